"""Thin ctypes binding of libnvfp4moe.so (the C ABI in include/nvfp4moe.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, outputs and workspaces are allocated with torch (device memory
and the current stream are all torch provides), and every step of the path
runs in the HIP kernels behind the C ABI.  There is no fallback: if the
library is missing or the device is not a gfx950 the call raises.
"""

import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnvfp4moe.so")

EPI_BF16 = 0
EPI_SWIGLU_NVFP4 = 1

_lib = None
_lock = threading.Lock()

c_void_p, c_int64, c_int, c_size_t = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/nvfp4moe.h
SIGNATURES = {
    "nvfp4_status_string": (ctypes.c_char_p, [c_int]),
    "nvfp4_last_error": (ctypes.c_char_p, []),
    "nvfp4_version": (c_int, []),
    "nvfp4_weight_layout": (c_int, [c_void_p, c_int64, c_int64, c_int64, c_int, c_void_p, c_void_p]),
    "nvfp4_packed_weight_bytes": (c_size_t, [c_int64, c_int64, c_int64, ctypes.POINTER(c_size_t)]),
    "nvfp4_pack_weights": (c_int, [c_void_p, c_void_p, c_int64, c_int64, c_int64, c_void_p, c_void_p,
                                   c_void_p]),
    "nvfp4_quantize_workspace_size": (c_size_t, [c_int64, c_int64, c_int64]),
    "nvfp4_quantize": (c_int, [c_void_p, c_int64, c_int64, c_int64, c_int64, c_void_p, c_void_p,
                               c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "nvfp4_moe_route_workspace_size": (c_size_t, [c_int64, c_int, c_int]),
    "nvfp4_moe_route": (c_int, [c_void_p, c_int64, c_int, c_int, c_void_p, c_void_p, c_void_p,
                                c_void_p, c_void_p, c_size_t, c_void_p]),
    "nvfp4_grouped_gemm_workspace_size": (c_size_t, []),
    "nvfp4_grouped_gemm_splitk_workspace_size": (c_size_t, [c_int, c_int64, c_int64, c_int64, c_int]),
    "nvfp4_router_topk": (c_int, [c_void_p, c_int64, c_int, c_int, c_void_p, c_void_p, c_void_p]),
    "nvfp4_grouped_gemm": (c_int, [c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_void_p,
                                   c_int, c_int64, c_int64, c_int64, c_void_p, c_void_p, c_void_p,
                                   c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                   c_size_t, c_void_p]),
    "nvfp4_quantize_scatter_workspace_size": (c_size_t, [c_int64, c_int64]),
    "nvfp4_quantize_scatter": (c_int, [c_void_p, c_int64, c_int64, c_int, c_void_p, c_void_p, c_int,
                                       c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "nvfp4_to_mx": (c_int, [c_void_p, c_void_p, c_int64, c_int64, c_void_p, c_void_p, c_void_p]),
    "nvfp4_moe_combine": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_int, c_int,
                                  c_int64, c_void_p, c_void_p]),
    "moe_expert_forward_workspace_size": (c_size_t, [c_int64, c_int64, c_int64, c_int, c_int]),
    "moe_expert_forward": (c_int, [c_void_p, c_int64, c_int64, c_int64, c_int, c_int, c_void_p,
                                   c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                   c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                   c_void_p]),
}
# the MX variants take the same arguments as their NVFP4 counterparts
SIGNATURES["nvfp4_mx_grouped_gemm"] = SIGNATURES["nvfp4_grouped_gemm"]
SIGNATURES["moe_expert_forward_mx"] = SIGNATURES["moe_expert_forward"]
SIGNATURES["moe_expert_forward_shared"] = SIGNATURES["moe_expert_forward"]
SIGNATURES["moe_expert_forward_shared_workspace_size"] = SIGNATURES["moe_expert_forward_workspace_size"]
SIGNATURES["moe_expert_forward_noalloc"] = (c_int, SIGNATURES["moe_expert_forward"][1][:17] + [c_void_p])


class Taps(ctypes.Structure):
    """nvfp4_moe_taps: optional device pointers for the intermediates."""
    _fields_ = [(n, c_void_p) for n in ("a_q", "a_sf", "gs_a", "expert_offsets", "perm", "inv_perm",
                                        "invalid_count", "h_f32", "h_q", "h_sf", "y_bf16")]


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                                   "`python -m nvfp4_block_scaled_04_amd.build`")
            handle = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(handle, name)
                fn.restype, fn.argtypes = res, args
            _lib = handle
    return _lib


class Nvfp4Error(RuntimeError):
    def __init__(self, status, where):
        L = lib()
        self.status = status
        super().__init__(f"{where}: {L.nvfp4_status_string(status).decode()} "
                         f"({status}): {L.nvfp4_last_error().decode()}")


def _check(status, where):
    if status != 0:
        raise Nvfp4Error(status, where)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _dev(t, dtype, name, shape=None, rows=False):
    """Check a device tensor; rows=True accepts a 2-D tensor whose rows are
    contiguous but spaced apart (a row stride), as the row-strided calls do."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if rows:
        if t.dim() != 2 or t.stride(1) != 1 or (t.shape[0] > 1 and t.stride(0) < t.shape[1]):
            raise ValueError(f"{name} must be 2-D with contiguous rows")
    elif not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    return t


def _workspace(nbytes, device):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ entry points

def weight_layout(w, interleave_gate_up):
    """(G, R, C) bf16 -> (G, C, R) bf16: K-major, optionally gate/up interleaved."""
    _dev(w, torch.bfloat16, "w")
    G, R, C = w.shape
    out = torch.empty((G, C, R), dtype=torch.bfloat16, device=w.device)
    _check(lib().nvfp4_weight_layout(_ptr(w), G, R, C, int(bool(interleave_gate_up)), _ptr(out),
                                     _stream(w.device)), "nvfp4_weight_layout")
    return out


class PackedWeight:
    """NVFP4 weights of E experts, N rows of K elements, in the GEMM's packed
    layout (nvfp4_pack_weights): flat uint8 codes `q` and scales `sf`."""

    def __init__(self, q, sf, E, N, K):
        self.q, self.sf, self.E, self.N, self.K = q, sf, E, N, K


def pack_weights(q, sf):
    """Row-major NVFP4 weights q (E, N, K/2), sf (E, N, K/16) -> PackedWeight."""
    _dev(q, torch.uint8, "q")
    E, N, Kh = q.shape
    K = Kh * 2
    _dev(sf, torch.uint8, "sf", (E, N, K // 16))
    L = lib()
    sfb = c_size_t(0)
    qb = L.nvfp4_packed_weight_bytes(E, N, K, ctypes.byref(sfb))
    qp = torch.empty(max(qb, 1), dtype=torch.uint8, device=q.device)
    sfp = torch.empty(max(sfb.value, 1), dtype=torch.uint8, device=q.device)
    _check(L.nvfp4_pack_weights(_ptr(q), _ptr(sf), E, N, K, _ptr(qp), _ptr(sfp), _stream(q.device)),
           "nvfp4_pack_weights")
    return PackedWeight(qp, sfp, E, N, K)


def quantize_scatter(x, inv_perm, offsets, k, out=None):
    """x (T, H) bf16 -> NVFP4 rows in expert order: (q (T*k, H/2), sf (T*k, H/16),
    gs (1,)); row inv_perm[t*k+j] holds token t (routed pairs only)."""
    _dev(x, torch.bfloat16, "x")
    T, H = x.shape
    E = offsets.shape[0] - 1
    _dev(inv_perm, torch.int32, "inv_perm", (T * k,))
    _dev(offsets, torch.int32, "offsets")
    dev = x.device
    if out is not None:
        q, sf, gs = out
    else:
        q = torch.empty((T * k, H // 2), dtype=torch.uint8, device=dev)
        sf = torch.empty((T * k, H // 16), dtype=torch.uint8, device=dev)
        gs = torch.empty((1,), dtype=torch.float32, device=dev)
    L = lib()
    ws = _workspace(L.nvfp4_quantize_scatter_workspace_size(T, H), dev)
    _check(L.nvfp4_quantize_scatter(_ptr(x), T, H, k, _ptr(inv_perm), _ptr(offsets), E, _ptr(q),
                                    _ptr(sf), _ptr(gs), _ptr(ws), ws.numel(), _stream(dev)),
           "nvfp4_quantize_scatter")
    return q, sf, gs


def to_mx(q, sf, out=None):
    """NVFP4 (q (R, C/2), E4M3 sf (R, C/16)) -> MXFP4 (q_mx (R, C/2), E8M0
    sc_mx (R, C/16), each scale byte stored twice); out may be (q, sf) for an
    in-place re-encoding."""
    _dev(q, torch.uint8, "q")
    Ch = q.shape[-1]
    C = Ch * 2
    _dev(sf, torch.uint8, "sf")
    if sf.numel() != q.numel() // 8:
        raise ValueError("sf must hold one byte per 16 elements of q")
    rows = q.numel() // Ch
    qm, sm = out if out is not None else (torch.empty_like(q), torch.empty_like(sf))
    _check(lib().nvfp4_to_mx(_ptr(q), _ptr(sf), rows, C, _ptr(qm), _ptr(sm), _stream(q.device)),
           "nvfp4_to_mx")
    return qm, sm


def quantize(x, groups=1, gs_in=None, out=None):
    """x (R, C) bf16 -> (q (R, C/2) u8, sf (R, C/16) u8, gs (groups,) f32).
    x's rows may be spaced apart (x.stride(0) >= C, e.g. a column slice)."""
    _dev(x, torch.bfloat16, "x", rows=True)
    R, C = x.shape
    if groups < 1 or R % groups:
        raise ValueError("rows must divide evenly into groups")
    dev = x.device
    if out is None:
        q = torch.empty((R, C // 2), dtype=torch.uint8, device=dev)
        sf = torch.empty((R, C // 16), dtype=torch.uint8, device=dev)
        gs = torch.empty((groups,), dtype=torch.float32, device=dev)
    else:
        q, sf, gs = out
    if gs_in is not None:
        _dev(gs_in, torch.float32, "gs_in", (groups,))
    L = lib()
    nbytes = L.nvfp4_quantize_workspace_size(groups, R // groups, C) if gs_in is None else 0
    ws = _workspace(nbytes, dev)
    ld_x = x.stride(0) if R > 1 else C      # a one-row tensor's row stride is arbitrary
    _check(L.nvfp4_quantize(_ptr(x), groups, R // groups, C, ld_x, _ptr(gs_in), _ptr(q),
                            _ptr(sf), _ptr(gs), _ptr(ws), nbytes, _stream(dev)), "nvfp4_quantize")
    return q, sf, gs


def moe_route(topk_ids, E):
    """topk_ids (T, k) int32 -> (offsets (E+1,), perm (T*k,), inv_perm (T*k,), invalid (1,))."""
    _dev(topk_ids, torch.int32, "topk_ids")
    T, k = topk_ids.shape
    dev = topk_ids.device
    off = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    perm = torch.empty((T * k,), dtype=torch.int32, device=dev)
    inv = torch.empty((T * k,), dtype=torch.int32, device=dev)
    bad = torch.empty((1,), dtype=torch.int32, device=dev)
    L = lib()
    nbytes = L.nvfp4_moe_route_workspace_size(T, k, E)
    ws = _workspace(nbytes, dev)
    _check(L.nvfp4_moe_route(_ptr(topk_ids), T, k, E, _ptr(off), _ptr(perm), _ptr(inv), _ptr(bad),
                             _ptr(ws), nbytes, _stream(dev)), "nvfp4_moe_route")
    return off, perm, inv, bad


def router_topk(logits, k, out=None):
    """logits (T, E) float32 -> (topk_ids (T, k) int32, topk_w (T, k) float32):
    the k largest logits (equal ones in increasing id) and a softmax over them."""
    _dev(logits, torch.float32, "logits")
    T, E = logits.shape
    if out is not None:
        ids, w = out
    else:
        ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
        w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _check(lib().nvfp4_router_topk(_ptr(logits), T, E, k, _ptr(ids), _ptr(w), _stream(logits.device)),
           "nvfp4_router_topk")
    return ids, w


def gemm_workspace_bytes():
    """Workspace bytes nvfp4_grouped_gemm needs (the tile scheduler's counters)."""
    return int(lib().nvfp4_grouped_gemm_workspace_size())


def gemm_splitk_workspace_bytes(epilogue, M, N, K, E):
    """Workspace bytes with which nvfp4_grouped_gemm may split K for this shape
    on the current device (gemm_workspace_bytes() when it would not)."""
    return int(lib().nvfp4_grouped_gemm_splitk_workspace_size(epilogue, M, N, K, E))


def grouped_gemm(epilogue, a_q, a_sf, gs_a, offsets, b: PackedWeight, gs_b, M, a_row_src=None,
                 a_row_div=1, gs_out=None, debug=False, out=None, workspace=None, mx=False):
    """Expert-grouped NVFP4 GEMM with packed B.  BF16 epilogue returns c (M, N)
    bf16; the SwiGLU epilogue returns (c_q (M, N/4), c_sf (M, N/32), h f32
    (M, N/2) or None).  workspace: uint8 tensor of at least
    gemm_workspace_bytes() (allocated here when None)."""
    E, N, K = b.E, b.N, b.K
    dev = b.q.device
    _dev(a_q, torch.uint8, "a_q")
    _dev(a_sf, torch.uint8, "a_sf")
    _dev(b.q, torch.uint8, "b.q")
    _dev(b.sf, torch.uint8, "b.sf")
    _dev(gs_a, torch.float32, "gs_a")
    _dev(gs_b, torch.float32, "gs_b", (E,))
    _dev(offsets, torch.int32, "offsets", (E + 1,))
    if a_row_src is not None:
        _dev(a_row_src, torch.int32, "a_row_src")
    if epilogue == EPI_BF16:
        c = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        c_q = c_sf = dbg = None
    else:
        I = N // 2
        c = None
        if out is not None:
            c_q, c_sf, dbg = out
        else:
            c_q = torch.empty((M, I // 2), dtype=torch.uint8, device=dev)
            c_sf = torch.empty((M, I // 16), dtype=torch.uint8, device=dev)
            dbg = torch.empty((M, I), dtype=torch.float32, device=dev) if debug else None
        _dev(gs_out, torch.float32, "gs_out")
    ws = workspace if workspace is not None else torch.empty(gemm_workspace_bytes(), dtype=torch.uint8,
                                                             device=dev)
    _dev(ws, torch.uint8, "workspace")
    fn = lib().nvfp4_mx_grouped_gemm if mx else lib().nvfp4_grouped_gemm
    _check(fn(epilogue, _ptr(a_q), _ptr(a_sf), _ptr(gs_a), _ptr(a_row_src), a_row_div, _ptr(offsets),
              E, M, N, K, _ptr(b.q), _ptr(b.sf), _ptr(gs_b), _ptr(gs_out), _ptr(c), _ptr(c_q),
              _ptr(c_sf), _ptr(dbg), _ptr(ws), ws.numel(), _stream(dev)),
           "nvfp4_mx_grouped_gemm" if mx else "nvfp4_grouped_gemm")
    return c if epilogue == EPI_BF16 else (c_q, c_sf, dbg)


def moe_combine(y, inv_perm, topk_w, offsets, out=None):
    """y (T*k, H) bf16 in expert order -> out (T, H) bf16."""
    _dev(y, torch.bfloat16, "y")
    _dev(topk_w, torch.float32, "topk_w")
    T, k = topk_w.shape
    H = y.shape[1]
    E = offsets.shape[0] - 1
    _dev(inv_perm, torch.int32, "inv_perm", (T * k,))
    _dev(offsets, torch.int32, "offsets")
    o = out if out is not None else torch.empty((T, H), dtype=torch.bfloat16, device=y.device)
    _check(lib().nvfp4_moe_combine(_ptr(y), _ptr(inv_perm), _ptr(topk_w), _ptr(offsets), T, k, E, H,
                                   _ptr(o), _stream(y.device)), "nvfp4_moe_combine")
    return o


class ExpertWeights:
    """NVFP4 expert weights as the forward reads them: packed L1 (`w1`, rows
    interleaved gate/up) and L2 (`w2`) weights with per-expert global scales;
    optionally the row-major NVFP4 arrays they were packed from."""

    def __init__(self, w1: PackedWeight, gs_w1, w2: PackedWeight, gs_w2, rowmajor=None, mx=False):
        self.w1, self.gs_w1, self.w2, self.gs_w2 = w1, gs_w1, w2, gs_w2
        self.rowmajor = rowmajor or {}
        self.mx = mx          # packed from nvfp4_to_mx output (MX variant)

    @property
    def E(self):
        return self.w1.E

    @property
    def I(self):
        return self.w1.N // 2

    @property
    def H(self):
        return self.w1.K


def forward_workspace(T, H, I, E, k, device):
    return _workspace(lib().moe_expert_forward_workspace_size(T, H, I, E, k), device)


def moe_expert_forward(x, topk_ids, topk_w, w: ExpertWeights, gs_h, out=None, taps=None,
                       workspace=None):
    """The whole expert forward.  ``taps``: dict name -> device tensor to
    receive intermediates (keys of ``Taps``)."""
    _dev(x, torch.bfloat16, "x")
    T, H = x.shape
    E, I = w.E, w.I
    k = topk_ids.shape[1]
    dev = x.device
    _dev(topk_ids, torch.int32, "topk_ids", (T, k))
    _dev(topk_w, torch.float32, "topk_w", (T, k))
    if w.H != H or w.w2.N != H or w.w2.K != I or w.w2.E != E:
        raise ValueError("weight shapes do not match x")
    _dev(w.gs_w1, torch.float32, "gs_w1", (E,))
    _dev(w.gs_w2, torch.float32, "gs_w2", (E,))
    _dev(gs_h, torch.float32, "gs_h", (1,))
    o = out if out is not None else torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    L = lib()
    nbytes = L.moe_expert_forward_workspace_size(T, H, I, E, k)
    ws = workspace if workspace is not None else _workspace(nbytes, dev)
    tp = None
    if taps:
        tp = Taps(**{name: t.data_ptr() for name, t in taps.items()})
    fn = L.moe_expert_forward_mx if w.mx else L.moe_expert_forward
    _check(fn(_ptr(x), T, H, I, E, k, _ptr(topk_ids), _ptr(topk_w), _ptr(w.w1.q), _ptr(w.w1.sf),
              _ptr(w.gs_w1), _ptr(w.w2.q), _ptr(w.w2.sf), _ptr(w.gs_w2), _ptr(gs_h), _ptr(o),
              ctypes.byref(tp) if tp is not None else None, _ptr(ws), ws.numel(), _stream(dev)),
           "moe_expert_forward_mx" if w.mx else "moe_expert_forward")
    return o


NOALLOC_SCRATCH_BYTES = 64 << 20      # NVFP4_NOALLOC_SCRATCH_BYTES


def moe_expert_forward_noalloc(x, topk_ids, topk_w, w: ExpertWeights, gs_h, out, taps=None):
    """The expert forward on the library's static scratch (no workspace and
    no allocation: the caller passes the output)."""
    _dev(x, torch.bfloat16, "x")
    T, H = x.shape
    E, I = w.E, w.I
    k = topk_ids.shape[1]
    _dev(topk_ids, torch.int32, "topk_ids", (T, k))
    _dev(topk_w, torch.float32, "topk_w", (T, k))
    if w.mx or w.H != H or w.w2.N != H or w.w2.K != I or w.w2.E != E:
        raise ValueError("NVFP4 weights matching x expected")
    _dev(w.gs_w1, torch.float32, "gs_w1", (E,))
    _dev(w.gs_w2, torch.float32, "gs_w2", (E,))
    _dev(gs_h, torch.float32, "gs_h", (1,))
    _dev(out, torch.bfloat16, "out", (T, H))
    tp = Taps(**{name: t.data_ptr() for name, t in taps.items()}) if taps else None
    _check(lib().moe_expert_forward_noalloc(
        _ptr(x), T, H, I, E, k, _ptr(topk_ids), _ptr(topk_w), _ptr(w.w1.q), _ptr(w.w1.sf),
        _ptr(w.gs_w1), _ptr(w.w2.q), _ptr(w.w2.sf), _ptr(w.gs_w2), _ptr(gs_h), _ptr(out),
        ctypes.byref(tp) if tp is not None else None, _stream(x.device)),
        "moe_expert_forward_noalloc")
    return out


def forward_shared_workspace(T, H, I, E, k, device):
    return _workspace(lib().moe_expert_forward_shared_workspace_size(T, H, I, E, k), device)


def moe_expert_forward_shared(x, topk_ids, topk_w, w: ExpertWeights, gs_h, out=None, taps=None,
                              workspace=None):
    """The expert forward plus one shared expert: ``w`` holds E + 1 experts,
    the routed ones first and the shared expert last; topk_ids index the E
    routed ones.  Taps are sized for T*(k+1) rows and E+2 offsets."""
    _dev(x, torch.bfloat16, "x")
    T, H = x.shape
    E, I = w.E - 1, w.I
    k = topk_ids.shape[1]
    dev = x.device
    _dev(topk_ids, torch.int32, "topk_ids", (T, k))
    _dev(topk_w, torch.float32, "topk_w", (T, k))
    if w.mx:
        raise ValueError("the shared-expert forward takes the NVFP4 weights")
    if E < 1 or w.H != H or w.w2.N != H or w.w2.K != I:
        raise ValueError("weight shapes do not match x (E + 1 experts expected)")
    _dev(w.gs_w1, torch.float32, "gs_w1", (E + 1,))
    _dev(w.gs_w2, torch.float32, "gs_w2", (E + 1,))
    _dev(gs_h, torch.float32, "gs_h", (1,))
    o = out if out is not None else torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    L = lib()
    ws = workspace if workspace is not None else forward_shared_workspace(T, H, I, E, k, dev)
    tp = Taps(**{name: t.data_ptr() for name, t in taps.items()}) if taps else None
    _check(L.moe_expert_forward_shared(_ptr(x), T, H, I, E, k, _ptr(topk_ids), _ptr(topk_w),
                                       _ptr(w.w1.q), _ptr(w.w1.sf), _ptr(w.gs_w1), _ptr(w.w2.q),
                                       _ptr(w.w2.sf), _ptr(w.gs_w2), _ptr(gs_h), _ptr(o),
                                       ctypes.byref(tp) if tp is not None else None, _ptr(ws),
                                       ws.numel(), _stream(dev)), "moe_expert_forward_shared")
    return o


def prepare_expert_weights(w1_list, w2_list, device, keep_rowmajor=True):
    """Logical bf16 weights -> ExpertWeights on the device.

    w1_list: iterable of chunks (Ec, H, 2I) bf16 ([gate | up]); w2_list of
    (Ec, I, H).  Each chunk goes through nvfp4_weight_layout (interleave +
    K-major) and nvfp4_quantize (one global scale per expert); the stacked
    result is packed with nvfp4_pack_weights.  keep_rowmajor keeps the
    row-major NVFP4 arrays (for bit-exact checks) in `.rowmajor`."""
    w1q, w1s, g1, w2q, w2s, g2 = [], [], [], [], [], []
    for w1c, w2c in zip(w1_list, w2_list):
        Ec = w1c.shape[0]
        l1 = weight_layout(w1c, True)                     # (Ec, 2I, H)
        q, s, g = quantize(l1.view(-1, l1.shape[2]), groups=Ec)
        w1q.append(q.view(Ec, l1.shape[1], -1)); w1s.append(s.view(Ec, l1.shape[1], -1)); g1.append(g)
        del l1
        l2 = weight_layout(w2c, False)                    # (Ec, H, I)
        q, s, g = quantize(l2.view(-1, l2.shape[2]), groups=Ec)
        w2q.append(q.view(Ec, l2.shape[1], -1)); w2s.append(s.view(Ec, l2.shape[1], -1)); g2.append(g)
        del l2
    cat = lambda xs: xs[0] if len(xs) == 1 else torch.cat(xs)
    w1q, w1s, w2q, w2s = cat(w1q), cat(w1s), cat(w2q), cat(w2s)
    p1, p2 = pack_weights(w1q, w1s), pack_weights(w2q, w2s)
    rm = dict(w1_q=w1q, w1_sf=w1s, w2_q=w2q, w2_sf=w2s) if keep_rowmajor else None
    return ExpertWeights(p1, cat(g1), p2, cat(g2), rm)


def mx_expert_weights(w: ExpertWeights, keep_rowmajor=True):
    """The MX variant's weights: the row-major NVFP4 arrays of ``w`` (built
    with keep_rowmajor=True) re-encoded with nvfp4_to_mx and packed; the
    global scales carry over."""
    if not w.rowmajor:
        raise ValueError("mx_expert_weights needs the row-major NVFP4 weights (keep_rowmajor=True)")
    r = w.rowmajor
    q1, s1 = to_mx(r["w1_q"], r["w1_sf"])
    q2, s2 = to_mx(r["w2_q"], r["w2_sf"])
    p1, p2 = pack_weights(q1, s1), pack_weights(q2, s2)
    rm = dict(w1_q=q1, w1_sf=s1, w2_q=q2, w2_sf=s2) if keep_rowmajor else None
    return ExpertWeights(p1, w.gs_w1, p2, w.gs_w2, rm, mx=True)
