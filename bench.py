"""Benchmark of the NVFP4 MoE expert forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill]

A step is one moe_expert_forward over one batch of synthetic, seeded input
resident in HBM: quantise -> route -> L1 grouped GEMM with the fused SwiGLU +
NVFP4 requant epilogue -> L2 grouped GEMM -> combine.  W untimed steps, then
K timed steps between device synchronisations; rank 0 prints one JSON line.

Besides the headline figures the line carries
  roofline      the dominant kernel (the L1 grouped GEMM) timed with HIP
                events on the stream the library launches on: algorithmic
                FLOPs per launch / average launch time vs the FP16 dense MFMA
                peak (the GEMM's operand dtype);
  stages        average time of every step of the path, each timed alone;
  cpu_baseline  the CPU oracle on a bounded sample of the same workload,
                timed on this host.
"""

import argparse
import json
import os
import sys
import threading
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import nvfp4_block_scaled_04_amd as nv  # noqa: E402
from nvfp4_block_scaled_04_amd import inputs as I  # noqa: E402

FP16_MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense FP16 MFMA
FP4_MFMA_PEAK_TFLOPS = 10100.0      # MI355X dense FP4 MFMA (not the operand dtype used here)
HBM_PEAK_GBS = 8000.0
RIDGE = FP16_MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)   # flop per byte
# HBM traffic of the L1 grouped GEMM per launch (bytes), from two rocprofv3
# --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch),
# each scaled by the ratio of known bytes to the counter's reading for a plain
# 1 GiB device copy (--copy-calibration).  Reported only while the GEMM
# sources hash to the value the counters were taken with; otherwise null.
TRAFFIC = {("prefill", "l1", "nvfp4"): 5400771207, ("prefill", "l2", "nvfp4"): 3261715108}
TRAFFIC_SRC_SHA = "cb98f150662afe23"


def gemm_src_sha():
    import hashlib
    h = hashlib.sha256()
    for f in ("gemm.hip", "device.hpp"):
        with open(os.path.join(ROOT, "nvfp4_block_scaled_04_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def moe_flops(T, H, Iw, k):
    """Algorithmic FLOPs of one forward: L1 (2I outputs) + L2 (H outputs)."""
    return 2.0 * T * k * (H * 2 * Iw + Iw * H)


def build_weights(w, dev, chunk=32, keep_rowmajor=False, n_experts=None):
    w1s, w2s = [], []
    n = w.E if n_experts is None else n_experts
    for e0 in range(0, n, chunk):
        es = range(e0, min(n, e0 + chunk))
        pairs = [I.make_expert_weights(w, e, dev) for e in es]
        w1s.append(torch.stack([p[0] for p in pairs]))
        w2s.append(torch.stack([p[1] for p in pairs]))
        del pairs
    ew = nv.prepare_expert_weights(w1s, w2s, dev, keep_rowmajor=keep_rowmajor)
    del w1s, w2s
    torch.cuda.empty_cache()
    return ew


class Events:
    """HIP events on the current stream (the one the library launches on)."""

    def __init__(self):
        self.s = torch.cuda.Event(enable_timing=True)
        self.e = torch.cuda.Event(enable_timing=True)

    def __enter__(self):
        self.s.record(torch.cuda.current_stream())
        return self

    def __exit__(self, *a):
        self.e.record(torch.cuda.current_stream())

    def ms(self):
        self.e.synchronize()
        return self.s.elapsed_time(self.e)


PEAK_CLOCK_MHZ = 2400.0             # the clock the published peaks are quoted at


class SmuSampler:
    """GFX clock (MHz) and socket power (W) from the SMU metrics table (via
    amdsmi), read every ~10 ms on a host thread while a measured region runs.
    The chip runs its power-limited clock under these kernels, so a fraction
    of the 2.4 GHz peak is reported together with the clock it ran at."""

    def __init__(self):
        self.h = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            self.amdsmi = amdsmi
            if len(handles) == 1:
                self.h = handles[0]
            else:
                bus = torch.cuda.get_device_properties(0).pci_bus_id
                for h in handles:
                    bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)
                    if int(bdf.split(":")[1], 16) == bus:
                        self.h = h
        except Exception:
            self.h = None
        self.samples = []
        self._stop = threading.Event()
        self._thread = None

    def power_cap_w(self):
        try:
            return self.amdsmi.amdsmi_get_power_cap_info(self.h)["power_cap"] / 1e6
        except Exception:
            return None

    def _run(self):
        while not self._stop.is_set():
            try:
                m = self.amdsmi.amdsmi_get_gpu_metrics_info(self.h)
                clk, pw = m.get("current_gfxclk"), m.get("current_socket_power")
                if isinstance(clk, (int, float)) and 0 < clk < 10000 and isinstance(pw, (int, float)):
                    self.samples.append((float(clk), float(pw)))
            except Exception:
                pass
            time.sleep(0.01)

    def __enter__(self):
        self.samples = []
        if self.h is not None:
            self._stop.clear()
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *a):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
            self._thread = None

    def summary(self):
        if not self.samples:
            return None
        c = np.array(self.samples)
        return {"gfxclk_mhz": round(float(c[:, 0].mean()), 1),
                "socket_power_w": round(float(c[:, 1].mean()), 1), "samples": int(len(c))}


SMU = None


def smu():
    global SMU
    if SMU is None:
        SMU = SmuSampler()
    return SMU


def nvfp4_bytes(rows, cols):
    """Codes + E4M3 scales of an NVFP4 (rows, cols) tensor."""
    return rows * cols * 0.5625


def timed_steps(fn, steps):
    """Wall-clock mean over `steps` calls bracketed by synchronisations, and
    per-step HIP-event times (ms) for percentiles."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s, e in evs:
        s.record(torch.cuda.current_stream())
        fn()
        e.record(torch.cuda.current_stream())
    torch.cuda.synchronize()
    mean = (time.perf_counter() - t0) * 1e3 / steps
    per = np.array([s.elapsed_time(e) for s, e in evs])
    pct = {"p10": round(float(np.percentile(per, 10)), 4), "p50": round(float(np.median(per)), 4),
           "p90": round(float(np.percentile(per, 90)), 4)}
    return mean, pct


def roofline(kernel, flops, nbytes, ms, traffic=None, peak=FP16_MFMA_PEAK_TFLOPS, clock=None):
    """Roofline object for one kernel: MFMA-bound (against the MFMA peak of
    its operand dtype) when its arithmetic intensity is above that ridge,
    else HBM-bound.  clock: SMU summary of the kernel's timing loop; the
    MFMA peak scales with the GFX clock, so the fraction of the peak at the
    clock the chip sustained is reported beside the fraction of the 2.4 GHz
    figure."""
    if flops / max(nbytes, 1.0) >= peak * 1e12 / (HBM_PEAK_GBS * 1e9):
        a = flops / (ms * 1e-3) / 1e12
        r = {"kernel": kernel, "bound": "mfma", "achieved": round(a, 2),
             "peak": peak, "unit": "TFLOP/s",
             "frac": round(a / peak, 4), "traffic": traffic, "ms": round(ms, 4)}
        if clock:
            r.update(gfxclk_mhz=clock["gfxclk_mhz"], socket_power_w=clock["socket_power_w"],
                     peak_at_clock=round(peak * clock["gfxclk_mhz"] / PEAK_CLOCK_MHZ, 1),
                     frac_at_clock=round(a / (peak * clock["gfxclk_mhz"] / PEAK_CLOCK_MHZ), 4))
        return r
    a = nbytes / (ms * 1e-3) / 1e9
    return {"kernel": kernel, "bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(a / HBM_PEAK_GBS, 4), "traffic": traffic}


def time_loop(fn, steps):
    torch.cuda.synchronize()
    ev = Events()
    with ev:
        for _ in range(steps):
            fn()
    return ev.ms() / steps


CLOCK_LOOPS = True


def sustained(fn, secs=2.0, settle=0.8):
    """Run fn back to back for `secs` seconds and return (ms per call over
    the whole loop by HIP events, SMU summary over the part after `settle`
    seconds).  The SMU metrics table lags the workload by a few hundred
    milliseconds, so the clock and power of a kernel are read from a loop
    of this length rather than from the short timed regions."""
    if not CLOCK_LOOPS:
        return None, None
    torch.cuda.synchronize()
    smp = smu()
    with smp:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(torch.cuda.current_stream())
        n = 0
        t_settle = None
        while time.perf_counter() - t0 < secs:
            fn()
            n += 1
            if n % 4 == 0:
                torch.cuda.synchronize()
                if t_settle is None and time.perf_counter() - t0 >= settle:
                    t_settle = len(smp.samples)
        e1.record(torch.cuda.current_stream())
        e1.synchronize()
    ms = e0.elapsed_time(e1) / n
    keep = smp.samples[t_settle:] if t_settle is not None else []
    if not keep:
        return ms, None
    c = np.array(keep)
    return ms, {"gfxclk_mhz": round(float(c[:, 0].mean()), 1),
                "socket_power_w": round(float(c[:, 1].mean()), 1), "samples": int(len(c)),
                "loop_ms": round(ms, 4), "loop_s": secs}


def bench_shared(w, steps, warmup, dev):
    """The forward plus one shared expert (E + 1 experts, the shared one
    last, every token through it with weight 1): whole-forward time only."""
    log(f"[bench] building weights for {w.name} + shared expert: E={w.E}+1 H={w.H} I={w.I}")
    ew = build_weights(w, dev, n_experts=w.E + 1)
    x = I.make_x(w, dev)
    ids_h, tw_h = I.make_routing(w)
    ids = torch.from_numpy(ids_h).to(dev)
    tw = torch.from_numpy(tw_h).to(dev)
    gs_h = torch.tensor([w.gs_h], dtype=torch.float32, device=dev)
    out = torch.empty((w.T, w.H), dtype=torch.bfloat16, device=dev)
    ws = nv.forward_shared_workspace(w.T, w.H, w.I, w.E, w.k, dev)
    step = lambda: nv.moe_expert_forward_shared(x, ids, tw, ew, gs_h, out=out, workspace=ws)
    for _ in range(warmup):
        step()
    ms_step, pct = timed_steps(step, steps)
    log(f"[bench] forward + shared expert {ms_step:.3f} ms/step")
    flops = moe_flops(w.T, w.H, w.I, w.k + 1)
    return flops / (ms_step * 1e-3) / 1e12, ms_step, pct


def bench_moe(w, steps, warmup, dev, mx=False):
    log(f"[bench] building weights for {w.name}: E={w.E} H={w.H} I={w.I}" + (" (MX variant)" if mx else ""))
    t0 = time.time()
    ew_nv = build_weights(w, dev, keep_rowmajor=mx)
    ew = nv.mx_expert_weights(ew_nv, keep_rowmajor=False) if mx else ew_nv
    x = I.make_x(w, dev)
    ids_h, tw_h = I.make_routing(w)
    ids = torch.from_numpy(ids_h).to(dev)
    tw = torch.from_numpy(tw_h).to(dev)
    gs_h = torch.tensor([w.gs_h], dtype=torch.float32, device=dev)
    out = torch.empty((w.T, w.H), dtype=torch.bfloat16, device=dev)
    ws = nv.forward_workspace(w.T, w.H, w.I, w.E, w.k, dev)
    torch.cuda.synchronize()
    log(f"[bench] inputs ready in {time.time() - t0:.1f}s; warmup {warmup}, timed {steps}")

    step = lambda: nv.moe_expert_forward(x, ids, tw, ew, gs_h, out=out, workspace=ws)
    for _ in range(warmup):
        step()
    ms_step, pct = timed_steps(step, steps)
    log(f"[bench] forward {ms_step:.3f} ms/step (p10/p50/p90 {pct['p10']}/{pct['p50']}/{pct['p90']})")
    step_clk = sustained(step)[1]
    log(f"[bench] forward sustained SMU reading: {step_clk}")

    # ---- each step alone, same kernels and arguments, events on the stream
    T, H, Iw, E, k = w.T, w.H, w.I, w.E, w.k
    M = T * k
    a_q, a_sf, gs_a = nv.quantize(x)
    off, perm, inv, bad = nv.moe_route(ids, E)
    h_q = torch.empty((M, Iw // 2), dtype=torch.uint8, device=dev)
    h_sf = torch.empty((M, Iw // 16), dtype=torch.uint8, device=dev)
    y = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    qbuf = (a_q, a_sf, gs_a)
    if mx:          # the GEMMs read MX operands: re-encode once, as the forward does
        nv.to_mx(a_q, a_sf, out=(a_q, a_sf))
    l1 = lambda: nv.grouped_gemm(nv.EPI_SWIGLU_NVFP4, a_q, a_sf, gs_a, off, ew.w1,
                                 ew.gs_w1, M, a_row_src=perm, a_row_div=k, gs_out=gs_h,
                                 out=(h_q, h_sf, None), mx=mx)
    if mx:
        l1()
        nv.to_mx(h_q, h_sf, out=(h_q, h_sf))
    l2 = lambda: nv.grouped_gemm(nv.EPI_BF16, h_q, h_sf, gs_h, off, ew.w2, ew.gs_w2,
                                 M, out=y, mx=mx)
    qx = torch.empty_like(a_q), torch.empty_like(a_sf), torch.empty_like(gs_a)
    stages = {
        "quantize": lambda: nv.quantize(x, out=qx),
        "route": lambda: nv.moe_route(ids, E),
        "l1_gemm_swiglu_requant": l1,
        "l2_gemm": l2,
        "combine": lambda: nv.moe_combine(y, inv, tw, off, out=out),
    }
    if not mx:
        # the alternative A path (not the forward's): quantise each token once
        # straight into its k expert-order rows, for L1 without the row gather
        sq = (torch.empty((M, H // 2), dtype=torch.uint8, device=dev),
              torch.empty((M, H // 16), dtype=torch.uint8, device=dev),
              torch.empty((1,), dtype=torch.float32, device=dev))
        stages["quantize_scatter"] = lambda: nv.quantize_scatter(x, inv, off, k, out=sq)
    if mx:
        stages["to_mx_x"] = lambda: nv.to_mx(qx[0], qx[1], out=(qx[0], qx[1]))
        hq2, hs2 = torch.empty_like(h_q), torch.empty_like(h_sf)
        stages["to_mx_h"] = lambda: nv.to_mx(h_q, h_sf, out=(hq2, hs2))
    st_ms = {}
    for name, fn in stages.items():
        fn()
        st_ms[name] = time_loop(fn, steps)
    # sustained loops for the clock and power the two GEMMs run at
    st_clk = {n: sustained(stages[n])[1] for n in ("l1_gemm_swiglu_requant", "l2_gemm")}
    log(f"[bench] sustained SMU readings: {st_clk}")
    log("[bench] stages (ms): " + ", ".join(f"{n}={v:.4f}" for n, v in st_ms.items()))
    # the step before the path (not in the timed forward, which takes ids and
    # weights): router top-k + softmax on N(0,1) logits of this shape
    logits = torch.from_numpy(I.make_router_logits(w)).to(dev)
    rbuf = (torch.empty((T, k), dtype=torch.int32, device=dev),
            torch.empty((T, k), dtype=torch.float32, device=dev))
    router = lambda: nv.router_topk(logits, k, out=rbuf)
    router()
    router_ms = time_loop(router, steps)

    l1_flops = 2.0 * M * (2 * Iw) * H
    l2_flops = 2.0 * M * H * Iw
    flops = moe_flops(T, H, Iw, k)
    # algorithmic bytes: weights of the experts that hold rows, each once;
    # A rows gathered, h written (L1); h read, y written (L2)
    n_live = int(np.unique(ids_h[(ids_h >= 0) & (ids_h < E)]).size)
    w1_bytes, w2_bytes = n_live * nvfp4_bytes(2 * Iw, H), n_live * nvfp4_bytes(H, Iw)
    l1_bytes = w1_bytes + nvfp4_bytes(M, H) + nvfp4_bytes(M, Iw)
    l2_bytes = w2_bytes + nvfp4_bytes(M, Iw) + 2.0 * M * H
    peak = FP4_MFMA_PEAK_TFLOPS if mx else FP16_MFMA_PEAK_TFLOPS
    roof = roofline("grouped_gemm_kernel<SwiGLU+NVFP4 epilogue> (L1)" + (" MX" if mx else ""),
                    l1_flops, l1_bytes, st_ms["l1_gemm_swiglu_requant"],
                    TRAFFIC.get((w.name, "l1", "mx" if mx else "nvfp4"))
                    if TRAFFIC_SRC_SHA == gemm_src_sha() else None,
                    peak=peak, clock=st_clk["l1_gemm_swiglu_requant"])
    extra = {
        "ms_percentiles": pct,
        "live_experts": n_live,
        "weight_stream_gbs": (w1_bytes + w2_bytes) / (ms_step * 1e-3) / 1e9,
        "l2_roofline": roofline("grouped_gemm_kernel<BF16 epilogue> (L2)" + (" MX" if mx else ""),
                                l2_flops, l2_bytes, st_ms["l2_gemm"],
                                TRAFFIC.get((w.name, "l2", "mx" if mx else "nvfp4"))
                                if TRAFFIC_SRC_SHA == gemm_src_sha() else None,
                                peak=peak, clock=st_clk["l2_gemm"]),
        "step_clock": step_clk,
        "tokens_per_s": T / (ms_step * 1e-3),
        "l2_gemm_tflops": l2_flops / (st_ms["l2_gemm"] * 1e-3) / 1e12,
        "quantize_gbs": (2 * T * H + 0.5625 * T * H) / (st_ms["quantize"] * 1e-3) / 1e9,
        "combine_gbs": (2 * M * H + 12 * M + 2 * T * H) / (st_ms["combine"] * 1e-3) / 1e9,
        "stages_ms": {n: round(v, 4) for n, v in st_ms.items()},
        "router_topk_ms": round(router_ms, 4),
    }
    if mx:
        # error study: the MX forward against the exact NVFP4 forward, same inputs
        ref = nv.moe_expert_forward(x, ids, tw, ew_nv, gs_h)
        got = nv.moe_expert_forward(x, ids, tw, ew, gs_h)
        a, b = ref.float().ravel(), got.float().ravel()
        extra["mx_vs_exact_cosine"] = round(float((a @ b) / (a.norm() * b.norm())), 6)
        extra["mx_vs_exact_maxabs_over_rms"] = round(float((a - b).abs().max() / a.pow(2).mean().sqrt()), 4)
        log(f"[bench] MX vs exact NVFP4 forward: cosine {extra['mx_vs_exact_cosine']}")
    return flops / (ms_step * 1e-3) / 1e12, ms_step, roof, extra, (x, ids_h, tw_h, ew_nv)


def bench_dense(w, steps, warmup, dev, mx=False):
    """The single NVFP4 linear (one expert): quantise A, then the GEMM with a
    BF16 epilogue; each timed alone, and both together as the step."""
    M, K, N = w.dense_mkn
    log(f"[bench] dense M={M} K={K} N={N}")
    a, b = I.make_dense(w, dev)
    bk = nv.weight_layout(b.view(1, K, N), False)[0]                     # (N, K)
    b_q, b_sf, gs_b = nv.quantize(bk)
    bp = nv.pack_weights(b_q.view(1, N, K // 2), b_sf.view(1, N, K // 16))
    bp_nv = bp
    if mx:
        bmq, bms = nv.to_mx(b_q, b_sf)
        bp = nv.pack_weights(bmq.view(1, N, K // 2), bms.view(1, N, K // 16))
    a_q, a_sf, gs_a = nv.quantize(a)
    off = torch.tensor([0, M], dtype=torch.int32, device=dev)
    c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    # a workspace large enough for split K (128 tiles cannot fill 256 CUs)
    gws = torch.empty(nv.gemm_splitk_workspace_bytes(nv.EPI_BF16, M, N, K, 1), dtype=torch.uint8,
                      device=dev)
    qbuf = (a_q, a_sf, gs_a)
    def quant():
        nv.quantize(a, out=qbuf)
        if mx:
            nv.to_mx(a_q, a_sf, out=(a_q, a_sf))
    gemm = lambda: nv.grouped_gemm(nv.EPI_BF16, a_q, a_sf, gs_a, off, bp, gs_b, M, out=c,
                                   workspace=gws, mx=mx)

    def step():
        quant()
        gemm()
    for _ in range(warmup):
        step()
    ms_step, pct = timed_steps(step, steps)
    st_ms = {"quantize": time_loop(quant, steps), "gemm": time_loop(gemm, steps)}
    gemm_clk = sustained(gemm)[1]
    log(f"[bench] dense step {ms_step:.4f} ms; stages (ms): " +
        ", ".join(f"{n}={v:.4f}" for n, v in st_ms.items()))
    flops = 2.0 * M * N * K
    nbytes = nvfp4_bytes(M, K) + nvfp4_bytes(N, K) + 2.0 * M * N
    roof = roofline("grouped_gemm_kernel<BF16 epilogue> (dense)" + (" MX" if mx else ""), flops,
                    nbytes, st_ms["gemm"],
                    peak=FP4_MFMA_PEAK_TFLOPS if mx else FP16_MFMA_PEAK_TFLOPS, clock=gemm_clk)
    extra = {"ms_percentiles": pct, "stages_ms": {n: round(v, 4) for n, v in st_ms.items()},
             "gemm_tflops": round(flops / (st_ms["gemm"] * 1e-3) / 1e12, 2),
             "split_k": gws.numel() > nv.gemm_workspace_bytes(),
             # A (16.5 MB) and B (8.3 MB) stay resident in the 256 MB last-level cache
             # between steps, unlike the MoE workloads' 6.3 GB of expert weights
             "cache": "warm",
             "quantize_gbs": round((2.0 * M * K + nvfp4_bytes(M, K)) / (st_ms["quantize"] * 1e-3) / 1e9, 1)}
    return flops / (ms_step * 1e-3) / 1e12, ms_step, roof, extra


def cpu_baseline(w, x, ids_h, tw_h, dev, budget_s=20.0):
    """The CPU oracle (as it stands) on a bounded sample of the workload:
    all rows of the first few experts through L1 -> SwiGLU -> requant -> L2,
    plus quantise and combine for the same share of tokens.  Weight
    quantisation is preparation on both sides and is not timed."""
    from threadpoolctl import threadpool_info
    from oracle import moe as O, quantize as Q, route as R

    xb = x.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    offsets, perm, inv, _ = R.route(ids_h, w.E)
    done_flops, t_total, experts = 0.0, 0.0, 0
    per_tok = moe_flops(1, w.H, w.I, w.k)
    gs_h = np.float32(w.gs_h)
    t0 = time.perf_counter()
    gs_a = Q.global_scale(xb)
    t_total += time.perf_counter() - t0
    for e in range(w.E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        w1, w2 = I.make_expert_weights(w, e, dev)
        prep = O.prepare_expert_weights(*[t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
                                          for t in (w1, w2)])
        tok = perm[lo:hi] // w.k
        t0 = time.perf_counter()
        codes, a_sf = Q.quantize_blocks(xb[tok], gs_a)          # this share of the quantise step
        h = O.l1_swiglu(Q.pack_codes(codes), a_sf, gs_a, prep["w1_q"], prep["w1_sf"], prep["gs_w1"])
        hc, hsf = Q.quantize_blocks(h, gs_h)
        y = O.l2(Q.pack_codes(hc), hsf, gs_h, prep["w2_q"], prep["w2_sf"], prep["gs_w2"])
        t_total += time.perf_counter() - t0
        done_flops += 2.0 * (hi - lo) * (w.H * 2 * w.I + w.I * w.H)
        experts += 1
        if t_total >= budget_s:
            break
    rows = int(offsets[experts]) if experts else 0
    # combine for the same number of rows' tokens (k rows per token)
    ntok = max(1, rows // w.k)
    ysim = np.zeros((w.T * w.k, w.H), np.uint16)
    t0 = time.perf_counter()
    O.combine(ysim, inv.reshape(w.T, w.k)[:ntok].ravel(), tw_h[:ntok], w.T * w.k)
    t_total += time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next((l.split(":", 1)[1].strip() for l in fh if l.startswith("model name")), "")
    except OSError:
        pass
    tflops = done_flops / t_total / 1e12
    return {"value": round(tflops, 6), "unit": "TFLOPS", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model,
            "sample": f"{experts} of {w.E} experts ({rows} of {w.T * w.k} expert rows): quantize "
                      f"+ L1 + SwiGLU + requant + L2 for their rows, combine for {ntok} tokens",
            "seconds": round(t_total, 2),
            "tokens_per_s": round(done_flops / per_tok / t_total, 3)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill", choices=sorted(I.WORKLOADS))
    ap.add_argument("--variant", default="nvfp4", choices=["nvfp4", "mx"],
                    help="nvfp4: exact E4M3/16 path (FP16 MFMA); mx: NVFP4 re-encoded to "
                         "E8M0/32 on the scaled FP4 MFMA")
    ap.add_argument("--shared", action="store_true",
                    help="add one shared expert (every token, weight 1) to the MoE forward")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the 2 s loops that read the SMU clock and power (for profiler runs)")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy 1 GiB device-to-device 3 times (counter calibration)")
    args = ap.parse_args()
    global CLOCK_LOOPS
    CLOCK_LOOPS = not args.no_clock
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel() * 4, "copies": 3}))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the expert-parallel "
              "sharding over several GPUs is a design note, not built.", file=sys.stderr)
        sys.exit(2)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    w = I.WORKLOADS[args.workload]
    mx = args.variant == "mx"
    common = {"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
              "scaling": "weak", "vs_baseline": None, "dtype": "fp4" if mx else "fp16",
              "variant": "mx (E2M1 + E8M0/32, scaled FP4 MFMA)" if mx else "nvfp4 (exact decode, FP16 MFMA)",
              "data": "synthetic (seeded; weights N(0,0.02), activations N(0,1))"}
    if w.dense_mkn:
        M, K, N = w.dense_mkn
        value, ms_step, roof, extra = bench_dense(w, args.steps, args.warmup, dev, mx)
        line = {"metric": f"NVFP4 dense linear TFLOPS, M={M} K={K} N={N} (quantize A + GEMM)",
                "value": round(value, 3), "unit": "TFLOPS", "ms_per_step": round(ms_step, 4),
                **common,
                "config": {"workload": f"dense M={M} K={K} N={N}", "rows": M, "k_dim": K,
                           "n_dim": N, "parallelism": "single GPU"},
                "frac_fp16_mfma_peak": round(value / FP16_MFMA_PEAK_TFLOPS, 4),
                "frac_fp4_mfma_peak": round(value / FP4_MFMA_PEAK_TFLOPS, 4),
                "roofline": roof, **extra, "cpu_baseline": None}
        print(json.dumps(line), flush=True)
        return
    if args.shared:
        value, ms_step, pct = bench_shared(w, args.steps, args.warmup, dev)
        line = {"metric": f"NVFP4 MoE fwd + shared expert TFLOPS, T={w.T} E={w.E}+1 top-{w.k}",
                "value": round(value, 3), "unit": "TFLOPS", "ms_per_step": round(ms_step, 4),
                **common,
                "config": {"workload": f"{w.name} + shared expert T={w.T} H={w.H} I={w.I} "
                                       f"E={w.E}+1 top-{w.k}+1", "parallelism": "single GPU"},
                "tokens_per_s": round(w.T / (ms_step * 1e-3), 1),
                "frac_fp16_mfma_peak": round(value / FP16_MFMA_PEAK_TFLOPS, 4),
                "ms_percentiles": pct, "cpu_baseline": None}
        print(json.dumps(line), flush=True)
        return
    value, ms_step, roof, extra, keep = bench_moe(w, args.steps, args.warmup, dev, mx)
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        x, ids_h, tw_h, _ = keep
        cpu = cpu_baseline(w, x, ids_h, tw_h, dev, args.cpu_budget)
        log(f"[bench] cpu oracle: {cpu}")
    line = {
        "metric": f"NVFP4 MoE fwd TFLOPS + tokens/s, T={w.T} E={w.E} top-{w.k}; % of MFMA peak",
        "value": round(value, 3), "unit": "TFLOPS", "ms_per_step": round(ms_step, 4), **common,
        "config": {"workload": f"{w.name} T={w.T} H={w.H} I={w.I} E={w.E} top-{w.k}",
                   "tokens": w.T, "hidden": w.H, "intermediate": w.I, "experts": w.E,
                   "top_k": w.k, "expert_rows": w.M, "parallelism": "single GPU"},
        "tokens_per_s": round(extra["tokens_per_s"], 1),
        "frac_fp16_mfma_peak": round(value / FP16_MFMA_PEAK_TFLOPS, 4),
        "frac_fp4_mfma_peak": round(value / FP4_MFMA_PEAK_TFLOPS, 4),
        "ms_percentiles": extra["ms_percentiles"],
        "roofline": roof,
        "l2_roofline": extra["l2_roofline"],
        "clock": dict(extra["step_clock"], power_cap_w=smu().power_cap_w(),
                      source="SMU gpu_metrics (amdsmi) every 10 ms over a 2 s loop of the step, "
                             "after 0.8 s")
        if extra["step_clock"] else None,
        "stages_ms": extra["stages_ms"],
        "router_topk_ms": extra["router_topk_ms"],
        "l2_gemm_tflops": round(extra["l2_gemm_tflops"], 2),
        "weight_stream_gbs": round(extra["weight_stream_gbs"], 1),
        "live_experts": extra["live_experts"],
        "quantize_gbs": round(extra["quantize_gbs"], 1),
        "combine_gbs": round(extra["combine_gbs"], 1),
        "cpu_baseline": cpu,
        **{n: extra[n] for n in ("mx_vs_exact_cosine", "mx_vs_exact_maxabs_over_rms") if n in extra},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
