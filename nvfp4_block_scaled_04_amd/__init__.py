"""NVFP4 block-scaled MoE expert forward for AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``libnvfp4moe.so`` behind the C ABI in
``include/nvfp4moe.h``; ``binding`` is a thin ctypes layer over it (argument
marshalling, torch for device memory and streams).  ``inputs`` draws the
seeded synthetic workloads.
"""

from .binding import (  # noqa: F401
    EPI_BF16, EPI_SWIGLU_NVFP4, ExpertWeights, Nvfp4Error, PackedWeight, Taps, forward_workspace,
    forward_shared_workspace, moe_expert_forward_shared, moe_expert_forward_noalloc,
    gemm_splitk_workspace_bytes, gemm_workspace_bytes,
    grouped_gemm, lib, moe_combine, moe_expert_forward, moe_route, mx_expert_weights, pack_weights,
    prepare_expert_weights, quantize, quantize_scatter, router_topk, to_mx, weight_layout,
)

__version__ = "0.1.0"
