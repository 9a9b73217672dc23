"""MI355X (gfx950) sparse Mixture-of-Experts layer with 2-, 3- and
4-bit block-quantised experts: HIP kernels behind a C ABI (include/moe.h), bound
here with ctypes."""

from ._lib import (  # noqa: F401
    FFN_REUSE_PLAN, FFN_SKIP_DOWN, FFN_SKIP_GATEUP, ROUTE_TAIL_SKIP, MoeError, QArena, QLayer, Shape, alloc_workspace, combine, dequant, expert_ffn, layer_forward, layer_forward_noalloc, lib,
    permute,
    quantize, read_error, repack, rmsnorm_bf16, route, workspace_bytes,
)
