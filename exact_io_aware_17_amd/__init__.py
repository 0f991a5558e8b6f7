"""MI355X-native exact attention: libfa (C-ABI, gfx950 HIP kernels) and its binding.

    from exact_io_aware_17_amd import fwd, bwd
    o, lse = fwd(q, k, v, causal=True)    # bf16, fp16 or fp32 GPU tensors: q [B, H, Nq, d],
                                          # k, v [B, Hkv, Nk, d]
    dq, dk, dv = bwd(q, k, v, o, lse, do, causal=True)

The library is loaded on first use; importing this package touches no GPU.
"""
from ._lib import (  # noqa: F401
    FA_DTYPE_BF16,
    FA_DTYPE_F16,
    FA_DTYPE_F32,
    FA_ERR_HIP,
    FA_ERR_INVALID_ARG,
    FA_BWD_DKDV_HEAD_SEQUENTIAL,
    FA_BWD_DQ_HEAD_SEQUENTIAL,
    FA_ERR_UNSUPPORTED,
    FA_FWD_ORDER_HEAD_SEQUENTIAL,
    FA_FWD_ORDER_HEAVY_FIRST,
    FA_FWD_ORDER_PAIRED,
    FA_MASK_CAUSAL,
    FA_MASK_CAUSAL_STRICT,
    FA_MASK_NONE,
    FA_OK,
    FaError,
    block_keys,
    bwd,
    bwd_tile_order,
    bwd_workspace_bytes,
    default_scale,
    dtype_code,
    fwd,
    fwd_noalloc,
    load,
    mask_kind,
    schedule,
    split_workspace_bytes,
    status_string,
    tile_order,
)
