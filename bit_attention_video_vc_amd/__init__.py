"""VC-Attention hot path for AMD Instinct MI355X (gfx950).

The compute runs in hand-written HIP kernels behind the C ABI in
include/vc.h (libvc.so, built in-tree by build.py).  This package is the thin
Python binding: it marshals torch tensors (device memory and the current HIP
stream) into that ABI and allocates the outputs.
"""
from .binding import (  # noqa: F401
    VcError, lib, lib_path, vsmooth_group, preprocess_quant, attn_fp8_fwd, attn_bf16_fwd,
    attn_fp8_fwd_dump, attn_fwd_dump, device_probe, unswizzle_v_codes, group_due, group_source, group_count, PermutationCache, P_EXPCAST, P_FP32EXP_E4M3, P_FP32_BF16, V_E4M3, V_NVFP4, V_MXFP4,
)
