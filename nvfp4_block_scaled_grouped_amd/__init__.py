"""MI355X-native NVFP4 block-scaled grouped GEMM.

The computation lives in the HIP library ``libnvfp4gg.so`` (csrc/nvfp4gg.hip,
C ABI in include/nvfp4gg.h); this package only binds it.
"""
from ._lib import (HIP_ERROR, INVALID_ARG, OK, UNSUPPORTED, GroupGemmCall, Nvfp4Error, blocked_scale_bytes,
                   dequant_f16, group_gemm, group_gemm_batched, group_gemm_batched_ptrs, group_gemm_ptrs, last_error, load,
                   set_max_frags, set_wait_limit, version)

__all__ = ["group_gemm", "group_gemm_ptrs", "group_gemm_batched", "group_gemm_batched_ptrs", "blocked_scale_bytes", "set_wait_limit", "set_max_frags", "GroupGemmCall", "dequant_f16", "load", "last_error", "version",
           "Nvfp4Error", "OK", "INVALID_ARG", "UNSUPPORTED", "HIP_ERROR"]
