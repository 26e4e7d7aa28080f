"""MI355X-native depthwise causal conv1d (width 4, fused bias + SiLU, BF16).

The compute path is the HIP library ``lib/libccv.so`` (gfx950) behind the
C-ABI declared in ``include/ccv.h``; this package is its thin Python binding.
"""
from .ops import (CcvError, bwd, causal_conv1d, causal_conv1d_update, check_flag, flag_tensor,
                  fwd, reset_flag, update, validate_cu_seqlens)

__all__ = ["causal_conv1d", "causal_conv1d_update", "validate_cu_seqlens", "check_flag",
           "reset_flag", "flag_tensor", "fwd", "bwd", "update", "CcvError"]
