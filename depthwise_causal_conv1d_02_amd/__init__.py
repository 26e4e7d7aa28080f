"""MI355X-native depthwise causal conv1d (width 4, fused bias + SiLU, BF16).

The compute path is the HIP library ``libccv.so`` (gfx950) behind the C-ABI
declared in ``include/ccv.h``; this package is its thin Python binding.
"""
