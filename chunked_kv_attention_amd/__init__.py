"""Same-step chunk attention on MI355X: Python face of libckv.so.

The library (include/ckv.h) does all the work: 3D RoPE + K/V append into
per-(layer, step) rings (optionally behind the QK-Norm), the clean
first-chunk sink, flash-style chunk attention over [sink | same-step window |
own chunk], cross-attention to a stored text context, and the streaming
causal 3D convolution of the video VAE decoder with its 2-frame temporal
cache (include/ckv_conv.h).  This package only
marshals arguments; it loads the library lazily and raises if it was not
built.
"""

from ._abi import (  # noqa: F401
    CKV_E_ARENA, CKV_E_HIP, CKV_E_INVALID, CKV_E_ORDER, CKV_E_STATE, CKV_OK, EXPORTS, LIB_PATH, MAX_TEXT_TOKENS, STEP_SINK,
    CONV_CACHE_T, Cache, CausalConv, CkvError, Config, ConvConfig, cache_bytes, conv_bytes, load, status_string,
)
