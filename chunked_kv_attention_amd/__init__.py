"""Same-step chunk attention on MI355X: Python face of libckv.so.

The library (include/ckv.h) does all the work: 3D RoPE + K/V append into
per-(layer, step) rings (optionally behind the QK-Norm), the clean
first-chunk sink, flash-style chunk attention over [sink | same-step window |
own chunk], and cross-attention to a stored text context.  This package only
marshals arguments; it loads the library lazily and raises if it was not
built.
"""

from ._abi import (  # noqa: F401
    CKV_E_ARENA, CKV_E_HIP, CKV_E_INVALID, CKV_E_ORDER, CKV_E_STATE, CKV_OK, EXPORTS, LIB_PATH, MAX_TEXT_TOKENS, STEP_SINK,
    Cache, CkvError, Config, cache_bytes, load, status_string,
)
