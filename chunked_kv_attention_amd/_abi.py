"""ctypes binding of libckv.so (include/ckv.h, include/ckv_conv.h): argument
marshalling only.

Every operation runs in the HIP library; this module checks tensor shapes and
dtypes, passes device pointers and the current HIP stream, and turns status
codes into exceptions.  It raises if the library has not been built.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libckv.so")

CKV_OK, CKV_E_INVALID, CKV_E_ORDER, CKV_E_STATE, CKV_E_ARENA, CKV_E_HIP = range(6)
STEP_SINK = -1
MAX_TEXT_TOKENS = 512

CONV_CACHE_T = 2

# Every symbol include/*.h declares.
EXPORTS = (
    "ckv_cache_bytes", "ckv_cache_create", "ckv_cache_create_dry", "ckv_cache_reset",
    "ckv_cache_destroy", "ckv_rope_append", "ckv_sink_build", "ckv_norm_rope_append",
    "ckv_norm_sink_build", "ckv_chunk_attention", "ckv_chunk_attention_static", "ckv_text_store",
    "ckv_cross_attention",
    "ckv_window", "ckv_ring_slot", "ckv_debug_copy_kv", "ckv_attention_splits",
    "ckv_status_string",
    "ckv_conv_bytes", "ckv_conv_create", "ckv_conv_create_dry", "ckv_conv_set_weights", "ckv_conv_reset",
    "ckv_causal_conv", "ckv_conv_position", "ckv_conv_splits", "ckv_conv_destroy",
)


class CkvConfig(ctypes.Structure):
    _fields_ = [
        ("num_layers", ctypes.c_int32),
        ("num_steps", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("grid_h", ctypes.c_int32),
        ("grid_w", ctypes.c_int32),
        ("first_chunk_frames", ctypes.c_int32),
        ("window_chunks", ctypes.c_int32),
        ("max_chunks", ctypes.c_int32),
        ("reserved0", ctypes.c_int32),
        ("rope_theta", ctypes.c_double),
        ("softmax_scale", ctypes.c_float),
        ("reserved1", ctypes.c_int32),
    ]


assert ctypes.sizeof(CkvConfig) == 56


class CkvConvConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("height", "width", "in_channels", "out_channels", "kt", "kh", "kw",
                                              "max_frames")]


class CkvSegment(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("kind", "first_slot", "chunk_first", "n_chunks", "n_tokens")]


class CkvError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


_lib = None


def load() -> ctypes.CDLL:
    """Load libckv.so once; raises if it was not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m chunked_kv_attention_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    cfgp = ctypes.POINTER(CkvConfig)
    sig = {
        "ckv_cache_bytes": (SZ, [cfgp]),
        "ckv_cache_create": (I32, [cfgp, P, SZ, ctypes.POINTER(P)]),
        "ckv_cache_create_dry": (I32, [cfgp, ctypes.POINTER(P)]),
        "ckv_cache_reset": (I32, [P]),
        "ckv_cache_destroy": (I32, [P]),
        "ckv_rope_append": (I32, [P, I32, I32, I32, P, P, P, P, P]),
        "ckv_sink_build": (I32, [P, I32, P, P, P, P, P]),
        "ckv_norm_rope_append": (I32, [P, I32, I32, I32, P, P, P, P, P, ctypes.c_float, P, P]),
        "ckv_norm_sink_build": (I32, [P, I32, P, P, P, P, P, ctypes.c_float, P, P]),
        "ckv_chunk_attention": (I32, [P, I32, I32, I32, P, P, P]),
        "ckv_chunk_attention_static": (I32, [P, I32, I32, I32, P, P, P]),
        "ckv_text_store": (I32, [P, I32, P, P, I32, P]),
        "ckv_cross_attention": (I32, [P, I32, I32, P, P, P]),
        "ckv_window": (I32, [P, I32, I32, I32, ctypes.POINTER(CkvSegment), I32, ctypes.POINTER(I32)]),
        "ckv_ring_slot": (I32, [P, I32, ctypes.POINTER(I32)]),
        "ckv_debug_copy_kv": (I32, [P, I32, I32, I32, P, P, P]),
        "ckv_attention_splits": (I32, [P, I32, I32]),
        "ckv_status_string": (ctypes.c_char_p, [I32]),
        "ckv_conv_bytes": (SZ, [ctypes.POINTER(CkvConvConfig)]),
        "ckv_conv_create": (I32, [ctypes.POINTER(CkvConvConfig), P, SZ, ctypes.POINTER(P)]),
        "ckv_conv_create_dry": (I32, [ctypes.POINTER(CkvConvConfig), ctypes.POINTER(P)]),
        "ckv_conv_set_weights": (I32, [P, P, P, P]),
        "ckv_conv_reset": (I32, [P]),
        "ckv_causal_conv": (I32, [P, P, I32, P, P]),
        "ckv_conv_position": (ctypes.c_int64, [P]),
        "ckv_conv_splits": (I32, [P, I32, ctypes.POINTER(I32)]),
        "ckv_conv_destroy": (I32, [P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(st: int) -> str:
    return load().ckv_status_string(int(st)).decode()


@dataclass(frozen=True)
class Config:
    num_layers: int
    num_steps: int
    num_heads: int
    head_dim: int
    grid_h: int
    grid_w: int
    first_chunk_frames: int
    window_chunks: int
    max_chunks: int
    rope_theta: float = 10000.0
    softmax_scale: float = 0.0

    def to_c(self) -> CkvConfig:
        return CkvConfig(self.num_layers, self.num_steps, self.num_heads, self.head_dim, self.grid_h,
                         self.grid_w, self.first_chunk_frames, self.window_chunks, self.max_chunks, 0,
                         float(self.rope_theta), float(self.softmax_scale), 0)

    @property
    def frame_tokens(self) -> int:
        return self.grid_h * self.grid_w

    def tokens(self, chunk: int) -> int:
        return (self.first_chunk_frames if chunk == 0 else 1) * self.frame_tokens


def cache_bytes(cfg: Config) -> int:
    c = cfg.to_c()
    return int(load().ckv_cache_bytes(ctypes.byref(c)))


def _check(st: int, what: str):
    if st != CKV_OK:
        raise CkvError(st, what)


def _same_device(t, arena, name):
    """The kernels run on the arena's GPU: a tensor on another GPU is refused."""
    if t.device != arena.device:
        raise ValueError(f"{name} is on {t.device}, the arena on {arena.device}")


class Cache:
    """One same-step K/V cache (sinks + per-(layer, step) rings) over a torch
    arena on the current device.  `dry=True` makes a host-only cache that
    validates and advances the schedule without touching a device; tensor
    arguments may then be any non-null 16-byte aligned integers."""

    def __init__(self, cfg: Config, dry: bool = False, device=None):
        self.cfg = cfg
        self.dry = dry
        self._lib = load()
        self._c = cfg.to_c()
        h = ctypes.c_void_p()
        if dry:
            self.arena = None
            _check(self._lib.ckv_cache_create_dry(ctypes.byref(self._c), ctypes.byref(h)), "ckv_cache_create_dry")
        else:
            import torch
            nbytes = self._lib.ckv_cache_bytes(ctypes.byref(self._c))
            if nbytes == 0:
                raise CkvError(CKV_E_INVALID, "ckv_cache_bytes")
            self.arena = torch.empty(int(nbytes), dtype=torch.uint8, device=device or "cuda")
            _check(self._lib.ckv_cache_create(ctypes.byref(self._c), self.arena.data_ptr(), int(nbytes),
                                              ctypes.byref(h)), "ckv_cache_create")
        self._h = h

    # -- helpers ---------------------------------------------------------
    def _ptr(self, t, shape, name):
        if self.dry and isinstance(t, int):
            return t
        import torch
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous bf16 device tensor")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        _same_device(t, self.arena, name)
        return t.data_ptr()

    def _stream(self, stream):
        if self.dry:
            return None
        import torch
        s = stream if stream is not None else torch.cuda.current_stream()
        return s.cuda_stream

    def _shape(self, chunk):
        return (self.cfg.tokens(chunk), self.cfg.num_heads, self.cfg.head_dim)

    # -- ABI calls ---------------------------------------------------------
    def rope_append(self, layer, step, chunk, q, k, v, q_rot, stream=None):
        sh = self._shape(chunk)
        _check(self._lib.ckv_rope_append(self._h, layer, step, chunk, self._ptr(q, sh, "q"), self._ptr(k, sh, "k"),
                                         self._ptr(v, sh, "v"), self._ptr(q_rot, sh, "q_rot"),
                                         self._stream(stream)), "ckv_rope_append")

    def sink_build(self, layer, q, k, v, q_rot, stream=None):
        sh = self._shape(0)
        _check(self._lib.ckv_sink_build(self._h, layer, self._ptr(q, sh, "q"), self._ptr(k, sh, "k"),
                                        self._ptr(v, sh, "v"), self._ptr(q_rot, sh, "q_rot"),
                                        self._stream(stream)), "ckv_sink_build")

    def _gain(self, g, name):
        if self.dry and isinstance(g, int):
            return g
        import torch
        width = self.cfg.num_heads * self.cfg.head_dim
        if not isinstance(g, torch.Tensor) or g.dtype != torch.float32 or not g.is_cuda or not g.is_contiguous():
            raise TypeError(f"{name} must be a contiguous float32 device tensor")
        if g.numel() != width:
            raise ValueError(f"{name} has {g.numel()} values, expected {width}")
        _same_device(g, self.arena, name)
        return g.data_ptr()

    def norm_rope_append(self, layer, step, chunk, q, k, v, q_gain, k_gain, eps, q_rot, stream=None):
        sh = self._shape(chunk)
        _check(self._lib.ckv_norm_rope_append(self._h, layer, step, chunk, self._ptr(q, sh, "q"), self._ptr(k, sh, "k"),
                                              self._ptr(v, sh, "v"), self._gain(q_gain, "q_gain"),
                                              self._gain(k_gain, "k_gain"), float(eps),
                                              self._ptr(q_rot, sh, "q_rot"), self._stream(stream)),
               "ckv_norm_rope_append")

    def norm_sink_build(self, layer, q, k, v, q_gain, k_gain, eps, q_rot, stream=None):
        sh = self._shape(0)
        _check(self._lib.ckv_norm_sink_build(self._h, layer, self._ptr(q, sh, "q"), self._ptr(k, sh, "k"),
                                             self._ptr(v, sh, "v"), self._gain(q_gain, "q_gain"),
                                             self._gain(k_gain, "k_gain"), float(eps), self._ptr(q_rot, sh, "q_rot"),
                                             self._stream(stream)), "ckv_norm_sink_build")

    def chunk_attention(self, layer, step, chunk, q_rot, out, stream=None):
        sh = self._shape(chunk)
        _check(self._lib.ckv_chunk_attention(self._h, layer, step, chunk, self._ptr(q_rot, sh, "q_rot"),
                                             self._ptr(out, sh, "out"), self._stream(stream)),
               "ckv_chunk_attention")

    def chunk_attention_static(self, layer, step, chunk, q_rot, out, stream=None):
        """ckv_chunk_attention_static: the same call with the split partials in
        the library's own static device array (allocates nothing)."""
        sh = self._shape(chunk)
        _check(self._lib.ckv_chunk_attention_static(self._h, layer, step, chunk, self._ptr(q_rot, sh, "q_rot"),
                                                    self._ptr(out, sh, "out"), self._stream(stream)),
               "ckv_chunk_attention_static")

    def text_store(self, layer, k_text, v_text, stream=None):
        """Store the layer's context: k_text, v_text [n_text][H][d] bf16 device tensors."""
        n = int(k_text.shape[0])
        sh = (n, self.cfg.num_heads, self.cfg.head_dim)
        _check(self._lib.ckv_text_store(self._h, layer, self._ptr(k_text, sh, "k_text"), self._ptr(v_text, sh, "v_text"),
                                        n, self._stream(stream)), "ckv_text_store")

    def text_store_rows(self, layer, k_ptr, v_ptr, n_text, stream=None):
        """Raw-pointer form (dry caches and tests of the argument checks)."""
        _check(self._lib.ckv_text_store(self._h, layer, k_ptr, v_ptr, n_text, self._stream(stream)), "ckv_text_store")

    def cross_attention(self, layer, chunk, q, out, stream=None):
        sh = self._shape(chunk)
        _check(self._lib.ckv_cross_attention(self._h, layer, chunk, self._ptr(q, sh, "q"), self._ptr(out, sh, "out"),
                                             self._stream(stream)), "ckv_cross_attention")

    def window(self, layer, step, chunk):
        segs = (CkvSegment * 4)()
        n = ctypes.c_int32()
        _check(self._lib.ckv_window(self._h, layer, step, chunk, segs, 4, ctypes.byref(n)), "ckv_window")
        return [dict(kind=s.kind, first_slot=s.first_slot, chunk_first=s.chunk_first, n_chunks=s.n_chunks,
                     n_tokens=s.n_tokens) for s in segs[: n.value]]

    def ring_slot(self, chunk):
        out = ctypes.c_int32()
        _check(self._lib.ckv_ring_slot(self._h, chunk, ctypes.byref(out)), "ckv_ring_slot")
        return out.value

    def debug_copy_kv(self, layer, step, chunk, k_out, v_out, stream=None):
        sh = self._shape(chunk)
        _check(self._lib.ckv_debug_copy_kv(self._h, layer, step, chunk, self._ptr(k_out, sh, "k_out"),
                                           self._ptr(v_out, sh, "v_out"), self._stream(stream)),
               "ckv_debug_copy_kv")

    def attention_splits(self, n_queries, n_keys):
        return int(self._lib.ckv_attention_splits(self._h, n_queries, n_keys))

    def reset(self):
        _check(self._lib.ckv_cache_reset(self._h), "ckv_cache_reset")

    def close(self):
        if getattr(self, "_h", None) and self._h.value:
            self._lib.ckv_cache_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


@dataclass(frozen=True)
class ConvConfig:
    """One causal Conv3d layer (include/ckv_conv.h): grid, channels, kernel,
    largest chunk."""
    height: int
    width: int
    in_channels: int
    out_channels: int
    kt: int = 3
    kh: int = 3
    kw: int = 3
    max_frames: int = 1

    def to_c(self) -> CkvConvConfig:
        return CkvConvConfig(self.height, self.width, self.in_channels, self.out_channels, self.kt, self.kh, self.kw,
                             self.max_frames)

    @property
    def taps(self) -> int:
        return self.kt * self.kh * self.kw


def conv_bytes(cfg: ConvConfig) -> int:
    c = cfg.to_c()
    return int(load().ckv_conv_bytes(ctypes.byref(c)))


class CausalConv:
    """Streaming causal Conv3d state (packed weights, bias, 2-frame cache)
    over a torch arena.  `dry=True` makes a host-only state whose calls
    validate and advance the position without a device; pointers may then be
    any 16-byte aligned integers."""

    def __init__(self, cfg: ConvConfig, dry: bool = False, device=None):
        self.cfg = cfg
        self.dry = dry
        self._lib = load()
        self._c = cfg.to_c()
        h = ctypes.c_void_p()
        if dry:
            self.arena = None
            _check(self._lib.ckv_conv_create_dry(ctypes.byref(self._c), ctypes.byref(h)), "ckv_conv_create_dry")
        else:
            import torch
            nbytes = self._lib.ckv_conv_bytes(ctypes.byref(self._c))
            if nbytes == 0:
                raise CkvError(CKV_E_INVALID, "ckv_conv_bytes")
            self.arena = torch.empty(int(nbytes), dtype=torch.uint8, device=device or "cuda")
            _check(self._lib.ckv_conv_create(ctypes.byref(self._c), self.arena.data_ptr(), int(nbytes),
                                             ctypes.byref(h)), "ckv_conv_create")
        self._h = h

    def _ptr(self, t, shape, name, optional=False):
        if t is None and optional:
            return None
        if self.dry and isinstance(t, int):
            return t
        import torch
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous bf16 device tensor")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        _same_device(t, self.arena, name)
        return t.data_ptr()

    def _stream(self, stream):
        if self.dry:
            return None
        import torch
        s = stream if stream is not None else torch.cuda.current_stream()
        return s.cuda_stream

    def set_weights(self, weight, bias=None, stream=None):
        """weight [C_out][C_in][kt][kh][kw] bf16 (Conv3d's layout), bias [C_out] bf16 or None."""
        c = self.cfg
        wp = self._ptr(weight, (c.out_channels, c.in_channels, c.kt, c.kh, c.kw), "weight")
        bp = self._ptr(bias, (c.out_channels,), "bias", optional=True)
        _check(self._lib.ckv_conv_set_weights(self._h, wp, bp, self._stream(stream)), "ckv_conv_set_weights")

    def __call__(self, x, y, stream=None):
        """x [frames][H][W][C_in] -> y [frames][H][W][C_out] (bf16, channels last)."""
        c = self.cfg
        frames = int(x.shape[0])
        xp = self._ptr(x, (frames, c.height, c.width, c.in_channels), "x")
        yp = self._ptr(y, (frames, c.height, c.width, c.out_channels), "y")
        _check(self._lib.ckv_causal_conv(self._h, xp, frames, yp, self._stream(stream)), "ckv_causal_conv")

    def call_raw(self, x_ptr, frames, y_ptr, stream=None):
        """Raw-pointer form (dry states and tests of the argument checks)."""
        _check(self._lib.ckv_causal_conv(self._h, x_ptr, frames, y_ptr, self._stream(stream)), "ckv_causal_conv")

    def set_weights_raw(self, w_ptr, b_ptr=None, stream=None):
        _check(self._lib.ckv_conv_set_weights(self._h, w_ptr, b_ptr, self._stream(stream)), "ckv_conv_set_weights")

    @property
    def position(self) -> int:
        return int(self._lib.ckv_conv_position(self._h))

    def splits(self, frames: int) -> int:
        """Parts of each split unit of a call (1: none split)."""
        return self.plan(frames)[1]

    def plan(self, frames: int):
        """(units run whole, parts of every later unit) for a call of `frames`."""
        whole = ctypes.c_int32()
        parts = int(self._lib.ckv_conv_splits(self._h, int(frames), ctypes.byref(whole)))
        return whole.value, parts

    def reset(self):
        _check(self._lib.ckv_conv_reset(self._h), "ckv_conv_reset")

    def close(self):
        if getattr(self, "_h", None) and self._h.value:
            self._lib.ckv_conv_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
