"""Plain CPU float64 oracle for the streaming causal 3D convolution of the
video VAE decoder.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this module; only
the tests, the package's smoke check and the benchmark's CPU-baseline leg may
call it.  It shares no code, tables or constants with the HIP path: it is the
plain definition of what that path computes, written out slowly in numpy
float64.

Source (web page; cited by title and section):
  [LG]  "Learning Video Generation from the Wan2.2 Source Code", Chapter 2,
        "Causal Convolution and Streaming Inference": a Conv3d whose time
        padding is moved entirely in front of the sequence (twice the
        per-side padding, none behind), spatial padding symmetric as usual;
        for streaming, the last CACHE_T = 2 input frames of each chunk are
        kept and put in front of the next chunk, and the front zero padding
        shrinks by the number of cached frames -- the same result as
        convolving the whole video at once.

Readings taken where the page is silent (each also listed in the design
notes of the repository):
  * The convolution is PyTorch's Conv3d (a cross-correlation, stride 1,
    dilation 1, no groups) with kernel (kt, kh, kw), kh and kw odd, spatial
    padding (kh-1)/2 and (kw-1)/2 on each side and time padding kt-1 in
    front; the layer shapes of the trained VAE are not on the page, so the
    channel counts, grid and kernel are inputs.
  * Activations are channels-last [T][H][W][C] here (the data is the same as
    the page's [C][T][H][W] tensor, transposed); weights keep Conv3d's layout
    [C_out][C_in][kt][kh][kw]; bias is per output channel.
  * When the front padding is smaller than the cache (kt - 1 < 2), the extra
    cached frames are dropped from the front (the page's padding accounting
    taken literally: a negative pad crops).
"""

from __future__ import annotations

import numpy as np

CACHE_T = 2  # frames kept between chunks ([LG] Ch.2, streaming paragraph)


def causal_conv3d(x: np.ndarray, weight: np.ndarray, bias=None) -> np.ndarray:
    """Whole-video causal convolution ([LG] Ch.2): zero-pad kt-1 frames in
    front of the time axis and (kh-1)/2, (kw-1)/2 on both sides of the
    spatial axes, then a valid cross-correlation.

    x: [T][H][W][C_in]; weight: [C_out][C_in][kt][kh][kw]; bias: [C_out] or
    None.  Returns [T][H][W][C_out] float64."""
    x = np.asarray(x, dtype=np.float64)
    weight = np.asarray(weight, dtype=np.float64)
    t_len, h, w, c_in = x.shape
    c_out, c_in_w, kt, kh, kw = weight.shape
    if c_in_w != c_in or kh % 2 == 0 or kw % 2 == 0:
        raise ValueError("shape mismatch or even spatial kernel")
    ph, pw = (kh - 1) // 2, (kw - 1) // 2
    padded = np.zeros((t_len + kt - 1, h + 2 * ph, w + 2 * pw, c_in))
    padded[kt - 1:, ph:ph + h, pw:pw + w, :] = x
    return _valid_conv(padded, weight, bias, t_len, h, w)


def _valid_conv(padded, weight, bias, t_len, h, w):
    """Valid cross-correlation of an already padded input: output frame t
    reads padded frames t .. t+kt-1 (one matmul over channels per tap)."""
    c_out, _, kt, kh, kw = weight.shape
    y = np.zeros((t_len, h, w, c_out))
    for a in range(kt):
        for b in range(kh):
            for c in range(kw):
                y += padded[a:a + t_len, b:b + h, c:c + w, :] @ weight[:, :, a, b, c].T
    if bias is not None:
        y += np.asarray(bias, dtype=np.float64)
    return y


class CausalConvStream:
    """Chunk-by-chunk causal convolution with a CACHE_T-frame cache ([LG]
    Ch.2, streaming paragraph): put the cached frames in front of the chunk,
    shrink the front zero padding by their number, convolve, then keep the
    last CACHE_T frames of (cache + chunk) for the next chunk."""

    def __init__(self, weight: np.ndarray, bias=None):
        self.weight = np.asarray(weight, dtype=np.float64)
        self.bias = None if bias is None else np.asarray(bias, dtype=np.float64)
        self.cache = None  # no history before the first chunk

    def reset(self):
        self.cache = None

    def __call__(self, x: np.ndarray) -> np.ndarray:
        x = np.asarray(x, dtype=np.float64)
        t_len, h, w, c_in = x.shape
        _, _, kt, kh, kw = self.weight.shape
        ph, pw = (kh - 1) // 2, (kw - 1) // 2
        front = kt - 1
        seq = x
        if self.cache is not None and front > 0:
            seq = np.concatenate([self.cache, x], axis=0)
            front -= self.cache.shape[0]
        if front < 0:
            seq = seq[-front:]  # more history cached than the kernel reaches
            front = 0
        padded = np.zeros((seq.shape[0] + front, h + 2 * ph, w + 2 * pw, c_in))
        padded[front:, ph:ph + h, pw:pw + w, :] = seq
        y = _valid_conv(padded, self.weight, self.bias, t_len, h, w)
        history = x if self.cache is None else np.concatenate([self.cache, x], axis=0)
        self.cache = history[-CACHE_T:].copy()
        return y


def conv_flops(frames: int, height: int, width: int, c_in: int, c_out: int, taps: int) -> int:
    """Multiply-adds x 2 of one call: every output value sums taps * C_in
    products."""
    return 2 * frames * height * width * c_out * c_in * taps
