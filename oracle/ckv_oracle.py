"""Plain CPU float64 oracle for same-step chunk attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this module; only
the tests, the package's smoke check and the benchmark's CPU-baseline leg may
call it.  It shares no code, tables or constants with the HIP path: it is the
plain definition of what that path computes, written out slowly and obviously
in numpy float64.

Sources (web pages; cited by title and section):
  [MC]  "PhysisServe -- Wan2.2 5B" model card: the "Inference profile" table
        and the paragraph after it (same-step KV, sink, schedule).
  [LG]  "Learning Video Generation from the Wan2.2 Source Code": Chapter 2
        (VAE strides, latent-shape formula, the 4n+1 rule, the 5B VAE),
        Chapter 3 ("Where Did the Prompt Go?": the text context), Chapter 4
        ("From Latent to Token", "3D RoPE: Letting Tokens Know Where They
        Are", the block forward pass), Chapter 8 ("What Does 75600^2
        Actually Mean?").
  [TI]  Wan2.2 docs index, "Wan2.2-TI2V-5B High-Compression Video Generation"
        (4x16x16 VAE, 4x32x32 with patchify) and "Run TI2V generation"
        (720P is 1280*704).

Readings taken where the pages are silent (each also listed in the design
notes of the repository):
  * RoPE base theta = 10000 (the pages name the frequency helper but do not
    print its body); each band's frequencies are normalised by the band's own
    width, w_j = theta^(-2j/D_band) -- textbook RoPE frequencies.  The base
    and the frequency formula are PARITY UNPINNED by the pages: no page prints
    a rotation angle.  Everything else in RoPE is pinned (band widths, band
    order, complex-multiplication convention, relative-position property).
  * Complex pairs are adjacent elements (x[2p], x[2p+1]) = (re, im).
  * Positions are absolute latent-frame indices: chunk 0 covers frames
    0..F0-1, chunk c >= 1 covers frame F0 + c - 1.
  * Tokens of a chunk are ordered frame-major, then patch row, then patch
    column.
  * Softmax scale 1/sqrt(head_dim); no mask inside the window.
  * The sink is stored once per layer and shared by every step.
  * Attention consumes the rotated q and k in bf16: the rotation itself is
    float64 ([LG] Ch.4 "3D RoPE" detail paragraph), but the backbone runs in
    bf16 ([LG] Ch.4, block forward pass) and its attention dependency takes
    half-precision inputs ([TI] install notes), so the rotated vectors are
    rounded to bf16 (nearest, ties to even) where they enter attention.
    Everything after that (scores, softmax, weighted sum) is float64.
    `OracleConfig.attention_inputs = "f64"` keeps them unrounded.
  * QK-Norm ([LG] Ch.4 "3D RoPE", detail paragraph: q and k are each passed
    through an RMSNorm after their linear layers): the norm runs over the
    whole projected vector of a token (all heads, H*d values -- the linear
    layer's output), y = x / sqrt(mean(x^2) + eps) * gain with one learned
    gain per channel; eps is an input (the pages print none; 1e-6 by
    default).  The norm's output is a bf16 activation of the bf16 backbone,
    so it is rounded to bf16 before the rotation.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# --------------------------------------------------------------------------
# Shapes and counts ([LG] Ch.2, Ch.4; [TI]; [MC] "Inference profile")
# --------------------------------------------------------------------------


def latent_frames(num_video_frames: int, temporal_stride: int = 4) -> int:
    """Latent frames of a video: (F - 1) // stride + 1 ([LG] Ch.2, "Where 4n+1
    Comes From": the first frame is encoded alone, then 4 frames per latent)."""
    if (num_video_frames - 1) % temporal_stride != 0:
        raise ValueError("frame count must be stride*n + 1")
    return (num_video_frames - 1) // temporal_stride + 1


def latent_shape(num_video_frames, height, width, vae_stride, z_dim):
    """(z, latent frames, H/sh, W/sw) ([LG] Ch.2, the target_shape formula)."""
    st, sh, sw = vae_stride
    return (z_dim, latent_frames(num_video_frames, st), height // sh, width // sw)


def tokens_per_frame(latent_h: int, latent_w: int, patch=(1, 2, 2)) -> int:
    """Patchify with kernel = stride = patch: one token per patch ([LG] Ch.4,
    "From Latent to Token")."""
    return (latent_h // patch[1]) * (latent_w // patch[2])


def chunk_frames(chunk: int, first_chunk_frames: int) -> int:
    """First chunk holds F0 latent frames, every later chunk one ([MC])."""
    return first_chunk_frames if chunk == 0 else 1


def chunk_first_frame(chunk: int, first_chunk_frames: int) -> int:
    """Absolute latent-frame index of a chunk's first frame (reading: absolute
    positions; chunk 0 starts at frame 0)."""
    return 0 if chunk == 0 else first_chunk_frames + chunk - 1


def chunk_tokens(chunk: int, grid_h: int, grid_w: int, first_chunk_frames: int) -> int:
    return chunk_frames(chunk, first_chunk_frames) * grid_h * grid_w


def token_positions(chunk: int, grid_h: int, grid_w: int, first_chunk_frames: int) -> np.ndarray:
    """(f, h, w) of every token of a chunk, in frame-major / row / column order.
    Returns int64 [n, 3]."""
    f0 = chunk_first_frame(chunk, first_chunk_frames)
    nf = chunk_frames(chunk, first_chunk_frames)
    out = []
    for f in range(nf):
        for h in range(grid_h):
            for w in range(grid_w):
                out.append((f0 + f, h, w))
    return np.asarray(out, dtype=np.int64).reshape(-1, 3)


def attention_flops(num_queries: int, num_keys: int, width: int) -> int:
    """2 matmuls x 2 FLOP per multiply-add: 4 * Lq * Lk * dim ([LG] Ch.8)."""
    return 4 * num_queries * num_keys * width


# --------------------------------------------------------------------------
# 3D RoPE ([LG] Ch.4, "3D RoPE")
# --------------------------------------------------------------------------


def rope_bands(head_dim: int):
    """Widths of the time, height and width bands of one head:
    d - 4*(d//6), 2*(d//6), 2*(d//6)  ([LG] Ch.4: 44/42/42 at d = 128)."""
    s = head_dim // 6
    return head_dim - 4 * s, 2 * s, 2 * s


def band_frequencies(band_width: int, theta: float) -> np.ndarray:
    """One rotation frequency per complex pair of a band:
    w_j = theta^(-2j / band_width), j = 0 .. band_width/2 - 1 (reading: the
    textbook RoPE frequencies, normalised by the band's own width)."""
    j = np.arange(band_width // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * j / float(band_width))


def rope_angles(positions: np.ndarray, head_dim: int, theta: float) -> np.ndarray:
    """Angle of every complex pair of every token, float64 [n, head_dim/2]:
    the time band takes f * w_t, then the height band h * w_h, then the width
    band w * w_w, concatenated in that order ([LG] Ch.4)."""
    dt, dh, dw = rope_bands(head_dim)
    pos = np.asarray(positions, dtype=np.float64)
    a_t = np.outer(pos[:, 0], band_frequencies(dt, theta))
    a_h = np.outer(pos[:, 1], band_frequencies(dh, theta))
    a_w = np.outer(pos[:, 2], band_frequencies(dw, theta))
    return np.concatenate([a_t, a_h, a_w], axis=1)


def rope3d(x: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """Rotate every head of every token by its 3D position, in float64.

    x is [n, heads, d]; each adjacent pair (x[2p], x[2p+1]) is read as the
    complex number x[2p] + i x[2p+1] and multiplied by e^{i angle_p}
    ([LG] Ch.4: applied to q and k by complex multiplication; the rotation is
    done in float64).  Returns float64 [n, heads, d]."""
    x = np.asarray(x, dtype=np.float64)
    n, _, d = x.shape
    ang = rope_angles(positions, d, theta)            # [n, d/2]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    re = x[:, :, 0::2]
    im = x[:, :, 1::2]
    out = np.empty_like(x)
    out[:, :, 0::2] = re * c - im * s
    out[:, :, 1::2] = re * s + im * c
    return out


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bf16 value (8 significant bits, ties to even) of float64 values,
    returned as float64.  Finite inputs in the normal bf16 range."""
    x = np.asarray(x, dtype=np.float64)
    mant, expo = np.frexp(x)                  # x = mant * 2^expo, 0.5 <= |mant| < 1
    return np.ldexp(np.rint(np.ldexp(mant, 8)), expo - 8)


# --------------------------------------------------------------------------
# Window membership ([MC] "Inference profile": up to W recent chunks plus the
# first-chunk sink without duplication; same-step reads)
# --------------------------------------------------------------------------


# --------------------------------------------------------------------------
# QK-Norm ([LG] Ch.4 "3D RoPE", detail paragraph)
# --------------------------------------------------------------------------


def rms_norm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm of every token's projected vector: x is [n, H, d] (or [n, H*d]);
    the mean of squares runs over all H*d values of a token, then each channel
    is scaled by its gain ([LG] Ch.4 "3D RoPE": q and k each go through an
    RMSNorm after their linear layers).  float64."""
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(x.shape[0], -1)
    g = np.asarray(gain, dtype=np.float64).reshape(-1)
    if g.shape[0] != flat.shape[1]:
        raise ValueError("one gain per channel of the projected vector")
    ms = np.mean(flat * flat, axis=1, keepdims=True)
    return (flat / np.sqrt(ms + eps) * g).reshape(x.shape)


def qk_norm_bf16(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """The norm's bf16 output (rounded once, nearest-even), as float64 values:
    what the rotation then reads."""
    return round_to_bf16(rms_norm(x, gain, eps))


def window_chunks(chunk: int, window: int) -> list:
    """Preceding chunks whose step-s K/V a chunk reads, oldest first.

    Chunk 0 reads none (it is generated before the rest).  A later chunk c
    reads the most recent `window` preceding chunks, never chunk 0's noisy
    entries (chunk 0 is present only as the clean sink): max(1, c-W) .. c-1."""
    if chunk <= 0:
        return []
    return list(range(max(1, chunk - window), chunk))


def window_key_count(chunk: int, window: int, grid_h: int, grid_w: int, first_chunk_frames: int) -> int:
    """Keys a chunk attends to: sink + window chunks + itself."""
    n1 = grid_h * grid_w
    if chunk == 0:
        return first_chunk_frames * n1
    return first_chunk_frames * n1 + len(window_chunks(chunk, window)) * n1 + n1


# --------------------------------------------------------------------------
# Softmax attention (the plain definition; [LG] Ch.8 names its two matmuls)
# --------------------------------------------------------------------------


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """o_i = sum_j softmax_j(scale * <q_i, k_j>) v_j, per head, float64.

    q [nq, H, d], k and v [nk, H, d] -> [nq, H, d].  Every query sees every
    key (no mask)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, nh, d = q.shape
    kh = np.ascontiguousarray(k.transpose(1, 0, 2))      # [H, nk, d]
    vh = np.ascontiguousarray(v.transpose(1, 0, 2))
    out = np.empty((nq, nh, v.shape[2]), dtype=np.float64)
    for h in range(nh):
        z = scale * (q[:, h, :] @ kh[h].T)               # [nq, nk]
        m = z.max(axis=1, keepdims=True)
        p = np.exp(z - m)
        p /= p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ vh[h]
    return out


def cross_attention(q: np.ndarray, k_text: np.ndarray, v_text: np.ndarray, n_text: int, scale: float) -> np.ndarray:
    """Cross-attention of video tokens to the text context ([LG] Ch.3 "Where
    Did the Prompt Go?": the prompt becomes up to 512 context vectors, trimmed
    to its real length, and every layer's cross-attention takes the video
    tokens as queries and the context as keys/values; Ch.4's block code passes
    the context lengths to it).  No position rotation, no mask beyond the
    real length: plain attention over the first n_text context rows.
    q [nq, H, d]; k_text, v_text [>= n_text, H, d]."""
    if not 1 <= n_text <= np.asarray(k_text).shape[0]:
        raise ValueError("n_text must be within the context")
    return attend(q, np.asarray(k_text)[:n_text], np.asarray(v_text)[:n_text], scale)


# --------------------------------------------------------------------------
# The rollout: who stores what, and what each call attends to
# ([MC] "Inference profile" and the paragraph after it)
# --------------------------------------------------------------------------


@dataclass
class OracleConfig:
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
    attention_inputs: str = "bf16"   # precision rotated q/k enter attention in

    @property
    def scale(self) -> float:
        return self.softmax_scale if self.softmax_scale > 0 else 1.0 / math.sqrt(self.head_dim)

    def tokens(self, chunk: int) -> int:
        return chunk_tokens(chunk, self.grid_h, self.grid_w, self.first_chunk_frames)

    def positions(self, chunk: int) -> np.ndarray:
        return token_positions(chunk, self.grid_h, self.grid_w, self.first_chunk_frames)


@dataclass
class OracleRollout:
    """Keeps every recorded K/V (no eviction: the window rule selects).

    noisy[(layer, step, chunk)] = (K_rot, V) recorded by chunk >= 1 at step;
    sink[layer] = (K_rot, V) of chunk 0's clean (sigma = 0) pass."""

    cfg: OracleConfig
    sink: dict = field(default_factory=dict)
    noisy: dict = field(default_factory=dict)

    def rotate(self, chunk: int, x) -> np.ndarray:
        """RoPE in float64, then the hand-off precision of attention's inputs."""
        r = rope3d(x, self.cfg.positions(chunk), self.cfg.rope_theta)
        return round_to_bf16(r) if self.cfg.attention_inputs == "bf16" else r

    def first_chunk_step(self, layer, step, q, k, v, rows=None):
        """Chunk 0, noisy step: self-attention within the chunk only."""
        qr, kr = self.rotate(0, q), self.rotate(0, k)
        qr = qr if rows is None else qr[rows]
        return attend(qr, kr, v, self.cfg.scale), (qr, kr)

    def sink_pass(self, layer, q, k, v, rows=None):
        """Chunk 0's extra clean pass: its rotated K and its V become the layer's
        sink; the pass itself attends within the chunk."""
        qr, kr = self.rotate(0, q), self.rotate(0, k)
        self.sink[layer] = (kr, np.asarray(v, dtype=np.float64))
        qr = qr if rows is None else qr[rows]
        return attend(qr, kr, v, self.cfg.scale), (qr, kr)

    def window_kv(self, layer, step, chunk, own_k, own_v):
        ks, vs = [self.sink[layer][0]], [self.sink[layer][1]]
        for j in window_chunks(chunk, self.cfg.window_chunks):
            kj, vj = self.noisy[(layer, step, j)]
            ks.append(kj)
            vs.append(vj)
        ks.append(own_k)
        vs.append(np.asarray(own_v, dtype=np.float64))
        return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)

    def chunk_step(self, layer, step, chunk, q, k, v, rows=None):
        """Chunk c >= 1 at step s: record (K_rot, V), then attend to
        [sink | same-step window | own]."""
        assert chunk >= 1
        qr, kr = self.rotate(chunk, q), self.rotate(chunk, k)
        self.noisy[(layer, step, chunk)] = (kr, np.asarray(v, dtype=np.float64))
        kw, vw = self.window_kv(layer, step, chunk, kr, v)
        qr = qr if rows is None else qr[rows]
        return attend(qr, kw, vw, self.cfg.scale), (qr, kr)
