"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module draws random numbers and rounds them to bf16; it holds none of the
attention arithmetic.  Every tensor is keyed by
(base_seed, prompt, layer, chunk, step_code, tensor_code), where step_code is
the denoising step index or `num_steps` for the first chunk's clean pass, and
tensor_code is 0 for q, 1 for k, 2 for v.

Values are float32 N(0, 1) from numpy's default generator, rounded to bf16 with
round-to-nearest-even, so both the HIP path and the float64 oracle consume the
exact same numbers.
"""

from __future__ import annotations

import numpy as np

TENSOR_CODES = {"q": 0, "k": 1, "v": 2}
CONV_TENSOR_CODES = {"x": 3, "weight": 4, "bias": 5}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bit patterns.
    Inputs here are finite."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    b32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b32.view(np.float32).astype(np.float64)


def normal_f32(shape, key) -> np.ndarray:
    rng = np.random.default_rng(np.random.SeedSequence([int(x) for x in key]))
    return rng.standard_normal(size=shape, dtype=np.float32)


def draw(shape, *, base_seed=0, prompt=0, layer=0, chunk=0, step_code=0, tensor="q") -> np.ndarray:
    """float32 N(0,1) tensor of the given shape for one (prompt, layer, chunk,
    step, tensor) key."""
    key = (base_seed, prompt, layer, chunk, step_code, TENSOR_CODES[tensor])
    return normal_f32(shape, key)


def draw_qkv_bits(n_tokens, num_heads, head_dim, **key):
    """q, k, v as bf16 bit patterns [n, H, d] (uint16)."""
    shape = (n_tokens, num_heads, head_dim)
    return tuple(f32_to_bf16_bits(draw(shape, tensor=t, **key)) for t in ("q", "k", "v"))


def peaky_key_rows(total_keys: int, fraction: float, seed_key) -> np.ndarray:
    """Indices of round(fraction * total_keys) window key rows, chosen by a
    seeded permutation; the workload scales those keys by 4 before rounding to
    get a peaky softmax."""
    count = int(round(fraction * total_keys))
    rng = np.random.default_rng(np.random.SeedSequence([int(x) for x in seed_key]))
    return np.sort(rng.permutation(total_keys)[:count])


def draw_conv_bits(shape, *, base_seed=0, layer=0, chunk=0, tensor="x", scale=1.0) -> np.ndarray:
    """bf16 bit patterns of a causal-convolution input: N(0,1) times `scale`
    (weights are drawn with scale 1/sqrt(fan-in) so outputs stay O(1)), keyed
    by (base_seed, layer, chunk, tensor) like the attention inputs."""
    key = (base_seed, 0, layer, chunk, 0, CONV_TENSOR_CODES[tensor])
    return f32_to_bf16_bits(normal_f32(shape, key) * np.float32(scale))
