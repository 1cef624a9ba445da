"""Cross-attention to the stored text context (through the C-ABI) against the
float64 oracle ("Learning Video Generation from the Wan2.2 Source Code",
Ch.3 "Where Did the Prompt Go?": video tokens attend to the context trimmed
to the prompt's real length).  Tolerance as for chunk attention: max |diff|
<= 2e-2 and relative L2 <= 5e-3 on the same bf16 inputs."""

import numpy as np
import pytest
import torch

import chunked_kv_attention_amd as C
import oracle.ckv_oracle as O
from chunked_kv_attention_amd import inputs as I
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

TINY = C.Config(num_layers=1, num_steps=2, num_heads=1, head_dim=64, grid_h=4, grid_w=4,
                first_chunk_frames=3, window_chunks=2, max_chunks=6)
PROFILE = C.Config(num_layers=2, num_steps=1, num_heads=24, head_dim=128, grid_h=22, grid_w=40,
                   first_chunk_frames=3, window_chunks=18, max_chunks=29)


def _bits(shape, seed):
    return I.f32_to_bf16_bits(np.random.default_rng(seed).standard_normal(shape).astype(np.float32))


def _case(cfg, cache, layer, chunk, n_text, seed, rows=None):
    H, d = cfg.num_heads, cfg.head_dim
    n = cfg.tokens(chunk)
    qb = _bits((n, H, d), seed)
    kb = _bits((n_text, H, d), seed + 1)
    vb = _bits((n_text, H, d), seed + 2)
    q, k, v = (G.to_dev(b) for b in (qb, kb, vb))
    out = torch.empty_like(q)
    print(f"  cross layer {layer} chunk {chunk} n_text {n_text}", flush=True)
    cache.text_store(layer, k, v)
    cache.cross_attention(layer, chunk, q, out)
    torch.cuda.synchronize()
    qf, kf, vf = (I.bf16_bits_to_f64(b) for b in (qb, kb, vb))
    if rows is not None:
        qf = qf[rows]
    ref = O.cross_attention(qf, kf, vf, n_text, 1.0 / np.sqrt(d))
    got = G.from_dev(out)
    if rows is not None:
        got = got[rows]
    return G.assert_attn_close(got, ref, f"cross chunk {chunk} n_text {n_text}")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    G.require_gpu()


@pytest.mark.parametrize("n_text", [1, 7, 64, 77, 300, 512])
def test_cross_attention_tiny(n_text):
    cache = C.Cache(TINY)
    for chunk in (0, 1):
        _case(TINY, cache, 0, chunk, n_text, seed=100 + n_text)


def test_cross_attention_profile_880_and_2640():
    cache = C.Cache(PROFILE)
    rows = G.sample_rows(880, 24, seed=3)
    mx, rl = _case(PROFILE, cache, 1, 5, 512, seed=7, rows=rows)
    print(f"  880 x 512: max abs {mx:.2e} rel L2 {rl:.2e}")
    _case(PROFILE, cache, 1, 6, 333, seed=8, rows=rows)                 # ragged context, key split tail
    _case(PROFILE, cache, 0, 0, 512, seed=9, rows=G.sample_rows(2640, 24, seed=4))


def test_context_is_per_layer_and_replaced():
    cache = C.Cache(PROFILE)
    rows = G.sample_rows(880, 16, seed=5)
    _case(PROFILE, cache, 0, 1, 512, seed=20, rows=rows)
    _case(PROFILE, cache, 1, 1, 96, seed=30, rows=rows)
    _case(PROFILE, cache, 0, 1, 40, seed=40, rows=rows)  # layer 0 replaced by a shorter context
