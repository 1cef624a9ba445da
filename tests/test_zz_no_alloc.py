"""ckv_chunk_attention_static (the entry point for callers that cannot
allocate: its split partials live in the library's static device array)
against ckv_chunk_attention on the same cache state, through the C-ABI: two
calls in a row, the second with a smaller input.  Both run the same kernels
with the same split, so their outputs must agree bit for bit (beyond the
attention bar of max |diff| <= 2e-2, rel-L2 <= 5e-3 against each other).
Also the call captured into a HIP graph and replayed."""

import numpy as np
import pytest
import torch

import chunked_kv_attention_amd as C
from chunked_kv_attention_amd import inputs as I
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _fill(cfg, last_chunk, seed):
    """A cache with the sink and chunks 1..last_chunk at step 0; returns it
    with the last chunk's rotated queries."""
    cache = C.Cache(cfg)
    H, d = cfg.num_heads, cfg.head_dim
    q0, k0, v0 = (G.to_dev(b) for b in I.draw_qkv_bits(cfg.tokens(0), H, d, base_seed=seed, chunk=0, step_code=1))
    cache.sink_build(0, q0, k0, v0, torch.empty_like(q0))
    q_rot = None
    for c in range(1, last_chunk + 1):
        q, k, v = (G.to_dev(b) for b in I.draw_qkv_bits(cfg.tokens(c), H, d, base_seed=seed, chunk=c))
        q_rot = torch.empty_like(q)
        cache.rope_append(0, 0, c, q, k, v, q_rot)
    return cache, q_rot


def _compare(cfg, chunk, seed):
    G.require_gpu()
    cache, q_rot = _fill(cfg, chunk, seed)
    n_keys = cfg.tokens(0) + cfg.tokens(1) * (min(chunk - 1, cfg.window_chunks) + 1)
    splits = cache.attention_splits(cfg.tokens(chunk), n_keys)
    ref, got = torch.empty_like(q_rot), torch.full_like(q_rot, float("nan"))
    print(f"  static scratch: {cfg.num_heads} heads x {cfg.tokens(chunk)} x {n_keys}, {splits} splits", flush=True)
    cache.chunk_attention(0, 0, chunk, q_rot, ref)
    cache.chunk_attention_static(0, 0, chunk, q_rot, got)
    torch.cuda.synchronize()
    a, b = G.from_dev(got), G.from_dev(ref)
    G.assert_attn_close(a, b, "static scratch against the arena scratch")
    np.testing.assert_array_equal(G.bits_of(got), G.bits_of(ref))
    return splits


def test_static_scratch_matches_arena_scratch_two_calls():
    # first call: the 3-head share at 880 x 19,360 (many key splits)
    big = C.Config(1, 1, 3, 128, 22, 40, 3, 18, 29)
    assert _compare(big, 19, seed=31) > 1
    # second call, smaller: 128 queries x 2,304 keys at head_dim 64 (4 splits)
    small = C.Config(1, 1, 2, 64, 8, 16, 3, 14, 17)
    assert _compare(small, 15, seed=32) == 4


def test_static_entry_point_replays_under_graph_capture():
    """The callers the entry point is for capture it into a HIP graph: one
    call (3 heads x 880 x 19,360, 24 key splits and the merge) captured, then
    replayed three times with the program's own eager work and
    synchronisations between the replays; every replay must equal the eager
    call bit for bit."""
    G.require_gpu()
    cfg = C.Config(1, 1, 3, 128, 22, 40, 3, 18, 29)
    cache, q_rot = _fill(cfg, 19, seed=33)
    eager = torch.empty_like(q_rot)
    cache.chunk_attention_static(0, 0, 19, q_rot, eager)
    torch.cuda.synchronize()
    want = G.bits_of(eager)
    out = torch.full_like(q_rot, float("nan"))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cache.chunk_attention_static(0, 0, 19, q_rot, out)
    other = torch.empty_like(q_rot)
    for replay in range(3):
        out.fill_(float("nan"))
        cache.chunk_attention(0, 0, 19, q_rot, other)  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        print(f"  graph replay {replay}", flush=True)
        np.testing.assert_array_equal(G.bits_of(out), want)
    np.testing.assert_array_equal(G.bits_of(other), want)
