"""Parity of the HIP path (through the C-ABI) with the float64 oracle.

Tolerances: RoPE outputs within 1 bf16 ulp of the oracle's float64 result
rounded to bf16 (V bit-exact); attention outputs max |diff| <= 2e-2 and
relative L2 <= 5e-3 against the oracle on the same bf16 inputs.  Small shapes
are compared on every element; full-size shapes on sampled rows (all heads,
all head dims) that include the first and last rows and tile edges."""

import dataclasses

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
PROFILE1 = C.Config(num_layers=1, num_steps=4, num_heads=24, head_dim=128, grid_h=22, grid_w=40,
                    first_chunk_frames=3, window_chunks=18, max_chunks=29)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    G.require_gpu()
    print(f"\n[gpu] {torch.cuda.get_device_name(0)} lib={C.LIB_PATH}", flush=True)


# ------------------------------------------------------------ RoPE + append --

def _rope_errors(got_bits, x_bits, pos, theta):
    """Checks a bf16 RoPE result against the float64 rotation.  Bound: half a
    bf16 ulp of the exact value (the final rounding) plus 2^-21 (|x0| + |x1|),
    which covers the float32 evaluation (cos/sin rounded to float32, two
    products and a sum, each within 2^-24 relative).  Returns the fraction of
    elements that equal the oracle's rounded value exactly."""
    x = I.bf16_bits_to_f64(x_bits)
    ref = O.rope3d(x, pos, theta)
    got = I.bf16_bits_to_f64(got_bits)
    pair = np.repeat(np.abs(x[..., 0::2]) + np.abs(x[..., 1::2]), 2, axis=-1)
    ulp = np.ldexp(1.0, (np.frexp(np.maximum(np.abs(ref), 2.0 ** -120))[1] - 1) - 7)
    bound = 0.5 * ulp + 2.0 ** -21 * pair
    over = np.abs(got - ref) > bound
    assert not over.any(), (np.argwhere(over)[:5], got[over][:5], ref[over][:5])
    return float((got == O.round_to_bf16(ref)).mean())


def _rope_case(cfg: C.Config, chunks):
    cache = C.Cache(cfg)
    H, d = cfg.num_heads, cfg.head_dim
    for c in chunks:
        n = cfg.tokens(c)
        key = dict(base_seed=7, layer=0, chunk=c, step_code=0 if c else cfg.num_steps)
        qb, kb, vb = I.draw_qkv_bits(n, H, d, **key)
        q, k, v = (G.to_dev(b) for b in (qb, kb, vb))
        qr = torch.empty_like(q)
        if c == 0:
            cache.sink_build(0, q, k, v, qr)
        else:
            cache.rope_append(0, 0, c, q, k, v, qr)
        k_out, v_out = torch.empty_like(q), torch.empty_like(q)
        cache.debug_copy_kv(0, C.STEP_SINK if c == 0 else 0, c, k_out, v_out)
        torch.cuda.synchronize()
        pos = O.token_positions(c, cfg.grid_h, cfg.grid_w, cfg.first_chunk_frames)
        exact_q = _rope_errors(G.bits_of(qr), qb, pos, cfg.rope_theta)
        exact_k = _rope_errors(G.bits_of(k_out), kb, pos, cfg.rope_theta)
        assert exact_q > 0.98 and exact_k > 0.98, (c, exact_q, exact_k)
        np.testing.assert_array_equal(G.bits_of(v_out), vb)  # V is stored untouched


def test_rope_append_tiny():
    _rope_case(TINY, [0, 1, 2, 3])


# ------------------------------------------------ QK-Norm + RoPE + append --

def _gains(cfg, seed):
    """Seeded per-channel gains (float32), q and k."""
    rng = np.random.default_rng(seed)
    w = cfg.num_heads * cfg.head_dim
    return [rng.normal(1.0, 0.3, w).astype(np.float32) for _ in range(2)]


def _norm_rope_errors(got_bits, x_bits, gain, eps, pos, theta):
    """QK-Norm then RoPE against the oracle.  y = bf16(rms_norm(x)) is what the
    oracle rotates; the kernel forms y in float32 and may land one bf16 ulp
    away where the exact value sits within float32 error of a rounding
    boundary, so at most 0.1% of elements may exceed the RoPE bound of
    _rope_errors, and only by the rotation of such a 1-ulp change of the pair.
    Returns the fraction equal to the oracle's rounded value."""
    y = O.qk_norm_bf16(I.bf16_bits_to_f64(x_bits), gain, eps)
    ref = O.rope3d(y, pos, theta)
    got = I.bf16_bits_to_f64(got_bits)
    ulp = lambda a: np.ldexp(1.0, (np.frexp(np.maximum(np.abs(a), 2.0 ** -120))[1] - 1) - 7)  # noqa: E731
    pair = np.repeat(np.abs(y[..., 0::2]) + np.abs(y[..., 1::2]), 2, axis=-1)
    pair_ulp = np.repeat(ulp(y[..., 0::2]) + ulp(y[..., 1::2]), 2, axis=-1)
    tight = 0.5 * ulp(ref) + 2.0 ** -21 * pair
    err = np.abs(got - ref)
    assert (err > tight).mean() <= 1e-3, (err > tight).mean()
    loose = tight + pair_ulp
    over = err > loose
    assert not over.any(), (np.argwhere(over)[:5], got[over][:5], ref[over][:5])
    return float((got == O.round_to_bf16(ref)).mean())


def _norm_rope_case(cfg: C.Config, chunks, eps=1e-6):
    cache = C.Cache(cfg)
    H, d = cfg.num_heads, cfg.head_dim
    gq, gk = _gains(cfg, 11)
    gq_dev, gk_dev = (torch.from_numpy(g).cuda() for g in (gq, gk))
    for c in chunks:
        n = cfg.tokens(c)
        key = dict(base_seed=9, layer=0, chunk=c, step_code=0 if c else cfg.num_steps)
        qb, kb, vb = I.draw_qkv_bits(n, H, d, **key)
        q, k, v = (G.to_dev(b) for b in (qb, kb, vb))
        qr = torch.empty_like(q)
        if c == 0:
            cache.norm_sink_build(0, q, k, v, gq_dev, gk_dev, eps, qr)
        else:
            cache.norm_rope_append(0, 0, c, q, k, v, gq_dev, gk_dev, eps, qr)
        k_out, v_out = torch.empty_like(q), torch.empty_like(q)
        cache.debug_copy_kv(0, C.STEP_SINK if c == 0 else 0, c, k_out, v_out)
        torch.cuda.synchronize()
        pos = O.token_positions(c, cfg.grid_h, cfg.grid_w, cfg.first_chunk_frames)
        exact_q = _norm_rope_errors(G.bits_of(qr), qb, gq, eps, pos, cfg.rope_theta)
        exact_k = _norm_rope_errors(G.bits_of(k_out), kb, gk, eps, pos, cfg.rope_theta)
        assert exact_q > 0.98 and exact_k > 0.98, (c, exact_q, exact_k)
        np.testing.assert_array_equal(G.bits_of(v_out), vb)  # V is not normalised
        print(f"  norm+rope chunk {c}: {exact_q:.4f} / {exact_k:.4f} of q / k equal to the rounded oracle", flush=True)


def test_norm_rope_append_tiny():
    _norm_rope_case(TINY, [0, 1, 2, 3])


def test_norm_rope_append_profile_shape():
    # 24 heads x 128: the norm spans 3072 values per token
    _norm_rope_case(PROFILE1, [0, 1, 2], eps=1e-6)


def test_norm_tiny_rollout_every_chunk_and_step():
    """The tiny rollout with QK-Norm in front of every append and the sink:
    every output element of every call against the oracle."""
    gq, gk = _gains(TINY, 12)
    r = G.Rollout(TINY, qk_norm=(gq, gk, 1e-6))
    r.run_first_chunk()
    r.run_chunks(range(1, 6))
    print(f"tiny norm rollout worst: max abs {r.worst[0]:.3e} rel L2 {r.worst[1]:.3e}")


def test_rope_append_profile_shape():
    # full 22 x 40 grid, 24 heads: the sink (frames 0..2) and chunks 1, 2
    _rope_case(PROFILE1, [0, 1, 2])


def test_rope_append_every_frame():
    # every latent frame of a 29-chunk rollout (frames 0..30) on the full grid
    _rope_case(C.Config(1, 1, 2, 128, 22, 40, 3, 18, 29), range(0, 29))


def test_ring_slot_placement_and_eviction():
    """Append 1..8 with W = 2 (3 slots): every live chunk reads back its own
    K/V from its slot; evicted chunks are refused."""
    cfg = C.Config(1, 1, 2, 64, 2, 4, 3, 2, 9)
    cache = C.Cache(cfg)
    q0, k0, v0 = (G.to_dev(b) for b in I.draw_qkv_bits(24, 2, 64, base_seed=3, chunk=0, step_code=1))
    cache.sink_build(0, q0, k0, v0, torch.empty_like(q0))
    stored = {}
    for c in range(1, 9):
        qb, kb, vb = I.draw_qkv_bits(8, 2, 64, base_seed=3, chunk=c)
        q, k, v = (G.to_dev(b) for b in (qb, kb, vb))
        cache.rope_append(0, 0, c, q, k, v, torch.empty_like(q))
        stored[c] = vb
        for j in range(1, c + 1):
            ko, vo = torch.empty_like(q), torch.empty_like(q)
            if j >= c - 2:
                cache.debug_copy_kv(0, 0, j, ko, vo)
                torch.cuda.synchronize()
                np.testing.assert_array_equal(G.bits_of(vo), stored[j])
            else:
                with pytest.raises(C.CkvError):
                    cache.debug_copy_kv(0, 0, j, ko, vo)


# --------------------------------------------------------------- attention --

def test_tiny_rollout_every_chunk_and_step():
    """1 layer, 1 head, d 64, 4x4 grid, 6 chunks, W = 2, 2 steps: every
    output element of every call."""
    r = G.Rollout(TINY)
    r.run_first_chunk()
    r.run_chunks(range(1, 6))
    print(f"tiny rollout worst: max abs {r.worst[0]:.3e} rel L2 {r.worst[1]:.3e}")


def test_config_rope_base_and_softmax_scale():
    """A rollout with a non-default RoPE base (500) and an explicit softmax
    scale (0.2 instead of 1/sqrt(64)) through both config fields; every
    output element of every call against the oracle given the same values."""
    cfg = dataclasses.replace(TINY, rope_theta=500.0, softmax_scale=0.2)
    r = G.Rollout(cfg, base_seed=17)
    r.run_first_chunk()
    r.run_chunks(range(1, 6))
    print(f"theta 500, scale 0.2: max abs {r.worst[0]:.3e} rel L2 {r.worst[1]:.3e}")


def test_reset_then_second_rollout():
    """A cache reused after ckv_cache_reset: a second rollout with new inputs
    matches a fresh oracle in every output, so no sink or ring entry of the
    first rollout leaks into it."""
    r = G.Rollout(TINY, base_seed=21)
    r.run_first_chunk()
    r.run_chunks(range(1, 6))
    r.cache.reset()
    r.oracle = O.OracleRollout(r.ocfg)
    r.oracle64 = O.OracleRollout(dataclasses.replace(r.ocfg, attention_inputs="f64"))
    r.seed = 22
    r.run_first_chunk()
    r.run_chunks(range(1, 6))
    print(f"after reset: max abs {r.worst[0]:.3e} rel L2 {r.worst[1]:.3e}")


def test_window_membership_on_device():
    """K = 0 makes the softmax uniform, so the output is the mean of the
    window's V; with V = chunk id + 1 the output reveals exactly which chunks
    the kernel read."""
    cfg = C.Config(1, 2, 2, 64, 2, 4, 3, 3, 12)
    cache = C.Cache(cfg)
    n0, n1 = cfg.tokens(0), cfg.tokens(1)
    zeros = lambda n: torch.zeros((n, 2, 64), dtype=torch.bfloat16, device="cuda")  # noqa: E731
    cache.sink_build(0, zeros(n0), zeros(n0), torch.full((n0, 2, 64), 1.0, dtype=torch.bfloat16, device="cuda"),
                     zeros(n0))
    for c in range(1, 12):
        for s in range(2):
            val = float(c + 1 + 100 * s)
            q = zeros(n1)
            qr, out = torch.empty_like(q), torch.empty_like(q)
            cache.rope_append(0, s, c, q, zeros(n1), torch.full_like(q, val), qr)
            cache.chunk_attention(0, s, c, qr, out)
            win = O.window_chunks(c, 3)
            expect = (n0 * 1.0 + sum(n1 * (j + 1 + 100 * s) for j in win) + n1 * val) / (n0 + n1 * (len(win) + 1))
            got = G.from_dev(out)
            assert np.abs(got - expect).max() <= abs(expect) * 2 ** -7, (c, s, got.ravel()[:4], expect)


def test_bootstrap_first_chunk_profile():
    """2640 queries x 2640 keys, 24 x 128: the 4 noisy steps of chunk 0 and the
    clean sink pass; sampled rows."""
    cfg = PROFILE1
    r = G.Rollout(cfg, rows_per_call=48)
    r.run_first_chunk()
    print(f"bootstrap worst: max abs {r.worst[0]:.3e} rel L2 {r.worst[1]:.3e}")


def _peaky_window_up_to_chunk_19(r, seed):
    """Sink + chunks 1..18 recorded unchecked, then chunk 19 checked: its
    window is 2640 + 18 x 880 + 880 = 19,360 keys, and 1% of them (194 rows,
    a seeded permutation over the whole window) are scaled x4 before RoPE
    (peaky softmax)."""
    total = 2640 + 18 * 880 + 880
    peaky = I.peaky_key_rows(total, 0.01, (seed, 0, 0))
    assert len(peaky) == 194

    def rows_of(chunk):
        lo = 0 if chunk == 0 else 2640 + 880 * (chunk - 1)
        hi = lo + (2640 if chunk == 0 else 880)
        return peaky[(peaky >= lo) & (peaky < hi)] - lo
    r.step("sink", 0, 0, 0, scale_rows=rows_of(0), check=False)
    for c in range(1, 19):
        r.step("chunk", 0, 0, c, scale_rows=rows_of(c), check=False)
    return r.step("chunk", 0, 0, 19, scale_rows=rows_of(19))


def test_single_chunk_880x19360_peaky():
    """Chunk 19 at one step: sink 2640 + 18 x 880 window + 880 self = 19,360
    keys; 1% of the window's keys scaled x4 before RoPE (peaky softmax)."""
    cfg = C.Config(1, 1, 24, 128, 22, 40, 3, 18, 29)
    r = G.Rollout(cfg, base_seed=11, rows_per_call=64, f64_bar=False)
    mx, rl2 = _peaky_window_up_to_chunk_19(r, 11)
    splits = r.cache.attention_splits(880, 19360)
    print(f"880x19360 peaky: max abs {mx:.3e} rel L2 {rl2:.3e} (splits {splits}); against "
          f"unrounded float64 q/k: max abs {r.worst64[0]:.3e} rel L2 {r.worst64[1]:.3e} (the two oracles "
          f"differ by {r.worst_pair[0]:.3e} / {r.worst_pair[1]:.3e})")
    assert splits > 1  # the split-key path and its merge are exercised


def test_single_chunk_880x19360_head_dim_64():
    """The head_dim-64 kernel at the full window: 24 heads x 64, chunk 19
    against 2640 + 18 x 880 + 880 = 19,360 keys (N(0,1) keys), sampled rows
    over every query tile, both oracles at the bar."""
    cfg = C.Config(1, 1, 24, 64, 22, 40, 3, 18, 29)
    r = G.Rollout(cfg, base_seed=21, rows_per_call=64)
    r.step("sink", 0, 0, 0, check=False)
    for c in range(1, 19):
        r.step("chunk", 0, 0, c, check=False)
    mx, rl2 = r.step("chunk", 0, 0, 19)
    splits = r.cache.attention_splits(880, 19360)
    print(f"880x19360 d=64: max abs {mx:.3e} rel L2 {rl2:.3e} (splits {splits}); against unrounded float64 "
          f"q/k: max abs {r.worst64[0]:.3e} rel L2 {r.worst64[1]:.3e}")
    assert splits > 1


def test_many_key_splits_three_heads_880x19360():
    """One GPU's share of 24 heads sharded 8 ways ("Learning Video Generation
    from the Wan2.2 Source Code", Ch.8, Ulysses: split heads, not the
    sequence): 3 heads x 880 queries x 19,360 keys, which fills the chip only
    with many key splits (24: 21 query tiles x 24 = 504 workgroups).  Chunk
    19 (peaky) and chunk 20 (its ring window wraps into two runs), sampled
    rows."""
    cfg = C.Config(1, 1, 3, 128, 22, 40, 3, 18, 29)
    r = G.Rollout(cfg, base_seed=13, rows_per_call=128, f64_bar=False)
    splits = r.cache.attention_splits(880, 19360)
    assert splits > 4, splits
    mx, rl2 = _peaky_window_up_to_chunk_19(r, 13)
    mx20, rl20 = r.step("chunk", 0, 0, 20)
    print(f"3 heads x 880 x 19360, {splits} splits: chunk 19 max abs {mx:.3e} rel L2 {rl2:.3e}; chunk 20 max abs "
          f"{mx20:.3e} rel L2 {rl20:.3e}; unrounded float64 q/k worst {r.worst64[0]:.3e} / {r.worst64[1]:.3e} "
          f"(oracles differ by {r.worst_pair[0]:.3e} / {r.worst_pair[1]:.3e})")


def test_four_key_splits_every_element():
    """2 heads x 64, 8 x 16 grid, window 14: from chunk 15 on the window holds
    384 + 14 x 128 + 128 = 2,304 keys (36 tiles), run as 4 key splits; every
    output element of every call against the oracle."""
    cfg = C.Config(1, 1, 2, 64, 8, 16, 3, 14, 17)
    r = G.Rollout(cfg, base_seed=6)
    assert r.cache.attention_splits(128, 2304) == 4
    r.run_first_chunk()
    r.run_chunks(range(1, 17))
    print(f"4-split d=64: max abs {r.worst[0]:.3e} rel L2 {r.worst[1]:.3e}")


def test_two_to_fourteen_key_splits_every_element():
    """1 head x 64, 16 x 16 grid (256 queries: 2 query tiles), first chunk of
    3 frames, window 24: chunk c (1..25) sees 768 + 256 c keys, so the split
    count climbs from 2 to 14 one step every two chunks.  That runs all three
    merge variants (up to 4 splits, one lane per 8 dims; 5..8 splits, lane
    pairs; 9..14, groups of four lanes, some of whose lanes hold no split);
    every output element of every call against the oracle."""
    cfg = C.Config(1, 1, 1, 64, 16, 16, 3, 24, 26)
    r = G.Rollout(cfg, base_seed=14)
    splits = [r.cache.attention_splits(256, 768 + 256 * c) for c in range(1, 26)]
    print(f"splits per chunk: {splits}")
    assert set(range(5, 9)) <= set(splits), splits
    assert any(p > 8 and p % 4 for p in splits), splits
    r.run_first_chunk()
    r.run_chunks(range(1, 26))
    print(f"2..14 splits d=64: max abs {r.worst[0]:.3e} rel L2 {r.worst[1]:.3e}")


@pytest.mark.timeout(600)
def test_rollout_one_layer_profile():
    """29 chunks x 4 steps, 24 x 128, 880 tokens per chunk after the 2640-token
    first chunk; W = 18 so the window grows, then evicts.  Sampled rows."""
    r = G.Rollout(PROFILE1, base_seed=5, rows_per_call=12)
    r.run_first_chunk()
    r.run_chunks(range(1, 29), progress=True)
    print(f"1-layer rollout worst: max abs {r.worst[0]:.3e} rel L2 {r.worst[1]:.3e}; against unrounded "
          f"float64 q/k: max abs {r.worst64[0]:.3e} rel L2 {r.worst64[1]:.3e}")


# ------------------------------------------------------------- edge cases --

@pytest.mark.parametrize("window", [0, 1, 8])
def test_window_extremes(window):
    """W = 0 (sink + self), W = 1, and W >= chunks (nothing evicted)."""
    cfg = C.Config(1, 1, 2, 128, 2, 8, 2, window, 9)
    r = G.Rollout(cfg, base_seed=window)
    r.run_first_chunk()
    r.run_chunks(range(1, 9))


def test_ragged_query_and_key_tiles_two_layers():
    """24 tokens per frame (not a multiple of the 128-row query tile or the
    64-key tile), first chunk of 5 frames, 2 layers x 3 steps interleaved."""
    cfg = C.Config(2, 3, 3, 128, 3, 8, 5, 4, 10)
    r = G.Rollout(cfg, base_seed=9)
    r.run_first_chunk()
    r.run_chunks(range(1, 10))


def test_partial_last_tile_in_either_buffer():
    """Windows of 64 .. 208 keys in steps of 16 (4 x 4 grid, window 9, one
    split): whole tiles only (64, 128, 192 keys), one whole tile then a
    partial one (80 .. 112: the partial tile sits in the second LDS buffer),
    two whole tiles then a partial one (144 .. 176: first buffer) and three
    whole tiles then a partial one (208: the odd leftover whole tile, then
    the second buffer); every output element of every call."""
    cfg = C.Config(1, 1, 2, 64, 4, 4, 3, 9, 13)
    r = G.Rollout(cfg, base_seed=12)
    keys = [48 + 16 * min(c - 1, 9) + 16 for c in range(1, 13)]
    assert sorted(set(k % 64 for k in keys)) == [0, 16, 32, 48]
    assert {k // 64 for k in keys if k % 64} == {1, 2, 3}
    assert all(r.cache.attention_splits(16, k) == 1 for k in keys)
    r.run_first_chunk()
    r.run_chunks(range(1, 13))
    print(f"partial tiles: max abs {r.worst[0]:.3e} rel L2 {r.worst[1]:.3e}")


def test_split_keys_path_head_dim_64():
    """A shape where the key range is split (and merged) with head_dim 64:
    8 x 8 frames, window 14 chunks, so the later windows reach 1,152 keys (18
    tiles: two splits of >= 8 tiles)."""
    cfg = C.Config(1, 1, 2, 64, 8, 8, 3, 14, 17)
    r = G.Rollout(cfg, base_seed=4)
    assert r.cache.attention_splits(64, 192 + 14 * 64 + 64) > 1
    r.run_first_chunk()
    r.run_chunks(range(1, 17))


def test_two_prompts_two_streams():
    """Two caches (prompts) on two streams, interleaved; each matches its oracle."""
    cfg = C.Config(1, 2, 2, 128, 2, 8, 3, 2, 6)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    a = G.Rollout(cfg, prompt=0, stream=s1)
    b = G.Rollout(cfg, prompt=1, stream=s2)
    for r in (a, b):
        r.run_first_chunk()
    for c in range(1, 6):
        a.run_chunks([c])
        b.run_chunks([c])


def test_errors_do_not_launch():
    cache = C.Cache(TINY)
    x = torch.zeros((TINY.tokens(1), 1, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(C.CkvError) as e:
        cache.rope_append(0, 0, 1, x, x, x, torch.empty_like(x))
    assert e.value.status == C.CKV_E_STATE
    with pytest.raises(ValueError):
        cache.chunk_attention(0, 0, 0, x, x)  # wrong shape for chunk 0


def test_repeated_calls_are_bit_identical():
    """The same call on the same cache gives the same bits every time (the
    kernels have no order-dependent reductions): chunk 19 of the profile at
    head_dim 128 (3 key splits + merge) and the 2640-token sink pass (one
    split), four calls each."""
    cfg = C.Config(1, 1, 24, 128, 22, 40, 3, 18, 29)
    cache = C.Cache(cfg)
    H, d = cfg.num_heads, cfg.head_dim
    qs = {}
    for c in range(0, 20):
        q, k, v = (G.to_dev(b) for b in I.draw_qkv_bits(cfg.tokens(c), H, d, base_seed=41, chunk=c,
                                                          step_code=1 if c == 0 else 0))
        qs[c] = torch.empty_like(q)
        if c == 0:
            cache.sink_build(0, q, k, v, qs[c])
        else:
            cache.rope_append(0, 0, c, q, k, v, qs[c])
    for step, chunk in ((0, 19), (C.STEP_SINK, 0)):
        outs = []
        for _ in range(4):
            o = torch.empty_like(qs[chunk])
            cache.chunk_attention(0, step, chunk, qs[chunk], o)
            torch.cuda.synchronize()
            outs.append(G.bits_of(o))
        for other in outs[1:]:
            np.testing.assert_array_equal(other, outs[0])
