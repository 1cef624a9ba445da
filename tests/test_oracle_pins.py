"""Pins of the float64 oracle to things other than itself.

Each test checks the oracle against a number the pages print (tests/golden/),
a closed form, an invariant of the mathematics, a brute-force computation on
tiny inputs, or an independent library routine.  test_oracle_mutations.py
plants plausible mistakes in the oracle and checks that these pins catch them.
"""

import collections
import os
import itertools
import math

import numpy as np
import pytest
import torch

import oracle.ckv_oracle as O
from tests.conftest import read_page_numbers, read_window_counts

RNG = np.random.default_rng(1234)


# ---------------------------------------------------------------- shapes --

def test_rope_band_widths_printed():
    pn = read_page_numbers()
    assert list(O.rope_bands(128)) == pn["rope_bands_d128"]
    assert sum(O.rope_bands(128)) == 128
    # head_dim 64 (tiny config): same rule, bands must still tile the head.
    assert sum(O.rope_bands(64)) == 64 and all(b % 2 == 0 for b in O.rope_bands(64))


def test_latent_shape_and_tokens_worked_example():
    pn = read_page_numbers()
    shape = O.latent_shape(81, 720, 1280, (4, 8, 8), 16)
    assert list(shape) == pn["latent_shape_81f_1280x720"]
    assert O.latent_frames(81) == pn["latent_frames_81"][0]
    per_frame = O.tokens_per_frame(shape[2], shape[3])
    assert per_frame == pn["tokens_per_frame_720p_a14b"][0]
    assert per_frame * shape[1] == pn["tokens_total_720p_a14b"][0]
    with pytest.raises(ValueError):
        O.latent_frames(80)


def test_5b_profile_token_counts_consistent():
    """1280x704 through the 5B VAE (4x16x16) and 2x2 patchify gives 22 x 40 =
    880 tokens per latent frame; 121 video frames are 31 latent frames = a
    3-frame first chunk plus 28 one-frame chunks = 29 chunks."""
    pn = read_page_numbers()
    w, h = (int(x) for x in pn["profile_width_height"])
    assert [w, h] == [int(x) for x in pn["ti2v_720p_width_height"]]
    st, sh, sw = (int(x) for x in pn["vae_stride_5b"])
    comp = [int(x) for x in pn["compression_with_patchify_5b"]]
    assert comp == [st, 2 * sh, 2 * sw]
    z = O.latent_shape(int(pn["video_frames_5b"][0]), h, w, (st, sh, sw), 48)
    assert O.tokens_per_frame(z[2], z[3]) == 880 == 22 * 40
    f0 = int(pn["profile_first_chunk_frames"][0])
    later = int(pn["profile_later_chunk_frames"][0])
    chunks = int(pn["profile_chunks"][0])
    assert z[1] == 31 == f0 + (chunks - 1) * later
    assert O.chunk_tokens(0, 22, 40, f0) == 2640
    assert O.chunk_tokens(5, 22, 40, f0) == 880


def test_flop_formula_worked_example():
    pn = read_page_numbers()
    flops = O.attention_flops(75600, 75600, 5120)
    assert float(f"{flops:.3g}") == pn["attention_flops_layer_a14b"][0]


def test_token_positions_brute_force():
    """Frame-major, then row, then column; absolute frame index."""
    gh, gw, f0 = 3, 5, 3
    for c in (0, 1, 4):
        pos = O.token_positions(c, gh, gw, f0)
        frames = range(0, f0) if c == 0 else [f0 + c - 1]
        expect = [(f, h, w) for f in frames for h in range(gh) for w in range(gw)]
        assert pos.tolist() == [list(t) for t in expect]


# ------------------------------------------------------------------ RoPE --

def _rand(*shape):
    return RNG.standard_normal(shape)


def test_rope_is_complex_multiplication():
    """Adjacent pairs are complex numbers multiplied by e^{i angle}."""
    x = _rand(7, 3, 128)
    pos = RNG.integers(0, 30, size=(7, 3))
    ang = O.rope_angles(pos, 128, 10000.0)
    z = x[:, :, 0::2] + 1j * x[:, :, 1::2]
    zr = z * np.exp(1j * ang)[:, None, :]
    got = O.rope3d(x, pos, 10000.0)
    np.testing.assert_allclose(got[:, :, 0::2], zr.real, atol=1e-13)
    np.testing.assert_allclose(got[:, :, 1::2], zr.imag, atol=1e-13)


@pytest.mark.parametrize("d", [64, 128])
def test_rope_band_layout(d):
    """A position on one axis rotates exactly that axis' band of dims:
    time first, then height, then width."""
    dt, dh, dw = O.rope_bands(d)
    x = _rand(1, 2, d)
    edges = {0: (0, dt), 1: (dt, dt + dh), 2: (dt + dh, d)}
    for axis in range(3):
        pos = np.zeros((1, 3), dtype=np.int64)
        pos[0, axis] = 5
        y = O.rope3d(x, pos, 10000.0)
        lo, hi = edges[axis]
        changed = np.abs(y - x).max(axis=(0, 1)) > 1e-12
        assert changed[lo:hi].all(), (axis, lo, hi)
        assert not changed[:lo].any() and not changed[hi:].any()


def _library_inv_freq(dim, theta):
    """Textbook RoPE frequencies from an independent library routine:
    transformers' default rotary parameters (RoFormer's 1 / base^(2j/dim),
    computed there in float32)."""
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaRotaryEmbedding

    cfg = LlamaConfig(hidden_size=dim, num_attention_heads=1, head_dim=dim,
                      rope_parameters={"rope_type": "default", "rope_theta": float(theta)})
    inv, _ = LlamaRotaryEmbedding.compute_default_rope_parameters(cfg)
    return inv.double().numpy()


def _roformer_freqs(dim, theta):
    """RoFormer's frequencies written out pair by pair: theta_j = base^(-2j/dim)."""
    return np.array([float(theta) ** (-2.0 * j / dim) for j in range(dim // 2)])


def _rope_1d(x, pos, freqs):
    """Textbook 1D rotary embedding over adjacent pairs (re, im): pair j of a
    token at position p is multiplied by exp(i p w_j).  x [n, H, D]."""
    z = x[..., 0::2] + 1j * x[..., 1::2]
    z = z * np.exp(1j * np.outer(pos, freqs))[:, None, :]
    out = np.empty_like(x)
    out[..., 0::2], out[..., 1::2] = z.real, z.imag
    return out


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("theta", [10000.0, 500.0])
def test_band_frequencies_are_textbook_rope_of_the_band_width(d, theta):
    """Each band's frequencies are the textbook RoPE frequencies of a head as
    wide as the band ("3D RoPE" section: the frequency helper is called once
    per band with the band's width): equal to a library routine's and to
    RoFormer's formula written out."""
    for width in O.rope_bands(d):
        got = O.band_frequencies(width, theta)
        np.testing.assert_allclose(got, _library_inv_freq(width, theta), rtol=1e-6)  # float32 there
        np.testing.assert_allclose(got, _roformer_freqs(width, theta), rtol=1e-14)
        assert got[0] == 1.0 and np.all(np.diff(got) < 0)


@pytest.mark.parametrize("d", [64, 128])
def test_each_band_is_1d_rope_when_other_coordinates_are_zero(d):
    """With two of (f, h, w) zero, 3D RoPE is textbook 1D RoPE of the third
    axis' band (frequencies from the library routine) and the identity on the
    other two bands."""
    dt, dh, dw = O.rope_bands(d)
    edges = [(0, dt), (dt, dt + dh), (dt + dh, d)]
    n = 9
    x = _rand(n, 2, d)
    for axis, (lo, hi) in enumerate(edges):
        pos = np.zeros((n, 3), dtype=np.int64)
        pos[:, axis] = np.arange(n) * 3 + 1          # up to 25, as far as the 5B grid reaches
        ref = x.copy()
        ref[:, :, lo:hi] = _rope_1d(x[:, :, lo:hi], pos[:, axis], _library_inv_freq(hi - lo, 1e4))
        # float32 library frequencies: angle error <= 25 * 2^-24 relative
        np.testing.assert_allclose(O.rope3d(x, pos, 1e4), ref, atol=2e-5)


def test_rope_identity_at_origin_and_norm():
    x = _rand(5, 2, 128)
    np.testing.assert_array_equal(O.rope3d(x, np.zeros((5, 3)), 10000.0), x)
    pos = RNG.integers(0, 1000, size=(5, 3))
    y = O.rope3d(x, pos, 10000.0)
    np.testing.assert_allclose(y[..., 0::2] ** 2 + y[..., 1::2] ** 2,
                               x[..., 0::2] ** 2 + x[..., 1::2] ** 2, rtol=1e-12)


def test_rope_relative_position_property():
    """<R_a q, R_b k> = <q, R_{b-a} k>: the score depends only on the
    coordinate difference ("3D RoPE" section)."""
    q, k = _rand(6, 1, 128), _rand(6, 1, 128)
    a = RNG.integers(0, 40, size=(6, 3))
    b = RNG.integers(0, 40, size=(6, 3))
    lhs = np.einsum("nhd,nhd->n", O.rope3d(q, a, 10000.0), O.rope3d(k, b, 10000.0))
    rhs = np.einsum("nhd,nhd->n", q, O.rope3d(k, b - a, 10000.0))
    np.testing.assert_allclose(lhs, rhs, rtol=1e-11, atol=1e-11)


def test_attention_shift_invariance_through_rope():
    """Shifting every token by the same (df, dh, dw) leaves attention unchanged."""
    q, k, v = _rand(5, 2, 64), _rand(9, 2, 64), _rand(9, 2, 64)
    pq = RNG.integers(0, 20, size=(5, 3))
    pk = RNG.integers(0, 20, size=(9, 3))
    shift = np.array([[7, -3, 11]])
    o1 = O.attend(O.rope3d(q, pq, 1e4), O.rope3d(k, pk, 1e4), v, 0.125)
    o2 = O.attend(O.rope3d(q, pq + shift, 1e4), O.rope3d(k, pk + shift, 1e4), v, 0.125)
    np.testing.assert_allclose(o1, o2, atol=1e-10)


# ----------------------------------------------------------------- window --

def _deque_windows(num_chunks, window):
    """Brute-force simulation: keep the last `window` noisy chunks in a FIFO;
    chunk 0 never enters it (it is only the sink); each chunk reads the FIFO
    before its own entry is appended."""
    hist = collections.deque(maxlen=window) if window > 0 else None
    out = {}
    for c in range(num_chunks):
        out[c] = list(hist) if (hist is not None and c >= 1) else []
        if c >= 1 and hist is not None:
            hist.append(c)
    return out


@pytest.mark.parametrize("window", [0, 1, 2, 5, 18, 40])
def test_window_matches_fifo_simulation(window):
    sim = _deque_windows(60, window)
    for c in range(60):
        assert O.window_chunks(c, window) == sim[c]
        assert 0 not in O.window_chunks(c, window)  # no duplication of chunk 0


def test_window_golden():
    windows, keys = read_window_counts()
    for (w, c), ids in windows.items():
        assert O.window_chunks(c, w) == ids, (w, c)
    for (gh, gw, f0, w, c), n in keys.items():
        assert O.window_key_count(c, w, gh, gw, f0) == n, (gh, gw, f0, w, c)


def test_window_no_eviction_when_window_covers_history():
    for c in range(1, 29):
        assert O.window_chunks(c, 28) == list(range(1, c))


# -------------------------------------------------------------- attention --

def test_single_key_returns_its_value():
    q, k, v = _rand(4, 3, 64), _rand(1, 3, 64), _rand(1, 3, 64)
    o = O.attend(q, k, v, 0.125)
    np.testing.assert_array_equal(o, np.broadcast_to(v, o.shape))


def test_zero_query_returns_mean_value():
    k, v = _rand(13, 2, 64), _rand(13, 2, 64)
    o = O.attend(np.zeros((3, 2, 64)), k, v, 0.125)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=0), o.shape), atol=1e-14)


def test_key_permutation_invariance():
    q, k, v = _rand(4, 2, 64), _rand(17, 2, 64), _rand(17, 2, 64)
    perm = RNG.permutation(17)
    np.testing.assert_allclose(O.attend(q, k, v, 0.2), O.attend(q, k[perm], v[perm], 0.2), atol=1e-13)


def test_segment_merge_equals_whole():
    """Softmax over a concatenation = log-sum-exp weighted merge of the
    per-segment softmaxes (what a split-key kernel relies on)."""
    q = _rand(3, 2, 32)
    segs = [(_rand(n, 2, 32), _rand(n, 2, 32)) for n in (5, 1, 9)]
    k = np.concatenate([s[0] for s in segs])
    v = np.concatenate([s[1] for s in segs])
    whole = O.attend(q, k, v, 0.3)
    num = 0
    den = 0
    for ks, vs in segs:
        z = 0.3 * np.einsum("qhd,khd->qhk", q, ks)
        lse = np.log(np.exp(z).sum(-1))                    # [q, h]
        num = num + np.exp(lse)[..., None] * O.attend(q, ks, vs, 0.3)
        den = den + np.exp(lse)[..., None]
    np.testing.assert_allclose(whole, num / den, atol=1e-13)


def test_brute_force_loops_tiny():
    nq, nk, nh, d = 3, 5, 2, 4
    q, k, v = _rand(nq, nh, d), _rand(nk, nh, d), _rand(nk, nh, d)
    scale = 0.7
    o = O.attend(q, k, v, scale)
    for i, h in itertools.product(range(nq), range(nh)):
        z = [scale * sum(q[i, h, t] * k[j, h, t] for t in range(d)) for j in range(nk)]
        e = [math.exp(x) for x in z]
        s = sum(e)
        for t in range(d):
            ref = sum(e[j] / s * v[j, h, t] for j in range(nk))
            assert abs(o[i, h, t] - ref) < 1e-12


def test_matches_torch_sdpa_float64():
    q, k, v = _rand(33, 4, 64), _rand(70, 4, 64), _rand(70, 4, 64)
    scale = 1.0 / 8.0
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2), torch.from_numpy(k).permute(1, 0, 2),
        torch.from_numpy(v).permute(1, 0, 2), scale=scale).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(O.attend(q, k, v, scale), ref, atol=1e-12)


# --------------------------------------------------------------- rollout --

def test_rollout_window_assembly_tiny():
    """Tiny rollout: the keys a chunk attends to are exactly sink, the window's
    same-step entries and its own, in that order; steps do not mix."""
    cfg = O.OracleConfig(1, 2, 1, 64, 4, 4, 3, 2, 6)
    ro = O.OracleRollout(cfg)
    mk = lambda n, tag: np.full((n, 1, 64), float(tag))  # noqa: E731
    ro.sink_pass(0, mk(48, 0), mk(48, 0), mk(48, -1))
    for c in range(1, 6):
        for s in range(2):
            tag = 10 * c + s
            ro.chunk_step(0, s, c, mk(16, tag), mk(16, tag), mk(16, tag))
            _, vw = ro.window_kv(0, s, c, mk(16, tag), mk(16, tag))
            ids = [-1] * 48 + [10 * j + s for j in O.window_chunks(c, 2) for _ in range(16)] + [tag] * 16
            assert vw[:, 0, 0].tolist() == [float(x) for x in ids]
            assert vw.shape[0] == O.window_key_count(c, 2, 4, 4, 3)


def test_first_chunk_step_attends_to_its_own_chunk_only():
    """Chunk 0's noisy steps come before every other chunk ("PhysisServe --
    Wan2.2 5B", paragraph after "Inference profile"), so they see only their
    own keys and record nothing.  Tagged values: a sink (V = -1) and a noisy
    entry (V = -2) already exist in the oracle; the step's own V is 3
    everywhere, so any other output means a foreign key was read.  With random
    V the step equals the plain softmax over its own rotated keys at frames
    0..F0-1, and a row subset equals those rows of the full result."""
    cfg = O.OracleConfig(1, 2, 2, 64, 2, 4, 3, 2, 5)
    ro = O.OracleRollout(cfg)
    n0 = cfg.tokens(0)
    ro.sink_pass(0, _rand(n0, 2, 64), _rand(n0, 2, 64), np.full((n0, 2, 64), -1.0))
    ro.chunk_step(0, 1, 1, _rand(8, 2, 64), _rand(8, 2, 64), np.full((8, 2, 64), -2.0))
    sink_k, sink_v = (a.copy() for a in ro.sink[0])
    noisy_keys = sorted(ro.noisy)
    q, k = _rand(n0, 2, 64), _rand(n0, 2, 64)
    o, _ = ro.first_chunk_step(0, 1, q, k, np.full((n0, 2, 64), 3.0))
    np.testing.assert_allclose(o, 3.0, rtol=1e-13)
    np.testing.assert_array_equal(ro.sink[0][0], sink_k)
    np.testing.assert_array_equal(ro.sink[0][1], sink_v)
    assert sorted(ro.noisy) == noisy_keys
    v = _rand(n0, 2, 64)
    o, (qr, kr) = ro.first_chunk_step(0, 0, q, k, v)
    pos = [(f, h, w) for f in range(3) for h in range(2) for w in range(4)]
    bf = O.round_to_bf16
    np.testing.assert_array_equal(kr, bf(O.rope3d(k, np.array(pos), 1e4)))
    z = (qr[:, 0] @ kr[:, 0].T) / 8.0
    p = np.exp(z - z.max(1, keepdims=True))
    np.testing.assert_allclose(o[:, 0], (p / p.sum(1, keepdims=True)) @ v[:, 0], atol=1e-13)
    rows = np.array([0, 5, n0 - 1])
    o_rows, _ = ro.first_chunk_step(0, 0, q, k, v, rows=rows)
    np.testing.assert_allclose(o_rows, o[rows], atol=1e-14)


def test_rollout_chunk_step_matches_direct_definition():
    cfg = O.OracleConfig(1, 1, 2, 64, 2, 4, 3, 2, 5)
    ro = O.OracleRollout(cfg)
    q0, k0, v0 = _rand(24, 2, 64), _rand(24, 2, 64), _rand(24, 2, 64)
    ro.sink_pass(0, q0, k0, v0)
    bf = O.round_to_bf16
    ks, vs = [bf(O.rope3d(k0, cfg.positions(0), 1e4))], [v0]
    for c in range(1, 5):
        q, k, v = _rand(8, 2, 64), _rand(8, 2, 64), _rand(8, 2, 64)
        o, _ = ro.chunk_step(0, 0, c, q, k, v)
        kr = bf(O.rope3d(k, cfg.positions(c), 1e4))
        win_k = [ks[0]] + [ks[j] for j in O.window_chunks(c, 2)] + [kr]
        win_v = [vs[0]] + [vs[j] for j in O.window_chunks(c, 2)] + [v]
        ref = O.attend(bf(O.rope3d(q, cfg.positions(c), 1e4)), np.concatenate(win_k), np.concatenate(win_v), 0.125)
        np.testing.assert_allclose(o, ref, atol=1e-13)
        ks.append(kr)
        vs.append(v)


# -------------------------------------------------------- bf16 hand-off --

def test_round_to_bf16_ties_and_library():
    """Ties go to the even significand; agrees with torch's float32 -> bfloat16
    conversion (round-to-nearest-even) on float32-representable values."""
    one = 1.0
    assert O.round_to_bf16(np.array([one + 2.0 ** -8]))[0] == 1.0                     # tie -> even
    assert O.round_to_bf16(np.array([one + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6      # tie -> even (up)
    assert O.round_to_bf16(np.array([one + 2.0 ** -8 + 2.0 ** -30]))[0] == 1.0 + 2.0 ** -7
    assert O.round_to_bf16(np.array([-(one + 2.0 ** -8)]))[0] == -1.0
    x = RNG.standard_normal(20000).astype(np.float32) * np.float32(37.0)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_to_bf16(x.astype(np.float64)), ref)


def test_rollout_rounds_rotated_qk_only():
    """The rollout hands bf16-rounded rotated q/k to attention; V untouched."""
    cfg = O.OracleConfig(1, 1, 2, 64, 2, 4, 3, 2, 5)
    ro = O.OracleRollout(cfg)
    q, k, v = _rand(24, 2, 64), _rand(24, 2, 64), _rand(24, 2, 64)
    _, (qr, kr) = ro.sink_pass(0, q, k, v)
    full = O.rope3d(k, cfg.positions(0), 1e4)
    np.testing.assert_array_equal(kr, O.round_to_bf16(full))
    np.testing.assert_array_equal(ro.sink[0][1], v)
    cfg64 = O.OracleConfig(1, 1, 2, 64, 2, 4, 3, 2, 5, attention_inputs="f64")
    _, (_, kr64) = O.OracleRollout(cfg64).sink_pass(0, q, k, v)
    np.testing.assert_array_equal(kr64, full)


# --------------------------------------------------------------------------
# QK-Norm ("Learning Video Generation from the Wan2.2 Source Code", Ch.4,
# "3D RoPE" detail paragraph): RMSNorm over each token's projected vector.
# --------------------------------------------------------------------------


def _read_qk_norm_golden():
    vals = {}
    with open(os.path.join(os.path.dirname(__file__), "golden", "qk_norm_worked.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split("=", 1)
                vals[k.strip()] = np.array([float(t) for t in v.split()])
    return vals


def test_qk_norm_worked_example():
    g = _read_qk_norm_golden()
    x = g["x"].reshape(1, 2, 2)
    np.testing.assert_allclose(O.rms_norm(x, np.ones(4), 0.0).reshape(-1), g["unit"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(O.rms_norm(x, g["gain"], 0.0).reshape(-1), g["scaled"], rtol=0, atol=1e-15)


def test_qk_norm_constant_vector_closed_form():
    # a constant vector c*1 normalises to sign(c) / sqrt(1 + eps / c^2)
    for c, eps in ((3.0, 0.0), (-0.5, 1e-6), (1e-3, 1e-6)):
        x = np.full((2, 3, 8), c)
        y = O.rms_norm(x, np.ones(24), eps)
        np.testing.assert_allclose(y, np.sign(c) / math.sqrt(1.0 + eps / (c * c)), rtol=1e-14)


def test_qk_norm_unit_rms_scale_invariance_and_gain():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((16, 24, 128))
    y = O.rms_norm(x, np.ones(24 * 128), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y.reshape(16, -1) ** 2, axis=1)), 1.0, rtol=1e-13)
    np.testing.assert_allclose(O.rms_norm(7.5 * x, np.ones(3072), 0.0), y, rtol=1e-13)
    gain = rng.standard_normal(3072)
    np.testing.assert_allclose(O.rms_norm(x, gain, 0.0), y * gain.reshape(24, 128), rtol=1e-13)


def test_qk_norm_spans_all_heads():
    # one head ten times larger: the norm couples the heads (per-head norms would not)
    x = np.ones((4, 3, 8))
    x[:, 0] *= 10.0
    y = O.rms_norm(x, np.ones(24), 0.0)
    # mean of squares (8 * 100 + 16) / 24 = 34: the small heads come out at 1/sqrt(34)
    np.testing.assert_allclose(y[:, 1:], 1.0 / math.sqrt(34.0), rtol=1e-14)
    np.testing.assert_allclose(y[:, 0], 10.0 / math.sqrt(34.0), rtol=1e-14)


def test_qk_norm_matches_torch_rms_norm_float64():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((5, 24, 128))
    gain = rng.uniform(0.5, 1.5, 3072)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x.reshape(5, -1)), (3072,), torch.from_numpy(gain), eps=1e-6)
    np.testing.assert_allclose(O.rms_norm(x, gain, 1e-6).reshape(5, -1), ref.numpy(), rtol=1e-13)


def test_qk_norm_bf16_output_is_rounded_norm():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((3, 2, 64))
    y = O.qk_norm_bf16(x, np.ones(128), 1e-6)
    t = torch.from_numpy(O.rms_norm(x, np.ones(128), 1e-6)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(y, t)


# --------------------------------------------------------------------------
# Cross-attention to the text context ("Learning Video Generation from the
# Wan2.2 Source Code", Ch.3 "Where Did the Prompt Go?")
# --------------------------------------------------------------------------


def test_cross_attention_uses_only_the_real_context_length():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((5, 2, 16))
    k = rng.standard_normal((12, 2, 16))
    v = rng.standard_normal((12, 2, 16))
    out = O.cross_attention(q, k, v, 7, 0.25)
    # rows past the real length (padding) change nothing
    k2, v2 = k.copy(), v.copy()
    k2[7:] = 100.0
    v2[7:] = -100.0
    np.testing.assert_array_equal(O.cross_attention(q, k2, v2, 7, 0.25), out)
    # brute force over the 7 real keys
    ref = np.empty_like(out)
    for i in range(5):
        for h in range(2):
            z = [0.25 * sum(q[i, h, e] * k[j, h, e] for e in range(16)) for j in range(7)]
            w = [math.exp(t - max(z)) for t in z]
            ref[i, h] = sum(w[j] * v[j, h] for j in range(7)) / sum(w)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)


def test_cross_attention_single_context_token():
    rng = np.random.default_rng(10)
    q = rng.standard_normal((3, 4, 8))
    k = rng.standard_normal((1, 4, 8))
    v = rng.standard_normal((1, 4, 8))
    np.testing.assert_allclose(O.cross_attention(q, k, v, 1, 0.5), np.broadcast_to(v, (3, 4, 8)), rtol=0, atol=1e-15)
