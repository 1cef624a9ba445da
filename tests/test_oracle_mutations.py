"""Plant plausible mistakes in the oracle (on the CPU) and check that at least
one pin in test_oracle_pins.py catches each of them."""

import numpy as np
import pytest

import oracle.ckv_oracle as O
import tests.test_oracle_pins as P


def _fails(fn):
    try:
        fn()
    except (AssertionError, ValueError, IndexError):
        return True
    return False


def _rope_sin_sign_flipped(x, positions, theta):
    x = np.asarray(x, dtype=np.float64)
    ang = O.rope_angles(positions, x.shape[2], theta)
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    out = np.empty_like(x)
    out[:, :, 0::2] = x[:, :, 0::2] * c + x[:, :, 1::2] * s
    out[:, :, 1::2] = -x[:, :, 0::2] * s + x[:, :, 1::2] * c
    return out


def _rope_half_split(x, positions, theta):
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[2]
    ang = O.rope_angles(positions, d, theta)
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    re, im = x[:, :, : d // 2], x[:, :, d // 2:]
    return np.concatenate([re * c - im * s, re * s + im * c], axis=2)


def _bands_swapped(d):
    t, h, w = (d - 4 * (d // 6), 2 * (d // 6), 2 * (d // 6))
    return h, t, w


def _angles_band_order_hwt(positions, head_dim, theta):
    dt, dh, dw = O.rope_bands(head_dim)
    pos = np.asarray(positions, dtype=np.float64)
    parts = [np.outer(pos[:, 1], O.band_frequencies(dh, theta)),
             np.outer(pos[:, 2], O.band_frequencies(dw, theta)),
             np.outer(pos[:, 0], O.band_frequencies(dt, theta))]
    return np.concatenate(parts, axis=1)


def _attend_no_scale(q, k, v, scale):
    return _ORIG_ATTEND(q, k, v, 1.0)


def _attend_swapped_kv(q, k, v, scale):
    return _ORIG_ATTEND(q, v, k, scale)


def _attend_no_normalise(q, k, v, scale):
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    out = np.empty((q.shape[0], q.shape[1], v.shape[2]))
    for h in range(q.shape[1]):
        z = scale * q[:, h] @ k[:, h].T
        out[:, h] = np.exp(z - z.max(1, keepdims=True)) @ v[:, h]
    return out


def _window_includes_chunk0(chunk, window):
    return [] if chunk <= 0 else list(range(max(0, chunk - window), chunk))


def _window_off_by_one(chunk, window):
    return [] if chunk <= 0 else list(range(max(1, chunk - window + 1), chunk))


def _tokens_transposed(chunk, gh, gw, f0):
    base = 0 if chunk == 0 else f0 + chunk - 1
    nf = f0 if chunk == 0 else 1
    return np.asarray([(base + f, h, w) for f in range(nf) for w in range(gw) for h in range(gh)]).reshape(-1, 3)


def _flops_one_matmul(lq, lk, width):
    return 2 * lq * lk * width


def _round_truncate(x):
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.trunc(np.ldexp(m, 8)), e - 8)


def _round_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.sign(m) * np.floor(np.abs(np.ldexp(m, 8)) + 0.5), e - 8)


_ORIG_ATTEND = O.attend

def _norm_per_head(x, gain, eps):
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gain, dtype=np.float64).reshape(x.shape[1:])


def _norm_mean_abs(x, gain, eps):
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(x.shape[0], -1)
    return (flat / (np.mean(np.abs(flat), axis=1, keepdims=True) + eps) * np.asarray(gain).reshape(-1)).reshape(x.shape)


def _norm_no_gain(x, gain, eps):
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(x.shape[0], -1)
    return (flat / np.sqrt(np.mean(flat * flat, axis=1, keepdims=True) + eps)).reshape(x.shape)


def _norm_eps_outside_root(x, gain, eps):
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(x.shape[0], -1)
    return (flat / (np.sqrt(np.mean(flat * flat, axis=1, keepdims=True)) + eps) * np.asarray(gain).reshape(-1)).reshape(x.shape)


def _norm_sum_not_mean(x, gain, eps):
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(x.shape[0], -1)
    return (flat / np.sqrt(np.sum(flat * flat, axis=1, keepdims=True) + eps) * np.asarray(gain).reshape(-1)).reshape(x.shape)


def _cross_over_padding(q, k_text, v_text, n_text, scale):
    return O.attend(q, k_text, v_text, scale)


def _freqs_without_two(band_width, theta):
    j = np.arange(band_width // 2, dtype=np.float64)
    return np.power(float(theta), -j / float(band_width))


def _angles_head_dim_normalised(positions, head_dim, theta):
    dt, dh, dw = O.rope_bands(head_dim)
    pos = np.asarray(positions, dtype=np.float64)
    f = lambda n: np.power(float(theta), -2.0 * np.arange(n // 2) / float(head_dim))  # noqa: E731
    return np.concatenate([np.outer(pos[:, 0], f(dt)), np.outer(pos[:, 1], f(dh)), np.outer(pos[:, 2], f(dw))], axis=1)


def _first_step_reads_sink(self, layer, step, q, k, v, rows=None):
    qr, kr = self.rotate(0, q), self.rotate(0, k)
    ks, vs = kr, np.asarray(v, dtype=np.float64)
    if layer in self.sink:
        ks = np.concatenate([self.sink[layer][0], kr])
        vs = np.concatenate([self.sink[layer][1], vs])
    qr = qr if rows is None else qr[rows]
    return O.attend(qr, ks, vs, self.cfg.scale), (qr, kr)


def _first_step_records_sink(self, layer, step, q, k, v, rows=None):
    qr, kr = self.rotate(0, q), self.rotate(0, k)
    self.sink[layer] = (kr, np.asarray(v, dtype=np.float64))
    qr = qr if rows is None else qr[rows]
    return O.attend(qr, kr, v, self.cfg.scale), (qr, kr)


MUTATIONS = [
    ("rope3d", _rope_sin_sign_flipped, [P.test_rope_is_complex_multiplication]),
    ("rope3d", _rope_half_split, [P.test_rope_is_complex_multiplication]),
    ("rope_bands", _bands_swapped, [P.test_rope_band_widths_printed]),
    ("rope_angles", _angles_band_order_hwt, [lambda: P.test_rope_band_layout(128)]),
    ("attend", _attend_no_scale, [P.test_matches_torch_sdpa_float64, P.test_brute_force_loops_tiny]),
    ("attend", _attend_swapped_kv, [P.test_single_key_returns_its_value, P.test_matches_torch_sdpa_float64]),
    ("attend", _attend_no_normalise, [P.test_zero_query_returns_mean_value, P.test_brute_force_loops_tiny]),
    ("window_chunks", _window_includes_chunk0, [lambda: P.test_window_matches_fifo_simulation(18), P.test_window_golden]),
    ("window_chunks", _window_off_by_one, [lambda: P.test_window_matches_fifo_simulation(2), P.test_window_golden]),
    ("token_positions", _tokens_transposed, [P.test_token_positions_brute_force]),
    ("attention_flops", _flops_one_matmul, [P.test_flop_formula_worked_example]),
    ("round_to_bf16", _round_truncate, [P.test_round_to_bf16_ties_and_library]),
    ("round_to_bf16", _round_ties_away, [P.test_round_to_bf16_ties_and_library]),
    ("rms_norm", _norm_per_head, [P.test_qk_norm_worked_example, P.test_qk_norm_spans_all_heads]),
    ("rms_norm", _norm_mean_abs, [P.test_qk_norm_worked_example, P.test_qk_norm_matches_torch_rms_norm_float64]),
    ("rms_norm", _norm_no_gain, [P.test_qk_norm_worked_example, P.test_qk_norm_unit_rms_scale_invariance_and_gain]),
    ("rms_norm", _norm_eps_outside_root, [P.test_qk_norm_constant_vector_closed_form]),
    ("cross_attention", _cross_over_padding, [P.test_cross_attention_uses_only_the_real_context_length]),
    ("rms_norm", _norm_sum_not_mean, [P.test_qk_norm_worked_example, P.test_qk_norm_unit_rms_scale_invariance_and_gain]),
    ("band_frequencies", _freqs_without_two,
     [lambda: P.test_band_frequencies_are_textbook_rope_of_the_band_width(128, 1e4),
      lambda: P.test_each_band_is_1d_rope_when_other_coordinates_are_zero(128)]),
    ("rope_angles", _angles_head_dim_normalised,
     [lambda: P.test_each_band_is_1d_rope_when_other_coordinates_are_zero(128),
      lambda: P.test_each_band_is_1d_rope_when_other_coordinates_are_zero(64)]),
    ("OracleRollout.first_chunk_step", _first_step_reads_sink, [P.test_first_chunk_step_attends_to_its_own_chunk_only]),
    ("OracleRollout.first_chunk_step", _first_step_records_sink, [P.test_first_chunk_step_attends_to_its_own_chunk_only]),
]


@pytest.mark.parametrize("name,mutant,pins", MUTATIONS, ids=[f"{m[0]}-{m[1].__name__}" for m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, mutant, pins):
    # sanity: the pins pass on the real oracle
    for pin in pins:
        assert not _fails(pin)
    target = O
    *owners, attr = name.split(".")
    for owner in owners:  # a method of an oracle class, e.g. OracleRollout.first_chunk_step
        target = getattr(target, owner)
    monkeypatch.setattr(target, attr, mutant)
    caught = [_fails(pin) for pin in pins]
    assert all(caught), f"planted mistake in {name} ({mutant.__name__}) not caught by {caught}"
