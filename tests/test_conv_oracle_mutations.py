"""Plant plausible mistakes in the causal-convolution oracle (on the CPU) and
check that at least one pin in test_conv_oracle_pins.py catches each."""

import numpy as np
import pytest

import oracle.causal_conv_oracle as CO
import tests.test_conv_oracle_pins as P

_ORIG_VALID = CO._valid_conv
_ORIG_CALL = CO.CausalConvStream.__call__


def _fails(fn, *args):
    try:
        fn(*args)
    except (AssertionError, ValueError, IndexError):
        return True
    return False


def _symmetric_time_padding(x, weight, bias=None):
    """Ordinary (non-causal) Conv3d: time padded on both sides."""
    x = np.asarray(x, dtype=np.float64)
    t_len, h, w, c_in = x.shape
    _, _, kt, kh, kw = weight.shape
    ph, pw, pt = (kh - 1) // 2, (kw - 1) // 2, (kt - 1) // 2
    padded = np.zeros((t_len + kt - 1, h + 2 * ph, w + 2 * pw, c_in))
    padded[pt:pt + t_len, ph:ph + h, pw:pw + w, :] = x
    return _ORIG_VALID(padded, np.asarray(weight, dtype=np.float64), bias, t_len, h, w)


def _flipped_kernel(padded, weight, bias, t_len, h, w):
    """True convolution (kernel reversed) instead of Conv3d's correlation."""
    return _ORIG_VALID(padded, weight[:, :, ::-1, ::-1, ::-1], bias, t_len, h, w)


def _no_bias(padded, weight, bias, t_len, h, w):
    return _ORIG_VALID(padded, weight, None, t_len, h, w)


def _transposed_weight(padded, weight, bias, t_len, h, w):
    """Spatial taps read (kw, kh) instead of (kh, kw)."""
    return _ORIG_VALID(padded, weight.transpose(0, 1, 2, 4, 3), bias, t_len, h, w)


def _cache_from_this_chunk_only(self, x):
    """Keeps the last 2 frames of the chunk alone (drops the older cached frame
    when a chunk has a single frame)."""
    y = _ORIG_CALL(self, x)
    self.cache = np.asarray(x, dtype=np.float64)[-CO.CACHE_T:].copy()
    return y


def _padding_not_reduced(self, x):
    """Puts the cache in front but still pads kt-1 zero frames."""
    x = np.asarray(x, dtype=np.float64)
    t_len, h, w, c_in = x.shape
    _, _, kt, kh, kw = self.weight.shape
    ph, pw = (kh - 1) // 2, (kw - 1) // 2
    seq = x if self.cache is None else np.concatenate([self.cache, x], axis=0)
    padded = np.zeros((seq.shape[0] + kt - 1, h + 2 * ph, w + 2 * pw, c_in))
    padded[kt - 1:, ph:ph + h, pw:pw + w, :] = seq
    y = _ORIG_VALID(padded, self.weight, self.bias, t_len, h, w)
    self.cache = seq[-CO.CACHE_T:].copy()
    return y


MUTATIONS = {
    "non-causal symmetric time padding": [("causal_conv3d", _symmetric_time_padding)],
    "flipped kernel (convolution)": [("_valid_conv", _flipped_kernel)],
    "bias dropped": [("_valid_conv", _no_bias)],
    "kh and kw swapped": [("_valid_conv", _transposed_weight)],
    "one cached frame": [("CACHE_T", 1)],
    "cache from the current chunk only": [("CausalConvStream.__call__", _cache_from_this_chunk_only)],
    "front padding not reduced by the cache": [("CausalConvStream.__call__", _padding_not_reduced)],
}

PINS = [
    (P.test_whole_video_matches_torch_conv3d_float64, [(3, 3, 3)]),
    (P.test_whole_video_matches_torch_conv3d_float64, [(3, 1, 3)]),
    (P.test_brute_force_loops_tiny, []),
    (P.test_streaming_equals_whole_video, [(3, 3, 3), [1, 1, 1, 1, 1, 1]]),
    (P.test_streaming_equals_whole_video, [(3, 3, 3), [3, 1, 1, 1]]),
    (P.test_oldest_tap_is_a_two_frame_delay, []),
    (P.test_cache_keeps_the_last_two_input_frames, []),
    (P.test_causality_future_frames_do_not_matter, []),
]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(monkeypatch, name):
    for target, value in MUTATIONS[name]:
        if target == "CausalConvStream.__call__":
            monkeypatch.setattr(CO.CausalConvStream, "__call__", value)
        else:
            monkeypatch.setattr(CO, target, value)
    caught = [pin.__name__ for pin, args in PINS if _fails(pin, *args)]
    assert caught, f"no pin catches: {name}"


def test_unmutated_oracle_passes_every_pin():
    for pin, args in PINS:
        pin(*args)
