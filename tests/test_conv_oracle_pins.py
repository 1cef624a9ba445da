"""Pins of the causal-convolution oracle to facts outside itself: torch's
Conv3d in float64 on explicitly padded input, brute-force loops, closed
forms (identity and pure-shift kernels, border counts), causality, and the
page's statement that chunked streaming with a 2-frame cache equals the
whole-video convolution ("Learning Video Generation from the Wan2.2 Source
Code", Chapter 2, "Causal Convolution and Streaming Inference")."""

import numpy as np
import pytest
import torch

import oracle.causal_conv_oracle as CO

KERNELS = [(3, 3, 3), (2, 3, 3), (1, 3, 3), (3, 1, 1), (1, 1, 1), (3, 1, 3)]


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def _torch_causal(x, weight, bias):
    """The page's layer, literally: pad the time axis by kt-1 frames in front
    and none behind, the spatial axes symmetrically, then Conv3d with no
    padding; [C][T][H][W] layout."""
    kt, kh, kw = weight.shape[2:]
    xt = torch.from_numpy(np.ascontiguousarray(x.transpose(3, 0, 1, 2)))[None]
    xt = torch.nn.functional.pad(xt, ((kw - 1) // 2, (kw - 1) // 2, (kh - 1) // 2, (kh - 1) // 2, kt - 1, 0))
    y = torch.nn.functional.conv3d(xt, torch.from_numpy(weight), None if bias is None else torch.from_numpy(bias))
    return y[0].numpy().transpose(1, 2, 3, 0)


@pytest.mark.parametrize("kernel", KERNELS)
def test_whole_video_matches_torch_conv3d_float64(kernel):
    x = _rand(1, 5, 6, 7, 3)
    w = _rand(2, 4, 3, *kernel)
    b = _rand(3, 4)
    np.testing.assert_allclose(CO.causal_conv3d(x, w, b), _torch_causal(x, w, b), rtol=0, atol=1e-12)


def test_brute_force_loops_tiny():
    x = _rand(4, 3, 3, 4, 2)
    w = _rand(5, 2, 2, 3, 3, 3)
    b = _rand(6, 2)
    T, H, W, Ci = x.shape
    Co = w.shape[0]
    ref = np.zeros((T, H, W, Co))
    for t in range(T):
        for i in range(H):
            for j in range(W):
                for o in range(Co):
                    acc = b[o]
                    for a in range(3):
                        for p in range(3):
                            for q in range(3):
                                tt, ii, jj = t + a - 2, i + p - 1, j + q - 1
                                if tt < 0 or not 0 <= ii < H or not 0 <= jj < W:
                                    continue
                                for c in range(Ci):
                                    acc += w[o, c, a, p, q] * x[tt, ii, jj, c]
                    ref[t, i, j, o] = acc
    np.testing.assert_allclose(CO.causal_conv3d(x, w, b), ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("chunks", [[1, 1, 1, 1, 1, 1], [3, 1, 1, 1], [2, 2, 2], [1, 2, 3], [6]])
def test_streaming_equals_whole_video(kernel, chunks):
    """The page's claim: caching the last 2 input frames and putting them in
    front of the next chunk gives the whole-video result, for any chunking."""
    x = _rand(7, sum(chunks), 4, 5, 3)
    w = _rand(8, 2, 3, *kernel)
    b = _rand(9, 2)
    stream = CO.CausalConvStream(w, b)
    outs, t0 = [], 0
    for n in chunks:
        outs.append(stream(x[t0:t0 + n]))
        t0 += n
    np.testing.assert_allclose(np.concatenate(outs), CO.causal_conv3d(x, w, b), rtol=0, atol=1e-12)


def test_reset_starts_a_new_video():
    x = _rand(10, 4, 3, 3, 2)
    w = _rand(11, 2, 2, 3, 3, 3)
    stream = CO.CausalConvStream(w)
    stream(_rand(12, 3, 3, 3, 2))
    stream.reset()
    got = np.concatenate([stream(x[:1]), stream(x[1:])])
    np.testing.assert_allclose(got, CO.causal_conv3d(x, w), rtol=0, atol=1e-12)


def test_identity_kernel_returns_input():
    """A kernel that is the identity at its newest-frame centre tap and zero
    elsewhere copies the input."""
    x = _rand(13, 4, 3, 5, 3)
    w = np.zeros((3, 3, 3, 3, 3))
    w[:, :, 2, 1, 1] = np.eye(3)
    np.testing.assert_array_equal(CO.causal_conv3d(x, w), x)


def test_oldest_tap_is_a_two_frame_delay():
    """Only the oldest time tap: y[t] = x[t - 2], zero for the first 2 frames
    (all time padding is in front)."""
    x = _rand(14, 5, 3, 4, 2)
    w = np.zeros((2, 2, 3, 3, 3))
    w[:, :, 0, 1, 1] = np.eye(2)
    y = CO.causal_conv3d(x, w)
    np.testing.assert_array_equal(y[:2], 0.0)
    np.testing.assert_array_equal(y[2:], x[:3])


def test_border_counts_of_an_all_ones_kernel():
    """All-ones input and kernel: each output counts the taps that land inside
    the video -- 9 / 6 / 4 spatial taps (interior / edge / corner) times the
    min(t + 1, 3) frames the causal window has reached."""
    x = np.ones((4, 4, 5, 1))
    w = np.ones((1, 1, 3, 3, 3))
    y = CO.causal_conv3d(x, w)[..., 0]
    rows = np.array([2, 3, 3, 2])[:, None]
    cols = np.array([2, 3, 3, 3, 2])[None, :]
    for t in range(4):
        np.testing.assert_array_equal(y[t], min(t + 1, 3) * rows * cols)


def test_causality_future_frames_do_not_matter():
    x = _rand(15, 6, 3, 3, 2)
    w = _rand(16, 2, 2, 3, 3, 3)
    x2 = x.copy()
    x2[4:] = _rand(17, 2, 3, 3, 2)
    np.testing.assert_array_equal(CO.causal_conv3d(x, w)[:4], CO.causal_conv3d(x2, w)[:4])


def test_cache_keeps_the_last_two_input_frames():
    x = _rand(18, 5, 2, 2, 1)
    w = _rand(19, 1, 1, 3, 3, 3)
    s = CO.CausalConvStream(w)
    s(x[:1])
    np.testing.assert_array_equal(s.cache, x[:1])  # only one frame of history so far
    s(x[1:2])
    np.testing.assert_array_equal(s.cache, x[:2])
    s(x[2:5])
    np.testing.assert_array_equal(s.cache, x[3:5])
    assert CO.CACHE_T == 2


def test_flops_count_matches_the_multiply_adds():
    T, H, W, Ci, Co, taps = 2, 3, 4, 5, 6, 27
    macs = sum(1 for _t in range(T) for _i in range(H) for _j in range(W) for _o in range(Co)
               for _k in range(taps * Ci))
    assert CO.conv_flops(T, H, W, Ci, Co, taps) == 2 * macs
