"""GPU parity of the streaming causal 3D convolution (include/ckv_conv.h)
against the float64 oracle ("Learning Video Generation from the Wan2.2
Source Code", Chapter 2, "Causal Convolution and Streaming Inference").

Both sides take the same bf16 inputs; the oracle convolves the whole video at
once (float64), the library streams it chunk by chunk through its 2-frame
cache (float32 accumulation, one bf16 rounding).  Bar: max |diff| <= 2e-2 and
relative L2 <= 5e-3, as for attention; weights are drawn N(0,1)/sqrt(fan-in)
so outputs are O(1)."""

import numpy as np
import pytest
import torch

import chunked_kv_attention_amd as C
import oracle.causal_conv_oracle as CO
from chunked_kv_attention_amd import inputs as I
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _layer(cfg: C.ConvConfig, seed: int, bias=True):
    fan_in = cfg.in_channels * cfg.taps
    wb = I.draw_conv_bits((cfg.out_channels, cfg.in_channels, cfg.kt, cfg.kh, cfg.kw), base_seed=seed,
                          tensor="weight", scale=1.0 / np.sqrt(fan_in))
    bb = I.draw_conv_bits((cfg.out_channels,), base_seed=seed, tensor="bias", scale=0.1) if bias else None
    return wb, bb


def _video(cfg: C.ConvConfig, frames: int, seed: int):
    return I.draw_conv_bits((frames, cfg.height, cfg.width, cfg.in_channels), base_seed=seed, tensor="x")


def _stream(cfg, state, xb, chunks):
    """Feed the video through the library chunk by chunk; bf16 output bits."""
    outs, t0 = [], 0
    for n in chunks:
        x = G.to_dev(xb[t0:t0 + n])
        y = torch.empty((n, cfg.height, cfg.width, cfg.out_channels), dtype=torch.bfloat16, device="cuda")
        state(x, y)
        outs.append(y)
        t0 += n
    torch.cuda.synchronize()
    return np.concatenate([G.from_dev(y) for y in outs])


def _check(got, ref, what, absum=None):
    """The stated bar, plus, given absum = the convolution of |x| with |W|
    (the sum of the absolute products behind each output): every output
    within half a bf16 ulp of the exact value plus 2^-16 * absum (float32
    accumulation error, far below what any indexing mistake would cause),
    and >= 98% equal to the oracle's correctly rounded value."""
    mx, rel = G.attn_errors(got, ref)
    assert mx <= G.MAX_ABS and rel <= G.REL_L2, f"{what}: max {mx:.3e} rel {rel:.3e}"
    if absum is not None:
        half_ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(ref), 2.0 ** -126))[1] - 9)
        bound = half_ulp + 2.0 ** -16 * absum
        over = np.abs(got - ref) > bound
        assert not over.any(), f"{what}: {int(over.sum())} outputs beyond the rounding bound"
        exact = (G.f64_to_bf16_bits(got) == G.f64_to_bf16_bits(ref)).mean()
        assert exact >= 0.98, f"{what}: only {exact:.4f} equal to the rounded oracle"
    return mx, rel


def _case(cfg, chunks, seed=1, bias=True, splits=None, hybrid=False):
    """Stream the video in `chunks`; `splits` (if given) is the parts of the
    split units every call must take; `hybrid` asks that some units run whole
    and the rest split."""
    G.require_gpu()
    print(f"[conv] {cfg} chunks={chunks} seed={seed} bias={bias}", flush=True)
    wb, bb = _layer(cfg, seed, bias)
    xb = _video(cfg, sum(chunks), seed)
    state = C.CausalConv(cfg)
    if splits is not None:
        assert all(state.splits(n) == splits for n in chunks)
    state.set_weights(G.to_dev(wb), None if bb is None else G.to_dev(bb))
    got = _stream(cfg, state, xb, chunks)
    if hybrid:  # the device's CU count is known after the first call
        units = -(-chunks[-1] * cfg.height * cfg.width // 128) * (cfg.out_channels // 128)
        whole, parts = state.plan(chunks[-1])
        assert 0 < whole < units and parts == cfg.kt, (whole, parts, units)
    x, w = I.bf16_bits_to_f64(xb), I.bf16_bits_to_f64(wb)
    ref = CO.causal_conv3d(x, w, None if bb is None else I.bf16_bits_to_f64(bb))
    absum = CO.causal_conv3d(np.abs(x), np.abs(w)) + (0.0 if bb is None else np.abs(I.bf16_bits_to_f64(bb)))
    assert state.position == sum(chunks)
    return _check(got, ref, f"{cfg} {chunks}", absum)


@pytest.mark.parametrize("chunks", [[1, 1, 1, 1], [1, 2, 1, 3], [4], [2, 2]])
def test_tiny_ragged_grid_every_chunking(chunks):
    """5 x 7 frames (35 pixels: tiles span rows and frames, ragged tail);
    small calls take the 3-way split of the reduction."""
    cfg = C.ConvConfig(height=5, width=7, in_channels=64, out_channels=128, max_frames=4)
    _case(cfg, chunks, splits=3)


def test_one_pass_path_with_three_time_taps():
    """A grid large enough that calls take one pass over all 27 taps (no
    split): 160 x 280 frames, 64 -> 128 channels, two one-frame chunks."""
    cfg = C.ConvConfig(height=160, width=280, in_channels=64, out_channels=128, max_frames=1)
    _case(cfg, [1, 1], seed=12, splits=1)


@pytest.mark.parametrize("kernel", [(2, 3, 3), (1, 3, 3), (3, 1, 1), (1, 1, 1), (3, 1, 3), (3, 3, 1)])
def test_kernel_shapes(kernel):
    kt, kh, kw = kernel
    cfg = C.ConvConfig(height=6, width=9, in_channels=64, out_channels=128, kt=kt, kh=kh, kw=kw, max_frames=3)
    _case(cfg, [1, 3, 1, 2], seed=2)


def test_last_round_split_path():
    """A call with more units than one round of workgroup slots: the first
    full round runs whole, the units of the partly filled last round run as 3
    parts (240 x 320 frames: 600 units on 256 CUs -> 512 whole + 88 x 3)."""
    cfg = C.ConvConfig(height=240, width=320, in_channels=64, out_channels=128, max_frames=1)
    _case(cfg, [1, 1], seed=13, hybrid=True)


def test_several_channel_tiles_and_blocks_no_bias():
    cfg = C.ConvConfig(height=8, width=12, in_channels=192, out_channels=256, max_frames=2)
    _case(cfg, [2, 1, 2, 1], seed=3, bias=False, splits=3)


def test_reset_and_new_weights():
    """After reset the next chunk has no history; new weights replace the old."""
    G.require_gpu()
    cfg = C.ConvConfig(height=4, width=6, in_channels=64, out_channels=128, max_frames=2)
    state = C.CausalConv(cfg)
    wb, bb = _layer(cfg, 4)
    state.set_weights(G.to_dev(wb), G.to_dev(bb))
    _stream(cfg, state, _video(cfg, 3, 40), [2, 1])
    state.reset()
    wb2, bb2 = _layer(cfg, 5)
    state.set_weights(G.to_dev(wb2), G.to_dev(bb2))
    xb = _video(cfg, 3, 41)
    got = _stream(cfg, state, xb, [1, 2])
    x, w, b = I.bf16_bits_to_f64(xb), I.bf16_bits_to_f64(wb2), I.bf16_bits_to_f64(bb2)
    ref = CO.causal_conv3d(x, w, b)
    _check(got, ref, "after reset", CO.causal_conv3d(np.abs(x), np.abs(w)) + np.abs(b))


def test_streaming_equals_one_call_bitwise():
    """The cache makes chunking invisible: every chunking gives the same bits
    (each output sums the same products in the same order)."""
    G.require_gpu()
    cfg = C.ConvConfig(height=6, width=10, in_channels=128, out_channels=128, max_frames=5)
    wb, bb = _layer(cfg, 6)
    xb = _video(cfg, 5, 6)
    outs = []
    for chunks in ([5], [1, 1, 1, 1, 1], [2, 3], [3, 1, 1]):
        state = C.CausalConv(cfg)
        state.set_weights(G.to_dev(wb), G.to_dev(bb))
        outs.append(_stream(cfg, state, xb, chunks))
    for o in outs[1:]:
        np.testing.assert_array_equal(o, outs[0])


def test_two_layers_on_two_streams():
    """Two independent states (two layers, or two videos) streamed on two HIP
    streams at once, chunks interleaved; each matches its own whole-video
    oracle."""
    G.require_gpu()
    cfg = C.ConvConfig(height=12, width=20, in_channels=128, out_channels=128, max_frames=2)
    chunks = [1, 2, 1, 2]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    cases = []
    for k in range(2):
        wb, bb = _layer(cfg, 20 + k)
        xb = _video(cfg, sum(chunks), 30 + k)
        state = C.CausalConv(cfg)
        w_dev, b_dev = G.to_dev(wb), G.to_dev(bb)
        torch.cuda.synchronize()  # uploads done before the other stream packs them
        state.set_weights(w_dev, b_dev, stream=streams[k])
        cases.append((state, wb, bb, xb, [w_dev, b_dev]))
    t0 = 0
    for n in chunks:
        for k, (state, _, _, xb, outs) in enumerate(cases):
            with torch.cuda.stream(streams[k]):
                x = G.to_dev(xb[t0:t0 + n])
                y = torch.empty((n, cfg.height, cfg.width, cfg.out_channels), dtype=torch.bfloat16, device="cuda")
                state(x, y, stream=streams[k])
                outs.append((x, y))
        t0 += n
    torch.cuda.synchronize()
    for state, wb, bb, xb, outs in cases:
        got = np.concatenate([G.from_dev(y) for _, y in outs[2:]])
        x, w, b = I.bf16_bits_to_f64(xb), I.bf16_bits_to_f64(wb), I.bf16_bits_to_f64(bb)
        ref = CO.causal_conv3d(x, w, b)
        _check(got, ref, "two streams", CO.causal_conv3d(np.abs(x), np.abs(w)) + np.abs(b))


def test_decoder_layer_shape_full_compare():
    """The 384-channel 3x3x3 layer on the 44 x 80 latent grid of the 1280x704
    profile, 3 one-frame chunks then a 2-frame chunk, every output compared."""
    cfg = C.ConvConfig(height=44, width=80, in_channels=384, out_channels=384, max_frames=2)
    mx, rel = _case(cfg, [1, 1, 1, 2], seed=7, splits=3)
    print(f"[conv] 44x80x384: max {mx:.3e} rel {rel:.3e}", flush=True)


def test_bench_shape_sampled_pixels():
    """The benchmarked layer (88 x 160 grid, 384 -> 384, 2-frame chunks) at
    full size: three chunks streamed, then 84 sampled output pixels of the
    last chunk (all channels; 20 of them in the units that split) computed
    one by one by the oracle from the frames that reach them."""
    G.require_gpu()
    cfg = C.ConvConfig(height=88, width=160, in_channels=384, out_channels=384, max_frames=2)
    print(f"[conv] {cfg} sampled", flush=True)
    wb, bb = _layer(cfg, 8)
    xb = _video(cfg, 6, 8)
    state = C.CausalConv(cfg)
    state.set_weights(G.to_dev(wb), G.to_dev(bb))
    got = _stream(cfg, state, xb, [2, 2, 2])
    whole, parts = state.plan(2)
    assert 0 < whole < 660 and parts == 3  # the last round's units split (660 units, 512 slots)
    x = I.bf16_bits_to_f64(xb)
    w = I.bf16_bits_to_f64(wb)
    b = I.bf16_bits_to_f64(bb)
    rng = np.random.default_rng(9)
    picks = [(t, int(rng.integers(cfg.height)), int(rng.integers(cfg.width))) for t in (4, 5) for _ in range(30)]
    picks += [(4, 0, 0), (5, cfg.height - 1, cfg.width - 1), (4, 0, cfg.width - 1), (5, cfg.height - 1, 0)]
    # pixels of the split units (unit >= 512 of the chunk: its second frame, rows >= 48)
    picks += [(5, int(rng.integers(48, cfg.height)), int(rng.integers(cfg.width))) for _ in range(20)]
    ref, out, absum = [], [], []
    for t, i, j in picks:
        # the oracle on the 3 x 3 x 3 neighbourhood that reaches (t, i, j)
        lo_i, lo_j = max(i - 1, 0), max(j - 1, 0)
        sub = x[t - 2:t + 1, lo_i:i + 2, lo_j:j + 2]
        ref.append(CO.causal_conv3d(sub, w, b)[2, i - lo_i, j - lo_j])
        absum.append(CO.causal_conv3d(np.abs(sub), np.abs(w))[2, i - lo_i, j - lo_j] + np.abs(b))
        out.append(got[t, i, j])
    _check(np.array(out), np.array(ref), "88x160x384 sampled", np.array(absum))
