"""Host-side rules of the causal-convolution C-ABI (include/ckv_conv.h),
exercised on a dry state: config and arena validation, argument checks, the
weights-first rule, and the stream position ("Learning Video Generation from
the Wan2.2 Source Code", Chapter 2, "Causal Convolution and Streaming
Inference": a chunk's history is the frames before it in the stream)."""

import ctypes

import pytest

import chunked_kv_attention_amd as C

FAKE = 0x10000  # aligned, never dereferenced by a dry state
BASE = C.ConvConfig(height=44, width=80, in_channels=384, out_channels=384, kt=3, kh=3, kw=3, max_frames=4)


def _cfg(**kw):
    return C.ConvConfig(**{**BASE.__dict__, **kw})


def test_bytes_cover_weights_bias_cache_zero_row_and_partials():
    taps = 27
    need = taps * 384 * 384 * 2 + 384 * 4 + C.CONV_CACHE_T * 44 * 80 * 384 * 2 + 384 * 2
    partials = 3 * 4 * 44 * 80 * 384 * 4  # kt splits of a 4-frame chunk, float32
    assert need + partials <= C.conv_bytes(BASE) <= need + partials + 5 * 256
    one_tap = _cfg(kt=1)  # no split possible: no partials
    need1 = 9 * 384 * 384 * 2 + 384 * 4 + C.CONV_CACHE_T * 44 * 80 * 384 * 2 + 384 * 2
    assert need1 <= C.conv_bytes(one_tap) <= need1 + 5 * 256


def test_split_policy():
    """Which units split their reduction by time offset (256 CUs assumed dry,
    two workgroups each = 512 slots): every unit when even the split parts
    fill at most two rounds; otherwise only a last, partly filled round whose
    parts fit in one round; never for kt = 1."""
    s = C.CausalConv(BASE, dry=True)
    assert [s.plan(f) for f in (1, 2, 3, 4)] == [(0, 3)] * 4        # 84..330 units of 44x80 frames
    assert s.splits(0) == 0 and s.splits(5) == 0
    big = C.CausalConv(_cfg(height=88, width=160, max_frames=3), dry=True)
    assert big.plan(1) == (0, 3)                                     # 330 units -> 990 parts
    assert big.plan(2) == (512, 3)                                   # 660 units: last 148 split -> 444 parts
    assert big.plan(3) == (990, 1)                                   # 990 units: last 478 would need 1434 parts
    assert C.CausalConv(_cfg(kt=1), dry=True).plan(1) == (84, 1)
    assert C.CausalConv(_cfg(kt=2), dry=True).plan(1) == (0, 2)
    exact = C.CausalConv(_cfg(height=64, width=256, out_channels=128, max_frames=8), dry=True)
    assert exact.plan(8) == (1024, 1)                                # 1024 units: two full rounds, no tail


@pytest.mark.parametrize("bad", [dict(in_channels=32), dict(in_channels=96), dict(out_channels=64),
                                 dict(out_channels=192), dict(kt=0), dict(kt=4), dict(kh=2), dict(kw=5),
                                 dict(height=0), dict(width=0), dict(max_frames=0)])
def test_invalid_configs_have_no_size(bad):
    assert C.conv_bytes(_cfg(**bad)) == 0
    with pytest.raises(C.CkvError) as e:
        C.CausalConv(_cfg(**bad), dry=True)
    assert e.value.status == C.CKV_E_INVALID


def test_arena_checks():
    lib = C.load()
    cfg = BASE.to_c()
    n = lib.ckv_conv_bytes(ctypes.byref(cfg))
    h = ctypes.c_void_p()
    assert lib.ckv_conv_create(ctypes.byref(cfg), ctypes.c_void_p(FAKE), n - 1, ctypes.byref(h)) == C.CKV_E_ARENA
    assert lib.ckv_conv_create(ctypes.byref(cfg), ctypes.c_void_p(FAKE + 16), n, ctypes.byref(h)) == C.CKV_E_ARENA
    assert lib.ckv_conv_create(ctypes.byref(cfg), None, n, ctypes.byref(h)) == C.CKV_E_ARENA
    assert lib.ckv_conv_create(ctypes.byref(cfg), ctypes.c_void_p(FAKE), n, ctypes.byref(h)) == C.CKV_OK
    assert lib.ckv_conv_destroy(h) == C.CKV_OK


def test_weights_first_then_position_advances_and_resets():
    s = C.CausalConv(BASE, dry=True)
    with pytest.raises(C.CkvError) as e:
        s.call_raw(FAKE, 1, FAKE * 1024)
    assert e.value.status == C.CKV_E_STATE
    assert s.position == 0
    with pytest.raises(C.CkvError):
        s.set_weights_raw(None)
    with pytest.raises(C.CkvError):
        s.set_weights_raw(FAKE + 8)
    s.set_weights_raw(FAKE, FAKE + 2)  # bias needs only bf16 alignment
    y = FAKE + (1 << 32)
    for n, pos in [(1, 1), (2, 3), (4, 7), (1, 8)]:
        s.call_raw(FAKE, n, y)
        assert s.position == pos
    s.reset()
    assert s.position == 0


def test_call_argument_checks_change_nothing():
    s = C.CausalConv(BASE, dry=True)
    s.set_weights_raw(FAKE)
    y = FAKE + (1 << 32)
    x_bytes = 44 * 80 * 384 * 2
    bad = [(FAKE, 0, y), (FAKE, 5, y), (FAKE, -1, y), (FAKE + 8, 1, y), (FAKE, 1, y + 8), (None, 1, y),
           (FAKE, 1, None), (FAKE, 1, FAKE), (FAKE, 2, FAKE + x_bytes), (FAKE + x_bytes // 2, 1, FAKE)]
    for xp, n, yp in bad:
        with pytest.raises(C.CkvError) as e:
            s.call_raw(xp, n, yp)
        assert e.value.status == C.CKV_E_INVALID, (xp, n, yp)
        assert s.position == 0
    s.call_raw(FAKE, 2, FAKE + 2 * x_bytes)  # adjacent, not overlapping
    assert s.position == 2
