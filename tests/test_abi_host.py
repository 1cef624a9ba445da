"""Host-side checks of the C-ABI library: exported symbols, arena sizing, the
ring indexer's slot map and window segments (bit-exact against the oracle's
window rule and a brute-force ring simulation), and the schedule's error codes
through dry caches.  No GPU needed."""

import ctypes
import os
import re

import pytest

import chunked_kv_attention_amd as C
import oracle.ckv_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROFILE = C.Config(num_layers=2, num_steps=4, num_heads=24, head_dim=128, grid_h=22, grid_w=40,
                   first_chunk_frames=3, window_chunks=18, max_chunks=29)
TINY = C.Config(1, 2, 1, 64, 4, 4, 3, 2, 6)
FAKE = 0x10000  # aligned, never dereferenced by a dry cache


def test_exports_match_header():
    declared = set()
    for name in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if name.endswith(".h"):
            header = open(os.path.join(ROOT, "include", name)).read()
            declared |= set(re.findall(r"^(?:[\w\s\*]+?)\b(ckv_\w+)\s*\(", header, flags=re.M))
    assert declared == set(C.EXPORTS)
    lib = ctypes.CDLL(C.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings():
    for st in range(6):
        assert C.status_string(st)
    assert C.status_string(99) == "unknown status"


def test_cache_bytes_covers_store():
    n1, n0, R = 880, 2640, 19
    H, d, L, S = 24, 128, 2, 4
    store = L * 2 * H * n0 * d * 2 + L * S * 2 * H * R * n1 * d * 2 + L * 2 * H * C.MAX_TEXT_TOKENS * d * 2
    nbytes = C.cache_bytes(PROFILE)
    assert store <= nbytes <= store + 4 * n0 * H * (d + 1) * 4 + (1 << 20)
    bad = [dict(head_dim=96), dict(grid_w=41), dict(num_layers=0), dict(window_chunks=-1),
           dict(rope_theta=0.5), dict(softmax_scale=-1.0)]
    for kw in bad:
        cfg = C.Config(**{**PROFILE.__dict__, **kw})
        assert C.cache_bytes(cfg) == 0, kw


def test_create_arena_errors():
    lib = C.load()
    cfg = PROFILE.to_c()
    need = lib.ckv_cache_bytes(ctypes.byref(cfg))
    h = ctypes.c_void_p()
    assert lib.ckv_cache_create(ctypes.byref(cfg), None, need, ctypes.byref(h)) == C.CKV_E_ARENA
    assert lib.ckv_cache_create(ctypes.byref(cfg), 0x10010, need, ctypes.byref(h)) == C.CKV_E_ARENA
    assert lib.ckv_cache_create(ctypes.byref(cfg), 0x10000, need - 1, ctypes.byref(h)) == C.CKV_E_ARENA
    bad = C.Config(**{**PROFILE.__dict__, "head_dim": 80}).to_c()
    assert lib.ckv_cache_create(ctypes.byref(bad), 0x10000, need, ctypes.byref(h)) == C.CKV_E_INVALID


def _segments_to_chunks(segs):
    ids = []
    for s in segs:
        if s["kind"] == 0:
            ids.append(("sink", 0))
        else:
            ids.extend(("ring", s["chunk_first"] + i) for i in range(s["n_chunks"]))
    return ids


@pytest.mark.parametrize("window", [0, 1, 2, 5, 18, 40])
def test_window_segments_match_oracle(window):
    cfg = C.Config(1, 1, 2, 64, 2, 4, 3, window, 60)
    cache = C.Cache(cfg, dry=True)
    for c in range(60):
        segs = cache.window(0, 0, c)
        ids = _segments_to_chunks(segs)
        assert ids[0] == ("sink", 0)
        if c == 0:
            assert ids == [("sink", 0)] and segs[0]["n_tokens"] == 24
            continue
        assert [i for _, i in ids[1:-1]] == O.window_chunks(c, window)  # bit-exact membership
        assert ids[-1] == ("ring", c)                                   # self is the newest entry
        assert sum(s["n_tokens"] for s in segs) == O.window_key_count(c, window, 2, 4, 3)
        assert len(segs) <= 3


@pytest.mark.parametrize("window", [0, 1, 2, 18])
def test_ring_slots_match_fifo_simulation(window):
    """Brute force: a ring of W+1 slots; each append takes the first free slot
    or evicts the oldest chunk.  Every chunk a window needs must be resident
    in the slot the segments point at."""
    R = window + 1
    cfg = C.Config(1, 1, 1, 64, 2, 4, 3, window, 60)
    cache = C.Cache(cfg, dry=True)
    slots = [None] * R
    for c in range(1, 60):
        if None in slots:
            target = slots.index(None)
        else:
            target = min(range(R), key=lambda i: slots[i])
        slots[target] = c
        assert cache.ring_slot(c) == target
        for s in cache.window(0, 0, c)[1:]:
            for i in range(s["n_chunks"]):
                assert slots[(s["first_slot"] + i) % R] == s["chunk_first"] + i
                assert s["first_slot"] + i < R  # runs never wrap inside themselves


def test_profile_key_counts():
    cache = C.Cache(PROFILE, dry=True)
    counts = {c: sum(s["n_tokens"] for s in cache.window(0, 0, c)) for c in range(29)}
    assert counts[0] == 2640 and counts[1] == 3520 and counts[2] == 4400
    assert all(counts[c] == 19360 for c in range(19, 29))
    assert max(counts.values()) == 19360


def test_dry_rollout_model_card_schedule():
    cache = C.Cache(PROFILE, dry=True)
    for _ in range(2):  # two rollouts, reset between them
        for s in range(4):
            for layer in range(2):
                cache.rope_append(layer, s, 0, FAKE, FAKE, FAKE, FAKE)
                cache.chunk_attention(layer, s, 0, FAKE, FAKE)
        for layer in range(2):
            cache.sink_build(layer, FAKE, FAKE, FAKE, FAKE)
            cache.chunk_attention(layer, C.STEP_SINK, 0, FAKE, FAKE)
        for c in range(1, 29):
            for s in range(4):
                for layer in range(2):
                    cache.rope_append(layer, s, c, FAKE, FAKE, FAKE, FAKE)
                    cache.chunk_attention(layer, s, c, FAKE, FAKE)
        cache.reset()


def _expect(status, fn, *args):
    with pytest.raises(C.CkvError) as e:
        fn(*args)
    assert e.value.status == status, str(e.value)


def test_schedule_errors():
    cache = C.Cache(TINY, dry=True)
    a = (FAKE, FAKE, FAKE, FAKE)
    # chunk >= 1 before the sink
    _expect(C.CKV_E_STATE, cache.rope_append, 0, 0, 1, *a)
    # chunk 0 attention before its append
    _expect(C.CKV_E_STATE, cache.chunk_attention, 0, 0, 0, FAKE, FAKE)
    _expect(C.CKV_E_STATE, cache.chunk_attention, 0, C.STEP_SINK, 0, FAKE, FAKE)
    cache.rope_append(0, 0, 0, *a)
    cache.chunk_attention(0, 0, 0, FAKE, FAKE)
    cache.rope_append(0, 1, 0, *a)
    # the sink area now holds step 1's chunk-0 K/V
    _expect(C.CKV_E_STATE, cache.chunk_attention, 0, 0, 0, FAKE, FAKE)
    cache.sink_build(0, *a)
    _expect(C.CKV_E_STATE, cache.sink_build, 0, *a)       # once per rollout
    _expect(C.CKV_E_STATE, cache.rope_append, 0, 0, 0, *a)  # would overwrite the sink
    cache.chunk_attention(0, C.STEP_SINK, 0, FAKE, FAKE)
    # order on one ring
    _expect(C.CKV_E_ORDER, cache.rope_append, 0, 0, 2, *a)
    _expect(C.CKV_E_ORDER, cache.chunk_attention, 0, 0, 1, FAKE, FAKE)
    cache.rope_append(0, 0, 1, *a)
    cache.chunk_attention(0, 0, 1, FAKE, FAKE)
    cache.chunk_attention(0, 0, 1, FAKE, FAKE)  # re-reading is allowed
    _expect(C.CKV_E_ORDER, cache.chunk_attention, 0, 1, 1, FAKE, FAKE)  # step 1 ring is separate
    cache.rope_append(0, 0, 2, *a)
    _expect(C.CKV_E_ORDER, cache.chunk_attention, 0, 0, 1, FAKE, FAKE)  # no longer the newest
    _expect(C.CKV_E_ORDER, cache.rope_append, 0, 0, 2, *a)  # no repeats
    # bad indices and pointers
    _expect(C.CKV_E_INVALID, cache.rope_append, 1, 0, 3, *a)
    _expect(C.CKV_E_INVALID, cache.rope_append, 0, 2, 3, *a)
    _expect(C.CKV_E_INVALID, cache.rope_append, 0, 0, 6, *a)
    _expect(C.CKV_E_INVALID, cache.rope_append, 0, 0, 3, FAKE + 8, FAKE, FAKE, FAKE)
    _expect(C.CKV_E_INVALID, cache.chunk_attention, 0, -1, 2, FAKE, FAKE)
    # a failing call changed nothing: the right next call still succeeds
    cache.rope_append(0, 0, 3, *a)
    cache.chunk_attention(0, 0, 3, FAKE, FAKE)
    # debug copies: live vs evicted (W = 2 keeps chunks 1..3 live after chunk 3... ring holds 3 slots)
    cache.debug_copy_kv(0, 0, 3, FAKE, FAKE)
    cache.debug_copy_kv(0, 0, 1, FAKE, FAKE)
    cache.rope_append(0, 0, 4, *a)
    _expect(C.CKV_E_STATE, cache.debug_copy_kv, 0, 0, 1, FAKE, FAKE)   # evicted by chunk 4
    _expect(C.CKV_E_STATE, cache.debug_copy_kv, 0, 0, 5, FAKE, FAKE)   # not appended yet
    cache.debug_copy_kv(0, C.STEP_SINK, 0, FAKE, FAKE)
    # reset forgets everything
    cache.reset()
    _expect(C.CKV_E_STATE, cache.rope_append, 0, 0, 1, *a)
    cache.rope_append(0, 0, 0, *a)


def test_attention_splits_policy():
    cache = C.Cache(PROFILE, dry=True)
    # 880 queries x 24 heads = 168 workgroups of 128 rows: split keys to fill two per CU
    assert cache.attention_splits(880, 19360) == 3
    # 2640 x 24 = 504 workgroups already fill the chip
    assert cache.attention_splits(2640, 2640) == 1
    # never fewer than 8 key tiles per split: a 512-row text context runs unsplit
    assert cache.attention_splits(880, 64 * 15) == 1
    assert cache.attention_splits(880, 512) == 1
    assert cache.attention_splits(880, 64 * 16) == 2
    # every chunk window of the rollout (>= 3,520 keys) keeps the 3-way split
    assert cache.attention_splits(880, 3520) == 3


def test_norm_entry_points_validate_and_follow_the_schedule():
    cache = C.Cache(TINY, dry=True)
    a = (FAKE, FAKE, FAKE)
    g = (FAKE, FAKE)
    # arguments of the norm: eps finite and > 0, gains non-null and 16-byte aligned
    for eps in (0.0, -1e-6, float("nan"), float("inf")):
        _expect(C.CKV_E_INVALID, cache.norm_sink_build, 0, *a, *g, eps, FAKE)
    _expect(C.CKV_E_INVALID, cache.norm_sink_build, 0, *a, 0, FAKE, 1e-6, FAKE)
    _expect(C.CKV_E_INVALID, cache.norm_sink_build, 0, *a, FAKE, FAKE + 4, 1e-6, FAKE)
    # the norm variants obey the plain calls' schedule rules
    _expect(C.CKV_E_STATE, cache.norm_rope_append, 0, 0, 1, *a, *g, 1e-6, FAKE)  # before the sink
    cache.norm_rope_append(0, 0, 0, *a, *g, 1e-6, FAKE)
    cache.chunk_attention(0, 0, 0, FAKE, FAKE)
    cache.norm_sink_build(0, *a, *g, 1e-6, FAKE)
    _expect(C.CKV_E_STATE, cache.norm_sink_build, 0, *a, *g, 1e-6, FAKE)  # once per rollout
    _expect(C.CKV_E_ORDER, cache.norm_rope_append, 0, 0, 2, *a, *g, 1e-6, FAKE)
    cache.norm_rope_append(0, 0, 1, *a, *g, 1e-6, FAKE)
    cache.rope_append(0, 0, 2, *a, FAKE)  # plain and norm appends share one ring order
    cache.chunk_attention(0, 0, 2, FAKE, FAKE)


def test_text_context_store_and_cross_attention_rules():
    cache = C.Cache(TINY, dry=True)
    # no context yet
    _expect(C.CKV_E_STATE, cache.cross_attention, 0, 1, FAKE, FAKE)
    # argument checks
    for n in (0, -1, C.MAX_TEXT_TOKENS + 1):
        _expect(C.CKV_E_INVALID, cache.text_store_rows, 0, FAKE, FAKE, n)
    _expect(C.CKV_E_INVALID, cache.text_store_rows, 1, FAKE, FAKE, 8)       # one layer only
    _expect(C.CKV_E_INVALID, cache.text_store_rows, 0, 0, FAKE, 8)          # null
    _expect(C.CKV_E_INVALID, cache.text_store_rows, 0, FAKE + 8, FAKE, 8)   # misaligned
    cache.text_store_rows(0, FAKE, FAKE, 77)
    cache.text_store_rows(0, FAKE, FAKE, C.MAX_TEXT_TOKENS)  # replaces
    # independent of the ring schedule: any chunk index, before any append
    cache.cross_attention(0, 0, FAKE, FAKE)
    cache.cross_attention(0, 5, FAKE, FAKE)
    _expect(C.CKV_E_INVALID, cache.cross_attention, 0, 6, FAKE, FAKE)
    _expect(C.CKV_E_INVALID, cache.cross_attention, 1, 1, FAKE, FAKE)
    cache.reset()  # a new rollout (prompt) forgets the context
    _expect(C.CKV_E_STATE, cache.cross_attention, 0, 1, FAKE, FAKE)


def test_cache_bytes_include_one_context_per_layer():
    one = C.cache_bytes(PROFILE)
    more = C.cache_bytes(C.Config(num_layers=PROFILE.num_layers + 1, num_steps=4, num_heads=24, head_dim=128, grid_h=22, grid_w=40,
                                  first_chunk_frames=3, window_chunks=18, max_chunks=29))
    # per layer: sink + 4 rings + the context's K and V^T (512 x 24 x 128 bf16 each)
    sink = 2 * 24 * 2640 * 128 * 2
    rings = 4 * 2 * 24 * 19 * 880 * 128 * 2
    text = 2 * 24 * 512 * 128 * 2
    assert more - one == sink + rings + text


def test_static_scratch_entry_point_follows_the_same_checks():
    """ckv_chunk_attention_static validates and orders exactly like
    ckv_chunk_attention (dry cache: no device work)."""
    lib = C.load()
    cfg = TINY.to_c()
    h = ctypes.c_void_p()
    assert lib.ckv_cache_create_dry(ctypes.byref(cfg), ctypes.byref(h)) == C.CKV_OK
    try:
        for fn in (lib.ckv_chunk_attention, lib.ckv_chunk_attention_static):
            assert fn(h, 0, 0, 1, FAKE, FAKE, None) == C.CKV_E_STATE      # no sink yet
            assert fn(None, 0, 0, 1, FAKE, FAKE, None) == C.CKV_E_INVALID
            assert fn(h, 0, 0, 1, FAKE + 8, FAKE, None) == C.CKV_E_INVALID  # misaligned
        assert lib.ckv_sink_build(h, 0, FAKE, FAKE, FAKE, FAKE, None) == C.CKV_OK
        assert lib.ckv_rope_append(h, 0, 0, 1, FAKE, FAKE, FAKE, FAKE, None) == C.CKV_OK
        for fn in (lib.ckv_chunk_attention, lib.ckv_chunk_attention_static):
            assert fn(h, 0, 0, 1, FAKE, FAKE, None) == C.CKV_OK
            assert fn(h, 0, 0, 2, FAKE, FAKE, None) == C.CKV_E_ORDER       # chunk 2 not appended
            assert fn(h, 0, C.STEP_SINK, 0, FAKE, FAKE, None) == C.CKV_OK
    finally:
        lib.ckv_cache_destroy(h)


def test_static_scratch_size_in_header_covers_every_split_call():
    """The header's CKV_STATIC_SCRATCH_BYTES holds the fp16 partials and
    float32 log-sum-exps of the largest split call the split policy allows
    (2 slots x 256 CUs x 128 query rows, head_dim 128)."""
    header = open(os.path.join(ROOT, "include", "ckv.h")).read()
    m = re.search(r"#define CKV_STATIC_SCRATCH_BYTES \(\(size_t\)(\d+) \* (\d+) \* (\d+) \* \((\d+) \* 2 \+ 4\)\)", header)
    assert m, "define not found"
    slots, cus, rows, d = (int(x) for x in m.groups())
    assert slots * cus * rows * (d * 2 + 4) == 2 * 256 * 128 * (128 * 2 + 4)
