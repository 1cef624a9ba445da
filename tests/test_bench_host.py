"""Host logic of bench.py (no GPU): the rollout's call list, its key counts
and FLOP accounting against the oracle's window rule and FLOP convention,
the HBM-counter summary's copy scaling and source check, and the refusal of
more than one GPU."""

import os
import subprocess
import sys

import pytest

import bench
import oracle.ckv_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_rollout_calls_order_and_count():
    cfg = bench.profile_config()
    calls = bench.rollout_calls(cfg)
    assert len(calls) == 4 + 1 + 28 * 4 == 117
    assert calls[:5] == [("first", 0, 0), ("first", 1, 0), ("first", 2, 0), ("first", 3, 0), ("sink", -1, 0)]
    # chunks 1..28 in order, each through its 4 steps
    assert calls[5:9] == [("chunk", s, 1) for s in range(4)]
    assert calls[-1] == ("chunk", 3, 28)
    assert [c for _, _, c in calls[5:]] == sorted(c for _, _, c in calls[5:])


def test_key_counts_and_flops_follow_the_window_rule():
    """keys_of and attn_flops agree with the oracle's window key count and
    4 * Lq * Lk * width convention for every chunk; the 880 x 19,360 call is
    209.35 GFLOP and one rollout 17.3664 TFLOP."""
    cfg = bench.profile_config()
    for c in range(cfg.max_chunks):
        if c == 0:
            assert bench.keys_of(cfg, 0) == cfg.tokens(0) == 2640
            continue
        keys = O.window_key_count(c, cfg.window_chunks, cfg.grid_h, cfg.grid_w, cfg.first_chunk_frames)
        assert bench.keys_of(cfg, c) == keys
        assert bench.attn_flops(cfg, c) == O.attention_flops(880, keys, cfg.num_heads * cfg.head_dim)
    assert bench.keys_of(cfg, 1) == 3520 and bench.keys_of(cfg, 19) == bench.keys_of(cfg, 28) == 19360
    assert bench.attn_flops(cfg, 19) == 4 * 880 * 19360 * 24 * 128 == 209_348_198_400
    total = sum(bench.attn_flops(cfg, c) for _, _, c in bench.rollout_calls(cfg))
    assert round(total / 1e12, 4) == 17.3664


def _write_csv(path, counter, rows):
    with open(path, "w") as f:
        f.write('"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value"\n')
        for i, (name, kib) in enumerate(rows):
            f.write(f'{i},"{name}","{counter}",{kib}\n')


def test_counter_summary_scales_by_the_copy_and_checks_the_source(tmp_path, monkeypatch):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) are scaled by what the same
    counter reads for the 1 GiB copy; the traffic is dropped when the kernel
    source no longer matches the summary's hash."""
    attn = "void ckv::(anonymous namespace)::chunk_attn_kernel<128>(ckv::AttnParams)"
    merge = "void ckv::(anonymous namespace)::attn_combine_kernel<128, 4, 1>(ckv::AttnParams)"
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    # the copy reads 1 GiB: FETCH_SIZE reports half of it, WRITE_SIZE all of it
    _write_csv(fetch, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 524288), (attn, 100000), (merge, 10000),
                                     (attn, 120000), ("other_kernel", 999999)])
    _write_csv(write, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 1048576), (attn, 8000), (merge, 2000),
                                     (attn, 9000)])
    out = tmp_path / "counters.txt"
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(out))
    bench.summarise_counters(str(fetch), str(write))
    text = out.read_text()
    vals = dict(line.split(" = ") for line in text.splitlines() if " = " in line and not line.startswith("#"))
    assert int(vals["attention_calls"]) == 2
    assert float(vals["fetch_scale"]) == pytest.approx(2.0)
    assert float(vals["write_scale"]) == pytest.approx(1.0)
    assert int(vals["fetch_bytes_per_call"]) == (100000 + 10000 + 120000) * 1024 * 2 // 2
    assert int(vals["write_bytes_per_call"]) == (8000 + 2000 + 9000) * 1024 // 2
    assert bench.read_counters() == pytest.approx(float(vals["traffic_bytes_per_call"]))
    other = tmp_path / "other.hip"
    other.write_text("// a different kernel source\n")
    monkeypatch.setattr(bench, "ATTN_SOURCE", str(other))
    assert bench.read_counters() is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single" in r.stderr
    assert r.stdout == ""
