"""Benchmark: same-step chunk attention over a full 29-chunk rollout on one GPU.

One step = one 1-layer rollout of the 1280x704 profile through the C-ABI:
chunk 0 (2640 tokens) for 4 denoising steps (RoPE + append, self-attention),
its clean sink pass (sink build + self-attention), then chunks 1..28 (880
tokens) x 4 steps (RoPE + ring append, chunk attention over sink + up to 18
same-step chunks + itself); 24 heads x 128, bf16.  Inputs (fresh seeded
N(0,1) q, k, v per chunk and step) are resident in HBM before timing starts.

Prints one JSON line.  `value` is algorithmic attention TFLOP/s over the
whole rollout (4 * n_q * n_k * 3072 per attention call, the convention of
"Learning Video Generation from the Wan2.2 Source Code", Chapter 8);
`ms_per_step` is milliseconds per rollout.  The roofline block is for the
dominant kernel, chunk attention (the MFMA kernel plus, when the key range is
split, its small merge kernel), over all of its launches in the timed
rollouts, timed with HIP events on the launch stream; the 880-query x
19,360-key launches (chunks 19..28) are also reported on their own.  After
the timed rollouts (outside them) it also reports the QK-Norm + RoPE + append
path, a device copy of the append's byte count, the cross-attention of an
880-token chunk to a 512-row text context, and two streaming causal Conv3d
layers of the VAE decoder (88x160 and 44x80 grids, 384 channels);
`--no-extras` skips these, so that a profiled run traces only the rollout's
launches.

`--workload rollout30x2` times the whole model's attention traffic (30 layers
x 2 prompts on 2 streams); `--workload attn880x19360` times the chunk-19
attention call alone, for per-kernel counter runs; `--workload
conv88x160x384` / `conv44x80x384` time one streaming causal Conv3d layer of
the VAE decoder (also reported as extras of the default line);
`--workload vendor_reference` times the platform's own bf16 GEMM (hipBLASLt)
and fused attention (torch SDPA) on the same GPU, for context.

`--counters FETCH.csv WRITE.csv` turns two rocprofv3 --pmc runs of
`bench.py --steps 1 --warmup 0 --no-cpu-baseline --no-extras --copy-calibration` (one for
FETCH_SIZE, one for WRITE_SIZE) into the HBM traffic per chunk-attention
call, scaled by what the same counters read for the plain 1 GiB copy, and
writes it with the kernel source's hash to profiles/.
"""

from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
COUNTERS_FILE = os.path.join(ROOT, "profiles", "chunk_attn_rollout_hbm_counters.txt")
ATTN_SOURCE = os.path.join(ROOT, "chunked_kv_attention_amd", "csrc", "chunk_attn.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=24, help="heads in the oracle's timed sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for HBM counter scaling)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the QK-Norm append, cross-attention and copy lines (profiling runs: only the "
                         "rollout's launches are traced)")
    ap.add_argument("--workload", choices=["rollout1", "rollout30x2", "attn880x19360", "attn3x880x19360",
                                           "conv88x160x384", "conv44x80x384", "vendor_reference"], default="rollout1",
                    help="rollout1: 1-layer 29-chunk rollout (default); rollout30x2: 30 layers x 2 prompts on "
                         "2 streams; attn880x19360: the peaky chunk-19 attention call alone, --steps times (for "
                         "per-kernel counter runs); attn3x880x19360: the same call for 3 heads (one GPU's share "
                         "of 8-way head sharding); conv88x160x384 / conv44x80x384: one streaming causal Conv3d "
                         "layer of the VAE decoder alone; vendor_reference: a hipBLASLt bf16 GEMM and torch's "
                         "fused SDPA on the 880 x 19,360 shape, for context")
    ap.add_argument("--counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise rocprofv3 FETCH_SIZE / WRITE_SIZE runs into the counters file and exit")
    return ap.parse_args()


def profile_config():
    import chunked_kv_attention_amd as C
    return C.Config(num_layers=1, num_steps=4, num_heads=24, head_dim=128, grid_h=22, grid_w=40,
                    first_chunk_frames=3, window_chunks=18, max_chunks=29)


def rollout_calls(cfg):
    """(kind, step, chunk) in rollout order: chunk 0's steps, its sink pass,
    then chunks 1.. x steps."""
    calls = [("first", s, 0) for s in range(cfg.num_steps)] + [("sink", -1, 0)]
    calls += [("chunk", s, c) for c in range(1, cfg.max_chunks) for s in range(cfg.num_steps)]
    return calls


def keys_of(cfg, chunk):
    n0, n1 = cfg.tokens(0), cfg.tokens(1)
    if chunk == 0:
        return n0
    return n0 + n1 * min(chunk - 1, cfg.window_chunks) + n1


def attn_flops(cfg, chunk):
    return 4 * cfg.tokens(chunk) * keys_of(cfg, chunk) * cfg.num_heads * cfg.head_dim


ATTN_KERNELS = ("chunk_attn_kernel", "attn_combine_kernel")
COPY_BYTES = 1 << 30


def source_hash():
    return hashlib.sha256(open(ATTN_SOURCE, "rb").read()).hexdigest()


def read_counters():
    """HBM traffic per chunk-attention call from committed rocprofv3 counter
    runs, valid only while the kernel source is unchanged."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    vals = {}
    for line in open(COUNTERS_FILE):
        line = line.split("#", 1)[0].strip()
        if "=" in line:
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != source_hash() or "traffic_bytes_per_call" not in vals:
        return None
    return float(vals["traffic_bytes_per_call"])


def summarise_counters(fetch_csv, write_csv):
    """Per-call HBM bytes of chunk attention from FETCH_SIZE / WRITE_SIZE (KiB
    per dispatch), each scaled by the reading of the same counter for the
    plain 1 GiB copy (copy reads 1 GiB and writes 1 GiB)."""
    import csv

    def load(path, counter):
        attn, copy = [], []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            kib = float(r["Counter_Value"])
            if any(k in name for k in ATTN_KERNELS):
                attn.append((int(r["Dispatch_Id"]), name, kib))
            elif "copyBuffer" in name or "copy" in name.lower():
                copy.append(kib)
        return attn, copy

    f_attn, f_copy = load(fetch_csv, "FETCH_SIZE")
    w_attn, w_copy = load(write_csv, "WRITE_SIZE")
    big_copy_f = max(f_copy)  # the 1 GiB copy dispatches
    big_copy_w = max(w_copy)
    fetch_scale = COPY_BYTES / (big_copy_f * 1024)
    write_scale = COPY_BYTES / (big_copy_w * 1024)
    calls = sum(1 for _, n, _ in f_attn if "chunk_attn_kernel" in n)
    fetch_bytes = sum(k for _, _, k in f_attn) * 1024 * fetch_scale / calls
    write_bytes = sum(k for _, _, k in w_attn) * 1024 * write_scale / calls
    lines = [
        "# HBM traffic of one chunk-attention call (chunk_attn_kernel + attn_combine_kernel),",
        "# averaged over every attention call of the profiled run (its timed and its instrumented",
        "# 1-layer 29-chunk rollout, 117 calls each).",
        "# Commands (run from the repository root; cd /tmp && export TMPDIR=/tmp first):",
        "#   rocprofv3 --pmc FETCH_SIZE -d OUT_F -o fetch --output-format csv -- "
        "python bench.py --steps 1 --warmup 0 --no-cpu-baseline --no-extras --copy-calibration",
        "#   rocprofv3 --pmc WRITE_SIZE -d OUT_W -o write --output-format csv -- "
        "python bench.py --steps 1 --warmup 0 --no-cpu-baseline --no-extras --copy-calibration",
        "#   python bench.py --counters OUT_F/fetch_counter_collection.csv OUT_W/write_counter_collection.csv",
        "# Scaling: the same counters read for the plain 1 GiB device copy (reads and writes 1 GiB).",
        f"copy_fetch_kib = {big_copy_f:.0f}",
        f"copy_write_kib = {big_copy_w:.0f}",
        f"fetch_scale = {fetch_scale:.4f}",
        f"write_scale = {write_scale:.4f}",
        f"attention_calls = {calls}",
        f"fetch_bytes_per_call = {fetch_bytes:.0f}",
        f"write_bytes_per_call = {write_bytes:.0f}",
        f"traffic_bytes_per_call = {fetch_bytes + write_bytes:.0f}",
        f"source_sha256 = {source_hash()}",
    ]
    os.makedirs(os.path.dirname(COUNTERS_FILE), exist_ok=True)
    with open(COUNTERS_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cpu_baseline(cfg, heads, calls=6):
    """The float64 oracle, untuned, on a bounded sample of the same workload
    (about 12 s of host work):
      * the rotation of the sink's and chunks 1..18's keys, then `calls`
        steady-state chunk steps at step 0 (chunks 19, 20, ...: rotate q/k,
        record K/V, attend 880 queries x 19,360 keys) for `heads` heads;
      * one first-chunk step (2640 x 2640 self-attention, the bootstrap of
        the 1280x704 profile), timed on its own.
    Rate = the steady-state attentions' algorithmic FLOPs / wall time
    (rotations included).  The whole 1-layer 29-chunk rollout is then
    extrapolated, not timed: each of its 117 attention calls at the rate
    measured for its kind (bootstrap rate for chunk 0's 5 calls, steady-state
    rate for the rest), plus the measured rotation time per call."""
    import numpy as np

    import oracle.ckv_oracle as O
    from chunked_kv_attention_amd import inputs as I

    ocfg = O.OracleConfig(1, cfg.num_steps, heads, cfg.head_dim, cfg.grid_h, cfg.grid_w,
                          cfg.first_chunk_frames, cfg.window_chunks, cfg.max_chunks)
    ro = O.OracleRollout(ocfg)
    last = 18 + calls
    data = {}
    for c in range(0, last + 1):
        n = cfg.tokens(c)
        data[c] = [I.bf16_bits_to_f64(b) for b in
                   I.draw_qkv_bits(n, heads, cfg.head_dim, base_seed=0, chunk=c, step_code=4 if c == 0 else 0)]
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    t0 = time.perf_counter()
    ro.sink[0] = (ro.rotate(0, data[0][1]), data[0][2])
    for c in range(1, 19):
        ro.noisy[(0, 0, c)] = (ro.rotate(c, data[c][1]), data[c][2])
    for c in range(19, last + 1):
        out, _ = ro.chunk_step(0, 0, c, *data[c])
        assert np.isfinite(out).all()
    dt = time.perf_counter() - t0
    flops = sum(4 * cfg.tokens(c) * keys_of(cfg, c) * heads * cfg.head_dim for c in range(19, last + 1))
    rate = flops / dt
    # one bootstrap step (chunk 0, 2640 x 2640), timed on its own
    t1 = time.perf_counter()
    out0, _ = ro.first_chunk_step(0, 0, *data[0])
    boot_s = time.perf_counter() - t1
    assert np.isfinite(out0).all()
    boot_flops = 4 * cfg.tokens(0) * cfg.tokens(0) * heads * cfg.head_dim
    # extrapolated 1-layer rollout (all heads): chunk 0's 5 calls at the
    # bootstrap rate, the 112 chunk calls at the steady-state rate (both rates
    # include the rotation of the call's own q and k)
    scale = cfg.num_heads / heads
    boot_rate = boot_flops / boot_s
    roll_s = sum(attn_flops(cfg, c) / (boot_rate if c == 0 else rate) for _, _, c in rollout_calls(cfg))
    cpu_model = platform.processor() or ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": rate / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "sample": (f"float64 numpy oracle: RoPE of the sink's and chunks 1..18's keys, then chunks "
                   f"19..{last} at step 0 (RoPE, record, attention 880 x 19,360 keys) for {heads} of 24 heads; "
                   f"{flops / 1e9:.1f} GFLOP in {dt:.2f} s; plus one 2640 x 2640 bootstrap step "
                   f"({boot_flops / 1e9:.1f} GFLOP in {boot_s:.2f} s)"),
        "seconds": dt, "host_cpus": os.cpu_count(), "cpu_model": cpu_model,
        "bootstrap_2640x2640_s": round(boot_s * scale, 3),
        "bootstrap_tflops": round(boot_rate / 1e12, 4),
        "rollout_1layer_s_extrapolated": round(roll_s, 1),
        "extrapolation": ("117 attention calls of the 1-layer 29-chunk rollout, each at the measured rate of its "
                          "kind (rotation included); not timed in full"),
    }


def rollout30x2(args):
    """30 layers x 2 prompts on 2 streams at the 1280x704 profile: one step is
    both prompts' full 30-layer 29-chunk rollouts (chunk -> step -> layer
    order), 1.042 PFLOP of algorithmic attention.  Every (prompt, layer,
    call) gets its own seeded q, k, v, all resident in HBM at once (≈ 123 GB
    of inputs beside 52 GB of caches), so no call rereads another call's
    inputs from a cache."""
    import torch

    import chunked_kv_attention_amd as C

    base = profile_config()
    cfg = C.Config(num_layers=30, num_steps=base.num_steps, num_heads=base.num_heads, head_dim=base.head_dim,
                   grid_h=base.grid_h, grid_w=base.grid_w, first_chunk_frames=base.first_chunk_frames,
                   window_chunks=base.window_chunks, max_chunks=base.max_chunks)
    H, d = cfg.num_heads, cfg.head_dim
    calls = rollout_calls(cfg)
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    # inputs[prompt][call][layer] = (q, k, v): views into one bf16 tensor per
    # (prompt, call), filled a few layers at a time (bounded float32 temporary)
    inputs = [[], []]
    for prompt in range(2):
        for i, (_, _, chunk) in enumerate(calls):
            n = cfg.tokens(chunk)
            block = torch.empty((cfg.num_layers, 3, n, H, d), device=dev, dtype=torch.bfloat16)
            gen.manual_seed(50000 * (prompt + 1) + i)
            for l0 in range(0, cfg.num_layers, 5):
                l1 = min(cfg.num_layers, l0 + 5)
                block[l0:l1] = torch.randn((l1 - l0, 3, n, H, d), generator=gen, device=dev, dtype=torch.float32)
            inputs[prompt].append([(block[layer, 0], block[layer, 1], block[layer, 2])
                                   for layer in range(cfg.num_layers)])
    caches = [C.Cache(cfg), C.Cache(cfg)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    bufs = [{n: (torch.empty((n, H, d), device=dev, dtype=torch.bfloat16),
                 torch.empty((n, H, d), device=dev, dtype=torch.bfloat16)) for n in (cfg.tokens(0), cfg.tokens(1))}
            for _ in range(2)]
    torch.cuda.synchronize()

    def run():
        for c in caches:
            c.reset()
        for i, (kind, step, chunk) in enumerate(calls):
            for layer in range(cfg.num_layers):
                for prompt in range(2):
                    q, k, v = inputs[prompt][i][layer]
                    qr, out = bufs[prompt][q.shape[0]]
                    s = streams[prompt]
                    if kind == "sink":
                        caches[prompt].sink_build(layer, q, k, v, qr, stream=s)
                    else:
                        caches[prompt].rope_append(layer, step, chunk, q, k, v, qr, stream=s)
                    caches[prompt].chunk_attention(layer, C.STEP_SINK if kind == "sink" else step, chunk, qr, out,
                                                   stream=s)

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    flops = 2 * cfg.num_layers * sum(attn_flops(cfg, c) for _, _, c in calls)
    result = {
        "metric": "same-step chunk-attn TFLOP/s + % bf16 MFMA peak; ms per 29-chunk rollout",
        "value": round(flops / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "30-layer 29-chunk same-step rollout at 1280x704 for 2 prompts on 2 streams "
                        "(24 heads x 128; distinct inputs for every prompt, layer and call)",
            "global_batch": 2,
            "seq_len": 19360,
            "parallelism": "none (1 GPU, 2 streams)",
            "algorithmic_tflop_per_step": round(flops / 1e12, 2),
            "cache_gb_per_prompt": round(caches[0].arena.numel() / 1e9, 2),
        },
        "pct_bf16_peak": round(100 * flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "ms_per_30_layer_rollout_both_prompts": round(ms, 2),
        "roofline": None,
    }
    print(json.dumps(result), flush=True)


def single_call_timing(heads=24, calls=50, warmup=60, peaky=True, spread=True):
    """One chunk-attention call shape on its own: 880 queries x 19,360 keys
    (chunk 19: sink 2640 + 18 x 880 window + 880 self), `heads` heads x 128.
    A 1-layer cache gets the sink and chunks 1..19 at step 0 from seeded
    N(0,1) bf16 inputs; with `peaky`, round(1% x 19,360) = 194 of the window's
    key rows (a seeded permutation over all 19,360 positions) are scaled by 4
    before RoPE, for a peaky softmax.  Then `calls` event-timed calls of chunk
    19's attention on the launch stream after `warmup` untimed ones (one event
    pair around them all: the mean), and with `spread` the same number again
    with an event pair around each call (median, p10, p90).  The default
    warm-up is long because a series of identical heavy calls first slows
    down by up to a third (the clock drops under the sustained matrix load)
    and settles again within about 50 calls.
    heads = 3 is one GPU's share of 24 heads sharded 8 ways."""
    import torch

    import chunked_kv_attention_amd as C
    from chunked_kv_attention_amd import inputs as I

    cfg = dataclasses.replace(profile_config(), num_steps=1, num_heads=heads)
    d = cfg.head_dim
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    n0, n1 = cfg.tokens(0), cfg.tokens(1)
    total = keys_of(cfg, 19)
    rows = I.peaky_key_rows(total, 0.01, (7, heads, 19)) if peaky else []

    def rnd(n):
        return torch.randn((n, heads, d), generator=gen, device=dev, dtype=torch.float32)

    def key_rows(chunk, k):
        lo = 0 if chunk == 0 else n0 + n1 * (chunk - 1)
        sel = [r - lo for r in rows if lo <= r < lo + k.shape[0]]
        if sel:
            k[torch.tensor(sel, device=dev)] *= 4.0
        return k.to(torch.bfloat16)

    cache = C.Cache(cfg)
    q0 = rnd(n0).to(torch.bfloat16)
    cache.sink_build(0, q0, key_rows(0, rnd(n0)), rnd(n0).to(torch.bfloat16), torch.empty_like(q0))
    q_rot = torch.empty((n1, heads, d), device=dev, dtype=torch.bfloat16)
    for c in range(1, 20):
        cache.rope_append(0, 0, c, rnd(n1).to(torch.bfloat16), key_rows(c, rnd(n1)), rnd(n1).to(torch.bfloat16),
                          q_rot)
    out = torch.empty_like(q_rot)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        cache.chunk_attention(0, 0, 19, q_rot, out, stream=stream)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(calls):
        cache.chunk_attention(0, 0, 19, q_rot, out, stream=stream)
    stop.record(stream)
    torch.cuda.synchronize()
    us = 1e3 * start.elapsed_time(stop) / calls
    spread_us = None
    if spread:
        # the same calls again, an event pair around each one
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
        for a, b in pairs:
            a.record(stream)
            cache.chunk_attention(0, 0, 19, q_rot, out, stream=stream)
            b.record(stream)
        torch.cuda.synchronize()
        each = sorted(1e3 * a.elapsed_time(b) for a, b in pairs)

        def pct(q):
            return round(each[min(len(each) - 1, int(q * (len(each) - 1) + 0.5))], 2)

        spread_us = {"p10": pct(0.1), "median": pct(0.5), "p90": pct(0.9),
                     "note": "an event pair around each call (pair overhead included)"}

    flops = attn_flops(cfg, 19)
    tflops = flops / (us * 1e-6) / 1e12
    return {"us_per_call": round(us, 2), "tflops": round(tflops, 2),
            "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2), "launches_timed": calls,
            "per_call_events_us": spread_us,
            "key_splits": cache.attention_splits(n1, total), "heads": heads,
            "inputs": ("N(0,1) bf16; 194 of the 19,360 window key rows scaled x4 before RoPE (peaky softmax)"
                       if peaky else "N(0,1) bf16")}


def attn880x19360(args, heads=24):
    """`--workload attn880x19360` (24 heads) / `attn3x880x19360` (3 heads):
    the single peaky 880-query x 19,360-key call alone, `--steps` timed calls
    (also used for per-kernel counter runs, where the rollout's mix of call
    shapes would blur the counters)."""
    r = single_call_timing(heads, calls=args.steps, warmup=args.warmup, spread=False)
    print(json.dumps({
        "metric": "chunk-attn TFLOP/s, 880 queries x 19,360 keys",
        "value": r["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "us_per_call": r["us_per_call"],
        "higher_is_better": True,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"one chunk-attention call: 880 queries x 19,360 keys (sink + 18 chunks + self), "
                               f"{heads} heads x 128", "inputs": r["inputs"], "key_splits": r["key_splits"]},
        "pct_bf16_peak": r["pct_bf16_peak"],
    }), flush=True)


def appends_back_to_back(C, cfg, dev, stream, inputs, calls, gains=None, reps=4):
    """RoPE + append (QK-Norm + RoPE + append when `gains` is given) of the
    880-token chunks 1..28 at step 0, launched back to back into a fresh cache
    after its sink, with one event pair around the 28 appends (an event
    between two launches is a queue barrier); per-call time = the pair's time
    / 28, the median over `reps` - 1 timed repetitions after one warm-up."""
    import torch
    H, d = cfg.num_heads, cfg.head_dim
    cache = C.Cache(cfg)
    chunk_inputs = {c: inputs[i] for i, (kind, step, c) in enumerate(calls) if kind == "chunk" and step == 0}
    sink_in = next(inputs[i] for i, (kind, _, _) in enumerate(calls) if kind == "sink")
    n0, n1 = cfg.tokens(0), cfg.tokens(1)
    qr0 = torch.empty((n0, H, d), device=dev, dtype=torch.bfloat16)
    qr1 = torch.empty((n1, H, d), device=dev, dtype=torch.bfloat16)
    times = []
    for rep in range(reps):
        cache.reset()
        if gains is None:
            cache.sink_build(0, *sink_in, qr0, stream=stream)
        else:
            cache.norm_sink_build(0, *sink_in, *gains, 1e-6, qr0, stream=stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for c in range(1, 29):
            if gains is None:
                cache.rope_append(0, 0, c, *chunk_inputs[c], qr1, stream=stream)
            else:
                cache.norm_rope_append(0, 0, c, *chunk_inputs[c], *gains, 1e-6, qr1, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        if rep:
            times.append(e0.elapsed_time(e1) * 1e3 / 28)
    times.sort()
    us = times[len(times) // 2]
    nbytes = 6 * n1 * H * d * 2
    return {"us_per_call": round(us, 2), "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
            "pct_hbm_peak": round(100 * nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 2),
            "timing": "28 appends back to back between one event pair (chunks 1..28, step 0)"}


def norm_append_and_copy(C, cfg, dev, stream, inputs, calls):
    """QK-Norm + RoPE + append on the 880-token chunks (its own cache; gains
    seeded), and a plain device copy of the same byte count for context."""
    import torch
    H, d = cfg.num_heads, cfg.head_dim
    g = torch.Generator(device=dev)
    g.manual_seed(77)
    gains = [1.0 + 0.3 * torch.randn(H * d, generator=g, device=dev, dtype=torch.float32) for _ in range(2)]
    norm = appends_back_to_back(C, cfg, dev, stream, inputs, calls, gains)
    n1 = cfg.tokens(1)
    nbytes = 6 * n1 * H * d * 2
    # 16 distinct buffer pairs (0.5 GB), so the copies stream from HBM like the appends' fresh inputs
    pairs = [(torch.empty(nbytes // 2, dtype=torch.uint8, device=dev),   # read + write = the append's bytes
              torch.empty(nbytes // 2, dtype=torch.uint8, device=dev)) for _ in range(16)]
    for a, b in pairs:
        b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for r in range(48):
        a, b = pairs[r % 16]
        b.copy_(a)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_us = e0.elapsed_time(e1) * 1e3 / 48
    del pairs
    norm["note"] = "algorithmic bytes as rope_append_880 (the norm adds no pass over q and k)"
    return (norm,
            {"bytes_moved": nbytes, "us_per_copy": round(copy_us, 2),
             "gbs": round(nbytes / (copy_us * 1e-6) / 1e9, 1),
             "note": "device-to-device copy moving the append's byte count (half read, half written), event-timed"})


def cross_attention_timing(C, cfg, dev, stream):
    """Cross-attention of an 880-token chunk to a 512-row text context
    (seeded N(0,1) bf16), 50 calls after warm-up, event-timed."""
    import torch
    H, d = cfg.num_heads, cfg.head_dim
    g = torch.Generator(device=dev)
    g.manual_seed(88)
    k, v = (torch.randn((512, H, d), generator=g, device=dev).to(torch.bfloat16) for _ in range(2))
    q = torch.randn((880, H, d), generator=g, device=dev).to(torch.bfloat16)
    out = torch.empty_like(q)
    cache = C.Cache(dataclasses.replace(cfg, num_layers=1, num_steps=1))
    cache.text_store(0, k, v, stream=stream)
    for _ in range(5):
        cache.cross_attention(0, 1, q, out, stream=stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(50):
        cache.cross_attention(0, 1, q, out, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / 50
    flops = 4 * 880 * 512 * H * d
    return {"us_per_call": round(us, 2), "tflops": round(flops / (us * 1e-6) / 1e12, 2),
            "pct_bf16_peak": round(100 * flops / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 2),
            "key_splits": cache.attention_splits(880, 512)}


CONV_LAYERS = {
    # name: (H, W, C_in, C_out, frames per call) -- 3x3x3 causal Conv3d layers
    "conv88x160x384": (88, 160, 384, 384, 2),
    "conv44x80x384": (44, 80, 384, 384, 1),
}


def conv_timing(name, calls=40, warmup=4):
    """Streaming causal Conv3d through the C-ABI: `calls` chunks of one layer
    (seeded N(0,1) bf16 frames, weights N(0,1)/sqrt(fan-in)), event-timed on
    the launch stream; each call is the conv kernel plus the cache update.
    FLOPs = 2 * pixels * C_out * 27 * C_in per call."""
    import torch

    import chunked_kv_attention_amd as C

    h, w, ci, co, frames = CONV_LAYERS[name]
    cfg = C.ConvConfig(height=h, width=w, in_channels=ci, out_channels=co, max_frames=frames)
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(31)
    weight = (torch.randn((co, ci, 3, 3, 3), generator=g, device=dev) / (27 * ci) ** 0.5).to(torch.bfloat16)
    bias = (0.1 * torch.randn((co,), generator=g, device=dev)).to(torch.bfloat16)
    xs = [torch.randn((frames, h, w, ci), generator=g, device=dev).to(torch.bfloat16) for _ in range(4)]
    y = torch.empty((frames, h, w, co), device=dev, dtype=torch.bfloat16)
    state = C.CausalConv(cfg)
    stream = torch.cuda.current_stream()
    state.set_weights(weight, bias, stream=stream)
    for i in range(warmup):
        state(xs[i % 4], y, stream=stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(calls):
        state(xs[i % 4], y, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / calls
    flops = 2 * frames * h * w * co * 27 * ci
    tflops = flops / (us * 1e-6) / 1e12
    return {"us_per_call": round(us, 2), "tflops": round(tflops, 2),
            "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2), "gflop_per_call": round(flops / 1e9, 2),
            "layer": f"causal Conv3d 3x3x3, {ci}->{co} channels, {h}x{w} grid, {frames} frame(s) per call",
            "calls_timed": calls}


def conv_workload(args):
    """`--workload conv88x160x384` / `conv44x80x384`: one streaming causal
    Conv3d layer alone, `--steps` timed calls (for per-kernel profiles)."""
    r = conv_timing(args.workload, calls=args.steps, warmup=args.warmup)
    print(json.dumps({
        "metric": "streaming causal Conv3d TFLOP/s", "value": r["tflops"], "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "us_per_call": r["us_per_call"], "higher_is_better": True,
        "dtype": "bf16", "data": "synthetic", "config": {"workload": r["layer"]},
        "pct_bf16_peak": r["pct_bf16_peak"],
    }), flush=True)


def vendor_reference(args):
    """`--workload vendor_reference`: the platform's own libraries on the same
    GPU, for context beside the nominal peak: a plain bf16 GEMM (torch.mm on
    contiguous 8192 x 8192 operands, i.e. hipBLASLt) and torch's fused
    scaled_dot_product_attention on the 880-query x 19,360-key x 24-head x
    128 shape with contiguous bf16 Q, K, V.  Only the flash and
    memory-efficient backends are allowed (the math backend would run batched
    products over transposed bf16 views).  Event-timed, `--steps` (at least
    20) calls after `--warmup` (at least 3)."""
    import torch
    from torch.nn.attention import SDPBackend, sdpa_kernel

    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    reps, warm = max(args.steps, 20), max(args.warmup, 3)

    def timed(fn):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(reps):
            fn()
        stop.record()
        torch.cuda.synchronize()
        return 1e3 * start.elapsed_time(stop) / reps

    n = 8192
    a, b = (torch.randn((n, n), generator=gen, device=dev).to(torch.bfloat16) for _ in range(2))
    c = torch.empty((n, n), device=dev, dtype=torch.bfloat16)
    us_mm = timed(lambda: torch.mm(a, b, out=c))
    del a, b, c
    H, d, nq, nk = 24, 128, 880, 19360
    q = torch.randn((1, H, nq, d), generator=gen, device=dev).to(torch.bfloat16)
    k, v = (torch.randn((1, H, nk, d), generator=gen, device=dev).to(torch.bfloat16) for _ in range(2))
    with sdpa_kernel([SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION]):
        us_sdpa = timed(lambda: torch.nn.functional.scaled_dot_product_attention(q, k, v))
    attn = 4 * nq * nk * H * d
    mm_tflops = 2 * n ** 3 / (us_mm * 1e-6) / 1e12
    sdpa_tflops = attn / (us_sdpa * 1e-6) / 1e12
    print(json.dumps({
        "metric": "vendor library bf16 throughput (context)", "value": round(mm_tflops, 1), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": reps, "warmup": warm, "higher_is_better": True, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "torch.mm 8192 x 8192 x 8192 bf16 (hipBLASLt); torch SDPA (flash / mem-efficient "
                               "backend) 880 x 19,360 keys x 24 heads x 128, bf16"},
        "gemm_8192": {"us_per_call": round(us_mm, 1), "tflops": round(mm_tflops, 1),
                      "pct_bf16_peak": round(100 * mm_tflops / PEAK_BF16_TFLOPS, 2)},
        "sdpa_880x19360": {"us_per_call": round(us_sdpa, 1), "tflops": round(sdpa_tflops, 1),
                           "pct_bf16_peak": round(100 * sdpa_tflops / PEAK_BF16_TFLOPS, 2)},
    }), flush=True)


def main():
    args = parse()
    if args.counters:
        summarise_counters(*args.counters)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the same-step chunk attention path is built and timed on a single "
              "MI355X; sharding heads across GPUs is described in the design notes, not implemented. Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import chunked_kv_attention_amd as C

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    C.load()
    if args.workload == "rollout30x2":
        rollout30x2(args)
        return
    if args.workload == "attn880x19360":
        attn880x19360(args)
        return
    if args.workload == "attn3x880x19360":
        attn880x19360(args, heads=3)
        return
    if args.workload in CONV_LAYERS:
        conv_workload(args)
        return
    if args.workload == "vendor_reference":
        vendor_reference(args)
        return
    dev = torch.device("cuda:0")
    cfg = profile_config()
    H, d = cfg.num_heads, cfg.head_dim
    calls = rollout_calls(cfg)

    # Inputs: fresh seeded N(0,1) q, k, v for every call, resident in HBM.
    gen = torch.Generator(device=dev)
    inputs = {}
    for i, (kind, step, chunk) in enumerate(calls):
        n = cfg.tokens(chunk)
        gen.manual_seed(1000 + i)
        inputs[i] = [torch.randn((n, H, d), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
                     for _ in range(3)]
    q_rot = {n: torch.empty((n, H, d), device=dev, dtype=torch.bfloat16) for n in (cfg.tokens(0), cfg.tokens(1))}
    out = {n: torch.empty((n, H, d), device=dev, dtype=torch.bfloat16) for n in (cfg.tokens(0), cfg.tokens(1))}
    cache = C.Cache(cfg)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    total_flops = sum(attn_flops(cfg, c) for _, _, c in calls)
    big = [i for i, (kind, _, c) in enumerate(calls) if kind == "chunk" and keys_of(cfg, c) == 19360]
    append_idx = [i for i, (kind, _, c) in enumerate(calls) if kind == "chunk"]

    def run_rollout(events=None):
        cache.reset()
        for i, (kind, step, chunk) in enumerate(calls):
            q, k, v = inputs[i]
            n = q.shape[0]
            ev = events[i] if events is not None else None
            if ev is not None:
                ev[0].record(stream)
            if kind == "sink":
                cache.sink_build(0, q, k, v, q_rot[n], stream=stream)
            else:
                cache.rope_append(0, step, chunk, q, k, v, q_rot[n], stream=stream)
            if ev is not None:
                ev[1].record(stream)
            cache.chunk_attention(0, C.STEP_SINK if kind == "sink" else step, chunk, q_rot[n], out[n],
                                  stream=stream)
            if ev is not None:
                ev[2].record(stream)

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    for _ in range(args.warmup):
        run_rollout()
    torch.cuda.synchronize()

    # Timed rollouts: events only at the two ends (an event recorded between
    # two launches is a queue barrier that idles the GPU for microseconds).
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for k in range(args.steps):
        run_rollout()
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / args.steps

    # The same number of rollouts again, instrumented: event pairs around every
    # append and attention call give the per-launch figures (roofline, append).
    events = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in calls] for _ in range(args.steps)]
    torch.cuda.synchronize()
    i0 = torch.cuda.Event(enable_timing=True)
    i1 = torch.cuda.Event(enable_timing=True)
    i0.record(stream)
    for k in range(args.steps):
        run_rollout(events[k])
    i1.record(stream)
    torch.cuda.synchronize()
    instrumented_ms = i0.elapsed_time(i1) / args.steps

    attn_big_ms = [events[k][i][1].elapsed_time(events[k][i][2]) for k in range(args.steps) for i in big]
    attn_all_ms = sum(events[k][i][1].elapsed_time(events[k][i][2]) for k in range(args.steps)
                      for i in range(len(calls)))
    append_ms = [events[k][i][0].elapsed_time(events[k][i][1]) for k in range(args.steps) for i in append_idx]
    big_flops = attn_flops(cfg, 19)
    big_us = 1e3 * sum(attn_big_ms) / len(attn_big_ms)
    big_tflops = big_flops / (big_us * 1e-6) / 1e12
    attn_us_per_call = 1e3 * attn_all_ms / (args.steps * len(calls))
    attn_flops_per_call = total_flops / len(calls)
    attn_tflops = attn_flops_per_call / (attn_us_per_call * 1e-6) / 1e12
    append_bytes = 6 * cfg.tokens(1) * H * d * 2
    append_us = 1e3 * sum(append_ms) / len(append_ms)
    traffic = read_counters()

    result = {
        "metric": "same-step chunk-attn TFLOP/s + % bf16 MFMA peak; ms per 29-chunk rollout",
        "value": round(total_flops / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "1-layer 29-chunk same-step rollout at 1280x704: chunk 0 = 2640 tokens x 4 steps + "
                        "sink pass, chunks 1..28 = 880 tokens x 4 steps, window = sink + 18 same-step chunks "
                        "+ self (<= 19,360 keys), 24 heads x 128",
            "global_batch": 1,
            "seq_len": 19360,
            "parallelism": "none (1 GPU)",
            "attention_calls_per_step": len(calls),
            "algorithmic_tflop_per_step": round(total_flops / 1e12, 4),
        },
        "pct_bf16_peak": round(100 * total_flops / (ms_per_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "chunk_attn_880x19360_in_rollout": {
            "inputs": "N(0,1) bf16 (the rollout's own chunks 19..28)",
            "us_per_call": round(big_us, 2),
            "tflops": round(big_tflops, 2),
            "pct_bf16_peak": round(100 * big_tflops / PEAK_BF16_TFLOPS, 2),
            "launches_timed": len(attn_big_ms),
            "key_splits": cache.attention_splits(880, 19360),
        },
        "attention_share_of_step": round(attn_all_ms / (instrumented_ms * args.steps), 4),
        "ms_per_step_with_per_call_events": round(instrumented_ms, 3),
        "rope_append_880": appends_back_to_back(C, cfg, dev, stream, inputs, calls),
        "rope_append_880_event_pairs": {
            "us_per_call": round(append_us, 2),
            "gbs": round(append_bytes / (append_us * 1e-6) / 1e9, 1),
            "timing": "an event pair around every append of the instrumented rollouts (barrier cost included)",
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(attn_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "kernel": "chunk attention call (chunk_attn_kernel + attn_combine_kernel when split)",
            "launches_timed": args.steps * len(calls),
            "flops_per_launch": attn_flops_per_call,
            "us_per_launch": round(attn_us_per_call, 2),
            "timing": "HIP event pairs around every attention call of the instrumented rollouts",
            "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-scaled)",
        },
    }
    if not args.no_extras:
        # the single call as stated for the 880 x 19,360 shape (peaky keys), and
        # the 3-head share of 8-way head sharding (24 key splits)
        result["chunk_attn_880x19360"] = single_call_timing(24)
        result["chunk_attn_880x19360_3heads"] = single_call_timing(3)
        result["norm_rope_append_880"], result["device_copy_same_bytes"] = norm_append_and_copy(
            C, cfg, dev, stream, inputs, calls)
        result["cross_attn_880x512"] = cross_attention_timing(C, cfg, dev, stream)
        result["causal_conv_88x160x384"] = conv_timing("conv88x160x384")
        result["causal_conv_44x80x384"] = conv_timing("conv44x80x384")
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, args.cpu_heads)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
