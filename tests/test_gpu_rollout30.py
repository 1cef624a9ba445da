"""The full 30-layer rollout at 1280x704 for 2 prompts on 2 streams
(30 layers x 29 chunks x 4 steps, 24 heads x 128, bf16; per-(layer, step)
rings, 25.6 GB of cache per prompt), checked against the oracle on a seeded
sample of (prompt, layer, chunk, step) calls that includes chunks 1, 2, 19,
20 and 28 and both prompts.

Inputs are drawn on the device by torch's generator, seeded per (prompt,
layer, chunk, step, tensor), so the oracle side can redraw exactly the
tensors a sampled call needs (sink pass + window chunks + own) and copy them
to the host; they come from torch's RNG, not from the library."""

import numpy as np
import pytest
import torch

import chunked_kv_attention_amd as C
import oracle.ckv_oracle as O
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

CFG = C.Config(num_layers=30, num_steps=4, num_heads=24, head_dim=128, grid_h=22, grid_w=40,
               first_chunk_frames=3, window_chunks=18, max_chunks=29)
SINK_STEP = 4  # step code of the clean pass


def _seed(prompt, layer, chunk, step_code, tensor):
    return (((prompt * 64 + layer) * 32 + chunk) * 8 + step_code) * 4 + tensor + 12345


def _draw(prompt, layer, chunk, step_code):
    n = CFG.tokens(chunk)
    g = torch.Generator(device="cuda")
    out = []
    for t in range(3):
        g.manual_seed(_seed(prompt, layer, chunk, step_code, t))
        out.append(torch.randn((n, 24, 128), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16))
    return out


def _sample():
    rng = np.random.default_rng(2024)
    picks = set()
    for prompt in (0, 1):
        for chunk in (1, 2, 19, 20, 28):
            picks.add((prompt, int(rng.integers(0, 30)), chunk, int(rng.integers(0, 4))))
    while len(picks) < 20:
        picks.add((int(rng.integers(0, 2)), int(rng.integers(0, 30)), int(rng.integers(1, 29)), int(rng.integers(0, 4))))
    return sorted(picks)


@pytest.mark.timeout(900)
def test_rollout_30_layers_two_prompts_two_streams():
    G.require_gpu()
    sample = _sample()
    caches = [C.Cache(CFG), C.Cache(CFG)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    kept = {}
    n0, n1 = CFG.tokens(0), CFG.tokens(1)

    def call(prompt, kind, layer, step, chunk):
        cache, stream = caches[prompt], streams[prompt]
        with torch.cuda.stream(stream):
            q, k, v = _draw(prompt, layer, chunk, SINK_STEP if kind == "sink" else step)
            qr, out = torch.empty_like(q), torch.empty_like(q)
            if kind == "sink":
                cache.sink_build(layer, q, k, v, qr, stream=stream)
                cache.chunk_attention(layer, C.STEP_SINK, 0, qr, out, stream=stream)
            else:
                cache.rope_append(layer, step, chunk, q, k, v, qr, stream=stream)
                cache.chunk_attention(layer, step, chunk, qr, out, stream=stream)
            if (prompt, layer, chunk, step) in sample and kind == "chunk":
                kept[(prompt, layer, chunk, step)] = out

    for s in range(4):
        for layer in range(30):
            for prompt in (0, 1):
                call(prompt, "first", layer, s, 0)
    for layer in range(30):
        for prompt in (0, 1):
            call(prompt, "sink", layer, 0, 0)
    for c in range(1, 29):
        for s in range(4):
            for layer in range(30):
                for prompt in (0, 1):
                    call(prompt, "chunk", layer, s, c)
        if c % 7 == 0:
            print(f"  enqueued chunk {c}", flush=True)
    torch.cuda.synchronize()
    print(f"rollout done; checking {len(sample)} sampled calls", flush=True)
    worst = (0.0, 0.0)
    host = lambda ts: [G.from_dev(t) for t in ts]  # noqa: E731
    for prompt, layer, chunk, step in sample:
        rows = G.sample_rows(n1, 24, seed=prompt * 1000 + layer * 10 + chunk)
        got = G.from_dev(kept[(prompt, layer, chunk, step)])[rows]
        q0, k0, v0 = host(_draw(prompt, layer, 0, SINK_STEP))
        win = {j: host(_draw(prompt, layer, j, step))[1:] for j in O.window_chunks(chunk, 18)}
        q, k, v = host(_draw(prompt, layer, chunk, step))
        # the rotated q/k handed to attention in bf16, then unrounded float64
        for inputs in ("bf16", "f64"):
            ro = O.OracleRollout(O.OracleConfig(30, 4, 24, 128, 22, 40, 3, 18, 29, attention_inputs=inputs))
            ro.sink_pass(layer, q0, k0, v0, rows=np.array([0]))
            for j, (kj, vj) in win.items():
                ro.noisy[(layer, step, j)] = (ro.rotate(j, kj), vj)
            ref, _ = ro.chunk_step(layer, step, chunk, q, k, v, rows=rows)
            mx, rl2 = G.assert_attn_close(got, ref, f"prompt {prompt} layer {layer} chunk {chunk} step {step} ({inputs})")
            if inputs == "bf16":
                worst = (max(worst[0], mx), max(worst[1], rl2))
        print(f"  prompt {prompt} layer {layer} chunk {chunk} step {step}: max abs {mx:.2e} rel L2 {rl2:.2e}",
              flush=True)
    assert n0 == 2640
    print(f"30-layer x 2-prompt rollout: {len(sample)} sampled calls, worst max abs {worst[0]:.3e} "
          f"rel L2 {worst[1]:.3e}", flush=True)
