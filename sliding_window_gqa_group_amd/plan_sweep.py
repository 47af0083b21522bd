"""Sweeps of the split plans against the automatic planner, on the GPU, printed as markdown.

    python -m sliding_window_gqa_group_amd.plan_sweep chunk    # 32- to 256-row chunks
    python -m sliding_window_gqa_group_amd.plan_sweep gated    # the gated workload's splits
    python -m sliding_window_gqa_group_amd.plan_sweep large    # the large workload's splits

Every timing runs on rotating input copies (at least 320 MB, so each call reads its K/V from
HBM), after untimed calls, as the mean of back-to-back calls between two events on the stream
the library launches on. The knobs are the library's tuning settings (attn_tuning_set):
`chunk` sets the tiles per split of chunks of the decode heads (8 KV groups x 4 query heads,
d 128, full 4096-slot rings, 4 sinks); `gated` the workgroup target of the single gated
launch; `large` the tiles per split of the 2048-row chunk. The automatic plan is measured
last (after the others have warmed the GPU), and printed first.
"""
from __future__ import annotations

import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROTATE_BYTES = 320 << 20
WARM_S = 0.1


def _setup():
    sys.path.insert(0, os.path.dirname(HERE))
    import torch
    from sliding_window_gqa_group_amd import binding as B, inputs as gen
    return torch, B, gen


def _rotating(torch, base: dict):
    nbytes = sum(v.numel() * v.element_size() for v in base.values() if isinstance(v, torch.Tensor))
    n = max(1, min(32, -(-ROTATE_BYTES // nbytes)))
    return [base] + [{k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in base.items()}
                     for _ in range(n - 1)]


def _time(torch, fn, n_sets: int, steps: int) -> float:
    """us per call: rounds of n_sets untimed calls, each waited for, until WARM_S of wall time
    has passed (clocks up, code and buffers touched; waiting per round keeps the queue from
    holding seconds of calls), then `steps` back-to-back calls between two events."""
    import time
    t0, i = time.perf_counter(), 0
    while True:
        for _ in range(n_sets):
            fn(i)
            i += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= WARM_S:
            break
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for i in range(steps):
        fn(i)
    b.record(stream)
    b.synchronize()
    return a.elapsed_time(b) * 1e3 / steps


def _chunk_call(B, t, scale, out, ws):
    B.attn_window_chunk(t["ring_k"], t["ring_v"], t["meta"], t["sink_k"], t["sink_v"], t["q"],
                        t["chunk_k"], t["chunk_v"], scale, out=out, workspace=ws)


def sweep_chunk() -> str:
    torch, B, gen = _setup()
    dev = "cuda:0"
    ws = B.Workspace(dev)
    lines = ["| rows | knob (tiles per split) | plan (kernel, block, splits, keys per split) | us per call |",
             "|---|---|---|---|"]
    summary = ["", "| rows | automatic | sweep best | gap |", "|---|---|---|---|"]
    meta = gen.decode().meta.copy()
    for rows in (32, 64, 96, 128, 256):
        inp = gen.make_chunk(rows, 8, 4, 128, 4096, 4, meta, seed=7)
        base = gen.to_device(inp, dev)
        sets = _rotating(torch, base)
        out = torch.empty((inp.rows, inp.nh, inp.d), dtype=torch.float32, device=dev)
        res = []
        for tps in (5, 6, 7, 8, 9, 10, 12, 17, 22, 0):
            B.tuning_set(B.TUNE_TILES_PER_SPLIT, tps)
            plan = B.chunk_plan(rows, 8, 4, 128, 4096, 4)
            us = _time(torch, lambda i: _chunk_call(B, sets[i % len(sets)], inp.scale, out, ws), len(sets), 100)
            res.append((us, tps, plan))
            print(f"rows {rows} tps {tps}: {us:.1f} us", file=sys.stderr, flush=True)
        B.tuning_set(B.TUNE_TILES_PER_SPLIT, 0)
        res = [res[-1]] + res[:-1]
        for us, tps, plan in res:
            lines.append(f"| {rows} | {tps or 'automatic'} | {tuple(plan)} | {us:.1f} |")
        best = min(res)
        summary.append(f"| {rows} | {res[0][0]:.1f} us | {best[0]:.1f} us | {(res[0][0] / best[0] - 1) * 100:+.1f} % |")
        del sets, base
        torch.cuda.empty_cache()
    return "\n".join(lines + summary)


def sweep_gated() -> str:
    torch, B, gen = _setup()
    dev = "cuda:0"
    ws = B.Workspace(dev)
    g = gen.gated()
    sets = _rotating(torch, gen.to_device(g, dev))
    out = torch.empty((g.rows, g.nh, g.hd), dtype=torch.float32, device=dev)

    def call(i):
        t = sets[i % len(sets)]
        B.attn_window_gated(t["yq"], t["yk"], t["yv"], t["rope"], t["q_scale"], t["gate"],
                            t["gate_scale"], t["ring_k"], t["ring_v"], g.pos0, g.window, g.scale,
                            g.eps, out=out, workspace=ws)

    rows = []
    for tb in (64, 128, 192, 208, 256, 512, 0):
        B.tuning_set(B.TUNE_TARGET_BLOCKS, tb)
        us = _time(torch, call, len(sets), 200)
        rows.append(f"| {tb or 'automatic'} | {us:.2f} |")
        print(f"gated target {tb}: {us:.2f} us", file=sys.stderr, flush=True)
    B.tuning_set(B.TUNE_TARGET_BLOCKS, 0)
    return "\n".join(["| knob (workgroup target) | us per call |", "|---|---|", rows[-1]] + rows[:-1])


def sweep_large() -> str:
    torch, B, gen = _setup()
    dev = "cuda:0"
    ws = B.Workspace(dev)
    inp = gen.large()
    sets = _rotating(torch, gen.to_device(inp, dev))
    out = torch.empty((inp.rows, inp.nh, inp.d), dtype=torch.float32, device=dev)
    lines = ["| knob (tiles per split) | plan (kernel, block, splits, keys per split) | us per call |",
             "|---|---|---|"]
    rows = []
    for tps in (171, 205, 257, 0):
        B.tuning_set(B.TUNE_TILES_PER_SPLIT, tps)
        plan = B.chunk_plan(inp.rows, inp.ng, inp.hpg, inp.d, inp.w, inp.ns)
        us = _time(torch, lambda i: _chunk_call(B, sets[i % len(sets)], inp.scale, out, ws), len(sets), 5)
        rows.append(f"| {tps or 'automatic'} | {tuple(plan)} | {us:.1f} |")
        print(f"large tps {tps}: {us:.1f} us", file=sys.stderr, flush=True)
    B.tuning_set(B.TUNE_TILES_PER_SPLIT, 0)
    return "\n".join(lines + [rows[-1]] + rows[:-1])


if __name__ == "__main__":
    modes = {"chunk": sweep_chunk, "gated": sweep_gated, "large": sweep_large}
    if len(sys.argv) < 2 or sys.argv[1] not in modes:
        raise SystemExit(__doc__)
    print(modes[sys.argv[1]]())
