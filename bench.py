"""Throughput of windowed grouped-query attention on one MI355X.

Default workload: the decode call (1 row, 8 KV groups x 4 query heads, d=128, full 4096-slot
rings with seeded head offsets, 4 sinks). A step is one attn_window_chunk call on one of
`--sets` copies of the inputs at distinct addresses (>= 0.5 GB in total, so the 256 MB
Infinity Cache cannot hold them and the K/V stream comes from HBM). Prints ONE JSON line.

value = distinct K/V bytes per call / time per call (GB/s); rows/s and the fraction of the
8 TB/s HBM peak are reported beside it. `roofline` divides the call's algorithmic bytes by the
time per call from the HIP events that bracket the timed loop on the library's stream (a
second pass with an event pair around every call is reported beside it); its `traffic` is the
calibrated rocprofv3 FETCH_SIZE + WRITE_SIZE bytes of one call, when they were taken on the
current kernel sources. `cpu_baseline` times the CPU oracle on a bounded sample. `also` holds
the other workloads (timed on resident inputs, labelled hot-cache).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
F32_PEAK_TFLOPS = 157.3
METRIC = "KV GB/s and rows/s for windowed GQA attention; % of HBM peak"
KERNEL_NAMES = {1: "attn_dec_kernel", 2: "attn_mfma_kernel", 3: "attn_valu_kernel",
                4: "attn_mfma16_kernel"}
COUNTERS_FILE = os.path.join(ROOT, "profiles", "attn_dec_kernel_decode_counters.json")
CALIBRATION_COPY_BYTES = 64 << 20


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sliding_window_gqa_group_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on
    the current kernel sources; else None."""
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_digest") != kernel_source_digest():
        return None
    return c.get("hbm_bytes_per_launch")


def chunk_tensors(inp, torch, dev):
    from sliding_window_gqa_group_amd import inputs as gen
    t = gen.to_device(inp, dev)
    if inp.ns == 0:
        t["sink_k"] = t["sink_v"] = None
    return t


def run_chunk(B, t, scale, out, ws):
    return B.attn_window_chunk(t["ring_k"], t["ring_v"], t["meta"], t["sink_k"], t["sink_v"],
                               t["q"], t["chunk_k"], t["chunk_v"], scale, out=out, workspace=ws)


WARM_MS = 50.0


def time_calls(torch, fn, n_sets, steps, warmup):
    """(ms per step over a bracketed loop, mean and median per-call event ms).

    Untimed first: calls for at least WARM_MS of wall time (the GPU leaves its idle clocks;
    this workload's code and buffers are touched), then `warmup` calls. The step time comes
    from one pair of events around `steps` back-to-back calls; the per-call times from a second
    pass with an event pair around each call (both on the stream the library launches on,
    torch's current stream)."""
    stream = torch.cuda.current_stream()
    t0w, s = time.perf_counter(), 0
    while (time.perf_counter() - t0w) * 1e3 < WARM_MS:
        fn(s % n_sets)
        s += 1
        if s % 8 == 0:
            torch.cuda.synchronize()
    for s in range(warmup):
        fn(s % n_sets)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for s in range(steps):
        fn(s % n_sets)
    t1.record(stream)
    torch.cuda.synchronize()
    total = t0.elapsed_time(t1)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for s in range(steps):
        starts[s].record(stream)
        fn(s % n_sets)
        ends[s].record(stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    return total / steps, float(np.mean(per)), float(np.median(per))


def bench_decode(args, torch, B, gen, acct):
    dev = "cuda:0"
    inp = gen.decode()
    base = chunk_tensors(inp, torch, dev)
    sets = [base] + [{k: (v.clone() if v is not None else None) for k, v in base.items()}
                     for _ in range(args.sets - 1)]
    outs = [torch.empty((inp.rows, inp.nh, inp.d), dtype=torch.float32, device=dev)
            for _ in range(args.sets)]
    ws = B.Workspace(dev)
    ws.get(B.chunk_workspace_bytes(inp.rows, inp.ng, inp.hpg, inp.d, inp.w, inp.ns))

    # correctness gate on the timed configuration
    import oracle
    run_chunk(B, sets[0], inp.scale, outs[0], ws)
    torch.cuda.synchronize()
    ref = oracle.window_chunk(inp)
    got = outs[0].cpu().numpy()
    ok = bool(np.all(np.abs(got - ref) <= np.maximum(1e-4 * np.abs(ref), 1e-5)))
    if not ok:
        raise SystemExit("bench: decode output does not match the oracle")

    ms, ev_mean, ev_med = time_calls(torch, lambda i: run_chunk(B, sets[i], inp.scale, outs[i], ws),
                                     args.sets, args.steps, args.warmup)
    kv = acct.unique_kv_bytes(inp)
    tot = acct.total_bytes(inp)
    set_bytes = sum(v.numel() * v.element_size() for v in base.values() if v is not None)
    return inp, ms, ev_mean, ev_med, kv, tot, set_bytes


def cpu_baseline(inp, seconds: float):
    import oracle
    from sliding_window_gqa_group_amd import accounting as acct
    oracle.window_chunk(inp)   # load / warm
    n, t0 = 0, time.perf_counter()
    while True:
        oracle.window_chunk(inp)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds or n >= 10000:
            break
    per = el / n
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(acct.unique_kv_bytes(inp) / per / 1e9, 4), "unit": "GB/s",
            "cores": cores, "kind": "oracle",
            "sample": f"{n} full decode calls (f64 accumulation), {el:.1f} s wall, "
                      f"{per * 1e3:.3f} ms per call"}


def bench_others(args, torch, B, gen, acct):
    dev = "cuda:0"
    res = {}
    for name, make in (("tiny", gen.tiny), ("prefill", gen.prefill), ("large", gen.large)):
        inp = make()
        t = chunk_tensors(inp, torch, dev)
        out = torch.empty((inp.rows, inp.nh, inp.d), dtype=torch.float32, device=dev)
        ws = B.Workspace(dev)
        ws.get(B.chunk_workspace_bytes(inp.rows, inp.ng, inp.hpg, inp.d, inp.w, inp.ns))
        steps = 5 if name == "large" else 20
        ms, ev_mean, _ = time_calls(torch, lambda i: run_chunk(B, t, inp.scale, out, ws), 1, steps, 3)
        flops = acct.chunk_flops(inp)
        kern = B.chunk_plan(inp.rows, inp.ng, inp.hpg, inp.d, inp.w, inp.ns)
        res[name] = {"ms": round(ms, 5), "kv_gbs": round(acct.unique_kv_bytes(inp) / ms / 1e6, 2),
                     "rows_per_s": round(inp.rows / ms * 1e3, 1),
                     "tflops": round(flops / ms / 1e9, 3),
                     "tflops_frac_f32_peak": round(flops / ms / 1e9 / F32_PEAK_TFLOPS, 4),
                     "kernel": KERNEL_NAMES[kern[0]], "splits": kern[2],
                     "cache": "hot (inputs resident, reused)"}
        del t, out, ws
        torch.cuda.empty_cache()
    # decode over a 32768-slot window (268 MB of K/V per call): three input sets at distinct
    # addresses (805 MB, beyond the 256 MB Infinity Cache), so K/V come from HBM
    inp = gen.decode_long()
    base = chunk_tensors(inp, torch, dev)
    sets = [base] + [{k: (v.clone() if v is not None else None) for k, v in base.items()}
                     for _ in range(2)]
    outs = [torch.empty((inp.rows, inp.nh, inp.d), dtype=torch.float32, device=dev) for _ in range(3)]
    ws = B.Workspace(dev)
    ws.get(B.chunk_workspace_bytes(inp.rows, inp.ng, inp.hpg, inp.d, inp.w, inp.ns))
    ms, _, _ = time_calls(torch, lambda i: run_chunk(B, sets[i], inp.scale, outs[i], ws), 3, 60, 6)
    kern = B.chunk_plan(inp.rows, inp.ng, inp.hpg, inp.d, inp.w, inp.ns)
    res["decode_w32768"] = {"ms": round(ms, 5),
                            "kv_gbs": round(acct.unique_kv_bytes(inp) / ms / 1e6, 2),
                            "hbm_frac": round(acct.total_bytes(inp) / ms / 1e6 / HBM_PEAK_GBS, 4),
                            "rows_per_s": round(inp.rows / ms * 1e3, 1),
                            "kernel": KERNEL_NAMES[kern[0]], "splits": kern[2],
                            "keys_per_split": kern[3],
                            "cache": "rotating (3 input sets, 805 MB)"}
    del base, sets, outs, ws
    torch.cuda.empty_cache()
    for name, rows in (("decode_far_m32", 1), ("chunk64_far_m32", 64)):
        # the decode shapes with a far field of 32 landmarks per head in every group (full
        # rings, so every row evicts); the near-only call on the same inputs is timed beside it
        inp = gen.make_chunk(rows, 8, 4, 128, 4096, 4, gen.decode().meta.copy(), seed=7)
        inp.meta[:, 2] = 1000
        far = gen.make_far(inp, 32, seed=8)
        t = chunk_tensors(inp, torch, dev)
        f = gen.to_device(far, dev)
        out = torch.empty((inp.rows, inp.nh, inp.d), dtype=torch.float32, device=dev)
        ws = B.Workspace(dev)
        ws.get(B.chunk_far_workspace_bytes(inp.rows, inp.ng, inp.hpg, inp.d, inp.w, inp.ns, 32))

        def far_call(i):
            B.attn_window_chunk_far(t["ring_k"], t["ring_v"], t["meta"], t["sink_k"],
                                    t["sink_v"], t["q"], t["chunk_k"], t["chunk_v"],
                                    f["k_tilde"], f["q_tilde"], f["mu"], f["mz"], f["t_hat"],
                                    inp.scale, out=out, workspace=ws)
        ms, _, _ = time_calls(torch, far_call, 1, 20, 3)
        near_ms, _, _ = time_calls(torch, lambda i: run_chunk(B, t, inp.scale, out, ws), 1, 20, 3)
        res[name] = {"ms": round(ms, 5), "near_only_ms": round(near_ms, 5),
                     "kv_gbs": round(acct.unique_kv_bytes(inp) / ms / 1e6, 2),
                     "rows_per_s": round(inp.rows / ms * 1e3, 1), "landmarks": 32,
                     "cache": "hot (inputs resident, reused)"}
        del t, f, out, ws
        torch.cuda.empty_cache()
    # the gated one-row call with 32 landmarks per head, at the gated workload's head shapes
    # (16 query / 4 KV heads, hd 256, full 1024-slot rings); the same call with every far
    # count 0 (far part skipped) is timed beside it
    gf = gen.make_gated_far(16, 4, 256, 1024, 0, 32, [(1024, 0, 5000, 0)] * 4, seed=9,
                            scale=1 / 16)
    t = gen.to_device(gf, dev)
    out = torch.empty((16, 256), dtype=torch.float32, device=dev)
    ws = B.Workspace(dev)

    def gated_far_call(i, meta):
        B.attn_window_gated_far(t["q"], t["ring_k"], t["ring_v"], meta, None, None,
                                t["k_tilde"], t["mu"], t["mz"], t["t_hat"], t["gate"],
                                t["gate_scale"], gf.scale, out=out, workspace=ws)
    ms, _, _ = time_calls(torch, lambda i: gated_far_call(i, t["meta"]), 1, 20, 3)
    empty = t["meta"].clone()
    empty[:, 2] = 0
    near_ms, _, _ = time_calls(torch, lambda i: gated_far_call(i, empty), 1, 20, 3)
    res["gated_far_m32"] = {"ms": round(ms, 5), "far_empty_ms": round(near_ms, 5),
                            "kv_gbs": round(4 * 1024 * 256 * 8 / ms / 1e6, 2),
                            "landmarks": 32, "cache": "hot (inputs resident, reused)"}
    del t, out, ws
    torch.cuda.empty_cache()
    # encoder attention: one 9801-position sequence with 16 heads of 64 and no window (the
    # vision tower's shape), and 16 packed sequences of seeded lengths U[64, 1024] with 16
    # query / 4 KV heads of 64 and a symmetric window of 128
    rng = np.random.default_rng(11)
    for name, lens, nh, nk, win in (
            ("encoder_full_9801", [9801], 16, 16, 0),
            ("encoder_varlen_window128", [int(x) for x in rng.integers(64, 1025, size=16)], 16, 4, 128)):
        e = gen.make_encoder(lens, nh, nk, 64, win, seed=12)
        q = torch.from_numpy(e.q).to(dev)
        k = torch.from_numpy(e.k).to(dev)
        v = torch.from_numpy(e.v).to(dev)
        segs = torch.from_numpy(e.segs.view(np.int32).copy()).to(dev)
        out = torch.empty((e.q.shape[0], nh * 64), dtype=torch.float32, device=dev)
        mx = max(lens)
        ms, _, _ = time_calls(torch, lambda i: B.attn_encoder(q, k, v, segs, nh, nk, 64, e.scale,
                                                               window=win, max_len=mx, out=out),
                              1, 5 if name.endswith("9801") else 20, 2)
        flops = acct.encoder_flops(e)
        res[name] = {"ms": round(ms, 5), "tflops": round(flops / ms / 1e9, 3),
                     "tflops_frac_f32_peak": round(flops / ms / 1e9 / F32_PEAK_TFLOPS, 4),
                     "tokens": int(sum(lens)), "kernel": "enc_attn_kernel",
                     "cache": "hot (inputs resident, reused)"}
        del q, k, v, segs, out
        torch.cuda.empty_cache()
    g = gen.gated()
    t = gen.to_device(g, dev)
    out = torch.empty((g.rows, g.nh, g.hd), dtype=torch.float32, device=dev)

    def gated_call(i):
        B.attn_window_gated(t["yq"], t["yk"], t["yv"], t["rope"], t["q_scale"], t["gate"],
                            t["gate_scale"], t["ring_k"], t["ring_v"], g.pos0, g.window, g.scale,
                            g.eps, out=out)
    ms, _, _ = time_calls(torch, gated_call, 1, 20, 3)
    kv, tot, flops = acct.gated_counts(g)
    res["gated"] = {"ms": round(ms, 5), "kv_gbs": round(kv / ms / 1e6, 2),
                    "rows_per_s": round(g.rows / ms * 1e3, 1),
                    "tflops": round(flops / ms / 1e9, 3),
                    "tflops_frac_f32_peak": round(flops / ms / 1e9 / F32_PEAK_TFLOPS, 4),
                    "cache": "hot (inputs resident, reused)"}
    return res


def counter_run(args, torch, B, gen):
    """A short, untimed run for hardware-counter passes: one device-to-device copy of
    CALIBRATION_COPY_BYTES (reads and writes exactly that many bytes), then `calls` calls of one
    workload on rotating input sets, as the timed decode run makes them."""
    dev = "cuda:0"
    src = torch.empty(CALIBRATION_COPY_BYTES // 4, dtype=torch.float32, device=dev).normal_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    name = args.counter_run
    if name == "encoder":
        e = gen.make_encoder([9801], 16, 16, 64, 0, seed=12)
        q, k, v = (torch.from_numpy(a).to(dev) for a in (e.q, e.k, e.v))
        segs = torch.from_numpy(e.segs.view(np.int32).copy()).to(dev)
        out = torch.empty((9801, 16 * 64), dtype=torch.float32, device=dev)
        for _ in range(args.calls):
            B.attn_encoder(q, k, v, segs, 16, 16, 64, e.scale, max_len=9801, out=out)
    elif name == "decode_far":
        inp = gen.make_chunk(1, 8, 4, 128, 4096, 4, gen.decode().meta.copy(), seed=7)
        inp.meta[:, 2] = 1000
        far = gen.make_far(inp, 32, seed=8)
        t = chunk_tensors(inp, torch, dev)
        f = gen.to_device(far, dev)
        out = torch.empty((inp.rows, inp.nh, inp.d), dtype=torch.float32, device=dev)
        for _ in range(args.calls):
            B.attn_window_chunk_far(t["ring_k"], t["ring_v"], t["meta"], t["sink_k"],
                                    t["sink_v"], t["q"], t["chunk_k"], t["chunk_v"],
                                    f["k_tilde"], f["q_tilde"], f["mu"], f["mz"], f["t_hat"],
                                    inp.scale, out=out)
    elif name == "gated":
        g = gen.gated()
        t = gen.to_device(g, dev)
        out = torch.empty((g.rows, g.nh, g.hd), dtype=torch.float32, device=dev)
        for _ in range(args.calls):
            B.attn_window_gated(t["yq"], t["yk"], t["yv"], t["rope"], t["q_scale"], t["gate"],
                                t["gate_scale"], t["ring_k"], t["ring_v"], g.pos0, g.window,
                                g.scale, g.eps, out=out)
    else:
        inp = {"tiny": gen.tiny, "decode": gen.decode, "prefill": gen.prefill,
               "large": gen.large, "decode_long": gen.decode_long}[name]()
        base = chunk_tensors(inp, torch, dev)
        n_sets = {"tiny": args.sets, "decode": args.sets, "decode_long": 3}.get(name, 1)
        sets = [base] + [{k: (v.clone() if v is not None else None) for k, v in base.items()}
                         for _ in range(n_sets - 1)]
        out = torch.empty((inp.rows, inp.nh, inp.d), dtype=torch.float32, device=dev)
        ws = B.Workspace(dev)
        ws.get(B.chunk_workspace_bytes(inp.rows, inp.ng, inp.hpg, inp.d, inp.w, inp.ns))
        for i in range(args.calls):
            run_chunk(B, sets[i % n_sets], inp.scale, out, ws)
    torch.cuda.synchronize()
    print(f"counter run: {name}, {args.calls} calls, calibration copy {CALIBRATION_COPY_BYTES} B",
          flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=20, help="rotating input copies (>= 16)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-others", action="store_true")
    ap.add_argument("--counter-run", choices=["tiny", "decode", "prefill", "large", "gated",
                                              "encoder", "decode_far", "decode_long"],
                    help="untimed calls of one workload for rocprofv3 counter passes; no JSON")
    ap.add_argument("--calls", type=int, default=20)
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: measures one GPU only; run with --gpus 1 (the per-GPU "
              "sharding by KV group is described in the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    from sliding_window_gqa_group_amd import accounting as acct
    from sliding_window_gqa_group_amd import binding as B
    from sliding_window_gqa_group_amd import inputs as gen

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    B.load()
    if args.counter_run:
        counter_run(args, torch, B, gen)
        return
    inp, ms, ev_mean, ev_med, kv, tot, set_bytes = bench_decode(args, torch, B, gen, acct)
    value = kv / (ms * 1e-3) / 1e9
    plan = B.chunk_plan(inp.rows, inp.ng, inp.hpg, inp.d, inp.w, inp.ns)
    kname = KERNEL_NAMES[plan[0]]
    traffic = measured_traffic()
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0,1), numpy PCG64 seed 1)",
        "config": {"workload": "decode", "rows": inp.rows, "ng": inp.ng, "hpg": inp.hpg,
                   "nh": inp.nh, "d": inp.d, "w": inp.w, "ns": inp.ns, "ring": "full, seeded heads",
                   "input_sets": args.sets, "rotating_bytes": args.sets * set_bytes,
                   "kernel": kname, "splits": plan[2], "keys_per_split": plan[3]},
        "rows_per_s": round(inp.rows / (ms * 1e-3), 1),
        "hbm_frac": round(tot / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        # One launch = one attn_window_chunk call (the attention kernel and the split merge),
        # timed by the HIP events that bracket the timed loop on the library's stream.
        "roofline": {
            "bound": "hbm",
            "achieved": round(tot / (ms * 1e-3) / 1e9, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(tot / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": f"{kname} + split_merge_kernel, one attn_window_chunk call",
            "algorithmic_bytes_per_launch": tot,
            "launch_ms_mean": round(ms, 6),
            "per_call_event_ms_mean": round(ev_mean, 6),
            "per_call_event_ms_median": round(ev_med, 6),
        },
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    if not args.no_others:
        line["also"] = bench_others(args, torch, B, gen, acct)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
