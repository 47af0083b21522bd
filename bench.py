"""Throughput of windowed grouped-query attention on one MI355X.

Default workload: the decode call (1 row, 8 KV groups x 4 query heads, d=128, full 4096-slot
rings with seeded head offsets, 4 sinks). A step is one attn_window_chunk call on one of
`--sets` copies of the inputs at distinct addresses (>= 0.5 GB in total, so the 256 MB
Infinity Cache cannot hold them and the K/V stream comes from HBM). Prints ONE JSON line.

value = distinct K/V bytes per call / time per call (GB/s); rows/s and the fraction of the
8 TB/s HBM peak are reported beside it. `roofline` divides the call's algorithmic bytes by the
time per call from the HIP events that bracket the timed loop on the library's stream (a
second pass with an event pair around every call is reported beside it); beside the peak it
gives the rate of a plain streaming read of the same number of bytes, timed the same way in
the same run (the achievable rate for one launch of this size), and the fraction of it. Its
`traffic` is the calibrated rocprofv3 FETCH_SIZE + WRITE_SIZE bytes of one call, when they were
taken on the current kernel sources. `cpu_baseline` times the CPU oracle on the decode call;
every workload under `also` carries its own oracle timing (`cpu_oracle`) in the same units.
Every workload rotates through copies of its inputs that together exceed the Infinity Cache.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
F32_PEAK_TFLOPS = 157.3
METRIC = "KV GB/s and rows/s for windowed GQA attention; % of HBM peak"
KERNEL_NAMES = {1: "attn_dec_kernel", 2: "attn_mfma_kernel", 3: "attn_valu_kernel",
                4: "attn_mfma16_kernel", 5: "attn_decode_kernel"}
COUNTERS_FILE = os.path.join(ROOT, "profiles", "attn_decode_kernel_decode_counters.json")
CALIBRATION_COPY_BYTES = 64 << 20
# Rotating input copies of a workload together hold at least this many bytes (more than the
# 256 MB Infinity Cache), so that every call reads its inputs from HBM.
ROTATE_BYTES = 320 << 20
# Oracle timing: median of up to 3 runs, stopping once the runs took this long.
ORACLE_BUDGET_S = 10.0


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on
    the current kernel sources; else None."""
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    from sliding_window_gqa_group_amd.build import DECODE_SOURCES, source_digest
    if c.get("kernel_source_digest") != source_digest(DECODE_SOURCES):
        return None
    return c.get("hbm_bytes_per_launch")


def chunk_tensors(inp, torch, dev):
    from sliding_window_gqa_group_amd import inputs as gen
    t = gen.to_device(inp, dev)
    if inp.ns == 0:
        t["sink_k"] = t["sink_v"] = None
    return t


def rotating(torch, base: dict, max_sets: int = 32):
    """(copies of the tensors in `base`, at distinct addresses, that together hold at least
    ROTATE_BYTES; their count; their bytes)."""
    nbytes = sum(v.numel() * v.element_size() for v in base.values()
                 if isinstance(v, torch.Tensor))
    n = max(1, min(max_sets, -(-ROTATE_BYTES // nbytes)))
    sets = [base] + [{k: (v.clone() if isinstance(v, torch.Tensor) else v)
                      for k, v in base.items()} for _ in range(n - 1)]
    return sets, n, n * nbytes


def cache_label(n, nbytes):
    return f"rotating ({n} input sets, {nbytes / 1e6:.0f} MB)"


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


# ── host description ──────────────────────────────────────────────────────────────────────────

def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def gpu_clocks():
    """Current clock levels of card 0 as rocm-smi reports them (sclk, mclk, fclk, ...)."""
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True,
                           text=True, timeout=30)
        d = json.loads(r.stdout)
        card = d.get("card0") or next(iter(d.values()))
        return {k.rstrip(":").strip(): v for k, v in card.items()}
    except Exception as e:   # a missing tool must not cost the measurement
        return {"error": f"rocm-smi: {type(e).__name__}: {str(e)[:160]}"}


# ── CPU oracle timings (test infrastructure, timed beside the GPU numbers) ─────────────────

def time_oracle(fn, budget_s=ORACLE_BUDGET_S, max_runs=3):
    """(median seconds per run, runs): up to max_runs runs, fewer once budget_s is spent."""
    times = []
    for _ in range(max_runs):
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
        if sum(times) >= budget_s:
            break
    return statistics.median(times), len(times)


def oracle_entry(sec, runs, sample, scale=1.0, **units):
    """One cpu_oracle record: seconds per call of the full workload (the sample's time times
    `scale`), and each unit's value from `units` (name -> work per call, in that unit times
    seconds)."""
    import oracle
    per = sec * scale
    rec = {"ms": round(per * 1e3, 3), "cores": oracle.threads(), "runs": runs,
           "kind": "oracle (f64 accumulation)", "sample": sample}
    for name, work in units.items():
        rec[name] = round(work / per, 4)
    return rec


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
    return {"value": round(acct.unique_kv_bytes(inp) / per / 1e9, 4), "unit": "GB/s",
            "cores": oracle.threads(), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{n} full decode calls (f64 accumulation), {el:.1f} s wall, "
                      f"{per * 1e3:.3f} ms per call"}


# ── decode (the headline) and the plain-read leg ─────────────────────────────────────────────

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
    clocks = gpu_clocks()
    kv = acct.unique_kv_bytes(inp)
    tot = acct.total_bytes(inp)
    set_bytes = sum(v.numel() * v.element_size() for v in base.values() if v is not None)
    return inp, ms, ev_mean, ev_med, kv, tot, set_bytes, clocks


def bench_read(args, torch, B, nbytes):
    """Plain streaming reads timed like the decode call: `args.sets` buffers of `nbytes`
    (rounded up to 16) read in rotation, and one 1 GiB buffer read again and again (the
    steady-state rate, where launch costs vanish)."""
    dev = "cuda:0"
    n = -(-nbytes // 16) * 4
    bufs = [torch.empty(n, dtype=torch.float32, device=dev).normal_() for _ in range(args.sets)]
    sink = torch.zeros(256, dtype=torch.float32, device=dev)
    ms, _, _ = time_calls(torch, lambda i: B.read_probe(bufs[i], sink), args.sets, args.steps,
                          args.warmup)
    del bufs
    big = torch.empty(1 << 28, dtype=torch.float32, device=dev).normal_()
    ms_big, _, _ = time_calls(torch, lambda i: B.read_probe(big, sink), 1, 20, 3)
    del big
    torch.cuda.empty_cache()
    return n * 4, ms, ms_big


# ── the other workloads ──────────────────────────────────────────────────────────────────────

def bench_chunk_workload(name, inp, torch, B, acct, steps, oracle_scale_runs=3):
    """One chunk workload: GPU time on rotating inputs, and the oracle on the same inputs."""
    import oracle
    dev = "cuda:0"
    base = chunk_tensors(inp, torch, dev)
    base["out"] = torch.empty((inp.rows, inp.nh, inp.d), dtype=torch.float32, device=dev)
    sets, n, nbytes = rotating(torch, base)
    ws = B.Workspace(dev)
    ws.get(B.chunk_workspace_bytes(inp.rows, inp.ng, inp.hpg, inp.d, inp.w, inp.ns))
    ms, _, _ = time_calls(torch, lambda i: run_chunk(B, sets[i], inp.scale, sets[i]["out"], ws),
                          n, steps, 3)
    flops = acct.chunk_flops(inp)
    kv = acct.unique_kv_bytes(inp)
    kern = B.chunk_plan(inp.rows, inp.ng, inp.hpg, inp.d, inp.w, inp.ns)
    rec = {"ms": round(ms, 5), "kv_gbs": round(kv / ms / 1e6, 2),
           "hbm_frac": round(acct.total_bytes(inp) / ms / 1e6 / HBM_PEAK_GBS, 4),
           "rows_per_s": round(inp.rows / ms * 1e3, 1),
           "tflops": round(flops / ms / 1e9, 3),
           "tflops_frac_f32_peak": round(flops / ms / 1e9 / F32_PEAK_TFLOPS, 4),
           "kernel": KERNEL_NAMES[kern[0]], "splits": kern[2], "keys_per_split": kern[3],
           "cache": cache_label(n, nbytes)}
    del sets, base, ws
    torch.cuda.empty_cache()
    sec, runs = time_oracle(lambda: oracle.window_chunk(inp), max_runs=oracle_scale_runs)
    rec["cpu_oracle"] = oracle_entry(sec, runs, f"the full {name} call", kv_gbs=kv / 1e9,
                                     rows_per_s=inp.rows, tflops=flops / 1e12)
    return rec


def bench_others(args, torch, B, gen, acct):
    import oracle
    dev = "cuda:0"
    res = {}
    for name, make, steps in (("tiny", gen.tiny, 50), ("prefill", gen.prefill, 20),
                              ("large", gen.large, 5), ("decode_w32768", gen.decode_long, 60)):
        res[name] = bench_chunk_workload(name, make(), torch, B, acct, steps)
    for name, rows in (("decode_far_m32", 1), ("chunk64_far_m32", 64)):
        # the decode shapes with a far field of 32 landmarks per head in every group (full
        # rings, so every row evicts); the near-only call on the same inputs is timed beside it
        inp = gen.make_chunk(rows, 8, 4, 128, 4096, 4, gen.decode().meta.copy(), seed=7)
        inp.meta[:, 2] = 1000
        far = gen.make_far(inp, 32, seed=8)
        base = chunk_tensors(inp, torch, dev)
        base.update({"far_" + k: v for k, v in gen.to_device(far, dev).items()})
        base["out"] = torch.empty((inp.rows, inp.nh, inp.d), dtype=torch.float32, device=dev)
        sets, n, nbytes = rotating(torch, base)
        ws = B.Workspace(dev)
        ws.get(B.chunk_far_workspace_bytes(inp.rows, inp.ng, inp.hpg, inp.d, inp.w, inp.ns, 32))

        def far_call(i):
            t = sets[i]
            B.attn_window_chunk_far(t["ring_k"], t["ring_v"], t["meta"], t["sink_k"],
                                    t["sink_v"], t["q"], t["chunk_k"], t["chunk_v"],
                                    t["far_k_tilde"], t["far_q_tilde"], t["far_mu"], t["far_mz"],
                                    t["far_t_hat"], inp.scale, out=t["out"], workspace=ws)
        ms, _, _ = time_calls(torch, far_call, n, 20, 3)
        near_ms, _, _ = time_calls(
            torch, lambda i: run_chunk(B, sets[i], inp.scale, sets[i]["out"], ws), n, 20, 3)
        kv = acct.unique_kv_bytes(inp)
        res[name] = {"ms": round(ms, 5), "near_only_ms": round(near_ms, 5),
                     "kv_gbs": round(kv / ms / 1e6, 2),
                     "rows_per_s": round(inp.rows / ms * 1e3, 1), "landmarks": 32,
                     "cache": cache_label(n, nbytes)}
        del sets, base, ws
        torch.cuda.empty_cache()
        sec, runs = time_oracle(lambda: oracle.window_chunk_far(inp, far))
        res[name]["cpu_oracle"] = oracle_entry(sec, runs, f"the full {name} call",
                                               kv_gbs=kv / 1e9, rows_per_s=inp.rows)
    # the gated one-row call with 32 landmarks per head, at the gated workload's head shapes
    # (16 query / 4 KV heads, hd 256, full 1024-slot rings); the same call with every far
    # count 0 (far part skipped) is timed beside it
    gf = gen.make_gated_far(16, 4, 256, 1024, 0, 32, [(1024, 0, 5000, 0)] * 4, seed=9,
                            scale=1 / 16)
    base = gen.to_device(gf, dev)
    base["out"] = torch.empty((16, 256), dtype=torch.float32, device=dev)
    base["empty_meta"] = base["meta"].clone()
    base["empty_meta"][:, 2] = 0
    sets, n, nbytes = rotating(torch, base)
    ws = B.Workspace(dev)

    def gated_far_call(i, meta_key):
        t = sets[i]
        B.attn_window_gated_far(t["q"], t["ring_k"], t["ring_v"], t[meta_key], None, None,
                                t["k_tilde"], t["mu"], t["mz"], t["t_hat"], t["gate"],
                                t["gate_scale"], gf.scale, out=t["out"], workspace=ws)
    ms, _, _ = time_calls(torch, lambda i: gated_far_call(i, "meta"), n, 20, 3)
    near_ms, _, _ = time_calls(torch, lambda i: gated_far_call(i, "empty_meta"), n, 20, 3)
    kv = 4 * 1024 * 256 * 8
    res["gated_far_m32"] = {"ms": round(ms, 5), "far_empty_ms": round(near_ms, 5),
                            "kv_gbs": round(kv / ms / 1e6, 2), "landmarks": 32,
                            "cache": cache_label(n, nbytes)}
    del sets, base, ws
    torch.cuda.empty_cache()
    sec, runs = time_oracle(lambda: oracle.window_gated_far(gf))
    res["gated_far_m32"]["cpu_oracle"] = oracle_entry(sec, runs, "the full call", kv_gbs=kv / 1e9)
    # encoder attention: one 9801-position sequence with 16 heads of 64 and no window (the
    # vision tower's shape), and 16 packed sequences of seeded lengths U[64, 1024] with 16
    # query / 4 KV heads of 64 and a symmetric window of 128
    rng = np.random.default_rng(11)
    for name, lens, nh, nk, win in (
            ("encoder_full_9801", [9801], 16, 16, 0),
            ("encoder_varlen_window128", [int(x) for x in rng.integers(64, 1025, size=16)], 16, 4, 128)):
        e = gen.make_encoder(lens, nh, nk, 64, win, seed=12)
        base = {"q": torch.from_numpy(e.q).to(dev), "k": torch.from_numpy(e.k).to(dev),
                "v": torch.from_numpy(e.v).to(dev),
                "segs": torch.from_numpy(e.segs.view(np.int32).copy()).to(dev),
                "out": torch.empty((e.q.shape[0], nh * 64), dtype=torch.float32, device=dev)}
        sets, n, nbytes = rotating(torch, base)
        mx = max(lens)

        def enc_call(i):
            t = sets[i]
            B.attn_encoder(t["q"], t["k"], t["v"], t["segs"], nh, nk, 64, e.scale, window=win,
                           max_len=mx, out=t["out"])
        ms, _, _ = time_calls(torch, enc_call, n, 5 if name.endswith("9801") else 20, 2)
        flops = acct.encoder_flops(e)
        res[name] = {"ms": round(ms, 5), "tflops": round(flops / ms / 1e9, 3),
                     "tflops_frac_f32_peak": round(flops / ms / 1e9 / F32_PEAK_TFLOPS, 4),
                     "tokens": int(sum(lens)), "kernel": "enc_attn_kernel",
                     "cache": cache_label(n, nbytes)}
        del sets, base
        torch.cuda.empty_cache()
        if name.endswith("9801"):
            # bounded sample: 2 of the 16 heads (heads are independent; time scaled by 8)
            es = gen.make_encoder(lens, 2, 2, 64, win, seed=12)
            sec, runs = time_oracle(lambda: oracle.encoder_attention(es), max_runs=1)
            res[name]["cpu_oracle"] = oracle_entry(sec, runs, "2 of the 16 heads, time x 8",
                                                   scale=8.0, tflops=flops / 1e12)
        else:
            sec, runs = time_oracle(lambda: oracle.encoder_attention(e))
            res[name]["cpu_oracle"] = oracle_entry(sec, runs, "the full call",
                                                   tflops=flops / 1e12)
    g = gen.gated()
    base = gen.to_device(g, dev)
    base["out"] = torch.empty((g.rows, g.nh, g.hd), dtype=torch.float32, device=dev)
    sets, n, nbytes = rotating(torch, base)

    def gated_call(i):
        t = sets[i]
        B.attn_window_gated(t["yq"], t["yk"], t["yv"], t["rope"], t["q_scale"], t["gate"],
                            t["gate_scale"], t["ring_k"], t["ring_v"], g.pos0, g.window, g.scale,
                            g.eps, out=t["out"])
    ms, _, _ = time_calls(torch, gated_call, n, 20, 3)
    kv, tot, flops = acct.gated_counts(g)
    res["gated"] = {"ms": round(ms, 5), "kv_gbs": round(kv / ms / 1e6, 2),
                    "hbm_frac": round(tot / ms / 1e6 / HBM_PEAK_GBS, 4),
                    "rows_per_s": round(g.rows / ms * 1e3, 1),
                    "tflops": round(flops / ms / 1e9, 3),
                    "tflops_frac_f32_peak": round(flops / ms / 1e9 / F32_PEAK_TFLOPS, 4),
                    # width 256 and 256 query vectors per KV head: the single-launch plan
                    "kernel": "attn_gated_tiles_kernel",
                    "workspace_bytes": B.gated_workspace_bytes(g.rows, g.nh, g.nk, g.hd, g.window),
                    "cache": cache_label(n, nbytes)}
    del sets, base
    torch.cuda.empty_cache()
    sec, runs = time_oracle(lambda: oracle.window_gated(g))
    res["gated"]["cpu_oracle"] = oracle_entry(sec, runs, "the full gated call", kv_gbs=kv / 1e9,
                                              rows_per_s=g.rows, tflops=flops / 1e12)
    return res


def counter_run(args, torch, B, gen):
    """A short, untimed run for hardware-counter passes: one device-to-device copy of
    CALIBRATION_COPY_BYTES (reads and writes exactly that many bytes), then `calls` calls of one
    workload on rotating input sets, as the timed runs make them."""
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
    inp, ms, ev_mean, ev_med, kv, tot, set_bytes, clocks = bench_decode(args, torch, B, gen, acct)
    read_bytes, read_ms, read_big_ms = bench_read(args, torch, B, tot)
    achieved = tot / (ms * 1e-3) / 1e9
    read_gbs = read_bytes / (read_ms * 1e-3) / 1e9
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
        "hbm_frac": round(achieved / HBM_PEAK_GBS, 4),
        # One launch = one attn_window_chunk call, timed by the HIP events that bracket the
        # timed loop on the library's stream.
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "one attn_window_chunk call (all its launches)",
            "algorithmic_bytes_per_launch": tot,
            "launch_ms_mean": round(ms, 6),
            "per_call_event_ms_mean": round(ev_mean, 6),
            "per_call_event_ms_median": round(ev_med, 6),
            # a plain streaming read of the same bytes, timed the same way in this run
            "achievable_gbs": round(read_gbs, 2),
            "achievable_ms": round(read_ms, 6),
            "frac_of_achievable": round(achieved / read_gbs, 4),
            "read_1gib_gbs": round((1 << 30) / (read_big_ms * 1e-3) / 1e9, 2),
        },
        "gpu_clocks": clocks,
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    if not args.no_others:
        line["also"] = bench_others(args, torch, B, gen, acct)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
