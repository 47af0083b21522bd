"""Phase timing of the single-launch decode and gated kernels from in-kernel clock stamps.

    python -m sliding_window_gqa_group_amd.phase_stamps build             # any host: compiles
    python -m sliding_window_gqa_group_amd.phase_stamps run [calls]       # GPU: decode table
    python -m sliding_window_gqa_group_amd.phase_stamps gated [calls]     # GPU: gated table
    python -m sliding_window_gqa_group_amd.phase_stamps clock [calls]     # GPU: prefill/large clock

`build` compiles the library a second time with WINATTN_PHASE_STAMPS defined, into
libwinattn_stamps.so beside the normal one (the normal library has no stamp code). `run` loads
that library instead of the normal one and makes decode calls (1 row, 8 KV groups x 4 query
heads, d 128, full 4096-slot rings, 4 sinks) on 20 rotating input sets. Each recorded call is
the last of 8 back-to-back calls, as in the bench's timed loop; every wave of it wrote the
100 MHz real-time counter at its phase boundaries. The report gives, per phase, the spread over
all waves of the recorded calls of the time since the call's first wave started. `gated` does
the same for the gated workload's single launch (64 rows at pos0 20000, 16 query heads over 4
KV heads, hd 256, window 1024) on its rotating input sets, and reports the shader clock the waves
ran at (the shader-clock counter over the real-time counter). `clock` reports that clock for the
32x32 matrix-core kernel on the prefill and large workloads (one reading per workgroup).
"""
from __future__ import annotations

import ctypes
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
STAMPS_LIB = os.path.join(HERE, "libwinattn_stamps.so")
STAMPS_OBJDIR = os.path.join(HERE, "_build_stamps")
WORDS = 10   # u64 per wave: 9 phase stamps, then the XCD number
PHASES = [
    ("start", "the wave starts"),
    ("meta", "the group's metadata has arrived (every K/V load of the split is in flight)"),
    ("tile0", "the first ring tile's scores, softmax and value update are done"),
    ("tiles", "every ring tile is done"),
    ("merged", "lane groups and waves merged into LDS"),
    ("issued", "partial stores issued"),
    ("acked", "partial stores acknowledged device-wide"),
    ("flagged", "ready flags raised (waves of non-gathering splits end here)"),
    ("gathered", "a gatherer's column chunk folded and stored (gatherers only)"),
]


def build() -> str:
    sys.path.insert(0, os.path.dirname(HERE))
    from sliding_window_gqa_group_amd import build as b
    return b.build(defines=("WINATTN_PHASE_STAMPS",), lib=STAMPS_LIB, objdir=STAMPS_OBJDIR)


def run(calls: int = 10) -> str:
    sys.path.insert(0, os.path.dirname(HERE))
    import numpy as np
    import torch
    from sliding_window_gqa_group_amd import binding as B, inputs as gen

    lib = B.load(STAMPS_LIB)   # every binding call below goes to the timing build
    lib.attn_phase_stamps_set.argtypes = [ctypes.c_void_p]
    lib.attn_phase_stamps_set.restype = ctypes.c_int
    dev = "cuda:0"
    inp = gen.decode()
    base = gen.to_device(inp, dev)
    nsets = 20
    sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(nsets - 1)]
    outs = [torch.empty((inp.rows, inp.nh, inp.d), dtype=torch.float32, device=dev)
            for _ in range(nsets)]
    plan = B.chunk_plan(inp.rows, inp.ng, inp.hpg, inp.d, inp.w, inp.ns)
    nsplit = plan[2]
    waves = inp.ng * nsplit * 4
    ws = B.Workspace(dev)
    ws.get(B.chunk_workspace_bytes(inp.rows, inp.ng, inp.hpg, inp.d, inp.w, inp.ns))
    stamps = torch.zeros(waves * WORDS, dtype=torch.int64, device=dev)

    def call(i):
        t = sets[i % nsets]
        B.attn_window_chunk(t["ring_k"], t["ring_v"], t["meta"], t["sink_k"], t["sink_v"], t["q"],
                            t["chunk_k"], t["chunk_v"], inp.scale, out=outs[i % nsets], workspace=ws)

    def set_ptr(ptr):
        torch.cuda.synchronize()
        if lib.attn_phase_stamps_set(ctypes.c_void_p(ptr)) != 0:
            raise RuntimeError("attn_phase_stamps_set failed")
        torch.cuda.synchronize()

    set_ptr(0)
    print(f"plan {tuple(plan)}: warming up", file=sys.stderr, flush=True)
    for i in range(200):   # untimed: clocks up, code and buffers touched
        call(i)
    rel = [[] for _ in PHASES]
    ends = []
    xcd = np.zeros(8, dtype=np.int64)
    for r in range(calls):
        stamps.zero_()
        set_ptr(stamps.data_ptr())
        for i in range(8):
            call(r * 8 + i)
        set_ptr(0)
        t = stamps.cpu().numpy().reshape(waves, WORDS)
        if (t[:, 0] == 0).any():
            raise RuntimeError("a wave wrote no stamps")
        t0 = t[:, 0].min()
        for k in range(len(PHASES)):
            col = t[:, k]
            rel[k].append((col[col != 0] - t0) * 0.01)
        last = np.where(t[:, 8] != 0, t[:, 8], t[:, 7])
        last = np.where(last != 0, last, t[:, 5])
        ends.append((last.max() - t0) * 0.01)
        xcd += np.bincount((t[:, 9] & 0xF).astype(np.int64), minlength=8)[:8]
        print(f"recorded call {r + 1} of {calls}", file=sys.stderr, flush=True)

    lines = [f"Decode call: plan (kernel, queries per block, splits, keys per split) = {tuple(plan)}, "
             f"{inp.ng * nsplit} workgroups of 4 waves; {calls} recorded calls, each the last of 8 "
             "back-to-back calls on 20 rotating input sets. Times in us since the call's first "
             "wave started (100 MHz counter), over every wave that reached the phase.",
             "",
             "| phase | waves | min | p10 | p50 | p90 | max | meaning |",
             "|---|---|---|---|---|---|---|---|"]
    for k, (name, meaning) in enumerate(PHASES):
        v = np.concatenate(rel[k])
        lines.append(f"| {name} | {len(v)} | {v.min():.2f} | {np.percentile(v, 10):.2f} | "
                     f"{np.median(v):.2f} | {np.percentile(v, 90):.2f} | {v.max():.2f} | {meaning} |")
    e = np.array(ends)
    lines += ["", f"First wave start to last wave end: median {np.median(e):.2f} us "
              f"(min {e.min():.2f}, max {e.max():.2f}).",
              "Waves per XCD (hardware register XCC_ID): " + ", ".join(str(int(x)) for x in xcd) + "."]
    return "\n".join(lines)


GATED_WORDS = 14   # u64 per wave: 11 phase stamps, the XCD number, the shader clock at start and end
GATED_PHASES = [
    ("start", "the wave starts"),
    ("queries", "the block's unit queries are in the wave's registers (tile 0 requested)"),
    ("tile0 in", "tile 0 is in LDS (first barrier of the loop)"),
    ("tile0 done", "the wave's half of tile 0: scores, softmax, value products"),
    ("tile1 in", "tile 1 is in LDS"),
    ("tile1 done", "the wave's half of tile 1"),
    ("tiles", "every tile of the split is done"),
    ("folded", "the two key halves of each query set folded in LDS"),
    ("flagged", "partials stored, acknowledged, flags raised (non-gatherers end here)"),
    ("flags seen", "a gatherer has seen every split's flag (partials requested as seen)"),
    ("end", "a gatherer's outputs stored and drained"),
]


def run_gated(calls: int = 10) -> str:
    sys.path.insert(0, os.path.dirname(HERE))
    import numpy as np
    import torch
    from sliding_window_gqa_group_amd import binding as B, inputs as gen

    lib = B.load(STAMPS_LIB)   # every binding call below goes to the timing build
    lib.attn_gated_stamps_set.argtypes = [ctypes.c_void_p]
    lib.attn_gated_stamps_set.restype = ctypes.c_int
    dev = "cuda:0"
    g = gen.gated()
    base = gen.to_device(g, dev)
    nsets = 5   # 5 copies of the inputs (about 350 MB): each call reads its window from HBM
    sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(nsets - 1)]
    out = torch.empty((g.rows, g.nh, g.hd), dtype=torch.float32, device=dev)
    ws = B.Workspace(dev)
    max_blocks = 4096
    stamps = torch.zeros(max_blocks * 8 * GATED_WORDS, dtype=torch.int64, device=dev)
    nqs = -(-g.rows * (g.nh // g.nk) // 64)
    per_split = g.nk * nqs                   # workgroups per split index

    def call(i):
        t = sets[i % nsets]
        B.attn_window_gated(t["yq"], t["yk"], t["yv"], t["rope"], t["q_scale"], t["gate"],
                            t["gate_scale"], t["ring_k"], t["ring_v"], g.pos0, g.window, g.scale,
                            g.eps, out=out, workspace=ws)

    def set_ptr(ptr):
        torch.cuda.synchronize()
        if lib.attn_gated_stamps_set(ctypes.c_void_p(ptr)) != 0:
            raise RuntimeError("attn_gated_stamps_set failed")
        torch.cuda.synchronize()

    set_ptr(0)
    print("gated: warming up", file=sys.stderr, flush=True)
    for i in range(200):
        call(i)
    groups = {"all waves": [], "split 0": [], "last split": []}
    rel = {k: [[] for _ in GATED_PHASES] for k in groups}
    ends, nsplit, clocks = [], 0, []
    for r in range(calls):
        stamps.zero_()
        set_ptr(stamps.data_ptr())
        for i in range(8):
            call(r * 8 + i)
        set_ptr(0)
        t = stamps.cpu().numpy().reshape(max_blocks * 8, GATED_WORDS)
        live = t[:, 0] != 0
        waves = np.nonzero(live)[0]
        split = (waves // 8) // per_split
        nsplit = int(split.max()) + 1
        t = t[live]
        t0 = t[:, 0].min()
        # shader clock of each wave: clock cycles over real time from its start to its last stamp
        last = t[:, :11].max(axis=1)
        dt = (last - t[:, 0]) * 1e-8
        clocks.append(((t[:, 13] - t[:, 12]) / np.where(dt > 0, dt, np.nan)) * 1e-9)
        sel = {"all waves": np.ones(len(t), bool), "split 0": split == 0,
               "last split": split == nsplit - 1}
        for name, m in sel.items():
            for k in range(len(GATED_PHASES)):
                col = t[m, k]
                rel[name][k].append((col[col != 0] - t0) * 0.01)
        ends.append((t[:, :11].max() - t0) * 0.01)
        print(f"recorded call {r + 1} of {calls}", file=sys.stderr, flush=True)

    lines = [f"Gated call: {per_split * nsplit} workgroups of 8 waves ({nsplit} splits of each of "
             f"{per_split} query blocks); {calls} recorded calls, each the last of 8 back-to-back "
             f"calls on {nsets} rotating input sets. Times in us since the call's first wave "
             "started (100 MHz counter), medians over the waves of each group that reached the "
             "phase (split 0 holds the largest share of key blocks; the last split also makes "
             "the chunk rows' unit keys and gathers).",
             "",
             "| phase | waves | min | p50 all | p90 all | max | p50 split 0 | p50 last split | meaning |",
             "|---|---|---|---|---|---|---|---|---|"]
    for k, (name, meaning) in enumerate(GATED_PHASES):
        v = np.concatenate(rel["all waves"][k])
        if len(v) == 0:
            continue
        s0 = np.concatenate(rel["split 0"][k])
        sl = np.concatenate(rel["last split"][k])
        f = lambda a: f"{np.median(a):.2f}" if len(a) else "—"
        lines.append(f"| {name} | {len(v)} | {v.min():.2f} | {np.median(v):.2f} | "
                     f"{np.percentile(v, 90):.2f} | {v.max():.2f} | {f(s0)} | {f(sl)} | {meaning} |")
    e = np.array(ends)
    c = np.concatenate(clocks)
    c = c[np.isfinite(c)]
    lines += ["", f"First wave start to last stamp: median {np.median(e):.2f} us "
              f"(min {e.min():.2f}, max {e.max():.2f}).",
              f"Shader clock over each wave's life (shader-clock counter over the 100 MHz counter): "
              f"median {np.median(c):.3f} GHz (p10 {np.percentile(c, 10):.3f}, p90 {np.percentile(c, 90):.3f})."]
    return "\n".join(lines)


def run_clock(calls: int = 5) -> str:
    """The shader clock while the 32x32 matrix-core kernel runs the prefill and large workloads."""
    sys.path.insert(0, os.path.dirname(HERE))
    import numpy as np
    import torch
    from sliding_window_gqa_group_amd import binding as B, inputs as gen

    lib = B.load(STAMPS_LIB)
    lib.attn_mfma_clock_set.argtypes = [ctypes.c_void_p]
    lib.attn_mfma_clock_set.restype = ctypes.c_int
    dev = "cuda:0"
    ws = B.Workspace(dev)
    buf = torch.zeros(65536 * 4, dtype=torch.int64, device=dev)

    def set_ptr(ptr):
        torch.cuda.synchronize()
        if lib.attn_mfma_clock_set(ctypes.c_void_p(ptr)) != 0:
            raise RuntimeError("attn_mfma_clock_set failed")
        torch.cuda.synchronize()

    lines = ["| workload | workgroups | median clock | p10 | p90 | median workgroup life |",
             "|---|---|---|---|---|---|"]
    for name, inp, warm in (("prefill", gen.prefill(), 50), ("large", gen.large(), 3)):
        base = gen.to_device(inp, dev)
        sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(1 if name == "large" else 4)]
        out = torch.empty((inp.rows, inp.nh, inp.d), dtype=torch.float32, device=dev)

        def call(i):
            t = sets[i % len(sets)]
            B.attn_window_chunk(t["ring_k"], t["ring_v"], t["meta"], t["sink_k"], t["sink_v"],
                                t["q"], t["chunk_k"], t["chunk_v"], inp.scale, out=out, workspace=ws)

        set_ptr(0)
        for i in range(warm):
            call(i)
        cs, lives = [], []
        for r in range(calls):
            buf.zero_()
            set_ptr(buf.data_ptr())
            call(r)
            set_ptr(0)
            t = buf.cpu().numpy().reshape(-1, 4)
            t = t[t[:, 0] != 0]
            dt = (t[:, 2] - t[:, 0]) * 1e-8
            ok = dt > 0
            cs.append((t[ok, 3] - t[ok, 1]) / dt[ok] * 1e-9)
            lives.append(dt[ok] * 1e6)
        c, lv = np.concatenate(cs), np.concatenate(lives)
        lines.append(f"| {name} | {len(c) // calls} | {np.median(c):.3f} GHz | {np.percentile(c, 10):.3f} | "
                     f"{np.percentile(c, 90):.3f} | {np.median(lv):.1f} us |")
        print(f"clock: {name} done", file=sys.stderr, flush=True)
        del sets, base
        torch.cuda.empty_cache()
    return "\n".join(lines)


if __name__ == "__main__":
    if len(sys.argv) < 2 or sys.argv[1] not in ("build", "run", "gated", "clock"):
        raise SystemExit(__doc__)
    n = int(sys.argv[2]) if len(sys.argv) > 2 else None
    if sys.argv[1] == "build":
        print(build())
    elif sys.argv[1] == "run":
        print(run(n or 10))
    elif sys.argv[1] == "gated":
        print(run_gated(n or 10))
    else:
        print(run_clock(n or 5))
