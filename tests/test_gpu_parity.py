"""Parity of the HIP path (through the C-ABI) with the CPU oracle, on seeded synthetic inputs.

Bar (per element): |gpu - oracle| <= max(1e-4 * |oracle|, 1e-5). The named workloads run at
their full sizes in the launch plan the benchmark uses, and every output is compared.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
from sliding_window_gqa_group_amd import binding as B
from sliding_window_gqa_group_amd import inputs as gen

pytestmark = pytest.mark.gpu

RTOL, ATOL = 1e-4, 1e-5
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()   # fail loudly if the HIP library is missing
    yield
    for knob in (B.TUNE_FORCE_KERNEL, B.TUNE_TILES_PER_SPLIT, B.TUNE_TARGET_BLOCKS,
                 B.TUNE_MERGE_KERNEL, B.TUNE_XCD_MAP):
        B.tuning_set(knob, 0)


def assert_close(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = np.maximum(RTOL * np.abs(ref), ATOL)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err / bound), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements out of tolerance; worst at "
                             f"{i}: gpu {got[i]!r} oracle {ref[i]!r}")


def gpu_chunk(inp, out=None, workspace=None):
    t = gen.to_device(inp, DEV)
    ns = inp.ns
    res = B.attn_window_chunk(t["ring_k"], t["ring_v"], t["meta"],
                              t["sink_k"] if ns else None, t["sink_v"] if ns else None,
                              t["q"], t["chunk_k"], t["chunk_v"], inp.scale, out=out,
                              workspace=workspace)
    torch.cuda.synchronize()
    return res


def gpu_gated(inp):
    t = gen.to_device(inp, DEV)
    z = B.attn_window_gated(t["yq"], t["yk"], t["yv"], t["rope"], t["q_scale"], t["gate"],
                            t["gate_scale"], t["ring_k"], t["ring_v"], inp.pos0, inp.window,
                            inp.scale, inp.eps)
    torch.cuda.synchronize()
    return z.cpu().numpy(), t["ring_k"].cpu().numpy(), t["ring_v"].cpu().numpy()


def _case(name):
    print(f"[case] {name}", flush=True)


# ── the matrix-core operand layout the wide-chunk kernel relies on ────────────────────────────

def test_mfma_layout_probe():
    _case("mfma layout probe")
    out = B.mfma_layout_probe(DEV).cpu().numpy()
    for lane in range(64):
        for r in range(16):
            i = 8 * (r // 4) + 4 * (lane // 32) + r % 4
            j = lane % 32
            assert out[lane, r] == i + 64 * j, (lane, r, out[lane, r])


def test_mfma16_layout_probe():
    _case("mfma16 layout probe")
    out = B.mfma16_layout_probe(DEV).cpu().numpy()
    for lane in range(64):
        for r in range(4):
            i = 4 * (lane // 16) + r
            j = lane % 16
            assert out[lane, r] == i + 64 * j, (lane, r, out[lane, r])


# ── the named workloads ──────────────────────────────────────────────────────────────────────

def test_tiny():
    _case("tiny")
    inp = gen.tiny()
    assert_close(gpu_chunk(inp).cpu().numpy(), oracle.window_chunk(inp), "tiny")


def test_decode():
    _case("decode")
    inp = gen.decode()
    assert_close(gpu_chunk(inp).cpu().numpy(), oracle.window_chunk(inp), "decode")


def test_decode_long_window():
    """Decode over a 32768-slot full ring (the register kernel's loop instance, 16 tiles per
    split), and the same row over the large workload's per-group overrides and partial rings."""
    _case("decode, w = 32768")
    inp = gen.decode_long()
    assert_close(gpu_chunk(inp).cpu().numpy(), oracle.window_chunk(inp), "decode w=32768")
    _, meta = gen.large_meta(seed=6)
    inp = gen.make_chunk(1, 8, 4, 128, 32768, 4, meta, seed=6)
    assert_close(gpu_chunk(inp).cpu().numpy(), oracle.window_chunk(inp), "decode, overrides")


def test_prefill():
    """Every output of the 512-row chunk (the 32x32 matrix-core kernel at its benchmark plan)."""
    _case("prefill")
    inp = gen.prefill()
    assert_close(gpu_chunk(inp).cpu().numpy(), oracle.window_chunk(inp), "prefill")


def test_large():
    """Every output of the 2048-row chunk over 32768-slot rings with per-group overrides and
    partial rings (the paths that only run at full size: long windows, the split caps, the
    round-robin work order). The oracle needs about 30 s of one host's cores here."""
    _case("large")
    inp = gen.large()
    got = gpu_chunk(inp).cpu().numpy()
    assert_close(got, oracle.window_chunk(inp), "large")


def test_gated():
    _case("gated")
    inp = gen.gated()
    z, rk, rv = gpu_gated(inp)
    oz, ork, orv = oracle.window_gated(inp)
    assert_close(z, oz, "gated z")
    assert_close(rk, ork, "gated ring k")
    np.testing.assert_array_equal(rv, orv)


# ── shape sweep over both kernels and forced multi-split merges ──────────────────────────────

def _rand_meta(rng, ng, w, kind):
    meta = []
    for g in range(ng):
        k = kind if kind != "mix" else ["full", "partial", "empty", "override"][g % 4]
        if k == "full":
            meta.append((w, int(rng.integers(0, w)), 0, 0))
        elif k == "partial":
            meta.append((int(rng.integers(1, w)), int(rng.integers(0, w)), 0, 0))
        elif k == "empty":
            meta.append((0, int(rng.integers(0, w)), 0, 0))
        else:
            ov = int(rng.integers(1, w + 1))
            meta.append((int(rng.integers(0, ov + 1)), int(rng.integers(0, ov)), 0, ov))
    return meta


SWEEP = [
    # rows, ng, hpg, d, w, ns, meta kind
    (1, 2, 1, 64, 40, 0, "full"),
    (1, 3, 4, 128, 300, 4, "mix"),
    (2, 1, 2, 128, 70, 4, "partial"),
    (4, 2, 4, 256, 90, 4, "mix"),
    (15, 2, 4, 64, 33, 3, "full"),
    (16, 1, 8, 128, 100, 0, "override"),
    (17, 3, 4, 256, 50, 4, "mix"),
    (64, 2, 4, 128, 200, 4, "full"),
    (513, 1, 4, 64, 90, 2, "mix"),
    (33, 2, 1, 36, 60, 1, "partial"),
    (5, 1, 3, 100, 20, 2, "mix"),
    (40, 1, 32, 64, 64, 0, "full"),
    (130, 4, 2, 128, 129, 5, "mix"),
]

VARIANTS = {
    "auto": {},
    "register_many_splits": {B.TUNE_FORCE_KERNEL: 1, B.TUNE_TILES_PER_SPLIT: 1},
    "mfma_many_splits": {B.TUNE_FORCE_KERNEL: 2, B.TUNE_TILES_PER_SPLIT: 1},
    "lds_vector_many_splits": {B.TUNE_FORCE_KERNEL: 3, B.TUNE_TILES_PER_SPLIT: 1},
    "register_merge_launch": {B.TUNE_FORCE_KERNEL: 1, B.TUNE_TILES_PER_SPLIT: 1,
                              B.TUNE_MERGE_KERNEL: 2},
    "mfma_merge_launch": {B.TUNE_FORCE_KERNEL: 2, B.TUNE_TILES_PER_SPLIT: 1,
                          B.TUNE_MERGE_KERNEL: 2},
    "mfma_in_kernel_merge_other_order": {B.TUNE_FORCE_KERNEL: 2, B.TUNE_TILES_PER_SPLIT: 2,
                                         B.TUNE_MERGE_KERNEL: 1, B.TUNE_XCD_MAP: 2},
    "mfma16_many_splits": {B.TUNE_FORCE_KERNEL: 4, B.TUNE_TILES_PER_SPLIT: 1},
    # the single-launch slot-order kernel (shapes of at most 8 query vectors per group)
    "slot_order_one_tile": {B.TUNE_FORCE_KERNEL: 5, B.TUNE_TILES_PER_SPLIT: 1},
    "slot_order_four_tiles": {B.TUNE_FORCE_KERNEL: 5, B.TUNE_TILES_PER_SPLIT: 4},
    "mfma16_one_split_in_kernel_merge": {B.TUNE_FORCE_KERNEL: 4, B.TUNE_TILES_PER_SPLIT: 3,
                                         B.TUNE_MERGE_KERNEL: 1, B.TUNE_XCD_MAP: 2},
}


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("shape", SWEEP, ids=[f"r{s[0]}g{s[1]}h{s[2]}d{s[3]}w{s[4]}s{s[5]}{s[6]}" for s in SWEEP])
def test_sweep(shape, variant):
    rows, ng, hpg, d, w, ns, kind = shape
    _case(f"sweep {shape} {variant}")
    rng = np.random.default_rng(zlib.crc32(repr((shape, variant)).encode()))
    inp = gen.make_chunk(rows, ng, hpg, d, w, ns, _rand_meta(rng, ng, w, kind),
                         seed=int(rng.integers(1 << 30)))
    ref = oracle.window_chunk(inp)
    try:
        for knob, val in VARIANTS[variant].items():
            B.tuning_set(knob, val)
        got = gpu_chunk(inp).cpu().numpy()
    finally:
        for knob in VARIANTS[variant]:
            B.tuning_set(knob, 0)
    assert_close(got, ref, f"{shape} {variant}")


# Shapes on which the matrix-core launch takes its paired order under the whole-groups-per-XCD
# work order (the second half of each XCD's workgroups mirror their query blocks): items per
# XCD a multiple of twice the query blocks, with invalid items at the end of the last XCD's
# range. Checked against the oracle and bitwise against the round-robin order (the same splits
# merged in the same order), with the merge in the last split and in its own launch.
PAIRED = [
    # rows, ng, hpg, d, w, ns, meta kind, tiles per split
    (64, 5, 4, 128, 200, 4, "mix", 3),      # 2 query blocks, 3 splits: 4 items per XCD, 2 invalid
    (96, 3, 4, 64, 400, 2, "partial", 3),   # 3 blocks, 5 splits: 6 per XCD, 3 invalid
    (64, 7, 4, 128, 150, 3, "full", 3),     # 2 blocks, 2 splits: 4 per XCD, 4 invalid
    (128, 3, 4, 128, 260, 2, "mix", 2),     # 4 blocks, 5 splits: 8 per XCD, 4 invalid
]


@pytest.mark.parametrize("merge", [1, 2], ids=["merge_in_kernel", "merge_launch"])
@pytest.mark.parametrize("shape", PAIRED, ids=[f"r{s[0]}g{s[1]}d{s[3]}w{s[4]}t{s[7]}" for s in PAIRED])
def test_paired_order(shape, merge):
    rows, ng, hpg, d, w, ns, kind, tps = shape
    _case(f"paired order {shape} merge {merge}")
    rng = np.random.default_rng(zlib.crc32(repr((shape, "paired")).encode()))
    inp = gen.make_chunk(rows, ng, hpg, d, w, ns, _rand_meta(rng, ng, w, kind),
                         seed=int(rng.integers(1 << 30)))
    ref = oracle.window_chunk(inp)
    knobs = {B.TUNE_FORCE_KERNEL: 2, B.TUNE_TILES_PER_SPLIT: tps, B.TUNE_MERGE_KERNEL: merge}
    got = {}
    try:
        for knob, val in knobs.items():
            B.tuning_set(knob, val)
        for order in (2, 1):   # knob value - 1 = xcd_map
            B.tuning_set(B.TUNE_XCD_MAP, order)
            plan = B.chunk_plan(rows, ng, hpg, d, w, ns)
            nqb = -(-rows * hpg // 128)
            per_xcd = -(-plan[2] * nqb * ng // 8)
            assert plan[0] == 2 and per_xcd % (2 * nqb) == 0 and 8 * per_xcd > plan[2] * nqb * ng, plan
            got[order] = gpu_chunk(inp).cpu().numpy()
    finally:
        for knob in list(knobs) + [B.TUNE_XCD_MAP]:
            B.tuning_set(knob, 0)
    assert_close(got[2], ref, f"{shape} paired order")
    assert np.array_equal(got[2], got[1]), "paired and round-robin orders differ"


# The register kernel runs splits of at most three tiles (split 0 also carries the sink tiles) as
# a straight-line instance and longer ones as a two-buffer loop (its tile is 4096 / d keys):
# both instances, one or two sink tiles, and both merge paths.
DEC_INSTANCES = [
    # rows, ng, hpg, d, w, ns, meta kind, tiles per split, merge (0 auto, 1 in kernel, 2 launch)
    (1, 2, 4, 128, 300, 40, "mix", 1, 0),      # split 0: two sink tiles + one stream tile
    (1, 2, 4, 128, 300, 40, "full", 4, 0),     # six tiles in split 0: loop instance
    (1, 2, 4, 128, 300, 40, "mix", 1, 1),      # three-tile split 0, in-kernel merge
    (2, 1, 4, 64, 500, 70, "mix", 1, 0),       # d = 64: 64-key tiles, two sink tiles
    (2, 3, 4, 256, 100, 17, "partial", 2, 0),  # d = 256: 16-key tiles, 8 queries, loop
    (1, 3, 8, 256, 100, 17, "override", 1, 2), # 8 queries, separate merge launch
    (1, 2, 4, 128, 5000, 3, "full", 3, 0),     # three-tile stream splits, four in split 0: loop
    (1, 1, 4, 128, 4096, 4, "full", 2, 0),     # the decode shape at one group
    (1, 2, 4, 128, 90, 5, "full", 8, 0),       # one split of four tiles: loop
    (1, 2, 4, 128, 60, 40, "mix", 2, 0),       # one split: two sink and two stream tiles
    (1, 1, 4, 64, 50, 3, "full", 1, 0),        # one split of two tiles
    (2, 2, 4, 256, 200, 20, "mix", 4, 1),      # loop, in-kernel merge
]


@pytest.mark.parametrize("shape", DEC_INSTANCES,
                         ids=[f"r{s[0]}g{s[1]}h{s[2]}d{s[3]}w{s[4]}s{s[5]}{s[6]}t{s[7]}m{s[8]}"
                              for s in DEC_INSTANCES])
def test_register_kernel_instances(shape):
    rows, ng, hpg, d, w, ns, kind, tps, merge = shape
    _case(f"register kernel {shape}")
    rng = np.random.default_rng(zlib.crc32(repr(shape).encode()))
    inp = gen.make_chunk(rows, ng, hpg, d, w, ns, _rand_meta(rng, ng, w, kind),
                         seed=int(rng.integers(1 << 30)))
    ref = oracle.window_chunk(inp)
    knobs = {B.TUNE_FORCE_KERNEL: 1, B.TUNE_TILES_PER_SPLIT: tps, B.TUNE_MERGE_KERNEL: merge}
    try:
        for knob, val in knobs.items():
            B.tuning_set(knob, val)
        plan = B.chunk_plan(rows, ng, hpg, d, w, ns)
        assert plan[0] == 1, plan
        got = gpu_chunk(inp).cpu().numpy()
    finally:
        for knob in knobs:
            B.tuning_set(knob, 0)
    assert_close(got, ref, f"{shape}")


# The single-launch kernel that streams rings in slot order (kernel 5): every query of a group
# in one block, ring tiles of 4096 / d slots, split 0 also takes the sinks and the chunk's rows
# (more than one pass of them when they exceed a pass), the last split merges.
SLOT_ORDER_CASES = [
    # rows, ng, hpg, d, w, ns, meta kind, ring tiles per split
    (1, 8, 4, 128, 4096, 4, "full", 2),      # the decode workload's plan
    (1, 8, 4, 128, 4096, 4, "mix", 4),
    (1, 2, 4, 128, 300, 40, "mix", 1),       # 44 sinks and rows: three passes of extra keys
    (2, 3, 4, 256, 100, 17, "partial", 2),   # 8 queries, d = 256 (4 keys per pass)
    (8, 2, 1, 64, 50, 3, "mix", 1),          # 8 rows of one head
    (1, 1, 4, 36, 90, 0, "override", 3),     # d = 36, no sinks
    (3, 2, 2, 100, 77, 5, "mix", 2),         # 6 queries, ragged ring
    (1, 4, 1, 64, 1, 1, "full", 1),          # a one-slot ring
    (4, 1, 2, 128, 20, 0, "empty", 1),       # an empty ring: the chunk's rows only
    (6, 2, 1, 64, 8, 2, "override", 1),      # chunk longer than its group's window
    (1, 3, 4, 256, 5000, 2, "mix", 4),       # a long ring: 79 splits
    (1, 1, 4, 64, 16, 2, "full", 1),         # one split: no partials, output stored directly
    (1, 1, 4, 64, 8192, 2, "full", 1),       # 128 splits, the most the kernel takes
    (1, 16, 4, 128, 1024, 4, "mix", 1),      # 16 groups x 8 gatherers: 128 waiting, the cap
    (2, 16, 4, 128, 2048, 4, "partial", 2),  # 8 queries per block over 16 groups
]


@pytest.mark.parametrize("shape", SLOT_ORDER_CASES,
                         ids=[f"r{s[0]}g{s[1]}h{s[2]}d{s[3]}w{s[4]}s{s[5]}{s[6]}t{s[7]}"
                              for s in SLOT_ORDER_CASES])
def test_slot_order_kernel(shape):
    rows, ng, hpg, d, w, ns, kind, tiles = shape
    _case(f"slot-order kernel {shape}")
    rng = np.random.default_rng(zlib.crc32(repr(shape).encode()))
    inp = gen.make_chunk(rows, ng, hpg, d, w, ns, _rand_meta(rng, ng, w, kind),
                         seed=int(rng.integers(1 << 30)))
    # slots no row sees hold NaN: they are read (slot order) and must add exactly nothing
    for g in range(ng):
        live = _visible_slots(inp, g)
        for sl in range(w):
            if sl not in live:
                inp.ring_k[g, sl] = np.nan
                inp.ring_v[g, sl] = np.nan
    ref = oracle.window_chunk(inp)
    knobs = {B.TUNE_FORCE_KERNEL: 5, B.TUNE_TILES_PER_SPLIT: tiles}
    try:
        for knob, val in knobs.items():
            B.tuning_set(knob, val)
        plan = B.chunk_plan(rows, ng, hpg, d, w, ns)
        assert plan[0] == 5, plan
        got = gpu_chunk(inp).cpu().numpy()
        again = gpu_chunk(inp).cpu().numpy()   # the ready flags were left at zero
    finally:
        for knob in knobs:
            B.tuning_set(knob, 0)
    assert_close(got, ref, f"{shape}")
    # the last split folds the others' partials in the order they become ready, so a repeat
    # may differ in the last bits (never beyond the bar)
    assert_close(again, ref, f"{shape}, repeated")


GATED_SWEEP = [
    # rows, pos0, cap, window, nh, nk, hd
    (1, 5000, 4096, 1024, 8, 2, 128),
    (3, 2, 16, 8, 4, 4, 64),
    (20, 100, 300, 256, 8, 2, 64),
    (64, 20000, 8192, 1024, 16, 4, 256),
    (40, 10, 64, 25, 6, 3, 128),
    # widths the single launch takes (160 to 256, multiples of 32)
    (17, 3, 64, 40, 6, 2, 192),          # windows clipped at position 0, sets across rows
    (40, 100, 200, 16, 8, 8, 256),       # more rows than the window, one head per KV head
    (33, 5000, 2048, 512, 12, 3, 160),   # a partial last set
    (16, 0, 64, 8, 4, 4, 224),           # one set per KV head
    (4, 50, 128, 64, 8, 2, 256),
    (2, 50, 128, 64, 8, 2, 256),         # fewer than 16 query vectors per KV head
    # 64 query vectors or more per KV head: the tile form
    (80, 3, 200, 100, 8, 2, 256),        # windows clipped at position 0
    (70, 100, 300, 30, 8, 8, 192),       # more rows than the window, one head per KV head
    (64, 5, 128, 48, 16, 4, 224),
    (64, 300, 512, 64, 64, 16, 256),     # 64 blocks: 2 gatherers per block, 4 items per thread
    (64, 300, 192, 64, 128, 32, 256),    # 128 blocks: 1 gatherer per block, 8 items per thread
]

# plans of the gated call: automatic; the single launch with one, the automatic and many
# workgroups per set; the three-launch path (prepared queries, 16x16 matrix-core kernel)
GATED_VARIANTS = {
    "auto": {},
    "single_launch_one_split": {B.TUNE_FORCE_KERNEL: 6, B.TUNE_TARGET_BLOCKS: 1},
    "single_launch": {B.TUNE_FORCE_KERNEL: 6},
    "single_launch_many_splits": {B.TUNE_FORCE_KERNEL: 6, B.TUNE_TARGET_BLOCKS: 4096},
    "three_launches": {B.TUNE_FORCE_KERNEL: 4},
}


@pytest.mark.parametrize("variant", list(GATED_VARIANTS))
@pytest.mark.parametrize("shape", GATED_SWEEP, ids=[f"r{s[0]}p{s[1]}c{s[2]}w{s[3]}h{s[4]}k{s[5]}d{s[6]}" for s in GATED_SWEEP])
def test_gated_sweep(shape, variant):
    rows, pos0, cap, window, nh, nk, hd = shape
    _case(f"gated sweep {shape} {variant}")
    knobs = GATED_VARIANTS[variant]
    try:
        for knob, val in knobs.items():
            B.tuning_set(knob, val)
        for scale in (None, float(np.sqrt(hd))):   # 1/sqrt(hd) and a sharp nGPT-like softmax
            inp = gen.make_gated(rows, pos0, cap, window, nh, nk, hd, seed=rows + pos0, scale=scale)
            z, rk, rv = gpu_gated(inp)
            oz, ork, orv = oracle.window_gated(inp)
            assert_close(z, oz, f"gated {shape} {variant} scale={scale}")
            assert_close(rk, ork, "ring k")
            np.testing.assert_array_equal(rv, orv)
            # a second call on the same inputs: the ready flags were left at zero
            z2, _, _ = gpu_gated(inp)
            assert_close(z2, oz, f"gated {shape} {variant} scale={scale}, repeated")
    finally:
        for knob in knobs:
            B.tuning_set(knob, 0)


# ── strict: nothing outside the window is read, nothing outside out is written ───────────────

def _visible_slots(inp, g):
    ln, head, _, ov = (int(x) for x in inp.meta[g])
    wg = ov if ov else inp.w
    seen = set()
    for i in range(inp.rows):
        hi = ln + i + 1
        lo = hi - min(wg, hi)
        for x in range(lo, min(hi, ln)):
            seen.add((head + x) % wg)
    return seen


@pytest.mark.parametrize("rows,hpg", [(1, 4), (2, 4), (3, 4), (70, 4)])
def test_poisoned_slots_and_canaries(rows, hpg):
    _case(f"poison rows={rows}")
    ng, d, w, ns = 4, 128, 96, 2
    meta = [(96, 17, 0, 0), (50, 80, 0, 0), (40, 39, 0, 64), (0, 3, 0, 0)]
    inp = gen.make_chunk(rows, ng, hpg, d, w, ns, meta, seed=99)
    for g in range(ng):
        live = _visible_slots(inp, g)
        for s in range(w):
            if s not in live:
                inp.ring_k[g, s] = np.nan
                inp.ring_v[g, s] = np.nan
    # the full ring's oldest entry is evicted for every row
    assert np.isnan(inp.ring_k[0, 17]).all()
    ref = oracle.window_chunk(inp)
    nh = ng * hpg
    n = rows * nh * d
    guard = 64
    buf = torch.full((n + 2 * guard,), 7.25, dtype=torch.float32, device=DEV)
    out = buf[guard:guard + n].view(rows, nh, d)
    need = B.chunk_workspace_bytes(rows, ng, hpg, d, w, ns)
    ws = B.Workspace(DEV)
    ws.buf = torch.zeros(need + 4096, dtype=torch.uint8, device=DEV)
    ws.buf[need:] = 0xAB
    gpu_chunk(inp, out=out, workspace=ws)
    assert_close(out.cpu().numpy(), ref, "poisoned")
    b = buf.cpu().numpy()
    assert np.all(b[:guard] == 7.25) and np.all(b[guard + n:] == 7.25), "wrote outside out"
    assert np.all(ws.buf[need:].cpu().numpy() == 0xAB), "wrote outside the workspace"


# three launches; the register form; the tile form
@pytest.mark.parametrize("rows,nh,hd", [(6, 4, 64), (6, 8, 256), (24, 8, 256)])
def test_gated_untouched_slots(rows, nh, hd):
    _case(f"gated untouched slots rows={rows} nh={nh} hd={hd}")
    inp = gen.make_gated(rows, 40, 64, 16, nh, 2, hd, seed=5)
    read_or_written = set()
    for r in range(inp.rows):
        pos = inp.pos0 + r
        for p in range(max(0, pos + 1 - inp.window), pos + 1):
            read_or_written.add(p % inp.cap)
    untouched = [s for s in range(inp.cap) if s not in read_or_written]
    # the slots the rows write hold NaN before the call too: nothing may read them before the
    # call has written them
    written = sorted({(inp.pos0 + r) % inp.cap for r in range(inp.rows)})
    inp.ring_k[untouched] = np.nan
    inp.ring_v[untouched] = np.nan
    inp.ring_k[written] = np.nan
    inp.ring_v[written] = np.nan
    z, rk, rv = gpu_gated(inp)
    oz, ork, orv = oracle.window_gated(inp)
    assert_close(z, oz, "gated poisoned")
    assert np.isnan(rk[untouched]).all() and np.isnan(rv[untouched]).all()
    assert_close(rk[written], ork[written], "written ring keys")
    np.testing.assert_array_equal(rv[written], orv[written])


# ── invariants on the GPU ────────────────────────────────────────────────────────────────────

def test_ring_rotation_on_gpu():
    _case("rotation")
    inp = gen.make_chunk(9, 3, 4, 128, 80, 4, [(80, 11, 0, 0), (30, 70, 0, 0), (20, 5, 0, 40)], seed=3)
    base = gpu_chunk(inp).cpu().numpy()
    rot = gen.make_chunk(9, 3, 4, 128, 80, 4, inp.meta.copy(), seed=3)
    for g in range(3):
        ln, head, far, ov = (int(x) for x in inp.meta[g])
        wg = ov if ov else inp.w
        r = 7 * g + 5
        idx = (np.arange(wg) + r) % wg
        rot.ring_k[g, idx] = inp.ring_k[g, :wg]
        rot.ring_v[g, idx] = inp.ring_v[g, :wg]
        rot.meta[g] = (ln, (head + r) % wg, far, ov)
    assert_close(gpu_chunk(rot).cpu().numpy(), base, "rotation")


def test_chunk_equals_sequence_of_decodes_on_gpu():
    _case("chunk vs decodes")
    import test_oracle_pins as pins
    inp = gen.make_chunk(12, 2, 4, 128, 10, 2, [(10, 3, 0, 0), (4, 1, 0, 6)], seed=8)
    full = gpu_chunk(inp).cpu().numpy()
    state = gen.make_chunk(1, 2, 4, 128, 10, 2, inp.meta.copy(), seed=0)
    state.ring_k, state.ring_v = inp.ring_k.copy(), inp.ring_v.copy()
    state.sink_k, state.sink_v = inp.sink_k, inp.sink_v
    for i in range(inp.rows):
        state.q = inp.q[i:i + 1].copy()
        state.chunk_k = inp.chunk_k[i:i + 1].copy()
        state.chunk_v = inp.chunk_v[i:i + 1].copy()
        assert_close(gpu_chunk(state).cpu().numpy()[0], full[i], f"decode row {i}")
        for g in range(inp.ng):
            pins._push(state, g, inp.chunk_k[i, g], inp.chunk_v[i, g])


# ── ring commit + meta advance (the state a decode loop carries) ───────────────────────────

COMMIT_CASES = [
    # rows, ng, d, w, meta
    (1, 8, 128, 4096, "full"),
    (3, 3, 64, 20, "mix"),
    (25, 2, 128, 16, "mix"),        # chunk longer than the window
    (7, 4, 36, 9, "partial"),
    (40, 1, 256, 100, "override"),
    (1, 2, 4, 1, "full"),            # window of one
]


@pytest.mark.parametrize("shape", COMMIT_CASES, ids=[f"r{c[0]}g{c[1]}d{c[2]}w{c[3]}{c[4]}" for c in COMMIT_CASES])
def test_commit_matches_oracle(shape):
    rows, ng, d, w, kind = shape
    _case(f"commit {shape}")
    rng = np.random.default_rng(zlib.crc32(repr(shape).encode()))
    inp = gen.make_chunk(rows, ng, 1, d, w, 0, _rand_meta(rng, ng, w, kind),
                         seed=int(rng.integers(1 << 30)))
    inp.meta[:, 2] = rng.integers(0, 1000, size=ng)   # far counts carry through
    rk, rv, meta = oracle.window_commit(inp)
    t = gen.to_device(inp, DEV)
    B.attn_window_commit(t["ring_k"], t["ring_v"], t["meta"], t["chunk_k"], t["chunk_v"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(t["meta"].cpu().numpy().astype(np.uint32), meta)
    np.testing.assert_array_equal(t["ring_k"].cpu().numpy(), rk)
    np.testing.assert_array_equal(t["ring_v"].cpu().numpy(), rv)


def test_decode_loop_with_commit_on_gpu():
    """A stateful loop entirely on the GPU: attend one row, commit it, next row. Every row's
    output equals the oracle's chunk call on the starting state, and the final rings and meta
    equal the oracle's commit of the whole chunk."""
    _case("decode loop with commit")
    inp = gen.make_chunk(20, 3, 4, 128, 12, 2, [(12, 5, 3, 0), (2, 1, 0, 7), (0, 9, 0, 0)], seed=9)
    ref = oracle.window_chunk(inp)
    rk, rv, meta = oracle.window_commit(inp)
    t = gen.to_device(inp, DEV)
    out = torch.empty((1, inp.nh, inp.d), dtype=torch.float32, device=DEV)
    for i in range(inp.rows):
        B.attn_window_chunk(t["ring_k"], t["ring_v"], t["meta"], t["sink_k"], t["sink_v"],
                            t["q"][i:i + 1], t["chunk_k"][i:i + 1], t["chunk_v"][i:i + 1],
                            inp.scale, out=out)
        assert_close(out.cpu().numpy()[0], ref[i], f"decode row {i}")
        B.attn_window_commit(t["ring_k"], t["ring_v"], t["meta"], t["chunk_k"][i:i + 1],
                             t["chunk_v"][i:i + 1])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(t["meta"].cpu().numpy().astype(np.uint32), meta)
    np.testing.assert_array_equal(t["ring_k"].cpu().numpy(), rk)
    np.testing.assert_array_equal(t["ring_v"].cpu().numpy(), rv)


def test_repeated_calls_and_workspace_reuse():
    """Split counters reset themselves: back-to-back calls of different shapes on one workspace."""
    _case("workspace reuse")
    ws = B.Workspace(DEV)
    a = gen.make_chunk(1, 8, 4, 128, 2048, 4, [(2048, 100 * g, 0, 0) for g in range(8)], seed=1)
    b = gen.make_chunk(200, 2, 4, 128, 700, 3, [(700, 3, 0, 0), (300, 9, 0, 0)], seed=2)
    ra, rb = oracle.window_chunk(a), oracle.window_chunk(b)
    ws.get(max(B.chunk_workspace_bytes(1, 8, 4, 128, 2048, 4),
               B.chunk_workspace_bytes(200, 2, 4, 128, 700, 3)))
    ws.buf[64 * 1024:] = 0x55   # stale bytes everywhere but the counter region
    c = gen.make_chunk(40, 1, 1, 64, 40, 0, [(40, 7, 0, 0)], seed=3)
    rc = oracle.window_chunk(c)
    for it in range(3):
        assert_close(gpu_chunk(a, workspace=ws).cpu().numpy(), ra, "a")
        assert_close(gpu_chunk(b, workspace=ws).cpu().numpy(), rb, "b")
        try:
            B.tuning_set(B.TUNE_FORCE_KERNEL, 2 if it % 2 else 1)
            B.tuning_set(B.TUNE_TILES_PER_SPLIT, 1)
            assert_close(gpu_chunk(c, workspace=ws).cpu().numpy(), rc, "c")
        finally:
            B.tuning_set(B.TUNE_FORCE_KERNEL, 0)
            B.tuning_set(B.TUNE_TILES_PER_SPLIT, 0)


def test_degenerate_cases():
    _case("degenerate")
    # a window of one key (override 1, no sinks) returns the row's own value
    inp = gen.make_chunk(5, 2, 4, 64, 8, 0, [(1, 0, 0, 1), (0, 0, 0, 1)], seed=4)
    got = gpu_chunk(inp).cpu().numpy()
    for i in range(5):
        for gh in range(8):
            np.testing.assert_allclose(got[i, gh], inp.chunk_v[i, gh // 4], rtol=0, atol=1e-6)
    # an empty ring: plain causal attention over the chunk plus sinks
    inp = gen.make_chunk(50, 1, 4, 128, 64, 3, [(0, 0, 0, 0)], seed=6)
    assert_close(gpu_chunk(inp).cpu().numpy(), oracle.window_chunk(inp), "empty ring")
    # rows = 0 is rejected before any launch
    t = gen.to_device(inp, DEV)
    rc = B.load().attn_window_chunk(t["ring_k"].data_ptr(), t["ring_v"].data_ptr(),
                                    t["meta"].data_ptr(), None, None, t["q"].data_ptr(),
                                    t["chunk_k"].data_ptr(), t["chunk_v"].data_ptr(),
                                    t["q"].data_ptr(), 0, 1, 4, 128, 64, 0, 0.1, None, 0, None)
    assert rc == B.EINVAL
