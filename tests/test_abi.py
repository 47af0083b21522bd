"""The C-ABI library loads, exports every symbol include/winattn.h declares, and validates its
arguments on the host (CPU only: no call here reaches a kernel launch)."""
import ctypes

import numpy as np
import pytest

from sliding_window_gqa_group_amd import binding as B


@pytest.fixture(scope="module")
def lib():
    return B.load()


def test_exports_every_declared_symbol(lib):
    names = B.declared_functions()
    assert "attn_window_chunk" in names and "attn_window_gated" in names
    raw = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), f"{n} declared in include/winattn.h but not exported"


def test_version_and_strerror(lib):
    assert B.abi_version() == 1
    for code in (0, -1, -2, -3, -4):
        assert B.strerror(code)
    assert "unknown" in B.strerror(-99)


FAKE = 1 << 20   # a 16-byte aligned non-null address; never dereferenced (validation fails first)


def _chunk(lib, **kw):
    a = dict(ring_k=FAKE, ring_v=FAKE, meta=FAKE, sink_k=FAKE, sink_v=FAKE, q=FAKE, chunk_k=FAKE,
             chunk_v=FAKE, out=FAKE, rows=1, ng=1, hpg=1, d=64, w=16, ns=0, scale=0.125,
             ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.attn_window_chunk(a["ring_k"], a["ring_v"], a["meta"], a["sink_k"], a["sink_v"],
                                 a["q"], a["chunk_k"], a["chunk_v"], a["out"], a["rows"], a["ng"],
                                 a["hpg"], a["d"], a["w"], a["ns"], a["scale"], a["ws"], a["wsb"],
                                 a["stream"])


@pytest.mark.parametrize("kw", [
    dict(rows=0), dict(ng=0), dict(hpg=0), dict(w=0), dict(ns=-1), dict(d=0), dict(d=6),
    dict(d=260), dict(scale=float("inf")), dict(scale=float("nan")), dict(ring_k=None),
    dict(meta=None), dict(out=None), dict(chunk_v=None), dict(ns=2, sink_k=None),
    dict(q=FAKE + 4), dict(out=FAKE + 8), dict(meta=FAKE + 2),
])
def test_chunk_rejects_invalid_arguments(lib, kw):
    assert _chunk(lib, **kw) == B.EINVAL


def test_chunk_rejects_small_workspace(lib):
    need = B.chunk_workspace_bytes(1, 8, 4, 128, 4096, 4)
    assert need > 0
    assert _chunk(lib, ng=8, hpg=4, d=128, w=4096, ns=4, ws=None, wsb=0) == B.EWORKSPACE
    assert _chunk(lib, ng=8, hpg=4, d=128, w=4096, ns=4, ws=FAKE, wsb=need - 1) == B.EWORKSPACE


def _gated(lib, **kw):
    a = dict(yq=FAKE, yk=FAKE, yv=FAKE, rope=FAKE, q_scale=FAKE, gate=FAKE, gate_scale=FAKE,
             ring_k=FAKE, ring_v=FAKE, out=FAKE, rows=4, pos0=10, cap=16, window=8, nh=4, nk=2,
             hd=64, scale=0.125, eps=1e-6, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return lib.attn_window_gated(a["yq"], a["yk"], a["yv"], a["rope"], a["q_scale"], a["gate"],
                                 a["gate_scale"], a["ring_k"], a["ring_v"], a["out"], a["rows"],
                                 a["pos0"], a["cap"], a["window"], a["nh"], a["nk"], a["hd"],
                                 a["scale"], a["eps"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw", [
    dict(rows=0), dict(pos0=-1), dict(cap=10), dict(window=0), dict(nh=5), dict(nk=0),
    dict(hd=60), dict(hd=264), dict(hd=4), dict(eps=-1.0), dict(scale=float("nan")),
    dict(yq=None), dict(ring_v=None), dict(gate=FAKE + 4),
])
def test_gated_rejects_invalid_arguments(lib, kw):
    assert _gated(lib, **kw) == B.EINVAL


def test_gated_rejects_small_workspace(lib):
    need = B.gated_workspace_bytes(4, 4, 2, 64, 8)
    assert need > 0
    assert _gated(lib, ws=None, wsb=0) == B.EWORKSPACE
    assert _gated(lib, wsb=need - 1) == B.EWORKSPACE


def _commit(lib, **kw):
    a = dict(ring_k=FAKE, ring_v=FAKE, meta=FAKE, chunk_k=FAKE, chunk_v=FAKE, rows=1, ng=1,
             d=64, w=16, stream=None)
    a.update(kw)
    return lib.attn_window_commit(a["ring_k"], a["ring_v"], a["meta"], a["chunk_k"],
                                  a["chunk_v"], a["rows"], a["ng"], a["d"], a["w"], a["stream"])


@pytest.mark.parametrize("kw", [
    dict(rows=0), dict(ng=0), dict(w=0), dict(d=0), dict(d=6), dict(d=260), dict(ring_k=None),
    dict(meta=None), dict(chunk_v=None), dict(ring_v=FAKE + 4), dict(chunk_k=FAKE + 8),
    dict(meta=FAKE + 2),
])
def test_commit_rejects_invalid_arguments(lib, kw):
    assert _commit(lib, **kw) == B.EINVAL


def _chunk_far(lib, **kw):
    a = dict(ring_k=FAKE, ring_v=FAKE, meta=FAKE, sink_k=None, sink_v=None, q=FAKE,
             chunk_k=FAKE, chunk_v=FAKE, k_tilde=FAKE, q_tilde=FAKE, mu=FAKE, mz=FAKE,
             t_hat=FAKE, out=FAKE, rows=4, ng=2, hpg=2, d=64, w=16, ns=0, m=8, scale=0.125,
             ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return lib.attn_window_chunk_far(*a.values())


@pytest.mark.parametrize("kw", [
    dict(rows=0), dict(m=0), dict(d=6), dict(k_tilde=None), dict(q_tilde=None), dict(mu=None),
    dict(mz=None), dict(t_hat=None), dict(mu=FAKE + 4), dict(t_hat=FAKE + 8),
    dict(ns=2), dict(scale=float("nan")), dict(meta=FAKE + 1),
])
def test_chunk_far_rejects_invalid_arguments(lib, kw):
    assert _chunk_far(lib, **kw) == B.EINVAL


@pytest.mark.parametrize("kw", [dict(rows=65), dict(m=65)])
def test_chunk_far_rejects_unsupported_sizes(lib, kw):
    assert _chunk_far(lib, **kw) == B.EUNSUPPORTED


def test_chunk_far_needs_its_workspace(lib):
    need = B.chunk_far_workspace_bytes(4, 2, 2, 64, 16, 0, 8)
    assert need > 0
    # the far call keeps one more partial slot per query block and its eviction arrays
    assert need > B.chunk_workspace_bytes(4, 2, 2, 64, 16, 0) + 2 * 4 * 8 * 4 * 4
    assert _chunk_far(lib, ws=None) == B.EWORKSPACE
    assert _chunk_far(lib, wsb=need - 1) == B.EWORKSPACE
    assert B.chunk_far_workspace_bytes(65, 2, 2, 64, 16, 0, 8) == 0
    assert B.chunk_far_workspace_bytes(4, 2, 2, 64, 16, 0, 65) == 0
    assert B.chunk_far_workspace_bytes(4, 2, 2, 64, 16, 0, 0) == 0


def _commit_far(lib, **kw):
    a = dict(ring_k=FAKE, ring_v=FAKE, meta=FAKE, chunk_k=FAKE, chunk_v=FAKE, q_tilde=FAKE,
             mz=FAKE, t_hat=FAKE, rows=4, ng=2, hpg=2, d=64, w=16, m=8, scale=0.125,
             stream=None)
    a.update(kw)
    return lib.attn_window_commit_far(*a.values())


@pytest.mark.parametrize("kw", [
    dict(rows=0), dict(ng=0), dict(hpg=0), dict(m=0), dict(d=6), dict(q_tilde=None),
    dict(mz=None), dict(t_hat=None), dict(mz=FAKE + 4), dict(meta=None),
    dict(scale=float("inf")),
])
def test_commit_far_rejects_invalid_arguments(lib, kw):
    assert _commit_far(lib, **kw) == B.EINVAL


@pytest.mark.parametrize("kw", [dict(rows=65), dict(m=65)])
def test_commit_far_rejects_unsupported_sizes(lib, kw):
    assert _commit_far(lib, **kw) == B.EUNSUPPORTED


def _gated_far(lib, **kw):
    a = dict(q=FAKE, ring_k=FAKE, ring_v=FAKE, meta=FAKE, sink_k=None, sink_v=None,
             k_tilde=FAKE, mu=FAKE, mz=FAKE, t_hat=FAKE, gate=FAKE, gate_scale=FAKE, out=FAKE,
             nh=8, nk=2, hd=64, w=16, ns=0, m=8, scale=0.125, rect=0, ws=FAKE, wsb=1 << 30,
             stream=None)
    a.update(kw)
    return lib.attn_window_gated_far(*a.values())


@pytest.mark.parametrize("kw", [
    dict(nh=0), dict(nk=3), dict(hd=6), dict(hd=260), dict(w=0), dict(m=0), dict(rect=2),
    dict(q=None), dict(gate=None), dict(gate_scale=FAKE + 4), dict(t_hat=None), dict(ns=1),
    dict(meta=FAKE + 2), dict(scale=float("nan")),
])
def test_gated_far_rejects_invalid_arguments(lib, kw):
    assert _gated_far(lib, **kw) == B.EINVAL


def test_gated_far_limits_and_workspace(lib):
    assert _gated_far(lib, m=65) == B.EUNSUPPORTED
    need = B.gated_far_workspace_bytes(8, 2, 64, 16, 0, 8)
    assert need > 0
    assert _gated_far(lib, ws=None) == B.EWORKSPACE
    assert _gated_far(lib, wsb=need - 1) == B.EWORKSPACE
    assert B.gated_far_workspace_bytes(8, 2, 64, 16, 0, 65) == 0
    assert B.gated_far_workspace_bytes(8, 3, 64, 16, 0, 8) == 0


def _encoder(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, segs=FAKE, nseg=2, max_len=100, ldq=512,
             ldk=128, ldv=128, ldo=512, nh=8, nk=2, hd=64, window=0, scale=0.125, stream=None)
    a.update(kw)
    return lib.attn_encoder(*a.values())


@pytest.mark.parametrize("kw", [
    dict(nh=6, nk=4), dict(nk=0), dict(hd=6), dict(hd=0), dict(window=-1), dict(nseg=-1),
    dict(ldq=508), dict(ldk=126), dict(ldv=100), dict(ldo=500), dict(q=None), dict(out=FAKE + 4),
    dict(segs=None), dict(segs=FAKE + 2), dict(scale=float("inf")), dict(max_len=-1),
])
def test_encoder_rejects_invalid_arguments(lib, kw):
    assert _encoder(lib, **kw) == B.EINVAL


def test_encoder_limits(lib):
    assert _encoder(lib, hd=260, ldq=8 * 260, ldk=2 * 260, ldv=2 * 260, ldo=8 * 260) == B.EINVAL
    # nothing to do: no launch, success, even with no pointers at all
    assert _encoder(lib, nseg=0, q=None, segs=None) == B.OK
    assert _encoder(lib, max_len=0, q=None) == B.OK


def test_workspace_queries(lib):
    assert B.chunk_workspace_bytes(0, 1, 1, 64, 16, 0) == 0
    assert B.gated_workspace_bytes(1, 5, 2, 64, 8) == 0
    # a single-split plan needs no workspace at all
    kern, qb, splits, kps = B.chunk_plan(1, 1, 4, 64, 16, 2)
    assert (kern, splits) == (5, 1)
    assert B.chunk_workspace_bytes(1, 1, 4, 64, 16, 2) == 0
    # gated always holds its prepared queries
    assert B.gated_workspace_bytes(64, 16, 4, 256, 1024) >= 64 * 16 * 256 * 4


def test_plans_of_the_named_workloads(lib):
    # decode: the single-launch slot-order kernel, 64 splits of two 32-slot tiles per group
    # (512 workgroups, two per CU); over a 32768-slot window the two-launch register kernel,
    # 64 splits of 16 tiles
    assert B.chunk_plan(1, 8, 4, 128, 4096, 4) == (5, 4, 64, 64)
    assert B.chunk_plan(1, 8, 4, 128, 32768, 4) == (1, 4, 64, 512)
    assert B.chunk_plan(2, 8, 4, 128, 4096, 4) == (5, 8, 64, 64)  # two rows: 8 queries per block
    # 8 queries per block hold at most two ring tiles per split
    assert B.chunk_plan(1, 8, 8, 128, 8192, 4) == (5, 8, 128, 64)
    assert B.chunk_plan(4, 8, 4, 128, 4096, 4)[:2] == (4, 64)   # 16 queries: 16x16 matrix cores
    assert B.chunk_plan(64, 8, 4, 128, 4096, 4)[:2] == (4, 64)  # up to 256 queries per group
    assert B.chunk_plan(65, 8, 4, 128, 4096, 4)[:2] == (2, 128) # beyond: 32x32 matrix cores
    assert B.chunk_plan(512, 8, 4, 128, 4096, 4)[0] == 2        # prefill: matrix cores
    k, qb, splits, kps = B.chunk_plan(2048, 8, 8, 128, 32768, 4)
    assert k == 2 and splits * kps >= 4 + 32768 + 16
    # wide heads (the gated shape: 64 rows, 4 query heads per KV head, d = 256)
    k, qb, splits, kps = B.chunk_plan(64, 4, 4, 256, 1024, 0)
    assert (k, qb) == (4, 64)


def test_tuning_knobs_change_the_plan(lib):
    try:
        B.tuning_set(B.TUNE_FORCE_KERNEL, 2)
        assert B.chunk_plan(1, 8, 4, 128, 4096, 4)[0] == 2
        B.tuning_set(B.TUNE_FORCE_KERNEL, 1)
        B.tuning_set(B.TUNE_TILES_PER_SPLIT, 1)
        k, qb, splits, kps = B.chunk_plan(512, 8, 4, 128, 4096, 4)
        assert k == 1 and qb == 8 and kps == 32
        B.tuning_set(B.TUNE_FORCE_KERNEL, 3)
        k, qb, splits, kps = B.chunk_plan(512, 8, 4, 128, 4096, 4)
        assert k == 3 and qb == 16 and kps == 64
        B.tuning_set(B.TUNE_FORCE_KERNEL, 4)
        k, qb, splits, kps = B.chunk_plan(512, 8, 4, 128, 4096, 4)
        assert k == 4 and qb == 64 and kps == 32
    finally:
        B.tuning_set(B.TUNE_FORCE_KERNEL, 0)
        B.tuning_set(B.TUNE_TILES_PER_SPLIT, 0)
    with pytest.raises(B.WinattnError):
        B.tuning_set(99, 1)
    try:
        B.tuning_set(B.TUNE_FORCE_KERNEL, 5)
        B.tuning_set(B.TUNE_TILES_PER_SPLIT, 4)
        assert B.chunk_plan(1, 8, 4, 128, 4096, 4) == (5, 4, 32, 128)
        assert B.chunk_plan(2, 8, 4, 128, 4096, 4) == (5, 8, 64, 64)   # capped at two tiles
        assert B.chunk_plan(512, 8, 4, 128, 4096, 4)[0] == 2   # too many queries: automatic
        # the slot-order kernel's limits: 128 splits per group (two 64-bit masks of splits per
        # gatherer lane), 128 waiting gatherers over all groups
        B.tuning_set(B.TUNE_TILES_PER_SPLIT, 1)
        assert B.chunk_plan(1, 1, 4, 64, 8192, 2) == (5, 4, 128, 64)
        assert B.chunk_plan(1, 2, 4, 64, 8256, 2)[:3] == (1, 4, 129)   # 129 splits: another kernel
        assert B.chunk_plan(1, 16, 4, 128, 1024, 4) == (5, 4, 32, 32)   # 16 groups x 8 gatherers
    finally:
        B.tuning_set(B.TUNE_FORCE_KERNEL, 0)
        B.tuning_set(B.TUNE_TILES_PER_SPLIT, 0)
    with pytest.raises(B.WinattnError):
        B.tuning_set(B.TUNE_FORCE_KERNEL, 7)


def test_workspace_sizes_follow_the_tuning_knobs(lib):
    # the binding keeps workspace sizes per call shape; a knob that changes the plan must change
    # the size it reports
    shape = (1, 8, 4, 128, 4096, 4)
    auto = B.chunk_workspace_bytes(*shape)
    assert auto == lib.attn_window_chunk_workspace(*shape)
    try:
        B.tuning_set(B.TUNE_FORCE_KERNEL, 2)
        forced = B.chunk_workspace_bytes(*shape)
        assert forced == lib.attn_window_chunk_workspace(*shape) and forced != auto
    finally:
        B.tuning_set(B.TUNE_FORCE_KERNEL, 0)
    assert B.chunk_workspace_bytes(*shape) == auto


def test_one_row_far_plan_workspace(lib):
    # A one-row chunk call with a far field runs its far part inside the single-launch decode
    # kernel, one workgroup per head ahead of the splits: for the 4096-slot decode heads (8
    # groups x 4, d 128, 32-slot ring tiles) the 32 far workgroups and the splits fit two per
    # CU (512): 3 tiles per split, 43 splits, and one partial slot more per group for the far
    # part; then the f64 eviction arrays [nh][m][rows] (two) and [nh][m] (two), here m = 16.
    def al(x):
        return (x + 255) // 256 * 256

    def expect(nsplit):
        slots = 8 * (nsplit + 1) * 4
        return 65536 + al(slots * 128 * 4) + 2 * al(slots * 4) + 4 * al(32 * 16 * 8)
    need = B.chunk_far_workspace_bytes(1, 8, 4, 128, 4096, 4, 16)
    assert need == expect(43)
    try:
        B.tuning_set(B.TUNE_TILES_PER_SPLIT, 2)   # 64 splits: 68 ready flags per gatherer
        assert B.chunk_far_workspace_bytes(1, 8, 4, 128, 4096, 4, 16) == expect(64)
        B.tuning_set(B.TUNE_TILES_PER_SPLIT, 4)   # 32 splits
        assert B.chunk_far_workspace_bytes(1, 8, 4, 128, 4096, 4, 16) == expect(32)
    finally:
        B.tuning_set(B.TUNE_TILES_PER_SPLIT, 0)
    assert B.chunk_far_workspace_bytes(1, 8, 4, 128, 4096, 4, 16) == need


def test_gated_one_row_far_plan_workspace(lib):
    # The gated one-row far call at the gated heads (16 query / 4 KV heads, hd 256, 1024-slot
    # rings) runs in the single-launch decode kernel: 16-slot ring tiles (32 KiB of K and V),
    # two per split for at least 64 KiB, 32 splits per group plus the far slot; counters +
    # partials, no eviction arrays.
    def al(x):
        return (x + 255) // 256 * 256

    def expect(nsplit):
        slots = 4 * (nsplit + 1) * 4
        return 65536 + al(slots * 256 * 4) + 2 * al(slots * 4)
    assert B.gated_far_workspace_bytes(16, 4, 256, 1024, 0, 32) == expect(32)
    try:
        B.tuning_set(B.TUNE_TILES_PER_SPLIT, 4)
        assert B.gated_far_workspace_bytes(16, 4, 256, 1024, 0, 32) == expect(16)
        B.tuning_set(B.TUNE_TILES_PER_SPLIT, 1)   # 64 splits: 68 ready flags per gatherer
        assert B.gated_far_workspace_bytes(16, 4, 256, 1024, 0, 32) == expect(64)
    finally:
        B.tuning_set(B.TUNE_TILES_PER_SPLIT, 0)


def test_gated_single_launch_workspace(lib):
    # the gated call in one launch (kernel 6), tile form for the 64-row, 16/4-head, width-256
    # workload: 4 blocks of 64 query vectors per KV head, 16 splits each (256 workgroups):
    # counters + partials
    items = 4 * 4 * 16
    need = B.gated_workspace_bytes(64, 16, 4, 256, 1024)
    assert need == 65536 + items * 64 * 256 * 4 + 2 * items * 64 * 4
    # register form (16 to 63 query vectors per KV head): sets of 16, 4 splits each
    items = 2 * 2 * 16
    assert B.gated_workspace_bytes(8, 8, 2, 256, 1024) == 65536 + items * 16 * 256 * 4 + 2 * items * 16 * 4
    try:
        B.tuning_set(B.TUNE_TARGET_BLOCKS, 1)    # one workgroup per block: no partials at all
        assert B.gated_workspace_bytes(64, 16, 4, 256, 1024) == 0
        B.tuning_set(B.TUNE_TARGET_BLOCKS, 0)
        B.tuning_set(B.TUNE_FORCE_KERNEL, 6)     # fewer than 16 query vectors per KV head, forced
        assert B.gated_workspace_bytes(2, 8, 2, 256, 64) == 0
        B.tuning_set(B.TUNE_FORCE_KERNEL, 4)     # the three-launch path keeps its prepared queries
        assert B.gated_workspace_bytes(64, 16, 4, 256, 1024) >= 64 * 16 * 256 * 4
    finally:
        B.tuning_set(B.TUNE_FORCE_KERNEL, 0)
        B.tuning_set(B.TUNE_TARGET_BLOCKS, 0)
    # widths the single launch does not take keep the three-launch plan
    assert B.gated_workspace_bytes(64, 16, 4, 128, 1024) >= 64 * 16 * 128 * 4
    assert B.gated_workspace_bytes(64, 16, 4, 200, 1024) >= 64 * 16 * 200 * 4


def test_check_meta(lib):
    assert B.check_meta(np.array([[16, 5, 0, 0]]), 1, 16) == 0
    assert B.check_meta(np.array([[17, 0, 0, 0]]), 1, 16) == B.EINVAL     # len > w
    assert B.check_meta(np.array([[4, 4, 0, 4]]), 1, 16) == B.EINVAL      # head >= window
    assert B.check_meta(np.array([[3, 0, 0, 20]]), 1, 16) == B.EINVAL     # override > w
    assert B.check_meta(np.array([[0, 99, 7, 0]]), 1, 16) == 0            # empty ring: head free
    assert lib.attn_window_check_meta(None, 1, 16) == B.EINVAL


def test_workspace_init_validation(lib):
    assert lib.attn_workspace_init(None, 0, None) == 0
    assert lib.attn_workspace_init(None, 64, None) == B.EINVAL
    assert lib.attn_workspace_init(FAKE + 4, 64, None) == B.EINVAL


def _noalloc(lib, **kw):
    a = dict(ring_k=FAKE, ring_v=FAKE, meta=FAKE, sink_k=FAKE, sink_v=FAKE, q=FAKE, chunk_k=FAKE,
             chunk_v=FAKE, out=FAKE, rows=1, ng=1, hpg=1, d=64, w=16, ns=0, scale=0.125,
             stream=None)
    a.update(kw)
    return lib.attn_window_chunk_noalloc(a["ring_k"], a["ring_v"], a["meta"], a["sink_k"],
                                         a["sink_v"], a["q"], a["chunk_k"], a["chunk_v"], a["out"],
                                         a["rows"], a["ng"], a["hpg"], a["d"], a["w"], a["ns"],
                                         a["scale"], a["stream"])


@pytest.mark.parametrize("kw", [
    dict(rows=0), dict(d=6), dict(scale=float("nan")), dict(q=None), dict(ns=2, sink_v=None),
    dict(out=FAKE + 8),
])
def test_noalloc_rejects_invalid_arguments(lib, kw):
    assert _noalloc(lib, **kw) == B.EINVAL


def test_noalloc_rejects_plans_beyond_its_scratch(lib):
    """A call whose plan needs more than the static scratch is refused before any device work."""
    shape = dict(rows=2048, ng=8, hpg=8, d=128, w=32768, ns=4)
    need = B.chunk_workspace_bytes(*shape.values())
    assert need > B.NOALLOC_SCRATCH_BYTES
    assert _noalloc(lib, **shape) == B.EWORKSPACE
    import re
    hdr = open(B.HEADER).read()
    m = re.search(r"#define WINATTN_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == B.NOALLOC_SCRATCH_BYTES
