"""Parity of the far-field path (attn_window_chunk_far, attn_window_commit_far) with the CPU
oracle, on seeded synthetic far states (inputs.make_far).

Bar (per element): |gpu - oracle| <= max(1e-4 * |oracle|, 1e-5), as for the near path; ring
slots and meta bit-exact; far maxima of empty fields stay -inf on both sides.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
from sliding_window_gqa_group_amd import binding as B
from sliding_window_gqa_group_amd import inputs as gen
from test_gpu_parity import _case, _rand_meta, assert_close

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()
    yield
    for knob in (B.TUNE_FORCE_KERNEL, B.TUNE_TILES_PER_SPLIT, B.TUNE_TARGET_BLOCKS,
                 B.TUNE_MERGE_KERNEL, B.TUNE_XCD_MAP):
        B.tuning_set(knob, 0)


def _far_inputs(shape):
    rows, ng, hpg, d, w, ns, m, kind, mu_kind = shape
    rng = np.random.default_rng(zlib.crc32(repr(shape).encode()))
    meta = _rand_meta(rng, ng, w, kind)
    # far counts: some groups start with an empty far field, the rest with a non-empty one
    meta = [(a, b, int(rng.integers(1, 500)) if (g % 3) else 0, c)
            for g, (a, b, _, c) in enumerate(meta)]
    inp = gen.make_chunk(rows, ng, hpg, d, w, ns, meta, seed=int(rng.integers(1 << 30)))
    far = gen.make_far(inp, m, seed=int(rng.integers(1 << 30)), mu_kind=mu_kind)
    return inp, far


def gpu_chunk_far(inp, far, out=None, workspace=None):
    t = gen.to_device(inp, DEV)
    f = gen.to_device(far, DEV)
    ns = inp.ns
    res = B.attn_window_chunk_far(t["ring_k"], t["ring_v"], t["meta"],
                                  t["sink_k"] if ns else None, t["sink_v"] if ns else None,
                                  t["q"], t["chunk_k"], t["chunk_v"], f["k_tilde"],
                                  f["q_tilde"], f["mu"], f["mz"], f["t_hat"], inp.scale,
                                  out=out, workspace=workspace)
    torch.cuda.synchronize()
    return res.cpu().numpy()


def assert_mz_close(got, ref, m, what):
    got = np.asarray(got)
    ref = np.asarray(ref)
    np.testing.assert_array_equal(np.isneginf(got), np.isneginf(ref), err_msg=f"{what}: -inf")
    fin = ~np.isneginf(ref)
    assert_close(got[fin], ref[fin], what)


FAR_CASES = [
    # rows, ng, hpg, d, w, ns, m, meta kind, mu kind
    (1, 8, 4, 128, 4096, 4, 16, "full", "positive"),      # the decode workload with a far field
    (1, 2, 4, 64, 40, 0, 8, "mix", "positive"),
    (4, 2, 4, 256, 90, 4, 16, "mix", "signed"),
    (17, 3, 4, 128, 50, 4, 64, "mix", "positive"),
    (64, 2, 4, 128, 200, 4, 32, "full", "positive"),      # the largest far chunk
    (64, 1, 8, 64, 20, 2, 8, "partial", "positive"),      # chunk longer than the window
    (33, 2, 1, 36, 30, 1, 5, "partial", "signed"),
    (5, 1, 3, 100, 6, 2, 1, "override", "positive"),      # one landmark
    (64, 4, 4, 256, 64, 0, 64, "full", "signed"),         # 16x16 matrix-core near kernel
    (2, 3, 1, 64, 1, 0, 3, "full", "positive"),           # window of one
    (1, 2, 2, 256, 70, 3, 12, "mix", "signed"),           # one row at d = 256 (one launch)
]

FAR_VARIANTS = {
    "auto": {},
    "register_many_splits": {B.TUNE_FORCE_KERNEL: 1, B.TUNE_TILES_PER_SPLIT: 1},
    "mfma_many_splits": {B.TUNE_FORCE_KERNEL: 2, B.TUNE_TILES_PER_SPLIT: 1},
    "lds_vector_many_splits": {B.TUNE_FORCE_KERNEL: 3, B.TUNE_TILES_PER_SPLIT: 1},
    "mfma16_many_splits": {B.TUNE_FORCE_KERNEL: 4, B.TUNE_TILES_PER_SPLIT: 1},
    # asks for the in-kernel merge: the far slot still merges in the merge launch
    "mfma_in_kernel_merge_asked": {B.TUNE_FORCE_KERNEL: 2, B.TUNE_TILES_PER_SPLIT: 2,
                                   B.TUNE_MERGE_KERNEL: 1},
    # one-row calls: the far part inside the single-launch slot-order kernel (kernel 5) with
    # other split sizes than its plan picks (the 4096-slot decode: 64 splits, 68 ready flags
    # per gatherer, more workgroups than the GPU holds at once; with one tile, 128 splits and 4
    # far flags are more than a gatherer polls, and the two-launch register plan takes it;
    # small rings: a single split); other shapes take their usual plan
    "decode_one_launch_two_tiles": {B.TUNE_FORCE_KERNEL: 5, B.TUNE_TILES_PER_SPLIT: 2},
    "decode_one_launch_one_tile": {B.TUNE_FORCE_KERNEL: 5, B.TUNE_TILES_PER_SPLIT: 1},
}


@pytest.mark.parametrize("variant", list(FAR_VARIANTS))
@pytest.mark.parametrize("shape", FAR_CASES,
                         ids=[f"r{s[0]}g{s[1]}h{s[2]}d{s[3]}w{s[4]}s{s[5]}m{s[6]}{s[7]}{s[8][0]}"
                              for s in FAR_CASES])
def test_chunk_far_matches_oracle(shape, variant):
    _case(f"chunk far {shape} {variant}")
    inp, far = _far_inputs(shape)
    ref = oracle.window_chunk_far(inp, far)
    try:
        for knob, val in FAR_VARIANTS[variant].items():
            B.tuning_set(knob, val)
        got = gpu_chunk_far(inp, far)
    finally:
        for knob in FAR_VARIANTS[variant]:
            B.tuning_set(knob, 0)
    assert_close(got, ref, f"chunk far {shape} {variant}")


def test_chunk_far_with_empty_field_equals_chunk():
    """No far count anywhere and a chunk that evicts nothing: the near call's result."""
    _case("far empty = near")
    inp = gen.make_chunk(9, 2, 4, 128, 40, 3, [(20, 5, 0, 0), (3, 1, 0, 0)], seed=12)
    far = gen.make_far(inp, 8, seed=13)
    near = B.attn_window_chunk(*[gen.to_device(inp, DEV)[k] for k in
                                 ("ring_k", "ring_v", "meta", "sink_k", "sink_v", "q",
                                  "chunk_k", "chunk_v")], inp.scale)
    torch.cuda.synchronize()
    assert_close(gpu_chunk_far(inp, far), near.cpu().numpy(), "far empty")


COMMIT_FAR_CASES = [
    # rows, ng, hpg, d, w, m, meta kind
    (1, 8, 4, 128, 4096, 16, "full"),
    (3, 3, 2, 64, 20, 8, "mix"),
    (64, 2, 4, 128, 16, 32, "mix"),       # chunk longer than the window
    (7, 4, 1, 36, 9, 5, "partial"),
    (40, 1, 4, 256, 100, 64, "override"),
    (1, 2, 1, 4, 1, 1, "full"),           # window of one
]


@pytest.mark.parametrize("shape", COMMIT_FAR_CASES,
                         ids=[f"r{c[0]}g{c[1]}h{c[2]}d{c[3]}w{c[4]}m{c[5]}{c[6]}" for c in COMMIT_FAR_CASES])
def test_commit_far_matches_oracle(shape):
    rows, ng, hpg, d, w, m, kind = shape
    _case(f"commit far {shape}")
    inp, far = _far_inputs((rows, ng, hpg, d, w, 0, m, kind, "positive"))
    rk, rv, meta, mz, th = oracle.window_commit_far(inp, far)
    t = gen.to_device(inp, DEV)
    f = gen.to_device(far, DEV)
    B.attn_window_commit_far(t["ring_k"], t["ring_v"], t["meta"], t["chunk_k"], t["chunk_v"],
                             f["q_tilde"], f["mz"], f["t_hat"], inp.scale)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(t["meta"].cpu().numpy().astype(np.uint32), meta)
    np.testing.assert_array_equal(t["ring_k"].cpu().numpy(), rk)
    np.testing.assert_array_equal(t["ring_v"].cpu().numpy(), rv)
    assert_mz_close(f["mz"].cpu().numpy(), mz, m, "mz")
    assert_close(f["t_hat"].cpu().numpy(), th, "t_hat")


def test_far_decode_loop_on_gpu():
    """A stateful loop on the GPU: attend one row with the far field, commit it (far state,
    ring, meta), next row. Every row equals the oracle's far chunk call on the starting state;
    the final state equals the oracle's far commit of the whole chunk."""
    _case("far decode loop")
    inp = gen.make_chunk(24, 3, 4, 128, 10, 2, [(10, 4, 7, 0), (5, 1, 0, 6), (0, 3, 0, 0)],
                         seed=21)
    far = gen.make_far(inp, 12, seed=22)
    ref = oracle.window_chunk_far(inp, far)
    rk, rv, meta, mz, th = oracle.window_commit_far(inp, far)
    t = gen.to_device(inp, DEV)
    f = gen.to_device(far, DEV)
    out = torch.empty((1, inp.nh, inp.d), dtype=torch.float32, device=DEV)
    for i in range(inp.rows):
        B.attn_window_chunk_far(t["ring_k"], t["ring_v"], t["meta"], t["sink_k"], t["sink_v"],
                                t["q"][i:i + 1], t["chunk_k"][i:i + 1], t["chunk_v"][i:i + 1],
                                f["k_tilde"], f["q_tilde"], f["mu"], f["mz"], f["t_hat"],
                                inp.scale, out=out)
        assert_close(out.cpu().numpy()[0], ref[i], f"far decode row {i}")
        B.attn_window_commit_far(t["ring_k"], t["ring_v"], t["meta"], t["chunk_k"][i:i + 1],
                                 t["chunk_v"][i:i + 1], f["q_tilde"], f["mz"], f["t_hat"],
                                 inp.scale)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(t["meta"].cpu().numpy().astype(np.uint32), meta)
    np.testing.assert_array_equal(t["ring_k"].cpu().numpy(), rk)
    np.testing.assert_array_equal(t["ring_v"].cpu().numpy(), rv)
    assert_mz_close(f["mz"].cpu().numpy(), mz, far.m, "mz")
    assert_close(f["t_hat"].cpu().numpy(), th, "t_hat")


def test_far_workspace_reuse_with_stale_bytes():
    """The far call fills every slot it merges: stale bytes in the workspace do not leak."""
    _case("far workspace reuse")
    inp, far = _far_inputs((17, 3, 4, 128, 50, 4, 16, "mix", "positive"))
    ref = oracle.window_chunk_far(inp, far)
    ws = B.Workspace(DEV)
    ws.get(B.chunk_far_workspace_bytes(17, 3, 4, 128, 50, 4, 16))
    ws.buf[64 * 1024:] = 0x55
    for _ in range(2):
        assert_close(gpu_chunk_far(inp, far, workspace=ws), ref, "far with stale workspace")


def test_one_row_far_calls_leave_the_counters_at_zero():
    """One-row far calls take the single launch, whose far part and splits raise ready flags in
    the workspace's counter region: calls of different shapes on one workspace (stale bytes
    past the counters) each match the oracle, and the counters are all zero afterwards."""
    _case("one-row far calls, shared workspace")
    shapes = [(1, 8, 4, 128, 4096, 4, 16, "full", "positive"),
              (1, 2, 2, 256, 70, 3, 12, "mix", "signed"),
              (1, 3, 4, 64, 300, 0, 64, "partial", "signed"),
              (1, 8, 4, 128, 4096, 4, 16, "full", "positive")]
    need = max(B.chunk_far_workspace_bytes(*s[:7]) for s in shapes)
    ws = B.Workspace(DEV)
    ws.get(need)
    ws.buf[64 * 1024:] = 0x55
    for shape in shapes:
        inp, far = _far_inputs(shape)
        assert_close(gpu_chunk_far(inp, far, workspace=ws), oracle.window_chunk_far(inp, far),
                     f"one-row far {shape}")
        assert int(torch.count_nonzero(ws.buf[:64 * 1024])) == 0, f"counters left set after {shape}"
