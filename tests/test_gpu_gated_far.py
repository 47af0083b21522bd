"""Parity of the gated one-row far-field call (attn_window_gated_far) with the CPU oracle, on
seeded synthetic inputs (inputs.make_gated_far).

Bar (per element): |gpu - oracle| <= max(1e-4 * |oracle|, 1e-5), as for the other calls.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
from sliding_window_gqa_group_amd import binding as B
from sliding_window_gqa_group_amd import inputs as gen
from test_gpu_parity import _case, assert_close

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


def _inputs(shape):
    nh, nk, hd, w, ns, m, lens, fars, scale, rect, mu_kind = shape
    rng = np.random.default_rng(zlib.crc32(repr(shape).encode()))
    meta = []
    for kh in range(nk):
        ln = w if lens == "full" else int(rng.integers(0 if ns else 1, w + 1))
        fa = 0 if (fars == "mixed" and kh % 2) else int(rng.integers(1, 1000))
        meta.append((ln, int(rng.integers(0, w)), fa, 0))
    return gen.make_gated_far(nh, nk, hd, w, ns, m, meta, seed=int(rng.integers(1 << 30)),
                              scale=scale, rect=rect, mu_kind=mu_kind)


def gpu_gated_far(inp, workspace=None):
    t = gen.to_device(inp, DEV)
    ns = inp.ns
    z = B.attn_window_gated_far(t["q"], t["ring_k"], t["ring_v"], t["meta"],
                                t["sink_k"] if ns else None, t["sink_v"] if ns else None,
                                t["k_tilde"], t["mu"], t["mz"], t["t_hat"], t["gate"],
                                t["gate_scale"], inp.scale, rect=inp.rect, workspace=workspace)
    torch.cuda.synchronize()
    return z.cpu().numpy()


CASES = [
    # nh, nk, hd, w, ns, m, ring lens, far, scale, rect, mu
    (16, 4, 256, 1024, 0, 32, "full", "all", 1 / 16, 0, "positive"),     # the gated shapes, one row
    (16, 4, 256, 1024, 0, 32, "full", "mixed", 16.0, 1, "signed"),
    (32, 8, 128, 4096, 4, 16, "full", "mixed", 128 ** -0.5, 0, "positive"),   # decode shapes
    (8, 1, 64, 40, 2, 64, "partial", "all", 4.0, 1, "signed"),
    (12, 4, 36, 9, 1, 5, "partial", "mixed", 1.0, 0, "signed"),
    (32, 2, 128, 300, 3, 8, "partial", "all", 8.0, 1, "positive"),        # 16 heads per KV head
    (64, 2, 128, 200, 0, 16, "full", "mixed", 4.0, 0, "signed"),          # 32 heads per KV head
    (64, 2, 256, 100, 2, 8, "partial", "all", 2.0, 1, "positive"),
    (4, 4, 64, 1, 0, 3, "full", "all", 1.0, 0, "positive"),               # window of one
]

VARIANTS = {
    "auto": {},
    "register_many_splits": {B.TUNE_FORCE_KERNEL: 1, B.TUNE_TILES_PER_SPLIT: 1},
    "mfma_many_splits": {B.TUNE_FORCE_KERNEL: 2, B.TUNE_TILES_PER_SPLIT: 1},
    "lds_vector_many_splits": {B.TUNE_FORCE_KERNEL: 3, B.TUNE_TILES_PER_SPLIT: 1},
    "mfma16_many_splits": {B.TUNE_FORCE_KERNEL: 4, B.TUNE_TILES_PER_SPLIT: 1},
    # up to 8 query vectors per KV head: the far part inside the single-launch slot-order
    # kernel (kernel 5) with other splits than its plan picks (the gated heads, d 256: 64
    # splits and 68 ready flags per gatherer, or 16 splits, instead of 32); other shapes take
    # their usual plan
    "decode_one_launch_one_tile": {B.TUNE_FORCE_KERNEL: 5, B.TUNE_TILES_PER_SPLIT: 1},
    "decode_one_launch_four_tiles": {B.TUNE_FORCE_KERNEL: 5, B.TUNE_TILES_PER_SPLIT: 4},
}


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("shape", CASES, ids=[f"h{c[0]}k{c[1]}d{c[2]}w{c[3]}s{c[4]}m{c[5]}{c[6]}{c[7]}r{c[9]}{c[10][0]}" for c in CASES])
def test_gated_far_matches_oracle(shape, variant):
    _case(f"gated far {shape} {variant}")
    inp = _inputs(shape)
    ref = oracle.window_gated_far(inp)
    try:
        for knob, val in VARIANTS[variant].items():
            B.tuning_set(knob, val)
        got = gpu_gated_far(inp)
    finally:
        for knob in VARIANTS[variant]:
            B.tuning_set(knob, 0)
    assert_close(got, ref, f"gated far {shape} {variant}")


def test_gated_far_stale_workspace():
    _case("gated far stale workspace")
    inp = _inputs(CASES[2])
    ref = oracle.window_gated_far(inp)
    ws = B.Workspace(DEV)
    ws.get(B.gated_far_workspace_bytes(inp.nh, inp.nk, inp.hd, inp.w, inp.ns, inp.m))
    ws.buf[64 * 1024:] = 0x55
    for _ in range(2):
        assert_close(gpu_gated_far(inp, workspace=ws), ref, "gated far, stale workspace")


def test_gated_far_calls_leave_the_counters_at_zero():
    """The single launch's far part and splits raise ready flags in the workspace's counter
    region: gated one-row far calls of several shapes on one workspace (stale bytes past the
    counters) each match the oracle and leave the counters all zero."""
    _case("gated far calls, shared workspace")
    shapes = [CASES[0], CASES[2], CASES[3], CASES[4], CASES[0]]
    need = max(B.gated_far_workspace_bytes(*c[:6]) for c in shapes)
    ws = B.Workspace(DEV)
    ws.get(need)
    ws.buf[64 * 1024:] = 0x55
    for shape in shapes:
        inp = _inputs(shape)
        assert_close(gpu_gated_far(inp, workspace=ws), oracle.window_gated_far(inp),
                     f"gated far {shape}")
        assert int(torch.count_nonzero(ws.buf[:64 * 1024])) == 0, f"counters left set after {shape}"
