"""The allocation-free entry point (attn_window_chunk_noalloc) against attn_window_chunk, through
the C-ABI: the same kernels with the library's static per-device scratch in place of a caller
workspace. Two calls in a row, the second smaller (the scratch keeps the first call's bytes),
plus the decode workload in the in-kernel and separate-launch merge plans."""
import numpy as np
import pytest
import torch

from sliding_window_gqa_group_amd import binding as B
from sliding_window_gqa_group_amd import inputs as gen

pytestmark = pytest.mark.gpu

RTOL, ATOL = 1e-4, 1e-5
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()
    yield
    B.tuning_set(B.TUNE_MERGE_KERNEL, 0)


def _close(got, ref, what):
    got = got.cpu().numpy().astype(np.float64)
    ref = ref.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got)), what
    bad = np.abs(got - ref) > np.maximum(RTOL * np.abs(ref), ATOL)
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} out of tolerance"


def _both(inp):
    t = gen.to_device(inp, DEV)
    sk = t["sink_k"] if inp.ns else None
    sv = t["sink_v"] if inp.ns else None
    ref = B.attn_window_chunk(t["ring_k"], t["ring_v"], t["meta"], sk, sv, t["q"], t["chunk_k"],
                              t["chunk_v"], inp.scale)
    out = torch.full((inp.rows, inp.nh, inp.d), float("nan"), dtype=torch.float32, device=DEV)
    B.attn_window_chunk_noalloc(t["ring_k"], t["ring_v"], t["meta"], sk, sv, t["q"], t["chunk_k"],
                                t["chunk_v"], inp.scale, out)
    torch.cuda.synchronize()
    return out, ref


def test_noalloc_matches_workspace_call_twice_second_smaller():
    print("[case] noalloc: 64-row chunk then decode", flush=True)
    big = gen.make_chunk(64, 4, 4, 128, 2000, 4,
                         [(2000, 17, 0, 0), (900, 3, 0, 0), (512, 100, 0, 1024), (0, 0, 0, 0)],
                         seed=31)
    need = B.chunk_workspace_bytes(big.rows, big.ng, big.hpg, big.d, big.w, big.ns)
    assert 0 < need <= B.NOALLOC_SCRATCH_BYTES
    out, ref = _both(big)
    _close(out, ref, "64-row chunk")
    small = gen.decode()
    assert B.chunk_workspace_bytes(1, 8, 4, 128, 4096, 4) < need
    out, ref = _both(small)
    _close(out, ref, "decode after the 64-row chunk")


@pytest.mark.parametrize("merge", [1, 2])
def test_noalloc_decode_both_merge_plans(merge):
    print(f"[case] noalloc: decode, merge plan {merge}", flush=True)
    try:
        B.tuning_set(B.TUNE_MERGE_KERNEL, merge)
        for seed in (1, 2):
            out, ref = _both(gen.decode(seed=seed))
            _close(out, ref, f"decode seed {seed}")
    finally:
        B.tuning_set(B.TUNE_MERGE_KERNEL, 0)

