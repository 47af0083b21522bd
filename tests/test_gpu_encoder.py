"""Parity of the encoder call (attn_encoder) with the CPU oracle on seeded packed sequences
(inputs.make_encoder). Bar (per element): |gpu - oracle| <= max(1e-4 * |oracle|, 1e-5)."""
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
SENTINEL = 7.5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()
    yield


def gpu_encoder(inp, max_len=None):
    q = torch.from_numpy(inp.q).to(DEV)
    k = torch.from_numpy(inp.k).to(DEV)
    v = torch.from_numpy(inp.v).to(DEV)
    segs = torch.from_numpy(inp.segs.view(np.int32).copy()).to(DEV)
    out = torch.full((inp.q.shape[0], inp.nh * inp.hd + 4), SENTINEL, dtype=torch.float32, device=DEV)
    B.attn_encoder(q, k, v, segs, inp.nh, inp.nk, inp.hd, inp.scale, window=inp.window,
                   max_len=max_len, out=out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check(inp, what):
    ref = oracle.encoder_attention(inp, out=np.full((inp.q.shape[0], inp.nh * inp.hd + 4),
                                                     SENTINEL, np.float32))
    got = gpu_encoder(inp)
    assert_close(got, ref, what)


CASES = [
    # lens, nh, nk, hd, window, gap, pad
    ([1], 4, 4, 64, 0, 0, 0),
    ([7, 33, 128, 129, 200], 8, 2, 64, 0, 2, 4),
    ([500], 12, 4, 64, 5, 0, 0),
    ([64, 65, 300], 8, 1, 128, 0, 1, 4),
    ([257, 31], 16, 16, 64, 64, 3, 0),
    ([100, 90], 6, 2, 36, 3, 0, 8),        # padded head width
    ([150], 4, 2, 100, 1000, 0, 4),        # window wider than the sequence
    ([40, 41, 42], 8, 4, 128, 1, 2, 0),
    ([1, 1, 2, 3], 2, 1, 8, 0, 1, 0),
    ([96, 130], 8, 2, 256, 0, 1, 4),       # wide heads
    ([200], 4, 4, 200, 17, 0, 0),          # padded to 256
]


@pytest.mark.parametrize("case", CASES, ids=[f"l{len(c[0])}x{max(c[0])}h{c[1]}k{c[2]}d{c[3]}w{c[4]}" for c in CASES])
def test_encoder_matches_oracle(case):
    lens, nh, nk, hd, window, gap, pad = case
    _case(f"encoder {case}")
    inp = gen.make_encoder(lens, nh, nk, hd, window, seed=zlib.crc32(repr(case).encode()),
                           gap=gap, pad=pad)
    _check(inp, f"encoder {case}")


def test_encoder_packed_qkv_rows():
    """The page's layout: one buffer of q|k|v rows; q, k and v are column slices of it."""
    _case("encoder packed qkv")
    nh, nk, hd = 8, 2, 64
    lens = [77, 130, 5]
    base = gen.make_encoder(lens, nh, nk, hd, 0, seed=31, gap=1)
    tokens = base.q.shape[0]
    qkv = np.concatenate([base.q, base.k, base.v], axis=1)
    t = torch.from_numpy(qkv).to(DEV)
    q, k, v = t[:, :nh * hd], t[:, nh * hd:(nh + nk) * hd], t[:, (nh + nk) * hd:]
    segs = torch.from_numpy(base.segs.view(np.int32).copy()).to(DEV)
    out = torch.full((tokens, nh * hd), SENTINEL, dtype=torch.float32, device=DEV)
    B.attn_encoder(q, k, v, segs, nh, nk, hd, base.scale, out=out)
    torch.cuda.synchronize()
    ref = oracle.encoder_attention(base, out=np.full((tokens, nh * hd), SENTINEL, np.float32))
    assert_close(out.cpu().numpy(), ref, "packed qkv")


def test_encoder_long_sequence_full_attention():
    """One 2048-position sequence, 16 heads of 64 (the vision tower's head width)."""
    _case("encoder long full")
    inp = gen.make_encoder([2048], 16, 16, 64, 0, seed=41)
    _check(inp, "long full attention")


def test_encoder_max_len_above_every_length():
    """A larger max_len only reserves more (empty) blocks."""
    _case("encoder max_len")
    inp = gen.make_encoder([33, 70], 4, 2, 64, 2, seed=51)
    ref = oracle.encoder_attention(inp, out=np.full((inp.q.shape[0], inp.nh * inp.hd + 4),
                                                     SENTINEL, np.float32))
    assert_close(gpu_encoder(inp, max_len=1000), ref, "max_len 1000")


@pytest.mark.parametrize("order", [1, 2], ids=["round_robin", "runs_per_xcd"])
def test_encoder_work_orders(order):
    """Both XCD work orders give the oracle's result (the automatic one picks by sequence
    count)."""
    _case(f"encoder work order {order}")
    inp = gen.make_encoder([300, 17, 129, 64], 8, 2, 64, 0, seed=61, gap=1)
    try:
        B.tuning_set(B.TUNE_XCD_MAP, order)
        got = gpu_encoder(inp)
    finally:
        B.tuning_set(B.TUNE_XCD_MAP, 0)
    ref = oracle.encoder_attention(inp, out=np.full((inp.q.shape[0], inp.nh * inp.hd + 4),
                                                     SENTINEL, np.float32))
    assert_close(got, ref, f"work order {order}")
