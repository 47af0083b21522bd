"""Seeded synthetic inputs for windowed grouped-query attention over a ring buffer.

This module only draws numbers and lays them out; it holds none of the attention arithmetic.
Both the HIP path (through the binding) and the CPU oracle are fed from the arrays built here.

Layouts follow the header comment of the o1c page ("A sealed layer's attention for a chunk of
rows, on Metal"): ring k/v ``[g][w][d]``, sink k/v ``[g][ns][d]``, q ``[row][nh][d]``, chunk k/v
``[row][g][d]``, out ``[row][nh][d]``, and ``meta[g*4] = len | head | far_len | window``.
The gated layouts follow the dory page ("Dory's token path", ``dory_prep``): raw yq
``[row][nh][hd]``, yk/yv ``[row][nk][hd]``, a RoPE table row per position whose first half is
cos and second half sin, a learned query scale ``[nh][hd]``, a gate ``[row][nh*hd]`` with its scale
``[nh*hd]``, and a position-indexed ring ``[cap][nk][hd]``.

Draw order per config (numpy PCG64, seed = config index): meta draws, ring K, ring V, sink K,
sink V, q, chunk K, chunk V; gated: ring K, ring V, yq, yk, yv, q_scale, gate, gate_scale.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


@dataclass
class ChunkInputs:
    """Inputs of one windowed-attention call over a chunk of rows."""
    name: str
    rows: int
    ng: int
    hpg: int
    d: int
    w: int
    ns: int
    scale: float
    meta: np.ndarray          # uint32 [ng][4]
    ring_k: np.ndarray        # f32 [ng][w][d]
    ring_v: np.ndarray        # f32 [ng][w][d]
    sink_k: np.ndarray        # f32 [ng][ns][d]
    sink_v: np.ndarray        # f32 [ng][ns][d]
    q: np.ndarray             # f32 [rows][nh][d]
    chunk_k: np.ndarray       # f32 [rows][ng][d]
    chunk_v: np.ndarray       # f32 [rows][ng][d]
    seed: int = 0

    @property
    def nh(self) -> int:
        return self.ng * self.hpg


@dataclass
class GatedInputs:
    """Inputs of one gated unit-head windowed-attention call."""
    name: str
    rows: int
    pos0: int
    cap: int
    window: int
    nh: int
    nk: int
    hd: int
    scale: float
    eps: float
    yq: np.ndarray            # f32 [rows][nh][hd]
    yk: np.ndarray            # f32 [rows][nk][hd]
    yv: np.ndarray            # f32 [rows][nk][hd]
    rope: np.ndarray          # f32 [rows][hd]: cos | sin at position pos0+row
    q_scale: np.ndarray       # f32 [nh][hd]
    gate: np.ndarray          # f32 [rows][nh*hd]
    gate_scale: np.ndarray    # f32 [nh*hd]
    ring_k: np.ndarray        # f32 [cap][nk][hd] (state before the call)
    ring_v: np.ndarray        # f32 [cap][nk][hd]
    seed: int = 0


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def make_chunk(rows: int, ng: int, hpg: int, d: int, w: int, ns: int, meta, seed: int,
               name: str = "custom", scale: float | None = None) -> ChunkInputs:
    """Draw ring/sink/q/chunk tensors for given meta rows ``(len, head, far_len, window)``."""
    rng = np.random.Generator(np.random.PCG64(seed))
    meta = np.ascontiguousarray(np.asarray(meta, dtype=np.uint32).reshape(ng, 4))
    return _fill_chunk(rng, name, rows, ng, hpg, d, w, ns, meta, seed, scale)


def _fill_chunk(rng, name, rows, ng, hpg, d, w, ns, meta, seed, scale) -> ChunkInputs:
    nh = ng * hpg
    ring_k = _normal(rng, (ng, w, d))
    ring_v = _normal(rng, (ng, w, d))
    sink_k = _normal(rng, (ng, ns, d))
    sink_v = _normal(rng, (ng, ns, d))
    q = _normal(rng, (rows, nh, d))
    chunk_k = _normal(rng, (rows, ng, d))
    chunk_v = _normal(rng, (rows, ng, d))
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(d)))
    return ChunkInputs(name, rows, ng, hpg, d, w, ns, float(scale), meta, ring_k, ring_v,
                       sink_k, sink_v, q, chunk_k, chunk_v, seed)


def rope_table(rows: int, pos0: int, hd: int, base: float = 10000.0) -> np.ndarray:
    """cos | sin table for positions pos0..pos0+rows-1, computed in f64 and rounded to f32.

    Frequencies theta_i = p * base^(-2i/hd) for i < hd/2, pairing element i with i + hd/2
    (rotate-half). The table is an input of the gated call; the pages take it as a buffer.
    """
    half = hd // 2
    pos = np.arange(pos0, pos0 + rows, dtype=np.float64)[:, None]
    inv_freq = base ** (-2.0 * np.arange(half, dtype=np.float64) / hd)
    ang = pos * inv_freq[None, :]
    return np.ascontiguousarray(np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32))


def make_gated(rows: int, pos0: int, cap: int, window: int, nh: int, nk: int, hd: int, seed: int,
               name: str = "custom", scale: float | None = None, eps: float = 1e-6,
               rope_base: float = 10000.0) -> GatedInputs:
    rng = np.random.Generator(np.random.PCG64(seed))
    # State of the ring before the call: unit-norm keys (a Gaussian direction, normalised
    # without epsilon) and N(0,1) values in every slot.
    rk = rng.standard_normal(size=(cap, nk, hd), dtype=np.float32).astype(np.float64)
    rk /= np.linalg.norm(rk, axis=-1, keepdims=True)
    ring_k = np.ascontiguousarray(rk.astype(np.float32))
    ring_v = _normal(rng, (cap, nk, hd))
    yq = _normal(rng, (rows, nh, hd))
    yk = _normal(rng, (rows, nk, hd))
    yv = _normal(rng, (rows, nk, hd))
    q_scale = rng.uniform(0.5, 1.5, size=(nh, hd)).astype(np.float32)
    gate = _normal(rng, (rows, nh * hd))
    gate_scale = _normal(rng, (nh * hd,))
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(hd)))
    return GatedInputs(name, rows, pos0, cap, window, nh, nk, hd, float(scale), float(eps), yq, yk,
                       yv, rope_table(rows, pos0, hd, rope_base), q_scale, gate, gate_scale,
                       ring_k, ring_v, seed)


# ── The five named workloads ────────────────────────────────────────────────────────────────

def tiny() -> ChunkInputs:
    """1 row, 1 KV group of 4 query heads, d=64, w=16 full ring with head 5, 2 sinks."""
    return make_chunk(1, 1, 4, 64, 16, 2, [(16, 5, 0, 0)], seed=0, name="tiny")


def decode(seed: int = 1) -> ChunkInputs:
    """1 row, 8 KV groups x 4 heads, d=128, w=4096 full ring, seeded head offsets, 4 sinks."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ng, w = 8, 4096
    heads = rng.integers(0, w, size=ng)
    meta = np.array([(w, int(h), 0, 0) for h in heads], dtype=np.uint32)
    return _fill_chunk(rng, "decode", 1, ng, 4, 128, w, 4, meta, seed, None)


def prefill() -> ChunkInputs:
    """512 rows, 8 KV groups x 4 heads, d=128, w=4096, ring len 3000 head 0, 4 sinks."""
    return make_chunk(512, 8, 4, 128, 4096, 4, [(3000, 0, 0, 0)] * 8, seed=2, name="prefill")


def gated() -> GatedInputs:
    """64 rows at pos0=20000, cap 8192, window 1024, 16 q heads over 4 KV heads, hd=256."""
    return make_gated(64, 20000, 8192, 1024, 16, 4, 256, seed=3, name="gated")


def decode_long(seed: int = 5) -> ChunkInputs:
    """The decode shapes over a long window: 1 row, 8 KV groups x 4 heads, d=128, w=32768 full
    ring, seeded head offsets, 4 sinks (268 MB of K/V per call)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ng, w = 8, 32768
    heads = rng.integers(0, w, size=ng)
    meta = np.array([(w, int(h), 0, 0) for h in heads], dtype=np.uint32)
    return _fill_chunk(rng, "decode_long", 1, ng, 4, 128, w, 4, meta, seed, None)


def large_meta(seed: int = 4, ng: int = 8, w: int = 32768):
    """Per-group (len, head, 0, window override) for the Large workload, plus its generator."""
    rng = np.random.Generator(np.random.PCG64(seed))
    rows_meta = []
    for _ in range(ng):
        ov = int(rng.choice([0, 4096, 8192]))
        wg = ov if ov else w
        ln = int(rng.integers(0, wg + 1))
        hd = int(rng.integers(0, wg))
        rows_meta.append((ln, hd, 0, ov))
    return rng, np.array(rows_meta, dtype=np.uint32)


def large(seed: int = 4) -> ChunkInputs:
    """2048 rows, 8 KV groups x 8 heads, d=128, w=32768 with per-group overrides, 4 sinks."""
    rng, meta = large_meta(seed)
    return _fill_chunk(rng, "large", 2048, 8, 8, 128, 32768, 4, meta, seed, None)


CHUNK_CONFIGS = {"tiny": tiny, "decode": decode, "prefill": prefill, "large": large}
GATED_CONFIGS = {"gated": gated}


@dataclass
class FarState:
    """Synthetic far-field state of a chunk call: m landmarks per query head.

    k_tilde [ng][m][d] landmark keys, q_tilde [nh][m][d] landmark queries, mu [nh][m][m]
    mixing weights (row a, column b), mz [nh][2m] far maxima then far masses, t_hat [nh][m][d]
    far numerators. A group whose meta far_len is 0 has an empty far field (maxima -inf, masses
    and numerators 0)."""
    m: int
    k_tilde: np.ndarray
    q_tilde: np.ndarray
    mu: np.ndarray
    mz: np.ndarray
    t_hat: np.ndarray


def make_far(inp: ChunkInputs, m: int, seed: int, mu_kind: str = "positive") -> FarState:
    """Draw a far state for `inp` (its meta's far_len says which groups have one). Landmark
    keys and queries are N(0,1); mu is U(0,1) ("positive") or N(0,1) ("signed"); a non-empty
    field has maxima N(0,1), masses U(0.5, 4) and numerators N(0,1) scaled by the mass."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ng, hpg, d = inp.ng, inp.hpg, inp.d
    nh = ng * hpg
    k_tilde = rng.standard_normal((ng, m, d), dtype=np.float32)
    q_tilde = rng.standard_normal((nh, m, d), dtype=np.float32)
    if mu_kind == "signed":
        mu = rng.standard_normal((nh, m, m), dtype=np.float32)
    else:
        mu = rng.random((nh, m, m), dtype=np.float32)
    mz = np.zeros((nh, 2 * m), dtype=np.float32)
    mz[:, :m] = rng.standard_normal((nh, m), dtype=np.float32)
    mz[:, m:] = rng.uniform(0.5, 4.0, (nh, m)).astype(np.float32)
    t_hat = rng.standard_normal((nh, m, d), dtype=np.float32) * mz[:, m:, None]
    for g in range(ng):
        if int(inp.meta[g, 2]) == 0:
            sl = slice(g * hpg, (g + 1) * hpg)
            mz[sl, :m] = -np.inf
            mz[sl, m:] = 0.0
            t_hat[sl] = 0.0
    return FarState(m, k_tilde, q_tilde, mu, mz, np.ascontiguousarray(t_hat, dtype=np.float32))


@dataclass
class GatedFarInputs:
    """The gated one-row call with the far field: one query per head, the ring after the row's
    own push, sinks, and a far state per query head."""
    q: np.ndarray            # [nh][hd]
    ring_k: np.ndarray       # [nk][w][hd]
    ring_v: np.ndarray       # [nk][w][hd]
    meta: np.ndarray         # [nk][4] u32: len, head (unused), far count, window (unused)
    sink_k: np.ndarray       # [nk][ns][hd]
    sink_v: np.ndarray
    k_tilde: np.ndarray      # [nk][m][hd]
    mu: np.ndarray           # [nh][m][m]
    mz: np.ndarray           # [nh][2m]
    t_hat: np.ndarray        # [nh][m][hd]
    gate: np.ndarray         # [nh*hd]
    gate_scale: np.ndarray   # [nh*hd]
    scale: float
    rect: int

    @property
    def nh(self) -> int:
        return self.q.shape[0]

    @property
    def nk(self) -> int:
        return self.ring_k.shape[0]

    @property
    def hd(self) -> int:
        return self.q.shape[1]

    @property
    def w(self) -> int:
        return self.ring_k.shape[1]

    @property
    def ns(self) -> int:
        return self.sink_k.shape[1]

    @property
    def m(self) -> int:
        return self.mu.shape[1]


def _unit_rows(rng, shape) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32).astype(np.float64)
    x /= np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x.astype(np.float32)


def make_gated_far(nh: int, nk: int, hd: int, w: int, ns: int, m: int, meta, seed: int,
                   scale: float, rect: int = 0, mu_kind: str = "positive") -> GatedFarInputs:
    """Seeded inputs of the gated one-row far call, shaped like the gated path's prepped heads:
    ring, sink and landmark keys are unit vectors, the query is a unit vector times U(0.5, 1.5)
    per component (the learned query scale), values N(0,1); mu U(0,1) ("positive") or N(0,1)
    ("signed"); a head whose KV head has a far count gets far maxima N(0,1) * scale, masses
    U(0.5, 4) and numerators N(0,1) times the mass, the others the empty field (-inf, 0, 0);
    gate and gate_scale N(0,1). `meta` lists (len, head, far count, window) per KV head."""
    rng = np.random.Generator(np.random.PCG64(seed))
    meta = np.asarray(meta, dtype=np.uint32).reshape(nk, 4)
    q = _unit_rows(rng, (nh, hd)) * rng.uniform(0.5, 1.5, (nh, hd)).astype(np.float32)
    ring_k = _unit_rows(rng, (nk, w, hd))
    ring_v = rng.standard_normal((nk, w, hd), dtype=np.float32)
    sink_k = _unit_rows(rng, (nk, ns, hd)) if ns else np.zeros((nk, 0, hd), np.float32)
    sink_v = rng.standard_normal((nk, ns, hd), dtype=np.float32)
    k_tilde = _unit_rows(rng, (nk, m, hd))
    if mu_kind == "signed":
        mu = rng.standard_normal((nh, m, m), dtype=np.float32)
    else:
        mu = rng.random((nh, m, m), dtype=np.float32)
    mz = np.zeros((nh, 2 * m), dtype=np.float32)
    mz[:, :m] = rng.standard_normal((nh, m), dtype=np.float32) * np.float32(scale)
    mz[:, m:] = rng.uniform(0.5, 4.0, (nh, m)).astype(np.float32)
    t_hat = rng.standard_normal((nh, m, hd), dtype=np.float32) * mz[:, m:, None]
    gate = rng.standard_normal(nh * hd, dtype=np.float32)
    gate_scale = rng.standard_normal(nh * hd, dtype=np.float32)
    hpg = nh // nk
    for kh in range(nk):
        if int(meta[kh, 2]) == 0:
            sl = slice(kh * hpg, (kh + 1) * hpg)
            mz[sl, :m] = -np.inf
            mz[sl, m:] = 0.0
            t_hat[sl] = 0.0
    return GatedFarInputs(q.astype(np.float32), ring_k, ring_v, meta, sink_k, sink_v, k_tilde,
                          mu, mz, np.ascontiguousarray(t_hat, dtype=np.float32), gate,
                          gate_scale, float(np.float32(scale)), int(rect))


@dataclass
class EncoderInputs:
    """Encoder attention over packed sequences: q [tokens][ldq], k [tokens][ldk], v
    [tokens][ldv] (head h's values at h*hd of a row), segs [nseg][2] u32 (start, len)."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    segs: np.ndarray
    nh: int
    nk: int
    hd: int
    window: int
    scale: float


def make_encoder(lens, nh: int, nk: int, hd: int, window: int, seed: int, gap: int = 0,
                 pad: int = 0, scale: float | None = None) -> EncoderInputs:
    """Sequences of the given lengths packed one after another (`gap` unused rows between
    them), q/k/v rows N(0,1) with `pad` extra floats per row (row strides nh*hd + pad and
    nk*hd + pad); scale 1/sqrt(hd) unless given."""
    rng = np.random.Generator(np.random.PCG64(seed))
    segs, t = [], 0
    for ln in lens:
        segs.append((t, int(ln)))
        t += int(ln) + gap
    tokens = max(t, 1)
    q = rng.standard_normal((tokens, nh * hd + pad), dtype=np.float32)
    k = rng.standard_normal((tokens, nk * hd + pad), dtype=np.float32)
    v = rng.standard_normal((tokens, nk * hd + pad), dtype=np.float32)
    sc = float(np.float32(1.0 / np.sqrt(hd) if scale is None else scale))
    return EncoderInputs(q, k, v, np.asarray(segs, dtype=np.uint32).reshape(-1, 2), nh, nk, hd,
                         int(window), sc)


def to_device(inp, device="cuda"):
    """The arrays of a ChunkInputs / GatedInputs as contiguous torch tensors on `device`."""
    import torch
    out = {}
    for name, val in vars(inp).items():
        if isinstance(val, np.ndarray):
            if val.dtype == np.uint32:
                out[name] = torch.from_numpy(val.view(np.int32).copy()).to(device)
            else:
                out[name] = torch.from_numpy(np.ascontiguousarray(val)).to(device)
    return out
