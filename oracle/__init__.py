"""CPU oracle for windowed grouped-query attention (ctypes binding of ``oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package; the product path (the HIP library and its binding) never does, and shares
no code with it. Arrays are numpy, host memory; results are f32 computed in f64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

_f32p = ctypes.POINTER(ctypes.c_float)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_i32p = ctypes.POINTER(ctypes.c_int32)
_f64p = ctypes.POINTER(ctypes.c_double)


def compile_source(src: str, so: str) -> str:
    """gcc -O2 -fopenmp (strict IEEE: no fast-math) of one C file into a shared library."""
    tmp = so + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall",
                           "-Wno-unknown-pragmas", "-Wno-maybe-uninitialized", src, "-o", tmp,
                           "-lm"])
    os.replace(tmp, so)
    return so


def build(force: bool = True) -> str:
    """Compile liboracle.so next to its source."""
    if force or not os.path.exists(_SO):
        compile_source(_SRC, _SO)
    return _SO


def source_path() -> str:
    return _SRC


def load_library(path: str):
    """A ctypes handle on a compiled oracle library with its signatures declared."""
    lib = ctypes.CDLL(path)
    i, f = ctypes.c_int, ctypes.c_float
    lib.oracle_window_chunk.argtypes = [_f32p, _f32p, _u32p, _f32p, _f32p, _f32p, _f32p, _f32p,
                                        _f32p, i, i, i, i, i, i, f]
    lib.oracle_window_chunk_select.argtypes = [_f32p, _f32p, _u32p, _f32p, _f32p, _f32p,
                                               _f32p, _f32p, i, i, i, i, i, i, f, _i32p,
                                               _i32p, i, _f32p]
    lib.oracle_window_chunk_weights.argtypes = [_f32p, _f32p, _u32p, _f32p, _f32p, _f32p,
                                                _f32p, _f32p, i, i, i, i, i, i, f, i, i, _f64p]
    lib.oracle_window_gated.argtypes = [_f32p, _f32p, _f32p, _f32p, _f32p, _f32p, _f32p,
                                        _f32p, _f32p, _f32p, i, i, i, i, i, i, i, f, f]
    lib.oracle_meta_ok.argtypes = [_u32p, i, i]
    lib.oracle_window_commit.argtypes = [_f32p, _f32p, _u32p, _f32p, _f32p, i, i, i, i]
    lib.oracle_window_chunk_far.argtypes = [_f32p, _f32p, _u32p, _f32p, _f32p, _f32p, _f32p,
                                            _f32p, _f32p, _f32p, _f32p, _f32p, _f32p, _f32p,
                                            i, i, i, i, i, i, i, f]
    lib.oracle_window_commit_far.argtypes = [_f32p, _f32p, _u32p, _f32p, _f32p, _f32p, _f32p,
                                             _f32p, i, i, i, i, i, i, f]
    lib.oracle_window_gated_far.argtypes = [_f32p, _f32p, _f32p, _u32p, _f32p, _f32p, _f32p,
                                            _f32p, _f32p, _f32p, _f32p, _f32p, _f32p,
                                            i, i, i, i, i, i, f, i]
    lib.oracle_encoder_attention.argtypes = [_f32p, _f32p, _f32p, _f32p, _u32p, i, i, i, i, i,
                                             i, i, i, i, f]
    lib.oracle_threads.argtypes = []
    lib.oracle_threads.restype = ctypes.c_int
    for name in ("oracle_encoder_attention", "oracle_window_chunk", "oracle_window_chunk_select",
                 "oracle_window_chunk_weights", "oracle_window_gated", "oracle_meta_ok",
                 "oracle_window_commit", "oracle_window_chunk_far", "oracle_window_commit_far",
                 "oracle_window_gated_far"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        _lib = load_library(_SO)
    return _lib


def use_library(lib) -> None:
    """Route this module's calls through another compiled oracle (the mutation tests use it)."""
    global _lib
    _lib = lib


def _f32(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a, a.ctypes.data_as(_f32p)


def _opt_f32(a):
    if a is None or a.size == 0:
        return None, None
    return _f32(a)


def _chunk_ptrs(inp):
    arrs = {}
    arrs["rk"], prk = _f32(inp.ring_k)
    arrs["rv"], prv = _f32(inp.ring_v)
    arrs["meta"] = np.ascontiguousarray(inp.meta, dtype=np.uint32)
    pm = arrs["meta"].ctypes.data_as(_u32p)
    arrs["sk"], psk = _opt_f32(inp.sink_k)
    arrs["sv"], psv = _opt_f32(inp.sink_v)
    arrs["q"], pq = _f32(inp.q)
    arrs["ck"], pck = _f32(inp.chunk_k)
    arrs["cv"], pcv = _f32(inp.chunk_v)
    return arrs, (prk, prv, pm, psk, psv, pq, pck, pcv)


def window_chunk(inp) -> np.ndarray:
    """out [rows][nh][d] for a ChunkInputs-like object."""
    lib = _load()
    keep, ptrs = _chunk_ptrs(inp)
    out = np.zeros((inp.rows, inp.ng * inp.hpg, inp.d), dtype=np.float32)
    rc = lib.oracle_window_chunk(*ptrs, out.ctypes.data_as(_f32p), inp.rows, inp.ng, inp.hpg,
                                 inp.d, inp.w, inp.ns, inp.scale)
    if rc != 0:
        raise ValueError(f"oracle_window_chunk rejected its arguments (rc={rc})")
    return out


def window_chunk_select(inp, rows_sel, heads_sel) -> np.ndarray:
    """out[k] = output vector of (rows_sel[k], heads_sel[k]); shape [len][d]."""
    lib = _load()
    keep, ptrs = _chunk_ptrs(inp)
    rs = np.ascontiguousarray(rows_sel, dtype=np.int32)
    hs = np.ascontiguousarray(heads_sel, dtype=np.int32)
    out = np.zeros((rs.size, inp.d), dtype=np.float32)
    rc = lib.oracle_window_chunk_select(*ptrs, inp.rows, inp.ng, inp.hpg, inp.d, inp.w, inp.ns,
                                        inp.scale, rs.ctypes.data_as(_i32p),
                                        hs.ctypes.data_as(_i32p), rs.size,
                                        out.ctypes.data_as(_f32p))
    if rc != 0:
        raise ValueError(f"oracle_window_chunk_select rejected its arguments (rc={rc})")
    return out


def window_chunk_weights(inp, row: int, gh: int) -> np.ndarray:
    """Normalised weights of (row, gh) in key-list order: sinks, then window oldest->newest."""
    lib = _load()
    keep, ptrs = _chunk_ptrs(inp)
    wts = np.zeros(inp.ns + inp.w, dtype=np.float64)
    n = lib.oracle_window_chunk_weights(*ptrs, inp.rows, inp.ng, inp.hpg, inp.d, inp.w, inp.ns,
                                        inp.scale, row, gh, wts.ctypes.data_as(_f64p))
    if n < 0:
        raise ValueError("oracle_window_chunk_weights rejected its arguments")
    return wts[:n].copy()


def window_gated(inp):
    """(z [rows][nh][hd], ring_k after, ring_v after) for a GatedInputs-like object."""
    lib = _load()
    rk = np.array(inp.ring_k, dtype=np.float32, copy=True, order="C")
    rv = np.array(inp.ring_v, dtype=np.float32, copy=True, order="C")
    keep = [_f32(a) for a in (inp.yq, inp.yk, inp.yv, inp.rope, inp.q_scale, inp.gate,
                              inp.gate_scale)]
    out = np.zeros((inp.rows, inp.nh, inp.hd), dtype=np.float32)
    rc = lib.oracle_window_gated(*[p for _, p in keep], rk.ctypes.data_as(_f32p),
                                 rv.ctypes.data_as(_f32p), out.ctypes.data_as(_f32p), inp.rows,
                                 inp.pos0, inp.cap, inp.window, inp.nh, inp.nk, inp.hd, inp.scale,
                                 inp.eps)
    if rc != 0:
        raise ValueError(f"oracle_window_gated rejected its arguments (rc={rc})")
    return out, rk, rv


def window_commit(inp):
    """(ring_k, ring_v, meta) after pushing the chunk's K/V rows into the rings of a
    ChunkInputs-like object (inputs untouched)."""
    lib = _load()
    rk = np.array(inp.ring_k, dtype=np.float32, copy=True, order="C")
    rv = np.array(inp.ring_v, dtype=np.float32, copy=True, order="C")
    meta = np.array(inp.meta, dtype=np.uint32, copy=True, order="C")
    ck, pck = _f32(inp.chunk_k)
    cv, pcv = _f32(inp.chunk_v)
    rc = lib.oracle_window_commit(rk.ctypes.data_as(_f32p), rv.ctypes.data_as(_f32p),
                                  meta.ctypes.data_as(_u32p), pck, pcv, inp.rows, inp.ng, inp.d,
                                  inp.w)
    if rc != 0:
        raise ValueError(f"oracle_window_commit rejected its arguments (rc={rc})")
    return rk, rv, meta


def window_chunk_far(inp, far) -> np.ndarray:
    """out [rows][nh][d] of a chunk call with the far field `far` (a FarState-like object)."""
    lib = _load()
    keep, ptrs = _chunk_ptrs(inp)
    fk = [_f32(a) for a in (far.k_tilde, far.q_tilde, far.mu, far.mz, far.t_hat)]
    out = np.zeros((inp.rows, inp.ng * inp.hpg, inp.d), dtype=np.float32)
    rc = lib.oracle_window_chunk_far(*ptrs, *[p for _, p in fk], out.ctypes.data_as(_f32p),
                                     inp.rows, inp.ng, inp.hpg, inp.d, inp.w, inp.ns, far.m,
                                     inp.scale)
    if rc != 0:
        raise ValueError(f"oracle_window_chunk_far rejected its arguments (rc={rc})")
    return out


def window_commit_far(inp, far):
    """(ring_k, ring_v, meta, mz, t_hat) after committing the chunk with its far state (inputs
    untouched)."""
    lib = _load()
    rk = np.array(inp.ring_k, dtype=np.float32, copy=True, order="C")
    rv = np.array(inp.ring_v, dtype=np.float32, copy=True, order="C")
    meta = np.array(inp.meta, dtype=np.uint32, copy=True, order="C")
    mz = np.array(far.mz, dtype=np.float32, copy=True, order="C")
    th = np.array(far.t_hat, dtype=np.float32, copy=True, order="C")
    ck, pck = _f32(inp.chunk_k)
    cv, pcv = _f32(inp.chunk_v)
    qt, pqt = _f32(far.q_tilde)
    rc = lib.oracle_window_commit_far(rk.ctypes.data_as(_f32p), rv.ctypes.data_as(_f32p),
                                      meta.ctypes.data_as(_u32p), pck, pcv, pqt,
                                      mz.ctypes.data_as(_f32p), th.ctypes.data_as(_f32p),
                                      inp.rows, inp.ng, inp.hpg, inp.d, inp.w, far.m, inp.scale)
    if rc != 0:
        raise ValueError(f"oracle_window_commit_far rejected its arguments (rc={rc})")
    return rk, rv, meta, mz, th


def window_gated_far(inp) -> np.ndarray:
    """z [nh][hd] of the gated one-row call with the far field, for a GatedFarInputs-like
    object (q [nh][hd], ring_k/ring_v [nk][w][hd], meta [nk][4], sinks [nk][ns][hd] or empty,
    k_tilde [nk][m][hd], mu [nh][m][m], mz [nh][2m], t_hat [nh][m][hd], gate and gate_scale
    [nh*hd], scale, rect)."""
    lib = _load()
    nk, w, hd = inp.ring_k.shape
    nh = inp.q.shape[0]
    ns = inp.sink_k.shape[1] if inp.sink_k is not None else 0
    m = inp.mu.shape[1]
    keep = [_f32(a) for a in (inp.q, inp.ring_k, inp.ring_v)]
    meta = np.ascontiguousarray(inp.meta, dtype=np.uint32)
    sk = _f32(inp.sink_k) if ns else (None, None)
    sv = _f32(inp.sink_v) if ns else (None, None)
    rest = [_f32(a) for a in (inp.k_tilde, inp.mu, inp.mz, inp.t_hat, inp.gate, inp.gate_scale)]
    out = np.zeros((nh, hd), dtype=np.float32)
    rc = lib.oracle_window_gated_far(*[p for _, p in keep], meta.ctypes.data_as(_u32p), sk[1],
                                     sv[1], *[p for _, p in rest], out.ctypes.data_as(_f32p),
                                     nh, nk, hd, w, ns, m, inp.scale, int(inp.rect))
    if rc != 0:
        raise ValueError(f"oracle_window_gated_far rejected its arguments (rc={rc})")
    return out


def encoder_attention(inp, out=None) -> np.ndarray:
    """out [tokens][ldo] of encoder attention for an EncoderInputs-like object (q, k, v row
    arrays [tokens][ld*], segs [nseg][2] u32, nh, nk, hd, window, scale). Rows outside every
    sequence keep the values of `out` (zeros if not given)."""
    lib = _load()
    keep = [_f32(a) for a in (inp.q, inp.k, inp.v)]
    if out is None:
        out = np.zeros((inp.q.shape[0], inp.nh * inp.hd), dtype=np.float32)
    out = np.array(out, dtype=np.float32, copy=True, order="C")
    segs = np.ascontiguousarray(inp.segs, dtype=np.uint32)
    rc = lib.oracle_encoder_attention(*[p for _, p in keep], out.ctypes.data_as(_f32p),
                                      segs.ctypes.data_as(_u32p), segs.shape[0],
                                      inp.q.shape[1], inp.k.shape[1], inp.v.shape[1],
                                      out.shape[1], inp.nh, inp.nk, inp.hd, inp.window,
                                      inp.scale)
    if rc != 0:
        raise ValueError(f"oracle_encoder_attention rejected its arguments (rc={rc})")
    return out


def threads() -> int:
    """Threads the oracle's parallel loops use (its OpenMP team size)."""
    return int(_load().oracle_threads())


def meta_ok(meta, ng: int, w: int) -> bool:
    lib = _load()
    m = np.ascontiguousarray(meta, dtype=np.uint32)
    return bool(lib.oracle_meta_ok(m.ctypes.data_as(_u32p), ng, w))
