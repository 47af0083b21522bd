"""ctypes binding of libwinattn.so (include/winattn.h) over torch device tensors.

Argument marshalling only: every step of the attention runs in the library's HIP kernels on the
caller's (or torch's current) stream. Missing library => ImportError at first use; there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwinattn.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "winattn.h")

OK, EINVAL, EWORKSPACE, ELAUNCH, EUNSUPPORTED = 0, -1, -2, -3, -4
TUNE_FORCE_KERNEL, TUNE_TILES_PER_SPLIT, TUNE_TARGET_BLOCKS, TUNE_MERGE_KERNEL, TUNE_XCD_MAP = 1, 2, 3, 4, 5

_lib = None
_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t
_ip = ctypes.POINTER(ctypes.c_int)


class WinattnError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed with code {code}: {strerror(code)}")
        self.code = code


def load(path: str = LIB_PATH):
    """Load (once) and return the ctypes handle; raises ImportError if the library is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m sliding_window_gqa_group_amd.build` "
                          "or __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    lib.attn_window_chunk.argtypes = [_vp] * 9 + [_i] * 6 + [_f, _vp, _sz, _vp]
    lib.attn_window_chunk.restype = _i
    lib.attn_window_chunk_noalloc.argtypes = [_vp] * 9 + [_i] * 6 + [_f, _vp]
    lib.attn_window_chunk_noalloc.restype = _i
    lib.attn_window_chunk_workspace.argtypes = [_i] * 6
    lib.attn_window_chunk_workspace.restype = _sz
    lib.attn_window_gated.argtypes = [_vp] * 10 + [_i] * 7 + [_f, _f, _vp, _sz, _vp]
    lib.attn_window_gated.restype = _i
    lib.attn_window_gated_workspace.argtypes = [_i] * 5
    lib.attn_window_gated_workspace.restype = _sz
    lib.attn_workspace_init.argtypes = [_vp, _sz, _vp]
    lib.attn_workspace_init.restype = _i
    lib.attn_window_check_meta.argtypes = [_vp, _i, _i]
    lib.attn_window_check_meta.restype = _i
    lib.attn_window_chunk_plan.argtypes = [_i] * 6 + [_ip] * 4
    lib.attn_window_chunk_plan.restype = _i
    lib.attn_mfma_layout_probe.argtypes = [_vp, _vp]
    lib.attn_mfma_layout_probe.restype = _i
    lib.attn_window_commit.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp]
    lib.attn_window_commit.restype = _i
    lib.attn_mfma16_layout_probe.argtypes = [_vp, _vp]
    lib.attn_mfma16_layout_probe.restype = _i
    lib.attn_window_chunk_far.argtypes = [_vp] * 14 + [_i] * 7 + [_f, _vp, _sz, _vp]
    lib.attn_window_chunk_far.restype = _i
    lib.attn_window_chunk_far_workspace.argtypes = [_i] * 7
    lib.attn_window_chunk_far_workspace.restype = _sz
    lib.attn_window_commit_far.argtypes = [_vp] * 8 + [_i] * 6 + [_f, _vp]
    lib.attn_window_commit_far.restype = _i
    lib.attn_window_gated_far.argtypes = [_vp] * 13 + [_i] * 6 + [_f, _i, _vp, _sz, _vp]
    lib.attn_window_gated_far.restype = _i
    lib.attn_window_gated_far_workspace.argtypes = [_i] * 6
    lib.attn_window_gated_far_workspace.restype = _sz
    lib.attn_encoder.argtypes = [_vp] * 5 + [_i] * 10 + [_f, _vp]
    lib.attn_encoder.restype = _i
    lib.attn_read_probe.argtypes = [_vp, _sz, _vp, _vp]
    lib.attn_read_probe.restype = _i
    lib.attn_tuning_set.argtypes = [_i, _i]
    lib.attn_tuning_set.restype = _i
    lib.attn_strerror.argtypes = [_i]
    lib.attn_strerror.restype = ctypes.c_char_p
    lib.attn_abi_version.argtypes = []
    lib.attn_abi_version.restype = _i
    _lib = lib
    _ws_sizes.clear()
    return lib


def declared_functions(header: str = HEADER):
    """Names of the functions include/winattn.h declares."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", text)))


def strerror(code: int) -> str:
    return load().attn_strerror(int(code)).decode()


def abi_version() -> int:
    return load().attn_abi_version()


# Workspace sizes by call shape: they depend only on the shape and the tuning knobs, so they are
# asked of the library once per shape (cleared when a knob changes or a library is loaded).
_ws_sizes = {}


def tuning_set(knob: int, value: int) -> None:
    rc = load().attn_tuning_set(knob, value)
    _ws_sizes.clear()
    if rc != OK:
        raise WinattnError("attn_tuning_set", rc)


def chunk_workspace_bytes(rows, ng, hpg, d, w, ns) -> int:
    key = ("chunk", rows, ng, hpg, d, w, ns)
    n = _ws_sizes.get(key)
    if n is None:
        n = _ws_sizes[key] = int(load().attn_window_chunk_workspace(rows, ng, hpg, d, w, ns))
    return n


def gated_workspace_bytes(rows, nh, nk, hd, window) -> int:
    key = ("gated", rows, nh, nk, hd, window)
    n = _ws_sizes.get(key)
    if n is None:
        n = _ws_sizes[key] = int(load().attn_window_gated_workspace(rows, nh, nk, hd, window))
    return n


def chunk_far_workspace_bytes(rows, ng, hpg, d, w, ns, m) -> int:
    return load().attn_window_chunk_far_workspace(rows, ng, hpg, d, w, ns, m)


def gated_far_workspace_bytes(nh, nk, hd, w, ns, m) -> int:
    return load().attn_window_gated_far_workspace(nh, nk, hd, w, ns, m)


def chunk_plan(rows, ng, hpg, d, w, ns):
    """(kernel, query block, splits, keys per split) for these sizes, as
    attn_window_chunk_plan reports them (kernel numbers in include/winattn.h)."""
    vals = [ctypes.c_int(0) for _ in range(4)]
    rc = load().attn_window_chunk_plan(rows, ng, hpg, d, w, ns, *[ctypes.byref(v) for v in vals])
    if rc != OK:
        raise WinattnError("attn_window_chunk_plan", rc)
    return tuple(v.value for v in vals)


def check_meta(meta_host, ng: int, w: int) -> int:
    import numpy as np
    m = np.ascontiguousarray(meta_host, dtype=np.uint32)
    return load().attn_window_check_meta(m.ctypes.data, ng, w)


# ── workspaces ──────────────────────────────────────────────────────────────────────────────

class Workspace:
    """Zero-initialised device scratch for one stream; grows on demand (a growth is a fresh
    zeroed allocation, so the counters the library keeps there start at zero)."""

    def __init__(self, device):
        self.device = torch.device(device)
        self.buf = None

    def get(self, nbytes: int):
        if nbytes == 0:
            return None, 0
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        return self.buf.data_ptr(), self.buf.numel()


_workspaces = {}


def _default_workspace(device, stream_ptr):
    key = (torch.device(device).index, stream_ptr)
    ws = _workspaces.get(key)
    if ws is None:
        ws = _workspaces[key] = Workspace(device)
    return ws


def _ptr(t, name, dtypes=(torch.float32,)):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must have dtype {dtypes}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


# torch's current stream of a device as a raw handle, without building a Stream object (that
# costs about 2 us per call, as much as the rest of the argument marshalling); the public route
# where this torch build has no such accessor.
_raw_current_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_ptr(stream, device):
    if stream is None:
        if _raw_current_stream is not None:
            idx = device.index if device.index is not None else torch.cuda.current_device()
            return _raw_current_stream(idx)
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def attn_window_chunk(ring_k, ring_v, meta, sink_k, sink_v, q, chunk_k, chunk_v, scale,
                      out=None, workspace=None, stream=None):
    """out[rows][nh][d] = windowed GQA attention of a chunk (see include/winattn.h).

    ring_k/ring_v [ng][w][d], meta [ng][4] int32/uint32, sink_k/sink_v [ng][ns][d] (or None),
    q [rows][nh][d], chunk_k/chunk_v [rows][ng][d].
    """
    ng, w, d = ring_k.shape
    rows, nh, dq = q.shape
    if dq != d or nh % ng:
        raise ValueError("q must be [rows][ng*hpg][d] matching ring_k [ng][w][d]")
    ns = 0 if sink_k is None else sink_k.shape[1]
    if out is None:
        out = torch.empty((rows, nh, d), dtype=torch.float32, device=q.device)
    st = _stream_ptr(stream, q.device)
    need = chunk_workspace_bytes(rows, ng, nh // ng, d, w, ns)
    ws = workspace if workspace is not None else _default_workspace(q.device, st)
    wp, wb = ws.get(need)
    rc = load().attn_window_chunk(
        _ptr(ring_k, "ring_k"), _ptr(ring_v, "ring_v"),
        _ptr(meta, "meta", (torch.int32, torch.uint32)), _ptr(sink_k, "sink_k"),
        _ptr(sink_v, "sink_v"), _ptr(q, "q"), _ptr(chunk_k, "chunk_k"), _ptr(chunk_v, "chunk_v"),
        _ptr(out, "out"), rows, ng, nh // ng, d, w, ns, float(scale), wp, wb, st)
    if rc != OK:
        raise WinattnError("attn_window_chunk", rc)
    return out


NOALLOC_SCRATCH_BYTES = 32 << 20   # WINATTN_NOALLOC_SCRATCH_BYTES


def attn_window_chunk_noalloc(ring_k, ring_v, meta, sink_k, sink_v, q, chunk_k, chunk_v, scale,
                              out, stream=None):
    """attn_window_chunk with the library's static per-device scratch instead of a workspace
    (see attn_window_chunk_noalloc in include/winattn.h). `out` is required: nothing is
    allocated on this path."""
    ng, w, d = ring_k.shape
    rows, nh, dq = q.shape
    if dq != d or nh % ng or tuple(out.shape) != (rows, nh, d):
        raise ValueError("q and out must be [rows][ng*hpg][d] matching ring_k [ng][w][d]")
    ns = 0 if sink_k is None else sink_k.shape[1]
    rc = load().attn_window_chunk_noalloc(
        _ptr(ring_k, "ring_k"), _ptr(ring_v, "ring_v"),
        _ptr(meta, "meta", (torch.int32, torch.uint32)), _ptr(sink_k, "sink_k"),
        _ptr(sink_v, "sink_v"), _ptr(q, "q"), _ptr(chunk_k, "chunk_k"), _ptr(chunk_v, "chunk_v"),
        _ptr(out, "out"), rows, ng, nh // ng, d, w, ns, float(scale), _stream_ptr(stream, q.device))
    if rc != OK:
        raise WinattnError("attn_window_chunk_noalloc", rc)
    return out


def attn_window_gated(yq, yk, yv, rope, q_scale, gate, gate_scale, ring_k, ring_v, pos0, window,
                      scale, eps, out=None, workspace=None, stream=None):
    """z[rows][nh][hd] of the gated unit-head call; writes the rows' ring slots."""
    rows, nh, hd = yq.shape
    nk = yk.shape[1]
    cap = ring_k.shape[0]
    if out is None:
        out = torch.empty((rows, nh, hd), dtype=torch.float32, device=yq.device)
    st = _stream_ptr(stream, yq.device)
    need = gated_workspace_bytes(rows, nh, nk, hd, window)
    ws = workspace if workspace is not None else _default_workspace(yq.device, st)
    wp, wb = ws.get(need)
    rc = load().attn_window_gated(
        _ptr(yq, "yq"), _ptr(yk, "yk"), _ptr(yv, "yv"), _ptr(rope, "rope"),
        _ptr(q_scale, "q_scale"), _ptr(gate, "gate"), _ptr(gate_scale, "gate_scale"),
        _ptr(ring_k, "ring_k"), _ptr(ring_v, "ring_v"), _ptr(out, "out"), rows, int(pos0), cap,
        int(window), nh, nk, hd, float(scale), float(eps), wp, wb, st)
    if rc != OK:
        raise WinattnError("attn_window_gated", rc)
    return out


def mfma_layout_probe(device="cuda", stream=None):
    """[64][16] accumulator map of one 32x32x2 f32 matrix-core product (see the header)."""
    out = torch.full((64, 16), -1.0, dtype=torch.float32, device=device)
    rc = load().attn_mfma_layout_probe(out.data_ptr(), _stream_ptr(stream, out.device))
    if rc != OK:
        raise WinattnError("attn_mfma_layout_probe", rc)
    return out


def attn_window_commit(ring_k, ring_v, meta, chunk_k, chunk_v, stream=None) -> None:
    """Push the chunk's K/V rows [rows][ng][d] into the rings [ng][w][d] and advance meta
    [ng][4] in place (see attn_window_commit in include/winattn.h)."""
    ng, w, d = ring_k.shape
    rows = chunk_k.shape[0]
    if (tuple(ring_v.shape) != (ng, w, d) or tuple(chunk_k.shape) != (rows, ng, d)
            or tuple(chunk_v.shape) != (rows, ng, d) or tuple(meta.shape) != (ng, 4)):
        raise ValueError("attn_window_commit: rings [ng][w][d], chunk [rows][ng][d], meta [ng][4]")
    rc = load().attn_window_commit(
        _ptr(ring_k, "ring_k"), _ptr(ring_v, "ring_v"),
        _ptr(meta, "meta", (torch.int32, torch.uint32)), _ptr(chunk_k, "chunk_k"),
        _ptr(chunk_v, "chunk_v"), rows, ng, d, w, _stream_ptr(stream, ring_k.device))
    if rc != OK:
        raise WinattnError("attn_window_commit", rc)


def _far_shapes(ring_k, q_tilde, mz, t_hat):
    ng, w, d = ring_k.shape
    nh, m, dq = q_tilde.shape
    if dq != d or nh % ng or tuple(mz.shape) != (nh, 2 * m) or tuple(t_hat.shape) != (nh, m, d):
        raise ValueError("far state: q_tilde [nh][m][d], mz [nh][2m], t_hat [nh][m][d]")
    return ng, w, d, nh, m


def attn_window_chunk_far(ring_k, ring_v, meta, sink_k, sink_v, q, chunk_k, chunk_v, k_tilde,
                          q_tilde, mu, mz, t_hat, scale, out=None, workspace=None, stream=None):
    """out[rows][nh][d] = windowed GQA attention of a chunk plus the far field of landmark
    summaries (see attn_window_chunk_far in include/winattn.h). k_tilde [ng][m][d],
    q_tilde [nh][m][d], mu [nh][m][m], mz [nh][2m], t_hat [nh][m][d]."""
    ng, w, d, nh, m = _far_shapes(ring_k, q_tilde, mz, t_hat)
    rows = q.shape[0]
    if tuple(q.shape) != (rows, nh, d) or tuple(k_tilde.shape) != (ng, m, d) \
            or tuple(mu.shape) != (nh, m, m):
        raise ValueError("attn_window_chunk_far: q [rows][nh][d], k_tilde [ng][m][d], mu [nh][m][m]")
    ns = 0 if sink_k is None else sink_k.shape[1]
    if out is None:
        out = torch.empty((rows, nh, d), dtype=torch.float32, device=q.device)
    st = _stream_ptr(stream, q.device)
    need = chunk_far_workspace_bytes(rows, ng, nh // ng, d, w, ns, m)
    ws = workspace if workspace is not None else _default_workspace(q.device, st)
    wp, wb = ws.get(need)
    rc = load().attn_window_chunk_far(
        _ptr(ring_k, "ring_k"), _ptr(ring_v, "ring_v"),
        _ptr(meta, "meta", (torch.int32, torch.uint32)), _ptr(sink_k, "sink_k"),
        _ptr(sink_v, "sink_v"), _ptr(q, "q"), _ptr(chunk_k, "chunk_k"), _ptr(chunk_v, "chunk_v"),
        _ptr(k_tilde, "k_tilde"), _ptr(q_tilde, "q_tilde"), _ptr(mu, "mu"), _ptr(mz, "mz"),
        _ptr(t_hat, "t_hat"), _ptr(out, "out"), rows, ng, nh // ng, d, w, ns, m, float(scale),
        wp, wb, st)
    if rc != OK:
        raise WinattnError("attn_window_chunk_far", rc)
    return out


def attn_window_commit_far(ring_k, ring_v, meta, chunk_k, chunk_v, q_tilde, mz, t_hat, scale,
                           stream=None) -> None:
    """Update the far state (mz, t_hat) with the chunk's evictions, then push the chunk into
    the rings and advance meta, all in place (see attn_window_commit_far in
    include/winattn.h)."""
    ng, w, d, nh, m = _far_shapes(ring_k, q_tilde, mz, t_hat)
    rows = chunk_k.shape[0]
    if (tuple(ring_v.shape) != (ng, w, d) or tuple(chunk_k.shape) != (rows, ng, d)
            or tuple(chunk_v.shape) != (rows, ng, d) or tuple(meta.shape) != (ng, 4)):
        raise ValueError("attn_window_commit_far: rings [ng][w][d], chunk [rows][ng][d], meta [ng][4]")
    rc = load().attn_window_commit_far(
        _ptr(ring_k, "ring_k"), _ptr(ring_v, "ring_v"),
        _ptr(meta, "meta", (torch.int32, torch.uint32)), _ptr(chunk_k, "chunk_k"),
        _ptr(chunk_v, "chunk_v"), _ptr(q_tilde, "q_tilde"), _ptr(mz, "mz"), _ptr(t_hat, "t_hat"),
        rows, ng, nh // ng, d, w, m, float(scale), _stream_ptr(stream, ring_k.device))
    if rc != OK:
        raise WinattnError("attn_window_commit_far", rc)


def attn_window_gated_far(q, ring_k, ring_v, meta, sink_k, sink_v, k_tilde, mu, mz, t_hat,
                          gate, gate_scale, scale, rect=0, out=None, workspace=None, stream=None):
    """z [nh][hd] of the gated one-row call with the far field (see attn_window_gated_far in
    include/winattn.h): q [nh][hd], rings [nk][w][hd], meta [nk][4], sinks [nk][ns][hd] or
    None, k_tilde [nk][m][hd], mu [nh][m][m], mz [nh][2m], t_hat [nh][m][hd], gate and
    gate_scale [nh*hd]."""
    nk, w, hd = ring_k.shape
    nh = q.shape[0]
    m = mu.shape[1]
    if (tuple(q.shape) != (nh, hd) or nh % nk or tuple(k_tilde.shape) != (nk, m, hd)
            or tuple(mu.shape) != (nh, m, m) or tuple(mz.shape) != (nh, 2 * m)
            or tuple(t_hat.shape) != (nh, m, hd) or gate.numel() != nh * hd
            or gate_scale.numel() != nh * hd or tuple(meta.shape) != (nk, 4)):
        raise ValueError("attn_window_gated_far: inconsistent shapes")
    ns = 0 if sink_k is None else sink_k.shape[1]
    if out is None:
        out = torch.empty((nh, hd), dtype=torch.float32, device=q.device)
    st = _stream_ptr(stream, q.device)
    need = gated_far_workspace_bytes(nh, nk, hd, w, ns, m)
    ws = workspace if workspace is not None else _default_workspace(q.device, st)
    wp, wb = ws.get(need)
    rc = load().attn_window_gated_far(
        _ptr(q, "q"), _ptr(ring_k, "ring_k"), _ptr(ring_v, "ring_v"),
        _ptr(meta, "meta", (torch.int32, torch.uint32)), _ptr(sink_k, "sink_k"),
        _ptr(sink_v, "sink_v"), _ptr(k_tilde, "k_tilde"), _ptr(mu, "mu"), _ptr(mz, "mz"),
        _ptr(t_hat, "t_hat"), _ptr(gate, "gate"), _ptr(gate_scale, "gate_scale"),
        _ptr(out, "out"), nh, nk, hd, w, ns, m, float(scale), int(rect), wp, wb, st)
    if rc != OK:
        raise WinattnError("attn_window_gated_far", rc)
    return out


def _rows(t, name):
    if not isinstance(t, torch.Tensor) or t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D row-major view (rows, columns) with unit column stride")
    if not t.is_cuda or t.dtype != torch.float32:
        raise ValueError(f"{name} must be a float32 device tensor")
    return t.data_ptr(), t.stride(0)


def attn_encoder(q, k, v, segs, nh, nk, hd, scale, window=0, max_len=None, out=None,
                 stream=None):
    """Encoder attention over packed sequences (see attn_encoder in include/winattn.h).

    q [tokens][>= nh*hd], k and v [tokens][>= nk*hd], out [tokens][>= nh*hd]: 2-D row views
    (strided rows allowed, e.g. column slices of one packed q|k|v buffer); segs [nseg][2]
    int32/uint32 device tensor of (start, len); max_len defaults to the largest len (read
    from segs on the host)."""
    qp, ldq = _rows(q, "q")
    kp, ldk = _rows(k, "k")
    vp, ldv = _rows(v, "v")
    if out is None:
        out = torch.zeros((q.shape[0], nh * hd), dtype=torch.float32, device=q.device)
    op, ldo = _rows(out, "out")
    if tuple(segs.shape[1:]) != (2,) or not segs.is_contiguous():
        raise ValueError("segs must be a contiguous [nseg][2] tensor")
    nseg = segs.shape[0]
    if max_len is None:
        max_len = int(segs[:, 1].max().item()) if nseg else 0
    rc = load().attn_encoder(qp, kp, vp, op, _ptr(segs, "segs", (torch.int32, torch.uint32)),
                             nseg, int(max_len), ldq, ldk, ldv, ldo, nh, nk, hd, int(window),
                             float(scale), _stream_ptr(stream, q.device))
    if rc != OK:
        raise WinattnError("attn_encoder", rc)
    return out


def mfma16_layout_probe(device="cuda", stream=None):
    """[64][4] accumulator map of one 16x16x4 f32 matrix-core product (see the header)."""
    out = torch.full((64, 4), -1.0, dtype=torch.float32, device=device)
    rc = load().attn_mfma16_layout_probe(out.data_ptr(), _stream_ptr(stream, out.device))
    if rc != OK:
        raise WinattnError("attn_mfma16_layout_probe", rc)
    return out


def read_probe(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """One plain streaming read of every byte of the contiguous device tensor `src` (the
    achievable HBM read rate; see attn_read_probe in include/winattn.h). sink: 256 floats."""
    if sink.numel() < 256:
        raise ValueError("sink must hold 256 floats")
    rc = load().attn_read_probe(_ptr(src, "src", (src.dtype,)), src.numel() * src.element_size(),
                                _ptr(sink, "sink"), _stream_ptr(stream, src.device))
    if rc != OK:
        raise WinattnError("attn_read_probe", rc)


def workspace_init(buf: torch.Tensor, stream=None) -> None:
    st = _stream_ptr(stream, buf.device)
    rc = load().attn_workspace_init(buf.data_ptr(), buf.numel() * buf.element_size(), st)
    if rc != OK:
        raise WinattnError("attn_workspace_init", rc)
