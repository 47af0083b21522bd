"""Algorithmic work of one call: the bytes the method must move and the flops it must do.

These are the measurement formulas the throughput figures are quoted against; they count what
the definition requires (distinct K/V rows read once, QK^T and PV multiply-adds), not what any
kernel happens to do.
"""
from __future__ import annotations

import numpy as np


def _group_window(inp, g: int):
    ln, _, _, ov = (int(x) for x in inp.meta[g])
    return ln, (ov if ov else inp.w)


def unique_kv_keys(inp) -> int:
    """Distinct K/V rows of a chunk call: per group ns + min(wg, len0+1) + rows - 1."""
    total = 0
    for g in range(inp.ng):
        ln, wg = _group_window(inp, g)
        total += inp.ns + min(wg, ln + 1) + inp.rows - 1
    return total


def unique_kv_bytes(inp) -> int:
    return unique_kv_keys(inp) * inp.d * 4 * 2


def total_bytes(inp) -> int:
    """K/V rows + q + out + meta for a chunk call."""
    return unique_kv_bytes(inp) + 2 * inp.rows * inp.nh * inp.d * 4 + inp.ng * 16


def visible_triples(inp) -> int:
    """(row, query head, key) triples scored by a chunk call."""
    total = 0
    i = np.arange(inp.rows, dtype=np.int64)
    for g in range(inp.ng):
        ln, wg = _group_window(inp, g)
        total += int(np.sum(inp.ns + np.minimum(wg, ln + i + 1))) * inp.hpg
    return total


def chunk_flops(inp) -> int:
    """QK^T plus PV multiply-adds, 2 flops each: 4*d per visible triple."""
    return visible_triples(inp) * 4 * inp.d


def gated_counts(inp):
    """(distinct KV bytes read, total bytes, flops) for a gated call."""
    first = max(0, inp.pos0 + 1 - inp.window)
    last = inp.pos0 + inp.rows - 1
    positions = last - first + 1
    kv_read = positions * inp.nk * inp.hd * 4 * 2
    prior = (inp.pos0 - first) * inp.nk * inp.hd * 4 * 2
    inputs = (inp.yq.size + inp.yk.size + inp.yv.size + inp.rope.size + inp.q_scale.size +
              inp.gate.size + inp.gate_scale.size) * 4
    out = inp.rows * inp.nh * inp.hd * 4
    ring_writes = inp.rows * inp.nk * inp.hd * 4 * 2
    total = prior + inputs + out + ring_writes
    pos = inp.pos0 + np.arange(inp.rows, dtype=np.int64)
    keys = np.minimum(inp.window, pos + 1)
    flops = int(np.sum(keys)) * inp.nh * 4 * inp.hd
    return kv_read, total, flops


def encoder_flops(inp) -> int:
    """4 * hd flops (score and value products) per visible (position, query head, key) of an
    encoder call: a window of w keeps positions max(0, i - w) .. min(len, i + w + 1) - 1."""
    total = 0
    for _, ln in inp.segs:
        ln = int(ln)
        if inp.window == 0:
            keys = ln * ln
        else:
            i = np.arange(ln)
            keys = int(np.sum(np.minimum(ln, i + inp.window + 1) - np.maximum(0, i - inp.window)))
        total += keys
    return 4 * inp.hd * inp.nh * total
