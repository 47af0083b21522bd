"""Pins of the CPU oracle to things other than itself (CPU only).

Each test checks the oracle against a fact fixed by the pages' definition or by mathematics:
a brute force that simulates the ring pushes with a bounded deque, torch's f64 scaled-dot-product
attention, closed forms (uniform weights give the arithmetic-series mean of visible positions),
special cases (a one-key window returns its value), invariants (ring rotation, chunk == a
sequence of decodes, a group's override == that group alone with w = override), and hand-derived
worked examples under tests/golden/.

Definition followed (o1c page, "A sealed layer's attention for a chunk of rows, on Metal"):
row i of a group sees its ns sinks and the last min(wg, len0 + i + 1) entries of the stream
[ring entries oldest->newest, chunk rows 0..i]; wg is the per-group override or w (`wgf`).
"""
import collections
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from sliding_window_gqa_group_amd import inputs as gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ── Independent brute force: simulate the ring as a bounded deque ─────────────────────────────

def _ring_entries(inp, g):
    """(k, v) of the group's ring entries, oldest first, read by walking slots from the head."""
    ln, head, _, ov = (int(x) for x in inp.meta[g])
    wg = ov if ov else inp.w
    out, slot = [], head
    for _ in range(ln):
        out.append((inp.ring_k[g, slot].astype(np.float64), inp.ring_v[g, slot].astype(np.float64)))
        slot += 1
        if slot == wg:
            slot = 0
    return out, wg


def brute_chunk(inp):
    rows, ng, hpg, d = inp.rows, inp.ng, inp.hpg, inp.d
    out = np.zeros((rows, ng * hpg, d))
    for g in range(ng):
        entries, wg = _ring_entries(inp, g)
        window = collections.deque(entries, maxlen=wg)   # push evicts the oldest when full
        sinks = [(inp.sink_k[g, s].astype(np.float64), inp.sink_v[g, s].astype(np.float64))
                 for s in range(inp.ns)]
        for i in range(rows):
            window.append((inp.chunk_k[i, g].astype(np.float64), inp.chunk_v[i, g].astype(np.float64)))
            keys = sinks + list(window)
            for h in range(hpg):
                qv = inp.q[i, g * hpg + h].astype(np.float64)
                sc = [inp.scale * float(np.dot(qv, k)) for k, _ in keys]
                m = max(sc)
                p = [math.exp(s - m) for s in sc]
                tot = math.fsum(p)
                acc = np.zeros(d)
                for pj, (_, v) in zip(p, keys):
                    acc += pj * v
                out[i, g * hpg + h] = acc / tot
    return out


def _random_case(rng, d=None, ns=None, rows=None):
    ng = int(rng.integers(1, 4))
    hpg = int(rng.choice([1, 2, 3, 4]))
    d = int(d if d is not None else rng.choice([4, 8, 12, 16]))
    w = int(rng.integers(1, 10))
    ns = int(ns if ns is not None else rng.choice([0, 1, 3]))
    rows = int(rows if rows is not None else rng.integers(1, 7))
    meta = []
    for _ in range(ng):
        ov = int(rng.integers(0, w + 1)) if rng.random() < 0.4 else 0
        wg = ov if ov else w
        ln = int(rng.integers(0, wg + 1))
        head = int(rng.integers(0, wg)) if ln > 0 else int(rng.integers(0, wg))
        meta.append((ln, head, int(rng.integers(0, 5)), ov))
    return gen.make_chunk(rows, ng, hpg, d, w, ns, meta, seed=int(rng.integers(1 << 30)),
                          scale=float(rng.choice([0.25, 0.5, 1.0])))


def test_oracle_matches_deque_bruteforce():
    rng = np.random.default_rng(1234)
    for _ in range(300):
        inp = _random_case(rng)
        ref = brute_chunk(inp)
        got = oracle.window_chunk(inp)
        np.testing.assert_allclose(got, ref, rtol=3e-7, atol=1e-8)


# ── Library routine: torch f64 scaled-dot-product attention ──────────────────────────────────

def test_oracle_matches_torch_causal_gqa():
    """len0 = 0, ns = 0 and a window no shorter than the chunk: plain causal GQA attention."""
    rng = np.random.default_rng(7)
    for rows, ng, hpg, d in [(5, 2, 3, 8), (17, 1, 4, 16), (9, 3, 1, 12)]:
        w = rows + int(rng.integers(0, 4))
        inp = gen.make_chunk(rows, ng, hpg, d, w, 0, [(0, int(rng.integers(0, w)), 0, 0)] * ng,
                             seed=int(rng.integers(1 << 30)))
        q = torch.from_numpy(inp.q.astype(np.float64)).permute(1, 0, 2)[None]       # [1,nh,L,d]
        k = torch.from_numpy(inp.chunk_k.astype(np.float64)).permute(1, 0, 2)[None]  # [1,ng,L,d]
        v = torch.from_numpy(inp.chunk_v.astype(np.float64)).permute(1, 0, 2)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            q, k, v, is_causal=True, scale=inp.scale, enable_gqa=True)[0].permute(1, 0, 2).numpy()
        np.testing.assert_allclose(oracle.window_chunk(inp), ref, rtol=3e-7, atol=1e-8)


def test_oracle_matches_torch_with_window_mask():
    """Sinks + wrapped ring + chunk as one key panel and a boolean mask, through torch f64 SDPA."""
    rng = np.random.default_rng(8)
    for _ in range(20):
        inp = _random_case(rng, d=8)
        for g in range(inp.ng):
            entries, wg = _ring_entries(inp, g)
            ln = len(entries)
            keys = ([inp.sink_k[g, s] for s in range(inp.ns)] + [e[0] for e in entries] +
                    [inp.chunk_k[i, g] for i in range(inp.rows)])
            vals = ([inp.sink_v[g, s] for s in range(inp.ns)] + [e[1] for e in entries] +
                    [inp.chunk_v[i, g] for i in range(inp.rows)])
            K = torch.tensor(np.array(keys, dtype=np.float64))[None, None]
            V = torch.tensor(np.array(vals, dtype=np.float64))[None, None]
            n = K.shape[2]
            mask = torch.zeros(inp.rows, n, dtype=torch.bool)
            for i in range(inp.rows):
                mask[i, :inp.ns] = True
                end = ln + i + 1
                start = end - min(wg, end)
                mask[i, inp.ns + start: inp.ns + end] = True
            heads = slice(g * inp.hpg, (g + 1) * inp.hpg)
            Q = torch.tensor(inp.q[:, heads].astype(np.float64)).permute(1, 0, 2)[None]
            ref = torch.nn.functional.scaled_dot_product_attention(
                Q, K.expand(1, inp.hpg, n, inp.d), V.expand(1, inp.hpg, n, inp.d),
                attn_mask=mask, scale=inp.scale)[0].permute(1, 0, 2).numpy()
            np.testing.assert_allclose(oracle.window_chunk(inp)[:, heads], ref, rtol=3e-7, atol=1e-8)


# ── Closed forms and special cases ───────────────────────────────────────────────────────────

def _coded_case(rows, ng, hpg, w, ns, meta, d=4):
    """q = 0 (uniform weights); V carries (position code, 1, code^2, 0)."""
    inp = gen.make_chunk(rows, ng, hpg, d, w, ns, meta, seed=5)
    inp.q[:] = 0.0
    for g in range(ng):
        ln, head, _, ov = (int(x) for x in inp.meta[g])
        wg = ov if ov else w
        for x in range(ln):
            slot = (head + x) % wg
            inp.ring_v[g, slot, :3] = (x, 1.0, x * x)
        for i in range(rows):
            inp.chunk_v[i, g, :3] = (ln + i, 1.0, (ln + i) ** 2)
        for s in range(ns):
            inp.sink_v[g, s, :3] = (-1 - s, 1.0, (1 + s) ** 2)
    return inp


def test_uniform_weights_give_arithmetic_series_mean():
    cases = [
        (6, 2, 2, 8, 2, [(8, 3, 0, 0), (5, 2, 0, 6)]),
        (3, 1, 1, 16, 0, [(16, 5, 0, 0)]),
        (9, 3, 1, 5, 1, [(0, 0, 0, 0), (2, 4, 0, 0), (3, 1, 0, 3)]),
    ]
    for rows, ng, hpg, w, ns, meta in cases:
        inp = _coded_case(rows, ng, hpg, w, ns, meta)
        out = oracle.window_chunk(inp)
        for g in range(ng):
            ln, _, _, ov = meta[g]
            wg = ov if ov else w
            for i in range(rows):
                hi = ln + i + 1
                win = min(wg, hi)
                lo = hi - win
                n = ns + win
                pos_sum = (lo + hi - 1) * win / 2.0 - ns * (ns + 1) / 2.0
                sq_sum = (sum(x * x for x in range(lo, hi)) + sum((1 + s) ** 2 for s in range(ns)))
                for h in range(hpg):
                    o = out[i, g * hpg + h]
                    assert o[0] == pytest.approx(pos_sum / n, rel=1e-6, abs=1e-6)
                    assert o[1] == pytest.approx(1.0, rel=1e-7)
                    assert o[2] == pytest.approx(sq_sum / n, rel=1e-6)


def test_window_of_one_returns_own_value():
    inp = gen.make_chunk(7, 3, 2, 8, 5, 0, [(1, 0, 0, 1), (0, 0, 0, 1), (1, 0, 0, 1)], seed=11)
    out = oracle.window_chunk(inp)
    for i in range(inp.rows):
        for g in range(inp.ng):
            for h in range(inp.hpg):
                np.testing.assert_array_equal(out[i, g * inp.hpg + h], inp.chunk_v[i, g])


def test_one_hot_query_with_large_scale_selects_argmax_key():
    inp = gen.make_chunk(1, 1, 1, 8, 6, 0, [(6, 4, 0, 0)], seed=12, scale=200.0)
    inp.ring_k[:] = 0.0
    inp.chunk_k[:] = 0.0
    inp.q[:] = 0.0
    inp.q[0, 0, 3] = 1.0
    # logical entry x sits at slot (4 + x) % 6; row 0 sees x = 1..5 and itself
    target_slot = (4 + 2) % 6
    inp.ring_k[0, target_slot, 3] = 1.0
    inp.ring_k[0, (4 + 0) % 6, 3] = 2.0          # oldest entry: evicted for row 0, must not win
    out = oracle.window_chunk(inp)
    np.testing.assert_allclose(out[0, 0], inp.ring_v[0, target_slot], rtol=1e-6, atol=1e-6)


def test_weights_sum_to_one_and_count_matches_window():
    rng = np.random.default_rng(21)
    for _ in range(40):
        inp = _random_case(rng)
        i = int(rng.integers(0, inp.rows))
        gh = int(rng.integers(0, inp.ng * inp.hpg))
        g = gh // inp.hpg
        ln, _, _, ov = (int(x) for x in inp.meta[g])
        wg = ov if ov else inp.w
        wts = oracle.window_chunk_weights(inp, i, gh)
        assert wts.size == inp.ns + min(wg, ln + i + 1)
        assert math.fsum(wts) == pytest.approx(1.0, abs=1e-12)
        assert np.all(wts > 0)


# ── Invariants ───────────────────────────────────────────────────────────────────────────────

def test_ring_rotation_invariance_is_bitwise():
    rng = np.random.default_rng(31)
    for _ in range(30):
        inp = _random_case(rng)
        base = oracle.window_chunk(inp)
        rot = gen.make_chunk(inp.rows, inp.ng, inp.hpg, inp.d, inp.w, inp.ns, inp.meta.copy(), 0,
                             scale=inp.scale)
        for name in ("sink_k", "sink_v", "q", "chunk_k", "chunk_v"):
            setattr(rot, name, getattr(inp, name).copy())
        for g in range(inp.ng):
            ln, head, far, ov = (int(x) for x in inp.meta[g])
            wg = ov if ov else inp.w
            r = int(rng.integers(0, wg))
            # slot s moves to (s + r) mod wg; the head moves with it
            idx = (np.arange(wg) + r) % wg
            rot.ring_k[g, idx] = inp.ring_k[g, :wg]
            rot.ring_v[g, idx] = inp.ring_v[g, :wg]
            rot.ring_k[g, wg:] = inp.ring_k[g, wg:]
            rot.ring_v[g, wg:] = inp.ring_v[g, wg:]
            rot.meta[g] = (ln, (head + r) % wg, far, ov)
        np.testing.assert_array_equal(oracle.window_chunk(rot), base)


def _push(inp, g, k, v):
    """One ring push with the commit rules of the o1c page (`o1c_ring_commit`, `o1c_meta`):
    the row lands in slot (head + len) mod wg; a full ring advances its head instead."""
    ln, head, far, ov = (int(x) for x in inp.meta[g])
    wg = ov if ov else inp.w
    slot = (head + ln) % wg
    inp.ring_k[g, slot] = k
    inp.ring_v[g, slot] = v
    if ln + 1 <= wg:
        inp.meta[g] = (ln + 1, head, far, ov)
    else:
        inp.meta[g] = (wg, (head + 1) % wg, far + 1, ov)


def _decode_state(inp):
    """A one-row call sharing inp's rings (copied), meta (copied) and sinks."""
    state = gen.make_chunk(1, inp.ng, inp.hpg, inp.d, inp.w, inp.ns, inp.meta.copy(), 0,
                           scale=inp.scale)
    state.ring_k = inp.ring_k.copy()
    state.ring_v = inp.ring_v.copy()
    state.sink_k, state.sink_v = inp.sink_k, inp.sink_v
    return state


def _row_of(state, inp, i):
    state.q = inp.q[i:i + 1].copy()
    state.chunk_k = inp.chunk_k[i:i + 1].copy()
    state.chunk_v = inp.chunk_v[i:i + 1].copy()


def test_chunk_equals_sequence_of_decodes():
    """Row i of a chunk call == a one-row call after the rows before it were pushed: by the
    push rule written out here, and by the oracle's commit (row by row, and all rows before i
    in one commit)."""
    rng = np.random.default_rng(41)
    for _ in range(25):
        inp = _random_case(rng)
        full = oracle.window_chunk(inp)
        pushed, committed = _decode_state(inp), _decode_state(inp)
        for i in range(inp.rows):
            for state in (pushed, committed):
                _row_of(state, inp, i)
                np.testing.assert_allclose(oracle.window_chunk(state)[0], full[i], rtol=1e-7,
                                           atol=1e-9)
            for g in range(inp.ng):
                _push(pushed, g, inp.chunk_k[i, g], inp.chunk_v[i, g])
            committed.ring_k, committed.ring_v, committed.meta = oracle.window_commit(committed)
            np.testing.assert_array_equal(committed.meta, pushed.meta)
            np.testing.assert_array_equal(committed.ring_k, pushed.ring_k)
            # the rows before i + 1 in a single commit reach the same state
            if i >= 1:
                many = gen.make_chunk(i + 1, inp.ng, inp.hpg, inp.d, inp.w, inp.ns,
                                      inp.meta.copy(), 0, scale=inp.scale)
                many.ring_k, many.ring_v = inp.ring_k.copy(), inp.ring_v.copy()
                many.chunk_k = inp.chunk_k[:i + 1].copy()
                many.chunk_v = inp.chunk_v[:i + 1].copy()
                rk, rv, meta = oracle.window_commit(many)
                np.testing.assert_array_equal(meta, pushed.meta)
                np.testing.assert_array_equal(rk, pushed.ring_k)
                np.testing.assert_array_equal(rv, pushed.ring_v)


def _live_entries(ring_g, meta_g, w):
    """A group's ring entries oldest first, read as the attention reads them: entry x at slot
    (head + x) mod wg."""
    ln, head, _, ov = (int(x) for x in meta_g)
    wg = ov if ov else w
    return [ring_g[(head + x) % wg] for x in range(ln)]


def test_commit_matches_stream_bruteforce():
    """After a commit the ring, read through the attention's slot rule, holds the last
    min(wg, len + rows) entries of [old entries, chunk rows] (a bounded deque); length and far
    count follow; slots that hold no entry and slots past the group window keep their data."""
    from collections import deque
    rng = np.random.default_rng(77)
    for _ in range(300):
        inp = _random_case(rng, rows=int(rng.integers(1, 14)))
        rk, rv, meta = oracle.window_commit(inp)
        for g in range(inp.ng):
            ln0, head0, far0, ov = (int(x) for x in inp.meta[g])
            wg = ov if ov else inp.w
            ks = deque(_live_entries(inp.ring_k[g], inp.meta[g], inp.w), maxlen=wg)
            vs = deque(_live_entries(inp.ring_v[g], inp.meta[g], inp.w), maxlen=wg)
            for j in range(inp.rows):
                ks.append(inp.chunk_k[j, g])
                vs.append(inp.chunk_v[j, g])
            assert int(meta[g, 0]) == len(ks) == min(wg, ln0 + inp.rows)
            assert int(meta[g, 2]) == far0 + max(0, ln0 + inp.rows - wg)
            assert int(meta[g, 3]) == ov
            got_k = _live_entries(rk[g], meta[g], inp.w)
            got_v = _live_entries(rv[g], meta[g], inp.w)
            for a, b in zip(got_k, ks):
                np.testing.assert_array_equal(a, b)
            for a, b in zip(got_v, vs):
                np.testing.assert_array_equal(a, b)
            live = {(int(meta[g, 1]) + x) % wg for x in range(int(meta[g, 0]))}
            for slot in range(inp.w):
                if slot >= wg or slot not in live:
                    np.testing.assert_array_equal(rk[g, slot], inp.ring_k[g, slot])
                    np.testing.assert_array_equal(rv[g, slot], inp.ring_v[g, slot])


def test_group_override_equals_group_alone_restrided():
    rng = np.random.default_rng(51)
    inp = gen.make_chunk(6, 3, 2, 8, 12, 2, [(12, 7, 0, 0), (4, 3, 0, 5), (7, 2, 0, 9)], seed=52)
    full = oracle.window_chunk(inp)
    for g in range(inp.ng):
        ln, head, far, ov = (int(x) for x in inp.meta[g])
        wg = ov if ov else inp.w
        alone = gen.make_chunk(inp.rows, 1, inp.hpg, inp.d, wg, inp.ns, [(ln, head, far, 0)], 0,
                               scale=inp.scale)
        alone.ring_k = inp.ring_k[g:g + 1, :wg].copy()
        alone.ring_v = inp.ring_v[g:g + 1, :wg].copy()
        alone.sink_k = inp.sink_k[g:g + 1].copy()
        alone.sink_v = inp.sink_v[g:g + 1].copy()
        alone.q = inp.q[:, g * inp.hpg:(g + 1) * inp.hpg].copy()
        alone.chunk_k = inp.chunk_k[:, g:g + 1].copy()
        alone.chunk_v = inp.chunk_v[:, g:g + 1].copy()
        np.testing.assert_array_equal(oracle.window_chunk(alone),
                                      full[:, g * inp.hpg:(g + 1) * inp.hpg])


def test_select_matches_full():
    inp = gen.make_chunk(9, 2, 3, 16, 10, 2, [(10, 4, 0, 0), (6, 1, 0, 7)], seed=61)
    full = oracle.window_chunk(inp)
    rows = np.array([0, 8, 3, 5])
    heads = np.array([5, 0, 2, 4])
    np.testing.assert_array_equal(oracle.window_chunk_select(inp, rows, heads), full[rows, heads])


def test_invalid_meta_is_rejected():
    bad = [
        [(17, 0, 0, 0)],      # len beyond w
        [(4, 4, 0, 4)],       # head not below the window
        [(3, 0, 0, 20)],      # override beyond the storage stride w
    ]
    for meta in bad:
        inp = gen.make_chunk(2, 1, 2, 4, 16, 0, meta, seed=1)
        assert not oracle.meta_ok(inp.meta, 1, 16)
        with pytest.raises(ValueError):
            oracle.window_chunk(inp)


def test_golden_chunk_pow2():
    with open(os.path.join(GOLDEN, "chunk_pow2.json")) as f:
        gd = json.load(f)
    q = np.array([[[math.log(2) if x == "ln2" else x for x in hv] for hv in row] for row in gd["q"]],
                 dtype=np.float32)
    inp = gen.make_chunk(gd["rows"], gd["ng"], gd["hpg"], gd["d"], gd["w"], gd["ns"], gd["meta"], 0,
                         scale=gd["scale"])
    inp.ring_k = np.array(gd["ring_k"], dtype=np.float32)
    inp.ring_v = np.array(gd["ring_v"], dtype=np.float32)
    inp.sink_k = np.array(gd["sink_k"], dtype=np.float32)
    inp.sink_v = np.array(gd["sink_v"], dtype=np.float32)
    inp.chunk_k = np.array(gd["chunk_k"], dtype=np.float32)
    inp.chunk_v = np.array(gd["chunk_v"], dtype=np.float32)
    inp.q = q
    np.testing.assert_allclose(oracle.window_chunk(inp), np.array(gd["expected"]), rtol=gd["rtol"],
                               atol=1e-7)


# ── Gated variant ────────────────────────────────────────────────────────────────────────────

def _rotate_unit_complex(raw, rope_row, eps):
    """Rotate-half as complex multiplication: (x + iy)(c + is), then unit-normalise with eps."""
    half = raw.shape[-1] // 2
    z = raw[:half].astype(np.float64) + 1j * raw[half:].astype(np.float64)
    r = rope_row[:half].astype(np.float64) + 1j * rope_row[half:].astype(np.float64)
    rot = z * r
    vec = np.concatenate([rot.real, rot.imag])
    return vec / np.sqrt(np.sum(np.abs(rot) ** 2) + eps)


def brute_gated(inp):
    from scipy.special import expit
    rk = inp.ring_k.copy()
    rv = inp.ring_v.copy()
    for r in range(inp.rows):
        slot = (inp.pos0 + r) % inp.cap
        for kh in range(inp.nk):
            rk[slot, kh] = _rotate_unit_complex(inp.yk[r, kh], inp.rope[r], inp.eps).astype(np.float32)
            rv[slot, kh] = inp.yv[r, kh]
    hpg = inp.nh // inp.nk
    z = np.zeros((inp.rows, inp.nh, inp.hd))
    for r in range(inp.rows):
        pos = inp.pos0 + r
        positions = [p for p in range(0, pos + 1) if pos - p < inp.window]
        for a in range(inp.nh):
            kh = a // hpg
            qv = _rotate_unit_complex(inp.yq[r, a], inp.rope[r], inp.eps) * inp.q_scale[a]
            K = np.array([rk[p % inp.cap, kh] for p in positions], dtype=np.float64)
            V = np.array([rv[p % inp.cap, kh] for p in positions], dtype=np.float64)
            s = inp.scale * (K @ qv)
            p = np.exp(s - s.max())
            o = (p[:, None] * V).sum(0) / p.sum()
            gsl = slice(a * inp.hd, (a + 1) * inp.hd)
            z[r, a] = o * expit(inp.gate[r, gsl].astype(np.float64) * inp.gate_scale[gsl])
    return z, rk, rv


def test_gated_matches_complex_bruteforce():
    cases = [(3, 5, 8, 4, 4, 2, 8), (4, 0, 7, 4, 2, 2, 16), (2, 30, 9, 6, 6, 3, 4), (5, 2, 11, 7, 4, 1, 8)]
    for rows, pos0, cap, window, nh, nk, hd in cases:
        inp = gen.make_gated(rows, pos0, cap, window, nh, nk, hd, seed=rows * 100 + pos0, scale=0.7)
        z, rk, rv = oracle.window_gated(inp)
        bz, brk, brv = brute_gated(inp)
        np.testing.assert_allclose(rk, brk, rtol=2e-7, atol=1e-8)
        np.testing.assert_array_equal(rv, brv)
        np.testing.assert_allclose(z, bz, rtol=1e-6, atol=1e-8)


def test_gated_identity_table_is_pure_normalisation():
    inp = gen.make_gated(3, 0, 4, 2, 2, 1, 8, seed=71)
    inp.rope[:, :4] = 1.0
    inp.rope[:, 4:] = 0.0
    inp.yk[2] *= 3e-4          # a key whose sum of squares is comparable to eps
    _, rk, _ = oracle.window_gated(inp)
    for r in range(inp.rows):
        raw = inp.yk[r, 0].astype(np.float64)
        ss = float(np.sum(raw * raw))
        slot = (inp.pos0 + r) % inp.cap
        np.testing.assert_allclose(rk[slot, 0], raw / math.sqrt(ss + inp.eps), rtol=2e-7)
        assert float(np.sum(rk[slot, 0].astype(np.float64) ** 2)) == pytest.approx(ss / (ss + inp.eps), rel=1e-6)


def test_gated_rotation_preserves_norm():
    inp = gen.make_gated(4, 1000, 8, 4, 2, 2, 16, seed=72, eps=0.0)
    _, rk, _ = oracle.window_gated(inp)
    for r in range(inp.rows):
        for kh in range(inp.nk):
            k = rk[(inp.pos0 + r) % inp.cap, kh].astype(np.float64)
            assert float(np.dot(k, k)) == pytest.approx(1.0, abs=1e-6)


def test_rope_table_angle_steps_follow_the_frequency_law():
    """The rotation table's pair i (cos in column i, sin in column i + hd/2) turns by
    base^(-2i/hd) radians from one position to the next, read back from consecutive rows with
    atan2 (the f32 entries hold each angle to about 1e-7), and every pair lies on the unit
    circle. Every frequency is at most 1 radian, so the wrapped steps are the frequencies."""
    hd, base = 64, 10000.0
    t = gen.rope_table(9, 123, hd, base).astype(np.float64)
    half = hd // 2
    ang = np.arctan2(t[:, half:], t[:, :half])
    step = np.angle(np.exp(1j * (ang[1:] - ang[:-1])))
    freq = base ** (-2.0 * np.arange(half) / hd)
    np.testing.assert_allclose(step, np.broadcast_to(freq, step.shape), rtol=0, atol=1e-6)
    np.testing.assert_allclose(t[:, :half] ** 2 + t[:, half:] ** 2, 1.0, rtol=0, atol=1e-6)


def test_gated_output_depends_on_relative_positions_only():
    """With pos0 = 0 every key a row sees is a chunk row, rotated by the same table as the
    queries. With a query scale that is constant per head (the learned per-element scale does
    not commute with the rotation), scores <s R(p) q, R(p') k> depend on p - p' only: the
    table of positions c .. c + rows - 1 in place of 0 .. rows - 1 leaves the output unchanged
    up to the f32 rounding of the table. Rotating queries and keys by different pairings or
    angles, or only one of them, breaks this."""
    inp = gen.make_gated(6, 0, 16, 8, 4, 2, 16, seed=75, scale=0.8)
    inp.q_scale[:] = inp.q_scale[:, :1]
    z0, _, _ = oracle.window_gated(inp)
    for c in (1, 37, 1000):
        inp.rope = gen.rope_table(inp.rows, c, inp.hd)
        z1, _, _ = oracle.window_gated(inp)
        np.testing.assert_allclose(z1, z0, rtol=1e-5, atol=1e-7)
    # not vacuous: without rotation (the identity table) the relative angles are gone and the
    # output changes
    inp.rope[:, :inp.hd // 2] = 1.0
    inp.rope[:, inp.hd // 2:] = 0.0
    assert not np.allclose(oracle.window_gated(inp)[0], z0, rtol=1e-3)


def test_gated_zero_gate_is_half_of_chunk_attention():
    """gate = 0 gives z = attn / 2; the attention equals the chunk path on the prepped ring with
    ns = 0, window override = window, the ring tail as the ring and the new rows as the chunk."""
    inp = gen.make_gated(5, 9, 12, 6, 4, 2, 8, seed=73, scale=0.9)
    inp.gate[:] = 0.0
    z, rk, rv = oracle.window_gated(inp)
    hpg = inp.nh // inp.nk
    ln = min(inp.window - 1, inp.pos0)
    first = inp.pos0 - ln
    ch = gen.make_chunk(inp.rows, inp.nk, hpg, inp.hd, inp.window, 0,
                        [(ln, 0, 0, 0)] * inp.nk, seed=0, scale=inp.scale)
    for x in range(ln):
        ch.ring_k[:, x] = rk[(first + x) % inp.cap]
        ch.ring_v[:, x] = rv[(first + x) % inp.cap]
    for r in range(inp.rows):
        ch.chunk_k[r] = rk[(inp.pos0 + r) % inp.cap]
        ch.chunk_v[r] = rv[(inp.pos0 + r) % inp.cap]
        for a in range(inp.nh):
            ch.q[r, a] = (_rotate_unit_complex(inp.yq[r, a], inp.rope[r], inp.eps) * inp.q_scale[a])
    attn = oracle.window_chunk(ch)
    # q goes through f32 on the chunk side; allow for that rounding
    np.testing.assert_allclose(z, 0.5 * attn, rtol=2e-6, atol=1e-7)


def test_gated_rejects_small_cap():
    inp = gen.make_gated(4, 10, 6, 4, 2, 1, 8, seed=74)
    with pytest.raises(ValueError):
        oracle.window_gated(inp)      # cap 6 < window + rows - 1 = 7


def test_golden_gated_unit():
    with open(os.path.join(GOLDEN, "gated_unit.json")) as f:
        gd = json.load(f)
    inp = gen.make_gated(gd["rows"], gd["pos0"], gd["cap"], gd["window"], gd["nh"], gd["nk"],
                         gd["hd"], seed=0, scale=gd["scale"], eps=gd["eps"])
    for name in ("yq", "yk", "yv", "rope", "q_scale", "gate", "gate_scale"):
        setattr(inp, name, np.array(gd[name], dtype=np.float32))
    inp.ring_k = np.array(gd["ring_k_before"], dtype=np.float32)
    inp.ring_v = np.array(gd["ring_v_before"], dtype=np.float32)
    z, rk, rv = oracle.window_gated(inp)
    np.testing.assert_allclose(z, np.array(gd["expected_z"]), rtol=gd["rtol"], atol=gd["atol"])
    np.testing.assert_allclose(rk, np.array(gd["expected_ring_k"]), rtol=1e-7, atol=1e-8)
    np.testing.assert_array_equal(rv, np.array(gd["expected_ring_v"], dtype=np.float32))


# ── the far field (landmark summaries of evicted keys) ──────────────────────────────────────

def _far_case(rng, rows, m=1, hpg=1, far_len=None, d=8):
    ng = int(rng.integers(1, 4))
    w = int(rng.integers(2, 9))
    meta = []
    for _ in range(ng):
        ov = int(rng.integers(1, w + 1)) if rng.random() < 0.3 else 0
        wg = ov if ov else w
        ln = int(rng.integers(0, wg + 1))
        head = int(rng.integers(0, wg))
        fl = int(far_len if far_len is not None else rng.integers(0, 4))
        meta.append((ln, head, fl, ov))
    return gen.make_chunk(rows, ng, hpg, d, w, int(rng.choice([0, 2])), meta,
                          seed=int(rng.integers(1 << 30)), scale=float(rng.choice([0.3, 0.6])))


def _stream_entries(inp, g):
    """K, V of every entry a group has held so far, oldest first: its ring entries then chunk
    rows (the history before them is passed separately)."""
    ln, head, _, ov = (int(x) for x in inp.meta[g])
    wg = ov if ov else inp.w
    ks = [inp.ring_k[g, (head + x) % wg] for x in range(ln)]
    vs = [inp.ring_v[g, (head + x) % wg] for x in range(ln)]
    return ks, vs


def _exact_far_state(q, hist_k, hist_v, scale):
    """f64 summary (max, mass, numerator) of a key history against one landmark query."""
    if len(hist_k) == 0:
        return -np.inf, 0.0, np.zeros(q.shape[0])
    s = scale * (np.asarray(hist_k, np.float64) @ q.astype(np.float64))
    mx = s.max()
    e = np.exp(s - mx)
    return mx, e.sum(), e @ np.asarray(hist_v, np.float64)


def _history_setup(rng, inp, m=1):
    """Give each group a history of far_len evicted keys, every head one query shared by all
    rows, and an exact landmark 0 (q_tilde = that query). Returns (far, history per group)."""
    far = gen.make_far(inp, m, seed=int(rng.integers(1 << 30)))
    hist = []
    for g in range(inp.ng):
        n0 = int(inp.meta[g, 2])
        hk = rng.standard_normal((n0, inp.d)).astype(np.float32)
        hv = rng.standard_normal((n0, inp.d)).astype(np.float32)
        hist.append((hk, hv))
        for h in range(inp.hpg):
            gh = g * inp.hpg + h
            qh = rng.standard_normal(inp.d).astype(np.float32)
            inp.q[:, gh] = qh
            far.q_tilde[gh, 0] = qh
            mx, z, th = _exact_far_state(qh, hk, hv, inp.scale)
            far.mz[gh, 0], far.mz[gh, m] = mx, z
            far.t_hat[gh, 0] = th
    return far, hist


def _full_history_attention(inp, hist, i, gh):
    """Plain softmax of row i's query over every key its group has seen: sinks, the far
    history, all ring entries and chunk rows 0..i."""
    g = gh // inp.hpg
    ks, vs = _stream_entries(inp, g)
    keys = list(inp.sink_k[g]) + list(hist[g][0]) + ks + [inp.chunk_k[j, g] for j in range(i + 1)]
    vals = list(inp.sink_v[g]) + list(hist[g][1]) + vs + [inp.chunk_v[j, g] for j in range(i + 1)]
    q = inp.q[i, gh].astype(np.float64)
    s = inp.scale * (np.asarray(keys, np.float64) @ q)
    p = np.exp(s - s.max())
    return (p @ np.asarray(vals, np.float64)) / p.sum()


def test_far_empty_equals_near_attention():
    rng = np.random.default_rng(601)
    done = 0
    while done < 40:
        inp = _far_case(rng, rows=int(rng.integers(1, 5)), m=int(rng.integers(1, 4)),
                        hpg=int(rng.integers(1, 3)), far_len=0)
        wgs = [int(inp.meta[g, 3]) or inp.w for g in range(inp.ng)]
        if inp.rows > min(wgs):
            continue   # a chunk longer than a window evicts its own rows
        done += 1
        for g in range(inp.ng):   # no evictions: the chunk fits into every ring
            ov = int(inp.meta[g, 3])
            wg = ov if ov else inp.w
            inp.meta[g, 0] = min(int(inp.meta[g, 0]), max(0, wg - inp.rows))
        far = gen.make_far(inp, int(rng.integers(1, 4)), seed=int(rng.integers(1 << 30)))
        np.testing.assert_allclose(oracle.window_chunk_far(inp, far), oracle.window_chunk(inp),
                                   rtol=1e-6, atol=1e-7)


def test_far_exact_landmarks_give_full_history_attention():
    """One landmark whose query is the row's query summarises the evicted keys exactly. A row
    weighs landmark b by sum_a exp(scale <q, k_tilde_a>) mu[a][b] (not normalised), so with a
    zero landmark key and a mixing weight of 1 the weight is exactly 1: windowed attention plus
    the far field is then plain attention over everything the group has seen, evictions inside
    the chunk included."""
    rng = np.random.default_rng(602)
    for _ in range(60):
        inp = _far_case(rng, rows=int(rng.integers(1, 12)), hpg=int(rng.integers(1, 3)))
        far, hist = _history_setup(rng, inp)
        far.mu[:] = 1.0
        far.k_tilde[:] = 0.0
        got = oracle.window_chunk_far(inp, far)
        for i in range(inp.rows):
            for gh in range(inp.nh):
                np.testing.assert_allclose(got[i, gh], _full_history_attention(inp, hist, i, gh),
                                           rtol=2e-5, atol=2e-6)


def test_far_mixing_selects_the_landmark_its_row_names():
    """Landmark key 0 scores 0 and key 1 scores -400 against the row's query, so only row 0 of
    mu counts; mu[0] = (0, 1) routes the whole weight to landmark 1, which holds the exact
    history (mu is not symmetric: mu[1][0] = 0.7, so reading it transposed would weigh the
    exact state by 0.7 and landmark 0's unrelated state by 1)."""
    rng = np.random.default_rng(603)
    for _ in range(30):
        inp = _far_case(rng, rows=int(rng.integers(1, 6)), m=2, far_len=int(rng.integers(1, 4)))
        far, hist = _history_setup(rng, inp, m=2)
        for gh in range(inp.nh):   # move the exact summary to landmark 1
            far.q_tilde[gh, 1] = far.q_tilde[gh, 0]
            far.mz[gh, 1], far.mz[gh, 3] = far.mz[gh, 0], far.mz[gh, 2]
            far.t_hat[gh, 1] = far.t_hat[gh, 0]
            far.q_tilde[gh, 0] = rng.standard_normal(inp.d)
            far.mz[gh, 0] = far.mz[gh, 1] - 1.0
            far.mz[gh, 2] = 3.0
            far.t_hat[gh, 0] = rng.standard_normal(inp.d)
            far.mu[gh] = [[0.0, 1.0], [0.7, 0.0]]
        for g in range(inp.ng):
            q0 = inp.q[0, g * inp.hpg].astype(np.float64)
            far.k_tilde[g, 0] = 0.0
            far.k_tilde[g, 1] = -400.0 * q0 / (inp.scale * float(q0 @ q0))
        got = oracle.window_chunk_far(inp, far)
        for i in range(inp.rows):
            for gh in range(inp.nh):
                np.testing.assert_allclose(got[i, gh], _full_history_attention(inp, hist, i, gh),
                                           rtol=2e-5, atol=2e-6)


def test_far_negative_mass_is_dropped():
    """A negative far mass (mixing weight -1) drops the far part, evictions inside the chunk
    included: the result is the windowed attention alone."""
    rng = np.random.default_rng(604)
    for _ in range(30):
        inp = _far_case(rng, rows=int(rng.integers(1, 8)), far_len=int(rng.integers(1, 4)))
        far = gen.make_far(inp, 1, seed=int(rng.integers(1 << 30)))
        far.mu[:] = -1.0
        np.testing.assert_allclose(oracle.window_chunk_far(inp, far), oracle.window_chunk(inp),
                                   rtol=1e-6, atol=1e-7)


def test_far_commit_summarises_the_evicted_keys_exactly():
    rng = np.random.default_rng(605)
    for _ in range(60):
        inp = _far_case(rng, rows=int(rng.integers(1, 12)), m=2, hpg=int(rng.integers(1, 3)))
        far, hist = _history_setup(rng, inp, m=2)
        rk, rv, meta, mz, th = oracle.window_commit_far(inp, far)
        rk0, rv0, meta0 = oracle.window_commit(inp)
        np.testing.assert_array_equal(rk, rk0)
        np.testing.assert_array_equal(meta, meta0)
        for g in range(inp.ng):
            ks, vs = _stream_entries(inp, g)
            ks += [inp.chunk_k[j, g] for j in range(inp.rows)]
            vs += [inp.chunk_v[j, g] for j in range(inp.rows)]
            ov = int(inp.meta[g, 3])
            wg = ov if ov else inp.w
            nev = max(0, len(ks) - wg)   # the oldest entries leave the window
            hk = list(hist[g][0]) + ks[:nev]
            hv = list(hist[g][1]) + vs[:nev]
            assert int(meta[g, 2]) == int(inp.meta[g, 2]) + nev
            for h in range(inp.hpg):
                gh = g * inp.hpg + h
                mx, z, t = _exact_far_state(far.q_tilde[gh, 0], hk, hv, inp.scale)
                if nev == 0:   # untouched
                    np.testing.assert_array_equal(mz[gh], far.mz[gh])
                    np.testing.assert_array_equal(th[gh], far.t_hat[gh])
                    continue
                np.testing.assert_allclose(mz[gh, 0], mx, rtol=1e-6, atol=1e-6)
                np.testing.assert_allclose(mz[gh, 2], z, rtol=2e-6)
                np.testing.assert_allclose(th[gh, 0], t, rtol=2e-5, atol=2e-6)


def test_far_chunk_equals_sequence_of_decodes():
    """Row i of a chunk call with a far field == a one-row call on the state after the rows
    before it were committed with their far updates (any mixing, any landmark queries)."""
    rng = np.random.default_rng(606)
    for _ in range(25):
        inp = _far_case(rng, rows=int(rng.integers(1, 8)), m=int(rng.integers(1, 4)),
                        hpg=int(rng.integers(1, 3)))
        far = gen.make_far(inp, int(rng.integers(1, 4)), seed=int(rng.integers(1 << 30)),
                           mu_kind="positive")
        full = oracle.window_chunk_far(inp, far)
        state = _decode_state(inp)
        sfar = gen.FarState(far.m, far.k_tilde, far.q_tilde, far.mu, far.mz.copy(),
                            far.t_hat.copy())
        for i in range(inp.rows):
            _row_of(state, inp, i)
            np.testing.assert_allclose(oracle.window_chunk_far(state, sfar)[0], full[i],
                                       rtol=2e-5, atol=2e-6)
            state.ring_k, state.ring_v, state.meta, sfar.mz, sfar.t_hat = \
                oracle.window_commit_far(state, sfar)


# ── the gated one-row call with the far field (dory page, `dory_os` .. `dory_ogate`) ─────────

def _gated_far_case(rng, nk=2, hpg=2, hd=16, w=12, ns=2, m=1, far=3, scale=0.5):
    lens = [int(rng.integers(1, w + 1)) for _ in range(nk)]
    meta = [(lens[kh], int(rng.integers(0, w)), far, 0) for kh in range(nk)]
    return gen.make_gated_far(nk * hpg, nk, hd, w, ns, m, meta, seed=int(rng.integers(1 << 30)),
                              scale=scale)


def _gated_bruteforce(inp, extra=None):
    """sigmoid(gate * gate_scale) times f64 softmax attention (torch SDPA) of each head's query
    over its KV head's sinks, ring slots 0..len-1 and, if given, extra (K, V) rows per head."""
    out = np.zeros((inp.nh, inp.hd))
    hpg = inp.nh // inp.nk
    for gh in range(inp.nh):
        kh = gh // hpg
        ln = int(inp.meta[kh, 0])
        ks = [inp.sink_k[kh], inp.ring_k[kh, :ln]]
        vs = [inp.sink_v[kh], inp.ring_v[kh, :ln]]
        if extra is not None:
            ks.append(extra[gh][0])
            vs.append(extra[gh][1])
        k = torch.from_numpy(np.concatenate(ks).astype(np.float64))[None, None]
        v = torch.from_numpy(np.concatenate(vs).astype(np.float64))[None, None]
        q = torch.from_numpy(inp.q[gh].astype(np.float64))[None, None, None]
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=inp.scale)[0, 0, 0]
        g = torch.from_numpy((inp.gate[gh * inp.hd:(gh + 1) * inp.hd].astype(np.float64) *
                              inp.gate_scale[gh * inp.hd:(gh + 1) * inp.hd].astype(np.float64)))
        out[gh] = (o * torch.sigmoid(g)).numpy()
    return out


def _gated_exact_landmark(rng, inp, b=0, n_hist=None):
    """Landmark b of every head summarises a history of keys exactly for that head's query:
    returns the history per head."""
    hist = []
    m = inp.m
    for gh in range(inp.nh):
        n0 = n_hist if n_hist is not None else int(rng.integers(1, 6))
        hk = gen._unit_rows(rng, (n0, inp.hd))
        hv = rng.standard_normal((n0, inp.hd)).astype(np.float32)
        mx, z, th = _exact_far_state(inp.q[gh], hk, hv, inp.scale)
        inp.mz[gh, b], inp.mz[gh, m + b] = mx, z
        inp.t_hat[gh, b] = th
        hist.append((hk, hv))
    return hist


def test_gated_far_empty_field_is_gated_softmax():
    """No far count: the far state is never read and the result is the gated softmax over the
    sinks and the ring's slots 0..len-1. The state holds NaN on one pass and, on another, a
    finite state with positive weights and masses that would change the result if read."""
    rng = np.random.default_rng(701)
    for _ in range(20):
        inp = _gated_far_case(rng, nk=int(rng.integers(1, 4)), hpg=int(rng.integers(1, 4)),
                              ns=int(rng.integers(0, 3)), m=int(rng.integers(1, 4)), far=0,
                              scale=float(rng.choice([0.25, 4.0])))
        ref = _gated_bruteforce(inp)
        m = inp.m
        inp.mz[:, :m] = 3.0
        inp.mz[:, m:] = 2.0
        inp.t_hat[...] = 5.0
        np.testing.assert_allclose(oracle.window_gated_far(inp), ref, rtol=2e-6, atol=1e-7)
        for a in (inp.k_tilde, inp.mu, inp.mz, inp.t_hat):
            a[...] = np.nan
        np.testing.assert_allclose(oracle.window_gated_far(inp), ref, rtol=2e-6, atol=1e-7)


def test_gated_far_exact_landmark_gives_full_attention():
    """One landmark whose summary is exact for the head's query (zero landmark key, mixing
    weight 1): the gated call equals gated softmax over sinks, ring and the whole history."""
    rng = np.random.default_rng(702)
    for _ in range(20):
        inp = _gated_far_case(rng, nk=int(rng.integers(1, 4)), hpg=int(rng.integers(1, 4)),
                              ns=int(rng.integers(0, 3)), scale=float(rng.choice([0.25, 4.0])))
        inp.k_tilde[:] = 0.0
        inp.mu[:] = 1.0
        hist = _gated_exact_landmark(rng, inp)
        np.testing.assert_allclose(oracle.window_gated_far(inp), _gated_bruteforce(inp, hist),
                                   rtol=2e-5, atol=2e-6)


def test_gated_far_rect_clamps_negative_weights():
    """Landmark 0 is exact, landmark 1 gets weight -3 (mu row 0 = (1, -3), zero landmark keys)
    and a large mass. With rect the weight is clamped to 0: full attention with the history.
    Without it the far mass is negative and the far part is dropped: the near result."""
    rng = np.random.default_rng(703)
    for _ in range(20):
        inp = _gated_far_case(rng, m=2, scale=float(rng.choice([0.25, 4.0])))
        inp.k_tilde[:] = 0.0
        inp.mu[:] = 0.0
        inp.mu[:, 0, 0], inp.mu[:, 0, 1] = 1.0, -3.0
        hist = _gated_exact_landmark(rng, inp, b=0, n_hist=2)
        inp.mz[:, 1] = inp.mz[:, 0] + 2.0      # landmark 1: larger max and mass
        inp.mz[:, 3] = inp.mz[:, 2] * 5.0 + 1.0
        inp.rect = 1
        np.testing.assert_allclose(oracle.window_gated_far(inp), _gated_bruteforce(inp, hist),
                                   rtol=2e-5, atol=2e-6)
        inp.rect = 0
        np.testing.assert_allclose(oracle.window_gated_far(inp), _gated_bruteforce(inp),
                                   rtol=2e-6, atol=1e-7)


def test_gated_far_landmark_keys_of_the_rows_kv_head():
    """KV head kh's queries point along basis vector kh; its landmark key 1 is -200 times that
    vector (score -200 * |q| * scale) and key 0 is zero, so only row 0 of mu counts; mu[0] =
    (0, 1) routes the weight to landmark 1, which is exact; mu[1] = (0.7, 0) makes mu
    non-symmetric. Another KV head's landmark keys score 0 and would mix in landmark 0's
    unrelated state."""
    rng = np.random.default_rng(704)
    for _ in range(20):
        nk, hpg, hd = int(rng.integers(2, 4)), int(rng.integers(1, 3)), 16
        inp = _gated_far_case(rng, nk=nk, hpg=hpg, hd=hd, m=2, scale=1.0)
        for gh in range(inp.nh):
            kh = gh // hpg
            inp.q[gh] = 0.0
            inp.q[gh, kh] = float(rng.uniform(0.5, 1.5))
        inp.k_tilde[:] = 0.0
        for kh in range(nk):
            inp.k_tilde[kh, 1, kh] = -200.0
        inp.mu[:] = 0.0
        inp.mu[:, 0, 1] = 1.0
        inp.mu[:, 1, 0] = 0.7
        hist = _gated_exact_landmark(rng, inp, b=1)
        np.testing.assert_allclose(oracle.window_gated_far(inp), _gated_bruteforce(inp, hist),
                                   rtol=2e-5, atol=2e-6)


def test_gated_far_gate_zero_halves_the_ungated_result():
    """gate = 0 multiplies by sigmoid(0) = 1/2 exactly; a gate of 1e4 multiplies by 1."""
    rng = np.random.default_rng(705)
    for _ in range(10):
        inp = _gated_far_case(rng, nk=2, hpg=2, m=3, scale=2.0)
        inp.gate[:] = 0.0
        half = oracle.window_gated_far(inp)
        inp.gate[:] = 1e4
        inp.gate_scale[:] = 1.0
        full = oracle.window_gated_far(inp)
        np.testing.assert_array_equal(half, full * np.float32(0.5))


def test_gated_far_ring_storage_order_is_irrelevant():
    """The ring's live slots are a set: permuting slots 0..len-1 leaves the result unchanged."""
    rng = np.random.default_rng(706)
    for _ in range(10):
        inp = _gated_far_case(rng, nk=2, hpg=2, m=2, ns=1, scale=4.0)
        base = oracle.window_gated_far(inp)
        for kh in range(inp.nk):
            ln = int(inp.meta[kh, 0])
            perm = rng.permutation(ln)
            inp.ring_k[kh, :ln] = inp.ring_k[kh, perm]
            inp.ring_v[kh, :ln] = inp.ring_v[kh, perm]
        np.testing.assert_allclose(oracle.window_gated_far(inp), base, rtol=1e-6, atol=1e-7)


# ── encoder attention over packed sequences (egemma2 page, `eg_flash_body`, `eg_softmax`) ──

def _encoder_sdpa(inp, s, mask_fn=None):
    """f64 torch SDPA (non-causal, K/V heads repeated per group) of sequence s, optionally with
    a boolean keep-mask from mask_fn(len) -> [len][len]."""
    st, ln = int(inp.segs[s, 0]), int(inp.segs[s, 1])
    nh, nk, hd = inp.nh, inp.nk, inp.hd
    q = torch.from_numpy(inp.q[st:st + ln, :nh * hd].astype(np.float64)).view(ln, nh, hd)
    k = torch.from_numpy(inp.k[st:st + ln, :nk * hd].astype(np.float64)).view(ln, nk, hd)
    v = torch.from_numpy(inp.v[st:st + ln, :nk * hd].astype(np.float64)).view(ln, nk, hd)
    k = k.repeat_interleave(nh // nk, dim=1)
    v = v.repeat_interleave(nh // nk, dim=1)
    mask = None if mask_fn is None else torch.from_numpy(mask_fn(ln))
    o = torch.nn.functional.scaled_dot_product_attention(
        q.transpose(0, 1), k.transpose(0, 1).contiguous(), v.transpose(0, 1).contiguous(),
        attn_mask=mask, scale=inp.scale)
    return o.transpose(0, 1).reshape(ln, nh * hd).numpy()


def _band(window):
    def fn(n):
        i = np.arange(n)
        return np.abs(i[:, None] - i[None, :]) <= window
    return fn


def test_encoder_full_attention_matches_sdpa():
    rng = np.random.default_rng(801)
    for _ in range(12):
        nk = int(rng.integers(1, 4))
        nh = nk * int(rng.choice([1, 2, 4]))
        inp = gen.make_encoder([int(rng.integers(1, 80))], nh, nk, int(rng.choice([8, 16, 36])),
                               0, seed=int(rng.integers(1 << 30)), pad=int(rng.integers(0, 5)))
        got = oracle.encoder_attention(inp)
        np.testing.assert_allclose(got[:, :nh * inp.hd], _encoder_sdpa(inp, 0), rtol=2e-6, atol=1e-7)


def test_encoder_symmetric_window_matches_masked_sdpa():
    rng = np.random.default_rng(802)
    for _ in range(12):
        nk = int(rng.integers(1, 3))
        nh = nk * int(rng.choice([1, 3]))
        ln = int(rng.integers(2, 90))
        win = int(rng.integers(1, ln + 2))
        inp = gen.make_encoder([ln], nh, nk, 16, win, seed=int(rng.integers(1 << 30)))
        got = oracle.encoder_attention(inp)
        np.testing.assert_allclose(got[:, :nh * 16], _encoder_sdpa(inp, 0, _band(win)),
                                   rtol=2e-6, atol=1e-7)


def test_encoder_sequences_are_independent_and_gaps_untouched():
    """A packed call equals each sequence alone; rows between sequences keep their values."""
    rng = np.random.default_rng(803)
    for _ in range(8):
        lens = [int(x) for x in rng.integers(1, 40, size=int(rng.integers(1, 5)))]
        win = int(rng.choice([0, 1, 4]))
        inp = gen.make_encoder(lens, 4, 2, 8, win, seed=int(rng.integers(1 << 30)), gap=3, pad=2)
        sentinel = np.full((inp.q.shape[0], inp.nh * inp.hd + 1), 7.5, np.float32)
        got = oracle.encoder_attention(inp, out=sentinel)
        covered = np.zeros(inp.q.shape[0], bool)
        for s in range(len(lens)):
            st, ln = int(inp.segs[s, 0]), int(inp.segs[s, 1])
            covered[st:st + ln] = True
            mask = None if win == 0 else _band(win)
            np.testing.assert_allclose(got[st:st + ln, :inp.nh * inp.hd],
                                       _encoder_sdpa(inp, s, mask), rtol=2e-6, atol=1e-7)
        assert np.all(got[~covered] == 7.5)
        assert np.all(got[:, inp.nh * inp.hd:] == 7.5)


def test_encoder_uniform_weights_give_the_window_mean():
    """q = 0: every visible key weighs the same, so the output is the mean of the window's
    values: positions max(0, i - w) .. min(len, i + w + 1) - 1."""
    rng = np.random.default_rng(804)
    for win in (0, 1, 3, 50):
        inp = gen.make_encoder([23], 2, 1, 8, win, seed=int(rng.integers(1 << 30)))
        inp.q[:] = 0.0
        got = oracle.encoder_attention(inp)
        for i in range(23):
            lo, hi = (0, 23) if win == 0 else (max(0, i - win), min(23, i + win + 1))
            ref = inp.v[lo:hi, :8].astype(np.float64).mean(axis=0)
            for h in range(2):
                np.testing.assert_allclose(got[i, h * 8:(h + 1) * 8], ref, rtol=1e-6, atol=1e-7)


def test_encoder_key_order_is_irrelevant_without_a_window():
    rng = np.random.default_rng(805)
    inp = gen.make_encoder([37], 4, 2, 16, 0, seed=5)
    base = oracle.encoder_attention(inp)
    perm = rng.permutation(37)
    inp.k[:] = inp.k[perm]
    inp.v[:] = inp.v[perm]
    np.testing.assert_allclose(oracle.encoder_attention(inp), base, rtol=1e-6, atol=1e-7)
