"""The oracle's pins have teeth: plausible mistakes planted in a copy of the oracle fail them.

Each mutant is a one-line edit of ``oracle/oracle.c`` (a dropped term, a wrong sign, index or
operand), compiled on the CPU into a temporary library; the pin suite of test_oracle_pins.py is
then run against it and at least one pin must fail. The real oracle is restored afterwards.
"""
import os

import pytest

import oracle
import test_oracle_pins as pins

# (name, text in oracle.c, replacement)
MUTANTS = [
    ("window one short", "uint32_t win = wg < end ? wg : end;",
     "uint32_t win = wg - 1 < end ? wg - 1 : end;"),
    ("row excludes itself", "uint32_t end = len0 + (uint32_t)i + 1u;",
     "uint32_t end = len0 + (uint32_t)i + (i > 0 ? 0u : 1u);"),
    ("head offset ignored", "size_t slot = (size_t)((head0 + x) % wg);",
     "size_t slot = (size_t)(x % wg);"),
    ("modulus is w, not the group window", "size_t slot = (size_t)((head0 + x) % wg);",
     "size_t slot = (size_t)((head0 + x) % (uint32_t)w);"),
    ("override ignored", "return ov != 0u ? ov : (uint32_t)w;", "return (uint32_t)w;"),
    ("sinks dropped", "for (int s = 0; s < ns; ++s) {", "for (int s = 0; s < 0; ++s) {"),
    ("values read from keys", "vp[n] = ring_v + ((size_t)g * w + slot) * d;",
     "vp[n] = ring_k + ((size_t)g * w + slot) * d;"),
    ("chunk row of the wrong group", "kp[n] = chunk_k + (row * ng + g) * d;",
     "kp[n] = chunk_k + (row * ng + (ng - 1 - g)) * d;"),
    ("scale dropped", "sc[j] = scale * dot;", "sc[j] = dot;"),
    ("not normalised", "for (int e = 0; e < d; ++e) acc[e] /= l;",
     "for (int e = 0; e < d; ++e) acc[e] /= (l > 1.0 ? 1.0 : 1.0);"),
    ("query head of the wrong row", "const float *qv = q + ((size_t)i * nh + gh) * d;",
     "const float *qv = q + ((size_t)0 * nh + gh) * d;"),
    ("rotation sign", "double u = x * c - y * s, v = y * c + x * s;",
     "double u = x * c + y * s, v = y * c - x * s;"),
    ("sine of the neighbouring pair", "double c = rope_row[e], s = rope_row[half + e];",
     "double c = rope_row[e], s = rope_row[half + (e + 1) % half];"),
    ("key rotated with the previous row's table",
     "rotate_unit(yk + ((size_t)r * nk + kh) * hd, rope + (size_t)r * hd, hd, (double)eps, tmp);",
     "rotate_unit(yk + ((size_t)r * nk + kh) * hd, rope + (size_t)(r > 0 ? r - 1 : 0) * hd, hd, (double)eps, tmp);"),
    ("eps outside the square root", "double inv = 1.0 / sqrt(ss + eps);",
     "double inv = 1.0 / (sqrt(ss) + eps);"),
    ("gate sign", "z[e] = (float)(acc[e] / (1.0 + exp(-gs)));",
     "z[e] = (float)(acc[e] / (1.0 + exp(gs)));"),
    ("kv head interleaved", "int kh = a / hpg;", "int kh = a % nk;"),
    ("window start off by one", "long lo = pos + 1 > window ? pos + 1 - window : 0;",
     "long lo = pos + 1 > window ? pos - window : 0;"),
    ("query scale dropped", "for (int e = 0; e < hd; ++e) qd[e] *= (double)q_scale[(size_t)a * hd + e];",
     "for (int e = 0; e < hd; ++e) qd[e] *= 1.0;"),
    ("ring value not written", "vd[e] = vs[e];", "vd[e] = vd[e];"),
    ("commit slot ignores the head", "const uint32_t slot = (uint32_t)(((uint64_t)head + len) % wg);",
     "const uint32_t slot = (uint32_t)(((uint64_t)len) % wg);"),
    ("full ring keeps its head", "head = (head + 1) % wg;", "head = head % wg;"),
    ("far count not advanced", "far += 1;", "far += 0;"),
    ("commit takes the wrong group's row", "const float *ks = chunk_k + ((size_t)j * ng + g) * d;",
     "const float *ks = chunk_k + ((size_t)j * ng + (ng - 1 - g)) * d;"),
    ("far numerator not rescaled", "acc[c] += gb[b] * r[b] * (double)th[c];",
     "acc[c] += gb[b] * (double)th[c];"),
    ("mixing matrix transposed", "wb[b] += ea * (double)mu[((size_t)gh * m + a) * m + b];",
     "wb[b] += ea * (double)mu[((size_t)gh * m + b) * m + a];"),
    ("far mass one row behind", "far_den += gb[b] * z[(size_t)b * rows + i];",
     "far_den += gb[b] * z[(size_t)b * rows + (i > 0 ? i - 1 : 0)];"),
    ("negative far mass kept", "if (far_den >= 0.0) have = 1; else far_den = 0.0;", "have = 1;"),
    ("row's own eviction left out", "for (long j = j0 < 0 ? 0 : j0; j <= i; ++j) {",
     "for (long j = j0 < 0 ? 0 : j0; j < i; ++j) {"),
    ("old far mass not rescaled", "double acc = mass * r;", "double acc = mass;"),
    ("gain ignores the landmark max", "gb[b] = wb[b] * exp(f + mx[b] - cmax);",
     "gb[b] = wb[b] * exp(f - cmax);"),
    ("far-field call: query of the wrong row", "const float *qrow = q + ((size_t)i * nh + gh) * d;",
     "const float *qrow = q + ((size_t)0 * nh + gh) * d;"),
    ("far commit numerator not rescaled", "for (int c = 0; c < d; ++c) acc[c] = (double)th[c] * r;",
     "for (int c = 0; c < d; ++c) acc[c] = (double)th[c];"),
    ("gated far: rect ignored", "for (int b = 0; b < m; ++b) if (u[b] < 0.0) u[b] = 0.0;",
     "for (int b = 0; b < m; ++b) if (u[b] < 0.0) u[b] = u[b];"),
    ("gated far: empty far field read", "if (far > 0) {", "if (far >= 0) {"),
    ("gated far: one ring slot short", "const int n = ns + len;", "const int n = ns + len - (len > 1);"),
    ("gated far: landmark keys of KV head 0", "const float *kt = k_tilde + ((size_t)kh * m + a) * hd;",
     "const float *kt = k_tilde + ((size_t)0 * m + a) * hd;"),
    ("gated far: gate sign", "z[e] = (float)(acc[e] / den / (1.0 + exp(-gs)));",
     "z[e] = (float)(acc[e] / den / (1.0 + exp(gs)));"),
    ("gated far: far numerator dropped", "for (int e = 0; e < hd; ++e) acc[e] += gb[b] * (double)th[e];",
     "for (int e = 0; e < hd; ++e) acc[e] += 0.0 * gb[b] * (double)th[e];"),
    ("gated far: negative far mass kept", "have = far_den >= 0.0;   /* a negative far mass drops the far terms */",
     "have = 1;"),
    ("encoder: window one short on the right", "hi = i + window + 1 < len ? i + window + 1 : len;",
     "hi = i + window < len ? i + window : len;"),
    ("encoder: window one wide on the left", "lo = i > window ? i - window : 0;",
     "lo = i > window + 1 ? i - window - 1 : 0;"),
    ("encoder: KV heads interleaved", "h = (int)(rem % nh), kvh = h / group;",
     "h = (int)(rem % nh), kvh = h % nk;"),
    ("encoder: causal mask", "long lo = 0, hi = len;", "long lo = 0, hi = i + 1;"),
    ("encoder: keys from the start of the buffer",
     "kp[j] = k + (size_t)(start + lo + j) * ldk + (size_t)kvh * hd;",
     "kp[j] = k + (size_t)(lo + j) * ldk + (size_t)kvh * hd;"),
    ("encoder: values from the query row", "vp[j] = v + (size_t)(start + lo + j) * ldv + (size_t)kvh * hd;",
     "vp[j] = v + (size_t)(start + i) * ldv + (size_t)kvh * hd;"),
    ("gated far: mu transposed", "u[b] += ea * (double)mu[((size_t)gh * m + a) * m + b];",
     "u[b] += ea * (double)mu[((size_t)gh * m + b) * m + a];"),
]

PIN_TESTS = [getattr(pins, n) for n in dir(pins) if n.startswith("test_")]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(oracle.source_path()).read()
    assert src.count(old) == 1, f"mutation anchor not found once: {old!r}"
    mpath = os.path.join(tmp_path, "mutant.c")
    with open(mpath, "w") as f:
        f.write(src.replace(old, new))
    lib = oracle.load_library(oracle.compile_source(mpath, os.path.join(tmp_path, "libmutant.so")))
    caught = []
    try:
        oracle.use_library(lib)
        for t in PIN_TESTS:
            try:
                t()
            except (AssertionError, ValueError, FloatingPointError):
                caught.append(t.__name__)
    finally:
        oracle.use_library(None)
    assert caught, f"no pin caught the mutant '{name}'"
