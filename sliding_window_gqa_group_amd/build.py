"""Compile the HIP library libwinattn.so for gfx950 (in-tree, next to this file).

Each source is compiled to its own object in parallel, then the objects are linked into one
shared library (no relocatable device code: every kernel lives with its launcher).
"""
from __future__ import annotations

import hashlib
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libwinattn.so")
OBJDIR = os.path.join(HERE, "_build")
SOURCES = ["api.hip", "attn_dec.hip", "attn_valu.hip", "attn_mfma.hip", "attn_mfma16.hip",
           "gated_prep.hip", "ring_commit.hip", "far_field.hip",
           "enc_attn.hip", "attn_dec_far.hip", "read_probe.hip", "attn_decode.hip",
           "attn_gated.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions are kept out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
_NOISE = "packed-fp32-ops' is not a recognized feature"


# The sources the decode call's kernel is built from (its kernel, the shared device header, the
# launch declarations and the plan): counters taken on the decode call stay current while
# these are unchanged.
DECODE_SOURCES = ("api.hip", "attn_decode.hip", "attn_dec_block.h", "launch.h", "winattn_dev.h")


def source_digest(names=None) -> str:
    """Digest of kernel sources (`names` under csrc/, default every file there): measurements
    taken on other sources are not reported as current."""
    h = hashlib.sha256()
    for name in sorted(names if names is not None else os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if _NOISE not in ln]
    return res.returncode, msgs


def build(verbose: bool = False, defines=(), lib: str = LIB, objdir: str = OBJDIR) -> str:
    """Compile every source and link `lib`. `defines`: extra preprocessor macros (a timing
    build: see phase_stamps.py), with their own object folder and library name."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(objdir, exist_ok=True)
    extra = [f"-D{m}" for m in defines]
    jobs = []
    for s in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(s)[0] + ".o")
        jobs.append((obj, [hipcc, *HIPCC_FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-c",
                           os.path.join(CSRC, s), "-o", obj]))
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(lambda j: _run(j[1]), jobs))
    for (obj, cmd), (rc, msgs) in zip(jobs, results):
        if verbose:
            print(" ".join(cmd), flush=True)
        if rc != 0:
            raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + "\n".join(msgs))
        if verbose and msgs:
            print("\n".join(msgs))
    tmp = lib + ".tmp"
    link = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *[o for o, _ in jobs], "-o", tmp]
    rc, msgs = _run(link)
    if verbose:
        print(" ".join(link), flush=True)
    if rc != 0:
        raise RuntimeError("link failed:\n" + "\n".join(msgs))
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
