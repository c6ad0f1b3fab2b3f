"""Build libfa_gfx950.so in-tree with hipcc (gfx950 only).

    python -m exact_io_aware_tile_amd.build

Each source compiles to an object under ``exact_io_aware_tile_amd/_build``
(in parallel), then hipcc links the shared library next to this file.  The
packed-fp32 target feature is disabled for every device pass.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfa_gfx950.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

SOURCES = ["fa_api.cpp", "fa_fwd_bf16.hip", "fa_fwd_bf16_d256.hip", "fa_fwd_fp8.hip", "fa_fwd_f32.hip", "fa_decode.hip", "fa_merge.hip"]
# The race-check library: the same library with the prefill pipelines' hand
# ordered waits and barriers replaced by full ones (FA_SYNC_CHECK); only the
# tests load it, to compare it bit for bit with the product.
SYNC_CHECK_LIB = os.path.join(BUILD, "libfa_gfx950_synccheck.so")
SYNC_CHECK_SOURCES = ["fa_fwd_bf16.hip", "fa_fwd_bf16_d256.hip", "fa_fwd_fp8.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument", "-I" + INCLUDE,
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; drop that note.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if err.strip():
        print(err, file=sys.stderr)


def _link(objs, out):
    tmp = out + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, out)


def build(out: str = LIB, jobs: int | None = None, verbose: bool = False, sync_check: bool = True) -> str:
    """Compile every source and link the library; with sync_check, also the
    race-check library (SYNC_CHECK_LIB) from the same sources."""
    os.makedirs(BUILD, exist_ok=True)
    objs, chk_objs, cmds = [], [], []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        if src in SYNC_CHECK_SOURCES:
            chk = os.path.join(BUILD, os.path.splitext(src)[0] + ".synccheck.o")
            chk_objs.append(chk)
            if sync_check:
                cmds.append([HIPCC, *FLAGS, "-DFA_SYNC_CHECK", "-c", os.path.join(CSRC, src), "-o", chk])
        else:
            chk_objs.append(obj)
    jobs = jobs or min(len(cmds), 8)
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(_run, cmds))
    _link(objs, out)
    if sync_check:
        _link(chk_objs, SYNC_CHECK_LIB)
    if verbose:
        print(f"built {out}" + (f" and {SYNC_CHECK_LIB}" if sync_check else ""))
    return out


if __name__ == "__main__":
    build(verbose=True)
