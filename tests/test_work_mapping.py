"""The prefill work mapping is a bijection (CPU only).

Builds ``tests/work_mapping_check.cpp`` with hipcc for the host (it includes
the kernels' own ``fa_workmap.h``, so the code checked is the code the kernels
run) and runs it: over query-tile counts, pair counts, GQA group sizes and
chunk sizes (0 = the plain heaviest-first order, and sizes that do and do not
divide the XCD's pairs) every workgroup index maps to a distinct in-range
(query tile, pair), in the same order as the mapping written with plain
integer divisions; and the multiply-and-shift division the mapping uses
equals integer division exhaustively for small operands and on edge and
random operands up to 2^31 - 1.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def test_prefill_work_mapping_is_a_bijection(tmp_path):
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    exe = tmp_path / "work_mapping_check"
    subprocess.run([HIPCC, "-O1", "-std=c++17", "--offload-arch=gfx950", os.path.join(HERE, "work_mapping_check.cpp"),
                    "-o", str(exe)], check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok")
