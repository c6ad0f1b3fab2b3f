"""Race check of the prefill pipelines' hand-ordered LDS ring.

The prefill kernels replace the workgroup barrier's release fence with a
plain ``s_barrier`` and wait, per wave, for exactly the LDS-DMA loads the
next phase reads (``wait_vmcnt<N>`` counted by hand).  A mistake there -- a
ring stage read before its loads landed, or refilled while another wave
still reads it -- would not necessarily show as a wrong answer on every run.

The race-check library (``_build/libfa_gfx950_synccheck.so``, built by
``build()`` from the same sources with FA_SYNC_CHECK) drains every memory
operation at each such wait and uses a full ``__syncthreads`` at each
barrier, so it cannot read a stage early.  Each case here runs the product
and the checking build on the same inputs and requires identical bits in O and LSE:
the arithmetic is the same instruction stream, so any difference is a
synchronisation error of the product.  Cases cover 1, 2 and 3 key tiles
(the pipeline's prologue and drain), many tiles with a ragged tail, several
query tiles, packed and paged keys, FP8, dropout, head dims 64/128/256, and
the full-size workload shapes.
"""
import contextlib
import os

import numpy as np
import pytest

from exact_io_aware_tile_amd import build as hipbuild
from exact_io_aware_tile_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def libs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_io_aware_tile_amd import fa
    prod = fa.lib()
    if not os.path.exists(hipbuild.SYNC_CHECK_LIB):
        pytest.fail("the race-check library is not built (python -m exact_io_aware_tile_amd.build)")
    chk = fa.load(hipbuild.SYNC_CHECK_LIB)
    return fa, prod, chk


@contextlib.contextmanager
def using(fa, L):
    saved = fa._lib
    fa._lib = L
    try:
        yield
    finally:
        fa._lib = saved


def both(libs, fn):
    """Run fn(fa) with the product and with the checking build; compare every
    output tensor bit for bit."""
    fa, prod, chk = libs
    with using(fa, prod):
        a = fn(fa)
    torch.cuda.synchronize()
    with using(fa, chk):
        b = fn(fa)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        if x is None:
            continue
        assert x.dtype == y.dtype and x.shape == y.shape
        assert torch.equal(x.contiguous().view(torch.uint8), y.contiguous().view(torch.uint8))


def bf(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


# key counts giving 1, 2 and 3 key tiles, and many with a ragged tail
# (64-key tiles at head dims 64/128 and in FP8, 32-key tiles at 256)
def nks(d):
    t = 32 if d == 256 else 64
    return [t, 2 * t, 3 * t, 1000]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_dense_bf16(libs, d, causal):
    for nk in nks(d):
        for nq in (nk, 300):
            c = inputs.dense_case(900 + nk + d, 1, nq, nk, 4, 2, d)
            q, k, v = bf(c["q"]), bf(c["k"]), bf(c["v"])
            both(libs, lambda fa: fa.fa_fwd(q, k, v, causal=causal))


@pytest.mark.parametrize("d", [64, 128, 256])
def test_varlen_bf16(libs, d):
    c = inputs.varlen_case(910 + d, [1, 64, 130, 700, 0, 33], 4, 2, d)
    q, k, v, cu = bf(c["q"]), bf(c["k"]), bf(c["v"]), i32(c["cu_seqlens"])
    both(libs, lambda fa: fa.fa_fwd_varlen(q, k, v, cu, c["max_seqlen"], causal=True))


@pytest.mark.parametrize("d", [64, 128, 256])
def test_paged_bf16(libs, d):
    c = inputs.paged_prefill_case(920 + d, [1, 130, 64, 300, 7], [1, 333, 64, 1000, 200], 8, 2, d, pad_blocks=1)
    q, kp, vp = bf(c["q"]), bf(c["k_pool"]), bf(c["v_pool"])
    bt, cu, sl = i32(c["block_table"]), i32(c["cu_seqlens_q"]), i32(c["seq_lens"])
    both(libs, lambda fa: fa.fa_fwd_paged(q, kp, vp, bt, cu, sl, c["max_seqlen_q"], 1000, causal=True))


@pytest.mark.parametrize("causal", [False, True])
def test_fp8(libs, causal):
    for nk in nks(128):
        c = inputs.fp8_case(930 + nk, 1, nk, nk, 4, 2, 128)
        q, k, v = u8(c["q"]), u8(c["k"]), u8(c["v"])
        both(libs, lambda fa: fa.fa_fwd_fp8(q, k, v, c["descale"], causal=causal))
    c = inputs.fp8_varlen_case(931, [1, 64, 130, 700], 4, 2, 128)
    q, k, v, cu = u8(c["q"]), u8(c["k"]), u8(c["v"]), i32(c["cu_seqlens"])
    both(libs, lambda fa: fa.fa_fwd_varlen_fp8(q, k, v, cu, c["max_seqlen"], c["descale"], causal=causal))
    c = inputs.paged_prefill_fp8_case(932, [1, 130, 300], [1, 333, 1000], 8, 2, 128)
    q, kp, vp = u8(c["q"]), u8(c["k_pool"]), u8(c["v_pool"])
    bt, cu, sl = i32(c["block_table"]), i32(c["cu_seqlens_q"]), i32(c["seq_lens"])
    both(libs, lambda fa: fa.fa_fwd_paged_fp8(q, kp, vp, bt, cu, sl, c["max_seqlen_q"], 1000, c["descale"],
                                              causal=causal))


@pytest.mark.parametrize("d", [128, 256])
def test_dropout(libs, d):
    for nk in nks(d):
        c = inputs.dense_case(940 + nk, 1, nk, nk, 4, 2, d)
        q, k, v = bf(c["q"]), bf(c["k"]), bf(c["v"])
        both(libs, lambda fa: fa.fa_fwd_dropout(q, k, v, dropout_p=0.1, seed=5, causal=True))
    c = inputs.varlen_case(941, [1, 64, 300], 4, 2, d)
    q, k, v, cu = bf(c["q"]), bf(c["k"]), bf(c["v"]), i32(c["cu_seqlens"])
    both(libs, lambda fa: fa.fa_fwd_varlen_dropout(q, k, v, cu, c["max_seqlen"], dropout_p=0.3, seed=6))


def test_full_size_workloads(libs):
    """Workloads 2 (B 4, H 32, N 2048, d 128, causal) and 7 (the same in
    FP8): every workgroup of the real grid, all CUs busy at once."""
    w = inputs.workload(2)
    q, k, v = bf(w["q"]), bf(w["k"]), bf(w["v"])
    both(libs, lambda fa: fa.fa_fwd(q, k, v, causal=True))
    del q, k, v
    c = inputs.fp8_case(7, 4, 2048, 2048, 32, 32, 128)
    q, k, v = u8(c["q"]), u8(c["k"]), u8(c["v"])
    both(libs, lambda fa: fa.fa_fwd_fp8(q, k, v, c["descale"], causal=True))
