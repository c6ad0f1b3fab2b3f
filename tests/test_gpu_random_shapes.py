"""Seeded random configurations of every entry point against the fp64 oracle.

Each case draws its shape from a fixed seed (batch, lengths with ragged
tails, GQA group, head dim, causal flag, dropout rate, split count), so the
sweep covers combinations the hand-picked parity cases do not, and is the
same on every run.  Tolerances are those of ``test_gpu_parity`` (bf16,
FP8) and ``test_gpu_dropout``.
"""
import numpy as np
import pytest

import oracle
from exact_io_aware_tile_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

BF16 = (2e-2, 2e-3)
FP8 = (0.08, 0.006)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_io_aware_tile_amd import fa
    fa.lib()
    return fa


def bdev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def u8dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def check(og, lg, o_ref, lse_ref, tol, what, s=1.0):
    err = np.abs(og - o_ref)
    assert np.isfinite(og).all(), what
    assert err.max() <= tol[0] * s, f"{what}: max |dO| {err.max():.3e}"
    assert err.mean() <= tol[1] * s, f"{what}: mean |dO| {err.mean():.3e}"
    fin = np.isfinite(lse_ref)
    np.testing.assert_array_equal(np.isfinite(lg), fin, err_msg=what)
    if fin.any():
        assert np.abs(lg[fin] - lse_ref[fin]).max() <= 1e-3, f"{what}: LSE"


def draw(i):
    rng = np.random.default_rng([7000, i])
    group = int(rng.choice([1, 2, 4, 8]))
    hkv = int(rng.integers(1, 4))
    return rng, group, hkv


@pytest.mark.parametrize("i", range(12))
def test_random_dense(gpu, i):
    rng, group, hkv = draw(i)
    d = int(rng.choice([64, 128, 256]))
    B = int(rng.integers(1, 4))
    nq = int(rng.integers(1, 700))
    nk = int(rng.integers(1, 700)) if rng.random() < 0.3 else nq
    causal = bool(rng.random() < 0.6)
    case = inputs.dense_case(7100 + i, B, nq, nk, hkv * group, hkv, d, dtype="bf16")
    o, lse = gpu.fa_fwd(*(bdev(case[n]) for n in ("q", "k", "v")), causal=causal)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.dense(case["q"], case["k"], case["v"], causal=causal)
    check(host(o).transpose(0, 2, 1, 3), lse.cpu().numpy().astype(np.float64), o_ref, l_ref, BF16,
          f"dense B={B} nq={nq} nk={nk} H={hkv * group}/{hkv} d={d} causal={causal}")


@pytest.mark.parametrize("i", range(10))
def test_random_varlen(gpu, i):
    rng, group, hkv = draw(100 + i)
    d = int(rng.choice([64, 128, 256]))
    lens = rng.integers(0, 600, size=int(rng.integers(1, 9)))
    causal = bool(rng.random() < 0.7)
    case = inputs.varlen_case(7200 + i, lens, hkv * group, hkv, d, dtype="bf16")
    cu = torch.from_numpy(case["cu_seqlens"]).cuda()
    if case["total"] == 0:
        return
    o, lse = gpu.fa_fwd_varlen(*(bdev(case[n]) for n in ("q", "k", "v")), cu, case["max_seqlen"], causal=causal)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.varlen(case["q"], case["k"], case["v"], case["cu_seqlens"], causal=causal)
    check(host(o).transpose(1, 0, 2), lse.cpu().numpy().astype(np.float64), o_ref, l_ref, BF16,
          f"varlen lens={lens.tolist()} H={hkv * group}/{hkv} d={d} causal={causal}")


@pytest.mark.parametrize("i", range(10))
def test_random_paged_prefill(gpu, i):
    rng, group, hkv = draw(200 + i)
    d = int(rng.choice([64, 128, 256]))
    n = int(rng.integers(1, 7))
    k_lens = rng.integers(0, 1500, size=n)
    q_lens = np.array([int(rng.integers(0, max(1, L) + 1)) if rng.random() < 0.8 else int(rng.integers(0, 300))
                       for L in k_lens])
    causal = bool(rng.random() < 0.7)
    case = inputs.paged_prefill_case(7300 + i, q_lens, k_lens, hkv * group, hkv, d, pad_blocks=int(rng.integers(0, 3)))
    if case["total_q"] == 0:
        return
    o, lse = gpu.fa_fwd_paged(bdev(case["q"]), bdev(case["k_pool"]), bdev(case["v_pool"]),
                              torch.from_numpy(case["block_table"]).cuda(),
                              torch.from_numpy(case["cu_seqlens_q"]).cuda(),
                              torch.from_numpy(case["seq_lens"]).cuda(), case["max_seqlen_q"],
                              int(case["seq_lens"].max(initial=0)), causal=causal)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.paged_prefill(case["q"], case["k_pool"], case["v_pool"], case["block_table"],
                                        case["cu_seqlens_q"], case["seq_lens"], causal=causal)
    check(host(o).transpose(1, 0, 2), lse.cpu().numpy().astype(np.float64), o_ref, l_ref, BF16,
          f"paged prefill q={q_lens.tolist()} k={k_lens.tolist()} H={hkv * group}/{hkv} d={d} causal={causal}")


@pytest.mark.parametrize("i", range(10))
def test_random_decode(gpu, i):
    rng, group, hkv = draw(300 + i)
    d = int(rng.choice([64, 128, 256]))
    lens = rng.integers(0, 3000, size=int(rng.integers(1, 12)))
    splits = int(rng.choice([0, 1, 5, 64]))
    fp8 = bool(rng.random() < 0.5)
    maxlen = int(lens.max())
    if fp8:
        case = inputs.paged_fp8_case(7400 + i, lens, hkv * group, hkv, d, pad_blocks=int(rng.integers(0, 3)))
        kp, vp = u8dev(case["k_pool"]), u8dev(case["v_pool"])
    else:
        case = inputs.paged_case(7400 + i, lens, hkv * group, hkv, d, pad_blocks=int(rng.integers(0, 3)))
        kp, vp = bdev(case["k_pool"]), bdev(case["v_pool"])
    bt, sl = torch.from_numpy(case["block_table"]).cuda(), torch.from_numpy(case["seq_lens"]).cuda()
    if fp8:
        o, lse = gpu.fa_decode_paged_fp8(bdev(case["q"]), kp, vp, bt, sl, maxlen, case["descale"], num_splits=splits)
    else:
        o, lse = gpu.fa_decode_paged(bdev(case["q"]), kp, vp, bt, sl, maxlen, num_splits=splits)
    torch.cuda.synchronize()
    if fp8:
        o_ref, l_ref = oracle.decode_paged_fp8(case["q"], case["k_pool"], case["v_pool"], case["block_table"],
                                               case["seq_lens"], case["descale"])
    else:
        o_ref, l_ref = oracle.decode_paged(case["q"], case["k_pool"], case["v_pool"], case["block_table"],
                                           case["seq_lens"])
    check(host(o), lse.cpu().numpy().astype(np.float64), o_ref, l_ref, BF16,
          f"decode fp8={fp8} lens={lens.tolist()} H={hkv * group}/{hkv} d={d} splits={splits}")


@pytest.mark.parametrize("i", range(8))
def test_random_fp8(gpu, i):
    rng, group, hkv = draw(400 + i)
    causal = bool(rng.random() < 0.6)
    if rng.random() < 0.5:
        B, nq = int(rng.integers(1, 3)), int(rng.integers(1, 600))
        nk = int(rng.integers(1, 600)) if rng.random() < 0.3 else nq
        case = inputs.fp8_case(7500 + i, B, nq, nk, hkv * group, hkv, 128)
        o, lse = gpu.fa_fwd_fp8(*(u8dev(case[n]) for n in ("q", "k", "v")), case["descale"], causal=causal)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.fp8_dense(case["q"], case["k"], case["v"], case["descale"], causal=causal)
        og = host(o).transpose(0, 2, 1, 3)
        what = f"fp8 dense B={B} nq={nq} nk={nk}"
    else:
        lens = rng.integers(0, 600, size=int(rng.integers(1, 7)))
        case = inputs.fp8_varlen_case(7500 + i, lens, hkv * group, hkv, 128)
        if case["total"] == 0:
            return
        o, lse = gpu.fa_fwd_varlen_fp8(*(u8dev(case[n]) for n in ("q", "k", "v")),
                                       torch.from_numpy(case["cu_seqlens"]).cuda(), case["max_seqlen"],
                                       case["descale"], causal=causal)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.fp8_varlen(case["q"], case["k"], case["v"], case["cu_seqlens"], case["descale"],
                                         causal=causal)
        og = host(o).transpose(1, 0, 2)
        what = f"fp8 varlen lens={lens.tolist()}"
    check(og, lse.cpu().numpy().astype(np.float64), o_ref, l_ref, FP8, f"{what} H={hkv * group}/{hkv} causal={causal}")


@pytest.mark.parametrize("i", range(8))
def test_random_dropout(gpu, i):
    rng, group, hkv = draw(500 + i)
    d = int(rng.choice([64, 128, 256]))
    p = float(rng.choice([0.05, 0.1, 0.3, 0.6]))
    seed, offset = int(rng.integers(0, 2**63)), int(rng.integers(0, 2**32))
    causal = bool(rng.random() < 0.7)
    t = oracle.dropout_threshold(p)
    s = 256.0 / (256 - t)
    if rng.random() < 0.5:
        B, nq = int(rng.integers(1, 3)), int(rng.integers(1, 500))
        case = inputs.dense_case(7600 + i, B, nq, nq, hkv * group, hkv, d, dtype="bf16")
        o, lse = gpu.fa_fwd_dropout(*(bdev(case[n]) for n in ("q", "k", "v")), dropout_p=p, seed=seed,
                                    offset=offset, causal=causal)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.dense_dropout(case["q"], case["k"], case["v"], causal=causal, dropout_p=p, seed=seed,
                                            offset=offset)
        og = host(o).transpose(0, 2, 1, 3)
        what = f"dropout dense B={B} n={nq}"
    else:
        lens = rng.integers(0, 500, size=int(rng.integers(1, 6)))
        case = inputs.varlen_case(7600 + i, lens, hkv * group, hkv, d, dtype="bf16")
        if case["total"] == 0:
            return
        o, lse = gpu.fa_fwd_varlen_dropout(*(bdev(case[n]) for n in ("q", "k", "v")),
                                           torch.from_numpy(case["cu_seqlens"]).cuda(), case["max_seqlen"],
                                           dropout_p=p, seed=seed, offset=offset, causal=causal)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.varlen_dropout(case["q"], case["k"], case["v"], case["cu_seqlens"], causal=causal,
                                             dropout_p=p, seed=seed, offset=offset)
        og = host(o).transpose(1, 0, 2)
        what = f"dropout varlen lens={lens.tolist()}"
    check(og, lse.cpu().numpy().astype(np.float64), o_ref, l_ref, BF16,
          f"{what} H={hkv * group}/{hkv} d={d} p={p} causal={causal}", s=s)
