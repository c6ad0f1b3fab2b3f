"""GPU parity of attention dropout (bf16 prefill, dense and packed) against the
fp64 oracle, through the C ABI.

* Keep decisions are compared bit for bit: with q = 0 every visible key has
  weight exactly 1 / n and each value row is a unit vector, so each output
  coordinate times n / scale is an integer count of kept keys, recovered
  exactly from the bf16 output and compared with the oracle's count.
* Outputs on random inputs: dropout scales every kept weight by
  s = 256 / (256 - t), so O is no longer a convex combination and both
  rounding errors of the bf16 path (the weights rounded to bf16 for P.V, the
  output rounded to bf16) scale with s: max |dO| <= 2e-2 * s and mean
  |dO| <= 2e-3 * s.  LSE does not depend on dropout and must equal the LSE
  of the plain kernel bit for bit (and the oracle's within 1e-3).
* p = 0 is the plain kernel bit for bit; the same (seed, offset) gives the
  same output; another seed or offset gives another mask.
"""
import numpy as np
import pytest

import oracle
from exact_io_aware_tile_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_io_aware_tile_amd import fa
    fa.lib()
    return fa


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def bf16_bits(x):
    return inputs.f32_to_bf16(np.asarray(x, np.float32))


def check(og, lg, o_ref, lse_ref, s, what):
    err = np.abs(og - o_ref)
    assert np.isfinite(og).all(), f"{what}: non-finite output"
    assert err.max() <= 2e-2 * s, f"{what}: max |dO| = {err.max():.3e} > {2e-2 * s:.3e}"
    assert err.mean() <= 2e-3 * s, f"{what}: mean |dO| = {err.mean():.3e} > {2e-3 * s:.3e}"
    fin = np.isfinite(lse_ref)
    np.testing.assert_array_equal(np.isfinite(lg), fin, err_msg=f"{what}: LSE finiteness")
    if fin.any():
        assert np.abs(lg[fin] - lse_ref[fin]).max() <= 1e-3, f"{what}: LSE"


def onehot_case(B, N, H, d):
    """q = 0, k random, v[j] = e_(j mod d) (bf16 bit patterns)."""
    q = np.zeros((B, N, H, d), np.float32)
    k = np.random.default_rng(N + d).standard_normal((B, N, H, d)).astype(np.float32)
    v = np.zeros((B, N, H, d), np.float32)
    v[:, np.arange(N), :, np.arange(N) % d] = 1.0
    return bf16_bits(q), bf16_bits(k), bf16_bits(v)


def kept_counts(o, n, s):
    """Per-coordinate kept-key counts from O = count * s / n."""
    return np.rint(o * n[..., None] / s).astype(np.int64)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 300, 3, 64), (1, 1000, 2, 128), (1, 64, 1, 64), (1, 1, 2, 128),
                                   (2, 300, 3, 256), (1, 33, 1, 256)])
@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_keep_decisions_bitwise(gpu, shape, causal, p):
    B, N, H, d = shape
    q, k, v = onehot_case(B, N, H, d)
    seed, offset = 0x0123456789ABCDEF, 7 + N
    t = oracle.dropout_threshold(p)
    s = 256.0 / (256 - t)
    o, lse = gpu.fa_fwd_dropout(dev(q), dev(k), dev(v), dropout_p=p, seed=seed, offset=offset, causal=causal)
    torch.cuda.synchronize()
    o_ref, _ = oracle.dense_dropout(q, k, v, causal=causal, dropout_p=p, seed=seed, offset=offset)
    og = host(o).transpose(0, 2, 1, 3)  # [B, H, N, d]
    n = np.broadcast_to((np.arange(N) + 1.0) if causal else np.full(N, float(N)), (B, H, N))
    got, want = kept_counts(og, n, s), kept_counts(o_ref, n, s)
    np.testing.assert_array_equal(got, want)
    # and the counts really are integers on the GPU side (no stray weights)
    np.testing.assert_allclose(og, want * s / n[..., None], rtol=2 ** -8, atol=0)
    # q = 0: every visible score is 0, so LSE = ln n whatever is dropped
    np.testing.assert_allclose(lse.cpu().numpy(), np.log(n), rtol=0, atol=1e-5)


def test_packed_keep_decisions_bitwise(gpu):
    lens = [1, 130, 0, 64, 257, 7, 128]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, H, d = int(cu[-1]), 2, 128
    q = np.zeros((T, H, d), np.float32)
    k = np.random.default_rng(5).standard_normal((T, H, d)).astype(np.float32)
    v = np.zeros((T, H, d), np.float32)
    for a, b in zip(cu[:-1], cu[1:]):
        v[a:b, :, :][np.arange(b - a), :, np.arange(b - a) % d] = 1.0
    q, k, v = bf16_bits(q), bf16_bits(k), bf16_bits(v)
    p, seed, offset = 0.3, 2 ** 40 + 3, 11
    s = 256.0 / (256 - oracle.dropout_threshold(p))
    for causal in (True, False):
        o, _ = gpu.fa_fwd_varlen_dropout(dev(q), dev(k), dev(v), torch.from_numpy(cu).cuda(), max(lens),
                                         dropout_p=p, seed=seed, offset=offset, causal=causal)
        torch.cuda.synchronize()
        o_ref, _ = oracle.varlen_dropout(q, k, v, cu, causal=causal, dropout_p=p, seed=seed, offset=offset)
        og = host(o).transpose(1, 0, 2)  # [H, T, d]
        n = np.zeros(T)
        for a, b in zip(cu[:-1], cu[1:]):
            n[a:b] = (np.arange(b - a) + 1.0) if causal else float(b - a)
        n = np.broadcast_to(n, (H, T))
        np.testing.assert_array_equal(kept_counts(og, n, s), kept_counts(o_ref, n, s))


DENSE = [
    # B, Nq, Nk, Hq, Hkv, d
    (2, 65, 65, 4, 2, 64),
    (1, 255, 255, 2, 2, 128),
    (1, 300, 300, 3, 1, 64),
    (1, 1000, 1000, 2, 2, 128),
    (1, 17, 200, 2, 2, 128),
    (1, 200, 70, 2, 2, 64),
    (1, 300, 300, 4, 2, 256),
    (1, 70, 200, 2, 2, 256),
]


@pytest.mark.parametrize("p", [0.1, 0.5])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", DENSE)
def test_dense_dropout_parity(gpu, shape, causal, p):
    B, Nq, Nk, Hq, Hkv, d = shape
    case = inputs.dense_case(300 + Nq + d, B, Nq, Nk, Hq, Hkv, d, dtype="bf16")
    q, k, v = (dev(case[n]) for n in ("q", "k", "v"))
    seed = 1000 + Nq
    o, lse = gpu.fa_fwd_dropout(q, k, v, dropout_p=p, seed=seed, causal=causal)
    _, lse_plain = gpu.fa_fwd(q, k, v, causal=causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.dense_dropout(case["q"], case["k"], case["v"], causal=causal, dropout_p=p, seed=seed)
    s = 256.0 / (256 - oracle.dropout_threshold(p))
    check(host(o).transpose(0, 2, 1, 3), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref, s,
          f"{shape} causal={causal} p={p}")
    if d == 64:
        # At head dim 64 the plain kernel takes 128-key tiles and the dropout
        # kernel 64-key ones, so the running max moves at different points:
        # the two LSEs agree to fp32 rounding of the sums, not bit for bit.
        assert torch.allclose(lse, lse_plain, rtol=0, atol=2e-6), "LSE must not depend on dropout"
    else:
        assert torch.equal(lse, lse_plain), "LSE must not depend on dropout"


@pytest.mark.parametrize("d", [64, 128, 256])
def test_varlen_dropout_parity(gpu, d):
    lens = [1, 130, 0, 64, 257, 7, 128]
    case = inputs.varlen_case(400 + d, lens, 4, 2, d, dtype="bf16")
    q, k, v = (dev(case[n]) for n in ("q", "k", "v"))
    cu = torch.from_numpy(case["cu_seqlens"]).cuda()
    p, seed, offset = 0.2, 77, 5
    o, lse = gpu.fa_fwd_varlen_dropout(q, k, v, cu, case["max_seqlen"], dropout_p=p, seed=seed, offset=offset,
                                       causal=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.varlen_dropout(case["q"], case["k"], case["v"], case["cu_seqlens"], causal=True,
                                           dropout_p=p, seed=seed, offset=offset)
    s = 256.0 / (256 - oracle.dropout_threshold(p))
    check(host(o).transpose(1, 0, 2), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref, s, f"varlen d={d}")


def test_single_packed_sequence_equals_dense_bitwise(gpu):
    """One sequence of N tokens numbers its rows h * N + i in both layouts."""
    N, H, d = 700, 3, 128
    case = inputs.dense_case(9, 1, N, N, H, H, d, dtype="bf16")
    q, k, v = (dev(case[n]) for n in ("q", "k", "v"))
    od, ld = gpu.fa_fwd_dropout(q, k, v, dropout_p=0.25, seed=5, offset=1, causal=True)
    cu = torch.tensor([0, N], dtype=torch.int32).cuda()
    ov, lv = gpu.fa_fwd_varlen_dropout(q[0], k[0], v[0], cu, N, dropout_p=0.25, seed=5, offset=1, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(od[0], ov)
    assert torch.equal(ld[0], lv)


def test_zero_probability_is_plain_and_masks_are_reproducible(gpu):
    case = inputs.dense_case(21, 2, 333, 333, 4, 2, 128, dtype="bf16")
    q, k, v = (dev(case[n]) for n in ("q", "k", "v"))
    o0, l0 = gpu.fa_fwd(q, k, v, causal=True)
    o1, l1 = gpu.fa_fwd_dropout(q, k, v, dropout_p=0.0, seed=3, causal=True)
    a, _ = gpu.fa_fwd_dropout(q, k, v, dropout_p=0.3, seed=3, offset=0, causal=True)
    b, _ = gpu.fa_fwd_dropout(q, k, v, dropout_p=0.3, seed=3, offset=0, causal=True)
    c, _ = gpu.fa_fwd_dropout(q, k, v, dropout_p=0.3, seed=3, offset=1, causal=True)
    e, _ = gpu.fa_fwd_dropout(q, k, v, dropout_p=0.3, seed=4, offset=0, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    assert torch.equal(a, b)
    assert not torch.equal(a, c) and not torch.equal(a, e)


def test_dropout_workload_sampled(gpu):
    """The causal prefill workload (B=4, H=32, N=2048, d=128) with p = 0.1, on
    sampled rows (tile edges and the last rows included)."""
    case = inputs.workload(2)
    B, N, H = case["batch"], case["nq"], case["hq"]
    rng = np.random.default_rng(12)
    ids = set(rng.integers(0, B * H * N, size=256).tolist())
    for i in (0, 63, 64, 255, 256, N - 65, N - 64, N - 1):
        ids.add(int(rng.integers(0, B * H)) * N + i)
    rows = np.array(sorted(ids), dtype=np.int64)
    q, k, v = (dev(case[n]) for n in ("q", "k", "v"))
    p, seed, offset = 0.1, 0xC0FFEE, 2
    o, lse = gpu.fa_fwd_dropout(q, k, v, dropout_p=p, seed=seed, offset=offset, causal=case["causal"])
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.dense_dropout(case["q"], case["k"], case["v"], causal=case["causal"], dropout_p=p,
                                          seed=seed, offset=offset, rows=rows)
    og = host(o).transpose(0, 2, 1, 3).reshape(-1, case["d"])[rows]
    lg = lse.cpu().numpy().astype(np.float64).reshape(-1)[rows]
    check(og, lg, o_ref, lse_ref, 256.0 / (256 - oracle.dropout_threshold(p)), "workload sampled rows")
