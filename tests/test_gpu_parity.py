"""GPU parity: the HIP kernels, called through the C ABI, against the fp64 oracle.

Tolerances: fp32 I/O max |dO| <= 1e-5; bf16 I/O max |dO| <= 2e-2 and mean
|dO| <= 2e-3; max |dLSE| <= 1e-3 (natural log).  Inputs are the seeded
generators of exact_io_aware_tile_amd.inputs; the oracle sees exactly the
bytes the GPU sees.
"""
import math

import numpy as np
import pytest

import oracle
from exact_io_aware_tile_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, None), "bf16": (2e-2, 2e-3)}
LSE_TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_io_aware_tile_amd import fa
    fa.lib()  # must load; no fallback exists
    return fa


def dev(a, dtype):
    """Host array (float32, or uint16 bf16 bits) -> GPU tensor with the same bytes."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.cuda()


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def check(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what=""):
    tmax, tmean = TOL[dtype]
    err = np.abs(o_gpu - o_ref)
    assert np.isfinite(o_gpu).all(), f"{what}: non-finite output"
    assert err.max() <= tmax, f"{what}: max |dO| = {err.max():.3e} > {tmax}"
    if tmean is not None:
        assert err.mean() <= tmean, f"{what}: mean |dO| = {err.mean():.3e} > {tmean}"
    if lse_gpu is not None:
        fin = np.isfinite(lse_ref)
        np.testing.assert_array_equal(np.isfinite(lse_gpu), fin, err_msg=f"{what}: LSE finiteness")
        np.testing.assert_array_equal(lse_gpu[~fin], lse_ref[~fin])
        if fin.any():
            e = np.abs(lse_gpu[fin] - lse_ref[fin]).max()
            assert e <= LSE_TOL, f"{what}: max |dLSE| = {e:.3e}"


def run_dense(fa, case, causal, rows=None):
    dt = case["dtype"]
    q, k, v = (dev(case[n], dt) for n in ("q", "k", "v"))
    o, lse = fa.fa_fwd(q, k, v, causal=causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.dense(case["q"], case["k"], case["v"], causal=causal, rows=rows)
    og = host(o).transpose(0, 2, 1, 3)  # [B, Hq, Nq, d]
    lg = lse.cpu().numpy().astype(np.float64)
    if rows is not None:
        og = og.reshape(-1, og.shape[-1])[rows]
        lg = lg.reshape(-1)[rows]
    return og, lg, o_ref, lse_ref


DENSE_SHAPES = [
    # B, Nq, Nk, Hq, Hkv, d
    (1, 1, 1, 1, 1, 64),
    (2, 17, 17, 2, 2, 64),
    (1, 63, 63, 2, 1, 128),
    (1, 64, 64, 1, 1, 128),
    (2, 65, 65, 4, 2, 64),
    (1, 255, 255, 2, 2, 128),
    (1, 300, 300, 3, 1, 64),
    (1, 1000, 1000, 2, 2, 128),
    (1, 17, 200, 2, 2, 128),   # fewer queries than keys (end-aligned causal)
    (1, 200, 70, 2, 2, 64),    # more queries than keys: first rows see nothing when causal
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", DENSE_SHAPES)
def test_dense_parity(gpu, shape, causal, dtype):
    B, Nq, Nk, Hq, Hkv, d = shape
    case = inputs.dense_case(100 + Nq + d, B, Nq, Nk, Hq, Hkv, d, dtype=dtype)
    og, lg, o_ref, lse_ref = run_dense(gpu, case, causal)
    check(og, lg, o_ref, lse_ref, dtype, f"{shape} causal={causal} {dtype}")


D256_SHAPES = [
    # B, Nq, Nk, Hq, Hkv, d -- head_dim 256 (16 rows per wave, 32-key tiles)
    (1, 1, 1, 1, 1, 256),
    (2, 17, 17, 2, 2, 256),
    (1, 31, 31, 2, 1, 256),
    (1, 127, 127, 2, 1, 256),
    (1, 128, 128, 1, 1, 256),
    (2, 129, 129, 4, 2, 256),
    (1, 300, 300, 3, 1, 256),
    (1, 1000, 1000, 2, 2, 256),
    (1, 17, 200, 2, 2, 256),
    (1, 200, 70, 2, 2, 256),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", D256_SHAPES)
def test_d256_parity(gpu, shape, causal):
    B, Nq, Nk, Hq, Hkv, d = shape
    case = inputs.dense_case(500 + Nq, B, Nq, Nk, Hq, Hkv, d, dtype="bf16")
    og, lg, o_ref, lse_ref = run_dense(gpu, case, causal)
    check(og, lg, o_ref, lse_ref, "bf16", f"{shape} causal={causal} d=256")


@pytest.mark.parametrize("causal", [True, False])
def test_d256_varlen_parity(gpu, causal):
    lens = [1, 130, 0, 64, 257, 7, 128, 31]
    case = inputs.varlen_case(256, lens, 4, 2, 256, dtype="bf16")
    og, lg, o_ref, lse_ref = run_varlen(gpu, case, causal)
    check(og, lg, o_ref, lse_ref, "bf16", f"varlen d=256 causal={causal}")


def test_d256_workload_sampled(gpu):
    case = inputs.workload(9)
    B, N, H = case["batch"], case["nq"], case["hq"]
    rows = sample_rows(np.random.default_rng(9), B, H, N, 256)
    og, lg, o_ref, lse_ref = run_dense(gpu, case, case["causal"], rows=rows)
    check(og, lg, o_ref, lse_ref, "bf16", "d=256 workload sampled rows")


def test_d256_empty_keys(gpu):
    q = torch.randn(1, 40, 2, 256, device="cuda").to(torch.bfloat16)
    k = torch.zeros(1, 0, 2, 256, device="cuda", dtype=torch.bfloat16)
    o, lse = gpu.fa_fwd(q, k, k, causal=False)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_workload1_fp32(gpu):
    case = inputs.workload(1)
    og, lg, o_ref, lse_ref = run_dense(gpu, case, case["causal"])
    check(og, lg, o_ref, lse_ref, "f32", "fp32 N=256 d=64")


def test_worked_example_on_gpu(gpu):
    """Row 1, 0.5, 2, 1.5 | 3, 0.2, 1, 2.5 from the merge-rule worked example on
    the "FlashAttention" page of tachyon.techntrek.in: with q = 8 e0, k_j =
    row_j e0 (scale 1/8) and V = identity, O is the softmax row and
    exp(LSE - 3) is the merged l printed as 2.611."""
    row = np.array([1.0, 0.5, 2.0, 1.5, 3.0, 0.2, 1.0, 2.5], dtype=np.float32)
    d, n = 64, 8
    q = np.zeros((1, 1, 1, d), np.float32)
    q[0, 0, 0, 0] = 8.0
    k = np.zeros((1, n, 1, d), np.float32)
    k[0, :, 0, 0] = row
    v = np.zeros((1, n, 1, d), np.float32)
    v[0, np.arange(n), 0, np.arange(n)] = 1.0
    o, lse = gpu.fa_fwd(dev(q, "f32"), dev(k, "f32"), dev(v, "f32"), causal=False, scale=0.125)
    torch.cuda.synchronize()
    w = host(o)[0, 0, 0, :n]
    L = float(lse.cpu()[0, 0, 0])
    assert abs(math.exp(L - 3.0) - 2.611) < 1e-3
    assert abs(math.exp(L - 2.0) * w[:4].sum() - 2.198) < 1e-3
    assert abs(math.exp(L - 3.0) * w[4:].sum() - 1.803) < 1e-3
    o_ref, l_ref = oracle.dense(q, k, v, causal=False, scale=0.125)
    np.testing.assert_allclose(w, o_ref[0, 0, 0, :n], atol=1e-6, rtol=0)
    assert abs(L - l_ref[0, 0, 0]) < 1e-5
    assert abs(w.sum() - 1.0) < 1e-5


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_closed_forms_on_gpu(gpu, dtype):
    B, N, H, d = 1, 300, 2, 128
    case = inputs.dense_case(7, B, N, N, H, H, d, dtype=dtype)
    ones = np.ones((B, N, H, d), np.float32)
    v1 = inputs.f32_to_bf16(ones) if dtype == "bf16" else ones
    q, k = dev(case["q"], dtype), dev(case["k"], dtype)
    o, _ = gpu.fa_fwd(q, k, dev(v1, dtype), causal=True)
    assert np.abs(host(o) - 1.0).max() <= TOL[dtype][0]
    # q = 0: uniform weights, LSE = ln(i + 1) under the causal mask
    zq = torch.zeros_like(q)
    o, lse = gpu.fa_fwd(zq, k, dev(case["v"], dtype), causal=True)
    torch.cuda.synchronize()
    ln = np.log(np.arange(1, N + 1))
    assert np.abs(lse.cpu().numpy()[0] - ln[None]).max() < 1e-4
    vv = (inputs.bf16_to_f32(case["v"]) if dtype == "bf16" else case["v"]).astype(np.float64)
    mean = np.cumsum(vv[0], axis=0) / np.arange(1, N + 1)[:, None, None]
    assert np.abs(host(o)[0] - mean).max() <= TOL[dtype][0]


@pytest.mark.parametrize("d", [64, 128, 256])
def test_prefix_property_on_gpu(gpu, d):
    """Causal row i equals non-causal attention of query i over keys 0..i
    (a separate call with seqlen_k = i + 1)."""
    N, H = 300, 2
    case = inputs.dense_case(40 + d, 1, N, N, H, H, d, dtype="bf16")
    q, k, v = (dev(case[n], "bf16") for n in ("q", "k", "v"))
    o, lse = gpu.fa_fwd(q, k, v, causal=True)
    for i in (0, 1, 31, 63, 64, 127, 128, 255, 256, 299):
        oi, li = gpu.fa_fwd(q[:, i:i + 1].contiguous(), k[:, :i + 1].contiguous(), v[:, :i + 1].contiguous(),
                            causal=False)
        torch.cuda.synchronize()
        assert (o[:, i:i + 1].float() - oi.float()).abs().max().item() <= TOL["bf16"][0], i
        assert (lse[:, :, i:i + 1] - li).abs().max().item() <= 1e-4, i


@pytest.mark.parametrize("d", [64, 128, 256])
def test_identity_values_give_softmax_rows(gpu, d):
    """V = identity (N_k = d keys): O row i is the weight row P_i, which sums
    to one and matches the oracle's weights."""
    N, H = d, 2
    case = inputs.dense_case(60 + d, 1, N, N, H, H, d, dtype="bf16")
    eye = np.zeros((1, N, H, d), np.float32)
    eye[0, np.arange(N), :, np.arange(N)] = 1.0
    v = inputs.f32_to_bf16(eye)
    for causal in (False, True):
        o, _ = gpu.fa_fwd(dev(case["q"], "bf16"), dev(case["k"], "bf16"), dev(v, "bf16"), causal=causal)
        torch.cuda.synchronize()
        og = host(o)
        assert np.abs(og.sum(-1) - 1.0).max() <= 2e-2
        o_ref, _ = oracle.dense(case["q"], case["k"], v, causal=causal)
        check(og.transpose(0, 2, 1, 3), None, o_ref, None, "bf16", f"identity d={d} causal={causal}")


def test_strided_views(gpu):
    B, N, H, d = 2, 130, 2, 128
    big = inputs.dense_case(8, B, N, N, 2 * H, 2 * H, d, dtype="bf16")
    q = dev(big["q"], "bf16")[:, :, 1::2]  # head stride 2*d
    k = dev(big["k"], "bf16")[:, :, :H]
    v = dev(big["v"], "bf16")[:, :, H:]
    out = torch.empty((B, N, 2 * H, d), dtype=torch.bfloat16, device="cuda")[:, :, ::2]
    o, lse = gpu.fa_fwd(q, k, v, causal=True, out=out)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.dense(big["q"][:, :, 1::2], big["k"][:, :, :H], big["v"][:, :, H:], causal=True)
    check(host(o).transpose(0, 2, 1, 3), lse.cpu().numpy().astype(np.float64), o_ref, l_ref, "bf16",
          "strided")


def _spread_rows(src, row_stride, fill=float("nan")):
    """Device copy of a contiguous [1, N, 1, d] tensor whose rows lie row_stride
    elements apart in one buffer filled with FILL elsewhere (a stray read of
    the gaps shows up as a non-finite output)."""
    _, N, _, d = src.shape
    buf = torch.full(((N - 1) * row_stride + d,), fill, dtype=src.dtype, device="cuda")
    view = buf.as_strided((1, N, 1, d), (0, row_stride, d, 1))
    view.copy_(src)
    return view


@pytest.mark.parametrize("d", [128, 256])
def test_max_kv_row_stride(gpu, d):
    """k/v rows 2^24 elements apart (the largest stride the bf16 kernels'
    32-bit lane offsets accept), over several tiles and a ragged tail."""
    N = 100
    case = inputs.dense_case(70 + d, 1, N, N, 1, 1, d, dtype="bf16")
    q = dev(case["q"], "bf16")
    k = _spread_rows(dev(case["k"], "bf16"), 1 << 24)
    v = _spread_rows(dev(case["v"], "bf16"), 1 << 24)
    for causal in (False, True):
        o, lse = gpu.fa_fwd(q, k, v, causal=causal)
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle.dense(case["q"], case["k"], case["v"], causal=causal)
        check(host(o).transpose(0, 2, 1, 3), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref, "bf16",
              f"k/v row stride 2^24 d={d} causal={causal}")
    del k, v
    torch.cuda.empty_cache()


def test_max_kv_row_stride_fp8(gpu):
    N = 100
    case = inputs.fp8_case(75, 1, N, N, 1, 1, 128)
    q = torch.from_numpy(case["q"]).cuda()
    k = _spread_rows(torch.from_numpy(case["k"]).cuda(), 1 << 24, fill=0x7F)  # 0x7F: E4M3 NaN
    v = _spread_rows(torch.from_numpy(case["v"]).cuda(), 1 << 24, fill=0x7F)
    o, lse = gpu.fa_fwd_fp8(q, k, v, case["descale"], causal=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.fp8_dense(case["q"], case["k"], case["v"], case["descale"], causal=True)
    check_fp8(host(o).transpose(0, 2, 1, 3), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref,
              "fp8 k/v row stride 2^24")
    del k, v
    torch.cuda.empty_cache()


@pytest.mark.parametrize("d", [128, 256])
def test_decode_max_token_stride(gpu, d):
    """Pool tokens 2^26 elements apart (the largest token stride the decode
    kernel's 32-bit lane offsets accept), two sequences over two blocks."""
    lens = [20, 9]
    case = inputs.paged_case(80 + d, lens, 2, 1, d)
    nb = case["k_pool"].shape[0]
    ts = 1 << 26
    def spread(a):
        buf = torch.full(((nb * 16 - 1) * ts + d,), float("nan"), dtype=torch.bfloat16, device="cuda")
        view = buf.as_strided((nb, 1, 16, d), (16 * ts, 16 * ts, ts, 1))
        view.copy_(dev(a, "bf16"))
        return view
    kp, vp = spread(case["k_pool"]), spread(case["v_pool"])
    o, lse = decode_gpu(gpu, case, k_pool=kp, v_pool=vp)
    o_ref, lse_ref = oracle.decode_paged(case["q"], case["k_pool"], case["v_pool"], case["block_table"],
                                         case["seq_lens"])
    check(host(o), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref, "bf16", f"decode token stride 2^26 d={d}")
    del kp, vp
    torch.cuda.empty_cache()


def test_concurrent_streams_bitwise(gpu):
    """Calls are re-entrant on distinct streams: a prefill and a decode
    enqueued on two (default-priority) streams at once give the bits each
    gives alone."""
    c = inputs.dense_case(90, 2, 700, 700, 4, 2, 128, dtype="bf16")
    q, k, v = (dev(c[n], "bf16") for n in ("q", "k", "v"))
    p = inputs.paged_case(91, [3000, 17, 900], 8, 2, 128)
    dq, kp, vp = dev(p["q"], "bf16"), dev(p["k_pool"], "bf16"), dev(p["v_pool"], "bf16")
    bt, sl = torch.from_numpy(p["block_table"]).cuda(), torch.from_numpy(p["seq_lens"]).cuda()
    o1, l1 = gpu.fa_fwd(q, k, v, causal=True)
    d1, dl1 = gpu.fa_decode_paged(dq, kp, vp, bt, sl, 3000)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            a = gpu.fa_fwd(q, k, v, causal=True, stream=s1)
        with torch.cuda.stream(s2):
            b = gpu.fa_decode_paged(dq, kp, vp, bt, sl, 3000, stream=s2)
        outs.append((a, b))
    torch.cuda.synchronize()
    for (o2, l2), (d2, dl2) in outs:
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        assert torch.equal(d1, d2) and torch.equal(dl1, dl2)


def test_empty_keys(gpu):
    q = torch.randn(1, 5, 2, 64, device="cuda").to(torch.bfloat16)
    k = torch.zeros(1, 0, 2, 64, device="cuda", dtype=torch.bfloat16)
    o, lse = gpu.fa_fwd(q, k, k, causal=False)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def sample_rows(rng, B, H, N, n):
    """Row ids (b*H + h)*N + i: random rows plus tile edges and the last row."""
    ids = set(rng.integers(0, B * H * N, size=n).tolist())
    for i in (0, 1, 63, 64, 127, 128, N - 129, N - 128, N - 65, N - 64, N - 2, N - 1):
        if 0 <= i < N:
            ids.add(int(rng.integers(0, B * H)) * N + i)
    return np.array(sorted(ids), dtype=np.int64)


@pytest.mark.parametrize("wl", [2, 3])
def test_prefill_workloads_sampled(gpu, wl):
    case = inputs.workload(wl)
    B, N, H = case["batch"], case["nq"], case["hq"]
    rows = sample_rows(np.random.default_rng(wl), B, H, N, 384)
    og, lg, o_ref, lse_ref = run_dense(gpu, case, case["causal"], rows=rows)
    check(og, lg, o_ref, lse_ref, "bf16", f"workload {wl} sampled rows")


def test_prefill_full_size_properties(gpu):
    """At full size every output row is a convex combination of value rows
    (inside their per-dimension range) and every LSE is finite."""
    case = inputs.workload(3)
    q, k, v = (dev(case[n], "bf16") for n in ("q", "k", "v"))
    o, lse = gpu.fa_fwd(q, k, v, causal=True)
    of = o.float()
    assert torch.isfinite(of).all() and torch.isfinite(lse).all()
    vf = v.float()
    vmin = torch.cummin(vf, dim=1).values  # causal: keys 0..i
    vmax = torch.cummax(vf, dim=1).values
    # o is divided by the sum of the weights P.V took, so the fp32 row is a
    # convex combination of value rows up to fp32 rounding, and rounding it
    # to bf16 (monotone, the hull's bounds being bf16 values) cannot leave
    # the hull: only fp32 rounding noise is allowed.
    slack = 1e-3
    assert bool((of >= vmin - slack).all()) and bool((of <= vmax + slack).all())
    # LSE >= the row's own diagonal score (that key is always visible)
    diag = (q.float() * k.float()).sum(-1) / math.sqrt(case["d"])  # [B, N, H]
    assert bool((lse.permute(0, 2, 1) >= diag - 1e-3).all())


# --------------------------------------------------------------------------
# packed variable-length
# --------------------------------------------------------------------------
def run_varlen(fa, case, causal, rows=None):
    q, k, v = (dev(case[n], case["dtype"]) for n in ("q", "k", "v"))
    cu = torch.from_numpy(case["cu_seqlens"]).cuda()
    o, lse = fa.fa_fwd_varlen(q, k, v, cu, case["max_seqlen"], causal=causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.varlen(case["q"], case["k"], case["v"], case["cu_seqlens"], causal=causal,
                                   rows=rows)
    og = host(o).transpose(1, 0, 2)  # [Hq, T, d]
    lg = lse.cpu().numpy().astype(np.float64)
    if rows is not None:
        og = og.reshape(-1, og.shape[-1])[rows]
        lg = lg.reshape(-1)[rows]
    return og, lg, o_ref, lse_ref


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("d", [64, 128])
def test_varlen_parity(gpu, d, causal, dtype):
    lens = [1, 130, 0, 64, 257, 7, 128]
    case = inputs.varlen_case(200 + d, lens, 4, 2, d, dtype=dtype)
    og, lg, o_ref, lse_ref = run_varlen(gpu, case, causal)
    check(og, lg, o_ref, lse_ref, dtype, f"varlen d={d} causal={causal}")


def test_varlen_workload_sampled(gpu):
    case = inputs.workload(4)
    T, H = case["total"], case["hq"]
    rng = np.random.default_rng(4)
    rows = set(rng.integers(0, H * T, size=384).tolist())
    cu = case["cu_seqlens"]
    for s in range(len(cu) - 1):  # first and last token of every sequence
        for t in (cu[s], cu[s + 1] - 1):
            rows.add(int(rng.integers(0, H)) * T + int(t))
    rows = np.array(sorted(rows), dtype=np.int64)
    og, lg, o_ref, lse_ref = run_varlen(gpu, case, True, rows=rows)
    check(og, lg, o_ref, lse_ref, "bf16", "varlen workload sampled rows")


def test_varlen_matches_dense_per_sequence(gpu):
    lens = [100, 300, 5]
    case = inputs.varlen_case(9, lens, 2, 2, 128, dtype="bf16")
    q, k, v = (dev(case[n], "bf16") for n in ("q", "k", "v"))
    cu = torch.from_numpy(case["cu_seqlens"]).cuda()
    o, lse = gpu.fa_fwd_varlen(q, k, v, cu, max(lens), causal=True)
    for s, L in enumerate(lens):
        a, b = case["cu_seqlens"][s], case["cu_seqlens"][s + 1]
        od, ld = gpu.fa_fwd(q[None, a:b], k[None, a:b], v[None, a:b], causal=True)
        # identical tiling of identical data: identical bits
        assert torch.equal(o[a:b], od[0])
        assert torch.equal(lse[:, a:b], ld[0])


# --------------------------------------------------------------------------
# paged decode
# --------------------------------------------------------------------------
def decode_gpu(fa, case, num_splits=0, k_pool=None, v_pool=None, table=None):
    q = dev(case["q"], "bf16")
    kp = dev(case["k_pool"], "bf16") if k_pool is None else k_pool
    vp = dev(case["v_pool"], "bf16") if v_pool is None else v_pool
    bt = torch.from_numpy(case["block_table"]).cuda() if table is None else table
    sl = torch.from_numpy(case["seq_lens"]).cuda()
    maxlen = int(case["seq_lens"].max(initial=0))
    o, lse = fa.fa_decode_paged(q, kp, vp, bt, sl, maxlen, num_splits=num_splits)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("group", [1, 2, 3, 4, 8, 16])
@pytest.mark.parametrize("num_splits", [0, 1, 3, 50])
def test_decode_parity(gpu, group, num_splits):
    # lengths: one token, a full block, a block and one token, a zero-length
    # sequence in the middle, tails of every residue class mod 16
    lens = [1, 16, 17, 100, 0, 333, 48, 1000]
    hkv = 2
    case = inputs.paged_case(300 + group, lens, hkv * group, hkv, 128, pad_blocks=2)
    o, lse = decode_gpu(gpu, case, num_splits=num_splits)
    o_ref, lse_ref = oracle.decode_paged(case["q"], case["k_pool"], case["v_pool"], case["block_table"],
                                         case["seq_lens"])
    check(host(o), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref, "bf16",
          f"decode group={group} splits={num_splits}")


@pytest.mark.parametrize("d", [64, 256])
@pytest.mark.parametrize("group", [1, 4, 16])
@pytest.mark.parametrize("num_splits", [0, 1, 7])
def test_decode_head_dims(gpu, d, group, num_splits):
    lens = [1, 16, 17, 100, 0, 333, 48, 1000]
    hkv = 2
    case = inputs.paged_case(340 + group + d, lens, hkv * group, hkv, d, pad_blocks=2)
    o, lse = decode_gpu(gpu, case, num_splits=num_splits)
    o_ref, lse_ref = oracle.decode_paged(case["q"], case["k_pool"], case["v_pool"], case["block_table"],
                                         case["seq_lens"])
    check(host(o), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref, "bf16",
          f"decode d={d} group={group} splits={num_splits}")


@pytest.mark.parametrize("d", [64, 256])
def test_decode_head_dims_paged_equals_contiguous_bitwise(gpu, d):
    lens = [700, 17, 1024, 33]
    case = inputs.paged_case(350 + d, lens, 8, 2, d)
    o1, l1 = decode_gpu(gpu, case, num_splits=0)
    bt = case["block_table"]
    order = np.concatenate([bt[b, :(L + 15) // 16] for b, L in enumerate(lens)]).astype(np.int64)
    idx = torch.from_numpy(order).cuda()
    kp = dev(case["k_pool"], "bf16")[idx].contiguous()
    vp = dev(case["v_pool"], "bf16")[idx].contiguous()
    table = np.full_like(bt, -1)
    pos = 0
    for b, L in enumerate(lens):
        nb = (L + 15) // 16
        table[b, :nb] = np.arange(pos, pos + nb)
        pos += nb
    o2, l2 = decode_gpu(gpu, case, num_splits=0, k_pool=kp, v_pool=vp, table=torch.from_numpy(table).cuda())
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def decode_fp8_gpu(fa, case, num_splits=0, k_pool=None, v_pool=None, table=None):
    q = dev(case["q"], "bf16")
    kp = torch.from_numpy(case["k_pool"]).cuda() if k_pool is None else k_pool
    vp = torch.from_numpy(case["v_pool"]).cuda() if v_pool is None else v_pool
    bt = torch.from_numpy(case["block_table"]).cuda() if table is None else table
    sl = torch.from_numpy(case["seq_lens"]).cuda()
    maxlen = int(case["seq_lens"].max(initial=0))
    o, lse = fa.fa_decode_paged_fp8(q, kp, vp, bt, sl, maxlen, case["descale"], num_splits=num_splits)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("group", [1, 4, 16])
@pytest.mark.parametrize("num_splits", [0, 3])
def test_decode_fp8_kv_parity(gpu, d, group, num_splits):
    """FP8 KV cache: the codes are widened exactly, so the bf16 decode
    tolerance applies to the attention of q over descale * value(code)."""
    lens = [1, 16, 17, 100, 0, 333, 48, 1000]
    hkv = 2
    case = inputs.paged_fp8_case(360 + group + d, lens, hkv * group, hkv, d, pad_blocks=2)
    o, lse = decode_fp8_gpu(gpu, case, num_splits=num_splits)
    o_ref, lse_ref = oracle.decode_paged_fp8(case["q"], case["k_pool"], case["v_pool"], case["block_table"],
                                             case["seq_lens"], case["descale"])
    check(host(o), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref, "bf16",
          f"fp8 kv decode d={d} group={group} splits={num_splits}")


def test_decode_fp8_kv_paged_equals_contiguous_bitwise(gpu):
    lens = [5000, 17, 1024, 333]
    case = inputs.paged_fp8_case(370, lens, 32, 8, 128)
    o1, l1 = decode_fp8_gpu(gpu, case)
    bt = case["block_table"]
    order = np.concatenate([bt[b, :(L + 15) // 16] for b, L in enumerate(lens)]).astype(np.int64)
    idx = torch.from_numpy(order).cuda()
    kp = torch.from_numpy(case["k_pool"]).cuda()[idx].contiguous()
    vp = torch.from_numpy(case["v_pool"]).cuda()[idx].contiguous()
    table = np.full_like(bt, -1)
    pos = 0
    for b, L in enumerate(lens):
        nb = (L + 15) // 16
        table[b, :nb] = np.arange(pos, pos + nb)
        pos += nb
    o2, l2 = decode_fp8_gpu(gpu, case, k_pool=kp, v_pool=vp, table=torch.from_numpy(table).cuda())
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_fp8_kv_matches_bf16_decode_of_widened_pools(gpu):
    """The FP8 instance equals the bf16 kernel run on the widened pools with
    the descales folded into the pool values (both sides exact in bf16 when
    the descale is a power of two)."""
    lens = [300, 17, 64]
    case = inputs.paged_fp8_case(371, lens, 8, 2, 128)
    case["descale"] = (0.25, 0.5)
    o8, l8 = decode_fp8_gpu(gpu, case)
    kw = torch.from_numpy(case["k_pool"]).cuda().view(torch.float8_e4m3fn).float() * 0.25
    vw = torch.from_numpy(case["v_pool"]).cuda().view(torch.float8_e4m3fn).float() * 0.5
    o16, l16 = decode_gpu(gpu, case, k_pool=kw.to(torch.bfloat16), v_pool=vw.to(torch.bfloat16))
    assert (o8.float() - o16.float()).abs().max().item() <= 2e-2
    assert (l8 - l16).abs().max().item() <= 1e-5


@pytest.mark.parametrize("lens", [[0, 0, 5], [5, 0, 0], [0], [16, 0, 16, 0, 1]])
def test_decode_empty_sequences(gpu, lens):
    case = inputs.paged_case(330 + len(lens), lens, 8, 2, 128, pad_blocks=1)
    for ns in (0, 2, 9):
        o, lse = decode_gpu(gpu, case, num_splits=ns)
        o_ref, lse_ref = oracle.decode_paged(case["q"], case["k_pool"], case["v_pool"], case["block_table"],
                                             case["seq_lens"])
        check(host(o), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref, "bf16",
              f"decode lens={lens} splits={ns}")


def test_decode_paged_equals_contiguous_bitwise(gpu):
    lens = [5000, 17, 1024, 333, 4097]
    case = inputs.paged_case(310, lens, 32, 8, 128)
    o1, l1 = decode_gpu(gpu, case, num_splits=0)
    # the same logical keys, blocks laid out in table order, identity table
    bt = case["block_table"]
    order = np.concatenate([bt[b, :(L + 15) // 16] for b, L in enumerate(lens)]).astype(np.int64)
    idx = torch.from_numpy(order).cuda()
    kp = dev(case["k_pool"], "bf16").index_select(0, idx)
    vp = dev(case["v_pool"], "bf16").index_select(0, idx)
    ident = np.full_like(bt, -1)
    pos = 0
    for b, L in enumerate(lens):
        nb = (L + 15) // 16
        ident[b, :nb] = np.arange(pos, pos + nb)
        pos += nb
    o2, l2 = decode_gpu(gpu, case, num_splits=0, k_pool=kp, v_pool=vp,
                        table=torch.from_numpy(ident).cuda())
    assert torch.equal(o1, o2)
    assert torch.equal(l1, l2)


def test_decode_token_major_pool(gpu):
    lens = [40, 300]
    case = inputs.paged_case(320, lens, 8, 2, 128)
    o1, l1 = decode_gpu(gpu, case)
    kt = dev(np.ascontiguousarray(case["k_pool"].transpose(0, 2, 1, 3)), "bf16").transpose(1, 2)
    vt = dev(np.ascontiguousarray(case["v_pool"].transpose(0, 2, 1, 3)), "bf16").transpose(1, 2)
    o2, l2 = decode_gpu(gpu, case, k_pool=kt, v_pool=vt)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_workload_sampled(gpu):
    case = inputs.workload(5)
    o, lse = decode_gpu(gpu, case)
    B, H = case["q"].shape[:2]
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([rng.integers(0, B * H, size=96),
                                     [int(np.argmax(case["seq_lens"])) * H, int(np.argmin(case["seq_lens"])) * H]]))
    o_ref, lse_ref = oracle.decode_paged(case["q"], case["k_pool"], case["v_pool"], case["block_table"],
                                         case["seq_lens"], rows=rows)
    og = host(o).reshape(B * H, -1)[rows]
    lg = lse.cpu().numpy().astype(np.float64).reshape(-1)[rows]
    check(og, lg, o_ref, lse_ref, "bf16", "decode workload sampled")


# --------------------------------------------------------------------------
# chunked prefill over the paged pool
# --------------------------------------------------------------------------
def paged_prefill_gpu(fa, case, causal=True, k_pool=None, v_pool=None, table=None):
    q = dev(case["q"], "bf16")
    kp = dev(case["k_pool"], "bf16") if k_pool is None else k_pool
    vp = dev(case["v_pool"], "bf16") if v_pool is None else v_pool
    bt = torch.from_numpy(case["block_table"]).cuda() if table is None else table
    cu = torch.from_numpy(case["cu_seqlens_q"]).cuda()
    sl = torch.from_numpy(case["seq_lens"]).cuda()
    o, lse = fa.fa_fwd_paged(q, kp, vp, bt, cu, sl, case["max_seqlen_q"], int(case["seq_lens"].max(initial=0)),
                             causal=causal)
    torch.cuda.synchronize()
    return o, lse


def run_paged_prefill(fa, case, causal, rows=None):
    o, lse = paged_prefill_gpu(fa, case, causal)
    o_ref, lse_ref = oracle.paged_prefill(case["q"], case["k_pool"], case["v_pool"], case["block_table"],
                                          case["cu_seqlens_q"], case["seq_lens"], causal=causal, rows=rows)
    og = host(o).transpose(1, 0, 2)  # [Hq, Tq, d]
    lg = lse.cpu().numpy().astype(np.float64)
    if rows is not None:
        og = og.reshape(-1, og.shape[-1])[rows]
        lg = lg.reshape(-1)[rows]
    return og, lg, o_ref, lse_ref


# chunk of one query, chunk = whole context, chunk longer than its keys,
# a sequence without keys, one without queries, several key tiles with
# ragged tails and several query tiles
PAGED_Q = [1, 130, 7, 5, 64, 300, 6, 257, 0]
PAGED_K = [1, 333, 7, 0, 1000, 300, 4, 600, 40]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("group", [1, 4])
def test_paged_prefill_parity(gpu, group, d, causal):
    case = inputs.paged_prefill_case(400 + 10 * group + d, PAGED_Q, PAGED_K, 2 * group, 2, d, pad_blocks=1)
    og, lg, o_ref, lse_ref = run_paged_prefill(gpu, case, causal)
    check(og, lg, o_ref, lse_ref, "bf16", f"paged prefill group={group} d={d} causal={causal}")


@pytest.mark.parametrize("d", [128, 256])
def test_paged_prefill_whole_context_is_varlen_bitwise(gpu, d):
    # a chunk that is the whole context reads exactly the keys the packed
    # kernel reads, in the same tiles: identical bits
    lens = [300, 64, 17, 700]
    case = inputs.paged_prefill_case(410 + d, lens, lens, 8, 2, d)
    o1, l1 = paged_prefill_gpu(gpu, case, causal=True)
    bs = case["block_size"]
    kp, vp = dev(case["k_pool"], "bf16"), dev(case["v_pool"], "bf16")
    ks, vs = [], []
    for s, L in enumerate(lens):
        t = torch.arange(L, device="cuda")
        phys = torch.from_numpy(case["block_table"][s]).cuda().long()[t // bs]
        ks.append(kp[phys, :, t % bs])
        vs.append(vp[phys, :, t % bs])
    k, v = torch.cat(ks).contiguous(), torch.cat(vs).contiguous()
    cu = torch.from_numpy(case["cu_seqlens_q"]).cuda()
    o2, l2 = gpu.fa_fwd_varlen(dev(case["q"], "bf16"), k, v, cu, max(lens), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(l1, l2)


@pytest.mark.parametrize("d", [128, 256])
def test_paged_prefill_pool_order_bitwise(gpu, d):
    q_lens, k_lens = [512, 33, 200], [2000, 33, 1500]
    case = inputs.paged_prefill_case(420 + d, q_lens, k_lens, 16, 4, d)
    o1, l1 = paged_prefill_gpu(gpu, case)
    bt = case["block_table"]
    order = np.concatenate([bt[b, :(L + 15) // 16] for b, L in enumerate(k_lens)]).astype(np.int64)
    idx = torch.from_numpy(order).cuda()
    kp = dev(case["k_pool"], "bf16").index_select(0, idx)
    vp = dev(case["v_pool"], "bf16").index_select(0, idx)
    ident = np.full_like(bt, -1)
    pos = 0
    for b, L in enumerate(k_lens):
        nb = (L + 15) // 16
        ident[b, :nb] = np.arange(pos, pos + nb)
        pos += nb
    o2, l2 = paged_prefill_gpu(gpu, case, k_pool=kp, v_pool=vp, table=torch.from_numpy(ident).cuda())
    assert torch.equal(o1, o2)
    assert torch.equal(l1, l2)
    # token-major pool [blocks, 16, Hkv, d] viewed with the same logical shape
    kt = dev(np.ascontiguousarray(case["k_pool"].transpose(0, 2, 1, 3)), "bf16").transpose(1, 2)
    vt = dev(np.ascontiguousarray(case["v_pool"].transpose(0, 2, 1, 3)), "bf16").transpose(1, 2)
    o3, l3 = paged_prefill_gpu(gpu, case, k_pool=kt, v_pool=vt)
    assert torch.equal(o1, o3)
    assert torch.equal(l1, l3)


def paged_prefill_fp8_gpu(fa, case, causal=True, k_pool=None, v_pool=None, table=None):
    q = torch.from_numpy(case["q"]).cuda()
    kp = torch.from_numpy(case["k_pool"]).cuda() if k_pool is None else k_pool
    vp = torch.from_numpy(case["v_pool"]).cuda() if v_pool is None else v_pool
    bt = torch.from_numpy(case["block_table"]).cuda() if table is None else table
    cu = torch.from_numpy(case["cu_seqlens_q"]).cuda()
    sl = torch.from_numpy(case["seq_lens"]).cuda()
    o, lse = fa.fa_fwd_paged_fp8(q, kp, vp, bt, cu, sl, case["max_seqlen_q"], int(case["seq_lens"].max(initial=0)),
                                 case["descale"], causal=causal)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("group", [1, 4])
def test_paged_prefill_fp8_parity(gpu, group, causal):
    case = inputs.paged_prefill_fp8_case(620 + group, PAGED_Q, PAGED_K, 2 * group, 2, 128, pad_blocks=1)
    o, lse = paged_prefill_fp8_gpu(gpu, case, causal)
    o_ref, lse_ref = oracle.paged_prefill_fp8(case["q"], case["k_pool"], case["v_pool"], case["block_table"],
                                              case["cu_seqlens_q"], case["seq_lens"], case["descale"], causal=causal)
    check_fp8(host(o).transpose(1, 0, 2), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref,
              f"fp8 paged prefill group={group} causal={causal}")


def test_paged_prefill_fp8_pool_order_bitwise(gpu):
    q_lens, k_lens = [512, 33, 200], [2000, 33, 1500]
    case = inputs.paged_prefill_fp8_case(630, q_lens, k_lens, 16, 4, 128)
    o1, l1 = paged_prefill_fp8_gpu(gpu, case)
    bt = case["block_table"]
    order = np.concatenate([bt[b, :(L + 15) // 16] for b, L in enumerate(k_lens)]).astype(np.int64)
    idx = torch.from_numpy(order).cuda()
    kp = torch.from_numpy(case["k_pool"]).cuda().index_select(0, idx)
    vp = torch.from_numpy(case["v_pool"]).cuda().index_select(0, idx)
    ident = np.full_like(bt, -1)
    pos = 0
    for b, L in enumerate(k_lens):
        nb = (L + 15) // 16
        ident[b, :nb] = np.arange(pos, pos + nb)
        pos += nb
    o2, l2 = paged_prefill_fp8_gpu(gpu, case, k_pool=kp, v_pool=vp, table=torch.from_numpy(ident).cuda())
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_paged_prefill_fp8_whole_context_is_varlen_fp8_bitwise(gpu):
    lens = [300, 64, 17, 700]
    case = inputs.paged_prefill_fp8_case(640, lens, lens, 8, 2, 128)
    o1, l1 = paged_prefill_fp8_gpu(gpu, case)
    kp, vp = torch.from_numpy(case["k_pool"]).cuda(), torch.from_numpy(case["v_pool"]).cuda()
    ks, vs = [], []
    for s_, L in enumerate(lens):
        t = torch.arange(L, device="cuda")
        phys = torch.from_numpy(case["block_table"][s_]).cuda().long()[t // 16]
        ks.append(kp[phys, :, t % 16])
        vs.append(vp[phys, :, t % 16])
    k, v = torch.cat(ks).contiguous(), torch.cat(vs).contiguous()
    cu = torch.from_numpy(case["cu_seqlens_q"]).cuda()
    o2, l2 = gpu.fa_fwd_varlen_fp8(torch.from_numpy(case["q"]).cuda(), k, v, cu, max(lens), case["descale"],
                                   causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_paged_prefill_workload_sampled(gpu):
    case = inputs.workload(6)
    T, H = case["total_q"], case["hq"]
    rng = np.random.default_rng(6)
    rows = set(rng.integers(0, H * T, size=256).tolist())
    cu = case["cu_seqlens_q"]
    for s in range(len(cu) - 1):  # first and last query of every chunk
        for t in (cu[s], cu[s + 1] - 1):
            rows.add(int(rng.integers(0, H)) * T + int(t))
    rows = np.array(sorted(rows), dtype=np.int64)
    og, lg, o_ref, lse_ref = run_paged_prefill(gpu, case, True, rows=rows)
    check(og, lg, o_ref, lse_ref, "bf16", "paged prefill workload sampled rows")


# --------------------------------------------------------------------------
# FP8 E4M3 prefill
# --------------------------------------------------------------------------
# Tolerance of the FP8 path against the fp64 oracle on the same descaled
# inputs.  Scores and LSE are computed in fp32 from exact FP8 products: LSE
# keeps LSE_TOL.  O differs by the E4M3 rounding of the weights fed to P.V
# (relative error up to 2^-4 per weight; O is normalised by the sum of the
# rounded weights, so it stays a convex combination of V rows and the error
# scales with the spread of the V rows that carry weight: largest for rows
# with two or three comparable keys, about 2^-5 * |v_i - v_j|) plus bf16
# output rounding (2^-9 relative).  With unit-variance V: max |dO| <= 0.08,
# mean |dO| <= 0.006.
FP8_TOL = (0.08, 0.006)


def run_fp8(fa, case, causal, rows=None):
    q, k, v = (torch.from_numpy(case[n]).cuda() for n in ("q", "k", "v"))
    o, lse = fa.fa_fwd_fp8(q, k, v, case["descale"], causal=causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.fp8_dense(case["q"], case["k"], case["v"], case["descale"], causal=causal, rows=rows)
    og = host(o).transpose(0, 2, 1, 3)
    lg = lse.cpu().numpy().astype(np.float64)
    if rows is not None:
        og = og.reshape(-1, og.shape[-1])[rows]
        lg = lg.reshape(-1)[rows]
    return og, lg, o_ref, lse_ref


def check_fp8(og, lg, o_ref, lse_ref, what):
    tmax, tmean = FP8_TOL
    err = np.abs(og - o_ref)
    assert np.isfinite(og).all(), f"{what}: non-finite output"
    assert err.max() <= tmax, f"{what}: max |dO| = {err.max():.3e} > {tmax}"
    assert err.mean() <= tmean, f"{what}: mean |dO| = {err.mean():.3e} > {tmean}"
    fin = np.isfinite(lse_ref)
    np.testing.assert_array_equal(np.isfinite(lg), fin, err_msg=f"{what}: LSE finiteness")
    np.testing.assert_array_equal(lg[~fin], lse_ref[~fin])
    if fin.any():
        e = np.abs(lg[fin] - lse_ref[fin]).max()
        assert e <= LSE_TOL, f"{what}: max |dLSE| = {e:.3e}"


@pytest.mark.parametrize("causal", [True, False])
def test_fp8_varlen_parity(gpu, causal):
    lens = [1, 130, 0, 64, 257, 7, 128, 300]
    case = inputs.fp8_varlen_case(610, lens, 4, 2, 128)
    q, k, v = (torch.from_numpy(case[n]).cuda() for n in ("q", "k", "v"))
    cu = torch.from_numpy(case["cu_seqlens"]).cuda()
    o, lse = gpu.fa_fwd_varlen_fp8(q, k, v, cu, case["max_seqlen"], case["descale"], causal=causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.fp8_varlen(case["q"], case["k"], case["v"], case["cu_seqlens"], case["descale"],
                                       causal=causal)
    check_fp8(host(o).transpose(1, 0, 2), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref,
              f"fp8 varlen causal={causal}")


def test_fp8_varlen_single_sequence_equals_dense_bitwise(gpu):
    N = 700
    case = inputs.fp8_case(611, 1, N, N, 3, 3, 128)
    q, k, v = (torch.from_numpy(case[n]).cuda() for n in ("q", "k", "v"))
    od, ld = gpu.fa_fwd_fp8(q, k, v, case["descale"], causal=True)
    cu = torch.tensor([0, N], dtype=torch.int32).cuda()
    ov, lv = gpu.fa_fwd_varlen_fp8(q[0], k[0], v[0], cu, N, case["descale"], causal=True)
    torch.cuda.synchronize()
    assert torch.equal(od[0], ov)
    assert torch.equal(ld[0], lv)


FP8_SHAPES = [
    # B, Nq, Nk, Hq, Hkv
    (1, 1, 1, 1, 1),
    (1, 64, 64, 1, 1),
    (1, 300, 300, 2, 2),
    (2, 513, 513, 4, 2),
    (2, 100, 260, 2, 1),   # more keys than queries (end-aligned causal)
    (1, 300, 77, 2, 2),    # more queries than keys: early causal rows see no key
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", FP8_SHAPES)
def test_fp8_parity(gpu, shape, causal):
    B, Nq, Nk, Hq, Hkv = shape
    case = inputs.fp8_case(810 + Nq + Nk, B, Nq, Nk, Hq, Hkv, 128)
    og, lg, o_ref, lse_ref = run_fp8(gpu, case, causal)
    check_fp8(og.reshape(-1, 128), lg.reshape(-1), o_ref.reshape(-1, 128), lse_ref.reshape(-1),
              f"fp8 {shape} causal={causal}")


def test_fp8_single_key_returns_that_value(gpu):
    # one visible key: its weight is 1 (exact in E4M3), so O = v_descale * v
    # up to the bf16 rounding of the output
    case = inputs.fp8_case(830, 2, 40, 40, 2, 2, 128)
    og, lg, o_ref, lse_ref = run_fp8(gpu, case, True)
    v = inputs.e4m3_to_f32(case["v"]).astype(np.float64) * float(case["descale"][2])
    first = og[:, :, 0, :]          # [B, Hq, d]: row 0 sees key 0 only
    np.testing.assert_allclose(first, v[:, 0, :, :], rtol=2.0 ** -8, atol=0)


def test_fp8_empty_keys(gpu):
    case = inputs.fp8_case(831, 1, 20, 1, 2, 2, 128)
    q = torch.from_numpy(case["q"]).cuda()
    kv = torch.empty((1, 0, 2, 128), dtype=torch.uint8, device="cuda")
    o, lse = gpu.fa_fwd_fp8(q, kv, kv, case["descale"], causal=False)
    torch.cuda.synchronize()
    assert torch.all(o == 0)
    assert torch.all(torch.isneginf(lse))


def test_fp8_workload_sampled(gpu):
    case = inputs.workload(7)
    B, N, H = case["batch"], case["nq"], case["hq"]
    rng = np.random.default_rng(7)
    rows = set(rng.integers(0, B * H * N, size=384).tolist())
    for b in range(B):  # tile edges and the last row of some heads
        for i in (0, 1, 255, 256, 1023, N - 1):
            rows.add((b * H + int(rng.integers(0, H))) * N + i)
    rows = np.array(sorted(rows), dtype=np.int64)
    og, lg, o_ref, lse_ref = run_fp8(gpu, case, True, rows=rows)
    check_fp8(og, lg, o_ref, lse_ref, "fp8 workload sampled rows")
