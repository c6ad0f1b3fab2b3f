"""GPU parity of fa_merge_states against the fp64 oracle.

* seeded partial results (``inputs.merge_case``) over head dims 64/128/256,
  bf16 and fp32, 1..8 parts, ragged row counts, with and without shards
  that saw no key (lse -inf, output NaN);
* ring attention over key shards on one GPU (bf16, and fp32 at the fp32 bound): each query chunk's results
  against the key shards before it (plain) and its own shard (causal), from
  fa_fwd, merged, against the oracle's causal attention over the whole
  sequence;
* flash-decoding split across devices: paged decode over two halves of
  every block table, merged, against the oracle's decode over all keys;
* the bench-size merge (8 shard results of B=1, N=8192, H=32, d=128) on
  sampled rows.

Tolerances: bf16 output within 2^-8 of |o| plus 1e-6 (one bf16 rounding of
an fp32 merge), fp32 output within 1e-5, lse within 2e-5; composed paths
(ring, split decode) at the bf16 attention tolerance of ``test_gpu_parity``.
"""
import numpy as np
import pytest

import oracle
from exact_io_aware_tile_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

BF16 = (2e-2, 2e-3)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_io_aware_tile_amd import fa
    fa.lib()
    return fa


def bdev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def odev(a, dtype):
    return bdev(a) if dtype == "bf16" else torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def oracle_merge(c, rows=None):
    """Oracle on the case's layout: o_parts [P,B,S,H,d] -> rows ordered as lse [P,B,H,S]."""
    o = c["o_parts"].transpose(0, 1, 3, 2, 4)
    lse = c["lse_parts"]
    if rows is not None:
        o, lse = o[:, :, :, rows], lse[:, :, :, rows]
    return oracle.merge_states(o, lse)


def check_merge(og, lg, o_ref, l_ref, dtype, what):
    og = og.transpose(0, 2, 1, 3)  # [B,S,H,d] -> [B,H,S,d]
    fin = np.isfinite(l_ref)
    np.testing.assert_array_equal(np.isfinite(lg), fin, err_msg=what)
    assert (og[~fin] == 0).all(), what
    assert np.isfinite(og).all(), what
    err = np.abs(og - o_ref)
    bound = (2.0 ** -8) * np.abs(o_ref) + 1e-6 if dtype == "bf16" else 1e-5
    assert (err <= bound).all(), f"{what}: worst |dO| {err.max():.3e}"
    if fin.any():
        assert np.abs(lg[fin] - l_ref[fin]).max() <= 2e-5, f"{what}: lse"


@pytest.mark.parametrize("P,B,S,H,d,dtype,empty", [
    (1, 1, 9, 2, 128, "bf16", 0.0),
    (2, 2, 7, 3, 64, "bf16", 0.3),
    (3, 1, 130, 4, 128, "bf16", 0.2),
    (8, 2, 33, 5, 256, "bf16", 0.5),
    (4, 1, 17, 3, 64, "f32", 0.25),
    (5, 2, 65, 2, 128, "f32", 0.0),
    (2, 1, 40, 8, 256, "f32", 0.6),
])
def test_merge_parity(gpu, P, B, S, H, d, dtype, empty):
    c = inputs.merge_case(8000 + P * 10 + d, P, B, S, H, d, dtype=dtype, empty_frac=empty)
    o, lse = gpu.fa_merge_states(odev(c["o_parts"], dtype), torch.from_numpy(c["lse_parts"]).cuda())
    torch.cuda.synchronize()
    o_ref, l_ref = oracle_merge(c)
    check_merge(host(o), lse.cpu().numpy().astype(np.float64), o_ref, l_ref, dtype,
                f"merge P={P} B={B} S={S} H={H} d={d} {dtype} empty={empty}")


def test_merge_all_parts_empty(gpu):
    c = inputs.merge_case(8100, 3, 1, 6, 2, 128, empty_frac=0.0)
    c["lse_parts"][:] = -np.inf
    o, lse = gpu.fa_merge_states(bdev(c["o_parts"]), torch.from_numpy(c["lse_parts"]).cuda())
    torch.cuda.synchronize()
    assert (host(o) == 0).all()
    assert np.isneginf(lse.cpu().numpy()).all()


def test_merge_without_lse_and_into_out(gpu):
    c = inputs.merge_case(8101, 3, 1, 20, 4, 128, empty_frac=0.1)
    out = torch.full((1, 20, 4, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    o, lse = gpu.fa_merge_states(bdev(c["o_parts"]), torch.from_numpy(c["lse_parts"]).cuda(), out=out,
                                 return_lse=False)
    torch.cuda.synchronize()
    assert lse is None and o.data_ptr() == out.data_ptr()
    o_ref, l_ref = oracle_merge(c)
    check_merge(host(o), l_ref, o_ref, l_ref, "bf16", "merge without lse")


@pytest.mark.parametrize("N,chunks,H,Hkv,d", [(1024, 4, 4, 4, 128), (768, 3, 8, 2, 64), (600, 3, 4, 2, 256)])
def test_ring_attention_over_key_shards(gpu, N, chunks, H, Hkv, d):
    case = inputs.dense_case(8200 + d, 1, N, N, H, Hkv, d, dtype="bf16")
    q, k, v = (bdev(case[n]) for n in ("q", "k", "v"))
    o_ref, l_ref = oracle.dense(case["q"], case["k"], case["v"], causal=True)
    cl = N // chunks
    for c in range(chunks):
        qs = slice(c * cl, (c + 1) * cl)
        os_, ls_ = [], []
        for s in range(c + 1):
            ks = slice(s * cl, (s + 1) * cl)
            o_p, l_p = gpu.fa_fwd(q[:, qs].contiguous(), k[:, ks].contiguous(), v[:, ks].contiguous(),
                                  causal=(s == c))
            os_.append(o_p)
            ls_.append(l_p)
        o, lse = gpu.fa_merge_states(torch.stack(os_).contiguous(), torch.stack(ls_).contiguous())
        torch.cuda.synchronize()
        og = host(o).transpose(0, 2, 1, 3)
        err = np.abs(og - o_ref[:, :, qs])
        what = f"ring N={N} chunk {c}/{chunks} H={H}/{Hkv} d={d}"
        assert err.max() <= BF16[0] and err.mean() <= BF16[1], f"{what}: {err.max():.3e}"
        assert np.abs(lse.cpu().numpy() - l_ref[:, :, qs]).max() <= 1e-3, what


@pytest.mark.parametrize("kv8", [False, True])
def test_decode_split_over_two_shards(gpu, kv8):
    lens = np.array([0, 1, 15, 16, 17, 300, 1024, 2047, 3001, 5000])
    H, Hkv, d = 8, 2, 128
    mk = inputs.paged_fp8_case if kv8 else inputs.paged_case
    case = mk(8300 + kv8, lens, H, Hkv, d, pad_blocks=1)
    conv = (lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()) if kv8 else bdev
    kp, vp = conv(case["k_pool"]), conv(case["v_pool"])
    bt = case["block_table"]
    nb = bt.shape[1]
    half = (nb + 1) // 2
    os_, ls_ = [], []
    for lo, hi in ((0, half), (half, nb)):
        sl = np.clip(lens - 16 * lo, 0, 16 * (hi - lo)).astype(np.int32)
        bts = np.ascontiguousarray(bt[:, lo:hi]) if hi > lo else np.zeros((len(lens), 1), np.int32)
        args = (bdev(case["q"]), kp, vp, torch.from_numpy(bts).cuda(), torch.from_numpy(sl).cuda(),
                int(max(16 * (hi - lo), 0)))
        if kv8:
            o_p, l_p = gpu.fa_decode_paged_fp8(*args, case["descale"])
        else:
            o_p, l_p = gpu.fa_decode_paged(*args)
        os_.append(o_p.reshape(len(lens), 1, H, d))
        ls_.append(l_p.reshape(len(lens), H, 1))
    o, lse = gpu.fa_merge_states(torch.stack(os_).contiguous(), torch.stack(ls_).contiguous())
    torch.cuda.synchronize()
    if kv8:
        o_ref, l_ref = oracle.decode_paged_fp8(case["q"], case["k_pool"], case["v_pool"], bt, case["seq_lens"],
                                               case["descale"])
    else:
        o_ref, l_ref = oracle.decode_paged(case["q"], case["k_pool"], case["v_pool"], bt, case["seq_lens"])
    og = host(o).reshape(len(lens), H, d)
    lg = lse.cpu().numpy().reshape(len(lens), H).astype(np.float64)
    np.testing.assert_array_equal(np.isfinite(lg), np.isfinite(l_ref))
    err = np.abs(og - o_ref)
    assert err.max() <= BF16[0] and err.mean() <= BF16[1], f"split decode kv8={kv8}: {err.max():.3e}"
    fin = np.isfinite(l_ref)
    assert np.abs(lg[fin] - l_ref[fin]).max() <= 1e-3


def test_merge_bench_size_sampled(gpu):
    c = inputs.workload(12)
    o, lse = gpu.fa_merge_states(bdev(c["o_parts"]), torch.from_numpy(c["lse_parts"]).cuda())
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(12).choice(c["seqlen"], 512, replace=False))
    o_ref, l_ref = oracle_merge(c, rows)
    og = o[:, torch.from_numpy(rows).cuda()]
    check_merge(host(og), lse[:, :, torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64), o_ref,
                l_ref, "bf16", "merge workload 12 sampled")


@pytest.mark.parametrize("d", [64, 128])
def test_ring_attention_fp32(gpu, d):
    """fp32 ring over two key shards: the merged result keeps the fp32 bound."""
    N, chunks, H = 512, 2, 2
    case = inputs.dense_case(8400 + d, 1, N, N, H, H, d, dtype="f32")
    q, k, v = (torch.from_numpy(case[n]).cuda() for n in ("q", "k", "v"))
    o_ref, l_ref = oracle.dense(case["q"], case["k"], case["v"], causal=True)
    cl = N // chunks
    for c in range(chunks):
        qs = slice(c * cl, (c + 1) * cl)
        parts = [gpu.fa_fwd(q[:, qs].contiguous(), k[:, s * cl:(s + 1) * cl].contiguous(),
                            v[:, s * cl:(s + 1) * cl].contiguous(), causal=(s == c)) for s in range(c + 1)]
        o, lse = gpu.fa_merge_states(torch.stack([p[0] for p in parts]).contiguous(),
                                     torch.stack([p[1] for p in parts]).contiguous())
        torch.cuda.synchronize()
        err = np.abs(o.cpu().numpy().astype(np.float64).transpose(0, 2, 1, 3) - o_ref[:, :, qs])
        assert err.max() <= 1e-5, f"fp32 ring d={d} chunk {c}: {err.max():.3e}"
        assert np.abs(lse.cpu().numpy() - l_ref[:, :, qs]).max() <= 1e-5
