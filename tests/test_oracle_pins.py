"""Pins of the fp64 CPU oracle against facts that do not come from the oracle.

Each pin targets a different plausible mistake (a dropped term, a wrong sign,
a wrong index, a transposed operand, a wrong mask direction or group map):

 1. worked example of the merge rule ("FlashAttention", tachyon.techntrek.in,
    "For engineers / Show the maths"): l after tile 1, tile 2's own l~, and
    the merged l, read back out of the oracle's O and LSE;
 2. rows are normalised: V = ones gives O = 1; V = identity gives weights that
    sum to 1;
 3. closed form q = 0: O is the mean of the visible values, LSE = ln |visible|;
 4. a single visible key: O = v_0, LSE = s_0;
 5. causal direction: row 0 sees key 0 only; the last row sees everything;
 6. prefix property (causal row i == non-causal over keys 0..i), the
    accumulator statement in "S12 FlashAttention", "Explore / Try it";
 7. end-aligned causal mask when Nk > Nq;
 8. GQA contiguous groups (q head h reads kv head h // group);
 9. strided (non-contiguous) inputs equal a contiguous copy;
10. key permutation invariance (non-causal);
11. shifting every score by c leaves O and adds c to LSE;
12. O is affine in V;
13. independent brute force (``oracle/twin.py``) on tiny shapes;
14. library special case: torch's scaled_dot_product_attention and
    logsumexp in fp64 on the CPU;
15. varlen == dense per sequence;
16. paged decode == dense over the gathered keys, and invariant to the pool
    order;
17. bf16 bit patterns are widened exactly.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import twin
from exact_io_aware_tile_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def test_worked_example_merge_rule():
    ex = json.load(open(os.path.join(GOLDEN, "worked_example_merge.json")))
    row = np.array(ex["row"], dtype=np.float64)
    n, d, tile = row.size, 64, ex["tile"]
    # q = 8 e_0 and k_j = row_j e_0 make the scaled score exactly row_j (scale 1/8).
    q = np.zeros((1, 1, 1, d))
    q[0, 0, 0, 0] = 8.0
    k = np.zeros((1, n, 1, d))
    k[0, :, 0, 0] = row
    v = np.zeros((1, n, 1, d))
    v[0, np.arange(n), 0, np.arange(n)] = 1.0  # V = identity: O row = softmax weights
    o, lse = oracle.dense(q, k, v, causal=False)
    w = o[0, 0, 0, :n]
    L = lse[0, 0, 0]
    tol = ex["tolerance_vs_printed"]
    pr = ex["printed"]
    # weights are a distribution
    assert abs(w.sum() - 1.0) < 1e-14 and (w > 0).all()
    # merged l at m = 3 equals the full-row sum: exp(LSE - 3)
    assert abs(math.exp(L - pr["merged"]["m"]) - pr["merged"]["l"]) < tol
    # l after tile 1 at m = 2: sum of tile-1 weights rescaled to that max
    l1 = math.exp(L - pr["after_tile_1"]["m"]) * w[:tile].sum()
    assert abs(l1 - pr["after_tile_1"]["l"]) < tol
    # tile 2's own l~ at m~ = 3
    l2 = math.exp(L - pr["tile_2_own"]["m_tile"]) * w[tile:].sum()
    assert abs(l2 - pr["tile_2_own"]["l_tile"]) < tol
    # the merge rule itself, from the printed m's and the oracle's pieces
    merged = math.exp(2.0 - 3.0) * l1 + math.exp(3.0 - 3.0) * l2
    assert abs(merged - math.exp(L - 3.0)) < 1e-12
    # the row max is the printed m = 3 and the weights are ordered like the scores
    assert np.argmax(w) == np.argmax(row)
    for a in range(n):  # weights are ordered like the scores (equal scores, equal weights)
        for b in range(n):
            if row[a] < row[b]:
                assert w[a] < w[b]
            elif row[a] == row[b]:
                assert abs(w[a] - w[b]) < 1e-16


@pytest.mark.parametrize("causal", [False, True])
def test_rows_normalised(causal):
    B, N, H, d = 2, 37, 3, 16
    q, k = rnd(1, B, N, H, d), rnd(2, B, N, H, d)
    v = np.ones((B, N, H, d))
    o, _ = oracle.dense(q, k, v, causal=causal)
    assert np.abs(o - 1.0).max() < 1e-14
    # identity values: weights over keys sum to 1, all non-negative
    n = 12
    vi = np.zeros((1, n, 1, n))
    vi[0, np.arange(n), 0, np.arange(n)] = 1.0
    o, _ = oracle.dense(rnd(3, 1, n, 1, n), rnd(4, 1, n, 1, n), vi, causal=causal)
    s = o[0, 0].sum(axis=1)
    assert np.abs(s - 1.0).max() < 1e-14 and (o >= 0).all()
    if causal:  # weights on masked keys are exactly zero
        assert np.all(np.triu(o[0, 0], 1) == 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_is_mean(causal):
    B, N, H, d = 1, 29, 2, 8
    q = np.zeros((B, N, H, d))
    k, v = rnd(5, B, N, H, d), rnd(6, B, N, H, d)
    o, lse = oracle.dense(q, k, v, causal=causal)
    for h in range(H):
        for i in range(N):
            nvis = i + 1 if causal else N
            np.testing.assert_allclose(o[0, h, i], v[0, :nvis, h].mean(axis=0), rtol=0, atol=1e-14)
            assert abs(lse[0, h, i] - math.log(nvis)) < 1e-14


def test_single_key():
    d = 32
    q, k, v = rnd(7, 1, 5, 2, d), rnd(8, 1, 1, 2, d), rnd(9, 1, 1, 2, d)
    o, lse = oracle.dense(q, k, v, causal=False)
    for h in range(2):
        for i in range(5):
            np.testing.assert_array_equal(o[0, h, i], v[0, 0, h])
            s0 = float(np.dot(q[0, i, h], k[0, 0, h])) / math.sqrt(d)
            assert abs(lse[0, h, i] - s0) < 1e-13


def test_causal_direction():
    N, d = 9, 8
    q, k, v = rnd(10, 1, N, 1, d), rnd(11, 1, N, 1, d), rnd(12, 1, N, 1, d)
    o, lse = oracle.dense(q, k, v, causal=True)
    np.testing.assert_array_equal(o[0, 0, 0], v[0, 0, 0])  # row 0 sees key 0 only
    on, ln = oracle.dense(q, k, v, causal=False)
    np.testing.assert_allclose(o[0, 0, -1], on[0, 0, -1], atol=1e-15, rtol=0)
    assert abs(lse[0, 0, -1] - ln[0, 0, -1]) < 1e-15


def test_causal_prefix_property():
    N, d = 23, 16
    q, k, v = rnd(13, 1, N, 2, d), rnd(14, 1, N, 2, d), rnd(15, 1, N, 2, d)
    o, lse = oracle.dense(q, k, v, causal=True)
    for i in [0, 1, 7, 22]:
        op, lp = oracle.dense(q[:, i:i + 1], k[:, :i + 1], v[:, :i + 1], causal=False)
        np.testing.assert_allclose(o[0, :, i], op[0, :, 0], atol=1e-14, rtol=0)
        np.testing.assert_allclose(lse[0, :, i], lp[0, :, 0], atol=1e-14, rtol=0)


def test_causal_end_aligned_when_more_keys():
    Nq, Nk, d = 5, 12, 8
    q, k, v = rnd(16, 1, Nq, 1, d), rnd(17, 1, Nk, 1, d), rnd(18, 1, Nk, 1, d)
    o, _ = oracle.dense(q, k, v, causal=True)
    for i in range(Nq):
        last = i + Nk - Nq
        op, _ = oracle.dense(q[:, i:i + 1], k[:, :last + 1], v[:, :last + 1], causal=False)
        np.testing.assert_allclose(o[0, 0, i], op[0, 0, 0], atol=1e-14, rtol=0)
    # more queries than keys: the first rows see nothing
    o2, l2 = oracle.dense(rnd(19, 1, 6, 1, d), k[:, :3], v[:, :3], causal=True)
    assert np.all(o2[0, 0, :3] == 0.0) and np.all(np.isneginf(l2[0, 0, :3]))
    assert np.all(np.isfinite(l2[0, 0, 3:]))


def test_gqa_group_mapping():
    B, N, Hq, Hkv, d = 1, 7, 6, 3, 8
    q, k = rnd(20, B, N, Hq, d), rnd(21, B, N, Hkv, d)
    v = np.zeros((B, N, Hkv, d))
    for g in range(Hkv):
        v[:, :, g, :] = 10.0 * (g + 1)
    o, _ = oracle.dense(q, k, v, causal=False)
    for h in range(Hq):
        assert np.allclose(o[0, h], 10.0 * (h // (Hq // Hkv) + 1), atol=1e-12)


def test_strided_inputs():
    B, N, H, d = 2, 19, 3, 16
    big = rnd(22, B, N, H + 2, 2 * d)
    q = big[:, :, 1:H + 1, :d]  # non-contiguous view
    k, v = rnd(23, B, N, H, d), rnd(24, B, N, H, d)
    o1, l1 = oracle.dense(q, k, v, causal=True)
    o2, l2 = oracle.dense(np.ascontiguousarray(q), k, v, causal=True)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_key_permutation_invariance():
    B, N, H, d = 1, 31, 2, 8
    q, k, v = rnd(25, B, 4, H, d), rnd(26, B, N, H, d), rnd(27, B, N, H, d)
    perm = np.random.default_rng(0).permutation(N)
    o1, l1 = oracle.dense(q, k, v, causal=False)
    o2, l2 = oracle.dense(q, k[:, perm], v[:, perm], causal=False)
    np.testing.assert_allclose(o1, o2, atol=1e-14, rtol=0)
    np.testing.assert_allclose(l1, l2, atol=1e-14, rtol=0)


def test_score_shift():
    # one extra coordinate adds the same constant c to every score of a row
    N, d, c = 13, 8, 2.5
    q, k, v = rnd(28, 1, 3, 1, d), rnd(29, 1, N, 1, d), rnd(30, 1, N, 1, d)
    scale = 0.37
    q2 = np.concatenate([q, np.ones((1, 3, 1, 1))], axis=-1)
    k2 = np.concatenate([k, np.full((1, N, 1, 1), c / scale)], axis=-1)
    v2 = np.concatenate([v, np.zeros((1, N, 1, 1))], axis=-1)
    o1, l1 = oracle.dense(q, k, v, causal=False, scale=scale)
    o2, l2 = oracle.dense(q2, k2, v2, causal=False, scale=scale)
    np.testing.assert_allclose(o2[..., :d], o1, atol=1e-13, rtol=0)
    np.testing.assert_allclose(l2, l1 + c, atol=1e-13, rtol=0)


def test_affine_in_values():
    q, k, v = rnd(31, 1, 6, 2, 8), rnd(32, 1, 10, 2, 8), rnd(33, 1, 10, 2, 8)
    o1, _ = oracle.dense(q, k, v, causal=True)
    o2, _ = oracle.dense(q, k, 3.0 * v - 1.5, causal=True)
    np.testing.assert_allclose(o2, 3.0 * o1 - 1.5, atol=1e-13, rtol=0)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 1, 1, 1, 1), (2, 5, 7, 4, 2, 3), (1, 9, 9, 2, 1, 8),
                                   (1, 16, 16, 1, 1, 8), (1, 6, 3, 2, 2, 4)])
def test_brute_force_twin(shape, causal):
    B, Nq, Nk, Hq, Hkv, d = shape
    q, k, v = rnd(34, B, Nq, Hq, d), rnd(35, B, Nk, Hkv, d), rnd(36, B, Nk, Hkv, d)
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.dense(q, k, v, causal=causal)
    ot, lt = twin.dense(q, k, v, causal, scale)
    ot, lt = np.array(ot, dtype=np.float64), np.array(lt, dtype=np.float64)
    np.testing.assert_allclose(o, ot, atol=1e-12, rtol=0)
    fin = np.isfinite(lt)
    np.testing.assert_array_equal(fin, np.isfinite(lse))
    np.testing.assert_allclose(lse[fin], lt[fin], atol=1e-12, rtol=0)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 64, 64, 4, 2, 32), (1, 200, 200, 2, 2, 64),
                                   (1, 37, 90, 2, 1, 16), (1, 512, 512, 1, 1, 128)])
def test_torch_sdpa_fp64(shape, causal):
    torch = pytest.importorskip("torch")
    B, Nq, Nk, Hq, Hkv, d = shape
    q, k, v = rnd(37, B, Nq, Hq, d), rnd(38, B, Nk, Hkv, d), rnd(39, B, Nk, Hkv, d)
    o, lse = oracle.dense(q, k, v, causal=causal)
    grp = Hq // Hkv
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(grp, dim=1)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(grp, dim=1)
    mask = None
    if causal:
        i = torch.arange(Nq)[:, None]
        j = torch.arange(Nk)[None, :]
        mask = j <= i + (Nk - Nq)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12, rtol=0)
    s = (tq @ tk.transpose(-1, -2)) / math.sqrt(d)
    if mask is not None:
        s = s.masked_fill(~mask, float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), atol=1e-12, rtol=0)


def test_varlen_equals_dense_per_sequence():
    lens = [1, 17, 5, 64, 0, 33]
    H, d = 2, 16
    c = inputs.varlen_case(40, lens, H, H, d, dtype="f32")
    q, k, v, cu = c["q"], c["k"], c["v"], c["cu_seqlens"]
    for causal in (False, True):
        o, lse = oracle.varlen(q, k, v, cu, causal=causal)
        for s, L in enumerate(lens):
            a, b = cu[s], cu[s + 1]
            if L == 0:
                continue
            od, ld = oracle.dense(q[None, a:b], k[None, a:b], v[None, a:b], causal=causal)
            np.testing.assert_array_equal(o[:, a:b], od[0])
            np.testing.assert_array_equal(lse[:, a:b], ld[0])


def test_decode_equals_dense_over_gathered_keys():
    lens = [1, 16, 17, 100, 33]
    Hq, Hkv, d, bs = 8, 2, 32, 16
    c = inputs.paged_case(41, lens, Hq, Hkv, d, block_size=bs, pad_blocks=2)
    o, lse = oracle.decode_paged(c["q"], c["k_pool"], c["v_pool"], c["block_table"], c["seq_lens"])
    qf = inputs.bf16_to_f32(c["q"]).astype(np.float64)
    kp = inputs.bf16_to_f32(c["k_pool"]).astype(np.float64)
    vp = inputs.bf16_to_f32(c["v_pool"]).astype(np.float64)
    for b, L in enumerate(lens):
        t = np.arange(L)
        phys = c["block_table"][b, t // bs]
        kk = kp[phys, :, t % bs]  # [L, Hkv, d]
        vv = vp[phys, :, t % bs]
        od, ld = oracle.dense(qf[b][None, None], kk[None], vv[None], causal=False)
        np.testing.assert_allclose(o[b], od[0, :, 0], atol=1e-14, rtol=0)
        np.testing.assert_allclose(lse[b], ld[0, :, 0], atol=1e-14, rtol=0)
    # the same logical keys in a differently ordered pool give identical results
    nb = c["num_blocks"]
    perm = np.random.default_rng(9).permutation(nb)
    inv = np.argsort(perm)
    kp2, vp2 = c["k_pool"][perm], c["v_pool"][perm]
    bt2 = np.where(c["block_table"] >= 0, inv[np.maximum(c["block_table"], 0)], -1).astype(np.int32)
    o2, l2 = oracle.decode_paged(c["q"], kp2, vp2, bt2, c["seq_lens"])
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, l2)


def test_decode_token_major_pool_layout():
    # pool stored [num_blocks, block, Hkv, d] and passed as a strided view
    lens = [20, 40]
    c = inputs.paged_case(42, lens, 4, 2, 16, block_size=16)
    o, lse = oracle.decode_paged(c["q"], c["k_pool"], c["v_pool"], c["block_table"], c["seq_lens"])
    kt = np.ascontiguousarray(c["k_pool"].transpose(0, 2, 1, 3)).transpose(0, 2, 1, 3)
    vt = np.ascontiguousarray(c["v_pool"].transpose(0, 2, 1, 3)).transpose(0, 2, 1, 3)
    o2, l2 = oracle.decode_paged(c["q"], kt, vt, c["block_table"], c["seq_lens"])
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, l2)


def test_bf16_widened_exactly():
    c = inputs.dense_case(43, 1, 20, 20, 2, 2, 16, dtype="bf16")
    o1, l1 = oracle.dense(c["q"], c["k"], c["v"], causal=True)
    w = {n: inputs.bf16_to_f32(c[n]).astype(np.float64) for n in ("q", "k", "v")}
    o2, l2 = oracle.dense(w["q"], w["k"], w["v"], causal=True)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_row_subset_matches_full():
    c = inputs.dense_case(44, 2, 33, 33, 4, 2, 16, dtype="bf16")
    o, lse = oracle.dense(c["q"], c["k"], c["v"], causal=True)
    rows = np.array([0, 5, 32, 33 * 3 + 7, 33 * 7 + 32])
    os_, ls = oracle.dense(c["q"], c["k"], c["v"], causal=True, rows=rows)
    np.testing.assert_array_equal(os_, o.reshape(-1, 16)[rows])
    np.testing.assert_array_equal(ls, lse.reshape(-1)[rows])


def test_bad_arguments_rejected():
    q = np.zeros((1, 4, 3, 8))
    k = np.zeros((1, 4, 2, 8))
    with pytest.raises(ValueError):
        oracle.dense(q, k, k, causal=False)  # 3 q heads over 2 kv heads
    c = inputs.paged_case(45, [20], 2, 1, 8)
    bt = c["block_table"].copy()
    bt[0, 0] = c["num_blocks"] + 5
    with pytest.raises(ValueError):
        oracle.decode_paged(c["q"], c["k_pool"], c["v_pool"], bt, c["seq_lens"])
