"""Pins of the oracle's merge of partial attention results (CPU only).

``oracle.merge_states`` follows "FlashAttention" (tachyon.techntrek.in),
"For engineers / Show the maths": partial states over disjoint key sets
combine by rescaling to the larger max and adding.  Its pins:

* key partition: attention over a random partition of the keys into parts
  (non-contiguous index sets), each computed by the oracle's dense
  definition, merges to attention over all keys (fp64, 1e-12);
* causal ring: query chunk c merged from its full blocks s < c and its
  causal diagonal block equals the rows of the causal attention over the
  whole sequence, the split one GPU per chunk would run ("S12
  FlashAttention", "What this unlocks beyond speed", ring attention);
* the page's worked example (printed to three decimals) and its closed form
  from the printed row;
* the page's pairwise (m, l, o) merge (``oracle.recurrence.combine``) applied
  part after part;
* special cases: one part is the identity, parts with lse = -inf are
  skipped whatever their output holds, rows no part saw are 0 / -inf, and a
  common shift of every lse shifts the merged lse only.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import recurrence

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _qkv(seed, n, nk, h=2, d=16):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((1, n, h, d)), rng.standard_normal((1, nk, h, d)),
            rng.standard_normal((1, nk, h, d)))


def test_key_partition_reaches_full_attention():
    q, k, v = _qkv(1, 12, 40)
    o_full, l_full = oracle.dense(q, k, v, causal=False)
    perm = np.random.default_rng(2).permutation(40)
    parts = [np.sort(perm[:7]), np.sort(perm[7:25]), np.sort(perm[25:])]
    os_, ls_ = [], []
    for idx in parts:
        o_p, l_p = oracle.dense(q, k[:, idx], v[:, idx], causal=False)
        os_.append(o_p)
        ls_.append(l_p)
    # a part that saw no key: lse -inf, output garbage
    os_.append(np.full_like(os_[0], np.nan))
    ls_.append(np.full_like(ls_[0], -np.inf))
    o, lse = oracle.merge_states(np.stack(os_), np.stack(ls_))
    np.testing.assert_allclose(o, o_full, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, l_full, rtol=0, atol=1e-12)


def test_causal_ring_chunks_merge_to_causal_attention():
    n, chunks = 48, 3
    q, k, v = _qkv(3, n, n, h=3, d=8)
    o_full, l_full = oracle.dense(q, k, v, causal=True)  # [1, H, N, d], [1, H, N]
    c_len = n // chunks
    for c in range(chunks):
        qc = q[:, c * c_len:(c + 1) * c_len]
        os_, ls_ = [], []
        for s in range(c + 1):
            ks, vs = k[:, s * c_len:(s + 1) * c_len], v[:, s * c_len:(s + 1) * c_len]
            o_p, l_p = oracle.dense(qc, ks, vs, causal=(s == c))
            os_.append(o_p)
            ls_.append(l_p)
        o, lse = oracle.merge_states(np.stack(os_), np.stack(ls_))
        rows = slice(c * c_len, (c + 1) * c_len)
        np.testing.assert_allclose(o, o_full[:, :, rows], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, l_full[:, :, rows], rtol=0, atol=1e-12)


def test_worked_example_as_two_parts():
    ex = json.load(open(os.path.join(GOLDEN, "worked_example_merge.json")))
    pr = ex["printed"]
    lse1 = pr["after_tile_1"]["m"] + np.log(pr["after_tile_1"]["l"])
    lse2 = pr["tile_2_own"]["m_tile"] + np.log(pr["tile_2_own"]["l_tile"])
    # outputs 1 and 0: the merged output is part 1's share of the weight
    o, lse = oracle.merge_states(np.array([[[1.0]], [[0.0]]]), np.array([[lse1], [lse2]]))
    merged_l = pr["merged"]["l"]
    assert abs(lse[0] - (pr["merged"]["m"] + np.log(merged_l))) < ex["tolerance_vs_printed"]
    share = np.exp(pr["after_tile_1"]["m"] - pr["merged"]["m"]) * pr["after_tile_1"]["l"] / merged_l
    assert abs(o[0, 0] - share) < ex["tolerance_vs_printed"]
    # closed form from the printed row: log-sum-exp of each tile, then of the row
    row = np.array(ex["row"])
    t = ex["tile"]
    lse_t = [np.log(np.exp(row[:t]).sum()), np.log(np.exp(row[t:]).sum())]
    _, lse_m = oracle.merge_states(np.zeros((2, 1, 1)), np.array(lse_t)[:, None])
    assert abs(lse_m[0] - np.log(np.exp(row).sum())) < 1e-13


def test_matches_pairwise_recurrence_merge():
    rng = np.random.default_rng(5)
    P, d = 5, 6
    states = [(float(rng.normal(0, 4)), float(rng.uniform(0.5, 9)), rng.standard_normal(d)) for _ in range(P)]
    rows = [recurrence.Rows(np.array([m_]), np.array([l_]), o_[None]) for m_, l_, o_ in states]
    acc = rows[0]
    for st in rows[1:]:
        acc = recurrence.combine(acc, st)
    m, l, ou = float(acc.mx[0]), float(acc.total[0]), acc.acc[0]
    o_parts = np.stack([(o_ / l_)[None] for _, l_, o_ in states])
    lse_parts = np.array([[m_ + np.log(l_)] for m_, l_, _ in states])
    o, lse = oracle.merge_states(o_parts, lse_parts)
    np.testing.assert_allclose(o[0], ou / l, rtol=0, atol=1e-13)
    assert abs(lse[0] - (m + np.log(l))) < 1e-13


def test_special_cases():
    rng = np.random.default_rng(6)
    o1 = rng.standard_normal((1, 7, 4))
    l1 = rng.normal(0, 3, (1, 7))
    o, lse = oracle.merge_states(o1, l1)
    np.testing.assert_array_equal(o, o1[0])
    np.testing.assert_array_equal(lse, l1[0])
    # every part empty for row 2; part 1 empty for row 4 (garbage output)
    o2 = rng.standard_normal((2, 7, 4))
    l2 = rng.normal(0, 3, (2, 7))
    l2[:, 2] = -np.inf
    l2[1, 4] = -np.inf
    o2[1, 4] = np.inf
    o, lse = oracle.merge_states(o2, l2)
    np.testing.assert_array_equal(o[2], 0.0)
    assert lse[2] == -np.inf
    np.testing.assert_allclose(o[4], o2[0, 4], rtol=0, atol=1e-15)
    assert lse[4] == l2[0, 4]
    assert np.isfinite(o).all()
    # a common shift of every lse moves the merged lse only
    o_s, lse_s = oracle.merge_states(o2, l2 + 7.25)
    np.testing.assert_allclose(o_s, o, rtol=0, atol=1e-14)
    fin = np.isfinite(lse)
    np.testing.assert_allclose(lse_s[fin], lse[fin] + 7.25, rtol=0, atol=1e-12)


@pytest.mark.parametrize("lse_shape", [(3, 5), (2, 6)])
def test_shape_mismatch_rejected(lse_shape):
    with pytest.raises(ValueError):
        oracle.merge_states(np.zeros((2, 5, 4)), np.zeros(lse_shape))
