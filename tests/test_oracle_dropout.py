"""Pins of the oracle's attention dropout, CPU only.

* ``oracle.philox4x32_10`` reproduces the generator's published known-answer
  vectors (``tests/golden/philox4x32_10_kat.json``, with their source);
* the keep decisions the attention oracle applies are exactly the ones the
  documented counter layout, byte selection and threshold give with that
  pinned generator: with q = 0 every visible key has weight 1/n, and one-hot
  value rows make O show each key's kept / dropped factor;
* probability 0 is the plain oracle bit for bit, LSE never depends on
  dropout, the keep rate matches (256 - t) / 256 within binomial bounds and
  the kept weights are scaled by 256 / (256 - t) (the output is unbiased);
* a single packed sequence (B = 1, one head) numbers rows like the dense
  layout, so the packed and dense dropout oracles agree bit for bit.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.json")


def test_philox_known_answers():
    kat = json.load(open(GOLDEN))
    for vec in kat["vectors"]:
        ctr = [int(x, 16) for x in vec["ctr"]]
        key = [int(x, 16) for x in vec["key"]]
        out = [int(x, 16) for x in vec["out"]]
        np.testing.assert_array_equal(oracle.philox4x32_10(ctr, key), np.array(out, np.uint32))


def _keep(seed, offset, row, j, t):
    w = oracle.philox4x32_10([j // 16, row & 0xFFFFFFFF, row >> 32, offset & 0xFFFFFFFF],
                             [seed & 0xFFFFFFFF, seed >> 32])
    byte = (int(w[(j % 16) // 4]) >> (8 * (j % 4))) & 0xFF
    return byte >= t


def _onehot_case(B, N, H, causal_n=None):
    q = np.zeros((B, N, H, N), np.float64)
    k = np.random.default_rng(1).standard_normal((B, N, H, N))
    v = np.zeros((B, N, H, N), np.float64)
    for j in range(N):
        v[:, j, :, j] = 1.0  # key j's value is the unit vector e_j
    return q, k, v


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_keep_decisions_follow_the_counter_layout(p):
    B, N, H = 2, 40, 3
    seed, offset = 0x1234_5678_9ABC_DEF0, 77
    q, k, v = _onehot_case(B, N, H)
    t = oracle.dropout_threshold(p)
    o, lse = oracle.dense_dropout(q, k, v, causal=False, dropout_p=p, seed=seed, offset=offset)
    scale = 256.0 / (256 - t)
    for b in range(B):
        for h in range(H):
            for i in (0, 7, N - 1):
                row = (b * H + h) * N + i
                expect = np.array([scale / N if _keep(seed, offset, row, j, t) else 0.0 for j in range(N)])
                np.testing.assert_allclose(o[b, h, i], expect, rtol=1e-12, atol=0)


def test_zero_probability_is_plain_and_lse_ignores_dropout():
    rng = np.random.default_rng(2)
    q, k, v = (rng.standard_normal((2, 33, 2, 16)) for _ in range(3))
    o0, l0 = oracle.dense(q, k, v, causal=True)
    o1, l1 = oracle.dense_dropout(q, k, v, causal=True, dropout_p=0.0, seed=5)
    np.testing.assert_array_equal(o0, o1)
    np.testing.assert_array_equal(l0, l1)
    o2, l2 = oracle.dense_dropout(q, k, v, causal=True, dropout_p=0.3, seed=5)
    np.testing.assert_array_equal(l0, l2)
    assert not np.array_equal(o0, o2)


def test_keep_rate_and_unbiased_scaling():
    B, N, H = 4, 64, 8
    q, k, v = _onehot_case(B, N, H)
    p = 0.25
    t = oracle.dropout_threshold(p)
    o, _ = oracle.dense_dropout(q, k, v, causal=False, dropout_p=p, seed=99)
    kept = (o > 0).sum()
    total = o.size
    rate = (256 - t) / 256
    sd = np.sqrt(total * rate * (1 - rate))
    assert abs(kept - total * rate) < 5 * sd
    # every kept factor is exactly scale / N; the row sums average to one
    np.testing.assert_allclose(o[o > 0], 256.0 / (256 - t) / N, rtol=1e-12)
    assert abs(o.sum(axis=-1).mean() - 1.0) < 5 * np.sqrt((1 - rate) / rate / N / (B * H * N))


def test_single_packed_sequence_numbers_rows_like_dense():
    rng = np.random.default_rng(3)
    N, d = 50, 8
    q, k, v = (rng.standard_normal((1, N, 1, d)) for _ in range(3))
    od, ld = oracle.dense_dropout(q, k, v, causal=True, dropout_p=0.4, seed=11, offset=3)
    ov, lv = oracle.varlen_dropout(q[0], k[0], v[0], np.array([0, N], np.int32), causal=True,
                                   dropout_p=0.4, seed=11, offset=3)
    np.testing.assert_array_equal(od[0], ov)
    np.testing.assert_array_equal(ld[0], lv)


def test_threshold_rule():
    assert oracle.dropout_threshold(0.0) == 0
    assert oracle.dropout_threshold(0.5) == 128
    assert oracle.dropout_threshold(0.1) == 26
    with pytest.raises(ValueError):
        oracle.dropout_threshold(1.0)


def test_packed_keep_decisions_use_head_major_rows_and_local_keys():
    cu = np.array([0, 19, 20, 45], np.int32)
    T, H = int(cu[-1]), 2
    d = 32  # >= the longest sequence: one-hot values per local key
    q = np.zeros((T, H, d))
    k = np.random.default_rng(4).standard_normal((T, H, d))
    v = np.zeros((T, H, d))
    for s in range(len(cu) - 1):
        for j in range(cu[s + 1] - cu[s]):
            v[cu[s] + j, :, j] = 1.0
    p, seed, offset = 0.3, 2**40 + 5, 9
    t = oracle.dropout_threshold(p)
    o, _ = oracle.varlen_dropout(q, k, v, cu, causal=False, dropout_p=p, seed=seed, offset=offset)
    scale = 256.0 / (256 - t)
    for h in range(H):
        for s in range(len(cu) - 1):
            n = int(cu[s + 1] - cu[s])
            for tok in range(cu[s], cu[s + 1]):
                expect = np.zeros(d)
                for j in range(n):
                    expect[j] = scale / n if _keep(seed, offset, h * T + tok, j, t) else 0.0
                np.testing.assert_allclose(o[h, tok], expect, rtol=1e-12, atol=0)


def test_sampled_rows_match_full_output():
    rng = np.random.default_rng(5)
    q, k, v = (rng.standard_normal((2, 37, 4, 16)) for _ in range(3))
    o, lse = oracle.dense_dropout(q, k, v, causal=True, dropout_p=0.2, seed=7)
    rows = np.array([0, 5, 36, 37 * 4 + 3, 2 * 4 * 37 - 1], np.int64)
    os_, ls = oracle.dense_dropout(q, k, v, causal=True, dropout_p=0.2, seed=7, rows=rows)
    np.testing.assert_array_equal(os_, o.reshape(-1, 16)[rows])
    np.testing.assert_array_equal(ls, lse.reshape(-1)[rows])
