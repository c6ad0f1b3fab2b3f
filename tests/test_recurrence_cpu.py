"""The pages' method, run in fp64 on the CPU, reaches the oracle's definition.

Mirrors the self-test described under "Run it locally" in "S12 FlashAttention"
(llminference.xinbetween.com): tiled, paged and flash-decoding (4 workers)
agree with the materialised-score reference to ~1e-15 across random inputs,
tile sizes and lengths; and the fully-masked-first-tile NaN from the callout
"exp(-inf - -inf) is NaN" appears without the guard and disappears with it.
Also pins the per-tile statistics of the worked example on the
"FlashAttention" page of tachyon.techntrek.in ("For engineers / Show the
maths").
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import recurrence as rec

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TOL = 1e-12


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def test_worked_example_tile_stats():
    ex = json.load(open(os.path.join(GOLDEN, "worked_example_merge.json")))
    st = rec.tile_stats(ex["row"], ex["tile"])
    pr, tol = ex["printed"], ex["tolerance_vs_printed"]
    assert st[0]["m"] == pr["after_tile_1"]["m"]
    assert abs(st[0]["l"] - pr["after_tile_1"]["l"]) < tol
    assert st[1]["m_tile"] == pr["tile_2_own"]["m_tile"]
    assert abs(st[1]["l_tile"] - pr["tile_2_own"]["l_tile"]) < tol
    assert st[1]["m"] == pr["merged"]["m"]
    assert abs(st[1]["l"] - pr["merged"]["l"]) < tol
    # "exactly the full-row sum"
    full = float(np.exp(np.array(ex["row"]) - 3.0).sum())
    assert abs(st[1]["l"] - full) < 1e-14
    # recomputed to full precision from the printed row
    assert abs(st[0]["l"] - 2.1975402610) < 1e-9
    assert abs(st[1]["l_tile"] - 1.8026760056) < 1e-9
    assert abs(st[1]["l"] - 2.6111058888) < 1e-9


@pytest.mark.parametrize("tile", [1, 4, 64, 1000])
@pytest.mark.parametrize("n", [1, 7, 64, 130])
def test_tiled_equals_oracle(tile, n):
    d = 16
    q, k, v = rnd(n, d), rnd(n + 1, n, d), rnd(n + 2, n, d)
    o, lse = oracle.dense(q[None, None, None], k[None, :, None], v[None, :, None], causal=False)
    of, lf = rec.stream(q, k, v, tile, 1.0 / math.sqrt(d))
    np.testing.assert_allclose(of, o[0, 0, 0], atol=TOL, rtol=0)
    assert abs(lf - lse[0, 0, 0]) < TOL


def test_tiled_causal_equals_oracle():
    N, d, tile = 70, 8, 16
    q, k, v = rnd(50, N, d), rnd(51, N, d), rnd(52, N, d)
    o, lse = oracle.dense(q[None, :, None], k[None, :, None], v[None, :, None], causal=True)
    for i in range(N):
        vis = np.arange(N) <= i
        of, lf = rec.stream(q[i], k, v, tile, 1.0 / math.sqrt(d), visible=vis)
        np.testing.assert_allclose(of, o[0, 0, i], atol=TOL, rtol=0)
        assert abs(lf - lse[0, 0, i]) < TOL


def test_intermediate_state_is_prefix_softmax():
    """Before the last tile the accumulator is the exact softmax over the keys
    seen so far ("S12 FlashAttention", "Explore / Try it")."""
    N, d, tile = 40, 8, 8
    q, k, v = rnd(53, d), rnd(54, N, d), rnd(55, N, d)
    scale = 1.0 / math.sqrt(d)
    st = rec.empty(1, d)
    for start in range(0, N, tile):
        st = rec.absorb(st, ((k[start:start + tile] @ q) * scale)[None], v[start:start + tile])
        o_part, l_part = rec.readout(st)
        o_part, l_part = o_part[0], l_part[0]
        seen = start + tile
        o, lse = oracle.dense(q[None, None, None], k[None, :seen, None], v[None, :seen, None],
                              causal=False)
        np.testing.assert_allclose(o_part, o[0, 0, 0], atol=TOL, rtol=0)
        assert abs(l_part - lse[0, 0, 0]) < TOL


@pytest.mark.parametrize("seq_len", [1, 15, 16, 17, 95])
def test_paged_equals_oracle(seq_len):
    d, bs = 8, 16
    nb = (seq_len + bs - 1) // bs + 3
    rng = np.random.default_rng(seq_len)
    k_cache, v_cache = rng.standard_normal((nb, bs, d)), rng.standard_normal((nb, bs, d))
    table = rng.permutation(nb)
    q = rng.standard_normal(d)
    t = np.arange(seq_len)
    kk, vv = k_cache[table[t // bs], t % bs], v_cache[table[t // bs], t % bs]
    o, lse = oracle.dense(q[None, None, None], kk[None, :, None], vv[None, :, None], causal=False)
    op, lp = rec.paged(q, table, k_cache, v_cache, seq_len, bs, 1.0 / math.sqrt(d))
    np.testing.assert_allclose(op, o[0, 0, 0], atol=TOL, rtol=0)
    assert abs(lp - lse[0, 0, 0]) < TOL


@pytest.mark.parametrize("n", [4, 9, 1000])
def test_split_four_workers_equals_oracle(n):
    d = 16
    q, k, v = rnd(60, d), rnd(61, n, d), rnd(62, n, d)
    o, lse = oracle.dense(q[None, None, None], k[None, :, None], v[None, :, None], causal=False)
    os_, ls = rec.split(q, k, v, workers=4, tile=16, scale=1.0 / math.sqrt(d))
    np.testing.assert_allclose(os_, o[0, 0, 0], atol=TOL, rtol=0)
    assert abs(ls - lse[0, 0, 0]) < TOL


def test_fully_masked_first_tile_nan_and_guard():
    N, d, tile = 32, 8, 8
    q, k, v = rnd(63, d), rnd(64, N, d), rnd(65, N, d)
    vis = np.arange(N) >= tile  # the whole first tile is masked
    with np.errstate(invalid="ignore"):
        o_bad, _ = rec.stream(q, k, v, tile, 0.5, visible=vis, guard=False)
    assert np.isnan(o_bad).all()
    o_ok, l_ok = rec.stream(q, k, v, tile, 0.5, visible=vis, guard=True)
    o, lse = oracle.dense(q[None, None, None], k[None, tile:, None], v[None, tile:, None],
                          causal=False, scale=0.5)
    np.testing.assert_allclose(o_ok, o[0, 0, 0], atol=TOL, rtol=0)
    assert abs(l_ok - lse[0, 0, 0]) < TOL


def test_merge_with_empty_state_is_identity():
    d = 4
    st = rec.absorb(rec.empty(1, d), np.array([[0.3, -1.0]]), rnd(66, 2, d))
    for m in (rec.combine(st, rec.empty(1, d)), rec.combine(rec.empty(1, d), st)):
        assert m.mx[0] == st.mx[0] and m.total[0] == st.total[0] and np.array_equal(m.acc, st.acc)


def test_many_rows_at_once_equal_one_row_at_a_time():
    N, d = 45, 8
    q, k, v = rnd(67, 6, d), rnd(68, N, d), rnd(69, N, d)
    vis = np.arange(N)[None, :] <= (np.arange(6)[:, None] * 7 + 3)
    o, lse = rec.stream(q, k, v, 16, 0.4, visible=vis)
    for i in range(6):
        oi, li = rec.stream(q[i], k, v, 16, 0.4, visible=vis[i])
        np.testing.assert_allclose(o[i], oi, atol=1e-15, rtol=0)
        assert abs(lse[i] - li) < 1e-15
