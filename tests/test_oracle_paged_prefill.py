"""Pins of the oracle's chunked (paged) prefill, CPU only.

``oracle.paged_prefill`` is pinned against things other than itself:

* a chunk of one query per sequence is the paged decode (a different C
  function with its own addressing);
* with the keys gathered through the block table, each sequence's chunk is
  dense attention with Nq = chunk, Nk = context and the end-aligned causal
  mask (``oracle.dense``, separate code);
* a chunk that is the whole context is the packed causal attention
  (``oracle.varlen``);
* the pure-Python brute force (``oracle.twin``) on tiny shapes with 2-token
  blocks;
* a permuted pool with the matching table gives identical results;
* a chunk longer than the context leaves its first rows without keys
  (o = 0, LSE = -inf), the reading for fully masked rows.
"""
import math

import numpy as np

import oracle
from oracle import twin
from exact_io_aware_tile_amd import inputs


def _f64(a):
    return inputs.bf16_to_f32(a).astype(np.float64)


def _gather(c, s, L):
    bs = c["block_size"]
    t = np.arange(L)
    phys = c["block_table"][s, t // bs]
    return _f64(c["k_pool"])[phys, :, t % bs], _f64(c["v_pool"])[phys, :, t % bs]  # [L, Hkv, d]


def test_chunk_of_one_is_decode():
    k_lens = [1, 16, 17, 100, 33]
    c = inputs.paged_prefill_case(51, [1] * 5, k_lens, 8, 2, 32, pad_blocks=1)
    o, lse = oracle.paged_prefill(c["q"], c["k_pool"], c["v_pool"], c["block_table"], c["cu_seqlens_q"],
                                  c["seq_lens"], causal=True)
    od, ld = oracle.decode_paged(c["q"], c["k_pool"], c["v_pool"], c["block_table"], c["seq_lens"])
    np.testing.assert_array_equal(o.transpose(1, 0, 2), od)  # [Hq, T, d] vs [B, Hq, d]
    np.testing.assert_array_equal(lse.T, ld)


def test_chunks_equal_dense_over_gathered_keys():
    q_lens, k_lens = [7, 1, 40, 16], [50, 9, 40, 100]
    Hq, Hkv, d = 4, 2, 16
    for causal in (True, False):
        c = inputs.paged_prefill_case(52, q_lens, k_lens, Hq, Hkv, d)
        o, lse = oracle.paged_prefill(c["q"], c["k_pool"], c["v_pool"], c["block_table"],
                                      c["cu_seqlens_q"], c["seq_lens"], causal=causal)
        q = _f64(c["q"])
        cu = c["cu_seqlens_q"]
        for s, (nq, L) in enumerate(zip(q_lens, k_lens)):
            kk, vv = _gather(c, s, L)
            od, ld = oracle.dense(q[cu[s]:cu[s + 1]][None], kk[None], vv[None], causal=causal)
            np.testing.assert_allclose(o[:, cu[s]:cu[s + 1]], od[0], atol=1e-14, rtol=0)
            np.testing.assert_allclose(lse[:, cu[s]:cu[s + 1]], ld[0], atol=1e-14, rtol=0)


def test_whole_context_chunk_is_varlen():
    lens = [5, 33, 64, 17]
    Hq, Hkv, d = 4, 4, 8
    c = inputs.paged_prefill_case(53, lens, lens, Hq, Hkv, d)
    o, lse = oracle.paged_prefill(c["q"], c["k_pool"], c["v_pool"], c["block_table"], c["cu_seqlens_q"],
                                  c["seq_lens"], causal=True)
    k = np.concatenate([_gather(c, s, L)[0] for s, L in enumerate(lens)])
    v = np.concatenate([_gather(c, s, L)[1] for s, L in enumerate(lens)])
    ov, lv = oracle.varlen(_f64(c["q"]), k, v, c["cu_seqlens_q"], causal=True)
    np.testing.assert_allclose(o, ov, atol=1e-14, rtol=0)
    np.testing.assert_allclose(lse, lv, atol=1e-14, rtol=0)


def test_brute_force_twin():
    q_lens, k_lens = [3, 2, 4], [5, 7, 2]
    Hq, Hkv, d, bs = 2, 1, 4, 2
    c = inputs.paged_prefill_case(54, q_lens, k_lens, Hq, Hkv, d, block_size=bs)
    q = _f64(c["q"])
    cu = c["cu_seqlens_q"]
    for causal in (True, False):
        o, lse = oracle.paged_prefill(c["q"], c["k_pool"], c["v_pool"], c["block_table"],
                                      c["cu_seqlens_q"], c["seq_lens"], causal=causal)
        for s, (nq, L) in enumerate(zip(q_lens, k_lens)):
            kk, vv = _gather(c, s, L)
            for h in range(Hq):
                qs = [list(q[t, h]) for t in range(cu[s], cu[s + 1])]
                vis = (lambda i, j: j <= i + (L - nq)) if causal else (lambda i, j: True)
                ot, lt = twin.attention(qs, [list(x) for x in kk[:, 0]], [list(x) for x in vv[:, 0]],
                                        1.0 / math.sqrt(d), vis)
                for i in range(nq):
                    if math.isinf(lt[i]):
                        assert lse[h, cu[s] + i] == -np.inf
                        np.testing.assert_array_equal(o[h, cu[s] + i], 0.0)
                    else:
                        np.testing.assert_allclose(o[h, cu[s] + i], ot[i], atol=1e-12, rtol=0)
                        assert abs(lse[h, cu[s] + i] - lt[i]) < 1e-12


def test_pool_order_does_not_matter():
    q_lens, k_lens = [9, 30], [60, 33]
    c = inputs.paged_prefill_case(55, q_lens, k_lens, 4, 2, 16, pad_blocks=2)
    args = (c["cu_seqlens_q"], c["seq_lens"])
    o, lse = oracle.paged_prefill(c["q"], c["k_pool"], c["v_pool"], c["block_table"], *args, causal=True)
    perm = np.random.default_rng(3).permutation(c["num_blocks"])
    inv = np.argsort(perm)
    bt2 = np.where(c["block_table"] >= 0, inv[np.maximum(c["block_table"], 0)], -1).astype(np.int32)
    o2, l2 = oracle.paged_prefill(c["q"], c["k_pool"][perm], c["v_pool"][perm], bt2, *args, causal=True)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, l2)


def test_chunk_longer_than_context_starts_without_keys():
    # 6 queries over 4 keys, causal end-aligned: query i sees keys t <= i - 2
    c = inputs.paged_prefill_case(56, [6], [4], 2, 2, 8)
    o, lse = oracle.paged_prefill(c["q"], c["k_pool"], c["v_pool"], c["block_table"], c["cu_seqlens_q"],
                                  c["seq_lens"], causal=True)
    assert np.all(lse[:, :2] == -np.inf) and np.all(o[:, :2] == 0.0)
    assert np.all(np.isfinite(lse[:, 2:]))
    # query 2 sees exactly key 0: its output is v_0 and its LSE the one score
    kk, vv = _gather(c, 0, 4)
    q = _f64(c["q"])
    for h in range(2):
        np.testing.assert_allclose(o[h, 2], vv[0, h], atol=1e-14, rtol=0)
        assert abs(lse[h, 2] - q[2, h] @ kk[0, h] / math.sqrt(8)) < 1e-12
