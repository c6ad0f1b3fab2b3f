"""Pins of the oracle's FP8 E4M3 path and of the FP8 input recipe, CPU only.

* ``oracle.decode_e4m3`` against torch's ``float8_e4m3fn`` widening (a
  library routine) for all 256 codes, and against values the format
  definition fixes (1.0, the largest finite 448, the smallest normal 2^-6, the
  smallest subnormal 2^-9, negative zero, NaN);
* ``oracle.fp8_dense`` composes decoding, per-tensor descaling and the dense
  oracle: scaling V's descale scales O and leaves LSE alone; Q's and K's
  descales enter only through their product with the score scale; decoding
  and descaling by hand and calling ``oracle.dense`` gives the same bits;
* ``inputs.f32_to_e4m3`` rounds to nearest-even and saturates, checked
  against torch's conversion and on constructed ties.
"""
import math

import numpy as np
import pytest

import oracle
from exact_io_aware_tile_amd import inputs

torch = pytest.importorskip("torch")


def test_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.decode_e4m3(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    np.testing.assert_array_equal(np.isnan(mine), nan)
    np.testing.assert_array_equal(mine[~nan], ref[~nan])
    # sign of zero too
    assert math.copysign(1.0, mine[0x80]) == -1.0


def test_decode_closed_forms():
    v = oracle.decode_e4m3(np.array([0x38, 0x7E, 0x08, 0x01, 0x07, 0xB8, 0x80, 0x7F, 0xFF, 0x3C], np.uint8))
    assert v[0] == 1.0
    assert v[1] == 448.0
    assert v[2] == 2.0 ** -6
    assert v[3] == 2.0 ** -9
    assert v[4] == 7 * 2.0 ** -9
    assert v[5] == -1.0
    assert v[6] == 0.0 and math.copysign(1.0, v[6]) == -1.0
    assert np.isnan(v[7]) and np.isnan(v[8])
    assert v[9] == 1.5


def _case(seed, B=2, N=37, H=2, d=16):
    c = inputs.fp8_case(seed, B, N, N, H, H, d)
    return c["q"], c["k"], c["v"], tuple(float(x) for x in c["descale"])


def test_fp8_dense_equals_dense_on_widened_inputs():
    q8, k8, v8, (qd, kd, vd) = _case(71)
    for causal in (False, True):
        o, lse = oracle.fp8_dense(q8, k8, v8, (qd, kd, vd), causal=causal)
        q = torch.from_numpy(q8).view(torch.float8_e4m3fn).double().numpy() * qd
        k = torch.from_numpy(k8).view(torch.float8_e4m3fn).double().numpy() * kd
        v = torch.from_numpy(v8).view(torch.float8_e4m3fn).double().numpy() * vd
        o2, l2 = oracle.dense(q, k, v, causal=causal)
        np.testing.assert_array_equal(o, o2)
        np.testing.assert_array_equal(lse, l2)


def test_fp8_varlen_equals_fp8_dense_per_sequence():
    lens = [5, 0, 23, 1]
    c = inputs.fp8_varlen_case(72, lens, 4, 2, 16)
    cu, ds = c["cu_seqlens"], tuple(float(x) for x in c["descale"])
    for causal in (False, True):
        o, lse = oracle.fp8_varlen(c["q"], c["k"], c["v"], cu, ds, causal=causal)
        for s, L in enumerate(lens):
            if L == 0:
                continue
            a, b = cu[s], cu[s + 1]
            od, ld = oracle.fp8_dense(c["q"][None, a:b], c["k"][None, a:b], c["v"][None, a:b], ds, causal=causal)
            np.testing.assert_array_equal(o[:, a:b], od[0])
            np.testing.assert_array_equal(lse[:, a:b], ld[0])


def test_decode_paged_fp8_equals_decode_on_hand_decoded_pools():
    c = inputs.paged_fp8_case(73, [5, 0, 40, 17], 4, 2, 16)
    kd, vd = (float(x) for x in c["descale"])
    o, lse = oracle.decode_paged_fp8(c["q"], c["k_pool"], c["v_pool"], c["block_table"], c["seq_lens"], (kd, vd))
    q = torch.from_numpy(c["q"].view(np.int16)).view(torch.bfloat16).double().numpy()
    kp = torch.from_numpy(c["k_pool"]).view(torch.float8_e4m3fn).double().numpy() * kd
    vp = torch.from_numpy(c["v_pool"]).view(torch.float8_e4m3fn).double().numpy() * vd
    o2, l2 = oracle.decode_paged(q, kp, vp, c["block_table"], c["seq_lens"])
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, l2)
    # V's descale scales O only; K's acts through the scores
    o3, l3 = oracle.decode_paged_fp8(c["q"], c["k_pool"], c["v_pool"], c["block_table"], c["seq_lens"],
                                     (kd, 2 * vd))
    np.testing.assert_allclose(o3, 2 * o, rtol=1e-14, atol=0)
    np.testing.assert_array_equal(l3, lse)


def test_paged_prefill_fp8_equals_paged_prefill_on_hand_decoded_inputs():
    c = inputs.paged_prefill_fp8_case(74, [3, 0, 20], [40, 5, 20], 4, 2, 16)
    ds = tuple(float(x) for x in c["descale"])
    for causal in (False, True):
        o, lse = oracle.paged_prefill_fp8(c["q"], c["k_pool"], c["v_pool"], c["block_table"], c["cu_seqlens_q"],
                                          c["seq_lens"], ds, causal=causal)
        wid = [torch.from_numpy(c[n]).view(torch.float8_e4m3fn).double().numpy() * f
               for n, f in zip(("q", "k_pool", "v_pool"), ds)]
        o2, l2 = oracle.paged_prefill(*wid, c["block_table"], c["cu_seqlens_q"], c["seq_lens"], causal=causal)
        np.testing.assert_array_equal(o, o2)
        np.testing.assert_array_equal(lse, l2)


def test_v_descale_scales_output_only():
    q8, k8, v8, (qd, kd, vd) = _case(72)
    o1, l1 = oracle.fp8_dense(q8, k8, v8, (qd, kd, vd), causal=True)
    o2, l2 = oracle.fp8_dense(q8, k8, v8, (qd, kd, 4 * vd), causal=True)
    np.testing.assert_allclose(o2, 4 * o1, rtol=1e-15, atol=0)
    np.testing.assert_array_equal(l1, l2)


def test_qk_descales_act_through_the_score_scale():
    q8, k8, v8, (qd, kd, vd) = _case(73)
    d = q8.shape[-1]
    base = 1.0 / math.sqrt(d)
    o1, l1 = oracle.fp8_dense(q8, k8, v8, (2 * qd, kd, vd), causal=False)
    o2, l2 = oracle.fp8_dense(q8, k8, v8, (qd, 2 * kd, vd), causal=False)
    o3, l3 = oracle.fp8_dense(q8, k8, v8, (qd, kd, vd), causal=False, scale=2 * base)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(o1, o3, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l3, rtol=0, atol=1e-12)


def test_input_rounding_matches_torch_and_saturates():
    x = (np.random.default_rng(5).standard_normal(200000) * 60).astype(np.float32)
    mine = inputs.f32_to_e4m3(x)
    ref = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(mine, ref)
    # ties between neighbours go to the even code; beyond 448 saturates
    ties = np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -11, 500.0, -1e6, 464.0], np.float32)
    np.testing.assert_array_equal(inputs.f32_to_e4m3(ties), [0x38, 0x3A, 0x00, 0x01, 0x7E, 0xFE, 0x7E])
    # widening back is exact
    codes = np.arange(0, 255, dtype=np.uint8)
    codes = codes[(codes & 0x7F) != 0x7F]
    np.testing.assert_array_equal(inputs.e4m3_to_f32(codes).astype(np.float64), oracle.decode_e4m3(codes))


def test_fp8_case_descale_is_amax_over_448():
    c = inputs.fp8_case(74, 1, 64, 64, 2, 2, 32)
    for name, stream, dsc in (("q", inputs.STREAM_Q, c["descale"][0]), ("v", inputs.STREAM_V, c["descale"][2])):
        x = inputs.normal_f32(74, stream, c[name].shape)
        assert dsc == np.float32(np.abs(x).max() / 448.0)
        # the largest magnitude maps to (almost) the top of the range
        assert inputs.e4m3_to_f32(c[name]).max() <= 448.0
        assert np.abs(inputs.e4m3_to_f32(c[name])).max() >= 416.0
