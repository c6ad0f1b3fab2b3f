"""The seeded input generators: determinism, the documented recipe, exact bf16
rounding (checked against torch's own float32 -> bfloat16 conversion)."""
import hashlib

import numpy as np
import pytest

from exact_io_aware_tile_amd import inputs


def test_chunked_draw_matches_recipe():
    n = inputs.CHUNK + 1000
    a = inputs.normal_f32(7, 1, (n,))
    first = np.random.default_rng([7, 1, 0]).standard_normal(inputs.CHUNK, dtype=np.float32)
    second = np.random.default_rng([7, 1, 1]).standard_normal(1000, dtype=np.float32)
    np.testing.assert_array_equal(a[:inputs.CHUNK], first)
    np.testing.assert_array_equal(a[inputs.CHUNK:], second)


def test_deterministic_and_seed_sensitive():
    a = inputs.dense_case(3, 1, 40, 40, 2, 2, 16)
    b = inputs.dense_case(3, 1, 40, 40, 2, 2, 16)
    c = inputs.dense_case(4, 1, 40, 40, 2, 2, 16)
    for n in ("q", "k", "v"):
        assert hashlib.sha256(a[n].tobytes()).digest() == hashlib.sha256(b[n].tobytes()).digest()
        assert not np.array_equal(a[n], c[n])
    assert not np.array_equal(a["q"], a["k"])


def test_bf16_round_nearest_even_matches_torch():
    torch = pytest.importorskip("torch")
    x = inputs.normal_f32(11, 0, (100000,)) * np.float32(37.0)
    # include exact ties: values halfway between two bf16 neighbours
    ties = (np.arange(1, 2001, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ours = inputs.f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(inputs.bf16_to_f32(ours),
                                  torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_spike_rows_are_exact_powers_of_two():
    c = inputs.dense_case(3, 1, 500, 500, 2, 2, 8, dtype="bf16", spike_frac=0.01)
    plain = inputs.dense_case(3, 1, 500, 500, 2, 2, 8, dtype="bf16")
    sp = c["spikes"]
    assert sp.shape == (1, 2, 5)
    kf, pf = inputs.bf16_to_f32(c["k"]), inputs.bf16_to_f32(plain["k"])
    for h in range(2):
        rows = sp[0, h]
        assert len(set(rows.tolist())) == 5
        np.testing.assert_array_equal(kf[0, rows, h], 8.0 * pf[0, rows, h])
        other = np.setdiff1d(np.arange(500), rows)
        np.testing.assert_array_equal(kf[0, other, h], pf[0, other, h])
    np.testing.assert_array_equal(c["q"], plain["q"])
    np.testing.assert_array_equal(c["v"], plain["v"])


def test_varlen_recipe():
    lens = inputs.varlen_lengths(4, 16, 128, 4096)
    assert lens.shape == (16,) and lens.min() >= 128 and lens.max() <= 4096
    c = inputs.varlen_case(4, [3, 0, 5], 2, 1, 8)
    assert list(c["cu_seqlens"]) == [0, 3, 3, 8]
    assert c["q"].shape == (8, 2, 8) and c["k"].shape == (8, 1, 8)


def test_paged_recipe():
    lens = [1, 16, 17, 40]
    c = inputs.paged_case(5, lens, 4, 2, 8, block_size=16, pad_blocks=1)
    nb = [1, 1, 2, 3]
    assert c["num_blocks"] == sum(nb)
    bt = c["block_table"]
    assert bt.shape == (4, 4)
    used = np.concatenate([bt[b, :n] for b, n in enumerate(nb)])
    assert sorted(used.tolist()) == list(range(sum(nb)))  # every pool slot used once
    for b, n in enumerate(nb):
        assert np.all(bt[b, n:] == -1)
    assert c["k_pool"].shape == (7, 2, 16, 8) and c["q"].shape == (4, 4, 8)


def test_small_named_workloads():
    w1 = inputs.workload(1)
    assert w1["q"].dtype == np.float32 and w1["q"].shape == (1, 256, 1, 64) and not w1["causal"]
    w4 = inputs.workload(4)
    assert w4["q"].dtype == np.uint16 and w4["q"].shape == (w4["total"], 32, 64)
    assert w4["total"] == int(w4["lengths"].sum()) and len(w4["cu_seqlens"]) == 17
