"""GPU parity at shapes where the prefill work mapping takes the XCD's pairs
in chunks that do not divide them, with a GQA group of three (K/V of one kv
head within 4 MB: chunk = whole groups, the last chunk shorter), packed and
dense.  Tolerances are those of ``test_gpu_parity`` (bf16)."""
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


def check(og, lg, o_ref, l_ref, what):
    err = np.abs(og - o_ref)
    assert np.isfinite(og).all(), what
    assert err.max() <= BF16[0] and err.mean() <= BF16[1], f"{what}: max |dO| {err.max():.3e}"
    fin = np.isfinite(l_ref)
    np.testing.assert_array_equal(np.isfinite(lg), fin, err_msg=what)
    assert np.abs(lg[fin] - l_ref[fin]).max() <= 1e-3, what


def test_packed_chunks_not_dividing_with_group_three(gpu):
    # 32 sequences x 6 q heads = 192 pairs, 24 per XCD; K/V of one kv head at
    # 1200 tokens, d = 128 is 614 KB -> chunks of 6 groups x 3 = 18 pairs (18 + 6).
    lens = np.random.default_rng(9100).integers(1, 1201, size=32)
    lens[0] = 1200
    case = inputs.varlen_case(9100, lens, 6, 2, 128, dtype="bf16")
    o, lse = gpu.fa_fwd_varlen(*(bdev(case[n]) for n in ("q", "k", "v")), torch.from_numpy(case["cu_seqlens"]).cuda(),
                               case["max_seqlen"], causal=True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.varlen(case["q"], case["k"], case["v"], case["cu_seqlens"], causal=True)
    check(o.float().cpu().numpy().astype(np.float64).transpose(1, 0, 2), lse.cpu().numpy().astype(np.float64),
          o_ref, l_ref, "packed, chunks of 18 of 24 pairs, group 3")


@pytest.mark.parametrize("causal", [True, False])
def test_dense_chunks_of_eight_pairs(gpu, causal):
    # B = 16, H = 16: 256 pairs, 32 per XCD; 1000 keys at d = 128 is 512 KB
    # of K/V -> chunks of 8 pairs; N = 1000 leaves a ragged last query tile.
    case = inputs.dense_case(9101, 16, 1000, 1000, 16, 16, 128, dtype="bf16")
    o, lse = gpu.fa_fwd(*(bdev(case[n]) for n in ("q", "k", "v")), causal=causal)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, 16 * 16 * 1000, 97), [16 * 16 * 1000 - 1]]))
    o_ref, l_ref = oracle.dense(case["q"], case["k"], case["v"], causal=causal, rows=rows)
    og = o.float().cpu().numpy().astype(np.float64).transpose(0, 2, 1, 3).reshape(-1, 128)[rows]
    lg = lse.cpu().numpy().astype(np.float64).reshape(-1)[rows]
    check(og, lg, o_ref, l_ref, f"dense chunks of 8 causal={causal}")  # oracle rows: (b * H + h) * N + i
