"""fa_decode_paged_noalloc, the decode entry point for callers that cannot
allocate, against fa_decode_paged with a caller workspace.

Both run the same kernels with the same split count, so their outputs must be
identical bit for bit; the library-held workspace keeps the previous call's
partial states, so two calls in a row (the second one smaller, with fewer
parts and sequences) must each match their own reference.
"""
import numpy as np
import pytest

from exact_io_aware_tile_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_io_aware_tile_amd import fa as m
    m.lib()
    return m


def bf(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def run_both(fa, case, num_splits):
    q, kp, vp = bf(case["q"]), bf(case["k_pool"]), bf(case["v_pool"])
    bt = torch.from_numpy(case["block_table"]).cuda()
    sl = torch.from_numpy(case["seq_lens"]).cuda()
    maxlen = int(case["seq_lens"].max(initial=0))
    o_ref, l_ref = fa.fa_decode_paged(q, kp, vp, bt, sl, maxlen, num_splits=num_splits)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((q.shape[0], q.shape[1]), float("nan"), dtype=torch.float32, device="cuda")
    fa.fa_decode_paged_noalloc(q, kp, vp, bt, sl, maxlen, num_splits=num_splits, out=out, lse=lse)
    torch.cuda.synchronize()
    return o_ref, l_ref, out, lse


def test_noalloc_matches_workspace_call_twice(fa):
    # the batch-64 decode workload with its automatic split (384 parts on a
    # 256-CU device), then a smaller call with an explicit split
    big = inputs.workload(5)
    o_ref, l_ref, o, lse = run_both(fa, big, 0)
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(lse, l_ref)
    small = inputs.paged_case(801, [1, 300, 0, 5000], 16, 4, 128)
    o_ref, l_ref, o, lse = run_both(fa, small, 7)
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(lse[torch.isfinite(l_ref)], l_ref[torch.isfinite(l_ref)])
    assert torch.equal(torch.isinf(lse), torch.isinf(l_ref))


@pytest.mark.parametrize("d", [64, 256])
def test_noalloc_other_head_dims(fa, d):
    case = inputs.paged_case(802 + d, [17, 900, 2048], 8, 2, d)
    o_ref, l_ref, o, lse = run_both(fa, case, 0)
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(lse, l_ref)


def test_noalloc_rejects_oversize_without_launch(fa):
    case = inputs.paged_case(803, [16] * 64, 32, 8, 128)
    q, kp, vp = bf(case["q"]), bf(case["k_pool"]), bf(case["v_pool"])
    bt = torch.from_numpy(case["block_table"]).cuda()
    sl = torch.from_numpy(case["seq_lens"]).cuda()
    out = torch.zeros_like(q)
    # 32 heads x (2000 + 64) slots x 132 floats = 34.9 MB > the 16 MiB held
    with pytest.raises(fa.FAError, match="library holds"):
        fa.fa_decode_paged_noalloc(q, kp, vp, bt, sl, 16, num_splits=2000, out=out)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(out)) == 0
