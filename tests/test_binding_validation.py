"""The Python binding rejects tensors that disagree with the call before it
touches the GPU or the library.

The C ABI trusts the sizes it is given (it receives raw pointers), so a
short output, a value tensor shorter than the keys or an operand of the wrong
dtype would be read or written out of bounds on the device.  Every check
here runs on CPU tensors: the binding validates shapes and dtypes before its
device check, so each case must raise its own error, not "tensors must be on
the GPU".
"""
import pytest
import torch

from exact_io_aware_tile_amd import fa

bf, f32, u8, i32 = torch.bfloat16, torch.float32, torch.uint8, torch.int32


def z(*shape, dt=bf):
    return torch.zeros(shape, dtype=dt)


def dense_ok(dt=bf):
    return dict(q=z(2, 10, 4, 64, dt=dt), k=z(2, 12, 2, 64, dt=dt), v=z(2, 12, 2, 64, dt=dt))


def raises(exc, match, fn, *a, **kw):
    with pytest.raises(exc, match=match) as e:
        fn(*a, **kw)
    assert "on the GPU" not in str(e.value)


@pytest.mark.parametrize("change,exc,match", [
    (dict(v=z(2, 11, 2, 64)), ValueError, "v must have shape"),
    (dict(k=z(2, 12, 2, 128), v=z(2, 12, 2, 128)), ValueError, "k must have shape"),
    (dict(k=z(3, 12, 2, 64), v=z(3, 12, 2, 64)), ValueError, "k must have shape"),
    (dict(k=z(2, 12, 2, 64, dt=f32), v=z(2, 12, 2, 64, dt=f32)), TypeError, "k must be"),
    (dict(v=z(2, 12, 2, 64, dt=f32)), TypeError, "v must be"),
    (dict(out=z(2, 9, 4, 64)), ValueError, "out must have shape"),
    (dict(out=z(2, 10, 4, 64, dt=f32)), TypeError, "out must be"),
    (dict(lse=z(2, 4, 9, dt=f32)), ValueError, "lse must have shape"),
    (dict(lse=z(2, 4, 10, dt=bf)), TypeError, "lse must be"),
    (dict(lse=z(2, 10, 4, dt=f32).transpose(1, 2)), ValueError, "lse must be contiguous"),
    (dict(q=z(2, 10, 4)), ValueError, "q must be a 4-D"),
])
def test_dense_rejects(change, exc, match):
    kw = dense_ok()
    kw.update(change)
    q, k, v = kw.pop("q"), kw.pop("k"), kw.pop("v")
    raises(exc, match, fa.fa_fwd, q, k, v, **kw)
    raises(exc, match, fa.fa_fwd_dropout, q, k, v, dropout_p=0.1, seed=1, **kw)


def test_dense_rejects_unsupported_dtype():
    kw = dense_ok(dt=torch.float16)
    raises(TypeError, "unsupported dtype", fa.fa_fwd, kw["q"], kw["k"], kw["v"])


@pytest.mark.parametrize("change,exc,match", [
    (dict(q=z(2, 10, 4, 64)), TypeError, "uint8"),
    (dict(v=z(2, 11, 2, 64, dt=u8)), ValueError, "v must have shape"),
    (dict(out=z(2, 10, 4, 64, dt=f32)), TypeError, "out must be"),
    (dict(lse=z(2, 4, 11, dt=f32)), ValueError, "lse must have shape"),
])
def test_dense_fp8_rejects(change, exc, match):
    kw = dense_ok(dt=u8)
    kw.update(change)
    q, k, v = kw.pop("q"), kw.pop("k"), kw.pop("v")
    raises(exc, match, fa.fa_fwd_fp8, q, k, v, (1.0, 1.0, 1.0), **kw)


def varlen_ok(dt=bf):
    return dict(q=z(30, 4, 64, dt=dt), k=z(30, 2, 64, dt=dt), v=z(30, 2, 64, dt=dt),
                cu=torch.tensor([0, 10, 30], dtype=i32))


@pytest.mark.parametrize("change,exc,match", [
    (dict(k=z(29, 2, 64)), ValueError, "k must have shape"),
    (dict(v=z(30, 1, 64)), ValueError, "v must have shape"),
    (dict(cu=torch.tensor([0, 10, 30], dtype=torch.int64)), TypeError, "cu_seqlens must be"),
    (dict(cu=torch.zeros(2, 2, dtype=i32)), ValueError, "cu_seqlens must be a 1-D"),
    (dict(out=z(30, 4, 32)), ValueError, "out must have shape"),
    (dict(lse=z(30, 4, dt=f32)), ValueError, "lse must have shape"),
])
def test_varlen_rejects(change, exc, match):
    kw = varlen_ok()
    kw.update(change)
    q, k, v, cu = kw.pop("q"), kw.pop("k"), kw.pop("v"), kw.pop("cu")
    raises(exc, match, fa.fa_fwd_varlen, q, k, v, cu, 20, **kw)
    raises(exc, match, fa.fa_fwd_varlen_dropout, q, k, v, cu, 20, dropout_p=0.1, seed=1, **kw)


def test_varlen_fp8_rejects_mixed_dtypes():
    kw = varlen_ok(dt=u8)
    raises(TypeError, "uint8", fa.fa_fwd_varlen_fp8, kw["q"], kw["k"], z(30, 2, 64), kw["cu"], 20, (1, 1, 1))
    raises(ValueError, "out must have shape", fa.fa_fwd_varlen_fp8, kw["q"], kw["k"], kw["v"], kw["cu"], 20,
           (1, 1, 1), out=z(30, 4, 64)[:20])


def decode_ok(pool_dt=bf):
    return dict(q=z(3, 8, 128), kp=z(20, 2, 16, 128, dt=pool_dt), vp=z(20, 2, 16, 128, dt=pool_dt),
                bt=torch.zeros(3, 5, dtype=i32), sl=torch.ones(3, dtype=i32))


@pytest.mark.parametrize("change,exc,match", [
    (dict(q=z(3, 8, 128, dt=f32)), TypeError, "q must be"),
    (dict(kp=z(20, 2, 16, 128, dt=f32), vp=z(20, 2, 16, 128, dt=f32)), TypeError, "k_pool must be"),
    (dict(vp=z(19, 2, 16, 128)), ValueError, "v_pool must have shape"),
    (dict(kp=z(20, 2, 16, 64), vp=z(20, 2, 16, 64)), ValueError, "head_dim"),
    (dict(bt=torch.zeros(2, 5, dtype=i32)), ValueError, "block_table must have shape"),
    (dict(bt=torch.zeros(3, 5, dtype=torch.int64)), TypeError, "block_table must be"),
    (dict(bt=torch.zeros(5, 3, dtype=i32).t()), ValueError, "block_table must be contiguous"),
    (dict(sl=torch.ones(4, dtype=i32)), ValueError, "seq_lens must have shape"),
    (dict(sl=torch.ones(3, dtype=torch.int64)), TypeError, "seq_lens must be"),
    (dict(out=z(3, 8, 64)), ValueError, "out must have shape"),
    (dict(lse=z(3, 7, dt=f32)), ValueError, "lse must have shape"),
    (dict(lse=z(3, 8)), TypeError, "lse must be"),
])
def test_decode_rejects(change, exc, match):
    kw = decode_ok()
    kw.update(change)
    args = [kw.pop(n) for n in ("q", "kp", "vp", "bt", "sl")]
    raises(exc, match, fa.fa_decode_paged, *args, 64, **kw)
    if not kw:
        raises(exc, match, fa.fa_decode_paged_workspace_size, *args, 64)
        raises(exc, match, fa.fa_decode_paged_num_splits, *args, 64)


def test_decode_fp8_rejects():
    kw = decode_ok(pool_dt=u8)
    args = [kw[n] for n in ("q", "kp", "vp", "bt", "sl")]
    raises(TypeError, "uint8", fa.fa_decode_paged_fp8, args[0], z(20, 2, 16, 128), *args[2:], 64, (1, 1))
    raises(ValueError, "seq_lens must have shape", fa.fa_decode_paged_fp8, *args[:4], torch.ones(2, dtype=i32), 64,
           (1, 1))
    raises(TypeError, "q must be", fa.fa_decode_paged_fp8_workspace_size, z(3, 8, 128, dt=f32), *args[1:], 64,
           (1, 1))


def paged_ok(dt=bf):
    return dict(q=z(12, 8, 128, dt=dt), kp=z(20, 2, 16, 128, dt=dt), vp=z(20, 2, 16, 128, dt=dt),
                bt=torch.zeros(2, 5, dtype=i32), cu=torch.tensor([0, 4, 12], dtype=i32),
                sk=torch.tensor([30, 60], dtype=i32))


@pytest.mark.parametrize("change,exc,match", [
    (dict(bt=torch.zeros(3, 5, dtype=i32)), ValueError, "block_table must have shape"),
    (dict(sk=torch.tensor([30], dtype=i32)), ValueError, "seq_lens_k must have shape"),
    (dict(vp=z(20, 2, 16, 128)[:, :1]), ValueError, "v_pool must have shape"),
    (dict(out=z(11, 8, 128)), ValueError, "out must have shape"),
    (dict(lse=z(8, 11, dt=f32)), ValueError, "lse must have shape"),
])
def test_paged_prefill_rejects(change, exc, match):
    kw = paged_ok()
    kw.update(change)
    args = [kw.pop(n) for n in ("q", "kp", "vp", "bt", "cu", "sk")]
    raises(exc, match, fa.fa_fwd_paged, *args, 8, 80, **kw)


def test_paged_prefill_fp8_rejects():
    kw = paged_ok(dt=u8)
    args = [kw[n] for n in ("q", "kp", "vp", "bt", "cu", "sk")]
    raises(TypeError, "uint8", fa.fa_fwd_paged_fp8, z(12, 8, 128), *args[1:], 8, 80, (1, 1, 1))
    raises(ValueError, "out must have shape", fa.fa_fwd_paged_fp8, *args, 8, 80, (1, 1, 1), out=z(12, 8, 64))


def test_merge_rejects():
    o_parts, lse_parts = z(3, 1, 5, 2, 64), z(3, 1, 2, 5, dt=f32)
    raises(ValueError, "out must have shape", fa.fa_merge_states, o_parts, lse_parts, out=z(1, 5, 2, 32))
    raises(ValueError, "lse must have shape", fa.fa_merge_states, o_parts, lse_parts, lse=z(1, 5, 2, dt=f32))
    raises(ValueError, "lse_parts must be", fa.fa_merge_states, o_parts, z(2, 1, 2, 5, dt=f32))
