"""Host-side checks of the C ABI (no GPU needed, no kernel launched).

* libfa_gfx950.so loads and exports every function include/fa.h declares;
* the ctypes mirrors of the argument structs have the C layout (checked
  against gcc's sizeof/offsetof of include/fa.h);
* every invalid argument is rejected with its status before any launch, and
  no-op calls return FA_OK without touching memory;
* workspace and split sizing follow the documented rules.
"""
import ctypes
import os
import re
import subprocess

import pytest

from exact_io_aware_tile_amd import fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fa.LIB_PATH):
        pytest.fail("libfa_gfx950.so is not built (python -m exact_io_aware_tile_amd.build)")
    return fa.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert set(names) == set(fa.SYMBOLS)
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True, text=True)
    exported = {l.split()[-1] for l in out.stdout.splitlines() if " T " in l}
    assert set(names) <= exported
    # nothing else of the library's own leaks out under the fa_ prefix
    assert {e for e in exported if e.startswith("fa_")} == set(names)


def test_no_unresolved_library_symbols():
    """Every kernel launch stub the library references is defined in it (a
    missing stub only shows up when the library is loaded)."""
    out = subprocess.run(["nm", "-D", "--undefined-only", fa.LIB_PATH], capture_output=True, text=True)
    own = [l for l in out.stdout.splitlines() if "_ZN2fa" in l or "device_stub" in l]
    assert own == []


def test_abi_version_and_strings(L):
    with open(os.path.join(ROOT, "include", "fa.h")) as f:
        declared = int(re.search(r"#define FA_ABI_VERSION (\d+)", f.read()).group(1))
    assert L.fa_abi_version() == declared == 10
    for st in range(6):
        assert L.fa_status_string(st)
    assert L.fa_status_string(0) == b"ok"


STRUCTS = {
    "fa_fwd_args": fa.FwdArgs,
    "fa_fwd_varlen_args": fa.FwdVarlenArgs,
    "fa_fwd_paged_args": fa.FwdPagedArgs,
    "fa_fwd_fp8_args": fa.FwdFp8Args,
    "fa_decode_paged_args": fa.DecodePagedArgs,
    "fa_dropout_args": fa.DropoutArgs,
    "fa_fwd_varlen_fp8_args": fa.FwdVarlenFp8Args,
    "fa_decode_paged_fp8_args": fa.DecodePagedFp8Args,
    "fa_fwd_paged_fp8_args": fa.FwdPagedFp8Args,
    "fa_merge_states_args": fa.MergeStatesArgs,
}


def test_struct_layout_matches_header(tmp_path):
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "fa.h"', "int main(void) {"]
    for cname, py in STRUCTS.items():
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines += ["return 0; }"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    got = {}
    for line in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.splitlines():
        s, f, v = line.split()
        got[(s, f)] = int(v)
    for cname, py in STRUCTS.items():
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert got[(cname, f)] == getattr(py, f).offset, (cname, f)


def fwd_args(**kw):
    a = fa.FwdArgs()
    a.batch, a.seqlen_q, a.seqlen_k, a.heads_q, a.heads_kv, a.head_dim = 1, 8, 8, 2, 2, 64
    a.dtype, a.scale, a.causal = fa.FA_BF16, 0.125, 1
    a.q = a.k = a.v = a.o = 0x1000
    for arr in (a.q_stride, a.k_stride, a.v_stride, a.o_stride):
        arr[:] = [8 * 2 * 64, 2 * 64, 64]
    for k, v in kw.items():
        if k.endswith("_stride"):
            getattr(a, k)[:] = v
        else:
            setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(heads_q=3), fa.FA_ERR_BAD_SHAPE),
    (dict(heads_kv=0), fa.FA_ERR_BAD_SHAPE),
    (dict(batch=-1), fa.FA_ERR_BAD_SHAPE),
    (dict(seqlen_k=-2), fa.FA_ERR_BAD_SHAPE),
    (dict(head_dim=96), fa.FA_ERR_UNSUPPORTED),
    (dict(head_dim=256, dtype=fa.FA_F32), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=7), fa.FA_ERR_UNSUPPORTED),
    (dict(scale=0.0), fa.FA_ERR_BAD_SHAPE),
    (dict(scale=float("nan")), fa.FA_ERR_BAD_SHAPE),
    (dict(q=None), fa.FA_ERR_NULL_POINTER),
    (dict(o=None), fa.FA_ERR_NULL_POINTER),
    (dict(q=0x1002), fa.FA_ERR_BAD_SHAPE),
    (dict(k_stride=[1024, 129, 64]), fa.FA_ERR_BAD_SHAPE),
    (dict(v_stride=[1024, -128, 64]), fa.FA_ERR_BAD_SHAPE),
    (dict(k_stride=[1 << 30, (1 << 24) + 8, 64]), fa.FA_ERR_UNSUPPORTED),
])
def test_fwd_rejects_before_launch(L, kw, status):
    a = fwd_args(**kw)
    assert L.fa_fwd(ctypes.byref(a), None) == status
    assert L.fa_last_error()


def test_fwd_empty_is_noop(L):
    for kw in (dict(batch=0), dict(seqlen_q=0)):
        a = fwd_args(q=None, k=None, v=None, o=None, **kw)
        assert L.fa_fwd(ctypes.byref(a), None) == fa.FA_OK
        assert L.fa_last_error() == b""
    assert L.fa_fwd(None, None) == fa.FA_ERR_NULL_POINTER


def fp8_args(**kw):
    a = fa.FwdFp8Args()
    a.batch, a.seqlen_q, a.seqlen_k, a.heads_q, a.heads_kv, a.head_dim = 1, 8, 8, 2, 2, 128
    a.q_descale = a.k_descale = a.v_descale = 0.01
    a.scale, a.causal = 0.088, 1
    a.q = a.k = a.v = a.o = 0x1000
    for arr in (a.q_stride, a.k_stride, a.v_stride):
        arr[:] = [8 * 2 * 128, 2 * 128, 128]
    a.o_stride[:] = [8 * 2 * 128, 2 * 128, 128]
    for k, v in kw.items():
        if k.endswith("_stride"):
            getattr(a, k)[:] = v
        else:
            setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(heads_q=3), fa.FA_ERR_BAD_SHAPE),
    (dict(head_dim=64), fa.FA_ERR_UNSUPPORTED),
    (dict(q_descale=0.0), fa.FA_ERR_BAD_SHAPE),
    (dict(v_descale=float("inf")), fa.FA_ERR_BAD_SHAPE),
    (dict(scale=-1.0), fa.FA_ERR_BAD_SHAPE),
    (dict(q=None), fa.FA_ERR_NULL_POINTER),
    (dict(k=None), fa.FA_ERR_NULL_POINTER),
    (dict(q_stride=[2048, 264, 8]), fa.FA_ERR_BAD_SHAPE),   # 8-byte q stride
    (dict(o_stride=[2048, 260, 128]), fa.FA_ERR_BAD_SHAPE),
    (dict(v=0x1008), fa.FA_ERR_BAD_SHAPE),
    (dict(k_stride=[1 << 30, (1 << 24) + 16, 128]), fa.FA_ERR_UNSUPPORTED),
])
def test_fp8_rejects_before_launch(L, kw, status):
    a = fp8_args(**kw)
    assert L.fa_fwd_fp8(ctypes.byref(a), None) == status
    assert L.fa_last_error()


def test_fp8_empty_is_noop(L):
    for kw in (dict(batch=0), dict(seqlen_q=0)):
        a = fp8_args(q=None, k=None, v=None, o=None, **kw)
        assert L.fa_fwd_fp8(ctypes.byref(a), None) == fa.FA_OK


def dropout_args(p=0.1, seed=1, offset=0):
    d = fa.DropoutArgs()
    d.p, d.seed, d.offset = p, seed, offset
    return d


@pytest.mark.parametrize("dkw,kw,status", [
    (dict(p=-0.1), {}, fa.FA_ERR_BAD_SHAPE),
    (dict(p=1.0), {}, fa.FA_ERR_BAD_SHAPE),
    (dict(p=float("nan")), {}, fa.FA_ERR_BAD_SHAPE),
    (dict(p=255.5 / 256), {}, fa.FA_ERR_BAD_SHAPE),       # rounds to t = 256
    (dict(p=0.3), dict(dtype=fa.FA_F32), fa.FA_ERR_UNSUPPORTED),
    (dict(p=0.3), dict(heads_q=3, heads_kv=2), fa.FA_ERR_BAD_SHAPE),
    (dict(p=0.3), dict(q=None), fa.FA_ERR_NULL_POINTER),
])
def test_dropout_rejects_before_launch(L, dkw, kw, status):
    a, d = fwd_args(**kw), dropout_args(**dkw)
    assert L.fa_fwd_dropout(ctypes.byref(a), ctypes.byref(d), None) == status
    assert L.fa_last_error()
    v = varlen_args(**kw)
    assert L.fa_fwd_varlen_dropout(ctypes.byref(v), ctypes.byref(d), None) == status
    assert L.fa_last_error()


def test_dropout_null_and_noop(L):
    a, v = fwd_args(), varlen_args()
    assert L.fa_fwd_dropout(ctypes.byref(a), None, None) == fa.FA_ERR_NULL_POINTER
    assert L.fa_fwd_varlen_dropout(ctypes.byref(v), None, None) == fa.FA_ERR_NULL_POINTER
    d = dropout_args(p=0.5)
    e = fwd_args(q=None, k=None, v=None, o=None, batch=0)
    assert L.fa_fwd_dropout(ctypes.byref(e), ctypes.byref(d), None) == fa.FA_OK
    # p rounding to t = 0 is plain attention, allowed for fp32 too
    e = fwd_args(q=None, k=None, v=None, o=None, batch=0, dtype=fa.FA_F32)
    assert L.fa_fwd_dropout(ctypes.byref(e), ctypes.byref(dropout_args(p=0.5 / 256)), None) == fa.FA_OK


def varlen_fp8_args(**kw):
    a = fa.FwdVarlenFp8Args()
    a.num_seqs, a.total_tokens, a.max_seqlen, a.heads_q, a.heads_kv, a.head_dim = 2, 10, 6, 2, 1, 128
    a.q_descale = a.k_descale = a.v_descale = 0.01
    a.scale, a.causal = 0.088, 1
    a.q = a.k = a.v = a.o = a.cu_seqlens = 0x1000
    a.q_stride[:] = [2 * 128, 128]
    a.o_stride[:] = [2 * 128, 128]
    a.k_stride[:] = a.v_stride[:] = [128, 128]
    for k, v in kw.items():
        if k.endswith("_stride"):
            getattr(a, k)[:] = v
        else:
            setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(heads_q=3, heads_kv=2), fa.FA_ERR_BAD_SHAPE),
    (dict(num_seqs=-1), fa.FA_ERR_BAD_SHAPE),
    (dict(head_dim=64), fa.FA_ERR_UNSUPPORTED),
    (dict(k_descale=0.0), fa.FA_ERR_BAD_SHAPE),
    (dict(v_descale=float("nan")), fa.FA_ERR_BAD_SHAPE),
    (dict(cu_seqlens=None), fa.FA_ERR_NULL_POINTER),
    (dict(q_stride=[264, 8]), fa.FA_ERR_BAD_SHAPE),
    (dict(o=0x1008), fa.FA_ERR_BAD_SHAPE),
    (dict(k_stride=[(1 << 24) + 16, 128]), fa.FA_ERR_UNSUPPORTED),
])
def test_varlen_fp8_rejects_before_launch(L, kw, status):
    a = varlen_fp8_args(**kw)
    assert L.fa_fwd_varlen_fp8(ctypes.byref(a), None) == status
    assert L.fa_last_error()


def test_varlen_fp8_empty_is_noop(L):
    for kw in (dict(num_seqs=0), dict(max_seqlen=0), dict(total_tokens=0)):
        a = varlen_fp8_args(q=None, k=None, v=None, o=None, cu_seqlens=None, **kw)
        assert L.fa_fwd_varlen_fp8(ctypes.byref(a), None) == fa.FA_OK


def varlen_args(**kw):
    a = fa.FwdVarlenArgs()
    a.num_seqs, a.total_tokens, a.max_seqlen, a.heads_q, a.heads_kv, a.head_dim = 2, 10, 6, 2, 1, 64
    a.dtype, a.scale, a.causal = fa.FA_BF16, 0.125, 1
    a.q = a.k = a.v = a.o = a.cu_seqlens = 0x1000
    for arr in (a.q_stride, a.o_stride):
        arr[:] = [2 * 64, 64]
    for arr in (a.k_stride, a.v_stride):
        arr[:] = [64, 64]
    for k, v in kw.items():
        if k.endswith("_stride"):
            getattr(a, k)[:] = v
        else:
            setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(heads_q=3, heads_kv=2), fa.FA_ERR_BAD_SHAPE),
    (dict(num_seqs=-1), fa.FA_ERR_BAD_SHAPE),
    (dict(head_dim=32), fa.FA_ERR_UNSUPPORTED),
    (dict(cu_seqlens=None), fa.FA_ERR_NULL_POINTER),
    (dict(q_stride=[100, 64]), fa.FA_ERR_BAD_SHAPE),
    (dict(o=0x1008), fa.FA_ERR_BAD_SHAPE),
    (dict(v_stride=[(1 << 24) + 8, 64]), fa.FA_ERR_UNSUPPORTED),
])
def test_varlen_rejects_before_launch(L, kw, status):
    a = varlen_args(**kw)
    assert L.fa_fwd_varlen(ctypes.byref(a), None) == status


def test_varlen_empty_is_noop(L):
    for kw in (dict(num_seqs=0), dict(max_seqlen=0), dict(total_tokens=0)):
        a = varlen_args(q=None, k=None, v=None, o=None, cu_seqlens=None, **kw)
        assert L.fa_fwd_varlen(ctypes.byref(a), None) == fa.FA_OK


def paged_args(**kw):
    a = fa.FwdPagedArgs()
    a.num_seqs, a.total_q, a.max_seqlen_q, a.max_seqlen_k = 3, 40, 20, 300
    a.heads_q, a.heads_kv, a.head_dim, a.block_size = 8, 2, 128, 16
    a.max_blocks_per_seq, a.num_blocks = 20, 64
    a.scale, a.causal = 0.088, 1
    a.q = a.k_pool = a.v_pool = a.block_table = a.cu_seqlens_q = a.seq_lens_k = a.o = 0x1000
    a.pool_stride[:] = [2 * 16 * 128, 16 * 128, 128]
    a.q_stride[:] = [8 * 128, 128]
    a.o_stride[:] = [8 * 128, 128]
    for k, v in kw.items():
        if k.endswith("_stride"):
            getattr(a, k)[:] = v
        else:
            setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(heads_q=7), fa.FA_ERR_BAD_SHAPE),
    (dict(total_q=-1), fa.FA_ERR_BAD_SHAPE),
    (dict(head_dim=96), fa.FA_ERR_UNSUPPORTED),
    (dict(block_size=32), fa.FA_ERR_UNSUPPORTED),
    (dict(max_seqlen_k=20 * 16 + 1), fa.FA_ERR_BAD_SHAPE),
    (dict(scale=-1.0), fa.FA_ERR_BAD_SHAPE),
    (dict(cu_seqlens_q=None), fa.FA_ERR_NULL_POINTER),
    (dict(seq_lens_k=None), fa.FA_ERR_NULL_POINTER),
    (dict(block_table=None), fa.FA_ERR_NULL_POINTER),
    (dict(k_pool=None), fa.FA_ERR_NULL_POINTER),
    (dict(q_stride=[8 * 128, 100]), fa.FA_ERR_BAD_SHAPE),
    (dict(o=0x1004), fa.FA_ERR_BAD_SHAPE),
    (dict(pool_stride=[1 << 40, 16 * 128, (1 << 24) + 8]), fa.FA_ERR_UNSUPPORTED),
])
def test_paged_prefill_rejects_before_launch(L, kw, status):
    a = paged_args(**kw)
    assert L.fa_fwd_paged(ctypes.byref(a), None) == status
    assert L.fa_last_error()


@pytest.mark.parametrize("kw,dkw,status", [
    (dict(head_dim=64), {}, fa.FA_ERR_UNSUPPORTED),
    (dict(), dict(q_descale=0.0), fa.FA_ERR_BAD_SHAPE),
    (dict(), dict(v_descale=float("nan")), fa.FA_ERR_BAD_SHAPE),
    (dict(q_stride=[8 * 128 + 8, 128]), {}, fa.FA_ERR_BAD_SHAPE),   # 8-byte multiple, not 16
    (dict(heads_q=3), {}, fa.FA_ERR_BAD_SHAPE),
    (dict(q=None), {}, fa.FA_ERR_NULL_POINTER),
])
def test_paged_prefill_fp8_rejects_before_launch(L, kw, dkw, status):
    a = fa.FwdPagedFp8Args()
    a.base = paged_args(**kw)
    a.q_descale = a.k_descale = a.v_descale = 0.01
    for k, v in dkw.items():
        setattr(a, k, v)
    assert L.fa_fwd_paged_fp8(ctypes.byref(a), None) == status
    assert L.fa_last_error()
    assert L.fa_fwd_paged_fp8(None, None) == fa.FA_ERR_NULL_POINTER


def test_paged_prefill_empty_is_noop(L):
    for kw in (dict(num_seqs=0), dict(max_seqlen_q=0), dict(total_q=0)):
        a = paged_args(q=None, k_pool=None, v_pool=None, block_table=None, cu_seqlens_q=None,
                       seq_lens_k=None, o=None, **kw)
        assert L.fa_fwd_paged(ctypes.byref(a), None) == fa.FA_OK
    assert L.fa_fwd_paged(None, None) == fa.FA_ERR_NULL_POINTER


def decode_args(**kw):
    a = fa.DecodePagedArgs()
    a.batch, a.heads_q, a.heads_kv, a.head_dim, a.block_size = 4, 32, 8, 128, 16
    a.max_blocks_per_seq, a.num_blocks, a.max_seq_len = 64, 200, 1000
    a.scale, a.num_splits = 0.088, 0
    a.q = a.k_pool = a.v_pool = a.block_table = a.seq_lens = a.o = a.workspace = 0x1000
    a.pool_stride[:] = [8 * 16 * 128, 16 * 128, 128]
    a.q_stride[:] = [32 * 128, 128]
    a.o_stride[:] = [32 * 128, 128]
    for k, v in kw.items():
        if k.endswith("_stride"):
            getattr(a, k)[:] = v
        else:
            setattr(a, k, v)
    if "workspace_bytes" not in kw:
        a.workspace_bytes = 0
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(heads_q=30), fa.FA_ERR_BAD_SHAPE),
    (dict(heads_kv=1), fa.FA_ERR_UNSUPPORTED),   # group 32 > 16
    (dict(pool_stride=[8 * 16 * 128, 16 * 128, (1 << 26) + 8]), fa.FA_ERR_UNSUPPORTED),
    (dict(head_dim=96), fa.FA_ERR_UNSUPPORTED),
    (dict(block_size=32), fa.FA_ERR_UNSUPPORTED),
    (dict(max_seq_len=64 * 16 + 1), fa.FA_ERR_BAD_SHAPE),
    (dict(batch=-3), fa.FA_ERR_BAD_SHAPE),
    (dict(num_splits=-1), fa.FA_ERR_BAD_SHAPE),
    (dict(block_table=None), fa.FA_ERR_NULL_POINTER),
    (dict(workspace=None), fa.FA_ERR_NULL_POINTER),
    (dict(pool_stride=[8 * 16 * 128, 16 * 128, 100]), fa.FA_ERR_BAD_SHAPE),
    (dict(v_pool=0x1010 + 4), fa.FA_ERR_BAD_SHAPE),
    (dict(), fa.FA_ERR_WORKSPACE_TOO_SMALL),
])
def test_decode_rejects_before_launch(L, kw, status):
    a = decode_args(**kw)
    assert L.fa_decode_paged(ctypes.byref(a), None) == status
    assert L.fa_last_error()


@pytest.mark.parametrize("kw,dkw,status", [
    (dict(), dict(k_descale=0.0), fa.FA_ERR_BAD_SHAPE),
    (dict(), dict(v_descale=float("inf")), fa.FA_ERR_BAD_SHAPE),
    (dict(pool_stride=[8 * 16 * 128, 16 * 128, 120]), {}, fa.FA_ERR_BAD_SHAPE),   # 120-byte token stride
    (dict(head_dim=96), {}, fa.FA_ERR_UNSUPPORTED),
    (dict(heads_q=30), {}, fa.FA_ERR_BAD_SHAPE),
    (dict(workspace=None), {}, fa.FA_ERR_NULL_POINTER),
    (dict(), {}, fa.FA_ERR_WORKSPACE_TOO_SMALL),
])
def test_decode_fp8_rejects_before_launch(L, kw, dkw, status):
    a = fa.DecodePagedFp8Args()
    a.base = decode_args(**kw)
    a.k_descale, a.v_descale = 0.01, 0.02
    for k, v in dkw.items():
        setattr(a, k, v)
    assert L.fa_decode_paged_fp8(ctypes.byref(a), None) == status
    assert L.fa_last_error()
    assert L.fa_decode_paged_fp8(None, None) == fa.FA_ERR_NULL_POINTER


def test_decode_fp8_sizes(L):
    a = fa.DecodePagedFp8Args()
    a.base = decode_args(num_splits=6)
    a.k_descale, a.v_descale = 0.01, 0.02
    assert L.fa_decode_paged_fp8_num_splits(ctypes.byref(a)) == 6
    assert L.fa_decode_paged_fp8_workspace_size(ctypes.byref(a)) == 32 * (6 + 4) * (128 + 4) * 4
    # automatic: twelve wave slots per CU (three per SIMD) for FP8 pools,
    # still capped at about one part per 4 blocks of the largest batch
    a.base = decode_args(max_seq_len=64 * 16, max_blocks_per_seq=64, batch=64)
    ns8 = L.fa_decode_paged_fp8_num_splits(ctypes.byref(a))
    ns16 = L.fa_decode_paged_num_splits(ctypes.byref(a.base))
    assert ns8 >= ns16 and 1 <= ns8 <= 64 * 64 // 4
    assert L.fa_decode_paged_fp8_num_splits(None) == 0
    assert L.fa_decode_paged_fp8_workspace_size(None) == 0


def test_decode_workspace_scales_with_head_dim(L):
    for d in (64, 128, 256):
        a = decode_args(num_splits=5, head_dim=d)
        assert L.fa_decode_paged_workspace_size(ctypes.byref(a)) == 32 * (5 + 4) * (d + 4) * 4


def test_decode_sizes(L):
    # Explicit num_splits: that many parts of the concatenated block list per
    # kv head; the workspace holds (parts + batch) slots of 128 + 4 floats
    # per query head.
    a = decode_args(num_splits=4)
    assert L.fa_decode_paged_num_splits(ctypes.byref(a)) == 4
    assert L.fa_decode_paged_workspace_size(ctypes.byref(a)) == 32 * (4 + 4) * (128 + 4) * 4
    a = decode_args(num_splits=7)
    assert L.fa_decode_paged_num_splits(ctypes.byref(a)) == 7
    # Automatic: one part per wave slot (8 per CU) spread over the 8 kv
    # heads, at most about one part per 4 blocks of the largest batch
    # (4 sequences x ceil(1000 / 16) = 252 blocks -> 63).
    a = decode_args()
    ns = L.fa_decode_paged_num_splits(ctypes.byref(a))
    assert ns == 63
    assert L.fa_decode_paged_workspace_size(ctypes.byref(a)) == 32 * (63 + 4) * (128 + 4) * 4
    a = decode_args(max_seq_len=64 * 16, max_blocks_per_seq=64, batch=64)
    ns = L.fa_decode_paged_num_splits(ctypes.byref(a))
    assert 1 <= ns <= 64 * 64 // 4
    bad = decode_args(head_dim=96)
    assert L.fa_decode_paged_workspace_size(ctypes.byref(bad)) == 0
    assert L.fa_decode_paged_num_splits(ctypes.byref(bad)) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(heads_q=30), fa.FA_ERR_BAD_SHAPE),
    (dict(head_dim=96), fa.FA_ERR_UNSUPPORTED),
    (dict(block_table=None), fa.FA_ERR_NULL_POINTER),
    (dict(o=None), fa.FA_ERR_NULL_POINTER),
    # 64 sequences x 32 heads x (1000 + 64) slots x 132 floats: 36 MB > 16 MiB
    (dict(num_splits=1000, batch=64, max_seq_len=64 * 16), fa.FA_ERR_WORKSPACE_TOO_SMALL),
])
def test_decode_noalloc_rejects_before_launch(L, kw, status):
    a = decode_args(**kw)
    a.workspace, a.workspace_bytes = None, 0
    assert L.fa_decode_paged_noalloc(ctypes.byref(a), None) == status
    assert L.fa_last_error()


def test_decode_noalloc_limit(L):
    assert L.fa_decode_paged_noalloc_max_bytes() == 16 << 20
    # the batch-64 decode workload with its automatic split fits
    a = decode_args(batch=64, max_seq_len=32768, max_blocks_per_seq=2048)
    assert 0 < L.fa_decode_paged_workspace_size(ctypes.byref(a)) <= L.fa_decode_paged_noalloc_max_bytes()


def test_decode_empty_batch_is_noop(L):
    a = decode_args(batch=0, q=None, k_pool=None, v_pool=None, block_table=None, seq_lens=None,
                    o=None, workspace=None)
    assert L.fa_decode_paged(ctypes.byref(a), None) == fa.FA_OK


def test_binding_refuses_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(fa, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        fa.lib(str(tmp_path / "missing.so"))


def merge_args(**kw):
    d = dict(num_parts=2, batch=1, seqlen=5, heads=3, head_dim=128, dtype=fa.FA_BF16, o_parts=0x1000,
             lse_parts=0x2000, o=0x3000, lse=0x4000)
    d.update(kw)
    return fa.MergeStatesArgs(*(d[f] for f, _ in fa.MergeStatesArgs._fields_))


@pytest.mark.parametrize("kw,status", [
    (dict(num_parts=0), fa.FA_ERR_BAD_SHAPE),
    (dict(batch=-1), fa.FA_ERR_BAD_SHAPE),
    (dict(heads=-2), fa.FA_ERR_BAD_SHAPE),
    (dict(head_dim=96), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=7), fa.FA_ERR_UNSUPPORTED),
    (dict(o_parts=None), fa.FA_ERR_NULL_POINTER),
    (dict(lse_parts=None), fa.FA_ERR_NULL_POINTER),
    (dict(o=None), fa.FA_ERR_NULL_POINTER),
    (dict(o=0x3008), fa.FA_ERR_BAD_SHAPE),
    (dict(lse=0x4004), fa.FA_ERR_BAD_SHAPE),
    (dict(num_parts=1 << 20, batch=1 << 10, seqlen=1 << 10), fa.FA_ERR_UNSUPPORTED),
    (dict(num_parts=1, batch=1 << 10, seqlen=1 << 13, heads=1 << 4), fa.FA_ERR_UNSUPPORTED),  # 2^34 per part
])
def test_merge_rejects_before_launch(L, kw, status):
    a = merge_args(**kw)
    assert L.fa_merge_states(ctypes.byref(a), None) == status
    assert L.fa_last_error()


def test_merge_empty_is_noop(L):
    for kw in (dict(batch=0), dict(seqlen=0), dict(heads=0)):
        a = merge_args(o_parts=None, lse_parts=None, o=None, lse=None, **kw)
        assert L.fa_merge_states(ctypes.byref(a), None) == fa.FA_OK
        assert L.fa_last_error() == b""
    assert L.fa_merge_states(None, None) == fa.FA_ERR_NULL_POINTER
