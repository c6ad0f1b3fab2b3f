"""Thin ctypes binding over libfa_gfx950.so (declared in include/fa.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of the attention runs in the library's kernels.  There is
no fallback -- if the library is missing or a call is rejected, an exception
is raised.

Layouts (see include/fa.h):
    fa_fwd:          q [B, Nq, Hq, d], k/v [B, Nk, Hkv, d] -> o like q, lse [B, Hq, Nq]
    fa_fwd_fp8:      as fa_fwd with uint8 E4M3 q/k/v and per-tensor descale factors -> o bf16
    fa_fwd_varlen:   q [T, Hq, d], k/v [T, Hkv, d], cu_seqlens int32 [S+1] -> o, lse [Hq, T]
    fa_fwd_varlen_fp8: as fa_fwd_varlen with uint8 E4M3 q/k/v and descale factors -> o bf16
    fa_fwd_dropout, fa_fwd_varlen_dropout: as fa_fwd / fa_fwd_varlen (bf16) with dropout
                     of the weights drawn from (dropout_p, seed, offset)
    fa_fwd_paged:    q [Tq, Hq, d] (chunks packed by cu_seqlens_q int32 [S+1]), pools and
                     block_table as for decode, seq_lens_k int32 [S] -> o like q, lse [Hq, Tq]
    fa_decode_paged_fp8: as fa_decode_paged with uint8 E4M3 pools and (k, v) descale factors
    fa_decode_paged: q [B, Hq, d], pools [blocks, Hkv, 16, d] (or any strides with d
                     contiguous), block_table int32 [B, max_blocks], seq_lens int32 [B]
                     -> o [B, Hq, d], lse [B, Hq]
"""
from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfa_gfx950.so")

FA_OK, FA_ERR_NULL_POINTER, FA_ERR_BAD_SHAPE, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE_TOO_SMALL, FA_ERR_HIP = range(6)
FA_F32, FA_BF16 = 0, 1

_P, _I32, _I64, _F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float


class FwdArgs(ctypes.Structure):
    _fields_ = [("q", _P), ("k", _P), ("v", _P), ("o", _P), ("lse", _P),
                ("batch", _I32), ("seqlen_q", _I32), ("seqlen_k", _I32), ("heads_q", _I32),
                ("heads_kv", _I32), ("head_dim", _I32),
                ("q_stride", _I64 * 3), ("k_stride", _I64 * 3), ("v_stride", _I64 * 3),
                ("o_stride", _I64 * 3),
                ("dtype", ctypes.c_int), ("scale", _F), ("causal", _I32)]


class FwdFp8Args(ctypes.Structure):
    _fields_ = [("q", _P), ("k", _P), ("v", _P), ("o", _P), ("lse", _P),
                ("batch", _I32), ("seqlen_q", _I32), ("seqlen_k", _I32), ("heads_q", _I32),
                ("heads_kv", _I32), ("head_dim", _I32),
                ("q_stride", _I64 * 3), ("k_stride", _I64 * 3), ("v_stride", _I64 * 3),
                ("o_stride", _I64 * 3),
                ("q_descale", _F), ("k_descale", _F), ("v_descale", _F), ("scale", _F), ("causal", _I32)]


class FwdVarlenArgs(ctypes.Structure):
    _fields_ = [("q", _P), ("k", _P), ("v", _P), ("o", _P), ("lse", _P), ("cu_seqlens", _P),
                ("num_seqs", _I32), ("total_tokens", _I32), ("max_seqlen", _I32), ("heads_q", _I32),
                ("heads_kv", _I32), ("head_dim", _I32),
                ("q_stride", _I64 * 2), ("k_stride", _I64 * 2), ("v_stride", _I64 * 2),
                ("o_stride", _I64 * 2),
                ("dtype", ctypes.c_int), ("scale", _F), ("causal", _I32)]


class FwdVarlenFp8Args(ctypes.Structure):
    _fields_ = [("q", _P), ("k", _P), ("v", _P), ("o", _P), ("lse", _P), ("cu_seqlens", _P),
                ("num_seqs", _I32), ("total_tokens", _I32), ("max_seqlen", _I32), ("heads_q", _I32),
                ("heads_kv", _I32), ("head_dim", _I32),
                ("q_stride", _I64 * 2), ("k_stride", _I64 * 2), ("v_stride", _I64 * 2),
                ("o_stride", _I64 * 2),
                ("q_descale", _F), ("k_descale", _F), ("v_descale", _F), ("scale", _F), ("causal", _I32)]


class DropoutArgs(ctypes.Structure):
    _fields_ = [("p", ctypes.c_double), ("seed", ctypes.c_uint64), ("offset", ctypes.c_uint32)]


class DecodePagedArgs(ctypes.Structure):
    _fields_ = [("q", _P), ("k_pool", _P), ("v_pool", _P), ("pool_stride", _I64 * 3),
                ("block_table", _P), ("seq_lens", _P), ("o", _P), ("lse", _P),
                ("q_stride", _I64 * 2), ("o_stride", _I64 * 2),
                ("batch", _I32), ("heads_q", _I32), ("heads_kv", _I32), ("head_dim", _I32),
                ("block_size", _I32), ("max_blocks_per_seq", _I32), ("num_blocks", _I32),
                ("max_seq_len", _I32), ("scale", _F), ("num_splits", _I32),
                ("workspace", _P), ("workspace_bytes", ctypes.c_size_t)]


class DecodePagedFp8Args(ctypes.Structure):
    _fields_ = [("base", DecodePagedArgs), ("k_descale", _F), ("v_descale", _F)]


class FwdPagedArgs(ctypes.Structure):
    _fields_ = [("q", _P), ("k_pool", _P), ("v_pool", _P), ("pool_stride", _I64 * 3),
                ("block_table", _P), ("cu_seqlens_q", _P), ("seq_lens_k", _P), ("o", _P), ("lse", _P),
                ("q_stride", _I64 * 2), ("o_stride", _I64 * 2),
                ("num_seqs", _I32), ("total_q", _I32), ("max_seqlen_q", _I32), ("max_seqlen_k", _I32),
                ("heads_q", _I32), ("heads_kv", _I32), ("head_dim", _I32), ("block_size", _I32),
                ("max_blocks_per_seq", _I32), ("num_blocks", _I32), ("scale", _F), ("causal", _I32)]


class FwdPagedFp8Args(ctypes.Structure):
    _fields_ = [("base", FwdPagedArgs), ("q_descale", _F), ("k_descale", _F), ("v_descale", _F)]


class MergeStatesArgs(ctypes.Structure):
    _fields_ = [("num_parts", _I32), ("batch", _I32), ("seqlen", _I32), ("heads", _I32), ("head_dim", _I32),
                ("dtype", ctypes.c_int), ("o_parts", _P), ("lse_parts", _P), ("o", _P), ("lse", _P)]


SYMBOLS = ("fa_fwd", "fa_fwd_dropout", "fa_fwd_fp8", "fa_fwd_varlen", "fa_fwd_varlen_dropout", "fa_fwd_varlen_fp8", "fa_fwd_paged", "fa_fwd_paged_fp8", "fa_decode_paged", "fa_decode_paged_workspace_size",
           "fa_decode_paged_num_splits", "fa_decode_paged_fp8", "fa_decode_paged_fp8_workspace_size",
           "fa_decode_paged_fp8_num_splits", "fa_decode_paged_noalloc", "fa_decode_paged_noalloc_max_bytes",
           "fa_merge_states", "fa_status_string", "fa_last_error", "fa_abi_version")

_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{detail} (status {status})")
        self.status = status


def lib(path: str = LIB_PATH):
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    _lib = load(path)
    return _lib


def load(path: str):
    """Load a build of the library from ``path`` with the argument types set
    (``lib()`` caches the product; tests load other builds with this)."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m exact_io_aware_tile_amd.build`")
    L = ctypes.CDLL(path)
    L.fa_fwd.argtypes = [ctypes.POINTER(FwdArgs), _P]
    L.fa_fwd.restype = ctypes.c_int
    L.fa_fwd_fp8.argtypes = [ctypes.POINTER(FwdFp8Args), _P]
    L.fa_fwd_fp8.restype = ctypes.c_int
    L.fa_fwd_varlen.argtypes = [ctypes.POINTER(FwdVarlenArgs), _P]
    L.fa_fwd_varlen.restype = ctypes.c_int
    L.fa_fwd_varlen_fp8.argtypes = [ctypes.POINTER(FwdVarlenFp8Args), _P]
    L.fa_fwd_varlen_fp8.restype = ctypes.c_int
    L.fa_fwd_dropout.argtypes = [ctypes.POINTER(FwdArgs), ctypes.POINTER(DropoutArgs), _P]
    L.fa_fwd_dropout.restype = ctypes.c_int
    L.fa_fwd_varlen_dropout.argtypes = [ctypes.POINTER(FwdVarlenArgs), ctypes.POINTER(DropoutArgs), _P]
    L.fa_fwd_varlen_dropout.restype = ctypes.c_int
    L.fa_fwd_paged.argtypes = [ctypes.POINTER(FwdPagedArgs), _P]
    L.fa_fwd_paged.restype = ctypes.c_int
    L.fa_decode_paged.argtypes = [ctypes.POINTER(DecodePagedArgs), _P]
    L.fa_decode_paged.restype = ctypes.c_int
    L.fa_decode_paged_noalloc.argtypes = [ctypes.POINTER(DecodePagedArgs), _P]
    L.fa_decode_paged_noalloc.restype = ctypes.c_int
    L.fa_decode_paged_noalloc_max_bytes.argtypes = []
    L.fa_decode_paged_noalloc_max_bytes.restype = ctypes.c_size_t
    L.fa_fwd_paged_fp8.argtypes = [ctypes.POINTER(FwdPagedFp8Args), _P]
    L.fa_fwd_paged_fp8.restype = ctypes.c_int
    L.fa_decode_paged_fp8.argtypes = [ctypes.POINTER(DecodePagedFp8Args), _P]
    L.fa_decode_paged_fp8.restype = ctypes.c_int
    L.fa_decode_paged_fp8_workspace_size.argtypes = [ctypes.POINTER(DecodePagedFp8Args)]
    L.fa_decode_paged_fp8_workspace_size.restype = ctypes.c_size_t
    L.fa_decode_paged_fp8_num_splits.argtypes = [ctypes.POINTER(DecodePagedFp8Args)]
    L.fa_decode_paged_fp8_num_splits.restype = _I32
    L.fa_decode_paged_workspace_size.argtypes = [ctypes.POINTER(DecodePagedArgs)]
    L.fa_decode_paged_workspace_size.restype = ctypes.c_size_t
    L.fa_decode_paged_num_splits.argtypes = [ctypes.POINTER(DecodePagedArgs)]
    L.fa_decode_paged_num_splits.restype = _I32
    L.fa_merge_states.argtypes = [ctypes.POINTER(MergeStatesArgs), _P]
    L.fa_merge_states.restype = ctypes.c_int
    L.fa_status_string.argtypes = [ctypes.c_int]
    L.fa_status_string.restype = ctypes.c_char_p
    L.fa_last_error.argtypes = []
    L.fa_last_error.restype = ctypes.c_char_p
    L.fa_abi_version.argtypes = []
    L.fa_abi_version.restype = _I32
    return L


def _check(status: int) -> None:
    if status != FA_OK:
        L = lib()
        raise FAError(status, f"{L.fa_status_string(status).decode()}: {L.fa_last_error().decode()}")


# ---------------------------------------------------------------------------
# torch marshalling helpers (torch is only memory + streams here)
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return FA_F32
    if t.dtype == torch.bfloat16:
        return FA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use torch.float32 or torch.bfloat16")


def _dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
    _same_device(*ts)
    for t in ts:
        if t is not None and t.dim() > 0 and t.stride(-1) != 1:
            raise ValueError("the last dimension must be contiguous")


def _need(t, name, shape=None, dtype=None, contiguous=False, optional=False):
    """Reject a tensor whose shape, dtype or layout disagrees with the call:
    the library trusts the sizes it is given, so a short output or a
    mismatched operand would be read or written out of bounds."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ndim(t, name, n):
    if t is None or t.dim() != n:
        raise ValueError(f"{name} must be a {n}-D tensor")


def _same_device(*ts):
    ref = next(t for t in ts if t is not None)
    for t in ts:
        if t is not None and t.device != ref.device:
            raise ValueError(f"all tensors must be on {ref.device}, got one on {t.device}")


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dropout_args(dropout_p, seed, offset):
    d = DropoutArgs()
    d.p = float(dropout_p)
    d.seed = int(seed) & (2**64 - 1)
    d.offset = int(offset) & (2**32 - 1)
    return d


def fa_fwd(q, k, v, *, causal: bool = False, scale: float | None = None, out=None, lse=None,
           return_lse: bool = True, stream=None):
    """Dense attention.  Returns (o, lse) (lse is None when return_lse is False)."""
    a, out, lse = _fwd_args(q, k, v, causal, scale, out, lse, return_lse)
    _check(lib().fa_fwd(ctypes.byref(a), _stream(stream)))
    return out, lse


def fa_fwd_dropout(q, k, v, *, dropout_p: float, seed: int, offset: int = 0, causal: bool = False,
                   scale: float | None = None, out=None, lse=None, return_lse: bool = True, stream=None):
    """Dense attention with dropout of the weights (bf16).  Returns (o, lse)."""
    a, out, lse = _fwd_args(q, k, v, causal, scale, out, lse, return_lse)
    d = _dropout_args(dropout_p, seed, offset)
    _check(lib().fa_fwd_dropout(ctypes.byref(a), ctypes.byref(d), _stream(stream)))
    return out, lse


def _check_dense(q, k, v, out, lse, qdt, odt):
    """Shapes and dtypes of a dense call: q [B, Nq, Hq, d], k and v
    [B, Nk, Hkv, d], out [B, Nq, Hq, d], lse [B, Hq, Nq] fp32 contiguous."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _ndim(t, n, 4)
    B, Nq, Hq, d = q.shape
    _, Nk, Hkv, _ = k.shape
    _need(q, "q", dtype=qdt)
    _need(k, "k", (B, Nk, Hkv, d), qdt)
    _need(v, "v", (B, Nk, Hkv, d), qdt)
    _need(out, "out", (B, Nq, Hq, d), odt, optional=True)
    _need(lse, "lse", (B, Hq, Nq), torch.float32, contiguous=True, optional=True)


def _fwd_args(q, k, v, causal, scale, out, lse, return_lse):
    torch = _torch()
    _dtype_code(q)
    _check_dense(q, k, v, out, lse, q.dtype, q.dtype)
    _dev(q, k, v, out, lse)
    B, Nq, Hq, d = q.shape
    _, Nk, Hkv, _ = k.shape
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    a = FwdArgs()
    a.q, a.k, a.v, a.o, a.lse = _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse)
    a.batch, a.seqlen_q, a.seqlen_k, a.heads_q, a.heads_kv, a.head_dim = B, Nq, Nk, Hq, Hkv, d
    for name, t in (("q_stride", q), ("k_stride", k), ("v_stride", v), ("o_stride", out)):
        getattr(a, name)[:] = list(t.stride()[:3])
    a.dtype = _dtype_code(q)
    a.scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    a.causal = int(bool(causal))
    return a, out, lse


def fa_fwd_fp8(q, k, v, descale, *, causal: bool = False, scale: float | None = None, out=None, lse=None,
               return_lse: bool = True, stream=None):
    """Dense attention over FP8 E4M3 codes (uint8 tensors q [B, Nq, Hq, d], k/v
    [B, Nk, Hkv, d]) standing for descale[i] * value(code).  Returns (o, lse)
    with o in bf16."""
    torch = _torch()
    for t in (q, k, v):
        if t is not None and t.dtype != torch.uint8:
            raise TypeError("fa_fwd_fp8 takes E4M3 codes as uint8 tensors")
    _check_dense(q, k, v, out, lse, torch.uint8, torch.bfloat16)
    _dev(q, k, v, out, lse)
    B, Nq, Hq, d = q.shape
    _, Nk, Hkv, _ = k.shape
    if out is None:
        out = torch.empty((B, Nq, Hq, d), dtype=torch.bfloat16, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    a = FwdFp8Args()
    a.q, a.k, a.v, a.o, a.lse = _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse)
    a.batch, a.seqlen_q, a.seqlen_k, a.heads_q, a.heads_kv, a.head_dim = B, Nq, Nk, Hq, Hkv, d
    for name, t in (("q_stride", q), ("k_stride", k), ("v_stride", v), ("o_stride", out)):
        getattr(a, name)[:] = list(t.stride()[:3])
    a.q_descale, a.k_descale, a.v_descale = (float(x) for x in descale)
    a.scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    a.causal = int(bool(causal))
    _check(lib().fa_fwd_fp8(ctypes.byref(a), _stream(stream)))
    return out, lse


def fa_fwd_varlen(q, k, v, cu_seqlens, max_seqlen: int, *, causal: bool = True,
                  scale: float | None = None, out=None, lse=None, return_lse: bool = True,
                  stream=None):
    """Packed variable-length attention.  ``max_seqlen`` is a host-side bound."""
    a, out, lse = _varlen_args(q, k, v, cu_seqlens, max_seqlen, causal, scale, out, lse, return_lse)
    _check(lib().fa_fwd_varlen(ctypes.byref(a), _stream(stream)))
    return out, lse


def fa_fwd_varlen_dropout(q, k, v, cu_seqlens, max_seqlen: int, *, dropout_p: float, seed: int,
                          offset: int = 0, causal: bool = True, scale: float | None = None, out=None,
                          lse=None, return_lse: bool = True, stream=None):
    """Packed variable-length attention with dropout of the weights (bf16)."""
    a, out, lse = _varlen_args(q, k, v, cu_seqlens, max_seqlen, causal, scale, out, lse, return_lse)
    d = _dropout_args(dropout_p, seed, offset)
    _check(lib().fa_fwd_varlen_dropout(ctypes.byref(a), ctypes.byref(d), _stream(stream)))
    return out, lse


def _check_varlen(q, k, v, cu_seqlens, out, lse, qdt, odt):
    """Shapes and dtypes of a packed call: q [T, Hq, d], k and v [T, Hkv, d],
    cu_seqlens int32 [S + 1] contiguous, out [T, Hq, d], lse [Hq, T] fp32."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _ndim(t, n, 3)
    _ndim(cu_seqlens, "cu_seqlens", 1)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    _need(q, "q", dtype=qdt)
    _need(k, "k", (T, Hkv, d), qdt)
    _need(v, "v", (T, Hkv, d), qdt)
    _need(cu_seqlens, "cu_seqlens", dtype=torch.int32, contiguous=True)
    if cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens needs at least one entry")
    _need(out, "out", (T, Hq, d), odt, optional=True)
    _need(lse, "lse", (Hq, T), torch.float32, contiguous=True, optional=True)


def _varlen_args(q, k, v, cu_seqlens, max_seqlen, causal, scale, out, lse, return_lse):
    torch = _torch()
    _dtype_code(q)
    _check_varlen(q, k, v, cu_seqlens, out, lse, q.dtype, q.dtype)
    _dev(q, k, v, out, lse, cu_seqlens)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((Hq, T), dtype=torch.float32, device=q.device)
    a = FwdVarlenArgs()
    a.q, a.k, a.v, a.o, a.lse = _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse)
    a.cu_seqlens = _ptr(cu_seqlens)
    a.num_seqs, a.total_tokens, a.max_seqlen = cu_seqlens.numel() - 1, T, int(max_seqlen)
    a.heads_q, a.heads_kv, a.head_dim = Hq, Hkv, d
    for name, t in (("q_stride", q), ("k_stride", k), ("v_stride", v), ("o_stride", out)):
        getattr(a, name)[:] = list(t.stride()[:2])
    a.dtype = _dtype_code(q)
    a.scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    a.causal = int(bool(causal))
    return a, out, lse


def fa_fwd_varlen_fp8(q, k, v, cu_seqlens, max_seqlen: int, descale, *, causal: bool = True,
                      scale: float | None = None, out=None, lse=None, return_lse: bool = True, stream=None):
    """Packed attention over FP8 E4M3 codes (uint8 q [T, Hq, d], k/v [T, Hkv, d])
    standing for descale[i] * value(code).  Returns (o, lse), o in bf16."""
    torch = _torch()
    for t in (q, k, v):
        if t is not None and t.dtype != torch.uint8:
            raise TypeError("fa_fwd_varlen_fp8 takes E4M3 codes as uint8 tensors")
    _check_varlen(q, k, v, cu_seqlens, out, lse, torch.uint8, torch.bfloat16)
    _dev(q, k, v, out, lse, cu_seqlens)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    if out is None:
        out = torch.empty((T, Hq, d), dtype=torch.bfloat16, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((Hq, T), dtype=torch.float32, device=q.device)
    a = FwdVarlenFp8Args()
    a.q, a.k, a.v, a.o, a.lse = _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse)
    a.cu_seqlens = _ptr(cu_seqlens)
    a.num_seqs, a.total_tokens, a.max_seqlen = cu_seqlens.numel() - 1, T, int(max_seqlen)
    a.heads_q, a.heads_kv, a.head_dim = Hq, Hkv, d
    for name, t in (("q_stride", q), ("k_stride", k), ("v_stride", v), ("o_stride", out)):
        getattr(a, name)[:] = list(t.stride()[:2])
    a.q_descale, a.k_descale, a.v_descale = (float(x) for x in descale)
    a.scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    a.causal = int(bool(causal))
    _check(lib().fa_fwd_varlen_fp8(ctypes.byref(a), _stream(stream)))
    return out, lse


def _check_pools(k_pool, v_pool, d, dt):
    """Pools [num_blocks, heads_kv, block_size, d] (any strides with d
    contiguous), k and v alike."""
    _ndim(k_pool, "k_pool", 4)
    _ndim(v_pool, "v_pool", 4)
    if k_pool.shape[3] != d:
        raise ValueError(f"pools must have head_dim {d}, got {k_pool.shape[3]}")
    _need(k_pool, "k_pool", dtype=dt)
    _need(v_pool, "v_pool", tuple(k_pool.shape), dt)
    if tuple(k_pool.stride()) != tuple(v_pool.stride()):
        raise ValueError("k_pool and v_pool must share shape and strides")


def _check_paged_prefill(q, k_pool, v_pool, block_table, cu_seqlens_q, seq_lens_k, out, lse, qdt, odt):
    torch = _torch()
    _ndim(q, "q", 3)
    Tq, Hq, d = q.shape
    _need(q, "q", dtype=qdt)
    _check_pools(k_pool, v_pool, d, qdt)
    _ndim(cu_seqlens_q, "cu_seqlens_q", 1)
    _need(cu_seqlens_q, "cu_seqlens_q", dtype=torch.int32, contiguous=True)
    S = cu_seqlens_q.numel() - 1
    if S < 0:
        raise ValueError("cu_seqlens_q needs at least one entry")
    _ndim(block_table, "block_table", 2)
    _need(block_table, "block_table", (S, block_table.shape[1]), torch.int32, contiguous=True)
    _need(seq_lens_k, "seq_lens_k", (S,), torch.int32, contiguous=True)
    _need(out, "out", (Tq, Hq, d), odt, optional=True)
    _need(lse, "lse", (Hq, Tq), torch.float32, contiguous=True, optional=True)


def _fwd_paged_args(q, k_pool, v_pool, block_table, cu_seqlens_q, seq_lens_k, max_seqlen_q, max_seqlen_k,
                    causal, scale):
    Tq, Hq, d = q.shape
    nb, Hkv, bs, _ = k_pool.shape
    if tuple(k_pool.stride()) != tuple(v_pool.stride()) or k_pool.shape != v_pool.shape:
        raise ValueError("k_pool and v_pool must share shape and strides")
    a = FwdPagedArgs()
    a.q, a.k_pool, a.v_pool = _ptr(q), _ptr(k_pool), _ptr(v_pool)
    a.pool_stride[:] = list(k_pool.stride()[:3])
    a.block_table, a.cu_seqlens_q, a.seq_lens_k = _ptr(block_table), _ptr(cu_seqlens_q), _ptr(seq_lens_k)
    a.q_stride[:] = list(q.stride()[:2])
    a.num_seqs, a.total_q = cu_seqlens_q.numel() - 1, Tq
    a.max_seqlen_q, a.max_seqlen_k = int(max_seqlen_q), int(max_seqlen_k)
    a.heads_q, a.heads_kv, a.head_dim, a.block_size = Hq, Hkv, d, bs
    a.max_blocks_per_seq = block_table.shape[1] if block_table is not None else 0
    a.num_blocks = nb
    a.scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    a.causal = int(bool(causal))
    return a


def fa_fwd_paged(q, k_pool, v_pool, block_table, cu_seqlens_q, seq_lens_k, max_seqlen_q: int,
                 max_seqlen_k: int, *, causal: bool = True, scale: float | None = None, out=None, lse=None,
                 return_lse: bool = True, stream=None):
    """Chunked prefill over a paged KV pool (bf16).  ``max_seqlen_q`` and
    ``max_seqlen_k`` are host-side bounds.  Returns (o, lse)."""
    torch = _torch()
    for t in (q, k_pool, v_pool):
        if t is not None and t.dtype != torch.bfloat16:
            raise TypeError("fa_fwd_paged takes bf16 q and pools")
    _check_paged_prefill(q, k_pool, v_pool, block_table, cu_seqlens_q, seq_lens_k, out, lse, torch.bfloat16,
                         torch.bfloat16)
    _dev(q, k_pool, v_pool, block_table, cu_seqlens_q, seq_lens_k, out, lse)
    Tq, Hq, _ = q.shape
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((Hq, Tq), dtype=torch.float32, device=q.device)
    a = _fwd_paged_args(q, k_pool, v_pool, block_table, cu_seqlens_q, seq_lens_k, max_seqlen_q, max_seqlen_k,
                        causal, scale)
    a.o, a.lse = _ptr(out), _ptr(lse)
    a.o_stride[:] = list(out.stride()[:2])
    _check(lib().fa_fwd_paged(ctypes.byref(a), _stream(stream)))
    return out, lse


def _check_decode(q, k_pool, v_pool, block_table, seq_lens, out, lse, workspace, pool_dt):
    """q [B, Hq, d] bf16, pools [blocks, Hkv, 16, d] of pool_dt, block_table
    int32 [B, max_blocks] contiguous, seq_lens int32 [B], out [B, Hq, d] bf16,
    lse [B, Hq] fp32 contiguous, workspace contiguous."""
    torch = _torch()
    _ndim(q, "q", 3)
    B, Hq, d = q.shape
    _need(q, "q", dtype=torch.bfloat16)
    _check_pools(k_pool, v_pool, d, pool_dt)
    _ndim(block_table, "block_table", 2)
    _need(block_table, "block_table", (B, block_table.shape[1]), torch.int32, contiguous=True)
    _need(seq_lens, "seq_lens", (B,), torch.int32, contiguous=True)
    _need(out, "out", (B, Hq, d), torch.bfloat16, optional=True)
    _need(lse, "lse", (B, Hq), torch.float32, contiguous=True, optional=True)
    _need(workspace, "workspace", contiguous=True, optional=True)


def _decode_args(q, k_pool, v_pool, block_table, seq_lens, max_seq_len, scale, num_splits):
    B, Hq, d = q.shape
    nb, Hkv, bs, _ = k_pool.shape
    if tuple(k_pool.stride()) != tuple(v_pool.stride()) or k_pool.shape != v_pool.shape:
        raise ValueError("k_pool and v_pool must share shape and strides")
    a = DecodePagedArgs()
    a.q, a.k_pool, a.v_pool = _ptr(q), _ptr(k_pool), _ptr(v_pool)
    ps = k_pool.stride()
    a.pool_stride[:] = [ps[0], ps[1], ps[2]]
    a.block_table, a.seq_lens = _ptr(block_table), _ptr(seq_lens)
    a.q_stride[:] = list(q.stride()[:2])
    a.batch, a.heads_q, a.heads_kv, a.head_dim, a.block_size = B, Hq, Hkv, d, bs
    a.max_blocks_per_seq = block_table.shape[1] if block_table is not None else 0
    a.num_blocks, a.max_seq_len = nb, int(max_seq_len)
    a.scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    a.num_splits = int(num_splits)
    return a


def fa_decode_paged_workspace_size(q, k_pool, v_pool, block_table, seq_lens, max_seq_len: int, *,
                                   num_splits: int = 0) -> int:
    _check_decode(q, k_pool, v_pool, block_table, seq_lens, None, None, None, _torch().bfloat16)
    a = _decode_args(q, k_pool, v_pool, block_table, seq_lens, max_seq_len, None, num_splits)
    return int(lib().fa_decode_paged_workspace_size(ctypes.byref(a)))


def fa_decode_paged_num_splits(q, k_pool, v_pool, block_table, seq_lens, max_seq_len: int, *,
                               num_splits: int = 0) -> int:
    _check_decode(q, k_pool, v_pool, block_table, seq_lens, None, None, None, _torch().bfloat16)
    a = _decode_args(q, k_pool, v_pool, block_table, seq_lens, max_seq_len, None, num_splits)
    return int(lib().fa_decode_paged_num_splits(ctypes.byref(a)))


def fa_decode_paged(q, k_pool, v_pool, block_table, seq_lens, max_seq_len: int, *,
                    scale: float | None = None, num_splits: int = 0, out=None, lse=None,
                    return_lse: bool = True, workspace=None, stream=None):
    """Paged single-token decode.  Returns (o, lse)."""
    torch = _torch()
    _check_decode(q, k_pool, v_pool, block_table, seq_lens, out, lse, workspace, torch.bfloat16)
    _dev(q, k_pool, v_pool, block_table, seq_lens, out, lse, workspace)
    B, Hq, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    a = _decode_args(q, k_pool, v_pool, block_table, seq_lens, max_seq_len, scale, num_splits)
    a.o, a.lse = _ptr(out), _ptr(lse)
    a.o_stride[:] = list(out.stride()[:2])
    need = int(lib().fa_decode_paged_workspace_size(ctypes.byref(a)))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    a.workspace, a.workspace_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    _check(lib().fa_decode_paged(ctypes.byref(a), _stream(stream)))
    return out, lse


def fa_decode_paged_noalloc(q, k_pool, v_pool, block_table, seq_lens, max_seq_len: int, *,
                            scale: float | None = None, num_splits: int = 0, out, lse=None, stream=None):
    """Paged single-token decode that allocates nothing: the caller passes
    ``out`` (and optionally ``lse``); the partial states go to the library's
    own per-device workspace.  Returns (out, lse)."""
    torch = _torch()
    _check_decode(q, k_pool, v_pool, block_table, seq_lens, out, lse, None, torch.bfloat16)
    _dev(q, k_pool, v_pool, block_table, seq_lens, out, lse)
    a = _decode_args(q, k_pool, v_pool, block_table, seq_lens, max_seq_len, scale, num_splits)
    a.o, a.lse = _ptr(out), _ptr(lse)
    a.o_stride[:] = list(out.stride()[:2])
    a.workspace, a.workspace_bytes = None, 0
    _check(lib().fa_decode_paged_noalloc(ctypes.byref(a), _stream(stream)))
    return out, lse


def fa_decode_paged_fp8(q, k_pool, v_pool, block_table, seq_lens, max_seq_len: int, descale, *,
                        scale: float | None = None, num_splits: int = 0, out=None, lse=None,
                        return_lse: bool = True, workspace=None, stream=None):
    """Paged single-token decode over an FP8 KV cache: uint8 E4M3 pools
    standing for descale[0] * value(k code) and descale[1] * value(v code);
    q and o bf16.  Returns (o, lse)."""
    torch = _torch()
    for t in (k_pool, v_pool):
        if t is not None and t.dtype != torch.uint8:
            raise TypeError("fa_decode_paged_fp8 takes E4M3 pools as uint8 tensors")
    _check_decode(q, k_pool, v_pool, block_table, seq_lens, out, lse, workspace, torch.uint8)
    _dev(q, k_pool, v_pool, block_table, seq_lens, out, lse, workspace)
    B, Hq, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    a = DecodePagedFp8Args()
    a.base = _decode_args(q, k_pool, v_pool, block_table, seq_lens, max_seq_len, scale, num_splits)
    a.base.o, a.base.lse = _ptr(out), _ptr(lse)
    a.base.o_stride[:] = list(out.stride()[:2])
    a.k_descale, a.v_descale = (float(x) for x in descale)
    need = int(lib().fa_decode_paged_fp8_workspace_size(ctypes.byref(a)))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    a.base.workspace, a.base.workspace_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    _check(lib().fa_decode_paged_fp8(ctypes.byref(a), _stream(stream)))
    return out, lse


def _decode_fp8_args(q, k_pool, v_pool, block_table, seq_lens, max_seq_len, descale, num_splits):
    _check_decode(q, k_pool, v_pool, block_table, seq_lens, None, None, None, _torch().uint8)
    a = DecodePagedFp8Args()
    a.base = _decode_args(q, k_pool, v_pool, block_table, seq_lens, max_seq_len, None, num_splits)
    a.k_descale, a.v_descale = (float(x) for x in descale)
    return a


def fa_decode_paged_fp8_workspace_size(q, k_pool, v_pool, block_table, seq_lens, max_seq_len: int, descale, *,
                                       num_splits: int = 0) -> int:
    a = _decode_fp8_args(q, k_pool, v_pool, block_table, seq_lens, max_seq_len, descale, num_splits)
    return int(lib().fa_decode_paged_fp8_workspace_size(ctypes.byref(a)))


def fa_decode_paged_fp8_num_splits(q, k_pool, v_pool, block_table, seq_lens, max_seq_len: int, descale, *,
                                   num_splits: int = 0) -> int:
    a = _decode_fp8_args(q, k_pool, v_pool, block_table, seq_lens, max_seq_len, descale, num_splits)
    return int(lib().fa_decode_paged_fp8_num_splits(ctypes.byref(a)))


def fa_fwd_paged_fp8(q, k_pool, v_pool, block_table, cu_seqlens_q, seq_lens_k, max_seqlen_q: int,
                     max_seqlen_k: int, descale, *, causal: bool = True, scale: float | None = None, out=None,
                     lse=None, return_lse: bool = True, stream=None):
    """Chunked prefill over an FP8 KV cache: uint8 E4M3 q [Tq, Hq, d] and pools
    standing for descale[i] * value(code) (q, k, v).  Returns (o, lse), o bf16."""
    torch = _torch()
    for t in (q, k_pool, v_pool):
        if t is not None and t.dtype != torch.uint8:
            raise TypeError("fa_fwd_paged_fp8 takes E4M3 q and pools as uint8 tensors")
    _check_paged_prefill(q, k_pool, v_pool, block_table, cu_seqlens_q, seq_lens_k, out, lse, torch.uint8,
                         torch.bfloat16)
    _dev(q, k_pool, v_pool, block_table, cu_seqlens_q, seq_lens_k, out, lse)
    Tq, Hq, d = q.shape
    if out is None:
        out = torch.empty((Tq, Hq, d), dtype=torch.bfloat16, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((Hq, Tq), dtype=torch.float32, device=q.device)
    a = FwdPagedFp8Args()
    a.base = _fwd_paged_args(q, k_pool, v_pool, block_table, cu_seqlens_q, seq_lens_k, max_seqlen_q, max_seqlen_k,
                             causal, scale)
    a.base.o, a.base.lse = _ptr(out), _ptr(lse)
    a.base.o_stride[:] = list(out.stride()[:2])
    a.q_descale, a.k_descale, a.v_descale = (float(x) for x in descale)
    _check(lib().fa_fwd_paged_fp8(ctypes.byref(a), _stream(stream)))
    return out, lse


def fa_merge_states(o_parts, lse_parts, *, out=None, lse=None, return_lse: bool = True, stream=None):
    """Merge P results over disjoint key sets: o_parts [P, B, S, H, D] and
    lse_parts [P, B, H, S] (contiguous) -> (o [B, S, H, D], lse [B, H, S])."""
    torch = _torch()
    if o_parts.dim() != 5 or lse_parts.dim() != 4:
        raise ValueError("o_parts must be [P, B, S, H, D] and lse_parts [P, B, H, S]")
    P, B, S, H, D = o_parts.shape
    if tuple(lse_parts.shape) != (P, B, H, S) or lse_parts.dtype != torch.float32:
        raise ValueError(f"lse_parts must be fp32 {(P, B, H, S)}, got {tuple(lse_parts.shape)} {lse_parts.dtype}")
    if not (o_parts.is_contiguous() and lse_parts.is_contiguous()):
        raise ValueError("o_parts and lse_parts must be contiguous")
    _need(out, "out", (B, S, H, D), o_parts.dtype, contiguous=True, optional=True)
    _need(lse, "lse", (B, H, S), torch.float32, contiguous=True, optional=True)
    _dev(o_parts, lse_parts, out, lse)
    if out is None:
        out = torch.empty((B, S, H, D), dtype=o_parts.dtype, device=o_parts.device)
    if lse is None and return_lse:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=o_parts.device)
    if not out.is_contiguous() or tuple(out.shape) != (B, S, H, D) or out.dtype != o_parts.dtype:
        raise ValueError("out must be a contiguous [B, S, H, D] tensor of o_parts' dtype")
    a = MergeStatesArgs(P, B, S, H, D, _dtype_code(o_parts), _ptr(o_parts), _ptr(lse_parts), _ptr(out), _ptr(lse))
    _check(lib().fa_merge_states(ctypes.byref(a), _stream(stream)))
    return out, lse
