"""fp64 CPU oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the bench's CPU-baseline leg
may import this package.  The GPU library never imports it, and it never
imports the GPU library: the two share no code.

``oracle.c`` is the definition (materialised score row, textbook softmax,
double precision); this module compiles it with gcc and wraps it with ctypes.
``twin.py`` is an independent pure-Python brute force used to pin it, and
``recurrence.py`` is the pages' tiled / paged / split recurrence in fp64,
used to show that the method reaches the definition.

Every function here is pinned by ``tests/test_oracle_*.py``; see the pin list
in each test module's docstring.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

F64, F32, BF16 = 0, 1, 2


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (plain -O2, OpenMP, no fast-math)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
           src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _load(path: str = _LIB):
    global _lib
    if _lib is not None and path == _LIB:
        return _lib
    if not os.path.exists(path) or (path == _LIB and os.path.getmtime(path) < os.path.getmtime(_SRC)):
        build(out=path)
    lib = ctypes.CDLL(path)
    P, I, I64, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
    U64, U32 = ctypes.c_uint64, ctypes.c_uint32
    lib.oracle_attn_dense.argtypes = [P, P, P, I, I, I, I, I, I, I, P, P, P, I, D, P, I64, P, P, I]
    lib.oracle_attn_varlen.argtypes = [P, P, P, I, P, I, I, I, I, P, P, P, I, D, P, I64, P, P, I]
    lib.oracle_attn_decode_paged.argtypes = [P, P, P, I, P, P, P, I, P, I, I, I, I, I, I, D, P,
                                             I64, P, P, I]
    lib.oracle_attn_paged_prefill.argtypes = [P, P, P, I, P, I, P, P, P, I, P, I, I, I, I, I, I, D,
                                              P, I64, P, P, I]
    lib.oracle_max_threads.argtypes = [I]
    lib.oracle_attn_dense_dropout.argtypes = [P, P, P, I, I, I, I, I, I, I, P, P, P, I, D, I, U64, U32, P,
                                              I64, P, P, I]
    lib.oracle_attn_varlen_dropout.argtypes = [P, P, P, I, P, I, I, I, I, P, P, P, I, D, I, U64, U32, P,
                                               I64, P, P, I]
    lib.oracle_philox4x32_10.argtypes = [P, P, P]
    lib.oracle_philox4x32_10.restype = None
    lib.oracle_decode_e4m3.argtypes = [P, P, I64]
    lib.oracle_decode_e4m3.restype = None
    lib.oracle_merge_states.argtypes = [I64, I64, I64, P, P, P, P]
    lib.oracle_merge_states.restype = None
    for f in (lib.oracle_attn_dense, lib.oracle_attn_varlen, lib.oracle_attn_decode_paged,
              lib.oracle_attn_paged_prefill, lib.oracle_max_threads):
        f.restype = I
    if path == _LIB:
        _lib = lib
    return lib


def load_library(path: str):
    """Load an oracle build from an explicit path (used to test planted mistakes)."""
    return _load(path)


def threads(n: int = 0) -> int:
    """Set (n > 0) and return the OpenMP thread count the oracle will use."""
    return _load().oracle_max_threads(int(n))


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float64:
        return F64
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"unsupported dtype {a.dtype}: use float64, float32 or uint16 (bf16 bits)")


def _strides(a: np.ndarray, n: int) -> np.ndarray:
    st = [s // a.itemsize for s in a.strides]
    if st[-1] != 1:
        raise ValueError("last dimension must be contiguous")
    return np.asarray(st[:n], dtype=np.int64)


def _ptr(a):
    return None if a is None else a.ctypes.data


def _rows(rows):
    if rows is None:
        return None, 0
    r = np.ascontiguousarray(rows, dtype=np.int64)
    return r, int(r.size)


def dense(q, k, v, *, causal: bool, scale: float | None = None, rows=None, nthreads: int = 0,
          lib=None):
    """Dense batched attention.  q [B, Nq, Hq, d]; k, v [B, Nk, Hkv, d].

    Returns (o, lse).  With rows=None: o [B, Hq, Nq, d] and lse [B, Hq, Nq];
    otherwise rows are flattened ids (b*Hq + h)*Nq + i and o is [nrows, d].
    Default scale is 1/sqrt(d) in double precision.
    """
    lib = lib or _load()
    B, Nq, Hq, d = q.shape
    _, Nk, Hkv, _ = k.shape
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    r, nr = _rows(rows)
    n = nr if r is not None else B * Hq * Nq
    o = np.zeros((n, d), dtype=np.float64)
    lse = np.zeros(n, dtype=np.float64)
    qs, ks, vs = _strides(q, 3), _strides(k, 3), _strides(v, 3)
    st = lib.oracle_attn_dense(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, Nq, Nk, Hq, Hkv, d,
                               _ptr(qs), _ptr(ks), _ptr(vs), int(bool(causal)), scale, _ptr(r),
                               nr, _ptr(o), _ptr(lse), int(nthreads))
    if st:
        raise ValueError(f"oracle_attn_dense failed with status {st}")
    if r is None:
        return o.reshape(B, Hq, Nq, d), lse.reshape(B, Hq, Nq)
    return o, lse


def varlen(q, k, v, cu_seqlens, *, causal: bool, scale: float | None = None, rows=None,
           nthreads: int = 0, lib=None):
    """Packed attention.  q [T, Hq, d]; k, v [T, Hkv, d]; cu_seqlens [S+1].

    With rows=None: o [Hq, T, d], lse [Hq, T]; else rows are h*T + t.
    """
    lib = lib or _load()
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    r, nr = _rows(rows)
    n = nr if r is not None else Hq * T
    o = np.zeros((n, d), dtype=np.float64)
    lse = np.zeros(n, dtype=np.float64)
    qs, ks, vs = _strides(q, 2), _strides(k, 2), _strides(v, 2)
    st = lib.oracle_attn_varlen(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(cu), len(cu) - 1,
                                Hq, Hkv, d, _ptr(qs), _ptr(ks), _ptr(vs), int(bool(causal)), scale,
                                _ptr(r), nr, _ptr(o), _ptr(lse), int(nthreads))
    if st:
        raise ValueError(f"oracle_attn_varlen failed with status {st}")
    if r is None:
        return o.reshape(Hq, T, d), lse.reshape(Hq, T)
    return o, lse


def decode_paged(q, k_pool, v_pool, block_table, seq_lens, *, scale: float | None = None,
                 rows=None, nthreads: int = 0, lib=None):
    """Paged single-token decode.  q [B, Hq, d]; pools [num_blocks, Hkv, block, d]
    (any strides with d contiguous; k and v pools must share strides);
    block_table [B, max_blocks] int32; seq_lens [B] int32.

    With rows=None: o [B, Hq, d], lse [B, Hq]; else rows are b*Hq + h.
    """
    lib = lib or _load()
    B, Hq, d = q.shape
    nb, Hkv, bs, _ = k_pool.shape
    if k_pool.strides != v_pool.strides or k_pool.shape != v_pool.shape:
        raise ValueError("k and v pools must have the same shape and strides")
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    r, nr = _rows(rows)
    n = nr if r is not None else B * Hq
    o = np.zeros((n, d), dtype=np.float64)
    lse = np.zeros(n, dtype=np.float64)
    qs, ps = _strides(q, 2), _strides(k_pool, 3)
    st = lib.oracle_attn_decode_paged(_ptr(q), _ptr(k_pool), _ptr(v_pool), _dtype_code(q),
                                      _ptr(qs), _ptr(ps), _ptr(bt), bt.shape[1], _ptr(sl), B, Hq,
                                      Hkv, d, bs, nb, scale, _ptr(r), nr, _ptr(o), _ptr(lse),
                                      int(nthreads))
    if st:
        raise ValueError(f"oracle_attn_decode_paged failed with status {st}")
    if r is None:
        return o.reshape(B, Hq, d), lse.reshape(B, Hq)
    return o, lse


def paged_prefill(q, k_pool, v_pool, block_table, cu_seqlens_q, seq_lens_k, *, causal: bool,
                  scale: float | None = None, rows=None, nthreads: int = 0, lib=None):
    """Chunked prefill over a paged pool.  q packed [Tq, Hq, d] with
    cu_seqlens_q [S+1]; pools [num_blocks, Hkv, block, d] (k and v share
    strides); block_table [S, max_blocks] int32; seq_lens_k [S] int32 (each
    sequence's whole context).  Causal: query i of a chunk of n sees key t iff
    t <= i + (seq_lens_k - n).

    With rows=None: o [Hq, Tq, d], lse [Hq, Tq]; else rows are h*Tq + t.
    """
    lib = lib or _load()
    T, Hq, d = q.shape
    nb, Hkv, bs, _ = k_pool.shape
    if k_pool.strides != v_pool.strides or k_pool.shape != v_pool.shape:
        raise ValueError("k and v pools must have the same shape and strides")
    cu = np.ascontiguousarray(cu_seqlens_q, dtype=np.int32)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens_k, dtype=np.int32)
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    r, nr = _rows(rows)
    n = nr if r is not None else Hq * T
    o = np.zeros((n, d), dtype=np.float64)
    lse = np.zeros(n, dtype=np.float64)
    qs, ps = _strides(q, 2), _strides(k_pool, 3)
    st = lib.oracle_attn_paged_prefill(_ptr(q), _ptr(k_pool), _ptr(v_pool), _dtype_code(q), _ptr(cu),
                                       len(cu) - 1, _ptr(qs), _ptr(ps), _ptr(bt), bt.shape[1], _ptr(sl),
                                       Hq, Hkv, d, bs, nb, int(bool(causal)), scale, _ptr(r), nr,
                                       _ptr(o), _ptr(lse), int(nthreads))
    if st:
        raise ValueError(f"oracle_attn_paged_prefill failed with status {st}")
    if r is None:
        return o.reshape(Hq, T, d), lse.reshape(Hq, T)
    return o, lse


def visible_pairs_dense(nq: int, nk: int, causal: bool) -> int:
    """Number of visible (query, key) pairs of one head."""
    if not causal:
        return nq * nk
    return sum(max(0, min(nk, i + (nk - nq) + 1)) for i in range(nq))


def decode_e4m3(codes, *, lib=None) -> np.ndarray:
    """FP8 E4M3 codes (uint8) -> their exact values in float64 (see
    oracle_decode_e4m3 for the format)."""
    L = lib or _load()
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    L.oracle_decode_e4m3(_ptr(c), _ptr(out), c.size)
    return out


def fp8_dense(q8, k8, v8, descale, *, causal: bool, scale: float | None = None, rows=None,
              nthreads: int = 0, lib=None):
    """Dense attention over FP8 E4M3 inputs with per-tensor descale factors.

    The inputs stand for the real tensors q = descale[0] * value(q8), k =
    descale[1] * value(k8), v = descale[2] * value(v8); the result is the
    exact attention of those (``dense`` on the widened, scaled tensors), with
    the same layouts and return values as ``dense``.  The scale defaults to
    1/sqrt(d).
    """
    qd, kd, vd = (float(x) for x in descale)
    q = decode_e4m3(q8, lib=lib) * qd
    k = decode_e4m3(k8, lib=lib) * kd
    v = decode_e4m3(v8, lib=lib) * vd
    return dense(q, k, v, causal=causal, scale=scale, rows=rows, nthreads=nthreads, lib=lib)


def fp8_varlen(q8, k8, v8, cu_seqlens, descale, *, causal: bool, scale: float | None = None, rows=None,
               nthreads: int = 0, lib=None):
    """Packed attention over FP8 E4M3 inputs with per-tensor descale factors:
    ``varlen`` on descale[i] * value(code), with the layouts and return values
    of ``varlen``."""
    qd, kd, vd = (float(x) for x in descale)
    q = decode_e4m3(q8, lib=lib) * qd
    k = decode_e4m3(k8, lib=lib) * kd
    v = decode_e4m3(v8, lib=lib) * vd
    return varlen(q, k, v, cu_seqlens, causal=causal, scale=scale, rows=rows, nthreads=nthreads, lib=lib)


def _widen(x):
    """bf16 bit patterns (uint16) -> float64 exactly; floats pass through."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def decode_paged_fp8(q, k8_pool, v8_pool, block_table, seq_lens, descale, *, scale: float | None = None,
                     rows=None, nthreads: int = 0, lib=None):
    """Paged decode over FP8 E4M3 pools with per-tensor descale factors
    (k, v): ``decode_paged`` on q (bf16 widened exactly) and the pools
    descale * value(code), with the layouts and return values of
    ``decode_paged``."""
    kd, vd = (float(x) for x in descale)
    kp = decode_e4m3(k8_pool, lib=lib) * kd
    vp = decode_e4m3(v8_pool, lib=lib) * vd
    return decode_paged(_widen(q), kp, vp, block_table, seq_lens, scale=scale, rows=rows, nthreads=nthreads,
                        lib=lib)


def paged_prefill_fp8(q8, k8_pool, v8_pool, block_table, cu_seqlens_q, seq_lens_k, descale, *, causal: bool,
                      scale: float | None = None, rows=None, nthreads: int = 0, lib=None):
    """Chunked prefill with FP8 E4M3 queries and pools and per-tensor descale
    factors (q, k, v): ``paged_prefill`` on descale[i] * value(code)."""
    qd, kd, vd = (float(x) for x in descale)
    q = decode_e4m3(q8, lib=lib) * qd
    kp = decode_e4m3(k8_pool, lib=lib) * kd
    vp = decode_e4m3(v8_pool, lib=lib) * vd
    return paged_prefill(q, kp, vp, block_table, cu_seqlens_q, seq_lens_k, causal=causal, scale=scale, rows=rows,
                         nthreads=nthreads, lib=lib)


def dropout_threshold(p: float) -> int:
    """Byte threshold t of a dropout probability: t = rint(256 p), p in [0, 1)
    with t <= 255; a weight is kept iff its random byte >= t, with probability
    (256 - t) / 256, and kept weights are scaled by 256 / (256 - t)."""
    t = int(np.rint(float(p) * 256.0))
    if not (0.0 <= float(p) < 1.0) or t > 255:
        raise ValueError("dropout probability must be in [0, 255.5/256)")
    return t


def philox4x32_10(ctr, key, *, lib=None):
    """One Philox-4x32-10 block: 4 uint32 counter words, 2 key words -> 4 words."""
    L = lib or _load()
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    L.oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def dense_dropout(q, k, v, *, causal: bool, dropout_p: float, seed: int, offset: int = 0,
                  scale: float | None = None, rows=None, nthreads: int = 0, lib=None):
    """``dense`` with dropout of the normalised weights: the weight of row
    (b, h, i) on key j is kept iff byte j % 16 of Philox-4x32-10(counter {j /
    16, row, row >> 32, offset}, key {seed, seed >> 32}) is >= the threshold
    of ``dropout_threshold``, row = (b * Hq + h) * Nq + i."""
    L = lib or _load()
    B, Nq, Hq, d = q.shape
    _, Nk, Hkv, _ = k.shape
    t = dropout_threshold(dropout_p)
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    r, nr = _rows(rows)
    n = nr if r is not None else B * Hq * Nq
    o = np.zeros((n, d), dtype=np.float64)
    lse = np.zeros(n, dtype=np.float64)
    qs, ks, vs = _strides(q, 3), _strides(k, 3), _strides(v, 3)
    st = L.oracle_attn_dense_dropout(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, Nq, Nk, Hq, Hkv, d,
                                     _ptr(qs), _ptr(ks), _ptr(vs), int(bool(causal)), scale, t,
                                     int(seed) & (2**64 - 1), int(offset) & (2**32 - 1), _ptr(r), nr,
                                     _ptr(o), _ptr(lse), int(nthreads))
    if st:
        raise ValueError(f"oracle_attn_dense_dropout failed with status {st}")
    if r is None:
        return o.reshape(B, Hq, Nq, d), lse.reshape(B, Hq, Nq)
    return o, lse


def varlen_dropout(q, k, v, cu_seqlens, *, causal: bool, dropout_p: float, seed: int, offset: int = 0,
                   scale: float | None = None, rows=None, nthreads: int = 0, lib=None):
    """``varlen`` with dropout; the row of (h, token t) is h * T + t and keys
    are numbered within their sequence."""
    L = lib or _load()
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    t = dropout_threshold(dropout_p)
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    r, nr = _rows(rows)
    n = nr if r is not None else Hq * T
    o = np.zeros((n, d), dtype=np.float64)
    lse = np.zeros(n, dtype=np.float64)
    qs, ks, vs = _strides(q, 2), _strides(k, 2), _strides(v, 2)
    st = L.oracle_attn_varlen_dropout(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(cu), len(cu) - 1,
                                      Hq, Hkv, d, _ptr(qs), _ptr(ks), _ptr(vs), int(bool(causal)), scale,
                                      t, int(seed) & (2**64 - 1), int(offset) & (2**32 - 1), _ptr(r), nr,
                                      _ptr(o), _ptr(lse), int(nthreads))
    if st:
        raise ValueError(f"oracle_attn_varlen_dropout failed with status {st}")
    if r is None:
        return o.reshape(Hq, T, d), lse.reshape(Hq, T)
    return o, lse


def merge_states(o_parts, lse_parts, *, lib=None):
    """Merge P attention results of the same rows over disjoint key sets
    ("FlashAttention", tachyon.techntrek.in, "For engineers / Show the
    maths", the (m, l, o) merge rule over P states): o_parts [P, ..., d]
    (bf16 bit patterns as uint16, or floats) and lse_parts [P, ...] (natural
    log, -inf = the part saw no key) -> (o [..., d], lse [...]) in fp64."""
    lib = lib or _load()
    o_parts = np.ascontiguousarray(_widen(o_parts))
    lse_parts = np.ascontiguousarray(np.asarray(lse_parts, dtype=np.float64))
    P, d = o_parts.shape[0], o_parts.shape[-1]
    rows_shape = o_parts.shape[1:-1]
    if lse_parts.shape != (P,) + rows_shape:
        raise ValueError(f"lse_parts {lse_parts.shape} does not match o_parts {o_parts.shape}")
    R = int(np.prod(rows_shape, dtype=np.int64))
    o = np.zeros(rows_shape + (d,), dtype=np.float64)
    lse = np.zeros(rows_shape, dtype=np.float64)
    lib.oracle_merge_states(P, R, d, _ptr(o_parts), _ptr(lse_parts), _ptr(o), _ptr(lse))
    return o, lse
