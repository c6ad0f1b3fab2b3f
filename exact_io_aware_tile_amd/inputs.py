"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module draws random numbers and lays them out; it holds none of the
attention arithmetic.  Both the GPU library and the CPU oracle are fed from
the same host bytes produced here.

Recipe
------
* Every normal tensor is drawn as float32 N(0, 1) in C order of its logical
  layout, in fixed chunks of ``CHUNK`` elements; chunk ``c`` of stream ``s``
  under seed ``seed`` comes from ``numpy.random.default_rng([seed, s, c])``
  (PCG64).  The values therefore do not depend on how many threads draw them.
* Streams: q = 0, k = 1, v = 2 (the pages' q, k, v order), 3 for the new
  queries of a chunked prefill.  Integer draws
  (lengths, permutations, spike rows) use ``default_rng([seed, 100 + n])``.
* bf16 tensors are the float32 draws rounded to nearest-even, kept as raw
  ``uint16`` bit patterns; ``bf16_to_f32`` widens them back exactly.
* fp8 tensors are FP8 E4M3 codes (``uint8``) of the float32 draws divided by
  a per-tensor descale factor amax / 448 (float32), rounded to nearest-even
  and saturated at +-448; the tensor they stand for is descale * value(code).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 22
STREAM_Q, STREAM_K, STREAM_V = 0, 1, 2
STREAM_QCHUNK = 3  # queries of a chunked prefill


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_f32(seed: int, stream: int, shape) -> np.ndarray:
    """float32 N(0,1) array of ``shape`` drawn chunk by chunk (see module doc)."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK

    def fill(c: int) -> None:
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        rng = np.random.default_rng([seed, stream, c])
        out[lo:hi] = rng.standard_normal(hi - lo, dtype=np.float32)

    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16, nearest-even, returned as uint16 bit patterns.

    Inputs here are finite normals, so no NaN/inf special-casing is needed.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)

    def conv(lo: int, hi: int) -> None:
        u = flat[lo:hi].view(np.uint32)
        r = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
        out[lo:hi] = (r >> np.uint32(16)).astype(np.uint16)

    n = flat.size
    if n <= CHUNK:
        conv(0, n)
    else:
        spans = [(lo, min(n, lo + CHUNK)) for lo in range(0, n, CHUNK)]
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(lambda s: conv(*s), spans))
    return out.reshape(x.shape)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32, exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# The 127 non-negative finite E4M3 values in code order (codes 0x00..0x7E):
# subnormals m * 2^-9, then (1 + m/8) * 2^(e-7); increasing with the code.
_E4M3_POS = np.array([m * 2.0**-9 if e == 0 else (1 + m / 8) * 2.0**(e - 7)
                      for e in range(16) for m in range(8)][:127], dtype=np.float64)
E4M3_MAX = 448.0


def f32_to_e4m3(x: np.ndarray) -> np.ndarray:
    """Round float32 to FP8 E4M3 codes (uint8): nearest value, ties to the even
    code, magnitudes above 448 saturated to 448.  Inputs are finite.

    Normal range (|x| >= 2^-6): the float32 mantissa is rounded to 3 bits,
    ties to even, in integer arithmetic on the bit pattern (a carry moves the
    exponent); subnormal range: multiples of 2^-9, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    a = np.abs(x)
    bits = a.view(np.uint32)
    r = (bits + np.uint32(0x7FFFF) + ((bits >> np.uint32(20)) & np.uint32(1))) & np.uint32(0xFFF00000)
    e = (r >> np.uint32(23)).astype(np.int32) - (127 - 7)
    code = (e << 3) | ((r >> np.uint32(20)) & np.uint32(7)).astype(np.int32)
    sub = a < np.float32(2.0 ** -6)
    code = np.where(sub, np.rint(a * np.float32(512.0)).astype(np.int32), code)
    code = np.where(a >= np.float32(E4M3_MAX), 126, np.minimum(code, 126)).astype(np.uint8)
    return np.where(np.signbit(x), code | np.uint8(0x80), code).astype(np.uint8)


def e4m3_to_f32(c: np.ndarray) -> np.ndarray:
    """Widen E4M3 codes (uint8, no NaN codes) to float32, exactly."""
    c = np.asarray(c, dtype=np.uint8)
    v = _E4M3_POS[np.minimum(c & np.uint8(0x7F), 126)].astype(np.float32)
    return np.where(c >= 0x80, -v, v)


def _chunked(fn, x: np.ndarray, out_dtype):
    """fn applied to C-order chunks of x (threads: numpy releases the GIL)."""
    flat = np.ascontiguousarray(x).reshape(-1)
    out = np.empty(flat.size, dtype=out_dtype)
    nchunks = (flat.size + CHUNK - 1) // CHUNK

    def run(c: int) -> None:
        out[c * CHUNK:(c + 1) * CHUNK] = fn(flat[c * CHUNK:(c + 1) * CHUNK])

    if nchunks <= 1:
        for c in range(nchunks):
            run(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(run, range(nchunks)))
    return out.reshape(np.shape(x))


def to_fp8(x: np.ndarray):
    """Per-tensor scaled E4M3: (codes, descale) with descale = amax / 448."""
    x = np.asarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    starts = range(0, flat.size, CHUNK)
    with ThreadPoolExecutor(_threads()) as ex:
        amax = max(ex.map(lambda i: float(np.max(np.abs(flat[i:i + CHUNK]))), starts), default=0.0)
    descale = np.float32(amax / E4M3_MAX if amax > 0 else 1.0)
    return _chunked(lambda c: f32_to_e4m3(c / descale), x, np.uint8), descale


def _maybe_bf16(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return f32_to_bf16(x)
    raise ValueError(f"dtype must be 'f32' or 'bf16', got {dtype!r}")


# --------------------------------------------------------------------------
# dense batched attention: q [B, Nq, Hq, d], k/v [B, Nk, Hkv, d]
# --------------------------------------------------------------------------
def dense_case(seed: int, batch: int, nq: int, nk: int, hq: int, hkv: int, d: int,
               dtype: str = "bf16", spike_frac: float = 0.0, spike_mult: float = 8.0) -> dict:
    """Seeded dense case.  ``spike_frac`` > 0 multiplies round(spike_frac*nk)
    key rows per (batch, head), chosen without replacement, by ``spike_mult``
    (a power of two, so the scaling is exact after rounding)."""
    q = normal_f32(seed, STREAM_Q, (batch, nq, hq, d))
    k = normal_f32(seed, STREAM_K, (batch, nk, hkv, d))
    v = normal_f32(seed, STREAM_V, (batch, nk, hkv, d))
    spikes = None
    if spike_frac > 0.0:
        nsp = int(round(spike_frac * nk))
        rng = np.random.default_rng([seed, 102])
        spikes = np.empty((batch, hkv, nsp), dtype=np.int64)
        for b in range(batch):
            for h in range(hkv):
                rows = np.sort(rng.choice(nk, size=nsp, replace=False))
                spikes[b, h] = rows
                k[b, rows, h, :] *= np.float32(spike_mult)
    return {
        "q": _maybe_bf16(q, dtype), "k": _maybe_bf16(k, dtype), "v": _maybe_bf16(v, dtype),
        "dtype": dtype, "batch": batch, "nq": nq, "nk": nk, "hq": hq, "hkv": hkv, "d": d,
        "spikes": spikes,
    }


def fp8_case(seed: int, batch: int, nq: int, nk: int, hq: int, hkv: int, d: int) -> dict:
    """Seeded dense case in FP8 E4M3 with per-tensor descale factors (the same
    float32 draws as ``dense_case``)."""
    q8, qd = to_fp8(normal_f32(seed, STREAM_Q, (batch, nq, hq, d)))
    k8, kd = to_fp8(normal_f32(seed, STREAM_K, (batch, nk, hkv, d)))
    v8, vd = to_fp8(normal_f32(seed, STREAM_V, (batch, nk, hkv, d)))
    return {"q": q8, "k": k8, "v": v8, "descale": (qd, kd, vd), "dtype": "fp8",
            "batch": batch, "nq": nq, "nk": nk, "hq": hq, "hkv": hkv, "d": d}


# --------------------------------------------------------------------------
# packed variable-length: q/k/v [T, H, d] with cu_seqlens [S+1]
# --------------------------------------------------------------------------
def varlen_lengths(seed: int, nseq: int, lo: int, hi: int) -> np.ndarray:
    """nseq integer lengths, uniform on [lo, hi] inclusive."""
    rng = np.random.default_rng([seed, 100])
    return rng.integers(lo, hi, size=nseq, endpoint=True).astype(np.int64)


def varlen_case(seed: int, lengths, hq: int, hkv: int, d: int, dtype: str = "bf16") -> dict:
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    t = int(cu[-1])
    q = normal_f32(seed, STREAM_Q, (t, hq, d))
    k = normal_f32(seed, STREAM_K, (t, hkv, d))
    v = normal_f32(seed, STREAM_V, (t, hkv, d))
    return {
        "q": _maybe_bf16(q, dtype), "k": _maybe_bf16(k, dtype), "v": _maybe_bf16(v, dtype),
        "cu_seqlens": cu, "lengths": lengths, "total": t, "max_seqlen": int(lengths.max(initial=0)),
        "dtype": dtype, "hq": hq, "hkv": hkv, "d": d,
    }


def fp8_varlen_case(seed: int, lengths, hq: int, hkv: int, d: int) -> dict:
    """Packed case in FP8 E4M3 with per-tensor descale factors (the same
    float32 draws as ``varlen_case``)."""
    c = varlen_case(seed, lengths, hq, hkv, d, dtype="f32")
    q8, qd = to_fp8(c["q"])
    k8, kd = to_fp8(c["k"])
    v8, vd = to_fp8(c["v"])
    c.update(q=q8, k=k8, v=v8, descale=(qd, kd, vd), dtype="fp8")
    return c


# --------------------------------------------------------------------------
# paged decode: q [B, Hq, d]; pools [num_blocks, Hkv, block, d]; table [B, max_blocks]
# --------------------------------------------------------------------------
def paged_case(seed: int, seq_lens, hq: int, hkv: int, d: int, block_size: int = 16,
               pad_blocks: int = 0) -> dict:
    """One query token per sequence over a shuffled block pool (bf16).

    num_blocks = sum(ceil(L/block)).  One seeded permutation of the pool
    indices is dealt out in order: sequence b receives the next ceil(L_b/block)
    entries.  Table slots past a sequence's last block hold -1.
    ``pad_blocks`` extra unused slots are appended to every table row.
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    nblk = (seq_lens + block_size - 1) // block_size
    num_blocks = int(nblk.sum())
    max_blocks = int(nblk.max(initial=0)) + int(pad_blocks)
    perm = np.random.default_rng([seed, 101]).permutation(num_blocks).astype(np.int32)
    table = np.full((len(seq_lens), max(1, max_blocks)), -1, dtype=np.int32)
    pos = 0
    for b, nb in enumerate(nblk):
        table[b, :nb] = perm[pos:pos + nb]
        pos += int(nb)
    q = normal_f32(seed, STREAM_Q, (len(seq_lens), hq, d))
    kp = normal_f32(seed, STREAM_K, (num_blocks, hkv, block_size, d))
    vp = normal_f32(seed, STREAM_V, (num_blocks, hkv, block_size, d))
    return {
        "q": f32_to_bf16(q), "k_pool": f32_to_bf16(kp), "v_pool": f32_to_bf16(vp),
        "block_table": table, "seq_lens": seq_lens.astype(np.int32), "num_blocks": num_blocks,
        "block_size": block_size, "hq": hq, "hkv": hkv, "d": d, "dtype": "bf16",
    }


def paged_fp8_case(seed: int, seq_lens, hq: int, hkv: int, d: int, block_size: int = 16,
                   pad_blocks: int = 0) -> dict:
    """``paged_case`` with the K and V pools in FP8 E4M3 (per-tensor descale
    amax/448 of the same float32 draws); q stays bf16."""
    c = paged_case(seed, seq_lens, hq, hkv, d, block_size=block_size, pad_blocks=pad_blocks)
    nb = c["num_blocks"]
    k8, kd = to_fp8(normal_f32(seed, STREAM_K, (nb, hkv, block_size, d)))
    v8, vd = to_fp8(normal_f32(seed, STREAM_V, (nb, hkv, block_size, d)))
    c.update(k_pool=k8, v_pool=v8, descale=(kd, vd), dtype="fp8")
    return c


def paged_prefill_case(seed: int, q_lens, k_lens, hq: int, hkv: int, d: int, block_size: int = 16,
                       pad_blocks: int = 0) -> dict:
    """Chunks of new queries over a shuffled block pool (bf16).

    Sequence s has k_lens[s] keys in the pool (laid out as in paged_case) and
    q_lens[s] new queries, packed into q [sum(q_lens), hq, d] with
    cu_seqlens_q.  The queries are drawn from a stream of their own, so the
    pool is the same as paged_case's for the same seed and k_lens.
    """
    c = paged_case(seed, k_lens, hq, hkv, d, block_size=block_size, pad_blocks=pad_blocks)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    cu = np.zeros(len(q_lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(q_lens)
    t = int(cu[-1])
    c["q"] = f32_to_bf16(normal_f32(seed, STREAM_QCHUNK, (t, hq, d)))
    c.update(cu_seqlens_q=cu, q_lens=q_lens, total_q=t, max_seqlen_q=int(q_lens.max(initial=0)),
             k_lens=np.asarray(k_lens, dtype=np.int64))
    return c


def paged_prefill_fp8_case(seed: int, q_lens, k_lens, hq: int, hkv: int, d: int, block_size: int = 16,
                           pad_blocks: int = 0) -> dict:
    """``paged_prefill_case`` in FP8 E4M3: the same float32 draws of the
    queries and pools, each tensor with its per-tensor descale amax/448."""
    c = paged_prefill_case(seed, q_lens, k_lens, hq, hkv, d, block_size=block_size, pad_blocks=pad_blocks)
    nb = c["num_blocks"]
    q8, qd = to_fp8(normal_f32(seed, STREAM_QCHUNK, (c["total_q"], hq, d)))
    k8, kd = to_fp8(normal_f32(seed, STREAM_K, (nb, hkv, block_size, d)))
    v8, vd = to_fp8(normal_f32(seed, STREAM_V, (nb, hkv, block_size, d)))
    c.update(q=q8, k_pool=k8, v_pool=v8, descale=(qd, kd, vd), dtype="fp8")
    return c


# --------------------------------------------------------------------------
# the five named workloads
# --------------------------------------------------------------------------
# --------------------------------------------------------------------------
# partial results to merge: o_parts [P, B, S, H, d], lse_parts [P, B, H, S]
# --------------------------------------------------------------------------
def merge_case(seed: int, parts: int, batch: int, seqlen: int, heads: int, d: int, dtype: str = "bf16",
               empty_frac: float = 0.0) -> dict:
    """Seeded partial attention results of the same rows over ``parts`` key
    shards: outputs N(0, 0.3^2) (a normalised output is a convex combination
    of value rows), log-sum-exps 4 + N(0, 2^2) (shards of a few hundred keys
    whose max scores differ by a few units).  A fraction ``empty_frac`` of
    (part, row) entries is marked as a shard that saw no key: lse -inf and
    an output row of NaN, which a merge must ignore."""
    o = normal_f32(seed, 201, (parts, batch, seqlen, heads, d)) * np.float32(0.3)
    lse = normal_f32(seed, 202, (parts, batch, heads, seqlen)) * np.float32(2.0) + np.float32(4.0)
    if empty_frac > 0.0:
        rng = np.random.default_rng([seed, 203])
        empty = rng.random((parts, batch, heads, seqlen)) < empty_frac
        lse[empty] = -np.inf
        o[np.transpose(empty, (0, 1, 3, 2))] = np.nan
    return {"o_parts": _maybe_bf16(o, dtype), "lse_parts": lse, "dtype": dtype, "parts": parts,
            "batch": batch, "seqlen": seqlen, "heads": heads, "d": d}


def workload(n: int) -> dict:
    """The five synthetic workloads (seed = workload number):

    1. fp32 single head, batch 1, N = 256, d = 64, non-causal;
    2. bf16 MHA causal prefill, batch 4, 32 heads, N = 2048, d = 128;
    3. bf16 causal prefill, batch 1, 32 heads, N = 8192, d = 128, 1% of key
       rows per head scaled by 8;
    4. bf16 causal varlen prefill, 16 sequences of length U{128..4096},
       32 heads, d = 64;
    5. bf16 paged GQA decode, batch 64, 32 q heads / 8 kv heads, d = 128,
       lengths U{1024..32768}, 16-token blocks.

    Beyond these: 6. bf16 chunked prefill over the paged pool, 16 sequences
    with contexts U{1024..8192}, each adding a causal chunk of its last 512
    tokens, 32 q heads / 8 kv heads, d = 128; 7. workload 2 in FP8 E4M3 with
    per-tensor descale factors; 8. workload 2 with attention dropout p = 0.1
    (the usual training rate), seed 8, offset 0; 9. bf16 causal GQA prefill
    at head_dim 256, batch 2, 16 q heads / 8 kv heads, N = 4096 (the shape of
    a head_dim-256 model's prefill); 10. bf16 paged GQA decode at head_dim
    256, batch 32, 16 q heads / 8 kv heads, lengths U{1024..16384}; 11.
    workload 5 with an FP8 E4M3 KV cache (per-tensor descale amax/448); 12.
    the merge of 8 key-shard results of workload 3's shape (batch 1,
    N = 8192, 32 heads, d = 128, bf16): what each GPU of an 8-way ring over
    the keys merges for its queries.
    """
    if n == 1:
        c = dense_case(1, 1, 256, 256, 1, 1, 64, dtype="f32")
        c.update(causal=False, name="fp32 single-head N=256 d=64")
        return c
    if n == 2:
        c = dense_case(2, 4, 2048, 2048, 32, 32, 128, dtype="bf16")
        c.update(causal=True, name="bf16 causal MHA prefill B=4 H=32 N=2048 d=128")
        return c
    if n == 3:
        c = dense_case(3, 1, 8192, 8192, 32, 32, 128, dtype="bf16", spike_frac=0.01)
        c.update(causal=True, name="bf16 causal prefill B=1 H=32 N=8192 d=128, 1% key rows x8")
        return c
    if n == 4:
        lens = varlen_lengths(4, 16, 128, 4096)
        c = varlen_case(4, lens, 32, 32, 64, dtype="bf16")
        c.update(causal=True, name="bf16 causal varlen prefill 16 seqs U{128..4096} H=32 d=64")
        return c
    if n == 5:
        lens = varlen_lengths(5, 64, 1024, 32768)
        c = paged_case(5, lens, 32, 8, 128, block_size=16)
        c.update(name="bf16 paged GQA decode B=64 Hq=32 Hkv=8 d=128 L~U{1024..32768} block 16")
        return c
    if n == 11:
        lens = varlen_lengths(5, 64, 1024, 32768)
        c = paged_fp8_case(5, lens, 32, 8, 128, block_size=16)
        c.update(name="fp8 kv paged GQA decode B=64 Hq=32 Hkv=8 d=128 L~U{1024..32768} block 16")
        return c
    if n == 10:
        lens = varlen_lengths(10, 32, 1024, 16384)
        c = paged_case(10, lens, 16, 8, 256, block_size=16)
        c.update(name="bf16 paged GQA decode B=32 Hq=16 Hkv=8 d=256 L~U{1024..16384} block 16")
        return c
    if n == 9:
        c = dense_case(9, 2, 4096, 4096, 16, 8, 256, dtype="bf16")
        c.update(causal=True, name="bf16 causal GQA prefill B=2 Hq=16 Hkv=8 N=4096 d=256")
        return c
    if n == 8:
        c = workload(2)
        c.update(dropout_p=0.1, seed=8, offset=0,
                 name="bf16 causal MHA prefill B=4 H=32 N=2048 d=128, dropout p=0.1")
        return c
    if n == 7:
        c = fp8_case(7, 4, 2048, 2048, 32, 32, 128)
        c.update(causal=True, name="fp8 e4m3 causal MHA prefill B=4 H=32 N=2048 d=128")
        return c
    if n == 12:
        c = merge_case(12, 8, 1, 8192, 32, 128, dtype="bf16")
        c.update(name="merge of 8 key-shard results B=1 N=8192 H=32 d=128 bf16")
        return c
    if n == 6:
        k_lens = varlen_lengths(6, 16, 1024, 8192)
        c = paged_prefill_case(6, np.full(16, 512), k_lens, 32, 8, 128, block_size=16)
        c.update(causal=True,
                 name="bf16 chunked paged prefill 16 seqs ctx U{1024..8192} chunk 512 Hq=32 Hkv=8 d=128")
        return c
    raise ValueError(f"no workload {n}")
