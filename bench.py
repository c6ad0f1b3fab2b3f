#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one fa_fwd call on the headline workload: bf16 causal MHA prefill,
batch 4, 32 heads, N = 2048, d = 128 (seeded synthetic N(0,1) inputs,
already resident in HBM).  Each workload first runs its step untimed for
0.3 s (the clock ramps up under sustained load), then W warm-up steps, then
K steps timed between barrier + synchronisation with HIP events on the
launch stream.  The paged GQA decode
workload (batch 64, 32/8 heads, d = 128, lengths U{1024..32768}) is timed the
same way and reported in "decode"; the long-context, varlen, chunked paged
prefill, FP8 prefill, dropout prefill and head_dim 256 prefill workloads are
reported in "extra" (FP8 against the 5.0 PFLOP/s dense fp8 peak), as is a
head_dim 256 paged decode workload, the paged decode workload over an FP8
KV cache and the merge of 8 key-shard results of the long-context shape
(GB/s).

One JSON line is printed.  "roofline" is the prefill kernel's algorithmic
TFLOP/s (4*d flops per visible query/key pair) against the 2.5 PFLOP/s dense
bf16 MFMA peak; "cpu_baseline" is the fp64 oracle timed on this host's cores
on a bounded sample of the same workload's rows, and "parity" compares the
outputs the timed steps left behind with the oracle on sampled rows (the
oracle runs only in that final leg, after all GPU timing).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "prefill": ["exact_io_aware_tile_amd/csrc/fa_fwd_bf16.hip"],
    "long": ["exact_io_aware_tile_amd/csrc/fa_fwd_bf16.hip"],
    "decode": ["exact_io_aware_tile_amd/csrc/fa_decode.hip"],
    "chunked": ["exact_io_aware_tile_amd/csrc/fa_fwd_bf16.hip"],
    "fp8": ["exact_io_aware_tile_amd/csrc/fa_fwd_fp8.hip"],
    "dropout": ["exact_io_aware_tile_amd/csrc/fa_fwd_bf16.hip"],
    "d256": ["exact_io_aware_tile_amd/csrc/fa_fwd_bf16_d256.hip"],
    "varlen": ["exact_io_aware_tile_amd/csrc/fa_fwd_bf16.hip"],
    "decode_d256": ["exact_io_aware_tile_amd/csrc/fa_decode.hip"],
    "decode_fp8": ["exact_io_aware_tile_amd/csrc/fa_decode.hip"],
    "merge": ["exact_io_aware_tile_amd/csrc/fa_merge.hip"],
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall-clock budget of the oracle CPU baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--only", nargs="+", choices=["prefill", "decode", "long", "varlen", "chunked", "fp8", "dropout",
                                                 "d256", "decode_d256", "decode_fp8", "merge", "copy"],
                    default=None,
                    help="run only these workloads and print one JSON line each (for profiler "
                         "runs); 'copy' runs a plain 1 GiB device copy used to calibrate the "
                         "HBM byte counters")
    return ap.parse_args()


def sources_digest(kind: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind] + ["exact_io_aware_tile_amd/csrc/fa_device.h",
                                       "exact_io_aware_tile_amd/csrc/fa_internal.h"]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kind: str):
    """HBM bytes per launch from the committed counter summary, or None when
    the summary is absent or the kernel source changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)[kind]
    except (OSError, KeyError, ValueError):
        return None
    if t.get("source_digest") != sources_digest(kind):
        return None
    return t.get("bytes_per_launch")


def bf16_dev(a, torch, np):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


INPUT_KEYS = ("q", "k", "v", "k_pool", "v_pool", "block_table", "seq_lens", "cu_seqlens", "cu_seqlens_q",
              "o_parts", "lse_parts")


def input_digest(case) -> str:
    """sha256 of the host bytes of every input array of a workload (the bytes
    copied to the device), in INPUT_KEYS order."""
    import numpy as np
    h = hashlib.sha256()
    for key in INPUT_KEYS:
        a = case.get(key)
        if isinstance(a, np.ndarray):
            h.update(key.encode())
            h.update(np.ascontiguousarray(a).view(np.uint8).reshape(-1).data)
    return h.hexdigest()


SETTLE_S = 0.3  # untimed seconds of the same step before the warm-up steps


def time_steps(fn, steps, warmup, torch):
    # The GPU leaves its idle clock only after some time under load (the
    # inputs are built on the host for seconds before); the same step runs
    # untimed for SETTLE_S seconds so that the timed steps see the clock of
    # sustained work, then the W warm-up steps, then exactly K timed steps.
    t_end = time.perf_counter() + SETTLE_S
    while time.perf_counter() < t_end:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t0.record(stream)
    for _ in range(steps):
        fn()
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    return t0.elapsed_time(t1) / steps, wall / steps * 1e3  # ms per step (events, wall)


def time_cold(fn, reps, torch, flush):
    """Per-launch HIP-event times (ms) with a write of FLUSH (larger than the
    256 MB last-level cache) between launches, outside the timed window."""
    stream = torch.cuda.current_stream()
    times = []
    for r in range(reps):
        flush.fill_(r & 0x7F)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        fn()
        t1.record(stream)
        torch.cuda.synchronize()
        times.append(t0.elapsed_time(t1))
    times.sort()
    return times[0], times[len(times) // 2]


def copy_bandwidth(torch, reps=10):
    """Device-to-device copy of 1 GiB: bytes read + written per second (GB/s),
    a measured ceiling for a streaming kernel on this GPU."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(reps):
        b.copy_(a)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps
    del a, b
    return 2 * n / (ms * 1e-3) / 1e9


def prefill_flops(case) -> float:
    d, B, H = case["d"], case["batch"], case["hq"]
    nq, nk = case["nq"], case["nk"]
    if case["causal"]:
        pairs = sum(max(0, min(nk, i + (nk - nq) + 1)) for i in range(nq))
    else:
        pairs = nq * nk
    return 4.0 * d * pairs * B * H


def edge_rows(rng, heads, n, extra):
    """Row ids h*n + i (of one sequence of n rows over `heads` heads): random
    rows plus rows at the edges of 64- and 256-row tiles and the last rows."""
    ids = set(rng.integers(0, heads * n, size=extra).tolist())
    for i in (0, 1, 63, 64, 255, 256, n - 257, n - 256, n - 65, n - 64, n - 2, n - 1):
        if 0 <= i < n:
            ids.add(int(rng.integers(0, heads)) * n + i)
    return np.array(sorted(ids), dtype=np.int64)


def parity_stats(o_gpu, lse_gpu, o_ref, lse_ref, max_tol=2e-2, mean_tol=2e-3, lse_tol=1e-3):
    err = np.abs(o_gpu - o_ref)
    fin = np.isfinite(lse_ref)
    lerr = np.abs(lse_gpu[fin] - lse_ref[fin])
    finite_ok = bool(np.isfinite(o_gpu).all() and (np.isfinite(lse_gpu) == fin).all())
    st = {"rows": int(o_gpu.shape[0]), "max_abs_do": float(err.max()), "mean_abs_do": float(err.mean()),
          "max_abs_dlse": float(lerr.max()) if lerr.size else 0.0}
    st["within_contract"] = bool(finite_ok and st["max_abs_do"] <= max_tol and st["mean_abs_do"] <= mean_tol
                                 and st["max_abs_dlse"] <= lse_tol)
    return st


def oracle_leg(legs, seconds):
    """The only part of the bench that runs the fp64 oracle (test
    infrastructure, never on the measured path), after all GPU timing:

    * cpu_baseline: the oracle, untuned, timed on this host's cores on random
      query rows of the headline workload for about `seconds`;
    * parity: the outputs the timed GPU steps left in their buffers, compared
      with the oracle on sampled rows (the baseline's own rows for the
      headline, plus tile edges; a bounded sample for the other legs)."""
    import oracle
    threads = oracle.threads(0)
    try:
        threads = oracle.threads(len(os.sched_getaffinity(0)))
    except AttributeError:
        pass
    parity = {}
    base = None
    for key, (case, res) in legs.items():
        outs = res.get("outputs")
        if outs is None:
            continue
        og, lg = outs
        rng = np.random.default_rng(1234)
        if key == "prefill":
            B, N, H, d = case["batch"], case["nq"], case["hq"], case["d"]
            o_rows = og.reshape(B, N, H, d).transpose(0, 2, 1, 3).reshape(B * H * N, d)
            l_rows = lg.reshape(-1)
            flops, done, errs = 0.0, [], []
            t0 = time.perf_counter()
            first = True
            while first or time.perf_counter() - t0 < seconds:
                rows = rng.integers(0, B * H * N, size=256)
                if first:  # tile edges of a random (b, h)
                    bh = int(rng.integers(0, B * H))
                    rows = np.concatenate([rows, bh * N + edge_rows(rng, 1, N, 0)])
                first = False
                o_ref, l_ref = oracle.dense(case["q"], case["k"], case["v"], causal=True, rows=rows,
                                            nthreads=threads)
                flops += float(4.0 * d * (rows % N + 1).sum())
                done.append(rows)
                errs.append((o_rows[rows], l_rows[rows], o_ref, l_ref))
            el = time.perf_counter() - t0
            n_rows = int(sum(r.size for r in done))
            n_distinct = int(np.unique(np.concatenate(done)).size)
            base = {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
                    "sample": f"{n_rows} query rows ({n_distinct} distinct) drawn uniformly with replacement, "
                              f"256 at a time, from the workload's {B * H * N} (b, h, i) rows, plus each batch's "
                              f"tile-edge rows; fp64 materialised-score oracle, {el:.1f} s wall"}
            parity[key] = parity_stats(*(np.concatenate([e[i] for e in errs]) for i in range(4)))
        elif key == "long":
            B, N, H, d = case["batch"], case["nq"], case["hq"], case["d"]
            rows = edge_rows(rng, B * H, N, 192)
            o_rows = og.reshape(B, N, H, d).transpose(0, 2, 1, 3).reshape(B * H * N, d)
            o_ref, l_ref = oracle.dense(case["q"], case["k"], case["v"], causal=True, rows=rows, nthreads=threads)
            parity[key] = parity_stats(o_rows[rows], lg.reshape(-1)[rows], o_ref, l_ref)
        elif key == "varlen":
            T, H, d = case["total"], case["hq"], case["d"]
            rows = set(rng.integers(0, H * T, size=256).tolist())
            cu = case["cu_seqlens"]
            for sq in range(len(cu) - 1):
                for t in (cu[sq], cu[sq + 1] - 1):
                    rows.add(int(rng.integers(0, H)) * T + int(t))
            rows = np.array(sorted(rows), dtype=np.int64)
            o_rows = og.reshape(T, H, d).transpose(1, 0, 2).reshape(H * T, d)
            o_ref, l_ref = oracle.varlen(case["q"], case["k"], case["v"], cu, causal=True, rows=rows,
                                         nthreads=threads)
            parity[key] = parity_stats(o_rows[rows], lg.reshape(-1)[rows], o_ref, l_ref)
        elif key == "decode":
            B, H, d = case["q"].shape
            rows = np.array(sorted(set(rng.integers(0, B * H, size=128).tolist())), dtype=np.int64)
            o_ref, l_ref = oracle.decode_paged(case["q"], case["k_pool"], case["v_pool"], case["block_table"],
                                               case["seq_lens"], rows=rows, nthreads=threads)
            parity[key] = parity_stats(og.reshape(B * H, d)[rows], lg.reshape(-1)[rows], o_ref, l_ref)
    return base, parity


def host_outputs(o, lse):
    """The timed steps' output buffers, copied to the host as float64."""
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def run_prefill(fa, case, steps, warmup, torch, np, kind, flush=None):
    q, k, v = (bf16_dev(case[n], torch, np) for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty((case["batch"], case["hq"], case["nq"]), dtype=torch.float32, device="cuda")

    if "dropout_p" in case:
        def step():
            fa.fa_fwd_dropout(q, k, v, dropout_p=case["dropout_p"], seed=case["seed"], offset=case["offset"],
                              causal=case["causal"], out=o, lse=lse)
    else:
        def step():
            fa.fa_fwd(q, k, v, causal=case["causal"], out=o, lse=lse)

    ms, wall_ms = time_steps(step, steps, warmup, torch)
    outputs = host_outputs(o, lse) if kind in ("prefill", "long") else None
    flops = prefill_flops(case)
    tf = flops / (ms * 1e-3) / 1e12
    traffic = measured_traffic(kind)
    cold = None
    if flush is not None:
        mn, med = time_cold(step, 20, torch, flush)
        cold = {"min_us": round(mn * 1e3, 1), "median_us": round(med * 1e3, 1),
                "tflops_at_min": round(flops / (mn * 1e-3) / 1e12, 2),
                "tflops_at_median": round(flops / (med * 1e-3) / 1e12, 2)}
    return {
        "ms": ms, "wall_ms": wall_ms, "tflops": tf, "flops": flops, "cold": cold, "outputs": outputs,
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": traffic},
    }


def run_varlen(fa, case, steps, warmup, torch, np):
    q, k, v = (bf16_dev(case[n], torch, np) for n in ("q", "k", "v"))
    cu = torch.from_numpy(case["cu_seqlens"]).cuda()
    o = torch.empty_like(q)
    lse = torch.empty((case["hq"], case["total"]), dtype=torch.float32, device="cuda")

    def step():
        fa.fa_fwd_varlen(q, k, v, cu, case["max_seqlen"], causal=True, out=o, lse=lse)

    ms, wall_ms = time_steps(step, steps, warmup, torch)
    lens = case["lengths"].astype(np.float64)
    flops = float(4.0 * case["d"] * case["hq"] * (lens * (lens + 1) / 2).sum())
    tf = flops / (ms * 1e-3) / 1e12
    return {"ms": ms, "tflops": tf, "flops": flops, "outputs": host_outputs(o, lse),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                         "traffic": measured_traffic("varlen")}}


def run_paged_prefill(fa, case, steps, warmup, torch, np):
    q = bf16_dev(case["q"], torch, np)
    kp = bf16_dev(case["k_pool"], torch, np)
    vp = bf16_dev(case["v_pool"], torch, np)
    bt = torch.from_numpy(case["block_table"]).cuda()
    cu = torch.from_numpy(case["cu_seqlens_q"]).cuda()
    sl = torch.from_numpy(case["seq_lens"]).cuda()
    maxk = int(case["seq_lens"].max())
    o = torch.empty_like(q)
    lse = torch.empty((case["hq"], case["total_q"]), dtype=torch.float32, device="cuda")

    def step():
        fa.fa_fwd_paged(q, kp, vp, bt, cu, sl, case["max_seqlen_q"], maxk, causal=True, out=o, lse=lse)

    ms, wall_ms = time_steps(step, steps, warmup, torch)
    pairs = 0
    for nq, nk in zip(case["q_lens"].tolist(), case["k_lens"].tolist()):
        i = np.arange(nq, dtype=np.int64)
        pairs += int(np.clip(i + (nk - nq) + 1, 0, nk).sum())
    flops = 4.0 * case["d"] * case["hq"] * pairs
    tf = flops / (ms * 1e-3) / 1e12
    return {"ms": ms, "tflops": tf, "flops": flops,
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                         "traffic": measured_traffic("chunked")}}


def run_fp8(fa, case, steps, warmup, torch, np):
    q, k, v = (torch.from_numpy(case[n]).cuda() for n in ("q", "k", "v"))
    o = torch.empty(case["q"].shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((case["batch"], case["hq"], case["nq"]), dtype=torch.float32, device="cuda")

    def step():
        fa.fa_fwd_fp8(q, k, v, case["descale"], causal=case["causal"], out=o, lse=lse)

    ms, wall_ms = time_steps(step, steps, warmup, torch)
    flops = prefill_flops(case)
    tf = flops / (ms * 1e-3) / 1e12
    return {"ms": ms, "tflops": tf, "flops": flops,
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_FP8_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_FP8_TFLOPS, 4),
                         "traffic": measured_traffic("fp8")}}


def run_decode(fa, case, steps, warmup, torch, np, flush=None, kind="decode"):
    kv8 = case["dtype"] == "fp8"
    q = bf16_dev(case["q"], torch, np)
    kp = torch.from_numpy(case["k_pool"]).cuda() if kv8 else bf16_dev(case["k_pool"], torch, np)
    vp = torch.from_numpy(case["v_pool"]).cuda() if kv8 else bf16_dev(case["v_pool"], torch, np)
    bt = torch.from_numpy(case["block_table"]).cuda()
    sl = torch.from_numpy(case["seq_lens"]).cuda()
    maxlen = int(case["seq_lens"].max())
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    if kv8:
        ws = torch.empty(fa.fa_decode_paged_fp8_workspace_size(q, kp, vp, bt, sl, maxlen, case["descale"]),
                         dtype=torch.uint8, device="cuda")
        splits = fa.fa_decode_paged_fp8_num_splits(q, kp, vp, bt, sl, maxlen, case["descale"])
    else:
        ws = torch.empty(fa.fa_decode_paged_workspace_size(q, kp, vp, bt, sl, maxlen), dtype=torch.uint8,
                         device="cuda")
        splits = fa.fa_decode_paged_num_splits(q, kp, vp, bt, sl, maxlen)

    if kv8:
        def step():
            fa.fa_decode_paged_fp8(q, kp, vp, bt, sl, maxlen, case["descale"], out=o, lse=lse, workspace=ws)
    else:
        def step():
            fa.fa_decode_paged(q, kp, vp, bt, sl, maxlen, out=o, lse=lse, workspace=ws)

    ms, wall_ms = time_steps(step, steps, warmup, torch)
    outputs = host_outputs(o, lse) if kind == "decode" else None
    L = case["seq_lens"].astype(np.int64)
    hkv, d, bs = case["hkv"], case["d"], case["block_size"]
    kv_bytes = float(2 * hkv * d * (1 if kv8 else 2) * L.sum())
    other = float(q.numel() * 2 + o.numel() * 2 + 4 * ((L + bs - 1) // bs).sum() + 4 * L.size)
    nbytes = kv_bytes + other
    gbs = nbytes / (ms * 1e-3) / 1e9
    traffic = measured_traffic(kind)
    cold = None
    if flush is not None:
        mn, med = time_cold(step, 20, torch, flush)
        cold = {"min_us": round(mn * 1e3, 1), "median_us": round(med * 1e3, 1),
                "gbs_at_median": round(nbytes / (med * 1e-3) / 1e9, 1)}
    return {"ms": ms, "gbs": gbs, "bytes": nbytes, "kv_bytes": kv_bytes, "num_splits": splits, "cold": cold,
            "outputs": outputs,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic}}


def run_merge(fa, case, steps, warmup, torch, np):
    """Merge of P key-shard results: algorithmic bytes = P x (output rows +
    their lse) read + one output (rows + lse) written."""
    o_parts = bf16_dev(case["o_parts"], torch, np)
    lse_parts = torch.from_numpy(case["lse_parts"]).cuda()
    P, B, S, H, D = case["o_parts"].shape
    o = torch.empty((B, S, H, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")

    def step():
        fa.fa_merge_states(o_parts, lse_parts, out=o, lse=lse)

    ms, _ = time_steps(step, steps, warmup, torch)
    rows = B * S * H
    nbytes = float((P + 1) * rows * (2 * D + 4))
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"ms": ms, "gbs": gbs, "bytes": nbytes,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": measured_traffic("merge")}}


def run_copy(torch, steps):
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    for _ in range(max(1, steps)):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": max(1, steps)}))


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only; --gpus must be 1 "
                                   f"(got {args.gpus}). Multi-GPU sharding is described, not built."}))
        sys.exit(2)
    import numpy as np
    import torch

    from exact_io_aware_tile_amd import fa, inputs

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    fa.lib()
    torch.cuda.set_device(0)

    only = set(args.only or [])

    def want(name, default=True):
        return name in only if only else default

    out = {}
    # 512 MB written between cold launches (outside their timed window) so
    # that no input stays in the 256 MB last-level cache.
    flush = None if only else torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    if want("prefill"):
        case = inputs.workload(2)
        res = run_prefill(fa, case, args.steps, args.warmup, torch, np, "prefill", flush)
        out["prefill"] = (case, res)
    if want("long", not args.no_extra):
        case = inputs.workload(3)
        out["long"] = (case, run_prefill(fa, case, max(5, args.steps // 5), max(2, args.warmup // 5), torch, np,
                                         "long", flush))
    if want("varlen", not args.no_extra):
        case = inputs.workload(4)
        out["varlen"] = (case, run_varlen(fa, case, max(5, args.steps // 2), max(2, args.warmup // 2), torch, np))
    if want("chunked", not args.no_extra):
        case = inputs.workload(6)
        out["chunked"] = (case, run_paged_prefill(fa, case, max(5, args.steps // 2), max(2, args.warmup // 2),
                                                  torch, np))
    if want("fp8", not args.no_extra):
        case = inputs.workload(7)
        out["fp8"] = (case, run_fp8(fa, case, args.steps, args.warmup, torch, np))
    if want("dropout", not args.no_extra):
        case = inputs.workload(8)
        out["dropout"] = (case, run_prefill(fa, case, args.steps, args.warmup, torch, np, "dropout"))
    if want("d256", not args.no_extra):
        case = inputs.workload(9)
        out["d256"] = (case, run_prefill(fa, case, max(5, args.steps // 2), max(2, args.warmup // 2), torch, np,
                                         "d256"))
    if want("decode_d256", not args.no_extra):
        case = inputs.workload(10)
        out["decode_d256"] = (case, run_decode(fa, case, args.steps, args.warmup, torch, np, kind="decode_d256"))
    if want("decode_fp8", not args.no_extra):
        case = inputs.workload(11)
        out["decode_fp8"] = (case, run_decode(fa, case, args.steps, args.warmup, torch, np, kind="decode_fp8"))
    if want("merge", not args.no_extra):
        case = inputs.workload(12)
        out["merge"] = (case, run_merge(fa, case, args.steps, args.warmup, torch, np))
    if want("decode", not args.no_decode):
        case = inputs.workload(5)
        out["decode"] = (case, run_decode(fa, case, args.steps, args.warmup, torch, np, flush))
    if want("copy", False):
        run_copy(torch, args.steps)

    if only:
        for k, (case, res) in out.items():
            print(json.dumps({"workload": case["name"],
                              **{a: b for a, b in res.items() if a not in ("roofline", "outputs")},
                              "roofline": res["roofline"]}))
        return

    case, res = out["prefill"]
    line = {
        "metric": "attn fwd TFLOP/s (% bf16 MFMA peak); paged decode HBM GB/s (% peak)",
        "value": round(res["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["wall_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), resident in HBM)",
        "config": {"workload": case["name"], "batch": case["batch"], "heads": case["hq"],
                   "seq_len": case["nq"], "head_dim": case["d"], "causal": True,
                   "algorithmic_gflop_per_step": round(res["flops"] / 1e9, 3)},
        "roofline": res["roofline"],
        "kernel_ms": round(res["ms"], 4),
        "basis": "warm: K back-to-back launches on one stream, inputs resident in HBM (201 MB of q/k/v, "
                 "which the 256 MB last-level cache can hold); 'cold' times single launches after a 512 MB "
                 "device write evicted that cache",
        "cold": res["cold"],
        "inputs": {"seed": 2, "sha256": input_digest(case),
                   "recipe": "numpy default_rng([seed, stream, chunk]) N(0,1) float32, RNE to bf16"},
    }
    if "decode" in out:
        dcase, dres = out["decode"]
        line["decode"] = {"workload": dcase["name"], "value": round(dres["gbs"], 1), "unit": "GB/s",
                          "ms_per_step": round(dres["ms"], 4), "algorithmic_bytes": dres["bytes"],
                          "num_splits": dres["num_splits"], "roofline": dres["roofline"], "cold": dres["cold"],
                          "inputs": {"seed": 5, "sha256": input_digest(dcase)}}
        del flush
        flush = None
        line["decode"]["copy_gbs"] = round(copy_bandwidth(torch), 1)
    extra = []
    seeds = {"long": 3, "varlen": 4, "chunked": 6, "fp8": 7, "dropout": 8, "d256": 9, "decode_d256": 10,
             "decode_fp8": 11, "merge": 12}
    for key in ("long", "varlen", "chunked", "fp8", "dropout", "d256", "decode_d256", "decode_fp8", "merge"):
        if key in out:
            c, r = out[key]
            if "gbs" in r:
                e = {"workload": c["name"], "value": round(r["gbs"], 1), "unit": "GB/s",
                     "ms_per_step": round(r["ms"], 4), "roofline": r["roofline"]}
            else:
                e = {"workload": c["name"], "value": round(r["tflops"], 2), "unit": "TFLOP/s",
                     "ms_per_step": round(r["ms"], 4), "roofline": r["roofline"]}
            if r.get("cold"):
                e["cold"] = r["cold"]
            e["inputs"] = {"seed": seeds[key], "sha256": input_digest(c)}
            extra.append(e)
    if extra:
        line["extra"] = extra
    line["context"] = ("pages' figures (other hardware): 2-4x wall-clock over standard attention; "
                       "FlashAttention-1 25-40% and FlashAttention-2 50-73% of A100 peak")
    if not args.no_cpu_baseline:
        base, parity = oracle_leg(out, args.cpu_seconds)
        line["cpu_baseline"] = base
        line["parity"] = {"what": "the timed steps' outputs against the fp64 oracle on sampled rows "
                                  "(contract: max |dO| <= 2e-2, mean |dO| <= 2e-3, max |dLSE| <= 1e-3)",
                          **parity}
    print(json.dumps(line))


if __name__ == "__main__":
    main()
