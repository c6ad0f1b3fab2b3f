"""The pages' online-softmax method in fp64 on the CPU -- TEST INFRASTRUCTURE ONLY.

These helpers follow the method's steps in the pages' order and notation so
that tests can show, on the CPU and in double precision, that the method
reaches the oracle's textbook definition (to ~1e-15, as the "Run it locally"
note of "S12 FlashAttention" expects) for any tile size, through a block
table, and when the keys are split across workers and merged.  The GPU
kernels do not use this module.

Sources (page titles and sections):
* "S12 FlashAttention" (llminference.xinbetween.com), "Core idea / The
  solution": per tile, m_new = max(m, max s); alpha = exp(m - m_new);
  p = exp(s - m_new); l = alpha*l + sum p; o = alpha*o + p @ v; final o / l.
* same page, "Build it / Implementation": the paged loop puts a block table
  in front of the key access; a block holds n = min(block, seq_len -
  logical*block) keys and the walk stops when n <= 0.  The callout
  "exp(-inf - -inf) is NaN" describes the fully masked first tile and the
  guard.
* same page, "What this unlocks beyond speed" (flash-decoding) and
  "Exercises" 1: split the keys across workers and combine their (m, l, o).
* "FlashAttention" (tachyon.techntrek.in/learn/flash-attention), "For
  engineers / Show the maths": m_new = max(m, m~),
  l_new = e^(m - m_new) l + e^(m~ - m_new) l~.
"""
from __future__ import annotations

import numpy as np


def init_state(d: int):
    """(m, l, o) before any key: m = -inf, l = 0, o = 0."""
    return -np.inf, 0.0, np.zeros(d, dtype=np.float64)


def update(state, s, v_tile, guard: bool = True):
    """One tile of the recurrence.  s: scaled scores of the tile (masked keys
    are -inf); v_tile: the tile's value rows.

    With guard=False this is the recurrence exactly as printed, which turns
    into NaN when the running max and the tile max are both -inf.  With
    guard=True a tile whose every key is masked leaves the state unchanged.
    """
    m, l, o = state
    s = np.asarray(s, dtype=np.float64)
    m_new = max(m, float(np.max(s))) if s.size else m
    if guard and m_new == -np.inf:
        return state
    with np.errstate(invalid="ignore"):
        alpha = np.exp(m - m_new)
        p = np.exp(s - m_new)
    l = alpha * l + p.sum()
    o = alpha * o + p @ np.asarray(v_tile, dtype=np.float64)
    return m_new, l, o


def finish(state):
    """o / l and the log-sum-exp m + ln l (a row with no visible key: 0, -inf)."""
    m, l, o = state
    if l == 0.0:
        return np.zeros_like(o), -np.inf
    return o / l, m + np.log(l)


def flash_row(q, k, v, tile: int, scale: float, visible=None, guard: bool = True):
    """Tiled online softmax for one query row.  visible: optional bool mask
    over keys.  Returns (o, lse)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    state = init_state(v.shape[1])
    for start in range(0, k.shape[0], tile):
        s = (k[start:start + tile] @ q) * scale
        if visible is not None:
            s = np.where(visible[start:start + tile], s, -np.inf)
        state = update(state, s, v[start:start + tile], guard=guard)
    return finish(state)


def paged_row(q, block_table, k_cache, v_cache, seq_len: int, block_size: int, scale: float):
    """The paged loop: the same recurrence with a block table in front of the
    key access.  k_cache / v_cache: [num_blocks, block_size, d]."""
    q = np.asarray(q, dtype=np.float64)
    state = init_state(k_cache.shape[-1])
    for logical, physical in enumerate(block_table):
        n = min(block_size, seq_len - logical * block_size)
        if n <= 0:
            break
        k_blk = np.asarray(k_cache[physical, :n], dtype=np.float64)
        v_blk = np.asarray(v_cache[physical, :n], dtype=np.float64)
        state = update(state, (k_blk @ q) * scale, v_blk)
    return finish(state)


def merge(a, b):
    """Combine two (m, l, o) states: rescale both to the larger max and add."""
    m1, l1, o1 = a
    m2, l2, o2 = b
    m = max(m1, m2)
    if m == -np.inf:
        return a
    w1, w2 = np.exp(m1 - m), np.exp(m2 - m)
    return m, w1 * l1 + w2 * l2, w1 * o1 + w2 * o2


def split_row(q, k, v, workers: int, tile: int, scale: float):
    """Flash-decoding: contiguous key ranges per worker, each runs the
    recurrence alone, then the partial states are merged."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = k.shape[0]
    bounds = np.linspace(0, n, workers + 1).round().astype(int)
    parts = []
    for w in range(workers):
        st = init_state(v.shape[1])
        for start in range(bounds[w], bounds[w + 1], tile):
            stop = min(start + tile, bounds[w + 1])
            st = update(st, (k[start:stop] @ q) * scale, v[start:stop])
        parts.append(st)
    total = init_state(v.shape[1])
    for p in parts:
        total = merge(total, p)
    return finish(total)


def tile_stats(scores, tile: int):
    """For a row of (already scaled) scores: per tile, the tile's own
    (m~, l~) and the running (m, l) after it."""
    scores = np.asarray(scores, dtype=np.float64)
    out = []
    m, l = -np.inf, 0.0
    for start in range(0, scores.size, tile):
        s = scores[start:start + tile]
        mt = float(s.max())
        lt = float(np.exp(s - mt).sum())
        m_new = max(m, mt)
        l = np.exp(m - m_new) * l + np.exp(mt - m_new) * lt
        m = m_new
        out.append({"m_tile": mt, "l_tile": lt, "m": m, "l": float(l)})
    return out
