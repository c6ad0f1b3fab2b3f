"""The pages' online-softmax method in fp64 on the CPU -- TEST INFRASTRUCTURE ONLY.

The tests use these helpers to show, on the CPU and in double precision,
that the streaming method reaches the oracle's textbook definition (to
~1e-15, the agreement the "Run it locally" note of "S12 FlashAttention"
expects) for any tile size, through a block table, and when the keys are
split across workers and the partial states merged.  The GPU kernels do not
use this module, and it does not use them.

What is computed (page titles and sections):
* "S12 FlashAttention" (llminference.xinbetween.com), "Core idea / The
  solution": a state (running max m, running sum l, unnormalised output o)
  absorbs one key tile at a time -- m moves to the larger of m and the
  tile's max, the old l and o shrink by exp(m_old - m_new), the tile's
  weights exp(s - m_new) add to l and their value-weighted sum to o -- and
  the result is o / l.
* same page, "Build it / Implementation": a block table sits in front of the
  key access, a block holding min(block, seq_len - i*block) keys; its callout
  "exp(-inf - -inf) is NaN" is the fully masked first tile and its guard.
* same page, "What this unlocks beyond speed" and "Exercises" 1: split one
  row's keys across workers and combine their states.
* "FlashAttention" (tachyon.techntrek.in/learn/flash-attention), "For
  engineers / Show the maths": two states combine by rescaling both to the
  larger max and adding.

Layout here: a state covers R query rows at once -- ``mx`` [R], ``total``
[R], ``acc`` [R, d] -- and a tile's scores arrive as an [R, n] matrix, so one
call advances every row.  One-row helpers wrap that with R = 1.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass
class Rows:
    """Streaming state of R query rows: running max, running sum of
    exp(score - max), and the value rows summed under the same weights."""
    mx: np.ndarray     # [R]
    total: np.ndarray  # [R]
    acc: np.ndarray    # [R, d]


def empty(rows: int, d: int) -> Rows:
    """The state before any key: max -inf, nothing summed."""
    return Rows(np.full(rows, -np.inf), np.zeros(rows), np.zeros((rows, d)))


def absorb(st: Rows, scores, values, guard: bool = True) -> Rows:
    """Advance every row by one key tile.  ``scores`` [R, n]: the tile's scaled
    scores, -inf for a key the row may not see; ``values`` [n, d].

    guard=False applies the update as the pages write it, which yields NaN in
    a row whose running max and tile max are both -inf (0 * exp(nan)).  With
    guard=True such a row keeps its state: a tile the row cannot see adds
    nothing.
    """
    s = np.atleast_2d(np.asarray(scores, dtype=np.float64))
    vals = np.asarray(values, dtype=np.float64).reshape(s.shape[1], -1)
    if s.shape[1] == 0:
        return st
    new_mx = np.maximum(st.mx, s.max(axis=1))
    with np.errstate(invalid="ignore"):
        shrink = np.exp(st.mx - new_mx)            # alpha of every row
        w = np.exp(s - new_mx[:, None])            # the tile's weights
    total = shrink * st.total + w.sum(axis=1)
    acc = shrink[:, None] * st.acc + w @ vals
    if guard:
        dead = new_mx == -np.inf
        total = np.where(dead, st.total, total)
        acc = np.where(dead[:, None], st.acc, acc)
    return Rows(new_mx, total, acc)


def readout(st: Rows):
    """(O, LSE) of every row: acc / total and mx + ln(total); a row that saw
    no key (total exactly 0) reads 0 and -inf.  NaN passes through."""
    seen = st.total != 0
    with np.errstate(divide="ignore", invalid="ignore"):
        o = np.where(seen[:, None], st.acc / np.where(seen, st.total, 1.0)[:, None], 0.0)
        lse = np.where(seen, st.mx + np.log(np.where(seen, st.total, 1.0)), -np.inf)
    return o, lse


def combine(a: Rows, b: Rows) -> Rows:
    """Merge two states of the same rows over disjoint key sets."""
    top = np.maximum(a.mx, b.mx)
    ref = np.where(top == -np.inf, 0.0, top)     # rows neither state has seen stay empty
    wa, wb = np.exp(a.mx - ref), np.exp(b.mx - ref)
    return Rows(top, wa * a.total + wb * b.total, wa[:, None] * a.acc + wb[:, None] * b.acc)


def stream(q, k, v, tile: int, scale: float, visible=None, guard: bool = True):
    """Tiled attention of the rows of ``q`` [R, d] (or one row [d]) over keys
    ``k``, values ``v`` [n, d], taking ``tile`` keys per step.  ``visible``:
    optional bool mask [R, n] (or [n] for one row).  Returns (O, LSE) with
    the leading row axis dropped for a one-row query."""
    q = np.asarray(q, dtype=np.float64)
    one = q.ndim == 1
    qm = np.atleast_2d(q)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    mask = None if visible is None else np.atleast_2d(np.asarray(visible, dtype=bool))
    st = empty(qm.shape[0], v.shape[1])
    for lo in range(0, k.shape[0], tile):
        hi = min(lo + tile, k.shape[0])
        s = (qm @ k[lo:hi].T) * scale
        if mask is not None:
            s = np.where(mask[:, lo:hi], s, -np.inf)
        st = absorb(st, s, v[lo:hi], guard=guard)
    o, lse = readout(st)
    return (o[0], float(lse[0])) if one else (o, lse)


def paged_slots(table, seq_len: int, block_size: int) -> np.ndarray:
    """Flat pool positions (block * block_size + slot) of keys 0 .. seq_len-1
    of a sequence whose logical block i is ``table[i]``."""
    pos = np.arange(seq_len)
    return np.asarray(table)[pos // block_size] * block_size + pos % block_size


def paged(q, table, k_cache, v_cache, seq_len: int, block_size: int, scale: float):
    """The recurrence over a paged cache ``[num_blocks, block_size, d]``: the
    sequence's keys are gathered through the table (one index per key) and
    streamed one pool block per step."""
    d = k_cache.shape[-1]
    where = paged_slots(table, seq_len, block_size)
    keys = np.asarray(k_cache, dtype=np.float64).reshape(-1, d)[where]
    vals = np.asarray(v_cache, dtype=np.float64).reshape(-1, d)[where]
    return stream(q, keys, vals, block_size, scale)


def split(q, k, v, workers: int, tile: int, scale: float):
    """Flash-decoding for one row: ``workers`` contiguous key ranges each
    stream alone from an empty state; the partial states are then combined."""
    q = np.atleast_2d(np.asarray(q, dtype=np.float64))
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    cuts = np.linspace(0, k.shape[0], workers + 1).round().astype(int)
    merged = empty(1, v.shape[1])
    for w in range(workers):
        part = empty(1, v.shape[1])
        for lo in range(cuts[w], cuts[w + 1], tile):
            hi = min(lo + tile, cuts[w + 1])
            part = absorb(part, (q @ k[lo:hi].T) * scale, v[lo:hi])
        merged = combine(merged, part)
    o, lse = readout(merged)
    return o[0], float(lse[0])


def tile_stats(scores, tile: int):
    """For one row of scaled scores: per tile, the tile's own max and sum
    (m~, l~) and the running (m, l) after absorbing it."""
    s = np.asarray(scores, dtype=np.float64)
    st = empty(1, 1)
    out = []
    for lo in range(0, s.size, tile):
        part = s[lo:lo + tile]
        own_m = float(part.max())
        own_l = float(np.exp(part - own_m).sum())
        st = absorb(st, part[None, :], np.zeros((part.size, 1)))
        out.append({"m_tile": own_m, "l_tile": own_l, "m": float(st.mx[0]), "l": float(st.total[0])})
    return out
