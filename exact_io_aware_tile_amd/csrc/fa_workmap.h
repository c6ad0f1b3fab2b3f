// fa_workmap.h -- the prefill work mapping (workgroup index -> query tile and
// (sequence, head) pair) with its divisions prepared on the host.  Shared by
// the host API, the prefill kernels and the host-side bijection check.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Division of an int in [0, 2^31) by a divisor d >= 1 fixed for a launch, as
// one 32x32 -> 64-bit multiply and a shift (Granlund and Montgomery,
// "Division by invariant integers using multiplication", PLDI 1994):
// n / d = (n * mul) >> shift with shift = 31 + ceil(log2 d) and
// mul = ceil(2^shift / d) < 2^32.  With e = mul * d - 2^shift in [0, d),
// n * e < 2^31 * d <= 2^shift, so the product never reaches the next
// multiple of 2^shift / d early and the quotient is exact.  In a kernel the
// operands are wave-uniform, so this is three scalar instructions where a
// runtime division takes a chain of vector-ALU reciprocal steps.
struct IntDiv {
  uint32_t mul;
  uint32_t shift;
};

inline IntDiv make_intdiv(int32_t d) {
  uint32_t l = 0;
  while (l < 31 && (int64_t(1) << l) < d) ++l;  // ceil(log2 d)
  const uint32_t shift = 31 + l;
  const uint64_t mul = ((uint64_t(1) << shift) + (uint64_t)d - 1) / (uint64_t)d;
  return IntDiv{(uint32_t)mul, shift};
}

__host__ __device__ __forceinline__ int32_t idiv(int32_t n, IntDiv f) {
  return (int32_t)(((uint64_t)(uint32_t)n * f.mul) >> f.shift);
}

// Work item of prefill workgroup w of nwg = num_qtiles x (sequence, query
// head) pairs: query tile qt and pair bh = b * heads_q + h.  Workgroups are
// dealt round-robin to the 8 XCDs and each XCD starts its items in order as
// its CUs free up.  When the GQA groups (the `group` query heads that share a
// KV head) split evenly over the XCDs ("balanced"), group g goes to XCD
// g mod 8: every XCD then holds a share of every sequence, so the causal work
// of packed sequences of different lengths balances across XCDs, and the
// heads of a group share its K/V in one XCD's L2.  Each XCD starts with the
// heaviest causal items (the last query tiles of all its px pairs), then the
// ones before, and so on.  With chunk > 0 the XCD's pairs are taken `chunk`
// at a time (a multiple of the group) and each chunk's items run heaviest
// first before the next chunk starts: the XCD's CUs then work on few pairs
// at once and their query tiles share each K/V tile through the L2, where a
// heaviest-first order over many long packed sequences would keep more K/V
// in flight than the L2 holds.  Otherwise items are dealt in (pair, query
// tile) order, heaviest tile first.
struct WorkMap {
  int32_t num_qtiles;
  int32_t group;
  int32_t balanced;
  int32_t px;       // pairs per XCD (balanced; 1 otherwise)
  int32_t chunk;    // pairs per chunk, <= px (px: the XCD's pairs form one chunk)
  int32_t last_cn;  // pairs in the XCD's last chunk
  IntDiv by_qtiles, by_group, by_chunk_items, by_chunk, by_last_cn;
};

// chunk as the host picks it (0: none).  No chunking is one chunk of the
// XCD's px pairs, so both cases take the same steps.
inline WorkMap make_workmap(int32_t nwg, int32_t num_qtiles, int32_t group, int32_t chunk) {
  WorkMap m{};
  m.num_qtiles = num_qtiles;
  m.group = group;
  const int32_t npairs = nwg / num_qtiles;
  m.balanced = (npairs / group) % 8 == 0 && npairs % group == 0 ? 1 : 0;
  m.px = m.balanced ? npairs / 8 : 1;
  m.chunk = (chunk > 0 && chunk < m.px) ? chunk : m.px;
  m.last_cn = m.px - (m.px - 1) / m.chunk * m.chunk;
  m.by_qtiles = make_intdiv(num_qtiles);
  m.by_group = make_intdiv(group);
  m.by_chunk_items = make_intdiv(m.chunk * num_qtiles);
  m.by_chunk = make_intdiv(m.chunk);
  m.by_last_cn = make_intdiv(m.last_cn);
  return m;
}

// Query tile qt and pair bh (= sequence * heads_q + head) of workgroup w.
// Both orders are formed and one is selected, so that a kernel takes no
// branch here and loads the whole map at once.
__host__ __device__ inline void prefill_work_item(const WorkMap& m, int32_t w, int32_t& qt, int32_t& bh) {
  // balanced: XCD w % 8, rank j on it; its chunk of pairs starting at c0
  const int32_t j = w >> 3;
  const int32_t c0 = idiv(j, m.by_chunk_items) * m.chunk;
  const bool last = c0 + m.chunk > m.px;
  const int32_t cn = last ? m.last_cn : m.chunk;  // pairs in this chunk
  const int32_t r = j - c0 * m.num_qtiles;
  const int32_t rq = idiv(r, last ? m.by_last_cn : m.by_chunk);
  const int32_t k = c0 + (r - rq * cn);  // the XCD's k-th pair
  const int32_t kg = idiv(k, m.by_group);
  const int32_t bh_x = ((kg << 3) + (w & 7)) * m.group + (k - kg * m.group);
  // otherwise: pair w / num_qtiles, its tiles heaviest first
  const int32_t wq = idiv(w, m.by_qtiles);
  qt = m.num_qtiles - 1 - (m.balanced ? rq : w - wq * m.num_qtiles);
  bh = m.balanced ? bh_x : wq;
}

}  // namespace fa
