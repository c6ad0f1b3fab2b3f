// fa_decode.hip -- paged single-token decode with grouped-query heads, split
// across waves (flash-decoding) and merged by a second kernel.
//
// Sources: "S12 FlashAttention" (llminference.xinbetween.com):
//   * "What this unlocks beyond speed": tiles need not be contiguous -- each
//     can be a block fetched through the block table; with one query the
//     keys are split across thread blocks and the partial (m, l, o) states
//     are combined at the end;
//   * "How this composes with what you already built": one loop over the
//     block table that loads the KV head shared by the query's group and
//     updates (m, l, o);
//   * "Build it / Implementation" (paged excerpt): block i holds
//     min(block, seq_len - i*block) keys and the walk stops when that is <= 0;
//     the same section's remedy for exp(-inf - -inf): a finite initial max.
// The merge of two partial states is the rule printed on the "FlashAttention"
// page of tachyon.techntrek.in ("For engineers / Show the maths"):
// m = max(m1, m2), l = e^(m1-m) l1 + e^(m2-m) l2, and o rescales the same way.
//
// Work division (balanced split).  For one KV head, the key blocks of all
// sequences, concatenated in batch order, form one list of U blocks.  It is
// cut into P equal parts (P = num_splits, by default one per wave slot of
// the device), one wave each, so every wave streams the same number of
// blocks and all finish together whatever the mix of lengths.  A part may
// end inside a sequence and may cover several short ones: it leaves one
// partial state per (sequence, part) piece.  Piece (sequence b, part w) of
// a query head is stored in that head's slot w + b -- unique, because
// walking the pieces in order increases w, b or both -- so the workspace
// holds P + batch slots per query head.  The cut depends only on logical
// block positions: a permuted pool gives bit-identical results.
//
// Split kernel, gfx950 mapping: one wave per (part, kv head); all query
// heads of the group (up to 16) ride in the 16 columns of the matrix
// products, so every K/V byte is loaded once for the whole group.
//   * scores S^T[16 tokens x 16 heads] = K Q^T on v_mfma_f32_16x16x32_bf16:
//     lane l loads the A operand straight from the pool -- token l%16, dims
//     32s + 8(l/16) .. +7 for s = 0..3 -- and holds Q of head l%16 as B;
//   * the accumulator leaves lane l with tokens 4(l/16) .. +3 of head l%16,
//     which is exactly the B operand layout of the second product
//     O^T += V^T P^T (v_mfma_f32_16x16x16bf16_1k), so the weights never move
//     between lanes; the lazy softmax per head runs on those 4 values;
//   * V^T comes from a 4 KB LDS copy of the value block read with
//     ds_read_b64_tr_b16 (four tokens of one dim per lane); the 16-byte
//     chunks of each row are XOR-swizzled so the transposed reads of a
//     half-wave hit distinct banks;
//   * K and V of the next block are in flight (a two-block register ring)
//     while one is consumed; the pool is read with non-temporal loads.
// Lazy correction: weights are formed against the head's current reference
// max until one would exceed 2^8; only then is the reference moved (the max
// over the four lane groups holding that head) and (o, l) rescaled.
// FP8 pools (KV8): K and V blocks are E4M3 bytes, widened to bf16 in
// registers right after the load (exact: every E4M3 value is a bf16 value),
// so the products and the LDS copy are the bf16 ones; the K descale factor
// is folded into the score scale and the V descale into the combine.  A
// 16-byte K load then covers two score steps: the contraction is relabelled
// so that step 2u + h takes head dims 64u + 16(l/16) + 8h .. +7 (Q is loaded
// with the same relabelling).
#include <mutex>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

// Device memory of the allocation-free decode entry point: the split
// kernel's partial states live here instead of in a caller workspace.  One
// copy per GPU, held until the process ends; every call on a GPU reuses it,
// so calls that overlap on one GPU race.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

constexpr int kBlock = 16;
constexpr float kLazyLog2 = 8.f;    // largest weight 2^8 against a stale reference
constexpr float kInitMax = -1e30f;  // finite initial reference max
constexpr int kMlStride = 4;        // workspace floats per partial: m, l, lb, unused
constexpr int kSplitWavesPerCu = 12; // occupancy the split kernel is built for (bf16, head_dim 64 / 128)

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ f32x4 zero4() {
  f32x4 z = {0.f, 0.f, 0.f, 0.f};
  return z;
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc, false);
}

__device__ __forceinline__ int clamp_len(int L, int maxlen) { return L < 0 ? 0 : (L > maxlen ? maxlen : L); }

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
  return x;
}

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

// Key blocks of sequence b.
__device__ __forceinline__ int seq_blocks(const DecodeParams& p, int b) {
  return (clamp_len(p.seq_lens[b], p.max_seq_len) + kBlock - 1) / kBlock;
}

// U: key blocks of the whole batch (per kv head).
__device__ int total_blocks(const DecodeParams& p, int lane) {
  int s = 0;
  for (int c0 = 0; c0 < p.batch; c0 += 64)
    if (c0 + lane < p.batch) s += seq_blocks(p, c0 + lane);
  return __builtin_amdgcn_readfirstlane(wave_sum(s));
}

// The sequence b holding list position x (0 <= x < U) and the position of
// b's first block.
__device__ void locate(const DecodeParams& p, int lane, int x, int& b_out, int& first_out) {
  int base = 0;
  for (int c0 = 0; c0 < p.batch; c0 += 64) {
    const int nb = c0 + lane < p.batch ? seq_blocks(p, c0 + lane) : 0;
    const int incl = wave_incl_scan(nb, lane) + base;
    const uint64_t hit = __ballot(incl > x);
    if (hit) {
      const int j = __builtin_ctzll(hit);
      b_out = c0 + j;
      first_out = __shfl(incl - nb, j, 64);
      return;
    }
    base = __shfl(incl, 63, 64);
  }
  b_out = p.batch;
  first_out = base;
}

// Position in a walk over the block list: sequence b, its block blk, its
// block count nb and length L (all wave-uniform).
struct Cursor {
  int b, blk, nb, L;
};

__device__ __forceinline__ void cursor_seq(const DecodeParams& p, Cursor& c, int b) {
  c.b = b;
  c.L = clamp_len(p.seq_lens[b], p.max_seq_len);
  c.nb = (c.L + kBlock - 1) / kBlock;
}

// Next block; past a sequence's last block, the next sequence with keys.
// Only called while blocks remain in the wave's part, so such a sequence exists.
__device__ __forceinline__ void cursor_next(const DecodeParams& p, Cursor& c) {
  if (++c.blk < c.nb) return;
  c.blk = 0;
  do {
    cursor_seq(p, c, c.b + 1);
  } while (c.nb == 0);
}

// 16 bytes of the KV pool, read once: a non-temporal load (streams past the
// caches instead of displacing lines that are reused).
__device__ __forceinline__ uint4 load_stream(const char* p) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Physical 16-byte chunk of logical chunk c in value row r of the LDS copy
// (D / 8 chunks per row).
template <int D>
__device__ __forceinline__ int swz(int r, int c) {
  return D >= 128 ? c ^ (2 * (r & 3) + 8 * ((r >> 2) & 1)) : c ^ (2 * (r & 3));
}

// One block as this lane loads it: k[s] = token l%16, dims 32s + 8(l/16)
// .. +7 (score A operand); v[s] = token s * 64/(D/8) + l / (D/8), dims
// 8(l % (D/8)) .. +7 (D/32 loads each).
template <int D, bool KV8>
struct Blk {
  uint4 k[KV8 ? D / 64 : D / 32];
  uint4 v[KV8 ? D / 64 : D / 32];
};

// Blocks in flight per wave: a ring of two.  The waves are bound by their
// per-block chain of waits rather than by bytes in flight, so registers
// serve better as more waves per SIMD than as a deeper ring (measured on
// B=64 Hq=32 Hkv=8 d=128, lengths U{1024..32768}, against a four-block ring:
// E4M3 pools 424 -> 393 us at four waves instead of three, bf16 pools
// 698 -> 686 us at three instead of two).  At head_dim 256 with bf16 pools a
// block is 16 KB per operand and two blocks already take most registers; a
// ring of four there, consumed two blocks per step, measured the same as two
// (B=32 Hq=16 Hkv=8, lengths U{1024..16384}: 441 us either way), the reads
// already running within a few percent of a plain read of the same blocks.

// Two E4M3 bytes (0, 1 or, with HI, 2, 3 of w) -> two bf16, exactly (scale 1).
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
// Eight E4M3 bytes (two words) -> eight bf16.
__device__ __forceinline__ uint4 e4m3x8_bf16x8(uint32_t a, uint32_t b) {
  return make_uint4(e4m3x2_bf16x2<false>(a), e4m3x2_bf16x2<true>(a), e4m3x2_bf16x2<false>(b),
                    e4m3x2_bf16x2<true>(b));
}

// Waves per SIMD the split kernel is built for: three (at most 168
// registers; head_dim 128 takes 164), or one at head_dim 256 (its ring,
// accumulator and Q fragments need more than 256 registers; the rest goes to
// the accumulation registers), or four with E4M3 pools (128 registers: the
// two 64-bit row pointers used only at piece boundaries spill).
template <int D, bool KV8 = false>
constexpr int split_waves_per_simd() { return D == 256 ? 1 : (KV8 ? 4 : 3); }

template <int D, bool KV8>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(split_waves_per_simd<D, KV8>(),
                                                                     split_waves_per_simd<D, KV8>()))) void
decode_split_kernel(const DecodeParams p) {
  constexpr int kD = D;
  constexpr int ES = KV8 ? 1 : 2;       // bytes per pool element
  constexpr int NS = D / 32;            // 32-dim steps of the score product
  constexpr int NL = KV8 ? D / 64 : NS; // 16-byte loads per lane per operand and block
  constexpr int VCH = D / 8;            // 16-byte bf16 chunks of a value row in LDS
  constexpr int VCHL = D * ES / 16;     // 16-byte pieces of a value row in the pool
  constexpr int VTPL = 64 / VCHL;       // value rows per load instruction
  const int part = blockIdx.x;
  const int g = blockIdx.y;  // kv head; query heads g*G .. g*G + G - 1
  const int G = p.group;
  const int lane = threadIdx.x;
  const int j = lane >> 4;   // lane group
  const int n = lane & 15;   // token (K operand), head (scores), dim (V^T)
  __shared__ __attribute__((aligned(16))) uint16_t v_s[kBlock * kD];

  const int U = total_blocks(p, lane);
  const int x0 = (int)((int64_t)part * U / p.num_splits);
  const int x1 = (int)((int64_t)(part + 1) * U / p.num_splits);
  if (x0 >= x1) return;
  const int n_units = x1 - x0;
  int b_first, first;
  locate(p, lane, x0, b_first, first);
  b_first = __builtin_amdgcn_readfirstlane(b_first);
  first = __builtin_amdgcn_readfirstlane(first);

  Cursor ic, pc;  // issue and process positions
  cursor_seq(p, ic, b_first);
  ic.blk = x0 - first;
  pc = ic;

  // Loads address a block through a wave-uniform 64-bit base (scalar
  // registers) plus a per-lane 32-bit byte offset that is the same for every
  // block (the host keeps it below 2^31).
  const char* __restrict__ kpool = (const char*)p.k_pool + (int64_t)g * p.p_hs * ES;
  const char* __restrict__ vpool = (const char*)p.v_pool + (int64_t)g * p.p_hs * ES;
  // Load s of a block adds 64 s bytes to the key offset (an immediate) and
  // s VTPL rows to the value base (a uniform step), so one per-lane offset
  // per operand serves every load.
  const uint32_t koff = KV8 ? (uint32_t)(n * p.p_ts + 16 * j) : (uint32_t)((n * p.p_ts + 8 * j) * 2);
  const uint32_t voff = (uint32_t)((lane / VCHL) * p.p_ts * ES + 16 * (lane % VCHL));
  const int64_t vstep = (int64_t)VTPL * p.p_ts * ES;

  // Q of head n as the B operand of the score product (zero for columns
  // past the group).
  uint4 qf[NS];
  auto load_q = [&](int b) {
    const uint16_t* qr = (const uint16_t*)p.q + (int64_t)b * p.q_bs + (int64_t)(g * G + n) * p.q_hs;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int dim = KV8 ? 64 * (s >> 1) + 16 * j + 8 * (s & 1) : 32 * s + 8 * j;
      qf[s] = n < G ? *(const uint4*)(qr + dim) : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  load_q(pc.b);

  f32x4 o[D / 16];  // O^T: o[db][r] = dim 16db + 4j + r of head n
  float m, l, lb;  // reference max (base 2), fp32 weight sum, bf16 weight sum
  auto reset = [&]() {
    m = kInitMax;
    l = 0.f;
    lb = 0.f;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) o[db] = zero4();
  };
  reset();

  int n_issued = 0;
  auto issue = [&](Blk<D, KV8>& B) {
    if (n_issued < n_units) {
      const int64_t base = (int64_t)p.block_table[(int64_t)ic.b * p.max_blocks + ic.blk] * p.p_bs * ES;
      const char* kb = kpool + base;
      const char* vb = vpool + base;
#pragma unroll
      for (int s = 0; s < NL; ++s) B.k[s] = load_stream(kb + koff + 64 * s);
#pragma unroll
      for (int s = 0; s < NL; ++s) B.v[s] = load_stream(vb + s * vstep + voff);
      if (++n_issued < n_units) cursor_next(p, ic);
    }
  };

  const uint32_t ones2 = 0x3F803F80u;  // bf16 pair (1, 1)
  const float cs = p.scale_log2;
  const int tk = n >> 2, tq = n & 3;

  // One block through the recurrence; tokens at or past VALID hold no key
  // (only a sequence's last block has such tokens).
  auto process = [&](const Blk<D, KV8>& B, int valid) {
    // Values to LDS (row = token, swizzled bf16 chunks).
#pragma unroll
    for (int s = 0; s < NL; ++s) {
      const int r = s * VTPL + lane / VCHL;
      if (KV8) {
        const int c = 2 * (lane % VCHL);  // 16 E4M3 bytes = bf16 chunks c, c + 1
        *(uint4*)&v_s[r * kD + swz<D>(r, c) * 8] = e4m3x8_bf16x8(B.v[s].x, B.v[s].y);
        *(uint4*)&v_s[r * kD + swz<D>(r, c + 1) * 8] = e4m3x8_bf16x8(B.v[s].z, B.v[s].w);
      } else {
        *(uint4*)&v_s[r * kD + swz<D>(r, lane % VCH) * 8] = B.v[s];
      }
    }
    // Scores: sc[r] = S[token 4j + r][head n].
    f32x4 sc = zero4();
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      uint4 ka;
      if (KV8)
        ka = (s & 1) ? e4m3x8_bf16x8(B.k[s >> 1].z, B.k[s >> 1].w) : e4m3x8_bf16x8(B.k[s >> 1].x, B.k[s >> 1].y);
      else
        ka = B.k[s];
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka), __builtin_bit_cast(bf16x8, qf[s]),
                                                  sc, 0, 0, 0);
    }
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = 4 * j + r < valid ? sc[r] * cs : -INFINITY;
    const float xm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    if (__any(xm > m + kLazyLog2)) {
      float mx = fmaxf(xm, __shfl_xor(xm, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mn = fmaxf(m, mx);
      const float al = exp2_fast(m - mn);
      m = mn;
      l *= al;
      lb *= al;
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[db][r] *= al;
    }
    float pw[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pw[r] = exp2_fast(x[r] - m);
    l += (pw[0] + pw[1]) + (pw[2] + pw[3]);
    const uint32_t p01 = pack_bf16x2(pw[0], pw[1]);
    const uint32_t p23 = pack_bf16x2(pw[2], pw[3]);
    lb = dot2(p01, ones2, lb);
    lb = dot2(p23, ones2, lb);
    const i16x4 pb = __builtin_bit_cast(i16x4, make_uint2(p01, p23));
    // Value tokens past the end may hold anything: clear them so that a
    // zero weight cannot meet a NaN.
    uint32_t keep0 = 0xFFFFFFFFu, keep1 = 0xFFFFFFFFu;
    if (valid < kBlock) {
      keep0 = (4 * j + 0 < valid ? 0x0000FFFFu : 0u) | (4 * j + 1 < valid ? 0xFFFF0000u : 0u);
      keep1 = (4 * j + 2 < valid ? 0x0000FFFFu : 0u) | (4 * j + 3 < valid ? 0xFFFF0000u : 0u);
    }
    // O^T += V^T P^T per 16-dim block: lane 4k+q of group j reads token
    // 4j + k, dims 16db + 4q .. +3; the transposed read leaves lane n with
    // dim 16db + n of tokens 4j .. 4j+3.
    const int vr = 4 * j + tk;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const i16x4 vt = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)&v_s[vr * kD + swz<D>(vr, 2 * db + (tq >> 1)) * 8 + 4 * (tq & 1)]);
      uint2 w = __builtin_bit_cast(uint2, vt);
      w.x &= keep0;
      w.y &= keep1;
      o[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, w), pb, o[db], 0, 0, 0);
    }
  };

  // End of a piece: sum the four lane groups' weight sums and store the
  // piece's partial state for the group's heads in slot part + b.
  const int S = p.num_splits + p.batch;
  auto flush = [&](int b) {
    float lt = l + __shfl_xor(l, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    float lbt = lb + __shfl_xor(lb, 16, 64);
    lbt += __shfl_xor(lbt, 32, 64);
    if (n < G) {
      const int64_t row = (int64_t)(g * G + n) * S + part + b;
      float* dst = p.ws_o + row * kD + 4 * j;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) *(f32x4*)(dst + 16 * db) = o[db];
      if (j == 0) *(float4*)(p.ws_ml + row * kMlStride) = make_float4(m, lt, lbt, 0.f);
    }
  };

  int n_done = 0;
  auto step = [&](const Blk<D, KV8>& B) {
    if (n_done >= n_units) return;
    const bool last_blk = pc.blk == pc.nb - 1;
    process(B, last_blk ? pc.L - pc.blk * kBlock : kBlock);
    ++n_done;
    if (last_blk || n_done == n_units) {
      flush(pc.b);
      if (n_done < n_units) {
        reset();
        cursor_next(p, pc);
        load_q(pc.b);
      }
    } else {
      ++pc.blk;
    }
  };

  // The scheduling barriers keep each ring refill where it is written, one
  // block ahead of its use, instead of letting the scheduler sink the loads
  // next to their consumers.
  Blk<D, KV8> R0, R1;
  issue(R0);
  issue(R1);
  __builtin_amdgcn_sched_barrier(0);
  for (int u = 0; u < n_units; u += 2) {
    step(R0);
    __builtin_amdgcn_sched_barrier(0);
    issue(R0);
    __builtin_amdgcn_sched_barrier(0);
    step(R1);
    __builtin_amdgcn_sched_barrier(0);
    issue(R1);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One wave per (sequence, query head): merge the partial states of the
// sequence's pieces.  Pieces of sequence b are those of the parts holding
// its first and last blocks and every non-empty part between; part w holds
// list positions [w*U/P, (w+1)*U/P), so position x lies in part
// ceil((x+1)*P/U) - 1.
template <int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(const DecodeParams p) {
  constexpr int kD = D;
  constexpr int DPL = D / 64;  // output dims per lane
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int lane = threadIdx.x;
  const int U = total_blocks(p, lane);
  // first block position of sequence b, and its block count
  int first = 0;
  for (int c0 = 0; c0 < b; c0 += 64)
    if (c0 + lane < b) first += seq_blocks(p, c0 + lane);
  first = __builtin_amdgcn_readfirstlane(wave_sum(first));
  const int nb = seq_blocks(p, b);

  const int P = p.num_splits;
  const int S = P + p.batch;
  float M = -INFINITY, l = 0.f, lb = 0.f;
  float oa[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) oa[i] = 0.f;
  if (nb > 0) {
    const int w0 = (int)(((int64_t)(first + 1) * P + U - 1) / U) - 1;
    const int w1 = (int)(((int64_t)(first + nb) * P + U - 1) / U) - 1;
    const int64_t row0 = (int64_t)h * S + b;
    // Parts with an empty range (possible when U < P) hold no piece.
    auto empty = [&](int w) { return (int64_t)w * U / P == (int64_t)(w + 1) * U / P; };
    // One pass over the pieces, four at a time with all their loads issued
    // together: the group's max moves the reference M and what was merged
    // so far is rescaled by 2^(M_old - M_new).  Past w1 the index is clamped
    // (a valid address) and, like an empty part, the piece is dead; a dead
    // piece's workspace row is never used (it may hold anything).
    for (int w = w0; w <= w1; w += 4) {
      float4 ml[4];
      float v[4][DPL];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int wu = min(w + u, w1);
        ml[u] = *(const float4*)(p.ws_ml + (row0 + wu) * kMlStride);
        const float* src = p.ws_o + (row0 + wu) * kD + DPL * lane;
#pragma unroll
        for (int i = 0; i < DPL; ++i) v[u][i] = src[i];
        if (w + u > w1 || empty(w + u)) ml[u].x = -INFINITY;
      }
      const float gm = fmaxf(fmaxf(ml[0].x, ml[1].x), fmaxf(ml[2].x, ml[3].x));
      if (gm == -INFINITY) continue;
      const float Mn = fmaxf(M, gm);
      const float a = exp2_fast(M - Mn);  // 0 while nothing was merged (M = -inf)
      l *= a;
      lb *= a;
#pragma unroll
      for (int i = 0; i < DPL; ++i) oa[i] *= a;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool live = ml[u].x != -INFINITY;
        const float wt = live ? exp2_fast(ml[u].x - Mn) : 0.f;
        l = __builtin_fmaf(wt, ml[u].y, l);
        lb = __builtin_fmaf(wt, ml[u].z, lb);
#pragma unroll
        for (int i = 0; i < DPL; ++i) oa[i] = live ? __builtin_fmaf(wt, v[u][i], oa[i]) : oa[i];
      }
      M = Mn;
    }
  }
  // o / lb: the weights P.V used, so the row is a convex combination of
  // value rows up to fp32 rounding (times the V descale of FP8 pools); LSE
  // from the fp32 weights.
  const float inv = lb > 0.f ? p.o_scale / lb : 0.f;
  uint16_t* orow = (uint16_t*)p.o + (int64_t)b * p.o_bs + (int64_t)h * p.o_hs;
  if constexpr (DPL == 1) {
    orow[lane] = (uint16_t)(pack_bf16x2(oa[0] * inv, 0.f) & 0xFFFFu);
  } else {
#pragma unroll
    for (int i = 0; i < DPL; i += 2) *(uint32_t*)(orow + DPL * lane + i) = pack_bf16x2(oa[i] * inv, oa[i + 1] * inv);
  }
  if (p.lse && lane == 0)
    p.lse[(int64_t)b * p.heads_q + h] = l > 0.f ? (M + log2_fast(l)) * kLn2 : -INFINITY;
}

}  // namespace

int decode_num_parts(int num_splits, int batch, int heads_q, int group, int max_seq_len, int head_dim,
                     bool kv8) {
  if (num_splits > 0) return num_splits;
  // One part per wave slot of the device (the split kernel is built for three
  // waves per SIMD, twelve per CU; one and four at head_dim 256; four and
  // sixteen for FP8 pools below 256), spread over the kv heads; no more parts
  // than about one per 4 blocks of the largest possible batch.
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  const int64_t heads_kv = group > 0 ? heads_q / group : 1;
  const int waves_per_cu =
      head_dim == 256 ? 4 * split_waves_per_simd<256>() : (kv8 ? 4 * split_waves_per_simd<128, true>() : kSplitWavesPerCu);
  int64_t parts = (int64_t)cus * waves_per_cu / (heads_kv > 0 ? heads_kv : 1);
  const int64_t max_units = (int64_t)batch * ((max_seq_len + kBlock - 1) / kBlock);
  if (parts > (max_units + 3) / 4) parts = (max_units + 3) / 4;
  if (parts < 1) parts = 1;
  return (int)parts;
}

hipError_t decode_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kDecodeScratchMaxDevices) return hipErrorInvalidDevice;
  // The array's name is a host-side stand-in: its device address is looked
  // up once per device, with that device current, and used from then on.
  static std::mutex mu;
  static void* addr[kDecodeScratchMaxDevices] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!a) return hipErrorInvalidSymbol;
    addr[dev] = a;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

size_t decode_workspace_bytes(int parts, int batch, int heads_q, int head_dim) {
  const size_t rows = (size_t)heads_q * (size_t)(parts + batch);
  return rows * ((size_t)head_dim + kMlStride) * sizeof(float);
}

namespace {
template <int D>
hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  if (p.kv8)
    hipLaunchKernelGGL((decode_split_kernel<D, true>), dim3(p.num_splits, p.heads_kv), dim3(64), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_split_kernel<D, false>), dim3(p.num_splits, p.heads_kv), dim3(64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel<D>, dim3(p.heads_q, p.batch), dim3(64), 0, stream, p);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_decode_paged(const DecodeParams& p, int head_dim, hipStream_t stream) {
  if (head_dim == 128) return launch_decode<128>(p, stream);
  if (head_dim == 64) return launch_decode<64>(p, stream);
  if (head_dim == 256) return launch_decode<256>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
