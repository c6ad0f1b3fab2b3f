// fa_internal.h -- parameter blocks and launchers shared by the host API and
// the kernel translation units of libfa_gfx950.so.  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_workmap.h"

namespace fa {

// Query rows handled by one prefill workgroup.
constexpr int kFwdRowsPerTileBf16 = 256;
constexpr int kFwdRowsPerTileBf16D256 = 128;  // head_dim 256: 16 rows per wave
constexpr int kFwdRowsPerTileF32 = 128;
// The bf16 prefill kernel addresses rows inside a 64-key tile with 32-bit
// byte offsets: key/value row strides (elements) are limited to 2^24.
constexpr int64_t kFwdMaxKvRowStrideBf16 = int64_t(1) << 24;
// The FP8 prefill kernel: 256 query rows per workgroup, head_dim 128.
constexpr int kFwdRowsPerTileFp8 = 256;
// Paged prefill reads 16-token blocks.
constexpr int kFwdPagedBlock = 16;

// One prefill launch: dense batched attention or packed variable-length
// sequences.  All strides are in elements.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;                 // may be null
  const int32_t* cu_seqlens;  // null: dense; else packed sequences
  int64_t q_bs, q_ss, q_hs;   // batch (dense only), token, head strides
  int64_t k_bs, k_ss, k_hs;
  int64_t v_bs, v_ss, v_hs;
  int64_t o_bs, o_ss, o_hs;
  int32_t batch;     // dense batch, or number of packed sequences
  int32_t seqlen_q;  // dense lengths; for packed sequences: max_seqlen bound
  int32_t seqlen_k;
  int32_t total_tokens;  // packed only: LSE row stride
  int32_t heads_q;
  int32_t group;         // heads_q / heads_kv
  int32_t num_qtiles;    // query tiles per (sequence, head)
  int32_t causal;
  float scale_log2;      // scale * log2(e): scores are kept in base 2
                         // (fp8: times the q and k descale factors)
  float o_scale;         // fp8: the v descale factor, applied to O
  // Paged keys and values (chunked prefill, bf16): when `paged` is set,
  // q / o / lse are packed by cu_seqlens (the new queries of each sequence),
  // k / v point at the two pools, and key t of sequence s is token t % 16
  // of pool block block_table[s * max_blocks + t / 16]; the sequence has
  // seq_lens_k[s] keys (clamped to [0, seqlen_k]).
  int32_t paged;
  const int32_t* block_table;
  const int32_t* seq_lens_k;
  int32_t max_blocks;
  int64_t p_bs, p_hs, p_ts;  // pool strides: block, head, token
  // Dropout (bf16, dense and packed; drop_t == 0: none).  The weight of row
  // r (its index in the LSE layout) on key j of its sequence is kept iff
  // byte j % 16 of Philox-4x32-10(counter {j / 16, r, r >> 32, drop_offset},
  // key {seed lo, seed hi}) is >= drop_t; O is then scaled by drop_scale.
  int32_t drop_t;
  uint32_t drop_seed_lo, drop_seed_hi, drop_offset;
  float drop_scale;
  // Work mapping: 0 = every XCD runs its pairs' heaviest items first; > 0 =
  // pairs taken that many at a time (packed sequences, see prefill_work_item).
  int32_t wi_chunk;
  WorkMap wmap;     // the mapping of this launch (set_work_map)
  IntDiv by_heads;  // pair -> (sequence, head)
};

// The work mapping of a prefill launch over num_qtiles * heads_q * batch
// workgroups, with its divisors prepared here rather than in every
// workgroup.
inline void set_work_map(FwdParams& p) {
  const int64_t nwg = (int64_t)p.num_qtiles * p.heads_q * p.batch;
  p.wmap = nwg > 0 ? make_workmap((int32_t)nwg, p.num_qtiles, p.group, p.wi_chunk) : make_workmap(1, 1, 1, 0);
  p.by_heads = make_intdiv(p.heads_q > 0 ? p.heads_q : 1);
}

// Paged decode: query heads per kv head (one wave serves the whole group),
// and the largest pool token stride (elements) the kernel's 32-bit per-lane
// offsets inside a block can address.
constexpr int kDecodeMaxGroup = 16;
constexpr int64_t kDecodeMaxTokenStride = int64_t(1) << 26;

// Paged decode: split kernel followed by the combine kernel.
struct DecodeParams {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  int64_t p_bs, p_hs, p_ts;  // pool strides: block, head, token
  int64_t q_bs, q_hs;
  int64_t o_bs, o_hs;
  const int32_t* block_table;
  const int32_t* seq_lens;
  void* o;
  float* lse;
  float* ws_o;   // [heads_q, num_splits + batch, head_dim] fp32 partial o
  float* ws_ml;  // [heads_q, num_splits + batch, 4] fp32 partial (m, l, lb, -), m in base 2
  int32_t batch, heads_q, heads_kv, group, max_blocks, max_seq_len;
  int32_t num_splits;  // parts the block list of one kv head is cut into
  float scale_log2;    // FP8 pools: times the K descale factor
  int32_t kv8;         // pools hold E4M3 bytes (strides then count bytes)
  float o_scale;       // multiplies O: 1, or the V descale factor of FP8 pools
};

hipError_t launch_fwd_bf16(const FwdParams& p, int head_dim, hipStream_t stream);
hipError_t launch_fwd_bf16_d256(const FwdParams& p, hipStream_t stream);
// Query rows per prefill workgroup of the bf16 kernels.
inline int fwd_rows_per_tile_bf16(int head_dim) {
  return head_dim == 256 ? kFwdRowsPerTileBf16D256 : kFwdRowsPerTileBf16;
}
hipError_t launch_fwd_fp8(const FwdParams& p, int head_dim, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdParams& p, int head_dim, hipStream_t stream);
hipError_t launch_decode_paged(const DecodeParams& p, int head_dim, hipStream_t stream);
// Parts for a requested num_splits (0: one per wave slot of the current
// device, or of a 256-CU device when none can be queried).
int decode_num_parts(int num_splits, int batch, int heads_q, int group, int max_seq_len, int head_dim, bool kv8);
size_t decode_workspace_bytes(int parts, int batch, int heads_q, int head_dim);
// Library-held decode workspace (one per device, for callers that cannot
// allocate): its size, and its address on the current device.
constexpr size_t kDecodeScratchBytes = size_t(16) << 20;
constexpr int kDecodeScratchMaxDevices = 64;
hipError_t decode_scratch(void** ptr);

// Merge of P partial (o, lse) states of the same rows.
struct MergeParams {
  const void* o_parts;    // [parts][rows][head_dim], bf16 or fp32
  const float* lse_parts; // [parts][batch][heads][seqlen]
  void* o;                // [rows][head_dim]
  float* lse;             // [batch][heads][seqlen] or null
  int64_t rows;           // batch * seqlen * heads, in that (row-major) order
  int64_t part_elems;     // rows * head_dim
  int64_t part_rows;      // rows
  int32_t parts, seqlen, heads, head_dim;
  int32_t f32;
  IntDiv by_heads, by_seqlen;  // row -> (batch, seqlen, head) (rows * head_dim / 8 < 2^31)
};
hipError_t launch_merge(const MergeParams& p, hipStream_t stream);

}  // namespace fa
