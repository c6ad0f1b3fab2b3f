// fa_api.cpp -- the C ABI of include/fa.h: host-side validation, parameter
// blocks and launch.  Nothing here touches device memory; every check runs
// before any launch, and a rejected call launches nothing.
//
// The parameter block carries strides, data type, masking mode and sequence
// layout to the kernels, the role "FlashAttention: The Algorithm That Beat
// the Memory Wall" (repo-explainer.com, "How the Repo Connects Python to
// Bare-Metal CUDA") gives the host glue.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/fa.h"
#include "fa_internal.h"

#define FA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

fa_status fail(fa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

fa_status ok() {
  g_last_error.clear();
  return FA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Vector loads move 16 bytes: every row start must be 16-byte aligned.
bool strides_ok(const int64_t* s, int n, int64_t elems16) {
  for (int i = 0; i < n; ++i)
    if (s[i] < 0 || s[i] % elems16) return false;
  return true;
}

float scale_log2(float scale) { return (float)((double)scale * 1.4426950408889634073599); }

constexpr int kDecodeBlock = 16;

// Pairs per chunk of the prefill work mapping: whole GQA groups, as many as
// keep their K/V (at the longest length) within one XCD's 4 MB L2.  Below
// four pairs a chunk is too small to balance its causal items and the plain
// order (0) is used: measured on MI355X, the chunked order cuts the K/V
// re-reads of packed and chunked-paged prefill several-fold and is a few
// percent faster there and at B=4 N=2048, and slower with one pair per chunk.
int32_t wi_chunk(int max_seqlen, int head_dim, int elem_bytes, int group) {
  const double kv = 2.0 * (double)max_seqlen * head_dim * elem_bytes;  // K and V of one kv head
  const double c = std::floor((4 << 20) / (kv > 1.0 ? kv : 1.0)) * group;
  return c < 4.0 ? 0 : c > 65536.0 ? 65536 : (int32_t)c;  // 65536 or more pairs: one chunk, the plain order
}

fa_status check_decode(const fa_decode_paged_args* a) {
  if (!a) return fail(FA_ERR_NULL_POINTER, "fa_decode_paged: args is NULL");
  if (a->batch < 0 || a->heads_q <= 0 || a->heads_kv <= 0 || a->max_seq_len < 0 ||
      a->max_blocks_per_seq < 0 || a->num_blocks < 0 || a->num_splits < 0)
    return fail(FA_ERR_BAD_SHAPE, "fa_decode_paged: negative or zero size");
  if (a->heads_q % a->heads_kv)
    return fail(FA_ERR_BAD_SHAPE, "fa_decode_paged: heads_q (%d) is not a multiple of heads_kv (%d)",
                a->heads_q, a->heads_kv);
  const int group = a->heads_q / a->heads_kv;
  if (group > fa::kDecodeMaxGroup)
    return fail(FA_ERR_UNSUPPORTED, "fa_decode_paged: heads_q / heads_kv = %d, supported up to %d", group,
                fa::kDecodeMaxGroup);
  if (a->head_dim != 64 && a->head_dim != 128 && a->head_dim != 256)
    return fail(FA_ERR_UNSUPPORTED, "fa_decode_paged: head_dim %d, supported 64, 128 and 256", a->head_dim);
  if (a->block_size != kDecodeBlock)
    return fail(FA_ERR_UNSUPPORTED, "fa_decode_paged: block_size %d, supported 16", a->block_size);
  if ((int64_t)a->max_seq_len > (int64_t)a->max_blocks_per_seq * a->block_size)
    return fail(FA_ERR_BAD_SHAPE, "fa_decode_paged: max_seq_len %d exceeds max_blocks_per_seq * block_size",
                a->max_seq_len);
  if (a->batch > 65535) return fail(FA_ERR_UNSUPPORTED, "fa_decode_paged: batch %d > 65535", a->batch);
  if ((int64_t)a->batch * ((a->max_seq_len + kDecodeBlock - 1) / kDecodeBlock) > 0x7fffffffLL)
    return fail(FA_ERR_UNSUPPORTED, "fa_decode_paged: batch * max_seq_len / block_size exceeds 2^31");
  if (a->pool_stride[2] > fa::kDecodeMaxTokenStride)
    return fail(FA_ERR_UNSUPPORTED, "fa_decode_paged: pool token stride above %lld elements",
                (long long)fa::kDecodeMaxTokenStride);
  if (a->num_splits > 65535)
    return fail(FA_ERR_UNSUPPORTED, "fa_decode_paged: num_splits %d > 65535", a->num_splits);
  return FA_OK;
}

// Parts the key-block list is cut into; -1 if the device cannot be queried.
int decode_parts(const fa_decode_paged_args* a, bool kv8) {
  return fa::decode_num_parts(a->num_splits, a->batch, a->heads_q, a->heads_q / a->heads_kv, a->max_seq_len,
                              a->head_dim, kv8);
}


// Dropout arguments -> byte threshold t = rint(256 p) (ties to even), seed
// and offset in the parameter block; t == 0 leaves dropout off.
fa_status set_dropout(const fa_dropout_args* d, fa_dtype dtype, const char* fn, fa::FwdParams& p) {
  if (!d) return fail(FA_ERR_NULL_POINTER, "%s: dropout args is NULL", fn);
  if (!(d->p >= 0.0) || !(d->p < 1.0))
    return fail(FA_ERR_BAD_SHAPE, "%s: dropout probability must be in [0, 1)", fn);
  const double t = std::nearbyint(256.0 * d->p);
  if (t > 255.0) return fail(FA_ERR_BAD_SHAPE, "%s: dropout probability rounds to 256/256", fn);
  if (t > 0.0 && dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "%s: dropout is built for bf16", fn);
  p.drop_t = (int32_t)t;
  p.drop_seed_lo = (uint32_t)d->seed;
  p.drop_seed_hi = (uint32_t)(d->seed >> 32);
  p.drop_offset = d->offset;
  p.drop_scale = (float)(256.0 / (256.0 - t));
  return FA_OK;
}

fa_status fwd_dense(const fa_fwd_args* a, const fa_dropout_args* drop, const char* fn, void* stream) {
  if (!a) return fail(FA_ERR_NULL_POINTER, "%s: args is NULL", fn);
  if (a->batch < 0 || a->seqlen_q < 0 || a->seqlen_k < 0 || a->heads_q <= 0 || a->heads_kv <= 0)
    return fail(FA_ERR_BAD_SHAPE, "%s: negative or zero size", fn);
  if (a->heads_q % a->heads_kv)
    return fail(FA_ERR_BAD_SHAPE, "%s: heads_q (%d) is not a multiple of heads_kv (%d)", fn, a->heads_q,
                a->heads_kv);
  if (a->dtype != FA_F32 && a->dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "%s: dtype %d", fn, (int)a->dtype);
  if (a->head_dim != 64 && a->head_dim != 128 && !(a->head_dim == 256 && a->dtype == FA_BF16))
    return fail(FA_ERR_UNSUPPORTED, "%s: head_dim %d, supported 64 and 128 (and 256 for bf16)", fn, a->head_dim);
  if (!(a->scale > 0.f) || !std::isfinite(a->scale))
    return fail(FA_ERR_BAD_SHAPE, "%s: scale must be positive and finite", fn);
  fa::FwdParams p{};
  if (drop) {
    const fa_status st = set_dropout(drop, a->dtype, fn, p);
    if (st != FA_OK) return st;
  }
  if (a->batch == 0 || a->seqlen_q == 0) return ok();
  if (!a->q || !a->o) return fail(FA_ERR_NULL_POINTER, "%s: q and o are required", fn);
  if (a->seqlen_k > 0 && (!a->k || !a->v))
    return fail(FA_ERR_NULL_POINTER, "%s: k and v are required when seqlen_k > 0", fn);
  const int64_t e16 = a->dtype == FA_BF16 ? 8 : 4;
  if (!strides_ok(a->q_stride, 3, e16) || !strides_ok(a->k_stride, 3, e16) || !strides_ok(a->v_stride, 3, e16) ||
      !strides_ok(a->o_stride, 3, e16))
    return fail(FA_ERR_BAD_SHAPE, "%s: strides must be non-negative multiples of %lld elements", fn,
                (long long)e16);
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o))
    return fail(FA_ERR_BAD_SHAPE, "%s: q, k, v, o must be 16-byte aligned", fn);
  if (a->dtype == FA_BF16 &&
      (a->k_stride[1] > fa::kFwdMaxKvRowStrideBf16 || a->v_stride[1] > fa::kFwdMaxKvRowStrideBf16))
    return fail(FA_ERR_UNSUPPORTED, "%s: bf16 k/v row strides above %lld elements", fn,
                (long long)fa::kFwdMaxKvRowStrideBf16);
  const int64_t rows = a->dtype == FA_BF16 ? fa::fwd_rows_per_tile_bf16(a->head_dim) : fa::kFwdRowsPerTileF32;
  const int64_t qtiles = (a->seqlen_q + rows - 1) / rows;
  if (qtiles * a->heads_q * a->batch > 0x7fffffffLL) return fail(FA_ERR_UNSUPPORTED, "%s: grid too large", fn);

  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.o = a->o;
  p.lse = a->lse;
  p.cu_seqlens = nullptr;
  p.q_bs = a->q_stride[0], p.q_ss = a->q_stride[1], p.q_hs = a->q_stride[2];
  p.k_bs = a->k_stride[0], p.k_ss = a->k_stride[1], p.k_hs = a->k_stride[2];
  p.v_bs = a->v_stride[0], p.v_ss = a->v_stride[1], p.v_hs = a->v_stride[2];
  p.o_bs = a->o_stride[0], p.o_ss = a->o_stride[1], p.o_hs = a->o_stride[2];
  p.batch = a->batch;
  p.seqlen_q = a->seqlen_q;
  p.seqlen_k = a->seqlen_k;
  p.total_tokens = 0;
  p.heads_q = a->heads_q;
  p.group = a->heads_q / a->heads_kv;
  p.num_qtiles = (int32_t)qtiles;
  p.wi_chunk = wi_chunk(a->seqlen_k, a->head_dim, a->dtype == FA_BF16 ? 2 : 4, p.group);
  fa::set_work_map(p);
  p.causal = a->causal ? 1 : 0;
  p.scale_log2 = scale_log2(a->scale);
  hipStream_t s = (hipStream_t)stream;
  const hipError_t e = a->dtype == FA_BF16 ? fa::launch_fwd_bf16(p, a->head_dim, s)
                                           : fa::launch_fwd_f32(p, a->head_dim, s);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

fa_status fwd_varlen(const fa_fwd_varlen_args* a, const fa_dropout_args* drop, const char* fn, void* stream) {
  if (!a) return fail(FA_ERR_NULL_POINTER, "%s: args is NULL", fn);
  if (a->num_seqs < 0 || a->total_tokens < 0 || a->max_seqlen < 0 || a->heads_q <= 0 || a->heads_kv <= 0)
    return fail(FA_ERR_BAD_SHAPE, "%s: negative or zero size", fn);
  if (a->heads_q % a->heads_kv)
    return fail(FA_ERR_BAD_SHAPE, "%s: heads_q (%d) is not a multiple of heads_kv (%d)", fn, a->heads_q,
                a->heads_kv);
  if (a->dtype != FA_F32 && a->dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "%s: dtype %d", fn, (int)a->dtype);
  if (a->head_dim != 64 && a->head_dim != 128 && !(a->head_dim == 256 && a->dtype == FA_BF16))
    return fail(FA_ERR_UNSUPPORTED, "%s: head_dim %d, supported 64 and 128 (and 256 for bf16)", fn, a->head_dim);
  if (!(a->scale > 0.f) || !std::isfinite(a->scale))
    return fail(FA_ERR_BAD_SHAPE, "%s: scale must be positive and finite", fn);
  fa::FwdParams p{};
  if (drop) {
    const fa_status st = set_dropout(drop, a->dtype, fn, p);
    if (st != FA_OK) return st;
  }
  if (a->num_seqs == 0 || a->max_seqlen == 0 || a->total_tokens == 0) return ok();
  if (!a->q || !a->k || !a->v || !a->o || !a->cu_seqlens)
    return fail(FA_ERR_NULL_POINTER, "%s: q, k, v, o and cu_seqlens are required", fn);
  const int64_t e16 = a->dtype == FA_BF16 ? 8 : 4;
  if (!strides_ok(a->q_stride, 2, e16) || !strides_ok(a->k_stride, 2, e16) || !strides_ok(a->v_stride, 2, e16) ||
      !strides_ok(a->o_stride, 2, e16))
    return fail(FA_ERR_BAD_SHAPE, "%s: strides must be non-negative multiples of %lld elements", fn,
                (long long)e16);
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o))
    return fail(FA_ERR_BAD_SHAPE, "%s: q, k, v, o must be 16-byte aligned", fn);
  if (a->dtype == FA_BF16 &&
      (a->k_stride[0] > fa::kFwdMaxKvRowStrideBf16 || a->v_stride[0] > fa::kFwdMaxKvRowStrideBf16))
    return fail(FA_ERR_UNSUPPORTED, "%s: bf16 k/v token strides above %lld elements", fn,
                (long long)fa::kFwdMaxKvRowStrideBf16);
  const int64_t rows = a->dtype == FA_BF16 ? fa::fwd_rows_per_tile_bf16(a->head_dim) : fa::kFwdRowsPerTileF32;
  const int64_t qtiles = (a->max_seqlen + rows - 1) / rows;
  if (qtiles * a->heads_q * a->num_seqs > 0x7fffffffLL) return fail(FA_ERR_UNSUPPORTED, "%s: grid too large", fn);

  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.o = a->o;
  p.lse = a->lse;
  p.cu_seqlens = a->cu_seqlens;
  p.q_bs = 0, p.q_ss = a->q_stride[0], p.q_hs = a->q_stride[1];
  p.k_bs = 0, p.k_ss = a->k_stride[0], p.k_hs = a->k_stride[1];
  p.v_bs = 0, p.v_ss = a->v_stride[0], p.v_hs = a->v_stride[1];
  p.o_bs = 0, p.o_ss = a->o_stride[0], p.o_hs = a->o_stride[1];
  p.batch = a->num_seqs;
  p.seqlen_q = a->max_seqlen;
  p.seqlen_k = a->max_seqlen;
  p.total_tokens = a->total_tokens;
  p.heads_q = a->heads_q;
  p.group = a->heads_q / a->heads_kv;
  p.num_qtiles = (int32_t)qtiles;
  p.wi_chunk = wi_chunk(a->max_seqlen, a->head_dim, a->dtype == FA_BF16 ? 2 : 4, p.group);
  fa::set_work_map(p);
  p.causal = a->causal ? 1 : 0;
  p.scale_log2 = scale_log2(a->scale);
  hipStream_t s = (hipStream_t)stream;
  const hipError_t e = a->dtype == FA_BF16 ? fa::launch_fwd_bf16(p, a->head_dim, s)
                                           : fa::launch_fwd_f32(p, a->head_dim, s);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

}  // namespace

FA_EXPORT fa_status fa_fwd(const fa_fwd_args* a, void* stream) { return fwd_dense(a, nullptr, "fa_fwd", stream); }

FA_EXPORT fa_status fa_fwd_dropout(const fa_fwd_args* a, const fa_dropout_args* d, void* stream) {
  if (!d) return fail(FA_ERR_NULL_POINTER, "fa_fwd_dropout: dropout args is NULL");
  return fwd_dense(a, d, "fa_fwd_dropout", stream);
}

FA_EXPORT fa_status fa_fwd_varlen(const fa_fwd_varlen_args* a, void* stream) {
  return fwd_varlen(a, nullptr, "fa_fwd_varlen", stream);
}

FA_EXPORT fa_status fa_fwd_varlen_dropout(const fa_fwd_varlen_args* a, const fa_dropout_args* d, void* stream) {
  if (!d) return fail(FA_ERR_NULL_POINTER, "fa_fwd_varlen_dropout: dropout args is NULL");
  return fwd_varlen(a, d, "fa_fwd_varlen_dropout", stream);
}

FA_EXPORT fa_status fa_fwd_fp8(const fa_fwd_fp8_args* a, void* stream) {
  if (!a) return fail(FA_ERR_NULL_POINTER, "fa_fwd_fp8: args is NULL");
  if (a->batch < 0 || a->seqlen_q < 0 || a->seqlen_k < 0 || a->heads_q <= 0 || a->heads_kv <= 0)
    return fail(FA_ERR_BAD_SHAPE, "fa_fwd_fp8: negative or zero size");
  if (a->heads_q % a->heads_kv)
    return fail(FA_ERR_BAD_SHAPE, "fa_fwd_fp8: heads_q (%d) is not a multiple of heads_kv (%d)", a->heads_q,
                a->heads_kv);
  if (a->head_dim != 128)
    return fail(FA_ERR_UNSUPPORTED, "fa_fwd_fp8: head_dim %d, supported 128", a->head_dim);
  if (!(a->scale > 0.f) || !std::isfinite(a->scale))
    return fail(FA_ERR_BAD_SHAPE, "fa_fwd_fp8: scale must be positive and finite");
  for (float d : {a->q_descale, a->k_descale, a->v_descale})
    if (!(d > 0.f) || !std::isfinite(d))
      return fail(FA_ERR_BAD_SHAPE, "fa_fwd_fp8: descale factors must be positive and finite");
  if (a->batch == 0 || a->seqlen_q == 0) return ok();
  if (!a->q || !a->o) return fail(FA_ERR_NULL_POINTER, "fa_fwd_fp8: q and o are required");
  if (a->seqlen_k > 0 && (!a->k || !a->v))
    return fail(FA_ERR_NULL_POINTER, "fa_fwd_fp8: k and v are required when seqlen_k > 0");
  if (!strides_ok(a->q_stride, 3, 16) || !strides_ok(a->k_stride, 3, 16) || !strides_ok(a->v_stride, 3, 16) ||
      !strides_ok(a->o_stride, 3, 8))
    return fail(FA_ERR_BAD_SHAPE, "fa_fwd_fp8: strides must be non-negative multiples of 16 bytes");
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o))
    return fail(FA_ERR_BAD_SHAPE, "fa_fwd_fp8: q, k, v, o must be 16-byte aligned");
  if (a->k_stride[1] > fa::kFwdMaxKvRowStrideBf16 || a->v_stride[1] > fa::kFwdMaxKvRowStrideBf16)
    return fail(FA_ERR_UNSUPPORTED, "fa_fwd_fp8: k/v sequence strides above %lld elements",
                (long long)fa::kFwdMaxKvRowStrideBf16);
  const int64_t qtiles = (a->seqlen_q + fa::kFwdRowsPerTileFp8 - 1) / fa::kFwdRowsPerTileFp8;
  if (qtiles * a->heads_q * a->batch > 0x7fffffffLL) return fail(FA_ERR_UNSUPPORTED, "fa_fwd_fp8: grid too large");

  fa::FwdParams p{};
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.o = a->o;
  p.lse = a->lse;
  p.cu_seqlens = nullptr;
  p.q_bs = a->q_stride[0], p.q_ss = a->q_stride[1], p.q_hs = a->q_stride[2];
  p.k_bs = a->k_stride[0], p.k_ss = a->k_stride[1], p.k_hs = a->k_stride[2];
  p.v_bs = a->v_stride[0], p.v_ss = a->v_stride[1], p.v_hs = a->v_stride[2];
  p.o_bs = a->o_stride[0], p.o_ss = a->o_stride[1], p.o_hs = a->o_stride[2];
  p.batch = a->batch;
  p.seqlen_q = a->seqlen_q;
  p.seqlen_k = a->seqlen_k;
  p.heads_q = a->heads_q;
  p.group = a->heads_q / a->heads_kv;
  p.num_qtiles = (int32_t)qtiles;
  p.wi_chunk = wi_chunk(a->seqlen_k, a->head_dim, 1, p.group);
  fa::set_work_map(p);
  p.causal = a->causal ? 1 : 0;
  p.scale_log2 = (float)((double)a->scale * a->q_descale * a->k_descale * 1.4426950408889634073599);
  p.o_scale = a->v_descale;
  const hipError_t e = fa::launch_fwd_fp8(p, a->head_dim, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "fa_fwd_fp8: launch failed: %s", hipGetErrorString(e));
  return ok();
}

FA_EXPORT fa_status fa_fwd_varlen_fp8(const fa_fwd_varlen_fp8_args* a, void* stream) {
  if (!a) return fail(FA_ERR_NULL_POINTER, "fa_fwd_varlen_fp8: args is NULL");
  if (a->num_seqs < 0 || a->total_tokens < 0 || a->max_seqlen < 0 || a->heads_q <= 0 || a->heads_kv <= 0)
    return fail(FA_ERR_BAD_SHAPE, "fa_fwd_varlen_fp8: negative or zero size");
  if (a->heads_q % a->heads_kv)
    return fail(FA_ERR_BAD_SHAPE, "fa_fwd_varlen_fp8: heads_q (%d) is not a multiple of heads_kv (%d)",
                a->heads_q, a->heads_kv);
  if (a->head_dim != 128)
    return fail(FA_ERR_UNSUPPORTED, "fa_fwd_varlen_fp8: head_dim %d, supported 128", a->head_dim);
  if (!(a->scale > 0.f) || !std::isfinite(a->scale))
    return fail(FA_ERR_BAD_SHAPE, "fa_fwd_varlen_fp8: scale must be positive and finite");
  for (float d : {a->q_descale, a->k_descale, a->v_descale})
    if (!(d > 0.f) || !std::isfinite(d))
      return fail(FA_ERR_BAD_SHAPE, "fa_fwd_varlen_fp8: descale factors must be positive and finite");
  if (a->num_seqs == 0 || a->max_seqlen == 0 || a->total_tokens == 0) return ok();
  if (!a->q || !a->k || !a->v || !a->o || !a->cu_seqlens)
    return fail(FA_ERR_NULL_POINTER, "fa_fwd_varlen_fp8: q, k, v, o and cu_seqlens are required");
  if (!strides_ok(a->q_stride, 2, 16) || !strides_ok(a->k_stride, 2, 16) || !strides_ok(a->v_stride, 2, 16) ||
      !strides_ok(a->o_stride, 2, 8))
    return fail(FA_ERR_BAD_SHAPE, "fa_fwd_varlen_fp8: strides must be non-negative multiples of 16 bytes");
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o))
    return fail(FA_ERR_BAD_SHAPE, "fa_fwd_varlen_fp8: q, k, v, o must be 16-byte aligned");
  if (a->k_stride[0] > fa::kFwdMaxKvRowStrideBf16 || a->v_stride[0] > fa::kFwdMaxKvRowStrideBf16)
    return fail(FA_ERR_UNSUPPORTED, "fa_fwd_varlen_fp8: k/v token strides above %lld elements",
                (long long)fa::kFwdMaxKvRowStrideBf16);
  const int64_t qtiles = (a->max_seqlen + fa::kFwdRowsPerTileFp8 - 1) / fa::kFwdRowsPerTileFp8;
  if (qtiles * a->heads_q * a->num_seqs > 0x7fffffffLL)
    return fail(FA_ERR_UNSUPPORTED, "fa_fwd_varlen_fp8: grid too large");

  fa::FwdParams p{};
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.o = a->o;
  p.lse = a->lse;
  p.cu_seqlens = a->cu_seqlens;
  p.q_bs = 0, p.q_ss = a->q_stride[0], p.q_hs = a->q_stride[1];
  p.k_bs = 0, p.k_ss = a->k_stride[0], p.k_hs = a->k_stride[1];
  p.v_bs = 0, p.v_ss = a->v_stride[0], p.v_hs = a->v_stride[1];
  p.o_bs = 0, p.o_ss = a->o_stride[0], p.o_hs = a->o_stride[1];
  p.batch = a->num_seqs;
  p.seqlen_q = a->max_seqlen;
  p.seqlen_k = a->max_seqlen;
  p.total_tokens = a->total_tokens;
  p.heads_q = a->heads_q;
  p.group = a->heads_q / a->heads_kv;
  p.num_qtiles = (int32_t)qtiles;
  p.wi_chunk = wi_chunk(a->max_seqlen, a->head_dim, 1, p.group);
  fa::set_work_map(p);
  p.causal = a->causal ? 1 : 0;
  p.scale_log2 = (float)((double)a->scale * a->q_descale * a->k_descale * 1.4426950408889634073599);
  p.o_scale = a->v_descale;
  const hipError_t e = fa::launch_fwd_fp8(p, a->head_dim, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "fa_fwd_varlen_fp8: launch failed: %s", hipGetErrorString(e));
  return ok();
}

namespace {
// Chunked prefill over a paged pool: bf16, or FP8 E4M3 queries and pools
// with descale factors (fp8 != nullptr: q, k, v descales).
fa_status paged_impl(const fa_fwd_paged_args* a, const float* fp8, const char* fn, void* stream) {
  if (!a) return fail(FA_ERR_NULL_POINTER, "%s: args is NULL", fn);
  if (a->num_seqs < 0 || a->total_q < 0 || a->max_seqlen_q < 0 || a->max_seqlen_k < 0 || a->heads_q <= 0 ||
      a->heads_kv <= 0 || a->max_blocks_per_seq < 0 || a->num_blocks < 0)
    return fail(FA_ERR_BAD_SHAPE, "%s: negative or zero size", fn);
  if (a->heads_q % a->heads_kv)
    return fail(FA_ERR_BAD_SHAPE, "%s: heads_q (%d) is not a multiple of heads_kv (%d)", fn, a->heads_q,
                a->heads_kv);
  if (fp8 ? a->head_dim != 128 : (a->head_dim != 64 && a->head_dim != 128 && a->head_dim != 256))
    return fail(FA_ERR_UNSUPPORTED, "%s: head_dim %d, supported %s", fn, a->head_dim, fp8 ? "128" : "64, 128 and 256");
  if (fp8)
    for (int i = 0; i < 3; ++i)
      if (!(fp8[i] > 0.f) || !std::isfinite(fp8[i]))
        return fail(FA_ERR_BAD_SHAPE, "%s: descale factors must be positive and finite", fn);
  if (a->block_size != fa::kFwdPagedBlock)
    return fail(FA_ERR_UNSUPPORTED, "%s: block_size %d, supported %d", fn, a->block_size,
                fa::kFwdPagedBlock);
  if ((int64_t)a->max_seqlen_k > (int64_t)a->max_blocks_per_seq * a->block_size)
    return fail(FA_ERR_BAD_SHAPE, "%s: max_seqlen_k %d exceeds max_blocks_per_seq * block_size", fn,
                a->max_seqlen_k);
  if (!(a->scale > 0.f) || !std::isfinite(a->scale))
    return fail(FA_ERR_BAD_SHAPE, "%s: scale must be positive and finite", fn);
  if (a->num_seqs == 0 || a->max_seqlen_q == 0 || a->total_q == 0) return ok();
  if (!a->q || !a->o || !a->cu_seqlens_q || !a->seq_lens_k)
    return fail(FA_ERR_NULL_POINTER, "%s: q, o, cu_seqlens_q and seq_lens_k are required", fn);
  if (a->max_seqlen_k > 0 && (!a->k_pool || !a->v_pool || !a->block_table))
    return fail(FA_ERR_NULL_POINTER, "%s: pools and block_table are required when max_seqlen_k > 0", fn);
  // 16-byte loads and stores: q and pool strides are multiples of 16 bytes
  // (elements: 8 bf16 or 16 E4M3), o strides of 8 bf16 elements
  if (!strides_ok(a->pool_stride, 3, fp8 ? 16 : 8) || !strides_ok(a->q_stride, 2, fp8 ? 16 : 8) ||
      !strides_ok(a->o_stride, 2, 8))
    return fail(FA_ERR_BAD_SHAPE, "%s: strides must be non-negative multiples of 16 bytes", fn);
  if (!aligned16(a->q) || !aligned16(a->k_pool) || !aligned16(a->v_pool) || !aligned16(a->o))
    return fail(FA_ERR_BAD_SHAPE, "%s: q, pools and o must be 16-byte aligned", fn);
  if (a->pool_stride[2] > fa::kFwdMaxKvRowStrideBf16)
    return fail(FA_ERR_UNSUPPORTED, "%s: pool token stride above %lld elements", fn,
                (long long)fa::kFwdMaxKvRowStrideBf16);
  const int64_t rows = fp8 ? fa::kFwdRowsPerTileFp8 : fa::fwd_rows_per_tile_bf16(a->head_dim);
  const int64_t qtiles = (a->max_seqlen_q + rows - 1) / rows;
  if (qtiles * a->heads_q * a->num_seqs > 0x7fffffffLL)
    return fail(FA_ERR_UNSUPPORTED, "%s: grid too large", fn);

  fa::FwdParams p{};
  p.q = a->q;
  p.k = a->k_pool;
  p.v = a->v_pool;
  p.o = a->o;
  p.lse = a->lse;
  p.cu_seqlens = a->cu_seqlens_q;
  p.q_bs = 0, p.q_ss = a->q_stride[0], p.q_hs = a->q_stride[1];
  p.o_bs = 0, p.o_ss = a->o_stride[0], p.o_hs = a->o_stride[1];
  p.batch = a->num_seqs;
  p.seqlen_q = a->max_seqlen_q;
  p.seqlen_k = a->max_seqlen_k;
  p.total_tokens = a->total_q;
  p.heads_q = a->heads_q;
  p.group = a->heads_q / a->heads_kv;
  p.num_qtiles = (int32_t)qtiles;
  p.wi_chunk = wi_chunk(a->max_seqlen_k, a->head_dim, fp8 ? 1 : 2, p.group);
  fa::set_work_map(p);
  p.causal = a->causal ? 1 : 0;
  p.scale_log2 = fp8 ? (float)((double)a->scale * fp8[0] * fp8[1] * 1.4426950408889634073599) : scale_log2(a->scale);
  p.o_scale = fp8 ? fp8[2] : 1.f;
  p.paged = 1;
  p.block_table = a->block_table;  // with max_seqlen_k == 0 neither table nor pools are read
  p.seq_lens_k = a->seq_lens_k;
  p.max_blocks = a->max_blocks_per_seq;
  p.p_bs = a->pool_stride[0], p.p_hs = a->pool_stride[1], p.p_ts = a->pool_stride[2];
  const hipError_t e = fp8 ? fa::launch_fwd_fp8(p, a->head_dim, (hipStream_t)stream)
                           : fa::launch_fwd_bf16(p, a->head_dim, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}
}  // namespace

FA_EXPORT fa_status fa_fwd_paged(const fa_fwd_paged_args* a, void* stream) {
  return paged_impl(a, nullptr, "fa_fwd_paged", stream);
}

FA_EXPORT fa_status fa_fwd_paged_fp8(const fa_fwd_paged_fp8_args* a, void* stream) {
  if (!a) return fail(FA_ERR_NULL_POINTER, "fa_fwd_paged_fp8: args is NULL");
  const float ds[3] = {a->q_descale, a->k_descale, a->v_descale};
  return paged_impl(&a->base, ds, "fa_fwd_paged_fp8", stream);
}

namespace {
size_t decode_workspace(const fa_decode_paged_args* a, bool kv8) {
  if (check_decode(a) != FA_OK) return 0;
  const int parts = decode_parts(a, kv8);
  if (parts < 1) {
    fail(FA_ERR_HIP, "fa_decode_paged_workspace_size: cannot query the current device");
    return 0;
  }
  return fa::decode_workspace_bytes(parts, a->batch, a->heads_q, a->head_dim);
}

int32_t decode_splits(const fa_decode_paged_args* a, bool kv8) {
  if (check_decode(a) != FA_OK) return 0;
  const int parts = decode_parts(a, kv8);
  if (parts < 1) {
    fail(FA_ERR_HIP, "fa_decode_paged_num_splits: cannot query the current device");
    return 0;
  }
  return parts;
}
}  // namespace

FA_EXPORT size_t fa_decode_paged_workspace_size(const fa_decode_paged_args* a) { return decode_workspace(a, false); }

FA_EXPORT int32_t fa_decode_paged_num_splits(const fa_decode_paged_args* a) { return decode_splits(a, false); }

FA_EXPORT size_t fa_decode_paged_fp8_workspace_size(const fa_decode_paged_fp8_args* a) {
  return a ? decode_workspace(&a->base, true) : 0;
}

FA_EXPORT int32_t fa_decode_paged_fp8_num_splits(const fa_decode_paged_fp8_args* a) {
  return a ? decode_splits(&a->base, true) : 0;
}

namespace {
// Paged decode over bf16 pools, or E4M3 pools (kv8) with descale factors.
// no_alloc: the partial states go to the library's own per-device scratch
// array instead of the caller's workspace (whose fields are then ignored).
fa_status decode_impl(const fa_decode_paged_args* a, bool kv8, float k_descale, float v_descale, const char* fn,
                      void* stream, bool no_alloc = false) {
  const fa_status st = check_decode(a);
  if (st != FA_OK) return st;
  if (!(a->scale > 0.f) || !std::isfinite(a->scale))
    return fail(FA_ERR_BAD_SHAPE, "%s: scale must be positive and finite", fn);
  if (kv8 && (!(k_descale > 0.f) || !std::isfinite(k_descale) || !(v_descale > 0.f) || !std::isfinite(v_descale)))
    return fail(FA_ERR_BAD_SHAPE, "%s: descale factors must be positive and finite", fn);
  if (a->batch == 0) return ok();
  if (!a->q || !a->seq_lens || !a->o || (!no_alloc && !a->workspace))
    return fail(FA_ERR_NULL_POINTER, "%s: q, seq_lens, o and workspace are required", fn);
  if (a->max_seq_len > 0 && (!a->k_pool || !a->v_pool || !a->block_table))
    return fail(FA_ERR_NULL_POINTER, "%s: pools and block_table are required when max_seq_len > 0", fn);
  // 16-byte loads: pool strides are multiples of 16 bytes (8 bf16 elements, 16 E4M3 bytes)
  if (!strides_ok(a->pool_stride, 3, kv8 ? 16 : 8) || !strides_ok(a->q_stride, 2, 8) || !strides_ok(a->o_stride, 2, 8))
    return fail(FA_ERR_BAD_SHAPE, "%s: strides must be non-negative multiples of 16 bytes", fn);
  if (!aligned16(a->q) || !aligned16(a->k_pool) || !aligned16(a->v_pool) || !aligned16(a->o) ||
      (!no_alloc && !aligned16(a->workspace)))
    return fail(FA_ERR_BAD_SHAPE, "%s: q, pools, o and workspace must be 16-byte aligned", fn);
  const int parts = decode_parts(a, kv8);
  if (parts < 1) return fail(FA_ERR_HIP, "%s: cannot query the current device", fn);
  const size_t need = fa::decode_workspace_bytes(parts, a->batch, a->heads_q, a->head_dim);
  void* ws = a->workspace;
  if (no_alloc) {
    if (need > fa::kDecodeScratchBytes)
      return fail(FA_ERR_WORKSPACE_TOO_SMALL,
                  "%s: these arguments need %zu bytes of partial states, the library holds %zu (lower num_splits "
                  "or the batch, or call fa_decode_paged with a workspace)",
                  fn, need, fa::kDecodeScratchBytes);
    const hipError_t e = fa::decode_scratch(&ws);
    if (e != hipSuccess) return fail(FA_ERR_HIP, "%s: scratch address: %s", fn, hipGetErrorString(e));
  } else if (a->workspace_bytes < need) {
    return fail(FA_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu bytes, need %zu", fn, a->workspace_bytes, need);
  }

  fa::DecodeParams p{};
  p.q = a->q;
  p.k_pool = a->k_pool;
  p.v_pool = a->v_pool;
  p.p_bs = a->pool_stride[0], p.p_hs = a->pool_stride[1], p.p_ts = a->pool_stride[2];
  p.q_bs = a->q_stride[0], p.q_hs = a->q_stride[1];
  p.o_bs = a->o_stride[0], p.o_hs = a->o_stride[1];
  p.block_table = a->block_table;
  p.seq_lens = a->seq_lens;
  p.o = a->o;
  p.lse = a->lse;
  p.num_splits = parts;
  const size_t rows = (size_t)a->heads_q * (size_t)(parts + a->batch);
  p.ws_o = (float*)ws;
  p.ws_ml = p.ws_o + rows * a->head_dim;
  p.batch = a->batch;
  p.heads_q = a->heads_q;
  p.heads_kv = a->heads_kv;
  p.group = a->heads_q / a->heads_kv;
  p.max_blocks = a->max_blocks_per_seq;
  p.max_seq_len = a->max_seq_len;
  p.scale_log2 = kv8 ? (float)((double)a->scale * k_descale * 1.4426950408889634073599) : scale_log2(a->scale);
  p.kv8 = kv8 ? 1 : 0;
  p.o_scale = kv8 ? v_descale : 1.f;
  const hipError_t e = fa::launch_decode_paged(p, a->head_dim, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}
}  // namespace

FA_EXPORT fa_status fa_decode_paged(const fa_decode_paged_args* a, void* stream) {
  return decode_impl(a, false, 1.f, 1.f, "fa_decode_paged", stream);
}

FA_EXPORT fa_status fa_decode_paged_noalloc(const fa_decode_paged_args* a, void* stream) {
  return decode_impl(a, false, 1.f, 1.f, "fa_decode_paged_noalloc", stream, true);
}

FA_EXPORT size_t fa_decode_paged_noalloc_max_bytes(void) { return fa::kDecodeScratchBytes; }

FA_EXPORT fa_status fa_decode_paged_fp8(const fa_decode_paged_fp8_args* a, void* stream) {
  if (!a) return fail(FA_ERR_NULL_POINTER, "fa_decode_paged_fp8: args is NULL");
  return decode_impl(&a->base, true, a->k_descale, a->v_descale, "fa_decode_paged_fp8", stream);
}

FA_EXPORT fa_status fa_merge_states(const fa_merge_states_args* a, void* stream) {
  if (!a) return fail(FA_ERR_NULL_POINTER, "fa_merge_states: args is NULL");
  if (a->num_parts < 1 || a->batch < 0 || a->seqlen < 0 || a->heads < 0)
    return fail(FA_ERR_BAD_SHAPE, "fa_merge_states: num_parts must be >= 1 and sizes >= 0");
  if (a->head_dim != 64 && a->head_dim != 128 && a->head_dim != 256)
    return fail(FA_ERR_UNSUPPORTED, "fa_merge_states: head_dim %d (supported: 64, 128, 256)", a->head_dim);
  if (a->dtype != FA_BF16 && a->dtype != FA_F32)
    return fail(FA_ERR_UNSUPPORTED, "fa_merge_states: dtype %d", (int)a->dtype);
  const int64_t rows = (int64_t)a->batch * a->seqlen * a->heads;
  if (rows == 0) return ok();
  if ((double)a->num_parts * (double)rows * a->head_dim >= 1099511627776.0)
    return fail(FA_ERR_UNSUPPORTED, "fa_merge_states: more than 2^40 input elements");
  if (rows * a->head_dim >= (int64_t(1) << 34))
    return fail(FA_ERR_UNSUPPORTED, "fa_merge_states: 2^34 or more elements per part");
  if (!a->o_parts || !a->lse_parts || !a->o) return fail(FA_ERR_NULL_POINTER, "fa_merge_states: NULL tensor");
  if (!aligned16(a->o_parts) || !aligned16(a->lse_parts) || !aligned16(a->o) || (a->lse && !aligned16(a->lse)))
    return fail(FA_ERR_BAD_SHAPE, "fa_merge_states: pointers must be 16-byte aligned");
  fa::MergeParams p{};
  p.o_parts = a->o_parts;
  p.lse_parts = a->lse_parts;
  p.o = a->o;
  p.lse = a->lse;
  p.rows = rows;
  p.part_elems = rows * a->head_dim;
  p.part_rows = rows;
  p.parts = a->num_parts;
  p.seqlen = a->seqlen;
  p.heads = a->heads;
  p.head_dim = a->head_dim;
  p.f32 = a->dtype == FA_F32;
  p.by_heads = fa::make_intdiv(a->heads > 0 ? a->heads : 1);
  p.by_seqlen = fa::make_intdiv(a->seqlen > 0 ? a->seqlen : 1);
  const hipError_t e = fa::launch_merge(p, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "fa_merge_states: %s", hipGetErrorString(e));
  return ok();
}

FA_EXPORT const char* fa_status_string(fa_status status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL_POINTER: return "null pointer";
    case FA_ERR_BAD_SHAPE: return "bad shape or layout";
    case FA_ERR_UNSUPPORTED: return "unsupported configuration";
    case FA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case FA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

FA_EXPORT const char* fa_last_error(void) { return g_last_error.c_str(); }

FA_EXPORT int32_t fa_abi_version(void) { return FA_ABI_VERSION; }
