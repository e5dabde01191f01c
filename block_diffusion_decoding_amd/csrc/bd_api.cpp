// C ABI of libbd: argument validation and dispatch to the HIP launchers.
// Every check here runs on the host before anything is enqueued, so the error
// paths need no GPU.  The entry points are declared, with their contracts, in
// include/bd.h.
#include "bd.h"
#include "bd_kernels.hpp"

#include <climits>
#include <cmath>
#include <cstdint>
#include <initializer_list>

namespace {

thread_local int g_last_hip_error = 0;

constexpr long long kMaxGrid = 0x7fffffffLL;

bd_status hip_status(hipError_t e) {
  if (e == hipSuccess) return BD_OK;
  g_last_hip_error = (int)e;
  return BD_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The product of non-negative sizes exceeds limit (>= 0), found without
// overflow: while the running product is at most limit, one more factor up to
// INT_MAX keeps it below 2^62.
bool exceeds(long long limit, std::initializer_list<long long> factors) {
  long long p = 1;
  for (const long long f : factors) {
    if (f != 0 && p > limit / f) return true;
    p *= f;
  }
  return p > limit;
}

// Sizes of an attention call: positive, whole query-head groups, and a grid
// that fits (one workgroup per (batch, head, row tile) at most).
bool attn_sizes_ok(int batch, int seqlen, int hq, int hkv) {
  if (batch <= 0 || seqlen <= 0 || hq <= 0 || hkv <= 0 || hq % hkv != 0) return false;
  return !exceeds(kMaxGrid, {batch, hq, seqlen});
}

// Rows of a commit call, and its reduce grid, that fit.
bool commit_rows_ok(int n_seq, int blk_len, int vocab) {
  if (n_seq <= 0 || blk_len <= 0 || vocab <= 0 || vocab > BD_MAX_VOCAB || blk_len > bd::kCommitMaxBlock)
    return false;
  const long long rows = (long long)n_seq * blk_len;
  return !exceeds(kMaxGrid, {rows, bd::commit_chunks_per_row(rows, vocab)});
}

float resolve_scale(float scale, int head_dim) { return scale > 0.f ? scale : 1.0f / std::sqrt((float)head_dim); }

bd_status check_attn_shape(int batch, int seqlen, int hq, int hkv, int d, int blk, bd_dtype dtype, float scale) {
  if (batch <= 0 || seqlen <= 0 || hq <= 0 || hkv <= 0 || d <= 0 || blk <= 0) return BD_ERR_SHAPE;
  if (hq % hkv != 0) return BD_ERR_SHAPE;
  if (std::isnan(scale) || std::isinf(scale)) return BD_ERR_VALUE;
  if (dtype == BD_BF16) {
    if (d != 128) return BD_ERR_UNSUPPORTED;
  } else if (dtype == BD_F32) {
    if (d > 128) return BD_ERR_UNSUPPORTED;
  } else {
    return BD_ERR_UNSUPPORTED;
  }
  if (!attn_sizes_ok(batch, seqlen, hq, hkv)) return BD_ERR_SHAPE;
  return BD_OK;
}

bd_status commit_common(const void* logits, int64_t row_stride, int n_seq, int blk_len, int vocab, bd_dtype dtype,
                        float threshold, const float* thresholds, bd_fallback fallback, int32_t* tokens,
                        uint8_t* masked, float* conf, int32_t* pred, int32_t* n_committed, int32_t* n_masked_left,
                        void* workspace, size_t ws_bytes, hipStream_t stream, bool noalloc = false) {
  if (!logits || !tokens || !masked) return BD_ERR_NULL;
  if (n_seq <= 0 || blk_len <= 0 || vocab <= 0 || row_stride < vocab) return BD_ERR_SHAPE;
  if (blk_len > bd::kCommitMaxBlock) return BD_ERR_UNSUPPORTED;
  if (dtype != BD_F32 && dtype != BD_BF16) return BD_ERR_UNSUPPORTED;
  if (std::isnan(threshold)) return BD_ERR_VALUE;
  if (fallback != BD_FALLBACK_NONE && fallback != BD_FALLBACK_TOP1) return BD_ERR_VALUE;
  if (!commit_rows_ok(n_seq, blk_len, vocab)) return BD_ERR_SHAPE;
  const size_t need = bd::commit_workspace_bytes(n_seq, blk_len, vocab);
  if (noalloc) {
    if (need > bd::kNoAllocScratchBytes) return BD_ERR_SCRATCH;
  } else if (!workspace || ws_bytes < need) {
    return BD_ERR_WORKSPACE;
  } else if (!aligned16(workspace)) {
    return BD_ERR_ALIGNMENT;
  }
  bd::CommitArgs a{logits, row_stride, n_seq, blk_len, vocab, dtype == BD_BF16, threshold, thresholds,
                   fallback == BD_FALLBACK_TOP1, tokens, masked, conf, pred, n_committed, n_masked_left, workspace};
  return hip_status(noalloc ? bd::launch_commit_noalloc(a, stream) : bd::launch_commit(a, stream));
}

static_assert(bd::kNoAllocScratchBytes == BD_NOALLOC_SCRATCH_BYTES, "scratch size of the header and the kernels");

}  // namespace

extern "C" {

const char* bd_status_string(bd_status s) {
  switch (s) {
    case BD_OK: return "ok";
    case BD_ERR_NULL: return "required pointer is NULL";
    case BD_ERR_SHAPE: return "invalid or inconsistent sizes";
    case BD_ERR_UNSUPPORTED: return "dtype / head_dim combination not supported";
    case BD_ERR_WORKSPACE: return "workspace missing or too small";
    case BD_ERR_VALUE: return "scalar argument out of its domain";
    case BD_ERR_HIP: return "HIP runtime error";
    case BD_ERR_ALIGNMENT: return "tensor or workspace pointer not 16-byte aligned";
    case BD_ERR_SCRATCH: return "problem exceeds the fixed scratch of the no-allocation entry point";
  }
  return "unknown status";
}

int bd_last_hip_error(void) { return g_last_hip_error; }

int bd_version(void) { return 100; }

bd_status bd_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int batch, int seqlen,
                      int n_q_heads, int n_kv_heads, int head_dim, int block_size, float softmax_scale,
                      bd_dtype dtype, hipStream_t stream) {
  if (!q || !k || !v || !o) return BD_ERR_NULL;
  bd_status st = check_attn_shape(batch, seqlen, n_q_heads, n_kv_heads, head_dim, block_size, dtype, softmax_scale);
  if (st != BD_OK) return st;
  bd::AttnShape s{batch, seqlen, n_q_heads, n_kv_heads, head_dim, block_size,
                  resolve_scale(softmax_scale, head_dim)};
  if (dtype == BD_BF16) {
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return BD_ERR_ALIGNMENT;
    return hip_status(bd::launch_attn_fwd_bf16(q, k, v, o, lse, s, stream));
  }
  return hip_status(bd::launch_attn_fwd_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                                            static_cast<const float*>(v), static_cast<float*>(o), lse, s,
                                            stream));
}

size_t bd_attn_bwd_workspace_size(int batch, int seqlen, int n_q_heads, int n_kv_heads, int head_dim) {
  if (head_dim <= 0 || !attn_sizes_ok(batch, seqlen, n_q_heads, n_kv_heads)) return 0;
  return bd::attn_bwd_workspace_bytes(batch, seqlen, n_q_heads);
}

bd_status bd_attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* d_o, void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes, int batch,
                      int seqlen, int n_q_heads, int n_kv_heads, int head_dim, int block_size,
                      float softmax_scale, bd_dtype dtype, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse || !d_o || !dq || !dk || !dv) return BD_ERR_NULL;
  bd_status st = check_attn_shape(batch, seqlen, n_q_heads, n_kv_heads, head_dim, block_size, dtype, softmax_scale);
  if (st != BD_OK) return st;
  const size_t need = bd::attn_bwd_workspace_bytes(batch, seqlen, n_q_heads);
  if (!workspace || ws_bytes < need) return BD_ERR_WORKSPACE;
  if (!aligned16(workspace)) return BD_ERR_ALIGNMENT;
  bd::AttnShape s{batch, seqlen, n_q_heads, n_kv_heads, head_dim, block_size,
                  resolve_scale(softmax_scale, head_dim)};
  if (dtype == BD_BF16) {
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(d_o) || !aligned16(dq) ||
        !aligned16(dk) || !aligned16(dv))
      return BD_ERR_ALIGNMENT;
    const hipError_t e = bd::launch_attn_bwd_bf16(q, k, v, o, lse, d_o, dq, dk, dv, workspace, s, stream);
    if (e == hipErrorNotSupported) return BD_ERR_UNSUPPORTED;
    return hip_status(e);
  }
  return hip_status(bd::launch_attn_bwd_f32(
      static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
      static_cast<const float*>(o), lse, static_cast<const float*>(d_o), static_cast<float*>(dq),
      static_cast<float*>(dk), static_cast<float*>(dv), workspace, s, stream));
}

size_t bd_attn_decode_workspace_size(int n_seq, int blk_len, int max_prefix_len, int n_q_heads, int n_kv_heads,
                                     int head_dim) {
  if (max_prefix_len < 0 || head_dim <= 0 || !attn_sizes_ok(n_seq, blk_len, n_q_heads, n_kv_heads) ||
      (long long)max_prefix_len + blk_len > kMaxGrid / 2)
    return 0;
  bd::DecodeShape s{n_seq, blk_len, max_prefix_len, n_q_heads, n_kv_heads, head_dim, 1.f};
  return bd::decode_workspace_bytes(s, 1);
}

bd_status bd_attn_decode_block(const void* q_blk, const void* k_blk, const void* v_blk, const void* k_cache,
                               const void* v_cache, const int64_t* prefix_start, const int32_t* prefix_len,
                               int max_prefix_len, void* o, float* lse, int n_seq, int blk_len, int n_q_heads,
                               int n_kv_heads, int head_dim, float softmax_scale, bd_dtype dtype, void* workspace,
                               size_t ws_bytes, hipStream_t stream) {
  if (!q_blk || !k_blk || !v_blk || !o || !prefix_start || !prefix_len) return BD_ERR_NULL;
  if (max_prefix_len > 0 && (!k_cache || !v_cache)) return BD_ERR_NULL;
  if (n_seq <= 0 || blk_len <= 0 || max_prefix_len < 0) return BD_ERR_SHAPE;
  bd_status st = check_attn_shape(n_seq, blk_len, n_q_heads, n_kv_heads, head_dim, 1, dtype, softmax_scale);
  if (st != BD_OK) return st;
  if ((long long)max_prefix_len + blk_len > kMaxGrid / 2) return BD_ERR_SHAPE;
  bd::DecodeShape s{n_seq, blk_len, max_prefix_len, n_q_heads, n_kv_heads, head_dim,
                    resolve_scale(softmax_scale, head_dim)};
  if (dtype == BD_BF16) {
    if (!aligned16(q_blk) || !aligned16(k_blk) || !aligned16(v_blk) || !aligned16(o) ||
        (k_cache && !aligned16(k_cache)) || (v_cache && !aligned16(v_cache)))
      return BD_ERR_ALIGNMENT;
    const size_t need = bd::decode_workspace_bytes(s, 1);
    if (!workspace || ws_bytes < need) return BD_ERR_WORKSPACE;
    if (!aligned16(workspace)) return BD_ERR_ALIGNMENT;
    return hip_status(bd::launch_decode_bf16(q_blk, k_blk, v_blk, k_cache, v_cache, prefix_start, prefix_len, o,
                                             lse, workspace, s, stream));
  }
  return hip_status(bd::launch_decode_f32(
      static_cast<const float*>(q_blk), static_cast<const float*>(k_blk), static_cast<const float*>(v_blk),
      static_cast<const float*>(k_cache), static_cast<const float*>(v_cache), prefix_start, prefix_len,
      static_cast<float*>(o), lse, s, stream));
}

bd_status bd_attn_decode_block_paged(const void* q_blk, const void* k_blk, const void* v_blk, const void* k_pages,
                                     const void* v_pages, const int32_t* block_table, int max_pages_per_seq,
                                     int page_size, const int32_t* prefix_len, int max_prefix_len, void* o,
                                     float* lse, int n_seq, int blk_len, int n_q_heads, int n_kv_heads, int head_dim,
                                     float softmax_scale, bd_dtype dtype, void* workspace, size_t ws_bytes,
                                     hipStream_t stream) {
  if (!q_blk || !k_blk || !v_blk || !o || !prefix_len) return BD_ERR_NULL;
  if (max_prefix_len > 0 && (!k_pages || !v_pages || !block_table)) return BD_ERR_NULL;
  if (n_seq <= 0 || blk_len <= 0 || max_prefix_len < 0 || max_pages_per_seq < 0) return BD_ERR_SHAPE;
  if (page_size <= 0 || page_size % 32 != 0) return BD_ERR_UNSUPPORTED;
  if ((long long)max_pages_per_seq * page_size < max_prefix_len) return BD_ERR_SHAPE;
  bd_status st = check_attn_shape(n_seq, blk_len, n_q_heads, n_kv_heads, head_dim, 1, dtype, softmax_scale);
  if (st != BD_OK) return st;
  if (dtype != BD_BF16) return BD_ERR_UNSUPPORTED;
  if ((long long)max_prefix_len + blk_len > kMaxGrid / 2) return BD_ERR_SHAPE;
  if (!aligned16(q_blk) || !aligned16(k_blk) || !aligned16(v_blk) || !aligned16(o) ||
      (k_pages && !aligned16(k_pages)) || (v_pages && !aligned16(v_pages)))
    return BD_ERR_ALIGNMENT;
  bd::DecodeShape s{n_seq, blk_len, max_prefix_len, n_q_heads, n_kv_heads, head_dim,
                    resolve_scale(softmax_scale, head_dim)};
  const size_t need = bd::decode_workspace_bytes(s, 1);
  if (!workspace || ws_bytes < need) return BD_ERR_WORKSPACE;
  if (!aligned16(workspace)) return BD_ERR_ALIGNMENT;
  return hip_status(bd::launch_decode_bf16_paged(q_blk, k_blk, v_blk, k_pages, v_pages, block_table,
                                                 max_pages_per_seq, page_size, prefix_len, o, lse, workspace, s,
                                                 stream));
}

bd_status bd_kv_append_block(const void* k_blk, const void* v_blk, void* k_pages, void* v_pages,
                             const int32_t* block_table, int max_pages_per_seq, int page_size, int32_t* prefix_len,
                             const int32_t* n_masked_left, int n_seq, int blk_len, int n_kv_heads, int head_dim,
                             bd_dtype dtype, hipStream_t stream) {
  if (!k_blk || !v_blk || !k_pages || !v_pages || !block_table || !prefix_len) return BD_ERR_NULL;
  if (n_seq <= 0 || blk_len <= 0 || n_kv_heads <= 0 || head_dim <= 0 || max_pages_per_seq <= 0) return BD_ERR_SHAPE;
  if (page_size <= 0) return BD_ERR_SHAPE;
  // a row's elements, and the block's 16-byte pieces, are counted in int
  if (exceeds(INT_MAX, {n_kv_heads, head_dim}) || exceeds(8LL * INT_MAX, {blk_len, n_kv_heads, head_dim}))
    return BD_ERR_SHAPE;
  if (dtype != BD_BF16) return BD_ERR_UNSUPPORTED;
  if ((n_kv_heads * head_dim) % 8 != 0) return BD_ERR_UNSUPPORTED;
  if (!aligned16(k_blk) || !aligned16(v_blk) || !aligned16(k_pages) || !aligned16(v_pages)) return BD_ERR_ALIGNMENT;
  return hip_status(bd::launch_kv_append_bf16(k_blk, v_blk, k_pages, v_pages, block_table, max_pages_per_seq,
                                              page_size, prefix_len, n_masked_left, n_seq, blk_len, n_kv_heads,
                                              head_dim, stream));
}

size_t bd_confidence_commit_workspace_size(int n_seq, int blk_len, int vocab) {
  if (!commit_rows_ok(n_seq, blk_len, vocab)) return 0;
  return bd::commit_workspace_bytes(n_seq, blk_len, vocab);
}

bd_status bd_confidence_commit(const void* logits, int64_t row_stride, int n_seq, int blk_len, int vocab,
                               bd_dtype dtype, float threshold, bd_fallback fallback, int32_t* tokens,
                               uint8_t* masked, float* conf, int32_t* pred, int32_t* n_committed,
                               int32_t* n_masked_left, void* workspace, size_t ws_bytes, hipStream_t stream) {
  return commit_common(logits, row_stride, n_seq, blk_len, vocab, dtype, threshold, nullptr, fallback, tokens,
                       masked, conf, pred, n_committed, n_masked_left, workspace, ws_bytes, stream);
}

bd_status bd_confidence_commit_noalloc(const void* logits, int64_t row_stride, int n_seq, int blk_len, int vocab,
                                       bd_dtype dtype, float threshold, bd_fallback fallback, int32_t* tokens,
                                       uint8_t* masked, float* conf, int32_t* pred, int32_t* n_committed,
                                       int32_t* n_masked_left, hipStream_t stream) {
  return commit_common(logits, row_stride, n_seq, blk_len, vocab, dtype, threshold, nullptr, fallback, tokens,
                       masked, conf, pred, n_committed, n_masked_left, nullptr, 0, stream, true);
}

bd_status bd_confidence_commit_rowwise(const void* logits, int64_t row_stride, int n_seq, int blk_len, int vocab,
                                       bd_dtype dtype, const float* thresholds, bd_fallback fallback,
                                       int32_t* tokens, uint8_t* masked, float* conf, int32_t* pred,
                                       int32_t* n_committed, int32_t* n_masked_left, void* workspace,
                                       size_t ws_bytes, hipStream_t stream) {
  if (!thresholds) return BD_ERR_NULL;
  return commit_common(logits, row_stride, n_seq, blk_len, vocab, dtype, 0.f, thresholds, fallback, tokens,
                       masked, conf, pred, n_committed, n_masked_left, workspace, ws_bytes, stream);
}

size_t bd_confidence_commit_sampled_workspace_size(int n_seq, int blk_len, int vocab) {
  if (!commit_rows_ok(n_seq, blk_len, vocab)) return 0;
  return bd::commit_sampled_workspace_bytes(n_seq, blk_len, vocab);
}

bd_status bd_confidence_commit_sampled(const void* logits, int64_t row_stride, int n_seq, int blk_len, int vocab,
                                       bd_dtype dtype, float temperature, uint64_t seed, uint64_t step, int top_k,
                                       float top_p, float threshold, bd_fallback fallback, int32_t* tokens,
                                       uint8_t* masked,
                                       float* conf, int32_t* pred, int32_t* n_committed, int32_t* n_masked_left,
                                       void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!logits || !tokens || !masked) return BD_ERR_NULL;
  if (n_seq <= 0 || blk_len <= 0 || vocab <= 0 || row_stride < vocab) return BD_ERR_SHAPE;
  if (blk_len > bd::kCommitMaxBlock) return BD_ERR_UNSUPPORTED;
  if (dtype != BD_F32 && dtype != BD_BF16) return BD_ERR_UNSUPPORTED;
  if (std::isnan(threshold)) return BD_ERR_VALUE;
  if (!(temperature > 0.f) || std::isinf(temperature)) return BD_ERR_VALUE;
  if (top_k < 0 || !(top_p > 0.f && top_p <= 1.f)) return BD_ERR_VALUE;
  if (fallback != BD_FALLBACK_NONE && fallback != BD_FALLBACK_TOP1) return BD_ERR_VALUE;
  const bool truncate = top_k > 0 || top_p < 1.f;
  if (truncate && vocab > bd::sample_truncated_max_vocab(dtype == BD_BF16)) return BD_ERR_UNSUPPORTED;
  if (!commit_rows_ok(n_seq, blk_len, vocab)) return BD_ERR_SHAPE;
  const size_t need = bd::commit_sampled_workspace_bytes(n_seq, blk_len, vocab);
  if (!workspace || ws_bytes < need) return BD_ERR_WORKSPACE;
  if (!aligned16(workspace)) return BD_ERR_ALIGNMENT;
  bd::CommitArgs a{logits, row_stride, n_seq, blk_len, vocab, dtype == BD_BF16, threshold, nullptr,
                   fallback == BD_FALLBACK_TOP1, tokens, masked, conf, pred, n_committed, n_masked_left, workspace};
  if (truncate)
    return hip_status(bd::launch_commit_sampled_truncated(a, temperature, seed, step, top_k, top_p, stream));
  return hip_status(bd::launch_commit_sampled(a, temperature, seed, step, stream));
}

size_t bd_lmhead_commit_workspace_size(int n_seq, int blk_len, int vocab) {
  if (n_seq <= 0 || blk_len <= 0 || vocab <= 0 || vocab > BD_MAX_VOCAB || blk_len > bd::kCommitMaxBlock) return 0;
  if ((long long)n_seq * blk_len > kMaxGrid / 256) return 0;
  return bd::lmhead_workspace_bytes(n_seq, blk_len);
}

bd_status bd_lmhead_commit(const void* hidden, int64_t hidden_stride, const void* weight, int64_t weight_stride,
                           int n_seq, int blk_len, int hidden_dim, int vocab, float threshold, bd_fallback fallback,
                           int32_t* tokens, uint8_t* masked, float* conf, int32_t* pred, int32_t* n_committed,
                           int32_t* n_masked_left, void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!hidden || !weight || !tokens || !masked) return BD_ERR_NULL;
  if (n_seq <= 0 || blk_len <= 0 || vocab <= 0 || vocab > BD_MAX_VOCAB || hidden_dim <= 0) return BD_ERR_SHAPE;
  if (hidden_stride < hidden_dim || weight_stride < hidden_dim) return BD_ERR_SHAPE;
  if (blk_len > bd::kCommitMaxBlock) return BD_ERR_UNSUPPORTED;
  if (hidden_dim % 64 != 0 || hidden_dim > bd::lmhead_max_hidden()) return BD_ERR_UNSUPPORTED;
  if (!aligned16(hidden) || !aligned16(weight) || hidden_stride % 8 != 0 || weight_stride % 8 != 0)
    return BD_ERR_ALIGNMENT;
  if (std::isnan(threshold)) return BD_ERR_VALUE;
  if (fallback != BD_FALLBACK_NONE && fallback != BD_FALLBACK_TOP1) return BD_ERR_VALUE;
  if ((long long)n_seq * blk_len > kMaxGrid / 256) return BD_ERR_SHAPE;
  const size_t need = bd::lmhead_workspace_bytes(n_seq, blk_len);
  if (!workspace || ws_bytes < need) return BD_ERR_WORKSPACE;
  if (!aligned16(workspace)) return BD_ERR_ALIGNMENT;
  bd::LmHeadArgs a;
  a.hidden = hidden;
  a.hidden_stride = hidden_stride;
  a.weight = weight;
  a.weight_stride = weight_stride;
  a.hidden_dim = hidden_dim;
  a.commit = bd::CommitArgs{nullptr, 0, n_seq, blk_len, vocab, 1, threshold, nullptr,
                            fallback == BD_FALLBACK_TOP1, tokens, masked, conf, pred, n_committed, n_masked_left,
                            workspace};
  return hip_status(bd::launch_lmhead_commit(a, stream));
}

}  // extern "C"
