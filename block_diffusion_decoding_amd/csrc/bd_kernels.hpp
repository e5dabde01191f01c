// Host-side launchers of the libbd kernels.  Arguments have been validated by
// the C-ABI layer (bd_api.cpp) before any of these is called.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace bd {

struct AttnShape {
  int batch, seqlen, n_q_heads, n_kv_heads, head_dim, block_size;
  float scale;  // resolved softmax scale (> 0)
};

// ---- full-sequence block-causal attention ---------------------------------
hipError_t launch_attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                                const AttnShape& s, hipStream_t st);
hipError_t launch_attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                               const AttnShape& s, hipStream_t st);

size_t attn_bwd_workspace_bytes(int batch, int seqlen, int n_q_heads);
hipError_t launch_attn_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                                const float* lse, const void* d_o, void* dq, void* dk, void* dv,
                                void* ws, const AttnShape& s, hipStream_t st);
hipError_t launch_attn_bwd_f32(const float* q, const float* k, const float* v, const float* o,
                               const float* lse, const float* d_o, float* dq, float* dk, float* dv,
                               void* ws, const AttnShape& s, hipStream_t st);

// ---- one block against a prefix KV cache -----------------------------------
struct DecodeShape {
  int n_seq, blk_len, max_prefix_len, n_q_heads, n_kv_heads, head_dim;
  float scale;
};
size_t decode_workspace_bytes(const DecodeShape& s, int is_bf16);
hipError_t launch_decode_bf16(const void* q_blk, const void* k_blk, const void* v_blk,
                              const void* k_cache, const void* v_cache, const int64_t* prefix_start,
                              const int32_t* prefix_len, void* o, float* lse, void* ws,
                              const DecodeShape& s, hipStream_t st);
// The same with the prefix in pages (page_size a multiple of 32).
hipError_t launch_decode_bf16_paged(const void* q_blk, const void* k_blk, const void* v_blk, const void* k_pages,
                                    const void* v_pages, const int32_t* block_table, int max_pages, int page_size,
                                    const int32_t* prefix_len, void* o, float* lse, void* ws, const DecodeShape& s,
                                    hipStream_t st);
hipError_t launch_kv_append_bf16(const void* k_blk, const void* v_blk, void* k_pages, void* v_pages,
                                 const int32_t* block_table, int max_pages, int page_size, int32_t* prefix_len,
                                 const int32_t* n_masked_left, int n_seq, int blk_len, int n_kv_heads, int head_dim,
                                 hipStream_t st);
hipError_t launch_decode_f32(const float* q_blk, const float* k_blk, const float* v_blk,
                             const float* k_cache, const float* v_cache, const int64_t* prefix_start,
                             const int32_t* prefix_len, float* o, float* lse, const DecodeShape& s,
                             hipStream_t st);

// ---- confidence-threshold commit -------------------------------------------
struct CommitArgs {
  const void* logits;
  int64_t row_stride;
  int n_seq, blk_len, vocab;
  int is_bf16;
  float threshold;
  const float* thresholds;   // per row (device), or null: `threshold` for every row
  int fallback_top1;
  int32_t* tokens;
  uint8_t* masked;
  float* conf;
  int32_t* pred;
  int32_t* n_committed;
  int32_t* n_masked_left;
  void* ws;
};
int commit_chunks_per_row(long long rows, int vocab);
size_t commit_workspace_bytes(int n_seq, int blk_len, int vocab);
hipError_t launch_commit(const CommitArgs& a, hipStream_t st);
// The same with the partials in the library's fixed device scratch array (a.ws is ignored);
// the caller has checked commit_workspace_bytes() <= kNoAllocScratchBytes.
constexpr size_t kNoAllocScratchBytes = (size_t)4 << 20;
hipError_t launch_commit_noalloc(const CommitArgs& a, hipStream_t st);
// Sampled predictions at `temperature` (Philox4x32-10 keyed by seed, row, step).
size_t commit_sampled_workspace_bytes(int n_seq, int blk_len, int vocab);
hipError_t launch_commit_sampled(const CommitArgs& a, float temperature, uint64_t seed, uint64_t step,
                                 hipStream_t st);
// Sampled predictions after top-k / top-p truncation (one workgroup per row, the
// row held in registers: vocab at most sample_truncated_max_vocab); the
// workspace holds the per-row confidence and id (rows * 8 bytes).
int sample_truncated_max_vocab(int is_bf16);
hipError_t launch_commit_sampled_truncated(const CommitArgs& a, float temperature, uint64_t seed, uint64_t step,
                                           int top_k, float top_p, hipStream_t st);
// The decide step alone, on nchunk partials per row at `part` ([row][chunk]).
hipError_t launch_commit_decide(const void* part, int nchunk, const CommitArgs& a, hipStream_t st);

constexpr int kCommitMaxBlock = 1024;  // largest blk_len the commit kernel takes

// ---- output projection fused with the confidence reduce ---------------------
struct LmHeadArgs {
  const void* hidden;   // [rows, hidden_dim] bf16
  int64_t hidden_stride;
  const void* weight;   // [vocab, hidden_dim] bf16
  int64_t weight_stride;
  int hidden_dim;
  CommitArgs commit;    // logits unused; vocab, state, outputs and workspace as for the commit
};
int lmhead_max_hidden();
size_t lmhead_workspace_bytes(int n_seq, int blk_len);
hipError_t launch_lmhead_commit(const LmHeadArgs& a, hipStream_t st);

}  // namespace bd
