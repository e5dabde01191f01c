/*
 * bd.h -- C ABI of the block-diffusion decoding hot path on MI355X (gfx950).
 *
 * The method (MinerU-Diffusion) decodes the output token sequence block by
 * block.  Inside a block of L' tokens every token attends to every other token
 * of the block; across blocks attention is causal: a token attends to all
 * earlier blocks and to no later block (paper.rainbus.top digest, method step
 * 3; hysenlabs.com editorial "The idea: OCR as inverse rendering"; OpenDataLab
 * blog, Fig. 2).  The earlier blocks are held as a KV cache (digest, novelty
 * paragraph).  After each denoising step every still-masked position whose
 * prediction confidence exceeds a threshold T is confirmed (digest, method
 * steps 4 and 6: T = 0.95, temperature 1, no top-k / top-p).
 *
 * Conventions shared by every entry point:
 *   - Every buffer argument is DEVICE memory owned by the caller.  The library
 *     never allocates or frees memory; scratch space is the caller's
 *     `workspace`, sized by the matching *_workspace_size() query, whose base
 *     must be 16-byte aligned (BD_ERR_ALIGNMENT otherwise; hipMalloc returns
 *     such addresses).
 *   - Tensors are dense and row-major with the innermost dimension last:
 *     q/o [batch, seqlen, n_q_heads, head_dim], k/v [batch, seqlen, n_kv_heads,
 *     head_dim] ("BSHD"); lse [batch, n_q_heads, seqlen] float32, natural log.
 *   - `dtype` selects the element type of q/k/v/o/dO/dq/dk/dv and logits:
 *     BD_F32 (float32) or BD_BF16 (bfloat16).  Accumulation is float32.
 *   - Grouped-query attention: query head h reads KV head h / (n_q_heads /
 *     n_kv_heads); n_q_heads must be a multiple of n_kv_heads.
 *   - softmax_scale <= 0 selects 1/sqrt(head_dim); a NaN scale is BD_ERR_VALUE.
 *   - bf16 tensors (and float32 logits) are read with 16-byte vector loads: their
 *     base pointers must be 16-byte aligned (BD_ERR_ALIGNMENT otherwise;
 *     logits fall back to scalar loads instead).
 *   - Calls are asynchronous: they validate the arguments, enqueue kernels on
 *     `stream` and return.  A non-BD_OK status means nothing was enqueued,
 *     except BD_ERR_HIP, which reports a failed launch (bd_last_hip_error()
 *     gives the hipError_t).  Faults inside a kernel surface at the caller's
 *     next synchronisation.
 *   - The library keeps no mutable global state except a thread-local last HIP
 *     error, values set once per process and never changed afterwards (kernel
 *     launch attributes, each device's compute-unit count; set under a lock or
 *     a once-flag) and, for bd_confidence_commit_noalloc only, a fixed device
 *     scratch array per GPU; calls on different streams may run concurrently as
 *     long as their output and workspace buffers do not overlap.
 */
#ifndef BD_H_
#define BD_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enumerations are int-sized.  In C++ their underlying type is fixed to
 * int, so that every int a caller passes (from C, or through a binding) is a
 * value the library may test and reject with a status. */
#ifdef __cplusplus
#define BD_INT_ENUM enum : int
#else
#define BD_INT_ENUM enum
#endif

typedef BD_INT_ENUM {
  BD_OK = 0,
  BD_ERR_NULL = 1,         /* a required pointer is NULL */
  BD_ERR_SHAPE = 2,        /* a size is non-positive or inconsistent */
  BD_ERR_UNSUPPORTED = 3,  /* dtype / head_dim combination not compiled in */
  BD_ERR_WORKSPACE = 4,    /* workspace NULL or smaller than the query returns */
  BD_ERR_VALUE = 5,        /* a scalar argument is out of its domain (e.g. NaN threshold) */
  BD_ERR_HIP = 6,          /* a HIP runtime call failed */
  BD_ERR_ALIGNMENT = 7,    /* a bf16 tensor or workspace pointer is not 16-byte aligned */
  BD_ERR_SCRATCH = 8       /* the problem needs more scratch than the fixed buffer of a
                              no-allocation entry point holds */
} bd_status;

typedef BD_INT_ENUM { BD_F32 = 0, BD_BF16 = 1 } bd_dtype;

/* What a block does when none of its masked tokens clears the threshold. */
typedef BD_INT_ENUM {
  BD_FALLBACK_NONE = 0,  /* commit nothing; the block stays as it is */
  BD_FALLBACK_TOP1 = 1   /* commit the single most confident masked token (lowest row on ties) */
} bd_fallback;

/* ------------------------------------------------------------------------
 * Block-causal attention over whole sequences (training / prefill).
 *
 * Query i may attend key j exactly when floor(j / block_size) <=
 * floor(i / block_size) (digest, method step 3).  seqlen need not be a
 * multiple of block_size: the last block is then short.
 *
 *   q  [batch, seqlen, n_q_heads, head_dim]   in
 *   k  [batch, seqlen, n_kv_heads, head_dim]  in
 *   v  [batch, seqlen, n_kv_heads, head_dim]  in
 *   o  [batch, seqlen, n_q_heads, head_dim]   out
 *   lse [batch, n_q_heads, seqlen] float32    out, may be NULL (natural-log
 *        log-sum-exp of the scaled scores of each row; bd_attn_bwd needs it)
 *
 * Supported: BD_BF16 with head_dim 128 (matrix-core path); BD_F32 with
 * head_dim <= 128 (vector path).
 * ---------------------------------------------------------------------- */
bd_status bd_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      int batch, int seqlen, int n_q_heads, int n_kv_heads, int head_dim,
                      int block_size, float softmax_scale, bd_dtype dtype, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Gradients of bd_attn_fwd for the loss sum(o * d_o) (the masked-token
 * training objective of the blog's Fig. 2 back-propagates through this).
 *
 *   q, k, v, o, lse   as produced / consumed by bd_attn_fwd (lse required)
 *   d_o [batch, seqlen, n_q_heads, head_dim]       in
 *   dq  [batch, seqlen, n_q_heads, head_dim]       out
 *   dk, dv [batch, seqlen, n_kv_heads, head_dim]   out (summed over the query
 *        heads of each group)
 *   workspace of bd_attn_bwd_workspace_size() bytes (bf16: two float32
 *        arrays [batch, n_q_heads, seqlen rounded up to 64] holding -D, with
 *        D = rowsum(d_o * o), and -lse / scale, then the counters that hand
 *        out work items to the compute units; fp32: D per row); contents on
 *        entry are ignored.
 *
 * Supported: as bd_attn_fwd.  Deterministic: every output element is summed
 * by one workgroup in one fixed order (the counters only decide which
 * workgroup computes which block of outputs), so repeated calls give
 * bit-identical results.
 * ---------------------------------------------------------------------- */
size_t bd_attn_bwd_workspace_size(int batch, int seqlen, int n_q_heads, int n_kv_heads, int head_dim);
bd_status bd_attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* d_o, void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes,
                      int batch, int seqlen, int n_q_heads, int n_kv_heads, int head_dim,
                      int block_size, float softmax_scale, bd_dtype dtype, hipStream_t stream);

/* ------------------------------------------------------------------------
 * One block per sequence against that sequence's KV-cache prefix (one
 * denoising step of decoding; digest, novelty paragraph on KV-cache reuse).
 *
 * The block is the newest block of its sequence, so each of its tokens sees
 * every prefix token and every token of the block: keys are
 * cache[prefix_start[s] .. prefix_start[s] + prefix_len[s]) followed by the
 * block's own k_blk/v_blk rows, all unmasked.
 *
 *   q_blk [n_seq, blk_len, n_q_heads, head_dim]     in
 *   k_blk, v_blk [n_seq, blk_len, n_kv_heads, head_dim]  in (the block's own
 *        keys and values, recomputed by the model at every step)
 *   k_cache, v_cache [total_rows, n_kv_heads, head_dim]  in (packed, ragged;
 *        may be NULL only if every prefix_len is 0)
 *   prefix_start int64[n_seq], prefix_len int32[n_seq]  in, DEVICE memory;
 *        prefix_len[s] must lie in [0, max_prefix_len]
 *   max_prefix_len  host value, an upper bound of prefix_len (sizes the grid;
 *        with this packed cache a larger prefix_len still gives the exact
 *        result, only the split of the work is then unbalanced)
 *   o [n_seq, blk_len, n_q_heads, head_dim]        out
 *   lse [n_seq, n_q_heads, blk_len] float32        out, may be NULL
 *   workspace of bd_attn_decode_workspace_size() bytes (split-KV partial
 *        softmax states); contents on entry are ignored.
 *
 * Supported: as bd_attn_fwd.
 * ---------------------------------------------------------------------- */
size_t bd_attn_decode_workspace_size(int n_seq, int blk_len, int max_prefix_len,
                                     int n_q_heads, int n_kv_heads, int head_dim);
bd_status bd_attn_decode_block(const void* q_blk, const void* k_blk, const void* v_blk,
                               const void* k_cache, const void* v_cache,
                               const int64_t* prefix_start, const int32_t* prefix_len, int max_prefix_len,
                               void* o, float* lse, int n_seq, int blk_len,
                               int n_q_heads, int n_kv_heads, int head_dim, float softmax_scale,
                               bd_dtype dtype, void* workspace, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * One block against a prefix cache held in pages (the cache layout of the
 * serving engines the pages name for the model, SGLang and the Nano-vLLM
 * adaptation: editorial, "The model, the weights and the serving stack").  The attention is exactly that of
 * bd_attn_decode_block; only where prefix row j of sequence s lives differs:
 *
 *   k_pages, v_pages [n_pages * page_size, n_kv_heads, head_dim] bf16: page p
 *        holds cache rows p*page_size .. p*page_size + page_size - 1;
 *   block_table int32[n_seq][max_pages_per_seq] (device): prefix row j of
 *        sequence s is row block_table[s][j / page_size] * page_size +
 *        j % page_size;
 *   page_size a multiple of 32 (BD_ERR_UNSUPPORTED otherwise);
 *   max_pages_per_seq * page_size >= max_prefix_len (BD_ERR_SHAPE otherwise).
 * bf16 only.  The workspace is that of bd_attn_decode_block
 * (bd_attn_decode_workspace_size).  Other arguments as bd_attn_decode_block.
 * ---------------------------------------------------------------------- */
bd_status bd_attn_decode_block_paged(const void* q_blk, const void* k_blk, const void* v_blk, const void* k_pages,
                                     const void* v_pages, const int32_t* block_table, int max_pages_per_seq,
                                     int page_size, const int32_t* prefix_len, int max_prefix_len, void* o,
                                     float* lse, int n_seq, int blk_len, int n_q_heads, int n_kv_heads, int head_dim,
                                     float softmax_scale, bd_dtype dtype, void* workspace, size_t ws_bytes,
                                     hipStream_t stream);

/* ------------------------------------------------------------------------
 * Append finished blocks to the paged cache (digest, novelty paragraph: the
 * block structure lets later blocks reuse the KV cache of earlier ones).  For
 * every sequence s with n_masked_left[s] == 0 (every sequence when
 * n_masked_left is NULL): rows t = 0 .. blk_len-1 of k_blk[s] / v_blk[s]
 * ([n_seq, blk_len, n_kv_heads, head_dim] bf16) are written to prefix rows
 * prefix_len[s] + t (addressed as in bd_attn_decode_block_paged), then
 * prefix_len[s] += blk_len (int32[n_seq], device, in/out).  The caller
 * allocates the pages first: a block whose rows would pass
 * max_pages_per_seq * page_size is left out (prefix_len unchanged).
 * page_size any positive value; bf16 only.
 * ---------------------------------------------------------------------- */
bd_status bd_kv_append_block(const void* k_blk, const void* v_blk, void* k_pages, void* v_pages,
                             const int32_t* block_table, int max_pages_per_seq, int page_size, int32_t* prefix_len,
                             const int32_t* n_masked_left, int n_seq, int blk_len, int n_kv_heads, int head_dim,
                             bd_dtype dtype, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Confidence-threshold commit (digest, method steps 4 and 6).
 *
 * logits [n_seq * blk_len rows, vocab], row r at logits + r * row_stride
 * elements (row_stride >= vocab).  Rows r = s * blk_len .. s * blk_len +
 * blk_len - 1 form the current block of sequence s.  vocab is at most
 * BD_MAX_VOCAB (BD_ERR_SHAPE beyond; the workspace query then returns 0).
 *
 * For each row with masked[r] != 0 on entry:
 *   pred[r] = lowest id v with logits[r][v] = max_v logits[r][v]
 *   conf[r] = 1 / sum_v exp(logits[r][v] - max)   (largest softmax probability
 *             at temperature 1 over the full vocabulary)
 *   A row holding NaN or +Inf, or only -Inf, gets conf = NaN and pred = -1.
 * Then per block s: the rows with conf > threshold (strict) are committed; if
 * there are none and fallback == BD_FALLBACK_TOP1, the masked row with the
 * largest non-NaN conf is committed (lowest row on ties).  Committing row r
 * sets tokens[r] = pred[r] and masked[r] = 0.
 *
 *   tokens int32[n_seq*blk_len], masked uint8[n_seq*blk_len]   in/out
 *   conf float32[n_seq*blk_len], pred int32[n_seq*blk_len]     out, may be
 *        NULL; written only for rows masked on entry
 *   n_committed, n_masked_left int32[n_seq]                    out, may be NULL
 *   workspace of bd_confidence_commit_workspace_size() bytes; contents on
 *        entry are ignored.
 * Rows with masked[r] == 0 on entry are neither read nor written.  A
 * threshold outside (0, 1) is legal (>= 1: fallback only; < 1/vocab: every
 * masked row commits); a NaN threshold is BD_ERR_VALUE.
 * ---------------------------------------------------------------------- */
#define BD_MAX_VOCAB (1 << 30)
size_t bd_confidence_commit_workspace_size(int n_seq, int blk_len, int vocab);
bd_status bd_confidence_commit(const void* logits, int64_t row_stride, int n_seq, int blk_len, int vocab,
                               bd_dtype dtype, float threshold, bd_fallback fallback,
                               int32_t* tokens, uint8_t* masked, float* conf, int32_t* pred,
                               int32_t* n_committed, int32_t* n_masked_left,
                               void* workspace, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * bd_confidence_commit without a workspace argument and without any memory
 * allocation, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Arguments, results and errors as bd_confidence_commit.  The per-chunk
 * partials that bd_confidence_commit keeps in the caller's workspace live here
 * in a file-scope device array of BD_NOALLOC_SCRATCH_BYTES bytes, one per GPU,
 * held from the library's load until the process ends.  A shape whose
 * bd_confidence_commit_workspace_size() exceeds it returns BD_ERR_SCRATCH
 * (nothing is enqueued); 4 MiB covers every shape of at most 262144 rows
 * (n_seq * blk_len), whatever the vocabulary.
 *
 * The array is not cleared between calls (each call writes every partial it
 * reads).  All calls on one GPU share its array: two calls that may overlap in
 * time on the same GPU (different streams, or different host threads without
 * ordering) race on it and must be serialised by the caller.  The calling
 * thread's current device must be the device of `stream`; the array's device
 * address is looked up (hipGetSymbolAddress) on the first call per device.
 * ---------------------------------------------------------------------- */
#define BD_NOALLOC_SCRATCH_BYTES (4u << 20)
bd_status bd_confidence_commit_noalloc(const void* logits, int64_t row_stride, int n_seq, int blk_len, int vocab,
                                       bd_dtype dtype, float threshold, bd_fallback fallback,
                                       int32_t* tokens, uint8_t* masked, float* conf, int32_t* pred,
                                       int32_t* n_committed, int32_t* n_masked_left, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Confidence commit with a threshold per position (digest, weaknesses,
 * point 2: the global threshold could give way to local ones that follow the
 * complexity of each region).
 *
 * As bd_confidence_commit, except that row r commits when
 * conf[r] > thresholds[r]:
 *   thresholds float32[n_seq*blk_len] (device), read for masked rows only;
 *        a NaN entry never passes (that row can still be a block's fallback).
 * The fallback rule is unchanged: a block none of whose masked rows passes
 * its own threshold commits its most confident masked row (BD_FALLBACK_TOP1).
 * thresholds == NULL is BD_ERR_NULL; the workspace is the same as for
 * bd_confidence_commit.
 * ---------------------------------------------------------------------- */
bd_status bd_confidence_commit_rowwise(const void* logits, int64_t row_stride, int n_seq, int blk_len, int vocab,
                                       bd_dtype dtype, const float* thresholds, bd_fallback fallback,
                                       int32_t* tokens, uint8_t* masked, float* conf, int32_t* pred,
                                       int32_t* n_committed, int32_t* n_masked_left, void* workspace,
                                       size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Confidence commit with sampled predictions.  The pages decode with
 * temperature 1.0, top-k 0 and top-p 1.0 (digest, method step 6): tokens drawn
 * from the full softmax with no truncation.  bd_confidence_commit takes the
 * argmax; this call samples:
 *
 *   p_v = softmax(logits[r] / temperature)_v over the ids that the truncation
 *         keeps (all of them for top_k = 0, top_p = 1, as on the pages);
 *   u   = (w + 1/2) / 2^32, w = word 0 of Philox4x32-10 (Salmon et al., SC
 *         2011) of counter (r, step mod 2^32, step >> 32, 0) under key
 *         (seed mod 2^32, seed >> 32);
 *   pred[r] = the first kept id v whose cumulative probability sum_{w<=v} p_w
 *         exceeds u (inverse-CDF sampling in id order);
 *   conf[r] = p_pred (renormalised over the kept ids).
 * Truncation, after the temperature: top_k >= 1 keeps the ids whose logit is
 * at least the top_k-th largest finite logit (ties kept together; 0 = off);
 * then top_p in (0, 1] keeps, of those, the ids down to the first logit value
 * (in decreasing order) at which their renormalised probability reaches top_p
 * (nucleus sampling, Holtzman et al., ICLR 2020; ties kept together; 1 = off).
 * Then the threshold rule, the fallback and the state update of
 * bd_confidence_commit.  Invalid rows as there (conf NaN, pred -1).
 *   temperature > 0 and finite, top_k >= 0, 0 < top_p <= 1 (BD_ERR_VALUE
 *   otherwise); a new `step` per denoising step gives fresh draws; the same
 *   (seed, step) repeats them.
 *   With truncation on, vocab is at most 155648 (bf16) or 77824 (fp32)
 *   (BD_ERR_UNSUPPORTED otherwise): one workgroup holds a row in registers.
 *   workspace of bd_confidence_commit_sampled_workspace_size() bytes;
 *   contents on entry are ignored.  Other arguments as bd_confidence_commit.
 * Without truncation the id is found by rescanning, for each masked row, only
 * the vocabulary chunk in which the running sum passes u (one extra read of
 * 1/k of the row for k chunks per row); with it, each row is read once.
 * ---------------------------------------------------------------------- */
size_t bd_confidence_commit_sampled_workspace_size(int n_seq, int blk_len, int vocab);
bd_status bd_confidence_commit_sampled(const void* logits, int64_t row_stride, int n_seq, int blk_len, int vocab,
                                       bd_dtype dtype, float temperature, uint64_t seed, uint64_t step, int top_k,
                                       float top_p, float threshold, bd_fallback fallback, int32_t* tokens,
                                       uint8_t* masked,
                                       float* conf, int32_t* pred, int32_t* n_committed, int32_t* n_masked_left,
                                       void* workspace, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Output projection fused with the confidence commit.  The commit acts on the
 * prediction of each masked position (digest, method step 4), the decoder's
 * distribution over the shared vocabulary (method step 1): the softmax of the
 * logits that the output projection makes from the last hidden states.  Here
 * the logits are never stored:
 *
 *   logits[r][v] = sum_k hidden[r][k] * weight[v][k]   (fp32 accumulation)
 *
 * and the rows then follow bd_confidence_commit exactly (conf, pred, the
 * threshold rule, the fallback, the state update), with conf and pred taken
 * from the fp32 logits.
 *
 *   hidden [n_seq*blk_len, hidden_dim] bf16, row r at hidden + r*hidden_stride
 *   weight [vocab, hidden_dim] bf16, row v at weight + v*weight_stride
 *        (both base pointers 16-byte aligned, strides multiples of 8 elements:
 *        BD_ERR_ALIGNMENT otherwise)
 *   hidden_dim a multiple of 64, at most 2048 (BD_ERR_UNSUPPORTED otherwise)
 *   threshold, fallback, tokens, masked, conf, pred, n_committed,
 *        n_masked_left: as bd_confidence_commit
 *   workspace of bd_lmhead_commit_workspace_size() bytes (per-row partial
 *        states); contents on entry are ignored.
 * Each group of 32 rows that holds a masked row reads the whole weight once
 * (one block of 32 rows: the weight is streamed from HBM once).
 * ---------------------------------------------------------------------- */
size_t bd_lmhead_commit_workspace_size(int n_seq, int blk_len, int vocab);
bd_status bd_lmhead_commit(const void* hidden, int64_t hidden_stride, const void* weight, int64_t weight_stride,
                           int n_seq, int blk_len, int hidden_dim, int vocab, float threshold, bd_fallback fallback,
                           int32_t* tokens, uint8_t* masked, float* conf, int32_t* pred, int32_t* n_committed,
                           int32_t* n_masked_left, void* workspace, size_t ws_bytes, hipStream_t stream);

/* Human-readable name of a status code (static storage; never NULL). */
const char* bd_status_string(bd_status s);

/* hipError_t of the most recent BD_ERR_HIP returned on the calling thread. */
int bd_last_hip_error(void);

/* Library version as major * 10000 + minor * 100 + patch. */
int bd_version(void);

#ifdef __cplusplus
}
#endif
#endif /* BD_H_ */
