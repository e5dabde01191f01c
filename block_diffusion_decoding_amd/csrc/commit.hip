// Confidence-threshold commit (MinerU-Diffusion "confidence dynamic scheduling":
// paper.rainbus.top digest, method steps 4 and 6).
//
// Two kernels on the caller's stream:
//   1. commit_reduce: one workgroup per (masked row, vocabulary chunk) streams
//      its chunk of logits from HBM once, with 16-byte coalesced loads, and
//      reduces it to (max, lowest argmax, sum exp(x - max), invalid flag).
//      Rows not masked on entry are skipped without touching their logits.
//   2. commit_decide: one workgroup per block merges the chunk partials of its
//      rows (associative merge: max, lowest id on ties, rescaled sums), forms
//      conf = 1 / sum, and applies the threshold / fallback rule.
// The HBM traffic is the logits of the masked rows plus a few bytes per row.
#include "bd_device.hpp"
#include "bd_kernels.hpp"

namespace bd {

namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 8192;  // vocabulary entries per workgroup and row

struct Partial {
  float m;    // max of the chunk (-inf if the chunk holds only -inf)
  float s;    // sum over the chunk of exp(x - m)
  int idx;    // lowest id reaching m
  int bad;    // chunk holds a NaN or +Inf
};

// Merge (m2, s2, i2) into (m, s, i).  Sums are kept relative to their max.
__device__ __forceinline__ void merge_state(float& m, float& s, int& idx, float m2, float s2, int i2) {
  if (m2 > m) {
    s = s * exp2_fast((m - m2) * kLog2e) + s2;
    m = m2;
    idx = i2;
  } else if (m2 == m) {
    s += s2;
    idx = min(idx, i2);
  } else {
    s += s2 * exp2_fast((m2 - m) * kLog2e);
  }
}

template <typename T> struct Vec;
template <> struct Vec<uint16_t> {
  static constexpr int N = 8;
  __device__ static void load(const uint16_t* p, float* x) {
    uint4 u = ldg16(p);
    x[0] = bf16_bits_to_f32(u.x & 0xffffu); x[1] = bf16_bits_to_f32(u.x >> 16);
    x[2] = bf16_bits_to_f32(u.y & 0xffffu); x[3] = bf16_bits_to_f32(u.y >> 16);
    x[4] = bf16_bits_to_f32(u.z & 0xffffu); x[5] = bf16_bits_to_f32(u.z >> 16);
    x[6] = bf16_bits_to_f32(u.w & 0xffffu); x[7] = bf16_bits_to_f32(u.w >> 16);
  }
  __device__ static float scalar(const uint16_t* p) { return bf16_bits_to_f32(*p); }
};
template <> struct Vec<float> {
  static constexpr int N = 4;
  __device__ static void load(const float* p, float* x) {
    float4 f = *reinterpret_cast<const float4*>(p);
    x[0] = f.x; x[1] = f.y; x[2] = f.z; x[3] = f.w;
  }
  __device__ static float scalar(const float* p) { return *p; }
};

// Fold VEC values starting at vocabulary id `base` into the running state.
template <int N>
__device__ __forceinline__ void fold(const float* x, int base, int valid, float& m, float& s, int& idx,
                                     int& bad) {
  float vmax = kNegInf;
  int vidx = 0x7fffffff;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    if (j < valid) {
      bad |= (x[j] != x[j]) | (x[j] == __builtin_huge_valf());
      if (x[j] > vmax) { vmax = x[j]; vidx = base + j; }
    }
  }
  if (vmax > m) {
    s *= exp2_fast((m - vmax) * kLog2e);
    m = vmax;
    idx = vidx;
  }
  if (m != kNegInf) {
    const float mb = m * kLog2e;
#pragma unroll
    for (int j = 0; j < N; ++j)
      if (j < valid) s += exp2_fast(__builtin_fmaf(x[j], kLog2e, -mb));
  }
}

template <typename T, bool kVector>
__global__ __launch_bounds__(kThreads) void commit_reduce(const T* __restrict__ logits, int64_t row_stride,
                                                          int vocab, int nchunk,
                                                          const uint8_t* __restrict__ masked,
                                                          Partial* __restrict__ part) {
  const int row = blockIdx.x / nchunk;
  const int chunk = blockIdx.x - row * nchunk;
  if (!masked[row]) return;
  const int tid = threadIdx.x;
  const T* base = logits + (int64_t)row * row_stride;
  const int c0 = chunk * kChunk;
  const int c1 = min(vocab, c0 + kChunk);

  float m = kNegInf, s = 0.f;
  int idx = 0x7fffffff, bad = 0;
  if (kVector) {
    constexpr int N = Vec<T>::N;
    constexpr int kIter = kChunk / (N * kThreads);
    float x[kIter][N];
    int pos[kIter];
#pragma unroll
    for (int it = 0; it < kIter; ++it) {
      pos[it] = c0 + (it * kThreads + tid) * N;
      if (pos[it] + N <= c1) Vec<T>::load(base + pos[it], x[it]);
    }
#pragma unroll
    for (int it = 0; it < kIter; ++it) {
      const int p = pos[it];
      if (p + N <= c1) {
        fold<N>(x[it], p, N, m, s, idx, bad);
      } else if (p < c1) {
        float t[N];
        const int valid = c1 - p;
#pragma unroll
        for (int j = 0; j < N; ++j) t[j] = (j < valid) ? Vec<T>::scalar(base + p + j) : 0.f;
        fold<N>(t, p, valid, m, s, idx, bad);
      }
    }
  } else {
    for (int p = c0 + tid; p < c1; p += kThreads) {
      float t = Vec<T>::scalar(base + p);
      fold<1>(&t, p, 1, m, s, idx, bad);
    }
  }

  // wave reduction
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    float m2 = __shfl_xor(m, off, 64), s2 = __shfl_xor(s, off, 64);
    int i2 = __shfl_xor(idx, off, 64), b2 = __shfl_xor(bad, off, 64);
    merge_state(m, s, idx, m2, s2, i2);
    bad |= b2;
  }
  __shared__ Partial red[kThreads / 64];
  const int wave = tid >> 6;
  if ((tid & 63) == 0) red[wave] = Partial{m, s, idx, bad};
  __syncthreads();
  if (tid == 0) {
    Partial r = red[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) {
      merge_state(r.m, r.s, r.idx, red[w].m, red[w].s, red[w].idx);
      r.bad |= red[w].bad;
    }
    part[(int64_t)row * nchunk + chunk] = r;
  }
}

__global__ __launch_bounds__(kThreads) void commit_decide(const Partial* __restrict__ part, int nchunk,
                                                          int blk_len, float threshold, int fallback_top1,
                                                          int32_t* __restrict__ tokens,
                                                          uint8_t* __restrict__ masked,
                                                          float* __restrict__ conf_out,
                                                          int32_t* __restrict__ pred_out,
                                                          int32_t* __restrict__ n_committed,
                                                          int32_t* __restrict__ n_left) {
  __shared__ float s_conf[kCommitMaxBlock];
  __shared__ int s_pred[kCommitMaxBlock];
  __shared__ float s_best_c[kThreads / 64];
  __shared__ int s_best_r[kThreads / 64];
  const int g = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t row0 = (int64_t)g * blk_len;

  int above = 0;
  float best_c = kNegInf;
  int best_r = 0x7fffffff;
  for (int r = tid; r < blk_len; r += kThreads) {
    const int64_t row = row0 + r;
    float c = __builtin_nanf("");
    int p = -2;  // -2: not masked on entry
    if (masked[row]) {
      const Partial* pp = part + row * nchunk;
      float m = pp[0].m, s = pp[0].s;
      int idx = pp[0].idx, bad = pp[0].bad;
      for (int k = 1; k < nchunk; ++k) {
        merge_state(m, s, idx, pp[k].m, pp[k].s, pp[k].idx);
        bad |= pp[k].bad;
      }
      const bool invalid = bad || (m == kNegInf);
      c = invalid ? __builtin_nanf("") : 1.0f / s;
      p = invalid ? -1 : idx;
      if (conf_out) conf_out[row] = c;
      if (pred_out) pred_out[row] = p;
      above |= (c > threshold);
      if (!invalid && (c > best_c || (c == best_c && r < best_r))) { best_c = c; best_r = r; }
    }
    s_conf[r] = c;
    s_pred[r] = p;
  }
  const int any_above = __syncthreads_or(above);

  int chosen_row = -1;
  if (!any_above && fallback_top1) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      float c2 = __shfl_xor(best_c, off, 64);
      int r2 = __shfl_xor(best_r, off, 64);
      if (c2 > best_c || (c2 == best_c && r2 < best_r)) { best_c = c2; best_r = r2; }
    }
    if ((tid & 63) == 0) { s_best_c[tid >> 6] = best_c; s_best_r[tid >> 6] = best_r; }
    __syncthreads();
    float bc = s_best_c[0];
    int br = s_best_r[0];
    for (int w = 1; w < kThreads / 64; ++w) {
      if (s_best_c[w] > bc || (s_best_c[w] == bc && s_best_r[w] < br)) { bc = s_best_c[w]; br = s_best_r[w]; }
    }
    chosen_row = (br < blk_len) ? br : -1;
  }

  int committed = 0, left = 0;
  for (int r = tid; r < blk_len; r += kThreads) {
    const int p = s_pred[r];
    if (p == -2) continue;
    const float c = s_conf[r];
    const bool take = any_above ? (c > threshold) : (r == chosen_row);
    if (take) {
      tokens[row0 + r] = p;
      masked[row0 + r] = 0;
      ++committed;
    } else {
      ++left;
    }
  }
  __shared__ int s_cnt[2];
  if (tid == 0) { s_cnt[0] = 0; s_cnt[1] = 0; }
  __syncthreads();
  if (committed) atomicAdd(&s_cnt[0], committed);
  if (left) atomicAdd(&s_cnt[1], left);
  __syncthreads();
  if (tid == 0) {
    if (n_committed) n_committed[g] = s_cnt[0];
    if (n_left) n_left[g] = s_cnt[1];
  }
}

}  // namespace

int commit_chunks_per_row(int vocab, int /*is_bf16*/) { return (vocab + kChunk - 1) / kChunk; }

size_t commit_workspace_bytes(int n_seq, int blk_len, int vocab, int is_bf16) {
  return (size_t)n_seq * blk_len * commit_chunks_per_row(vocab, is_bf16) * sizeof(Partial);
}

hipError_t launch_commit(const CommitArgs& a, hipStream_t st) {
  const int nchunk = commit_chunks_per_row(a.vocab, a.is_bf16);
  const int64_t rows = (int64_t)a.n_seq * a.blk_len;
  Partial* part = reinterpret_cast<Partial*>(a.ws);
  const int elem = a.is_bf16 ? 2 : 4;
  const bool vec = ((uintptr_t)a.logits % 16 == 0) && ((a.row_stride * elem) % 16 == 0);
  dim3 grid((unsigned)(rows * nchunk));
  if (a.is_bf16) {
    const uint16_t* lg = reinterpret_cast<const uint16_t*>(a.logits);
    if (vec) hipLaunchKernelGGL((commit_reduce<uint16_t, true>), grid, dim3(kThreads), 0, st, lg, a.row_stride, a.vocab, nchunk, a.masked, part);
    else hipLaunchKernelGGL((commit_reduce<uint16_t, false>), grid, dim3(kThreads), 0, st, lg, a.row_stride, a.vocab, nchunk, a.masked, part);
  } else {
    const float* lg = reinterpret_cast<const float*>(a.logits);
    if (vec) hipLaunchKernelGGL((commit_reduce<float, true>), grid, dim3(kThreads), 0, st, lg, a.row_stride, a.vocab, nchunk, a.masked, part);
    else hipLaunchKernelGGL((commit_reduce<float, false>), grid, dim3(kThreads), 0, st, lg, a.row_stride, a.vocab, nchunk, a.masked, part);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(commit_decide, dim3(a.n_seq), dim3(kThreads), 0, st, part, nchunk, a.blk_len, a.threshold,
                     a.fallback_top1, a.tokens, a.masked, a.conf, a.pred, a.n_committed, a.n_masked_left);
  return hipGetLastError();
}

}  // namespace bd
