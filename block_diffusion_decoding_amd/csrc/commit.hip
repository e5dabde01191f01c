// Confidence-threshold commit (MinerU-Diffusion "confidence dynamic scheduling":
// paper.rainbus.top digest, method steps 4 and 6).
//
// Two kernels on the caller's stream:
//   1. commit_reduce: one workgroup per (masked row, vocabulary chunk) streams
//      its chunk of logits from HBM once (16-byte non-temporal loads, 64
//      bytes per thread in flight ahead of the arithmetic) and reduces it to
//      (max, lowest argmax, sum exp(x - max), invalid flag).  Rows not masked on entry are
//      skipped without touching their logits.  The chunk count per row is
//      chosen so that about 8192 workgroups are launched: several per row even
//      when many rows are decoded together, so that the few rows still masked
//      late in a decode loop still spread over the whole chip, and many per
//      row for a single block.
//   2. commit_decide: one workgroup per block merges the chunk partials of its
//      rows (associative merge: max, lowest id on ties, rescaled sums; eight
//      threads per row), forms conf = 1 / sum, and applies the threshold
//      (one for every row, or one per row) and the fallback rule.
// The HBM traffic is the logits of the masked rows plus a few bytes per row.
#include "bd_device.hpp"
#include "bd_kernels.hpp"
#include "commit_common.hpp"

#include <algorithm>

#ifndef BD_COMMIT_TARGET_WGS
#define BD_COMMIT_TARGET_WGS 8192
#endif

namespace bd {

namespace {

constexpr int kThreads = 256;
constexpr int kStep = 2048;          // vocabulary entries per workgroup and load step (bf16)
constexpr int kTargetWGs = BD_COMMIT_TARGET_WGS;   // workgroups the chunking aims for
constexpr int kMinChunk = 4096;      // fewest vocabulary entries per chunk
constexpr int kDecideLanes = 8;      // threads merging one row's partials
constexpr int kMergeBatch = 8;       // partial loads in flight per merging thread

template <typename T> struct Vec;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
template <> struct Vec<uint16_t> {
  static constexpr int N = 8;
  typedef u32x4 Raw;
  __device__ static Raw load(const uint16_t* p) { return __builtin_nontemporal_load(reinterpret_cast<const Raw*>(p)); }
  __device__ static void unpack(const Raw& u, float* x) {
    x[0] = __uint_as_float(u.x << 16); x[1] = __uint_as_float(u.x & 0xffff0000u);
    x[2] = __uint_as_float(u.y << 16); x[3] = __uint_as_float(u.y & 0xffff0000u);
    x[4] = __uint_as_float(u.z << 16); x[5] = __uint_as_float(u.z & 0xffff0000u);
    x[6] = __uint_as_float(u.w << 16); x[7] = __uint_as_float(u.w & 0xffff0000u);
  }
  __device__ static float scalar(const uint16_t* p) { return bf16_bits_to_f32(*p); }
};
template <> struct Vec<float> {
  static constexpr int N = 4;
  typedef f32x4 Raw;
  __device__ static Raw load(const float* p) { return __builtin_nontemporal_load(reinterpret_cast<const Raw*>(p)); }
  __device__ static void unpack(const Raw& f, float* x) { x[0] = f.x; x[1] = f.y; x[2] = f.z; x[3] = f.w; }
  __device__ static float scalar(const float* p) { return *p; }
};

template <typename T, bool kVector>
__global__ __launch_bounds__(kThreads) void commit_reduce(const T* __restrict__ logits, int64_t row_stride,
                                                          int vocab, int nchunk, int chunk_len,
                                                          const uint8_t* __restrict__ masked,
                                                          Partial* __restrict__ part) {
  const int row = blockIdx.x / nchunk;
  const int chunk = blockIdx.x - row * nchunk;
  if (!masked[row]) return;
  const int tid = threadIdx.x;
  const T* base = logits + (int64_t)row * row_stride;
  const int c0 = chunk * chunk_len;
  const int c1 = min(vocab, c0 + chunk_len);

  RowState st;
  if (kVector) {
    constexpr int N = Vec<T>::N;
    constexpr int kA = 32 / N;   // rounds of loads in flight (64 bytes per thread)
    typedef typename Vec<T>::Raw Raw;
    const int full = c0 + ((c1 - c0) / (N * kThreads)) * (N * kThreads);   // end of whole vector rounds
    const int nv = (full - c0) / (N * kThreads);                          // vector rounds in the chunk
    const T* p = base + c0 + tid * N;
    auto at = [&](int v) __attribute__((always_inline)) { return p + v * kThreads * N; };
    auto fold = [&](const Raw& r, int v) __attribute__((always_inline)) {
      float x[N];
      Vec<T>::unpack(r, x);
      fold_vec<N>(x, c0 + (v * kThreads + tid) * N, st);
    };
    Raw buf[kA];
    if (nv >= 2 * kA) {
      // Unconditional loads up to the end of the loop, so that the wait
      // before each fold covers only the load it needs.
#pragma unroll
      for (int u = 0; u < kA; ++u) buf[u] = Vec<T>::load(at(u));
      int v0 = 0;
      for (; v0 + 2 * kA <= nv; v0 += kA) {
#pragma unroll
        for (int u = 0; u < kA; ++u) {
          fold(buf[u], v0 + u);
          buf[u] = Vec<T>::load(at(v0 + u + kA));
        }
      }
      // kA <= nv - v0 < 2 kA rounds left; buf holds rounds v0 .. v0 + kA - 1
#pragma unroll
      for (int u = 0; u < kA; ++u) {
        fold(buf[u], v0 + u);
        if (v0 + u + kA < nv) buf[u] = Vec<T>::load(at(v0 + u + kA));
      }
#pragma unroll
      for (int u = 0; u < kA; ++u)
        if (v0 + kA + u < nv) fold(buf[u], v0 + kA + u);
    } else {
      // a short chunk: at most two batches of kA rounds
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int u = 0; u < kA; ++u)
          if (h * kA + u < nv) buf[u] = Vec<T>::load(at(h * kA + u));
#pragma unroll
        for (int u = 0; u < kA; ++u)
          if (h * kA + u < nv) fold(buf[u], h * kA + u);
      }
    }
    for (int q = full + tid; q < c1; q += kThreads) fold_one(Vec<T>::scalar(base + q), q, st);
  } else {
    for (int q = c0 + tid; q < c1; q += kThreads) fold_one(Vec<T>::scalar(base + q), q, st);
  }
  st.bad |= (st.s != st.s) | (st.m == __builtin_huge_valf());

  // wave reduction
  float m = st.m, s = st.s;
  int idx = st.idx, bad = st.bad;
  if (m == kNegInf) s = 0.f;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    float m2 = __shfl_xor(m, off, 64), s2 = __shfl_xor(s, off, 64);
    int i2 = __shfl_xor(idx, off, 64), b2 = __shfl_xor(bad, off, 64);
    if (!bad && !b2) merge_state(m, s, idx, m2, s2, i2);
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
      if (!r.bad && !red[w].bad) merge_state(r.m, r.s, r.idx, red[w].m, red[w].s, red[w].idx);
      r.bad |= red[w].bad;
    }
    part[(int64_t)row * nchunk + chunk] = r;
  }
}

// kLanes threads per row merge its partials; kThr threads per workgroup.
template <int kLanes, int kThr>
__global__ __launch_bounds__(kThr) void commit_decide(const Partial* __restrict__ part, int nchunk,
                                                          int blk_len, float threshold,
                                                          const float* __restrict__ thr_rows, int fallback_top1,
                                                          int32_t* __restrict__ tokens,
                                                          uint8_t* __restrict__ masked,
                                                          float* __restrict__ conf_out,
                                                          int32_t* __restrict__ pred_out,
                                                          int32_t* __restrict__ n_committed,
                                                          int32_t* __restrict__ n_left) {
  __shared__ float s_conf[kCommitMaxBlock];
  __shared__ int s_pred[kCommitMaxBlock];
  __shared__ unsigned char s_pass[kCommitMaxBlock];
  __shared__ float s_best_c[kThr / 64];
  __shared__ int s_best_r[kThr / 64];
  const int g = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t row0 = (int64_t)g * blk_len;

  // kLanes threads per row merge its chunk partials (strided), then
  // combine across the group; the group's first thread finishes the row.
  int above = 0;
  float best_c = kNegInf;
  int best_r = 0x7fffffff;
  const int sub = tid % kLanes;
  for (int r0 = 0; r0 < blk_len; r0 += kThr / kLanes) {
    const int r = r0 + tid / kLanes;
    const bool in = r < blk_len;
    const int64_t row = row0 + (in ? r : 0);
    const bool msk = in && masked[row];
    float m = kNegInf, s = 0.f;
    int idx = 0x7fffffff, bad = 0;
    if (msk) {
      // partials in batches of kMergeBatch loads per round trip to memory
      const Partial* pp = part + row * nchunk;
      for (int kb = sub; kb < nchunk; kb += kMergeBatch * kLanes) {
        Partial q[kMergeBatch];
#pragma unroll
        for (int i = 0; i < kMergeBatch; ++i)
          if (kb + i * kLanes < nchunk) q[i] = pp[kb + i * kLanes];
#pragma unroll
        for (int i = 0; i < kMergeBatch; ++i)
          if (kb + i * kLanes < nchunk) {
            if (!bad && !q[i].bad) merge_state(m, s, idx, q[i].m, q[i].s, q[i].idx);
            bad |= q[i].bad;
          }
      }
    }
#pragma unroll
    for (int off = 1; off < kLanes; off <<= 1) {
      float m2 = __shfl_xor(m, off, 64), s2 = __shfl_xor(s, off, 64);
      int i2 = __shfl_xor(idx, off, 64), b2 = __shfl_xor(bad, off, 64);
      if (!bad && !b2) merge_state(m, s, idx, m2, s2, i2);
      bad |= b2;
    }
    if (in && sub == 0) {
      float c = __builtin_nanf("");
      int pr = -2;  // -2: not masked on entry
      if (msk) {
        const bool invalid = bad || (m == kNegInf);
        c = invalid ? __builtin_nanf("") : 1.0f / s;
        pr = invalid ? -1 : idx;
        if (conf_out) conf_out[row] = c;
        if (pred_out) pred_out[row] = pr;
        const bool pass = c > (thr_rows ? thr_rows[row] : threshold);   // false for a NaN threshold
        above |= pass;
        s_pass[r] = pass;
        if (!invalid && (c > best_c || (c == best_c && r < best_r))) { best_c = c; best_r = r; }
      }
      s_conf[r] = c;
      s_pred[r] = pr;
    }
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
    for (int w = 1; w < kThr / 64; ++w) {
      if (s_best_c[w] > bc || (s_best_c[w] == bc && s_best_r[w] < br)) { bc = s_best_c[w]; br = s_best_r[w]; }
    }
    chosen_row = (br < blk_len) ? br : -1;
  }

  int committed = 0, left = 0;
  for (int r = tid; r < blk_len; r += kThr) {
    const int p = s_pred[r];
    if (p == -2) continue;
    const float c = s_conf[r];
    const bool take = any_above ? (s_pass[r] != 0) : (r == chosen_row);
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

// Vocabulary entries per chunk for rows x vocab logits: about kTargetWGs
// workgroups in all, chunks of at least kMinChunk entries, a multiple of
// kStep (so that every chunk but a row's last starts and ends on whole steps).
int commit_chunk_len(long long rows, int vocab) {
  const long long want = std::max<long long>(1, (kTargetWGs + rows - 1) / rows);
  const long long most = std::max<long long>(1, (vocab + kMinChunk - 1) / kMinChunk);
  const long long nchunk = std::min(want, most);
  const long long len = (vocab + nchunk - 1) / nchunk;
  return (int)(((len + kStep - 1) / kStep) * kStep);
}

}  // namespace

int commit_chunks_per_row(long long rows, int vocab) {
  const int len = commit_chunk_len(rows, vocab);
  return (vocab + len - 1) / len;
}

size_t commit_workspace_bytes(int n_seq, int blk_len, int vocab) {
  const long long rows = (long long)n_seq * blk_len;
  return (size_t)rows * commit_chunks_per_row(rows, vocab) * sizeof(Partial);
}

hipError_t launch_commit(const CommitArgs& a, hipStream_t st) {
  const int64_t rows = (int64_t)a.n_seq * a.blk_len;
  const int chunk_len = commit_chunk_len(rows, a.vocab);
  const int nchunk = (a.vocab + chunk_len - 1) / chunk_len;
  Partial* part = reinterpret_cast<Partial*>(a.ws);
  const int elem = a.is_bf16 ? 2 : 4;
  const bool vec = ((uintptr_t)a.logits % 16 == 0) && ((a.row_stride * elem) % 16 == 0);
  dim3 grid((unsigned)(rows * nchunk));
  if (a.is_bf16) {
    const uint16_t* lg = reinterpret_cast<const uint16_t*>(a.logits);
    if (vec) hipLaunchKernelGGL((commit_reduce<uint16_t, true>), grid, dim3(kThreads), 0, st, lg, a.row_stride, a.vocab, nchunk, chunk_len, a.masked, part);
    else hipLaunchKernelGGL((commit_reduce<uint16_t, false>), grid, dim3(kThreads), 0, st, lg, a.row_stride, a.vocab, nchunk, chunk_len, a.masked, part);
  } else {
    const float* lg = reinterpret_cast<const float*>(a.logits);
    if (vec) hipLaunchKernelGGL((commit_reduce<float, true>), grid, dim3(kThreads), 0, st, lg, a.row_stride, a.vocab, nchunk, chunk_len, a.masked, part);
    else hipLaunchKernelGGL((commit_reduce<float, false>), grid, dim3(kThreads), 0, st, lg, a.row_stride, a.vocab, nchunk, chunk_len, a.masked, part);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_commit_decide(part, nchunk, a, st);
}

hipError_t launch_commit_decide(const void* part, int nchunk, const CommitArgs& a, hipStream_t st) {
  // Rows with many partials (the fused projection: one per workgroup) get 32 threads each.
  const Partial* pp = reinterpret_cast<const Partial*>(part);
  if (nchunk >= 64)
    hipLaunchKernelGGL((commit_decide<32, 1024>), dim3(a.n_seq), dim3(1024), 0, st, pp, nchunk, a.blk_len,
                       a.threshold, a.thresholds, a.fallback_top1, a.tokens, a.masked, a.conf, a.pred,
                       a.n_committed, a.n_masked_left);
  else
    hipLaunchKernelGGL((commit_decide<kDecideLanes, kThreads>), dim3(a.n_seq), dim3(kThreads), 0, st, pp, nchunk,
                       a.blk_len, a.threshold, a.thresholds, a.fallback_top1, a.tokens, a.masked, a.conf, a.pred,
                       a.n_committed, a.n_masked_left);
  return hipGetLastError();
}

}  // namespace bd
