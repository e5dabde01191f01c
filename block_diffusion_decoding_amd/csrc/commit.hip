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
#include <mutex>
#include <utility>

#ifndef BD_COMMIT_TARGET_WGS
#define BD_COMMIT_TARGET_WGS 8192
#endif
#ifndef BD_SAMPLE_CHUNK_MULT
#define BD_SAMPLE_CHUNK_MULT 4
#endif

namespace bd {

namespace {

constexpr int kThreads = 256;
constexpr int kStep = 2048;          // vocabulary entries per workgroup and load step (bf16)
constexpr int kTargetWGs = BD_COMMIT_TARGET_WGS;   // workgroups the chunking aims for
// Sampling rescans one chunk per row: finer chunks keep that rescan short.
constexpr int kSampleTargetWGs = BD_SAMPLE_CHUNK_MULT * BD_COMMIT_TARGET_WGS;
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
                                                          Partial* __restrict__ part, float c) {
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
      fold_vec<N>(x, c0 + (v * kThreads + tid) * N, st, c);
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
    for (int q = full + tid; q < c1; q += kThreads) fold_one(Vec<T>::scalar(base + q), q, st, c);
  } else {
    for (int q = c0 + tid; q < c1; q += kThreads) fold_one(Vec<T>::scalar(base + q), q, st, c);
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
    if (!bad && !b2) merge_state(m, s, idx, m2, s2, i2, c);
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
      if (!r.bad && !red[w].bad) merge_state(r.m, r.s, r.idx, red[w].m, red[w].s, red[w].idx, c);
      r.bad |= red[w].bad;
    }
    part[(int64_t)row * nchunk + chunk] = r;
  }
}

// kLanes threads per row merge its partials; kThr threads per workgroup.
// With row_conf / row_pred set, each masked row's (conf, id) is taken from
// them (a prediction made elsewhere, e.g. sampled) and no partial is read.
template <int kLanes, int kThr>
__global__ __launch_bounds__(kThr) void commit_decide(const Partial* __restrict__ part, int nchunk,
                                                          const float* __restrict__ row_conf,
                                                          const int32_t* __restrict__ row_pred,
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
    if (msk && !row_conf) {
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
        bool invalid;
        if (row_conf) {
          pr = row_pred[row];
          invalid = pr < 0;
          c = invalid ? __builtin_nanf("") : row_conf[row];
        } else {
          invalid = bad || (m == kNegInf);
          c = invalid ? __builtin_nanf("") : 1.0f / s;
          pr = invalid ? -1 : idx;
        }
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
// Computed in 64 bits: for vocabularies up to 2^30 the length fits an int.
int commit_chunk_len(long long rows, int vocab, long long target_wgs = kTargetWGs) {
  const long long v = vocab;
  const long long want = std::max<long long>(1, (target_wgs + rows - 1) / rows);
  const long long most = std::max<long long>(1, (v + kMinChunk - 1) / kMinChunk);
  const long long nchunk = std::min(want, most);
  const long long len = (v + nchunk - 1) / nchunk;
  return (int)(((len + kStep - 1) / kStep) * kStep);
}

// ---- sampled predictions ----------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
// as 1, 2, 3", SC 2011): ten rounds of the two 32 x 32 -> 64-bit products of
// counter words 0 and 2, the key bumped by the Weyl constants between rounds;
// word 0 of the output block.
__device__ __forceinline__ uint32_t philox_word0(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                                 uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
    const uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return c0;
}

// One workgroup per masked row: merge the row's chunk partials (max M, sum S of
// 2^((x - M) c)), draw u for (seed, row, step), find the chunk in which the
// running sum (chunks in id order) passes u S, rescan that chunk in id order
// (each thread a contiguous slice, a workgroup scan of the slice sums) and take
// the first id whose running sum passes u S.  conf = 2^((x_id - M) c) / S.
template <typename T, bool kVector>
__global__ __launch_bounds__(kThreads) void sample_locate(const T* __restrict__ logits, int64_t row_stride,
                                                          int vocab, int nchunk, int chunk_len,
                                                          const uint8_t* __restrict__ masked,
                                                          const Partial* __restrict__ part, float c, uint32_t seed_lo,
                                                          uint32_t seed_hi, uint32_t step_lo, uint32_t step_hi,
                                                          float* __restrict__ row_conf,
                                                          int32_t* __restrict__ row_pred) {
  constexpr int N = Vec<T>::N;
  const int row = blockIdx.x;
  if (!masked[row]) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float s_M, s_S, s_res;
  __shared__ int s_chunk, s_ok;
  __shared__ float s_wsum[kThreads / 64];
  __shared__ int s_found, s_last, s_idx;

  if (wave == 0) {
    // total over the chunks, then the chunk holding the target (chunks of 64 at a time)
    Partial tot{kNegInf, 0.f, 0x7fffffff, 0};
    for (int k0 = 0; k0 < nchunk; k0 += 64) {
      Partial q{kNegInf, 0.f, 0x7fffffff, 0};
      if (k0 + lane < nchunk) q = part[(int64_t)row * nchunk + k0 + lane];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        Partial o{__shfl_xor(q.m, off, 64), __shfl_xor(q.s, off, 64), __shfl_xor(q.idx, off, 64),
                  __shfl_xor(q.bad, off, 64)};
        merge_partial(q, o, c);
      }
      merge_partial(tot, q, c);
    }
    const bool ok = !tot.bad && tot.m != kNegInf;
    // the last chunk holding a finite value (a target past the end, from rounding, takes its last id)
    int last_chunk = 0;
    for (int k0 = 0; k0 < nchunk; k0 += 64) {
      const bool fin = k0 + lane < nchunk && part[(int64_t)row * nchunk + k0 + lane].m != kNegInf;
      const unsigned long long b = __builtin_amdgcn_ballot_w64(fin);
      if (b) last_chunk = k0 + 63 - __builtin_clzll(b);
    }
    const uint32_t w = philox_word0((uint32_t)row, step_lo, step_hi, 0u, seed_lo, seed_hi);
    const float u = (float)(((double)w + 0.5) * (1.0 / 4294967296.0));
    const float target = u * tot.s;
    int chunk = last_chunk;
    float before = 0.f;
    bool found = false;
    if (ok) {
      for (int k0 = 0; k0 < nchunk && !found; k0 += 64) {
        float v = 0.f;
        if (k0 + lane < nchunk) {
          const Partial q = part[(int64_t)row * nchunk + k0 + lane];
          v = q.m == kNegInf ? 0.f : q.s * exp2_fast((q.m - tot.m) * c);
        }
        float incl = v;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const float y = __shfl_up(incl, off, 64);
          if (lane >= off) incl += y;
        }
        const unsigned long long hit = __builtin_amdgcn_ballot_w64(k0 + lane < nchunk && before + incl > target);
        if (hit) {
          // the chunks before the crossing one sum to lane l-1's inclusive value, the
          // very sum the crossing test found not to pass the target: target - before >= 0
          const int l = __builtin_ctzll(hit);
          chunk = k0 + l;
          const float excl = __shfl(incl, l > 0 ? l - 1 : 0, 64);
          if (l > 0) before += excl;
          found = true;
        } else {
          before += __shfl(incl, 63, 64);
        }
      }
    }
    if (lane == 0) {
      s_ok = ok;
      s_M = tot.m;
      s_S = tot.s;
      s_chunk = chunk;
      s_res = found ? target - before : 3.4e38f;   // past the end: the last id of positive weight
      s_found = 0x7fffffff;
      s_last = -1;
      s_idx = tot.idx;
    }
  }
  __syncthreads();
  if (!s_ok) {
    if (tid == 0) {
      row_conf[row] = __builtin_nanf("");
      row_pred[row] = -1;
    }
    return;
  }
  const float M = s_M, res = s_res, mb = s_M * c;
  const T* base = logits + (int64_t)row * row_stride;
  const int e0 = s_chunk * chunk_len, e1 = min(vocab, e0 + chunk_len);
  // this thread's contiguous slice [a0, a1) of the chunk, N-aligned
  const int per = ((e1 - e0 + kThreads - 1) / kThreads + N - 1) / N * N;
  const int a0 = min(e1, e0 + tid * per), a1 = min(e1, a0 + per);
  auto weight = [&](float x) __attribute__((always_inline)) { return exp2_fast(__builtin_fmaf(x, c, -mb)); };
  float sum = 0.f;
  int last_pos = -1;
  const int vend = kVector ? a0 + (a1 - a0) / N * N : a0;   // end of whole vectors of the slice
  if (kVector) {
#pragma unroll 4
    for (int v = a0; v < vend; v += N) {
      float x[N];
      Vec<T>::unpack(Vec<T>::load(base + v), x);
#pragma unroll
      for (int j = 0; j < N; ++j) {
        const float q = weight(x[j]);
        sum += q;
        last_pos = q > 0.f ? v + j : last_pos;
      }
    }
  }
  for (int v = vend; v < a1; ++v) {   // the slice's scalar part (all of it without vector loads)
    const float q = weight(Vec<T>::scalar(base + v));
    sum += q;
    last_pos = q > 0.f ? v : last_pos;
  }
  // scan of the slice sums (thread order = id order); each thread's interval
  // [lower, upper) takes its ends from the same sums as its neighbours', so the
  // intervals tile the chunk without gaps and exactly one brackets a target
  // below the chunk total
  float incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  float prev = __shfl_up(incl, 1, 64);
  if (lane == 0) prev = 0.f;
  if (lane == 63) s_wsum[wave] = incl;
  atomicMax(&s_last, last_pos);
  __syncthreads();
  float wbase = 0.f;
  for (int w = 0; w < wave; ++w) wbase += s_wsum[w];
  const float pre = wbase + prev, upper = wbase + incl;
  if (pre <= res && res < upper) {
    // Rescan the slice in id order for the first running sum past the target:
    // whole vectors four loads at a time (the slice was just read: cache hits),
    // the running sum kept per vector, then the elements of the crossing vector.
    float run = pre;
    int hit = -1;
    int v = a0;
    for (; v < vend && hit < 0; v += 4 * N) {
      float vs[4];
      float xs[4][N];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (v + i * N < vend) Vec<T>::unpack(Vec<T>::load(base + v + i * N), xs[i]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vs[i] = 0.f;
        if (v + i * N < vend)
#pragma unroll
          for (int j = 0; j < N; ++j) vs[i] += weight(xs[i][j]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (hit < 0 && v + i * N < vend) {
          if (run + vs[i] > res) {
            float r2 = run;
#pragma unroll
            for (int j = 0; j < N; ++j) {
              r2 += weight(xs[i][j]);
              if (hit < 0 && r2 > res) hit = v + i * N + j;
            }
            if (hit < 0) hit = v + i * N + N - 1;   // rounding: the vector's last id
          }
          run += vs[i];
        }
      }
    }
    for (int e = vend; e < a1 && hit < 0; ++e) {   // the slice's scalar tail
      run += weight(Vec<T>::scalar(base + e));
      if (run > res) hit = e;
    }
    atomicMin(&s_found, hit >= 0 ? hit : a1 - 1);   // one thread brackets the target; min guards ties
  }
  __syncthreads();
  if (tid == 0) {
    // the bracketing id; else (rounding) the chunk's last id of positive weight; else the argmax
    const int id = s_found != 0x7fffffff ? s_found : (s_last >= 0 ? s_last : s_idx);
    row_pred[row] = id;
    row_conf[row] = weight(Vec<T>::scalar(base + id)) / s_S;
  }
}

// ---- sampling under top-k / top-p truncation ----------------------------------
// One workgroup of 512 threads (two waves per SIMD, so that a thread has 256
// registers) per masked row holds the whole row in registers (kTrVec 16-byte
// vectors per thread; vector j of thread t holds ids (512 j + t) N .. + N - 1),
// so the row is read from HBM once:
//   1. the largest order key (a total order on the values, -0 taken as +0),
//      the invalid flag and the count of finite values (workgroup reductions);
//   2. the cut, the order key of the smallest kept value.  bf16 rows: counts
//      per 16-bit key in an LDS histogram (one bin per representable value,
//      windows of 32768 keys below the row maximum, at most two), whose running
//      count and mass (count times the value's weight) over decreasing values
//      place the top-k and then the top-p cut exactly, with no exponential per
//      element.  fp32 rows: bisection over the 32-bit key, one workgroup count
//      or mass reduction per step.
//   3. inverse CDF over the kept ids in id order: vector totals across the
//      workgroup give the vector holding u times the kept mass, a workgroup
//      scan of that vector's per-thread weights the thread, and a walk of its
//      N ids the id.  conf = weight / kept mass.
constexpr int kTrThreads = 512;
constexpr int kTrWaves = kTrThreads / 64;
constexpr int kTrVec = 38;                           // 16-byte vectors per thread
constexpr int kHistBins = 32768;                     // histogram window (keys)
constexpr int kHistPerThread = kHistBins / kTrThreads;
// One pad word after every 64 bins: the 64 bins a thread scans start 65 words
// after its neighbour's, so a wave's scan reads fall in distinct banks.
constexpr int kHistWords = kHistBins + kHistBins / 64;
constexpr size_t kHistBytes = kHistWords * sizeof(uint32_t);
static_assert(kHistPerThread == 64, "one pad word per thread's bins");
__device__ __forceinline__ uint32_t hist_at(uint32_t off) { return off + (off >> 6); }
constexpr size_t kPsBytes = (size_t)kTrVec * kTrThreads * sizeof(float);   // per-thread vector sums
static_assert(kPsBytes <= kHistBytes, "the vector sums reuse the histogram's space");

// The row is held as order keys: unsigned integers in the order of the values
// (sign bit flipped for positive values, all bits for negative ones; -0 taken
// as +0), so that the cut is a key and equal values share one key.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
template <typename T> struct TrElem;
template <> struct TrElem<uint16_t> {
  static constexpr int N = 8;
  static constexpr uint32_t kNegInfKey = 0x007Fu;        // key of -inf
  static constexpr uint32_t kPosInfKey = 0xFF80u;        // key of +inf (NaNs lie outside the two)
  __device__ __forceinline__ static uint32_t key(const u32x4& r, int e) {
    const uint32_t w = r[e >> 1];
    return (e & 1) ? (w >> 16) : (w & 0xFFFFu);
  }
  __device__ __forceinline__ static uint32_t to_key(uint32_t b) {
    b = b == 0x8000u ? 0u : b;
    return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
  }
  __device__ __forceinline__ static float value_of_key(uint32_t k) { return __uint_as_float(((k & 0x8000u) ? (k & 0x7FFFu) : (~k & 0xFFFFu)) << 16); }
  __device__ __forceinline__ static uint32_t fetch(const uint16_t* p) { return *p; }
  __device__ __forceinline__ static void put(u32x4& r, int e, uint32_t k) {
    const uint32_t w = r[e >> 1];
    r[e >> 1] = (e & 1) ? ((w & 0xFFFFu) | (k << 16)) : ((w & 0xFFFF0000u) | k);
  }
  // Both halves of each word at once (packed 16-bit integer operations):
  // flip the sign bit of positive values and every bit of negative ones, then
  // move -0 (key 0x7FFF) up to +0's key.
  __device__ __forceinline__ static void to_keys(u32x4& r) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = r[i];
      const uint32_t neg = __builtin_bit_cast(uint32_t, __builtin_bit_cast(s16x2, w) >> (short)15);
      const uint32_t k = w ^ (neg | 0x80008000u);
      const u16x2 nz = __builtin_elementwise_min(__builtin_bit_cast(u16x2, k ^ 0x7FFF7FFFu), u16x2{1, 1});
      r[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, k) + (u16x2{1, 1} - nz));
    }
  }
  // Largest and smallest key and the count of keys above -inf's, for both
  // halves at once (count halves hold at most 4 kTrVec).  (The elements are
  // copied out before the bit casts: a bit cast of a vector element in place
  // reads element 0 with this compiler.)
  __device__ __forceinline__ static void scan_keys(const u32x4& r, u16x2& kmax, u16x2& kmin, u16x2& nfin) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = r[i];
      const u16x2 k = __builtin_bit_cast(u16x2, w);
      kmax = __builtin_elementwise_max(kmax, k);
      kmin = __builtin_elementwise_min(kmin, k);
      nfin += __builtin_elementwise_min(k - u16x2{(unsigned short)kNegInfKey, (unsigned short)kNegInfKey}, u16x2{1, 1});
    }
  }
  // Largest key of the vector.
  __device__ __forceinline__ static uint32_t vmax(const u32x4& r) {
    const uint32_t w0 = r[0], w1 = r[1], w2 = r[2], w3 = r[3];
    const u16x2 m = __builtin_elementwise_max(
        __builtin_elementwise_max(__builtin_bit_cast(u16x2, w0), __builtin_bit_cast(u16x2, w1)),
        __builtin_elementwise_max(__builtin_bit_cast(u16x2, w2), __builtin_bit_cast(u16x2, w3)));
    return max((uint32_t)m.x, (uint32_t)m.y);
  }
};
template <> struct TrElem<float> {
  static constexpr int N = 4;
  static constexpr uint32_t kNegInfKey = 0x007FFFFFu;
  static constexpr uint32_t kPosInfKey = 0xFF800000u;
  __device__ __forceinline__ static uint32_t key(const u32x4& r, int e) { return r[e]; }
  __device__ __forceinline__ static uint32_t to_key(uint32_t b) {
    b = b == 0x80000000u ? 0u : b;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  }
  __device__ __forceinline__ static float value_of_key(uint32_t k) { return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k); }
  __device__ __forceinline__ static uint32_t fetch(const float* p) { return __float_as_uint(*p); }
  __device__ __forceinline__ static void put(u32x4& r, int e, uint32_t k) { r[e] = k; }
  __device__ __forceinline__ static void to_keys(u32x4& r) {
#pragma unroll
    for (int e = 0; e < N; ++e) r[e] = to_key(r[e]);
  }
  __device__ __forceinline__ static uint32_t vmax(const u32x4& r) { return max(max(r[0], r[1]), max(r[2], r[3])); }
};

// Opaque to the optimiser, placed before the work on each vector of every
// pass: a pass recomputes what it needs from the keys instead of keeping
// per-element values alive from an earlier pass, and the vectors of a pass
// are processed in turn rather than all interleaved (either would spill).
__device__ __forceinline__ void tr_fence(u32x4& v) { asm volatile("" : "+v"(v)); }

// r[j] for a workgroup-uniform j, by selects (no indexed register access).
__device__ __forceinline__ u32x4 tr_pick(const u32x4 (&r)[kTrVec], int j) {
  u32x4 v = r[0];
#pragma unroll
  for (int i = 1; i < kTrVec; ++i) {
    const bool h = i == j;
    v.x = h ? r[i].x : v.x;
    v.y = h ? r[i].y : v.y;
    v.z = h ? r[i].z : v.z;
    v.w = h ? r[i].w : v.w;
  }
  return v;
}

struct TrShared {
  float redf[kTrWaves];
  uint32_t redu[kTrWaves];
  float vtot[kTrVec];
  uint32_t cut_off;              // offset (below the largest key) of the smallest kept value
  float cut_mass;                // running mass through that value
  int first_thr, last_id, id;
};

// Workgroup-uniform values (read from LDS) moved to scalar registers, so that
// branches on them are scalar branches.
__device__ __forceinline__ uint32_t tr_uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ float tr_uni(float v) { return __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(v))); }
__device__ __forceinline__ int tr_uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Workgroup sums (every thread gets the same total; fixed order).
__device__ __forceinline__ float tr_sum(float v, TrShared& sh, int lane, int wave) {
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) sh.redf[wave] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < kTrWaves; ++w) t += sh.redf[w];
  return tr_uni(t);
}
__device__ __forceinline__ uint32_t tr_sum(uint32_t v, TrShared& sh, int lane, int wave) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  __syncthreads();
  if (lane == 0) sh.redu[wave] = v;
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (int w = 0; w < kTrWaves; ++w) t += sh.redu[w];
  return tr_uni(t);
}
__device__ __forceinline__ uint32_t tr_max(uint32_t v, TrShared& sh, int lane, int wave) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = max(v, (uint32_t)__shfl_xor(v, m, 64));
  __syncthreads();
  if (lane == 0) sh.redu[wave] = v;
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (int w = 0; w < kTrWaves; ++w) t = max(t, sh.redu[w]);
  return tr_uni(t);
}

// Exclusive workgroup scan in thread order: c (exact) and m (fp32, fixed order).
__device__ __forceinline__ void tr_scan(uint32_t c, float m, uint32_t& c_ex, float& m_ex, uint32_t& c_tot,
                                        float& m_tot, TrShared& sh, int lane, int wave) {
  uint32_t ci = c;
  float mi = m;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t yc = __shfl_up(ci, off, 64);
    const float ym = __shfl_up(mi, off, 64);
    if (lane >= off) {
      ci += yc;
      mi += ym;
    }
  }
  uint32_t cx = __shfl_up(ci, 1, 64);
  float mx = __shfl_up(mi, 1, 64);
  if (lane == 0) {
    cx = 0;
    mx = 0.f;
  }
  __syncthreads();
  if (lane == 63) {
    sh.redu[wave] = ci;
    sh.redf[wave] = mi;
  }
  __syncthreads();
  uint32_t cb = 0, ct = 0;
  float mb = 0.f, mt = 0.f;
#pragma unroll
  for (int w = 0; w < kTrWaves; ++w) {
    if (w < wave) {
      cb += sh.redu[w];
      mb += sh.redf[w];
    }
    ct += sh.redu[w];
    mt += sh.redf[w];
  }
  c_ex = cb + cx;
  m_ex = mb + mx;
  c_tot = tr_uni(ct);
  m_tot = tr_uni(mt);
}

template <typename T, bool kVector>
__global__ __launch_bounds__(kTrThreads) void sample_truncated(const T* __restrict__ logits, int64_t row_stride,
                                                               int vocab, const uint8_t* __restrict__ masked,
                                                               float c, int top_k, float top_p, uint32_t seed_lo,
                                                               uint32_t seed_hi, uint32_t step_lo, uint32_t step_hi,
                                                               float* __restrict__ row_conf,
                                                               int32_t* __restrict__ row_pred) {
  using E = TrElem<T>;
  constexpr int N = E::N;
  constexpr bool kHist = sizeof(T) == 2;
  extern __shared__ __attribute__((aligned(16))) uint32_t hist[];
  __shared__ TrShared sh;
  const int row = blockIdx.x;
  if (!masked[row]) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const T* base = logits + (int64_t)row * row_stride;

  // ---- the row into registers: every whole vector first (clamped addresses,
  // no branch between the loads), then the ragged or missing ones by element
  u32x4 r[kTrVec];
  if (kVector) {
    const int last_full = (vocab / N - 1) * N;   // vocab >= N on this path
#pragma unroll
    for (int j = 0; j < kTrVec; ++j) {
      const int v0 = min((j * kTrThreads + tid) * N, last_full);
      r[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + v0));
    }
  }
#pragma unroll
  for (int j = 0; j < kTrVec; ++j) {
    const int v0 = (j * kTrThreads + tid) * N;
    if (!kVector || v0 + N > vocab) {
      // ids past the row hold -inf's key (never kept)
#pragma unroll
      for (int e = 0; e < N; ++e) E::put(r[j], e, v0 + e < vocab ? E::to_key(E::fetch(base + v0 + e)) : E::kNegInfKey);
    } else {
      E::to_keys(r[j]);
    }
  }

  // ---- 1. largest key, invalid flag (a NaN or +inf), finite count
  uint32_t kmax = 0, nfin = 0, bad = 0;
  if constexpr (kHist) {
    // a valid row has no key above +inf's or below -inf's; then the largest key
    // is the largest finite one unless every value is -inf (no finite count)
    u16x2 mx{0, 0}, mn{0xFFFF, 0xFFFF}, nf{0, 0};
#pragma unroll
    for (int j = 0; j < kTrVec; ++j) {
      tr_fence(r[j]);
      E::scan_keys(r[j], mx, mn, nf);
    }
    kmax = max((uint32_t)mx.x, (uint32_t)mx.y);
    bad = kmax >= E::kPosInfKey || min((uint32_t)mn.x, (uint32_t)mn.y) < E::kNegInfKey;
    nfin = (uint32_t)nf.x + (uint32_t)nf.y;
  } else {
#pragma unroll
    for (int j = 0; j < kTrVec; ++j) {
      tr_fence(r[j]);
#pragma unroll
      for (int e = 0; e < N; ++e) {
        const uint32_t k = E::key(r[j], e);
        const bool fin = k > E::kNegInfKey && k < E::kPosInfKey;
        bad |= k >= E::kPosInfKey || k < E::kNegInfKey;
        nfin += fin;
        kmax = fin ? max(kmax, k) : kmax;
      }
    }
  }
  bad = tr_max(bad, sh, lane, wave);
  nfin = tr_sum(nfin, sh, lane, wave);
  kmax = tr_max(kmax, sh, lane, wave);
  if (bad || nfin == 0) {
    if (tid == 0) {
      row_conf[row] = __builtin_nanf("");
      row_pred[row] = -1;
    }
    return;
  }
  const float M = E::value_of_key(kmax), mb = M * c;
  auto weight = [&](float x) __attribute__((always_inline)) { return exp2_fast(__builtin_fmaf(x, c, -mb)); };
  const bool need_k = top_k >= 1 && (uint32_t)top_k < nfin;
  const bool need_p = top_p < 1.f;

  // ---- 2. the cut
  uint32_t cut_key = E::kNegInfKey + 1;   // keep every finite value
  if constexpr (kHist) {
    // bins of window w: offsets kmax - key - 32768 w in [0, 32768)
    // With `rest`, also the mass of the finite values below the window (the
    // total mass then needs no second window).
    auto build = [&](uint32_t wbase, bool rest) __attribute__((always_inline)) {
      uint4* h4 = reinterpret_cast<uint4*>(hist);
      for (int i = tid; i < kHistWords / 4; i += kTrThreads) h4[i] = make_uint4(0, 0, 0, 0);
      __syncthreads();
      float rm = 0.f;
#pragma unroll
      for (int j = 0; j < kTrVec; ++j) {
        tr_fence(r[j]);
#pragma unroll
        for (int e = 0; e < N; ++e) {
          const uint32_t k = E::key(r[j], e);
          const uint32_t off = kmax - k - wbase;
          if (k > E::kNegInfKey && off < (uint32_t)kHistBins) atomicAdd(&hist[hist_at(off)], 1u);
          if (rest && k > E::kNegInfKey && off >= (uint32_t)kHistBins) rm += weight(E::value_of_key(k));
        }
        if (rest) asm volatile("" : "+v"(rm));
      }
      return rest ? tr_sum(rm, sh, lane, wave) : (__syncthreads(), 0.f);
    };
    // mass of bin i of this thread's 32 (count times the weight of its value), kept
    // out of fused multiply-adds so that the scan and the walk below round alike
    // (masses are only needed for top-p: with top-k alone the counts place the cut)
    auto mass_at = [&](uint32_t off, uint32_t cnt) __attribute__((always_inline)) {   // off: below the maximum
      return (cnt == 0 || !need_p) ? 0.f : __fmul_rn((float)cnt, weight(E::value_of_key(kmax - off)));
    };
    auto bin_mass = [&](uint32_t wbase, int i, uint32_t cnt) __attribute__((always_inline)) {
      return mass_at(wbase + (uint32_t)(tid * kHistPerThread + i), cnt);
    };
    uint32_t c_ex = 0, own_c = 0, c_tot = 0;
    float m_ex = 0.f, own_m = 0.f, m_tot = 0.f;
    auto scan = [&](uint32_t wbase, uint32_t cbase, float mbase) __attribute__((always_inline)) {
      own_c = 0;
      own_m = 0.f;
#pragma unroll 8
      for (int i = 0; i < kHistPerThread; ++i) {
        const uint32_t cnt = hist[tid * (kHistPerThread + 1) + i];
        own_c += cnt;
        own_m = __fadd_rn(own_m, bin_mass(wbase, i, cnt));
      }
      tr_scan(own_c, own_m, c_ex, m_ex, c_tot, m_tot, sh, lane, wave);
      c_ex += cbase;
      m_ex = __fadd_rn(mbase, m_ex);
      c_tot += cbase;
      m_tot = __fadd_rn(mbase, m_tot);
    };
    // The first bin whose running count reaches k (exact: one thread brackets it).
    // Its wave walks the bracketing thread's 64 bins, a bin per lane.
    auto find_count = [&](uint32_t wbase, uint32_t k) __attribute__((always_inline)) {
      if (c_ex < k && k <= c_ex + own_c) sh.first_thr = tid;
      __syncthreads();
      const int bt = tr_uni(sh.first_thr);
      if (wave == bt / 64) {
        const uint32_t off = wbase + (uint32_t)(bt * kHistPerThread + lane);
        const uint32_t cnt = hist[bt * (kHistPerThread + 1) + lane];
        uint32_t cc = cnt;
        float cm = mass_at(off, cnt);
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const uint32_t yc = __shfl_up(cc, d, 64);
          const float ym = __shfl_up(cm, d, 64);
          if (lane >= d) {
            cc += yc;
            cm += ym;
          }
        }
        const uint32_t cb = __shfl(c_ex, bt & 63, 64);
        const float mb0 = __shfl(m_ex, bt & 63, 64);
        const unsigned long long hit = __builtin_amdgcn_ballot_w64(cb + cc >= k);
        if (lane == __builtin_ctzll(hit)) {
          sh.cut_off = off;
          sh.cut_mass = __fadd_rn(mb0, cm);
        }
      }
      __syncthreads();
    };
    // The first bin whose running mass reaches the target: the first thread whose
    // running mass through its last bin does, then its bins in order (the last
    // one reaches it, as the sums are formed alike).  None: keep the window.
    auto find_mass = [&](uint32_t wbase, float target) __attribute__((always_inline)) {
      if (tid == 0) sh.first_thr = kTrThreads;
      __syncthreads();
      if (__fadd_rn(m_ex, own_m) >= target) atomicMin(&sh.first_thr, tid);
      __syncthreads();
      if (tid == sh.first_thr) {
        float lm = 0.f;
        for (int i = 0; i < kHistPerThread; ++i) {
          lm = __fadd_rn(lm, bin_mass(wbase, i, hist[tid * (kHistPerThread + 1) + i]));
          if (__fadd_rn(m_ex, lm) >= target) {
            sh.cut_off = wbase + (uint32_t)(tid * kHistPerThread + i);
            break;
          }
        }
      }
      __syncthreads();
    };
    // Windows are built one at a time, window 0 first (the largest values):
    // top-k needs the window holding the k-th largest value; top-p needs the
    // top-k mass (or, with top-k off, the total over both windows) and then the
    // window holding its crossing.  At most three builds.
    constexpr uint32_t kNone = 0xFFFFFFFFu;
    uint32_t off_k = kNone, off_p = kNone, tc0 = 0;
    float tm0 = 0.f, zk = 0.f;
    bool k_done = !need_k, z_known = need_k ? false : !need_p, p_done = !need_p;
    const bool want_rest = !need_k && need_p;   // the total mass from window 0's build
    float rest_m = 0.f;
    int want = 0;
#pragma unroll 1
    for (int it = 0; it < 4 && want >= 0; ++it) {
      const uint32_t wbase = want ? (uint32_t)kHistBins : 0u;
      const float rm = build(wbase, want_rest && want == 0);
      scan(wbase, want ? tc0 : 0u, want ? tm0 : 0.f);
      if (want == 0) {
        tc0 = c_tot;
        tm0 = m_tot;
        rest_m = rm;
      }
      int next = -1;
      if (!k_done) {
        if ((uint32_t)top_k <= c_tot) {
          if (tid == 0) sh.cut_off = kNone;
          __syncthreads();
          find_count(wbase, (uint32_t)top_k);
          off_k = tr_uni(sh.cut_off);
          zk = tr_uni(sh.cut_mass);
          k_done = z_known = true;
        } else {
          next = 1;
        }
      } else if (!z_known) {
        zk = __fadd_rn(tm0, rest_m);
        z_known = true;
      }
      if (next < 0 && !p_done) {
        const float target = top_p * zk;
        const int wp = (target <= tm0 || nfin == tc0) ? 0 : 1;
        if (wp == want) {
          if (tid == 0) sh.cut_off = kNone;
          __syncthreads();
          find_mass(wbase, target);
          off_p = tr_uni(sh.cut_off);
          p_done = true;
        } else {
          next = wp;
        }
      }
      want = next;
    }
    const uint32_t cut_off = min(off_k, off_p);
    if (cut_off != kNone) cut_key = kmax - cut_off;
  } else {
    // bisection over the order key: the largest key t with count (mass) of the
    // values at or above t reaching k (the top-p target)
    // (t is always above -inf's key)
    auto count_ge = [&](uint32_t t) __attribute__((always_inline)) {
      uint32_t n = 0;
#pragma unroll
      for (int j = 0; j < kTrVec; ++j) {
        tr_fence(r[j]);
#pragma unroll
        for (int e = 0; e < N; ++e) n += E::key(r[j], e) >= t;
      }
      return tr_sum(n, sh, lane, wave);
    };
    auto mass_ge = [&](uint32_t t) __attribute__((always_inline)) {
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < kTrVec; ++j) {
        tr_fence(r[j]);
#pragma unroll
        for (int e = 0; e < N; ++e) {
          const uint32_t k = E::key(r[j], e);
          s += k >= t ? weight(E::value_of_key(k)) : 0.f;
        }
        asm volatile("" : "+v"(s));
      }
      return tr_sum(s, sh, lane, wave);
    };
    uint32_t lo = E::kNegInfKey + 1;
    if (need_k) {
      uint32_t hi = kmax;
      while (lo < hi) {
        const uint32_t mid = lo + (hi - lo + 1) / 2;
        if (count_ge(mid) >= (uint32_t)top_k) lo = mid;
        else hi = mid - 1;
      }
    }
    if (need_p) {
      const float target = top_p * mass_ge(lo);
      uint32_t hi = kmax;
      while (lo < hi) {
        const uint32_t mid = lo + (hi - lo + 1) / 2;
        if (mass_ge(mid) >= target) lo = mid;
        else hi = mid - 1;
      }
    }
    cut_key = lo;
  }

  // ---- 3. inverse CDF over the kept ids, in id order.  Each thread's kept
  // weight per vector goes to LDS (the histogram's space), ps[j][t].
  auto kept_w = [&](uint32_t k) __attribute__((always_inline)) {
    return k >= cut_key ? weight(E::value_of_key(k)) : 0.f;
  };
  float* ps = reinterpret_cast<float*>(hist);
  __syncthreads();   // the histogram is no longer read
#pragma unroll
  for (int j = 0; j < kTrVec; ++j) {
    tr_fence(r[j]);
    float s = 0.f;
    if (E::vmax(r[j]) >= cut_key) {   // no exponentials for a vector with nothing kept
#pragma unroll
      for (int e = 0; e < N; ++e) s += kept_w(E::key(r[j], e));
    }
    asm volatile("" ::"v"(s));
    ps[j * kTrThreads + tid] = s;
  }
  if (tid == 0) {
    sh.last_id = -1;
    sh.first_thr = kTrThreads;
    sh.id = -1;
  }
  __syncthreads();
  // vector totals: wave w adds vectors w, w + 8, ... (eight consecutive threads' sums per lane)
  for (int j = wave; j < kTrVec; j += kTrWaves) {
    const float* q = ps + j * kTrThreads + lane * (kTrThreads / 64);
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < kTrThreads / 64; ++i) t += q[i];
    t = wave_sum(t);
    if (lane == 0) sh.vtot[j] = t;
  }
  __syncthreads();
  float Z = 0.f;
#pragma unroll
  for (int j = 0; j < kTrVec; ++j) Z += sh.vtot[j];
  Z = tr_uni(Z);
  const uint32_t wu = philox_word0((uint32_t)row, step_lo, step_hi, 0u, seed_lo, seed_hi);
  const float target = (float)(((double)wu + 0.5) * (1.0 / 4294967296.0)) * Z;
  int js = -1;
  float before = 0.f;
  for (int j = 0; j < kTrVec; ++j) {
    const float t = tr_uni(sh.vtot[j]);
    if (before + t > target) {
      js = j;
      break;
    }
    before += t;
  }
  // the first thread of vector js whose running weight passes the target
  const float sj = js >= 0 ? ps[js * kTrThreads + tid] : 0.f;
  const float res = target - before;
  float pre = 0.f;
  {
    uint32_t cdummy, ctot;
    float mtot;
    tr_scan(0u, sj, cdummy, pre, ctot, mtot, sh, lane, wave);
  }
  if (js >= 0 && pre + sj > res) atomicMin(&sh.first_thr, tid);
  __syncthreads();
  if (js >= 0 && tid == sh.first_thr) {
    // its ids in order: the running weight is formed as in sj, so the last one passes
    const u32x4 v = tr_pick(r, js);
    float lw = 0.f;
    int hit = -1;
#pragma unroll
    for (int e = 0; e < N; ++e) {
      lw += kept_w(E::key(v, e));
      if (hit < 0 && pre + lw > res) hit = (js * kTrThreads + tid) * N + e;
    }
    sh.id = hit;
  }
  __syncthreads();
  if (tr_uni(sh.id) < 0) {
    // rounding left no thread of vector js past the target: the last kept id of
    // that vector (the target lies at its end); with no vector past it, the
    // last kept id of the row
    int last = -1;
#pragma unroll
    for (int j = 0; j < kTrVec; ++j) {
      tr_fence(r[j]);
      if (js >= 0 && j != js) continue;
#pragma unroll
      for (int e = 0; e < N; ++e) last = E::key(r[j], e) >= cut_key ? (j * kTrThreads + tid) * N + e : last;
    }
    atomicMax(&sh.last_id, last);
    __syncthreads();
  }
  const int id = tr_uni(sh.id >= 0 ? sh.id : sh.last_id);
  if (tid == ((id / N) & (kTrThreads - 1))) {
    const u32x4 v = tr_pick(r, id / N / kTrThreads);
    const int ee = id % N;
    float w = 0.f;
#pragma unroll
    for (int e = 0; e < N; ++e)
      if (e == ee) w = kept_w(E::key(v, e));
    row_pred[row] = id;
    row_conf[row] = w / Z;
  }
}

hipError_t launch_decide(const void* part, int nchunk, const float* row_conf, const int32_t* row_pred,
                         const CommitArgs& a, hipStream_t st) {
  // Rows with many partials (the fused projection: one per workgroup) get 32 threads each.
  const Partial* pp = reinterpret_cast<const Partial*>(part);
  if (nchunk >= 64)
    hipLaunchKernelGGL((commit_decide<32, 1024>), dim3(a.n_seq), dim3(1024), 0, st, pp, nchunk, row_conf, row_pred,
                       a.blk_len, a.threshold, a.thresholds, a.fallback_top1, a.tokens, a.masked, a.conf, a.pred,
                       a.n_committed, a.n_masked_left);
  else
    hipLaunchKernelGGL((commit_decide<kDecideLanes, kThreads>), dim3(a.n_seq), dim3(kThreads), 0, st, pp, nchunk,
                       row_conf, row_pred, a.blk_len, a.threshold, a.thresholds, a.fallback_top1, a.tokens,
                       a.masked, a.conf, a.pred, a.n_committed, a.n_masked_left);
  return hipGetLastError();
}

}  // namespace

size_t commit_sampled_workspace_bytes(int n_seq, int blk_len, int vocab) {
  const long long rows = (long long)n_seq * blk_len;
  const int len = commit_chunk_len(rows, vocab, kSampleTargetWGs);
  return (size_t)rows * (((long long)vocab + len - 1) / len) * sizeof(Partial) + (size_t)rows * 8;
}

hipError_t launch_commit_sampled(const CommitArgs& a, float temperature, uint64_t seed, uint64_t step,
                                 hipStream_t st) {
  const int64_t rows = (int64_t)a.n_seq * a.blk_len;
  const int chunk_len = commit_chunk_len(rows, a.vocab, kSampleTargetWGs);
  const int nchunk = (int)(((long long)a.vocab + chunk_len - 1) / chunk_len);
  Partial* part = reinterpret_cast<Partial*>(a.ws);
  float* row_conf = reinterpret_cast<float*>(reinterpret_cast<char*>(a.ws) + (size_t)rows * nchunk * sizeof(Partial));
  int32_t* row_pred = reinterpret_cast<int32_t*>(row_conf + rows);
  const float c = kLog2e / temperature;
  const uint32_t sl = (uint32_t)seed, sh = (uint32_t)(seed >> 32), tl = (uint32_t)step, th = (uint32_t)(step >> 32);
  const int elem = a.is_bf16 ? 2 : 4;
  const bool vec = ((uintptr_t)a.logits % 16 == 0) && ((a.row_stride * elem) % 16 == 0);
  const dim3 grid((unsigned)(rows * nchunk)), rgrid((unsigned)rows), block(kThreads);
  if (a.is_bf16) {
    const uint16_t* lg = reinterpret_cast<const uint16_t*>(a.logits);
    if (vec) {
      hipLaunchKernelGGL((commit_reduce<uint16_t, true>), grid, block, 0, st, lg, a.row_stride, a.vocab, nchunk, chunk_len, a.masked, part, c);
      hipLaunchKernelGGL((sample_locate<uint16_t, true>), rgrid, block, 0, st, lg, a.row_stride, a.vocab, nchunk, chunk_len, a.masked, part, c, sl, sh, tl, th, row_conf, row_pred);
    } else {
      hipLaunchKernelGGL((commit_reduce<uint16_t, false>), grid, block, 0, st, lg, a.row_stride, a.vocab, nchunk, chunk_len, a.masked, part, c);
      hipLaunchKernelGGL((sample_locate<uint16_t, false>), rgrid, block, 0, st, lg, a.row_stride, a.vocab, nchunk, chunk_len, a.masked, part, c, sl, sh, tl, th, row_conf, row_pred);
    }
  } else {
    const float* lg = reinterpret_cast<const float*>(a.logits);
    if (vec) {
      hipLaunchKernelGGL((commit_reduce<float, true>), grid, block, 0, st, lg, a.row_stride, a.vocab, nchunk, chunk_len, a.masked, part, c);
      hipLaunchKernelGGL((sample_locate<float, true>), rgrid, block, 0, st, lg, a.row_stride, a.vocab, nchunk, chunk_len, a.masked, part, c, sl, sh, tl, th, row_conf, row_pred);
    } else {
      hipLaunchKernelGGL((commit_reduce<float, false>), grid, block, 0, st, lg, a.row_stride, a.vocab, nchunk, chunk_len, a.masked, part, c);
      hipLaunchKernelGGL((sample_locate<float, false>), rgrid, block, 0, st, lg, a.row_stride, a.vocab, nchunk, chunk_len, a.masked, part, c, sl, sh, tl, th, row_conf, row_pred);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_decide(part, nchunk, row_conf, row_pred, a, st);
}

int sample_truncated_max_vocab(int is_bf16) { return kTrVec * kTrThreads * (is_bf16 ? 8 : 4); }

hipError_t launch_commit_sampled_truncated(const CommitArgs& a, float temperature, uint64_t seed, uint64_t step,
                                           int top_k, float top_p, hipStream_t st) {
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [] {
    const std::pair<const void*, size_t> fs[] = {
        {reinterpret_cast<const void*>(&sample_truncated<uint16_t, true>), kHistBytes},
        {reinterpret_cast<const void*>(&sample_truncated<uint16_t, false>), kHistBytes},
        {reinterpret_cast<const void*>(&sample_truncated<float, true>), kPsBytes},
        {reinterpret_cast<const void*>(&sample_truncated<float, false>), kPsBytes}};
    for (const auto& f : fs) {
      const hipError_t e = hipFuncSetAttribute(f.first, hipFuncAttributeMaxDynamicSharedMemorySize, (int)f.second);
      if (e != hipSuccess) attr_err = e;
    }
  });
  if (attr_err != hipSuccess) return attr_err;
  const int64_t rows = (int64_t)a.n_seq * a.blk_len;
  float* row_conf = reinterpret_cast<float*>(a.ws);
  int32_t* row_pred = reinterpret_cast<int32_t*>(row_conf + rows);
  const float c = kLog2e / temperature;
  const uint32_t sl = (uint32_t)seed, sh = (uint32_t)(seed >> 32), tl = (uint32_t)step, th = (uint32_t)(step >> 32);
  const int elem = a.is_bf16 ? 2 : 4;
  const bool vec = ((uintptr_t)a.logits % 16 == 0) && ((a.row_stride * elem) % 16 == 0) && a.vocab >= 16 / elem;
  const dim3 grid((unsigned)rows), block(kTrThreads);
  if (a.is_bf16) {
    const uint16_t* lg = reinterpret_cast<const uint16_t*>(a.logits);
    if (vec) hipLaunchKernelGGL((sample_truncated<uint16_t, true>), grid, block, kHistBytes, st, lg, a.row_stride, a.vocab, a.masked, c, top_k, top_p, sl, sh, tl, th, row_conf, row_pred);
    else hipLaunchKernelGGL((sample_truncated<uint16_t, false>), grid, block, kHistBytes, st, lg, a.row_stride, a.vocab, a.masked, c, top_k, top_p, sl, sh, tl, th, row_conf, row_pred);
  } else {
    const float* lg = reinterpret_cast<const float*>(a.logits);
    if (vec) hipLaunchKernelGGL((sample_truncated<float, true>), grid, block, kPsBytes, st, lg, a.row_stride, a.vocab, a.masked, c, top_k, top_p, sl, sh, tl, th, row_conf, row_pred);
    else hipLaunchKernelGGL((sample_truncated<float, false>), grid, block, kPsBytes, st, lg, a.row_stride, a.vocab, a.masked, c, top_k, top_p, sl, sh, tl, th, row_conf, row_pred);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_decide(nullptr, 1, row_conf, row_pred, a, st);
}

int commit_chunks_per_row(long long rows, int vocab) {
  const long long len = commit_chunk_len(rows, vocab);
  return (int)(((long long)vocab + len - 1) / len);
}

size_t commit_workspace_bytes(int n_seq, int blk_len, int vocab) {
  const long long rows = (long long)n_seq * blk_len;
  return (size_t)rows * commit_chunks_per_row(rows, vocab) * sizeof(Partial);
}

hipError_t launch_commit(const CommitArgs& a, hipStream_t st) {
  const int64_t rows = (int64_t)a.n_seq * a.blk_len;
  const int chunk_len = commit_chunk_len(rows, a.vocab);
  const int nchunk = (int)(((long long)a.vocab + chunk_len - 1) / chunk_len);
  Partial* part = reinterpret_cast<Partial*>(a.ws);
  const int elem = a.is_bf16 ? 2 : 4;
  const bool vec = ((uintptr_t)a.logits % 16 == 0) && ((a.row_stride * elem) % 16 == 0);
  dim3 grid((unsigned)(rows * nchunk));
  if (a.is_bf16) {
    const uint16_t* lg = reinterpret_cast<const uint16_t*>(a.logits);
    if (vec) hipLaunchKernelGGL((commit_reduce<uint16_t, true>), grid, dim3(kThreads), 0, st, lg, a.row_stride, a.vocab, nchunk, chunk_len, a.masked, part, kLog2e);
    else hipLaunchKernelGGL((commit_reduce<uint16_t, false>), grid, dim3(kThreads), 0, st, lg, a.row_stride, a.vocab, nchunk, chunk_len, a.masked, part, kLog2e);
  } else {
    const float* lg = reinterpret_cast<const float*>(a.logits);
    if (vec) hipLaunchKernelGGL((commit_reduce<float, true>), grid, dim3(kThreads), 0, st, lg, a.row_stride, a.vocab, nchunk, chunk_len, a.masked, part, kLog2e);
    else hipLaunchKernelGGL((commit_reduce<float, false>), grid, dim3(kThreads), 0, st, lg, a.row_stride, a.vocab, nchunk, chunk_len, a.masked, part, kLog2e);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_commit_decide(part, nchunk, a, st);
}

// ---- no-allocation variant ---------------------------------------------------
// The chunk partials of bd_confidence_commit_noalloc live in this array, one copy
// per GPU (loaded with the code object).  In host code `scratch` names a host-side
// stand-in: kernels get the device address looked up below, never the name.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];   // device address of `scratch` on each device, once looked up
}  // namespace

// Device address of `scratch` on the calling thread's current device.
static hipError_t noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return hipSuccess;
}

hipError_t launch_commit_noalloc(const CommitArgs& a, hipStream_t st) {
  if (commit_workspace_bytes(a.n_seq, a.blk_len, a.vocab) > kNoAllocScratchBytes) return hipErrorInvalidValue;
  void* ws = nullptr;
  const hipError_t e = noalloc_scratch(&ws);
  if (e != hipSuccess) return e;
  CommitArgs b = a;
  b.ws = ws;
  return launch_commit(b, st);
}

hipError_t launch_commit_decide(const void* part, int nchunk, const CommitArgs& a, hipStream_t st) {
  return launch_decide(part, nchunk, nullptr, nullptr, a, st);
}


}  // namespace bd
