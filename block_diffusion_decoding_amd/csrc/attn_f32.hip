// fp32 vector-ALU path of the three attention entry points (forward, one
// block against a prefix cache, backward), for head_dim <= 128.
//
// One wave owns one query row (forward, decode, dQ) or one key row (dK/dV);
// each lane holds head_dim/64 entries and dot products are wave reductions.
// This path favours exactness over speed: it is the fp32 member of the kernel
// family and serves small problems.  Mask: query i sees key j iff
// floor(j / L') <= floor(i / L') (paper.rainbus.top digest, method step 3).
#include "bd_device.hpp"
#include "bd_kernels.hpp"

namespace bd {
namespace {

constexpr int kMaxPerLane = 2;  // head_dim <= 128

struct RowVec {
  float x[kMaxPerLane];
};

__device__ __forceinline__ RowVec load_row(const float* p, int d, int lane) {
  RowVec r;
#pragma unroll
  for (int e = 0; e < kMaxPerLane; ++e) {
    const int c = lane + 64 * e;
    r.x[e] = c < d ? p[c] : 0.f;
  }
  return r;
}

__device__ __forceinline__ float dot(const RowVec& a, const float* b, int d, int lane) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < kMaxPerLane; ++e) {
    const int c = lane + 64 * e;
    if (c < d) s += a.x[e] * b[c];
  }
  return wave_sum(s);
}

// Online-softmax attention of one query row over keys produced by `kv(j)`.
template <typename KV>
__device__ void attend_row(const RowVec& q, int nkeys, int d, float scale_log2, const KV& kv, float* o,
                           float* lse_out, int lane) {
  float m = kNegInf, l = 0.f;
  float acc[kMaxPerLane] = {0.f, 0.f};
  // Eight keys per step: their loads are in flight together and the online
  // update takes their common maximum (the same algebra as one key at a time).
  constexpr int kU = 8;
  int j = 0;
  for (; j + kU <= nkeys; j += kU) {
    float kx[kU][kMaxPerLane], vx[kU][kMaxPerLane];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const float* kr;
      const float* vr;
      kv(j + u, kr, vr);
#pragma unroll
      for (int e = 0; e < kMaxPerLane; ++e) {
        const int c = lane + 64 * e;
        kx[u][e] = c < d ? kr[c] : 0.f;
        vx[u][e] = c < d ? vr[c] : 0.f;
      }
    }
    float s[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < kMaxPerLane; ++e) part += q.x[e] * kx[u][e];
      s[u] = wave_sum(part) * scale_log2;
    }
    float m_new = m;
#pragma unroll
    for (int u = 0; u < kU; ++u) m_new = fmaxf(m_new, s[u]);
    const float alpha = exp2f(m - m_new);
    float pu[kU], psum = 0.f;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      pu[u] = exp2f(s[u] - m_new);
      psum += pu[u];
    }
    l = l * alpha + psum;
#pragma unroll
    for (int e = 0; e < kMaxPerLane; ++e) {
      float pv = 0.f;
#pragma unroll
      for (int u = 0; u < kU; ++u) pv += pu[u] * vx[u][e];
      acc[e] = acc[e] * alpha + pv;
    }
    m = m_new;
  }
  for (; j < nkeys; ++j) {
    const float* kr;
    const float* vr;
    kv(j, kr, vr);
    const float s = dot(q, kr, d, lane) * scale_log2;
    const float m_new = fmaxf(m, s);
    const float alpha = exp2f(m - m_new);
    const float pj = exp2f(s - m_new);
    l = l * alpha + pj;
#pragma unroll
    for (int e = 0; e < kMaxPerLane; ++e) {
      const int c = lane + 64 * e;
      acc[e] = acc[e] * alpha + (c < d ? pj * vr[c] : 0.f);
    }
    m = m_new;
  }
#pragma unroll
  for (int e = 0; e < kMaxPerLane; ++e) {
    const int c = lane + 64 * e;
    if (c < d) o[c] = acc[e] / l;
  }
  if (lse_out && lane == 0) *lse_out = (m + log2f(l)) * kLn2;
}

struct FwdF32 {
  const float *q, *k, *v;
  float *o, *lse;
  int B, L, Hq, Hkv, d, blk;
  float scale_log2;
};

__global__ __launch_bounds__(64) void attn_fwd_f32_rows(FwdF32 p) {
  const int64_t row = blockIdx.x;  // ((b * Hq + h) * L + i)
  const int i = (int)(row % p.L);
  const int h = (int)((row / p.L) % p.Hq);
  const int b = (int)(row / ((int64_t)p.L * p.Hq));
  const int g = h / (p.Hq / p.Hkv);
  const int lane = threadIdx.x;
  const RowVec q = load_row(p.q + (((int64_t)b * p.L + i) * p.Hq + h) * p.d, p.d, lane);
  const int64_t kv_rs = (int64_t)p.Hkv * p.d;
  const float* kb = p.k + (int64_t)b * p.L * kv_rs + (int64_t)g * p.d;
  const float* vb = p.v + (int64_t)b * p.L * kv_rs + (int64_t)g * p.d;
  auto kv = [&](int j, const float*& kr, const float*& vr) {
    kr = kb + j * kv_rs;
    vr = vb + j * kv_rs;
  };
  attend_row(q, key_limit(i, p.L, p.blk), p.d, p.scale_log2, kv,
             p.o + (((int64_t)b * p.L + i) * p.Hq + h) * p.d,
             p.lse ? p.lse + ((int64_t)b * p.Hq + h) * p.L + i : nullptr, lane);
}

struct DecF32 {
  const float *q, *kb, *vb, *kc, *vc;
  const int64_t* start;
  const int32_t* plen;
  float *o, *lse;
  int n_seq, T, Hq, Hkv, d;
  float scale_log2;
};

__global__ __launch_bounds__(64) void decode_f32_rows(DecF32 p) {
  const int64_t row = blockIdx.x;  // ((n * Hq + h) * T + t)
  const int t = (int)(row % p.T);
  const int h = (int)((row / p.T) % p.Hq);
  const int n = (int)(row / ((int64_t)p.T * p.Hq));
  const int g = h / (p.Hq / p.Hkv);
  const int lane = threadIdx.x;
  const int P = p.plen[n];
  const int64_t s0 = p.start[n];
  const int64_t rs = (int64_t)p.Hkv * p.d;
  const RowVec q = load_row(p.q + (((int64_t)n * p.T + t) * p.Hq + h) * p.d, p.d, lane);
  auto kv = [&](int j, const float*& kr, const float*& vr) {
    const int64_t off = j < P ? (s0 + j) * rs : ((int64_t)n * p.T + (j - P)) * rs;
    kr = (j < P ? p.kc : p.kb) + off + (int64_t)g * p.d;
    vr = (j < P ? p.vc : p.vb) + off + (int64_t)g * p.d;
  };
  attend_row(q, P + p.T, p.d, p.scale_log2, kv, p.o + (((int64_t)n * p.T + t) * p.Hq + h) * p.d,
             p.lse ? p.lse + ((int64_t)n * p.Hq + h) * p.T + t : nullptr, lane);
}

struct BwdF32 {
  const float *q, *k, *v, *o, *lse, *dO;
  float *dq, *dk, *dv, *Dsum;
  int B, L, Hq, Hkv, d, blk;
  float scale;
};

// D[b, h, i] = sum_c dO[b, i, h, c] * O[b, i, h, c]
__global__ __launch_bounds__(64) void bwd_f32_dsum(BwdF32 p) {
  const int64_t row = blockIdx.x;  // ((b * Hq + h) * L + i)
  const int i = (int)(row % p.L);
  const int h = (int)((row / p.L) % p.Hq);
  const int b = (int)(row / ((int64_t)p.L * p.Hq));
  const int64_t off = (((int64_t)b * p.L + i) * p.Hq + h) * p.d;
  const RowVec a = load_row(p.dO + off, p.d, threadIdx.x);
  const float s = dot(a, p.o + off, p.d, threadIdx.x);
  if (threadIdx.x == 0) p.Dsum[row] = s;
}

// dq_i = scale * sum_j P_ij (dP_ij - D_i) k_j over the keys row i sees.
__global__ __launch_bounds__(64) void bwd_f32_dq(BwdF32 p) {
  const int64_t row = blockIdx.x;
  const int i = (int)(row % p.L);
  const int h = (int)((row / p.L) % p.Hq);
  const int b = (int)(row / ((int64_t)p.L * p.Hq));
  const int g = h / (p.Hq / p.Hkv);
  const int lane = threadIdx.x;
  const int64_t off = (((int64_t)b * p.L + i) * p.Hq + h) * p.d;
  const RowVec q = load_row(p.q + off, p.d, lane);
  const RowVec dO = load_row(p.dO + off, p.d, lane);
  const float lse = p.lse[row], Di = p.Dsum[row];
  const int64_t rs = (int64_t)p.Hkv * p.d;
  const float* kb = p.k + (int64_t)b * p.L * rs + (int64_t)g * p.d;
  const float* vb = p.v + (int64_t)b * p.L * rs + (int64_t)g * p.d;
  float acc[kMaxPerLane] = {0.f, 0.f};
  const int nk = key_limit(i, p.L, p.blk);
  for (int j = 0; j < nk; ++j) {
    const float* kr = kb + j * rs;
    const float pj = expf(dot(q, kr, p.d, lane) * p.scale - lse);
    const float dp = dot(dO, vb + j * rs, p.d, lane);
    const float ds = pj * (dp - Di);
#pragma unroll
    for (int e = 0; e < kMaxPerLane; ++e) {
      const int c = lane + 64 * e;
      if (c < p.d) acc[e] += ds * kr[c];
    }
  }
#pragma unroll
  for (int e = 0; e < kMaxPerLane; ++e) {
    const int c = lane + 64 * e;
    if (c < p.d) p.dq[off + c] = acc[e] * p.scale;
  }
}

// dk_j = scale * sum dS_ij q_i, dv_j = sum P_ij dO_i over every query i that
// sees key j (blocks >= block of j) and every query head of the group.
__global__ __launch_bounds__(64) void bwd_f32_dkdv(BwdF32 p) {
  const int64_t row = blockIdx.x;  // ((b * Hkv + g) * L + j)
  const int j = (int)(row % p.L);
  const int g = (int)((row / p.L) % p.Hkv);
  const int b = (int)(row / ((int64_t)p.L * p.Hkv));
  const int G = p.Hq / p.Hkv;
  const int lane = threadIdx.x;
  const int64_t kv_off = (((int64_t)b * p.L + j) * p.Hkv + g) * p.d;
  const RowVec k = load_row(p.k + kv_off, p.d, lane);
  const RowVec v = load_row(p.v + kv_off, p.d, lane);
  float ak[kMaxPerLane] = {0.f, 0.f}, av[kMaxPerLane] = {0.f, 0.f};
  const int i0 = (j / p.blk) * p.blk;
  for (int h = g * G; h < (g + 1) * G; ++h) {
    for (int i = i0; i < p.L; ++i) {
      const int64_t qoff = (((int64_t)b * p.L + i) * p.Hq + h) * p.d;
      const int64_t srow = ((int64_t)b * p.Hq + h) * p.L + i;
      const float* qr = p.q + qoff;
      const float* dor = p.dO + qoff;
      const float pij = expf(dot(k, qr, p.d, lane) * p.scale - p.lse[srow]);
      const float dp = dot(v, dor, p.d, lane);
      const float ds = pij * (dp - p.Dsum[srow]);
#pragma unroll
      for (int e = 0; e < kMaxPerLane; ++e) {
        const int c = lane + 64 * e;
        if (c < p.d) {
          av[e] += pij * dor[c];
          ak[e] += ds * qr[c];
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < kMaxPerLane; ++e) {
    const int c = lane + 64 * e;
    if (c < p.d) {
      p.dk[kv_off + c] = ak[e] * p.scale;
      p.dv[kv_off + c] = av[e];
    }
  }
}

}  // namespace

hipError_t launch_attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                               const AttnShape& s, hipStream_t st) {
  FwdF32 p{q, k, v, o, lse, s.batch, s.seqlen, s.n_q_heads, s.n_kv_heads, s.head_dim, s.block_size,
           s.scale * kLog2e};
  const long long rows = (long long)s.batch * s.n_q_heads * s.seqlen;
  hipLaunchKernelGGL(attn_fwd_f32_rows, dim3((unsigned)rows), dim3(64), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_decode_f32(const float* q_blk, const float* k_blk, const float* v_blk, const float* k_cache,
                             const float* v_cache, const int64_t* prefix_start, const int32_t* prefix_len,
                             float* o, float* lse, const DecodeShape& s, hipStream_t st) {
  DecF32 p{q_blk, k_blk, v_blk, k_cache, v_cache, prefix_start, prefix_len, o, lse,
           s.n_seq, s.blk_len, s.n_q_heads, s.n_kv_heads, s.head_dim, s.scale * kLog2e};
  const long long rows = (long long)s.n_seq * s.n_q_heads * s.blk_len;
  hipLaunchKernelGGL(decode_f32_rows, dim3((unsigned)rows), dim3(64), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_f32(const float* q, const float* k, const float* v, const float* o, const float* lse,
                               const float* d_o, float* dq, float* dk, float* dv, void* ws, const AttnShape& s,
                               hipStream_t st) {
  BwdF32 p{q, k, v, o, lse, d_o, dq, dk, dv, reinterpret_cast<float*>(ws), s.batch, s.seqlen, s.n_q_heads,
           s.n_kv_heads, s.head_dim, s.block_size, s.scale};
  const long long qrows = (long long)s.batch * s.n_q_heads * s.seqlen;
  const long long krows = (long long)s.batch * s.n_kv_heads * s.seqlen;
  hipLaunchKernelGGL(bwd_f32_dsum, dim3((unsigned)qrows), dim3(64), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_f32_dq, dim3((unsigned)qrows), dim3(64), 0, st, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_f32_dkdv, dim3((unsigned)krows), dim3(64), 0, st, p);
  return hipGetLastError();
}

}  // namespace bd
