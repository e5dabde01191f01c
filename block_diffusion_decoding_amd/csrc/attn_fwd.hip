// Block-causal attention forward on the gfx950 matrix cores (bf16 in, fp32
// accumulate, bf16 out, fp32 natural-log LSE).
//
// Mask (paper.rainbus.top digest, method step 3; OpenDataLab blog, Fig. 2):
// query i sees key j iff floor(j / L') <= floor(i / L'), i.e. j < key_limit(i).
//
// Work decomposition
//   workgroup = NW waves = 32*NW consecutive query rows of one (batch, q head);
//   each wave owns 32 rows.  The workgroup walks key tiles of 64 from key 0 to
//   the largest key_limit of its rows, so tiles wholly in the future are never
//   loaded or multiplied: cost follows the block mask (about L^2/2), not L^2.
//   A tile a wave cannot see at all is skipped by that wave; a tile that
//   straddles the diagonal applies the mask per element; all others run
//   unmasked.
//
// Per wave and key tile (S^T formulation, see bd_device.hpp for layouts):
//   S^T[64 keys x 32 q] = K Q^T   (2 x 8 MFMA 32x32x16; Q^T stays in registers,
//                                   K rows come from LDS in sigma32 order)
//   online softmax per query column (one cross-lane exchange per tile)
//   O^T[128 d x 32 q] += V^T P^T   (4 x 4 MFMA 32x32x16; P^T comes straight
//                                   from the S^T accumulator, V^T from LDS)
// K and V tiles are staged global -> registers -> LDS, double buffered, with
// the next tile's global loads in flight during the current tile's MFMAs.  V is
// written to LDS transposed ([d][key]) so its A operand is one 16-byte read.
//
// Workgroups of one (batch, kv head) are handed to the same XCD (L2 reuse of
// K/V) and the most expensive query tiles are dispatched first.
#include "bd_device.hpp"
#include "bd_kernels.hpp"

#include <mutex>

namespace bd {
namespace {

constexpr int D = 128;
constexpr int KT = 64;                       // keys per tile
constexpr int KP = D + 8;                    // LDS pitch of a K row (elements)
constexpr int VP = KT + 8;                   // LDS pitch of a V^T row (elements)
constexpr int K_TILE = KT * KP;              // elements
constexpr int V_TILE = D * VP;
constexpr int kNW = 4;                       // waves per workgroup
constexpr int kThreads = kNW * 64;
constexpr size_t kSmemBytes = 2 * (K_TILE + V_TILE) * sizeof(uint16_t);

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int L, Hq, Hkv, G, blk, qtiles;
  float scale_log2;  // softmax scale * log2(e)
};

// One tile of K (row layout) and V (transposed) in flight, per thread.
struct TileRegs {
  static constexpr int KCH = (KT * D / 8) / kThreads;         // 16-byte K chunks / thread
  static constexpr int VTASK = (KT / 4) * (D / 8);            // (4 keys x 8 d) tasks per tile
  static constexpr int VPT = (VTASK + kThreads - 1) / kThreads;
  uint4 k[KCH];
  uint4 v[VPT][4];
};

__device__ __forceinline__ void load_tile(TileRegs& r, const uint16_t* kb, const uint16_t* vb, int64_t rs,
                                          int key0, int kend, int tid) {
  const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < TileRegs::KCH; ++i) {
    const int c = tid + i * kThreads;
    const int key = key0 + (c >> 4);
    r.k[i] = key < kend ? ldg16(kb + key * rs + (c & 15) * 8) : z;
  }
#pragma unroll
  for (int i = 0; i < TileRegs::VPT; ++i) {
    const int task = tid + i * kThreads;
    const int kq = task & 15, ch = task >> 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int key = key0 + kq * 4 + e;
      r.v[i][e] = (task < TileRegs::VTASK && key < kend) ? ldg16(vb + key * rs + ch * 8) : z;
    }
  }
}

__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

__device__ __forceinline__ void store_tile(const TileRegs& r, uint16_t* ks, uint16_t* vt, int tid) {
#pragma unroll
  for (int i = 0; i < TileRegs::KCH; ++i) {
    const int c = tid + i * kThreads;
    *reinterpret_cast<uint4*>(ks + (c >> 4) * KP + (c & 15) * 8) = r.k[i];
  }
#pragma unroll
  for (int i = 0; i < TileRegs::VPT; ++i) {
    const int task = tid + i * kThreads;
    if (task >= TileRegs::VTASK) continue;
    const int kq = task & 15, ch = task >> 4;
    const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&r.v[i][0]);
    const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&r.v[i][1]);
    const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&r.v[i][2]);
    const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&r.v[i][3]);
    uint16_t* dst = vt + (ch * 8) * VP + kq * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint2 lo = make_uint2(lo_pair(w0[e], w1[e]), lo_pair(w2[e], w3[e]));  // d = 8ch + 2e
      uint2 hi = make_uint2(hi_pair(w0[e], w1[e]), hi_pair(w2[e], w3[e]));  // d = 8ch + 2e + 1
      *reinterpret_cast<uint2*>(dst + (2 * e) * VP) = lo;
      *reinterpret_cast<uint2*>(dst + (2 * e + 1) * VP) = hi;
    }
  }
}

__global__ __launch_bounds__(kThreads) void attn_fwd_bf16_d128(FwdParams p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t* ks = smem;               // [2][KT][KP]
  uint16_t* vt = smem + 2 * K_TILE;  // [2][D][VP]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wid = xcd_remap(blockIdx.x, gridDim.x);
  const int per_group = p.qtiles * p.G;
  const int grp = wid / per_group;
  const int rem = wid - grp * per_group;
  const int b = grp / p.Hkv, kvh = grp - b * p.Hkv;
  const int qt = p.qtiles - 1 - rem / p.G;
  const int hq = kvh * p.G + rem % p.G;

  const int L = p.L;
  const int wg_r0 = qt * (32 * kNW);
  const int r0 = wg_r0 + wave * 32;
  const int kend_wg = key_limit(min(wg_r0 + 32 * kNW, L) - 1, L, p.blk);
  const int ntiles = (kend_wg + KT - 1) / KT;
  const bool active = r0 < L;
  const int kend_lo = active ? key_limit(r0, L, p.blk) : 0;
  const int kend_hi = active ? key_limit(min(r0 + 31, L - 1), L, p.blk) : 0;

  const int col = lane & 31, half = lane >> 5;
  const int qrow = r0 + col;
  const int kq = key_limit(min(qrow, L - 1), L, p.blk);

  const int64_t q_rs = (int64_t)p.Hq * D, kv_rs = (int64_t)p.Hkv * D;
  const uint16_t* qb = p.q + (int64_t)b * L * q_rs + (int64_t)hq * D;
  const uint16_t* kb = p.k + (int64_t)b * L * kv_rs + (int64_t)kvh * D;
  const uint16_t* vb = p.v + (int64_t)b * L * kv_rs + (int64_t)kvh * D;

  bf16x8 qreg[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (qrow < L) u = ldg16(qb + qrow * q_rs + 16 * t + 8 * half);
    qreg[t] = as_bf16x8(u);
  }

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = kNegInf, l_run = 0.f;

  TileRegs regs;
  load_tile(regs, kb, vb, kv_rs, 0, kend_wg, tid);
  store_tile(regs, ks, vt, tid);
  __syncthreads();

  const int krow_off = sigma32(col) * KP + 8 * half;
  const int vrow_off = col * VP + 8 * half;

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) load_tile(regs, kb, vb, kv_rs, (t + 1) * KT, kend_wg, tid);
    const int key0 = t * KT;
    if (active && key0 < kend_hi) {
      const uint16_t* K = ks + buf * K_TILE;
      const uint16_t* V = vt + buf * V_TILE;
      f32x16 sacc[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[h2][i] = 0.f;
        const uint16_t* kr = K + h2 * 32 * KP + krow_off;
#pragma unroll
        for (int ds = 0; ds < 8; ++ds)
          sacc[h2] = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(kr + 16 * ds), qreg[ds], sacc[h2]);
      }
      const bool partial = key0 + KT > kend_lo;
      float mx = kNegInf;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float s = sacc[h2][i] * p.scale_log2;
          if (partial) {
            const int key = key0 + 32 * h2 + 16 * (i >> 3) + 8 * half + (i & 7);
            if (key >= kq) s = kNegInf;
          }
          sacc[h2][i] = s;
          mx = fmaxf(mx, s);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2_fast(m_run - m_new);
      float psum = 0.f;
      bf16x8 pb[4];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          float pv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pv[e] = exp2_fast(sacc[h2][8 * j + e] - m_new);
            psum += pv[e];
          }
          pb[2 * h2 + j] = pack_bf16x8(pv);
        }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const uint16_t* vr = V + db * 32 * VP + vrow_off;
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
          oacc[db] = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(vr + 16 * s4), pb[s4], oacc[db]);
      }
    }
    if (t + 1 < ntiles) store_tile(regs, ks + (buf ^ 1) * K_TILE, vt + (buf ^ 1) * V_TILE, tid);
    __syncthreads();
  }

  if (!active) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (qrow >= L) return;
  const float inv = 1.0f / l_tot;
  uint16_t* orow = p.o + ((int64_t)b * L + qrow) * q_rs + (int64_t)hq * D;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint2 w = make_uint2(pack_bf16x2(oacc[db][4 * j] * inv, oacc[db][4 * j + 1] * inv),
                           pack_bf16x2(oacc[db][4 * j + 2] * inv, oacc[db][4 * j + 3] * inv));
      *reinterpret_cast<uint2*>(orow + 32 * db + 8 * j + 4 * half) = w;
    }
  if (p.lse && half == 0) p.lse[((int64_t)b * p.Hq + hq) * L + qrow] = (m_run + __log2f(l_tot)) * kLn2;
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                                const AttnShape& s, hipStream_t st) {
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [] {
    attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_fwd_bf16_d128),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSmemBytes);
  });
  if (attr_err != hipSuccess) return attr_err;
  FwdParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.L = s.seqlen;
  p.Hq = s.n_q_heads;
  p.Hkv = s.n_kv_heads;
  p.G = s.n_q_heads / s.n_kv_heads;
  p.blk = s.block_size;
  p.qtiles = (s.seqlen + 32 * kNW - 1) / (32 * kNW);
  p.scale_log2 = s.scale * kLog2e;
  const long long nblocks = (long long)s.batch * s.n_q_heads * p.qtiles;
  hipLaunchKernelGGL(attn_fwd_bf16_d128, dim3((unsigned)nblocks), dim3(kThreads), kSmemBytes, st, p);
  return hipGetLastError();
}

}  // namespace bd
