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
//                                   K rows are read from LDS in sigma32 order)
//   online softmax per query column (one cross-lane exchange per tile)
//   O^T[128 d x 32 q] += V^T P^T   (4 x 4 MFMA 32x32x16; P^T comes straight
//                                   from the S^T accumulator, V^T is read from
//                                   the row-major V tile with transposed LDS
//                                   reads)
// K and V tiles go global -> LDS directly (no register staging) into a
// two-stage ring of swizzled tiles: the next tile's loads are in flight while a
// tile is multiplied; one barrier per tile.  Every LDS read address is a
// per-lane register computed once plus a compile-time offset (the tile loop is
// unrolled by the ring depth).
//
// Softmax: the score scale is folded into the exponent (one FMA per score
// before exp2), and the running maximum used as the exponent offset is only
// raised -- with the matching rescale of O and of the row sum -- when a
// column's maximum grows by more than 2^8; exact either way, since O and the
// row sum always share the same offset.
//
// Workgroups of one (batch, kv head) are handed to the same XCD (L2 reuse of
// K/V) and the most expensive query tiles are dispatched first.
#include "bd_device.hpp"
#include "bd_kernels.hpp"

#include <mutex>
#include <type_traits>

namespace bd {
namespace {

constexpr int D = 128;
constexpr int KT = 64;                    // keys per tile
#ifndef BD_FWD_NW
#define BD_FWD_NW 8
#endif
#ifndef BD_FWD_NS
#define BD_FWD_NS 2
#endif
constexpr int kNW = BD_FWD_NW;            // waves per workgroup
constexpr int kNS = BD_FWD_NS;            // LDS ring depth (tiles)
constexpr int kThreads = kNW * 64;
constexpr int kTileBytes = KT * D * 2;    // 16 KB
constexpr int kStageBytes = 2 * kTileBytes;
constexpr size_t kSmemBytes = (size_t)kNS * kStageBytes;
constexpr float kRescaleSlack = 8.0f;     // log2 units

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int L, Hq, Hkv, G, blk, qtiles;
  float scale_log2;  // softmax scale * log2(e)
};

__global__ __launch_bounds__(kThreads) void attn_fwd_bf16_d128(FwdParams p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

  static_assert(kNS == 2, "the tile loop below is written for a two-stage ring");
  // prologue: tile 0 in flight
  if (ntiles > 0) {
    tile_dma<kNW>(lds0, kb, kv_rs, 0, kend_wg, wave, lane);
    tile_dma<kNW>(lds0 + kTileBytes, vb, kv_rs, 0, kend_wg, wave, lane);
  }

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
  float m_use = kNegInf, l_run = 0.f;
  const float c2 = p.scale_log2;

  // Per-lane LDS byte addresses (stage 0), so that every read below is this
  // register plus a compile-time offset.
  //   K A operand, d-step ds: row sigma32(col) (+32 for the second key block),
  //     logical chunk 2*ds + half.
  //   V^T A operand (transposed read), d-block db, k-step s4, half-read tt:
  //     row 16*s4 + 8*half + 4*tt + jj, logical chunk 4*db + 2*g1 + b, where
  //     jj = (lane%16)/4, g1 = (lane/16)%2, b = (lane%4)/2; with tile_swz the
  //     physical chunk is 4*(db^jj) + 2*(g1^half) + (b ^ tt ^ (s4%2)).
  uint32_t kaddr[8], vaddr[4][2];
  {
    const int krow = sigma32(col);
    const int kswz = tile_swz(krow);
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) kaddr[ds] = lds0 + krow * 256 + (((2 * ds + half) ^ kswz) << 4);
    const int li = lane & 15, jj = li >> 2, g1 = (lane >> 4) & 1, bb = (li & 3) >> 1;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int x = 0; x < 2; ++x)
        vaddr[db][x] = lds0 + kTileBytes + (8 * half + jj) * 256 +
                       ((4 * (db ^ jj) + 2 * (g1 ^ half) + (bb ^ x)) << 4) + 8 * (li & 1);
  }

  auto step = [&](auto stage_c, int t) {
    constexpr int S = decltype(stage_c)::value;
    constexpr uint32_t so = S * kStageBytes;
    vm_wait<0>();
    __syncthreads();
    if (t + 1 < ntiles) {
      const uint32_t st = lds0 + (1 - S) * kStageBytes;
      tile_dma<kNW>(st, kb, kv_rs, (t + 1) * KT, kend_wg, wave, lane);
      tile_dma<kNW>(st + kTileBytes, vb, kv_rs, (t + 1) * KT, kend_wg, wave, lane);
    }
    const int key0 = t * KT;
    if (!active || key0 >= kend_hi) return;

    f32x16 sacc[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[h2][i] = 0.f;
#pragma unroll
      for (int ds = 0; ds < 8; ++ds)
        sacc[h2] = mfma_32x32x16(lds_read_b128(kaddr[ds] + so + h2 * 32 * 256), qreg[ds], sacc[h2]);
    }
    // entry i of block h2 holds key key0 + 32*h2 + 16*(i/8) + 8*half + (i%8)
    float mx = kNegInf;
    if (key0 + KT > kend_lo) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + 32 * h2 + 16 * (i >> 3) + 8 * half + (i & 7);
          if (key >= kq) sacc[h2][i] = kNegInf;
          mx = fmaxf(mx, sacc[h2][i]);
        }
    } else {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[h2][i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * c2;
    const bool grow = mx > m_use + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float m_new = grow ? mx : m_use;
      const float alpha = exp2_fast(m_use - m_new);
      m_use = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    }
    const float nm = -m_use;
    float psum = 0.f;
    bf16x8 pb[4];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pv[e] = exp2_fast(__builtin_fmaf(sacc[h2][8 * j + e], c2, nm));
          psum += pv[e];
        }
        pb[2 * h2 + j] = pack_bf16x8(pv);
      }
    l_run += psum;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const i16x4 lo = lds_read_tr16(vaddr[db][s4 & 1] + so + (16 * s4) * 256);
        const i16x4 hi = lds_read_tr16(vaddr[db][(s4 & 1) ^ 1] + so + (16 * s4 + 4) * 256);
        oacc[db] = mfma_32x32x16(cat_i16x4(lo, hi), pb[s4], oacc[db]);
      }
  };

  for (int t = 0; t < ntiles; t += 2) {
    step(std::integral_constant<int, 0>(), t);
    if (t + 1 < ntiles) step(std::integral_constant<int, 1>(), t + 1);
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
  if (p.lse && half == 0) p.lse[((int64_t)b * p.Hq + hq) * L + qrow] = (m_use + __log2f(l_tot)) * kLn2;
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
