// Block-causal attention backward on the gfx950 matrix cores (bf16 in and out,
// fp32 accumulation).  Gradients of the loss sum(O * dO) with
//   P = exp(scale * Q K^T - LSE),  D_i = sum_c dO_ic O_ic,
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),
//   dQ = scale * dS K,  dK = scale * dS^T Q  (dK, dV summed over the query heads
//   of a group),
// under the block-causal mask (paper.rainbus.top digest, method step 3): query
// i sees key j iff floor(j / L') <= floor(i / L').
//
// Three kernels, no atomics (bit-for-bit deterministic):
//   bwd_prep  per (batch, head, row): D = rowsum(dO * O) and LSE * log2(e),
//             stored interleaved in the workspace.
//   bwd_dkdv  workgroup = 4 waves = 128 consecutive keys of one (batch, kv
//             head); each wave owns 32 keys with K and V in registers and walks
//             the query tiles (64 rows) of every query head of the group, from
//             the first query that can see its keys to the end of the sequence.
//             Q and dO tiles (and their D / LSE slices) go global -> LDS
//             directly into a three-stage ring of swizzled row-major tiles.  Per
//             32-query slice:
//               S  = Q K^T, dP = dO V^T        (A = Q / dO rows from LDS, in
//                                               sigma32 order)
//               dV^T += dO^T P, dK^T += Q^T dS (A = dO^T / Q^T by transposed
//                                               LDS reads, B = P / dS straight
//                                               from the accumulators)
//   bwd_dq    workgroup = 8 waves = 256 query rows of one (batch, q head), as
//             the forward: per 32-key half of a 64-key tile,
//             S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T (K^T by transposed
//             reads of the K tile), over the key tiles its rows can see; K and V
//             tiles in a two-stage direct-to-LDS ring.
#include "bd_device.hpp"
#include "bd_kernels.hpp"

#include <mutex>
#include <type_traits>

namespace bd {
namespace {

constexpr int D = 128;
constexpr int kTileBytes = 64 * D * 2;   // 16 KB: one 64-row bf16 tile

struct BwdParams {
  const uint16_t *q, *k, *v, *o, *dO;
  const float* lse;
  float2* dl;          // [B, Hq, L]: (D, LSE * log2 e)
  uint16_t *dq, *dk, *dv;
  int B, L, Hq, Hkv, G, blk;
  float scale, scale_log2;
};

// ---------------------------------------------------------------------------
// 16 lanes per row, rows of [B, L, Hq] in memory order.
__global__ __launch_bounds__(256) void bwd_prep(BwdParams p) {
  const int64_t gt = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gt >> 4;
  const int ch = (int)(gt & 15);
  const int64_t nrows = (int64_t)p.B * p.L * p.Hq;
  float s = 0.f;
  if (row < nrows) {
    const uint4 a = ldg16(p.dO + row * D + 8 * ch);
    const uint4 b = ldg16(p.o + row * D + 8 * ch);
    const uint32_t* wa = reinterpret_cast<const uint32_t*>(&a);
    const uint32_t* wb = reinterpret_cast<const uint32_t*>(&b);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s += bf16_bits_to_f32(wa[e] & 0xffffu) * bf16_bits_to_f32(wb[e] & 0xffffu);
      s += bf16_bits_to_f32(wa[e] >> 16) * bf16_bits_to_f32(wb[e] >> 16);
    }
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
  if (row < nrows && ch == 0) {
    const int h = (int)(row % p.Hq);
    const int64_t bi = row / p.Hq;
    const int i = (int)(bi % p.L), b = (int)(bi / p.L);
    const int64_t o = ((int64_t)b * p.Hq + h) * p.L + i;
    p.dl[o] = make_float2(s, p.lse[o] * kLog2e);
  }
}

// ---------------------------------------------------------------------------
// dK / dV
constexpr int kKvNW = 4;                       // waves per workgroup (32 keys each)
constexpr int kKvNS = 3;                       // ring depth (query tiles)
constexpr int kKvStage = 2 * kTileBytes + 512; // Q tile, dO tile, 64 x (D, LSE*log2e)
constexpr size_t kDkdvSmem = (size_t)kKvNS * kKvStage;

__global__ __launch_bounds__(kKvNW * 64) void bwd_dkdv(BwdParams p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int L = p.L;
  const int nkt = (L + 32 * kKvNW - 1) / (32 * kKvNW);
  const int wid = xcd_remap(blockIdx.x, gridDim.x);
  const int kt = wid % nkt;
  const int bk = wid / nkt;
  const int kvh = bk % p.Hkv, b = bk / p.Hkv;
  const int k0 = kt * 32 * kKvNW;
  const int kw0 = k0 + 32 * wave;          // this wave's first key
  const int key = kw0 + col;               // this lane's key (B-operand column)
  const int qmin_key = (min(key, L - 1) / p.blk) * p.blk;   // first query that sees `key`
  const int qmin_w = (min(kw0, L - 1) / p.blk) * p.blk;     // first query that sees any wave key
  const int qmin_w_hi = (min(kw0 + 31, L - 1) / p.blk) * p.blk;
  const int q_first = ((min(k0, L - 1) / p.blk) * p.blk / 64) * 64;
  const int nqt = (L - q_first + 63) / 64;
  const int n_iter = p.G * nqt;
  const bool wave_live = kw0 < L;

  const int64_t kv_rs = (int64_t)p.Hkv * D, q_rs = (int64_t)p.Hq * D;

  // this wave's share of iteration `it`'s tiles: Q, dO rows and the (D, LSE) slice
  auto issue = [&](int it) {
    const uint32_t st = lds0 + (uint32_t)(it % kKvNS) * kKvStage;
    const int hq = kvh * p.G + it / nqt;
    const int q0 = q_first + (it % nqt) * 64;
    const uint16_t* qb = p.q + (int64_t)b * L * q_rs + (int64_t)hq * D;
    const uint16_t* dob = p.dO + (int64_t)b * L * q_rs + (int64_t)hq * D;
    tile_dma<kKvNW>(st, qb, q_rs, q0, L, wave, lane);
    tile_dma<kKvNW>(st + kTileBytes, dob, q_rs, q0, L, wave, lane);
    // 64 float2 = 512 bytes: lanes 0..31 of every wave copy the same slice, rows
    // q0 + 2l and q0 + 2l + 1 to slots 2l, 2l + 1.  When only the first row of a
    // pair exists, the second read runs 8 bytes into the next head's rows (or
    // into the workspace's 16 bytes of slack); lanes wholly past the end read
    // from row 0.  Query rows past the end are masked below.
    const float2* dlb = p.dl + ((int64_t)b * p.Hq + hq) * L;
    const int r2 = q0 + 2 * lane;
    if (lane < 32) lds_dma16(dlb + (r2 < L ? r2 : 0), st + 2 * kTileBytes);
  };
  for (int u = 0; u < kKvNS - 1 && u < n_iter; ++u) issue(u);

  bf16x8 kreg[8], vreg[8];
  {
    const int64_t off = ((int64_t)b * L + min(key, L - 1)) * kv_rs + (int64_t)kvh * D + 8 * half;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      kreg[t] = as_bf16x8(key < L ? ldg16(p.k + off + 16 * t) : make_uint4(0, 0, 0, 0));
      vreg[t] = as_bf16x8(key < L ? ldg16(p.v + off + 16 * t) : make_uint4(0, 0, 0, 0));
    }
  }
  vm_wait<0>();

  f32x16 dk_acc[4], dv_acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) { dk_acc[db][i] = 0.f; dv_acc[db][i] = 0.f; }

  // Per-lane LDS offsets within a stage: A-operand rows of Q / dO in sigma32
  // order (logical chunk 2*ds + half), and the transposed-read addresses of Q^T /
  // dO^T (as the forward's V^T reads).
  uint32_t raddr[8], taddr[8];
  {
    const int rrow = sigma32(col);
    const int rswz = tile_swz(rrow);
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) raddr[ds] = rrow * 256 + (((2 * ds + half) ^ rswz) << 4);
    tr32_bases(taddr, 0, lane);
  }
  const float c2 = p.scale_log2;

  for (int it = 0; it < n_iter; ++it) {
    {
      const int pending = min(kKvNS - 2, n_iter - 1 - it);
      constexpr int per = 2 * (16 / kKvNW) + 1;
      if (pending >= 1) vm_wait<per>();
      else vm_wait<0>();
    }
    __syncthreads();
    if (it + kKvNS - 1 < n_iter) issue(it + kKvNS - 1);
    const int q0 = q_first + (it % nqt) * 64;
    if (!wave_live || q0 + 64 <= qmin_w) continue;      // no query of the tile sees this wave's keys
    const uint32_t st = lds0 + (uint32_t)(it % kKvNS) * kKvStage;
    const uint32_t Qt = st, dOt = st + kTileBytes;
    const float2* dl_s = reinterpret_cast<const float2*>(reinterpret_cast<const char*>(smem) + (st - lds0) + 2 * kTileBytes);
    const bool partial = q0 < qmin_w_hi;
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      if (q0 + 32 * qs + 32 <= qmin_w) continue;
      f32x16 s_acc, dp_acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) { s_acc[i] = 0.f; dp_acc[i] = 0.f; }
#pragma unroll
      for (int ds = 0; ds < 8; ++ds) {
        s_acc = mfma_32x32x16(lds_read_b128(Qt + 32 * qs * 256 + raddr[ds]), kreg[ds], s_acc);
        dp_acc = mfma_32x32x16(lds_read_b128(dOt + 32 * qs * 256 + raddr[ds]), vreg[ds], dp_acc);
      }
      // entry i of this lane holds query q0 + 32*qs + 16*(i/8) + 8*half + (i%8)
      float pv[16], dsv[16];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int qb0 = 32 * qs + 16 * j + 8 * half;
        const float4* src = reinterpret_cast<const float4*>(dl_s + qb0);
        float dd[8], ll[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float4 w = src[e];
          dd[2 * e] = w.x; ll[2 * e] = w.y; dd[2 * e + 1] = w.z; ll[2 * e + 1] = w.w;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = 8 * j + e;
          float pe = exp2_fast(__builtin_fmaf(s_acc[i], c2, -ll[e]));
          if (partial && (q0 + qb0 + e) < qmin_key) pe = 0.f;
          if (q0 + qb0 + e >= L) pe = 0.f;
          pv[i] = pe;
          dsv[i] = pe * (dp_acc[i] - dd[e]);
        }
      }
      const bf16x8 pb0 = pack_bf16x8(pv), pb1 = pack_bf16x8(pv + 8);
      const bf16x8 sb0 = pack_bf16x8(dsv), sb1 = pack_bf16x8(dsv + 8);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int s0 = 2 * qs;   // 16-row k-steps 2qs, 2qs+1 of the 64-row tile
        const bf16x8 dto0 = cat_i16x4(lds_read_tr16(dOt + taddr[tr32_idx(db, s0, 0)] + tr32_off(s0, 0)),
                                      lds_read_tr16(dOt + taddr[tr32_idx(db, s0, 1)] + tr32_off(s0, 1)));
        const bf16x8 dto1 = cat_i16x4(lds_read_tr16(dOt + taddr[tr32_idx(db, s0 + 1, 0)] + tr32_off(s0 + 1, 0)),
                                      lds_read_tr16(dOt + taddr[tr32_idx(db, s0 + 1, 1)] + tr32_off(s0 + 1, 1)));
        dv_acc[db] = mfma_32x32x16(dto0, pb0, dv_acc[db]);
        dv_acc[db] = mfma_32x32x16(dto1, pb1, dv_acc[db]);
        const bf16x8 qt0 = cat_i16x4(lds_read_tr16(Qt + taddr[tr32_idx(db, s0, 0)] + tr32_off(s0, 0)),
                                     lds_read_tr16(Qt + taddr[tr32_idx(db, s0, 1)] + tr32_off(s0, 1)));
        const bf16x8 qt1 = cat_i16x4(lds_read_tr16(Qt + taddr[tr32_idx(db, s0 + 1, 0)] + tr32_off(s0 + 1, 0)),
                                     lds_read_tr16(Qt + taddr[tr32_idx(db, s0 + 1, 1)] + tr32_off(s0 + 1, 1)));
        dk_acc[db] = mfma_32x32x16(qt0, sb0, dk_acc[db]);
        dk_acc[db] = mfma_32x32x16(qt1, sb1, dk_acc[db]);
      }
    }
  }

  if (key >= L) return;
  const int64_t off = ((int64_t)b * L + key) * kv_rs + (int64_t)kvh * D;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = 32 * db + 8 * j + 4 * half;
      const f32x16& a = dk_acc[db];
      const f32x16& c = dv_acc[db];
      *reinterpret_cast<uint2*>(p.dk + off + d0) =
          make_uint2(pack_bf16x2(a[4 * j] * p.scale, a[4 * j + 1] * p.scale),
                     pack_bf16x2(a[4 * j + 2] * p.scale, a[4 * j + 3] * p.scale));
      *reinterpret_cast<uint2*>(p.dv + off + d0) =
          make_uint2(pack_bf16x2(c[4 * j], c[4 * j + 1]), pack_bf16x2(c[4 * j + 2], c[4 * j + 3]));
    }
}

// ---------------------------------------------------------------------------
// dQ
constexpr int kDqNW = 8;
constexpr int kDqStage = 2 * kTileBytes;       // K tile, V tile
constexpr size_t kDqSmem = 2 * (size_t)kDqStage;

__global__ __launch_bounds__(kDqNW * 64) void bwd_dq(BwdParams p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int L = p.L;
  const int qtiles = (L + 32 * kDqNW - 1) / (32 * kDqNW);
  const int wid = xcd_remap(blockIdx.x, gridDim.x);
  const int per_group = qtiles * p.G;
  const int grp = wid / per_group, rem = wid - grp * per_group;
  const int b = grp / p.Hkv, kvh = grp - b * p.Hkv;
  const int qt = qtiles - 1 - rem / p.G;
  const int hq = kvh * p.G + rem % p.G;
  const int wg_r0 = qt * 32 * kDqNW, r0 = wg_r0 + 32 * wave;
  const int kend_wg = key_limit(min(wg_r0 + 32 * kDqNW, L) - 1, L, p.blk);
  const int ntiles = (kend_wg + 63) / 64;
  const bool active = r0 < L;
  const int kend_lo = active ? key_limit(r0, L, p.blk) : 0;
  const int kend_hi = active ? key_limit(min(r0 + 31, L - 1), L, p.blk) : 0;
  const int qrow = r0 + col;
  const int kq = key_limit(min(qrow, L - 1), L, p.blk);

  const int64_t q_rs = (int64_t)p.Hq * D, kv_rs = (int64_t)p.Hkv * D;
  const uint16_t* kb = p.k + (int64_t)b * L * kv_rs + (int64_t)kvh * D;
  const uint16_t* vb = p.v + (int64_t)b * L * kv_rs + (int64_t)kvh * D;
  auto issue = [&](int t) {
    const uint32_t st = lds0 + (uint32_t)(t & 1) * kDqStage;
    tile_dma<kDqNW>(st, kb, kv_rs, t * 64, kend_wg, wave, lane);
    tile_dma<kDqNW>(st + kTileBytes, vb, kv_rs, t * 64, kend_wg, wave, lane);
  };
  if (ntiles > 0) issue(0);

  bf16x8 qreg[8], doreg[8];
  {
    const int64_t off = ((int64_t)b * L + min(qrow, L - 1)) * q_rs + (int64_t)hq * D + 8 * half;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      qreg[t] = as_bf16x8(qrow < L ? ldg16(p.q + off + 16 * t) : make_uint4(0, 0, 0, 0));
      doreg[t] = as_bf16x8(qrow < L ? ldg16(p.dO + off + 16 * t) : make_uint4(0, 0, 0, 0));
    }
  }
  const float2 dl = p.dl[((int64_t)b * p.Hq + hq) * L + min(qrow, L - 1)];
  const float Dq = dl.x, nlse2 = -dl.y;
  vm_wait<0>();

  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

  uint32_t raddr[8], taddr[8];
  {
    const int rrow = sigma32(col);
    const int rswz = tile_swz(rrow);
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) raddr[ds] = lds0 + rrow * 256 + (((2 * ds + half) ^ rswz) << 4);
    tr32_bases(taddr, lds0, lane);
  }
  const float c2 = p.scale_log2;

  auto step = [&](auto stage_c, int t) {
    constexpr uint32_t so = decltype(stage_c)::value * kDqStage;
    vm_wait<0>();
    __syncthreads();
    if (t + 1 < ntiles) issue(t + 1);
    const int key0 = t * 64;
    if (!active || key0 >= kend_hi) return;
    const bool partial = key0 + 64 > kend_lo;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      f32x16 s_acc, dp_acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) { s_acc[i] = 0.f; dp_acc[i] = 0.f; }
#pragma unroll
      for (int ds = 0; ds < 8; ++ds) {
        s_acc = mfma_32x32x16(lds_read_b128(raddr[ds] + so + h2 * 32 * 256), qreg[ds], s_acc);
        dp_acc = mfma_32x32x16(lds_read_b128(raddr[ds] + so + kTileBytes + h2 * 32 * 256), doreg[ds], dp_acc);
      }
      // entry i holds key key0 + 32*h2 + 16*(i/8) + 8*half + (i%8)
      bf16x8 sb[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float dsv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = 8 * j + e;
          float pe = exp2_fast(__builtin_fmaf(s_acc[i], c2, nlse2));
          if (partial && key0 + 32 * h2 + 16 * j + 8 * half + e >= kq) pe = 0.f;
          dsv[e] = pe * (dp_acc[i] - Dq);
        }
        sb[j] = pack_bf16x8(dsv);
      }
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int s4 = 2 * h2 + j;
          const i16x4 lo = lds_read_tr16(taddr[tr32_idx(db, s4, 0)] + so + tr32_off(s4, 0));
          const i16x4 hi = lds_read_tr16(taddr[tr32_idx(db, s4, 1)] + so + tr32_off(s4, 1));
          acc[db] = mfma_32x32x16(cat_i16x4(lo, hi), sb[j], acc[db]);
        }
    }
  };
  for (int t = 0; t < ntiles; t += 2) {
    step(std::integral_constant<int, 0>(), t);
    if (t + 1 < ntiles) step(std::integral_constant<int, 1>(), t + 1);
  }

  if (!active || qrow >= L) return;
  uint16_t* out = p.dq + ((int64_t)b * L + qrow) * q_rs + (int64_t)hq * D;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x16& a = acc[db];
      *reinterpret_cast<uint2*>(out + 32 * db + 8 * j + 4 * half) =
          make_uint2(pack_bf16x2(a[4 * j] * p.scale, a[4 * j + 1] * p.scale),
                     pack_bf16x2(a[4 * j + 2] * p.scale, a[4 * j + 3] * p.scale));
    }
}

}  // namespace

size_t attn_bwd_workspace_bytes(int batch, int seqlen, int n_q_heads) {
  return (size_t)batch * n_q_heads * seqlen * sizeof(float2) + 16;
}

hipError_t launch_attn_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                const void* d_o, void* dq, void* dk, void* dv, void* ws, const AttnShape& s,
                                hipStream_t st) {
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [] {
    attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_dkdv),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)kDkdvSmem);
    if (attr_err == hipSuccess)
      attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_dq),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kDqSmem);
  });
  if (attr_err != hipSuccess) return attr_err;
  BwdParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<const uint16_t*>(o);
  p.dO = static_cast<const uint16_t*>(d_o);
  p.lse = lse;
  p.dl = static_cast<float2*>(ws);
  p.dq = static_cast<uint16_t*>(dq);
  p.dk = static_cast<uint16_t*>(dk);
  p.dv = static_cast<uint16_t*>(dv);
  p.B = s.batch;
  p.L = s.seqlen;
  p.Hq = s.n_q_heads;
  p.Hkv = s.n_kv_heads;
  p.G = s.n_q_heads / s.n_kv_heads;
  p.blk = s.block_size;
  p.scale = s.scale;
  p.scale_log2 = s.scale * kLog2e;
  const long long rows = (long long)s.batch * s.seqlen * s.n_q_heads;
  hipLaunchKernelGGL(bwd_prep, dim3((unsigned)((rows * 16 + 255) / 256)), dim3(256), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long nk = (long long)s.batch * s.n_kv_heads * ((s.seqlen + 32 * kKvNW - 1) / (32 * kKvNW));
  hipLaunchKernelGGL(bwd_dkdv, dim3((unsigned)nk), dim3(kKvNW * 64), kDkdvSmem, st, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long nq = (long long)s.batch * s.n_q_heads * ((s.seqlen + 32 * kDqNW - 1) / (32 * kDqNW));
  hipLaunchKernelGGL(bwd_dq, dim3((unsigned)nq), dim3(kDqNW * 64), kDqSmem, st, p);
  return hipGetLastError();
}

}  // namespace bd
