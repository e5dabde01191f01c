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
//   bwd_dsum  D for every (batch, head, row).
//   bwd_dkdv  workgroup = 4 waves = 128 consecutive keys of one (batch, kv
//             head); each wave owns 32 keys with K and V in registers and walks
//             the query tiles (64 rows, both layouts staged in LDS) of every
//             query head of the group, from the first query that can see its
//             keys to the end of the sequence.  Per 32-query slice:
//               S  = Q K^T, dP = dO V^T        (A = Q / dO rows from LDS)
//               dV^T += dO^T P, dK^T += Q^T dS (A = dO^T / Q^T from LDS,
//                                               B = P / dS from the accumulator)
//             The query rows of the A operand are read in sigma32 order so that
//             the S and dP accumulators are already in B-operand layout.
//   bwd_dq    workgroup = 4 waves = 128 query rows of one (batch, q head), as
//             the forward: S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T, over the
//             key tiles its rows can see (K in both layouts and V in LDS).
#include "bd_device.hpp"
#include "bd_kernels.hpp"

#include <mutex>

namespace bd {
namespace {

constexpr int D = 128;
constexpr int RP = D + 8;      // pitch of a row-layout tile [rows][D]
constexpr int TP = 64 + 8;     // pitch of a transposed tile [D][64 rows]
constexpr int ROW_TILE = 64 * RP;
constexpr int T_TILE = D * TP;
constexpr int kThreads = 256;

struct BwdParams {
  const uint16_t *q, *k, *v, *o, *dO;
  const float* lse;
  float* Dsum;
  uint16_t *dq, *dk, *dv;
  int B, L, Hq, Hkv, G, blk;
  float scale, scale_log2;
};

__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

// A 64-row x 128-column bf16 tile in flight: thread t holds rows 4*(t%16)..+3,
// columns 8*(t/16)..+7 (four 16-byte loads).
struct Tile64 {
  uint4 r[4];
};

template <typename RowPtr>
__device__ __forceinline__ void tile_load(Tile64& t, const RowPtr& row_ptr, int row0, int nrows, int tid) {
  const int rq = tid & 15, ch = tid >> 4;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r = row0 + 4 * rq + e;
    t.r[e] = r < nrows ? ldg16(row_ptr(r) + 8 * ch) : make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ void tile_store_rows(const Tile64& t, uint16_t* dst, int tid) {
  const int rq = tid & 15, ch = tid >> 4;
#pragma unroll
  for (int e = 0; e < 4; ++e) *reinterpret_cast<uint4*>(dst + (4 * rq + e) * RP + 8 * ch) = t.r[e];
}

__device__ __forceinline__ void tile_store_transposed(const Tile64& t, uint16_t* dst, int tid) {
  const int rq = tid & 15, ch = tid >> 4;
  const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&t.r[0]);
  const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&t.r[1]);
  const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&t.r[2]);
  const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&t.r[3]);
  uint16_t* base = dst + (8 * ch) * TP + 4 * rq;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    *reinterpret_cast<uint2*>(base + (2 * e) * TP) = make_uint2(lo_pair(w0[e], w1[e]), lo_pair(w2[e], w3[e]));
    *reinterpret_cast<uint2*>(base + (2 * e + 1) * TP) = make_uint2(hi_pair(w0[e], w1[e]), hi_pair(w2[e], w3[e]));
  }
}

// ---------------------------------------------------------------------------
// D = rowsum(dO * O): 16 lanes per row, rows of [B, L, Hq] in memory order.
__global__ __launch_bounds__(kThreads) void bwd_dsum(BwdParams p) {
  const int64_t gt = (int64_t)blockIdx.x * kThreads + threadIdx.x;
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
    p.Dsum[((int64_t)b * p.Hq + h) * p.L + i] = s;
  }
}

// ---------------------------------------------------------------------------
constexpr size_t kDkdvSmem = (2 * ROW_TILE + 2 * T_TILE) * sizeof(uint16_t) + 2 * 64 * sizeof(float);

__global__ __launch_bounds__(kThreads) void bwd_dkdv(BwdParams p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t* Qs = smem;                     // [64][RP]   rows = queries
  uint16_t* dOs = Qs + ROW_TILE;           // [64][RP]
  uint16_t* Qt = dOs + ROW_TILE;           // [D][TP]    rows = head dim
  uint16_t* dOt = Qt + T_TILE;             // [D][TP]
  float* lse2_s = reinterpret_cast<float*>(dOt + T_TILE);  // [64] lse * log2(e)
  float* D_s = lse2_s + 64;                                // [64]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int L = p.L;
  const int nkt = (L + 127) / 128;
  const int wid = xcd_remap(blockIdx.x, gridDim.x);
  const int kt = wid % nkt;
  const int bk = wid / nkt;
  const int kvh = bk % p.Hkv, b = bk / p.Hkv;
  const int k0 = kt * 128;
  const int kw0 = k0 + 32 * wave;          // this wave's first key
  const int key = kw0 + col;               // this lane's key (B-operand column)
  const int qmin_key = (min(key, L - 1) / p.blk) * p.blk;   // first query that sees `key`
  const int qmin_w = (min(kw0, L - 1) / p.blk) * p.blk;     // first query that sees any wave key
  const int qmin_w_hi = (min(kw0 + 31, L - 1) / p.blk) * p.blk;
  const int q_first = ((min(k0, L - 1) / p.blk) * p.blk / 64) * 64;
  const int nqt = (L - q_first + 63) / 64;

  const int64_t kv_rs = (int64_t)p.Hkv * D, q_rs = (int64_t)p.Hq * D;
  bf16x8 kreg[8], vreg[8];
  {
    const int64_t off = ((int64_t)b * L + key) * kv_rs + (int64_t)kvh * D + 8 * half;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      kreg[t] = as_bf16x8(key < L ? ldg16(p.k + off + 16 * t) : make_uint4(0, 0, 0, 0));
      vreg[t] = as_bf16x8(key < L ? ldg16(p.v + off + 16 * t) : make_uint4(0, 0, 0, 0));
    }
  }
  f32x16 dk_acc[4], dv_acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) { dk_acc[db][i] = 0.f; dv_acc[db][i] = 0.f; }

  const int arow = sigma32(col);
  const int n_iter = p.G * nqt;
  Tile64 tq, tdo;
  float pre_lse = 0.f, pre_D = 0.f;
  auto prefetch = [&](int it) {
    const int hq = kvh * p.G + it / nqt;
    const int q0 = q_first + (it % nqt) * 64;
    const uint16_t* qb = p.q + (int64_t)b * L * q_rs + (int64_t)hq * D;
    const uint16_t* db_ = p.dO + (int64_t)b * L * q_rs + (int64_t)hq * D;
    tile_load(tq, [&](int r) { return qb + r * q_rs; }, q0, L, tid);
    tile_load(tdo, [&](int r) { return db_ + r * q_rs; }, q0, L, tid);
    if (tid < 64) {
      const int qi = q0 + tid;
      const int64_t s = ((int64_t)b * p.Hq + hq) * L + qi;
      pre_lse = qi < L ? p.lse[s] * kLog2e : __builtin_huge_valf();
      pre_D = qi < L ? p.Dsum[s] : 0.f;
    }
  };

  prefetch(0);
  for (int it = 0; it < n_iter; ++it) {
    const int q0 = q_first + (it % nqt) * 64;
    __syncthreads();   // previous tile fully consumed
    tile_store_rows(tq, Qs, tid);
    tile_store_rows(tdo, dOs, tid);
    tile_store_transposed(tq, Qt, tid);
    tile_store_transposed(tdo, dOt, tid);
    if (tid < 64) { lse2_s[tid] = pre_lse; D_s[tid] = pre_D; }
    __syncthreads();
    if (it + 1 < n_iter) prefetch(it + 1);

    if (q0 + 64 <= qmin_w || kw0 >= L) continue;      // no query of the tile sees this wave's keys
    const bool partial = q0 < qmin_w_hi;
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      if (q0 + 32 * qs + 32 <= qmin_w) continue;
      f32x16 s_acc, dp_acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) { s_acc[i] = 0.f; dp_acc[i] = 0.f; }
      const uint16_t* qa = Qs + (32 * qs + arow) * RP + 8 * half;
      const uint16_t* da = dOs + (32 * qs + arow) * RP + 8 * half;
#pragma unroll
      for (int ds = 0; ds < 8; ++ds) {
        s_acc = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(qa + 16 * ds), kreg[ds], s_acc);
        dp_acc = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(da + 16 * ds), vreg[ds], dp_acc);
      }
      // entry i of this lane holds query q0 + 32*qs + 16*(i/8) + 8*half + (i%8)
      float pv[16], dsv[16];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int qb0 = 32 * qs + 16 * j + 8 * half;
        const float4 l0 = *reinterpret_cast<const float4*>(lse2_s + qb0);
        const float4 l1 = *reinterpret_cast<const float4*>(lse2_s + qb0 + 4);
        const float4 d0 = *reinterpret_cast<const float4*>(D_s + qb0);
        const float4 d1 = *reinterpret_cast<const float4*>(D_s + qb0 + 4);
        const float lv[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
        const float dv8[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = 8 * j + e;
          float pe = exp2_fast(s_acc[i] * p.scale_log2 - lv[e]);
          if (partial && (q0 + qb0 + e) < qmin_key) pe = 0.f;
          pv[i] = pe;
          dsv[i] = pe * (dp_acc[i] - dv8[e]);
        }
      }
      const bf16x8 pb0 = pack_bf16x8(pv), pb1 = pack_bf16x8(pv + 8);
      const bf16x8 sb0 = pack_bf16x8(dsv), sb1 = pack_bf16x8(dsv + 8);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const uint16_t* dta = dOt + (32 * db + col) * TP + 32 * qs + 8 * half;
        const uint16_t* qta = Qt + (32 * db + col) * TP + 32 * qs + 8 * half;
        dv_acc[db] = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(dta), pb0, dv_acc[db]);
        dv_acc[db] = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(dta + 16), pb1, dv_acc[db]);
        dk_acc[db] = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(qta), sb0, dk_acc[db]);
        dk_acc[db] = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(qta + 16), sb1, dk_acc[db]);
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
constexpr size_t kDqSmem = 2 * (2 * ROW_TILE + T_TILE) * sizeof(uint16_t);

__global__ __launch_bounds__(kThreads) void bwd_dq(BwdParams p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  // per buffer: K rows [64][RP], V rows [64][RP], K^T [D][TP]
  constexpr int BUF = 2 * ROW_TILE + T_TILE;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int L = p.L;
  const int qtiles = (L + 127) / 128;
  const int wid = xcd_remap(blockIdx.x, gridDim.x);
  const int per_group = qtiles * p.G;
  const int grp = wid / per_group, rem = wid - grp * per_group;
  const int b = grp / p.Hkv, kvh = grp - b * p.Hkv;
  const int qt = qtiles - 1 - rem / p.G;
  const int hq = kvh * p.G + rem % p.G;
  const int wg_r0 = qt * 128, r0 = wg_r0 + 32 * wave;
  const int kend_wg = key_limit(min(wg_r0 + 128, L) - 1, L, p.blk);
  const int ntiles = (kend_wg + 63) / 64;
  const bool active = r0 < L;
  const int kend_lo = active ? key_limit(r0, L, p.blk) : 0;
  const int kend_hi = active ? key_limit(min(r0 + 31, L - 1), L, p.blk) : 0;
  const int qrow = r0 + col;
  const int kq = key_limit(min(qrow, L - 1), L, p.blk);

  const int64_t q_rs = (int64_t)p.Hq * D, kv_rs = (int64_t)p.Hkv * D;
  const uint16_t* kb = p.k + (int64_t)b * L * kv_rs + (int64_t)kvh * D;
  const uint16_t* vb = p.v + (int64_t)b * L * kv_rs + (int64_t)kvh * D;
  bf16x8 qreg[8], doreg[8];
  {
    const int64_t off = ((int64_t)b * L + qrow) * q_rs + (int64_t)hq * D + 8 * half;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      qreg[t] = as_bf16x8(qrow < L ? ldg16(p.q + off + 16 * t) : make_uint4(0, 0, 0, 0));
      doreg[t] = as_bf16x8(qrow < L ? ldg16(p.dO + off + 16 * t) : make_uint4(0, 0, 0, 0));
    }
  }
  const int64_t srow = ((int64_t)b * p.Hq + hq) * L + min(qrow, L - 1);
  const float lse2 = p.lse[srow] * kLog2e;
  const float Dq = p.Dsum[srow];

  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

  Tile64 tk, tv;
  auto kptr = [&](int r) { return kb + r * kv_rs; };
  auto vptr = [&](int r) { return vb + r * kv_rs; };
  tile_load(tk, kptr, 0, kend_wg, tid);
  tile_load(tv, vptr, 0, kend_wg, tid);
  tile_store_rows(tk, smem, tid);
  tile_store_rows(tv, smem + ROW_TILE, tid);
  tile_store_transposed(tk, smem + 2 * ROW_TILE, tid);
  __syncthreads();
  const int arow = sigma32(col);

  for (int t = 0; t < ntiles; ++t) {
    uint16_t* cur = smem + (t & 1) * BUF;
    if (t + 1 < ntiles) {
      tile_load(tk, kptr, (t + 1) * 64, kend_wg, tid);
      tile_load(tv, vptr, (t + 1) * 64, kend_wg, tid);
    }
    const int key0 = t * 64;
    if (active && key0 < kend_hi) {
      const uint16_t* Ks = cur;
      const uint16_t* Vs = cur + ROW_TILE;
      const uint16_t* Kt = cur + 2 * ROW_TILE;
      f32x16 s_acc[2], dp_acc[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
        for (int i = 0; i < 16; ++i) { s_acc[h2][i] = 0.f; dp_acc[h2][i] = 0.f; }
        const uint16_t* ka = Ks + (32 * h2 + arow) * RP + 8 * half;
        const uint16_t* va = Vs + (32 * h2 + arow) * RP + 8 * half;
#pragma unroll
        for (int ds = 0; ds < 8; ++ds) {
          s_acc[h2] = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(ka + 16 * ds), qreg[ds], s_acc[h2]);
          dp_acc[h2] = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(va + 16 * ds), doreg[ds], dp_acc[h2]);
        }
      }
      const bool partial = key0 + 64 > kend_lo;
      bf16x8 sb[4];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          float dsv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int i = 8 * j + e;
            float pe = exp2_fast(s_acc[h2][i] * p.scale_log2 - lse2);
            if (partial && key0 + 32 * h2 + 16 * j + 8 * half + e >= kq) pe = 0.f;
            dsv[e] = pe * (dp_acc[h2][i] - Dq);
          }
          sb[2 * h2 + j] = pack_bf16x8(dsv);
        }
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const uint16_t* ka = Kt + (32 * db + col) * TP + 8 * half;
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
          acc[db] = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(ka + 16 * s4), sb[s4], acc[db]);
      }
    }
    if (t + 1 < ntiles) {
      uint16_t* nxt = smem + ((t + 1) & 1) * BUF;
      tile_store_rows(tk, nxt, tid);
      tile_store_rows(tv, nxt + ROW_TILE, tid);
      tile_store_transposed(tk, nxt + 2 * ROW_TILE, tid);
    }
    __syncthreads();
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
  return (size_t)batch * n_q_heads * seqlen * sizeof(float);
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
  p.Dsum = static_cast<float*>(ws);
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
  hipLaunchKernelGGL(bwd_dsum, dim3((unsigned)((rows * 16 + kThreads - 1) / kThreads)), dim3(kThreads), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long nk = (long long)s.batch * s.n_kv_heads * ((s.seqlen + 127) / 128);
  hipLaunchKernelGGL(bwd_dkdv, dim3((unsigned)nk), dim3(kThreads), kDkdvSmem, st, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long nq = (long long)s.batch * s.n_q_heads * ((s.seqlen + 127) / 128);
  hipLaunchKernelGGL(bwd_dq, dim3((unsigned)nq), dim3(kThreads), kDqSmem, st, p);
  return hipGetLastError();
}

}  // namespace bd
