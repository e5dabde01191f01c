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
//   bwd_prep  per (batch, head, row): -D = -rowsum(dO * O) and -LSE / scale,
//             two arrays [B, Hq, Lp] (rows padded to a multiple of 64 with
//             zeros), the starting values of the dP and S accumulators.
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

#include <algorithm>
#include <climits>
#include <mutex>
#include <type_traits>

namespace bd {
namespace {

constexpr int D = 128;
constexpr int kTileBytes = 64 * D * 2;   // 16 KB: one 64-row bf16 tile

struct BwdParams {
  const uint16_t *q, *k, *v, *o, *dO;
  const float* lse;
  float* negD;         // [B, Hq, Lp]: -D = -rowsum(dO * O); 0 in the padding rows
  float* nlse;         // [B, Hq, Lp]: -LSE / scale; 0 in the padding rows
  uint16_t *dq, *dk, *dv;
  unsigned* queue;     // [8]: next unclaimed item of each XCD's list (zeroed by bwd_prep)
  int B, L, Lp, Hq, Hkv, G, blk;
  float scale, scale_log2;
};

// ---------------------------------------------------------------------------
// 16 lanes per row, rows of [B, L, Hq] in memory order.  The first
// B * Hq * (Lp - L) threads also zero the padding rows.
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
    const int64_t bh = (int64_t)b * p.Hq + h;
    p.negD[bh * p.Lp + i] = -s;
    p.nlse[bh * p.Lp + i] = -p.lse[bh * p.L + i] / p.scale;
  }
  if (gt < 8) p.queue[gt] = 0u;
  const int pad = p.Lp - p.L;
  if (gt < (int64_t)p.B * p.Hq * pad) {
    const int64_t bh = gt / pad;
    const int64_t o = bh * p.Lp + p.L + (gt - bh * pad);
    p.negD[o] = 0.f;
    p.nlse[o] = 0.f;
  }
}

// ---------------------------------------------------------------------------
// dK / dV
//
// Workgroup = 8 waves = 4 pairs; pair g owns keys k0 + 32 g .. + 31 of one
// (batch, kv head) and walks the 64-row query tiles of every query head of the
// group from the first query that can see the workgroup's keys.  The two waves
// of a pair sit on one SIMD and split the work by kind:
//   score wave     K and V of the pair's keys in registers;
//                  S = Q K^T, dP = dO V^T (A = Q / dO rows from LDS, sigma32
//                  order; the accumulators start from -LSE/scale and -D of
//                  their query rows, so they end as S - LSE/scale, dP - D), then
//                  P = exp2((S - LSE/scale) scale log2 e), dS = P (dP - D) on
//                  the vector ALU, packed to bf16;
//   gradient wave  dV^T += dO^T P, dK^T += Q^T dS (A = dO^T / Q^T by transposed
//                  LDS reads, B = P / dS as the score wave packed them, read
//                  from an LDS exchange area), the dK / dV accumulators; it
//                  also issues the tile loads.
// Every tile takes two phases ended by workgroup barriers:
//   phase A(t)  score: store P / dS of tile t-1 to the exchange area, then the
//                      products of tile t;
//               gradient: issue the loads of tile t+1 (global -> LDS);
//   phase B(t)  score: the vector work of tile t (P / dS kept in registers);
//               gradient: the products of tile t-1, then wait for its loads.
// So the vector work of one wave overlaps the products of the other on the
// same SIMD, and products never wait on memory.  Ring stages: tile t+1 goes to
// the stage of tile t-2, whose last reads (the gradient products of t-2) ended
// in B(t-1).  (Measured alternatives: a double exchange area with half of the
// gradient products moved into phase A, 15-20 % slower; reading further ahead
// than four products, no change.)
constexpr int kKvNW = 8;                       // waves per workgroup
constexpr int kKvPairs = kKvNW / 2;            // 32 keys each
constexpr int kKvKeys = 32 * kKvPairs;         // keys per workgroup
constexpr int kKvNS = 3;                       // ring depth (query tiles)
// LDS: the Q tiles of the three stages, then their dO tiles, then their
// slices of -D and -LSE/scale (64 floats each), then the exchange areas of the
// pairs and the SIMD ids.  Every read is a per-lane base register plus an
// immediate offset below 64 KB (stage, slice and step are compile-time
// constants).
constexpr uint32_t kQRing = 0;
constexpr uint32_t kDORing = kQRing + kKvNS * kTileBytes;
constexpr uint32_t kDLRing = kDORing + kKvNS * kTileBytes;
constexpr uint32_t kXchOff = kDLRing + kKvNS * 512;
constexpr uint32_t kXchPair = 8 * 64 * 16;     // 8 operands of 16 bytes per lane
constexpr uint32_t kKvIdsOff = kXchOff + kKvPairs * kXchPair;
constexpr size_t kDkdvSmem = kKvIdsOff + 64;

// Products whose LDS operands are read ahead (a tuning knob of the build).
#ifndef BD_BWD_LOOK
#define BD_BWD_LOOK 4
#endif

template <int S>
using Stage = std::integral_constant<int, S>;

// Hide how a per-lane LDS base was derived, so that the compiler keeps it as
// its own register and every read from it fits the 16-bit offset field
// (otherwise it rebuilds it from another base plus an offset above 64 KB,
// one extra add per read).
__device__ __forceinline__ void opaque(uint32_t& x) { asm volatile("" : "+v"(x)); }

// Work item wid: the 128 keys kt * 128 .. of (batch, KV head) wid / nkt.
__device__ __forceinline__ void dkdv_item(const BwdParams& p, const int wid) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int L = p.L;
  const int nkt = (L + kKvKeys - 1) / kKvKeys;
  const int kt = wid % nkt;
  const int bk = wid / nkt;
  const int kvh = bk % p.Hkv, b = bk / p.Hkv;
  const int k0 = kt * kKvKeys;

  // Pairs: the two waves the hardware placed on one SIMD (HW_ID bits 5:4),
  // the first (by wave index) the score wave.  Otherwise waves 0-3 score and
  // 4-7 compute gradients, pair = wave % 4; the pairing only affects speed.
  const int simd = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_s_getreg((1 << 11) | (4 << 6) | 4) & 3);
  typedef __attribute__((address_space(3))) int lds_int;
  lds_int* simd_of = reinterpret_cast<lds_int*>((uintptr_t)(lds0 + kKvIdsOff));
  if (lane == 0) simd_of[wave] = simd;
  __syncthreads();
  int ids[kKvNW];
#pragma unroll
  for (int w = 0; w < kKvNW; ++w) ids[w] = __builtin_amdgcn_readfirstlane(simd_of[w]);
  bool paired = true;
  int rank = 0;
#pragma unroll
  for (int w = 0; w < kKvNW; ++w) {
    int same = 0;
#pragma unroll
    for (int x = 0; x < kKvNW; ++x) same += (ids[x] == ids[w]);
    paired = paired && same == 2;
    rank += (w < wave && ids[w] == simd);
  }
  const bool scorer = __builtin_amdgcn_readfirstlane(paired ? rank == 0 : wave < kKvPairs);
  const int gp = __builtin_amdgcn_readfirstlane(paired ? simd : (wave & (kKvPairs - 1)));

  const int kw0 = k0 + 32 * gp;            // the pair's first key
  const int key = kw0 + col;               // this lane's key (B-operand column)
  const int qmin_key = (min(key, L - 1) / p.blk) * p.blk;   // first query that sees `key`
  const int qmin_w = (min(kw0, L - 1) / p.blk) * p.blk;     // first query that sees any of the pair's keys
  const int qmin_w_hi = (min(kw0 + 31, L - 1) / p.blk) * p.blk;
  const int q_first = ((min(k0, L - 1) / p.blk) * p.blk / 64) * 64;
  const int nqt = (L - q_first + 63) / 64;
  const int n_iter = p.G * nqt;
  const bool pair_live = kw0 < L;
  const int64_t kv_rs = (int64_t)p.Hkv * D, q_rs = (int64_t)p.Hq * D;

  auto tile_q0 = [&](int it) __attribute__((always_inline)) { return q_first + (it % nqt) * 64; };
  // a tile some query of which sees the pair's keys (the same test in both waves of the pair)
  auto live = [&](int it) __attribute__((always_inline)) { return pair_live && tile_q0(it) + 64 > qmin_w; };

  uint32_t xch = lds0 + kXchOff + gp * kXchPair + lane * 16;   // + 1024 * operand
  opaque(xch);
  const float c2 = p.scale_log2;

  if (scorer) {
    // ------------------------------------------------------------ score wave
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
    __syncthreads();   // the gradient waves' loads of tile 0 are complete

    // A-operand rows of Q / dO in sigma32 order (logical chunk 2*ds + half),
    // stage 0; the -D / -LSE/scale slots of this lane's first query row.
    uint32_t rq[8], rdo[8];
    {
      const int rrow = sigma32(col);
      const int rswz = tile_swz(rrow);
#pragma unroll
      for (int ds = 0; ds < 8; ++ds) {
        rq[ds] = lds0 + kQRing + rrow * 256 + (((2 * ds + half) ^ rswz) << 4);
        rdo[ds] = rq[ds] - kQRing + kDORing;
        opaque(rdo[ds]);
      }
    }
    uint32_t dl_lane = lds0 + kDLRing + 4 * 8 * half;   // + 256 for -LSE/scale
    opaque(dl_lane);
    f32x16 acc[4];      // S of slices 0, 1 and dP of slices 0, 1: acc[2 * which + qs]
    bf16x8 pk[8];       // P / dS of the last tile: operand 4 qs + 2 kind + j (k-step 2 qs + j)

    // Products of a tile in stage S: step i multiplies d-step i/4 of slice
    // (i/2)%2, S (i even) or dP (i odd), so each accumulator recurs every 4
    // products; each step's operand row is read kLook steps ahead.  The
    // accumulators start from -LSE/scale (S) and -D (dP) of their query rows:
    // entry i of slice qs is query 32 qs + 16 (i/8) + 8 half + (i%8), so each
    // starting value is four 16-byte reads of the tile's slices.
    auto products = [&](auto sc) __attribute__((always_inline)) {
      constexpr uint32_t so = decltype(sc)::value * kTileBytes;
      constexpr uint32_t sl = decltype(sc)::value * 512;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int qs = a & 1;
        const uint32_t base = dl_lane + sl + (a < 2 ? 256u : 0u) + 4 * 32 * qs;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const f32x4 w = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(
              (uintptr_t)(base + 4 * 16 * (r >> 1) + 16 * (r & 1)));
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[a][4 * r + e] = w[e];
        }
      }
      constexpr int kLook = BD_BWD_LOOK;
      bf16x8 op[32];
      auto rd = [&](int i) __attribute__((always_inline)) {
        const int ds = i >> 2, qs = (i >> 1) & 1, which = i & 1;
        op[i] = lds_read_b128((which ? rdo[ds] : rq[ds]) + so + 32 * qs * 256);
      };
#pragma unroll
      for (int i = 0; i < kLook; ++i) rd(i);
      __builtin_amdgcn_sched_group_barrier(0x100, 16 + kLook, 0);
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        if (i + kLook < 32) rd(i + kLook);
        const int ds = i >> 2, qs = (i >> 1) & 1, which = i & 1;
        acc[2 * which + qs] = mfma_32x32x16(op[i], which ? vreg[ds] : kreg[ds], acc[2 * which + qs]);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i + kLook < 32) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    };

    // Vector work of a tile: P = exp2((S - LSE/scale) scale log2 e),
    // dS = P (dP - D).  Only tiles that reach below the pair's last key block or
    // past the sequence end need the mask.
    auto vector_work = [&](int it) __attribute__((always_inline)) {
      const int q0 = tile_q0(it);
      auto body = [&](auto masked_c) __attribute__((always_inline)) {
#pragma unroll
        for (int qs = 0; qs < 2; ++qs)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            float pv[8], dsv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int i = 8 * j + e;
              float pe = exp2_fast(acc[qs][i] * c2);
              if (decltype(masked_c)::value) {
                const int q = q0 + 32 * qs + 16 * j + 8 * half + e;
                if (q < qmin_key || q >= L) pe = 0.f;
              }
              pv[e] = pe;
              dsv[e] = pe * acc[2 + qs][i];
            }
            pk[4 * qs + j] = pack_bf16x8(pv);
            pk[4 * qs + 2 + j] = pack_bf16x8(dsv);
          }
      };
      if (q0 < qmin_w_hi || q0 + 64 > L) body(std::true_type());
      else body(std::false_type());
    };

    // Tile t in stage S (= t % 3): phase A(t), phase B(t).
    auto tile = [&](auto sc, int t) __attribute__((always_inline)) {
      if (t >= 1 && live(t - 1)) {
#pragma unroll
        for (int o = 0; o < 8; ++o)
          *reinterpret_cast<__attribute__((address_space(3))) bf16x8*>((uintptr_t)(xch + 1024 * o)) = pk[o];
      }
      if (t < n_iter && live(t)) products(sc);
      __syncthreads();
      if (t < n_iter && live(t)) vector_work(t);
      __syncthreads();
    };
    for (int t = 0; t <= n_iter; t += 3) {
      tile(Stage<0>(), t);
      if (t + 1 <= n_iter) tile(Stage<1>(), t + 1);
      if (t + 2 <= n_iter) tile(Stage<2>(), t + 2);
    }
    return;
  }

  // -------------------------------------------------------------- gradient wave
  // Loads of tile `it` into stage S: Q and dO rows (a quarter each) and the
  // -D and -LSE/scale slices (64 floats each, rows q0 .. q0 + 63 of the padded
  // arrays): lanes 0..15 of pair 0's wave copy four rows of -D each, lanes
  // 16..31 four rows of -LSE/scale.
  auto issue = [&](auto sc, int it) __attribute__((always_inline)) {
    constexpr int S = decltype(sc)::value;
    const int hq = kvh * p.G + it / nqt;
    const int q0 = tile_q0(it);
    const uint16_t* qb = p.q + (int64_t)b * L * q_rs + (int64_t)hq * D;
    const uint16_t* dob = p.dO + (int64_t)b * L * q_rs + (int64_t)hq * D;
    tile_dma<kKvPairs>(lds0 + kQRing + S * kTileBytes, qb, q_rs, q0, L, gp, lane);
    tile_dma<kKvPairs>(lds0 + kDORing + S * kTileBytes, dob, q_rs, q0, L, gp, lane);
    const int64_t bh = ((int64_t)b * p.Hq + hq) * p.Lp + q0;
    if (gp == 0 && lane < 32)
      lds_dma16((lane < 16 ? p.negD + bh + 4 * lane : p.nlse + bh + 4 * (lane - 16)), lds0 + kDLRing + S * 512);
  };

  if (n_iter > 0) issue(Stage<0>(), 0);
  vm_wait<0>();
  __syncthreads();

  f32x16 dk_acc[4], dv_acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) { dk_acc[db][i] = 0.f; dv_acc[db][i] = 0.f; }
  uint32_t tq[8], tdo[8];
  tr32_bases(tq, lds0 + kQRing, lane);
#pragma unroll
  for (int y = 0; y < 8; ++y) {
    tdo[y] = tq[y] - kQRing + kDORing;
    opaque(tdo[y]);
  }

  // Products of the tile in stage S (k-step s = 16 query rows): step i takes
  // k-step i/8, d-block (i/2)%4 and dV (i even) or dK (i odd), so each
  // accumulator recurs every 8 products; A operands kLook steps ahead.
  auto products = [&](auto sc) __attribute__((always_inline)) {
    constexpr uint32_t so = decltype(sc)::value * kTileBytes;
    bf16x8 bop[8];
#pragma unroll
    for (int o = 0; o < 8; ++o)
      bop[o] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>((uintptr_t)(xch + 1024 * o));
    constexpr int kLook = BD_BWD_LOOK;
    bf16x8 op[32];
    auto rd = [&](int i) __attribute__((always_inline)) {
      const int s4 = i >> 3, db = (i >> 1) & 3, which = i & 1;
      const uint32_t* t = which ? tq : tdo;    // dK: Q^T; dV: dO^T
      op[i] = cat_i16x4(lds_read_tr16(t[tr32_idx(db, s4, 0)] + so + tr32_off(s4, 0)),
                        lds_read_tr16(t[tr32_idx(db, s4, 1)] + so + tr32_off(s4, 1)));
    };
#pragma unroll
    for (int i = 0; i < kLook; ++i) rd(i);
    __builtin_amdgcn_sched_group_barrier(0x100, 8 + 2 * kLook, 0);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (i + kLook < 32) rd(i + kLook);
      const int s4 = i >> 3, db = (i >> 1) & 3, which = i & 1;
      // operand of k-step s4 = 2 qs + j: P at 4 qs + j, dS at 4 qs + 2 + j
      const bf16x8& bb = bop[4 * (s4 >> 1) + 2 * which + (s4 & 1)];
      if (which) dk_acc[db] = mfma_32x32x16(op[i], bb, dk_acc[db]);
      else dv_acc[db] = mfma_32x32x16(op[i], bb, dv_acc[db]);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i + kLook < 32) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  };

  // Tile t: phase A(t) issues the loads of tile t+1 (stage (t+1) % 3), phase
  // B(t) multiplies tile t-1 (stage (t+2) % 3) and waits for those loads.
  auto tile = [&](auto sc, int t) __attribute__((always_inline)) {
    constexpr int S = decltype(sc)::value;
    if (t + 1 < n_iter) issue(Stage<(S + 1) % kKvNS>(), t + 1);
    __syncthreads();
    if (t >= 1 && live(t - 1)) products(Stage<(S + 2) % kKvNS>());
    vm_wait<0>();
    __syncthreads();
  };
  for (int t = 0; t <= n_iter; t += 3) {
    tile(Stage<0>(), t);
    if (t + 1 <= n_iter) tile(Stage<1>(), t + 1);
    if (t + 2 <= n_iter) tile(Stage<2>(), t + 2);
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

// Work item wid: query tile qt (256 rows) of one query head, the most
// expensive tiles of a (batch, KV head) group first.
__device__ __forceinline__ void dq_item(const BwdParams& p, const int wid) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int L = p.L;
  const int qtiles = (L + 32 * kDqNW - 1) / (32 * kDqNW);
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
  uint32_t kv_off[2];
  tile_dma_offsets<kDqNW>(kv_off, kv_rs, wave, lane);
  auto issue = [&](int t) {
    const uint32_t st = lds0 + (uint32_t)(t & 1) * kDqStage;
    static_assert(kDqNW == 8, "eight waves share the K and V copies");
    if (t + 1 < ntiles) {   // all 64 rows exist: fixed per-lane offsets from the tile's base
      const int64_t row0 = (int64_t)t * 64 * kv_rs;
      tile_dma_pair8_full(st, kb + row0, st + kTileBytes, vb + row0, kv_off, wave);
    } else {
      tile_dma_pair8(st, kb, st + kTileBytes, vb, kv_rs, t * 64, kend_wg, wave, lane);
    }
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
  const int64_t bhq = ((int64_t)b * p.Hq + hq) * p.Lp + min(qrow, L - 1);
  const float Dq = -p.negD[bhq], nlse2 = p.nlse[bhq] * p.scale_log2;
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
      for (int i = 0; i < 16; ++i) { s_acc[i] = 0.f; dp_acc[i] = -Dq; }   // dP - D accumulates directly
#pragma unroll
      for (int ds = 0; ds < 8; ++ds) {
        s_acc = mfma_32x32x16(lds_read_b128(raddr[ds] + so + h2 * 32 * 256), qreg[ds], s_acc);
        dp_acc = mfma_32x32x16(lds_read_b128(raddr[ds] + so + kTileBytes + h2 * 32 * 256), doreg[ds], dp_acc);
      }
      // entry i holds key key0 + 32*h2 + 16*(i/8) + 8*half + (i%8)
      // dS = P (dP - D).  Only a half that reaches past some row's last key
      // is masked, by setting S to -inf (exp2 gives exactly 0), in a branch of
      // its own: folded into the exponentials the mask cost four vector
      // instructions per entry on every half (measured: dQ 3.2 -> 2.9 ms).
      bf16x8 sb[2];
      if (partial) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (key0 + 32 * h2 + 16 * (i >> 3) + 8 * half + (i & 7) >= kq) s_acc[i] = kNegInf;
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float dsv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) dsv[e] = exp2_fast(__builtin_fmaf(s_acc[8 * j + e], c2, nlse2)) * dp_acc[8 * j + e];
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

static_assert(kKvNW == kDqNW, "one workgroup shape for both kinds of work item");
constexpr size_t kQueuedSmem = kDkdvSmem > kDqSmem ? kDkdvSmem : kDqSmem;

__global__ __launch_bounds__(kKvNW * 64) void bwd_dkdv(BwdParams p) { dkdv_item(p, xcd_remap(blockIdx.x, gridDim.x)); }

__global__ __launch_bounds__(kDqNW * 64) void bwd_dq(BwdParams p) { dq_item(p, xcd_remap(blockIdx.x, gridDim.x)); }

// dK/dV and dQ items in one persistent launch (one workgroup per compute
// unit), so that no compute unit idles while another XCD still works: whole
// XCDs run at different clocks (per-CU busy time of a launch of one
// workgroup per item differs by up to 7 % (dK/dV) and 10 % (dQ) between the
// XCDs), and such a launch ends when its slowest XCD does.  XCD x's list
// holds the items xcd_remap gives it in the per-item launches: its nk / 8
// dK/dV items, then its nq / 8 dQ items, each kind's whole (batch, KV head)
// groups interleaved (first item of each group, then the second, ...; within
// a group the most expensive first), so each kind runs from its most to its
// least expensive items and the list ends on small dQ items.  A workgroup
// claims the next item of its own XCD's list (XCC_ID) with an atomic counter
// and, once that list is used up, of the other XCDs' lists in turn; every
// workgroup stops when all lists are, so the loop always ends.  The counters
// only hand out items: each output is computed by one workgroup in one fixed
// order whichever claims it, so the results do not depend on the schedule.
__global__ __launch_bounds__(kKvNW * 64) void bwd_queued(BwdParams p, int nk, int nq, int pgk, int pgq) {
  constexpr int kXcd = 8;
  __shared__ int pick[2];
  const int a = nk / kXcd, bq = nq / kXcd, per = a + bq;
  // groups per XCD and their stride (1 and 0 when a group spans XCDs)
  const int gk = a % pgk == 0 ? a / pgk : 1, sk = gk > 1 ? pgk : 0;
  const int gq = bq % pgq == 0 ? bq / pgq : 1, sq = gq > 1 ? pgq : 0;
  int from = (int)(__builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & (kXcd - 1));   // XCC_ID
  for (;;) {
    if (threadIdx.x == 0) {
      int q = -1, it = 0;
      for (int y = 0; y < kXcd && q < 0; ++y) {
        const int qq = (from + y) & (kXcd - 1);
        const int i = (int)atomicAdd(p.queue + qq, 1u);
        if (i < per) {
          q = qq;
          it = i;
        }
      }
      pick[0] = q;
      pick[1] = it;
    }
    __syncthreads();
    const int q = pick[0], it = pick[1];
    __syncthreads();   // pick is rewritten only after every wave has read it
    if (q < 0) break;
    from = q;
    if (it < a) {
      dkdv_item(p, q * a + (it % gk) * sk + it / gk);
    } else {
      const int j = it - a;
      dq_item(p, q * bq + (j % gq) * sq + j / gq);
    }
  }
}

// Compute units of the current device (cached per device).
int device_cus() {
  static std::mutex mu;
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (cus[dev] == 0 && hipDeviceGetAttribute(&cus[dev], hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus[dev] = -1;
  return cus[dev];
}

}  // namespace

size_t attn_bwd_workspace_bytes(int batch, int seqlen, int n_q_heads) {
  const size_t lp = ((size_t)seqlen + 63) / 64 * 64;
  return 2 * (size_t)batch * n_q_heads * lp * sizeof(float) + 64;   // -D, -LSE/scale, 8 work counters
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
    if (attr_err == hipSuccess)
      attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_queued),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kQueuedSmem);
  });
  if (attr_err != hipSuccess) return attr_err;
  BwdParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<const uint16_t*>(o);
  p.dO = static_cast<const uint16_t*>(d_o);
  p.lse = lse;
  p.Lp = (s.seqlen + 63) / 64 * 64;
  p.negD = static_cast<float*>(ws);
  p.nlse = p.negD + (size_t)s.batch * s.n_q_heads * p.Lp;
  p.queue = reinterpret_cast<unsigned*>(p.nlse + (size_t)s.batch * s.n_q_heads * p.Lp);
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
  const long long pad = (long long)s.batch * s.n_q_heads * (p.Lp - s.seqlen);
  const long long prep_threads = rows * 16 > pad ? rows * 16 : pad;
  hipLaunchKernelGGL(bwd_prep, dim3((unsigned)((prep_threads + 255) / 256)), dim3(256), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long nk = (long long)s.batch * s.n_kv_heads * ((s.seqlen + kKvKeys - 1) / kKvKeys);
  const long long nq = (long long)s.batch * s.n_q_heads * ((s.seqlen + 32 * kDqNW - 1) / (32 * kDqNW));
  const int cus = device_cus();
  if (nk % 8 == 0 && nq % 8 == 0 && cus > 0 && nk + nq <= INT_MAX) {
    const int nkt = (s.seqlen + kKvKeys - 1) / kKvKeys;
    const int nqt = (s.seqlen + 32 * kDqNW - 1) / (32 * kDqNW);
    hipLaunchKernelGGL(bwd_queued, dim3((unsigned)std::min<long long>(cus, nk + nq)), dim3(kKvNW * 64), kQueuedSmem,
                       st, p, (int)nk, (int)nq, nkt, nqt * (s.n_q_heads / s.n_kv_heads));
    return hipGetLastError();
  }
  hipLaunchKernelGGL(bwd_dkdv, dim3((unsigned)nk), dim3(kKvNW * 64), kDkdvSmem, st, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dq, dim3((unsigned)nq), dim3(kDqNW * 64), kDqSmem, st, p);
  return hipGetLastError();
}

}  // namespace bd
