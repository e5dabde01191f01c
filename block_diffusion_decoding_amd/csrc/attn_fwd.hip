// Block-causal attention forward on the gfx950 matrix cores (bf16 in, fp32
// accumulate, bf16 out, fp32 natural-log LSE).
//
// Mask (paper.rainbus.top digest, method step 3; OpenDataLab blog, Fig. 2):
// query i sees key j iff floor(j / L') <= floor(i / L'), i.e. j < key_limit(i).
//
// Work decomposition
//   workgroup = 8 waves = 256 consecutive query rows of one (batch, q head);
//   each wave owns 32 rows.  The workgroup walks key tiles of 64 from key 0 to
//   the largest key_limit of its rows, so tiles wholly in the future are never
//   loaded or multiplied: cost follows the block mask (about L^2/2), not L^2.
//   A tile a wave cannot see at all is skipped by that wave; a tile that
//   straddles the diagonal applies the mask per element; all others run
//   unmasked.
//
// Per wave and key tile (S^T formulation, see bd_device.hpp for layouts):
//   S^T[64 keys x 32 q] = K Q^T   (16 MFMA 32x32x16; Q^T stays in registers,
//                                   K rows are read from LDS in sigma32 order)
//   softmax per query column
//   O^T[128 d x 32 q] += V^T P^T   (16 MFMA 32x32x16; P^T comes straight from
//                                   the S^T accumulator, V^T is read from the
//                                   row-major V tile with transposed LDS reads)
//
// Two wave groups in antiphase ("ping-pong"): the two waves of each SIMD belong
// to different groups.  Each tile takes two phases ended by workgroup
// barriers; in every phase one group runs its matrix products (PV of the
// previous tile interleaved with QK of this one, operands read a few products
// ahead) while the other runs its softmax, so the SIMD's matrix pipe and vector
// ALU work at the same time.  K and V tiles go global -> LDS directly into
// three-stage rings of swizzled tiles; the loads are issued only by the group
// that is in its softmax phase and waited for two phases later, so matrix
// phases never wait on memory.
//
// Softmax: the score scale is folded into the exponent (one FMA per score
// before exp2).  The exponent offset of a column is not its running maximum: it
// is raised (with the matching rescale of O and of the row sum) only when a
// tile's exponentials would exceed 2^16, which in practice happens only on a
// column's first tile; O and the row sum always share the offset, so the result
// is exact up to rounding.
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
constexpr int kNW = 8;                    // waves per workgroup (two per SIMD)
constexpr int kThreads = kNW * 64;
constexpr int kTileBytes = KT * D * 2;    // 16 KB
constexpr int kNS = 3;                    // ring depth (K and V each)
constexpr uint32_t kKRing = 0;
constexpr uint32_t kVRing = kNS * kTileBytes;
constexpr uint32_t kIdsOff = 2 * kNS * kTileBytes;   // per-wave SIMD ids
constexpr size_t kSmemBytes = 2 * kNS * kTileBytes + 64;
constexpr float kSumLimit = 65536.0f;     // 2^16: largest accepted per-lane tile sum

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

  // SIMD of this wave (HW_ID bits 5:4), exchanged through LDS.  Wave groups:
  // normally the hardware places two waves on each SIMD: group A is the first
  // of the two (by wave index), group B the second, and gw (0..3) is the SIMD.
  // Otherwise waves 0-3 form A and 4-7 form B, gw = wave % 4.  Either way each
  // group has four waves with distinct gw (which split the group's tile
  // loads); the pairing only affects speed.
  const int simd = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_s_getreg((1 << 11) | (4 << 6) | 4) & 3);
  typedef __attribute__((address_space(3))) int lds_int;
  lds_int* simd_of = reinterpret_cast<lds_int*>((uintptr_t)(lds0 + kIdsOff));
  if (lane == 0) simd_of[wave] = simd;
  __syncthreads();
  int ids[kNW];
#pragma unroll
  for (int w = 0; w < kNW; ++w) ids[w] = __builtin_amdgcn_readfirstlane(simd_of[w]);
  bool paired = true;
  int rank = 0;
#pragma unroll
  for (int w = 0; w < kNW; ++w) {
    int same = 0;
#pragma unroll
    for (int x = 0; x < kNW; ++x) same += (ids[x] == ids[w]);
    paired = paired && same == 2;
    rank += (w < wave && ids[w] == simd);
  }
  const bool grp_a = __builtin_amdgcn_readfirstlane(paired ? rank == 0 : wave < 4);
  const int gw = __builtin_amdgcn_readfirstlane(paired ? simd : (wave & 3));

  // The workgroup's work item: query tile qt (256 rows) of query head hq.
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

  // Prologue: K tiles 0 and 1 and V tile 0 (issued by all waves), and the V
  // stage of tile -1 zero-filled (the first matrix phase multiplies it by
  // P = 0).
  for (int u = 0; u < 2 && u < ntiles; ++u)
    tile_dma<kNW>(lds0 + kKRing + u * kTileBytes, kb, kv_rs, u * KT, kend_wg, wave, lane);
  if (ntiles > 0) tile_dma<kNW>(lds0 + kVRing, vb, kv_rs, 0, kend_wg, wave, lane);
  {
    uint4* vz = reinterpret_cast<uint4*>(reinterpret_cast<char*>(smem) + kVRing + (kNS - 1) * kTileBytes);
    vz[tid] = make_uint4(0, 0, 0, 0);
    vz[tid + kThreads] = make_uint4(0, 0, 0, 0);
  }

  bf16x8 qreg[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (qrow < L) u = ldg16(qb + qrow * q_rs + 16 * t + 8 * half);
    qreg[t] = as_bf16x8(u);
  }
  vm_wait<0>();
  __syncthreads();

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_use = kNegInf, l_run = 0.f;
  const float c2 = p.scale_log2;

  // Per-lane LDS byte addresses, so that every read below is one of these
  // registers plus a compile-time offset.
  //   K A operand, d-step ds: row sigma32(col) (+32 for the second key block),
  //     logical chunk 2*ds + half (K stage of the current tile).
  //   V^T A operand: the transposed-read table of bd_device.hpp (V stage of the
  //     previous tile).
  uint32_t kaddr[8], vaddr[8];
  {
    const int krow = sigma32(col);
    const int kswz = tile_swz(krow);
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) kaddr[ds] = lds0 + kKRing + krow * 256 + (((2 * ds + half) ^ kswz) << 4);
    tr32_bases(vaddr, lds0 + kVRing + (kNS - 1) * kTileBytes, lane);
  }

  auto live = [&](int t) __attribute__((always_inline)) { return active && t * KT < kend_hi; };

  // Group loads: a group's four waves split one tile (4 x 1 KB each).  All
  // tiles but the workgroup's last have 64 existing rows and use fixed per-lane
  // offsets from a uniform base; the last one clamps its rows to kend_wg - 1.
  uint32_t dma_off[4];
  tile_dma_offsets<4>(dma_off, kv_rs, gw, lane);
  auto load_tile = [&](uint32_t lds_tile, const uint16_t* g, int u) __attribute__((always_inline)) {
    if (u + 1 < ntiles) tile_dma_full<4>(lds_tile, g + (int64_t)u * KT * kv_rs, dma_off, gw);
    else tile_dma<4>(lds_tile, g, kv_rs, u * KT, kend_wg, gw, lane);
  };
  f32x16 sacc[2];
  bf16x8 pb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) pb[j] = as_bf16x8(make_uint4(0, 0, 0, 0));

  // The products of a matrix phase, interleaved: PV product i (d-block i%4,
  // k-step i/4) and QK product i (key block i%2, d-step i/2) alternate, so
  // products into the same accumulator are 4 to 8 apart, and the operands of
  // the next kLook steps are read from LDS while a step is multiplied.  Two
  // steps (128 matrix-pipe cycles) of lookahead measured faster than four or
  // six: more reads in flight only back up the LDS queue that the matrix wave
  // issues into.
  auto mm = [&]() __attribute__((always_inline)) {
    constexpr int kLook = 2;
    bf16x8 vop[16], kop[16];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[h2][i] = 0.f;
    auto read_step = [&](int i) __attribute__((always_inline)) {
      const int db = i & 3, s4 = i >> 2;
      vop[i] = cat_i16x4(lds_read_tr16(vaddr[tr32_idx(db, s4, 0)] + tr32_off(s4, 0)),
                         lds_read_tr16(vaddr[tr32_idx(db, s4, 1)] + tr32_off(s4, 1)));
      kop[i] = lds_read_b128(kaddr[i >> 1] + (i & 1) * 32 * 256);
    };
#pragma unroll
    for (int i = 0; i < kLook; ++i) read_step(i);
    __builtin_amdgcn_sched_group_barrier(0x100, 3 * kLook, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + kLook < 16) read_step(i + kLook);
      oacc[i & 3] = mfma_32x32x16(vop[i], pb[i >> 2], oacc[i & 3]);
      sacc[i & 1] = mfma_32x32x16(kop[i], qreg[i >> 1], sacc[i & 1]);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      if (i + kLook < 16) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
    }
  };

  // P = exp2(S * scale * log2 e - m_use) packed to bf16, and this lane's share
  // of the row sums.  Per block of 8 scores: 8 FMAs, 8 exponentials, then the
  // sums (two partial sums) and packs, so that no exponential waits on the FMA
  // just before it.
  auto exp_tile = [&](float nm) __attribute__((always_inline)) {
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float x8[8], pv8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x8[e] = __builtin_fmaf(sacc[h2][8 * j + e], c2, nm);
#pragma unroll
        for (int e = 0; e < 8; ++e) pv8[e] = exp2_fast(x8[e]);
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          ps0 += pv8[e];
          ps1 += pv8[e + 1];
        }
        pb[2 * h2 + j] = pack_bf16x8(pv8);
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 1);   // FMAs
        __builtin_amdgcn_sched_group_barrier(0x400, 8, 1);   // exponentials
        __builtin_amdgcn_sched_group_barrier(0x002, 12, 1);  // sums, packs
      }
    return ps0 + ps1;
  };

  // Softmax of one tile.  The exponent offset m_use is not the running maximum:
  // it is raised only when the tile's exponentials with the current offset
  // would exceed 2^16 (or on a column's first visible tile, where it is -inf),
  // so the common case needs no maximum at all.  Either way O and the row sum
  // share the offset, so the result is exact up to rounding; values stay below
  // 2^16 times the row sum of an ordinary softmax.
  auto softmax = [&](int t) __attribute__((always_inline)) {
    const int key0 = t * KT;
    // entry i of block h2 holds key key0 + 32*h2 + 16*(i/8) + 8*half + (i%8)
    if (key0 + KT > kend_lo) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + 32 * h2 + 16 * (i >> 3) + 8 * half + (i & 7);
          if (key >= kq) sacc[h2][i] = kNegInf;
        }
    }
    float psum = exp_tile(-m_use);
    if (__builtin_amdgcn_ballot_w64(!(psum <= kSumLimit))) {
      float mx = kNegInf;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[h2][i]);
      mx = pair_max(mx) * c2;   // column maximum (both halves of the column)
      if (mx > m_use) {
        const float alpha = exp2_fast(m_use - mx);   // 0 while m_use is -inf
        m_use = mx;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      }
      // a column with no visible key so far keeps m_use = -inf and p = 0
      psum = exp_tile(m_use == kNegInf ? 0.f : -m_use);
    }
    l_run += psum;
  };

  // The softmax phase of tile ts (if this wave's rows see it).  Group B first
  // starts its load of V(ts+2).  At the end each wave waits for its group's
  // previous load (K(ts+1) or V(ts+1)) and leaves the one of tile ts+2 in
  // flight.
  auto s_phase = [&](int ts, bool load_v) __attribute__((always_inline)) {
    const int u = ts + 2;
    if (load_v && u < ntiles) load_tile(lds0 + kVRing + (u % kNS) * kTileBytes, vb, u);
    if (ts >= 0 && ts < ntiles && live(ts)) softmax(ts);
    if (u < ntiles) vm_wait<4>();
    else vm_wait<0>();
  };

  // The matrix phase of tile t: O += P(t-1) V(t-1) and S(t) = Q K(t)^T.  One
  // code path for every phase keeps the live ranges short: for t = 0 the PV
  // products multiply P = 0 by the zero-filled V stage, and when tile t is past
  // this wave's rows (or past the last tile) the QK products run on whatever
  // the K stage holds and their result is never used.  Afterwards kaddr moves
  // to the K stage of tile t+1 and vaddr to the V stage of tile t, and group A
  // starts its load of K(t+2).
  int kst = 0, vst = kNS - 1;   // ring stages of K(t) and V(t-1)
  auto m_phase = [&](int t, bool load_k) __attribute__((always_inline)) {
    if (live(t == 0 ? 0 : t - 1)) mm();
    const uint32_t dk = kst == kNS - 1 ? (uint32_t)(-(kNS - 1) * kTileBytes) : (uint32_t)kTileBytes;
    const uint32_t dv = vst == kNS - 1 ? (uint32_t)(-(kNS - 1) * kTileBytes) : (uint32_t)kTileBytes;
    kst = kst == kNS - 1 ? 0 : kst + 1;
    vst = vst == kNS - 1 ? 0 : vst + 1;
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) kaddr[ds] += dk;
#pragma unroll
    for (int y = 0; y < 8; ++y) vaddr[y] += dv;
    if (load_k && t + 2 < ntiles) load_tile(lds0 + kKRing + ((t + 2) % kNS) * kTileBytes, kb, t + 2);
  };

  // Schedule.  Every tile takes two phases, each ended by a workgroup
  // barrier.  Group A runs, in phase 2t, the products O += P(t-1) V(t-1) and
  // S(t) = Q K(t)^T, and in phase 2t+1 the softmax of S(t); group B runs the
  // same one phase later.  So in every phase one wave of each SIMD issues
  // matrix products while the other runs its softmax on the vector ALU.
  // Loads: A starts K(t+2) at the end of its matrix phase 2t, where the wave
  // only waits for its last products, so that the load issue stays off the
  // softmax phases that bound the loop; B starts V(t+1) at the start of its
  // softmax phase 2t.  A wave may issue its share of a tile while the other
  // waves still work, so a load goes only into a stage no wave reads in that
  // phase: with three stages per ring, K(t+2) and V(t+1) take the stages of
  // K(t-1) and V(t-2), last read in phase 2t-1.  (B cannot start V(t+2) after
  // its matrix phase 2t+1 as A does with K: its group's other waves may still
  // read V(t-1) there, in the stage that V(t+2) would take.)  The issuing
  // waves wait for K(t+2) at the end of phase 2t+3 and for V(t+1) at the end
  // of phase 2t+2; both are first read in phase 2t+4.
  if (grp_a) {
    for (int t = 0; t <= ntiles; ++t) {
      m_phase(t, true);
      __syncthreads();
      s_phase(t, false);
      __syncthreads();
    }
  } else {
    for (int t = 0; t <= ntiles; ++t) {
      s_phase(t - 1, true);
      __syncthreads();
      m_phase(t, false);
      __syncthreads();
    }
  }

  if (!active) return;
  const float l_tot = pair_sum(l_run);
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
