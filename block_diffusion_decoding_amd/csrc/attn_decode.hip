// One denoising step of block decoding: the current block of every sequence
// attends to that sequence's KV-cache prefix plus the block itself, with no
// mask (the block is the newest one; paper.rainbus.top digest, novelty
// paragraph on KV-cache reuse across blocks).
//
// Split-KV ("flash decoding") on gfx950:
//   decode_split  one workgroup per (sequence, kv head, row tile of 64 query
//                 rows = block tokens x the query heads of the group, key
//                 split).  Four waves own 16 query rows each and share K/V
//                 tiles of 32 keys copied global -> LDS directly into a ring of
//                 kNS swizzled stages (kNS-1 tiles of loads in flight; 48 KB of
//                 LDS, so three workgroups share a CU).  Per tile and wave:
//                   S^T[32 keys x 16 q] = K Q^T  (2 x 4 MFMA 16x16x32)
//                   O^T[128 d x 16 q]  += V^T P^T (8 MFMA 16x16x32, V^T read
//                                                  transposed from LDS)
//                 and writes its unnormalised partial (m, l, acc) in fp32.
//   decode_merge  combines the splits exactly: m = max m_s,
//                 l = sum l_s 2^(m_s - m), O = sum acc_s 2^(m_s - m) / l, and
//                 writes O (bf16) and LSE; 128 threads per query row, one per
//                 head-dim entry.
// Each K/V byte of the cache is read from HBM once per step.
#include "bd_device.hpp"
#include "bd_kernels.hpp"

#include <algorithm>
#include <mutex>

// Pipeline shape (compile-time): LDS ring depth and the workgroup count the
// split plan aims for.
#ifndef BD_DECODE_NS
#define BD_DECODE_NS 3
#endif
#ifndef BD_DECODE_TARGET_WGS
#define BD_DECODE_TARGET_WGS 4096
#endif

namespace bd {
namespace {

constexpr int D = 128;
constexpr int KT = 32;
constexpr int kNW = 4;
constexpr int kNS = BD_DECODE_NS;
constexpr int kThreads = kNW * 64;
constexpr int kRows = 64;                     // query rows per workgroup (4 waves x 16)
constexpr int kTileBytes = KT * D * 2;      // 8 KB
constexpr int kStageBytes = 2 * kTileBytes;
constexpr size_t kSmemBytes = (size_t)kNS * kStageBytes;
constexpr int kMergeRows = 2;                 // query rows per merge workgroup

struct DecParams {
  const uint16_t* q_blk;
  const uint16_t* k_blk;
  const uint16_t* v_blk;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int64_t* prefix_start;
  const int32_t* prefix_len;
  float2* part_ml;   // [unit][nsplit][kRows]
  float* part_acc;   // [unit][nsplit][kRows][D]
  uint16_t* o;
  float* lse;
  int n_seq, blk_len, Hq, Hkv, G, rows, row_tiles, nsplit, chunk;
  float scale_log2;
};

// Copy this wave's share of the 32-key tile starting at key `key0` of the
// sequence's key list (prefix rows of the cache, then the block's own rows) into
// the swizzled LDS tile.  Keys >= kend are clamped to kend - 1.
__device__ __forceinline__ void dec_tile_dma(uint32_t lds_tile, const uint16_t* cache, const uint16_t* blk,
                                             int64_t start, int P, int n, int kvh, int blk_len, int Hkv,
                                             int key0, int kend, int wave, int lane) {
  const int64_t rs = (int64_t)Hkv * D;
#pragma unroll
  for (int i = 0; i < KT / 4 / kNW; ++i) {
    const int nn = wave * (KT / 4 / kNW) + i;
    const int r = 4 * nn + (lane >> 4);
    const int c = (lane & 15) ^ tile_swz(r);
    const int j = min(key0 + r, kend - 1);
    const uint16_t* src = j < P ? cache + (start + j) * rs : blk + ((int64_t)n * blk_len + (j - P)) * rs;
    lds_dma16(src + kvh * D + 8 * c, lds_tile + nn * 1024);
  }
}

__global__ __launch_bounds__(kThreads) void decode_split(DecParams p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  // Workgroup order: kv head fastest, then row tile, then split, then sequence.
  // A cache row interleaves the kv heads, so the workgroups dispatched together
  // fetch neighbouring pieces of the same rows.
  int bid = blockIdx.x;
  const int kvh = bid % p.Hkv;
  bid /= p.Hkv;
  const int rt = bid % p.row_tiles;
  bid /= p.row_tiles;
  const int split = bid % p.nsplit;
  const int n = bid / p.nsplit;
  const int unit = (n * p.Hkv + kvh) * p.row_tiles + rt;

  const int P = p.prefix_len[n];
  const int64_t start = p.prefix_start[n];
  const int total = P + p.blk_len;
  const int k0 = split * p.chunk;
  if (k0 >= total) return;
  const int k1 = min(total, k0 + p.chunk);
  const int ntiles = (k1 - k0 + KT - 1) / KT;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, g4 = lane >> 4;
  const int rloc = wave * 16 + col;            // row within the tile
  const int r = rt * kRows + rloc;             // row within the unit: r = hl * blk_len + t
  const bool rvalid = r < p.rows;
  const int hl = rvalid ? r / p.blk_len : 0, tok = rvalid ? r % p.blk_len : 0;
  const int hq = kvh * p.G + hl;

#pragma unroll
  for (int s = 0; s < kNS - 1; ++s) {
    if (s < ntiles) {
      const uint32_t st = lds0 + s * kStageBytes;
      dec_tile_dma(st, p.k_cache, p.k_blk, start, P, n, kvh, p.blk_len, p.Hkv, k0 + s * KT, k1, wave, lane);
      dec_tile_dma(st + kTileBytes, p.v_cache, p.v_blk, start, P, n, kvh, p.blk_len, p.Hkv, k0 + s * KT, k1, wave,
                   lane);
    }
  }

  bf16x8 qreg[4];
  {
    const uint16_t* qr = p.q_blk + (((int64_t)n * p.blk_len + tok) * p.Hq + hq) * D + 8 * g4;
#pragma unroll
    for (int t = 0; t < 4; ++t) qreg[t] = as_bf16x8(rvalid ? ldg16(qr + 32 * t) : make_uint4(0, 0, 0, 0));
  }
  vm_wait<0>();

  f32x4 oacc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_use = kNegInf, l_run = 0.f;
  const float c2 = p.scale_log2;

  // A-operand row of 16-key block kb (0, 1) for lane row rho = col:
  //   key 8*(rho/4) + 4*kb + rho%4
  // so that accumulator entry i of lane (col, g4) in block kb holds key
  //   8*g4 + 4*kb + i,
  // the B-operand k-slice of the PV product over the tile's 32 keys.
  const int arow = 8 * (col >> 2) + (col & 3);
  constexpr int per_tile = 2 * (KT / 4 / kNW);

  for (int t = 0; t < ntiles; ++t) {
    const int pending = min(kNS - 2, ntiles - 1 - t);
    if (pending >= 3) vm_wait<3 * per_tile>();
    else if (pending == 2) vm_wait<2 * per_tile>();
    else if (pending == 1) vm_wait<per_tile>();
    else vm_wait<0>();
    __syncthreads();
    if (t + kNS - 1 < ntiles) {
      const uint32_t st = lds0 + ((t + kNS - 1) % kNS) * kStageBytes;
      const int kn = k0 + (t + kNS - 1) * KT;
      dec_tile_dma(st, p.k_cache, p.k_blk, start, P, n, kvh, p.blk_len, p.Hkv, kn, k1, wave, lane);
      dec_tile_dma(st + kTileBytes, p.v_cache, p.v_blk, start, P, n, kvh, p.blk_len, p.Hkv, kn, k1, wave, lane);
    }
    const int key0 = k0 + t * KT;
    const uint32_t Kt = lds0 + (t % kNS) * kStageBytes;
    const uint32_t Vt = Kt + kTileBytes;

    f32x4 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int row = 4 * kb + arow;
#pragma unroll
      for (int ds = 0; ds < 4; ++ds)
        sacc[kb] = mfma_16x16x32(lds_read_b128(Kt + tile_off(row, 4 * ds + g4)), qreg[ds], sacc[kb]);
    }
    float mx = kNegInf;
    if (key0 + KT > k1) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = key0 + 8 * g4 + 4 * kb + i;
          if (key >= k1) sacc[kb][i] = kNegInf;
          mx = fmaxf(mx, sacc[kb][i]);
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[kb][i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * c2;
    const bool grow = mx > m_use + 8.0f;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float m_new = grow ? mx : m_use;
      const float alpha = exp2_fast(m_use - m_new);
      m_use = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 8; ++db) oacc[db] *= alpha;
    }
    const float nm = -m_use;
    float psum = 0.f;
    float pv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pv[i] = exp2_fast(__builtin_fmaf(sacc[0][i], c2, nm));
      pv[4 + i] = exp2_fast(__builtin_fmaf(sacc[1][i], c2, nm));
      psum += pv[i] + pv[4 + i];
    }
    const bf16x8 pb = pack_bf16x8(pv);
    l_run += psum;
#pragma unroll
    for (int db = 0; db < 8; ++db) oacc[db] = mfma_16x16x32(tile_read_t16(Vt, db, 0, lane), pb, oacc[db]);
  }

  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  const int64_t slot = ((int64_t)unit * p.nsplit + split) * kRows + rloc;
  if (g4 == 0) p.part_ml[slot] = make_float2(m_use, l_tot);
  float* acc = p.part_acc + slot * D + 4 * g4;
#pragma unroll
  for (int db = 0; db < 8; ++db)
    *reinterpret_cast<float4*>(acc + 16 * db) = make_float4(oacc[db][0], oacc[db][1], oacc[db][2], oacc[db][3]);
}

// 128 threads per query row, one head-dim entry each; kMergeRows rows per workgroup.
__global__ __launch_bounds__(128 * kMergeRows) void decode_merge(DecParams p) {
  const int per_unit = kRows / kMergeRows;
  const int unit = blockIdx.x / per_unit;
  const int rloc = (blockIdx.x % per_unit) * kMergeRows + threadIdx.x / D;
  const int d = threadIdx.x % D;
  const int rt = unit % p.row_tiles;
  const int nk = unit / p.row_tiles;
  const int kvh = nk % p.Hkv, n = nk / p.Hkv;
  const int r = rt * kRows + rloc;
  if (r >= p.rows) return;
  const int total = p.prefix_len[n] + p.blk_len;
  const int ns = min(p.nsplit, (total + p.chunk - 1) / p.chunk);
  const int hl = r / p.blk_len, tok = r % p.blk_len;
  const int hq = kvh * p.G + hl;

  const int64_t base = (int64_t)unit * p.nsplit * kRows + rloc;
  // Loads of up to kBatch splits are issued together (the split count is small
  // but each load is a round trip to L2 / HBM).
  constexpr int kBatch = 8;
  float m = kNegInf;
  for (int s0 = 0; s0 < ns; s0 += kBatch) {
    float mb[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) mb[k] = (s0 + k < ns) ? p.part_ml[base + (int64_t)(s0 + k) * kRows].x : kNegInf;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) m = fmaxf(m, mb[k]);
  }
  float l = 0.f, acc = 0.f;
  for (int s0 = 0; s0 < ns; s0 += kBatch) {
    float2 ml[kBatch];
    float a[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int64_t slot = base + (int64_t)(s0 + k) * kRows;
      const bool ok = s0 + k < ns;
      ml[k] = ok ? p.part_ml[slot] : make_float2(kNegInf, 0.f);
      a[k] = ok ? p.part_acc[slot * D + d] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const float w = exp2_fast(ml[k].x - m);
      l += ml[k].y * w;
      acc += a[k] * w;
    }
  }
  const float o = acc / l;
  const uint16_t ob = __builtin_bit_cast(uint16_t, (__bf16)o);
  p.o[(((int64_t)n * p.blk_len + tok) * p.Hq + hq) * D + d] = ob;
  if (p.lse && d == 0) p.lse[((int64_t)n * p.Hq + hq) * p.blk_len + tok] = (m + __log2f(l)) * kLn2;
}

struct Plan {
  int row_tiles, nsplit, chunk;
  long long units;
};

Plan make_plan(const DecodeShape& s) {
  Plan pl;
  const int rows = s.blk_len * (s.n_q_heads / s.n_kv_heads);
  pl.row_tiles = (rows + kRows - 1) / kRows;
  pl.units = (long long)s.n_seq * s.n_kv_heads * pl.row_tiles;
  const long long total_max = (long long)s.max_prefix_len + s.blk_len;
  // Aim for about BD_DECODE_TARGET_WGS workgroups over the longest sequence's
  // splits, with splits of at least four tiles (128 keys).
  const long long want_splits = std::max<long long>(1, (BD_DECODE_TARGET_WGS + pl.units - 1) / pl.units);
  long long chunk = (total_max + want_splits - 1) / want_splits;
  chunk = std::max<long long>(4 * KT, ((chunk + KT - 1) / KT) * KT);
  pl.chunk = (int)chunk;
  pl.nsplit = (int)((total_max + chunk - 1) / chunk);
  return pl;
}

}  // namespace

size_t decode_workspace_bytes(const DecodeShape& s, int /*is_bf16*/) {
  const Plan pl = make_plan(s);
  return (size_t)pl.units * pl.nsplit * kRows * (sizeof(float2) + D * sizeof(float));
}

hipError_t launch_decode_bf16(const void* q_blk, const void* k_blk, const void* v_blk, const void* k_cache,
                              const void* v_cache, const int64_t* prefix_start, const int32_t* prefix_len,
                              void* o, float* lse, void* ws, const DecodeShape& s, hipStream_t st) {
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [] {
    attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_split),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSmemBytes);
  });
  if (attr_err != hipSuccess) return attr_err;
  const Plan pl = make_plan(s);
  DecParams p;
  p.q_blk = static_cast<const uint16_t*>(q_blk);
  p.k_blk = static_cast<const uint16_t*>(k_blk);
  p.v_blk = static_cast<const uint16_t*>(v_blk);
  p.k_cache = static_cast<const uint16_t*>(k_cache);
  p.v_cache = static_cast<const uint16_t*>(v_cache);
  p.prefix_start = prefix_start;
  p.prefix_len = prefix_len;
  p.part_ml = reinterpret_cast<float2*>(ws);
  p.part_acc = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) +
                                        (size_t)pl.units * pl.nsplit * kRows * sizeof(float2));
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.n_seq = s.n_seq;
  p.blk_len = s.blk_len;
  p.Hq = s.n_q_heads;
  p.Hkv = s.n_kv_heads;
  p.G = s.n_q_heads / s.n_kv_heads;
  p.rows = s.blk_len * p.G;
  p.row_tiles = pl.row_tiles;
  p.nsplit = pl.nsplit;
  p.chunk = pl.chunk;
  p.scale_log2 = s.scale * kLog2e;
  hipLaunchKernelGGL(decode_split, dim3((unsigned)(pl.units * pl.nsplit)), dim3(kThreads), kSmemBytes, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge, dim3((unsigned)(pl.units * (kRows / kMergeRows))), dim3(128 * kMergeRows), 0, st,
                     p);
  return hipGetLastError();
}

}  // namespace bd
