// One denoising step of block decoding: the current block of every sequence
// attends to that sequence's KV-cache prefix plus the block itself, with no
// mask (the block is the newest one; paper.rainbus.top digest, novelty
// paragraph on KV-cache reuse across blocks).
//
// Split-KV ("flash decoding") on gfx950:
//   decode_split  one workgroup per (sequence, kv head, row tile of 64 query
//                 rows = block tokens x the query heads of the group, key
//                 split).  Four waves own 16 query rows each and share K/V
//                 tiles of 64 keys staged global -> LDS (V transposed), double
//                 buffered.  Per tile and wave:
//                   S^T[64 keys x 16 q] = K Q^T  (4 x 4 MFMA 16x16x32)
//                   O^T[128 d x 16 q]  += V^T P^T (8 x 2 MFMA 16x16x32)
//                 and writes its unnormalised partial (m, l, acc) in fp32.
//   decode_merge  one workgroup per (sequence, kv head, row tile) combines the
//                 splits exactly: m = max m_s, l = sum l_s 2^(m_s - m),
//                 O = sum acc_s 2^(m_s - m) / l, and writes O (bf16) and LSE.
// Each K/V byte of the cache is read from HBM once per step.
#include "bd_device.hpp"
#include "bd_kernels.hpp"

#include <algorithm>
#include <mutex>

namespace bd {
namespace {

constexpr int D = 128;
constexpr int KT = 64;
constexpr int KP = D + 8;
constexpr int VP = KT + 8;
constexpr int K_TILE = KT * KP;
constexpr int V_TILE = D * VP;
constexpr int kThreads = 256;
constexpr int kRows = 64;                     // query rows per workgroup (4 waves x 16)
constexpr size_t kSmemBytes = 2 * (K_TILE + V_TILE) * sizeof(uint16_t);

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

__device__ __forceinline__ const uint16_t* key_ptr(const DecParams& p, const uint16_t* cache,
                                                   const uint16_t* blk, int64_t start, int P, int n,
                                                   int kvh, int j) {
  const int64_t rs = (int64_t)p.Hkv * D;
  return j < P ? cache + (start + j) * rs + kvh * D
               : blk + ((int64_t)n * p.blk_len + (j - P)) * rs + kvh * D;
}

__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

struct DecTileRegs {
  uint4 k[4];      // 4 chunks of 16 bytes of K
  uint4 v[4];      // 4 keys x 8 d of V
};

__device__ __forceinline__ void dec_load(DecTileRegs& r, const DecParams& p, int64_t start, int P, int n,
                                         int kvh, int key0, int kend, int tid) {
  const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + i * kThreads;
    const int key = key0 + (c >> 4);
    r.k[i] = key < kend ? ldg16(key_ptr(p, p.k_cache, p.k_blk, start, P, n, kvh, key) + (c & 15) * 8) : z;
  }
  const int kq = tid & 15, ch = tid >> 4;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int key = key0 + kq * 4 + e;
    r.v[e] = key < kend ? ldg16(key_ptr(p, p.v_cache, p.v_blk, start, P, n, kvh, key) + ch * 8) : z;
  }
}

__device__ __forceinline__ void dec_store(const DecTileRegs& r, uint16_t* ks, uint16_t* vt, int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + i * kThreads;
    *reinterpret_cast<uint4*>(ks + (c >> 4) * KP + (c & 15) * 8) = r.k[i];
  }
  const int kq = tid & 15, ch = tid >> 4;
  const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&r.v[0]);
  const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&r.v[1]);
  const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&r.v[2]);
  const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&r.v[3]);
  uint16_t* dst = vt + (ch * 8) * VP + kq * 4;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    *reinterpret_cast<uint2*>(dst + (2 * e) * VP) = make_uint2(lo_pair(w0[e], w1[e]), lo_pair(w2[e], w3[e]));
    *reinterpret_cast<uint2*>(dst + (2 * e + 1) * VP) = make_uint2(hi_pair(w0[e], w1[e]), hi_pair(w2[e], w3[e]));
  }
}

__global__ __launch_bounds__(kThreads) void decode_split(DecParams p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t* ks = smem;
  uint16_t* vt = smem + 2 * K_TILE;

  const int split = blockIdx.x % p.nsplit;
  const int unit = blockIdx.x / p.nsplit;
  const int rt = unit % p.row_tiles;
  const int nk = unit / p.row_tiles;
  const int kvh = nk % p.Hkv, n = nk / p.Hkv;

  const int P = p.prefix_len[n];
  const int64_t start = p.prefix_start[n];
  const int total = P + p.blk_len;
  const int k0 = split * p.chunk;
  if (k0 >= total) return;
  const int k1 = min(total, k0 + p.chunk);
  const int ntiles = (k1 - k0 + KT - 1) / KT;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, g4 = lane >> 4;
  const int rloc = wave * 16 + col;            // row within the tile
  const int r = rt * kRows + rloc;             // row within the unit: r = hl * blk_len + t
  const bool rvalid = r < p.rows;
  const int hl = rvalid ? r / p.blk_len : 0, tok = rvalid ? r % p.blk_len : 0;
  const int hq = kvh * p.G + hl;

  bf16x8 qreg[4];
  {
    const uint16_t* qr = p.q_blk + (((int64_t)n * p.blk_len + tok) * p.Hq + hq) * D + 8 * g4;
#pragma unroll
    for (int t = 0; t < 4; ++t) qreg[t] = as_bf16x8(rvalid ? ldg16(qr + 32 * t) : make_uint4(0, 0, 0, 0));
  }

  f32x4 oacc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  DecTileRegs regs;
  dec_load(regs, p, start, P, n, kvh, k0, k1, tid);
  dec_store(regs, ks, vt, tid);
  __syncthreads();

  // A-operand row of 16-key block kb for lane row rho = col:
  //   key 32*(kb/2) + 8*(rho/4) + 4*(kb%2) + rho%4
  // so that accumulator entry i of lane (col, g4) in block kb holds key
  //   32*(kb/2) + 8*g4 + 4*(kb%2) + i,
  // the B-operand k-slice of the PV product over keys 32*(kb/2) .. +31.
  const int arow = 8 * (col >> 2) + (col & 3);

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int key0 = k0 + t * KT;
    if (t + 1 < ntiles) dec_load(regs, p, start, P, n, kvh, key0 + KT, k1, tid);
    const uint16_t* K = ks + buf * K_TILE;
    const uint16_t* V = vt + buf * V_TILE;

    f32x4 sacc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint16_t* kr = K + (32 * (kb >> 1) + 4 * (kb & 1) + arow) * KP + 8 * g4;
#pragma unroll
      for (int ds = 0; ds < 4; ++ds)
        sacc[kb] = mfma_16x16x32(*reinterpret_cast<const bf16x8*>(kr + 32 * ds), qreg[ds], sacc[kb]);
    }
    const bool partial = key0 + KT > k1;
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float s = sacc[kb][i] * p.scale_log2;
        if (partial) {
          const int key = key0 + 32 * (kb >> 1) + 8 * g4 + 4 * (kb & 1) + i;
          if (key >= k1) s = kNegInf;
        }
        sacc[kb][i] = s;
        mx = fmaxf(mx, s);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2_fast(m_run - m_new);
    float psum = 0.f;
    bf16x8 pb[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      float pv[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[i] = exp2_fast(sacc[2 * s2][i] - m_new);
        pv[4 + i] = exp2_fast(sacc[2 * s2 + 1][i] - m_new);
        psum += pv[i] + pv[4 + i];
      }
      pb[s2] = pack_bf16x8(pv);
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      oacc[db] *= alpha;
      const uint16_t* vr = V + (16 * db + col) * VP + 8 * g4;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
        oacc[db] = mfma_16x16x32(*reinterpret_cast<const bf16x8*>(vr + 32 * s2), pb[s2], oacc[db]);
    }
    if (t + 1 < ntiles) dec_store(regs, ks + (buf ^ 1) * K_TILE, vt + (buf ^ 1) * V_TILE, tid);
    __syncthreads();
  }

  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  const int64_t slot = ((int64_t)unit * p.nsplit + split) * kRows + rloc;
  if (g4 == 0) p.part_ml[slot] = make_float2(m_run, l_tot);
  float* acc = p.part_acc + slot * D + 4 * g4;
#pragma unroll
  for (int db = 0; db < 8; ++db)
    *reinterpret_cast<float4*>(acc + 16 * db) = make_float4(oacc[db][0], oacc[db][1], oacc[db][2], oacc[db][3]);
}

// Thread layout: 4 threads per row, 32 head-dim entries each.
__global__ __launch_bounds__(kThreads) void decode_merge(DecParams p) {
  const int unit = blockIdx.x;
  const int rt = unit % p.row_tiles;
  const int nk = unit / p.row_tiles;
  const int kvh = nk % p.Hkv, n = nk / p.Hkv;
  const int total = p.prefix_len[n] + p.blk_len;
  const int ns = min(p.nsplit, (total + p.chunk - 1) / p.chunk);
  const int tid = threadIdx.x;
  const int rloc = tid >> 2, part = tid & 3;
  const int r = rt * kRows + rloc;
  if (r >= p.rows) return;
  const int hl = r / p.blk_len, tok = r % p.blk_len;
  const int hq = kvh * p.G + hl;

  const int64_t base = (int64_t)unit * p.nsplit * kRows + rloc;
  float m = kNegInf;
  for (int s = 0; s < ns; ++s) m = fmaxf(m, p.part_ml[base + (int64_t)s * kRows].x);
  float l = 0.f;
  float acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float2 ml = p.part_ml[base + (int64_t)s * kRows];
    const float w = exp2_fast(ml.x - m);
    l += ml.y * w;
    const float4* src = reinterpret_cast<const float4*>(p.part_acc + (base + (int64_t)s * kRows) * D + part * 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 a = src[i];
      acc[4 * i] += a.x * w;
      acc[4 * i + 1] += a.y * w;
      acc[4 * i + 2] += a.z * w;
      acc[4 * i + 3] += a.w * w;
    }
  }
  const float inv = 1.0f / l;
  uint16_t* orow = p.o + (((int64_t)n * p.blk_len + tok) * p.Hq + hq) * D + part * 32;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint4 w;
    w.x = pack_bf16x2(acc[8 * i] * inv, acc[8 * i + 1] * inv);
    w.y = pack_bf16x2(acc[8 * i + 2] * inv, acc[8 * i + 3] * inv);
    w.z = pack_bf16x2(acc[8 * i + 4] * inv, acc[8 * i + 5] * inv);
    w.w = pack_bf16x2(acc[8 * i + 6] * inv, acc[8 * i + 7] * inv);
    *reinterpret_cast<uint4*>(orow + 8 * i) = w;
  }
  if (p.lse && part == 0) p.lse[((int64_t)n * p.Hq + hq) * p.blk_len + tok] = (m + __log2f(l)) * kLn2;
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
  // Aim for about 2048 busy workgroups (8 per CU) while keeping each split at
  // least two tiles long, so that partial-state traffic stays small next to
  // the K/V bytes a split streams.
  const long long want_splits = std::max<long long>(1, (2048 + pl.units - 1) / pl.units);
  long long chunk = (total_max + want_splits - 1) / want_splits;
  chunk = std::max<long long>(2 * KT, ((chunk + KT - 1) / KT) * KT);
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
  hipLaunchKernelGGL(decode_merge, dim3((unsigned)pl.units), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace bd
