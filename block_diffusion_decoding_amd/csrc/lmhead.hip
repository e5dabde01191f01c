// Output projection ("LM head") fused with the confidence reduce of the commit
// (MinerU-Diffusion "confidence dynamic scheduling": paper.rainbus.top digest,
// method step 4; the prediction is the decoder's distribution over the shared
// vocabulary, method step 1).
//
//   logits[r, v] = sum_k hidden[r, k] * weight[v, k]      (never stored)
//   per masked row r: max, lowest argmax, sum exp(logit - max)
//
// then the commit's decide step (threshold, fallback, state update).
//
// lmhead_reduce: one workgroup of 8 waves per compute unit and tile of 32
// hidden rows.  The tile's hidden states sit in LDS; each wave streams a
// contiguous, balanced share of the vocabulary in blocks of 8 weight rows
// straight from HBM into the A operand of v_mfma_f32_16x16x32_bf16, with up to
// 16 loads of 16 bytes per lane in flight, and multiplies them by the hidden
// states read from LDS.  Load pattern: a product's A operand is 16 rows x 32 k
// (64 bytes of each row per load), which reads each 128-byte line with two
// loads; measured on a plain stream of the same bytes, 16 rows x 64 B per load
// reaches 5.5 TB/s and 8 rows x 128 B 6.2 TB/s.  So each weight row takes two
// product rows, holding the two 32-k halves of a 64-k window (8 rows x 128 B
// per load), and every step runs the products against both k-halves of the
// hidden states; a product row's result counts only against its own half
// (half of the matrix work is thrown away: the kernel uses about a tenth of
// the matrix cores).  At the end of each block the 8 x 32 logits fold into
// per-lane running (max, argmax, sum) states; at the end the waves' states
// merge into one partial per (row, workgroup).  With one tile (a block of 32
// rows) the weight is read from HBM once, so the kernel is bound by HBM (about
// 32 flop per weight byte); more tiles re-read it once per tile.
#include "bd_device.hpp"
#include "bd_kernels.hpp"
#include "commit_common.hpp"

#include <mutex>

namespace bd {
namespace {

constexpr int kRowsT = 32;        // hidden rows per tile (two 16-column product blocks)
constexpr int kVB = 8;            // weight rows per block (two product rows each)
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kXPad = 8;          // bf16 elements of padding per LDS row
constexpr int kGroups = 256;      // workgroups per tile: one per compute unit

size_t lds_bytes(int H) { return (size_t)kRowsT * (H + kXPad) * 2 + (size_t)kWaves * kRowsT * sizeof(Partial); }

struct LmParams {
  const uint16_t* x;    // [rows, H] bf16, row stride xs elements
  const uint16_t* w;    // [V, H] bf16, row stride wsd elements
  int64_t xs, wsd;
  int rows, H, V, nvb;  // nvb = ceil(V / kVB)
  const uint8_t* masked;
  Partial* part;        // [rows][kGroups]
};

__device__ __forceinline__ uint4 ldg16_nt(const uint16_t* p) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ Partial shfl_partial(const Partial& a, int off) {
  return Partial{__shfl_xor(a.m, off, 64), __shfl_xor(a.s, off, 64), __shfl_xor(a.idx, off, 64),
                 __shfl_xor(a.bad, off, 64)};
}

// kA: weight loads in flight per lane (16 bytes each), a divisor of the steps per block.
template <int kA>
__global__ __launch_bounds__(kThreads) void lmhead_reduce(LmParams p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wg = blockIdx.x % kGroups, rt = blockIdx.x / kGroups;
  const int row0 = rt * kRowsT;

  // A tile none of whose rows is masked has nothing to compute.
  const bool mine = tid < kRowsT && row0 + tid < p.rows && p.masked[row0 + tid] != 0;
  if (!__syncthreads_or(mine)) return;

  // The tile's hidden states -> LDS, rows past the end zero.
  const int xst = p.H + kXPad;
  const int c8 = p.H / 8;
  for (int c = tid; c < kRowsT * c8; c += kThreads) {
    const int r = c / c8, k8 = c - r * c8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row0 + r < p.rows) v = ldg16(p.x + (int64_t)(row0 + r) * p.xs + k8 * 8);
    *reinterpret_cast<uint4*>(smem + r * xst + k8 * 8) = v;
  }
  __syncthreads();

  // This wave's share of the vocabulary blocks.
  const int gw = wg * kWaves + wave, nw = kGroups * kWaves;
  const int b0 = (int)((int64_t)p.nvb * gw / nw), b1 = (int)((int64_t)p.nvb * (gw + 1) / nw);
  const int KS = p.H / 64;              // product steps per block (64 k each; a multiple of kA)

  // Operand layout (16x16x32).  A: lane l holds product row m = l%16, k = 8*(l/16)..+7 of the
  // product's 32; product row m is weight row m/2 of the block, k-half m%2 of the step's 64-k
  // window, so a load reads 128 contiguous bytes of each of 8 weight rows.  B: lane l holds
  // hidden row n = l%16 (second block: 16 + n), same k, from the low or high 32-k half.
  const int vr = lane & 15, kq = lane >> 4;
  const int wj = vr >> 1, wh = vr & 1;
  const uint16_t* xl0 = smem + vr * xst + 8 * kq;
  const uint16_t* xl1 = smem + (16 + vr) * xst + 8 * kq;

  // Weight stream cursor (block bl, step kl), advanced without branches (so the
  // compiler's waits before each product cover just the load it needs); rows
  // past V are clamped to V - 1 (their logits are dropped).
  int bl = b0, kl = 0;
  auto load_next = [&]() __attribute__((always_inline)) {
    const int v = min(bl * kVB + wj, p.V - 1);
    const uint4 r = ldg16_nt(p.w + (int64_t)v * p.wsd + kl * 64 + 32 * wh + 8 * kq);
    ++kl;
    const bool wrap = kl == KS;
    bl += wrap ? 1 : 0;
    kl = wrap ? 0 : kl;
    return r;
  };

  // Accumulators: (low, high k-half) x (hidden rows n, 16 + n).
  f32x4 lo0 = {0.f, 0.f, 0.f, 0.f}, hi0 = lo0, lo1 = lo0, hi1 = lo0;
  RowState st0, st1;   // hidden rows vr and 16 + vr
  auto fold_block = [&](int b) __attribute__((always_inline)) {
    // product rows 4*kq + i: i = 0, 1 are weight row 2*kq (low, high half),
    // i = 2, 3 weight row 2*kq + 1; each half counts from its own product
    const int id0 = b * kVB + 2 * kq;
    float x0[2], x1[2];
    x0[0] = lo0[0] + hi0[1];
    x0[1] = lo0[2] + hi0[3];
    x1[0] = lo1[0] + hi1[1];
    x1[1] = lo1[2] + hi1[3];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      if (id0 + i >= p.V) x0[i] = x1[i] = kNegInf;
    fold_vec<2>(x0, id0, st0);
    fold_vec<2>(x1, id0, st1);
    lo0 = hi0 = lo1 = hi1 = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  auto mma = [&](const uint4& a, int ks) __attribute__((always_inline)) {
    const bf16x8 A = as_bf16x8(a);
    const int k0 = ks * 64;
    const bf16x8 L0 = as_bf16x8(*reinterpret_cast<const uint4*>(xl0 + k0));
    const bf16x8 H0 = as_bf16x8(*reinterpret_cast<const uint4*>(xl0 + k0 + 32));
    const bf16x8 L1 = as_bf16x8(*reinterpret_cast<const uint4*>(xl1 + k0));
    const bf16x8 H1 = as_bf16x8(*reinterpret_cast<const uint4*>(xl1 + k0 + 32));
    lo0 = mfma_16x16x32(A, L0, lo0);
    hi0 = mfma_16x16x32(A, H0, hi0);
    lo1 = mfma_16x16x32(A, L1, lo1);
    hi1 = mfma_16x16x32(A, H1, hi1);
  };

  if (b1 > b0) {
    uint4 buf[kA];
#pragma unroll
    for (int u = 0; u < kA; ++u) {
      buf[u] = load_next();
      __builtin_amdgcn_sched_barrier(0);
    }
    // every block but the last: each step's slot is refilled kA steps ahead
    for (int b = b0; b < b1 - 1; ++b) {
      for (int g = 0; g < KS; g += kA) {
#pragma unroll
        for (int u = 0; u < kA; ++u) {
          mma(buf[u], g + u);
          buf[u] = load_next();
          __builtin_amdgcn_sched_barrier(0);   // keep the loads in the order they are consumed
        }
      }
      fold_block(b);
    }
    // the last block: no loads past its end
    for (int g = 0; g < KS - kA; g += kA) {
#pragma unroll
      for (int u = 0; u < kA; ++u) {
        mma(buf[u], g + u);
        buf[u] = load_next();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int u = 0; u < kA; ++u) mma(buf[u], KS - kA + u);
    fold_block(b1 - 1);
  }

  // Lanes vr, vr+16, vr+32, vr+48 hold the same two rows: merge them, then the waves.
  Partial q0 = to_partial(st0), q1 = to_partial(st1);
#pragma unroll
  for (int off = 16; off <= 32; off <<= 1) {
    merge_partial(q0, shfl_partial(q0, off));
    merge_partial(q1, shfl_partial(q1, off));
  }
  Partial* red = reinterpret_cast<Partial*>(smem + kRowsT * xst);
  if (lane < 16) {
    red[wave * kRowsT + vr] = q0;
    red[wave * kRowsT + 16 + vr] = q1;
  }
  __syncthreads();
  if (tid < kRowsT && row0 + tid < p.rows) {
    Partial r = red[tid];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) merge_partial(r, red[w * kRowsT + tid]);
    p.part[(int64_t)(row0 + tid) * kGroups + wg] = r;
  }
}

}  // namespace

int lmhead_max_hidden() { return 2048; }

size_t lmhead_workspace_bytes(int n_seq, int blk_len) {
  return (size_t)n_seq * blk_len * kGroups * sizeof(Partial);
}

hipError_t launch_lmhead_commit(const LmHeadArgs& a, hipStream_t st) {
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [] {
    const void* fns[] = {reinterpret_cast<const void*>(&lmhead_reduce<16>),
                         reinterpret_cast<const void*>(&lmhead_reduce<8>),
                         reinterpret_cast<const void*>(&lmhead_reduce<4>),
                         reinterpret_cast<const void*>(&lmhead_reduce<2>),
                         reinterpret_cast<const void*>(&lmhead_reduce<1>)};
    for (const void* f : fns) {
      attr_err = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes(2048));
      if (attr_err != hipSuccess) break;
    }
  });
  if (attr_err != hipSuccess) return attr_err;
  const CommitArgs& c = a.commit;
  const int rows = c.n_seq * c.blk_len;
  LmParams p;
  p.x = static_cast<const uint16_t*>(a.hidden);
  p.w = static_cast<const uint16_t*>(a.weight);
  p.xs = a.hidden_stride;
  p.wsd = a.weight_stride;
  p.rows = rows;
  p.H = a.hidden_dim;
  p.V = c.vocab;
  p.nvb = (c.vocab + kVB - 1) / kVB;
  p.masked = c.masked;
  p.part = reinterpret_cast<Partial*>(c.ws);
  const int tiles = (rows + kRowsT - 1) / kRowsT;
  const dim3 grid((unsigned)(tiles * kGroups)), block(kThreads);
  const size_t lds = lds_bytes(a.hidden_dim);
  const int ks = a.hidden_dim / 64;
  if (ks % 16 == 0) hipLaunchKernelGGL(lmhead_reduce<16>, grid, block, lds, st, p);
  else if (ks % 8 == 0) hipLaunchKernelGGL(lmhead_reduce<8>, grid, block, lds, st, p);
  else if (ks % 4 == 0) hipLaunchKernelGGL(lmhead_reduce<4>, grid, block, lds, st, p);
  else if (ks % 2 == 0) hipLaunchKernelGGL(lmhead_reduce<2>, grid, block, lds, st, p);
  else hipLaunchKernelGGL(lmhead_reduce<1>, grid, block, lds, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_commit_decide(c.ws, kGroups, c, st);
}

}  // namespace bd
