// Device-side building blocks shared by the gfx950 kernels of libbd.
//
// Matrix-core conventions used throughout (CDNA4 wave64):
//   v_mfma_f32_32x32x16_bf16  D[32x32] += A[32x16] * B[16x32]
//     A: lane l holds row (l % 32), k = 8*(l / 32) .. +7   (8 bf16 = 16 bytes)
//     B: lane l holds col (l % 32), k = 8*(l / 32) .. +7
//     D: lane l holds col (l % 32), rows 8*(i/4) + 4*(l/32) + (i%4), i = 0..15
//   v_mfma_f32_16x16x32_bf16  D[16x16] += A[16x32] * B[32x16]
//     A: lane l holds row (l % 16), k = 8*(l / 16) .. +7
//     B: lane l holds col (l % 16), k = 8*(l / 16) .. +7
//     D: lane l holds col (l % 16), rows 4*(l/16) + i, i = 0..3
// The GPU parity tests exercise every one of these layouts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ f32x16 mfma_32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Hardware base-2 exponential (v_exp_f32).  exp2(-inf) = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ bf16x8 pack_bf16x8(const float* p) {
  uint4 u;
  u.x = pack_bf16x2(p[0], p[1]);
  u.y = pack_bf16x2(p[2], p[3]);
  u.z = pack_bf16x2(p[4], p[5]);
  u.w = pack_bf16x2(p[6], p[7]);
  return as_bf16x8(u);
}

// Key index range visible to query row i under the block-causal mask:
// keys 0 .. key_limit(i) - 1.
__device__ __forceinline__ int key_limit(int i, int seqlen, int block_size) {
  long long e = ((long long)(i / block_size) + 1) * block_size;
  return e < seqlen ? (int)e : seqlen;
}

// Swap bits 2 and 3 of a 0..31 row index.  Loading the A operand of a 32x32x16
// product from row sigma32(l % 32) makes the accumulator of lane l hold, for
// entry i, key 16*(i/8) + 8*(l/32) + (i%8): exactly the k-slice that lane must
// supply as the B operand of the following 32x32x16 product over those keys.
__device__ __forceinline__ int sigma32(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

template <typename T>
__device__ __forceinline__ T wave_shfl_xor(T v, int m) { return __shfl_xor(v, m, 64); }

// LDS-free reductions across the 64 lanes of a wave.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void stg16(void* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }

// Workgroup index remapped so that the workgroups dispatched to one XCD
// (hardware hands them out round-robin: XCD = blockIdx % 8) receive a
// contiguous range of work items, which then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  constexpr int kXcd = 8;
  if (nblocks % kXcd != 0) return bid;
  return (bid % kXcd) * (nblocks / kXcd) + bid / kXcd;
}

}  // namespace bd
