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

// Round to nearest even; one v_cvt_pk_bf16_f32 on gfx950.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
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

// LDS-free reductions across the 64 lanes of a wave.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Combine the values of lanes l and l ^ 32 (v_permlane32_swap, no LDS
// traffic); both lanes of a pair get the bitwise-identical result.
__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
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


// ---------------------------------------------------------------------------
// 64-row x 128-column bf16 tiles in LDS (256-byte rows, no padding).  The 16
// byte chunks of row r are XOR-swizzled: logical chunk c sits at physical
// chunk c ^ tile_swz(r), with tile_swz mapping row bits (r2, r3, r0 ^ r4, r1)
// to chunk bits (0, 1, 2, 3).  Measured on gfx950, ds_read_b128 serves 16
// lanes of equal lane bits 1 and 5 together, each lane taking one 16-byte slot
// of a 512-byte bank window (row parity and physical chunk), and
// ds_read_b64_tr_b16 serves the lanes of a half-wave together over 64 four-byte
// banks.  Under that rule this swizzle is conflict-free for every read pattern
// of the kernels:
//   * 32x32 A operands read as rows: lanes at rows sigma32(l % 32) (+32), one
//     logical chunk per half-wave;
//   * 16x16 A operands read as rows: rows 8(l%16 / 4) + l%4 (+4), chunk l/16;
//   * 32x32 and 16x16 A operands read transposed (tr32_* and tile_read_t16).
// Rows 16 apart differ in tile_swz only by chunk bit 2 (bit r4), and rows 32
// apart not at all; the transposed-read address tables below rely on this.
__device__ __forceinline__ int tile_swz(int r) {
  return ((r >> 2) & 1) | (((r >> 3) & 1) << 1) | ((((r >> 0) ^ (r >> 4)) & 1) << 2) | (((r >> 1) & 1) << 3);
}
__device__ __forceinline__ uint32_t tile_off(int r, int c) { return (uint32_t)(r * 256 + ((c ^ tile_swz(r)) << 4)); }

// Global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4): lane l of
// the wave writes bytes [lds_base + 16 l, +16).  Issued through inline asm so
// that the compiler does not fence every later LDS read on it; the caller
// waits with vm_wait<N>() before a barrier.  M0 is restored afterwards.  A
// scalar write of M0 needs one wait state before an LDS-DMA load reads it (the
// compiler keeps that distance in the code it emits itself), hence the s_nop.
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(lds_base)
      : "memory");
}

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left unconstrained).
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Two copies to consecutive 1 KB LDS blocks in one asm statement (M0 saved and
// restored once, one wait state after each M0 write).
__device__ __forceinline__ void lds_dma16_x2(const void* g0, const void* g1, uint32_t l0) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %4\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g0), "v"(g1), "s"(l0), "s"(l0 + 1024)
      : "memory");
}

// Four copies in one asm statement, to any four 1 KB LDS blocks.
__device__ __forceinline__ void lds_dma16_x4(const void* g0, const void* g1, const void* g2, const void* g3,
                                             uint32_t l0, uint32_t l1, uint32_t l2, uint32_t l3) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %5\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %6\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %7\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %3, off\n\t"
      "s_mov_b32 m0, %8\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %4, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g0), "v"(g1), "v"(g2), "v"(g3), "s"(l0), "s"(l1), "s"(l2), "s"(l3)
      : "memory");
}

// Source address of copy i of this wave's share of a clamped tile (see tile_dma).
template <int NW>
__device__ __forceinline__ const uint16_t* tile_src(const uint16_t* g, int64_t rs, int row0, int nrows, int wave,
                                                    int lane, int i) {
  const int n = wave * (16 / NW) + i;
  const int r = 4 * n + (lane >> 4);
  const int c = (lane & 15) ^ tile_swz(r);
  const int row = min(row0 + r, nrows - 1);
  return g + row * rs + 8 * c;
}

// Copy this wave's share of a 64-row tile (rows row0 .. row0+63 of a row-major
// bf16 matrix with row stride `rs` elements; rows >= nrows are clamped to the
// last valid row) into the swizzled LDS tile at byte address `lds_tile`.
// The tile is 16 wave-instructions of 1 KB (4 rows each); wave w of NW issues
// instructions w*16/NW .. +16/NW-1.
template <int NW>
__device__ __forceinline__ void tile_dma(uint32_t lds_tile, const uint16_t* g, int64_t rs, int row0, int nrows,
                                         int wave, int lane) {
  static_assert(NW == 4 || NW == 8, "two or four copies per wave");
  constexpr int kPer = 16 / NW;
  const uint32_t l0 = lds_tile + wave * kPer * 1024;
  if constexpr (kPer == 2) {
    lds_dma16_x2(tile_src<NW>(g, rs, row0, nrows, wave, lane, 0), tile_src<NW>(g, rs, row0, nrows, wave, lane, 1),
                 l0);
  } else {
    lds_dma16_x4(tile_src<NW>(g, rs, row0, nrows, wave, lane, 0), tile_src<NW>(g, rs, row0, nrows, wave, lane, 1),
                 tile_src<NW>(g, rs, row0, nrows, wave, lane, 2), tile_src<NW>(g, rs, row0, nrows, wave, lane, 3),
                 l0, l0 + 1024, l0 + 2048, l0 + 3072);
  }
}

// Two tiles with the same rows (K and V of one key range) copied by eight
// waves, each wave's four copies in one asm statement.
__device__ __forceinline__ void tile_dma_pair8(uint32_t lds_a, const uint16_t* ga, uint32_t lds_b,
                                               const uint16_t* gb, int64_t rs, int row0, int nrows, int wave,
                                               int lane) {
  const uint32_t la = lds_a + wave * 2 * 1024, lb = lds_b + wave * 2 * 1024;
  lds_dma16_x4(tile_src<8>(ga, rs, row0, nrows, wave, lane, 0), tile_src<8>(ga, rs, row0, nrows, wave, lane, 1),
               tile_src<8>(gb, rs, row0, nrows, wave, lane, 0), tile_src<8>(gb, rs, row0, nrows, wave, lane, 1),
               la, la + 1024, lb, lb + 1024);
}

// K and V rows of one whole 64-row tile (both with the same row stride) copied
// by eight waves: per-lane byte offsets from tile_dma_offsets<8>, wave-uniform
// tile bases; each wave's four copies in one asm statement.
__device__ __forceinline__ void tile_dma_pair8_full(uint32_t lds_a, const uint16_t* ga_tile, uint32_t lds_b,
                                                    const uint16_t* gb_tile, const uint32_t* off, int wave) {
  const uint32_t la = lds_a + wave * 2 * 1024, lb = lds_b + wave * 2 * 1024;
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %5\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %3\n\t"
      "s_mov_b32 m0, %6\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %7\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %4\n\t"
      "s_mov_b32 m0, %8\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %4\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off[0]), "v"(off[1]), "s"(ga_tile), "s"(gb_tile), "s"(la), "s"(la + 1024), "s"(lb), "s"(lb + 1024)
      : "memory");
}

// The same copy for a tile whose 64 rows all exist: the per-lane byte offsets
// (from tile_dma_offsets) do not depend on the tile, only the uniform base
// `g_tile` (= row row0 of the matrix) does.
template <int NW>
__device__ __forceinline__ void tile_dma_offsets(uint32_t* off, int64_t rs, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 16 / NW; ++i) {
    const int n = wave * (16 / NW) + i;
    const int r = 4 * n + (lane >> 4);
    const int c = (lane & 15) ^ tile_swz(r);
    off[i] = (uint32_t)((r * rs + 8 * c) * 2);
  }
}
// With four waves each wave issues four 1 KB copies to consecutive LDS
// addresses; they go in one asm statement, so M0 is saved and restored once and
// each M0 write is followed by the one wait state the copy that reads it needs.
template <int NW>
__device__ __forceinline__ void tile_dma_full(uint32_t lds_tile, const uint16_t* g_tile, const uint32_t* off,
                                              int wave) {
  static_assert(NW == 4, "four copies per wave");
  const uint32_t l0 = lds_tile + wave * 4 * 1024;
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %6\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %5\n\t"
      "s_mov_b32 m0, %7\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %5\n\t"
      "s_mov_b32 m0, %8\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %3, %5\n\t"
      "s_mov_b32 m0, %9\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %4, %5\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]), "s"(g_tile), "s"(l0), "s"(l0 + 1024),
        "s"(l0 + 2048), "s"(l0 + 3072)
      : "memory");
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// Transposed LDS read: within each group of 16 lanes, lane i receives element
// i % 4 of the 8-byte chunks addressed by lanes 4j + i / 4, j = 0..3.
__device__ __forceinline__ i16x4 lds_read_tr16(uint32_t lds_addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<__attribute__((address_space(3))) i16x4*>((uintptr_t)lds_addr));
}

__device__ __forceinline__ bf16x8 lds_read_b128(uint32_t lds_addr) {
  return *reinterpret_cast<__attribute__((address_space(3))) bf16x8*>((uintptr_t)lds_addr);
}

// Four consecutive rows of one column, read transposed from a row-major
// swizzled tile T[row][d]: within each 16-lane group, lane i (i = lane % 16)
// receives T[row0 + j][dbase + i] for j = 0..3 (dbase a multiple of 8; row0
// and dbase may differ between groups).
__device__ __forceinline__ i16x4 tile_read_t4(uint32_t lds_tile, int row0, int dbase, int lane) {
  const int li = lane & 15;
  const int row = row0 + (li >> 2);
  const int d = dbase + 4 * (li & 3);
  return lds_read_tr16(lds_tile + tile_off(row, d >> 3) + 2 * (d & 7));
}

__device__ __forceinline__ bf16x8 cat_i16x4(i16x4 lo, i16x4 hi) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, w);
}

// A operand (rows = head dim, k = 32 tile rows 32*s .. 32*s+31) of a 16x16x32
// product, read transposed: lane l gets T[32s + 8(l/16) + r][16 db + l % 16]
// for r = 0..7.
__device__ __forceinline__ bf16x8 tile_read_t16(uint32_t lds_tile, int db, int s, int lane) {
  const int row0 = 32 * s + 8 * (lane >> 4);
  return cat_i16x4(tile_read_t4(lds_tile, row0, 16 * db, lane), tile_read_t4(lds_tile, row0 + 4, 16 * db, lane));
}

// Transposed 32x32x16 A operands (rows = head-dim entries 32 db .. 32 db + 31,
// k = tile rows 16 s4 .. 16 s4 + 15) are read as two ds_read_b64_tr_b16 per
// operand: read tt (0, 1) covers, for lane l, tile row 16 s4 + 8 (l/32) + 4 tt
// + (l%16)/4 at columns 32 db + 16 ((l/16)%2) + 4 (l%4) .. +3.  With tile_swz
// the physical chunk of that read depends on (db, s4, tt) only through tt,
// (db ^ s4) % 2 and db / 2, so 8 per-lane base addresses plus compile-time
// offsets cover all 32 reads of a 64 x 128 tile:
//   address(db, s4, tt) = base[tr32_idx(db, s4, tt)] + tr32_off(s4, tt).
__device__ __forceinline__ void tr32_bases(uint32_t* base, uint32_t lds_tile, int lane) {
  const int li = lane & 15, jj = li >> 2, g1 = (lane >> 4) & 1, bb = (li & 3) >> 1, half = lane >> 5;
#pragma unroll
  for (int y = 0; y < 8; ++y) {
    const int tt = y & 1, db = ((y >> 1) & 1) | ((y >> 2) << 1);   // the representative with s4 = 0
    base[y] = lds_tile + tile_off(8 * half + 4 * tt + jj, 4 * db + 2 * g1 + bb) + 8 * (li & 1) - 1024 * tt;
  }
}
__device__ constexpr int tr32_idx(int db, int s4, int tt) { return tt | (((db ^ s4) & 1) << 1) | ((db >> 1) << 2); }
__device__ constexpr uint32_t tr32_off(int s4, int tt) { return (uint32_t)((16 * s4 + 4 * tt) * 256); }

}  // namespace bd
