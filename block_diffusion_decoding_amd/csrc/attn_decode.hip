// One denoising step of block decoding: the current block of every sequence
// attends to that sequence's KV-cache prefix plus the block itself, with no
// mask (the block is the newest one; paper.rainbus.top digest, novelty
// paragraph on KV-cache reuse across blocks).
//
// Balanced split-KV on gfx950.  Per KV head and row tile (64 query rows = block
// tokens x the query heads of the group) the key tiles of all sequences form
// one line: sequence 0's tiles of 32 keys (prefix keys, then the block's own),
// then sequence 1's, and so on.  The line is cut into R equal contiguous
// ranges, one workgroup each, with R chosen so that about one workgroup per
// resident slot of the chip is launched: every workgroup streams the same
// number of tiles whatever the mix of prefix lengths.
//   decode_split  workgroup = (range, row tile, kv head), range fastest (so
//                 the lines of one range share an XCD).  Four waves own 16
//                 query rows each and share K/V tiles staged through
//                 registers into two swizzled LDS
//                 stages (two tiles in flight in registers while one is
//                 multiplied); the pipeline runs on across sequence
//                 boundaries.  Per tile and wave:
//                   S^T[32 keys x 16 q] = K Q^T  (2 x 4 MFMA 16x16x32)
//                   O^T[128 d x 16 q]  += V^T P^T (8 MFMA 16x16x32, V^T read
//                                                  transposed from LDS)
//                 A sequence that lies wholly inside the range gets its final
//                 rows (O, LSE) directly; any other segment of the range
//                 leaves a partial in slot range + sequence (distinct for
//                 every pair a range meets): (m, l) in fp32 and O / l in bf16.
//                 Outputs of segments that end inside the range wait in LDS
//                 and are stored after the streaming loop.
//   decode_merge  combines the partials of each sequence met by several
//                 ranges: m = max m_s, w_s = l_s 2^(m_s - m),
//                 O = sum w_s O_s / sum w_s, LSE = (m + log2 sum w_s) ln 2, in
//                 fp32 (exact but for the bf16 rounding of each O_s).
// Each K/V byte of the cache is read from HBM once per step.
#include "bd_device.hpp"
#include "bd_kernels.hpp"

#include <algorithm>
#include <mutex>

// The number of workgroups the plan aims for (256 compute units x 3 resident
// workgroups, a limit set by registers); a compile-time knob for tuning builds.
#ifndef BD_DECODE_TARGET_WGS
#define BD_DECODE_TARGET_WGS 768
#endif

namespace bd {
namespace {

constexpr int D = 128;
constexpr int KT = 32;
constexpr int kNW = 4;
constexpr int kThreads = kNW * 64;
constexpr int kRows = 64;                     // query rows per workgroup (4 waves x 16)
constexpr int kTileBytes = KT * D * 2;      // 8 KB
constexpr int kStageBytes = 2 * kTileBytes;
constexpr int kStashBytes = 16 * D * 2 + 16 * 8;           // per wave: 16 rows of bf16 O, (m, l)
constexpr size_t kSmemBytes = 2 * (size_t)kStageBytes + kNW * kStashBytes;   // two stages, the stash
constexpr int kPieces = KT / 4 / kNW;         // 16-byte pieces per thread per tile, of K and of V

__device__ __forceinline__ uint4 ldg16_nt(const void* p) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));

// One tile in flight in registers: this thread's pieces of K and of V.
struct Staged {
  uint4 k[kPieces], v[kPieces];
};

__device__ __forceinline__ void lds_write16(uint32_t lds_addr, const uint4& v) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 w = {v.x, v.y, v.z, v.w};
  *reinterpret_cast<__attribute__((address_space(3))) u32x4*>((uintptr_t)lds_addr) = w;
}
#ifndef BD_DECODE_MIN_RANGE
#define BD_DECODE_MIN_RANGE 8
#endif
#ifndef BD_DECODE_MERGE_BATCH
#define BD_DECODE_MERGE_BATCH 8
#endif
constexpr int kMinRangeTiles = BD_DECODE_MIN_RANGE;   // fewest tiles per range the plan aims for

struct DecParams {
  const uint16_t* q_blk;
  const uint16_t* k_blk;
  const uint16_t* v_blk;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int64_t* prefix_start;  // packed cache: first row of each sequence's prefix
  const int32_t* prefix_len;
  const int32_t* block_table;   // paged cache: [n_seq][max_pages] page of each page_size-key span
  int max_pages, page_size;
  float2* part_ml;   // [lane][R + n_seq][kRows]: (m, l) of each partial row
  uint16_t* part_o;  // [lane][R + n_seq][wave][dp][lane of wave][8]: bf16 O / l of each partial
  uint16_t* o;
  float* lse;
  int n_seq, blk_len, Hq, Hkv, G, rows, row_tiles, R;
  float scale_log2;
};

// Key tiles of sequence s: ceil((prefix_len + blk_len) / KT).
__device__ __forceinline__ int seq_tiles(const DecParams& p, int s) {
  return (p.prefix_len[s] + p.blk_len + KT - 1) / KT;
}

// A 64-bit value that is equal in every lane, made known to be wave-uniform.
__device__ __forceinline__ long long uniform64(long long v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((unsigned long long)v >> 32));
  return (long long)(((unsigned long long)hi << 32) | lo);
}

// Wave-level inclusive prefix sum (64 lanes).
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d, 64);
    if (lane >= d) v += u;
  }
  return v;
}

// Tiles of the line up to and including sequence c + lane, for the chunk of
// 64 sequences starting at c (0 past the last sequence), and the chunk total.
__device__ __forceinline__ int chunk_scan(const DecParams& p, int c, int lane, int& tiles, int& chunk_total) {
  const int s = c + lane;
  tiles = s < p.n_seq ? seq_tiles(p, s) : 0;
  const int incl = wave_incl_scan(tiles, lane);
  chunk_total = __shfl(incl, 63, 64);
  return incl;
}

// The total number of tiles of the line, the first tile x of range r, and the
// sequence s_at holding tile x with the number of tiles before it.  Every lane returns the same values.
// With at most 64 sequences the prefix lengths are read once.
__device__ void line_locate(const DecParams& p, int r, int lane, long long& total, long long& x, int& s_at,
                            long long& before) {
  int tiles0, tot0;
  const int incl0 = chunk_scan(p, 0, lane, tiles0, tot0);
  total = tot0;
  for (int c = 64; c < p.n_seq; c += 64) {
    int t, ct;
    chunk_scan(p, c, lane, t, ct);
    total += ct;
  }
  x = total * r / p.R;   // first tile of range r (ranges split the line evenly)
  s_at = -1;
  before = 0;
  long long acc = 0;
  for (int c = 0; c < p.n_seq; c += 64) {
    int t, ct, incl;
    if (c == 0) {
      t = tiles0;
      ct = tot0;
      incl = incl0;
    } else {
      incl = chunk_scan(p, c, lane, t, ct);
    }
    const unsigned long long hit = __builtin_amdgcn_ballot_w64(c + lane < p.n_seq && acc + incl > x);
    if (hit) {
      const int l = __builtin_ctzll(hit);
      s_at = c + l;
      before = acc + __shfl(incl, l, 64) - __shfl(t, l, 64);
      break;
    }
    acc += ct;
  }
}

// A position on the line: sequence s, its tile j, and that sequence's
// prefix length and tile count.  (Where the prefix rows live is looked up when
// a tile is fetched: keeping the first cache row in the cursor measured 6 %
// slower on the 64-sequence step, from the code the compiler makes of it.)
struct Cursor {
  int s, j, P, tiles;
};

// kPaged: the prefix lives in pages of page_size rows (a multiple of the
// 32-key tile, so a tile of the prefix lies in one page): prefix row j of
// sequence s is row block_table[s][j / page_size] * page_size + j % page_size
// of the page buffer.  Otherwise it is row prefix_start[s] + j of the packed
// cache.
template <bool kPaged>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void decode_split(DecParams p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  // Range fastest: the hardware deals workgroups to the XCDs in turn, so
  // with R a multiple of 8 every line (KV head, row tile) of range r runs on
  // one XCD, which then reads whole cache rows (all heads' 256-byte pieces),
  // and neighbouring ranges run on different XCDs.  Measured against the
  // KV head fastest (one XCD per head): 1.5-3.8 % faster on the 64-sequence
  // step; whole blocks of consecutive ranges per XCD were 4 % slower.
  int bid = blockIdx.x;
  const int r = bid % p.R;
  bid /= p.R;
  const int kvh = bid % p.Hkv;
  const int rt = bid / p.Hkv;
  const int lane_id = rt * p.Hkv + kvh;        // which line

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  const int col = lane & 15, g4 = lane >> 4;
  const int rloc = wave * 16 + col;            // row within the tile
  // partial slot of sequence s met by this range (distinct for every pair)
  auto slot_of = [&](int s) { return (int64_t)lane_id * (p.R + p.n_seq) + r + s; };

  // This workgroup's range [x0, x1) of the line.
  long long total, x0, before;
  int s0;
  line_locate(p, r, lane, total, x0, s0, before);
  total = uniform64(total);
  x0 = uniform64(x0);
  const long long x1 = total * (r + 1) / p.R;
  s0 = __builtin_amdgcn_readfirstlane(s0);
  before = uniform64(before);
  if (x0 >= x1) {
    // An empty range (the line is shorter than R) that falls inside a sequence
    // lies between that sequence's first and last ranges: it leaves a neutral
    // partial so the merge can take every range in between.
    if (x0 > before && g4 == 0) p.part_ml[slot_of(s0) * kRows + rloc] = make_float2(kNegInf, 0.f);
    return;
  }
  const int n_tiles = (int)(x1 - x0);

  // Wave-uniform: read through the constant address space, so the loads are
  // scalar and tracked by lgkmcnt, not by the vmcnt that the tile copies use.
  typedef __attribute__((address_space(4))) const int32_t c_i32;
  typedef __attribute__((address_space(4))) const int64_t c_i64;
  auto cursor_at = [&](int s, int j) {
    Cursor c;
    c.s = __builtin_amdgcn_readfirstlane(s);
    c.j = __builtin_amdgcn_readfirstlane(j);
    c.P = ((c_i32*)(uintptr_t)p.prefix_len)[c.s];
    c.tiles = (c.P + p.blk_len + KT - 1) / KT;
    return c;
  };
  // Physical cache row of prefix row j of sequence s (uniform j: a scalar load of the table).
  auto prow_uniform = [&](int s, int j) __attribute__((always_inline)) -> int64_t {
    const int pg = ((c_i32*)(uintptr_t)p.block_table)[(int64_t)s * p.max_pages + j / p.page_size];
    return (int64_t)pg * p.page_size + j % p.page_size;
  };
  auto prow_lane = [&](int s, int j) __attribute__((always_inline)) -> int64_t {
    const int pg = p.block_table[(int64_t)s * p.max_pages + j / p.page_size];
    return (int64_t)pg * p.page_size + j % p.page_size;
  };
  auto advance = [&](Cursor& c) {
    if (++c.j == c.tiles && c.s + 1 < p.n_seq) c = cursor_at(c.s + 1, 0);
  };

  // Loader: register-staged copies.  fetch() reads the next tile of the line
  // (cursor ld) into registers: each thread its two 16-byte pieces of K and of
  // V (rows 4*nn + lane/16 of the tile, logical chunk (lane%16) ^ swizzle);
  // put() writes them to an LDS stage at the swizzled positions.  A tile
  // wholly inside the cache prefix is 32 consecutive cache rows: a uniform
  // base plus fixed per-lane offsets.  (Measured on gfx950, this path streams
  // HBM at about 6.8 TB/s where global -> LDS copies reach about 6.0.)
  const int64_t rs = (int64_t)p.Hkv * D;
  uint32_t row_off[kPieces];
#pragma unroll
  for (int i = 0; i < kPieces; ++i) {
    const int nn = wave * kPieces + i;
    const int rr = 4 * nn + (lane >> 4);
    row_off[i] = (uint32_t)((rr * rs + 8 * ((lane & 15) ^ tile_swz(rr))) * 2);
  }
  Cursor ld = cursor_at(s0, (int)(x0 - before));
  // Every step issues exactly one fetch (past the range it repeats the last
  // tile, an L2 hit, without moving the cursor): with a fixed number of loads
  // between a fetch and its put, the compiler waits for just that fetch.
  auto fetch = [&](Staged& sg, bool adv) __attribute__((always_inline)) {
    const int key0 = ld.j * KT, kend = ld.P + p.blk_len;
    if (key0 + KT <= ld.P) {
      const int64_t prow0 = kPaged ? prow_uniform(ld.s, key0) : ((c_i64*)(uintptr_t)p.prefix_start)[ld.s] + key0;
      const int64_t row0 = prow0 * rs + (int64_t)kvh * D;
      const char* kg = reinterpret_cast<const char*>(p.k_cache + row0);
      const char* vg = reinterpret_cast<const char*>(p.v_cache + row0);
#pragma unroll
      for (int i = 0; i < kPieces; ++i) {
        sg.k[i] = ldg16_nt(kg + row_off[i]);
        sg.v[i] = ldg16_nt(vg + row_off[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kPieces; ++i) {
        const int nn = wave * kPieces + i;
        const int rr = 4 * nn + (lane >> 4);
        const int c = (lane & 15) ^ tile_swz(rr);
        const int j = min(key0 + rr, kend - 1);
        const int64_t grow = j < ld.P ? (kPaged ? prow_lane(ld.s, j) : p.prefix_start[ld.s] + j) : -1;
        const int64_t brow = ((int64_t)ld.s * p.blk_len + (j - ld.P));
        const uint16_t* ksrc = (grow >= 0 ? p.k_cache + grow * rs : p.k_blk + brow * rs) + kvh * D + 8 * c;
        const uint16_t* vsrc = (grow >= 0 ? p.v_cache + grow * rs : p.v_blk + brow * rs) + kvh * D + 8 * c;
        sg.k[i] = ldg16_nt(ksrc);
        sg.v[i] = ldg16_nt(vsrc);
      }
    }
    if (adv) advance(ld);
  };
  auto put = [&](const Staged& sg, int stage) __attribute__((always_inline)) {
    const uint32_t st = lds0 + stage * kStageBytes;
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const uint32_t dst = st + (wave * kPieces + i) * 1024 + lane * 16;
      lds_write16(dst, sg.k[i]);
      lds_write16(dst + kTileBytes, sg.v[i]);
    }
  };

  const int row = rt * kRows + rloc;           // row within the line: row = hl * blk_len + t
  const bool rvalid = row < p.rows;
  const int hl = rvalid ? row / p.blk_len : 0, tok = rvalid ? row % p.blk_len : 0;
  const int hq = kvh * p.G + hl;
  const float c2 = p.scale_log2;
  // A-operand row of 16-key block kb (0, 1) for lane row rho = col:
  //   key 8*(rho/4) + 4*kb + rho%4
  // so that accumulator entry i of lane (col, g4) in block kb holds key
  //   8*g4 + 4*kb + i,
  // the B-operand k-slice of the PV product over the tile's 32 keys.
  const int arow = 8 * (col >> 2) + (col & 3);
  // LDS byte offsets within a tile: K row 4*kb + arow, chunk g4 (ds = 0); the
  // two transposed V reads of d-block 0 (rows 8*g4 + 4*h + (lane%16)/4,
  // columns 4*(lane%4) .. +3, as tile_read_t16).
  uint32_t kbase[2], vbase[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) kbase[kb] = tile_off(4 * kb + arow, g4);
  {
    const int li = lane & 15;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int vr = 8 * g4 + 4 * h + (li >> 2);
      const int d = 4 * (li & 3);
      vbase[h] = tile_off(vr, d >> 3) + 2 * (d & 7);
    }
  }

  Cursor cc = cursor_at(s0, (int)(x0 - before));   // the tile being multiplied
  bf16x8 qreg[4];
  f32x4 oacc[8];
  float m_use = kNegInf, l_run = 0.f;
  // The Q loads of a segment are waited for here, once per segment.  Left to
  // itself the compiler would instead wait for them (vmcnt(0), which also
  // covers the tile copies in flight) before the first product of every tile.
  auto begin_segment = [&]() {
    const uint16_t* qr = p.q_blk + (((int64_t)cc.s * p.blk_len + tok) * p.Hq + hq) * D + 8 * g4;
#pragma unroll
    for (int t = 0; t < 4; ++t) qreg[t] = as_bf16x8(rvalid ? ldg16(qr + 32 * t) : make_uint4(0, 0, 0, 0));
    vm_wait<0>();
#pragma unroll
    for (int db = 0; db < 8; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_use = kNegInf;
    l_run = 0.f;
  };
  // Segment outputs.  A sequence that lies wholly inside this range gets its
  // final rows (O in bf16 and LSE); otherwise the segment leaves a partial:
  // (m, l) in fp32 and O / l in bf16.  Lane (c, g4) holds rows' entries
  // d = 16 db + 4 g4 + i; packed per pair of d-blocks into chunk dp, element e
  // = d-block 2 dp + e / 4, entry e % 4.
  //
  // A global store inside the streaming loop stalls it: vmcnt retires in
  // order, and the next wait for a tile waits for the store to be
  // acknowledged, which under the read stream is slow (measured: ≈ 60 µs on
  // the 64-sequence step).  So the output of a segment that ends before the
  // range does goes to this wave's LDS stash and reaches memory after the
  // loop (a rarer second such segment is stored directly).
  auto store_out = [&](int s, bool whole, float m, float l, const uint4* w) __attribute__((always_inline)) {
    if (whole) {
      if (!rvalid) return;
      uint16_t* orow = p.o + (((int64_t)s * p.blk_len + tok) * p.Hq + hq) * D + 4 * g4;
#pragma unroll
      for (int dp = 0; dp < 4; ++dp) {
        *reinterpret_cast<uint2*>(orow + 32 * dp) = make_uint2(w[dp].x, w[dp].y);
        *reinterpret_cast<uint2*>(orow + 32 * dp + 16) = make_uint2(w[dp].z, w[dp].w);
      }
      if (p.lse && g4 == 0) p.lse[((int64_t)s * p.Hq + hq) * p.blk_len + tok] = (m + __log2f(l)) * kLn2;
    } else {
      const int64_t slot = slot_of(s);
      if (g4 == 0) p.part_ml[slot * kRows + rloc] = make_float2(m, l);
      uint16_t* po = p.part_o + ((slot * kNW + wave) * 4) * 64 * 8 + lane * 8;
#pragma unroll
      for (int dp = 0; dp < 4; ++dp) stg16(po + dp * 64 * 8, w[dp]);
    }
  };
  const uint32_t stash = lds0 + 2 * kStageBytes + wave * kStashBytes;
  int st_s = -1;
  bool st_whole = false;
  bool seg_from0 = cc.j == 0;   // the current segment began at its sequence's first tile
  auto end_segment = [&](bool last) __attribute__((always_inline)) {
    float l_tot = l_run + __shfl_xor(l_run, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    const bool whole = seg_from0 && cc.j + 1 == cc.tiles;
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    uint4 w[4];
#pragma unroll
    for (int dp = 0; dp < 4; ++dp) {
      const f32x4 a0 = oacc[2 * dp], a1 = oacc[2 * dp + 1];
      w[dp] = make_uint4(pack_bf16x2(a0[0] * inv, a0[1] * inv), pack_bf16x2(a0[2] * inv, a0[3] * inv),
                         pack_bf16x2(a1[0] * inv, a1[1] * inv), pack_bf16x2(a1[2] * inv, a1[3] * inv));
    }
    if (last || st_s >= 0) {
      store_out(cc.s, whole, m_use, l_tot, w);
    } else {
#pragma unroll
      for (int dp = 0; dp < 4; ++dp) lds_write16(stash + (dp * 64 + lane) * 16, w[dp]);
      if (g4 == 0)
        *reinterpret_cast<__attribute__((address_space(3))) f32x2*>((uintptr_t)(stash + 16 * D * 2 + col * 8)) =
            f32x2{m_use, l_tot};
      st_s = __builtin_amdgcn_readfirstlane(cc.s);
      st_whole = whole;
    }
  };
  begin_segment();

  // Pipeline: tile t is multiplied from LDS stage t % 2 while tiles t+1 and
  // t+2 are in flight in the register buffers (tile u in buffer u % 2).  After
  // the products of tile t, tile t+1 goes to stage (t+1) % 2 (free: its
  // previous tile was multiplied before this step's barrier) and the buffer
  // fetches tile t+3.  The loop is unrolled by two so that the buffers are
  // addressed statically.
  Staged sa, sb;
  fetch(sa, n_tiles > 1);
  fetch(sb, n_tiles > 2);
  put(sa, 0);
  fetch(sa, n_tiles > 3);

  auto step = [&](int t, Staged& nxt) __attribute__((always_inline)) {
    __syncthreads();
    const int key0 = cc.j * KT;
    const int kend = cc.P + p.blk_len;
    const uint32_t Kt = lds0 + (t & 1) * kStageBytes;
    const uint32_t Vt = Kt + kTileBytes;

    // All operand reads of the tile first (V's do not depend on the softmax):
    // K rows 4*kb + arow at logical chunk 4*ds + g4, and V^T for d-block db by
    // two transposed reads.  The swizzle touches only chunk bits, so each
    // address is a per-lane base XOR a compile-time constant.
    bf16x8 kop[8], vop[8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) kop[4 * kb + ds] = lds_read_b128(Kt + (kbase[kb] ^ (uint32_t)(ds << 6)));
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ds = 0; ds < 4; ++ds)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) sacc[kb] = mfma_16x16x32(kop[4 * kb + ds], qreg[ds], sacc[kb]);
    if (key0 + KT > kend) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (key0 + 8 * g4 + 4 * kb + i >= kend) sacc[kb][i] = kNegInf;
    }
    // P = exp2(S * scale * log2 e - m_use).  The offset m_use is raised (with
    // the matching rescale of O and l) only when this lane's exponentials
    // would exceed 2^16, or while it is still -inf (the segment's first tile);
    // O and l always share it, so the result is exact up to rounding.
    auto exp8 = [&](float nm, float* pv) {
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[i] = exp2_fast(__builtin_fmaf(sacc[0][i], c2, nm));
        pv[4 + i] = exp2_fast(__builtin_fmaf(sacc[1][i], c2, nm));
        ps += pv[i] + pv[4 + i];
      }
      return ps;
    };
    float pv[8];
    float psum = exp8(-m_use, pv);
    if (__builtin_amdgcn_ballot_w64(!(psum <= 65536.0f))) {
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[kb][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * c2;   // the query row's maximum (its 4 lanes)
      if (mx > m_use) {
        const float alpha = exp2_fast(m_use - mx);   // 0 while m_use is -inf
        m_use = mx;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 8; ++db) oacc[db] *= alpha;
      }
      psum = exp8(m_use == kNegInf ? 0.f : -m_use, pv);
    }
    const bf16x8 pb = pack_bf16x8(pv);
    l_run += psum;
#pragma unroll
    for (int db = 0; db < 8; ++db)
      vop[db] = cat_i16x4(lds_read_tr16(Vt + (vbase[0] ^ (uint32_t)(db << 5))),
                          lds_read_tr16(Vt + (vbase[1] ^ (uint32_t)(db << 5))));
#pragma unroll
    for (int db = 0; db < 8; ++db) oacc[db] = mfma_16x16x32(vop[db], pb, oacc[db]);

    put(nxt, (t + 1) & 1);   // past the range: an unused copy into a stage nobody reads again
    fetch(nxt, t + 4 < n_tiles);

    // end of this sequence's segment: write its partial, move on
    const bool seq_done = cc.j + 1 == cc.tiles;
    if (seq_done || t + 1 == n_tiles) {
      end_segment(t + 1 == n_tiles);
      if (t + 1 < n_tiles) {
        cc = cursor_at(cc.s + 1, 0);
        seg_from0 = true;
        begin_segment();
      }
    } else {
      ++cc.j;
    }
  };
  // Whole pairs in the loop (both buffers fetched on every path to the back
  // edge, so the compiler's waits before each put cover just that buffer).
  int t = 0;
  for (; t + 1 < n_tiles; t += 2) {
    step(t, sb);
    step(t + 1, sa);
  }
  if (t < n_tiles) step(t, sb);
  if (st_s >= 0) {   // this wave's own stash: its LDS writes precede these reads
    uint4 w[4];
#pragma unroll
    for (int dp = 0; dp < 4; ++dp) {
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      const u32x4 v = *reinterpret_cast<__attribute__((address_space(3))) u32x4*>((uintptr_t)(stash + (dp * 64 + lane) * 16));
      w[dp] = make_uint4(v[0], v[1], v[2], v[3]);
    }
    const f32x2 ml = *reinterpret_cast<__attribute__((address_space(3))) f32x2*>((uintptr_t)(stash + 16 * D * 2 + col * 8));
    store_out(st_s, st_whole, ml[0], ml[1], w);
  }
}

// First tile and tile count of sequence n on the line, and the line's total.
// Every lane returns the same values.
__device__ void seq_span(const DecParams& p, int n, int lane, long long& total, long long& start, int& tiles_n) {
  total = 0;
  start = 0;
  tiles_n = 0;
  for (int c = 0; c < p.n_seq; c += 64) {
    int t, ct;
    const int incl = chunk_scan(p, c, lane, t, ct);
    if (n >= c && n < c + 64) {
      const int tn = __shfl(t, n - c, 64);
      start = total + __shfl(incl, n - c, 64) - tn;
      tiles_n = tn;
    }
    total += ct;
  }
}

// Merge: one workgroup per (sequence, line, block of 16 rows); thread
// (dp = t / 64, l = t % 64) owns row 16 * block + l % 16 and the eight entries
// of chunk dp.  The ranges that met sequence n are found from the same cut
// points as in decode_split (range r starts at tile floor(total r / R)); a
// sequence met by one range only was written whole there.  Otherwise
//   m = max m_s,  w_s = l_s 2^(m_s - m),  O = sum w_s O_s / sum w_s,
//   LSE = (m + log2 sum w_s) ln 2,
// in one online pass in fp32 (O_s = the partial's O / l_s, stored in bf16;
// ranges that are empty inside the sequence left l = 0 and are skipped).
__global__ __launch_bounds__(256) void decode_merge(DecParams p) {
  const int lanes = p.row_tiles * p.Hkv;
  int u = blockIdx.x;
  const int wb = u % kNW;
  u /= kNW;
  const int lane_id = u % lanes, n = u / lanes;
  const int kvh = lane_id % p.Hkv, rt = lane_id / p.Hkv;
  const int t = threadIdx.x, dp = t >> 6, ln = t & 63, col = ln & 15, g4 = ln >> 4;
  const int rloc = wb * 16 + col;
  const int row = rt * kRows + rloc;

  long long total, start;
  int tiles_n;
  seq_span(p, n, ln, total, start, tiles_n);
  if (tiles_n <= 0 || total <= 0) return;
  const int r_first = (int)(((start + 1) * p.R - 1) / total);
  const int r_last = (int)(((start + tiles_n) * p.R - 1) / total);
  if (r_first == r_last || row >= p.rows) return;

  // partials in batches of kBatch per round trip to memory
  constexpr int kBatch = BD_DECODE_MERGE_BATCH;
  float m = kNegInf, lsum = 0.f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int r0 = r_first; r0 <= r_last; r0 += kBatch) {
    f32x2 ml[kBatch];
    uint4 w[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int64_t slot = (int64_t)lane_id * (p.R + p.n_seq) + r0 + k + n;
      const bool ok = r0 + k <= r_last;
      const float2 v = ok ? p.part_ml[slot * kRows + rloc] : make_float2(kNegInf, 0.f);
      ml[k] = f32x2{v.x, v.y};
      w[k] = ok ? ldg16(p.part_o + ((slot * kNW + wb) * 4 + dp) * 64 * 8 + ln * 8) : make_uint4(0, 0, 0, 0);
    }
    float mb = m;
#pragma unroll
    for (int k = 0; k < kBatch; ++k)
      if (ml[k][1] > 0.f) mb = fmaxf(mb, ml[k][0]);
    const float a = m == kNegInf ? 0.f : exp2_fast(m - mb);   // rescale of what was summed so far
    lsum *= a;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= a;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      if (!(ml[k][1] > 0.f)) continue;   // empty ranges inside the sequence, and past the last
      const float bw = ml[k][1] * exp2_fast(ml[k][0] - mb);
      const uint32_t ww[4] = {w[k].x, w[k].y, w[k].z, w[k].w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        acc[e] += bw * bf16_bits_to_f32((e & 1) ? ww[e >> 1] >> 16 : ww[e >> 1] & 0xffffu);
      lsum += bw;
    }
    m = mb;
  }
  const float inv = 1.0f / lsum;
  const int hl = row / p.blk_len, tok = row % p.blk_len;
  const int hq = kvh * p.G + hl;
  uint16_t* orow = p.o + (((int64_t)n * p.blk_len + tok) * p.Hq + hq) * D + 32 * dp + 4 * g4;
  *reinterpret_cast<uint2*>(orow) = make_uint2(pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv));
  *reinterpret_cast<uint2*>(orow + 16) =
      make_uint2(pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv));
  if (p.lse && dp == 0 && g4 == 0) p.lse[((int64_t)n * p.Hq + hq) * p.blk_len + tok] = (m + __log2f(lsum)) * kLn2;
}

struct Plan {
  int row_tiles, lanes, R;
};

Plan make_plan(const DecodeShape& s) {
  Plan pl;
  const int rows = s.blk_len * (s.n_q_heads / s.n_kv_heads);
  pl.row_tiles = (rows + kRows - 1) / kRows;
  pl.lanes = s.n_kv_heads * pl.row_tiles;
  // Tiles of the line when every prefix has the largest length (an upper
  // bound: the ranges are cut from the actual line on the device).
  const long long line_max = (long long)s.n_seq * (((long long)s.max_prefix_len + s.blk_len + KT - 1) / KT);
  long long R = std::max<long long>(1, BD_DECODE_TARGET_WGS / pl.lanes);
  R = std::min<long long>(R, std::max<long long>(1, line_max / kMinRangeTiles));
  // A multiple of 8 puts the lines of a range on one XCD (workgroups go to
  // the 8 XCDs in turn): the nearest one, within the workgroup target.
  if (R >= 8) {
    const long long up = (R + 4) / 8 * 8;
    R = up * pl.lanes <= std::max<long long>(BD_DECODE_TARGET_WGS, 8LL * pl.lanes) ? up : R / 8 * 8;
  }
  pl.R = (int)R;
  return pl;
}

size_t part_slots(const DecodeShape& s, const Plan& pl) {
  return (size_t)pl.lanes * ((size_t)pl.R + s.n_seq) * kRows;
}

}  // namespace

size_t decode_workspace_bytes(const DecodeShape& s, int /*is_bf16*/) {
  const Plan pl = make_plan(s);
  return part_slots(s, pl) * (sizeof(float2) + D * sizeof(uint16_t));
}

namespace {

hipError_t launch_decode_impl(const void* q_blk, const void* k_blk, const void* v_blk, const void* k_cache,
                              const void* v_cache, const int64_t* prefix_start, const int32_t* block_table,
                              int max_pages, int page_size, const int32_t* prefix_len, void* o, float* lse,
                              void* ws, const DecodeShape& s, hipStream_t st) {
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [] {
    attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_split<false>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSmemBytes);
    if (attr_err == hipSuccess)
      attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_split<true>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSmemBytes);
  });
  if (attr_err != hipSuccess) return attr_err;
  const Plan pl = make_plan(s);
  const size_t slots = part_slots(s, pl);
  DecParams p;
  p.q_blk = static_cast<const uint16_t*>(q_blk);
  p.k_blk = static_cast<const uint16_t*>(k_blk);
  p.v_blk = static_cast<const uint16_t*>(v_blk);
  p.k_cache = static_cast<const uint16_t*>(k_cache);
  p.v_cache = static_cast<const uint16_t*>(v_cache);
  p.prefix_start = prefix_start;
  p.prefix_len = prefix_len;
  p.block_table = block_table;
  p.max_pages = max_pages;
  p.page_size = page_size;
  p.part_ml = reinterpret_cast<float2*>(ws);
  p.part_o = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(ws) + slots * sizeof(float2));
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.n_seq = s.n_seq;
  p.blk_len = s.blk_len;
  p.Hq = s.n_q_heads;
  p.Hkv = s.n_kv_heads;
  p.G = s.n_q_heads / s.n_kv_heads;
  p.rows = s.blk_len * p.G;
  p.row_tiles = pl.row_tiles;
  p.R = pl.R;
  p.scale_log2 = s.scale * kLog2e;
  const dim3 grid((unsigned)((long long)pl.R * pl.lanes));
  if (block_table) hipLaunchKernelGGL(decode_split<true>, grid, dim3(kThreads), kSmemBytes, st, p);
  else hipLaunchKernelGGL(decode_split<false>, grid, dim3(kThreads), kSmemBytes, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge, dim3((unsigned)((long long)s.n_seq * pl.lanes * kNW)), dim3(256), 0, st, p);
  return hipGetLastError();
}

// Append each finished block (n_masked_left[s] == 0, or every block without
// that array) to its sequence's pages: rows t of the block's K and V go to
// prefix row prefix_len[s] + t; then prefix_len[s] grows by blk_len.  One
// workgroup per sequence; 16-byte copies.  A block whose rows would pass the
// sequence's last page is left out (the caller allocates pages first).
__global__ __launch_bounds__(256) void kv_append(const uint16_t* __restrict__ k_blk,
                                                 const uint16_t* __restrict__ v_blk, uint16_t* __restrict__ k_pages,
                                                 uint16_t* __restrict__ v_pages,
                                                 const int32_t* __restrict__ block_table, int max_pages,
                                                 int page_size, int32_t* __restrict__ prefix_len,
                                                 const int32_t* __restrict__ n_masked_left, int blk_len,
                                                 int row_elems) {
  const int s = blockIdx.x;
  if (n_masked_left && n_masked_left[s] != 0) return;
  const int P = prefix_len[s];
  if ((int64_t)P + blk_len > (int64_t)max_pages * page_size) return;
  const int per_row = row_elems / 8;   // 16-byte pieces per row
  for (int c = threadIdx.x; c < blk_len * per_row; c += blockDim.x) {
    const int t = c / per_row, k8 = c - t * per_row;
    const int j = P + t;
    const int64_t dst = ((int64_t)block_table[(int64_t)s * max_pages + j / page_size] * page_size + j % page_size) *
                            row_elems + k8 * 8;
    const int64_t src = ((int64_t)s * blk_len + t) * row_elems + k8 * 8;
    *reinterpret_cast<uint4*>(k_pages + dst) = *reinterpret_cast<const uint4*>(k_blk + src);
    *reinterpret_cast<uint4*>(v_pages + dst) = *reinterpret_cast<const uint4*>(v_blk + src);
  }
  __syncthreads();   // every thread has read P
  if (threadIdx.x == 0) prefix_len[s] = P + blk_len;
}

}  // namespace

hipError_t launch_decode_bf16(const void* q_blk, const void* k_blk, const void* v_blk, const void* k_cache,
                              const void* v_cache, const int64_t* prefix_start, const int32_t* prefix_len,
                              void* o, float* lse, void* ws, const DecodeShape& s, hipStream_t st) {
  return launch_decode_impl(q_blk, k_blk, v_blk, k_cache, v_cache, prefix_start, nullptr, 0, 0, prefix_len, o, lse,
                            ws, s, st);
}

hipError_t launch_decode_bf16_paged(const void* q_blk, const void* k_blk, const void* v_blk, const void* k_pages,
                                    const void* v_pages, const int32_t* block_table, int max_pages, int page_size,
                                    const int32_t* prefix_len, void* o, float* lse, void* ws, const DecodeShape& s,
                                    hipStream_t st) {
  return launch_decode_impl(q_blk, k_blk, v_blk, k_pages, v_pages, nullptr, block_table, max_pages, page_size,
                            prefix_len, o, lse, ws, s, st);
}

hipError_t launch_kv_append_bf16(const void* k_blk, const void* v_blk, void* k_pages, void* v_pages,
                                 const int32_t* block_table, int max_pages, int page_size, int32_t* prefix_len,
                                 const int32_t* n_masked_left, int n_seq, int blk_len, int n_kv_heads, int head_dim,
                                 hipStream_t st) {
  hipLaunchKernelGGL(kv_append, dim3((unsigned)n_seq), dim3(256), 0, st, static_cast<const uint16_t*>(k_blk),
                     static_cast<const uint16_t*>(v_blk), static_cast<uint16_t*>(k_pages),
                     static_cast<uint16_t*>(v_pages), block_table, max_pages, page_size, prefix_len, n_masked_left,
                     blk_len, n_kv_heads * head_dim);
  return hipGetLastError();
}

}  // namespace bd
