// Drives every entry point of include/bd.h through its argument checks and,
// with the runtime stand-ins of hip_runtime_stub.cpp, through the host side of
// its launchers, in a host-only build with the address and undefined-behaviour
// sanitizers.  Tensor arguments are host addresses that nothing dereferences
// (no kernel runs); each check states the status the contract in bd.h gives.
// Prints "abi driver: N checks passed" and exits 0, or lists the failures and
// exits 1; a sanitizer report aborts the process.
#include "bd.h"

#include <climits>
#include <cmath>
#include <cstdio>
#include <cstring>

extern long long g_stub_launches;

namespace {

int g_checks = 0, g_failed = 0;

void expect(bd_status got, bd_status want, const char* what, int line) {
  ++g_checks;
  if (got != want) {
    std::fprintf(stderr, "line %d: %s returned %d (%s), expected %d (%s)\n", line, what, (int)got,
                 bd_status_string(got), (int)want, bd_status_string(want));
    ++g_failed;
  }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

void expect_true(bool ok, const char* what, int line) {
  ++g_checks;
  if (!ok) {
    std::fprintf(stderr, "line %d: %s does not hold\n", line, what);
    ++g_failed;
  }
}
#define EXPECT_TRUE(cond) expect_true((cond), #cond, __LINE__)

alignas(16) char g_buf[4096];
void* const P = g_buf;          // a 16-byte aligned stand-in for any tensor
void* const M = g_buf + 2;      // a misaligned one
float* const F = reinterpret_cast<float*>(g_buf);
int32_t* const I32 = reinterpret_cast<int32_t*>(g_buf);
int64_t* const I64 = reinterpret_cast<int64_t*>(g_buf);
uint8_t* const U8 = reinterpret_cast<uint8_t*>(g_buf);
const hipStream_t S0 = nullptr;
const size_t kHuge = (size_t)1 << 60;   // a workspace size no call needs
const float kNaN = std::nanf("");
const float kInf = INFINITY;

void attention_forward() {
  EXPECT(bd_attn_fwd(nullptr, P, P, P, F, 1, 64, 2, 1, 128, 32, 0.f, BD_BF16, S0), BD_ERR_NULL);
  EXPECT(bd_attn_fwd(P, P, P, nullptr, F, 1, 64, 2, 1, 128, 32, 0.f, BD_BF16, S0), BD_ERR_NULL);
  EXPECT(bd_attn_fwd(P, P, P, P, F, 0, 64, 2, 1, 128, 32, 0.f, BD_BF16, S0), BD_ERR_SHAPE);
  EXPECT(bd_attn_fwd(P, P, P, P, F, 1, -5, 2, 1, 128, 32, 0.f, BD_BF16, S0), BD_ERR_SHAPE);
  EXPECT(bd_attn_fwd(P, P, P, P, F, 1, 64, 3, 2, 128, 32, 0.f, BD_BF16, S0), BD_ERR_SHAPE);
  EXPECT(bd_attn_fwd(P, P, P, P, F, 1, 64, 2, 1, 128, 0, 0.f, BD_BF16, S0), BD_ERR_SHAPE);
  EXPECT(bd_attn_fwd(P, P, P, P, F, 1, 64, 2, 1, 128, 32, kNaN, BD_BF16, S0), BD_ERR_VALUE);
  EXPECT(bd_attn_fwd(P, P, P, P, F, 1, 64, 2, 1, 128, 32, kInf, BD_BF16, S0), BD_ERR_VALUE);
  EXPECT(bd_attn_fwd(P, P, P, P, F, 1, 64, 2, 1, 64, 32, 0.f, BD_BF16, S0), BD_ERR_UNSUPPORTED);
  EXPECT(bd_attn_fwd(P, P, P, P, F, 1, 64, 2, 1, 256, 32, 0.f, BD_F32, S0), BD_ERR_UNSUPPORTED);
  EXPECT(bd_attn_fwd(P, P, P, P, F, 1, 64, 2, 1, 128, 32, 0.f, (bd_dtype)7, S0), BD_ERR_UNSUPPORTED);
  EXPECT(bd_attn_fwd(M, P, P, P, F, 1, 64, 2, 1, 128, 32, 0.f, BD_BF16, S0), BD_ERR_ALIGNMENT);
  // sizes whose product passes every integer width
  EXPECT(bd_attn_fwd(P, P, P, P, F, INT_MAX, INT_MAX, INT_MAX, 1, 128, 32, 0.f, BD_BF16, S0), BD_ERR_SHAPE);
  EXPECT(bd_attn_fwd(P, P, P, P, F, 1, INT_MAX, 65536, 1, 128, INT_MAX, 0.f, BD_BF16, S0), BD_ERR_SHAPE);
  const long long before = g_stub_launches;
  EXPECT(bd_attn_fwd(P, P, P, P, F, 2, 16384, 16, 8, 128, 32, 0.f, BD_BF16, S0), BD_OK);
  EXPECT(bd_attn_fwd(P, P, P, P, nullptr, 1, 77, 4, 2, 128, 5, 0.3f, BD_BF16, S0), BD_OK);
  EXPECT(bd_attn_fwd(P, P, P, P, F, 3, 129, 6, 3, 64, 200, 0.f, BD_F32, S0), BD_OK);
  EXPECT(bd_attn_fwd(P, P, P, P, F, 1, 1, 1, 1, 1, 1, 0.f, BD_F32, S0), BD_OK);
  EXPECT_TRUE(g_stub_launches >= before + 4);
}

void attention_backward() {
  const size_t ws = bd_attn_bwd_workspace_size(2, 16384, 16, 8, 128);
  EXPECT_TRUE(ws >= (size_t)2 * 2 * 16 * 16384 * 4);
  EXPECT_TRUE(bd_attn_bwd_workspace_size(0, 64, 2, 1, 128) == 0);
  EXPECT_TRUE(bd_attn_bwd_workspace_size(1, 64, 2, 0, 128) == 0);
  EXPECT_TRUE(bd_attn_bwd_workspace_size(1, 64, 3, 2, 128) == 0);
  // a shape the call rejects has no workspace size either
  EXPECT_TRUE(bd_attn_bwd_workspace_size(INT_MAX, INT_MAX, INT_MAX, 1, 128) == 0);
  EXPECT(bd_attn_bwd(P, P, P, P, nullptr, P, P, P, P, P, kHuge, 1, 64, 2, 1, 128, 32, 0.f, BD_BF16, S0),
         BD_ERR_NULL);
  EXPECT(bd_attn_bwd(P, P, P, P, F, P, P, P, nullptr, P, kHuge, 1, 64, 2, 1, 128, 32, 0.f, BD_BF16, S0),
         BD_ERR_NULL);
  EXPECT(bd_attn_bwd(P, P, P, P, F, P, P, P, P, nullptr, kHuge, 1, 64, 2, 1, 128, 32, 0.f, BD_BF16, S0),
         BD_ERR_WORKSPACE);
  EXPECT(bd_attn_bwd(P, P, P, P, F, P, P, P, P, P, ws - 1, 2, 16384, 16, 8, 128, 32, 0.f, BD_BF16, S0),
         BD_ERR_WORKSPACE);
  EXPECT(bd_attn_bwd(P, P, P, P, F, P, P, M, P, P, ws, 2, 16384, 16, 8, 128, 32, 0.f, BD_BF16, S0),
         BD_ERR_ALIGNMENT);
  EXPECT(bd_attn_bwd(P, P, P, P, F, P, P, P, P, M, ws, 2, 16384, 16, 8, 128, 32, 0.f, BD_BF16, S0),
         BD_ERR_ALIGNMENT);
  EXPECT(bd_attn_bwd(P, P, P, P, F, P, P, P, P, M, kHuge, 2, 100, 4, 4, 32, 16, 0.f, BD_F32, S0), BD_ERR_ALIGNMENT);
  EXPECT(bd_attn_bwd(P, P, P, P, F, P, P, P, P, P, kHuge, INT_MAX, INT_MAX, INT_MAX, 1, 128, 32, 0.f, BD_BF16,
                     S0),
         BD_ERR_SHAPE);
  EXPECT(bd_attn_bwd(P, P, P, P, F, P, P, P, P, P, ws, 2, 16384, 16, 8, 128, 32, 0.f, BD_BF16, S0), BD_OK);
  EXPECT(bd_attn_bwd(P, P, P, P, F, P, P, P, P, P, kHuge, 1, 200, 4, 2, 128, 7, 0.f, BD_BF16, S0), BD_OK);
  EXPECT(bd_attn_bwd(P, P, P, P, F, P, P, P, P, P, kHuge, 2, 100, 4, 4, 32, 16, 0.f, BD_F32, S0), BD_OK);
}

void decode() {
  const size_t ws = bd_attn_decode_workspace_size(64, 32, 16384, 16, 8, 128);
  EXPECT_TRUE(ws > 0);
  EXPECT_TRUE(bd_attn_decode_workspace_size(0, 32, 100, 16, 8, 128) == 0);
  EXPECT_TRUE(bd_attn_decode_workspace_size(1, 32, -1, 16, 8, 128) == 0);
  EXPECT_TRUE(bd_attn_decode_workspace_size(1, 32, 100, 16, 5, 128) == 0);
  // shapes the call rejects: no size, and no overflow on the way
  EXPECT_TRUE(bd_attn_decode_workspace_size(INT_MAX, INT_MAX, INT_MAX, INT_MAX, 1, 128) == 0);
  EXPECT_TRUE(bd_attn_decode_workspace_size(INT_MAX, 32, INT_MAX, 16, 8, 128) == 0);
  EXPECT(bd_attn_decode_block(P, P, P, P, P, nullptr, I32, 100, P, F, 2, 32, 16, 8, 128, 0.f, BD_BF16, P, kHuge,
                              S0),
         BD_ERR_NULL);
  EXPECT(bd_attn_decode_block(P, P, P, nullptr, P, I64, I32, 100, P, F, 2, 32, 16, 8, 128, 0.f, BD_BF16, P, kHuge,
                              S0),
         BD_ERR_NULL);
  EXPECT(bd_attn_decode_block(P, P, P, P, P, I64, I32, -1, P, F, 2, 32, 16, 8, 128, 0.f, BD_BF16, P, kHuge, S0),
         BD_ERR_SHAPE);
  EXPECT(bd_attn_decode_block(P, P, P, P, P, I64, I32, INT_MAX, P, F, 2, 32, 16, 8, 128, 0.f, BD_BF16, P, kHuge,
                              S0),
         BD_ERR_SHAPE);
  EXPECT(bd_attn_decode_block(P, P, P, P, P, I64, I32, 100, P, F, INT_MAX, INT_MAX, INT_MAX, 1, 128, 0.f, BD_BF16,
                              P, kHuge, S0),
         BD_ERR_SHAPE);
  EXPECT(bd_attn_decode_block(P, P, P, P, M, I64, I32, 100, P, F, 2, 32, 16, 8, 128, 0.f, BD_BF16, P, kHuge, S0),
         BD_ERR_ALIGNMENT);
  EXPECT(bd_attn_decode_block(P, P, P, P, P, I64, I32, 16384, P, F, 64, 32, 16, 8, 128, 0.f, BD_BF16, P, ws - 1,
                              S0),
         BD_ERR_WORKSPACE);
  EXPECT(bd_attn_decode_block(P, P, P, P, P, I64, I32, 16384, P, F, 64, 32, 16, 8, 128, 0.f, BD_BF16, M, ws, S0),
         BD_ERR_ALIGNMENT);
  EXPECT(bd_attn_decode_block(P, P, P, P, P, I64, I32, 16384, P, F, 64, 32, 16, 8, 128, kNaN, BD_BF16, P, ws, S0),
         BD_ERR_VALUE);
  EXPECT(bd_attn_decode_block(P, P, P, P, P, I64, I32, 16384, P, F, 64, 32, 16, 8, 128, 0.f, BD_BF16, P, ws, S0),
         BD_OK);
  // no prefix at all: the cache may be NULL
  EXPECT(bd_attn_decode_block(P, P, P, nullptr, nullptr, I64, I32, 0, P, F, 3, 7, 4, 2, 128, 0.f, BD_BF16, P,
                              kHuge, S0),
         BD_OK);
  EXPECT(bd_attn_decode_block(P, P, P, P, P, I64, I32, 100, P, nullptr, 3, 32, 4, 2, 64, 0.f, BD_F32, nullptr, 0,
                              S0),
         BD_OK);
  // one sequence past the bound's worth of ranges, and many sequences
  EXPECT(bd_attn_decode_block(P, P, P, P, P, I64, I32, 4096, P, F, 1, 32, 16, 8, 128, 0.f, BD_BF16, P, kHuge, S0),
         BD_OK);
  EXPECT(bd_attn_decode_block(P, P, P, P, P, I64, I32, 1000, P, F, 1000, 32, 16, 8, 128, 0.f, BD_BF16, P, kHuge,
                              S0),
         BD_OK);
}

void decode_paged() {
  EXPECT(bd_attn_decode_block_paged(P, P, P, P, P, nullptr, 8, 32, I32, 200, P, F, 2, 32, 16, 8, 128, 0.f,
                                    BD_BF16, P, kHuge, S0),
         BD_ERR_NULL);
  EXPECT(bd_attn_decode_block_paged(P, P, P, P, P, I32, 8, 48, I32, 200, P, F, 2, 32, 16, 8, 128, 0.f, BD_BF16, P,
                                    kHuge, S0),
         BD_ERR_UNSUPPORTED);
  EXPECT(bd_attn_decode_block_paged(P, P, P, P, P, I32, 8, 0, I32, 200, P, F, 2, 32, 16, 8, 128, 0.f, BD_BF16, P,
                                    kHuge, S0),
         BD_ERR_UNSUPPORTED);
  EXPECT(bd_attn_decode_block_paged(P, P, P, P, P, I32, 6, 32, I32, 200, P, F, 2, 32, 16, 8, 128, 0.f, BD_BF16, P,
                                    kHuge, S0),
         BD_ERR_SHAPE);
  // page counts and sizes whose product passes 32 bits
  EXPECT(bd_attn_decode_block_paged(P, P, P, P, P, I32, INT_MAX, INT_MAX - 31, I32, INT_MAX, P, F, 2, 32, 16, 8,
                                    128, 0.f, BD_BF16, P, kHuge, S0),
         BD_ERR_SHAPE);
  EXPECT(bd_attn_decode_block_paged(P, P, P, P, P, I32, INT_MAX, 1 << 30, I32, INT_MAX, P, F, 2, 32, 16, 8, 128,
                                    0.f, BD_BF16, P, kHuge, S0),
         BD_ERR_SHAPE);
  EXPECT(bd_attn_decode_block_paged(P, P, P, P, P, I32, 8, 32, I32, 200, P, F, 2, 32, 16, 8, 128, 0.f, BD_F32, P,
                                    kHuge, S0),
         BD_ERR_UNSUPPORTED);
  EXPECT(bd_attn_decode_block_paged(P, P, P, P, P, I32, 8, 32, I32, 200, P, F, 2, 32, 16, 8, 128, 0.f, BD_BF16, P,
                                    0, S0),
         BD_ERR_WORKSPACE);
  EXPECT(bd_attn_decode_block_paged(P, P, P, P, P, I32, 8, 32, I32, 200, P, F, 2, 32, 16, 8, 128, 0.f, BD_BF16, M,
                                    kHuge, S0),
         BD_ERR_ALIGNMENT);
  EXPECT(bd_attn_decode_block_paged(P, P, P, P, P, I32, 8, 32, I32, 200, P, F, 2, 32, 16, 8, 128, 0.f, BD_BF16, P,
                                    kHuge, S0),
         BD_OK);
  EXPECT(bd_attn_decode_block_paged(P, P, P, P, P, I32, 70, 256, I32, 16384, P, F, 64, 32, 16, 8, 128, 0.f, BD_BF16,
                                    P, kHuge, S0),
         BD_OK);
}

void kv_append() {
  EXPECT(bd_kv_append_block(P, P, P, P, nullptr, 8, 32, I32, I32, 2, 32, 8, 128, BD_BF16, S0), BD_ERR_NULL);
  EXPECT(bd_kv_append_block(P, P, P, P, I32, 8, 0, I32, I32, 2, 32, 8, 128, BD_BF16, S0), BD_ERR_SHAPE);
  EXPECT(bd_kv_append_block(P, P, P, P, I32, 0, 32, I32, I32, 2, 32, 8, 128, BD_BF16, S0), BD_ERR_SHAPE);
  EXPECT(bd_kv_append_block(P, P, P, P, I32, 8, 32, I32, I32, 2, 32, 8, 128, BD_F32, S0), BD_ERR_UNSUPPORTED);
  EXPECT(bd_kv_append_block(P, P, P, P, I32, 8, 32, I32, I32, 2, 32, 3, 5, BD_BF16, S0), BD_ERR_UNSUPPORTED);
  // a row wider than any index type: rejected, not wrapped
  EXPECT(bd_kv_append_block(P, P, P, P, I32, 8, 32, I32, I32, 2, 32, 1 << 20, 1 << 12, BD_BF16, S0), BD_ERR_SHAPE);
  EXPECT(bd_kv_append_block(M, P, P, P, I32, 8, 32, I32, I32, 2, 32, 8, 128, BD_BF16, S0), BD_ERR_ALIGNMENT);
  EXPECT(bd_kv_append_block(P, P, P, P, I32, 8, 32, I32, nullptr, 2, 32, 8, 128, BD_BF16, S0), BD_OK);
  EXPECT(bd_kv_append_block(P, P, P, P, I32, 8, 32, I32, I32, 64, 32, 8, 128, BD_BF16, S0), BD_OK);
}

void commit() {
  const int V = 151936;
  const size_t ws = bd_confidence_commit_workspace_size(64, 32, V);
  EXPECT_TRUE(ws > 0);
  EXPECT_TRUE(bd_confidence_commit_workspace_size(0, 32, V) == 0);
  EXPECT_TRUE(bd_confidence_commit_workspace_size(64, 32, -3) == 0);
  EXPECT_TRUE(bd_confidence_commit_workspace_size(INT_MAX, 1024, INT_MAX) == 0);
  EXPECT(bd_confidence_commit(nullptr, V, 64, 32, V, BD_BF16, 0.95f, BD_FALLBACK_TOP1, I32, U8, F, I32, I32, I32, P,
                              ws, S0),
         BD_ERR_NULL);
  EXPECT(bd_confidence_commit(P, V - 1, 64, 32, V, BD_BF16, 0.95f, BD_FALLBACK_TOP1, I32, U8, F, I32, I32, I32, P,
                              ws, S0),
         BD_ERR_SHAPE);
  EXPECT(bd_confidence_commit(P, V, 1, 1025, V, BD_BF16, 0.95f, BD_FALLBACK_TOP1, I32, U8, F, I32, I32, I32, P,
                              kHuge, S0),
         BD_ERR_UNSUPPORTED);
  EXPECT(bd_confidence_commit(P, V, 64, 32, V, (bd_dtype)9, 0.95f, BD_FALLBACK_TOP1, I32, U8, F, I32, I32, I32, P,
                              ws, S0),
         BD_ERR_UNSUPPORTED);
  EXPECT(bd_confidence_commit(P, V, 64, 32, V, BD_BF16, kNaN, BD_FALLBACK_TOP1, I32, U8, F, I32, I32, I32, P, ws,
                              S0),
         BD_ERR_VALUE);
  EXPECT(bd_confidence_commit(P, V, 64, 32, V, BD_BF16, 0.95f, (bd_fallback)2, I32, U8, F, I32, I32, I32, P, ws,
                              S0),
         BD_ERR_VALUE);
  EXPECT(bd_confidence_commit(P, V, 64, 32, V, BD_BF16, 0.95f, BD_FALLBACK_TOP1, I32, U8, F, I32, I32, I32, P,
                              ws - 1, S0),
         BD_ERR_WORKSPACE);
  EXPECT(bd_confidence_commit(P, V, 64, 32, V, BD_BF16, 0.95f, BD_FALLBACK_TOP1, I32, U8, F, I32, I32, I32, M,
                              ws, S0),
         BD_ERR_ALIGNMENT);
  EXPECT(bd_confidence_commit_rowwise(P, V, 64, 32, V, BD_BF16, F, BD_FALLBACK_TOP1, I32, U8, F, I32, I32, I32, M,
                                      ws, S0),
         BD_ERR_ALIGNMENT);
  EXPECT(bd_confidence_commit(P, INT64_MAX, INT_MAX, 1024, INT_MAX, BD_BF16, 0.95f, BD_FALLBACK_TOP1, I32, U8, F,
                              I32, I32, I32, P, kHuge, S0),
         BD_ERR_SHAPE);
  EXPECT(bd_confidence_commit(P, V, 64, 32, V, BD_BF16, 0.95f, BD_FALLBACK_TOP1, I32, U8, F, I32, I32, I32, P, ws,
                              S0),
         BD_OK);
  EXPECT(bd_confidence_commit(M, 77, 3, 5, 77, BD_F32, 2.f, BD_FALLBACK_NONE, I32, U8, nullptr, nullptr, nullptr,
                              nullptr, P, kHuge, S0),
         BD_OK);
  // the no-allocation form: the same checks, and its fixed scratch as the limit
  EXPECT(bd_confidence_commit_noalloc(P, V, 64, 32, V, BD_BF16, 0.95f, BD_FALLBACK_TOP1, I32, U8, F, I32, I32, I32,
                                      S0),
         BD_OK);
  EXPECT(bd_confidence_commit_noalloc(P, V, 262144 / 32, 32, V, BD_BF16, 0.95f, BD_FALLBACK_TOP1, I32, U8, F, I32,
                                      I32, I32, S0),
         BD_OK);
  EXPECT(bd_confidence_commit_noalloc(P, V, 262144 / 32 + 1, 32, V, BD_BF16, 0.95f, BD_FALLBACK_TOP1, I32, U8, F,
                                      I32, I32, I32, S0),
         BD_ERR_SCRATCH);
  EXPECT(bd_confidence_commit_noalloc(nullptr, V, 64, 32, V, BD_BF16, 0.95f, BD_FALLBACK_TOP1, I32, U8, F, I32,
                                      I32, I32, S0),
         BD_ERR_NULL);
  // one threshold per row
  EXPECT(bd_confidence_commit_rowwise(P, V, 64, 32, V, BD_BF16, nullptr, BD_FALLBACK_TOP1, I32, U8, F, I32, I32,
                                      I32, P, ws, S0),
         BD_ERR_NULL);
  EXPECT(bd_confidence_commit_rowwise(P, V, 64, 32, V, BD_BF16, F, BD_FALLBACK_TOP1, I32, U8, F, I32, I32, I32, P,
                                      ws, S0),
         BD_OK);
}

void commit_sampled() {
  const int V = 151936;
  const size_t ws = bd_confidence_commit_sampled_workspace_size(64, 32, V);
  EXPECT_TRUE(ws > 0);
  EXPECT_TRUE(bd_confidence_commit_sampled_workspace_size(64, 0, V) == 0);
  EXPECT_TRUE(bd_confidence_commit_sampled_workspace_size(INT_MAX, 1024, INT_MAX) == 0);
  auto call = [&](int n_seq, int vocab, float temp, int top_k, float top_p, float thr, size_t ws_bytes) {
    return bd_confidence_commit_sampled(P, vocab, n_seq, 32, vocab, BD_BF16, temp, 7, 3, top_k, top_p, thr,
                                        BD_FALLBACK_TOP1, I32, U8, F, I32, I32, I32, P, ws_bytes, S0);
  };
  EXPECT(call(64, V, 0.f, 0, 1.f, 0.9f, ws), BD_ERR_VALUE);
  EXPECT(call(64, V, -1.f, 0, 1.f, 0.9f, ws), BD_ERR_VALUE);
  EXPECT(call(64, V, kInf, 0, 1.f, 0.9f, ws), BD_ERR_VALUE);
  EXPECT(call(64, V, kNaN, 0, 1.f, 0.9f, ws), BD_ERR_VALUE);
  EXPECT(call(64, V, 1.f, -1, 1.f, 0.9f, ws), BD_ERR_VALUE);
  EXPECT(call(64, V, 1.f, 0, 0.f, 0.9f, ws), BD_ERR_VALUE);
  EXPECT(call(64, V, 1.f, 0, 1.5f, 0.9f, ws), BD_ERR_VALUE);
  EXPECT(call(64, V, 1.f, 0, kNaN, 0.9f, ws), BD_ERR_VALUE);
  EXPECT(call(64, V, 1.f, 0, 1.f, kNaN, ws), BD_ERR_VALUE);
  EXPECT(call(64, 155649, 1.f, 50, 1.f, 0.9f, kHuge), BD_ERR_UNSUPPORTED);
  EXPECT(call(64, V, 1.f, 0, 1.f, 0.9f, ws - 1), BD_ERR_WORKSPACE);
  EXPECT(bd_confidence_commit_sampled(P, V, 64, 32, V, BD_BF16, 1.f, 7, 3, 0, 1.f, 0.9f, BD_FALLBACK_TOP1, I32, U8,
                                      F, I32, I32, I32, M, ws, S0),
         BD_ERR_ALIGNMENT);
  EXPECT(call(INT_MAX / 32, INT_MAX, 1.f, 0, 1.f, 0.9f, kHuge), BD_ERR_SHAPE);
  EXPECT(call(64, V, 1.f, 0, 1.f, 0.9f, ws), BD_OK);
  EXPECT(call(64, V, 0.7f, 50, 1.f, 0.9f, ws), BD_OK);
  EXPECT(call(64, V, 1.f, 0, 0.9f, 0.9f, ws), BD_OK);
  EXPECT(call(1, 155648, 1.f, 1, 0.5f, 0.9f, kHuge), BD_OK);
}

void lmhead() {
  const int V = 151936, H = 2048;
  const size_t ws = bd_lmhead_commit_workspace_size(1, 32, V);
  EXPECT_TRUE(ws > 0);
  EXPECT_TRUE(bd_lmhead_commit_workspace_size(1, 0, V) == 0);
  EXPECT_TRUE(bd_lmhead_commit_workspace_size(INT_MAX, 1024, V) == 0);
  auto call = [&](const void* hidden, int64_t hs, int64_t wsd, int n_seq, int hidden_dim, float thr, size_t wsb) {
    return bd_lmhead_commit(hidden, hs, P, wsd, n_seq, 32, hidden_dim, V, thr, BD_FALLBACK_TOP1, I32, U8, F, I32,
                            I32, I32, P, wsb, S0);
  };
  EXPECT(call(nullptr, H, H, 1, H, 0.9f, ws), BD_ERR_NULL);
  EXPECT(call(P, H - 1, H, 1, H, 0.9f, ws), BD_ERR_SHAPE);
  EXPECT(call(P, H, H, 1, 100, 0.9f, ws), BD_ERR_UNSUPPORTED);
  EXPECT(call(P, 4096, 4096, 1, 4096, 0.9f, ws), BD_ERR_UNSUPPORTED);
  EXPECT(call(M, H, H, 1, H, 0.9f, ws), BD_ERR_ALIGNMENT);
  EXPECT(call(P, H + 4, H, 1, H, 0.9f, ws), BD_ERR_ALIGNMENT);
  EXPECT(call(P, H, H, 1, H, kNaN, ws), BD_ERR_VALUE);
  EXPECT(call(P, H, H, INT_MAX, H, 0.9f, kHuge), BD_ERR_SHAPE);
  EXPECT(call(P, H, H, 1, H, 0.9f, ws - 1), BD_ERR_WORKSPACE);
  EXPECT(bd_lmhead_commit(P, H, P, H, 1, 32, H, V, 0.9f, BD_FALLBACK_TOP1, I32, U8, F, I32, I32, I32, M, ws, S0),
         BD_ERR_ALIGNMENT);
  EXPECT(call(P, H, H, 1, H, 0.9f, ws), BD_OK);
  EXPECT(call(P, 1024, 1024, 4, 1024, 0.5f, kHuge), BD_OK);
}

void strings_and_version() {
  for (int s = 0; s <= 8; ++s) {
    const char* t = bd_status_string((bd_status)s);
    EXPECT_TRUE(t != nullptr && std::strcmp(t, "unknown status") != 0);
  }
  EXPECT_TRUE(std::strcmp(bd_status_string((bd_status)99), "unknown status") == 0);
  EXPECT_TRUE(std::strcmp(bd_status_string((bd_status)-1), "unknown status") == 0);
  EXPECT_TRUE(bd_version() > 0);
  EXPECT_TRUE(bd_last_hip_error() == 0);
}

}  // namespace

int main() {
  attention_forward();
  attention_backward();
  decode();
  decode_paged();
  kv_append();
  commit();
  commit_sampled();
  lmhead();
  strings_and_version();
  if (g_failed) {
    std::fprintf(stderr, "abi driver: %d of %d checks failed\n", g_failed, g_checks);
    return 1;
  }
  std::printf("abi driver: %d checks passed, %lld launches\n", g_checks, g_stub_launches);
  return 0;
}
