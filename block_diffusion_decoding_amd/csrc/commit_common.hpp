// Per-row confidence state shared by the commit kernels (the logits reduce and
// the fused output-projection reduce) and their decide step.
//
// A row's (max m, lowest argmax idx, sum of exp(x - m)) is associative: chunks
// of the vocabulary reduce on their own and merge in any grouping, with the
// lowest id kept on ties; a NaN or +Inf anywhere marks the row invalid.
#pragma once

#include "bd_device.hpp"

namespace bd {

struct Partial {
  float m;    // max of the chunk (-inf if the chunk holds only -inf)
  float s;    // sum over the chunk of exp(x - m)
  int idx;    // lowest id reaching m
  int bad;    // chunk holds a NaN or +Inf
};

// The sums below are of exp((x - m) / tau) = 2^((x - m) c) with the exponent
// scale c = log2(e) / tau (tau = 1, i.e. c = log2 e, for the plain softmax).
//
// Merge (m2, s2, i2) into (m, s, i).  Sums are kept relative to their max.
__device__ __forceinline__ void merge_state(float& m, float& s, int& idx, float m2, float s2, int i2,
                                            float c = kLog2e) {
  if (m2 > m) {
    s = s * exp2_fast((m - m2) * c) + s2;
    m = m2;
    idx = i2;
  } else if (m2 == m) {
    s += s2;
    idx = min(idx, i2);
  } else {
    s += s2 * exp2_fast((m2 - m) * c);
  }
}

// Running per-thread state over the ids it has seen (in increasing order):
// m = max, idx = lowest id reaching m, s = sum exp(x - m), bad = a NaN was
// summed before a later rescale could hide it.  A NaN element makes s NaN; a
// +Inf element makes m +Inf and s NaN; an element -Inf contributes 0.
struct RowState {
  float m = kNegInf, s = 0.f;
  float mb = 0.f;   // m * c once m is finite; 0 while m = -inf (then every exponent is -inf)
  int idx = 0x7fffffff, bad = 0;
};

// A new maximum mx > st.m at id: rescale the sum (a NaN summed so far is
// recorded first, since the rescale by 0 could hide it).
__device__ __forceinline__ void raise_max(RowState& st, float mx, int id, float c = kLog2e) {
  st.bad |= st.s != st.s;
  st.s = st.m == kNegInf ? 0.f : st.s * exp2_fast((st.m - mx) * c);
  st.m = mx;
  st.mb = mx * c;
  st.idx = id;
}

// Fold the N values starting at vocabulary id `base` (all valid).
template <int N>
__device__ __forceinline__ void fold_vec(const float* x, int base, RowState& st, float c = kLog2e) {
  float vmax = x[0];
#pragma unroll
  for (int j = 1; j < N; ++j) vmax = fmaxf(vmax, x[j]);
  if (vmax > st.m) {   // new maximum (rare after the first few vectors)
    int j0 = N - 1;
#pragma unroll
    for (int j = N - 2; j >= 0; --j) j0 = x[j] == vmax ? j : j0;
    raise_max(st, vmax, base + j0, c);
  }
  float e[N];
#pragma unroll
  for (int j = 0; j < N; ++j) e[j] = exp2_fast(__builtin_fmaf(x[j], c, -st.mb));
#pragma unroll
  for (int w = 1; w < N; w *= 2)
#pragma unroll
    for (int j = 0; j < N; j += 2 * w) e[j] += e[j + w];
  st.s += e[0];
}

// A single value (ragged tail / unaligned rows).
__device__ __forceinline__ void fold_one(float x, int id, RowState& st, float c = kLog2e) {
  if (x > st.m) raise_max(st, x, id, c);
  st.s += exp2_fast(__builtin_fmaf(x, c, -st.mb));
}

// The state as a partial, with NaN / +Inf folded into the flag.
__device__ __forceinline__ Partial to_partial(const RowState& st) {
  Partial r{st.m, st.s, st.idx, st.bad | (st.s != st.s) | (st.m == __builtin_huge_valf())};
  if (r.m == kNegInf) r.s = 0.f;
  return r;
}

// Merge q into p (an invalid side makes the result invalid).
__device__ __forceinline__ void merge_partial(Partial& p, const Partial& q, float c = kLog2e) {
  if (!p.bad && !q.bad) merge_state(p.m, p.s, p.idx, q.m, q.s, q.idx, c);
  p.bad |= q.bad;
}

}  // namespace bd
