// Cumulative-mass block selection ("streaming top-k" of the explainer's
// section 3.1: blocks are taken in descending score until their running sum
// reaches gamma).  Defined here as: the fewest indices, taken in descending
// value with ties broken by lower index first, whose sum is >= gamma * sum(x);
// gamma >= 1 takes every index.
//
// One wave does the whole search with fixed-order fp32 sums (lane partials,
// then a butterfly), so results are reproducible run to run.  Two methods:
//  * greedy: the maxima are extracted in exactly that order (value descending,
//    lowest index among equal values) until the running sum reaches gamma*T
//    -- used when that takes at most GS extractions (by default kGreedySteps,
//    half as many for rows of more than 1024 values, whose extraction steps
//    cost twice as much; callers whose rows rarely finish in few steps pass
//    fewer);
//  * bisection: the cut value theta = x_(k*) is the largest t with
//    sum_{x >= t} x >= gamma * T, found by bisection over the bit patterns of
//    non-negative floats (ordered like the values); everything above theta
//    is taken, plus the lowest-index ties at theta still needed.
#pragma once

#include "fp_common.hpp"

namespace fp {

// x[0..n) in LDS (values >= 0; elements visited as j = lane + 64 k).  Selected
// bits are OR-ed into words[0 .. ceil(n/32)) (LDS, cleared by the caller).
__device__ __forceinline__ void wave_select_lds(const float *x, int n, float gamma, uint32_t *words) {
  const int lane = threadIdx.x & 63;
  float part = 0.0f, mxl = 0.0f;
  for (int j = lane; j < n; j += 64) {
    part += x[j];
    mxl = fmaxf(mxl, x[j]);
  }
  const float T = wave_sum(part);
  const float target = gamma * T;
  if (gamma >= 1.0f || !(target > 0.0f)) {   // everything, or an all-zero input (index 0)
    const bool all = gamma >= 1.0f;
    for (int j = lane; j < n; j += 64)
      if (all || j == 0) atomicOr(&words[j >> 5], 1u << (j & 31));
    return;
  }
  // f(lo) >= target (f(0) = T), f(hi) = 0 < target (hi is above the maximum)
  uint32_t lo = 0u, hi = __float_as_uint(wave_max(mxl)) + 1u;
  while (hi - lo > 1u) {
    const uint32_t mid = lo + ((hi - lo) >> 1);
    const float th = __uint_as_float(mid);
    float s = 0.0f;
#pragma unroll 8
    for (int j = lane; j < n; j += 64) s += (x[j] >= th) ? x[j] : 0.0f;
    s = wave_sum(s);
    if (s >= target) lo = mid; else hi = mid;
  }
  const float th = __uint_as_float(lo);
  float a = 0.0f;
  int eq = 0;
  for (int j = lane; j < n; j += 64) {
    if (x[j] > th) a += x[j];
    eq += (x[j] == th) ? 1 : 0;
  }
  const float A = wave_sum(a);
  const int neq = wave_sum_int(eq);
  int c = 1;
  while (c < neq && A + (float)c * th < target) ++c;
  int carried = 0;                          // ties taken in index order
  for (int base = 0; base < n; base += 64) {
    const int j = base + lane;
    const float xv = j < n ? x[j] : -1.0f;
    const bool is_eq = (j < n) && (xv == th);
    const uint64_t eqm = __ballot(is_eq);
    const int rank = carried + __popcll(eqm & ((1ull << lane) - 1ull));
    const bool take = (j < n) && (xv > th || (is_eq && rank < c));
    if (take) atomicOr(&words[j >> 5], 1u << (j & 31));
    carried += __popcll(eqm);
  }
}

constexpr int kGreedySteps = 24;

// n <= 64 * VPL: the values live in registers (VPL per lane, element lane + 64 k
// in slot k), so every pass of the search is unrolled register work.  Per-lane
// sums visit the elements in the same order for any VPL (absent slots add 0),
// so the selection does not depend on which VPL serves a row.
// wave_select_vals takes the values already in registers: v[k] = element lane + 64 k, or -1 for
// the slots past n.
template <int VPL, int GS = (VPL > 16 ? kGreedySteps / 2 : kGreedySteps)>
__device__ __forceinline__ void wave_select_vals(const float (&v)[VPL], int n, float gamma, uint32_t *words) {
  static_assert(VPL >= 1 && VPL <= 32, "one bit of `taken` per slot");
  const int lane = threadIdx.x & 63;
  float part = 0.0f, mxl = 0.0f;
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    if (lane + 64 * k < n) {
      part += v[k];
      mxl = fmaxf(mxl, v[k]);
    }
  }
  const float T = wave_sum(part);
  const float target = gamma * T;
  if (gamma >= 1.0f || !(target > 0.0f)) {
    const bool all = gamma >= 1.0f;
    for (int j = lane; j < n; j += 64)
      if (all || j == 0) atomicOr(&words[j >> 5], 1u << (j & 31));
    return;
  }
  // greedy extraction
  constexpr int steps = GS;
  uint32_t taken = 0u;
  float cum = 0.0f;
  bool done = false;
  for (int step = 0; step < steps && step < n; ++step) {
    float bv = -1.0f;
    int bk = -1;
#pragma unroll
    for (int k = 0; k < VPL; ++k)
      if (!((taken >> k) & 1u) && v[k] > bv) {
        bv = v[k];
        bk = k;
      }
    const float M = wave_max(bv);
    const int jmin = wave_min_int((bk >= 0 && bv == M) ? lane + 64 * bk : 0x7fffffff);
    if (lane == (jmin & 63)) taken |= 1u << (jmin >> 6);
    cum += M;
    if (cum >= target) {
      done = true;
      break;
    }
  }
  if (done) {
#pragma unroll
    for (int k = 0; k < VPL; ++k)
      if ((taken >> k) & 1u) {
        const int j = lane + 64 * k;
        atomicOr(&words[j >> 5], 1u << (j & 31));
      }
    return;
  }
  // bisection
  uint32_t lo = 0u, hi = __float_as_uint(wave_max(mxl)) + 1u;
  while (hi - lo > 1u) {
    const uint32_t mid = lo + ((hi - lo) >> 1);
    const float th = __uint_as_float(mid);
    float sacc = 0.0f;
#pragma unroll
    for (int k = 0; k < VPL; ++k) sacc += (v[k] >= th) ? v[k] : 0.0f;   // v = -1 never counts
    sacc = wave_sum(sacc);
    if (sacc >= target) lo = mid; else hi = mid;
  }
  const float th = __uint_as_float(lo);
  float a = 0.0f;
  int eq = 0;
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    if (v[k] > th) a += v[k];
    eq += (v[k] == th) ? 1 : 0;
  }
  const float A = wave_sum(a);
  const int neq = wave_sum_int(eq);
  int c = 1;
  while (c < neq && A + (float)c * th < target) ++c;
  int carried = 0;
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    const int j = lane + 64 * k;
    const bool is_eq = (v[k] == th);
    const uint64_t eqm = __ballot(is_eq);
    const int rank = carried + __popcll(eqm & ((1ull << lane) - 1ull));
    if (v[k] > th || (is_eq && rank < c)) atomicOr(&words[j >> 5], 1u << (j & 31));
    carried += __popcll(eqm);
  }
}


template <int VPL>
__device__ __forceinline__ void wave_select_reg(const float *x, int n, float gamma, uint32_t *words) {
  const int lane = threadIdx.x & 63;
  float v[VPL];
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    const int j = lane + 64 * k;
    v[k] = j < n ? x[j] : -1.0f;             // -1: not an element
  }
  wave_select_vals<VPL>(v, n, gamma, words);
}

// The register form sized to the row (the cost of a search pass grows with VPL),
// up to MAXV values per lane; longer rows search in LDS.  MAXV = 32 costs about
// 20 more registers than 16, so kernels whose occupancy matters take 32 only
// when their rows can exceed 1024 elements.
template <int MAXV = 16>
__device__ __forceinline__ void wave_select(const float *x, int n, float gamma, uint32_t *words) {
  static_assert(MAXV == 16 || MAXV == 32, "register forms for up to 1024 or 2048 elements");
  if (n <= 256) wave_select_reg<4>(x, n, gamma, words);
  else if (n <= 512) wave_select_reg<8>(x, n, gamma, words);
  else if (n <= 1024) wave_select_reg<16>(x, n, gamma, words);
  else if (MAXV == 32 && n <= 2048) wave_select_reg<MAXV>(x, n, gamma, words);
  else wave_select_lds(x, n, gamma, words);
}

}  // namespace fp
