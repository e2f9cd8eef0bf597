// Cumulative-mass block selection ("streaming top-k" of the explainer's
// section 3.1: blocks are taken in descending score until their running sum
// reaches gamma).  Defined here as: the fewest indices, taken in descending
// value with ties broken by lower index first, whose sum is >= gamma * sum(x);
// gamma >= 1 takes every index.
//
// Instead of sorting, the cut value theta = x_(k*) is found exactly by a
// bisection over the bit patterns of non-negative floats (ordered like the
// values): theta is the largest value t with sum_{x >= t} x >= gamma * T.
// Everything above theta is taken, plus the lowest-index ties at theta that
// are still needed.  Sums are fp64 with a fixed reduction order.
#pragma once

#include "fp_common.hpp"

namespace fp {

__device__ __forceinline__ void set_bit_lds(uint32_t *m, int j) { atomicOr(&m[j >> 5], 1u << (j & 31)); }

// Whole workgroup: x[0..n) in LDS (values >= 0), result bits in lmask (LDS,
// ceil(n/32) words, cleared here).  redd: LDS double[>= nwaves], redi: int[>= nwaves].
__device__ void block_select(const float *x, int n, float gamma, uint32_t *lmask, double *redd,
                             int *redi) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int nw = (n + 31) >> 5;
  for (int w = tid; w < nw; w += nt) lmask[w] = 0u;
  double part = 0.0;
  for (int j = tid; j < n; j += nt) part += (double)x[j];
  const double T = block_sum(part, redd);   // contains barriers: lmask clear is visible
  if (gamma >= 1.0f) {
    for (int j = tid; j < n; j += nt) set_bit_lds(lmask, j);
    __syncthreads();
    return;
  }
  const double target = (double)gamma * T;
  if (!(target > 0.0)) {                    // all-zero input: the first index in order is 0
    if (tid == 0) lmask[0] = 1u;
    __syncthreads();
    return;
  }
  uint32_t lo = 0u, hi = 0x7f800000u;       // f(lo) >= target > f(hi)
  while (hi - lo > 1u) {
    const uint32_t mid = lo + ((hi - lo) >> 1);
    const float th = __uint_as_float(mid);
    double s = 0.0;
    for (int j = tid; j < n; j += nt) s += (x[j] >= th) ? (double)x[j] : 0.0;
    s = block_sum(s, redd);
    if (s >= target) lo = mid; else hi = mid;
  }
  const float th = __uint_as_float(lo);
  double a = 0.0;
  int eq = 0;
  for (int j = tid; j < n; j += nt) {
    if (x[j] > th) a += (double)x[j];
    eq += (x[j] == th) ? 1 : 0;
  }
  const double A = block_sum(a, redd);
  const int neq = block_sum_int(eq, redi);
  int c = 1;
  while (c < neq && A + (double)c * (double)th < target) ++c;
  for (int j = tid; j < n; j += nt)
    if (x[j] > th || (neq <= c && x[j] == th)) set_bit_lds(lmask, j);
  if (neq > c && tid == 0) {                // rare: only some ties at the cut are needed
    int taken = 0;
    for (int j = 0; j < n && taken < c; ++j)
      if (x[j] == th) { set_bit_lds(lmask, j); ++taken; }
  }
  __syncthreads();
}

// One wave: x[0..n) in LDS (values >= 0).  Returns, per lane, nothing; the
// selected bits are OR-ed into words[0 .. ceil(n/32)) (a per-wave LDS array
// the caller clears).  Elements are visited as j = lane + 64 * k.
__device__ void wave_select(const float *x, int n, float gamma, uint32_t *words) {
  const int lane = threadIdx.x & 63;
  double part = 0.0;
  for (int j = lane; j < n; j += 64) part += (double)x[j];
  const double T = wave_sum(part);
  if (gamma >= 1.0f || !(gamma * T > 0.0)) {
    const bool all = gamma >= 1.0f;
    for (int j = lane; j < n; j += 64)
      if (all || j == 0) atomicOr(&words[j >> 5], 1u << (j & 31));
    return;
  }
  const double target = (double)gamma * T;
  uint32_t lo = 0u, hi = 0x7f800000u;
  while (hi - lo > 1u) {
    const uint32_t mid = lo + ((hi - lo) >> 1);
    const float th = __uint_as_float(mid);
    double s = 0.0;
    for (int j = lane; j < n; j += 64) s += (x[j] >= th) ? (double)x[j] : 0.0;
    s = wave_sum(s);
    if (s >= target) lo = mid; else hi = mid;
  }
  const float th = __uint_as_float(lo);
  double a = 0.0;
  int eq = 0;
  for (int j = lane; j < n; j += 64) {
    if (x[j] > th) a += (double)x[j];
    eq += (x[j] == th) ? 1 : 0;
  }
  const double A = wave_sum(a);
  const int neq = wave_sum_int(eq);
  int c = 1;
  while (c < neq && A + (double)c * (double)th < target) ++c;
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

}  // namespace fp
