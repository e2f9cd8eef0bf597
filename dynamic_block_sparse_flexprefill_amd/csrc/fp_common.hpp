// Device helpers shared by the gfx950 kernels of libfpattn: vector types,
// matrix-core (MFMA) wrappers, bf16 conversion and wave / workgroup
// reductions.  gfx950 only (wave64, 32x32 MFMA tiles).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kD = 128;                 // head dimension
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -3.0e38f;     // finite "minus infinity" for running maxima

// ---------------------------------------------------------------- MFMA
// 32x32x16 bf16 -> fp32.  Operand A: lane l holds row (l % 32) and 8
// consecutive k values of half (l / 32); B likewise with column (l % 32).
// Result: acc[r] is row 8*(r/4) + 4*(l/32) + (r%4), column l % 32.
__device__ __forceinline__ f32x16 mfma_bf16(const u32x4 a, const u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 32x32x32 int8 -> int32, same lane roles with 16 int8 k values per lane.
__device__ __forceinline__ i32x16 mfma_i8(const u32x4 a, const u32x4 b, i32x16 c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a),
                                               __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
}

// Row index (within a 32x32 tile) of accumulator element r on lane `lane`.
__device__ __forceinline__ int acc_row(int r, int lane) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// Two fp32 -> packed bf16 (round to nearest even; one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
// 2^x on the transcendental unit, without a denormal fix-up (results below 2^-126 flush
// to zero).  Inputs here are at most the rescale headroom: 16 in the statistics, 24 in
// the attention.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- direct-to-LDS loads
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// One direct load: the 64 lanes' 16 B from g fill LDS bytes [lds, lds + 1024),
// lane L writing bytes [16 L, 16 L + 16).  Issued from inline assembly: the
// compiler then neither tracks the LDS write (so it inserts no wait for it
// before unrelated LDS reads) nor reuses M0; the caller waits for vmcnt(0)
// before the barrier that publishes the buffer.
__device__ __forceinline__ void lds_dma16(const void *g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}

// Wave-uniform LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(const lds_u8 *)p);
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima), as a builtin
// so that the compiler's own wait placement knows of it.
constexpr int kWaitVm0 = 0x0f70;

// ---------------------------------------------------------------- reductions
// Butterfly partners without LDS traffic: steps 0-3 are DPP moves inside each
// 16-lane row (lane ^ 1, lane ^ 2, then the mirrors i <-> 7 - i and
// i <-> 15 - i, which pair lanes holding equal partial results), step 4 pairs
// rows 0/1 and 2/3 (v_permlane16_swap), step 5 the two 32-lane halves
// (v_permlane32_swap).  Each step combines a lane with exactly one partner, so
// after step k every lane of a 2^(k+1)-lane group holds the same value.
template <int STEP>
__device__ __forceinline__ uint32_t bfly_partner(uint32_t v) {
  if constexpr (STEP == 0) return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, true);
  else if constexpr (STEP == 1) return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, true);
  else if constexpr (STEP == 2) return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xF, 0xF, true);
  else if constexpr (STEP == 3) return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xF, 0xF, true);
  else if constexpr (STEP == 4) {
    const auto s = __builtin_amdgcn_permlane16_swap(v, v, false, false);   // {own or row below, own or row above}
    return ((threadIdx.x >> 4) & 1) ? s[0] : s[1];
  } else {
    const auto s = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return ((threadIdx.x >> 5) & 1) ? s[0] : s[1];
  }
}
template <int STEP, typename T>
__device__ __forceinline__ T bfly(T x) {
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, bfly_partner<STEP>(__builtin_bit_cast(uint32_t, x)));
  } else {
    static_assert(sizeof(T) == 8, "32- or 64-bit values");
    const u32x2 w = __builtin_bit_cast(u32x2, x);
    return __builtin_bit_cast(T, u32x2{bfly_partner<STEP>(w[0]), bfly_partner<STEP>(w[1])});
  }
}
// The value of lane ^ 32.
template <typename T>
__device__ __forceinline__ T xor32(T x) { return bfly<5>(x); }

// Reduction over the first NSTEP butterfly steps (6: the whole wave, 5: each 32-lane half).
template <int NSTEP, typename T, typename Op>
__device__ __forceinline__ T bfly_reduce(T x, Op op) {
  x = op(x, bfly<0>(x));
  x = op(x, bfly<1>(x));
  x = op(x, bfly<2>(x));
  x = op(x, bfly<3>(x));
  if constexpr (NSTEP > 4) x = op(x, bfly<4>(x));
  if constexpr (NSTEP > 5) x = op(x, bfly<5>(x));
  return x;
}
template <typename T>
__device__ __forceinline__ T wave_sum(T x) { return bfly_reduce<6>(x, [](T a, T b) { return a + b; }); }
__device__ __forceinline__ float wave_max(float x) { return bfly_reduce<6>(x, [](float a, float b) { return fmaxf(a, b); }); }
__device__ __forceinline__ int wave_sum_int(int x) { return bfly_reduce<6>(x, [](int a, int b) { return a + b; }); }
__device__ __forceinline__ int wave_min_int(int x) { return bfly_reduce<6>(x, [](int a, int b) { return min(a, b); }); }
// Sum over each 32-lane half.
__device__ __forceinline__ float half_sum(float x) { return bfly_reduce<5>(x, [](float a, float b) { return a + b; }); }

// Workgroup-wide sum / max; `red` is LDS scratch of at least (blockDim/64)
// elements.  Every thread gets the result.  The order of additions is fixed
// (wave butterflies, then waves in index order), so results are reproducible.
template <typename T>
__device__ __forceinline__ T block_sum(T x, T *red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  x = wave_sum(x);
  __syncthreads();
  if (lane == 0) red[w] = x;
  __syncthreads();
  T s = red[0];
  for (int i = 1; i < nw; ++i) s += red[i];
  return s;
}
__device__ __forceinline__ float block_max(float x, float *red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  x = wave_max(x);
  __syncthreads();
  if (lane == 0) red[w] = x;
  __syncthreads();
  float s = red[0];
  for (int i = 1; i < nw; ++i) s = fmaxf(s, red[i]);
  return s;
}
__device__ __forceinline__ int block_sum_int(int x, int *red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  x = wave_sum_int(x);
  __syncthreads();
  if (lane == 0) red[w] = x;
  __syncthreads();
  int s = red[0];
  for (int i = 1; i < nw; ++i) s += red[i];
  return s;
}

}  // namespace fp
