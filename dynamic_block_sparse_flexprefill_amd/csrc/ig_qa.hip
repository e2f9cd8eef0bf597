// Query-aware rows of sparse-index generation.
//
// The re-telling ("FPGA加速动态稀疏注意力技术解析与优化", maplevalley.com.cn)
// section 1.1 describes the query-aware pattern as choosing key blocks from
// the current query content, with block-level index generation for every
// query block; the explainer ("FPGA24成果：FAST-Prefill稀疏注意力加速器",
// yunpan.plus) section 1.2 says its blocks spread over different rows and
// columns.  Read here as, for query block i of a query-aware head h:
//   e[j] = sigma * mean(Q_h block i) . mean(K_g block j),  j <= i
//   J(h, i) = Sel(softmax_{j<=i}(e), gamma) u {0, i}
// with Sel the cumulative-mass selection (explainer section 3.1).
//
// Only the Q blocks of heads the divergence test labelled query-aware are
// read.  One workgroup per (head, R consecutive query blocks): the R pooled
// queries share every pooled-key read; each wave then selects its rows and
// writes them as bit sets (one bit per key block).
#include "fp_common.hpp"
#include "fp_internal.hpp"
#include "fp_select.hpp"

namespace fp {
namespace {

struct QaArgs {
  const uint8_t *Q;
  const float *sQ;
  int S, N, B, G, R, nw32;
  float sigma, gamma;
  const uint8_t *pattern;
  const float *kbar;
  uint32_t *qabits;
};

constexpr int kQaThreads = 256;

template <bool I8>
__global__ void __launch_bounds__(kQaThreads) k_ig_qa(QaArgs a) {
  const int h = blockIdx.y;
  if (a.pattern[h] != FP_PATTERN_QUERY_AWARE) return;
  extern __shared__ __attribute__((aligned(16))) float smem[];
  const int N = a.N, B = a.B, S = a.S, R = a.R;
  const int i0 = blockIdx.x * R;
  const int rows = min(R, N - i0);
  const int g = h / a.G;
  float *ev = smem;                       // [R][N] logits / weights
  float *qb = ev + (size_t)R * N;         // [R][128] pooled queries
  float *tmp = qb + R * 128;              // [32][128] partial sums
  uint32_t *words = (uint32_t *)(tmp + 32 * 128);   // [4 waves][nw32]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // 1. Pool each query block (16-byte loads; rows split over thread groups).
  constexpr int EPC = I8 ? 16 : 8;        // elements per 16-byte chunk
  constexpr int CPR = 128 / EPC;          // chunks per row
  constexpr int RG = kQaThreads / CPR;    // row groups
  const int ch = tid % CPR, rg = tid / CPR;
  for (int r = 0; r < rows; ++r) {
    float acc[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = 0.0f;
    const size_t tok0 = (size_t)h * S + (size_t)(i0 + r) * B;
    for (int row = rg; row < B; row += RG) {
      const size_t tok = tok0 + row;
      const u32x4 v = *(const u32x4 *)(a.Q + tok * (I8 ? 128 : 256) + ch * 16);
      if (!I8) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += bf16lo(v[e]);
          acc[2 * e + 1] += bf16hi(v[e]);
        }
      } else {
        const float s = a.sQ[tok];
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] += s * (float)(int8_t)((v[e >> 2] >> (8 * (e & 3))) & 0xff);
      }
    }
#pragma unroll
    for (int e = 0; e < EPC; ++e) tmp[rg * 128 + ch * EPC + e] = acc[e];
    __syncthreads();
    if (tid < 128) {
      float s = 0.0f;
      for (int q = 0; q < RG; ++q) s += tmp[q * 128 + tid];
      qb[r * 128 + tid] = s / (float)B;
    }
    __syncthreads();
  }

  // 2. Pooled logits e[r][j] for j <= i0 + r.
  const int jmax = i0 + rows - 1;
  for (int j = tid; j <= jmax; j += kQaThreads) {
    const float4 *kr = (const float4 *)(a.kbar + ((size_t)g * N + j) * 128);
    float acc[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[r] = 0.0f;
    for (int c = 0; c < 32; ++c) {
      const float4 k4 = kr[c];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        if (r < rows) {
          const float *q = qb + r * 128 + 4 * c;
          acc[r] += q[0] * k4.x + q[1] * k4.y + q[2] * k4.z + q[3] * k4.w;
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 8; ++r)
      if (r < rows && j <= i0 + r) ev[(size_t)r * N + j] = a.sigma * acc[r];
  }
  __syncthreads();

  // 3. One wave per row: softmax weights, selection, bit-set row.
  uint32_t *wd = words + wave * a.nw32;
  for (int r = wave; r < rows; r += kQaThreads / 64) {
    const int i = i0 + r, n = i + 1;
    float *x = ev + (size_t)r * N;
    float mx = kNegBig;
    for (int j = lane; j < n; j += 64) mx = fmaxf(mx, x[j]);
    mx = wave_max(mx);
    for (int j = lane; j < n; j += 64) x[j] = expf(x[j] - mx);
    const int nwr = (i >> 5) + 1;
    for (int w = lane; w < nwr; w += 64) wd[w] = 0u;
    wave_select(x, n, a.gamma, wd);
    if (lane == 0) {
      atomicOr(&wd[0], 1u);
      atomicOr(&wd[i >> 5], 1u << (i & 31));
    }
    uint32_t *dst = a.qabits + ((size_t)h * N + i) * a.nw32;
    for (int w = lane; w < nwr; w += 64) dst[w] = wd[w];
  }
}

}  // namespace

hipError_t launch_ig_qa(const Plan &p, bool i8, const void *Q, const float *sQ, float gamma,
                        const uint8_t *pattern, const Work &w, hipStream_t st) {
  QaArgs a;
  a.Q = (const uint8_t *)Q;
  a.sQ = sQ;
  a.S = p.S; a.N = p.N; a.B = p.B; a.G = p.G; a.nw32 = p.nw32;
  a.R = p.N >= 2048 ? (p.N >= 4096 ? 2 : 4) : 8;
  a.sigma = 1.0f / sqrtf((float)p.d);
  a.gamma = gamma;
  a.pattern = pattern;
  a.kbar = w.kbar;
  a.qabits = w.qabits;
  const size_t lds = sizeof(float) * ((size_t)a.R * p.N + a.R * 128 + 32 * 128) +
                     sizeof(uint32_t) * 4 * p.nw32;
  dim3 grid((p.N + a.R - 1) / a.R, p.Hq);
  if (i8) {
    hipError_t e = hipFuncSetAttribute((const void *)k_ig_qa<true>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_ig_qa<true>, grid, dim3(kQaThreads), lds, st, a);
  } else {
    hipError_t e = hipFuncSetAttribute((const void *)k_ig_qa<false>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_ig_qa<false>, grid, dim3(kQaThreads), lds, st, a);
  }
  return hipGetLastError();
}

}  // namespace fp
