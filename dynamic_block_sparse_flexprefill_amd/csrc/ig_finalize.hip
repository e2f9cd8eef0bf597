// Per-head finalisation of sparse-index generation.
//
// Flex-Prefill's pattern decision, as the explainer ("FPGA24成果：FAST-Prefill
// 稀疏注意力加速器", yunpan.plus) section 1.2 and the re-telling
// ("FPGA加速动态稀疏注意力技术解析与优化", maplevalley.com.cn) section 1.1
// describe it: the last query block is the representative query; a
// Jensen-Shannon divergence decides per head between the query-aware and the
// vertical-slash pattern (threshold tau, typically 0.1).  Read here as:
//   p  = softmax_j(sigma * mean(Q_last) . mean(K_j))   pooled estimate
//   v  = vertical block mass,  sl = slash block mass (from the statistics pass)
//   D  = JSD(p, v) with the natural log; query-aware iff D < tau.
// For vertical-slash heads the key-block columns Sel(v, gamma) and the
// diagonal offsets Sel(sl, gamma) are chosen here (explainer section 3.1,
// cumulative threshold gamma); the rows are expanded later.
//
// One workgroup per query head; every per-head vector of length N lives in LDS.
#include <float.h>

#include "fp_common.hpp"
#include "fp_internal.hpp"
#include "fp_select.hpp"

namespace fp {
namespace {

struct FinArgs {
  const uint8_t *Q;
  const float *sQ;
  int S, N, B, G, nw32;
  float sigma, gamma, tau;
  const float *lo, *hi, *kbar;
  const float *pe;          // pooled-estimate logits [Hq][N] from the statistics, or NULL
  uint8_t *pattern;
  float *jsd, *stats;
  uint32_t *sel;
};

constexpr int kFinThreads = 1024;
constexpr int kFinRowGroups = 32;     // row groups of the last-block query mean (LDS: [32][128] partials)

template <bool I8>
__global__ void __launch_bounds__(kFinThreads) k_ig_finalize(FinArgs a) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  const int N = a.N, B = a.B, S = a.S;
  float *ev = smem;                 // [N] logits, then softmax weights
  float *vv = ev + N;               // [N] vertical mass
  float *sv = vv + N;               // [N] slash mass
  float *qb = sv + N;               // [128] mean query of the last block
  float *qpart = qb + 128;          // [kFinRowGroups][128] row-group partial sums
  uint32_t *msk = (uint32_t *)(qpart + kFinRowGroups * 128);   // [2][nw32]
  __shared__ double redd[kFinThreads / 64];
  __shared__ float redf[kFinThreads / 64];
  const int tid = threadIdx.x, h = blockIdx.x, g = h / a.G;

  if (a.pe) {
    // the statistics pass already formed sigma * mean(Q_last) . mean(K_j)
    for (int j = tid; j < N; j += kFinThreads) ev[j] = a.pe[(size_t)h * N + j];
  } else {
  // Mean of the last query block: 16-byte loads, rows split over RG groups
  // (the threads past RG * CPR only join the barriers), group partials
  // combined in order.
  {
    constexpr int RB = I8 ? 128 : 256, CPR = RB / 16, EPC = I8 ? 16 : 8;
    constexpr int RG = kFinThreads / CPR < kFinRowGroups ? kFinThreads / CPR : kFinRowGroups;
    const int ch = tid % CPR, rg = tid / CPR;
    float acc[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = 0.0f;
    const size_t tok0 = (size_t)h * S + (S - B);
#pragma unroll 8
    for (int r = rg; r < B && rg < RG; r += RG) {
      const u32x4 v = *(const u32x4 *)(a.Q + (tok0 + r) * RB + ch * 16);
      if (!I8) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += bf16lo(v[e]);
          acc[2 * e + 1] += bf16hi(v[e]);
        }
      } else {
        const float sc = a.sQ[tok0 + r];
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] += sc * (float)(int8_t)((v[e >> 2] >> (8 * (e & 3))) & 0xffu);
      }
    }
    if (rg < RG) {
#pragma unroll
      for (int e = 0; e < EPC; ++e) qpart[rg * 128 + ch * EPC + e] = acc[e];
    }
    __syncthreads();
    if (tid < 128) {
      float sum = 0.0f;
      for (int q = 0; q < RG; ++q) sum += qpart[q * 128 + tid];
      qb[tid] = sum / (float)B;
    }
    __syncthreads();
  }

  // Pooled logits against every mean-pooled key block: a wave takes 16 blocks at a time,
  // four adjacent lanes per block, each lane a contiguous quarter (32 columns, 128 bytes);
  // the four partial dots are combined across the lanes.
  {
    const int wv = tid >> 6, ln = tid & 63, rr = ln >> 2, qq = ln & 3;
    const float *qp = qb + 32 * qq;
    for (int j0 = wv * 16; j0 < N; j0 += (kFinThreads / 64) * 16) {
      const int j = j0 + rr;
      float acc = 0.0f;
      if (j < N) {
        const float4 *kr = (const float4 *)(a.kbar + ((size_t)g * N + j) * 128 + 32 * qq);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const float4 k4 = kr[c];
          acc += qp[4 * c] * k4.x + qp[4 * c + 1] * k4.y + qp[4 * c + 2] * k4.z + qp[4 * c + 3] * k4.w;
        }
      }
      acc += bfly<0>(acc);
      acc += bfly<1>(acc);
      if (qq == 0 && j < N) ev[j] = a.sigma * acc;
    }
  }
  __syncthreads();   // ev[j] is read below by thread j, not by the lane that wrote it
  }
  float mx = kNegBig;
  for (int j = tid; j < N; j += kFinThreads) mx = fmaxf(mx, ev[j]);
  mx = block_max(mx, redf);
  double zpart = 0.0;
  for (int j = tid; j < N; j += kFinThreads) {
    const float w = expf(ev[j] - mx);
    ev[j] = w;
    zpart += (double)w;
  }
  const double Z = block_sum(zpart, redd);

  // Vertical and slash mass; divergence.
  const float *lo = a.lo + (size_t)h * N, *hi = a.hi + (size_t)h * N;
  double dpart = 0.0;
  for (int j = tid; j < N; j += kFinThreads) {
    const float p = (float)((double)ev[j] / Z);
    ev[j] = p;
    const float v = lo[j] + hi[j];
    vv[j] = v;
    sv[j] = lo[N - 1 - j] + (j <= N - 2 ? hi[N - 2 - j] : 0.0f);
    // x log2(x / m) in fp32 with the hardware log2 (error about 1e-7 of the term's weight x, far
    // below the divergence's use against tau), summed in double; a ratio below the smallest normal
    // float contributes less than 1e-36 and is left out
    const float m = 0.5f * (p + v);
    float term = 0.0f;
    if (p > 0.0f) {
      const float r = __fdividef(p, m);
      if (r >= FLT_MIN) term += p * __log2f(r);
    }
    if (v > 0.0f) {
      const float r = __fdividef(v, m);
      if (r >= FLT_MIN) term += v * __log2f(r);
    }
    dpart += (double)term;
  }
  const double D = 0.5 * 0.6931471805599453 * block_sum(dpart, redd);   // natural log: ln 2 * log2
  const bool qa = D < (double)a.tau;
  if (tid == 0) {
    a.jsd[h] = (float)D;
    a.pattern[h] = qa ? FP_PATTERN_QUERY_AWARE : FP_PATTERN_VERTICAL_SLASH;
  }
  if (a.stats) {
    const size_t HN = (size_t)gridDim.x * N;
    for (int j = tid; j < N; j += kFinThreads) {
      a.stats[(size_t)h * N + j] = vv[j];
      a.stats[HN + (size_t)h * N + j] = sv[j];
      a.stats[2 * HN + (size_t)h * N + j] = ev[j];
    }
  }

  // Vertical-slash heads: wave 0 selects columns, wave 1 diagonal offsets.
  uint32_t *out = a.sel + (size_t)h * 2 * a.nw32;
  const int wave = tid >> 6;
  if (wave < 2) {
    uint32_t *m = msk + wave * a.nw32;
    for (int w = tid & 63; w < a.nw32; w += 64) m[w] = 0u;
    if (!qa) wave_select<32>(wave == 0 ? vv : sv, N, a.gamma, m);
    for (int w = tid & 63; w < a.nw32; w += 64) out[wave * a.nw32 + w] = m[w];
  }
}

}  // namespace

hipError_t launch_ig_finalize(const Plan &p, bool i8, const void *Q, const float *sQ,
                              float gamma, float tau, const fp_index_out *out, const Work &w,
                              hipStream_t st, bool have_pe) {
  FinArgs a;
  a.Q = (const uint8_t *)Q;
  a.sQ = sQ;
  a.S = p.S; a.N = p.N; a.B = p.B; a.G = p.G; a.nw32 = p.nw32;
  a.sigma = 1.0f / sqrtf((float)p.d);
  a.gamma = gamma; a.tau = tau;
  a.lo = w.lo; a.hi = w.hi; a.kbar = w.kbar;
  a.pe = have_pe ? w.pe : nullptr;
  a.pattern = out->pattern; a.jsd = out->jsd; a.stats = out->stats;
  a.sel = w.sel;
  const size_t lds = sizeof(float) * (3 * (size_t)p.N + 128 + kFinRowGroups * 128) + sizeof(uint32_t) * 2 * p.nw32;
  const void *fn = i8 ? (const void *)k_ig_finalize<true> : (const void *)k_ig_finalize<false>;
  hipError_t e = ensure_dyn_lds(fn, lds);
  if (e != hipSuccess) return e;
  if (i8)
    hipLaunchKernelGGL(k_ig_finalize<true>, dim3(p.Hq), dim3(kFinThreads), lds, st, a);
  else
    hipLaunchKernelGGL(k_ig_finalize<false>, dim3(p.Hq), dim3(kFinThreads), lds, st, a);
  return hipGetLastError();
}

}  // namespace fp
