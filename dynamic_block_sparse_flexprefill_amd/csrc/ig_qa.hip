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
// Only the Q blocks of the heads the divergence test labelled query-aware are
// read.  k_qa_rows16 (N <= 2048) pools its own 16 query blocks -- one wave per
// block, each load instruction covering consecutive rows (1 KiB contiguous for
// bf16), partial column sums combined across lanes at the end -- so the HBM
// read of Q overlaps the scoring and selection of other workgroups; it then
// scores those blocks against the pooled keys, and each wave selects its rows
// and writes them as bit sets (one bit per key block).  For N > 2048, k_pool_q
// writes the means to the workspace first and k_qa_rows scores from there.
#include "fp_common.hpp"
#include "fp_internal.hpp"
#include "fp_select.hpp"

namespace fp {
namespace {

constexpr int kQaThreads = 256;

struct PoolArgs {
  const uint8_t *Q;
  const float *sQ;
  int S, N;
  const uint8_t *pattern;
  float *qbar;       // [Hq][N][128]
};

// Column sums of one query block (B rows from token tok0) by one wave: lane
// (rr, ch) adds rows rr, rr + RPL, ... of 16-byte column chunk ch in order, then
// the RPL partial sums of each chunk are combined across lanes; afterwards lanes
// with rr == 0 hold the block's sums of columns ch * EPC .. ch * EPC + EPC - 1.
template <int B, bool I8> struct PoolGeo {
  static constexpr int RB = I8 ? 128 : 256, CPR = RB / 16, EPC = I8 ? 16 : 8;
  static constexpr int RPL = 64 / CPR;          // rows read together by one wave
};

template <int B, bool I8>
__device__ __forceinline__ void pool_block(const uint8_t *Q, const float *sQ, size_t tok0,
                                           float acc[PoolGeo<B, I8>::EPC]) {
  using PG = PoolGeo<B, I8>;
  const int lane = threadIdx.x & 63, ch = lane % PG::CPR, rr = lane / PG::CPR;
  const uint8_t *p = Q + (tok0 + rr) * PG::RB + ch * 16;
#pragma unroll
  for (int e = 0; e < PG::EPC; ++e) acc[e] = 0.0f;
#pragma unroll 8
  for (int r = 0; r < B; r += PG::RPL) {
    const u32x4 v = *(const u32x4 *)(p + (size_t)r * PG::RB);
    if (!I8) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += bf16lo(v[e]);
        acc[2 * e + 1] += bf16hi(v[e]);
      }
    } else {
      const float s = sQ[tok0 + r + rr];
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] += s * (float)(int8_t)((v[e >> 2] >> (8 * (e & 3))) & 0xffu);
    }
  }
  // lanes ch, ch + CPR, ... hold partial sums of the same columns
#pragma unroll
  for (int e = 0; e < PG::EPC; ++e) {
    if (PG::CPR == 16) {
      acc[e] += bfly<4>(acc[e]);
      acc[e] += bfly<5>(acc[e]);
    } else {
      acc[e] += __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(acc[e]), __float_as_int(acc[e]), 0x128, 0xF, 0xF, true));   // lane (i + 8) mod 16
      acc[e] += bfly<4>(acc[e]);
      acc[e] += bfly<5>(acc[e]);
    }
  }
}

// One wave per query block; the means go to qbar (used when N > 2048).
template <int B, bool I8>
__global__ void __launch_bounds__(kQaThreads) k_pool_q(PoolArgs a) {
  const int h = blockIdx.y;
  if (a.pattern[h] != FP_PATTERN_QUERY_AWARE) return;
  using PG = PoolGeo<B, I8>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int blk = blockIdx.x * (kQaThreads / 64) + wave, ch = lane % PG::CPR, rr = lane / PG::CPR;
  if (blk >= a.N) return;
  float acc[PG::EPC];
  pool_block<B, I8>(a.Q, a.sQ, (size_t)h * a.S + (size_t)blk * B, acc);
  if (rr == 0) {
    float4 *dst = (float4 *)(a.qbar + ((size_t)h * a.N + blk) * 128 + ch * PG::EPC);
#pragma unroll
    for (int e = 0; e < PG::EPC / 4; ++e)
      dst[e] = make_float4(acc[4 * e] / B, acc[4 * e + 1] / B, acc[4 * e + 2] / B, acc[4 * e + 3] / B);
  }
}

struct QaArgs {
  const uint8_t *Q;  // query tokens (pooled in the 16-row kernel)
  const float *sQ;
  int S, N, G, R, nw32;
  float sigma, gamma;
  const uint8_t *pattern;
  const float *qbar, *kbar;
  uint32_t *rowbits;
};

// Softmax weights and selection of one row of n logits (LDS) whose values fit the register form:
// one LDS read per value, the maximum, the exponentials and the search all in registers.
template <int VPL>
__device__ __forceinline__ void select_row_reg(const float *x, int n, float gamma, uint32_t *wd) {
  const int lane = threadIdx.x & 63;
  float v[VPL];
  float mx = kNegBig;
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    const int j = lane + 64 * k;
    v[k] = j < n ? x[j] : kNegBig;
    mx = fmaxf(mx, v[k]);
  }
  mx = wave_max(mx);
#pragma unroll
  for (int k = 0; k < VPL; ++k) v[k] = lane + 64 * k < n ? __expf(v[k] - mx) : -1.0f;   // -1: not an element
  // rows of more than 512 blocks: 8 greedy extractions before the bisection measured faster than 24
  // on the 128K layers (the selected set is the same either way)
  wave_select_vals<VPL, (VPL >= 16 ? 8 : kGreedySteps)>(v, n, gamma, wd);
}

// One wave per row of logits ev[r][0..i0+r]: softmax weights, selection
// ([E] 3.1 cumulative-gamma rule), block 0 and the diagonal forced in, and the
// row's bit set written to rowbits.  words: LDS, (blockDim / 64) * nw32 words.
// Rows of up to 64 * MAXV values select in registers (the form sized to the row); longer rows
// keep their weights in LDS.
template <int MAXV>
__device__ void select_rows(const QaArgs &a, int h, int i0, int rows, float *ev, uint32_t *words) {
  const int N = a.N, lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwv = blockDim.x >> 6;
  uint32_t *wd = words + wave * a.nw32;
  for (int r = wave; r < rows; r += nwv) {
    const int i = i0 + r, n = i + 1;
    float *x = ev + (size_t)r * N;
    const int nwr = (i >> 5) + 1;
    for (int w = lane; w < nwr; w += 64) wd[w] = 0u;
    if (n <= 256) {
      select_row_reg<4>(x, n, a.gamma, wd);
    } else if (n <= 512) {
      select_row_reg<8>(x, n, a.gamma, wd);
    } else if (n <= 1024) {
      select_row_reg<16>(x, n, a.gamma, wd);
    } else if (MAXV == 32 && n <= 2048) {
      select_row_reg<32>(x, n, a.gamma, wd);
    } else {
      float mx = kNegBig;
#pragma unroll 8
      for (int j = lane; j < n; j += 64) mx = fmaxf(mx, x[j]);
      mx = wave_max(mx);
#pragma unroll 8
      for (int j = lane; j < n; j += 64) x[j] = __expf(x[j] - mx);
      wave_select_lds(x, n, a.gamma, wd);
    }
    if (lane == 0) {
      atomicOr(&wd[0], 1u);
      atomicOr(&wd[i >> 5], 1u << (i & 31));
    }
    uint32_t *dst = a.rowbits + ((size_t)h * N + i) * a.nw32;
    for (int w = lane; w < nwr; w += 64) dst[w] = wd[w];
  }
}

// Logits of 16 query-aware rows on the fp32 matrix cores (16x16x4): the
// workgroup first pools its 16 query blocks (two per wave, read straight from
// Q) into LDS; those means are the A operand (lane l: row l % 16, quarter
// l / 16 of every 16-wide slice of d), each wave sweeps 16-column tiles of
// K-bar as the B operand, 32 products per tile; rows then select as above.
// Used while 16 rows of logits fit in LDS (N <= 2048); WIDE (N > 1024) selects rows
// of up to 2048 blocks in registers.
constexpr int kQa16Threads = 512;
// PRE: the pooled queries come from the caller (a.qbar, [Hq][N][128], e.g. from the projection
// epilogue) instead of being pooled here from Q.
template <int B, bool I8, bool WIDE, bool PRE>
__global__ void __launch_bounds__(kQa16Threads) k_qa_rows16(QaArgs a) {
  const int h = blockIdx.y;
  if (a.pattern[h] != FP_PATTERN_QUERY_AWARE) return;
  extern __shared__ __attribute__((aligned(16))) float smem[];
  const int N = a.N;
  const int i0 = blockIdx.x * 16;
  const int rows = min(16, N - i0);
  const int g = h / a.G;
  float *ev = smem;                                   // [16][N] logits / weights
  float *qs = ev + (size_t)16 * N;                    // [16][128] pooled queries
  uint32_t *words = (uint32_t *)(qs + 16 * 128);      // [8 waves][nw32]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, q = lane >> 4, rl = lane & 15;

  if constexpr (PRE) {
    for (int k = threadIdx.x; k < rows * 32; k += kQa16Threads)
      ((float4 *)qs)[k] = ((const float4 *)(a.qbar + ((size_t)h * N + i0) * 128))[k];
  } else {
    using PG = PoolGeo<B, I8>;
    const int ch = lane % PG::CPR, rr = lane / PG::CPR;
    for (int r = wave; r < rows; r += kQa16Threads / 64) {
      float acc[PG::EPC];
      pool_block<B, I8>(a.Q, a.sQ, (size_t)h * a.S + (size_t)(i0 + r) * B, acc);
      if (rr == 0) {
        float4 *dst = (float4 *)(qs + r * 128 + ch * PG::EPC);
#pragma unroll
        for (int e = 0; e < PG::EPC / 4; ++e)
          dst[e] = make_float4(acc[4 * e] / B, acc[4 * e + 1] / B, acc[4 * e + 2] / B, acc[4 * e + 3] / B);
      }
    }
  }
  __syncthreads();

  f32x4 qa[8];
  const float *qrow = qs + min(rl, rows - 1) * 128 + 4 * q;
#pragma unroll
  for (int t = 0; t < 8; ++t) qa[t] = *(const f32x4 *)(qrow + 16 * t);
  const int ntile = (i0 + rows - 1) / 16 + 1;         // column tiles covering j <= i0 + rows - 1
  auto ldk = [&](int jt, f32x4 *kb) {
    const float *krow = a.kbar + ((size_t)g * N + min(jt * 16 + rl, N - 1)) * 128 + 4 * q;
#pragma unroll
    for (int t = 0; t < 8; ++t) kb[t] = *(const f32x4 *)(krow + 16 * t);
  };
  f32x4 kn[8];
  if (wave < ntile) ldk(wave, kn);
  for (int jt = wave; jt < ntile; jt += kQa16Threads / 64) {
    f32x4 kb[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) kb[t] = kn[t];
    if (jt + kQa16Threads / 64 < ntile) ldk(jt + kQa16Threads / 64, kn);
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[t][e], kb[t][e], acc, 0, 0, 0);
    const int col = jt * 16 + rl;                      // acc[r]: row 4q + r, column col
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * q + r;
      if (row < rows && col <= i0 + row) ev[(size_t)row * N + col] = a.sigma * acc[r];
    }
  }
  __syncthreads();
  select_rows<WIDE ? 32 : 16>(a, h, i0, rows, ev, words);
}

__global__ void __launch_bounds__(kQaThreads) k_qa_rows(QaArgs a) {
  const int h = blockIdx.y;
  if (a.pattern[h] != FP_PATTERN_QUERY_AWARE) return;
  extern __shared__ __attribute__((aligned(16))) float smem[];
  const int N = a.N, R = a.R;
  const int i0 = blockIdx.x * R;
  const int rows = min(R, N - i0);
  const int g = h / a.G;
  float *ev = smem;                       // [R][N] logits / weights
  float *qb = ev + (size_t)R * N;         // [R][128] pooled queries
  uint32_t *words = (uint32_t *)(qb + R * 128);   // [4 waves][nw32]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  for (int k = tid; k < rows * 128; k += kQaThreads) qb[k] = a.qbar[((size_t)h * N + i0) * 128 + k];
  __syncthreads();

  // Pooled logits e[r][j] for j <= i0 + r.
  const int jmax = i0 + rows - 1;
  for (int j = tid; j <= jmax; j += kQaThreads) {
    const float4 *kr = (const float4 *)(a.kbar + ((size_t)g * N + j) * 128);
    float acc[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[r] = 0.0f;
#pragma unroll 8
    for (int c = 0; c < 32; ++c) {
      const float4 k4 = kr[c];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        if (r < rows) {
          const float4 q = *(const float4 *)(qb + r * 128 + 4 * c);
          acc[r] += q.x * k4.x + q.y * k4.y + q.z * k4.z + q.w * k4.w;
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 8; ++r)
      if (r < rows && j <= i0 + r) ev[(size_t)r * N + j] = a.sigma * acc[r];
  }
  __syncthreads();

  select_rows<16>(a, h, i0, rows, ev, words);
}

template <int B, bool I8>
hipError_t run_pool(const Plan &p, const PoolArgs &a, hipStream_t st) {
  constexpr int BPW = kQaThreads / 64;
  hipLaunchKernelGGL((k_pool_q<B, I8>), dim3((p.N + BPW - 1) / BPW, p.Hq), dim3(kQaThreads), 0, st, a);
  return hipGetLastError();
}

template <int B, bool I8, bool WIDE, bool PRE>
hipError_t launch_qa16(const Plan &p, const QaArgs &a, hipStream_t st) {
  const size_t lds = sizeof(float) * ((size_t)16 * p.N + 16 * 128) + sizeof(uint32_t) * 8 * p.nw32;
  const void *fn = (const void *)k_qa_rows16<B, I8, WIDE, PRE>;
  hipError_t e = ensure_dyn_lds(fn, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_qa_rows16<B, I8, WIDE, PRE>), dim3((p.N + 15) / 16, p.Hq), dim3(kQa16Threads), lds, st, a);
  return hipGetLastError();
}

template <int B, bool I8, bool PRE = false>
hipError_t run_qa16(const Plan &p, const QaArgs &a, hipStream_t st) {
  return p.N > 1024 ? launch_qa16<B, I8, true, PRE>(p, a, st) : launch_qa16<B, I8, false, PRE>(p, a, st);
}

}  // namespace

hipError_t launch_ig_qa(const Plan &p, bool i8, const void *Q, const float *sQ, float gamma,
                        const uint8_t *pattern, const Work &w, hipStream_t st, const float *qbar_in) {
  QaArgs a;
  a.Q = (const uint8_t *)Q;
  a.sQ = sQ;
  a.S = p.S; a.N = p.N; a.G = p.G; a.nw32 = p.nw32;
  a.R = p.N >= 2048 ? (p.N >= 4096 ? 2 : 4) : 8;
  a.sigma = 1.0f / sqrtf((float)p.d);
  a.gamma = gamma;
  a.pattern = pattern;
  a.qbar = w.qbar;
  a.kbar = w.kbar;
  a.rowbits = w.rowbits;
  if (qbar_in) {   // pooled queries from the caller: no read of Q at all
    a.qbar = qbar_in;
    if (p.N <= 2048) {
      if (p.B == 64) return run_qa16<64, false, true>(p, a, st);
      if (p.B == 128) return run_qa16<128, false, true>(p, a, st);
      return run_qa16<256, false, true>(p, a, st);
    }
    const size_t lds = sizeof(float) * ((size_t)a.R * p.N + a.R * 128) + sizeof(uint32_t) * 4 * p.nw32;
    hipError_t e = ensure_dyn_lds((const void *)k_qa_rows, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_qa_rows, dim3((p.N + a.R - 1) / a.R, p.Hq), dim3(kQaThreads), lds, st, a);
    return hipGetLastError();
  }
  if (p.N <= 2048) {   // pooling fused into the row kernel
    if (p.B == 64) return i8 ? run_qa16<64, true>(p, a, st) : run_qa16<64, false>(p, a, st);
    if (p.B == 128) return i8 ? run_qa16<128, true>(p, a, st) : run_qa16<128, false>(p, a, st);
    return i8 ? run_qa16<256, true>(p, a, st) : run_qa16<256, false>(p, a, st);
  }
  PoolArgs pa;
  pa.Q = (const uint8_t *)Q;
  pa.sQ = sQ;
  pa.S = p.S; pa.N = p.N;
  pa.pattern = pattern;
  pa.qbar = w.qbar;
  hipError_t e;
  if (p.B == 64) e = i8 ? run_pool<64, true>(p, pa, st) : run_pool<64, false>(p, pa, st);
  else if (p.B == 128) e = i8 ? run_pool<128, true>(p, pa, st) : run_pool<128, false>(p, pa, st);
  else e = i8 ? run_pool<256, true>(p, pa, st) : run_pool<256, false>(p, pa, st);
  if (e != hipSuccess) return e;
  const size_t lds = sizeof(float) * ((size_t)a.R * p.N + a.R * 128) + sizeof(uint32_t) * 4 * p.nw32;
  e = ensure_dyn_lds((const void *)k_qa_rows, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_qa_rows, dim3((p.N + a.R - 1) / a.R, p.Hq), dim3(kQaThreads), lds, st, a);
  return hipGetLastError();
}

}  // namespace fp
