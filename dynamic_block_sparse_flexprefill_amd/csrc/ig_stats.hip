// Last-block statistics for sparse-index generation.
//
// Explainer ("FPGA24成果：FAST-Prefill稀疏注意力加速器", yunpan.plus) section
// 3.1: key blocks stream from HBM in increasing block order, the last query
// block Q_last is multiplied against each one, and only compact per-head
// block statistics are kept -- vertical mass (attention summed along key
// columns) and slash mass (summed along diagonals).  Section 2.1 describes the
// b x S intermediate this avoids; nothing of that size is written here.
//
// The attention is the causal row softmax of section 1.1 for the b rows
// t_r = S - b + r of the last block.  With L_r the row's softmax denominator,
// the per-head outputs are, for each key block j,
//   lo[j] = (1/b) sum_r sum_{c <= r} exp(s_r[jb+c] - M_r) / L_r
//   hi[j] = (1/b) sum_r sum_{c >  r} exp(s_r[jb+c] - M_r) / L_r
// so that vertical mass v[j] = lo[j] + hi[j], and the slash mass of offset
// block o (token diagonal t_r - k pooled by b) is lo[N-1-o] + hi[N-2-o].
// Every key block is also mean-pooled into kbar[g][j][:] for the pooled
// estimate of Flex-Prefill's pattern test (explainer section 1.2).
//
// Two forms.  The single-pass kernel (k_ig_stats1, below) streams K once and
// keeps per-(row, block) partials on chip until one grid-wide barrier; it is
// used whenever those partials fit in LDS with one workgroup per CU.  The
// fallback streams K twice: pass 1 gathers each row's running maximum and
// exponential sum per chunk of key blocks, a combine step merges the chunks,
// and pass 2 streams K again to bin the normalised attention.
//
// Work split: one workgroup per (KV group g, contiguous chunk of key blocks);
// all G query heads of the group share each staged key block.  Each wave owns
// TPW tiles of 32 last-block query rows and keeps their Q fragments in
// registers; scores are computed transposed (keys x queries) on the 32x32x16
// bf16 (or 32x32x32 int8) matrix cores so that every lane holds one query row.
#include "fp_common.hpp"
#include "fp_internal.hpp"

namespace fp {
namespace {

struct StatArgs {
  const uint8_t *Q;   // bf16 or int8 [Hq, S, 128]
  const float *sQ;    // int8 only: [Hq, S]
  const uint8_t *K;   // bf16 or int8 [Hkv, S, 128]
  const float *sK;    // int8 only: [Hkv, S]
  int S, N, G, nch, cpb;
  float c2;           // (1/sqrt(d)) * log2(e)
  float2 *part;       // [Hq*B*nch] (max, sum) per row and chunk (log2 domain)
  float2 *rowml;      // [Hq*B] merged (max, sum)
  float *lo, *hi;     // [Hq*N]
  float *kbar;        // [Hkv*N*128]
  float *pe;          // [Hq*N] pooled-estimate logits (single pass only)
  float sigma;        // 1/sqrt(d)
};

template <bool I8> struct Tile;
template <> struct Tile<false> {   // bf16: 8 k-steps of 16, 272-byte LDS rows
  static constexpr int KS = 8, RowBytes = 256, Stride = 272;
};
template <> struct Tile<true> {    // int8: 4 k-steps of 32, 144-byte LDS rows
  static constexpr int KS = 4, RowBytes = 128, Stride = 144;
};

// Copy key block j of KV head g into LDS (rows padded to Tile::Stride bytes).
template <int B, bool I8>
__device__ __forceinline__ void stage_k(const StatArgs &a, int g, int j, uint8_t *ks, float *sk) {
  constexpr int CPR = Tile<I8>::RowBytes / 16;   // 16-byte chunks per row
  const uint8_t *src = a.K + ((size_t)g * a.S + (size_t)j * B) * Tile<I8>::RowBytes;
  for (int c = threadIdx.x; c < B * CPR; c += blockDim.x) {
    const int row = c / CPR, col = c % CPR;
    u32x4 v = *(const u32x4 *)(src + (size_t)row * Tile<I8>::RowBytes + col * 16);
    *(u32x4 *)(ks + row * Tile<I8>::Stride + col * 16) = v;
  }
  if (I8) {
    for (int r = threadIdx.x; r < B; r += blockDim.x) sk[r] = a.sK[(size_t)g * a.S + (size_t)j * B + r];
  }
}

// Exact int32 scores of one 32-key tile (kt) of the staged int8 block against one 32-query
// tile: acc[r] <-> key kt*32 + acc_row(r, lane), query lane % 32.
__device__ __forceinline__ i32x16 tile_raw_i8(const uint8_t *ks, const u32x4 *qf, int kt) {
  const int lane = threadIdx.x & 63;
  const uint8_t *arow = ks + (kt * 32 + (lane & 31)) * Tile<true>::Stride + 16 * (lane >> 5);
  i32x16 acc = {};
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = mfma_i8(*(const u32x4 *)(arow + 32 * s), qf[s], acc);
  return acc;
}

// Scores of one 32-key tile (kt) against one 32-query tile: x[r] in log2 units.
template <bool I8>
__device__ __forceinline__ void tile_scores(const uint8_t *ks, const float *sk, const u32x4 *qf,
                                            float qscale, int kt, float c2, float x[16]) {
  const int lane = threadIdx.x & 63;
  if (!I8) {
    const uint8_t *arow = ks + (kt * 32 + (lane & 31)) * Tile<I8>::Stride + 16 * (lane >> 5);
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < 8; ++s) acc = mfma_bf16(*(const u32x4 *)(arow + 32 * s), qf[s], acc);
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = acc[r] * c2;
  } else {
    const i32x16 acc = tile_raw_i8(ks, qf, kt);
#pragma unroll
    for (int r = 0; r < 16; ++r)
      x[r] = (float)acc[r] * (c2 * qscale) * sk[kt * 32 + acc_row(r, lane)];
  }
}

template <int B, int TPW, bool I8, int PASS>
__global__ void __launch_bounds__(1024) k_ig_stats(StatArgs a) {
  constexpr int QT = B / 32;                 // query tiles per head
  __shared__ __attribute__((aligned(16))) uint8_t ks[B * Tile<I8>::Stride];
  __shared__ float sk[I8 ? B : 1];
  __shared__ float red[64 * 2];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int chunk = blockIdx.x, g = blockIdx.y;
  const int G = a.G, S = a.S, N = a.N;
  const int ntiles = G * QT;
  const int j0 = chunk * a.cpb, j1 = min(N, j0 + a.cpb);

  // Q fragments of this wave's tiles (rows of the last query block).
  u32x4 qf[TPW][Tile<I8>::KS];
  float qscale[TPW], ml_m[TPW], ml_l[TPW], wrow[TPW];
  int qrow[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int t = wave * TPW + u;
    const int tt = t < ntiles ? t : 0;
    const int hh = tt / QT, row = (tt % QT) * 32 + (lane & 31);
    const int h = g * G + hh;
    qrow[u] = row;
    const size_t tok = (size_t)h * S + (S - B) + row;
    const uint8_t *qp = a.Q + tok * Tile<I8>::RowBytes + 16 * (lane >> 5);
#pragma unroll
    for (int s = 0; s < Tile<I8>::KS; ++s) qf[u][s] = *(const u32x4 *)(qp + 32 * s);
    qscale[u] = I8 ? a.sQ[tok] : 1.0f;
    ml_m[u] = kNegBig;
    ml_l[u] = 0.0f;
    wrow[u] = 0.0f;
    if (PASS == 2) {
      const float2 ml = a.rowml[(size_t)h * B + row];
      ml_m[u] = ml.x;
      wrow[u] = 1.0f / ((float)B * ml.y);
    }
  }

  for (int j = j0; j < j1; ++j) {
    __syncthreads();
    stage_k<B, I8>(a, g, j, ks, sk);
    __syncthreads();
    const bool diag = (j == N - 1);

    if (PASS == 2) {
      // Mean-pooled key block (fp32, rows summed in order).
      for (int dd = threadIdx.x; dd < 128; dd += blockDim.x) {
        float s = 0.0f;
        for (int r = 0; r < B; ++r) {
          float kv;
          if (!I8) kv = bf16_to_f32(*(const uint16_t *)(ks + r * Tile<I8>::Stride + 2 * dd));
          else kv = sk[r] * (float)(int8_t)ks[r * Tile<I8>::Stride + dd];
          s += kv;
        }
        a.kbar[((size_t)g * N + j) * 128 + dd] = s / (float)B;
      }
    }

#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int t = wave * TPW + u;
      if (t >= ntiles) continue;
      float lo_acc = 0.0f, hi_acc = 0.0f;
      for (int kt = 0; kt < QT; ++kt) {
        float x[16];
        tile_scores<I8>(ks, sk, qf[u], qscale[u], kt, a.c2, x);
        if (PASS == 1) {
          float mx = kNegBig;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int c = kt * 32 + acc_row(r, lane);
            if (diag && c > qrow[u]) x[r] = kNegBig;
            mx = fmaxf(mx, x[r]);
          }
          const float mnew = fmaxf(ml_m[u], mx);
          float sum = 0.0f;
#pragma unroll
          for (int r = 0; r < 16; ++r) sum += (x[r] == kNegBig) ? 0.0f : exp2f(x[r] - mnew);
          ml_l[u] = ml_l[u] * exp2f(ml_m[u] - mnew) + sum;
          ml_m[u] = mnew;
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int c = kt * 32 + acc_row(r, lane);
            const float e = exp2f(x[r] - ml_m[u]);
            if (c <= qrow[u]) lo_acc += e;
            else if (!diag) hi_acc += e;
          }
        }
      }
      if (PASS == 2) {
        lo_acc = wave_sum(lo_acc * wrow[u]);
        hi_acc = wave_sum(hi_acc * wrow[u]);
        if (lane == 0) {
          red[2 * t] = lo_acc;
          red[2 * t + 1] = hi_acc;
        }
      }
    }
    if (PASS == 2) {
      __syncthreads();
      if (threadIdx.x < G) {
        const int hh = threadIdx.x;
        float l = 0.0f, hsum = 0.0f;
        for (int q = 0; q < QT; ++q) {
          l += red[2 * (hh * QT + q)];
          hsum += red[2 * (hh * QT + q) + 1];
        }
        const size_t o = (size_t)(g * G + hh) * N + j;
        a.lo[o] = l;
        a.hi[o] = hsum;
      }
    }
  }

  if (PASS == 1) {
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int t = wave * TPW + u;
      float m = ml_m[u], l = ml_l[u];
      const float mo = xor32(m), lo = xor32(l);
      const float M = fmaxf(m, mo);
      const float L = l * exp2f(m - M) + lo * exp2f(mo - M);
      if (t < ntiles && lane < 32) {
        const int h = g * G + t / QT;
        a.part[((size_t)h * B + qrow[u]) * a.nch + chunk] = make_float2(M, L);
      }
    }
  }
}

// Merge the per-chunk (max, sum) of every last-block row, chunks in order.
__global__ void k_ig_combine(const float2 *part, float2 *rowml, int rows, int nch) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  const float2 *p = part + (size_t)r * nch;
  float M = kNegBig;
  for (int c = 0; c < nch; ++c) M = fmaxf(M, p[c].x);
  float L = 0.0f;
  for (int c = 0; c < nch; ++c) L += p[c].y * exp2f(p[c].x - M);
  rowml[r] = make_float2(M, L);
}

// ------------------------------------------------------------------ single pass
//
// K is streamed once.  Each workgroup keeps, for every last-block row of its
// KV group and every key block of its chunk, the lower / upper split sums
// exp2(x - m_ref) in LDS, where m_ref is the row's running reference maximum
// (raised only when a score exceeds it by more than kHeadroom, rescaling the
// partials already stored).  After one grid-wide barrier the per-chunk
// (m_ref, sum) pairs of every row are merged in chunk order, identically in
// every workgroup, and each workgroup normalises its own blocks.  All
// workgroups must be resident at once (see the launcher below).

constexpr float kHeadroom = 16.0f;

struct Stat1Args {
  StatArgs s;
  unsigned int *bar;   // grid barrier counter (zeroed by the status kernel)
  int32_t *status;
};

// Every workgroup arrives, then waits until all have; the wait is bounded so
// every wave exits even if the launch did not keep all workgroups resident.
// The counter is polled with relaxed loads (each acquire load would also
// invalidate the L2 of the polling workgroup's XCD); one fence follows the wait.
__device__ void grid_barrier(unsigned int *bar, unsigned int nblocks, int32_t *status) {
  __syncthreads();
  if (threadIdx.x == 0) {
    // release before the (relaxed) arrival, acquire after the (relaxed) wait: the two
    // fences pair up, so neither needs the other half of a full fence
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    atomicAdd(bar, 1u);
    unsigned int spins = 0;
    while (__hip_atomic_load(bar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < nblocks) {
      __builtin_amdgcn_s_sleep(4);
      if (++spins > (1u << 24)) {
        atomicOr((unsigned int *)status, (unsigned int)FP_STATUS_WAIT_TIMEOUT);
        break;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

template <int B, int NT, bool I8>
struct KStage {
  static constexpr int RB = Tile<I8>::RowBytes, CPR = RB / 16, PIECES = B * CPR;
  static constexpr int KP = (PIECES + NT - 1) / NT;
  u32x4 r[KP];
  float s;
  // Every thread issues the same KP (+1) loads (indices past the block repeat its last
  // piece and are never stored), so the number of loads in flight is the same on every
  // path and the wait before a stage's store leaves the other stage's loads in flight.
  __device__ __forceinline__ void load(const StatArgs &a, int g, int j) {
    const size_t row0 = (size_t)g * a.S + (size_t)j * B;
    const uint8_t *src = a.K + row0 * RB;
#pragma unroll
    for (int u = 0; u < KP; ++u) {
      const int idx = min((int)threadIdx.x + u * NT, PIECES - 1);
      r[u] = *(const u32x4 *)(src + (size_t)idx * 16);
    }
    if (I8) s = a.sK[row0 + min((int)threadIdx.x, B - 1)];
  }
  // bf16: column sums of this thread's pieces (all in 16-byte column chunk
  // threadIdx.x % CPR, since NT is a multiple of CPR), rows in order.
  __device__ __forceinline__ void colsum(float acc[8]) const {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int u = 0; u < KP; ++u) {
      if ((int)threadIdx.x + u * NT < PIECES) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          acc[2 * w] += bf16lo(r[u][w]);
          acc[2 * w + 1] += bf16hi(r[u][w]);
        }
      }
    }
  }
  __device__ __forceinline__ void store(uint8_t *ks, float *sk) const {
#pragma unroll
    for (int u = 0; u < KP; ++u) {
      const int idx = threadIdx.x + u * NT;
      if (idx < PIECES) *(u32x4 *)(ks + (idx / CPR) * Tile<I8>::Stride + (idx % CPR) * 16) = r[u];
    }
    if (I8 && threadIdx.x < B) sk[threadIdx.x] = s;
  }
};

// KBS: the chunk's pooled key blocks are kept in LDS and written after the block loop
// (no stores among the loads of the K stream); otherwise each block's is stored at once.
template <int B, int NT, int TPW, bool I8, bool KBS>
__global__ void __launch_bounds__(NT) k_ig_stats1(Stat1Args args) {
  const StatArgs &a = args.s;
  constexpr int QT = B / 32, NWV = NT / 64, RG = NT / 64;
  extern __shared__ __attribute__((aligned(16))) float part[];   // [NWV*TPW][cpb][32][2]
  __shared__ __attribute__((aligned(16))) uint8_t ks[B * Tile<I8>::Stride];
  __shared__ float sk[I8 ? B : 1];
  __shared__ float kpart[RG][128];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int chunk = blockIdx.x, g = blockIdx.y;
  const int G = a.G, S = a.S, N = a.N, cpb = a.cpb;
  const int ntiles = G * QT;
  const int j0 = chunk * cpb, nb = min(N, j0 + cpb) - j0;
  constexpr int NTL = NWV * TPW;                                  // tile slots
  float *red = part + (size_t)NTL * cpb * 64;                     // [cpb][NTL][2]
  float *qsm = red + (size_t)cpb * NTL * 2;                       // [G][128] mean of each last query block
  float *kbs = qsm + (size_t)G * 128;                             // [cpb][128] pooled key blocks (KBS)

  u32x4 qf[TPW][Tile<I8>::KS];
  float qscale[TPW], mref[TPW], lsum[TPW];
  int qrow[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int t = wave * TPW + u;
    const int tt = t < ntiles ? t : 0;
    const int h = g * G + tt / QT, row = (tt % QT) * 32 + (lane & 31);
    qrow[u] = row;
    const size_t tok = (size_t)h * S + (S - B) + row;
    const uint8_t *qp = a.Q + tok * Tile<I8>::RowBytes + 16 * (lane >> 5);
#pragma unroll
    for (int s = 0; s < Tile<I8>::KS; ++s) qf[u][s] = *(const u32x4 *)(qp + 32 * s);
    qscale[u] = (I8 ? a.sQ[tok] : 1.0f) * a.c2;
    mref[u] = -1e30f;
    lsum[u] = 0.0f;
  }

  // Mean of each of the group's last query blocks, for the pooled estimate, summed through
  // the staging buffer ks before the K stream starts: thread (16-byte column chunk, head,
  // row group) adds its rows in order, then the row groups are combined in order.
  {
    constexpr int CPR = Tile<I8>::RowBytes / 16, EPC = I8 ? 16 : 8, KSB = B * Tile<I8>::Stride;
    const int R = max(1, min(NT / (CPR * G), KSB / (G * 512)));
    float *qpart = (float *)ks;                                   // [G][R][128]
    const int tid = threadIdx.x;
    if (tid < CPR * G * R) {
      const int ch = tid % CPR, hh = (tid / CPR) % G, rg = tid / (CPR * G);
      const size_t tok0 = (size_t)(g * G + hh) * S + (S - B);
      float acc[EPC];
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[e] = 0.0f;
      for (int r = rg; r < B; r += R) {
        const u32x4 v = *(const u32x4 *)(a.Q + (tok0 + r) * Tile<I8>::RowBytes + ch * 16);
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
#pragma unroll
      for (int e = 0; e < EPC; ++e) qpart[(hh * R + rg) * 128 + ch * EPC + e] = acc[e];
    }
    __syncthreads();
    for (int k = tid; k < G * 128; k += NT) {
      const int hh = k / 128, dd = k % 128;
      float sm = 0.0f;
      for (int q = 0; q < R; ++q) sm += qpart[(hh * R + q) * 128 + dd];
      qsm[k] = sm / (float)B;
    }
    __syncthreads();                                              // ks is about to stage K
  }

  // The Q fragments (and scales) are waited for here, before any K block is in flight:
  // otherwise the compiler, unable to prove them loaded inside the block loop, waits for
  // every outstanding load at their first use there, including the next blocks' prefetch.
  __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)

  // K blocks stream through registers two blocks ahead of their use (two stages, alternating)
  KStage<B, NT, I8> stg0, stg1;
  stg0.load(a, g, j0);                      // nb >= 1 for every workgroup of the grid
  stg1.load(a, g, j0 + min(1, nb - 1));
  auto block = [&](int jj, KStage<B, NT, I8> &stg) {
    const int j = j0 + jj;
    // (the previous block's closing barrier has already retired every read of ks, sk and kpart)
    if constexpr (!I8) {
      // bf16 mean-pooled key block from the staged registers: lanes l, l + 16, l + 32,
      // l + 48 of a wave hold the same column chunk; each wave's sums go to kpart[wave]
      static_assert(NT % KStage<B, NT, I8>::CPR == 0 && KStage<B, NT, I8>::CPR == 16, "column chunk per lane");
      float cs[8];
      stg.colsum(cs);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        cs[e] += bfly<4>(cs[e]);
        cs[e] += bfly<5>(cs[e]);
      }
      if (lane < 16) {
#pragma unroll
        for (int e = 0; e < 8; ++e) kpart[wave][8 * lane + e] = cs[e];
      }
    }
    stg.store(ks, sk);
    __syncthreads();
    // unconditional, so every path through the loop has the same loads in flight (past the
    // chunk's end the stage re-reads its last block, still in L2, and is never stored)
    stg.load(a, g, j0 + min(jj + 2, nb - 1));
    const bool diag = (j == N - 1);
    if constexpr (!I8) {
      if (threadIdx.x < 128) {
        float sm = 0.0f;
        for (int q = 0; q < RG; ++q) sm += kpart[q][threadIdx.x];
        if constexpr (KBS) kbs[jj * 128 + threadIdx.x] = sm / (float)B;
        else a.kbar[((size_t)g * N + j) * 128 + threadIdx.x] = sm / (float)B;
      }
    }

    // int8: mean-pooled key block from LDS: RG row groups of two columns per thread (one 2-column read
    // per row, rows rg, rg + RG, ... in two interleaved partial sums), combined in order
    if constexpr (I8) {
      const int dp = threadIdx.x & 63, rg = threadIdx.x >> 6;
      float s0 = 0.0f, s1 = 0.0f, t0 = 0.0f, t1 = 0.0f;
#pragma unroll 4
      for (int r = rg; r < B; r += 2 * RG) {
        const int r2 = r + RG;
        if (!I8) {
          const uint32_t v = *(const uint32_t *)(ks + r * Tile<I8>::Stride + 4 * dp);
          s0 += __uint_as_float(v << 16);
          s1 += __uint_as_float(v & 0xffff0000u);
          if (r2 < B) {
            const uint32_t w = *(const uint32_t *)(ks + r2 * Tile<I8>::Stride + 4 * dp);
            t0 += __uint_as_float(w << 16);
            t1 += __uint_as_float(w & 0xffff0000u);
          }
        } else {
          const uint32_t v = *(const uint16_t *)(ks + r * Tile<I8>::Stride + 2 * dp);
          s0 += sk[r] * (float)(int8_t)(v & 0xffu);
          s1 += sk[r] * (float)(int8_t)(v >> 8);
          if (r2 < B) {
            const uint32_t w = *(const uint16_t *)(ks + r2 * Tile<I8>::Stride + 2 * dp);
            t0 += sk[r2] * (float)(int8_t)(w & 0xffu);
            t1 += sk[r2] * (float)(int8_t)(w >> 8);
          }
        }
      }
      kpart[rg][2 * dp] = s0 + t0;
      kpart[rg][2 * dp + 1] = s1 + t1;
    }

#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int t = wave * TPW + u;
      if (t >= ntiles) continue;
      float lo_acc = 0.0f, hi_acc = 0.0f;
      float *prow = part + ((size_t)(wave * TPW + u) * cpb) * 64;   // [cpb][32][2] of this tile
      const int tq = t % QT;            // this wave's 32 query rows are tq*32 .. tq*32+31
      bool piped = false;
      if constexpr (TPW == 1 && NT <= 768 && B <= 128) {
        if (!diag) {
          // Software-pipelined form for every block but the last: the wave visits its key
          // tiles in the order tq + 1, tq + 2, ... (mod QT), so the one tile whose keys fall on
          // both sides of the query rows (kt == tq) comes last, at a fixed position; the
          // products of the next tile are issued between the exponentials of the current
          // one.  The tile loop has no branch: the new reference maximum is chosen by a
          // select and the running sums are rescaled every tile (by exactly 1 where the
          // maximum stays); the partials stored for earlier blocks are rescaled once, after
          // the loop, by the product of the block's factors, 2^(m_start - m_end).
          piped = true;
          const float m_start = mref[u];
          auto tile = [&](int kt) {
            if constexpr (!I8) {
              const uint8_t *arow = ks + (kt * 32 + (lane & 31)) * Tile<I8>::Stride + 16 * (lane >> 5);
              f32x16 acc = {};
#pragma unroll
              for (int s = 0; s < 8; ++s) acc = mfma_bf16(*(const u32x4 *)(arow + 32 * s), qf[u][s], acc);
              return acc;
            } else {
              float x[16];
              tile_scores<I8>(ks, sk, qf[u], 1.0f, kt, 1.0f, x);
              f32x16 r;
#pragma unroll
              for (int e = 0; e < 16; ++e) r[e] = x[e];
              return r;
            }
          };
          f32x16 nx = tile((tq + 1) % QT);
#pragma unroll
          for (int pos = 0; pos < QT; ++pos) {
            const int kt = (tq + 1 + pos) % QT;
            const f32x16 x = nx;
            if (pos + 1 < QT) nx = tile((tq + 2 + pos) % QT);
            float mx = fmaxf(x[0], x[1]);
#pragma unroll
            for (int r = 2; r < 16; ++r) mx = fmaxf(mx, x[r]);
            mx = fmaxf(mx, xor32(mx)) * qscale[u];
            const bool grow = mx > mref[u] + kHeadroom;
            const float mnew = grow ? mx : mref[u];
            const float alpha = fast_exp2(mref[u] - mnew);   // exactly 1 where the maximum stays
            lo_acc *= alpha;
            hi_acc *= alpha;
            lsum[u] *= alpha;
            mref[u] = mnew;
            const float qs = qscale[u], mneg = -mnew;
            if (pos + 1 < QT) {
              // all keys of the tile lie on one side of the wave's query rows
              float e = 0.0f;
#pragma unroll
              for (int r = 0; r < 16; ++r) e += fast_exp2(fmaf(x[r], qs, mneg));
              const bool below = kt < tq;
              lo_acc += below ? e : 0.0f;
              hi_acc += below ? 0.0f : e;
            } else {
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const float e = fast_exp2(fmaf(x[r], qs, mneg));
                if (kt * 32 + acc_row(r, lane) <= qrow[u]) lo_acc += e;
                else hi_acc += e;
              }
            }
            // the tile's sums are needed here (an empty use), so they stay with the next
            // tile's products instead of sinking below the branch after the loop
            asm volatile("" ::"v"(lo_acc), "v"(hi_acc));
            if (pos + 1 < QT && !I8) {
              // interleave: the next tile's products, one operand read ahead, each followed by
              // a share of this tile's vector work
              __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
              for (int g8 = 0; g8 < 8; ++g8) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
              }
            }
          }
          const bool moved = mref[u] != m_start;
          if (__any(moved)) {
            const float ab = fast_exp2(m_start - mref[u]);
            if (moved && lane < 32)
              for (int q = 0; q < jj; ++q) {
                prow[q * 64 + 2 * lane] *= ab;
                prow[q * 64 + 2 * lane + 1] *= ab;
              }
          }
        }
      }
      for (int kt = 0; kt < (piped ? 0 : QT); ++kt) {
        if (diag && kt > tq) break;     // keys after every query row of the tile
        float x[16];
        tile_scores<I8>(ks, sk, qf[u], 1.0f, kt, 1.0f, x);
        const bool split = (kt == tq);  // the only key tile holding both c <= r and c > r
        // raw scores: the scale (>= 0) is applied to the maximum and inside the exponent;
        // keys after the row (diagonal block) are left out of both
        float mx;
        if (split && diag) {
          asm volatile("" ::: "memory");   // a real branch: the masked form runs for one tile of one block
          mx = -INFINITY;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (kt * 32 + acc_row(r, lane) <= qrow[u]) mx = fmaxf(mx, x[r]);
        } else {
          mx = x[0];
#pragma unroll
          for (int r = 1; r < 16; ++r) mx = fmaxf(mx, x[r]);
        }
        mx = fmaxf(mx, xor32(mx));
        mx = mx > -INFINITY ? mx * qscale[u] : -INFINITY;
        const bool grow = mx > mref[u] + kHeadroom;
        if (__any(grow)) {
          const float mnew = grow ? mx : mref[u];
          const float alpha = fast_exp2(mref[u] - mnew);
          lo_acc *= alpha;
          hi_acc *= alpha;
          lsum[u] *= alpha;
          if (grow && lane < 32)
            for (int q = 0; q < jj; ++q) {
              prow[q * 64 + 2 * lane] *= alpha;
              prow[q * 64 + 2 * lane + 1] *= alpha;
            }
          mref[u] = mnew;
        }
        const float qs = qscale[u], mneg = -mref[u];
        if (!split) {
          float e = 0.0f;
#pragma unroll
          for (int r = 0; r < 16; ++r) e += fast_exp2(fmaf(x[r], qs, mneg));
          if (kt < tq) lo_acc += e;
          else hi_acc += e;
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float e = fast_exp2(fmaf(x[r], qs, mneg));
            if (kt * 32 + acc_row(r, lane) <= qrow[u]) lo_acc += e;
            else if (!diag) hi_acc += e;
          }
        }
      }
      lo_acc += xor32(lo_acc);
      hi_acc += xor32(hi_acc);
      lsum[u] += lo_acc + hi_acc;
      if (lane < 32) {
        prow[jj * 64 + 2 * lane] = lo_acc;
        prow[jj * 64 + 2 * lane + 1] = hi_acc;
      }
    }
    __syncthreads();
    if constexpr (I8) {
      if (threadIdx.x < 128) {
        float sm = 0.0f;
        for (int q = 0; q < RG; ++q) sm += kpart[q][threadIdx.x];
        if constexpr (KBS) kbs[jj * 128 + threadIdx.x] = sm / (float)B;
        else a.kbar[((size_t)g * N + j) * 128 + threadIdx.x] = sm / (float)B;
      }
    }
  };
  // pairs of blocks, then an odd last block: no block of the loop body is conditional
  int jj = 0;
  for (; jj + 1 < nb; jj += 2) {
    block(jj, stg0);
    block(jj + 1, stg1);
  }
  if (jj < nb) block(jj, stg0);

  // per-chunk (m_ref, sum) of every row, then the grid-wide merge.  Stored chunk-major,
  // [head][chunk][row], so that a wave's 32 rows are one contiguous 256-byte store here
  // and one contiguous load per chunk in the merge (row-major, each lane's pairs would
  // sit in a different cache line: 32 lines per instruction, and as many dirty lines
  // for the barrier's release to write back)
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int t = wave * TPW + u;
    if (t < ntiles && lane < 32) {
      const int h = g * G + t / QT;
      a.part[((size_t)h * a.nch + chunk) * B + qrow[u]] = make_float2(mref[u], lsum[u]);
    }
  }
  grid_barrier(args.bar, gridDim.x * gridDim.y, args.status);
  if constexpr (KBS) {
    // the chunk's pooled key blocks (read only by later kernels): written after the K stream,
    // so no stores sit among its loads, and after the barrier, so its fence has little to write back
    for (int k = threadIdx.x; k < nb * 128; k += NT) a.kbar[((size_t)g * N + j0) * 128 + k] = kbs[k];
  }
  // pooled-estimate logits of the chunk's blocks, sigma * mean(Q_last) . mean(K_j) (K-bar from
  // LDS, or as this workgroup stored it before the barrier)
  for (int k = threadIdx.x; k < G * nb; k += NT) {
    const int hh = k % G, q = k / G;
    const float4 *kr = (const float4 *)(KBS ? kbs + (size_t)q * 128 : a.kbar + ((size_t)g * N + j0 + q) * 128);
    const float4 *qr = (const float4 *)(qsm + hh * 128);
    float sm = 0.0f;
#pragma unroll 8
    for (int c = 0; c < 32; ++c) {
      const float4 kv = kr[c], qv = qr[c];
      sm += qv.x * kv.x + qv.y * kv.y + qv.z * kv.z + qv.w * kv.w;
    }
    a.pe[(size_t)(g * G + hh) * N + j0 + q] = a.sigma * sm;
  }

#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int t = wave * TPW + u;
    if (t >= ntiles) continue;
    const int h = g * G + t / QT;
    const float2 *pp = a.part + (size_t)h * a.nch * B + qrow[u];   // chunk c at pp[c * B]
    // the row's per-chunk pairs, up to 32 loaded together (one memory round trip per batch);
    // batches merge into the running (M, L), chunks in order
    float M = kNegBig, L = 0.0f;
    constexpr int CB = 32;
    for (int c0 = 0; c0 < a.nch; c0 += CB) {
      float2 v[CB];
#pragma unroll
      for (int k = 0; k < CB; ++k) v[k] = c0 + k < a.nch ? pp[(size_t)(c0 + k) * B] : make_float2(kNegBig, 0.0f);
      float Mb = M;
#pragma unroll
      for (int k = 0; k < CB; ++k) Mb = fmaxf(Mb, v[k].x);
      float Lb = L * exp2f(M - Mb);
#pragma unroll
      for (int k = 0; k < CB; ++k) Lb += v[k].y * exp2f(v[k].x - Mb);
      M = Mb;
      L = Lb;
    }
    const float wr = exp2f(mref[u] - M) / ((float)B * L);
    const float *prow = part + ((size_t)(wave * TPW + u) * cpb) * 64;
    for (int q = 0; q < nb; ++q) {
      // lanes 0..31: lower split of their row; lanes 32..63: upper split
      float v = wr * prow[q * 64 + 2 * (lane & 31) + (lane >> 5)];
      v = half_sum(v);
      if ((lane & 31) == 0) red[(q * NTL + t) * 2 + (lane >> 5)] = v;
    }
  }
  __syncthreads();
  for (int k = threadIdx.x; k < G * nb; k += NT) {
    const int hh = k % G, q = k / G;
    float lo = 0.0f, hi = 0.0f;
    for (int tq = 0; tq < QT; ++tq) {
      lo += red[(q * NTL + hh * QT + tq) * 2];
      hi += red[(q * NTL + hh * QT + tq) * 2 + 1];
    }
    const size_t o = (size_t)(g * G + hh) * N + j0 + q;
    a.lo[o] = lo;
    a.hi[o] = hi;
  }
}

template <int B, int TPW, bool I8>
hipError_t run(const Plan &p, const StatArgs &a, hipStream_t st) {
  const int nwaves = (p.G * B / 32 + TPW - 1) / TPW;
  dim3 grid(p.nch, p.Hkv), block(64 * nwaves);
  hipLaunchKernelGGL((k_ig_stats<B, TPW, I8, 1>), grid, block, 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = p.Hq * B;
  hipLaunchKernelGGL(k_ig_combine, dim3((rows + 255) / 256), dim3(256), 0, st, a.part, a.rowml,
                     rows, p.nch);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((k_ig_stats<B, TPW, I8, 2>), grid, block, 0, st, a);
  return hipGetLastError();
}

template <bool I8>
hipError_t dispatch(const Plan &p, const StatArgs &a, hipStream_t st) {
  const int tiles = p.G * p.B / 32;      // at most 64 (G*b <= 2048)
  if (p.B == 64) {
    if (tiles <= 16) return run<64, 1, I8>(p, a, st);
    if (tiles <= 32) return run<64, 2, I8>(p, a, st);
    return run<64, 4, I8>(p, a, st);
  }
  if (p.B == 128) {
    if (tiles <= 16) return run<128, 1, I8>(p, a, st);
    if (tiles <= 32) return run<128, 2, I8>(p, a, st);
    return run<128, 4, I8>(p, a, st);
  }
  if (tiles <= 16) return run<256, 1, I8>(p, a, st);
  if (tiles <= 32) return run<256, 2, I8>(p, a, st);
  return run<256, 4, I8>(p, a, st);
}


// Single pass when every workgroup (one per CU) can hold its chunk's partials
// in LDS and all are co-resident; *used tells the caller whether it ran.  The
// pooled key blocks stay in LDS too when they fit (for 64-token blocks, whose
// chunks are twice as long, they are otherwise stored block by block).
template <int B, int NT, int TPW, bool I8, bool KBS>
hipError_t launch1(const Plan &p, const StatArgs &a, size_t lds, unsigned int *bar, int32_t *status,
                   hipStream_t st, bool *used) {
  const int cus = cu_count();
  const void *fn = (const void *)k_ig_stats1<B, NT, TPW, I8, KBS>;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, NT, lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1 || (long)a.nch * p.Hkv > (long)per_cu * cus) return hipSuccess;
  // The grid (one workgroup per CU, at most per_cu per CU) fits the device at
  // once, and the launch follows the previous kernel of the stream, so all
  // workgroups are resident together; the barrier's wait is bounded anyway.
  Stat1Args args{a, bar, status};
  hipLaunchKernelGGL((k_ig_stats1<B, NT, TPW, I8, KBS>), dim3(a.nch, p.Hkv), dim3(NT), lds, st, args);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  *used = true;
  return hipSuccess;
}

template <int B, int NT, int TPW, bool I8>
hipError_t run1(const Plan &p, StatArgs a, unsigned int *bar, int32_t *status, hipStream_t st,
                bool *used) {
  *used = false;
  constexpr int NTL = NT / 64 * TPW;
  const int cus = cu_count();
  if (cus <= 0) return hipSuccess;
  int nch = cus / p.Hkv;
  if (nch > p.N) nch = p.N;
  if (nch < 1 || nch > p.nch) return hipSuccess;
  const int cpb = (p.N + nch - 1) / nch;
  nch = (p.N + cpb - 1) / cpb;
  a.nch = nch;
  a.cpb = cpb;
  const size_t lds = sizeof(float) * ((size_t)NTL * cpb * 64 + (size_t)cpb * NTL * 2 + (size_t)p.G * 128);
  const size_t lds_kbs = lds + sizeof(float) * (size_t)cpb * 128;
  const size_t static_lds = B * Tile<I8>::Stride + 4 * (NT / 64) * 128 + (I8 ? 4 * B : 4);
  if (lds_kbs + static_lds <= 160 * 1024)
    return launch1<B, NT, TPW, I8, true>(p, a, lds_kbs, bar, status, st, used);
  if constexpr (B == 64) {
    if (lds + static_lds <= 160 * 1024) return launch1<B, NT, TPW, I8, false>(p, a, lds, bar, status, st, used);
  }
  return hipSuccess;
}

template <bool I8>
hipError_t dispatch1(const Plan &p, const StatArgs &a, unsigned int *bar, int32_t *status,
                     hipStream_t st, bool *used) {
  const int tiles = p.G * p.B / 32;
  if (p.B == 64) {
    if (tiles <= 4) return run1<64, 256, 1, I8>(p, a, bar, status, st, used);
    if (tiles <= 8) return run1<64, 512, 1, I8>(p, a, bar, status, st, used);
    if (tiles <= 12) return run1<64, 768, 1, I8>(p, a, bar, status, st, used);
    if (tiles <= 16) return run1<64, 1024, 1, I8>(p, a, bar, status, st, used);
    if (tiles <= 32) return run1<64, 1024, 2, I8>(p, a, bar, status, st, used);
    return run1<64, 1024, 4, I8>(p, a, bar, status, st, used);
  }
  if (p.B == 128) {
    if (tiles <= 4) return run1<128, 256, 1, I8>(p, a, bar, status, st, used);
    if (tiles <= 8) return run1<128, 512, 1, I8>(p, a, bar, status, st, used);
    if (tiles <= 12) return run1<128, 768, 1, I8>(p, a, bar, status, st, used);
    if (tiles <= 16) return run1<128, 1024, 1, I8>(p, a, bar, status, st, used);
    if (tiles <= 32) return run1<128, 1024, 2, I8>(p, a, bar, status, st, used);
    return run1<128, 1024, 4, I8>(p, a, bar, status, st, used);
  }
  if (tiles <= 8) return run1<256, 512, 1, I8>(p, a, bar, status, st, used);
  if (tiles <= 16) return run1<256, 1024, 1, I8>(p, a, bar, status, st, used);
  if (tiles <= 32) return run1<256, 1024, 2, I8>(p, a, bar, status, st, used);
  return run1<256, 1024, 4, I8>(p, a, bar, status, st, used);
}

// Test hook: the int32 tile Q8[h, i*B + r] . K8[g, j*B + c] through the single-pass kernel's own
// staging (KStage register stage, padded LDS rows) and int8 tile code, at the workgroup size the
// kernel runs with for this shape; out[c * B + r].  The scale slot of the stage reads bytes of K
// (in bounds, unused).
template <int B, int NT>
__global__ void __launch_bounds__(NT) k_probe_stats_i8(const uint8_t *Q, const uint8_t *K, int S, int h, int g,
                                                       int i, int j, int32_t *out) {
  __shared__ __attribute__((aligned(16))) uint8_t ks[B * Tile<true>::Stride];
  __shared__ float sk[B];
  StatArgs a{};
  a.Q = Q;
  a.K = K;
  a.sK = (const float *)K;
  a.S = S;
  KStage<B, NT, true> stg;
  stg.load(a, g, j);
  stg.store(ks, sk);
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave >= B / 32) return;
  const int qr = wave * 32 + (lane & 31);
  const uint8_t *qp = Q + ((size_t)h * S + (size_t)i * B + qr) * Tile<true>::RowBytes + 16 * (lane >> 5);
  u32x4 qf[Tile<true>::KS];
#pragma unroll
  for (int s = 0; s < Tile<true>::KS; ++s) qf[s] = *(const u32x4 *)(qp + 32 * s);
  for (int kt = 0; kt < B / 32; ++kt) {
    const i32x16 acc = tile_raw_i8(ks, qf, kt);
#pragma unroll
    for (int r = 0; r < 16; ++r) out[(size_t)(kt * 32 + acc_row(r, lane)) * B + qr] = acc[r];
  }
}

template <int B, int NT>
hipError_t probe1(const Plan &p, const int8_t *Q8, const int8_t *K8, int h, int i, int j, int32_t *out,
                  hipStream_t st) {
  hipLaunchKernelGGL((k_probe_stats_i8<B, NT>), dim3(1), dim3(NT), 0, st, (const uint8_t *)Q8,
                     (const uint8_t *)K8, p.S, h, h / p.G, i, j, out);
  return hipGetLastError();
}

}  // namespace

// The workgroup size follows dispatch1 (tiles = G * b / 32).
hipError_t launch_probe_stats_i8(const Plan &p, const int8_t *Q8, const int8_t *K8, int h, int i, int j,
                                 int32_t *out, hipStream_t st) {
  const int tiles = p.G * p.B / 32;
  if (p.B == 64) {
    if (tiles <= 4) return probe1<64, 256>(p, Q8, K8, h, i, j, out, st);
    if (tiles <= 8) return probe1<64, 512>(p, Q8, K8, h, i, j, out, st);
    if (tiles <= 12) return probe1<64, 768>(p, Q8, K8, h, i, j, out, st);
    return probe1<64, 1024>(p, Q8, K8, h, i, j, out, st);
  }
  if (p.B == 128) {
    if (tiles <= 4) return probe1<128, 256>(p, Q8, K8, h, i, j, out, st);
    if (tiles <= 8) return probe1<128, 512>(p, Q8, K8, h, i, j, out, st);
    if (tiles <= 12) return probe1<128, 768>(p, Q8, K8, h, i, j, out, st);
    return probe1<128, 1024>(p, Q8, K8, h, i, j, out, st);
  }
  if (tiles <= 8) return probe1<256, 512>(p, Q8, K8, h, i, j, out, st);
  return probe1<256, 1024>(p, Q8, K8, h, i, j, out, st);
}

int cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev] = n;
  }
  return cache[dev];
}

hipError_t launch_ig_stats(const Plan &p, bool i8, const void *Q, const float *sQ, const void *K,
                           const float *sK, const Work &w, int32_t *status, hipStream_t st,
                           bool two_pass, bool *have_pe) {
  StatArgs a;
  a.Q = (const uint8_t *)Q;
  a.sQ = sQ;
  a.K = (const uint8_t *)K;
  a.sK = sK;
  a.S = p.S; a.N = p.N; a.G = p.G; a.nch = p.nch; a.cpb = p.cpb;
  a.c2 = kLog2e / sqrtf((float)p.d);
  a.part = w.part; a.rowml = w.rowml; a.lo = w.lo; a.hi = w.hi; a.kbar = w.kbar;
  a.pe = w.pe;
  a.sigma = 1.0f / sqrtf((float)p.d);
  *have_pe = false;
  bool used = false;
  // two_pass (the test entry point fp_index_two_pass) selects the two-pass form for any shape, so
  // that it can be checked at sizes whose single-pass partials would fit in LDS
  if (!two_pass) {
    hipError_t e = i8 ? dispatch1<true>(p, a, w.bar, status, st, &used)
                      : dispatch1<false>(p, a, w.bar, status, st, &used);
    *have_pe = used;
    if (e != hipSuccess || used) return e;
  }
  return i8 ? dispatch<true>(p, a, st) : dispatch<false>(p, a, st);
}

}  // namespace fp
