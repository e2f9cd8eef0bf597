// Sparse index set -> CSR -> grouped-query job list.
//
// The explainer ("FPGA24成果：FAST-Prefill稀疏注意力加速器", yunpan.plus)
// section 3.2 turns the sparse index sets into a compact job list before
// attention runs, with per-block use counts.  Here the index set of row
// (h, i) becomes CSR row h*N + i (key blocks ascending); the job of (KV group
// g, query block i) is the union of the G rows of that group's query heads,
// each entry carrying the bit mask of heads that use the block (the heads of
// a group share K/V, which is what staged blocks are reused for), and jobs
// are ordered by decreasing work so the longest start first.
//
// Every row is handled as a bit set over key blocks.  Vertical-slash rows are
// expanded on the fly from the two selections,
//   J(h, i) = {j in V : j <= i} u {i - o : o in Sl, o <= i} u {0, i};
// query-aware rows (and, in fp_build_jobs, every row of a given CSR) come
// from the row bit-set buffer.  One wave handles one job: lanes own 32-bit
// words of the rows, popcounts give the counts, OR gives the union.  Counts
// are turned into offsets by one scan launch (rows and jobs side by side),
// then a second pass over the same words writes columns and job entries.
//
// Equal-length sequences of a batch can run as one call with their heads side
// by side; the job order is then ranked per sequence, and the split and merge
// kernels at the end of this file move between that folded form and each
// sequence's own outputs.
#include "fp_common.hpp"
#include "fp_internal.hpp"

namespace fp {
namespace {

__global__ void k_status_init(int32_t *status, unsigned int *bar) {
  status[0] = 0;
  if (bar) bar[0] = 0u;
}

// Bits o..o+31 (o may be negative) of a bit set of nw words; absent bits are 0.
__device__ __forceinline__ uint32_t bits32(const uint32_t *m, int nw, int o) {
  const int k = o >> 5, sh = o & 31;
  const uint32_t lo = (k >= 0 && k < nw) ? m[k] : 0u;
  const uint32_t hi = (k + 1 >= 0 && k + 1 < nw) ? m[k + 1] : 0u;
  return sh == 0 ? lo : ((lo >> sh) | (hi << (32 - sh)));
}

// Bits of columns j <= i in word w.
__device__ __forceinline__ uint32_t causal_mask_word(int i, int w) {
  const int wi = i >> 5;
  if (w < wi) return 0xffffffffu;
  if (w > wi) return 0u;
  const int b = i & 31;
  return b == 31 ? 0xffffffffu : ((1u << (b + 1)) - 1u);
}

struct JobArgs {
  int N, G, Hkv, nw32;
  int share;                // heads of a KV group with the same pattern share the union of their rows
  const uint8_t *pattern;   // NULL: every row comes from rowbits
  const uint32_t *sel;      // [Hq][2][nw32]
  const uint32_t *rowbits;  // [Hq][N][nw32]
  int32_t *row_ptr, *col_idx;
  int32_t *job_ptr, *job_blk;
  uint32_t *job_mask;
  int32_t *jwork;
};

// Word w of the bit set of row (h, i).
__device__ __forceinline__ uint32_t row_word(const JobArgs &a, int h, int i, int w) {
  uint32_t word;
  if (!a.pattern || a.pattern[h] == FP_PATTERN_QUERY_AWARE) {
    word = a.rowbits[((size_t)h * a.N + i) * a.nw32 + w];
  } else {
    const uint32_t *vm = a.sel + (size_t)h * 2 * a.nw32;
    const uint32_t *sm = vm + a.nw32;
    // column j = 32w + k lies on slash offset o = i - j; the offsets for
    // k = 31..0 are the 32 consecutive bits from i - 32w - 31, bit-reversed.
    const uint32_t s = __builtin_bitreverse32(bits32(sm, a.nw32, i - 32 * w - 31));
    word = vm[w] | s;
    if (w == 0) word |= 1u;
    if (w == (i >> 5)) word |= 1u << (i & 31);
  }
  return word & causal_mask_word(i, w);
}

constexpr int kMaxG = 16;                 // the job mask holds one bit per head of a group
constexpr int kJobWaves = 4;

// Inclusive prefix sum over the wave (32-bit): Hillis-Steele inside each
// 16-lane row with DPP row shifts (lanes shifted in from outside the row add
// 0), then the totals of the earlier rows (lanes 15, 31, 47) are added.
__device__ __forceinline__ int wave_scan_incl(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);   // row_shr:8
  const int t0 = __builtin_amdgcn_readlane(x, 15), t1 = __builtin_amdgcn_readlane(x, 31),
            t2 = __builtin_amdgcn_readlane(x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row >= 1 ? t0 : 0) + (row >= 2 ? t1 : 0) + (row >= 3 ? t2 : 0);
}


// Pass 1 (WRITE = false): row counts (when ROWS) and union counts / work per job.
// Pass 2 (WRITE = true): columns of the rows (when ROWS) and job entries.
// GM >= G bounds the per-head arrays (registers) at compile time.
template <int GM, bool ROWS, bool WRITE>
__global__ void __launch_bounds__(64 * kJobWaves) k_jobs(JobArgs a) {
  const int lane = threadIdx.x & 63;
  const int job = blockIdx.x * kJobWaves + (threadIdx.x >> 6);
  if (job >= a.Hkv * a.N) return;
  const int g = job / a.N, i = job % a.N, G = a.G;
  const int nwi = (i >> 5) + 1;
  int rbase[GM];
  int ucarry = 0, work = 0, ucount = 0;
  int rcount[GM];
#pragma unroll
  for (int hh = 0; hh < GM; ++hh) {
    rcount[hh] = 0;
    rbase[hh] = 0;
    if (WRITE && ROWS && hh < G) rbase[hh] = a.row_ptr[(g * G + hh) * a.N + i];
  }
  const int jb = WRITE ? a.job_ptr[job] : 0, je = WRITE ? a.job_ptr[job + 1] : 0;
  for (int w0 = 0; w0 < nwi; w0 += 64) {
    const int w = w0 + lane;
    uint32_t wd[GM];
    uint32_t U = 0u;
#pragma unroll
    for (int hh = 0; hh < GM; ++hh) {
      wd[hh] = (hh < G && w < nwi) ? row_word(a, g * G + hh, i, w) : 0u;
      U |= wd[hh];
    }
    if (a.share) {
      // head-pattern sharing: each head takes the union of the rows of its group's heads
      // that have its pattern
      uint32_t uq = 0u, uv = 0u;
#pragma unroll
      for (int hh = 0; hh < GM; ++hh) {
        if (hh >= G) continue;
        if (a.pattern[g * G + hh] == FP_PATTERN_QUERY_AWARE) uq |= wd[hh];
        else uv |= wd[hh];
      }
#pragma unroll
      for (int hh = 0; hh < GM; ++hh)
        if (hh < G) wd[hh] = a.pattern[g * G + hh] == FP_PATTERN_QUERY_AWARE ? uq : uv;
    }
    if (!WRITE) {
#pragma unroll
      for (int hh = 0; hh < GM; ++hh)
        if (hh < G) rcount[hh] += wave_sum_int(__popc(wd[hh]));
      ucount += wave_sum_int(__popc(U));
    } else {
      if (ROWS) {
#pragma unroll
        for (int hh = 0; hh < GM; ++hh) {
          if (hh >= G) continue;
          const int r = (g * G + hh) * a.N + i;
          const int c = __popc(wd[hh]);
          const int incl = wave_scan_incl(c);
          int pos = rbase[hh] + incl - c;
          const int end = a.row_ptr[r + 1];
          uint32_t m = wd[hh];
          while (m && pos < end) {
            a.col_idx[pos++] = 32 * w + (__ffs(m) - 1);
            m &= m - 1u;
          }
          rbase[hh] += __builtin_amdgcn_readlane(incl, 63);
        }
      }
      const int c = __popc(U);
      const int incl = wave_scan_incl(c);
      int pos = jb + ucarry + incl - c;
      uint32_t m = U;
      while (m && pos < je) {
        const int b = __ffs(m) - 1;
        m &= m - 1u;
        uint32_t hm = 0u;
#pragma unroll
        for (int hh = 0; hh < GM; ++hh) hm |= ((wd[hh] >> b) & 1u) << hh;
        a.job_blk[pos] = 32 * w + b;
        a.job_mask[pos] = hm;
        ++pos;
      }
      ucarry += __builtin_amdgcn_readlane(incl, 63);
    }
  }
  if (!WRITE && lane == 0) {
#pragma unroll
    for (int hh = 0; hh < GM; ++hh) {
      if (hh >= G) continue;
      work += rcount[hh];
      if (ROWS) a.row_ptr[(g * G + hh) * a.N + i + 1] = rcount[hh];
    }
    a.job_ptr[job + 1] = ucount;
    a.jwork[job] = work;
  }
}

// Bit sets of the rows of a caller-supplied CSR (columns outside [0, i] are
// dropped: such blocks hold no key a query of block i may attend to).
__global__ void k_csr_to_bits(const int32_t *row_ptr, const int32_t *col_idx, int64_t ccap, int N,
                              int nw32, int rows, uint32_t *rowbits) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  const int i = r % N;
  uint32_t *dst = rowbits + (size_t)r * nw32;
  for (int w = 0; w <= (i >> 5); ++w) dst[w] = 0u;
  const int64_t e = min((int64_t)row_ptr[r + 1], ccap);
  for (int64_t p = max((int64_t)row_ptr[r], (int64_t)0); p < e; ++p) {
    const int j = col_idx[p];
    if (j >= 0 && j <= i) dst[j >> 5] |= 1u << (j & 31);
  }
}

// In-place scans, one array per workgroup: x[1..n] hold counts; afterwards
// x[k] = sum of the first k counts, clamped to cap (x[0] = 0).  A total above
// cap sets `bit` in status.  Tiles of 8 elements per thread, loaded coalesced.
constexpr int kScanThreads = 1024;
struct ScanJob {
  int32_t *x;
  int n;
  int64_t cap;
  uint32_t bit;
};
// In-place exclusive scan of counts x[1..n] into offsets x[0..n] (x[0] = 0),
// clamped to cap (the overflow is reported through `bit`).  Tiles of
// kScanThreads * 8 counts; a tile's total fits 32 bits (counts <= N <= 8192),
// the running carry is 64-bit.  One workgroup does a whole array, so its global
// accesses are kept coalesced: a tile is loaded lane-consecutively into LDS,
// each thread scans 8 consecutive counts from there, and the offsets go back
// through LDS the same way (one pad word per 32 keeps both LDS patterns free of
// bank conflicts).
__device__ void scan_counts(const ScanJob &s, int32_t *status) {
  constexpr int E = 8, T = kScanThreads;
  __shared__ int wtot[T / 64];
  __shared__ int stage[T * E + T * E / 32];
  auto at = [](int i) { return i + (i >> 5); };
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  long long carry = 0;
  for (int base = 0; base < s.n; base += T * E) {
#pragma unroll
    for (int u = 0; u < E; ++u) {
      const int k = base + u * T + tid;
      stage[at(u * T + tid)] = k < s.n ? s.x[1 + k] : 0;
    }
    __syncthreads();
    int v[E];
    int loc = 0;
#pragma unroll
    for (int u = 0; u < E; ++u) {
      v[u] = stage[at(tid * E + u)];
      loc += v[u];
    }
    const int incl = wave_scan_incl(loc);
    if (lane == 63) wtot[wave] = incl;
    __syncthreads();
    int t = lane < T / 64 ? wtot[lane] : 0;
    t = wave_scan_incl(t);
    const int wpre = wave > 0 ? __builtin_amdgcn_readlane(t, wave - 1) : 0;
    const int tile = __builtin_amdgcn_readlane(t, T / 64 - 1);
    long long run = carry + wpre + (incl - loc);
#pragma unroll
    for (int u = 0; u < E; ++u) {
      run += v[u];
      stage[at(tid * E + u)] = (int32_t)(run < s.cap ? run : s.cap);
    }
    __syncthreads();                               // (wtot is rewritten only after the next one)
#pragma unroll
    for (int u = 0; u < E; ++u) {
      const int k = base + u * T + tid;
      if (k < s.n) s.x[1 + k] = stage[at(u * T + tid)];
    }
    carry += tile;
    __syncthreads();                               // stage is refilled by the next tile
  }
  if (tid == 0) {
    s.x[0] = 0;
    if (carry > s.cap) atomicOr((unsigned int *)status, s.bit);
  }
}

// Job order by decreasing work, ties by lower job index: every job has the
// unique key (work << 32) | ~job.  Step 1 sorts each KV group's N keys in LDS
// (one workgroup per group, bitonic); step 2 places every job at its rank,
// i.e. its position in its own group plus, for each other group of the same
// sequence, the number of larger keys there (binary search).  With several
// sequences side by side (gps groups each), each sequence's jobs are ranked
// among themselves and fill that sequence's gps * N slots of the order.
constexpr int kSortThreads = 1024;
constexpr int kSortMax = 16384;
__device__ __forceinline__ unsigned long long job_key(const int32_t *jwork, int job) {
  return ((unsigned long long)(uint32_t)jwork[job] << 32) | (0xffffffffu - (uint32_t)job);
}

__device__ void sort_group(const int32_t *jwork, int N, int g, unsigned long long *sorted,
                           unsigned long long *keys) {
  const int tid = threadIdx.x;
  int P = 1;
  while (P < N) P <<= 1;
  for (int k = tid; k < P; k += kSortThreads) keys[k] = k < N ? job_key(jwork, g * N + k) : 0ull;
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = tid; t < P / 2; t += kSortThreads) {
        const int pos = 2 * t - (t & (stride - 1));
        const int q = pos + stride;
        const bool desc = (pos & size) == 0;
        const unsigned long long x = keys[pos], y = keys[q];
        if ((x < y) == desc) {
          keys[pos] = y;
          keys[q] = x;
        }
      }
      __syncthreads();
    }
  }
  for (int k = tid; k < N; k += kSortThreads) sorted[(size_t)g * N + k] = keys[k];
}

// One launch for both steps that follow the count pass: workgroups 0 .. nscan-1
// scan the job (and row) counts; the next Hkv workgroups each sort one KV
// group's job keys (the sort needs only the job work).
static_assert(kScanThreads == kSortThreads, "the scans and sorts share one launch");
__global__ void __launch_bounds__(kScanThreads) k_scan_sort(ScanJob s0, ScanJob s1, int nscan, int32_t *status,
                                                            const int32_t *jwork, int N,
                                                            unsigned long long *sorted) {
  extern __shared__ unsigned long long keys[];
  const int blk = blockIdx.x;
  if (blk < nscan) scan_counts(blk == 0 ? s0 : s1, status);
  else sort_group(jwork, N, blk - nscan, sorted, keys);
}

// With LDS, every workgroup first copies all Hkv * N sorted keys into LDS (at most
// kRankLdsKeys) and searches there.
constexpr int kRankLdsKeys = 16384;       // 128 KiB of keys
template <bool LDS>
__global__ void k_rank_jobs(const unsigned long long *sorted, int N, int Hkv, int gps, int32_t *order) {
  extern __shared__ unsigned long long skeys[];
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (LDS) {
    for (int t = threadIdx.x; t < Hkv * N; t += blockDim.x) skeys[t] = sorted[t];
    __syncthreads();
  }
  if (e >= Hkv * N) return;
  const unsigned long long *src = LDS ? skeys : sorted;
  const int g = e / N, k = e % N;
  const int s0 = g / gps * gps;                              // the sequence's first group
  const unsigned long long key = src[e];
  int rank = k;
  for (int o = s0; o < s0 + gps; ++o) {
    if (o == g) continue;
    const unsigned long long *l = src + (size_t)o * N;      // descending
    int lo = 0, hi = N;                                      // count of entries > key
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (l[mid] > key) lo = mid + 1; else hi = mid;
    }
    rank += lo;
  }
  order[(size_t)s0 * N + rank] = (int32_t)(0xffffffffu - (uint32_t)(key & 0xffffffffull));
}

template <int GM, bool WRITE>
hipError_t run_jobs(const Plan &p, const JobArgs &a, hipStream_t st, bool rows) {
  const dim3 grid((p.Hkv * p.N + kJobWaves - 1) / kJobWaves), block(64 * kJobWaves);
  if (rows) hipLaunchKernelGGL((k_jobs<GM, true, WRITE>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((k_jobs<GM, false, WRITE>), grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t build(const Plan &p, const fp_index_out *io, const Work &w, hipStream_t st, bool rows,
                 bool share = false) {
  JobArgs a;
  a.N = p.N; a.G = p.G; a.Hkv = p.Hkv; a.nw32 = p.nw32;
  a.share = rows && share;
  a.pattern = rows ? io->pattern : nullptr;
  a.sel = w.sel;
  a.rowbits = w.rowbits;
  a.row_ptr = io->row_ptr; a.col_idx = io->col_idx;
  a.job_ptr = io->job_ptr; a.job_blk = io->job_blk; a.job_mask = io->job_mask;
  a.jwork = w.jwork;
  const int jobs = p.Hkv * p.N, rcount = p.Hq * p.N;
  hipError_t e;
  if (p.G <= 1) e = run_jobs<1, false>(p, a, st, rows);
  else if (p.G <= 2) e = run_jobs<2, false>(p, a, st, rows);
  else if (p.G <= 4) e = run_jobs<4, false>(p, a, st, rows);
  else if (p.G <= 8) e = run_jobs<8, false>(p, a, st, rows);
  else e = run_jobs<kMaxG, false>(p, a, st, rows);
  if (e != hipSuccess) return e;
  const ScanJob sj{io->job_ptr, jobs, io->job_cap, (uint32_t)FP_STATUS_JOB_OVERFLOW};
  const ScanJob sr{io->row_ptr, rcount, io->col_cap, (uint32_t)FP_STATUS_CSR_OVERFLOW};
  const int nscan = rows ? 2 : 1;
  // every supported N (at most 8192, checked by make_plan) sorts a group in LDS
  static_assert(kSortMax >= 8192, "a KV group's job keys fit in LDS for every supported N");
  int P = 1;
  while (P < p.N) P <<= 1;
  const size_t slds = sizeof(unsigned long long) * P;
  e = ensure_dyn_lds((const void *)k_scan_sort, slds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_scan_sort, dim3(nscan + p.Hkv), dim3(kScanThreads), slds, st, sj, sr, nscan,
                     io->status, w.jwork, p.N, w.jkeys);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (p.G <= 1) e = run_jobs<1, true>(p, a, st, rows);
  else if (p.G <= 2) e = run_jobs<2, true>(p, a, st, rows);
  else if (p.G <= 4) e = run_jobs<4, true>(p, a, st, rows);
  else if (p.G <= 8) e = run_jobs<8, true>(p, a, st, rows);
  else e = run_jobs<kMaxG, true>(p, a, st, rows);
  if (e != hipSuccess) return e;
  if (jobs <= kRankLdsKeys) {
    const size_t lds = sizeof(unsigned long long) * jobs;
    e = ensure_dyn_lds((const void *)k_rank_jobs<true>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_rank_jobs<true>, dim3((jobs + 1023) / 1024), dim3(1024), lds, st, w.jkeys, p.N, p.Hkv,
                       p.seq_groups, io->job_order);
  } else {
    hipLaunchKernelGGL(k_rank_jobs<false>, dim3((jobs + 255) / 256), dim3(256), 0, st, w.jkeys, p.N, p.Hkv,
                       p.seq_groups, io->job_order);
  }
  return hipGetLastError();
}

// Use counters of the key blocks ([E] 3.2: each block's consumer count, kept while the job
// list is built, drives the liveness of the block in the cache).  One thread per job (g, i)
// adds 1 to uses[g][j] and the number of heads in the entry's mask to head_uses[g][j] for
// every entry j of the job; integer atomics, so the counts do not depend on the order.
__global__ void k_zero_uses(int32_t *uses, int32_t *head_uses, int n) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= n) return;
  uses[k] = 0;
  if (head_uses) head_uses[k] = 0;
}
__global__ void k_block_uses(const int32_t *job_ptr, const int32_t *job_blk, const uint32_t *job_mask, int N,
                             int jobs, int32_t *uses, int32_t *head_uses) {
  const int job = blockIdx.x * blockDim.x + threadIdx.x;
  if (job >= jobs) return;
  const int g = job / N, i = job % N;
  for (int e = job_ptr[job]; e < job_ptr[job + 1]; ++e) {
    const int j = job_blk[e];
    if (j < 0 || j > i) continue;                  // not a key block this job may use
    atomicAdd(uses + (size_t)g * N + j, 1);
    if (head_uses) atomicAdd(head_uses + (size_t)g * N + j, __popc(job_mask[e]));
  }
}

}  // namespace

hipError_t launch_block_uses(const Plan &p, const fp_index_out *jobs, int32_t *uses, int32_t *head_uses,
                             hipStream_t st) {
  const int n = p.Hkv * p.N;
  hipLaunchKernelGGL(k_zero_uses, dim3((n + 255) / 256), dim3(256), 0, st, uses, head_uses, n);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_block_uses, dim3((n + 255) / 256), dim3(256), 0, st, jobs->job_ptr, jobs->job_blk,
                     jobs->job_mask, p.N, n, uses, head_uses);
  return hipGetLastError();
}

hipError_t launch_status_init(int32_t *status, unsigned int *bar, hipStream_t st) {
  hipLaunchKernelGGL(k_status_init, dim3(1), dim3(1), 0, st, status, bar);
  return hipGetLastError();
}

hipError_t launch_rows_and_jobs(const Plan &p, const fp_index_out *out, const Work &w,
                                hipStream_t st, bool share) {
  return build(p, out, w, st, true, share);
}

hipError_t launch_jobs(const Plan &p, const fp_index_out *io, const Work &w, hipStream_t st) {
  const int rows = p.Hq * p.N;
  hipLaunchKernelGGL(k_csr_to_bits, dim3((rows + 255) / 256), dim3(256), 0, st, io->row_ptr,
                     io->col_idx, io->col_cap, p.N, p.nw32, rows, w.rowbits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return build(p, io, w, st, false);
}

// ---------------------------------------------------------------------------
// Equal-length sequences run side by side.  A batch of k sequences of one length is one call with
// k * Hq query heads and k * Hkv KV heads: every quantity is per head or per KV group, and the job
// order and the attention's chunk rotation are taken per sequence (Plan::seq_groups).  These two
// kernels move between that folded form and the caller's per-sequence outputs; one workgroup per
// sequence.

// Index outputs of the folded call -> each sequence's fp_index_out, with that output's own
// capacities: row and job offsets rebased to the sequence and clamped to its capacity, columns and
// job entries copied up to it, the overflow bits set in its status word as a call of its own would.
__global__ void __launch_bounds__(1024) k_split_index(FoldArgs a) {
  const int t = a.t0 + blockIdx.x;                           // the sequence within the folded call
  const fp_index_out &o = a.seq[blockIdx.x];
  const int nr = a.Hq * a.N, nj = a.Hkv * a.N;
  const size_t rb = (size_t)t * nr, jb = (size_t)t * nj;
  const int r0 = a.f.row_ptr[rb], rtot = a.f.row_ptr[rb + nr] - r0;
  const int j0 = a.f.job_ptr[jb], jtot = a.f.job_ptr[jb + nj] - j0;
  for (int r = threadIdx.x; r <= nr; r += blockDim.x)
    o.row_ptr[r] = (int32_t)min((int64_t)(a.f.row_ptr[rb + r] - r0), o.col_cap);
  const int nc = (int)min((int64_t)rtot, o.col_cap);
  for (int q = threadIdx.x; q < nc; q += blockDim.x) o.col_idx[q] = a.f.col_idx[r0 + q];
  for (int j = threadIdx.x; j <= nj; j += blockDim.x)
    o.job_ptr[j] = (int32_t)min((int64_t)(a.f.job_ptr[jb + j] - j0), o.job_cap);
  const int ne = (int)min((int64_t)jtot, o.job_cap);
  for (int q = threadIdx.x; q < ne; q += blockDim.x) {
    o.job_blk[q] = a.f.job_blk[j0 + q];
    o.job_mask[q] = a.f.job_mask[j0 + q];
  }
  for (int q = threadIdx.x; q < nj; q += blockDim.x) o.job_order[q] = a.f.job_order[jb + q] - (int32_t)jb;
  for (int h = threadIdx.x; h < a.Hq; h += blockDim.x) {
    o.pattern[h] = a.f.pattern[(size_t)t * a.Hq + h];
    o.jsd[h] = a.f.jsd[(size_t)t * a.Hq + h];
  }
  if (o.stats && a.f.stats) {
    const size_t HNf = (size_t)a.k * nr;                       // folded [3][k * Hq][N]
    for (int e = threadIdx.x; e < 3 * nr; e += blockDim.x) {
      const int c = e / nr, q = e - c * nr;
      o.stats[e] = a.f.stats[c * HNf + rb + q];
    }
  }
  if (threadIdx.x == 0)
    o.status[0] = a.f.status[0] | (rtot > o.col_cap ? (int32_t)FP_STATUS_CSR_OVERFLOW : 0) |
                  (jtot > o.job_cap ? (int32_t)FP_STATUS_JOB_OVERFLOW : 0);
}

// Each sequence's job list -> the folded one: job offsets shifted by the entries of the sequences
// before it, entries copied after theirs, and the orders interleaved (position q * k + t holds
// sequence t's q-th job), which keeps every sequence's longest jobs first.  Launches cover
// consecutive groups of sequences in order; a group starts from the offset the previous one wrote
// (the folded job_ptr at its first sequence).
__global__ void __launch_bounds__(1024) k_merge_jobs(FoldArgs a) {
  const int t = a.t0 + blockIdx.x;
  const fp_index_out &in = a.seq[blockIdx.x];
  const int nj = a.Hkv * a.N;
  // offsets are kept within a sequence's worst case (the merged list has room for exactly that
  // much per sequence), whatever the input holds
  const int cap = (int)((int64_t)nj * (a.N + 1) / 2);
  auto clampj = [&](int v) { return min(max(v, 0), cap); };
  int off = a.t0 == 0 ? 0 : a.f.job_ptr[(size_t)a.t0 * nj];
  for (int u = 0; u < (int)blockIdx.x; ++u) off += clampj(a.seq[u].job_ptr[nj]);
  const int tot = clampj(in.job_ptr[nj]);
  for (int j = threadIdx.x; j <= nj; j += blockDim.x) a.f.job_ptr[(size_t)t * nj + j] = off + clampj(in.job_ptr[j]);
  for (int q = threadIdx.x; q < tot; q += blockDim.x) {
    a.f.job_blk[off + q] = in.job_blk[q];
    a.f.job_mask[off + q] = in.job_mask[q];
  }
  for (int q = threadIdx.x; q < nj; q += blockDim.x)
    a.f.job_order[(size_t)q * a.k + t] = in.job_order[q] + t * nj;
}

hipError_t launch_split_index(const FoldArgs &a, hipStream_t st) {
  hipLaunchKernelGGL(k_split_index, dim3(a.n), dim3(1024), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_merge_jobs(const FoldArgs &a, hipStream_t st) {
  hipLaunchKernelGGL(k_merge_jobs, dim3(a.n), dim3(1024), 0, st, a);
  return hipGetLastError();
}

}  // namespace fp
