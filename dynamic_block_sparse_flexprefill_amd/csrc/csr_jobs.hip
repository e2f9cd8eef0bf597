// Sparse index set -> CSR -> grouped-query job list.
//
// The explainer ("FPGA24成果：FAST-Prefill稀疏注意力加速器", yunpan.plus)
// section 3.2 turns the sparse index sets into a compact job list before
// attention runs, with per-block use counts.  Here the index set of row
// (h, i) becomes CSR row h*N + i (key blocks ascending); the job of (KV group
// g, query block i) is the union of the G rows of that group's query heads,
// each entry carrying the bit mask of heads that use the block (the heads of
// a group share K/V, which is what the staged blocks are reused for), and
// jobs are ordered by decreasing work so the longest start first.
//
// Vertical-slash rows are expanded here from the two selections:
//   J(h, i) = {j in V : j <= i} u {i - o : o in Sl, o <= i} u {0, i};
// query-aware rows arrive as bit sets.
#include "fp_common.hpp"
#include "fp_internal.hpp"

namespace fp {
namespace {

__global__ void k_status_init(int32_t *status) { status[0] = 0; }

// Bits j..j+31 (j may be negative) of a bit set of nw words; absent bits are 0.
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

struct RowArgs {
  int N, nw32, Hq;
  const uint8_t *pattern;
  const uint32_t *sel;     // [Hq][2][nw32]
  const uint32_t *qabits;  // [Hq][N][nw32]
  int32_t *row_ptr;
  int32_t *col_idx;
  int64_t cap;
  int32_t *status;
};

// Word w of the bit set of row (h, i).
__device__ __forceinline__ uint32_t row_word(const RowArgs &a, int h, int i, int w, bool qa) {
  uint32_t word;
  if (qa) {
    word = a.qabits[((size_t)h * a.N + i) * a.nw32 + w];
  } else {
    const uint32_t *vm = a.sel + (size_t)h * 2 * a.nw32;
    const uint32_t *sm = vm + a.nw32;
    // column j = 32w + k is on slash offset o = i - j; offsets for k = 31..0
    // are the 32 consecutive bits starting at i - 32w - 31, bit-reversed.
    const uint32_t s = __builtin_bitreverse32(bits32(sm, a.nw32, i - 32 * w - 31));
    word = vm[w] | s;
    if (w == 0) word |= 1u;
    if (w == (i >> 5)) word |= 1u << (i & 31);
  }
  return word & causal_mask_word(i, w);
}

__global__ void k_rows_count(RowArgs a) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= a.Hq * a.N) return;
  const int h = r / a.N, i = r % a.N;
  const bool qa = a.pattern[h] == FP_PATTERN_QUERY_AWARE;
  int cnt = 0;
  for (int w = 0; w <= (i >> 5); ++w) cnt += __popc(row_word(a, h, i, w, qa));
  a.row_ptr[r + 1] = cnt;
}

__global__ void k_rows_write(RowArgs a) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= a.Hq * a.N) return;
  const int h = r / a.N, i = r % a.N;
  const bool qa = a.pattern[h] == FP_PATTERN_QUERY_AWARE;
  int pos = a.row_ptr[r];
  const int end = a.row_ptr[r + 1];
  for (int w = 0; w <= (i >> 5) && pos < end; ++w) {
    uint32_t m = row_word(a, h, i, w, qa);
    while (m && pos < end) {
      const int b = __ffs(m) - 1;
      m &= m - 1u;
      a.col_idx[pos++] = 32 * w + b;
    }
  }
}

// In-place scan: a[1..n] hold counts; afterwards a[k] = sum of the first k
// counts, clamped to cap (a[0] = 0).  A total above cap sets `bit` in status.
constexpr int kScanThreads = 1024;
__global__ void __launch_bounds__(kScanThreads) k_scan_counts(int32_t *a, int n, int64_t cap,
                                                              int32_t *status, uint32_t bit) {
  __shared__ long long wsum[kScanThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int seg = (n + kScanThreads - 1) / kScanThreads;
  const int beg = 1 + tid * seg, end = min(n + 1, beg + seg);
  long long local = 0;
  for (int k = beg; k < end; ++k) local += a[k];
  // inclusive wave scan
  long long x = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const long long y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  long long base = 0;
  for (int w = 0; w < wave; ++w) base += wsum[w];
  long long run = base + x - local;     // exclusive prefix of this segment
  for (int k = beg; k < end; ++k) {
    run += a[k];
    a[k] = (int32_t)(run < cap ? run : cap);
  }
  if (tid == 0) a[0] = 0;
  if (tid == kScanThreads - 1) {
    long long total = 0;
    for (int w = 0; w < kScanThreads / 64; ++w) total += wsum[w];
    if (total > cap) atomicOr((unsigned int *)status, bit);
  }
}

struct JobArgs {
  int N, G, Hkv;
  const int32_t *row_ptr, *col_idx;
  int32_t *job_ptr, *job_blk;
  uint32_t *job_mask;
  int32_t *jwork;
  int64_t cap;
  int64_t ccap;   // entries of col_idx
};

constexpr int kMaxG = 16;

// G-way merge of the rows of job (g, i); WRITE selects counting or writing.
template <bool WRITE>
__global__ void k_jobs(JobArgs a) {
  const int job = blockIdx.x * blockDim.x + threadIdx.x;
  if (job >= a.Hkv * a.N) return;
  const int g = job / a.N, i = job % a.N;
  int p[kMaxG], e[kMaxG];
  int work = 0;
  for (int hh = 0; hh < a.G; ++hh) {
    const int r = (g * a.G + hh) * a.N + i;
    e[hh] = (int)min((int64_t)a.row_ptr[r + 1], a.ccap);
    p[hh] = min(a.row_ptr[r], e[hh]);
    work += e[hh] - p[hh];
  }
  int cnt = 0;
  int pos = WRITE ? a.job_ptr[job] : 0;
  const int end = WRITE ? a.job_ptr[job + 1] : 0;
  while (true) {
    int cur = 0x7fffffff;
    for (int hh = 0; hh < a.G; ++hh)
      if (p[hh] < e[hh]) cur = min(cur, a.col_idx[p[hh]]);
    if (cur == 0x7fffffff) break;
    uint32_t m = 0u;
    for (int hh = 0; hh < a.G; ++hh)
      if (p[hh] < e[hh] && a.col_idx[p[hh]] == cur) {
        m |= 1u << hh;
        ++p[hh];
      }
    if (WRITE) {
      if (pos >= end) break;
      a.job_blk[pos] = cur;
      a.job_mask[pos] = m;
      ++pos;
    } else {
      ++cnt;
    }
  }
  if (!WRITE) {
    a.job_ptr[job + 1] = cnt;
    a.jwork[job] = work;
  }
}

// Job order by decreasing work, ties by lower job index (bitonic sort in LDS).
constexpr int kSortThreads = 1024;
constexpr int kSortMax = 16384;
__global__ void __launch_bounds__(kSortThreads) k_jobs_order(const int32_t *jwork, int n, int N,
                                                             int Hkv, int32_t *order) {
  extern __shared__ unsigned long long keys[];
  const int tid = threadIdx.x;
  if (n > kSortMax) {   // too many to sort in LDS: latest query blocks first
    for (int k = tid; k < n; k += kSortThreads) {
      const int i = N - 1 - k / Hkv, g = k % Hkv;
      order[k] = g * N + i;
    }
    return;
  }
  int P = 1;
  while (P < n) P <<= 1;
  for (int k = tid; k < P; k += kSortThreads)
    keys[k] = k < n ? (((unsigned long long)(uint32_t)jwork[k] << 32) | (0xffffffffu - (uint32_t)k)) : 0ull;
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
  for (int k = tid; k < n; k += kSortThreads) order[k] = (int32_t)(0xffffffffu - (uint32_t)(keys[k] & 0xffffffffull));
}

}  // namespace

hipError_t launch_status_init(int32_t *status, hipStream_t st) {
  hipLaunchKernelGGL(k_status_init, dim3(1), dim3(1), 0, st, status);
  return hipGetLastError();
}

hipError_t launch_rows_to_csr(const Plan &p, const fp_index_out *out, const Work &w,
                              hipStream_t st) {
  RowArgs a;
  a.N = p.N; a.nw32 = p.nw32; a.Hq = p.Hq;
  a.pattern = out->pattern; a.sel = w.sel; a.qabits = w.qabits;
  a.row_ptr = out->row_ptr; a.col_idx = out->col_idx; a.cap = out->col_cap;
  a.status = out->status;
  const int rows = p.Hq * p.N;
  hipLaunchKernelGGL(k_rows_count, dim3((rows + 255) / 256), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_scan_counts, dim3(1), dim3(kScanThreads), 0, st, out->row_ptr, rows,
                     out->col_cap, out->status, (uint32_t)FP_STATUS_CSR_OVERFLOW);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_rows_write, dim3((rows + 255) / 256), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_jobs(const Plan &p, const fp_index_out *io, const Work &w, hipStream_t st) {
  JobArgs a;
  a.N = p.N; a.G = p.G; a.Hkv = p.Hkv;
  a.row_ptr = io->row_ptr; a.col_idx = io->col_idx;
  a.job_ptr = io->job_ptr; a.job_blk = io->job_blk; a.job_mask = io->job_mask;
  a.jwork = w.jwork;
  a.cap = io->job_cap;
  a.ccap = io->col_cap;
  const int jobs = p.Hkv * p.N;
  const dim3 grid((jobs + 127) / 128), block(128);
  hipLaunchKernelGGL(k_jobs<false>, grid, block, 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_scan_counts, dim3(1), dim3(kScanThreads), 0, st, io->job_ptr, jobs,
                     io->job_cap, io->status, (uint32_t)FP_STATUS_JOB_OVERFLOW);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_jobs<true>, grid, block, 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  int P = 1;
  while (P < jobs) P <<= 1;
  const size_t lds = jobs <= kSortMax ? sizeof(unsigned long long) * P : 0;
  if (lds > 0) {
    e = hipFuncSetAttribute((const void *)k_jobs_order, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_jobs_order, dim3(1), dim3(kSortThreads), lds, st, w.jwork, jobs, p.N,
                     p.Hkv, io->job_order);
  return hipGetLastError();
}

}  // namespace fp
