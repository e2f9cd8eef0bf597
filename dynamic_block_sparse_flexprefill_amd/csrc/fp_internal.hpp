// Host-side plan (shape checks and workspace carving) and the launchers each
// kernel file exports to the C-ABI layer.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fpattn.h"

namespace fp {

// Everything the launchers need about one problem, derived from fp_shape.
struct Plan {
  int S, B, Hq, Hkv, d, N, G;
  int seq_groups;    // KV groups per sequence: Hkv, or fewer when several equal-length sequences
                     // run as one call with their heads side by side (job order and chunk
                     // rotation are then taken per sequence)
  int nw32;          // 32-bit words per row bitmask: ceil(N / 32)
  int nch;           // key-block chunks of the statistics (stats_chunks)
  // workspace layout (byte offsets from the workspace base)
  size_t off_lohi;   // float2 [Hq*N*B]    per-(row, key block) split sums of the statistics
  size_t off_ml;     // float2 [Hq*nch*B]  per-(row, chunk) (reference max, sum)
  size_t off_rowml;  // float2 [Hq*B]      per-row (max, 1 / (b * sum))
  size_t off_qlast;  // float  [Hq*128]    mean of each head's last query block
  size_t off_lo;     // float  [Hq*N]      lower-split block mass
  size_t off_hi;     // float  [Hq*N]      upper-split block mass
  size_t off_kbar;   // float  [Hkv*N*d]   mean-pooled key blocks
  size_t off_sel;    // u32    [Hq*2*nw32] vertical / slash selections (bit sets)
  size_t off_rowbits; // u32   [Hq*N*nw32] row bit sets (query-aware rows; every row in fp_build_jobs)
  size_t off_qbar;   // float  [Hq*N*d]    mean-pooled query blocks (query-aware heads)
  size_t off_pe;     // float  [Hq*N]      pooled-estimate logits sigma * qbar_last . kbar_j
  size_t off_jwork;  // int32  [Hkv*N]     work per grouped job
  size_t off_bar;    // u32    [64]        [32]: unit counter of the persistent attention kernel
  size_t off_jkeys;  // u64    [Hkv*N]     per-group sorted job keys
  size_t off_utab;   // int4   [Hkv*N*b/32] attention work units {job, first entry, chunks, start}
  size_t total;      // bytes every call but fp_attn_i8 needs
  size_t off_vw;     // bf16   [Hkv*S*d]   fp_attn_i8: the int8 V codes widened to bf16
  size_t total_i8;   // bytes fp_attn_i8 needs (fp_workspace_bytes variant 1)
};

// Validates the shape (FP_EINVAL / FP_EUNSUPPORTED) and fills *p.
int make_plan(const fp_shape *s, Plan *p);

// Typed views of the workspace.
struct Work {
  float2 *lohi, *ml, *rowml;
  float *qlast;
  float *lo, *hi, *kbar;
  uint32_t *sel, *rowbits;
  float *qbar;
  float *pe;
  int32_t *jwork;
  unsigned int *bar;
  unsigned long long *jkeys;
  int4 *utab;
};
Work carve(const Plan &p, void *ws);

// ---- launchers: each returns hipSuccess or the launch error.
// Key-block chunks of the statistics for a shape (chunk boundaries depend on the shape only).
int stats_chunks(int B, int G, int N);
// Statistics of the last query block against every key block (K streamed once), then merged:
// lo, hi, kbar and the pooled-estimate logits pe in the workspace.
hipError_t launch_ig_stats(const Plan &p, bool i8, const void *Q, const float *sQ,
                           const void *K, const float *sK, const Work &w, hipStream_t st,
                           int32_t *status = nullptr);
// Per head: pooled estimate, divergence, pattern, vertical / slash selection.
// have_pe: the pooled-estimate logits are in w.pe (else they are computed here).
hipError_t launch_ig_finalize(const Plan &p, bool i8, const void *Q, const float *sQ,
                              float gamma, float tau, const fp_index_out *out,
                              const Work &w, hipStream_t st, bool have_pe);
// Query-aware rows: pooled queries of every block against pooled keys.
// qbar_in (or NULL): pooled queries [Hq][N][128] from the caller, so Q is not read.
hipError_t launch_ig_qa(const Plan &p, bool i8, const void *Q, const float *sQ, float gamma,
                        const uint8_t *pattern, const Work &w, hipStream_t st, const float *qbar_in = nullptr);
// QKV projection Y = X W^T with the fused epilogue (rotation, bf16 head-major store, block means,
// optional int8 codes and scales); see qkv_proj.hip.
hipError_t launch_qkv_proj(int S, int D, int Hq, int Hkv, int b, const void *X, const void *W, const float *cosT,
                           const float *sinT, void *Q, void *K, void *V, float *qbar, float *kbar, int8_t *Q8,
                           float *sQ, int8_t *K8, float *sK, int8_t *V8, float *sV, hipStream_t st);
// Row bit sets -> CSR rows, grouped-query job list and its work order.
// share: heads of a KV group with the same pattern take the union of their rows.
hipError_t launch_rows_and_jobs(const Plan &p, const fp_index_out *out, const Work &w,
                                hipStream_t st, bool share = false);
// Use counters of the key blocks from a job list: uses[g][j] job entries, head_uses[g][j] (or NULL)
// (head, query block) pairs per key block.
hipError_t launch_block_uses(const Plan &p, const fp_index_out *jobs, int32_t *uses, int32_t *head_uses,
                             hipStream_t st);
// Caller-supplied CSR -> grouped-query job list and its work order.
hipError_t launch_jobs(const Plan &p, const fp_index_out *io, const Work &w, hipStream_t st);
// status[0] = 0 and, when bar is not NULL, bar[0] = 0
hipError_t launch_status_init(int32_t *status, unsigned int *bar, hipStream_t st);

// Equal-length sequences run as one call (side by side): the folded call's outputs f (in the
// workspace, k sequences) and the own outputs seq[0..n) of its sequences t0 .. t0 + n - 1 (the
// caller's, passed by value, at most kFoldArgs per launch).
constexpr int kFoldRun = 64;        // sequences per folded call
constexpr int kFoldArgs = 24;       // sequences per split or merge launch (kernel arguments)
struct FoldArgs {
  fp_index_out f;
  fp_index_out seq[kFoldArgs];
  int k, t0, n, Hq, Hkv, N;         // Hq, Hkv: one sequence's heads
};
// Folded index outputs -> each sequence's fp_index_out (rebased, clamped to its capacities).
hipError_t launch_split_index(const FoldArgs &a, hipStream_t st);
// Each sequence's job list -> the folded job list (job fields of f).
hipError_t launch_merge_jobs(const FoldArgs &a, hipStream_t st);
// Block-sparse attention over the CSR rows.
// compute units of the current device (cached; 0 if the query fails)
int cu_count();
hipError_t ensure_dyn_lds(const void *fn, size_t bytes);
int occupancy_per_cu(const void *fn, int threads);
// nseg > 1: split-KV schedule of fp_attn_split (bf16, b >= 128): the nsplit longest jobs in nseg
// segments each, partial rows in `part`, merged by a combine kernel.
hipError_t launch_attn(const Plan &p, bool i8, const void *Q, const float *sQ, const void *K,
                       const float *sK, const void *V, const float *sV, const fp_index_out *csr,
                       void *O, unsigned int *ctr, int4 *utab, hipStream_t st, int nsplit = 0,
                       int nseg = 1, float *part = nullptr, uint16_t *vw = nullptr);
// Partial-output floats per split slot (G heads x b rows x padded row).
size_t attn_split_slot_floats(const Plan &p);
// One exact int8 score tile through the W8A8 attention kernel's staging and tile code.
hipError_t launch_probe_attn_i8(const Plan &p, const int8_t *Q8, const int8_t *K8, int h, int i,
                                int j, int32_t *out, hipStream_t st);
// The same through the single-pass statistics kernel's staging and tile code.
hipError_t launch_probe_stats_i8(const Plan &p, const int8_t *Q8, const int8_t *K8, int h, int i,
                                 int j, int32_t *out, hipStream_t st);

}  // namespace fp
