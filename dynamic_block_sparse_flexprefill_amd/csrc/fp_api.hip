// C-ABI layer of libfpattn: argument validation, workspace carving and the
// launch sequence of each call.  No device memory is allocated here and no
// call synchronises the stream.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "fp_internal.hpp"

// Scratch of fp_index_static: one buffer per GPU, held by the library's code object for the
// life of the process.  Host code never uses this name as an address (on the host it is only a
// stand-in for the symbol); the device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) unsigned char scratch[FP_STATIC_SCRATCH_BYTES];

namespace fp {

static size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

int make_plan(const fp_shape *s, Plan *p) {
  if (!s || !p) return FP_EINVAL;
  if (s->S <= 0 || s->b <= 0 || s->Hq <= 0 || s->Hkv <= 0 || s->d <= 0) return FP_EINVAL;
  if (s->S % s->b != 0 || s->Hq % s->Hkv != 0) return FP_EINVAL;
  if (s->d != 128 || (s->b != 64 && s->b != 128 && s->b != 256)) return FP_EUNSUPPORTED;
  const int N = s->S / s->b, G = s->Hq / s->Hkv;
  if (N > 8192 || (int64_t)G * s->b > 2048 || G > 16) return FP_EUNSUPPORTED;
  memset(p, 0, sizeof(*p));
  p->S = s->S; p->B = s->b; p->Hq = s->Hq; p->Hkv = s->Hkv; p->d = s->d;
  p->N = N; p->G = G;
  p->seq_groups = s->Hkv;
  p->nw32 = (N + 31) / 32;
  p->nch = stats_chunks(s->b, G, N);
  size_t o = 0;
  const size_t Hq = s->Hq, Hkv = s->Hkv, B = s->b;
  p->off_lohi = o;   o = align_up(o + sizeof(float2) * Hq * (size_t)N * B);
  p->off_ml = o;     o = align_up(o + sizeof(float2) * Hq * B * p->nch);
  p->off_rowml = o;  o = align_up(o + sizeof(float2) * Hq * B);
  p->off_qlast = o;  o = align_up(o + sizeof(float) * Hq * 128);
  p->off_lo = o;     o = align_up(o + sizeof(float) * Hq * N);
  p->off_hi = o;     o = align_up(o + sizeof(float) * Hq * N);
  p->off_kbar = o;   o = align_up(o + sizeof(float) * Hkv * N * 128);
  p->off_sel = o;    o = align_up(o + sizeof(uint32_t) * Hq * 2 * p->nw32);
  p->off_rowbits = o; o = align_up(o + sizeof(uint32_t) * Hq * (size_t)N * p->nw32);
  // pooled queries go through the workspace only in the two-launch query-aware path (N > 2048)
  p->off_qbar = o;   o = align_up(o + (N > 2048 ? sizeof(float) * Hq * (size_t)N * 128 : 0));
  p->off_pe = o;     o = align_up(o + sizeof(float) * Hq * (size_t)N);
  p->off_jwork = o;  o = align_up(o + sizeof(int32_t) * Hkv * N);
  p->off_bar = o;    o = align_up(o + 256);
  p->off_jkeys = o;  o = align_up(o + sizeof(unsigned long long) * Hkv * N);
  p->off_utab = o;   o = align_up(o + sizeof(int4) * Hkv * N * (B / 32));
  p->total = o;
  p->off_vw = o;     o = align_up(o + sizeof(uint16_t) * Hkv * (size_t)s->S * 128);
  p->total_i8 = o;
  return FP_OK;
}

Work carve(const Plan &p, void *ws) {
  char *b = (char *)ws;
  Work w;
  w.lohi = (float2 *)(b + p.off_lohi);
  w.ml = (float2 *)(b + p.off_ml);
  w.rowml = (float2 *)(b + p.off_rowml);
  w.qlast = (float *)(b + p.off_qlast);
  w.lo = (float *)(b + p.off_lo);
  w.hi = (float *)(b + p.off_hi);
  w.kbar = (float *)(b + p.off_kbar);
  w.sel = (uint32_t *)(b + p.off_sel);
  w.rowbits = (uint32_t *)(b + p.off_rowbits);
  w.qbar = (float *)(b + p.off_qbar);
  w.pe = (float *)(b + p.off_pe);
  w.jwork = (int32_t *)(b + p.off_jwork);
  w.bar = (unsigned int *)(b + p.off_bar);
  w.jkeys = (unsigned long long *)(b + p.off_jkeys);
  w.utab = (int4 *)(b + p.off_utab);
  return w;
}

}  // namespace fp

using namespace fp;

static int check_params(float gamma, float tau) {
  if (!(gamma > 0.0f) || !(gamma <= 1.0f)) return FP_EINVAL;  // also rejects NaN
  if (!(tau >= 0.0f)) return FP_EINVAL;
  return FP_OK;
}

static int check_out(const Plan &p, const fp_index_out *o, bool need_pattern) {
  if (!o || !o->row_ptr || !o->col_idx || !o->job_ptr || !o->job_blk || !o->job_mask ||
      !o->job_order || !o->status)
    return FP_EINVAL;
  if (need_pattern && (!o->pattern || !o->jsd)) return FP_EINVAL;
  if (o->col_cap < (int64_t)p.Hq * p.N || o->job_cap < (int64_t)p.Hkv * p.N) return FP_EINVAL;
  if (o->col_cap > INT32_MAX || o->job_cap > INT32_MAX) return FP_EINVAL;
  return FP_OK;
}

#define FP_LAUNCH(call)                          \
  do {                                           \
    if ((call) != hipSuccess) return FP_EHIP;    \
  } while (0)

extern "C" {

int fp_version(void) { return 100; }

const char *fp_strerror(int code) {
  switch (code) {
    case FP_OK: return "ok";
    case FP_EINVAL: return "invalid argument (null pointer, S % b != 0, Hq % Hkv != 0, gamma not in (0,1], tau < 0 or NaN, or a capacity below one entry per row)";
    case FP_EUNSUPPORTED: return "unsupported shape (needs d = 128, b in {64, 128, 256}, S/b <= 8192, Hq/Hkv <= 16, (Hq/Hkv)*b <= 2048)";
    case FP_EWORKSPACE: return "workspace smaller than fp_workspace_bytes()";
    case FP_ECAPACITY: return "CSR capacity exceeded (device status)";
    case FP_EHIP: return "HIP launch or query failed";
    case FP_EJOBCAPACITY: return "job-list capacity exceeded (device status)";
    case FP_ETIMEOUT: return "a bounded device-side wait gave up (device status)";
    case FP_ESCRATCH: return "shape needs more scratch than fp_index_static's buffer (FP_STATIC_SCRATCH_BYTES)";
    default: return "unknown fpattn error code";
  }
}

int fp_workspace_bytes(const fp_shape *shape, int variant, size_t *bytes) {
  if (!bytes || (variant != 0 && variant != 1)) return FP_EINVAL;
  Plan p;
  int rc = make_plan(shape, &p);
  if (rc) return rc;
  *bytes = variant == 1 ? p.total_i8 : p.total;
  return FP_OK;
}

int64_t fp_csr_capacity(const fp_shape *shape) {
  Plan p;
  int rc = make_plan(shape, &p);
  if (rc) return rc;
  return (int64_t)p.Hq * p.N * (p.N + 1) / 2;
}

int64_t fp_job_capacity(const fp_shape *shape) {
  Plan p;
  int rc = make_plan(shape, &p);
  if (rc) return rc;
  return (int64_t)p.Hkv * p.N * (p.N + 1) / 2;
}

// The index launches for a validated plan and workspace.
static int index_launch(const Plan &p, bool i8, const void *Q, const float *sQ, const void *K, const float *sK,
                        float gamma, float tau, const fp_index_out *out, void *ws, hipStream_t st, bool share,
                        const float *qbar_in) {
  Work w = carve(p, ws);
  FP_LAUNCH(launch_ig_stats(p, i8, Q, sQ, K, sK, w, st, out->status));   // also clears the status word
  FP_LAUNCH(launch_ig_finalize(p, i8, Q, sQ, gamma, tau, out, w, st, true));
  FP_LAUNCH(launch_ig_qa(p, i8, Q, sQ, gamma, out->pattern, w, st, qbar_in));
  FP_LAUNCH(launch_rows_and_jobs(p, out, w, st, share));
  return FP_OK;
}

static int index_common(const fp_shape *shape, bool i8, const void *Q, const float *sQ,
                        const void *K, const float *sK, float gamma, float tau,
                        fp_index_out *out, void *ws, size_t ws_bytes, void *stream,
                        bool share = false, const float *qbar_in = nullptr) {
  Plan p;
  int rc = make_plan(shape, &p);
  if (rc) return rc;
  if (!Q || !K || (i8 && (!sQ || !sK))) return FP_EINVAL;
  if ((rc = check_params(gamma, tau))) return rc;
  if ((rc = check_out(p, out, true))) return rc;
  if (!ws || ws_bytes < p.total) return ws ? FP_EWORKSPACE : FP_EINVAL;
  return index_launch(p, i8, Q, sQ, K, sK, gamma, tau, out, ws, (hipStream_t)stream, share, qbar_in);
}

int fp_index(const fp_shape *shape, const void *Q, const void *K, float gamma, float tau,
             fp_index_out *out, void *ws, size_t ws_bytes, void *stream) {
  return index_common(shape, false, Q, nullptr, K, nullptr, gamma, tau, out, ws, ws_bytes,
                      stream);
}

int fp_index_i8(const fp_shape *shape, const int8_t *Q8, const float *sQ, const int8_t *K8,
                const float *sK, float gamma, float tau, fp_index_out *out, void *ws,
                size_t ws_bytes, void *stream) {
  return index_common(shape, true, Q8, sQ, K8, sK, gamma, tau, out, ws, ws_bytes, stream);
}

// Device address of this GPU's scratch buffer, looked up once per device with that device
// current; NULL if the lookup fails.
static void *static_scratch() {
  static std::mutex mu;
  static void *ptr[64] = {nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    ptr[dev] = p;
  }
  return ptr[dev];
}

int fp_index_static(const fp_shape *shape, const void *Q, const void *K, float gamma, float tau,
                    fp_index_out *out, void *stream) {
  Plan p;
  int rc = make_plan(shape, &p);
  if (rc) return rc;
  if (!Q || !K || !out) return FP_EINVAL;
  if ((rc = check_params(gamma, tau))) return rc;
  if ((rc = check_out(p, out, true))) return rc;
  if (p.total > (size_t)FP_STATIC_SCRATCH_BYTES) return FP_ESCRATCH;
  void *ws = static_scratch();
  if (!ws) return FP_EHIP;
  return index_common(shape, false, Q, nullptr, K, nullptr, gamma, tau, out, ws, FP_STATIC_SCRATCH_BYTES,
                      stream);
}

int fp_index_pooled(const fp_shape *shape, const void *Q, const void *K, const float *qbar, float gamma,
                    float tau, fp_index_out *out, void *ws, size_t ws_bytes, void *stream) {
  if (!qbar) return FP_EINVAL;
  return index_common(shape, false, Q, nullptr, K, nullptr, gamma, tau, out, ws, ws_bytes, stream, false, qbar);
}

int fp_qkv_project(const fp_shape *shape, int D, const void *X, const void *W, const float *rope_cos,
                   const float *rope_sin, void *Q, void *K, void *V, float *qbar, float *kbar, int8_t *Q8,
                   float *sQ, int8_t *K8, float *sK, int8_t *V8, float *sV, void *stream) {
  if (!shape) return FP_EINVAL;
  const fp_shape &s = *shape;
  if (s.S <= 0 || s.Hq <= 0 || s.Hkv <= 0 || s.Hq % s.Hkv != 0 || D <= 0 || s.b <= 0) return FP_EINVAL;
  if (!X || !W || !Q || !K || !V || (!rope_cos) != (!rope_sin)) return FP_EINVAL;
  const bool any8 = Q8 || sQ || K8 || sK || V8 || sV, all8 = Q8 && sQ && K8 && sK && V8 && sV;
  if (any8 && !all8) return FP_EINVAL;
  if (s.d != 128 || s.S % 128 != 0 || D % 64 != 0) return FP_EUNSUPPORTED;
  if ((qbar || kbar) && s.b != 64 && s.b != 128) return FP_EUNSUPPORTED;
  if ((long)s.S * D >= (1L << 31) || (long)(s.Hq + 2 * s.Hkv) * 128 * D >= (1L << 31)) return FP_EUNSUPPORTED;
  FP_LAUNCH(launch_qkv_proj(s.S, D, s.Hq, s.Hkv, s.b, X, W, rope_cos, rope_sin, Q, K, V, qbar, kbar, Q8, sQ, K8, sK,
                            V8, sV, (hipStream_t)stream));
  return FP_OK;
}

int fp_index_shared(const fp_shape *shape, int variant, const void *Q, const float *sQ,
                    const void *K, const float *sK, float gamma, float tau, fp_index_out *out,
                    void *ws, size_t ws_bytes, void *stream) {
  if (variant != 0 && variant != 1) return FP_EINVAL;
  return index_common(shape, variant == 1, Q, sQ, K, sK, gamma, tau, out, ws, ws_bytes, stream, true);
}

int fp_block_uses(const fp_shape *shape, const fp_index_out *jobs, int32_t *uses, int32_t *head_uses,
                  void *stream) {
  Plan p;
  int rc = make_plan(shape, &p);
  if (rc) return rc;
  if (!jobs || !jobs->job_ptr || !jobs->job_blk || !jobs->job_mask || !uses) return FP_EINVAL;
  FP_LAUNCH(launch_block_uses(p, jobs, uses, head_uses, (hipStream_t)stream));
  return FP_OK;
}

int fp_build_jobs(const fp_shape *shape, fp_index_out *io, void *ws, size_t ws_bytes,
                  void *stream) {
  Plan p;
  int rc = make_plan(shape, &p);
  if (rc) return rc;
  if ((rc = check_out(p, io, false))) return rc;
  if (!ws || ws_bytes < p.total) return ws ? FP_EWORKSPACE : FP_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  Work w = carve(p, ws);
  FP_LAUNCH(launch_status_init(io->status, nullptr, st));
  FP_LAUNCH(launch_jobs(p, io, w, st));
  return FP_OK;
}

// The attention launches for a validated plan and workspace.
static int attn_launch(const Plan &p, bool i8, const void *Q, const float *sQ, const void *K, const float *sK,
                       const void *V, const float *sV, const fp_index_out *csr, void *O, void *ws, hipStream_t st) {
  const Work w = carve(p, ws);
  FP_LAUNCH(launch_attn(p, i8, Q, sQ, K, sK, V, sV, csr, O, w.bar + 32, w.utab, st, 0, 1, nullptr,
                        i8 ? (uint16_t *)((char *)ws + p.off_vw) : nullptr));
  return FP_OK;
}

static int attn_common(const fp_shape *shape, bool i8, const void *Q, const float *sQ,
                       const void *K, const float *sK, const void *V, const float *sV,
                       const fp_index_out *csr, void *O, void *ws, size_t ws_bytes,
                       void *stream) {
  Plan p;
  int rc = make_plan(shape, &p);
  if (rc) return rc;
  if (!Q || !K || !V || !O || (i8 && (!sQ || !sK || !sV))) return FP_EINVAL;
  if (!csr || !csr->row_ptr || !csr->col_idx || !csr->job_ptr || !csr->job_blk ||
      !csr->job_mask || !csr->job_order)
    return FP_EINVAL;
  const size_t need = i8 ? p.total_i8 : p.total;
  if (!ws || ws_bytes < need) return ws ? FP_EWORKSPACE : FP_EINVAL;
  return attn_launch(p, i8, Q, sQ, K, sK, V, sV, csr, O, ws, (hipStream_t)stream);
}

int fp_attn(const fp_shape *shape, const void *Q, const void *K, const void *V,
            const fp_index_out *csr, void *O, void *ws, size_t ws_bytes, void *stream) {
  return attn_common(shape, false, Q, nullptr, K, nullptr, V, nullptr, csr, O, ws, ws_bytes,
                     stream);
}

// fp_attn_split workspace: fp_attn's, then the split unit table and the partial slots.
static int split_layout(const Plan &p, int nsplit, int nseg, size_t *utab_off, size_t *part_off, size_t *total) {
  if (nsplit < 0 || nseg < 2 || nseg > 64) return FP_EINVAL;
  if (p.B < 128) return FP_EUNSUPPORTED;
  const long jobs = (long)p.Hkv * p.N, ns = nsplit < jobs ? nsplit : jobs;
  const size_t units = (size_t)(jobs + ns * (nseg - 1)) * (p.B / 32);
  *utab_off = align_up(p.total);
  *part_off = align_up(*utab_off + sizeof(int4) * units);
  *total = align_up(*part_off + sizeof(float) * (size_t)ns * nseg * attn_split_slot_floats(p));
  return FP_OK;
}

int fp_attn_split_workspace_bytes(const fp_shape *shape, int nsplit, int nseg, size_t *bytes) {
  Plan p;
  int rc = make_plan(shape, &p);
  if (rc) return rc;
  if (!bytes) return FP_EINVAL;
  size_t uo, po;
  return split_layout(p, nsplit, nseg, &uo, &po, bytes);
}

int fp_attn_split(const fp_shape *shape, const void *Q, const void *K, const void *V,
                  const fp_index_out *csr, int nsplit, int nseg, void *O, void *ws, size_t ws_bytes,
                  void *stream) {
  Plan p;
  int rc = make_plan(shape, &p);
  if (rc) return rc;
  if (!Q || !K || !V || !O || !csr || !csr->row_ptr || !csr->col_idx || !csr->job_ptr || !csr->job_blk ||
      !csr->job_mask || !csr->job_order)
    return FP_EINVAL;
  size_t uo, po, total;
  if ((rc = split_layout(p, nsplit, nseg, &uo, &po, &total))) return rc;
  if (!ws || ws_bytes < total) return ws ? FP_EWORKSPACE : FP_EINVAL;
  const Work w = carve(p, ws);
  char *b = (char *)ws;
  FP_LAUNCH(launch_attn(p, false, Q, nullptr, K, nullptr, V, nullptr, csr, O, w.bar + 32, (int4 *)(b + uo),
                        (hipStream_t)stream, nsplit, nseg, (float *)(b + po)));
  return FP_OK;
}

int fp_attn_i8(const fp_shape *shape, const int8_t *Q8, const float *sQ, const int8_t *K8,
               const float *sK, const int8_t *V8, const float *sV, const fp_index_out *csr,
               void *O, void *ws, size_t ws_bytes, void *stream) {
  return attn_common(shape, true, Q8, sQ, K8, sK, V8, sV, csr, O, ws, ws_bytes, stream);
}

// Ragged batches: every sequence is checked before anything is enqueued; the
// workspace must cover the longest sequence's plan (its int8 attention form for
// fp_attn_i8_batch) and is reused in order.
static int batch_check(const fp_shape *shape, int nseq, const int32_t *seqlens, size_t ws_bytes,
                       const fp_index_out *outs, bool need_pattern, bool i8_attn = false) {
  if (!shape || nseq < 1 || !seqlens || !outs) return FP_EINVAL;
  size_t need = 0;
  for (int s = 0; s < nseq; ++s) {
    fp_shape one = *shape;
    one.S = seqlens[s];
    Plan p;
    int rc = make_plan(&one, &p);
    if (rc) return rc;
    const fp_index_out *o = outs + s;
    if (need_pattern) {
      if ((rc = check_out(p, o, true))) return rc;
    } else if (!o->row_ptr || !o->col_idx || !o->job_ptr || !o->job_blk || !o->job_mask || !o->job_order) {
      return FP_EINVAL;
    }
    const size_t t = i8_attn ? p.total_i8 : p.total;
    need = t > need ? t : need;
  }
  return ws_bytes < need ? FP_EWORKSPACE : FP_OK;
}

// Runs of equal-length sequences (up to kFoldRun of them, each of at most kFoldMaxN key blocks) run
// as one call with their heads side by side, when the workspace holds that call's layout: a batch
// of short sequences is otherwise a chain of small launches per sequence.  Longer sequences gain
// nothing from it and would need folded capacities of Hq * N^2 / 2 entries each.
constexpr int kFoldMaxN = 256;

// The plan of k sequences of length S side by side (job order and chunk rotation per sequence).
// FP_EUNSUPPORTED when the folded call's worst-case column or job count would not fit the 32-bit
// offsets of its outputs (such runs go one sequence at a time).
static int fold_plan(const fp_shape *shape, int S, int k, Plan *p) {
  fp_shape f = *shape;
  f.S = S;
  f.Hq = shape->Hq * k;
  f.Hkv = shape->Hkv * k;
  const int rc = make_plan(&f, p);
  if (rc) return rc;
  const int64_t worst = (int64_t)p->Hq * p->N * (p->N + 1) / 2;   // columns (jobs: Hkv <= Hq)
  if (worst > INT32_MAX) return FP_EUNSUPPORTED;
  p->seq_groups = shape->Hkv;
  return FP_OK;
}

// Workspace of a folded index call: its own workspace, then the folded outputs with room for every
// sequence's worst case (so the folded call itself never overflows).
struct FoldIndexLayout {
  size_t row_ptr, col_idx, job_ptr, job_blk, job_mask, job_order, pattern, jsd, stats, status, total;
};
static FoldIndexLayout fold_index_layout(const Plan &pf, int k, bool stats) {
  const size_t N = pf.N, nr = (size_t)pf.Hq * N, nj = (size_t)pf.Hkv * N;
  const size_t ccap = nr * (N + 1) / 2, jcap = nj * (N + 1) / 2;   // k sequences' worst cases
  FoldIndexLayout L;
  size_t o = pf.total;
  L.row_ptr = o;   o = align_up(o + sizeof(int32_t) * (nr + 1));
  L.col_idx = o;   o = align_up(o + sizeof(int32_t) * ccap);
  L.job_ptr = o;   o = align_up(o + sizeof(int32_t) * (nj + 1));
  L.job_blk = o;   o = align_up(o + sizeof(int32_t) * jcap);
  L.job_mask = o;  o = align_up(o + sizeof(uint32_t) * jcap);
  L.job_order = o; o = align_up(o + sizeof(int32_t) * nj);
  L.pattern = o;   o = align_up(o + pf.Hq);
  L.jsd = o;       o = align_up(o + sizeof(float) * pf.Hq);
  L.stats = o;     o = align_up(o + (stats ? sizeof(float) * 3 * nr : 0));
  L.status = o;    o = align_up(o + sizeof(int32_t));
  L.total = o;
  (void)k;
  return L;
}

// Workspace of a folded attention call: its own workspace (with the int8 V widening for W8A8), then
// the merged job list.
struct FoldAttnLayout {
  size_t job_ptr, job_blk, job_mask, job_order, total;
};
static FoldAttnLayout fold_attn_layout(const Plan &pf, bool i8) {
  const size_t N = pf.N, nj = (size_t)pf.Hkv * N, jcap = nj * (N + 1) / 2;
  FoldAttnLayout L;
  size_t o = i8 ? pf.total_i8 : pf.total;
  L.job_ptr = o;   o = align_up(o + sizeof(int32_t) * (nj + 1));
  L.job_blk = o;   o = align_up(o + sizeof(int32_t) * jcap);
  L.job_mask = o;  o = align_up(o + sizeof(uint32_t) * jcap);
  L.job_order = o; o = align_up(o + sizeof(int32_t) * nj);
  L.total = o;
  return L;
}

// The run of equal-length sequences that starts at s: its length (1 if it is not folded).
static int fold_run(const fp_shape *shape, int nseq, const int32_t *seqlens, int s) {
  if (seqlens[s] / shape->b > kFoldMaxN) return 1;
  int e = s + 1;
  while (e < nseq && e - s < kFoldRun && seqlens[e] == seqlens[s]) ++e;
  return e - s;
}

// Sequence s's tensors follow sequence s - 1's: element bytes 2 (bf16) or 1 (int8), and the
// int8 forms' per-token scales likewise, one fp32 per head and token.
static int index_batch_common(const fp_shape *shape, bool i8, int nseq, const int32_t *seqlens,
                              const void *Q, const float *sQ, const void *K, const float *sK, float gamma,
                              float tau, fp_index_out *outs, void *ws, size_t ws_bytes, void *stream) {
  if (!Q || !K || !ws || (i8 && (!sQ || !sK))) return FP_EINVAL;
  int rc = check_params(gamma, tau);
  if (rc || (rc = batch_check(shape, nseq, seqlens, ws_bytes, outs, true))) return rc;
  const size_t eb = i8 ? 1 : 2;
  hipStream_t st = (hipStream_t)stream;
  const uint8_t *q = (const uint8_t *)Q, *k = (const uint8_t *)K;
  for (int s = 0; s < nseq;) {
    fp_shape one = *shape;
    one.S = seqlens[s];
    int run = fold_run(shape, nseq, seqlens, s);
    Plan pf;
    FoldIndexLayout L{};
    bool stats = false;
    for (int t = s; t < s + run; ++t) stats = stats || outs[t].stats != nullptr;
    if (run >= 2 && (rc = fold_plan(shape, one.S, run, &pf)) == FP_OK) L = fold_index_layout(pf, run, stats);
    if (run >= 2 && rc == FP_OK && ws_bytes >= L.total) {
      char *b = (char *)ws;
      FoldArgs fa{};
      fa.k = run; fa.Hq = shape->Hq; fa.Hkv = shape->Hkv; fa.N = pf.N;
      fp_index_out &f = fa.f;
      f.row_ptr = (int32_t *)(b + L.row_ptr);
      f.col_idx = (int32_t *)(b + L.col_idx);
      f.col_cap = (int64_t)pf.Hq * pf.N * (pf.N + 1) / 2;
      f.job_ptr = (int32_t *)(b + L.job_ptr);
      f.job_blk = (int32_t *)(b + L.job_blk);
      f.job_mask = (uint32_t *)(b + L.job_mask);
      f.job_cap = (int64_t)pf.Hkv * pf.N * (pf.N + 1) / 2;
      f.job_order = (int32_t *)(b + L.job_order);
      f.pattern = (uint8_t *)(b + L.pattern);
      f.jsd = (float *)(b + L.jsd);
      f.stats = stats ? (float *)(b + L.stats) : nullptr;
      f.status = (int32_t *)(b + L.status);
      if ((rc = index_launch(pf, i8, q, sQ, k, sK, gamma, tau, &f, ws, st, false, nullptr))) return rc;
      for (fa.t0 = 0; fa.t0 < run; fa.t0 += kFoldArgs) {
        fa.n = std::min(kFoldArgs, run - fa.t0);
        for (int t = 0; t < fa.n; ++t) fa.seq[t] = outs[s + fa.t0 + t];
        FP_LAUNCH(launch_split_index(fa, st));
      }
    } else {
      run = 1;
      if ((rc = index_common(&one, i8, q, sQ, k, sK, gamma, tau, outs + s, ws, ws_bytes, stream))) return rc;
    }
    q += (size_t)run * one.Hq * one.S * one.d * eb;
    k += (size_t)run * one.Hkv * one.S * one.d * eb;
    if (i8) {
      sQ += (size_t)run * one.Hq * one.S;
      sK += (size_t)run * one.Hkv * one.S;
    }
    s += run;
  }
  return FP_OK;
}

static int attn_batch_common(const fp_shape *shape, bool i8, int nseq, const int32_t *seqlens, const void *Q,
                             const float *sQ, const void *K, const float *sK, const void *V, const float *sV,
                             const fp_index_out *csrs, void *O, void *ws, size_t ws_bytes, void *stream) {
  if (!Q || !K || !V || !O || !ws || (i8 && (!sQ || !sK || !sV))) return FP_EINVAL;
  int rc = batch_check(shape, nseq, seqlens, ws_bytes, csrs, false, i8);
  if (rc) return rc;
  const size_t eb = i8 ? 1 : 2;
  hipStream_t st = (hipStream_t)stream;
  const uint8_t *q = (const uint8_t *)Q, *k = (const uint8_t *)K, *v = (const uint8_t *)V;
  uint8_t *o = (uint8_t *)O;
  for (int s = 0; s < nseq;) {
    fp_shape one = *shape;
    one.S = seqlens[s];
    int run = fold_run(shape, nseq, seqlens, s);
    Plan pf;
    FoldAttnLayout L{};
    if (run >= 2 && (rc = fold_plan(shape, one.S, run, &pf)) == FP_OK) L = fold_attn_layout(pf, i8);
    if (run >= 2 && rc == FP_OK && ws_bytes >= L.total) {
      char *b = (char *)ws;
      FoldArgs fa{};
      fa.k = run; fa.Hq = shape->Hq; fa.Hkv = shape->Hkv; fa.N = pf.N;
      fa.f.job_ptr = (int32_t *)(b + L.job_ptr);
      fa.f.job_blk = (int32_t *)(b + L.job_blk);
      fa.f.job_mask = (uint32_t *)(b + L.job_mask);
      fa.f.job_order = (int32_t *)(b + L.job_order);
      for (fa.t0 = 0; fa.t0 < run; fa.t0 += kFoldArgs) {   // in order: each group continues the last
        fa.n = std::min(kFoldArgs, run - fa.t0);
        for (int t = 0; t < fa.n; ++t) fa.seq[t] = csrs[s + fa.t0 + t];
        FP_LAUNCH(launch_merge_jobs(fa, st));
      }
      if ((rc = attn_launch(pf, i8, q, sQ, k, sK, v, sV, &fa.f, o, ws, st))) return rc;
    } else {
      run = 1;
      if ((rc = attn_common(&one, i8, q, sQ, k, sK, v, sV, csrs + s, o, ws, ws_bytes, stream))) return rc;
    }
    const size_t qn = (size_t)run * one.Hq * one.S, kn = (size_t)run * one.Hkv * one.S;
    q += qn * one.d * eb;
    o += qn * one.d * 2;                          // bf16 output
    k += kn * one.d * eb;
    v += kn * one.d * eb;
    if (i8) {
      sQ += qn;
      sK += kn;
      sV += kn;
    }
    s += run;
  }
  return FP_OK;
}

int fp_batch_workspace_bytes(const fp_shape *shape, int nseq, const int32_t *seqlens, int variant, size_t *bytes) {
  if (!shape || !bytes || nseq < 1 || !seqlens || (variant != 0 && variant != 1)) return FP_EINVAL;
  size_t need = 0;
  for (int s = 0; s < nseq;) {
    fp_shape one = *shape;
    one.S = seqlens[s];
    Plan p;
    int rc = make_plan(&one, &p);
    if (rc) return rc;
    size_t t = variant == 1 ? p.total_i8 : p.total;
    const int run = fold_run(shape, nseq, seqlens, s);
    Plan pf;
    if (run >= 2 && fold_plan(shape, one.S, run, &pf) == FP_OK) {   // (else the run goes one at a time)
      const size_t fi = fold_index_layout(pf, run, true).total, fa = fold_attn_layout(pf, variant == 1).total;
      t = std::max(t, std::max(fi, fa));
    }
    need = std::max(need, t);
    s += run;
  }
  *bytes = need;
  return FP_OK;
}

int fp_index_batch(const fp_shape *shape, int nseq, const int32_t *seqlens, const void *Q, const void *K,
                   float gamma, float tau, fp_index_out *outs, void *ws, size_t ws_bytes, void *stream) {
  return index_batch_common(shape, false, nseq, seqlens, Q, nullptr, K, nullptr, gamma, tau, outs, ws,
                            ws_bytes, stream);
}

int fp_attn_batch(const fp_shape *shape, int nseq, const int32_t *seqlens, const void *Q, const void *K,
                  const void *V, const fp_index_out *csrs, void *O, void *ws, size_t ws_bytes, void *stream) {
  return attn_batch_common(shape, false, nseq, seqlens, Q, nullptr, K, nullptr, V, nullptr, csrs, O, ws,
                           ws_bytes, stream);
}

int fp_index_i8_batch(const fp_shape *shape, int nseq, const int32_t *seqlens, const int8_t *Q8,
                      const float *sQ, const int8_t *K8, const float *sK, float gamma, float tau,
                      fp_index_out *outs, void *ws, size_t ws_bytes, void *stream) {
  return index_batch_common(shape, true, nseq, seqlens, Q8, sQ, K8, sK, gamma, tau, outs, ws, ws_bytes,
                            stream);
}

int fp_attn_i8_batch(const fp_shape *shape, int nseq, const int32_t *seqlens, const int8_t *Q8,
                     const float *sQ, const int8_t *K8, const float *sK, const int8_t *V8, const float *sV,
                     const fp_index_out *csrs, void *O, void *ws, size_t ws_bytes, void *stream) {
  return attn_batch_common(shape, true, nseq, seqlens, Q8, sQ, K8, sK, V8, sV, csrs, O, ws, ws_bytes,
                           stream);
}

int fp_probe_qk_i8(const fp_shape *shape, const int8_t *Q8, const int8_t *K8, int h, int i,
                   int j, int path, int32_t *out, void *stream) {
  Plan p;
  int rc = make_plan(shape, &p);
  if (rc) return rc;
  if (!Q8 || !K8 || !out) return FP_EINVAL;
  if (h < 0 || h >= p.Hq || i < 0 || i >= p.N || j < 0 || j >= p.N) return FP_EINVAL;
  if (path != FP_PROBE_ATTN && path != FP_PROBE_STATS) return FP_EINVAL;
  if (path == FP_PROBE_ATTN) FP_LAUNCH(launch_probe_attn_i8(p, Q8, K8, h, i, j, out, (hipStream_t)stream));
  else FP_LAUNCH(launch_probe_stats_i8(p, Q8, K8, h, i, j, out, (hipStream_t)stream));
  return FP_OK;
}

}  // extern "C"
