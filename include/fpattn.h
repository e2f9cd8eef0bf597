/*
 * fpattn.h -- C ABI of the dynamic block-sparse prefill attention library
 * (libfpattn.so, HIP kernels for AMD gfx950 / MI355X).
 *
 * The method is the one the FAST-Prefill write-ups describe for Flex-Prefill:
 *   [E] "FPGA24成果：FAST-Prefill稀疏注意力加速器，长上下文LLM推理提速2.5倍"
 *       (yunpan.plus explainer), sections 1.1, 1.2, 2.1, 3.1-3.3, 4.2;
 *   [R] "FPGA加速动态稀疏注意力技术解析与优化" (maplevalley.com.cn re-telling),
 *       sections 1.1, 2.2, 3.2, 3.3.
 * Two stages, each one call:
 *   fp_index  -- sparse-index generation ([E] 3.1): the last query block is
 *                scored against every key block in increasing block order;
 *                per head, vertical (column) and slash (diagonal) block mass
 *                and a pooled-query x pooled-key estimate are accumulated; a
 *                Jensen-Shannon divergence against tau picks the
 *                query-aware or the vertical-slash pattern ([E] 1.2, [R] 1.1);
 *                blocks are taken in descending score until the cumulative
 *                mass reaches gamma ([E] 3.1), block 0 and the diagonal block
 *                are always kept, and the result is a CSR of key blocks per
 *                (head, query block) plus a grouped-query job list ([E] 3.2).
 *   fp_attn   -- block-sparse causal attention over that CSR ([E] 1.1, 1.2
 *                figure 3): each query block attends only to its listed key
 *                blocks, with the causal mask inside the diagonal block.
 * The *_i8 variants are the W8A8 form ([E] 3.3 and 4.2, [R] 3.3): Q and K
 * (and V) arrive as int8 with one fp32 scale per (head, token); Q.K^T is an
 * int8 product with int32 accumulation, P.V runs in bf16.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Pointers named as device pointers must point to device memory of the
 *    current HIP device; "host" marks host memory.  Layouts are dense
 *    row-major.  Q is [Hq, S, d], K and V are [Hkv, S, d] (head-major, one
 *    sequence); query head h reads KV head h / (Hq / Hkv).
 *  - The caller owns every buffer.  The library allocates nothing on the
 *    device and keeps no state between calls apart from a cached
 *    device-property query.  Scratch memory comes in through `ws`, of at
 *    least fp_workspace_bytes() bytes; concurrent calls need separate
 *    workspaces.
 *  - Every call validates its arguments on the host, then only enqueues work
 *    on `stream` (a hipStream_t; NULL = the default stream) and returns
 *    without synchronising.  Outputs are valid once that stream has reached
 *    the point of the call; inputs must stay alive until then.
 *  - Return value: FP_OK (0) or a negative FP_E* code.  When a code is
 *    returned nothing was enqueued.  Data-dependent failures (CSR or job
 *    capacity exceeded) cannot be known on the host: the kernels set bits in
 *    the device status word (fp_index_out.status) and stop writing past the
 *    capacity; read it after the stream synchronises.
 *  - Identical inputs give bit-identical outputs (no floating-point atomics),
 *    on any device: the statistics of fp_index cut the key blocks into
 *    chunks whose boundaries depend on the shape only, whatever number of
 *    workgroups runs them.
 *  - Supported shapes: d = 128; b in {64, 128, 256}; S a positive multiple
 *    of b with S / b <= 8192; Hq a multiple of Hkv; G <= 16 and G * b <= 2048
 *    where G = Hq / Hkv; gamma in (0, 1]; tau >= 0.
 */
#ifndef FPATTN_H
#define FPATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP_OK            0
#define FP_EINVAL       (-1) /* null pointer, S % b != 0, Hq % Hkv != 0, gamma not in (0,1], tau < 0 or NaN */
#define FP_EUNSUPPORTED (-2) /* d != 128, b not in {64,128,256}, N > 8192, G > 16, G*b > 2048 */
#define FP_EWORKSPACE   (-3) /* workspace smaller than fp_workspace_bytes() */
#define FP_ECAPACITY    (-4) /* (device status bit 1) CSR capacity exceeded */
#define FP_EHIP         (-5) /* a HIP launch or query failed */
#define FP_EJOBCAPACITY (-6) /* (device status bit 2) job-list capacity exceeded */
#define FP_ETIMEOUT     (-7) /* (device status bit 3, no longer set) a bounded device-side wait gave up */
#define FP_ESCRATCH     (-8) /* fp_index_static: shape needs more than FP_STATIC_SCRATCH_BYTES */

/* Device status word bits (fp_index_out.status[0]); 0 = success. */
#define FP_STATUS_CSR_OVERFLOW 1u
#define FP_STATUS_JOB_OVERFLOW 2u
#define FP_STATUS_WAIT_TIMEOUT 4u   /* reserved: no kernel waits on another workgroup */

/* Pattern codes written to fp_index_out.pattern ([E] 1.2, [R] 1.1). */
#define FP_PATTERN_VERTICAL_SLASH 0
#define FP_PATTERN_QUERY_AWARE    1

/* Problem shape (host struct).  N = S / b blocks. */
typedef struct fp_shape {
  int32_t S;    /* tokens in the sequence                 */
  int32_t b;    /* block size in tokens ([E] 1.2: 128/256) */
  int32_t Hq;   /* query heads                            */
  int32_t Hkv;  /* key/value heads                        */
  int32_t d;    /* head dimension (must be 128)           */
} fp_shape;

/*
 * Index output (host struct of device pointers).  Row r = h * N + i is the
 * key-block set J(h, i) of query block i of head h, columns ascending; job
 * (g, i), index g * N + i, is the union over the G query heads of KV group g
 * of J(h, i), each block carrying a bit mask of the heads that use it (bit
 * h - g*G).  job_order lists the job indices by decreasing work
 * sum_h |J(h, i)| (ties: lower index first).
 */
typedef struct fp_index_out {
  int32_t  *row_ptr;    /* device [Hq*N + 1]                                    */
  int32_t  *col_idx;    /* device [col_cap]                                     */
  int64_t   col_cap;    /* host: capacity of col_idx (fp_csr_capacity() is the
                           worst case, gamma = 1)                               */
  int32_t  *job_ptr;    /* device [Hkv*N + 1]                                   */
  int32_t  *job_blk;    /* device [job_cap] key block of each job entry         */
  uint32_t *job_mask;   /* device [job_cap] head mask of each job entry         */
  int64_t   job_cap;    /* host: capacity of job_blk / job_mask
                           (fp_job_capacity() is the worst case)                */
  int32_t  *job_order;  /* device [Hkv*N]                                       */
  uint8_t  *pattern;    /* device [Hq], FP_PATTERN_*  (NULL allowed in
                           fp_build_jobs only)                                  */
  float    *jsd;        /* device [Hq] Jensen-Shannon divergence D_h (natural
                           log, no square root)  (NULL allowed in fp_build_jobs) */
  float    *stats;      /* device [3][Hq][N] or NULL: vertical mass v, slash
                           mass sl and pooled estimate p of every head          */
  int32_t  *status;     /* device [1] status word, FP_STATUS_* bits, written by
                           every call that fills this struct (set to 0 first)   */
} fp_index_out;

/* Library version (major * 10000 + minor * 100 + patch). */
int fp_version(void);

/* Static text for an FP_* code (never NULL). */
const char *fp_strerror(int code);

/*
 * Scratch bytes for this shape: variant 0 covers fp_index, fp_index_i8,
 * fp_build_jobs and fp_attn; variant 1 also fp_attn_i8, which keeps a bf16
 * widening of V8 there (2 * Hkv * S * d bytes more).  One workspace of the
 * size returned for variant 1 serves every call.  Writes *bytes (host).
 */
int fp_workspace_bytes(const fp_shape *shape, int variant, size_t *bytes);

/* Worst-case CSR entries Hq * N * (N + 1) / 2 (every causal block kept);
 * negative FP_E* code on an invalid shape. */
int64_t fp_csr_capacity(const fp_shape *shape);

/* Worst-case job entries Hkv * N * (N + 1) / 2; negative FP_E* on error. */
int64_t fp_job_capacity(const fp_shape *shape);

/*
 * Sparse-index generation, bf16 inputs ([E] 3.1, 1.2; [R] 1.1, 3.2).
 *   Q: device bf16 [Hq, S, d];  K: device bf16 [Hkv, S, d].
 *   gamma: cumulative-mass threshold in (0, 1] (gamma = 1 keeps every causal
 *          block); tau: divergence threshold (>= 0), D_h < tau selects the
 *          query-aware pattern.
 * Definitions (sigma = 1/sqrt(d), t_r = S - b + r for the b rows of the last
 * query block, softmax over keys k <= t_r):
 *   v[j]  = (1/b) sum_r sum_{k in block j} a_r[k]             (vertical mass)
 *   sl[o] = (1/b) sum_r sum_{k <= t_r, (t_r - k) / b = o} a_r[k] (slash mass)
 *   p     = softmax_j(sigma * mean(Q_last) . mean(K_j))       (pooled estimate)
 *   D     = JSD(p, v);  query-aware iff D < tau.
 *   Sel(x, gamma): fewest indices in descending value (ties: lower index
 *   first) whose sum reaches gamma * sum(x).
 *   vertical-slash rows: J(h,i) = {j in Sel(v) : j <= i}
 *                        u {i - o : o in Sel(sl), o <= i} u {0, i};
 *   query-aware rows:    J(h,i) = Sel(softmax_{j<=i}(sigma * mean(Q_i) .
 *                        mean(K_j))) u {0, i}.
 * Fills every field of *out (device writes only); out->stats may be NULL.
 * K is read from HBM once, in increasing block order; nothing of size
 * Hq x S is written to memory.  Errors: FP_EINVAL, FP_EUNSUPPORTED,
 * FP_EWORKSPACE, FP_EHIP; capacity overflow through out->status.
 */
int fp_index(const fp_shape *shape, const void *Q, const void *K,
             float gamma, float tau, fp_index_out *out,
             void *ws, size_t ws_bytes, void *stream);

/*
 * W8A8 sparse-index generation ([E] 3.3, 4.2; [R] 3.3).
 *   Q8: device int8 [Hq, S, d], sQ: device fp32 [Hq, S];
 *   K8: device int8 [Hkv, S, d], sK: device fp32 [Hkv, S].
 * Scores are sigma * sQ[t] * sK[k] * (Q8[t] . K8[k]) with the integer dot
 * product exact (int8 x int8 -> int32); pooled vectors use the dequantised
 * values s * x8.  Otherwise as fp_index.
 */
int fp_index_i8(const fp_shape *shape, const int8_t *Q8, const float *sQ,
                const int8_t *K8, const float *sK, float gamma, float tau,
                fp_index_out *out, void *ws, size_t ws_bytes, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): fp_index
 * with its scratch in a buffer of FP_STATIC_SCRATCH_BYTES that the library
 * holds on each GPU it runs on, from the first call on that GPU until the
 * process ends, instead of a caller workspace.  The call itself allocates
 * nothing and calls no allocating routine.  Arguments, outputs and errors
 * as fp_index, plus FP_ESCRATCH (nothing enqueued) when
 * fp_workspace_bytes(shape, 0) exceeds FP_STATIC_SCRATCH_BYTES (64 MiB covers
 * the 3B-shaped layer at S = 131072 with b = 64 or 128).  The buffer keeps
 * the last call's contents; what must start at zero is cleared by the call's
 * own kernels.  Every call on one GPU uses the same buffer: calls that
 * overlap on one GPU (different streams, or other host threads) race and
 * must be serialised by the caller; calls on one stream are ordered.  The
 * outputs equal fp_index's for the same inputs.
 */
#define FP_STATIC_SCRATCH_BYTES (64u << 20)
int fp_index_static(const fp_shape *shape, const void *Q, const void *K,
                    float gamma, float tau, fp_index_out *out, void *stream);

/*
 * The QKV projection that precedes the path, with the later stages' pooling
 * and quantisation fused into its epilogue ([E] 1.1: Q, K, V are
 * projections of the input; [E] 3.1: one fused streaming pipeline; [E] 3.3,
 * 4.2: W8A8 activations).  Y = X W^T on the bf16 matrix cores with fp32
 * accumulation, then per 128-token x 128-column output tile (one head):
 *   - the rotary embedding on the Q and K heads (rotate-half pairs (c, c+64):
 *     y_c' = y_c cos - y_{c+64} sin, y_{c+64}' = y_{c+64} cos + y_c sin);
 *   - rounding to bf16 (nearest even) and the head-major store;
 *   - qbar / kbar (or NULL): the fp32 mean of each b-token block of the
 *     rounded Q / K values, i.e. the pooled vectors fp_index would otherwise
 *     compute by reading Q and K back (fp_index_pooled takes qbar);
 *   - optionally Q8/sQ, K8/sK, V8/sV: symmetric per-(head, token) int8 codes
 *     of the rounded values, s = max|x| / 127 (1 for a zero row), codes
 *     rint(x / s) clamped to +-127, fp32 arithmetic (the inputs of
 *     fp_index_i8 / fp_attn_i8); all six NULL or all six set.
 *   shape: S, b, Hq, Hkv, d of the layer (d = 128; S a multiple of 128;
 *          b in {64, 128} when qbar or kbar is requested);
 *   D: model dimension, a positive multiple of 64;
 *   X: device bf16 [S, D];  W: device bf16 [(Hq + 2 Hkv) * 128, D], rows in
 *      the order Q heads, K heads, V heads (row h*128 + c is output column c
 *      of head h);
 *   rope_cos, rope_sin: device fp32 [S, 64] (position t, frequency c), or
 *      both NULL for no rotation;
 *   Q: device bf16 [Hq, S, 128]; K, V: device bf16 [Hkv, S, 128];
 *   qbar: device fp32 [Hq, S / b, 128]; kbar: device fp32 [Hkv, S / b, 128];
 *   Q8: device int8 [Hq, S, 128], sQ: fp32 [Hq, S]; K8, V8, sK, sV likewise
 *      over Hkv.
 * Errors: FP_EINVAL (null or inconsistent pointers, non-positive sizes,
 * Hq % Hkv != 0), FP_EUNSUPPORTED (d, S, D or b outside the above, or an
 * operand of 2^31 elements or more), FP_EHIP.
 */
int fp_qkv_project(const fp_shape *shape, int D, const void *X, const void *W,
                   const float *rope_cos, const float *rope_sin, void *Q, void *K, void *V,
                   float *qbar, float *kbar, int8_t *Q8, float *sQ, int8_t *K8, float *sK,
                   int8_t *V8, float *sV, void *stream);

/*
 * fp_index with the pooled query blocks supplied by the caller (for example
 * by fp_qkv_project's epilogue): qbar is device fp32 [Hq, N, 128], the mean
 * of each block of b queries of each head.  The query-aware rows then score
 * qbar against the pooled keys without reading Q; Q is read only for the
 * last query block.  Otherwise as fp_index (bf16); FP_EINVAL if qbar is NULL.
 */
int fp_index_pooled(const fp_shape *shape, const void *Q, const void *K, const float *qbar,
                    float gamma, float tau, fp_index_out *out,
                    void *ws, size_t ws_bytes, void *stream);

/*
 * Head-pattern sharing ([R] 5, item 1: compress the sparse pattern by letting
 * similar heads share one).  As fp_index (variant 0; sQ, sK ignored) or
 * fp_index_i8 (variant 1), except that every query head h of KV group g gets
 * the union of the index sets of the heads of g whose pattern equals h's:
 *   J'(h, i) = U { J(h', i) : h' in g, pattern(h') = pattern(h) }.
 * Heads with the same pattern in a group then have identical rows, and every
 * job-list entry of a group whose heads share one pattern carries all of
 * them.  pattern, jsd and stats are those of fp_index; the rows, the job list
 * and its order follow the shared sets.  Errors as fp_index; FP_EINVAL for
 * another variant.
 */
int fp_index_shared(const fp_shape *shape, int variant, const void *Q, const float *sQ,
                    const void *K, const float *sK, float gamma, float tau,
                    fp_index_out *out, void *ws, size_t ws_bytes, void *stream);

/*
 * Rebuild the grouped-query job list (job_ptr, job_blk, job_mask, job_order)
 * from a CSR already in io->row_ptr / io->col_idx (rows sorted ascending,
 * every column <= its query block).  fp_index calls this itself; it is
 * exported so that a CSR from elsewhere can drive fp_attn ([E] 3.2: the
 * sparse index set is turned into a compact job list).  Writes io->status.
 */
int fp_build_jobs(const fp_shape *shape, fp_index_out *io,
                  void *ws, size_t ws_bytes, void *stream);

/*
 * Use counters of the key blocks ([E] 3.2: the consumer count of each KV
 * block, the input of the liveness-driven cache), from the job list of an
 * fp_index / fp_build_jobs result (job_ptr, job_blk, job_mask; read only):
 *   uses[g * N + j]      = number of jobs (g, i) whose entry list holds j,
 *   head_uses[g * N + j] = number of (head, query block) pairs of group g
 *                          whose index set holds j (NULL: not computed).
 *   uses, head_uses: device int32 [Hkv * N], every element written.
 * Errors: FP_EINVAL, FP_EUNSUPPORTED, FP_EHIP.
 */
int fp_block_uses(const fp_shape *shape, const fp_index_out *jobs, int32_t *uses,
                  int32_t *head_uses, void *stream);

/*
 * Block-sparse causal attention, bf16 ([E] 1.1 and 1.2 figure 3).
 *   Q: device bf16 [Hq, S, d]; K, V: device bf16 [Hkv, S, d];
 *   csr: the fields row_ptr, col_idx, job_ptr, job_blk, job_mask, job_order
 *        of an fp_index / fp_build_jobs result (read only);
 *   O: device bf16 [Hq, S, d], every element written.
 * For query token t of block i of head h: O[h,t] = sum over keys k <= t whose
 * block is in J(h,i) of softmax_k(sigma * Q[h,t] . K[g,k]) * V[g,k]; fp32
 * softmax and accumulation, one rounding to bf16 at the end.  fp_index always
 * keeps block i; a row of a caller's CSR (fp_build_jobs) may leave it out, and
 * an empty row, which has no keys to attend to, gives O = 0 for its block.
 * Errors: FP_EINVAL, FP_EUNSUPPORTED, FP_EWORKSPACE, FP_EHIP.
 */
int fp_attn(const fp_shape *shape, const void *Q, const void *K, const void *V,
            const fp_index_out *csr, void *O,
            void *ws, size_t ws_bytes, void *stream);

/*
 * Split-KV schedule of the same attention ([E] 3.2: the attention unit walks
 * KV blocks and accumulates each query block's partial result under its key
 * until every consumer is served).  The nsplit longest jobs (the first
 * nsplit of job_order; clamped to the job count) are cut into nseg segments
 * of consecutive job-list entries; each segment runs as its own work unit and
 * writes every row's unnormalised partial output with its running maximum
 * and weight sum (m, l) to a slot keyed by (job, segment); a combine step
 * then merges a job's slots, O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s
 * with M = max_s m_s, and writes bf16 O.  The other jobs run as in fp_attn.
 * The result is fp_attn's up to floating-point rounding order.
 *   nsplit >= 0, 2 <= nseg <= 64; bf16 only, b in {128, 256}
 *   (FP_EUNSUPPORTED for b = 64); ws: at least
 *   fp_attn_split_workspace_bytes(shape, nsplit, nseg) bytes.
 * Arguments otherwise as fp_attn.  Errors: FP_EINVAL, FP_EUNSUPPORTED,
 * FP_EWORKSPACE, FP_EHIP.
 */
int fp_attn_split_workspace_bytes(const fp_shape *shape, int nsplit, int nseg, size_t *bytes);
int fp_attn_split(const fp_shape *shape, const void *Q, const void *K, const void *V,
                  const fp_index_out *csr, int nsplit, int nseg, void *O,
                  void *ws, size_t ws_bytes, void *stream);

/*
 * W8A8 block-sparse attention ([E] 3.3, 4.2; [R] 3.3).  Scores use the exact
 * int8 dot product scaled by sigma * sQ * sK; P.V uses bf16 P against V taken
 * as bf16(sV * v8), rounded once per call.
 *   V8: device int8 [Hkv, S, d], sV: device fp32 [Hkv, S]; O: device bf16.
 *   ws: at least fp_workspace_bytes(shape, 1) bytes (the call first widens V8
 *   to bf16 in it).
 */
int fp_attn_i8(const fp_shape *shape, const int8_t *Q8, const float *sQ,
               const int8_t *K8, const float *sK, const int8_t *V8,
               const float *sV, const fp_index_out *csr, void *O,
               void *ws, size_t ws_bytes, void *stream);

/*
 * Ragged batches of independent sequences (bf16), e.g. several prompts of
 * different lengths in one call.  Sequence s has S_s = seqlens[s] tokens (host
 * array, each a multiple of shape->b; shape->S is ignored) and is packed after
 * sequence s - 1 in its own head-major layout: Q holds [Hq, S_s, d] blocks one
 * after another, K (and V, O) [Hkv, S_s, d] (O like Q).  (A batch of equal
 * lengths is also one call of fp_index / fp_attn with B*Hq and B*Hkv heads,
 * since every quantity is per head or per KV group.)
 *   outs / csrs: host array of nseq index outputs, one per sequence, each
 *                sized for its own S_s as in fp_index.
 *   ws: at least fp_workspace_bytes of the longest sequence.  The sequences
 *       run in order on the stream and reuse it.  A run of up to 64
 *       consecutive sequences of one length S with S/b <= 256 runs as one
 *       call with its heads side by side (every quantity is per head or per
 *       KV group) when ws holds that call's layout; fp_batch_workspace_bytes
 *       gives the size that allows it for every run.  The outputs are the same
 *       bit for bit either way: job order and chunk order are taken per
 *       sequence, and each sequence's outputs keep its own capacities.
 *   csrs (attention): each as written by fp_index / fp_build_jobs for its
 *       sequence.
 * Every sequence is checked before anything is enqueued (FP_EINVAL,
 * FP_EUNSUPPORTED, FP_EWORKSPACE as for one sequence); FP_EHIP if a launch
 * fails, after the earlier sequences have been enqueued.  Each sequence's
 * capacity overflow is reported through its own status word.
 */
int fp_index_batch(const fp_shape *shape, int nseq, const int32_t *seqlens,
                   const void *Q, const void *K, float gamma, float tau,
                   fp_index_out *outs, void *ws, size_t ws_bytes, void *stream);
int fp_attn_batch(const fp_shape *shape, int nseq, const int32_t *seqlens,
                  const void *Q, const void *K, const void *V,
                  const fp_index_out *csrs, void *O,
                  void *ws, size_t ws_bytes, void *stream);

/*
 * Workspace bytes with which every run of equal-length sequences of a batch
 * (see above) runs as one call: seqlens as for the batch calls (host array),
 * shape->S ignored; variant 0 for fp_index_batch, fp_attn_batch and
 * fp_index_i8_batch, 1 for fp_attn_i8_batch (or for all four).  Host only.
 * Returns FP_EINVAL (null pointers, nseq < 1, variant not 0 or 1) or the
 * shape errors of fp_workspace_bytes.
 */
int fp_batch_workspace_bytes(const fp_shape *shape, int nseq, const int32_t *seqlens, int variant,
                             size_t *bytes);

/*
 * The same for W8A8 inputs (as fp_index_i8 / fp_attn_i8): Q8, K8, V8 packed
 * like Q, K, V above (one byte per element), and the per-token scales packed
 * the same way, sQ as [Hq, S_s] blocks and sK, sV as [Hkv, S_s] blocks one
 * after another.  O is bf16, packed like Q.  Null scales give FP_EINVAL.
 */
int fp_index_i8_batch(const fp_shape *shape, int nseq, const int32_t *seqlens,
                      const int8_t *Q8, const float *sQ, const int8_t *K8,
                      const float *sK, float gamma, float tau,
                      fp_index_out *outs, void *ws, size_t ws_bytes, void *stream);
int fp_attn_i8_batch(const fp_shape *shape, int nseq, const int32_t *seqlens,
                     const int8_t *Q8, const float *sQ, const int8_t *K8,
                     const float *sK, const int8_t *V8, const float *sV,
                     const fp_index_out *csrs, void *O,
                     void *ws, size_t ws_bytes, void *stream);

/*
 * Test hook for the W8A8 score product ([E] 3.3: INT8 x INT8 with INT32
 * accumulation): out[c][r] = Q8[h, i*b + r] . K8[h / G, j*b + c] (exact
 * int32) for r, c in [0, b), computed through the staging and int8
 * matrix-core tile code of one of the two kernels that use it, at the
 * workgroup size that kernel runs with for this shape:
 *   path FP_PROBE_ATTN:  fp_attn_i8's kernel (direct-to-LDS loads of the
 *                        int8 key rows into padded LDS rows);
 *   path FP_PROBE_STATS: fp_index_i8's streaming statistics kernel
 *                        (direct loads into padded LDS rows, up to 128
 *                        keys per staging unit).
 *   out: device int32 [b, b] (key-major: out[c * b + r]).
 * Errors: FP_EINVAL (null pointer, h, i or j out of range, unknown path),
 * FP_EUNSUPPORTED, FP_EHIP.
 */
#define FP_PROBE_ATTN  0
#define FP_PROBE_STATS 1
int fp_probe_qk_i8(const fp_shape *shape, const int8_t *Q8, const int8_t *K8,
                   int h, int i, int j, int path, int32_t *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FPATTN_H */
