// Block-sparse causal attention over the grouped-query job list.
//
// The explainer ("FPGA24成果：FAST-Prefill稀疏注意力加速器", yunpan.plus)
// section 1.1 gives the attention softmax(Q K^T / sqrt(d_k)) V; section 1.2
// (figure 3) restricts each query block to the key/value blocks its sparse
// index names.  For query token t of block i and head h, the keys are those
// k <= t whose block is in J(h, i); the softmax runs over exactly those keys.
// The softmax is taken chunk by chunk against a running reference maximum
// (the re-telling "FPGA加速动态稀疏注意力技术解析与优化", section 3.3,
// normalises attention scores block-wise to avoid overflow).
//
// W8A8 (explainer sections 3.3 and 4.2): Q.K^T on the int8 matrix cores with
// int32 accumulation, scaled by sigma * sQ[t] * sK[k]; P.V in bf16 against V
// taken as bf16(sV[k] * v8[k]), formed once per call (k_widen_v8), so the chunk
// stream stages V and runs P.V exactly as in the bf16 form.
//
// Kernel layout.  The explainer's section 2.2 notes that grouped-query heads
// re-fetch the same K/V blocks; section 3.2 schedules sparse attention from a
// compact job list.  A job is (KV group g, query block i) with the union of
// the G heads' key blocks; a work unit is a job or a share of its query
// tiles.  The kernel is persistent: one workgroup per CU takes units in job
// order (longest first), the first ones statically and the rest from an
// atomic counter.  Each key block is staged in LDS once, 128 keys at a time,
// and used by every head of the group whose mask bit is set; one wave owns
// one (head, 32-query tile).  One stream of chunks runs across units: while
// chunk c is computed from one LDS buffer, chunk c + 1 is copied into the
// other by direct global-to-LDS loads.  Scores are computed transposed,
// S^T = K Q^T, on the 32x32x16 matrix cores so that every lane owns one query
// row; its softmax weights are then already the operand of O^T += V^T P^T,
// whose V^T operand comes from LDS transpose reads of the key-major V rows.
#include <algorithm>

#include "fp_common.hpp"
#include "fp_internal.hpp"

namespace fp {
namespace {

struct AttnArgs {
  const uint8_t *Q, *K, *V;
  const float *sQ, *sK, *sV;
  const int32_t *job_ptr, *job_blk, *job_order;
  const uint32_t *job_mask;
  uint16_t *O;
  int S, N, B, G, qpw, parts;
  float c2;
  float *part;        // split-KV units only: fp32 partial outputs, [slot][G][b][kPartStride]
};

// Split-KV units (fp_attn_split): a partial output row holds the unnormalised O^T row (128 fp32), the
// reference maximum m (log2 units) and the weight sum l, padded to 16 bytes.
constexpr int kPartStride = 132;

constexpr int kChunkDl = 128;                // keys per staged chunk
// Lazy-rescale headroom: weights stay below 2^24 before a rescale, so O^T (at
// most 2^24 times the key count times max |V|) stays far inside fp32.
constexpr float kRescaleDl = 24.0f;
constexpr float kRescaleSumDl = 16777216.0f;   // 2^kRescaleDl

template <bool I8> struct KL {
  static constexpr int Stride = I8 ? 144 : 272;        // LDS bytes per staged key row (padded)
};

// Q fragments (operand B of S^T = K Q^T) for query token `tok` of this lane.
template <bool I8>
__device__ __forceinline__ void load_q(const uint8_t *Q, size_t tok, u32x4 qf[8]) {
  const int hf = (threadIdx.x & 63) >> 5;
  if (!I8) {
    const uint8_t *p = Q + tok * 256 + 16 * hf;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = *(const u32x4 *)(p + 32 * s);
  } else {
    const uint8_t *p = Q + tok * 128 + 16 * hf;
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[s] = *(const u32x4 *)(p + 32 * s);
  }
}

// Raw scores of 32 staged keys (rows key0..key0+31 of ks) against the wave's
// 32 queries: transposed tile, acc[r] <-> key key0 + acc_row(r), query lane%32.
template <bool I8>
__device__ __forceinline__ void raw_scores(const uint8_t *ks, int key0, const u32x4 qf[8],
                                           float x[16]) {
  const int lane = threadIdx.x & 63;
  const uint8_t *arow = ks + (key0 + (lane & 31)) * KL<I8>::Stride + 16 * (lane >> 5);
  if (!I8) {
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < 8; ++s) acc = mfma_bf16(*(const u32x4 *)(arow + 32 * s), qf[s], acc);
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = acc[r];
  } else {
    i32x16 acc = {};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mfma_i8(*(const u32x4 *)(arow + 32 * s), qf[s], acc);
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = (float)acc[r];
  }
}

// ---------------------------------------------------------------------------
// bf16 path with direct-to-LDS staging.  Each 128-key chunk of K and V is
// copied from global memory into LDS by global_load_lds_dwordx4 (lane L of one
// instruction fills bytes [16L, 16L+16) of a 1 KiB LDS span, from any global
// address the lane names), so staging costs no registers and no ALU work.
//  * K keeps rows of 17 slots of 16 B (272 B: the 32 rows one score tile
//    reads at one column fall in distinct bank groups); the pad slot receives
//    a duplicate of the row's last slot.
//  * V keeps its natural key-major rows of 256 B, the 16 B slot c of key row
//    r stored at c ^ 4 (r & 3).  The V^T operand of O^T += V^T P^T is read
//    with the LDS transpose read ds_read_b64_tr_b16: in each 16-lane block,
//    lane i receives element i % 4 of the 4-element rows addressed by lanes
//    i / 4, i / 4 + 4, i / 4 + 8, i / 4 + 12.  Lane 4e + q of a block
//    addresses key row e, columns 4q .. 4q + 3 of its 16-column slice, so the
//    block receives 16 columns x 4 consecutive keys, transposed.

namespace dl {
constexpr int KSlots = 17;                          // 16 B slots per staged K row
constexpr int KRow = KSlots * 16;                   // 272 B
constexpr int KBuf = kChunkDl * KRow;                 // 34816 B
constexpr int VBuf = kChunkDl * 256;                  // 32768 B
constexpr int KLoads = kChunkDl * KSlots / 64;        // 34 one-KiB loads
constexpr int VLoads = VBuf / 1024;                 // 32
static_assert(kChunkDl * KSlots % 64 == 0, "K staging must be whole 1 KiB spans");
// int8 form: K rows of 128 B staged as 9 slots (144 B); V rows of the widened
// bf16 copy staged as in the bf16 form; one more load carries the chunk's K and
// V scales.
constexpr int KSlots8 = 9;
constexpr int KRow8 = KSlots8 * 16;                 // 144 B
constexpr int KBuf8 = kChunkDl * KRow8;             // 18432 B
constexpr int KLoads8 = kChunkDl * KSlots8 / 64;    // 18
static_assert(kChunkDl * KSlots8 % 64 == 0, "K staging must be whole 1 KiB spans");
static_assert(kChunkDl == 128, "the scale load covers 128 keys");
}  // namespace dl

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Issue this wave's share of the direct loads of one chunk (rows from kg/vg).
__device__ __forceinline__ void dl_issue(const uint8_t *kg, const uint8_t *vg, uint32_t kb, uint32_t vb,
                                         int wave, int nw) {
  const int lane = threadIdx.x & 63;
  for (int u = wave; u < dl::KLoads + dl::VLoads; u += nw) {
    if (u < dl::KLoads) {
      const int s = 64 * u + lane, row = s / dl::KSlots, c = min(s - row * dl::KSlots, 15);
      lds_dma16(kg + row * 256 + 16 * c, kb + 1024 * u);
    } else {
      const int v = u - dl::KLoads, row = 4 * v + (lane >> 4), c = (lane & 15) ^ (4 * (lane >> 4));
      lds_dma16(vg + row * 256 + 16 * c, vb + 1024 * v);
    }
  }
}

// int8: this wave's share of the direct loads of one chunk: the int8 K rows (9-slot rows, as
// dl_issue's 17-slot ones), the bf16 V rows of the widened copy (exactly as dl_issue; none when vg
// is null, for the probe) and the scales (sK then sV, 128 each, one load).
__device__ __forceinline__ void dl_issue8(const uint8_t *kg, const uint8_t *vg, const float *skg, const float *svg,
                                          uint32_t kb, uint32_t vb, uint32_t sb, int wave, int nw) {
  const int lane = threadIdx.x & 63;
  const int nv = vg ? dl::VLoads : 0;
  for (int u = wave; u < dl::KLoads8 + nv + 1; u += nw) {
    if (u < dl::KLoads8) {
      const int s = 64 * u + lane, row = s / dl::KSlots8, c = min(s - row * dl::KSlots8, 7);
      lds_dma16(kg + row * 128 + 16 * c, kb + 1024 * u);
    } else if (u < dl::KLoads8 + nv) {
      const int v = u - dl::KLoads8, row = 4 * v + (lane >> 4), c = (lane & 15) ^ (4 * (lane >> 4));
      lds_dma16(vg + row * 256 + 16 * c, vb + 1024 * v);
    } else {
      lds_dma16(lane < 32 ? skg + 4 * lane : svg + 4 * (lane - 32), sb);
    }
  }
}

// Two-source forms for 64-key blocks: LDS rows 0..63 from the rows at ka/va (first block),
// rows 64..127 from those at kb_/vb_ (second block); otherwise as dl_issue / dl_issue8.
__device__ __forceinline__ void dl_issue2(const uint8_t *ka, const uint8_t *va, const uint8_t *kb_,
                                          const uint8_t *vb_, uint32_t kb, uint32_t vb, int wave, int nw) {
  const int lane = threadIdx.x & 63;
  for (int u = wave; u < dl::KLoads + dl::VLoads; u += nw) {
    if (u < dl::KLoads) {
      const int s = 64 * u + lane, row = s / dl::KSlots, c = min(s - row * dl::KSlots, 15);
      lds_dma16((row < 64 ? ka + row * 256 : kb_ + (row - 64) * 256) + 16 * c, kb + 1024 * u);
    } else {
      const int v = u - dl::KLoads, row = 4 * v + (lane >> 4), c = (lane & 15) ^ (4 * (lane >> 4));
      lds_dma16((row < 64 ? va + row * 256 : vb_ + (row - 64) * 256) + 16 * c, vb + 1024 * v);
    }
  }
}
__device__ __forceinline__ void dl_issue8_2(const uint8_t *ka, const uint8_t *va, const float *ska,
                                            const float *sva, const uint8_t *kb_, const uint8_t *vb_,
                                            const float *skb, const float *svb, uint32_t kb, uint32_t vb,
                                            uint32_t sb, int wave, int nw) {
  const int lane = threadIdx.x & 63;
  const int nv = va ? dl::VLoads : 0;
  for (int u = wave; u < dl::KLoads8 + nv + 1; u += nw) {
    if (u < dl::KLoads8) {
      const int s = 64 * u + lane, row = s / dl::KSlots8, c = min(s - row * dl::KSlots8, 7);
      lds_dma16((row < 64 ? ka + row * 128 : kb_ + (row - 64) * 128) + 16 * c, kb + 1024 * u);
    } else if (u < dl::KLoads8 + nv) {
      const int v = u - dl::KLoads8, row = 4 * v + (lane >> 4), c = (lane & 15) ^ (4 * (lane >> 4));
      lds_dma16((row < 64 ? va + row * 256 : vb_ + (row - 64) * 256) + 16 * c, vb + 1024 * v);
    } else {
      // lanes 0..15 / 16..31: sK of the two blocks, 32..47 / 48..63: sV
      const int q = lane >> 4, o = 4 * (lane & 15);
      lds_dma16(q == 0 ? ska + o : q == 1 ? skb + o : q == 2 ? sva + o : svb + o, sb);
    }
  }
}

// fp_attn_i8: the int8 V codes times their per-token scale, rounded to bf16 once per call, in the
// key-major layout the chunk stream stages from; P.V then runs exactly as in the bf16 form.  Thread
// t converts the 16 codes at byte 16 t (all of one token's row: 128 codes are 8 threads).
__global__ void __launch_bounds__(256) k_widen_v8(const uint8_t *v8, const float *sv, uint16_t *vw, size_t n16) {
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n16) return;
  const u32x4 in = *(const u32x4 *)(v8 + 16 * t);
  const float sc = sv[t >> 3];
  uint32_t w[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t word = in[k >> 1] >> (16 * (k & 1));
    w[k] = pack_bf16x2(sc * (float)(int8_t)(word & 0xffu), sc * (float)(int8_t)((word >> 8) & 0xffu));
  }
  u32x4 *o = (u32x4 *)(vw + 16 * t);
  o[0] = u32x4{w[0], w[1], w[2], w[3]};
  o[1] = u32x4{w[4], w[5], w[6], w[7]};
}

// An LDS byte address the compiler cannot fold constants into (keeps the
// per-read offsets small enough for the instruction's immediate field).
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ u32x4 tr_pair(uint32_t addr) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(size_t)addr);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(size_t)(addr + 8 * 256));
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
  return u32x4{l2[0], l2[1], h2[0], h2[1]};
}

// A load of a value every lane shares, kept on the vector memory path (an
// opaque VGPR zero in the address): such loads are waited on through vmcnt,
// which the chunk loop only drains at its barriers.  Scalar loads would share
// lgkmcnt with the LDS operand reads and stall the first of them.
template <typename T>
__device__ __forceinline__ T vload(const T *p) {
  int z = 0;
  asm volatile("" : "+v"(z));
  return p[z];
}
__device__ __forceinline__ int sgpr(int v) { return __builtin_amdgcn_readfirstlane(v); }

// A job-list entry (key block and head mask) by two scalar loads, waited for inside the same asm
// statement, so the chunk loop holds no vector load the compiler tracks (its own wait for one
// would also wait for the prefetch below).  Issued right after a chunk barrier, where no LDS read
// is outstanding; consecutive entries share a scalar-cache line.
__device__ __forceinline__ void sload_entry(const int *pb, const uint32_t *pm, int &jv, uint32_t &mv) {
  asm volatile("s_load_dword %0, %2, 0x0\n\ts_load_dword %1, %3, 0x0\n\ts_waitcnt lgkmcnt(0)"
               : "=s"(jv), "=s"(mv)
               : "s"(pb), "s"(pm)
               : "memory");
}

// One dword per lane from global memory into LDS (M0 + 4 * lane), by a direct load.
__device__ __forceinline__ void lds_dma4(const void *g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}

// L2 prefetch of the K rows of a chunk a step ahead of its own loads: one dword of every 128-byte
// line (kbytes from kg) is read into a small LDS sink that nothing reads, so the HBM fetch of chunk
// c + 2 overlaps chunk c and the loads of c + 2, issued during chunk c + 1, find its K rows in L2.
// (K is read first in a chunk; prefetching V as well, or touching every 64 or 32 bytes, measured
// slower.)  Wave w covers lines 64 w .. 64 w + 63; returns whether this wave issued a load
// (uniform in the wave).
constexpr int kPfLine = 128;
__device__ __forceinline__ bool dl_prefetch(const uint8_t *kg, int kbytes, uint32_t sink, int wave) {
  const int lane = threadIdx.x & 63;
  const int nl = kbytes / kPfLine;
  if (64 * wave >= nl) return false;
  lds_dma4(kg + (size_t)kPfLine * min(64 * wave + lane, nl - 1), sink);
  return true;
}
// The same for the K rows of two 64-key blocks (kbytes each; the second from kg2 unless null).
__device__ __forceinline__ bool dl_prefetch2(const uint8_t *kg1, const uint8_t *kg2, int kbytes, uint32_t sink,
                                             int wave) {
  const int lane = threadIdx.x & 63;
  const int n1 = kbytes / kPfLine, nl = kg2 ? 2 * n1 : n1;
  if (64 * wave >= nl) return false;
  const int line = min(64 * wave + lane, nl - 1);
  lds_dma4(line < n1 ? kg1 + (size_t)kPfLine * line : kg2 + (size_t)kPfLine * (line - n1), sink);
  return true;
}
constexpr int kWaitVm1 = 0x0f71;     // s_waitcnt vmcnt(1): all but the youngest vector memory op

// One unit of work: job (KV group g, query block i) in the job order, query
// tile share `part` of it, its first job-list entry p0, chunk count and the
// chunk the rotated visiting order starts from.
struct Unit {
  int u, g, i, part, p0, n, total, rot;        // n: job-list entries, total: chunks
  bool empty;                                  // no job-list entry: one chunk that computes nothing
  int slot;                                    // split-KV unit: its partial-output slot (else -1)
};

// Job-list entry of one chunk: key block jv and head mask maskv (as loaded,
// made scalar where used), 128-key chunk kc of the block, KV group g.  With
// 64-key blocks a chunk holds two consecutive entries, the second in jv2/maskv2.
struct Ent {
  int jv;
  uint32_t maskv;
  int kc, g;
  int jv2;                                     // 64-key blocks: the chunk's second entry (-1: none)
  uint32_t maskv2;
};

// Persistent form: one workgroup per compute unit takes units in job order
// (the first two statically, later ones from an atomic counter) and runs one
// continuous chunk stream across them, so the next unit's first chunk is
// loaded while the current unit's last chunk is computed.  A workgroup stops
// at the first unit index past the end; indices only grow, so none is lost.
//
// SPLIT (fp_attn_split): a unit may cover a contiguous range of its job's entries (a split-KV
// segment).  Such a unit's table entry carries -1 - slot in place of the rotation, and instead of
// normalising and writing O it writes its unnormalised rows with their (m, l) to partial slot
// `slot`; k_attn_combine merges a job's slots afterwards.
template <int NT, bool I8, bool PAIR, bool SPLIT>
__global__ void __launch_bounds__(NT) k_attn_dl(AttnArgs a, const int4 *utab, int nunits, unsigned int *ctr) {
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf[2][I8 ? dl::KBuf8 : dl::KBuf];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf[2][dl::VBuf];
  __shared__ __attribute__((aligned(16))) float sbuf[2][I8 ? 2 * kChunkDl : 4];   // int8: sK, sV of the chunk
  __shared__ int s_claim[2];
  __shared__ __attribute__((aligned(256))) uint32_t s_sink[64];   // prefetch sink (never read)
  const int lane = threadIdx.x & 63, hf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr int NW = NT / 64;
  const int N = a.N, S = a.S, B = a.B;
  const int nck = B / kChunkDl;                 // 128-key chunks per block (0 with 64-key blocks)
  const int hh = wave / a.qpw;
  const bool live = hh < a.G;                    // else a spare wave: it only stages and waits
  const float qscale = a.c2;

  auto unit_from = [&](int u, const int4 &t) -> Unit {
    Unit x{u, 0, 0, 0, 0, 0, 0, 0, true, -1};
    if (u >= nunits) return x;
    const int job = sgpr(t.x);
    x.part = u % a.parts;
    x.g = job / N;
    x.i = job - x.g * N;
    x.p0 = sgpr(t.y);
    x.n = sgpr(t.z);
    x.total = PAIR ? (x.n + 1) >> 1 : x.n * nck;
    x.rot = sgpr(t.w);
    if constexpr (SPLIT) {
      if (x.rot < 0) {
        x.slot = -1 - x.rot;
        x.rot = 0;
      }
    }
    x.empty = x.total == 0;
    if (x.empty) x.total = 1;
    return x;
  };
  auto fetch = [&](const Unit &x, int c) -> Ent {
    if (c >= x.total || x.empty) return Ent{-1, 0u, 0, 0, -1, 0u};
    int cr = c + x.rot;
    cr = cr >= x.total ? cr - x.total : cr;
    if constexpr (PAIR) {
      const int e = sgpr(x.p0 + 2 * cr);
      int jv, jv2 = -1;
      uint32_t mv, mv2 = 0u;
      sload_entry(a.job_blk + e, a.job_mask + e, jv, mv);
      if (2 * cr + 1 < x.n) sload_entry(a.job_blk + e + 1, a.job_mask + e + 1, jv2, mv2);
      return Ent{jv, mv, 0, x.g, jv2, mv2};
    } else {
      const int e = sgpr(x.p0 + cr / nck);
      int jv;
      uint32_t mv;
      sload_entry(a.job_blk + e, a.job_mask + e, jv, mv);
      return Ent{jv, mv, cr % nck, x.g, -1, 0u};
    }
  };
  auto issue = [&](const Ent &en, int b) {
    const int j = sgpr(en.jv);
    if (PAIR && j >= 0 && j < N) {
      // second block: a missing or out-of-range one repeats the first (loaded, never run)
      int j2 = sgpr(en.jv2);
      j2 = j2 >= 0 && j2 < N ? j2 : j;
      const size_t ra = (size_t)en.g * S + (size_t)j * B, rb = (size_t)en.g * S + (size_t)j2 * B;
      if constexpr (!I8) {
        dl_issue2(a.K + ra * 256, a.V + ra * 256, a.K + rb * 256, a.V + rb * 256, lds_addr(kbuf[b]),
                  lds_addr(vbuf[b]), wave, NW);
      } else {
        dl_issue8_2(a.K + ra * 128, a.V + ra * 256, a.sK + ra, a.sV + ra, a.K + rb * 128, a.V + rb * 256,
                    a.sK + rb, a.sV + rb, lds_addr(kbuf[b]), lds_addr(vbuf[b]), lds_addr(sbuf[b]), wave, NW);
      }
    } else if (!PAIR && j >= 0 && j < N) {
      const size_t row0 = (size_t)en.g * S + (size_t)j * B + en.kc * kChunkDl;
      if constexpr (!I8) {
        dl_issue(a.K + row0 * 256, a.V + row0 * 256, lds_addr(kbuf[b]), lds_addr(vbuf[b]), wave, NW);
      } else {
        dl_issue8(a.K + row0 * 128, a.V + row0 * 256, a.sK + row0, a.sV + row0, lds_addr(kbuf[b]),
                  lds_addr(vbuf[b]), lds_addr(sbuf[b]), wave, NW);
      }
    }
  };
  // the L2 prefetch of an entry's chunk (its K rows); whether this wave issued a load
  auto prefetch = [&](const Ent &en) -> bool {
    if constexpr (PAIR) {
      // both 64-key blocks of the chunk (a missing or out-of-range second one is not touched)
      const int j = sgpr(en.jv), j2 = sgpr(en.jv2);
      if (!(j >= 0 && j < N)) return false;
      const int rb = B * (I8 ? 128 : 256);
      const uint8_t *k1 = a.K + ((size_t)en.g * S + (size_t)j * B) * (I8 ? 128 : 256);
      const uint8_t *k2 = j2 >= 0 && j2 < N ? a.K + ((size_t)en.g * S + (size_t)j2 * B) * (I8 ? 128 : 256) : nullptr;
      return dl_prefetch2(k1, k2, rb, lds_addr(s_sink), wave);
    } else {
      const int j = sgpr(en.jv);
      if (!(j >= 0 && j < N)) return false;
      const size_t row0 = (size_t)en.g * S + (size_t)j * B + en.kc * kChunkDl;
      return dl_prefetch(a.K + row0 * (I8 ? 128 : 256), kChunkDl * (I8 ? 128 : 256), lds_addr(s_sink), wave);
    }
  };
  if ((int)blockIdx.x >= nunits) return;
  Unit cur = unit_from(blockIdx.x, vload(utab + blockIdx.x));
  int nxt_id = blockIdx.x + gridDim.x;                // claimed unit that follows cur
  Unit nxt{nunits, 0, 0, 0, 0, 0, 0, 0, true, -1};
  int parity = 0;
  Ent e0 = fetch(cur, 0), e1 = fetch(cur, 1);
  issue(e0, 0);

  // per-lane operand offsets: K rows (lane % 32) at column half hf; V^T per 32-column tile
  const int kl = (lane & 31) * dl::KRow + 16 * hf;
  const int j16 = lane & 15, bb = (lane >> 4) & 1;
  int vl[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) vl[dt] = (4 * hf + (j16 >> 2)) * 256 + 64 * (dt ^ (j16 >> 2)) + 32 * bb + 8 * (j16 & 3);

  int kk = 0;                                    // chunks streamed so far (LDS buffer parity)
  while (true) {
    // unit start: Q fragments, the table entry of the next unit and a claim for the one after it
    // are all in flight together and waited for once
    unsigned int claim = 0u;
    if (threadIdx.x == 0) {
      int z = 0;                                   // per-lane address: a plain returning atomic, waited below
      asm volatile("" : "+v"(z));
      claim = atomicAdd(ctr + z, 1u);
    }
    const int4 ntab = vload(utab + min(nxt_id, nunits - 1));   // (ignored past the end)
    // query tile of this wave, rotated by head: the waves sharing a SIMD (wave % 4) then hold
    // different tiles, which evens out the per-SIMD work on diagonal blocks
    const int qtok0 = cur.i * B + (cur.part * a.qpw + (wave + hh) % a.qpw) * 32;
    const int qtok = qtok0 + (lane & 31);
    const size_t tok = (size_t)(cur.g * a.G + (live ? hh : 0)) * S + qtok;
    u32x4 qf[8];
    load_q<I8>(a.Q, tok, qf);
    const float qsc = I8 ? qscale * a.sQ[tok] : qscale;
    f32x16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
    float m = -1e30f, l = 0.0f;
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    if (threadIdx.x == 0) s_claim[parity] = 2 * gridDim.x + (int)claim;
    nxt = unit_from(nxt_id, ntab);
    auto stream = [&](int c) -> Ent { return c < cur.total ? fetch(cur, c) : fetch(nxt, c - cur.total); };
    if (cur.total == 1) e1 = fetch(nxt, 0);        // the stream's next chunk lies in nxt, unknown until now
    __syncthreads();

    for (int c = 0; c < cur.total; ++c, ++kk) {
      const int buf = kk & 1;
      issue(e1, buf ^ 1);                          // the next chunk of the stream (no-op past its end)
      const Ent e2 = stream(c + 2);
      const bool pf = prefetch(e2);                // after the loads above: the youngest op of the wave
      const int j0 = sgpr(e0.jv);
      const uint32_t mask0 = (uint32_t)sgpr((int)e0.maskv);
      const int key0 = j0 * B + e0.kc * kChunkDl;
      // 64-key blocks: each half runs on its own (this wave's head in its mask, a key at or
      // before the tile's last query); otherwise both halves follow the one entry
      const int j2 = PAIR ? sgpr(e0.jv2) : -1;
      const int key2 = j2 * B;
      const bool ok0 = live && j0 >= 0 && j0 < N && ((mask0 >> hh) & 1u) && key0 <= qtok0 + 31;
      const bool run_a = ok0 && (!PAIR || key0 <= qtok0 + 31);
      const bool run_b = PAIR ? live && j0 >= 0 && j0 < N && j2 >= 0 && j2 < N &&
                                    (((uint32_t)sgpr((int)e0.maskv2) >> hh) & 1u) && key2 <= qtok0 + 31
                              : ok0;
      if (run_a || run_b) {
        const bool diag = key0 + kChunkDl - 1 > qtok0;
        const uint32_t kp = opaque(lds_addr(kbuf[buf]) + kl);
        // int8 K rows: KL<true>::Stride bytes each
        const uint32_t kp8 = I8 ? opaque(lds_addr(kbuf[buf]) + (lane & 31) * KL<true>::Stride + 16 * hf) : 0u;
        uint32_t vp[4];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) vp[dt] = opaque(lds_addr(vbuf[buf]) + vl[dt]);
        const float *sks = sbuf[buf];
        bool piped = false;
        if constexpr (!PAIR && NT <= 768) {
          if (!diag) {
            // Every key of the chunk precedes the wave's first query: no tile is masked or
            // skipped, and the four tiles run software-pipelined with P.V one tile behind.
            // The P.V products of tile kt - 1 are issued in the same basic block as the
            // softmax of tile kt, so the matrix cores work while the wave computes
            // exponentials.  The new reference maximum is chosen without a branch; only the
            // (rare) rescale of O is one, placed after tile kt - 1 has been added.
            piped = true;
            auto qk = [&](int kb) {
              f32x16 acc = {};
              if constexpr (!I8) {
#pragma unroll
                for (int s = 0; s < 8; ++s)
                  acc = mfma_bf16(*(const __attribute__((address_space(3))) u32x4 *)(size_t)(kp + kb * dl::KRow + 32 * s),
                                  qf[s], acc);
              } else {
                // int32 tile on the int8 matrix cores (K rows of KL<true>::Stride bytes), times
                // the key scales of its rows
                i32x16 ia = {};
#pragma unroll
                for (int s = 0; s < 4; ++s)
                  ia = mfma_i8(*(const __attribute__((address_space(3))) u32x4 *)(size_t)(kp8 + kb * KL<true>::Stride + 32 * s),
                               qf[s], ia);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                  const f32x4 s4 = *(const f32x4 *)(sks + kb + 8 * q + 4 * hf);
#pragma unroll
                  for (int e = 0; e < 4; ++e) acc[4 * q + e] = (float)ia[4 * q + e] * s4[e];
                }
              }
              return acc;
            };
            // softmax weights of one tile (bf16 pairs), first against the current reference
            // maximum m with no maximum pass: a score above m + kRescaleDl gives a weight above
            // 2^kRescaleDl, so the tile's sum reaching that bound (or infinity, as while m is
            // unset) is the only case that can need a new maximum.  Only then is the tile's
            // maximum taken and, where it exceeds m + kRescaleDl, m raised and the weights redone;
            // m therefore moves exactly as under a maximum pass of every tile.
            auto weights = [&](const f32x16 &sc, u32x4 pf[2], float &alpha, bool ilv) {
              auto eval = [&]() {
                float lt = 0.0f;
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                  for (int w = 0; w < 4; ++w) {
                    const uint32_t pw = pack_bf16x2(fast_exp2(fmaf(sc[8 * s2 + 2 * w], qsc, -m)),
                                                    fast_exp2(fmaf(sc[8 * s2 + 2 * w + 1], qsc, -m)));
                    pf[s2][w] = pw;
                    lt = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw),
                                                         __builtin_bit_cast(bf16x2_t, 0x3f803f80u), lt, false);
                  }
                return lt;
              };
              float lt = eval();
              if (ilv) {
                // one basic block holds this tile's products, the previous tile's P.V products and
                // this tile's weights: the products each follow their operand reads (one ahead),
                // and the weights fill the P.V products' read waits
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
                for (int s = 0; s < 7; ++s) {
                  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                  __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
                for (int s = 0; s < 7; ++s) {
                  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                  __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                  __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              }
              bool grew = false;
              if (__any(!(lt < kRescaleSumDl))) {
                float mx = fmaxf(sc[0], sc[1]);
#pragma unroll
                for (int r = 2; r < 16; ++r) mx = fmaxf(mx, sc[r]);
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
                mx = fmaxf(mx, fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]))) * qsc;
                const bool grow = mx > m + kRescaleDl;
                if (__any(grow)) {
                  const float mnew = grow ? mx : m;
                  alpha = fast_exp2(m - mnew);           // exactly 1 where the maximum stays
                  m = mnew;
                  l *= alpha;
                  lt = eval();
                  grew = true;
                }
              }
              l += lt;
              return grew;
            };
            auto pv = [&](int kb, const u32x4 pf[2]) {
#pragma unroll
              for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
                  o[dt] = mfma_bf16(tr_pair(vp[dt] + (kb + 16 * s2) * 256), pf[s2], o[dt]);
            };
            u32x4 pp[2];
            float alpha;
            if (weights(qk(0), pp, alpha, false)) {
#pragma unroll
              for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
            }
#pragma unroll
            for (int kt = 1; kt < kChunkDl / 32; ++kt) {
              const f32x16 sc = qk(32 * kt);
              pv(32 * (kt - 1), pp);
              u32x4 pn[2];
              if (weights(sc, pn, alpha, true)) {
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
              }
              pp[0] = pn[0];
              pp[1] = pn[1];
            }
            pv(kChunkDl - 32, pp);
          }
        }
        if constexpr (PAIR && NT <= 512) {
          // Two 64-key blocks: the halves that have work for this wave run pipelined (two or four
          // tiles) when all their keys precede the wave's first query.  (Up to 8 waves: the two
          // pipelined bodies need more than the 12-wave register budget.)
          if ((run_a || run_b) && (!run_a || key0 + 63 <= qtok0) && (!run_b || key2 + 63 <= qtok0)) {
            piped = true;
            auto qk = [&](int kb) {
              f32x16 acc = {};
              if constexpr (!I8) {
#pragma unroll
                for (int s = 0; s < 8; ++s)
                  acc = mfma_bf16(*(const __attribute__((address_space(3))) u32x4 *)(size_t)(kp + kb * dl::KRow + 32 * s),
                                  qf[s], acc);
              } else {
                // int32 tile on the int8 matrix cores (K rows of KL<true>::Stride bytes), times
                // the key scales of its rows
                i32x16 ia = {};
#pragma unroll
                for (int s = 0; s < 4; ++s)
                  ia = mfma_i8(*(const __attribute__((address_space(3))) u32x4 *)(size_t)(kp8 + kb * KL<true>::Stride + 32 * s),
                               qf[s], ia);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                  const f32x4 s4 = *(const f32x4 *)(sks + kb + 8 * q + 4 * hf);
#pragma unroll
                  for (int e = 0; e < 4; ++e) acc[4 * q + e] = (float)ia[4 * q + e] * s4[e];
                }
              }
              return acc;
            };
            // softmax weights of one tile (bf16 pairs), first against the current reference
            // maximum m with no maximum pass: a score above m + kRescaleDl gives a weight above
            // 2^kRescaleDl, so the tile's sum reaching that bound (or infinity, as while m is
            // unset) is the only case that can need a new maximum.  Only then is the tile's
            // maximum taken and, where it exceeds m + kRescaleDl, m raised and the weights redone;
            // m therefore moves exactly as under a maximum pass of every tile.
            auto weights = [&](const f32x16 &sc, u32x4 pf[2], float &alpha, bool ilv) {
              auto eval = [&]() {
                float lt = 0.0f;
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                  for (int w = 0; w < 4; ++w) {
                    const uint32_t pw = pack_bf16x2(fast_exp2(fmaf(sc[8 * s2 + 2 * w], qsc, -m)),
                                                    fast_exp2(fmaf(sc[8 * s2 + 2 * w + 1], qsc, -m)));
                    pf[s2][w] = pw;
                    lt = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw),
                                                         __builtin_bit_cast(bf16x2_t, 0x3f803f80u), lt, false);
                  }
                return lt;
              };
              float lt = eval();
              if (ilv) {
                // one basic block holds this tile's products, the previous tile's P.V products and
                // this tile's weights: the products each follow their operand reads (one ahead),
                // and the weights fill the P.V products' read waits
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
                for (int s = 0; s < 7; ++s) {
                  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                  __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
                for (int s = 0; s < 7; ++s) {
                  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                  __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                  __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              }
              bool grew = false;
              if (__any(!(lt < kRescaleSumDl))) {
                float mx = fmaxf(sc[0], sc[1]);
#pragma unroll
                for (int r = 2; r < 16; ++r) mx = fmaxf(mx, sc[r]);
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
                mx = fmaxf(mx, fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]))) * qsc;
                const bool grow = mx > m + kRescaleDl;
                if (__any(grow)) {
                  const float mnew = grow ? mx : m;
                  alpha = fast_exp2(m - mnew);           // exactly 1 where the maximum stays
                  m = mnew;
                  l *= alpha;
                  lt = eval();
                  grew = true;
                }
              }
              l += lt;
              return grew;
            };
            auto pv = [&](int kb, const u32x4 pf[2]) {
#pragma unroll
              for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
                  o[dt] = mfma_bf16(tr_pair(vp[dt] + (kb + 16 * s2) * 256), pf[s2], o[dt]);
            };
            auto run_tiles = [&](int t0, auto ntl) {
              constexpr int NTL = decltype(ntl)::value;
              u32x4 pp[2];
              float alpha;
              if (weights(qk(32 * t0), pp, alpha, false)) {
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
              }
#pragma unroll
              for (int kt = 1; kt < NTL; ++kt) {
                const f32x16 sc = qk(32 * (t0 + kt));
                pv(32 * (t0 + kt - 1), pp);
                u32x4 pn[2];
                if (weights(sc, pn, alpha, true)) {
#pragma unroll
                  for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
                }
                pp[0] = pn[0];
                pp[1] = pn[1];
              }
              pv(32 * (t0 + NTL - 1), pp);
            };
            if (run_a && run_b) run_tiles(0, std::integral_constant<int, 4>{});
            else run_tiles(run_a ? 0 : 2, std::integral_constant<int, 2>{});
          }
        }
#pragma unroll 1
        for (int kt = 0; kt < (piped ? 0 : kChunkDl / 32); ++kt) {
          const int kb = kt * 32;                  // LDS row of the tile
          const int key_t = PAIR ? (kt < 2 ? key0 : key2) + 32 * (kt & 1) : key0 + kb;   // its first key
          // a tile whose keys all follow the wave's last query contributes nothing
          if (PAIR ? !(kt < 2 ? run_a : run_b) || key_t > qtok0 + 31 : key_t > qtok0 + 31) continue;
          const bool diag_t = PAIR ? key_t + 31 > qtok0 : diag;
          float x[16];
          if constexpr (!I8) {
            f32x16 acc = {};
#pragma unroll
            for (int s = 0; s < 8; ++s)
              acc = mfma_bf16(*(const __attribute__((address_space(3))) u32x4 *)(size_t)(kp + kb * dl::KRow + 32 * s), qf[s], acc);
#pragma unroll
            for (int r = 0; r < 16; ++r) x[r] = acc[r];
          } else {
            // int32 tile (accumulator r of this lane is key kb + acc_row(r) = kb + 8 (r / 4) + 4 hf +
            // r % 4), times the key scales; the query scale enters with sigma below
            raw_scores<true>(kbuf[buf], kb, qf, x);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const f32x4 s4 = *(const f32x4 *)(sks + kb + 8 * q + 4 * hf);
#pragma unroll
              for (int e = 0; e < 4; ++e) x[4 * q + e] *= s4[e];
            }
          }
          if (diag_t) {
            // 4 * (lane / 32), the half-wave term of acc_row, computed here (one instruction the
            // compiler cannot hoist): kept live across the loop it is spilled, and its reload
            // waits for every load in flight, the next chunk's included
            int hw4;
            asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_and_b32 %0, 32, %0\n\tv_lshrrev_b32 %0, 3, %0" : "=v"(hw4));
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int row = 8 * (r >> 2) + hw4 + (r & 3);
              if (key_t + row > qtok) x[r] = -INFINITY;
            }
          }
          float mx = x[0];
#pragma unroll
          for (int r = 1; r < 16; ++r) mx = fmaxf(mx, x[r]);
          {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
            mx = fmaxf(mx, fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])));
            mx = mx > -INFINITY ? mx * qsc : -INFINITY;
          }
          const bool grow = mx > m + kRescaleDl;
          if (__any(grow)) {
            const float mnew = grow ? mx : m;
            const float alpha = fast_exp2(m - mnew);
            m = mnew;
            l *= alpha;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
          }
          u32x4 pf[2];
          if constexpr (!I8) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
              for (int w = 0; w < 4; ++w) {
                const uint32_t pw = pack_bf16x2(fast_exp2(fmaf(x[8 * s2 + 2 * w], qsc, -m)),
                                                fast_exp2(fmaf(x[8 * s2 + 2 * w + 1], qsc, -m)));
                pf[s2][w] = pw;
                l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw),
                                                    __builtin_bit_cast(bf16x2_t, 0x3f803f80u), l, false);
              }
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
              for (int s2 = 0; s2 < 2; ++s2)
                o[dt] = mfma_bf16(tr_pair(vp[dt] + (kb + 16 * s2) * 256), pf[s2], o[dt]);
          } else {
            // weights (summed into l), then P.V as in the bf16 form (the value scales are in the
            // widened V)
            float pv[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              pv[r] = fast_exp2(fmaf(x[r], qsc, -m));
              l += pv[r];
            }
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
              pf[s2] = u32x4{pack_bf16x2(pv[8 * s2 + 0], pv[8 * s2 + 1]), pack_bf16x2(pv[8 * s2 + 2], pv[8 * s2 + 3]),
                             pack_bf16x2(pv[8 * s2 + 4], pv[8 * s2 + 5]), pack_bf16x2(pv[8 * s2 + 6], pv[8 * s2 + 7])};
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
              for (int s2 = 0; s2 < 2; ++s2)
                o[dt] = mfma_bf16(tr_pair(vp[dt] + (kb + 16 * s2) * 256), pf[s2], o[dt]);
          }
        }
      }
      // this wave's loads of the next chunk have landed; its prefetch may still be in flight
      if (pf) __builtin_amdgcn_s_waitcnt(kWaitVm1);
      else __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __syncthreads();
      e0 = e1;
      e1 = e2;
    }

    l += xor32(l);
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    uint16_t *orow = a.O + tok * 128;
    bool direct = live;
    if constexpr (SPLIT) {
      if (live && cur.slot >= 0) {
        // split-KV segment: the unnormalised row (columns 32 dt + 8 j + 4 hf + (0..3) of this lane)
        // and its (m, l), for the combine step
        direct = false;
        const int r = qtok - cur.i * B;                        // row within the query block
        float *pr = a.part + (((size_t)cur.slot * a.G + hh) * B + r) * kPartStride;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            *(f32x4 *)(pr + 32 * dt + 8 * j + 4 * hf) =
                f32x4{o[dt][4 * j], o[dt][4 * j + 1], o[dt][4 * j + 2], o[dt][4 * j + 3]};
        if (hf == 0) *(float2 *)(pr + 128) = make_float2(m, l);
      }
    }
    if (direct) {
      // Lane (row, hf) holds columns 32 dt + 8 j + 4 hf + (0..3), j = 0..3, of its query row.
      // One swap with the other half-wave per 32-bit word (groups j = 0, 1 offered by the upper
      // half, j = 2, 3 by the lower) leaves each lane columns 32 dt + 16 hf + (0..15), stored as
      // two 16-byte pieces: half as many store instructions, each still covering 32 rows.
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t pa = pack_bf16x2(o[dt][2 * k] * inv, o[dt][2 * k + 1] * inv);        // j = 0, 1
          const uint32_t pb = pack_bf16x2(o[dt][8 + 2 * k] * inv, o[dt][8 + 2 * k + 1] * inv);  // j = 2, 3
          const auto sw = __builtin_amdgcn_permlane32_swap(pa, pb, false, false);
          lo[k] = sw[0];
          hi[k] = sw[1];
        }
        *(u32x4 *)(orow + dt * 32 + 16 * hf) = u32x4{lo[0], lo[1], hi[0], hi[1]};
        *(u32x4 *)(orow + dt * 32 + 16 * hf + 8) = u32x4{lo[2], lo[3], hi[2], hi[3]};
      }
    }

    cur = nxt;                                     // (every unit has a chunk barrier, which published the claim)
    if (cur.u >= nunits) break;
    nxt_id = s_claim[parity];
    parity ^= 1;
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);          // no prefetch outlives the workgroup's LDS
}

// Unit table {job, first job-list entry, entry count, rotated start chunk} and a zeroed claim counter.
// The rotation hashes the job's index within its sequence (jps jobs per sequence), so a sequence run
// side by side with others visits its chunks in the same order as when run alone.
__global__ void k_attn_prep(const int32_t *job_order, const int32_t *job_ptr, int nunits, int parts,
                            int nck, int jps, int4 *utab, unsigned int *ctr) {
  const int u = blockIdx.x * blockDim.x + threadIdx.x;
  if (u == 0) ctr[0] = 0u;
  if (u >= nunits) return;
  const int job = job_order[u / parts];
  const int p0 = job_ptr[job], n = job_ptr[job + 1] - p0;
  const int total = nck > 0 ? n * nck : (n + 1) >> 1;    // chunks (nck = 0: two 64-key blocks each)
  // chunks start at a per-job offset so that workgroups do not all fetch the same (sink) blocks at once
  const int rot = total > 0 ? (int)(((unsigned)(job % jps) * 2654435761u) % (unsigned)total) : 0;
  utab[u] = int4{job, p0, n, rot};
}

// Unit table of fp_attn_split: the nsplit longest jobs (the first in job order) are cut into nseg
// segments of consecutive entries, unit (segment, part); the other jobs follow as in k_attn_prep.
// A segment's entry carries -1 - slot (slot = job rank * nseg + segment) in place of the rotation.
__global__ void k_attn_prep_split(const int32_t *job_order, const int32_t *job_ptr, int nunits, int parts,
                                  int nck, int nsplit, int nseg, int4 *utab, unsigned int *ctr) {
  const int u = blockIdx.x * blockDim.x + threadIdx.x;
  if (u == 0) ctr[0] = 0u;
  if (u >= nunits) return;
  const int nsu = nsplit * nseg * parts;
  if (u < nsu) {
    const int js = u / parts, k = js / nseg, seg = js % nseg;
    const int job = job_order[k];
    const int p0 = job_ptr[job], n = job_ptr[job + 1] - p0;
    const int s0 = (int)((long)n * seg / nseg), s1 = (int)((long)n * (seg + 1) / nseg);
    utab[u] = int4{job, p0 + s0, s1 - s0, -1 - (k * nseg + seg)};
  } else {
    const int job = job_order[nsplit + (u - nsu) / parts];
    const int p0 = job_ptr[job], n = job_ptr[job + 1] - p0;
    const int total = nck > 0 ? n * nck : (n + 1) >> 1;
    const int rot = total > 0 ? (int)(((unsigned)job * 2654435761u) % (unsigned)total) : 0;
    utab[u] = int4{job, p0, n, rot};
  }
}

// Keyed combine of fp_attn_split: for every row of the nsplit split jobs, merge the nseg partial
// rows (m_s, l_s, O_s): M = max m_s, O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s, as bf16.
// One wave per (job rank, head, row); lane c covers columns 2c and 2c + 1.
__global__ void __launch_bounds__(256) k_attn_combine(const float *part, const int32_t *job_order, int N, int S,
                                                      int B, int G, int nsplit, int nseg, uint16_t *O) {
  const int lane = threadIdx.x & 63;
  const int rowid = blockIdx.x * 4 + (threadIdx.x >> 6);          // (k, hh, r)
  if (rowid >= nsplit * G * B) return;
  const int r = rowid % B, hh = (rowid / B) % G, k = rowid / (B * G);
  const int job = job_order[k], g = job / N, i = job % N;
  float M = -3.0e38f;
  for (int sg = 0; sg < nseg; ++sg) {
    const float *pr = part + (((size_t)(k * nseg + sg) * G + hh) * B + r) * kPartStride;
    M = fmaxf(M, pr[128]);
  }
  float L = 0.0f, o0 = 0.0f, o1 = 0.0f;
  for (int sg = 0; sg < nseg; ++sg) {
    const float *pr = part + (((size_t)(k * nseg + sg) * G + hh) * B + r) * kPartStride;
    const float2 ml = *(const float2 *)(pr + 128);
    const float w = ml.y > 0.0f ? exp2f(ml.x - M) : 0.0f;
    const float2 ov = *(const float2 *)(pr + 2 * lane);
    L += w * ml.y;
    o0 += w * ov.x;
    o1 += w * ov.y;
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  uint16_t *orow = O + ((size_t)(g * G + hh) * S + (size_t)i * B + r) * 128;
  *(uint32_t *)(orow + 2 * lane) = pack_bf16x2(o0 * inv, o1 * inv);
}

// Test hook: out[c * B + r] = Q8[h, i*B + r] . K8[g, j*B + c] through the W8A8 attention kernel's
// own staging (direct-to-LDS loads of dl_issue8, or dl_issue8_2 for 64-key blocks, without the V
// rows) and its int8 tile code, at the workgroup size the kernel runs with for this shape; the
// accumulator rows are mapped back to keys as the kernel's masking does.  The scale slot of the
// loads reads bytes of the same key block (in bounds, never used).
template <int NT>
__global__ void __launch_bounds__(NT) k_probe_attn_i8(const uint8_t *Q, const uint8_t *K, int S, int B, int h,
                                                      int g, int i, int j, int32_t *out) {
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf[dl::KBuf8];
  __shared__ __attribute__((aligned(16))) float sbuf[2 * kChunkDl];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr int NW = NT / 64;
  const int nchunk = B >= kChunkDl ? B / kChunkDl : 1;
  for (int kc = 0; kc < nchunk; ++kc) {
    __syncthreads();                                          // the previous chunk's reads are done
    const uint8_t *kg = K + ((size_t)g * S + (size_t)j * B + kc * kChunkDl) * 128;
    const float *junk = (const float *)kg;
    if (B >= kChunkDl)
      dl_issue8(kg, nullptr, junk, junk, lds_addr(kbuf), 0u, lds_addr(sbuf), wave, NW);
    else   // 64-key blocks: both halves of the chunk carry block j
      dl_issue8_2(kg, nullptr, junk, junk, kg, nullptr, junk, junk, lds_addr(kbuf), 0u, lds_addr(sbuf),
                  wave, NW);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    const int keys = B >= kChunkDl ? kChunkDl : B;            // keys of block j in this chunk
    for (int qt = wave; qt < B / 32; qt += NW) {
      const int qr = qt * 32 + (lane & 31);
      u32x4 qf[8];
      load_q<true>(Q, (size_t)h * S + (size_t)i * B + qr, qf);
      for (int kb = 0; kb < keys; kb += 32) {
        float x[16];
        raw_scores<true>(kbuf, kb, qf, x);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kc * kChunkDl + kb + acc_row(r, lane);
          out[(size_t)key * B + qr] = (int32_t)x[r];
        }
      }
    }
  }
}

// Query tiles per attention workgroup: the largest divisor of b/32 keeping G * qpw <= 12 waves.
static int attn_qpw(const Plan &p) {
  const int qtiles = p.B / 32;
  int qpw = 1;
  for (int d = 1; d <= qtiles; d <<= 1)
    if (qtiles % d == 0 && p.G * d <= 12) qpw = d;
  return qpw;
}

// split: {nsplit, nseg} of fp_attn_split, or nullptr for the plain schedule.
template <int NT, bool I8, bool PAIR, bool SPLIT>
hipError_t run_attn_dl(const Plan &p, const AttnArgs &a, unsigned int *ctr, int4 *utab, const int *split,
                       hipStream_t st) {
  const int jobs = p.Hkv * p.N;
  const int nsplit = SPLIT ? std::min(split[0], jobs) : 0, nseg = SPLIT ? split[1] : 1;
  const int nunits = (jobs + nsplit * (nseg - 1)) * a.parts;
  const int per_cu = occupancy_per_cu((const void *)k_attn_dl<NT, I8, PAIR, SPLIT>, NT);
  const int cus = cu_count();
  const int grid = std::max(1, std::min(nunits, std::max(1, per_cu) * std::max(1, cus)));
  if (SPLIT)
    hipLaunchKernelGGL(k_attn_prep_split, dim3((nunits + 255) / 256), dim3(256), 0, st, a.job_order, a.job_ptr,
                       nunits, a.parts, p.B / kChunkDl, nsplit, nseg, utab, ctr);
  else
    hipLaunchKernelGGL(k_attn_prep, dim3((nunits + 255) / 256), dim3(256), 0, st, a.job_order, a.job_ptr,
                       nunits, a.parts, p.B / kChunkDl, p.seq_groups * p.N, utab, ctr);
  hipLaunchKernelGGL((k_attn_dl<NT, I8, PAIR, SPLIT>), dim3(grid), dim3(NT), 0, st, a, (const int4 *)utab, nunits,
                     ctr);
  if (SPLIT && nsplit > 0) {
    const int rows = nsplit * p.G * p.B;
    hipLaunchKernelGGL(k_attn_combine, dim3((rows + 3) / 4), dim3(256), 0, st, (const float *)a.part, a.job_order,
                       p.N, p.S, p.B, p.G, nsplit, nseg, a.O);
  }
  return hipGetLastError();
}

template <bool I8, bool PAIR, bool SPLIT = false>
hipError_t dispatch_attn(const Plan &p, const AttnArgs &a, unsigned int *ctr, int4 *utab, hipStream_t st,
                         const int *split = nullptr) {
  const int need = 64 * p.G * a.qpw;                 // G * qpw <= 16 (G <= 16, G * b <= 2048)
  if (need <= 256) return run_attn_dl<256, I8, PAIR, SPLIT>(p, a, ctr, utab, split, st);
  if (need <= 512) return run_attn_dl<512, I8, PAIR, SPLIT>(p, a, ctr, utab, split, st);
  if (need <= 768) return run_attn_dl<768, I8, PAIR, SPLIT>(p, a, ctr, utab, split, st);
  return run_attn_dl<1024, I8, PAIR, SPLIT>(p, a, ctr, utab, split, st);
}

}  // namespace

hipError_t launch_attn(const Plan &p, bool i8, const void *Q, const float *sQ, const void *K,
                       const float *sK, const void *V, const float *sV, const fp_index_out *csr,
                       void *O, unsigned int *ctr, int4 *utab, hipStream_t st, int nsplit, int nseg,
                       float *part, uint16_t *vw) {
  AttnArgs a;
  a.part = part;
  a.Q = (const uint8_t *)Q; a.K = (const uint8_t *)K; a.V = (const uint8_t *)V;
  if (i8) {   // the chunk stream reads V from its bf16 widening
    if (!vw) return hipErrorInvalidValue;
    const size_t n16 = (size_t)p.Hkv * p.S * 128 / 16;
    hipLaunchKernelGGL(k_widen_v8, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, st, (const uint8_t *)V, sV, vw, n16);
    a.V = (const uint8_t *)vw;
  }
  a.sQ = sQ; a.sK = sK; a.sV = sV;
  a.job_ptr = csr->job_ptr; a.job_blk = csr->job_blk; a.job_order = csr->job_order;
  a.job_mask = csr->job_mask;
  a.O = (uint16_t *)O;
  a.S = p.S; a.N = p.N; a.B = p.B; a.G = p.G;
  a.c2 = kLog2e / sqrtf((float)p.d);
  // query tiles per workgroup: the largest divisor of b/32 keeping G * qpw <= 12 waves; the
  // workgroup size is the next supported one (256, 512, 768 or 1024 threads), spare waves idle
  const int qpw = attn_qpw(p);
  a.qpw = qpw;
  a.parts = p.B / 32 / qpw;
  if (nseg > 1) {   // split-KV schedule (bf16, b >= 128)
    const int split[2] = {nsplit, nseg};
    return dispatch_attn<false, false, true>(p, a, ctr, utab, st, split);
  }
  if (p.B == 64)   // two 64-key blocks per 128-key chunk
    return i8 ? dispatch_attn<true, true>(p, a, ctr, utab, st) : dispatch_attn<false, true>(p, a, ctr, utab, st);
  return i8 ? dispatch_attn<true, false>(p, a, ctr, utab, st) : dispatch_attn<false, false>(p, a, ctr, utab, st);
}

size_t attn_split_slot_floats(const Plan &p) { return (size_t)p.G * p.B * kPartStride; }

hipError_t launch_probe_attn_i8(const Plan &p, const int8_t *Q8, const int8_t *K8, int h, int i, int j,
                                int32_t *out, hipStream_t st) {
  // the workgroup size dispatch_attn picks for this shape
  const int need = 64 * p.G * attn_qpw(p);
  const uint8_t *q = (const uint8_t *)Q8, *k = (const uint8_t *)K8;
  const int g = h / p.G;
  if (need <= 256) hipLaunchKernelGGL(k_probe_attn_i8<256>, dim3(1), dim3(256), 0, st, q, k, p.S, p.B, h, g, i, j, out);
  else if (need <= 512) hipLaunchKernelGGL(k_probe_attn_i8<512>, dim3(1), dim3(512), 0, st, q, k, p.S, p.B, h, g, i, j, out);
  else if (need <= 768) hipLaunchKernelGGL(k_probe_attn_i8<768>, dim3(1), dim3(768), 0, st, q, k, p.S, p.B, h, g, i, j, out);
  else hipLaunchKernelGGL(k_probe_attn_i8<1024>, dim3(1), dim3(1024), 0, st, q, k, p.S, p.B, h, g, i, j, out);
  return hipGetLastError();
}

}  // namespace fp
