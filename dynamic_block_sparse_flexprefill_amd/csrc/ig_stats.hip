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
// t_r = S - b + r of the last block.  With M_r the row's maximum and L_r its
// softmax denominator, the per-head outputs are, for each key block j,
//   lo[j] = (1/b) sum_r sum_{c <= r} exp(s_r[jb+c] - M_r) / L_r
//   hi[j] = (1/b) sum_r sum_{c >  r} exp(s_r[jb+c] - M_r) / L_r
// so that vertical mass v[j] = lo[j] + hi[j], and the slash mass of offset
// block o (token diagonal t_r - k pooled by b) is lo[N-1-o] + hi[N-2-o].
// Every key block is also mean-pooled into kbar[g][j][:] for the pooled
// estimate of Flex-Prefill's pattern test (explainer section 1.2).
//
// Two kernels.  k_ig_stream reads K once, in increasing block order: one
// workgroup per (KV group g, contiguous range of key blocks) -- all G query
// heads of the group share each staged block -- cut into chunks of CB blocks
// whose boundaries depend only on the shape.  For every row and block it keeps
// the lower / upper split sums exp2(x - m) against the row's reference maximum
// m of the current chunk (raised lazily, rescaling what the chunk already
// holds), and at each chunk's end writes them with the chunk's (m, sum) pair.
// k_ig_merge then forms every row's (M, L) from its chunk pairs, the block
// masses lo, hi from the per-(row, block) sums, and the pooled-estimate
// logits.  There is no grid-wide barrier and no limit on S from LDS, and the
// results do not depend on how many workgroups run or where.
//
// Each wave of k_ig_stream owns TPW tiles of 32 last-block query rows and
// keeps their Q fragments in registers; scores are computed transposed (keys x
// queries) on the 32x32x16 bf16 (or 32x32x32 int8) matrix cores so that every
// lane holds one query row.  Key blocks reach LDS by direct loads in units of
// up to 128 keys, two units in flight (the next one loads while the current
// one is used), one barrier per unit.
#include <algorithm>
#include <map>
#include <mutex>
#include <utility>

#include "fp_common.hpp"
#include "fp_internal.hpp"

namespace fp {
namespace {

template <bool I8> struct Tile;
template <> struct Tile<false> {   // bf16: 8 k-steps of 16, 272-byte LDS rows
  static constexpr int KS = 8, RowBytes = 256, Stride = 272;
};
template <> struct Tile<true> {    // int8: 4 k-steps of 32, 144-byte LDS rows
  static constexpr int KS = 4, RowBytes = 128, Stride = 144;
};

struct StreamArgs {
  const uint8_t *Q;   // bf16 or int8 [Hq, S, 128]
  const float *sQ;    // int8 only: [Hq, S]
  const uint8_t *K;   // bf16 or int8 [Hkv, S, 128]
  const float *sK;    // int8 only: [Hkv, S]
  int S, N, G;
  int nch, cpw;       // chunks, chunks per workgroup
  float c2;           // (1/sqrt(d)) * log2(e)
  float2 *lohi;       // [Hq][N][B]   (lo, hi) sums of every row and key block, against the chunk's m
  float2 *ml;         // [Hq][nch][B] (m, sum) of every row and chunk (log2 units)
  float *kbar;        // [Hkv][N][128]
  int32_t *status;    // the call's status word, cleared here (the index stage's first kernel); or null
};

constexpr float kHeadroom = 16.0f;   // a row's reference maximum is raised once a score exceeds it by this
constexpr float kHeadroomScale = 65536.0f;   // 2^kHeadroom

// Key blocks per chunk: at most 1024 keys, and the per-tile sums of a chunk ((lo, hi) of 32 rows
// per tile slot and block) within 32 KiB of LDS.  Depends only on the shape.
constexpr int chunk_blocks(int B, int ntl) {
  int cb = 1024 / B;
  while (cb > 1 && ntl * cb * 256 > 32 * 1024) cb >>= 1;
  return cb;
}

// Tile slots (waves x tiles per wave) of the streaming kernel's workgroup for G * b / 32 query tiles.
constexpr int tile_slots(int tiles) {
  return tiles <= 4 ? 4 : tiles <= 8 ? 8 : tiles <= 12 ? 12 : tiles <= 16 ? 16 : tiles <= 32 ? 32 : 64;
}

// Exact int32 scores of one 32-key tile (kt) of the staged int8 keys against one 32-query
// tile: acc[r] <-> key kt*32 + acc_row(r, lane), query lane % 32.
__device__ __forceinline__ i32x16 tile_raw_i8(const uint8_t *ks, const u32x4 *qf, int kt) {
  const int lane = threadIdx.x & 63;
  const uint8_t *arow = ks + (kt * 32 + (lane & 31)) * Tile<true>::Stride + 16 * (lane >> 5);
  i32x16 acc = {};
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = mfma_i8(*(const u32x4 *)(arow + 32 * s), qf[s], acc);
  return acc;
}

// Raw scores of one 32-key tile (kt) of the staged keys against one 32-query tile: bf16 dot
// products, or the int8 dot times the key scale (the query scale and sigma enter later).
template <bool I8>
__device__ __forceinline__ void tile_scores(const uint8_t *ks, const float *sk, const u32x4 *qf, int kt,
                                            float x[16]) {
  const int lane = threadIdx.x & 63;
  if (!I8) {
    const uint8_t *arow = ks + (kt * 32 + (lane & 31)) * Tile<I8>::Stride + 16 * (lane >> 5);
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < 8; ++s) acc = mfma_bf16(*(const u32x4 *)(arow + 32 * s), qf[s], acc);
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = acc[r];
  } else {
    const i32x16 acc = tile_raw_i8(ks, qf, kt);
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = (float)acc[r] * sk[kt * 32 + acc_row(r, lane)];
  }
}

// One staging unit: KS = min(b, 128) keys of one block, rows padded to Tile::Stride bytes.
template <int B, bool I8> struct Unit {
  static constexpr int KS = B < 128 ? B : 128;
  static constexpr int UPB = B / KS;                           // units per block
  static constexpr int Slots = Tile<I8>::Stride / 16;          // 17 (bf16) or 9 (int8) per row
  static constexpr int RowSlots = Tile<I8>::RowBytes / 16;     // 16 or 8
  static constexpr int Loads = KS * Slots / 64;                // 1 KiB direct loads per unit
  static constexpr int Bytes = KS * Tile<I8>::Stride;
  static_assert(KS * Slots % 64 == 0, "a unit is whole 1 KiB spans");
};

// This wave's share of the direct loads of unit `sub` of key block j of KV head g: LDS row r
// holds key row0 + r, its pad slot a copy of the row's last 16 bytes; int8 adds one load of the
// unit's key scales (lanes past KS / 4 repeat the last four).
template <int B, int NT, bool I8>
__device__ __forceinline__ void unit_issue(const StreamArgs &a, int g, int j, int sub, uint32_t kb, uint32_t sb,
                                           int wave) {
  using U = Unit<B, I8>;
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63;
  const size_t row0 = (size_t)g * a.S + (size_t)j * B + (size_t)sub * U::KS;
  const uint8_t *src = a.K + row0 * Tile<I8>::RowBytes;
  for (int u = wave; u < U::Loads; u += NW) {
    const int s = 64 * u + lane, row = s / U::Slots, c = min(s - row * U::Slots, U::RowSlots - 1);
    lds_dma16(src + row * Tile<I8>::RowBytes + 16 * c, kb + 1024 * u);
  }
  if (I8 && wave == NW - 1) lds_dma16(a.sK + row0 + min(4 * lane, U::KS - 4), sb);
}

// Column sums of the staged unit (for the block means), into cs: thread t covers the 16-byte column
// chunk t % CPR of rows t / CPR, t / CPR + NT / CPR, ... (bf16: 8 columns, int8: 16 columns scaled by
// the key scales).
template <int B, int NT, bool I8>
__device__ __forceinline__ void unit_colsum(const uint8_t *ks, const float *sk, float *cs) {
  using U = Unit<B, I8>;
  constexpr int CPR = U::RowSlots, EPC = I8 ? 16 : 8, RSTEP = NT / CPR;
  const int ch = threadIdx.x % CPR;
  for (int r = threadIdx.x / CPR; r < U::KS; r += RSTEP) {
    const u32x4 v = *(const u32x4 *)(ks + r * Tile<I8>::Stride + 16 * ch);
    if (!I8) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        cs[2 * e] += bf16lo(v[e]);
        cs[2 * e + 1] += bf16hi(v[e]);
      }
    } else {
      const float s = sk[r];
#pragma unroll
      for (int e = 0; e < EPC; ++e) cs[e] += s * (float)(int8_t)((v[e >> 2] >> (8 * (e & 3))) & 0xffu);
    }
  }
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// bf16 key-block sums on the matrix cores: O^T = K^T 1 for one 32-column slice, 16 keys per
// product.  The A operand (lane l: column l % 32, eight keys) comes from two LDS transpose reads
// (ds_read_b64_tr_b16): in each 16-lane block, lane j addresses key row j / 4 (+ 4 for the upper
// half-wave, + 8 for the second read) and columns 4 (j % 4) .. + 3 of its 16-column half, so the
// block receives 16 columns x 4 keys.  Which eight keys a lane holds does not matter against a B
// operand of ones, only that the 16 keys of a step are each held once.
template <int Stride>
__device__ __forceinline__ void ksum_step(uint32_t addr, f32x16 &acc) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(size_t)addr);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(size_t)(addr + 8 * Stride));
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
  const u32x4 ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
  acc = mfma_bf16(u32x4{l2[0], l2[1], h2[0], h2[1]}, ones, acc);
}

template <int B, int NT, int TPW, bool I8>
__global__ void __launch_bounds__(NT) k_ig_stream(StreamArgs a) {
  using U = Unit<B, I8>;
  constexpr int QT = B / 32, NW = NT / 64, NTL = NW * TPW, KTU = U::KS / 32;
  constexpr int CB = chunk_blocks(B, NTL);
  constexpr int CPR = U::RowSlots, EPC = I8 ? 16 : 8;
  static_assert(NT % CPR == 0 && 64 % CPR == 0, "a column chunk per lane");
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf[2][U::Bytes];
  __shared__ __attribute__((aligned(16))) float skb[2][I8 ? 256 : 4];
  __shared__ float part[NTL][CB][64];        // (lo, hi) per row of each tile slot and block of the chunk
  __shared__ float kpart[I8 ? 2 : 1][I8 ? NW : 1][128];   // int8: per-wave column sums of a block (by parity)
  if (a.status && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) a.status[0] = 0;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = blockIdx.y, G = a.G, S = a.S, N = a.N;
  const int ntiles = G * QT;
  const int c_begin = blockIdx.x * a.cpw, c_end = min(a.nch, c_begin + a.cpw);
  if (c_begin >= c_end) return;
  const int jb = c_begin * CB, je = min(N, c_end * CB);
  const int nunits = (je - jb) * U::UPB;

  // Q fragments of this wave's tiles (rows of the last query block)
  u32x4 qf[TPW][Tile<I8>::KS];
  float qscale[TPW], mref[TPW], lsum[TPW], lo_acc[TPW], hi_acc[TPW];
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
    lo_acc[u] = 0.0f;
    hi_acc[u] = 0.0f;
  }
  float cs[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) cs[e] = 0.0f;
  f32x16 ksum = {};                          // bf16: waves 0..3, column slice 32 * wave of the block sums
  static_assert(I8 || NW >= 4, "four waves sum the bf16 key blocks");

  unit_issue<B, NT, I8>(a, g, jb, 0, lds_addr(kbuf[0]), lds_addr(skb[0]), wave);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);     // the Q fragments and the first unit
  __syncthreads();

  for (int q = 0; q < nunits; ++q) {
    const int buf = q & 1;
    const int j = jb + q / U::UPB, sub = q % U::UPB;
    if (q + 1 < nunits)
      unit_issue<B, NT, I8>(a, g, jb + (q + 1) / U::UPB, (q + 1) % U::UPB, lds_addr(kbuf[buf ^ 1]),
                            lds_addr(skb[buf ^ 1]), wave);
    const uint8_t *ks = kbuf[buf];
    const float *sk = skb[buf];
    if constexpr (I8) {
      unit_colsum<B, NT, I8>(ks, sk, cs);
    } else if (wave < 4) {
      const uint32_t kaddr = lds_addr(ks) + (4 * (lane >> 5) + ((lane & 15) >> 2)) * Tile<false>::Stride +
                             2 * (32 * wave + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));
#pragma unroll
      for (int k0 = 0; k0 < U::KS; k0 += 16) ksum_step<Tile<false>::Stride>(kaddr + k0 * Tile<false>::Stride, ksum);
    }
    const bool diag = (j == N - 1);
    const int bc = (j - jb) % CB;            // block index within its chunk
    const bool block_end = sub == U::UPB - 1;

#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int t = wave * TPW + u;
      if (t >= ntiles) continue;
      float *prow = part[wave * TPW + u][0];
      const int tq = t % QT;                  // this tile's rows are tq*32 .. tq*32+31
      bool piped = false;
      if constexpr (TPW == 1 && B == 128) {
        if (!diag) {
          // Software-pipelined form for every block but the last (one 128-key unit per block):
          // the wave visits its key tiles in the order tq + 1, tq + 2, ... (mod 4), so the one
          // tile whose keys fall on both sides of the query rows (kt == tq) comes last, and the
          // products of the next tile are issued between the exponentials of the current one.
          // The tile loop has no branch: the new reference maximum is chosen by a select and the
          // running sums are rescaled every tile (by exactly 1 where the maximum stays); the sums
          // stored for earlier blocks of the chunk are rescaled once, after the loop.
          piped = true;
          const float m_start = mref[u];
          auto tile = [&](int kt) {
            float x[16];
            tile_scores<I8>(ks, sk, qf[u], kt, x);
            f32x16 r;
#pragma unroll
            for (int e = 0; e < 16; ++e) r[e] = x[e];
            return r;
          };
          f32x16 nx = tile((tq + 1) % QT);
#pragma unroll
          for (int pos = 0; pos < QT; ++pos) {
            const int kt = (tq + 1 + pos) % QT;
            const f32x16 x = nx;
            if (pos + 1 < QT) nx = tile((tq + 2 + pos) % QT);
            const float qs = qscale[u];
            // the tile's sums against the current reference maximum, without a maximum pass: a
            // score above the reference by more than the headroom makes its half-row sum exceed
            // 2^headroom (or overflow to infinity), which sends the wave to the rare path below
            auto sums = [&](float mneg, float &elo, float &ehi) {
              elo = 0.0f;
              ehi = 0.0f;
              if (pos + 1 < QT) {
                // all keys of the tile lie on one side of the wave's query rows; four partial sums
                // (a shorter dependency chain), combined in a fixed order
                float e4[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) e4[q] = fast_exp2(fmaf(x[q], qs, mneg));
#pragma unroll
                for (int r = 4; r < 16; ++r) e4[r & 3] += fast_exp2(fmaf(x[r], qs, mneg));
                const float e = (e4[0] + e4[1]) + (e4[2] + e4[3]);
                (kt < tq ? elo : ehi) = e;
              } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                  const float e = fast_exp2(fmaf(x[r], qs, mneg));
                  if (kt * 32 + acc_row(r, lane) <= qrow[u]) elo += e;
                  else ehi += e;
                }
              }
            };
            float elo, ehi;
            sums(-mref[u], elo, ehi);
            if (__any(!(elo + ehi <= kHeadroomScale))) {
              float mx = fmaxf(x[0], x[1]);
#pragma unroll
              for (int r = 2; r < 16; ++r) mx = fmaxf(mx, x[r]);
              mx = fmaxf(mx, xor32(mx)) * qs;
              const bool grow = mx > mref[u] + kHeadroom;
              if (__any(grow)) {
                const float mnew = grow ? mx : mref[u];
                const float alpha = fast_exp2(mref[u] - mnew);   // exactly 1 where the maximum stays
                lo_acc[u] *= alpha;
                hi_acc[u] *= alpha;
                lsum[u] *= alpha;
                mref[u] = mnew;
                sums(-mnew, elo, ehi);
              }
            }
            lo_acc[u] += elo;
            hi_acc[u] += ehi;
            // the tile's sums are needed here (an empty use), so they stay with the next tile's
            // products instead of sinking below the rescale after the loop
            asm volatile("" ::"v"(lo_acc[u]), "v"(hi_acc[u]));
            if (pos + 1 < QT && !I8) {
              // interleave: the next tile's products, one operand read ahead, each followed by a
              // share of this tile's vector work
              __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
              for (int g8 = 0; g8 < 8; ++g8) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
              }
            }
          }
          const bool moved = mref[u] != m_start;
          if (__any(moved)) {
            const float ab = fast_exp2(m_start - mref[u]);
            if (moved && lane < 32)
              for (int p = 0; p < bc; ++p) {
                prow[p * 64 + 2 * lane] *= ab;
                prow[p * 64 + 2 * lane + 1] *= ab;
              }
          }
        }
      }
      for (int ktl = 0; ktl < (piped ? 0 : KTU); ++ktl) {
        const int kt = sub * KTU + ktl;       // key tile within the block
        if (diag && kt > tq) break;           // keys after every query row of the tile
        float x[16];
        tile_scores<I8>(ks, sk, qf[u], ktl, x);
        const bool split = (kt == tq);        // the only key tile holding both c <= r and c > r
        float mx;
        if (split && diag) {
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
          const float alpha = fast_exp2(mref[u] - mnew);   // exactly 1 where the maximum stays
          lo_acc[u] *= alpha;
          hi_acc[u] *= alpha;
          lsum[u] *= alpha;
          if (grow && lane < 32)
            for (int p = 0; p < bc; ++p) {
              prow[p * 64 + 2 * lane] *= alpha;
              prow[p * 64 + 2 * lane + 1] *= alpha;
            }
          mref[u] = mnew;
        }
        const float qs = qscale[u], mneg = -mref[u];
        if (!split) {
          float e = 0.0f;
#pragma unroll
          for (int r = 0; r < 16; ++r) e += fast_exp2(fmaf(x[r], qs, mneg));
          if (kt < tq) lo_acc[u] += e;
          else hi_acc[u] += e;
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float e = fast_exp2(fmaf(x[r], qs, mneg));
            if (kt * 32 + acc_row(r, lane) <= qrow[u]) lo_acc[u] += e;
            else if (!diag) hi_acc[u] += e;
          }
        }
      }
      if (block_end) {
        const float lo = lo_acc[u] + xor32(lo_acc[u]), hi = hi_acc[u] + xor32(hi_acc[u]);
        lsum[u] += lo + hi;
        if (lane < 32) {
          prow[bc * 64 + 2 * lane] = lo;
          prow[bc * 64 + 2 * lane + 1] = hi;
        }
        lo_acc[u] = 0.0f;
        hi_acc[u] = 0.0f;
      }
    }
    if (!I8 && block_end && wave < 4) {
      // lanes 0 and 32 hold the block's column sums of this wave's slice (every column of O^T is the same)
      if ((lane & 31) == 0) {
        float *dst = a.kbar + ((size_t)g * N + j) * 128 + 32 * wave + 4 * (lane >> 5);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *(f32x4 *)(dst + 8 * q) = f32x4{ksum[4 * q] / B, ksum[4 * q + 1] / B, ksum[4 * q + 2] / B, ksum[4 * q + 3] / B};
      }
      ksum = f32x16{};
    }
    if constexpr (I8) {
      if (block_end) {
      // the block's column sums: lanes l, l + CPR, ... of a wave share a column chunk
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        if (CPR == 8)
          cs[e] += __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(cs[e]), __float_as_int(cs[e]), 0x128, 0xF, 0xF, true));
        cs[e] += bfly<4>(cs[e]);
        cs[e] += bfly<5>(cs[e]);
      }
      if (lane < CPR) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) kpart[(j - jb) & 1][wave][EPC * lane + e] = cs[e];
      }
#pragma unroll
      for (int e = 0; e < EPC; ++e) cs[e] = 0.0f;
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);    // this wave's loads of the next unit
    __syncthreads();                        // publishes the next unit and this block's column sums
    if (block_end) {
      if constexpr (I8) {
        if (threadIdx.x < 128) {
          float sm = 0.0f;
          for (int w = 0; w < NW; ++w) sm += kpart[(j - jb) & 1][w][threadIdx.x];
          a.kbar[((size_t)g * N + j) * 128 + threadIdx.x] = sm / (float)B;
        }
      }
      if (bc == CB - 1 || j == je - 1) {
        // the chunk's end: every row's (lo, hi) per block and its (m, sum), against the chunk's m
        const int c = (j - jb) / CB + c_begin, j0 = c * CB;
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
          const int t = wave * TPW + u;
          if (t >= ntiles || lane >= 32) continue;
          const int h = g * G + t / QT;
          const float *prow = part[wave * TPW + u][0];
          for (int p = 0; p <= bc; ++p)
            a.lohi[((size_t)h * N + j0 + p) * B + qrow[u]] = make_float2(prow[p * 64 + 2 * lane], prow[p * 64 + 2 * lane + 1]);
          a.ml[((size_t)h * a.nch + c) * B + qrow[u]] = make_float2(mref[u], lsum[u]);
        }
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
          mref[u] = -1e30f;
          lsum[u] = 0.0f;
        }
      }
    }
  }
}

// The merge, in two kernels.  k_ig_rows: for every row of every head its (M, 1 / (b L)) from the
// row's chunk pairs -- four threads per row, each an online merge of every fourth chunk in order,
// then the four merged in order -- and, in the workgroups past the rows, the column sums of every
// head's last query block (for the pooled estimate).  k_ig_merge: per head and range of key blocks,
//   lo[j] = sum_r lo_r[j] 2^(m_r,c(j) - M_r) / (b L_r),  hi likewise,
// and the pooled-estimate logits pe[j] = sigma * mean(Q_last) . kbar_j.  Every sum runs in a fixed
// order, so the results are reproducible.
struct MergeArgs {
  const uint8_t *Q;
  const float *sQ;
  const float2 *lohi, *ml;
  const float *kbar;
  float2 *rowml;      // [Hq][B] (M, 1 / (b L))
  float *qlast;       // [Hq][128] column sums of the last query block
  float *lo, *hi, *pe;
  int S, N, G, Hq, CB, nch;
  float sigma;
};
constexpr int kMergeThreads = 256;
constexpr int kMergeBlocks = 16;      // key blocks per k_ig_merge workgroup: four per wave
constexpr int kRowSplit = 4;          // threads per row in k_ig_rows

template <int B, bool I8>
__global__ void __launch_bounds__(kMergeThreads) k_ig_rows(MergeArgs a) {
  constexpr int ROWS = kMergeThreads / kRowSplit;          // rows per workgroup
  const int tid = threadIdx.x;
  const int nrow_wg = (a.Hq * B + ROWS - 1) / ROWS;
  if ((int)blockIdx.x < nrow_wg) {
    const int row = blockIdx.x * ROWS + tid / kRowSplit, part = tid % kRowSplit;
    float M = -3.0e38f, L = 0.0f;
    if (row < a.Hq * B) {
      const int h = row / B, r = row % B;
      const float2 *p = a.ml + (size_t)h * a.nch * B + r;
      // (loads of up to 32 chunk pairs in flight: 8.3 -> 6.3 us at 128K against 4)
#pragma unroll 32
      for (int c = part; c < a.nch; c += kRowSplit) {
        const float2 v = p[(size_t)c * B];
        const float Mn = fmaxf(M, v.x);
        L = L * exp2f(M - Mn) + v.y * exp2f(v.x - Mn);
        M = Mn;
      }
    }
    // the four partial merges of a row sit in consecutive lanes: combine them in order
#pragma unroll
    for (int k = 1; k < kRowSplit; ++k) {
      const float Mo = __shfl(M, (tid & ~(kRowSplit - 1)) + k), Lo = __shfl(L, (tid & ~(kRowSplit - 1)) + k);
      if (part == 0) {
        const float Mn = fmaxf(M, Mo);
        L = L * exp2f(M - Mn) + Lo * exp2f(Mo - Mn);
        M = Mn;
      }
    }
    if (part == 0 && row < a.Hq * B) a.rowml[row] = make_float2(M, 1.0f / ((float)B * L));
  } else {
    // column sums of the last query block of head h: column tid % 128, rows in two halves
    __shared__ float qs[128];
    const int h = blockIdx.x - nrow_wg, col = tid & 127, half = tid >> 7;
    const size_t tok0 = (size_t)h * a.S + (a.S - B);
    float sm = 0.0f;
    for (int r = half * (B / 2); r < (half + 1) * (B / 2); ++r) {
      if (!I8) sm += bf16_to_f32(((const uint16_t *)a.Q)[(tok0 + r) * 128 + col]);
      else sm += a.sQ[tok0 + r] * (float)((const int8_t *)a.Q)[(tok0 + r) * 128 + col];
    }
    if (half == 1) qs[col] = sm;
    __syncthreads();
    if (half == 0) a.qlast[(size_t)h * 128 + col] = (sm + qs[col]) / (float)B;
  }
}

template <int B, bool I8>
__global__ void __launch_bounds__(kMergeThreads) k_ig_merge(MergeArgs a) {
  constexpr int NWV = kMergeThreads / 64;
  const int h = blockIdx.y, g = h / a.G, N = a.N, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j0 = blockIdx.x * kMergeBlocks, nb = min(kMergeBlocks, N - j0);
  const int c_lo = j0 / a.CB, c_hi = (j0 + nb - 1) / a.CB;
  __shared__ float w[kMergeBlocks][B];                   // weight of row r's sums in chunk c_lo + k
  // weights of the range's chunks
  for (int k = tid; k < (c_hi - c_lo + 1) * B; k += kMergeThreads) {
    const int c = c_lo + k / B, r = k % B;
    const float2 rm = a.rowml[(size_t)h * B + r];
    w[c - c_lo][r] = exp2f(a.ml[((size_t)h * a.nch + c) * B + r].x - rm.x) * rm.y;
  }
  __syncthreads();
  // block masses and pooled-estimate logits: one wave per block, each lane RPL consecutive rows
  // (one 16- or 8-byte load) and two columns of the block's K-bar row; the wave's four blocks
  // have all their loads in flight together
  constexpr int RPL = B / 64;
  static_assert(kMergeBlocks == 4 * NWV, "four blocks per wave");
  const float2 qv = *(const float2 *)(a.qlast + (size_t)h * 128 + 2 * lane);
  float lo[4], hi[4], dq[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    lo[q] = 0.0f;
    hi[q] = 0.0f;
    dq[q] = 0.0f;
    const int k = 4 * wave + q;
    if (k < nb) {
      const int j = j0 + k, c = j / a.CB - c_lo;
      const float2 *src = a.lohi + ((size_t)h * N + j) * B + RPL * lane;
      const float2 kv = *(const float2 *)(a.kbar + ((size_t)g * N + j) * 128 + 2 * lane);
#pragma unroll
      for (int e = 0; e < RPL; ++e) {
        const float2 v = src[e];
        const float wv = w[c][RPL * lane + e];
        lo[q] += v.x * wv;
        hi[q] += v.y * wv;
      }
      dq[q] = qv.x * kv.x + qv.y * kv.y;
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float sl = wave_sum(lo[q]), sh = wave_sum(hi[q]), d = wave_sum(dq[q]);
    const int k = 4 * wave + q;
    if (lane == 0 && k < nb) {
      a.lo[(size_t)h * N + j0 + k] = sl;
      a.hi[(size_t)h * N + j0 + k] = sh;
      a.pe[(size_t)h * N + j0 + k] = a.sigma * d;
    }
  }
}

template <int B, int NT, int TPW, bool I8>
hipError_t run_stream(const Plan &p, StreamArgs a, hipStream_t st) {
  // about one workgroup per compute unit in all, each a contiguous range of chunks of its group
  const int cus = cu_count();
  int wpg = std::max(1, (cus > 0 ? cus : 256) / p.Hkv);
  wpg = std::min(wpg, a.nch);
  a.cpw = (a.nch + wpg - 1) / wpg;
  wpg = (a.nch + a.cpw - 1) / a.cpw;
  hipLaunchKernelGGL((k_ig_stream<B, NT, TPW, I8>), dim3(wpg, p.Hkv), dim3(NT), 0, st, a);
  return hipGetLastError();
}

// Workgroup size by query tiles G * b / 32: one wave per tile up to 16 waves, else 2 or 4 tiles a wave.
template <int B, bool I8>
hipError_t dispatch_stream(const Plan &p, const StreamArgs &a, hipStream_t st) {
  const int tiles = p.G * B / 32;
  if (tiles <= 4) return run_stream<B, 256, 1, I8>(p, a, st);
  if (tiles <= 8) return run_stream<B, 512, 1, I8>(p, a, st);
  if (tiles <= 12) return run_stream<B, 768, 1, I8>(p, a, st);
  if (tiles <= 16) return run_stream<B, 1024, 1, I8>(p, a, st);
  if (tiles <= 32) return run_stream<B, 1024, 2, I8>(p, a, st);
  return run_stream<B, 1024, 4, I8>(p, a, st);
}

// Test hook: the int32 tile Q8[h, i*B + r] . K8[g, j*B + c] through the streaming kernel's own
// staging (direct loads into padded LDS rows, one unit of up to 128 keys at a time) and int8 tile
// code, at the workgroup size the kernel runs with for this shape; out[c * B + r].  The scale load
// of the staging reads bytes of K instead of key scales (in bounds, unused).
template <int B, int NT>
__global__ void __launch_bounds__(NT) k_probe_stats_i8(const uint8_t *Q, const uint8_t *K, int S, int h, int g,
                                                       int i, int j, int32_t *out) {
  using U = Unit<B, true>;
  __shared__ __attribute__((aligned(1024))) uint8_t ks[U::Bytes];
  __shared__ __attribute__((aligned(16))) float sk[256];
  StreamArgs a{};
  a.Q = Q;
  a.K = K;
  a.sK = (const float *)K;
  a.S = S;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int sub = 0; sub < U::UPB; ++sub) {
    __syncthreads();
    unit_issue<B, NT, true>(a, g, j, sub, lds_addr(ks), lds_addr(sk), wave);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    for (int qt = wave; qt < B / 32; qt += NT / 64) {
      const int qr = qt * 32 + (lane & 31);
      const uint8_t *qp = Q + ((size_t)h * S + (size_t)i * B + qr) * Tile<true>::RowBytes + 16 * (lane >> 5);
      u32x4 qf[Tile<true>::KS];
#pragma unroll
      for (int s = 0; s < Tile<true>::KS; ++s) qf[s] = *(const u32x4 *)(qp + 32 * s);
      for (int kt = 0; kt < U::KS / 32; ++kt) {
        const i32x16 acc = tile_raw_i8(ks, qf, kt);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          out[(size_t)(sub * U::KS + kt * 32 + acc_row(r, lane)) * B + qr] = acc[r];
      }
    }
  }
}

template <int B, int NT>
hipError_t probe1(const Plan &p, const int8_t *Q8, const int8_t *K8, int h, int i, int j, int32_t *out,
                  hipStream_t st) {
  hipLaunchKernelGGL((k_probe_stats_i8<B, NT>), dim3(1), dim3(NT), 0, st, (const uint8_t *)Q8,
                     (const uint8_t *)K8, p.S, h, h / p.G, i, j, out);
  return hipGetLastError();
}

template <int B>
hipError_t probe_b(const Plan &p, const int8_t *Q8, const int8_t *K8, int h, int i, int j, int32_t *out,
                   hipStream_t st) {
  const int tiles = p.G * B / 32;
  if (tiles <= 4) return probe1<B, 256>(p, Q8, K8, h, i, j, out, st);
  if (tiles <= 8) return probe1<B, 512>(p, Q8, K8, h, i, j, out, st);
  if (tiles <= 12) return probe1<B, 768>(p, Q8, K8, h, i, j, out, st);
  return probe1<B, 1024>(p, Q8, K8, h, i, j, out, st);
}

}  // namespace

int stats_chunks(int B, int G, int N) {
  const int cb = chunk_blocks(B, tile_slots(G * B / 32));
  return (N + cb - 1) / cb;
}

// A kernel's dynamic-LDS limit raised to at least `bytes` on the current device.  The runtime call
// is made only when the limit has to grow, so repeated launches of one shape do no host work for
// it (a batch of short sequences is bound by the host's launch rate).
hipError_t ensure_dyn_lds(const void *fn, size_t bytes) {
  static std::mutex mu;
  static std::map<std::pair<int, const void *>, size_t> set;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  size_t &cur = set[{dev, fn}];
  if (bytes <= cur) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) cur = bytes;
  return e;
}

// Resident workgroups per compute unit of a kernel launched with `threads` threads and no dynamic
// LDS, on the current device (queried once per kernel and device; 0 if the query fails).
int occupancy_per_cu(const void *fn, int threads) {
  static std::mutex mu;
  static std::map<std::pair<int, const void *>, int> seen;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  auto it = seen.find({dev, fn});
  if (it != seen.end()) return it->second;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, threads, 0) != hipSuccess) n = 0;
  seen[{dev, fn}] = n;
  return n;
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
                           const float *sK, const Work &w, hipStream_t st, int32_t *status) {
  StreamArgs a;
  a.status = status;
  a.Q = (const uint8_t *)Q;
  a.sQ = sQ;
  a.K = (const uint8_t *)K;
  a.sK = sK;
  a.S = p.S; a.N = p.N; a.G = p.G;
  const int cb = chunk_blocks(p.B, tile_slots(p.G * p.B / 32));
  a.nch = (p.N + cb - 1) / cb;
  a.cpw = a.nch;
  a.c2 = kLog2e / sqrtf((float)p.d);
  a.lohi = w.lohi;
  a.ml = w.ml;
  a.kbar = w.kbar;
  hipError_t e;
  if (p.B == 64) e = i8 ? dispatch_stream<64, true>(p, a, st) : dispatch_stream<64, false>(p, a, st);
  else if (p.B == 128) e = i8 ? dispatch_stream<128, true>(p, a, st) : dispatch_stream<128, false>(p, a, st);
  else e = i8 ? dispatch_stream<256, true>(p, a, st) : dispatch_stream<256, false>(p, a, st);
  if (e != hipSuccess) return e;
  MergeArgs m;
  m.Q = (const uint8_t *)Q;
  m.sQ = sQ;
  m.lohi = w.lohi;
  m.ml = w.ml;
  m.kbar = w.kbar;
  m.rowml = w.rowml;
  m.qlast = w.qlast;
  m.lo = w.lo;
  m.hi = w.hi;
  m.pe = w.pe;
  m.S = p.S; m.N = p.N; m.G = p.G; m.Hq = p.Hq; m.CB = cb; m.nch = a.nch;
  m.sigma = 1.0f / sqrtf((float)p.d);
  const int rows_wg = (p.Hq * p.B + kMergeThreads / kRowSplit - 1) / (kMergeThreads / kRowSplit);
  const dim3 g1(rows_wg + p.Hq), g2((p.N + kMergeBlocks - 1) / kMergeBlocks, p.Hq), blk(kMergeThreads);
  if (p.B == 64) {
    if (i8) { hipLaunchKernelGGL((k_ig_rows<64, true>), g1, blk, 0, st, m); hipLaunchKernelGGL((k_ig_merge<64, true>), g2, blk, 0, st, m); }
    else { hipLaunchKernelGGL((k_ig_rows<64, false>), g1, blk, 0, st, m); hipLaunchKernelGGL((k_ig_merge<64, false>), g2, blk, 0, st, m); }
  } else if (p.B == 128) {
    if (i8) { hipLaunchKernelGGL((k_ig_rows<128, true>), g1, blk, 0, st, m); hipLaunchKernelGGL((k_ig_merge<128, true>), g2, blk, 0, st, m); }
    else { hipLaunchKernelGGL((k_ig_rows<128, false>), g1, blk, 0, st, m); hipLaunchKernelGGL((k_ig_merge<128, false>), g2, blk, 0, st, m); }
  } else {
    if (i8) { hipLaunchKernelGGL((k_ig_rows<256, true>), g1, blk, 0, st, m); hipLaunchKernelGGL((k_ig_merge<256, true>), g2, blk, 0, st, m); }
    else { hipLaunchKernelGGL((k_ig_rows<256, false>), g1, blk, 0, st, m); hipLaunchKernelGGL((k_ig_merge<256, false>), g2, blk, 0, st, m); }
  }
  return hipGetLastError();
}

// The workgroup size follows dispatch_stream (tiles = G * b / 32).
hipError_t launch_probe_stats_i8(const Plan &p, const int8_t *Q8, const int8_t *K8, int h, int i, int j,
                                 int32_t *out, hipStream_t st) {
  if (p.B == 64) return probe_b<64>(p, Q8, K8, h, i, j, out, st);
  if (p.B == 128) return probe_b<128>(p, Q8, K8, h, i, j, out, st);
  return probe_b<256>(p, Q8, K8, h, i, j, out, st);
}

}  // namespace fp
