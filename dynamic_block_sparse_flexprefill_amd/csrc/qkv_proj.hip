// QKV projection with the index stage's pooling and the W8A8 quantisation fused into its epilogue.
//
// The explainer ("FPGA24成果：FAST-Prefill稀疏注意力加速器", yunpan.plus) section 1.1 derives
// Q, K and V from the input by three projections; section 3.1 credits one fused streaming
// pipeline for avoiding intermediate traffic; sections 3.3 and 4.2 quantise the activations to
// int8 (W8A8).  Here one GEMM Y = X W^T (X: [S, D] bf16, W: [(Hq + 2 Hkv) * 128, D] bf16, rows
// grouped as the Q heads, then the K heads, then the V heads) produces every head's [S, 128]
// slice, and the epilogue of each 128-token x 128-column tile -- one head's share of one (or two,
// for 64-token blocks) key blocks -- does everything later stages would otherwise read the output
// back for:
//   * rotary position embedding on Q and K (rotate-half pairs (c, c + 64), caller's cos / sin),
//   * rounding to bf16 and the head-major store [H, S, 128],
//   * the block means of the rounded values (q-bar, k-bar: the pooled vectors of the pattern test
//     and of the query-aware rows, explainer section 1.2),
//   * optionally the symmetric per-(head, token) int8 codes and fp32 scales of the rounded values.
//
// Tiling: a workgroup of 8 waves computes one 256-token x 256-column output tile (two heads) on
// the 32x32x16 bf16 matrix cores, 128 x 64 per wave, with the K dimension streamed through LDS 64
// at a time in two stages: the next stage arrives by direct-to-LDS loads (global_load_lds_dwordx4,
// no registers) while the current one is multiplied.  Staged rows are 144 bytes (the pad slot
// repeats the row's last 16 bytes), so the 32 rows one operand read covers fall in distinct bank
// groups.  The epilogue then runs on the four 128 x 128 sub-tiles (one head, 128 tokens), two at
// a time through LDS as fp32.
#include "fp_common.hpp"
#include "fp_internal.hpp"

namespace fp {
namespace {

struct ProjArgs {
  const uint8_t *X, *W;          // bf16 [S, D], [n_out, D]
  const float *cosT, *sinT;      // [S, 64] or null (no rotation)
  uint16_t *Q, *K, *V;           // bf16 [H, S, 128]
  float *qbar, *kbar;            // [Hq, S / b, 128], [Hkv, S / b, 128] or null
  int8_t *Q8, *K8, *V8;          // int8 [H, S, 128] or null
  float *sQ, *sK, *sV;           // fp32 [H, S]
  int S, D, Hq, Hkv, b;
};

constexpr int kBK = 64;                          // K values per LDS stage
constexpr int kSlots = 9;                        // 16-byte slots per staged row (the ninth repeats the eighth)
constexpr int kRowB = kSlots * 16;               // 144 B
constexpr int kTM = 256, kTN = 256;              // workgroup tile: tokens x output columns
constexpr int kStage = (kTM + kTN) * kRowB;      // 73728 B
constexpr int kLoadsA = kTM * kSlots / 64;       // 36 one-KiB direct loads of X per stage
constexpr int kLoads = (kTM + kTN) * kSlots / 64;   // 72 (9 per wave)
constexpr int kThreads = 512;
constexpr int kTileRow = 132;                    // fp32 per row of an epilogue sub-tile
static_assert(kLoads % (kThreads / 64) == 0, "the same number of loads per wave");
static_assert(2 * 128 * kTileRow * 4 + 2 * 1024 * 4 <= 2 * kStage, "two epilogue sub-tiles and their column sums fit");

// Epilogue of one 128-token x 128-column sub-tile (token tile it, column tile = head ct) held as
// fp32 in LDS, by 256 threads t.  Sixteen threads share a token row, 8 columns each, so that every
// store instruction of a wave covers four consecutive rows of the head-major output (1 KiB of bf16,
// 512 B of int8): rotary (the partner column c +- 64 read from the tile), bf16 rounding and store,
// the int8 codes and scale of the rounded row (its maximum over the 16 threads), and the column sums
// of the rounded values of rows 0-63 and 64-127, reduced over the wave's four rows and left in
// red[wave of the sub-tile][half][column] for the block means.  No barrier inside.
__device__ void epi_tile(const ProjArgs &a, const float *tile, int it, int ct, int t, float *red) {
  const int S = a.S, Hq = a.Hq, Hkv = a.Hkv;
  const int kind = ct < Hq ? 0 : (ct < Hq + Hkv ? 1 : 2);   // Q, K or V head
  const int head = kind == 0 ? ct : (kind == 1 ? ct - Hq : ct - Hq - Hkv);
  uint16_t *dst = kind == 0 ? a.Q : (kind == 1 ? a.K : a.V);
  int8_t *dst8 = kind == 0 ? a.Q8 : (kind == 1 ? a.K8 : a.V8);
  float *dsts = kind == 0 ? a.sQ : (kind == 1 ? a.sK : a.sV);
  const bool rope = kind < 2 && a.cosT;
  const int j = t & 15, rr = t >> 4, c0 = 8 * j, pc = 8 * (j ^ 8), rc = 8 * (j & 7);
  const bool upper = j >= 8;                  // columns 64..127: the second member of each pair
  float sum[2][8];
#pragma unroll
  for (int hlf = 0; hlf < 2; ++hlf)
#pragma unroll
    for (int e = 0; e < 8; ++e) sum[hlf][e] = 0.0f;
#pragma unroll 2
  for (int p = 0; p < 8; ++p) {
    const int row = 16 * p + rr, tok = it * 128 + row;
    const float *tr = tile + row * kTileRow;
    float v[8];
    {
      const float4 x0 = *(const float4 *)(tr + c0), x1 = *(const float4 *)(tr + c0 + 4);
      const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      if (rope) {
        const float4 y0 = *(const float4 *)(tr + pc), y1 = *(const float4 *)(tr + pc + 4);
        const float y[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
        const float4 k0 = *(const float4 *)(a.cosT + (size_t)tok * 64 + rc), k1 = *(const float4 *)(a.cosT + (size_t)tok * 64 + rc + 4);
        const float4 n0 = *(const float4 *)(a.sinT + (size_t)tok * 64 + rc), n1 = *(const float4 *)(a.sinT + (size_t)tok * 64 + rc + 4);
        const float cs[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
        const float sn[8] = {n0.x, n0.y, n0.z, n0.w, n1.x, n1.y, n1.z, n1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = upper ? x[e] * cs[e] + y[e] * sn[e] : x[e] * cs[e] - y[e] * sn[e];
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = x[e];
      }
    }
    uint32_t pk[4];
    float r[8], amax = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      pk[q] = pack_bf16x2(v[2 * q], v[2 * q + 1]);
      r[2 * q] = bf16lo(pk[q]);
      r[2 * q + 1] = bf16hi(pk[q]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sum[p >> 2][e] += r[e];
      amax = fmaxf(amax, fabsf(r[e]));
    }
    *(u32x4 *)(dst + ((size_t)head * S + tok) * 128 + c0) = u32x4{pk[0], pk[1], pk[2], pk[3]};
    if (dst8) {
      // symmetric per-(head, token) int8 of the rounded row: s = max|x| / 127 (1 for a zero row),
      // codes rint(x / s) clamped to +-127, all in fp32 with IEEE division
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
      const float sc = amax > 0.0f ? amax / 127.0f : 1.0f;
      uint32_t w8[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float c = fminf(fmaxf(rintf(r[e] / sc), -127.0f), 127.0f);
        w8[e >> 2] |= ((uint32_t)(int)c & 0xffu) << (8 * (e & 3));
      }
      *(u32x2 *)(dst8 + ((size_t)head * S + tok) * 128 + c0) = u32x2{w8[0], w8[1]};
      if (j == 0) dsts[(size_t)head * S + tok] = sc;
    }
  }
  // column sums over this wave's four row groups (lanes l, l ^ 16, l ^ 32, l ^ 48), in a fixed order
#pragma unroll
  for (int hlf = 0; hlf < 2; ++hlf)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sum[hlf][e] += __shfl_xor(sum[hlf][e], 16);
      sum[hlf][e] += __shfl_xor(sum[hlf][e], 32);
    }
  if ((t & 63) < 16) {
    float *rw = red + (t >> 6) * 256;
#pragma unroll
    for (int hlf = 0; hlf < 2; ++hlf)
#pragma unroll
      for (int e = 0; e < 8; ++e) rw[hlf * 128 + c0 + e] = sum[hlf][e];
  }
}

__global__ void __launch_bounds__(kThreads) k_qkv_proj(ProjArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t sm[2 * kStage];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int D = a.D, S = a.S, nc = a.Hq + 2 * a.Hkv;
  // Tile order: column tiles (two heads) in bands of 4; within a band the workgroups that share a
  // token tile (its 1.5 MiB of X at D = 3072) run back to back on one XCD, so X is read from HBM
  // about once per band instead of once per column tile.  Workgroup ids reach the XCDs round robin
  // (id mod 8); with a token-tile count that is not a multiple of 8 the band is simply walked token
  // tile by token tile.
  int it, ctl;
  {
    const int nt = (S + kTM - 1) / kTM, nct = (nc + 1) / 2, per_band = nt * 4;
    const int id = blockIdx.x, nfull = nct / 4;
    int band, r, w;
    if (id < nfull * per_band) {
      band = id / per_band;
      r = id - band * per_band;
      w = 4;
    } else {
      band = nfull;
      r = id - nfull * per_band;
      w = nct - 4 * nfull;
    }
    int cl;
    if (nt % 8 == 0) {
      const int j = r >> 3, x = r & 7;
      it = 8 * (j / w) + x;
      cl = j % w;
    } else {
      it = r / w;
      cl = r % w;
    }
    ctl = 4 * band + cl;                      // token tile it (256 tokens), column tile ctl (heads 2 ctl, 2 ctl + 1)
  }
  const int wr = (wave & 1) * 128, wc = (wave >> 1) * 64;
  const uint32_t smb = lds_addr(sm);

  // this wave's 9 direct loads of stage st (K offset k0): X rows of the token tile, then W rows of
  // the column tile; rows past the ends (a 128-token last tile, an odd head count) repeat the last
  // row and are never stored
  auto issue = [&](int k0, int st) {
    for (int u = wave; u < kLoads; u += kThreads / 64) {
      const bool isa = u < kLoadsA;
      const int v = isa ? u : u - kLoadsA;
      const int sl = 64 * v + lane, row = sl / kSlots, c = min(sl - row * kSlots, 7);
      const uint8_t *src = isa ? a.X + ((size_t)min(it * kTM + row, S - 1) * D + k0 + 8 * c) * 2
                               : a.W + ((size_t)min(ctl * kTN + row, nc * 128 - 1) * D + k0 + 8 * c) * 2;
      lds_dma16(src, __builtin_amdgcn_readfirstlane(smb + st * kStage + (isa ? 0 : kTM * kRowB) + 1024 * v));
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = f32x16{};

  const int nk = D / kBK;
  issue(0, 0);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  const uint32_t ao = (wr + (lane & 31)) * kRowB + 16 * (lane >> 5);
  const uint32_t bo = kTM * kRowB + (wc + (lane & 31)) * kRowB + 16 * (lane >> 5);
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) issue((kt + 1) * kBK, st ^ 1);
    const uint8_t *base = sm + st * kStage;
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      u32x4 fa[4], fb[2];
#pragma unroll
      for (int m = 0; m < 4; ++m) fa[m] = *(const u32x4 *)(base + ao + m * 32 * kRowB + 32 * ks);
#pragma unroll
      for (int n = 0; n < 2; ++n) fb[n] = *(const u32x4 *)(base + bo + n * 32 * kRowB + 32 * ks);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = mfma_bf16(fa[mi], fb[ni], acc[mi][ni]);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);      // this wave's loads of the next stage
    __syncthreads();                          // every wave's, and no wave still reads this stage
  }

  // ---- epilogue, by token half th: the two 128 x 128 sub-tiles (one per head) to LDS as fp32
  // [token][column], written by the four waves whose rows they are; 256 threads per sub-tile
  float *tiles = (float *)sm;
  float *red = tiles + 2 * 128 * kTileRow;     // [sub-tile][4 waves][2 halves][128 columns]
  const int hs = tid >> 8, t = tid & 255;      // sub-tile (head 2 ctl + hs) of this thread
  for (int th = 0; th < 2; ++th) {
    if ((wave & 1) == th) {
      float *tl = tiles + (wc >> 7) * 128 * kTileRow;
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            tl[(32 * mi + acc_row(r, lane)) * kTileRow + (wc & 127) + 32 * ni + (lane & 31)] = acc[mi][ni][r];
    }
    __syncthreads();
    const int it128 = 2 * it + th, ct = 2 * ctl + hs;
    const bool valid = it128 < S / 128 && ct < nc;
    float *rd = red + hs * 1024;
    if (valid) epi_tile(a, tiles + hs * 128 * kTileRow, it128, ct, t, rd);
    __syncthreads();
    // block means of the rounded values (Q and K heads): the four waves' column sums in order
    const int kind = ct < a.Hq ? 0 : (ct < a.Hq + a.Hkv ? 1 : 2);
    const int head = kind == 0 ? ct : ct - a.Hq;
    float *bar = !valid ? nullptr : kind == 0 ? a.qbar : (kind == 1 ? a.kbar : nullptr);
    if (bar && t < 128) {
      float lo = 0.0f, hi = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        lo += rd[w * 256 + t];
        hi += rd[w * 256 + 128 + t];
      }
      const int nb = S / a.b;
      if (a.b == 64) {
        bar[((size_t)head * nb + 2 * it128) * 128 + t] = lo / 64.0f;
        bar[((size_t)head * nb + 2 * it128 + 1) * 128 + t] = hi / 64.0f;
      } else {
        bar[((size_t)head * nb + it128) * 128 + t] = (lo + hi) / 128.0f;
      }
    }
    __syncthreads();                          // before the next token half overwrites the sub-tiles
  }
}

}  // namespace

hipError_t launch_qkv_proj(int S, int D, int Hq, int Hkv, int b, const void *X, const void *W, const float *cosT,
                           const float *sinT, void *Q, void *K, void *V, float *qbar, float *kbar, int8_t *Q8,
                           float *sQ, int8_t *K8, float *sK, int8_t *V8, float *sV, hipStream_t st) {
  ProjArgs a;
  a.X = (const uint8_t *)X;
  a.W = (const uint8_t *)W;
  a.cosT = cosT;
  a.sinT = sinT;
  a.Q = (uint16_t *)Q;
  a.K = (uint16_t *)K;
  a.V = (uint16_t *)V;
  a.qbar = qbar;
  a.kbar = kbar;
  a.Q8 = Q8; a.K8 = K8; a.V8 = V8;
  a.sQ = sQ; a.sK = sK; a.sV = sV;
  a.S = S; a.D = D; a.Hq = Hq; a.Hkv = Hkv; a.b = b;
  const int nt = (S + kTM - 1) / kTM, nct = (Hq + 2 * Hkv + 1) / 2;
  hipLaunchKernelGGL(k_qkv_proj, dim3(nt * nct), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace fp
