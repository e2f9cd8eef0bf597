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
// Tiling: a workgroup of 4 waves computes one 128 x 128 output tile on the 32x32x16 bf16 matrix
// cores, 64 x 64 per wave, with the K dimension streamed through LDS 64 at a time in two stages
// (the next stage loaded into registers while the current one is multiplied).
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

constexpr int kBK = 64;               // K values per LDS stage
constexpr int kRow = kBK + 8;         // bf16 per padded LDS row (144 B: 16 consecutive rows hit distinct banks)
constexpr int kTileRow = 132;         // fp32 per row of the epilogue tile

__global__ void __launch_bounds__(256) k_qkv_proj(ProjArgs a) {
  // two stages of A (128 tokens) and B (128 output columns), reused as the fp32 epilogue tile
  __shared__ __attribute__((aligned(16))) uint16_t sm[2 * 2 * 128 * kRow];
  static_assert(sizeof(uint16_t) * 2 * 2 * 128 * kRow >= sizeof(float) * 128 * kTileRow, "epilogue tile fits");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int D = a.D, S = a.S;
  // Tile order: column tiles (heads) in bands of 8; within a band the workgroups that share a token
  // tile (its 786 KB of X at D = 3072) run back to back on one XCD, so X is read from HBM about
  // once per band instead of once per head.  Workgroup ids reach the XCDs round robin (id mod 8);
  // with S / 128 not a multiple of 8 the band is simply walked token tile by token tile.
  int it, ct;
  {
    const int nt = S / 128, nc = a.Hq + 2 * a.Hkv, per_band = nt * 8;
    const int id = blockIdx.x, nfull = nc / 8;
    int band, r, w;
    if (id < nfull * per_band) {
      band = id / per_band;
      r = id - band * per_band;
      w = 8;
    } else {
      band = nfull;
      r = id - nfull * per_band;
      w = nc - 8 * nfull;
    }
    int hl;
    if (nt % 8 == 0) {
      const int j = r >> 3, x = r & 7;
      it = 8 * (j / w) + x;
      hl = j % w;
    } else {
      it = r / w;
      hl = r % w;
    }
    ct = 8 * band + hl;                                      // token tile it, column tile (= head) ct
  }
  const int wr = (wave & 1) * 64, wc = (wave >> 1) * 64;
  const uint8_t *xg = a.X + (size_t)it * 128 * D * 2;
  const uint8_t *wg = a.W + (size_t)ct * 128 * D * 2;

  // global -> register staging: thread t holds 16-byte pieces t + 256 u (u < 4) of each operand
  u32x4 ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = tid + 256 * u, row = c >> 3, p = c & 7;
      ra[u] = *(const u32x4 *)(xg + ((size_t)row * D + k0 + 8 * p) * 2);
      rb[u] = *(const u32x4 *)(wg + ((size_t)row * D + k0 + 8 * p) * 2);
    }
  };
  auto sstore = [&](int st) {
    uint16_t *as = sm + st * 2 * 128 * kRow, *bs = as + 128 * kRow;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = tid + 256 * u, row = c >> 3, p = c & 7;
      *(u32x4 *)(as + row * kRow + 8 * p) = ra[u];
      *(u32x4 *)(bs + row * kRow + 8 * p) = rb[u];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = f32x16{};

  const int nk = D / kBK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * kBK);
    const uint16_t *as = sm + st * 2 * 128 * kRow, *bs = as + 128 * kRow;
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      u32x4 fa[2], fb[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        fa[m] = *(const u32x4 *)(as + (wr + 32 * m + (lane & 31)) * kRow + 16 * ks + 8 * (lane >> 5));
        fb[m] = *(const u32x4 *)(bs + (wc + 32 * m + (lane & 31)) * kRow + 16 * ks + 8 * (lane >> 5));
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = mfma_bf16(fa[mi], fb[ni], acc[mi][ni]);
    }
    if (kt + 1 < nk) sstore(st ^ 1);
    __syncthreads();
  }

  // ---- epilogue: the tile to LDS as fp32 [token][column]
  float *tile = (float *)sm;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        tile[(wr + 32 * mi + acc_row(r, lane)) * kTileRow + wc + 32 * ni + (lane & 31)] = acc[mi][ni][r];
  __syncthreads();

  const int Hq = a.Hq, Hkv = a.Hkv;
  const int kind = ct < Hq ? 0 : (ct < Hq + Hkv ? 1 : 2);   // Q, K or V head
  const int head = kind == 0 ? ct : (kind == 1 ? ct - Hq : ct - Hq - Hkv);
  uint16_t *dst = kind == 0 ? a.Q : (kind == 1 ? a.K : a.V);
  int8_t *dst8 = kind == 0 ? a.Q8 : (kind == 1 ? a.K8 : a.V8);
  float *dsts = kind == 0 ? a.sQ : (kind == 1 ? a.sK : a.sV);
  {
    // two threads per token: columns c and c + 64 for c in [32 h, 32 h + 32), h = tid & 1
    const int row = tid >> 1, h = tid & 1, tok = it * 128 + row;
    float *tr = tile + row * kTileRow;
    const bool rope = kind < 2 && a.cosT;
    uint32_t packed[32];
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 32; e += 2) {
      float v[2][2];     // [pair member][element]
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int c = 32 * h + e + q;
        const float x0 = tr[c], x1 = tr[c + 64];
        if (rope) {
          const float cs = a.cosT[(size_t)tok * 64 + c], sn = a.sinT[(size_t)tok * 64 + c];
          v[0][q] = x0 * cs - x1 * sn;
          v[1][q] = x1 * cs + x0 * sn;
        } else {
          v[0][q] = x0;
          v[1][q] = x1;
        }
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const uint32_t pw = pack_bf16x2(v[m][0], v[m][1]);
        packed[m * 16 + e / 2] = pw;
        const float r0 = bf16lo(pw), r1 = bf16hi(pw);
        tr[64 * m + 32 * h + e] = r0;           // the rounded values, for the means
        tr[64 * m + 32 * h + e + 1] = r1;
        amax = fmaxf(amax, fmaxf(fabsf(r0), fabsf(r1)));
      }
    }
    uint16_t *orow = dst + ((size_t)head * S + tok) * 128;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(u32x4 *)(orow + 64 * m + 32 * h + 8 * q) =
            u32x4{packed[m * 16 + 4 * q], packed[m * 16 + 4 * q + 1], packed[m * 16 + 4 * q + 2], packed[m * 16 + 4 * q + 3]};
    if (dst8) {
      // symmetric per-(head, token) int8 of the rounded row: s = max|x| / 127 (1 for a zero row),
      // codes rint(x / s) clamped to +-127, all in fp32 with IEEE division
      amax = fmaxf(amax, __shfl_xor(amax, 1));
      const float s = amax > 0.0f ? amax / 127.0f : 1.0f;
      int8_t *o8 = dst8 + ((size_t)head * S + tok) * 128;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        uint32_t w8[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          uint32_t word = 0u;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x = tr[64 * m + 32 * h + 4 * q + e];
            const float c = fminf(fmaxf(rintf(x / s), -127.0f), 127.0f);
            word |= ((uint32_t)(int)c & 0xffu) << (8 * e);
          }
          w8[q] = word;
        }
        *(u32x4 *)(o8 + 64 * m + 32 * h) = u32x4{w8[0], w8[1], w8[2], w8[3]};
        *(u32x4 *)(o8 + 64 * m + 32 * h + 16) = u32x4{w8[4], w8[5], w8[6], w8[7]};
      }
      if (h == 0) dsts[(size_t)head * S + tok] = s;
    }
  }
  __syncthreads();

  // block means of the rounded values (Q and K heads): column c, rows in order, 64 rows per thread
  float *bar = kind == 0 ? a.qbar : (kind == 1 ? a.kbar : nullptr);
  if (bar) {
    const int c = tid & 127, half = tid >> 7;
    float sum = 0.0f;
    for (int r = 64 * half; r < 64 * half + 64; ++r) sum += tile[r * kTileRow + c];
    const int nb = S / a.b;
    if (a.b == 64) {
      bar[((size_t)head * nb + 2 * it + half) * 128 + c] = sum / 64.0f;
    } else {
      float *part = tile;                                // the tile is no longer read past this barrier
      __syncthreads();
      if (half == 1) part[c] = sum;
      __syncthreads();
      if (half == 0) bar[((size_t)head * nb + it) * 128 + c] = (sum + part[c]) / 128.0f;
    }
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
  hipLaunchKernelGGL(k_qkv_proj, dim3((S / 128) * (Hq + 2 * Hkv)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace fp
