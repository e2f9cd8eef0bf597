// Block-sparse causal attention over a CSR of key blocks.
//
// The explainer ("FPGA24成果：FAST-Prefill稀疏注意力加速器", yunpan.plus)
// section 1.1 gives the attention softmax(Q K^T / sqrt(d_k)) V; section 1.2
// (figure 3) restricts each query block to the key/value blocks its sparse
// index names.  For query token t of block i and head h, the keys are those
// k <= t whose block is in J(h, i); the softmax runs over exactly those keys.
// The softmax is taken block by block with a running maximum (the re-telling
// "FPGA加速动态稀疏注意力技术解析与优化", section 3.3, normalises attention
// scores block-wise to avoid overflow).
//
// W8A8 (explainer sections 3.3 and 4.2): Q.K^T on the int8 matrix cores with
// int32 accumulation, scaled by sigma * sQ[t] * sK[k]; P.V in bf16 with the
// int8 values of V (exact in bf16) and sV folded into P.
//
// Kernel layout: one workgroup per CSR row (h, i), one wave per 32 queries.
// Each key block is staged in LDS once per workgroup: K row-major, V
// transposed.  Scores are computed transposed, S^T = K Q^T, on the 32x32
// matrix cores, so every lane owns one query row; its softmax weights are
// already in the operand layout of the next product O^T += V^T P^T.
#include "fp_common.hpp"
#include "fp_internal.hpp"

namespace fp {
namespace {

struct AttnArgs {
  const uint8_t *Q, *K, *V;
  const float *sQ, *sK, *sV;
  const int32_t *row_ptr, *col_idx;
  uint16_t *O;
  int S, N, Hq, G;
  float c2;
};

template <int B, bool I8> struct AttnLds {
  static constexpr int KStride = I8 ? 144 : 272;   // bytes per staged key row
  static constexpr int VStride = B + 4;             // bf16 elements per transposed V row
  static constexpr int KBytes = B * KStride;
  static constexpr int VBytes = 128 * VStride * 2;
};

// Stage key block j of KV head g: K rows (padded) and V transposed to [d][key] bf16.
template <int B, bool I8>
__device__ __forceinline__ void stage_kv(const uint8_t *K, const uint8_t *V, const float *sK,
                                         const float *sV, int S, int g, int j, uint8_t *ks,
                                         uint16_t *vt, float *sk, float *sv) {
  using L = AttnLds<B, I8>;
  constexpr int RB = I8 ? 128 : 256;                 // bytes per global row
  constexpr int CPR = RB / 16;
  const size_t row0 = (size_t)g * S + (size_t)j * B;
  const uint8_t *kb = K + row0 * RB;
  for (int c = threadIdx.x; c < B * CPR; c += blockDim.x) {
    const int r = c / CPR, col = c % CPR;
    *(u32x4 *)(ks + r * L::KStride + col * 16) = *(const u32x4 *)(kb + (size_t)r * RB + col * 16);
  }
  const uint8_t *vb = V + row0 * RB;
  uint32_t *vt32 = (uint32_t *)vt;
  for (int it = threadIdx.x; it < (B / 2) * CPR; it += blockDim.x) {
    const int dc = it % CPR, kp = it / CPR;
    const u32x4 a = *(const u32x4 *)(vb + (size_t)(2 * kp) * RB + dc * 16);
    const u32x4 b = *(const u32x4 *)(vb + (size_t)(2 * kp + 1) * RB + dc * 16);
    if (!I8) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t lo = (a[e >> 1] >> (16 * (e & 1))) & 0xffffu;
        const uint32_t hi = (b[e >> 1] >> (16 * (e & 1))) & 0xffffu;
        vt32[((dc * 8 + e) * L::VStride + 2 * kp) >> 1] = lo | (hi << 16);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float lo = (float)(int8_t)((a[e >> 2] >> (8 * (e & 3))) & 0xffu);
        const float hi = (float)(int8_t)((b[e >> 2] >> (8 * (e & 3))) & 0xffu);
        vt32[((dc * 16 + e) * L::VStride + 2 * kp) >> 1] = pack_bf16x2(lo, hi);
      }
    }
  }
  if (I8) {
    for (int r = threadIdx.x; r < B; r += blockDim.x) {
      sk[r] = sK[row0 + r];
      sv[r] = sV[row0 + r];
    }
  }
}

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

// Raw scores of key tile (32 keys starting at key0) against this wave's 32 queries.
template <bool I8>
__device__ __forceinline__ void raw_scores(const uint8_t *ks, int kstride, int key0,
                                           const u32x4 qf[8], f32x16 &accf, i32x16 &acci) {
  const int lane = threadIdx.x & 63;
  const uint8_t *arow = ks + (key0 + (lane & 31)) * kstride + 16 * (lane >> 5);
  if (!I8) {
    accf = f32x16{};
#pragma unroll
    for (int s = 0; s < 8; ++s) accf = mfma_bf16(*(const u32x4 *)(arow + 32 * s), qf[s], accf);
  } else {
    acci = i32x16{};
#pragma unroll
    for (int s = 0; s < 4; ++s) acci = mfma_i8(*(const u32x4 *)(arow + 32 * s), qf[s], acci);
  }
}

template <int B, bool I8>
__global__ void __launch_bounds__(2 * B) k_attn_rows(AttnArgs a) {
  using L = AttnLds<B, I8>;
  __shared__ __attribute__((aligned(16))) uint8_t ks[L::KBytes];
  __shared__ __attribute__((aligned(16))) uint16_t vt[128 * L::VStride];
  __shared__ float sk[I8 ? B : 1], sv[I8 ? B : 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, hf = lane >> 5;
  const int N = a.N, S = a.S;

  // Workgroup -> row, keeping consecutive rows (the heads of one query
  // block) on the same XCD: the hardware deals workgroups round-robin to 8.
  const int nblk = gridDim.x;
  int L8 = blockIdx.x;
  if ((nblk & 7) == 0) L8 = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
  const int i = N - 1 - L8 / a.Hq, h = L8 % a.Hq, g = h / a.G;
  const int row = h * N + i;
  const int qr = wave * 32 + (lane & 31);
  const size_t tok = (size_t)h * S + (size_t)i * B + qr;

  u32x4 qf[8];
  load_q<I8>(a.Q, tok, qf);
  const float qscale = I8 ? a.c2 * a.sQ[tok] : a.c2;

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
  float m = kNegBig, l = 0.0f;

  const int p0 = a.row_ptr[row], p1 = a.row_ptr[row + 1];
  for (int p = p0; p < p1; ++p) {
    const int j = a.col_idx[p];
    if (j < 0 || j >= N) continue;   // not a key block of this sequence (same for every thread)
    __syncthreads();
    stage_kv<B, I8>(a.K, a.V, a.sK, a.sV, S, g, j, ks, vt, sk, sv);
    __syncthreads();
    const int lim = qr + (i - j) * B;   // keys c > lim of this block are in the future
#pragma unroll 1
    for (int kc = 0; kc < B / 128; ++kc) {
      float x[4][16];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        f32x16 accf;
        i32x16 acci;
        raw_scores<I8>(ks, L::KStride, kc * 128 + kt * 32, qf, accf, acci);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = kc * 128 + kt * 32 + acc_row(r, lane);
          float v = I8 ? (float)acci[r] * qscale * sk[c] : accf[r] * qscale;
          x[kt][r] = (c > lim) ? kNegBig : v;
        }
      }
      float mx = kNegBig;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, x[kt][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mnew = fmaxf(m, mx);
      const float alpha = exp2f(m - mnew);
      float rs = 0.0f;
      u32x4 pf[4][2];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        float pv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = (x[kt][r] == kNegBig) ? 0.0f : exp2f(x[kt][r] - mnew);
          rs += e;
          pv[r] = I8 ? e * sv[kc * 128 + kt * 32 + acc_row(r, lane)] : e;
        }
#pragma unroll
        for (int s = 0; s < 2; ++s)
          pf[kt][s] = u32x4{pack_bf16x2(pv[8 * s + 0], pv[8 * s + 1]), pack_bf16x2(pv[8 * s + 2], pv[8 * s + 3]),
                            pack_bf16x2(pv[8 * s + 4], pv[8 * s + 5]), pack_bf16x2(pv[8 * s + 6], pv[8 * s + 7])};
      }
      rs += __shfl_xor(rs, 32, 64);
      l = l * alpha + rs;
      m = mnew;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const uint16_t *vrow = vt + (dt * 32 + (lane & 31)) * L::VStride + kc * 128 + 4 * hf;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const uint16_t *q = vrow + kt * 32 + 16 * s;
            const u32x2 v0 = *(const u32x2 *)q;
            const u32x2 v1 = *(const u32x2 *)(q + 8);
            o[dt] = mfma_bf16(u32x4{v0[0], v0[1], v1[0], v1[1]}, pf[kt][s], o[dt]);
          }
      }
    }
  }

  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  uint16_t *orow = a.O + tok * 128;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int d0 = dt * 32 + 8 * rq + 4 * hf;
      const u32x2 w = u32x2{pack_bf16x2(o[dt][4 * rq] * inv, o[dt][4 * rq + 1] * inv),
                            pack_bf16x2(o[dt][4 * rq + 2] * inv, o[dt][4 * rq + 3] * inv)};
      *(u32x2 *)(orow + d0) = w;
    }
}

// out[c * B + r] = Q8[h, i*B + r] . K8[g, j*B + c] through the int8 tile code.
template <int B>
__global__ void __launch_bounds__(2 * B) k_probe_qk_i8(const uint8_t *Q, const uint8_t *K, int S,
                                                       int h, int g, int i, int j, int32_t *out) {
  using L = AttnLds<B, true>;
  __shared__ __attribute__((aligned(16))) uint8_t ks[L::KBytes];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint8_t *kb = K + ((size_t)g * S + (size_t)j * B) * 128;
  for (int c = threadIdx.x; c < B * 8; c += blockDim.x) {
    const int r = c / 8, col = c % 8;
    *(u32x4 *)(ks + r * L::KStride + col * 16) = *(const u32x4 *)(kb + (size_t)r * 128 + col * 16);
  }
  __syncthreads();
  const int qr = wave * 32 + (lane & 31);
  u32x4 qf[8];
  load_q<true>(Q, (size_t)h * S + (size_t)i * B + qr, qf);
  for (int kt = 0; kt < B / 32; ++kt) {
    f32x16 accf;
    i32x16 acci;
    raw_scores<true>(ks, L::KStride, kt * 32, qf, accf, acci);
#pragma unroll
    for (int r = 0; r < 16; ++r) out[(size_t)(kt * 32 + acc_row(r, lane)) * B + qr] = acci[r];
  }
}

template <int B, bool I8>
hipError_t run_attn(const Plan &p, const AttnArgs &a, hipStream_t st) {
  hipLaunchKernelGGL((k_attn_rows<B, I8>), dim3(p.Hq * p.N), dim3(2 * B), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(const Plan &p, bool i8, const void *Q, const float *sQ, const void *K,
                       const float *sK, const void *V, const float *sV, const fp_index_out *csr,
                       void *O, hipStream_t st) {
  AttnArgs a;
  a.Q = (const uint8_t *)Q; a.K = (const uint8_t *)K; a.V = (const uint8_t *)V;
  a.sQ = sQ; a.sK = sK; a.sV = sV;
  a.row_ptr = csr->row_ptr; a.col_idx = csr->col_idx;
  a.O = (uint16_t *)O;
  a.S = p.S; a.N = p.N; a.Hq = p.Hq; a.G = p.G;
  a.c2 = kLog2e / sqrtf((float)p.d);
  if (p.B == 128) return i8 ? run_attn<128, true>(p, a, st) : run_attn<128, false>(p, a, st);
  return i8 ? run_attn<256, true>(p, a, st) : run_attn<256, false>(p, a, st);
}

hipError_t launch_probe_qk_i8(const Plan &p, const int8_t *Q8, const int8_t *K8, int h, int i,
                              int j, int32_t *out, hipStream_t st) {
  const int g = h / p.G;
  if (p.B == 128)
    hipLaunchKernelGGL(k_probe_qk_i8<128>, dim3(1), dim3(256), 0, st, (const uint8_t *)Q8,
                       (const uint8_t *)K8, p.S, h, g, i, j, out);
  else
    hipLaunchKernelGGL(k_probe_qk_i8<256>, dim3(1), dim3(512), 0, st, (const uint8_t *)Q8,
                       (const uint8_t *)K8, p.S, h, g, i, j, out);
  return hipGetLastError();
}

}  // namespace fp
