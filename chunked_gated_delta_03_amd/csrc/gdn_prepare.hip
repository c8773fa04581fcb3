// Prepare kernel: everything of one (chunk, head) that does not depend on the
// carried state. One workgroup of 4 waves per (chunk, head).
//
// Steps of the eager chunk algorithm on the hyper-parallel "Diff Coverage"
// page (gate build 2026-09-10; _prepare_gdn_chunks_for_summary), done here:
//   - optional L2 normalisation of q and k (the _l2norm helper, eps 1e-6
//     added to the sum of squares) -- kept as per-row factors rq, rk so the
//     bf16 inputs enter the MFMAs unrounded;
//   - optional sigmoid of beta;
//   - chunk-local cumulative sum G of the gate;
//   - A = -(beta k k^T * Gamma), strictly lower, Gamma[i,j] = exp(G_i - G_j)
//     with the mask applied before the exponential;
//   - T = (I - A)^-1 (the page's row-by-row forward substitution plus the
//     identity), computed blockwise: 16x16 diagonal blocks by substitution,
//     then the off-diagonal blocks T_ij = T_ii * sum_m A_im T_mj;
//   - the intra-chunk output matrix scale * (q k^T * Gamma), lower with the
//     diagonal (_run_prepared_gdn_chunks).
// The WY products U = T v_beta and W = T (k_beta e^G) are not formed here:
// the state kernel applies T to (beta v - c * (k S)) directly, which needs T
// and the per-row vectors only.
#include "gdn_kernels.h"

namespace gdn {

constexpr int kLdRow = kDim + 8;    // bf16 row stride of a 64 x 128 tile in LDS
constexpr int kLdF = kChunk + 1;    // fp32 row stride of a 64 x 64 matrix in LDS
constexpr int kLdQ = kChunk + 8;    // bf16 row stride of a 64 x 64 matrix in LDS


__device__ __forceinline__ float sumsq8(const uint4& v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float lo = __uint_as_float(w[i] << 16);
    float hi = __uint_as_float(w[i] & 0xFFFF0000u);
    s = fmaf(lo, lo, s);
    s = fmaf(hi, hi, s);
  }
  return s;
}

__global__ __launch_bounds__(256) void gdn_prepare_kernel(PrepareArgs a) {
  const int c = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g4 = lane >> 4;
  const int l16 = lane & 15;
  const ChunkInfo ci = a.geo.chunk(c);
  const int H = a.H;

  __shared__ uint16_t sk[kChunk * kLdRow];
  __shared__ uint16_t sq[kChunk * kLdRow];
  __shared__ float sA[kChunk * kLdF];
  __shared__ float sT[kChunk * kLdF];
  __shared__ float sP[4][16 * 17];
  __shared__ uint16_t sAqk[kChunk * kLdQ];
  __shared__ float sG[kChunk], sBeta[kChunk], sRq[kChunk], sRk[kChunk];

  const bool l2 = (a.flags & 1u) != 0;
  const bool sig = (a.flags & 2u) != 0;

  // ---- 1. q, k rows into LDS; per-row normalisation factors ---------------
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int idx = pass * 256 + tid;
    const int r = idx >> 4;
    const int cc = (idx & 15) * 8;
    uint4 kv = make_uint4(0, 0, 0, 0), qv = make_uint4(0, 0, 0, 0);
    if (r < ci.len) {
      const size_t off = ((size_t)(ci.tok0 + r) * H + h) * kDim + cc;
      kv = *reinterpret_cast<const uint4*>(a.k + off);
      qv = *reinterpret_cast<const uint4*>(a.q + off);
    }
    *reinterpret_cast<uint4*>(sk + r * kLdRow + cc) = kv;
    *reinterpret_cast<uint4*>(sq + r * kLdRow + cc) = qv;
    float ssk = sumsq8(kv), ssq = sumsq8(qv);
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) {
      ssk += __shfl_xor(ssk, m);
      ssq += __shfl_xor(ssq, m);
    }
    if ((tid & 15) == 0) {
      const bool valid = r < ci.len;
      sRk[r] = valid ? (l2 ? 1.0f / sqrtf(ssk + 1e-6f) : 1.0f) : 0.0f;
      sRq[r] = valid ? (l2 ? 1.0f / sqrtf(ssq + 1e-6f) : 1.0f) : 0.0f;
    }
  }

  // ---- 2. gate cumsum and beta (wave 0) -------------------------------------
  if (wave == 0) {
    const bool valid = lane < ci.len;
    const size_t th = (size_t)(ci.tok0 + lane) * H + h;
    float x = valid ? a.g[th] : 0.0f;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    sG[lane] = x;
    float b = valid ? bf2f(a.beta[th]) : 0.0f;
    if (sig && valid) b = 1.0f / (1.0f + expf(-b));
    sBeta[lane] = b;
  }
  __syncthreads();

  // ---- 3. Gram tiles on MFMA: k k^T (strictly lower) and q k^T (lower) ------
  // 10 lower 16x16 tiles each; job = kind*10 + tile, wave takes every 4th.
  for (int job = wave; job < 20; job += 4) {
    const int kind = job / 10;  // 0: k k^T, 1: q k^T
    int t = job % 10, I = 0;
    while (t > I) { t -= I + 1; ++I; }
    const int J = t;
    const uint16_t* left = kind == 0 ? sk : sq;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u16x8 av = *reinterpret_cast<const u16x8*>(left + (16 * I + l16) * kLdRow + 32 * s + 8 * g4);
      const u16x8 bv = *reinterpret_cast<const u16x8*>(sk + (16 * J + l16) * kLdRow + 32 * s + 8 * g4);
      acc = mfma16(av, bv, acc);
    }
    const int jc = 16 * J + l16;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * I + 4 * g4 + e;
      if (kind == 0) {
        float val = 0.0f;
        if (i > jc) val = -sBeta[i] * sRk[i] * sRk[jc] * acc[e] * expf(sG[i] - sG[jc]);
        sA[i * kLdF + jc] = val;
      } else {
        float val = 0.0f;
        if (i >= jc) val = a.scale * sRq[i] * sRk[jc] * acc[e] * expf(sG[i] - sG[jc]);
        sAqk[i * kLdQ + jc] = f2bf(val);
      }
    }
  }
  __syncthreads();

  // ---- 4a. diagonal 16x16 blocks of T by forward substitution --------------
  if (lane < 16) {
    const int base = 16 * wave;
    float t[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float val = (i == lane) ? 1.0f : 0.0f;
#pragma unroll
      for (int m = 0; m < i; ++m) val = fmaf(sA[(base + i) * kLdF + base + m], t[m], val);
      t[i] = val;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sT[(base + i) * kLdF + base + lane] = t[i];
  }
  __syncthreads();

  // ---- 4b. off-diagonal blocks, one block row at a time --------------------
  // T_ij = T_ii * sum_{m=j}^{i-1} A_im T_mj ; lane holds (row l16, cols 4*g4..+3)
  for (int I = 1; I < 4; ++I) {
    const int J = wave;
    if (J < I) {
      float p[4] = {0.f, 0.f, 0.f, 0.f};
      for (int M = J; M < I; ++M) {
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const float av = sA[(16 * I + l16) * kLdF + 16 * M + x];
#pragma unroll
          for (int e = 0; e < 4; ++e) p[e] = fmaf(av, sT[(16 * M + x) * kLdF + 16 * J + 4 * g4 + e], p[e]);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) sP[wave][l16 * 17 + 4 * g4 + e] = p[e];
    }
    __syncthreads();
    if (J < I) {
      float r[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const float tv = sT[(16 * I + l16) * kLdF + 16 * I + x];
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = fmaf(tv, sP[wave][x * 17 + 4 * g4 + e], r[e]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) sT[(16 * I + l16) * kLdF + 16 * J + 4 * g4 + e] = r[e];
    }
    __syncthreads();
  }

  // ---- 5. outputs ------------------------------------------------------------
  const size_t cm = (size_t)h * a.geo.NT + c;
  float* tdst = a.tmat + cm * (kChunk * kChunk);
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int idx = pass * 256 + tid;
    const int r = idx >> 4;
    const int c4 = (idx & 15) * 4;
    float4 val;
    const bool upper = (c4 >> 4) > (r >> 4);
    val.x = upper ? 0.f : sT[r * kLdF + c4 + 0];
    val.y = upper ? 0.f : sT[r * kLdF + c4 + 1];
    val.z = upper ? 0.f : sT[r * kLdF + c4 + 2];
    val.w = upper ? 0.f : sT[r * kLdF + c4 + 3];
    *reinterpret_cast<float4*>(tdst + r * kChunk + c4) = val;
  }
  uint16_t* qdst = a.aqk + cm * (kChunk * kChunk);
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int idx = pass * 256 + tid;
    const int r = idx >> 3;
    const int c8 = (idx & 7) * 8;
    u16x8 val;
#pragma unroll
    for (int e = 0; e < 8; ++e) val[e] = ((c8 >> 4) > (r >> 4)) ? (uint16_t)0 : sAqk[r * kLdQ + c8 + e];
    *reinterpret_cast<u16x8*>(qdst + r * kChunk + c8) = val;
  }
  if (tid < 64) {
    const int i = tid;
    const bool valid = i < ci.len;
    const float G = sG[i];
    const float Glast = sG[63];
    const float b = valid ? sBeta[i] : 0.f;
    const float rk = sRk[i], rq = sRq[i];
    float* vd = a.vec + cm * (kVecRows * kChunk);
    vd[0 * 64 + i] = b;
    vd[1 * 64 + i] = valid ? b * rk * expf(G) : 0.f;
    vd[2 * 64 + i] = valid ? rk * expf(Glast - G) : 0.f;
    vd[3 * 64 + i] = valid ? a.scale * rq * expf(G) : 0.f;
    vd[4 * 64 + i] = G;
    vd[5 * 64 + i] = rq;
    vd[6 * 64 + i] = rk;
    vd[7 * 64 + i] = (i == 0) ? expf(Glast) : 0.f;
  }
}

hipError_t launch_prepare(bool kda, const PrepareArgs& a, hipStream_t stream) {
  if (kda) return hipErrorNotSupported;
  dim3 grid(a.geo.NT, a.H);
  hipLaunchKernelGGL(gdn_prepare_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gdn
