// Reverse state pass of the KDA backward (per-key-channel log2 gate).
//
// The loss L = <dO, o> + <dS_T, S_T> is linear in the state entering each
// chunk, and its gradient dS flows backwards through the chunks. Per chunk,
// with the chunk form of the forward (the prepared-chunk algorithm of
// torch_chunk_gated_delta_rule on the hyper-parallel "Diff Coverage" page,
// gate build 2026-09-10, with the per-channel decays of the KDA stages on the
// kimi_delta_attention_ascendc.py coverage page) and dS the gradient w.r.t.
// the state leaving the chunk:
//   dV' = KG dS + Aqk^T dO                        (w.r.t. v_new)
//   dS <- diag(2^G_last) dS + QD^T dO - KDB^T T^T dV'
// with the operands, rows i and key channels d of the chunk,
//   KG[i,d]  = k[i,d] rk_i 2^(G_last,d - G_i,d),
//   QD[i,d]  = q[i,d] scale rq_i 2^G_i,d,
//   KDB[i,d] = k[i,d] beta_i rk_i 2^G_i,d,
// G the chunk-local cumulative log2 gate, rk, rq the L2-norm factors, T the
// WY inverse and Aqk the intra-chunk output matrix (scale rq rk included),
// all from the KDA prepare kernel. Every exponent is <= 0.
//
// One workgroup per (sequence, head, 16 value columns), fp32 arithmetic on
// the vector units: the operands of a chunk are formed in LDS, the 128 x 16
// block of dS is held in registers (thread t: column t % 16, rows 8 (t / 16)
// .. + 7). It stores, per chunk, dS before the update (the gradient w.r.t. the
// state leaving the chunk) and dV', and the gradient w.r.t. the initial state.
#include "gdn_bwd.h"

namespace gdn {

namespace {

constexpr int kLdO = kDim + 4;     // fp32 row stride of the 64 x 128 operands (16-byte rows)
constexpr int kLdM = kChunk + 1;   // fp32 row stride of T and Aqk
constexpr int kCols = 16;          // value columns per workgroup

struct alignas(16) KdaDhSmem {
  float kg[kChunk * kLdO];
  float qd[kChunk * kLdO];
  float kdb[kChunk * kLdO];
  float t[kChunk * kLdM];
  float p[kChunk * kLdM];
  float dO[kChunk * kCols];
  float ds[kDim * kCols];
  float dv[kChunk * kCols];
  float y[kChunk * kCols];
  float dec[kDim];
};

}  // namespace

__global__ __launch_bounds__(256) void kda_bwd_dh_kernel(KdaBwdArgs a) {
  __shared__ KdaDhSmem sm;
  const int tid = threadIdx.x;
  const int vb = blockIdx.x % (kDim / kCols);
  const int unit = blockIdx.x / (kDim / kCols);
  const int n = unit / a.H, h = unit - (unit / a.H) * a.H;
  const SeqInfo si = a.geo.seq(n);
  const int NT = a.geo.NT;
  const int col0 = vb * kCols;

  // dS block: column cc, rows 8 rg .. 8 rg + 7
  const int cc = tid & 15, rg = tid >> 4;
  float dS[8];
  const size_t sbase = ((size_t)n * a.H + h) * kDim * kDim;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    dS[e] = a.dsfinal ? a.dsfinal[sbase + (size_t)(8 * rg + e) * kDim + col0 + cc] : 0.0f;

  for (int jc = si.nch - 1; jc >= 0; --jc) {
    const int c = si.c0 + jc;
    const size_t cm = (size_t)h * NT + c;
    const int tok0 = si.tok0 + jc * kChunk;
    const int rem = si.len - jc * kChunk;
    const int len = rem < kChunk ? rem : kChunk;
    const float* gk = a.gk + cm * (kChunk * kDim);
    const float* vec = a.vec + cm * (kVecRows * kChunk);

    // operands: thread (row i, 32 channels from d0), all loads issued
    // together as 16-byte pieces; rows past the end are zero
    {
      const int i = tid >> 2, d0 = (tid & 3) * 32;
      const bool valid = i < len;
      const float rkb = vec[1 * kChunk + i], rk = vec[2 * kChunk + i], srq = vec[3 * kChunk + i];
      const size_t roff = ((size_t)(tok0 + (valid ? i : 0)) * a.H + h) * kDim + d0;
      uint4 kr[4], qr[4];
      float4 gr[8], gl[8];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        kr[p] = valid ? reinterpret_cast<const uint4*>(a.k + roff)[p] : make_uint4(0, 0, 0, 0);
        qr[p] = valid ? reinterpret_cast<const uint4*>(a.q + roff)[p] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        gr[p] = reinterpret_cast<const float4*>(gk + i * kDim + d0)[p];
        gl[p] = reinterpret_cast<const float4*>(gk + (kChunk - 1) * kDim + d0)[p];
      }
      // T (hi + lo) and Aqk rows: thread (row r, stored positions 16 qq ..
      // 16 qq + 15), scattered to their columns
      const int r = tid >> 2, qq = tid & 3;
      const uint16_t* tm = a.tmat + cm * (kChunk * 2 * kChunk) + r * (2 * kChunk) + 16 * qq;
      const uint16_t* aq = a.aqk + cm * (kChunk * kChunk) + r * kChunk + 16 * qq;
      const uint4 th0 = reinterpret_cast<const uint4*>(tm)[0], th1 = reinterpret_cast<const uint4*>(tm)[1];
      const uint4 tl0 = reinterpret_cast<const uint4*>(tm + kChunk)[0];
      const uint4 tl1 = reinterpret_cast<const uint4*>(tm + kChunk)[1];
      const uint4 a0 = reinterpret_cast<const uint4*>(aq)[0], a1 = reinterpret_cast<const uint4*>(aq)[1];
      float dov[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int idx = tid + 256 * e, ri = idx >> 4, cj = idx & 15;
        dov[e] = ri < len ? bf2f(a.dout[((size_t)(tok0 + ri) * a.H + h) * kDim + col0 + cj]) : 0.0f;
      }

      const uint32_t kw[16] = {kr[0].x, kr[0].y, kr[0].z, kr[0].w, kr[1].x, kr[1].y, kr[1].z, kr[1].w,
                               kr[2].x, kr[2].y, kr[2].z, kr[2].w, kr[3].x, kr[3].y, kr[3].z, kr[3].w};
      const uint32_t qw[16] = {qr[0].x, qr[0].y, qr[0].z, qr[0].w, qr[1].x, qr[1].y, qr[1].z, qr[1].w,
                               qr[2].x, qr[2].y, qr[2].z, qr[2].w, qr[3].x, qr[3].y, qr[3].z, qr[3].w};
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const float G[4] = {gr[p].x, gr[p].y, gr[p].z, gr[p].w};
        const float GL[4] = {gl[p].x, gl[p].y, gl[p].z, gl[p].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c2 = 4 * p + e, d = d0 + c2;
          const uint32_t kb = kw[c2 >> 1], qb = qw[c2 >> 1];
          const float kv = __uint_as_float((c2 & 1) ? (kb & 0xFFFF0000u) : (kb << 16));
          const float qv = __uint_as_float((c2 & 1) ? (qb & 0xFFFF0000u) : (qb << 16));
          const float eg = exp2_hw(G[e]);
          sm.kg[i * kLdO + d] = kv * rk * exp2_hw(GL[e] - G[e]);
          sm.qd[i * kLdO + d] = qv * srq * eg;
          sm.kdb[i * kLdO + d] = kv * rkb * eg;
        }
      }
      if (tid < kDim / 4) {
        const float4 l = reinterpret_cast<const float4*>(gk + (kChunk - 1) * kDim)[tid];
        sm.dec[4 * tid + 0] = exp2_hw(l.x);
        sm.dec[4 * tid + 1] = exp2_hw(l.y);
        sm.dec[4 * tid + 2] = exp2_hw(l.z);
        sm.dec[4 * tid + 3] = exp2_hw(l.w);
      }
      const uint32_t thw[8] = {th0.x, th0.y, th0.z, th0.w, th1.x, th1.y, th1.z, th1.w};
      const uint32_t tlw[8] = {tl0.x, tl0.y, tl0.z, tl0.w, tl1.x, tl1.y, tl1.z, tl1.w};
      const uint32_t aw[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int col = unperm_col(16 * qq + e);
        const uint32_t hw = thw[e >> 1], lw = tlw[e >> 1], pw = aw[e >> 1];
        const float hv = __uint_as_float((e & 1) ? (hw & 0xFFFF0000u) : (hw << 16));
        const float lv = __uint_as_float((e & 1) ? (lw & 0xFFFF0000u) : (lw << 16));
        sm.t[r * kLdM + col] = hv + lv;
        sm.p[r * kLdM + col] = __uint_as_float((e & 1) ? (pw & 0xFFFF0000u) : (pw << 16));
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.dO[tid + 256 * e] = dov[e];
    }
    // dS before the update: the gradient w.r.t. the state leaving the chunk
    float* dhn = a.dhn + cm * (kDim * kDim);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sm.ds[(8 * rg + e) * kCols + cc] = dS[e];
      dhn[(size_t)(8 * rg + e) * kDim + col0 + cc] = dS[e];
    }
    __syncthreads();

    // dV' = KG dS + Aqk^T dO: thread (row i, columns c4 .. c4 + 3)
    {
      const int i = tid >> 2, c4 = (tid & 3) * 4;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      auto fma4 = [](float s, const float4& x, float4& y) {
        y.x = fmaf(s, x.x, y.x); y.y = fmaf(s, x.y, y.y); y.z = fmaf(s, x.z, y.z); y.w = fmaf(s, x.w, y.w);
      };
      for (int d = 0; d < kDim; d += 4) {
        const float4 kg4 = *reinterpret_cast<const float4*>(sm.kg + i * kLdO + d);
        fma4(kg4.x, *reinterpret_cast<const float4*>(sm.ds + (d + 0) * kCols + c4), acc);
        fma4(kg4.y, *reinterpret_cast<const float4*>(sm.ds + (d + 1) * kCols + c4), acc);
        fma4(kg4.z, *reinterpret_cast<const float4*>(sm.ds + (d + 2) * kCols + c4), acc);
        fma4(kg4.w, *reinterpret_cast<const float4*>(sm.ds + (d + 3) * kCols + c4), acc);
      }
      for (int r = i; r < kChunk; ++r)  // Aqk is lower triangular (with its diagonal)
        fma4(sm.p[r * kLdM + i], *reinterpret_cast<const float4*>(sm.dO + r * kCols + c4), acc);
      *reinterpret_cast<float4*>(sm.dv + i * kCols + c4) = acc;
      *reinterpret_cast<float4*>(a.dvn + cm * (kChunk * kDim) + (size_t)i * kDim + col0 + c4) = acc;
    }
    __syncthreads();

    // Y = T^T dV' (T lower triangular): thread (row j, columns c4 .. c4 + 3)
    {
      const int j = tid >> 2, c4 = (tid & 3) * 4;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int i = j; i < kChunk; ++i) {
        const float tv = sm.t[i * kLdM + j];
        const float4 x = *reinterpret_cast<const float4*>(sm.dv + i * kCols + c4);
        acc.x = fmaf(tv, x.x, acc.x); acc.y = fmaf(tv, x.y, acc.y);
        acc.z = fmaf(tv, x.z, acc.z); acc.w = fmaf(tv, x.w, acc.w);
      }
      *reinterpret_cast<float4*>(sm.y + j * kCols + c4) = acc;
    }
    __syncthreads();

    // dS <- diag(2^G_last) dS + QD^T dO - KDB^T Y (this thread's 8 rows)
    {
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = sm.dec[8 * rg + e] * dS[e];
      for (int i = 0; i < kChunk; ++i) {
        const float dov = sm.dO[i * kCols + cc], yv = sm.y[i * kCols + cc];
        const float4 q0 = *reinterpret_cast<const float4*>(sm.qd + i * kLdO + 8 * rg);
        const float4 q1 = *reinterpret_cast<const float4*>(sm.qd + i * kLdO + 8 * rg + 4);
        const float4 k0 = *reinterpret_cast<const float4*>(sm.kdb + i * kLdO + 8 * rg);
        const float4 k1 = *reinterpret_cast<const float4*>(sm.kdb + i * kLdO + 8 * rg + 4);
        const float qa[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
        const float ka[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(qa[e], dov, fmaf(-ka[e], yv, acc[e]));
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) dS[e] = acc[e];
    }
    __syncthreads();  // the next chunk rewrites the operands
  }
  if (a.ds0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) a.ds0[sbase + (size_t)(8 * rg + e) * kDim + col0 + cc] = dS[e];
  }
}

hipError_t launch_kda_bwd_dh(const KdaBwdArgs& a, hipStream_t stream) {
  const unsigned grid = (unsigned)((size_t)a.geo.N * a.H * (kDim / kCols));
  hipLaunchKernelGGL(kda_bwd_dh_kernel, dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gdn
