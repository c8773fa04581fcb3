// Stage finalize kernel (GDN) and the launchers of the state kernels. The
// finalize stage computes, for one (chunk, head) from the stored entry state
// h and v_new (hyper-parallel "Diff Coverage" page, gate build 2026-09-10,
// _run_prepared_gdn_chunks):  o = (q * r) bf16(h) + Aqk bf16(v_new),
// r = scale * rq * exp(G).
#include "gdn_kernels.h"

namespace gdn {

constexpr int kLdRow = kDim + 8;   // bf16 row stride, 64 x 128 tiles
constexpr int kLdT = kChunk + 8;   // bf16 row stride, 128 x 64 and 64 x 64 tiles


// Stage finalize: o = r * (q bf16(h)) + Aqk bf16(v_new) for one (chunk, head);
// 4 waves, each 32 output columns.

__global__ __launch_bounds__(256) void gdn_finalize_kernel(FinArgs a) {
  const int c = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int g4 = lane >> 4;
  const int l16 = lane & 15;
  const int H = a.H;
  const ChunkInfo ci = a.geo.chunk(c);
  const size_t cm = (size_t)h * a.geo.NT + c;

  __shared__ uint16_t sq[kChunk * kLdRow];
  __shared__ uint16_t sAqk[kChunk * kLdT];
  __shared__ uint16_t shh[kDim * kLdRow];
  __shared__ uint16_t svn[kChunk * kLdRow];
  __shared__ float sR[kChunk];
  __shared__ uint16_t sO[kChunk * kLdRow];

  for (int idx = tid; idx < 1024; idx += 256) {
    const int r = idx >> 4, cc = (idx & 15) * 8;
    uint4 qv = make_uint4(0, 0, 0, 0);
    if (r < ci.len) qv = *reinterpret_cast<const uint4*>(a.q + ((size_t)(ci.tok0 + r) * H + h) * kDim + cc);
    *reinterpret_cast<uint4*>(sq + r * kLdRow + cc) = qv;
  }
  for (int idx = tid; idx < 64 * 64; idx += 256) {
    const int r = idx >> 6, cc = idx & 63;
    sAqk[r * kLdT + unperm_col(cc)] = a.aqk[cm * 4096 + idx];
  }
  for (int idx = tid; idx < kDim * kDim; idx += 256) {
    const int r = idx >> 7, cc = idx & 127;
    shh[r * kLdRow + cc] = f2bf(a.h[cm * (kDim * kDim) + idx]);
  }
  for (int idx = tid; idx < kChunk * kDim; idx += 256) {
    const int r = idx >> 7, cc = idx & 127;
    svn[r * kLdRow + cc] = f2bf(a.vnew[cm * (kChunk * kDim) + idx]);
  }
  if (tid < 64) sR[tid] = a.vec[cm * (kVecRows * kChunk) + 3 * kChunk + tid];
  __syncthreads();

#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int col = 32 * w + 16 * nt + l16;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      f32x4 O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u16x8 av = *reinterpret_cast<const u16x8*>(sq + (16 * it + l16) * kLdRow + 32 * s + 8 * g4);
        u16x8 bv;
#pragma unroll
        for (int e = 0; e < 8; ++e) bv[e] = shh[(32 * s + 8 * g4 + e) * kLdRow + col];
        O = mfma16(av, bv, O);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) O[e] *= sR[16 * it + 4 * g4 + e];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const u16x8 av = *reinterpret_cast<const u16x8*>(sAqk + (16 * it + l16) * kLdT + 32 * s + 8 * g4);
        u16x8 bv;
#pragma unroll
        for (int e = 0; e < 8; ++e) bv[e] = svn[(32 * s + 8 * g4 + e) * kLdRow + col];
        O = mfma16(av, bv, O);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) sO[(16 * it + 4 * g4 + e) * kLdRow + col] = f2bf(O[e]);
    }
  }
  __syncthreads();
  for (int idx = tid; idx < 1024; idx += 256) {
    const int r = idx >> 4, cc = (idx & 15) * 8;
    if (r < ci.len)
      *reinterpret_cast<uint4*>(a.o + ((size_t)(ci.tok0 + r) * H + h) * kDim + cc) =
          *reinterpret_cast<const uint4*>(sO + r * kLdRow + cc);
  }
}

// State summary apply, state_out = M state_in + S per (sequence, head)
// (_apply_gdn_state_summary on the 2026-09-10 coverage page), fp32. One WG
// per (unit, 16 rows of the output): the 16 rows of M are staged in LDS,
// thread (column c, row parity) accumulates 8 rows over the 128 contraction
// indices in order; state_in nullptr means zero.
__global__ __launch_bounds__(256) void summary_apply_kernel(const float* M, const float* S, const float* sin,
                                                            float* sout) {
  __shared__ __attribute__((aligned(16))) float sM[16 * kDim];
  const size_t u = blockIdx.x;
  const int r0 = 16 * blockIdx.y;
  const int tid = threadIdx.x;
  const float* Mu = M + u * kDim * kDim;
  const float* Su = S + u * kDim * kDim;
  float* Ou = sout + u * kDim * kDim;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int idx = p * 256 + tid;  // float4 index inside the 16 x 128 block
    reinterpret_cast<float4*>(sM)[idx] = reinterpret_cast<const float4*>(Mu + (size_t)r0 * kDim)[idx];
  }
  __syncthreads();
  const int c = tid & 127, rs = tid >> 7;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (sin) {
    const float* Iu = sin + u * kDim * kDim;
    for (int kk = 0; kk < kDim; ++kk) {
      const float x = Iu[(size_t)kk * kDim + c];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(sM[(rs + 2 * i) * kDim + kk], x, acc[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const size_t off = (size_t)(r0 + rs + 2 * i) * kDim + c;
    Ou[off] = acc[i] + Su[off];
  }
}

hipError_t launch_summary_apply(const float* M, const float* S, const float* sin, float* sout, long units,
                                hipStream_t stream) {
  hipLaunchKernelGGL(summary_apply_kernel, dim3((unsigned)units, kDim / 16), dim3(256), 0, stream, M, S, sin, sout);
  return hipGetLastError();
}

hipError_t launch_fwd(bool kda, bool store_h, bool compute_o, const FwdArgs& a, hipStream_t stream) {
  if (kda) return launch_kda_fwd(store_h, compute_o, a, stream);
  return launch_gdn_state(store_h, compute_o, a, stream);
}

hipError_t launch_finalize(bool kda, const FinArgs& a, hipStream_t stream) {
  if (kda) return launch_kda_finalize(a, stream);
  dim3 grid(a.geo.NT, a.H);
  hipLaunchKernelGGL(gdn_finalize_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gdn
