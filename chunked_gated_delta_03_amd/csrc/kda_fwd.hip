// Stage finalize kernel (KDA): for one (chunk, head), from the stored entry
// state h and v_new, o = (scale rq) * ((q * 2^G) bf16(h)) + Aqk bf16(v_new),
// the output step of the GDN chunk form (hyper-parallel "Diff Coverage" page,
// gate build 2026-09-10, _run_prepared_gdn_chunks) with a per-channel log2
// decay.
#include "gdn_state_common.h"

namespace gdn {

namespace {
using namespace st;
constexpr int kLdRow = kDim + 8;   // bf16 row stride, 64 x 128 tiles (permuted columns)
constexpr int kLdT = kChunk + 8;   // bf16 row stride, 64 x 64 tiles

}  // namespace

// Stage finalize, KDA: o = (scale rq) * ((q * 2^G) bf16(h)) + Aqk bf16(v_new).
__global__ __launch_bounds__(256) void kda_finalize_kernel(FinArgs a) {
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

  for (int idx = tid; idx < kChunk * kDim; idx += 256) {
    const int r = idx >> 7, d = idx & 127;
    float qv = 0.f;
    if (r < ci.len) qv = bf2f(a.q[((size_t)(ci.tok0 + r) * H + h) * kDim + d]);
    sq[r * kLdRow + d] = f2bf(qv * exp2_hw(a.gk[cm * (kChunk * kDim) + idx]));
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

hipError_t launch_kda_finalize(const FinArgs& a, hipStream_t stream) {
  dim3 grid(a.geo.NT, a.H);
  hipLaunchKernelGGL(kda_finalize_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gdn
