// Kimi Delta Attention state kernel (per-key-channel log2 gate): the
// sequential chunk pass, optionally fused with the output. One workgroup
// (4 waves) per (sequence, head, 64-column V-block), each wave 16 columns.
//
// Per chunk, with S (K x V) the state entering it, G the chunk-local
// cumulative log2 gate per channel (written by the prepare kernel) and
//   kd = k * 2^G,   kg = k * 2^(G_last - G),   qd = q * 2^G   (elementwise),
// the GDN chunk form of the hyper-parallel "Diff Coverage" page (gate build
// 2026-09-10, _run_prepared_gdn_chunks) with every decay per channel reads:
//   v_new = T (beta v - (beta rk) * (kd S))
//   o     = (scale rq) * (qd S) + Aqk v_new
//   S    <- diag(2^G_last) S + kg^T (rk * v_new)
// kd, kg and the right-hand sides that carry the state are bf16 hi + lo
// pairs (three products each), as in the GDN kernel.
#include "gdn_kernels.h"

namespace gdn {

namespace {
constexpr int kLdRow = kDim + 8;   // bf16 row stride, 64 x 128 tiles
constexpr int kLdT = kChunk + 8;   // bf16 row stride, 128 x 64 and 64 x 64 tiles
constexpr int kNW = 4;             // waves per workgroup
constexpr int kBV = 16 * kNW;      // V columns per workgroup
constexpr int kLdV = kBV + 8;
}  // namespace

__device__ __forceinline__ u16x8 frag8(const uint16_t* row, int s, int g4) {
  // contraction slots of K-step s for lane group g4: indices 32s+4g4+(0..3)
  // and 32s+16+4g4+(0..3), matching the accumulator rows of the B operand.
  return cat4(*reinterpret_cast<const u16x4*>(row + 32 * s + 4 * g4),
              *reinterpret_cast<const u16x4*>(row + 32 * s + 16 + 4 * g4));
}

template <bool STORE_H, bool COMPUTE_O>
__global__ __launch_bounds__(kNW * 64) void kda_fwd_kernel(FwdArgs a) {
  const int unit = blockIdx.x;
  const int n = unit / a.H;
  const int h = unit - n * a.H;
  const int vb = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int g4 = lane >> 4;
  const int l16 = lane & 15;
  const int H = a.H;
  const int colw = vb * kBV + w * 16;
  const SeqInfo si = a.geo.seq(n);

  __shared__ uint16_t skd_hi[kChunk * kLdRow];
  __shared__ uint16_t skd_lo[kChunk * kLdRow];
  __shared__ uint16_t skgT_hi[kDim * kLdT];
  __shared__ uint16_t skgT_lo[kDim * kLdT];
  __shared__ uint16_t sTh[kChunk * kLdT];
  __shared__ uint16_t sTl[kChunk * kLdT];
  __shared__ uint16_t sv[kChunk * kLdV];
  __shared__ float sVec[4 * kChunk];
  __shared__ float sDec[kDim];
  __shared__ uint16_t sqd[COMPUTE_O ? kChunk * kLdRow : 1];
  __shared__ uint16_t sAqk[COMPUTE_O ? kChunk * kLdT : 1];
  __shared__ uint16_t sO[COMPUTE_O ? kChunk * kLdV : 1];

  f32x4 S[8];
  const size_t sbase = ((size_t)n * H + h) * kDim * kDim;
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      S[t][e] = a.s0 ? a.s0[sbase + (size_t)(16 * t + 4 * g4 + e) * kDim + colw + l16] : 0.0f;

  const float* sBeta = sVec;
  const float* sC = sVec + kChunk;
  const float* sD = sVec + 2 * kChunk;
  const float* sR = sVec + 3 * kChunk;

  for (int jc = 0; jc < si.nch; ++jc) {
    const int c = si.c0 + jc;
    const int tok0 = si.tok0 + jc * kChunk;
    const int rem = si.len - jc * kChunk;
    const int len = rem < kChunk ? rem : kChunk;
    const size_t cm = (size_t)h * a.geo.NT + c;
    const float* gk = a.gk + cm * (kChunk * kDim);

    // ---- stage the chunk: each thread a 4-row x 8-channel block -----------
    {
      const int m0 = 4 * (tid & 15);
      const int d0 = 8 * (tid >> 4);
      float glast[8];
      {
        const float4 x0 = *reinterpret_cast<const float4*>(gk + 63 * kDim + d0);
        const float4 x1 = *reinterpret_cast<const float4*>(gk + 63 * kDim + d0 + 4);
        glast[0] = x0.x; glast[1] = x0.y; glast[2] = x0.z; glast[3] = x0.w;
        glast[4] = x1.x; glast[5] = x1.y; glast[6] = x1.z; glast[7] = x1.w;
      }
      uint16_t kgh[8][4], kgl[8][4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int m = m0 + rr;
        uint4 kv = make_uint4(0, 0, 0, 0), qv = make_uint4(0, 0, 0, 0);
        if (m < len) {
          const size_t off = ((size_t)(tok0 + m) * H + h) * kDim + d0;
          kv = *reinterpret_cast<const uint4*>(a.k + off);
          if constexpr (COMPUTE_O) qv = *reinterpret_cast<const uint4*>(a.q + off);
        }
        const float4 ga = *reinterpret_cast<const float4*>(gk + m * kDim + d0);
        const float4 gb = *reinterpret_cast<const float4*>(gk + m * kDim + d0 + 4);
        const float gv[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
        const uint32_t kw[4] = {kv.x, kv.y, kv.z, kv.w};
        const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
        u16x8 kdh, kdl, qdv;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float kx = bf2f((uint16_t)((e & 1) ? (kw[e >> 1] >> 16) : (kw[e >> 1] & 0xFFFFu)));
          const float qx = bf2f((uint16_t)((e & 1) ? (qw[e >> 1] >> 16) : (qw[e >> 1] & 0xFFFFu)));
          const float fd = exp2f(gv[e]);
          const float fg = exp2f(glast[e] - gv[e]);
          uint16_t hh, ll;
          split_bf(kx * fd, hh, ll);
          kdh[e] = hh; kdl[e] = ll;
          split_bf(kx * fg, hh, ll);
          kgh[e][rr] = hh; kgl[e][rr] = ll;
          qdv[e] = f2bf(qx * fd);
        }
        *reinterpret_cast<u16x8*>(skd_hi + m * kLdRow + d0) = kdh;
        *reinterpret_cast<u16x8*>(skd_lo + m * kLdRow + d0) = kdl;
        if constexpr (COMPUTE_O) *reinterpret_cast<u16x8*>(sqd + m * kLdRow + d0) = qdv;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        *reinterpret_cast<u16x4*>(skgT_hi + (d0 + e) * kLdT + m0) = u16x4{kgh[e][0], kgh[e][1], kgh[e][2], kgh[e][3]};
        *reinterpret_cast<u16x4*>(skgT_lo + (d0 + e) * kLdT + m0) = u16x4{kgl[e][0], kgl[e][1], kgl[e][2], kgl[e][3]};
      }
      if (tid < kDim) sDec[tid] = exp2f(gk[63 * kDim + tid]);
    }
    {
      const float* tsrc = a.tmat + cm * (kChunk * kChunk);
      for (int idx = tid; idx < 1024; idx += kNW * 64) {
        const int r = idx >> 4, c4 = (idx & 15) * 4;
        const float4 tv4 = reinterpret_cast<const float4*>(tsrc)[idx];
        const float tv[4] = {tv4.x, tv4.y, tv4.z, tv4.w};
        u16x4 hi, lo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uint16_t a0, a1;
          split_bf(tv[e], a0, a1);
          hi[e] = a0; lo[e] = a1;
        }
        *reinterpret_cast<u16x4*>(sTh + r * kLdT + c4) = hi;
        *reinterpret_cast<u16x4*>(sTl + r * kLdT + c4) = lo;
      }
      if constexpr (COMPUTE_O) {
        const uint16_t* asrc = a.aqk + cm * (kChunk * kChunk);
        for (int idx = tid; idx < 512; idx += kNW * 64) {
          const int r = idx >> 3, c8 = (idx & 7) * 8;
          *reinterpret_cast<uint4*>(sAqk + r * kLdT + c8) = reinterpret_cast<const uint4*>(asrc)[idx];
        }
      }
      for (int idx = tid; idx < 64 * kBV / 8; idx += kNW * 64) {
        const int r = idx / (kBV / 8), cu = idx - r * (kBV / 8);
        uint4 val = make_uint4(0, 0, 0, 0);
        if (r < len)
          val = *reinterpret_cast<const uint4*>(a.v + ((size_t)(tok0 + r) * H + h) * kDim + vb * kBV + cu * 8);
        *reinterpret_cast<uint4*>(sv + r * kLdV + cu * 8) = val;
      }
      const float* vsrc = a.vec + cm * (kVecRows * kChunk);
      if (tid < 64) reinterpret_cast<float4*>(sVec)[tid] = reinterpret_cast<const float4*>(vsrc)[tid];
    }
    __syncthreads();

    u16x8 Shi[4], Slo[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint16_t hh, ll;
        split_bf(S[2 * s][e], hh, ll);
        Shi[s][e] = hh; Slo[s][e] = ll;
        split_bf(S[2 * s + 1][e], hh, ll);
        Shi[s][4 + e] = hh; Slo[s][4 + e] = ll;
      }

    if constexpr (STORE_H) {
      float* hd = a.h_out + cm * (kDim * kDim);
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) hd[(size_t)(16 * t + 4 * g4 + e) * kDim + colw + l16] = S[t][e];
    }

    // X = kd S, three split products
    f32x4 X[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      X[it] = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint16_t* rh = skd_hi + (16 * it + l16) * kLdRow;
      const uint16_t* rl = skd_lo + (16 * it + l16) * kLdRow;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u16x8 ah = frag8(rh, s, g4);
        const u16x8 al = frag8(rl, s, g4);
        X[it] = mfma16(ah, Shi[s], X[it]);
        X[it] = mfma16(ah, Slo[s], X[it]);
        X[it] = mfma16(al, Shi[s], X[it]);
      }
    }

    u16x8 Yhi[2], Ylo[2];
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 16 * it + 4 * g4 + e;
        const float vv = bf2f(sv[m * kLdV + w * 16 + l16]);
        const float y = sBeta[m] * vv - sC[m] * X[it][e];
        uint16_t hh, ll;
        split_bf(y, hh, ll);
        Yhi[it >> 1][(it & 1) * 4 + e] = hh;
        Ylo[it >> 1][(it & 1) * 4 + e] = ll;
      }

    f32x4 VN[4];
#pragma unroll
    for (int io = 0; io < 4; ++io) {
      VN[io] = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint16_t* rh = sTh + (16 * io + l16) * kLdT;
      const uint16_t* rl = sTl + (16 * io + l16) * kLdT;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const u16x8 ah = frag8(rh, s, g4);
        const u16x8 al = frag8(rl, s, g4);
        VN[io] = mfma16(ah, Yhi[s], VN[io]);
        VN[io] = mfma16(ah, Ylo[s], VN[io]);
        VN[io] = mfma16(al, Yhi[s], VN[io]);
      }
    }

    if constexpr (STORE_H) {
      float* vd = a.vnew_out + cm * (kChunk * kDim);
#pragma unroll
      for (int io = 0; io < 4; ++io)
#pragma unroll
        for (int e = 0; e < 4; ++e) vd[(size_t)(16 * io + 4 * g4 + e) * kDim + colw + l16] = VN[io][e];
    }

    if constexpr (COMPUTE_O) {
      u16x8 VNb[2];
#pragma unroll
      for (int io = 0; io < 4; ++io)
#pragma unroll
        for (int e = 0; e < 4; ++e) VNb[io >> 1][(io & 1) * 4 + e] = f2bf(VN[io][e]);
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        f32x4 O = {0.f, 0.f, 0.f, 0.f};
        const uint16_t* row = sqd + (16 * it + l16) * kLdRow;
#pragma unroll
        for (int s = 0; s < 4; ++s) O = mfma16(frag8(row, s, g4), Shi[s], O);
#pragma unroll
        for (int e = 0; e < 4; ++e) O[e] *= sR[16 * it + 4 * g4 + e];
        const uint16_t* arow = sAqk + (16 * it + l16) * kLdT;
#pragma unroll
        for (int s = 0; s < 2; ++s) O = mfma16(frag8(arow, s, g4), VNb[s], O);
#pragma unroll
        for (int e = 0; e < 4; ++e) sO[(16 * it + 4 * g4 + e) * kLdV + w * 16 + l16] = f2bf(O[e]);
      }
    }

    // S <- diag(2^G_last) S + kg^T (rk * v_new)
    {
      u16x8 Zhi[2], Zlo[2];
#pragma unroll
      for (int io = 0; io < 4; ++io)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float z = sD[16 * io + 4 * g4 + e] * VN[io][e];
          uint16_t hh, ll;
          split_bf(z, hh, ll);
          Zhi[io >> 1][(io & 1) * 4 + e] = hh;
          Zlo[io >> 1][(io & 1) * 4 + e] = ll;
        }
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        f32x4 acc;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = S[t][e] * sDec[16 * t + 4 * g4 + e];
        const uint16_t* rh = skgT_hi + (16 * t + l16) * kLdT;
        const uint16_t* rl = skgT_lo + (16 * t + l16) * kLdT;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const u16x8 ah = frag8(rh, s, g4);
          const u16x8 al = frag8(rl, s, g4);
          acc = mfma16(ah, Zhi[s], acc);
          acc = mfma16(ah, Zlo[s], acc);
          acc = mfma16(al, Zhi[s], acc);
        }
        S[t] = acc;
      }
    }
    __syncthreads();

    if constexpr (COMPUTE_O) {
      for (int idx = tid; idx < 64 * kBV / 8; idx += kNW * 64) {
        const int r = idx / (kBV / 8), cu = idx - r * (kBV / 8);
        if (r < len)
          *reinterpret_cast<uint4*>(a.o + ((size_t)(tok0 + r) * H + h) * kDim + vb * kBV + cu * 8) =
              *reinterpret_cast<const uint4*>(sO + r * kLdV + cu * 8);
      }
      __syncthreads();
    }
  }

  if (a.sfinal) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) a.sfinal[sbase + (size_t)(16 * t + 4 * g4 + e) * kDim + colw + l16] = S[t][e];
  }
}

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
    sq[r * kLdRow + d] = f2bf(qv * exp2f(a.gk[cm * (kChunk * kDim) + idx]));
  }
  for (int idx = tid; idx < 64 * 64; idx += 256) {
    const int r = idx >> 6, cc = idx & 63;
    sAqk[r * kLdT + cc] = a.aqk[cm * 4096 + idx];
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

hipError_t launch_kda_fwd(bool store_h, bool compute_o, const FwdArgs& a, hipStream_t stream) {
  dim3 grid(a.geo.N * a.H, kDim / kBV);
  dim3 block(64 * kNW);
  if (store_h && !compute_o)
    hipLaunchKernelGGL((kda_fwd_kernel<true, false>), grid, block, 0, stream, a);
  else if (!store_h && compute_o)
    hipLaunchKernelGGL((kda_fwd_kernel<false, true>), grid, block, 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_kda_finalize(const FinArgs& a, hipStream_t stream) {
  dim3 grid(a.geo.NT, a.H);
  hipLaunchKernelGGL(kda_finalize_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gdn
