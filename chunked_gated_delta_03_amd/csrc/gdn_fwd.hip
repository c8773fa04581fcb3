// State kernel: the sequential chunk pass (chunk_fwd_h), optionally fused
// with the output (finalize). One workgroup per (sequence, head, V-block);
// the V-block is 16 columns per wave; chunks of the sequence are processed in
// order with the K x V state held in registers (MFMA accumulator layout).
//
// Per chunk, with S the state entering it (hyper-parallel "Diff Coverage"
// page, gate build 2026-09-10, _run_prepared_gdn_chunks and the state update
// of torch_chunk_gated_delta_rule):
//   v_new = U - W S = T (beta v - c * (k S)),     c = beta * rk * exp(G)
//   o     = (q * r) S + Aqk v_new,                r = scale * rq * exp(G)
//   S    <- exp(G_last) S + k^T (d * v_new),      d = rk * exp(G_last - G)
// where k, q are the raw bf16 rows and rk, rq their normalisation factors,
// so every MFMA operand taken from the inputs is exact. Operands that carry
// the state forward (S in k S, T and the right-hand side in T(...), d*v_new
// in the update) are split into bf16 hi + lo pairs, which gives the state
// path ~16 significant bits per operand with fp32 accumulation; the output
// products use single bf16 operands.
#include "gdn_kernels.h"

namespace gdn {

constexpr int kLdRow = kDim + 8;   // bf16 row stride, 64 x 128 tiles
constexpr int kLdT = kChunk + 8;   // bf16 row stride, 128 x 64 and 64 x 64 tiles


template <int NW>
struct Stage {
  static constexpr int NTH = NW * 64;
  static constexpr int BV = NW * 16;
  static constexpr int kLdV = BV + 8;
  static constexpr int NK = 1024 / NTH;        // uint4 per thread for a 64x128 bf16 tile
  static constexpr int NTM = 1024 / NTH;       // float4 per thread for 64x64 fp32
  static constexpr int NAQ = 512 / NTH;        // uint4 per thread for 64x64 bf16
  static constexpr int NVB = (64 * BV / 8 + NTH - 1) / NTH;  // uint4 per thread for v block
};

template <int NW, bool STORE_H, bool COMPUTE_O>
__global__ __launch_bounds__(NW * 64) void gdn_fwd_kernel(FwdArgs a) {
  using St = Stage<NW>;
  constexpr int NTH = St::NTH;
  constexpr int BV = St::BV;
  constexpr int kLdV = St::kLdV;

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
  const int colw = vb * BV + w * 16;  // first V column of this wave
  const SeqInfo si = a.geo.seq(n);

  __shared__ uint16_t sk[kChunk * kLdRow];
  __shared__ uint16_t skT[kDim * kLdT];
  __shared__ uint16_t sTh[kChunk * kLdT];
  __shared__ uint16_t sTl[kChunk * kLdT];
  __shared__ uint16_t sv[kChunk * kLdV];
  __shared__ float sVec[4 * kChunk];
  __shared__ float sDecay;
  __shared__ uint16_t sq[COMPUTE_O ? kChunk * kLdRow : 1];
  __shared__ uint16_t sAqk[COMPUTE_O ? kChunk * kLdT : 1];
  __shared__ uint16_t sO[COMPUTE_O ? kChunk * kLdV : 1];

  // ---- state in registers: 8 row tiles of 16 x 16 (rows 16t + 4g4 + e) ----
  f32x4 S[8];
  const size_t sbase = ((size_t)n * H + h) * kDim * kDim;
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      S[t][e] = a.s0 ? a.s0[sbase + (size_t)(16 * t + 4 * g4 + e) * kDim + colw + l16] : 0.0f;

  // ---- prefetch registers --------------------------------------------------
  uint4 rk[St::NK];
  uint4 rq[COMPUTE_O ? St::NK : 1];
  float4 rt[St::NTM];
  uint4 ra[COMPUTE_O ? St::NAQ : 1];
  uint4 rv[St::NVB];
  float4 rvec;
  float rdec;

  auto load = [&](int jc) {
    const int c = si.c0 + jc;
    const int tok0 = si.tok0 + jc * kChunk;
    const int rem = si.len - jc * kChunk;
    const int len = rem < kChunk ? rem : kChunk;
    const size_t cm = (size_t)h * a.geo.NT + c;
#pragma unroll
    for (int p = 0; p < St::NK; ++p) {
      const int idx = p * NTH + tid;
      const int r = idx >> 4, cc = (idx & 15) * 8;
      const size_t off = ((size_t)(tok0 + r) * H + h) * kDim + cc;
      rk[p] = r < len ? *reinterpret_cast<const uint4*>(a.k + off) : make_uint4(0, 0, 0, 0);
      if constexpr (COMPUTE_O)
        rq[p] = r < len ? *reinterpret_cast<const uint4*>(a.q + off) : make_uint4(0, 0, 0, 0);
    }
    const float* tsrc = a.tmat + cm * (kChunk * kChunk);
#pragma unroll
    for (int p = 0; p < St::NTM; ++p) rt[p] = reinterpret_cast<const float4*>(tsrc)[p * NTH + tid];
    if constexpr (COMPUTE_O) {
      const uint16_t* asrc = a.aqk + cm * (kChunk * kChunk);
#pragma unroll
      for (int p = 0; p < St::NAQ; ++p) ra[p] = reinterpret_cast<const uint4*>(asrc)[p * NTH + tid];
    }
#pragma unroll
    for (int p = 0; p < St::NVB; ++p) {
      const int idx = p * NTH + tid;
      const int r = idx / (BV / 8), cu = idx - r * (BV / 8);
      uint4 val = make_uint4(0, 0, 0, 0);
      if (idx < 64 * BV / 8 && r < len)
        val = *reinterpret_cast<const uint4*>(a.v + ((size_t)(tok0 + r) * H + h) * kDim + vb * BV + cu * 8);
      rv[p] = val;
    }
    const float* vsrc = a.vec + cm * (kVecRows * kChunk);
    if (tid < 64) rvec = reinterpret_cast<const float4*>(vsrc)[tid];  // rows 0..3 (beta, c, d, r)
    rdec = vsrc[7 * kChunk];
  };

  auto store = [&]() {
#pragma unroll
    for (int p = 0; p < St::NK; ++p) {
      const int idx = p * NTH + tid;
      const int r = idx >> 4, cc = (idx & 15) * 8;
      *reinterpret_cast<uint4*>(sk + r * kLdRow + cc) = rk[p];
      const uint32_t wv[4] = {rk[p].x, rk[p].y, rk[p].z, rk[p].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        skT[(cc + 2 * e) * kLdT + r] = (uint16_t)(wv[e] & 0xFFFFu);
        skT[(cc + 2 * e + 1) * kLdT + r] = (uint16_t)(wv[e] >> 16);
      }
      if constexpr (COMPUTE_O) *reinterpret_cast<uint4*>(sq + r * kLdRow + cc) = rq[p];
    }
#pragma unroll
    for (int p = 0; p < St::NTM; ++p) {
      const int idx = p * NTH + tid;
      const int r = idx >> 4, c4 = (idx & 15) * 4;
      u16x4 hi, lo;
      const float tv[4] = {rt[p].x, rt[p].y, rt[p].z, rt[p].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint16_t a0, a1;
        split_bf(tv[e], a0, a1);
        hi[e] = a0;
        lo[e] = a1;
      }
      *reinterpret_cast<u16x4*>(sTh + r * kLdT + c4) = hi;
      *reinterpret_cast<u16x4*>(sTl + r * kLdT + c4) = lo;
    }
    if constexpr (COMPUTE_O) {
#pragma unroll
      for (int p = 0; p < St::NAQ; ++p) {
        const int idx = p * NTH + tid;
        const int r = idx >> 3, c8 = (idx & 7) * 8;
        *reinterpret_cast<uint4*>(sAqk + r * kLdT + c8) = ra[p];
      }
    }
#pragma unroll
    for (int p = 0; p < St::NVB; ++p) {
      const int idx = p * NTH + tid;
      const int r = idx / (BV / 8), cu = idx - r * (BV / 8);
      if (idx < 64 * BV / 8) *reinterpret_cast<uint4*>(sv + r * kLdV + cu * 8) = rv[p];
    }
    if (tid < 64) reinterpret_cast<float4*>(sVec)[tid] = rvec;
    if (tid == 0) sDecay = rdec;
  };

  const float* sBeta = sVec;
  const float* sC = sVec + kChunk;
  const float* sD = sVec + 2 * kChunk;
  const float* sR = sVec + 3 * kChunk;

  if (si.nch > 0) load(0);
  for (int jc = 0; jc < si.nch; ++jc) {
    const int c = si.c0 + jc;
    const int tok0 = si.tok0 + jc * kChunk;
    const int rem = si.len - jc * kChunk;
    const int len = rem < kChunk ? rem : kChunk;
    store();
    __syncthreads();
    if (jc + 1 < si.nch) load(jc + 1);

    // -- S as B operands: K-step s uses state tiles 2s and 2s+1 ---------------
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
      const size_t cm = (size_t)h * a.geo.NT + c;
      float* hd = a.h_out + cm * (kDim * kDim);
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) hd[(size_t)(16 * t + 4 * g4 + e) * kDim + colw + l16] = S[t][e];
    }

    // -- X = k S  (64 x 16) ----------------------------------------------------
    f32x4 X[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      X[it] = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint16_t* row = sk + (16 * it + l16) * kLdRow + 4 * g4;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u16x8 av = cat4(*reinterpret_cast<const u16x4*>(row + 32 * s),
                              *reinterpret_cast<const u16x4*>(row + 32 * s + 16));
        X[it] = mfma16(av, Shi[s], X[it]);
        X[it] = mfma16(av, Slo[s], X[it]);
      }
    }

    // -- Y = beta v - c X, split for the T product -----------------------------
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

    // -- v_new = T Y  (64 x 16), three split products --------------------------
    f32x4 VN[4];
#pragma unroll
    for (int io = 0; io < 4; ++io) {
      VN[io] = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint16_t* rh = sTh + (16 * io + l16) * kLdT + 4 * g4;
      const uint16_t* rl = sTl + (16 * io + l16) * kLdT + 4 * g4;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const u16x8 ah = cat4(*reinterpret_cast<const u16x4*>(rh + 32 * s),
                              *reinterpret_cast<const u16x4*>(rh + 32 * s + 16));
        const u16x8 al = cat4(*reinterpret_cast<const u16x4*>(rl + 32 * s),
                              *reinterpret_cast<const u16x4*>(rl + 32 * s + 16));
        VN[io] = mfma16(ah, Yhi[s], VN[io]);
        VN[io] = mfma16(ah, Ylo[s], VN[io]);
        VN[io] = mfma16(al, Yhi[s], VN[io]);
      }
    }

    if constexpr (STORE_H) {
      const size_t cm = (size_t)h * a.geo.NT + c;
      float* vd = a.vnew_out + cm * (kChunk * kDim);
#pragma unroll
      for (int io = 0; io < 4; ++io)
#pragma unroll
        for (int e = 0; e < 4; ++e) vd[(size_t)(16 * io + 4 * g4 + e) * kDim + colw + l16] = VN[io][e];
    }

    // -- output: o = r * (q S_hi) + Aqk bf16(v_new) ----------------------------
    if constexpr (COMPUTE_O) {
      u16x8 VNb[2];
#pragma unroll
      for (int io = 0; io < 4; ++io)
#pragma unroll
        for (int e = 0; e < 4; ++e) VNb[io >> 1][(io & 1) * 4 + e] = f2bf(VN[io][e]);
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        f32x4 O = {0.f, 0.f, 0.f, 0.f};
        const uint16_t* row = sq + (16 * it + l16) * kLdRow + 4 * g4;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const u16x8 av = cat4(*reinterpret_cast<const u16x4*>(row + 32 * s),
                                *reinterpret_cast<const u16x4*>(row + 32 * s + 16));
          O = mfma16(av, Shi[s], O);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) O[e] *= sR[16 * it + 4 * g4 + e];
        const uint16_t* arow = sAqk + (16 * it + l16) * kLdT + 4 * g4;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const u16x8 av = cat4(*reinterpret_cast<const u16x4*>(arow + 32 * s),
                                *reinterpret_cast<const u16x4*>(arow + 32 * s + 16));
          O = mfma16(av, VNb[s], O);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) sO[(16 * it + 4 * g4 + e) * kLdV + w * 16 + l16] = f2bf(O[e]);
      }
    }

    // -- state update: S <- exp(G_last) S + k^T (d * v_new) --------------------
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
      const float dec = sDecay;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        f32x4 acc = S[t] * dec;
        const uint16_t* row = skT + (16 * t + l16) * kLdT + 4 * g4;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const u16x8 av = cat4(*reinterpret_cast<const u16x4*>(row + 32 * s),
                                *reinterpret_cast<const u16x4*>(row + 32 * s + 16));
          acc = mfma16(av, Zhi[s], acc);
          acc = mfma16(av, Zlo[s], acc);
        }
        S[t] = acc;
      }
    }
    __syncthreads();

    if constexpr (COMPUTE_O) {
      constexpr int NOU = 64 * BV / 8;  // uint4 of the o block
      for (int idx = tid; idx < NOU; idx += NTH) {
        const int r = idx / (BV / 8), cu = idx - r * (BV / 8);
        if (r < len)
          *reinterpret_cast<uint4*>(a.o + ((size_t)(tok0 + r) * H + h) * kDim + vb * BV + cu * 8) =
              *reinterpret_cast<const uint4*>(sO + r * kLdV + cu * 8);
      }
    }
  }

  if (a.sfinal) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) a.sfinal[sbase + (size_t)(16 * t + 4 * g4 + e) * kDim + colw + l16] = S[t][e];
  }
}

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

constexpr int kFwdWaves = 4;

hipError_t launch_fwd(bool kda, bool store_h, bool compute_o, const FwdArgs& a, hipStream_t stream) {
  if (kda) return launch_kda_fwd(store_h, compute_o, a, stream);
  dim3 grid(a.geo.N * a.H, kDim / (16 * kFwdWaves));
  dim3 block(64 * kFwdWaves);
  if (store_h && !compute_o)
    hipLaunchKernelGGL((gdn_fwd_kernel<kFwdWaves, true, false>), grid, block, 0, stream, a);
  else if (!store_h && compute_o)
    hipLaunchKernelGGL((gdn_fwd_kernel<kFwdWaves, false, true>), grid, block, 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_finalize(bool kda, const FinArgs& a, hipStream_t stream) {
  if (kda) return launch_kda_finalize(a, stream);
  dim3 grid(a.geo.NT, a.H);
  hipLaunchKernelGGL(gdn_finalize_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gdn
