// State kernel (GDN): the sequential chunk pass (chunk_fwd_h), fused with the
// output (finalize) for the whole-pass entry. One workgroup per (sequence,
// head, V-block of 16*NWC columns) with two kinds of waves:
//   - NWC compute waves, each holding a 128 x 16 block of the fp32 K x V state
//     in MFMA accumulators and running the chunk recurrence;
//   - kLoaders loader waves that, while the compute waves work on chunk c out
//     of one LDS buffer, stage chunk c+1 into the other (q, k rows, T split
//     into bf16 hi/lo, Aqk, v transposed, per-row vectors) and write the
//     output rows of chunk c-1 to HBM.
// One workgroup barrier per chunk.
//
// Per chunk, with S the state entering it (hyper-parallel "Diff Coverage"
// page, gate build 2026-09-10, _run_prepared_gdn_chunks and the state update
// of torch_chunk_gated_delta_rule):
//   v_new = U - W S = T (beta v - c * (k S)),     c = beta * rk * exp(G)
//   o     = (q * r) S + Aqk v_new,                r = scale * rq * exp(G)
//   S    <- exp(G_last) S + k^T (d * v_new),      d = rk * exp(G_last - G)
// k, q and v enter the MFMAs as the exact bf16 inputs; the operands that
// carry the state (S in k S, T and the right-hand side in T(...), d * v_new
// in the update) are bf16 hi + lo pairs with fp32 accumulation.
//
// LDS layouts. An MFMA 16x16x32 contraction step s takes, in lane group g4,
// the contraction indices 32s + 4 g4 + (0..3) and 32s + 16 + 4 g4 + (0..3):
// those are the accumulator rows the B operand (S, Y or Z) already holds in
// registers. Matrices read as A operands store their columns permuted so that
// these eight indices are adjacent (one 16-byte read):
//   column 32s + 16h + 4g + e  ->  position 32s + 8g + 4h + e.
// k^T for the state update is read from the same row-major k with the
// transposing LDS read (ds_read_b64_tr_b16).
#include "gdn_state_common.h"

namespace gdn {

namespace {
using namespace st;

constexpr int kLoaders = 4;              // loader waves per workgroup
constexpr int kLdK = kDim + 8;           // k, q rows (permuted columns), bf16
constexpr int kLdT2 = 2 * kChunk + 8;    // T rows: hi | lo (permuted), bf16
constexpr int kLdA = kChunk + 8;         // Aqk rows (permuted), bf16
constexpr int kLdVT = kChunk + 8;        // v^T rows (chunk rows in order), bf16

template <int NWC>
struct alignas(16) Smem {
  static constexpr int BV = 16 * NWC;
  static constexpr int kLdO = BV + 8;
  struct alignas(16) Buf {
    uint16_t k[kChunk * kLdK];
    uint16_t q[kChunk * kLdK];
    uint16_t t[kChunk * kLdT2];
    uint16_t aqk[kChunk * kLdA];
    uint16_t vt[BV * kLdVT];
    float vec[4 * kChunk];
    float dec[4];
  };
  Buf buf[2];
  uint16_t o[2][kChunk * kLdO];
};

}  // namespace

template <int NWC, bool STORE_H, bool COMPUTE_O>
__global__ __launch_bounds__((NWC + kLoaders) * 64) void gdn_state_kernel(FwdArgs a) {
  using SM = Smem<NWC>;
  constexpr int BV = SM::BV;
  constexpr int kLdO = SM::kLdO;
  __shared__ SM sm;

  const int unit = blockIdx.x;
  const int n = unit / a.H;
  const int h = unit - n * a.H;
  const int vb = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int H = a.H;
  const SeqInfo si = a.geo.seq(n);
  const bool compute = w < NWC;

  // ------------------------------------------------------------------ loaders
  const int ltid = tid - NWC * 64;  // 0 .. 64*kLoaders-1 on loader waves
  auto stage = [&](int jc, int b) {
    typename SM::Buf& B = sm.buf[b];
    const int c = si.c0 + jc;
    const int tok0 = si.tok0 + jc * kChunk;
    const int rem = si.len - jc * kChunk;
    const int len = rem < kChunk ? rem : kChunk;
    const size_t cm = (size_t)h * a.geo.NT + c;
    constexpr int NL = 64 * kLoaders;
    // k (and q): 16-byte pieces of rows, written as two permuted halves
    uint4 kr[1024 / NL], qr[1024 / NL];
#pragma unroll
    for (int p = 0; p < 1024 / NL; ++p) {
      const int idx = p * NL + ltid;
      const int r = idx >> 4, cc = (idx & 15) * 8;
      const size_t off = ((size_t)(tok0 + r) * H + h) * kDim + cc;
      kr[p] = r < len ? *reinterpret_cast<const uint4*>(a.k + off) : make_uint4(0, 0, 0, 0);
      if constexpr (COMPUTE_O) qr[p] = r < len ? *reinterpret_cast<const uint4*>(a.q + off) : make_uint4(0, 0, 0, 0);
    }
    float4 tr[1024 / NL];
    const float* tsrc = a.tmat + cm * (kChunk * kChunk);
#pragma unroll
    for (int p = 0; p < 1024 / NL; ++p) tr[p] = reinterpret_cast<const float4*>(tsrc)[p * NL + ltid];
    uint4 ar[512 / NL];
    if constexpr (COMPUTE_O) {
      const uint16_t* asrc = a.aqk + cm * (kChunk * kChunk);
#pragma unroll
      for (int p = 0; p < 512 / NL; ++p) ar[p] = reinterpret_cast<const uint4*>(asrc)[p * NL + ltid];
    }
    // v block as 4 rows x 4 columns per thread
    constexpr int NVB = 16 * (BV / 4);  // blocks
    u16x4 vr[4];
    const int vbk = ltid;
    const int vm0 = 4 * (vbk & 15), vc0 = 4 * (vbk >> 4);
    if (vbk < NVB) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = vm0 + e;
        vr[e] = r < len ? *reinterpret_cast<const u16x4*>(a.v + ((size_t)(tok0 + r) * H + h) * kDim + vb * BV + vc0)
                        : u16x4{0, 0, 0, 0};
      }
    }
    const float* vsrc = a.vec + cm * (kVecRows * kChunk);
    float4 vecr = make_float4(0.f, 0.f, 0.f, 0.f);
    if (ltid < 64) vecr = reinterpret_cast<const float4*>(vsrc)[ltid];
    float decr = 0.f;
    if (ltid == 64) decr = vsrc[7 * kChunk];

    // ---- LDS writes
#pragma unroll
    for (int p = 0; p < 1024 / NL; ++p) {
      const int idx = p * NL + ltid;
      const int r = idx >> 4, cc = (idx & 15) * 8;
      const u16x8 kv = __builtin_bit_cast(u16x8, kr[p]);
      *reinterpret_cast<u16x4*>(B.k + r * kLdK + perm_col(cc)) = u16x4{kv[0], kv[1], kv[2], kv[3]};
      *reinterpret_cast<u16x4*>(B.k + r * kLdK + perm_col(cc + 4)) = u16x4{kv[4], kv[5], kv[6], kv[7]};
      if constexpr (COMPUTE_O) {
        const u16x8 qv = __builtin_bit_cast(u16x8, qr[p]);
        *reinterpret_cast<u16x4*>(B.q + r * kLdK + perm_col(cc)) = u16x4{qv[0], qv[1], qv[2], qv[3]};
        *reinterpret_cast<u16x4*>(B.q + r * kLdK + perm_col(cc + 4)) = u16x4{qv[4], qv[5], qv[6], qv[7]};
      }
    }
#pragma unroll
    for (int p = 0; p < 1024 / NL; ++p) {
      const int idx = p * NL + ltid;
      const int r = idx >> 4, c4 = (idx & 15) * 4;
      uint32_t h0, h1, l0, l1;
      split2(tr[p].x, tr[p].y, h0, l0);
      split2(tr[p].z, tr[p].w, h1, l1);
      *reinterpret_cast<uint2*>(B.t + r * kLdT2 + perm_col(c4)) = make_uint2(h0, h1);
      *reinterpret_cast<uint2*>(B.t + r * kLdT2 + kChunk + perm_col(c4)) = make_uint2(l0, l1);
    }
    if constexpr (COMPUTE_O) {
#pragma unroll
      for (int p = 0; p < 512 / NL; ++p) {
        const int idx = p * NL + ltid;
        const int r = idx >> 3, c8 = (idx & 7) * 8;
        const u16x8 av = __builtin_bit_cast(u16x8, ar[p]);
        *reinterpret_cast<u16x4*>(B.aqk + r * kLdA + perm_col(c8)) = u16x4{av[0], av[1], av[2], av[3]};
        *reinterpret_cast<u16x4*>(B.aqk + r * kLdA + perm_col(c8 + 4)) = u16x4{av[4], av[5], av[6], av[7]};
      }
    }
    if (vbk < NVB) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<u16x4*>(B.vt + (vc0 + j) * kLdVT + vm0) = u16x4{vr[0][j], vr[1][j], vr[2][j], vr[3][j]};
    }
    if (ltid < 64) reinterpret_cast<float4*>(B.vec)[ltid] = vecr;
    if (ltid == 64) B.dec[0] = decr;
  };

  auto store_o = [&](int jc, int b) {
    const int tok0 = si.tok0 + jc * kChunk;
    const int rem = si.len - jc * kChunk;
    const int len = rem < kChunk ? rem : kChunk;
    constexpr int NOU = 64 * BV / 8;
    for (int idx = ltid; idx < NOU; idx += 64 * kLoaders) {
      const int r = idx / (BV / 8), cu = idx - r * (BV / 8);
      if (r < len)
        *reinterpret_cast<uint4*>(a.o + ((size_t)(tok0 + r) * H + h) * kDim + vb * BV + cu * 8) =
            *reinterpret_cast<const uint4*>(sm.o[b] + r * kLdO + cu * 8);
    }
  };

  // ------------------------------------------------------------------ compute
  const int g4 = lane >> 4;
  const int l16 = lane & 15;
  const int colw = vb * BV + w * 16;
  const size_t sbase = ((size_t)n * H + h) * kDim * kDim;
  f32x4 S[8];
  if (compute) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        S[t][e] = a.s0 ? a.s0[sbase + (size_t)(16 * t + 4 * g4 + e) * kDim + colw + l16] : 0.0f;
  }
  // transposing-read lane roles: group G = lane/16, row offset j, column quad qd
  const int trG = lane >> 4, trJ = (lane >> 2) & 3, trQ = lane & 3;

  if (!compute) stage(0, 0);
  __syncthreads();

  for (int jc = 0; jc < si.nch; ++jc) {
    const int b = jc & 1;
    if (compute) {
      const typename SM::Buf& B = sm.buf[b];
      const int c = si.c0 + jc;
      const size_t cm = (size_t)h * a.geo.NT + c;

      if constexpr (STORE_H) {
        float* hd = a.h_out + cm * (kDim * kDim);
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) hd[(size_t)(16 * t + 4 * g4 + e) * kDim + colw + l16] = S[t][e];
      }

      // X = k S: contraction step s uses state tiles 2s, 2s+1 (split just
      // before use); four independent accumulators per step
      u16x8 Shi[4], Slo[4];
      f32x4 X[4];
#pragma unroll
      for (int it = 0; it < 4; ++it) X[it] = f32x4{0.f, 0.f, 0.f, 0.f};
      {
        u16x8 fk[2][4];
#pragma unroll
        for (int it = 0; it < 4; ++it)
          fk[0][it] = *reinterpret_cast<const u16x8*>(B.k + (16 * it + l16) * kLdK + 8 * g4);
        split_tiles(S[0], S[1], Shi[0], Slo[0]);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          if (s + 1 < 4) {
#pragma unroll
            for (int it = 0; it < 4; ++it)
              fk[(s + 1) & 1][it] =
                  *reinterpret_cast<const u16x8*>(B.k + (16 * it + l16) * kLdK + 32 * (s + 1) + 8 * g4);
          }
#pragma unroll
          for (int it = 0; it < 4; ++it) X[it] = mfma16(fk[s & 1][it], Shi[s], X[it]);
          if (s + 1 < 4) split_tiles(S[2 * s + 2], S[2 * s + 3], Shi[s + 1], Slo[s + 1]);
#pragma unroll
          for (int it = 0; it < 4; ++it) X[it] = mfma16(fk[s & 1][it], Slo[s], X[it]);
        }
      }

      // first half of the output, o_inter = q S_hi (independent of v_new)
      f32x4 O[4];
      if constexpr (COMPUTE_O) {
#pragma unroll
        for (int it = 0; it < 4; ++it) O[it] = f32x4{0.f, 0.f, 0.f, 0.f};
        u16x8 fq[2][4];
#pragma unroll
        for (int it = 0; it < 4; ++it)
          fq[0][it] = *reinterpret_cast<const u16x8*>(B.q + (16 * it + l16) * kLdK + 8 * g4);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          if (s + 1 < 4) {
#pragma unroll
            for (int it = 0; it < 4; ++it)
              fq[(s + 1) & 1][it] =
                  *reinterpret_cast<const u16x8*>(B.q + (16 * it + l16) * kLdK + 32 * (s + 1) + 8 * g4);
          }
#pragma unroll
          for (int it = 0; it < 4; ++it) O[it] = mfma16(fq[s & 1][it], Shi[s], O[it]);
        }
      }

      // Y = beta v - c X for tiles 2h, 2h+1 -> B operand of contraction step h
      auto make_y = [&](int hh, u16x8& yhi, u16x8& ylo) {
        f32x4 y2[2];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const int it = 2 * hh + k2;
          const u16x4 vv = *reinterpret_cast<const u16x4*>(B.vt + (16 * w + l16) * kLdVT + 16 * it + 4 * g4);
          const float4 bt = *reinterpret_cast<const float4*>(B.vec + 16 * it + 4 * g4);
          const float4 cc = *reinterpret_cast<const float4*>(B.vec + kChunk + 16 * it + 4 * g4);
          y2[k2][0] = bt.x * bf2f(vv[0]) - cc.x * X[it][0];
          y2[k2][1] = bt.y * bf2f(vv[1]) - cc.y * X[it][1];
          y2[k2][2] = bt.z * bf2f(vv[2]) - cc.z * X[it][2];
          y2[k2][3] = bt.w * bf2f(vv[3]) - cc.w * X[it][3];
        }
        split_tiles(y2[0], y2[1], yhi, ylo);
      };

      // v_new = T Y, three split products, four independent accumulators
      f32x4 VN[4];
      {
        u16x8 th[4][2], tl[4][2];
#pragma unroll
        for (int io = 0; io < 4; ++io) {
          const uint16_t* row = B.t + (16 * io + l16) * kLdT2 + 8 * g4;
          th[io][0] = *reinterpret_cast<const u16x8*>(row);
          th[io][1] = *reinterpret_cast<const u16x8*>(row + 32);
          tl[io][0] = *reinterpret_cast<const u16x8*>(row + kChunk);
          tl[io][1] = *reinterpret_cast<const u16x8*>(row + kChunk + 32);
          VN[io] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        u16x8 Yhi[2], Ylo[2];
        make_y(0, Yhi[0], Ylo[0]);
#pragma unroll
        for (int io = 0; io < 4; ++io) VN[io] = mfma16(th[io][0], Yhi[0], VN[io]);
        make_y(1, Yhi[1], Ylo[1]);
#pragma unroll
        for (int io = 0; io < 4; ++io) VN[io] = mfma16(th[io][0], Ylo[0], VN[io]);
#pragma unroll
        for (int io = 0; io < 4; ++io) VN[io] = mfma16(tl[io][0], Yhi[0], VN[io]);
#pragma unroll
        for (int io = 0; io < 4; ++io) VN[io] = mfma16(th[io][1], Yhi[1], VN[io]);
#pragma unroll
        for (int io = 0; io < 4; ++io) VN[io] = mfma16(th[io][1], Ylo[1], VN[io]);
#pragma unroll
        for (int io = 0; io < 4; ++io) VN[io] = mfma16(tl[io][1], Yhi[1], VN[io]);
      }
      if constexpr (STORE_H) {
        float* vd = a.vnew_out + cm * (kChunk * kDim);
#pragma unroll
        for (int io = 0; io < 4; ++io)
#pragma unroll
          for (int e = 0; e < 4; ++e) vd[(size_t)(16 * io + 4 * g4 + e) * kDim + colw + l16] = VN[io][e];
      }

      // state update: S <- exp(G_last) S + k^T (d * v_new), eight accumulators;
      // contraction step s uses v_new tiles 2s, 2s+1
      auto make_z = [&](int hh, u16x8& zhi, u16x8& zlo) {
        f32x4 z2[2];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const int io = 2 * hh + k2;
          const float4 dd = *reinterpret_cast<const float4*>(B.vec + 2 * kChunk + 16 * io + 4 * g4);
          z2[k2][0] = dd.x * VN[io][0];
          z2[k2][1] = dd.y * VN[io][1];
          z2[k2][2] = dd.z * VN[io][2];
          z2[k2][3] = dd.w * VN[io][3];
        }
        split_tiles(z2[0], z2[1], zhi, zlo);
      };
      {
        u16x8 ak[2][8];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const uint16_t* col = B.k + perm_col(16 * t + 4 * trQ);
            const u16x4 r0 = tr_read(col + (32 * s + 4 * trG + trJ) * kLdK);
            const u16x4 r1 = tr_read(col + (32 * s + 16 + 4 * trG + trJ) * kLdK);
            ak[s][t] = cat4(r0, r1);
          }
        const float dec = B.dec[0];
        u16x8 Zhi[2], Zlo[2];
        make_z(0, Zhi[0], Zlo[0]);
#pragma unroll
        for (int t = 0; t < 8; ++t) S[t] = mfma16(ak[0][t], Zhi[0], S[t] * dec);
        make_z(1, Zhi[1], Zlo[1]);
#pragma unroll
        for (int t = 0; t < 8; ++t) S[t] = mfma16(ak[0][t], Zlo[0], S[t]);
#pragma unroll
        for (int t = 0; t < 8; ++t) S[t] = mfma16(ak[1][t], Zhi[1], S[t]);
#pragma unroll
        for (int t = 0; t < 8; ++t) S[t] = mfma16(ak[1][t], Zlo[1], S[t]);
      }

      // second half of the output: o = r * o_inter + Aqk bf16(v_new)
      if constexpr (COMPUTE_O) {
        u16x8 VNb[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          u32x4 p;
          p[0] = pack2(VN[2 * hh][0], VN[2 * hh][1]);
          p[1] = pack2(VN[2 * hh][2], VN[2 * hh][3]);
          p[2] = pack2(VN[2 * hh + 1][0], VN[2 * hh + 1][1]);
          p[3] = pack2(VN[2 * hh + 1][2], VN[2 * hh + 1][3]);
          VNb[hh] = __builtin_bit_cast(u16x8, p);
        }
        u16x8 fa[4][2];
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const uint16_t* arow = B.aqk + (16 * it + l16) * kLdA + 8 * g4;
          fa[it][0] = *reinterpret_cast<const u16x8*>(arow);
          fa[it][1] = *reinterpret_cast<const u16x8*>(arow + 32);
          const float4 rr = *reinterpret_cast<const float4*>(B.vec + 3 * kChunk + 16 * it + 4 * g4);
          O[it][0] *= rr.x; O[it][1] *= rr.y; O[it][2] *= rr.z; O[it][3] *= rr.w;
        }
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int it = 0; it < 4; ++it) O[it] = mfma16(fa[it][s], VNb[s], O[it]);
#pragma unroll
        for (int it = 0; it < 4; ++it)
#pragma unroll
          for (int e = 0; e < 4; ++e) sm.o[b][(16 * it + 4 * g4 + e) * kLdO + w * 16 + l16] = bfr(O[it][e]);
      }
    } else {
      if constexpr (COMPUTE_O) {
        if (jc >= 1) store_o(jc - 1, b ^ 1);
      }
      if (jc + 1 < si.nch) stage(jc + 1, b ^ 1);
    }
    __syncthreads();
  }

  if (compute) {
    if (a.sfinal) {
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) a.sfinal[sbase + (size_t)(16 * t + 4 * g4 + e) * kDim + colw + l16] = S[t][e];
    }
  } else {
    if constexpr (COMPUTE_O) {
      if (si.nch >= 1) store_o(si.nch - 1, (si.nch - 1) & 1);
    }
  }
}

constexpr int kStateComputeWaves = 2;

hipError_t launch_gdn_state(bool store_h, bool compute_o, const FwdArgs& a, hipStream_t stream) {
  constexpr int NWC = kStateComputeWaves;
  dim3 grid(a.geo.N * a.H, kDim / (16 * NWC));
  dim3 block(64 * (NWC + kLoaders));
  if (store_h && !compute_o)
    hipLaunchKernelGGL((gdn_state_kernel<NWC, true, false>), grid, block, 0, stream, a);
  else if (!store_h && compute_o)
    hipLaunchKernelGGL((gdn_state_kernel<NWC, false, true>), grid, block, 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace gdn
