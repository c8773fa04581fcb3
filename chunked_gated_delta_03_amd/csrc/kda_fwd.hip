// Kimi Delta Attention state kernel (per-key-channel log2 gate): the
// sequential chunk pass, optionally fused with the output. One workgroup per
// (sequence, head, V-block of 16*NWC columns): NWC compute waves hold the
// K x V state (each 128 x 16, MFMA accumulators) and run the recurrence;
// kLoaders loader waves build the operands of chunk c+1 in registers while
// chunk c is computed, then write them into LDS between two barriers.
//
// Per chunk, with S (K x V) the state entering it, G the chunk-local
// cumulative log2 gate per channel (written by the prepare kernel) and
//   kd = k * 2^G,   kg = k * 2^(G_last - G),   qd = q * 2^G   (elementwise),
// the GDN chunk form of the hyper-parallel "Diff Coverage" page (gate build
// 2026-09-10, _run_prepared_gdn_chunks) with every decay per channel reads:
//   v_new = T (beta v - (beta rk) * (kd S))
//   o     = (scale rq) * (qd S) + Aqk v_new
//   S    <- diag(2^G_last) S + kg^T (rk * v_new)
// kd, kg (bf16 hi + lo), S and the right-hand sides that carry the state
// use split products as in the GDN kernel.
#include "gdn_state_common.h"

namespace gdn {

namespace {
using namespace st;
constexpr int kLdRow = kDim + 8;   // bf16 row stride, 64 x 128 tiles (permuted columns)
constexpr int kLdT = kChunk + 8;   // bf16 row stride, 64 x 64 tiles
constexpr int kLdT2 = 2 * kChunk + 8;
constexpr int kLoadersK = 4;

template <int NWC>
struct alignas(16) KdaSmem {
  static constexpr int BV = 16 * NWC;
  static constexpr int kLdO = BV + 8;
  uint16_t kdh[kChunk * kLdRow];
  uint16_t kdl[kChunk * kLdRow];
  uint16_t kgh[kChunk * kLdRow];
  uint16_t kgl[kChunk * kLdRow];
  uint16_t qd[kChunk * kLdRow];
  uint16_t t[kChunk * kLdT2];
  uint16_t aqk[kChunk * kLdT];
  uint16_t vt[BV * kLdT];
  float vec[4 * kChunk];
  float dec[kDim];
  uint16_t o[2][kChunk * kLdO];
};
}  // namespace

template <int NWC, bool STORE_H, bool COMPUTE_O>
__global__ __launch_bounds__((NWC + kLoadersK) * 64) void kda_state_kernel(FwdArgs a) {
  using SM = KdaSmem<NWC>;
  constexpr int BV = SM::BV;
  constexpr int kLdO = SM::kLdO;
  constexpr int NL = 64 * kLoadersK;
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
  const int ltid = tid - NWC * 64;

  // ---------------------------------------------------------------- loaders
  // thread block of the elementwise k/q/G work: rows m0..m0+3, channels d0..d0+7
  const int m0 = 4 * (ltid & 15), d0 = 8 * (ltid >> 4);
  uint32_t rkdh[4][4], rkdl[4][4], rkgh[4][4], rkgl[4][4], rqd[4][4];
  uint4 rt[1024 / NL];
  uint4 ra[512 / NL];
  u16x4 rv[4];
  float4 rvec;
  float rdec;
  const int vm0 = 4 * (ltid & 15), vc0 = 4 * (ltid >> 4);
  constexpr int NVB = 16 * (BV / 4);

  auto build = [&](int jc) {
    const int c = si.c0 + jc;
    const int tok0 = si.tok0 + jc * kChunk;
    const int rem = si.len - jc * kChunk;
    const int len = rem < kChunk ? rem : kChunk;
    const size_t cm = (size_t)h * a.geo.NT + c;
    const float* gk = a.gk + cm * (kChunk * kDim);
    float glast[8];
    {
      const float4 x0 = *reinterpret_cast<const float4*>(gk + 63 * kDim + d0);
      const float4 x1 = *reinterpret_cast<const float4*>(gk + 63 * kDim + d0 + 4);
      glast[0] = x0.x; glast[1] = x0.y; glast[2] = x0.z; glast[3] = x0.w;
      glast[4] = x1.x; glast[5] = x1.y; glast[6] = x1.z; glast[7] = x1.w;
    }
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
#pragma unroll
      for (int pr = 0; pr < 4; ++pr) {
        const float k0 = __uint_as_float(kw[pr] << 16), k1 = __uint_as_float(kw[pr] & 0xFFFF0000u);
        const float q0 = __uint_as_float(qw[pr] << 16), q1 = __uint_as_float(qw[pr] & 0xFFFF0000u);
        const float fd0 = exp2f(gv[2 * pr]), fd1 = exp2f(gv[2 * pr + 1]);
        const float fg0 = exp2f(glast[2 * pr] - gv[2 * pr]), fg1 = exp2f(glast[2 * pr + 1] - gv[2 * pr + 1]);
        split2(k0 * fd0, k1 * fd1, rkdh[rr][pr], rkdl[rr][pr]);
        split2(k0 * fg0, k1 * fg1, rkgh[rr][pr], rkgl[rr][pr]);
        rqd[rr][pr] = pack2(q0 * fd0, q1 * fd1);
      }
    }
    const uint16_t* tsrc = a.tmat + cm * (kChunk * 2 * kChunk);
#pragma unroll
    for (int p = 0; p < 1024 / NL; ++p) rt[p] = reinterpret_cast<const uint4*>(tsrc)[p * NL + ltid];
    if constexpr (COMPUTE_O) {
      const uint16_t* asrc = a.aqk + cm * (kChunk * kChunk);
#pragma unroll
      for (int p = 0; p < 512 / NL; ++p) ra[p] = reinterpret_cast<const uint4*>(asrc)[p * NL + ltid];
    }
    if (ltid < NVB) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = vm0 + e;
        rv[e] = r < len ? *reinterpret_cast<const u16x4*>(a.v + ((size_t)(tok0 + r) * H + h) * kDim + vb * BV + vc0)
                        : u16x4{0, 0, 0, 0};
      }
    }
    const float* vsrc = a.vec + cm * (kVecRows * kChunk);
    if (ltid < 64) rvec = reinterpret_cast<const float4*>(vsrc)[ltid];
    if (ltid < kDim) rdec = exp2f(gk[63 * kDim + ltid]);
  };

  auto write = [&]() {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int off = (m0 + rr) * kLdRow;
      const int p0 = perm_col(d0), p1 = perm_col(d0 + 4);
      *reinterpret_cast<uint2*>(sm.kdh + off + p0) = make_uint2(rkdh[rr][0], rkdh[rr][1]);
      *reinterpret_cast<uint2*>(sm.kdh + off + p1) = make_uint2(rkdh[rr][2], rkdh[rr][3]);
      *reinterpret_cast<uint2*>(sm.kdl + off + p0) = make_uint2(rkdl[rr][0], rkdl[rr][1]);
      *reinterpret_cast<uint2*>(sm.kdl + off + p1) = make_uint2(rkdl[rr][2], rkdl[rr][3]);
      *reinterpret_cast<uint2*>(sm.kgh + off + p0) = make_uint2(rkgh[rr][0], rkgh[rr][1]);
      *reinterpret_cast<uint2*>(sm.kgh + off + p1) = make_uint2(rkgh[rr][2], rkgh[rr][3]);
      *reinterpret_cast<uint2*>(sm.kgl + off + p0) = make_uint2(rkgl[rr][0], rkgl[rr][1]);
      *reinterpret_cast<uint2*>(sm.kgl + off + p1) = make_uint2(rkgl[rr][2], rkgl[rr][3]);
      if constexpr (COMPUTE_O) {
        *reinterpret_cast<uint2*>(sm.qd + off + p0) = make_uint2(rqd[rr][0], rqd[rr][1]);
        *reinterpret_cast<uint2*>(sm.qd + off + p1) = make_uint2(rqd[rr][2], rqd[rr][3]);
      }
    }
    // T (hi | lo) and Aqk arrive with permuted columns: plain row copies
#pragma unroll
    for (int p = 0; p < 1024 / NL; ++p) {
      const int idx = p * NL + ltid;
      *reinterpret_cast<uint4*>(sm.t + (idx >> 4) * kLdT2 + 8 * (idx & 15)) = rt[p];
    }
    if constexpr (COMPUTE_O) {
#pragma unroll
      for (int p = 0; p < 512 / NL; ++p) {
        const int idx = p * NL + ltid;
        *reinterpret_cast<uint4*>(sm.aqk + (idx >> 3) * kLdT + 8 * (idx & 7)) = ra[p];
      }
    }
    if (ltid < NVB) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<u16x4*>(sm.vt + (vc0 + j) * kLdT + vm0) = u16x4{rv[0][j], rv[1][j], rv[2][j], rv[3][j]};
    }
    if (ltid < 64) reinterpret_cast<float4*>(sm.vec)[ltid] = rvec;
    if (ltid < kDim) sm.dec[ltid] = rdec;
  };

  auto store_o = [&](int jc, int b) {
    const int tok0 = si.tok0 + jc * kChunk;
    const int rem = si.len - jc * kChunk;
    const int len = rem < kChunk ? rem : kChunk;
    constexpr int NOU = 64 * BV / 8;
    for (int idx = ltid; idx < NOU; idx += NL) {
      const int r = idx / (BV / 8), cu = idx - r * (BV / 8);
      if (r < len)
        *reinterpret_cast<uint4*>(a.o + ((size_t)(tok0 + r) * H + h) * kDim + vb * BV + cu * 8) =
            *reinterpret_cast<const uint4*>(sm.o[b] + r * kLdO + cu * 8);
    }
  };

  // ---------------------------------------------------------------- compute
  const int g4 = lane >> 4;
  const int l16 = lane & 15;
  const int colw = vb * BV + w * 16;
  const size_t sbase = ((size_t)n * H + h) * kDim * kDim;
  const int trG = lane >> 4, trJ = (lane >> 2) & 3, trQ = lane & 3;
  // The two roles run separate loops with the same barrier sequence (two
  // barriers per chunk), so their loop-carried registers never overlap.
  if (!compute) {
    build(0);
    write();
    __syncthreads();
    for (int jc = 0; jc < si.nch; ++jc) {
      if constexpr (COMPUTE_O) {
        if (jc >= 1) store_o(jc - 1, (jc - 1) & 1);
      }
      if (jc + 1 < si.nch) build(jc + 1);
      __syncthreads();
      if (jc + 1 < si.nch) write();
      __syncthreads();
    }
    if constexpr (COMPUTE_O) {
      if (si.nch >= 1) store_o(si.nch - 1, (si.nch - 1) & 1);
    }
    return;
  }

  f32x4 S[8];
  u16x8 Shi[4], Slo[4];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      S[t][e] = a.s0 ? a.s0[sbase + (size_t)(16 * t + 4 * g4 + e) * kDim + colw + l16] : 0.0f;
#pragma unroll
  for (int s = 0; s < 4; ++s) split_tiles(S[2 * s], S[2 * s + 1], Shi[s], Slo[s]);
  __syncthreads();

  for (int jc = 0; jc < si.nch; ++jc) {
    const int b = jc & 1;
    {
      const int c = si.c0 + jc;
      const size_t cm = (size_t)h * a.geo.NT + c;
      if constexpr (STORE_H) {
        float* hd = a.h_out + cm * (kDim * kDim);
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) hd[(size_t)(16 * t + 4 * g4 + e) * kDim + colw + l16] = S[t][e];
      }

      // X = kd S (three split products), four accumulators
      f32x4 X[4];
#pragma unroll
      for (int it = 0; it < 4; ++it) X[it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u16x8 fh[4], fl[4];
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          fh[it] = *reinterpret_cast<const u16x8*>(sm.kdh + (16 * it + l16) * kLdRow + 32 * s + 8 * g4);
          fl[it] = *reinterpret_cast<const u16x8*>(sm.kdl + (16 * it + l16) * kLdRow + 32 * s + 8 * g4);
        }
#pragma unroll
        for (int it = 0; it < 4; ++it) X[it] = mfma16(fh[it], Shi[s], X[it]);
#pragma unroll
        for (int it = 0; it < 4; ++it) X[it] = mfma16(fh[it], Slo[s], X[it]);
#pragma unroll
        for (int it = 0; it < 4; ++it) X[it] = mfma16(fl[it], Shi[s], X[it]);
      }

      // o_inter = qd S_hi
      f32x4 O[4];
      if constexpr (COMPUTE_O) {
#pragma unroll
        for (int it = 0; it < 4; ++it) O[it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          u16x8 fq[4];
#pragma unroll
          for (int it = 0; it < 4; ++it)
            fq[it] = *reinterpret_cast<const u16x8*>(sm.qd + (16 * it + l16) * kLdRow + 32 * s + 8 * g4);
#pragma unroll
          for (int it = 0; it < 4; ++it) O[it] = mfma16(fq[it], Shi[s], O[it]);
        }
      }

      // Y = beta v - (beta rk) X, then v_new = T Y
      auto make_y = [&](int hh, u16x8& yhi, u16x8& ylo) {
        f32x4 y2[2];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const int it = 2 * hh + k2;
          const u16x4 vv = *reinterpret_cast<const u16x4*>(sm.vt + (16 * w + l16) * kLdT + 16 * it + 4 * g4);
          const float4 bt = *reinterpret_cast<const float4*>(sm.vec + 16 * it + 4 * g4);
          const float4 cc = *reinterpret_cast<const float4*>(sm.vec + kChunk + 16 * it + 4 * g4);
          y2[k2][0] = bt.x * bf2f(vv[0]) - cc.x * X[it][0];
          y2[k2][1] = bt.y * bf2f(vv[1]) - cc.y * X[it][1];
          y2[k2][2] = bt.z * bf2f(vv[2]) - cc.z * X[it][2];
          y2[k2][3] = bt.w * bf2f(vv[3]) - cc.w * X[it][3];
        }
        split_tiles(y2[0], y2[1], yhi, ylo);
      };
      f32x4 VN[4];
      {
        u16x8 th[4][2], tl[4][2];
#pragma unroll
        for (int io = 0; io < 4; ++io) {
          const uint16_t* row = sm.t + (16 * io + l16) * kLdT2 + 8 * g4;
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

      // output second half first (it only needs v_new): o = r o_inter + Aqk v_new
      if constexpr (COMPUTE_O) {
        const u16x8 vnb0 = pack_tiles(VN[0], VN[1]);
        const u16x8 vnb1 = pack_tiles(VN[2], VN[3]);
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const uint16_t* arow = sm.aqk + (16 * it + l16) * kLdT + 8 * g4;
          const float4 rr = *reinterpret_cast<const float4*>(sm.vec + 3 * kChunk + 16 * it + 4 * g4);
          O[it][0] *= rr.x; O[it][1] *= rr.y; O[it][2] *= rr.z; O[it][3] *= rr.w;
          O[it] = mfma16(*reinterpret_cast<const u16x8*>(arow), vnb0, O[it]);
          O[it] = mfma16(*reinterpret_cast<const u16x8*>(arow + 32), vnb1, O[it]);
        }
#pragma unroll
        for (int it = 0; it < 4; ++it)
#pragma unroll
          for (int e = 0; e < 4; ++e) sm.o[b][(16 * it + 4 * g4 + e) * kLdO + w * 16 + l16] = bfr(O[it][e]);
      }

      // S <- diag(2^G_last) S + kg^T (rk * v_new), three split products
      {
        u16x8 Zhi[2], Zlo[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          f32x4 z2[2];
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            const int io = 2 * hh + k2;
            const float4 dd = *reinterpret_cast<const float4*>(sm.vec + 2 * kChunk + 16 * io + 4 * g4);
            z2[k2][0] = dd.x * VN[io][0];
            z2[k2][1] = dd.y * VN[io][1];
            z2[k2][2] = dd.z * VN[io][2];
            z2[k2][3] = dd.w * VN[io][3];
          }
          split_tiles(z2[0], z2[1], Zhi[hh], Zlo[hh]);
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float4 dv = *reinterpret_cast<const float4*>(sm.dec + 16 * t + 4 * g4);
          S[t][0] *= dv.x; S[t][1] *= dv.y; S[t][2] *= dv.z; S[t][3] *= dv.w;
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          u16x8 gh[8], gl[8];
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const int pc = perm_col(16 * t + 4 * trQ);
            const int r0 = (32 * s + 4 * trG + trJ) * kLdRow + pc;
            const int r1 = (32 * s + 16 + 4 * trG + trJ) * kLdRow + pc;
            gh[t] = cat4(tr_read(sm.kgh + r0), tr_read(sm.kgh + r1));
            gl[t] = cat4(tr_read(sm.kgl + r0), tr_read(sm.kgl + r1));
          }
#pragma unroll
          for (int t = 0; t < 8; ++t) S[t] = mfma16(gh[t], Zhi[s], S[t]);
#pragma unroll
          for (int t = 0; t < 8; ++t) S[t] = mfma16(gh[t], Zlo[s], S[t]);
#pragma unroll
          for (int t = 0; t < 8; ++t) S[t] = mfma16(gl[t], Zhi[s], S[t]);
        }
      }
    }
    __syncthreads();
    // split the new state for the next chunk while the loaders write LDS
#pragma unroll
    for (int s = 0; s < 4; ++s) split_tiles(S[2 * s], S[2 * s + 1], Shi[s], Slo[s]);
    __syncthreads();
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

constexpr int kKdaComputeWaves = 2;

hipError_t launch_kda_fwd(bool store_h, bool compute_o, const FwdArgs& a, hipStream_t stream) {
  constexpr int NWC = kKdaComputeWaves;
  dim3 grid(a.geo.N * a.H, kDim / (16 * NWC));
  dim3 block(64 * (NWC + kLoadersK));
  if (store_h && !compute_o)
    hipLaunchKernelGGL((kda_state_kernel<NWC, true, false>), grid, block, 0, stream, a);
  else if (!store_h && compute_o)
    hipLaunchKernelGGL((kda_state_kernel<NWC, false, true>), grid, block, 0, stream, a);
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
