// Kimi Delta Attention state kernel (per-key-channel log2 gate): the
// sequential chunk pass, optionally fused with the output. One workgroup per
// (sequence, head, V-block of 16*NCB columns) with two kinds of waves:
//   - 2*NCB compute waves. Each 16-column slice of the fp32 K x V state is
//     held by a pair of waves, one per half of the K rows (64 x 16 each, in
//     MFMA accumulators); the pair exchanges its partial K-contractions
//     through LDS, as in the GDN state kernel;
//   - loader waves (8 in the whole pass, else 4) that stage the chunk's
//     decayed operands: in the whole pass they copy them from the prepare
//     kernel's output; in the stage entry they form them from k, q and the
//     cumulative gate.
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
// use split products as in the GDN kernel; qd is a single bf16 operand.
//
// LDS holds one chunk of most operands (the decayed operands alone are 80 KiB,
// too much to double-buffer). Each such array is rewritten for the next chunk
// only while the compute waves do not read it: kd and qd are read before the
// pair barrier, so the loaders write the next chunk's after it; Aqk, v and kg
// are read after the pair barrier, so the loaders write the next chunk's
// between the end of a chunk and the next pair barrier. T, the row vectors
// and the channel decays (read after the pair barrier) have two buffers in
// the whole pass and are written after the pair barrier with kd and qd: LDS
// writes before that barrier compete with the compute waves' reads there. Layouts and the state-row permutation are those of the GDN state
// kernel: 16-byte pieces of 256-byte rows at slot p ^ (r & 15), the
// transposed-read kg rows at p ^ kswz(r) (Aqk rows: p ^ ((r >> 1) & 7), v
// rows: p ^ vswz(r)), row i of state tile t is K index perm_col(16 t + i).
#include <type_traits>

#include "gdn_state_common.h"

namespace gdn {

namespace {
using namespace st;

// Loader waves per workgroup: 8 in the whole pass (its loaders' LDS stores
// sit nearly on the chunk's critical path; state kernel 375 -> 342 us on the
// B=2 T=8192 H=32 workload), 4 in the other forms, whose larger register sets
// would spill at 12 waves per workgroup.
__host__ __device__ constexpr int loaders_k(bool store_h, bool compute_o) { return (compute_o && !store_h) ? 8 : 4; }

template <int NCB>
struct alignas(16) KSmem {
  static constexpr int BV = 16 * NCB;
  static constexpr int NCW = 2 * NCB;    // compute waves
  uint16_t kdh[kChunk * kDim];           // k 2^G, hi and lo
  uint16_t kdl[kChunk * kDim];
  uint16_t qd[kChunk * kDim];            // q 2^G
  uint16_t kgh[kChunk * kDim];           // k 2^(G_last - G), hi and lo
  uint16_t kgl[kChunk * kDim];
  // T, the row vectors and the channel decays have two buffers (chunk
  // parity) in the whole pass, so the loaders write the next chunk's after
  // the pair barrier; the stage entry uses buffer 0 only
  uint16_t t[2][kChunk * 2 * kChunk];    // T hi | lo (permuted columns)
  uint16_t aqk[kChunk * kChunk];         // permuted columns
  uint16_t v[kChunk * BV];               // v rows of this V-block
  float vec[2][kVecRows * kChunk];
  float dec[2][kDim];                    // 2^G_last per channel
  f32x4 xch[NCW][6][64];
  uint16_t o[NCW][32 * 16];
};

}  // namespace

template <int NCB, bool STORE_H, bool COMPUTE_O>
__global__ __launch_bounds__((2 * NCB + loaders_k(STORE_H, COMPUTE_O)) * 64) void kda_state_kernel(FwdArgs a) {
  using SM = KSmem<NCB>;
  constexpr int BV = SM::BV;
  constexpr int NCW = SM::NCW;
  __shared__ SM sm;

  int n, h, vb;
  if (!state_unit(a.geo, a.H, kDim / (16 * NCB), n, h, vb)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = a.H;
  const SeqInfo si = a.geo.seq(n);
  const int last = si.nch - 1;

  // ------------------------------------------------------------- loaders
  if constexpr (COMPUTE_O) {
    if (w >= NCW && a.kdec) {
      // Whole pass with a.kdec: the decayed operands come from the prepare kernel; the
      // loaders copy them (16-byte pieces, loaded one chunk ahead) into the
      // same windows as below.
      constexpr int NL = 64 * loaders_k(STORE_H, COMPUTE_O);
      constexpr int PPR = BV / 8;
      const int ltid = tid - NCW * 64;
      const int pc = ltid & 15;
      // two register sets: the arrays written before the pair barrier (kg,
      // Aqk, v) and those written after it (kd, qd, T, row vectors, decays),
      // each loaded one chunk ahead in the window in which it is written
      u32x4 dh[1024 / NL], dl[1024 / NL], qq[1024 / NL], tr[1024 / NL], er, dr;  // after the barrier
      u32x4 gh[1024 / NL], gl[1024 / NL], ar[512 / NL], vr;                       // before it
      auto chunk_at = [&](int jc, int& tok0, int& len, size_t& cm) {
        tok0 = si.tok0 + jc * kChunk;
        const int rem = si.len - jc * kChunk;
        len = rem < kChunk ? rem : kChunk;
        cm = (size_t)h * a.geo.NT + si.c0 + jc;
      };
      auto fetch_early = [&](int jc) {
        int tok0, len;
        size_t cm;
        chunk_at(jc, tok0, len, cm);
        const uint16_t* kd = a.kdec + cm * kKdecElems;
#pragma unroll
        for (int p = 0; p < 1024 / NL; ++p) {
          const int idx = p * NL + ltid;
          dh[p] = reinterpret_cast<const u32x4*>(kd + kKdecKdh)[idx];
          dl[p] = reinterpret_cast<const u32x4*>(kd + kKdecKdl)[idx];
          qq[p] = reinterpret_cast<const u32x4*>(kd + kKdecQd)[idx];
          tr[p] = reinterpret_cast<const u32x4*>(a.tmat + cm * (kChunk * 2 * kChunk))[idx];
        }
        if (ltid < kVecRows * kChunk / 4) er = reinterpret_cast<const u32x4*>(a.vec + cm * (kVecRows * kChunk))[ltid];
        if (ltid < kDim / 4) dr = reinterpret_cast<const u32x4*>(kd + kKdecDec)[ltid];
      };
      auto fetch_late = [&](int jc) {
        int tok0, len;
        size_t cm;
        chunk_at(jc, tok0, len, cm);
        const uint16_t* kd = a.kdec + cm * kKdecElems;
#pragma unroll
        for (int p = 0; p < 1024 / NL; ++p) {
          const int idx = p * NL + ltid;
          gh[p] = reinterpret_cast<const u32x4*>(kd + kKdecKgh)[idx];
          gl[p] = reinterpret_cast<const u32x4*>(kd + kKdecKgl)[idx];
        }
#pragma unroll
        for (int p = 0; p < 512 / NL; ++p) ar[p] = reinterpret_cast<const u32x4*>(a.aqk + cm * (kChunk * kChunk))[p * NL + ltid];
        if (ltid < 64 * PPR) {
          const int r = ltid / PPR;
          vr = (r < len && !a.s_identity) ? *reinterpret_cast<const u32x4*>(a.v + ((size_t)(tok0 + r) * H + h) * kDim + vb * BV + 8 * (ltid % PPR))
                                          : u32x4{0, 0, 0, 0};
        }
      };
      auto put_early = [&](int tb) {  // kd, qd, T, row vectors, decays of the fetched chunk
#pragma unroll
        for (int p = 0; p < 1024 / NL; ++p) {
          const int idx = p * NL + ltid, r = idx >> 4;
          const int slot = 8 * (pc ^ (r & 15));
          *reinterpret_cast<u32x4*>(sm.kdh + r * kDim + slot) = dh[p];
          *reinterpret_cast<u32x4*>(sm.kdl + r * kDim + slot) = dl[p];
          *reinterpret_cast<u32x4*>(sm.qd + r * kDim + slot) = qq[p];
          *reinterpret_cast<u32x4*>(sm.t[tb] + r * (2 * kChunk) + slot) = tr[p];
        }
        if (ltid < kVecRows * kChunk / 4) *reinterpret_cast<u32x4*>(sm.vec[tb] + 4 * ltid) = er;
        if (ltid < kDim / 4) *reinterpret_cast<u32x4*>(sm.dec[tb] + 4 * ltid) = dr;
      };
      auto put_late = [&]() {  // kg, Aqk, v of the chunk about to start
#pragma unroll
        for (int p = 0; p < 1024 / NL; ++p) {
          const int idx = p * NL + ltid, r = idx >> 4;
          const int slot = 8 * (pc ^ kswz(r));
          *reinterpret_cast<u32x4*>(sm.kgh + r * kDim + slot) = gh[p];
          *reinterpret_cast<u32x4*>(sm.kgl + r * kDim + slot) = gl[p];
        }
#pragma unroll
        for (int p = 0; p < 512 / NL; ++p) {
          const int idx = p * NL + ltid, r = idx >> 3;
          *reinterpret_cast<u32x4*>(sm.aqk + r * kChunk + 8 * ((idx & 7) ^ ((r >> 1) & 7))) = ar[p];
        }
        if (ltid < 64 * PPR) {
        const int vrow = ltid / PPR;
        *reinterpret_cast<u32x4*>(sm.v + vrow * BV + 8 * ((ltid % PPR) ^ vswz<BV>(vrow))) = vr;
      }
      };
      // same barrier sequence as the stage loaders below. During chunk jc:
      // before the pair barrier, chunk jc's kg, Aqk, v go in and chunk
      // jc+1's are loaded; after it, chunk jc+1's kd, qd, T, row vectors and
      // decays go in and chunk jc+2's are loaded (past the end the last chunk
      // is repeated, harmlessly)
      if (si.nch > 0) {
        fetch_early(0);
        fetch_late(0);
        put_early(0);
        fetch_early(min(1, last));
      }
      __syncthreads();
      for (int jc = 0; jc < si.nch; ++jc) {
        put_late();
        fetch_late(min(jc + 1, last));
        __syncthreads();
        put_early((jc + 1) & 1);
        fetch_early(min(jc + 2, last));
        __syncthreads();
      }
      return;
    }
  }
  if (w >= NCW) {
    // Stage entry: the loaders form the decayed operands from k, q and the
    // cumulative gate.
    constexpr int NL = 64 * loaders_k(STORE_H, COMPUTE_O);
    constexpr int PPR = BV / 8;              // v pieces per row
    const int ltid = tid - NCW * 64;
    const int pc = ltid & 15;                // this lane's 8-channel piece of every row
    // loaded for the next chunk
    u32x4 kr[1024 / NL], qr[1024 / NL], tr[1024 / NL], ar[512 / NL], vr, er;
    float4 g0[1024 / NL], g1[1024 / NL], gl0, gl1;
    // formed for the next chunk, written in the window after the chunk boundary
    u32x4 kgh[1024 / NL], kgl[1024 / NL];
    float4 dec0, dec1;

    // k, q and the cumulative gate of chunk jc (for its build); T, Aqk, v
    // and the row vectors of chunk jc (for its late window)
    auto fetch_kqg = [&](int jc) {
      const int tok0 = si.tok0 + jc * kChunk;
      const int rem = si.len - jc * kChunk;
      const int len = rem < kChunk ? rem : kChunk;
      const size_t cm = (size_t)h * a.geo.NT + si.c0 + jc;
      const float* gk = a.gk + cm * (kChunk * kDim);
#pragma unroll
      for (int p = 0; p < 1024 / NL; ++p) {
        const int idx = p * NL + ltid, r = idx >> 4;
        const size_t off = ((size_t)(tok0 + r) * H + h) * kDim + 8 * pc;
        kr[p] = r < len ? *reinterpret_cast<const u32x4*>(a.k + off) : u32x4{0, 0, 0, 0};
        if constexpr (COMPUTE_O) qr[p] = r < len ? *reinterpret_cast<const u32x4*>(a.q + off) : u32x4{0, 0, 0, 0};
        g0[p] = *reinterpret_cast<const float4*>(gk + r * kDim + 8 * pc);
        g1[p] = *reinterpret_cast<const float4*>(gk + r * kDim + 8 * pc + 4);
      }
      gl0 = *reinterpret_cast<const float4*>(gk + 63 * kDim + 8 * pc);
      gl1 = *reinterpret_cast<const float4*>(gk + 63 * kDim + 8 * pc + 4);
    };
    auto fetch_tav = [&](int jc) {
      const int tok0 = si.tok0 + jc * kChunk;
      const int rem = si.len - jc * kChunk;
      const int len = rem < kChunk ? rem : kChunk;
      const size_t cm = (size_t)h * a.geo.NT + si.c0 + jc;
#pragma unroll
      for (int p = 0; p < 1024 / NL; ++p) tr[p] = reinterpret_cast<const u32x4*>(a.tmat + cm * (kChunk * 2 * kChunk))[p * NL + ltid];
      if constexpr (COMPUTE_O) {
#pragma unroll
        for (int p = 0; p < 512 / NL; ++p) ar[p] = reinterpret_cast<const u32x4*>(a.aqk + cm * (kChunk * kChunk))[p * NL + ltid];
      }
      if (ltid < 64 * PPR) {
        const int r = ltid / PPR;
        vr = (r < len && !a.s_identity) ? *reinterpret_cast<const u32x4*>(a.v + ((size_t)(tok0 + r) * H + h) * kDim + vb * BV + 8 * (ltid % PPR))
                     : u32x4{0, 0, 0, 0};
      }
      if (ltid < kVecRows * kChunk / 4) er = reinterpret_cast<const u32x4*>(a.vec + cm * (kVecRows * kChunk))[ltid];
    };

    // decayed operands of the fetched chunk: kd, qd written now, kg and the
    // channel decays kept in registers for the next window
    auto build = [&]() {
      const float gla[8] = {gl0.x, gl0.y, gl0.z, gl0.w, gl1.x, gl1.y, gl1.z, gl1.w};
#pragma unroll
      for (int p = 0; p < 1024 / NL; ++p) {
        const int idx = p * NL + ltid, r = idx >> 4;
        const int slot = 8 * (pc ^ (r & 15));
        const float ga[8] = {g0[p].x, g0[p].y, g0[p].z, g0[p].w, g1[p].x, g1[p].y, g1[p].z, g1[p].w};
        const uint32_t kw[4] = {kr[p][0], kr[p][1], kr[p][2], kr[p][3]};
        const uint32_t qw[4] = {qr[p][0], qr[p][1], qr[p][2], qr[p][3]};
        u32x4 dh, dl, qq, hh, ll;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float k0 = __uint_as_float(kw[e] << 16), k1 = __uint_as_float(kw[e] & 0xFFFF0000u);
          const float q0 = __uint_as_float(qw[e] << 16), q1 = __uint_as_float(qw[e] & 0xFFFF0000u);
          const float f0 = exp2_hw(ga[2 * e]), f1 = exp2_hw(ga[2 * e + 1]);
          const float d0 = exp2_hw(gla[2 * e] - ga[2 * e]), d1 = exp2_hw(gla[2 * e + 1] - ga[2 * e + 1]);
          uint32_t xh, xl;
          split2(k0 * f0, k1 * f1, xh, xl);
          dh[e] = xh;
          dl[e] = xl;
          qq[e] = pack2(q0 * f0, q1 * f1);
          split2(k0 * d0, k1 * d1, xh, xl);
          hh[e] = xh;
          ll[e] = xl;
        }
        *reinterpret_cast<u32x4*>(sm.kdh + r * kDim + slot) = dh;
        *reinterpret_cast<u32x4*>(sm.kdl + r * kDim + slot) = dl;
        if constexpr (COMPUTE_O) *reinterpret_cast<u32x4*>(sm.qd + r * kDim + slot) = qq;
        kgh[p] = hh;
        kgl[p] = ll;
      }
      if (ltid < 16) {
        dec0 = make_float4(exp2_hw(gl0.x), exp2_hw(gl0.y), exp2_hw(gl0.z), exp2_hw(gl0.w));
        dec1 = make_float4(exp2_hw(gl1.x), exp2_hw(gl1.y), exp2_hw(gl1.z), exp2_hw(gl1.w));
      }
    };

    // kg, T, Aqk, v, row vectors and channel decays of the built chunk
    auto put_late = [&]() {
#pragma unroll
      for (int p = 0; p < 1024 / NL; ++p) {
        const int idx = p * NL + ltid, r = idx >> 4;
        const int slot = 8 * (pc ^ kswz(r));
        *reinterpret_cast<u32x4*>(sm.kgh + r * kDim + slot) = kgh[p];
        *reinterpret_cast<u32x4*>(sm.kgl + r * kDim + slot) = kgl[p];
        *reinterpret_cast<u32x4*>(sm.t[0] + r * (2 * kChunk) + 8 * (pc ^ (r & 15))) = tr[p];
      }
      if constexpr (COMPUTE_O) {
#pragma unroll
        for (int p = 0; p < 512 / NL; ++p) {
          const int idx = p * NL + ltid, r = idx >> 3;
          *reinterpret_cast<u32x4*>(sm.aqk + r * kChunk + 8 * ((idx & 7) ^ ((r >> 1) & 7))) = ar[p];
        }
      }
      if (ltid < 64 * PPR) {
        const int vrow = ltid / PPR;
        *reinterpret_cast<u32x4*>(sm.v + vrow * BV + 8 * ((ltid % PPR) ^ vswz<BV>(vrow))) = vr;
      }
      if (ltid < kVecRows * kChunk / 4) *reinterpret_cast<u32x4*>(sm.vec[0] + 4 * ltid) = er;
      if (ltid < 16) {
        *reinterpret_cast<float4*>(sm.dec[0] + 8 * ltid) = dec0;
        *reinterpret_cast<float4*>(sm.dec[0] + 8 * ltid + 4) = dec1;
      }
    };

    // Same barrier sequence as the compute waves: one before the loop, two
    // per chunk. Chunk jc's late arrays go in before its pair barrier and
    // chunk jc+1's T, Aqk, v and row vectors are loaded; after the pair
    // barrier, chunk jc+1's decayed operands are built from the k, q and gate
    // loaded a chunk earlier, and chunk jc+2's are loaded (past the end the
    // last chunk is repeated, harmlessly). Every load has a chunk to arrive.
    if (si.nch > 0) {
      fetch_kqg(0);
      fetch_tav(0);
      build();
      fetch_kqg(min(1, last));
    }
    __syncthreads();
    for (int jc = 0; jc < si.nch; ++jc) {
      put_late();
      fetch_tav(min(jc + 1, last));
      __syncthreads();
      build();
      fetch_kqg(min(jc + 2, last));
      __syncthreads();
    }
    return;
  }

  // ------------------------------------------------------------- compute
  const int cb = w >> 1;         // 16-column slice of the V-block
  auto compute = [&](auto kh_c) {
    constexpr int kh = decltype(kh_c)::value;  // half of the K rows held by this wave
    const int g4 = lane >> 4;
    const int l16 = lane & 15;
    const int colw = vb * BV + cb * 16;
    const size_t sbase = ((size_t)n * H + h) * kDim * kDim;
    // S[t]: rows perm_col(64 kh + 16 t + 4 g4 + e), column colw + l16
    auto srow = [&](int t, int e) { return perm_col(64 * kh + 16 * t + 4 * g4 + e); };
    f32x4 S[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        S[t][e] = a.s_identity ? (srow(t, e) == colw + l16 ? 1.0f : 0.0f)
                               : (a.s0 ? a.s0[sbase + (size_t)srow(t, e) * kDim + colw + l16] : 0.0f);
    const int trG = lane >> 4, trJ = (lane >> 2) & 3, trQ = lane & 3;
    f32x4* xmine = &sm.xch[w][0][0];
    const f32x4* xpart = &sm.xch[w ^ 1][0][0];
    uint16_t* ostage = sm.o[w];

    auto store_o = [&](int jc) {
      const int tok0 = si.tok0 + jc * kChunk;
      const int rem = si.len - jc * kChunk;
      const int len = rem < kChunk ? rem : kChunk;
      const int r = 32 * kh + (lane >> 1);
      const u32x4 val = *reinterpret_cast<const u32x4*>(ostage + 8 * lane);
      if (r < len) *reinterpret_cast<u32x4*>(a.o + ((size_t)(tok0 + r) * H + h) * kDim + colw + 8 * (lane & 1)) = val;
    };

    __syncthreads();

    for (int jc = 0; jc < si.nch; ++jc) {
      const int c = si.c0 + jc;
      const size_t cm = (size_t)h * a.geo.NT + c;
      const int tb = (COMPUTE_O && a.kdec) ? (jc & 1) : 0;  // buffer of T, row vectors, decays

      if constexpr (COMPUTE_O) {
        if (jc >= 1) store_o(jc - 1);
      }
      if constexpr (STORE_H) {
        float* hd = a.h_out + cm * (kDim * kDim);
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) hd[(size_t)srow(t, e) * kDim + colw + l16] = S[t][e];
      }

      // partial X = kd S (three split products) and o_inter = qd S_hi over
      // this wave's K half (contraction steps 2 kh, 2 kh + 1)
      u16x8 Shi[2], Slo[2];
      split_tiles(S[0], S[1], Shi[0], Slo[0]);
      split_tiles(S[2], S[3], Shi[1], Slo[1]);
      f32x4 X[4], OI[4];
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        X[it] = f32x4{0.f, 0.f, 0.f, 0.f};
        OI[it] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int sp = 0; sp < 2; ++sp) {
        const int s = 2 * kh + sp;
        const int slot = 8 * ((4 * s + g4) ^ l16);
        u16x8 fh[4], fl[4], fq[4];
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          fh[it] = *reinterpret_cast<const u16x8*>(sm.kdh + (16 * it + l16) * kDim + slot);
          fl[it] = *reinterpret_cast<const u16x8*>(sm.kdl + (16 * it + l16) * kDim + slot);
          if constexpr (COMPUTE_O) fq[it] = *reinterpret_cast<const u16x8*>(sm.qd + (16 * it + l16) * kDim + slot);
        }
#pragma unroll
        for (int it = 0; it < 4; ++it) X[it] = mfma16(fh[it], Shi[sp], X[it]);
        if constexpr (COMPUTE_O) {
#pragma unroll
          for (int it = 0; it < 4; ++it) OI[it] = mfma16(fq[it], Shi[sp], OI[it]);
        }
#pragma unroll
        for (int it = 0; it < 4; ++it) X[it] = mfma16(fh[it], Slo[sp], X[it]);
#pragma unroll
        for (int it = 0; it < 4; ++it) X[it] = mfma16(fl[it], Shi[sp], X[it]);
      }

      // post the partial sums, then add the partner's
#pragma unroll
      for (int it = 0; it < 4; ++it) xmine[it * 64 + lane] = X[it];
      if constexpr (COMPUTE_O) {
#pragma unroll
        for (int i = 0; i < 2; ++i) xmine[(4 + i) * 64 + lane] = OI[2 * (1 - kh) + i];
      }
      __syncthreads();
#pragma unroll
      for (int it = 0; it < 4; ++it) X[it] += xpart[it * 64 + lane];
      f32x4 O[2];
      if constexpr (COMPUTE_O) {
#pragma unroll
        for (int i = 0; i < 2; ++i) O[i] = OI[2 * kh + i] + xpart[(4 + i) * 64 + lane];
      }

      // Y = beta v - (beta rk) X, then v_new = T Y
      auto make_y = [&](int hh, u16x8& yhi, u16x8& ylo) {
        f32x4 y2[2];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const int it = 2 * hh + k2;
          const u16x4 vv = tr_read(sm.v + (16 * it + 4 * g4 + trJ) * BV + 8 * ((2 * cb + (trQ >> 1)) ^ vswz<BV>(16 * it + 4 * g4 + trJ)) + 4 * (trQ & 1));
          const float4 bt = *reinterpret_cast<const float4*>(sm.vec[tb] + 16 * it + 4 * g4);
          const float4 cc = *reinterpret_cast<const float4*>(sm.vec[tb] + kChunk + 16 * it + 4 * g4);
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
          const uint16_t* row = sm.t[tb] + (16 * io + l16) * (2 * kChunk);
          th[io][0] = *reinterpret_cast<const u16x8*>(row + 8 * (g4 ^ l16));
          tl[io][0] = *reinterpret_cast<const u16x8*>(row + 8 * ((8 + g4) ^ l16));
          if (io >= 2) {  // T is lower triangular
            th[io][1] = *reinterpret_cast<const u16x8*>(row + 8 * ((4 + g4) ^ l16));
            tl[io][1] = *reinterpret_cast<const u16x8*>(row + 8 * ((12 + g4) ^ l16));
          }
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
        for (int io = 2; io < 4; ++io) VN[io] = mfma16(th[io][1], Yhi[1], VN[io]);
#pragma unroll
        for (int io = 2; io < 4; ++io) VN[io] = mfma16(th[io][1], Ylo[1], VN[io]);
#pragma unroll
        for (int io = 2; io < 4; ++io) VN[io] = mfma16(tl[io][1], Yhi[1], VN[io]);
      }
      if constexpr (STORE_H) {
        float* vd = a.vnew_out + cm * (kChunk * kDim);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const f32x4 vt = VN[2 * kh + i];
#pragma unroll
          for (int e = 0; e < 4; ++e) vd[(size_t)(16 * (2 * kh + i) + 4 * g4 + e) * kDim + colw + l16] = vt[e];
        }
      }

      // state update of this K half: S <- diag(2^G_last) S + kg^T (rk * v_new)
      auto make_z = [&](int hh, u16x8& zhi, u16x8& zlo) {
        f32x4 z2[2];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const int io = 2 * hh + k2;
          const float4 dd = *reinterpret_cast<const float4*>(sm.vec[tb] + 2 * kChunk + 16 * io + 4 * g4);
          z2[k2][0] = dd.x * VN[io][0];
          z2[k2][1] = dd.y * VN[io][1];
          z2[k2][2] = dd.z * VN[io][2];
          z2[k2][3] = dd.w * VN[io][3];
        }
        split_tiles(z2[0], z2[1], zhi, zlo);
      };
      {
        u16x8 gh[2][4], gl[2][4];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int c0 = perm_col(64 * kh + 16 * t + 4 * trQ);
            const int r0 = 32 * s + 4 * trG + trJ, r1 = r0 + 16;
            const int o0 = r0 * kDim + 8 * ((c0 >> 3) ^ kswz(r0)) + (c0 & 7);
            const int o1 = r1 * kDim + 8 * ((c0 >> 3) ^ kswz(r1)) + (c0 & 7);
            gh[s][t] = cat4(tr_read(sm.kgh + o0), tr_read(sm.kgh + o1));
            gl[s][t] = cat4(tr_read(sm.kgl + o0), tr_read(sm.kgl + o1));
          }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          // the 4 rows of tile t in lane group g4 are 4 consecutive channels
          const float4 dv = *reinterpret_cast<const float4*>(sm.dec[tb] + perm_col(64 * kh + 16 * t + 4 * g4));
          S[t][0] *= dv.x; S[t][1] *= dv.y; S[t][2] *= dv.z; S[t][3] *= dv.w;
        }
        u16x8 Zhi[2], Zlo[2];
        make_z(0, Zhi[0], Zlo[0]);
        make_z(1, Zhi[1], Zlo[1]);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
          for (int t = 0; t < 4; ++t) S[t] = mfma16(gh[s][t], Zhi[s], S[t]);
#pragma unroll
          for (int t = 0; t < 4; ++t) S[t] = mfma16(gh[s][t], Zlo[s], S[t]);
#pragma unroll
          for (int t = 0; t < 4; ++t) S[t] = mfma16(gl[s][t], Zhi[s], S[t]);
        }
      }

      // output rows of this wave, staged for the store at the next chunk
      if constexpr (COMPUTE_O) {
        const u16x8 VNb0 = pack_tiles(VN[0], VN[1]);
        const u16x8 VNb1 = kh == 1 ? pack_tiles(VN[2], VN[3]) : VNb0;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int it = 2 * kh + i;
          const int r = 16 * it + l16;
          const float4 rr = *reinterpret_cast<const float4*>(sm.vec[tb] + 3 * kChunk + 16 * it + 4 * g4);
          O[i][0] *= rr.x; O[i][1] *= rr.y; O[i][2] *= rr.z; O[i][3] *= rr.w;
          O[i] = mfma16(*reinterpret_cast<const u16x8*>(sm.aqk + r * kChunk + 8 * (g4 ^ ((r >> 1) & 7))), VNb0, O[i]);
          if (kh == 1)  // Aqk is lower triangular
            O[i] = mfma16(*reinterpret_cast<const u16x8*>(sm.aqk + r * kChunk + 8 * ((4 + g4) ^ ((r >> 1) & 7))), VNb1, O[i]);
#pragma unroll
          for (int e = 0; e < 4; ++e) ostage[(16 * i + 4 * g4 + e) * 16 + l16] = bfr(O[i][e]);
        }
      }
      __syncthreads();
    }

    if constexpr (COMPUTE_O) {
      if (si.nch >= 1) store_o(last);
    }
    if (a.sfinal) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) a.sfinal[sbase + (size_t)srow(t, e) * kDim + colw + l16] = S[t][e];
    }
  };
  if (w & 1)
    compute(std::integral_constant<int, 1>{});
  else
    compute(std::integral_constant<int, 0>{});
}

// Column slices per workgroup: 2 (four compute waves) when the (sequence,
// head) units times four V-blocks fill the chip, else 1.
hipError_t launch_kda_fwd(bool store_h, bool compute_o, const FwdArgs& a, hipStream_t stream) {
  const long units = (long)a.geo.N * a.H;
  const bool narrow = units * (kDim / 32) < 256;
  const dim3 grid1(state_grid(a.geo.N, a.H, kDim / 16)), grid2(state_grid(a.geo.N, a.H, kDim / 32));
  const int nl = loaders_k(store_h, compute_o);
  const dim3 block1(64 * (2 + nl)), block2(64 * (4 + nl));
  if (store_h && !compute_o) {
    if (narrow) hipLaunchKernelGGL((kda_state_kernel<1, true, false>), grid1, block1, 0, stream, a);
    else hipLaunchKernelGGL((kda_state_kernel<2, true, false>), grid2, block2, 0, stream, a);
  } else if (!store_h && compute_o) {
    if (narrow) hipLaunchKernelGGL((kda_state_kernel<1, false, true>), grid1, block1, 0, stream, a);
    else hipLaunchKernelGGL((kda_state_kernel<2, false, true>), grid2, block2, 0, stream, a);
  } else if (!store_h && !compute_o) {  // state only (state summary)
    if (narrow) hipLaunchKernelGGL((kda_state_kernel<1, false, false>), grid1, block1, 0, stream, a);
    else hipLaunchKernelGGL((kda_state_kernel<2, false, false>), grid2, block2, 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gdn
