// State kernel (GDN): the sequential chunk pass (chunk_fwd_h), fused with the
// output (finalize) for the whole-pass entry. One workgroup per (sequence,
// head, V-block of 16*NCB columns) with two kinds of waves:
//   - 2*NCB compute waves. Each 16-column slice of the fp32 K x V state is
//     held by a pair of waves, one per half of the K rows (64 x 16 each, in
//     MFMA accumulators), so a wave carries half of every K-contraction. A
//     compute wave also stores its output rows of chunk c-1 during chunk c;
//   - loader waves (8 in the whole pass, 4 in the other forms; see
//     loaders()) that write chunk c+1 (loaded into registers
//     during chunk c-1) into the other LDS buffer at the start of chunk c
//     and issue the loads of chunk c+2.
// Two workgroup barriers per chunk: one after the pairs have posted their
// partial sums, one when the chunk's buffers change hands.
//
// Per chunk, with S the state entering it (hyper-parallel "Diff Coverage"
// page, gate build 2026-09-10, _run_prepared_gdn_chunks and the state update
// of torch_chunk_gated_delta_rule):
//   v_new = U - W S = T (beta v - c * (k S)),     c = beta * rk * exp(G)
//   o     = (q * r) S + Aqk v_new,                r = scale * rq * exp(G)
//   S    <- exp(G_last) S + k^T (d * v_new),      d = rk * exp(G_last - G)
// In a pair, each wave forms k S and q S over its K half; the halves are
// summed through LDS. Both waves then form the whole v_new (T times the
// right-hand side), update their own K half of S, and finish 32 of the 64
// output rows. k, q and v enter the MFMAs as the exact bf16 inputs.
// Precision: the operands that carry the state are bf16 hi + lo pairs
// (about 16 significant bits) with fp32 accumulation: S in k S, T and the
// right-hand side beta v - c (k S) in T(...), and d * v_new in the update.
// Only q S (output side, which does not feed the state) uses bf16(S). In an
// fp32 simulation against the fp64 recurrence this keeps the final state
// within about 1e-5 of max |S| for every gate tested, including no decay at
// all over 8192 tokens; rounding S in k S or T to a single bf16 instead gives
// up to 1.7e-3 there (the errors it writes into the state persist when the
// gate barely decays), above the 1e-3 bar.
//
// Layouts. Row i of state tile t (16 K rows) holds K index perm_col(16 t + i):
// then the B operand of contraction step s built from tiles 2s, 2s+1 covers
// K indices 32s + 8g .. 32s + 8g + 7 in lane group g, which an A-operand
// fragment of a k or q row reads as one 16-byte piece in natural column
// order. k, q and T rows (256 bytes) are stored as 16-byte pieces: piece p of
// row r of T at slot p ^ (r & 15), of k and q at slot p ^ kswz(r) (see
// there), Aqk rows (128 bytes) at p ^ ((r >> 1) & 7) (the two rows that
// share a 256-byte bank line take the same slot in different halves), so that
// the 16 rows of a fragment read fall on distinct banks; T (hi | lo) and Aqk
// come from the prepare kernel with permuted columns. k^T for the update and
// the v columns are read with the transposing LDS read (ds_read_b64_tr_b16);
// the v rows of a 32-column block use the slot swizzle vswz.
//
// Register arrays are indexed with compile-time indices only (the compute
// loop is specialised per K half): an index that depends on the wave becomes
// an indexed register move, whose read of an MFMA result is not ordered
// after the MFMA, or a private-memory array.
#include <type_traits>

#include "gdn_state_common.h"

namespace gdn {

namespace {
using namespace st;

// Loader waves per workgroup. The loaders' stores into LDS end close to the
// compute waves' end barrier (they are nearly on the chunk's critical path),
// so the whole pass splits them over 8 waves (state kernel 145 -> 137 us on
// the B=4 T=4096 H=16 workload). The other forms (storing h and v_new, or
// state only) keep 4: at 12 waves per workgroup (3 per SIMD, at most 168
// registers each) their larger register sets would spill.
__host__ __device__ constexpr int loaders(bool store_h, bool compute_o) { return (compute_o && !store_h) ? 8 : 4; }

template <int NCB>
struct alignas(16) Smem {
  static constexpr int BV = 16 * NCB;
  static constexpr int NCW = 2 * NCB;    // compute waves
  struct alignas(16) Buf {
    uint16_t k[kChunk * kDim];           // swizzled 16-byte pieces
    uint16_t t[kChunk * 2 * kChunk];     // hi | lo, swizzled pieces
    uint16_t aqk[kChunk * kChunk];       // swizzled pieces (8 per row)
    uint16_t v[kChunk * BV];             // v rows of this V-block
    float vec[kVecRows * kChunk];
  };
  Buf buf[2];
  // q is read only before the pair barrier, and the loaders write the next
  // chunk's q after it: one buffer
  uint16_t q[kChunk * kDim];
  // per wave: its partial k S (4 tiles) and the partner's two tiles of its
  // partial q S; lane-major 16-byte slots
  f32x4 xch[NCW][6][64];
  // per wave: its 32 output rows x 16 columns (bf16) of the last chunk
  uint16_t o[NCW][32 * 16];
};

}  // namespace

template <int NCB, bool STORE_H, bool COMPUTE_O>
__global__ __launch_bounds__((2 * NCB + loaders(STORE_H, COMPUTE_O)) * 64) void gdn_state_kernel(FwdArgs a) {
  using SM = Smem<NCB>;
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
  if (w >= NCW) {
    // Chunk jc's operands as 16-byte pieces: loader lane ltid takes pieces
    // ltid + NL*p of each array, loads them into registers one chunk ahead
    // and writes them to their (swizzled) LDS slots. Rows of k, q, v past the
    // end of the sequence are zero.
    constexpr int NL = 64 * loaders(STORE_H, COMPUTE_O);
    constexpr int PPR = BV / 8;              // v pieces per row
    const int ltid = tid - NCW * 64;
    u32x4 kr[1024 / NL], qr[1024 / NL], tr[1024 / NL], ar[512 / NL], vr, er;
    auto fetch = [&](int jc) {
      const int tok0 = si.tok0 + jc * kChunk;
      const int rem = si.len - jc * kChunk;
      const int len = rem < kChunk ? rem : kChunk;
      const size_t cm = (size_t)h * a.geo.NT + si.c0 + jc;
#pragma unroll
      for (int p = 0; p < 1024 / NL; ++p) {
        const int idx = p * NL + ltid, r = idx >> 4;
        const size_t off = ((size_t)(tok0 + r) * H + h) * kDim + 8 * (idx & 15);
        kr[p] = r < len ? *reinterpret_cast<const u32x4*>(a.k + off) : u32x4{0, 0, 0, 0};
        if constexpr (COMPUTE_O) qr[p] = r < len ? *reinterpret_cast<const u32x4*>(a.q + off) : u32x4{0, 0, 0, 0};
        tr[p] = reinterpret_cast<const u32x4*>(a.tmat + cm * (kChunk * 2 * kChunk))[idx];
      }
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
    // part 0: k, q; part 1: T, Aqk, v, row vectors
    auto put = [&](int b, int part) {
      typename SM::Buf& B = sm.buf[b];
#pragma unroll
      for (int p = 0; p < 1024 / NL; ++p) {
        const int idx = p * NL + ltid, r = idx >> 4;
        if (part == 0) {
          const int slot = 8 * ((idx & 15) ^ kswz(r));
          *reinterpret_cast<u32x4*>(B.k + r * kDim + slot) = kr[p];
          if constexpr (COMPUTE_O) *reinterpret_cast<u32x4*>(sm.q + r * kDim + slot) = qr[p];
        } else {
          *reinterpret_cast<u32x4*>(B.t + r * (2 * kChunk) + 8 * ((idx & 15) ^ (r & 15))) = tr[p];
        }
      }
      if (part == 0) return;
      if constexpr (COMPUTE_O) {
#pragma unroll
        for (int p = 0; p < 512 / NL; ++p) {
          const int idx = p * NL + ltid, r = idx >> 3;
          *reinterpret_cast<u32x4*>(B.aqk + r * kChunk + 8 * ((idx & 7) ^ ((r >> 1) & 7))) = ar[p];
        }
      }
      if (ltid < 64 * PPR) {
        const int vrow = ltid / PPR;
        *reinterpret_cast<u32x4*>(B.v + vrow * BV + 8 * ((ltid % PPR) ^ vswz<BV>(vrow))) = vr;
      }
      if (ltid < kVecRows * kChunk / 4) *reinterpret_cast<u32x4*>(B.vec + 4 * ltid) = er;
    };
    // Same barrier sequence as the compute waves: one before the loop, two
    // per chunk. During chunk jc, after the pair barrier (so that the LDS
    // writes do not compete with the compute waves' reads before it), chunk
    // jc+1 goes into the buffer chunk jc-1 released and the loads of chunk
    // jc+2 are issued. Both run unconditionally (past the end the last chunk
    // is repeated, harmlessly), so no load waits for another.
    if (si.nch > 0) {
      fetch(0);
      put(0, 0);
      put(0, 1);
      fetch(min(1, last));
    }
    __syncthreads();
    for (int jc = 0; jc < si.nch; ++jc) {
      const int bn = (jc & 1) ^ 1;
      __syncthreads();
      put(bn, 0);
      put(bn, 1);
      fetch(min(jc + 2, last));
      __syncthreads();
    }
    return;
  }

  // ------------------------------------------------------------- compute
  // The K half is a compile-time constant of each specialisation below, so
  // every register-array index is static.
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
    // transposing-read lane roles: group G = lane/16, row offset j, column quad
    const int trG = lane >> 4, trJ = (lane >> 2) & 3, trQ = lane & 3;
    f32x4* xmine = &sm.xch[w][0][0];
    const f32x4* xpart = &sm.xch[w ^ 1][0][0];
    uint16_t* ostage = sm.o[w];

    // output rows 32 kh .. 32 kh + 31 of chunk jc, staged in ostage, to HBM
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
      const int b = jc & 1;
      const typename SM::Buf& B = sm.buf[b];
      const int c = si.c0 + jc;
      const size_t cm = (size_t)h * a.geo.NT + c;

      // output rows of chunk jc-1
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

      // partial X = k S and o_inter = q S_hi over this wave's K half
      // (contraction steps 2 kh, 2 kh + 1)
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
        const int slot = 8 * ((4 * s + g4) ^ kswz(l16));
        u16x8 fk[4], fq[4];
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          fk[it] = *reinterpret_cast<const u16x8*>(B.k + (16 * it + l16) * kDim + slot);
          if constexpr (COMPUTE_O) fq[it] = *reinterpret_cast<const u16x8*>(sm.q + (16 * it + l16) * kDim + slot);
        }
#pragma unroll
        for (int it = 0; it < 4; ++it) X[it] = mfma16(fk[it], Shi[sp], X[it]);
        if constexpr (COMPUTE_O) {
#pragma unroll
          for (int it = 0; it < 4; ++it) OI[it] = mfma16(fq[it], Shi[sp], OI[it]);
        }
#pragma unroll
        for (int it = 0; it < 4; ++it) X[it] = mfma16(fk[it], Slo[sp], X[it]);
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

      // Y = beta v - c X for tiles 2h, 2h+1 -> B operand of contraction step h.
      // The v values of rows 16 it + 4 g4 + j, column 16 cb + l16 come from
      // a transposing read of the v rows.
      auto make_y = [&](int hh, u16x8& yhi, u16x8& ylo) {
        f32x4 y2[2];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const int it = 2 * hh + k2;
          const u16x4 vv = tr_read(B.v + (16 * it + 4 * g4 + trJ) * BV + 8 * ((2 * cb + (trQ >> 1)) ^ vswz<BV>(16 * it + 4 * g4 + trJ)) + 4 * (trQ & 1));
          const float4 bt = *reinterpret_cast<const float4*>(B.vec + 16 * it + 4 * g4);
          const float4 cc = *reinterpret_cast<const float4*>(B.vec + kChunk + 16 * it + 4 * g4);
          y2[k2][0] = bt.x * bf2f(vv[0]) - cc.x * X[it][0];
          y2[k2][1] = bt.y * bf2f(vv[1]) - cc.y * X[it][1];
          y2[k2][2] = bt.z * bf2f(vv[2]) - cc.z * X[it][2];
          y2[k2][3] = bt.w * bf2f(vv[3]) - cc.w * X[it][3];
        }
        split_tiles(y2[0], y2[1], yhi, ylo);
      };

      // v_new = T Y (all 64 rows), three split products, four accumulators.
      // T is lower triangular: rows 0..31 have no terms in contraction step 1.
      f32x4 VN[4];
      {
        u16x8 th[4][2], tl[4][2];
#pragma unroll
        for (int io = 0; io < 4; ++io) {
          const uint16_t* row = B.t + (16 * io + l16) * (2 * kChunk);
          th[io][0] = *reinterpret_cast<const u16x8*>(row + 8 * (g4 ^ l16));
          tl[io][0] = *reinterpret_cast<const u16x8*>(row + 8 * ((8 + g4) ^ l16));
          if (io >= 2) {
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

      // state update of this K half: S <- exp(G_last) S + k^T (d * v_new);
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
        // A operand of tile t: row i is K index perm_col(64 kh + 16 t + i);
        // lane (trG, 4 trJ + trQ) reads the 4 columns starting at
        // perm_col(64 kh + 16 t + 4 trQ) of token row 32 s + 4 trG + trJ (+16)
        u16x8 ak[2][4];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int c0 = perm_col(64 * kh + 16 * t + 4 * trQ);
            const int r0 = 32 * s + 4 * trG + trJ, r1 = r0 + 16;
            const u16x4 x0 = tr_read(B.k + r0 * kDim + 8 * ((c0 >> 3) ^ kswz(r0)) + (c0 & 7));
            const u16x4 x1 = tr_read(B.k + r1 * kDim + 8 * ((c0 >> 3) ^ kswz(r1)) + (c0 & 7));
            ak[s][t] = cat4(x0, x1);
          }
        const float dec = B.vec[7 * kChunk];
        u16x8 Zhi[2], Zlo[2];
        make_z(0, Zhi[0], Zlo[0]);
#pragma unroll
        for (int t = 0; t < 4; ++t) S[t] = mfma16(ak[0][t], Zhi[0], S[t] * dec);
        make_z(1, Zhi[1], Zlo[1]);
#pragma unroll
        for (int t = 0; t < 4; ++t) S[t] = mfma16(ak[0][t], Zlo[0], S[t]);
#pragma unroll
        for (int t = 0; t < 4; ++t) S[t] = mfma16(ak[1][t], Zhi[1], S[t]);
#pragma unroll
        for (int t = 0; t < 4; ++t) S[t] = mfma16(ak[1][t], Zlo[1], S[t]);
      }

      // output rows of this wave: o = r * o_inter + Aqk bf16(v_new), staged
      // for the store at the start of the next chunk
      if constexpr (COMPUTE_O) {
        const u16x8 VNb0 = pack_tiles(VN[0], VN[1]);
        const u16x8 VNb1 = kh == 1 ? pack_tiles(VN[2], VN[3]) : VNb0;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int it = 2 * kh + i;
          const int r = 16 * it + l16;
          const float4 rr = *reinterpret_cast<const float4*>(B.vec + 3 * kChunk + 16 * it + 4 * g4);
          O[i][0] *= rr.x; O[i][1] *= rr.y; O[i][2] *= rr.z; O[i][3] *= rr.w;
          O[i] = mfma16(*reinterpret_cast<const u16x8*>(B.aqk + r * kChunk + 8 * (g4 ^ ((r >> 1) & 7))), VNb0, O[i]);
          if (kh == 1)  // Aqk is lower triangular
            O[i] = mfma16(*reinterpret_cast<const u16x8*>(B.aqk + r * kChunk + 8 * ((4 + g4) ^ ((r >> 1) & 7))), VNb1, O[i]);
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

// Column slices per workgroup: 2 (four waves) when the (sequence, head)
// units times four V-blocks fill the chip, else 1.
hipError_t launch_gdn_state(bool store_h, bool compute_o, const FwdArgs& a, hipStream_t stream) {
  const long units = (long)a.geo.N * a.H;
  const bool narrow = units * (kDim / 32) < 256;
  const dim3 grid1(state_grid(a.geo.N, a.H, kDim / 16)), grid2(state_grid(a.geo.N, a.H, kDim / 32));
  const int nl = loaders(store_h, compute_o);
  const dim3 block1(64 * (2 + nl)), block2(64 * (4 + nl));
  if (store_h && !compute_o) {
    if (narrow) hipLaunchKernelGGL((gdn_state_kernel<1, true, false>), grid1, block1, 0, stream, a);
    else hipLaunchKernelGGL((gdn_state_kernel<2, true, false>), grid2, block2, 0, stream, a);
  } else if (!store_h && compute_o) {
    if (narrow) hipLaunchKernelGGL((gdn_state_kernel<1, false, true>), grid1, block1, 0, stream, a);
    else hipLaunchKernelGGL((gdn_state_kernel<2, false, true>), grid2, block2, 0, stream, a);
  } else if (!store_h && !compute_o) {  // state only (state summary)
    if (narrow) hipLaunchKernelGGL((gdn_state_kernel<1, false, false>), grid1, block1, 0, stream, a);
    else hipLaunchKernelGGL((gdn_state_kernel<2, false, false>), grid2, block2, 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gdn
