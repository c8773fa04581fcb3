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
// One workgroup per (sequence, head, 32 value columns), the four of a
// (sequence, head) dispatched to one XCD, 512 threads: the operands of a
// chunk are formed in LDS (fp32), the products run on v_mfma_f32_16x16x4f32
// (exact fp32 operands, fp32 accumulation) in 16 x 16 tiles, and the
// 128 x 32 block of dS is held in registers in that instruction's
// accumulator layout (wave w: rows 16 w .. 16 w + 15; lane (g, l): rows
// 16 w + 4 g + e, columns l and 16 + l). With 32 columns the grid is one workgroup per compute
// unit for 64 (sequence, head) units, and the per-chunk operands are formed
// by four workgroups per unit rather than eight. It stores, per chunk, dS
// before the update (the gradient w.r.t. the state leaving the chunk) and
// dV', and the gradient w.r.t. the initial state.
#include "gdn_bwd.h"

namespace gdn {

namespace {

constexpr int kLdO = kDim + 4;     // fp32 row stride of the 64 x 128 operands (16-byte rows)
constexpr int kLdM = kChunk + 1;   // row stride of T (fp32) and Aqk (bf16)
constexpr int kCols = 32;          // value columns per workgroup
constexpr int kLdC = kCols + 4;    // fp32 row stride of the 32-column arrays: rows 4 apart
                                   // (the four lane groups of an MFMA operand) on distinct banks

struct alignas(16) KdaDhSmem {
  float kg[kChunk * kLdO];
  float qd[kChunk * kLdO];
  float kdb[kChunk * kLdO];
  float t[kChunk * kLdM];
  uint16_t p[kChunk * kLdM];         // Aqk, exact in bf16
  float dO[kChunk * kLdC];
  union {
    float ds[kDim * kLdC];           // dS, read by the dV' products
    float y[kChunk * kLdC];          // then T^T dV'
  } u;
  float dv[kChunk * kLdC];
  float dec[kDim];
};

}  // namespace

__global__ __launch_bounds__(512) void kda_bwd_dh_kernel(KdaBwdArgs a) {
  __shared__ KdaDhSmem sm;
  const int tid = threadIdx.x;
  // the value-column blocks of one (sequence, head) on one XCD, where they
  // share the L2 copy of the chunk operands; longest sequences first
  int n, h, vb;
  if (!state_unit(a.geo, a.H, kDim / kCols, n, h, vb)) return;
  const SeqInfo si = a.geo.seq(n);
  const int NT = a.geo.NT;
  const int col0 = vb * kCols;

  // dS block in the accumulator layout: dS[ct][e] is row 16 w + 4 g + e,
  // column 16 ct + l of the block
  const int lane = tid & 63, l = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  f32x4 dS[2];
  const size_t sbase = ((size_t)n * a.H + h) * kDim * kDim;
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      dS[ct][e] = a.dsfinal ? a.dsfinal[sbase + (size_t)(16 * w + 4 * g + e) * kDim + col0 + 16 * ct + l] : 0.0f;

  // one chunk's global operands, loaded into registers a chunk ahead:
  // thread (row fi, channels fd0 .. fd0 + 15; stored T / Aqk positions
  // 8 fq .. 8 fq + 7); rows past the end are zero
  const int fi = tid >> 3, fd0 = (tid & 7) * 16, fq = tid & 7;
  uint4 kr[2], qr[2], th, tl, av;
  float4 gr[4], gl[4], decv;
  float rkb, rk, srq, dov[4];
  auto fetch = [&](int jc) {
    const size_t cm = (size_t)h * NT + si.c0 + jc;
    const int tok0 = si.tok0 + jc * kChunk;
    const int rem = si.len - jc * kChunk;
    const int len = rem < kChunk ? rem : kChunk;
    const float* gk = a.gk + cm * (kChunk * kDim);
    const float* vec = a.vec + cm * (kVecRows * kChunk);
    const bool valid = fi < len;
    rkb = vec[1 * kChunk + fi];
    rk = vec[2 * kChunk + fi];
    srq = vec[3 * kChunk + fi];
    const size_t roff = ((size_t)(tok0 + (valid ? fi : 0)) * a.H + h) * kDim + fd0;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      kr[p] = valid ? reinterpret_cast<const uint4*>(a.k + roff)[p] : make_uint4(0, 0, 0, 0);
      qr[p] = valid ? reinterpret_cast<const uint4*>(a.q + roff)[p] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      gr[p] = reinterpret_cast<const float4*>(gk + fi * kDim + fd0)[p];
      gl[p] = reinterpret_cast<const float4*>(gk + (kChunk - 1) * kDim + fd0)[p];
    }
    if (tid < kDim / 4) decv = reinterpret_cast<const float4*>(gk + (kChunk - 1) * kDim)[tid];
    const uint16_t* tm = a.tmat + cm * (kChunk * 2 * kChunk) + fi * (2 * kChunk) + 8 * fq;
    th = *reinterpret_cast<const uint4*>(tm);
    tl = *reinterpret_cast<const uint4*>(tm + kChunk);
    av = *reinterpret_cast<const uint4*>(a.aqk + cm * (kChunk * kChunk) + fi * kChunk + 8 * fq);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = tid + 512 * e, ri = idx >> 5, cj = idx & 31;
      dov[e] = ri < len ? bf2f(a.dout[((size_t)(tok0 + ri) * a.H + h) * kDim + col0 + cj]) : 0.0f;
    }
  };
  if (si.nch > 0) fetch(si.nch - 1);

  for (int jc = si.nch - 1; jc >= 0; --jc) {
    const int c = si.c0 + jc;
    const size_t cm = (size_t)h * NT + c;

    // this chunk's operands from the registers into LDS, then the next
    // chunk's loads go out
    {
      const int i = fi, d0 = fd0;
      const uint32_t kw[8] = {kr[0].x, kr[0].y, kr[0].z, kr[0].w, kr[1].x, kr[1].y, kr[1].z, kr[1].w};
      const uint32_t qw[8] = {qr[0].x, qr[0].y, qr[0].z, qr[0].w, qr[1].x, qr[1].y, qr[1].z, qr[1].w};
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float G[4] = {gr[p].x, gr[p].y, gr[p].z, gr[p].w};
        const float GL[4] = {gl[p].x, gl[p].y, gl[p].z, gl[p].w};
        float kg4[4], qd4[4], kb4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c2 = 4 * p + e;
          const uint32_t kb = kw[c2 >> 1], qb = qw[c2 >> 1];
          const float kv = __uint_as_float((c2 & 1) ? (kb & 0xFFFF0000u) : (kb << 16));
          const float qv = __uint_as_float((c2 & 1) ? (qb & 0xFFFF0000u) : (qb << 16));
          const float eg = exp2_hw(G[e]);
          kg4[e] = kv * rk * exp2_hw(GL[e] - G[e]);
          qd4[e] = qv * srq * eg;
          kb4[e] = kv * rkb * eg;
        }
        const int d = d0 + 4 * p;
        *reinterpret_cast<float4*>(sm.kg + i * kLdO + d) = make_float4(kg4[0], kg4[1], kg4[2], kg4[3]);
        *reinterpret_cast<float4*>(sm.qd + i * kLdO + d) = make_float4(qd4[0], qd4[1], qd4[2], qd4[3]);
        *reinterpret_cast<float4*>(sm.kdb + i * kLdO + d) = make_float4(kb4[0], kb4[1], kb4[2], kb4[3]);
      }
      if (tid < kDim / 4) {
        sm.dec[4 * tid + 0] = exp2_hw(decv.x);
        sm.dec[4 * tid + 1] = exp2_hw(decv.y);
        sm.dec[4 * tid + 2] = exp2_hw(decv.z);
        sm.dec[4 * tid + 3] = exp2_hw(decv.w);
      }
      const uint32_t thw[4] = {th.x, th.y, th.z, th.w};
      const uint32_t tlw[4] = {tl.x, tl.y, tl.z, tl.w};
      const uint32_t aw[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int col = unperm_col(8 * fq + e);
        const uint32_t hw = thw[e >> 1], lw = tlw[e >> 1], pw = aw[e >> 1];
        const float hv = __uint_as_float((e & 1) ? (hw & 0xFFFF0000u) : (hw << 16));
        const float lv = __uint_as_float((e & 1) ? (lw & 0xFFFF0000u) : (lw << 16));
        sm.t[i * kLdM + col] = hv + lv;
        sm.p[i * kLdM + col] = (uint16_t)((e & 1) ? (pw >> 16) : (pw & 0xFFFFu));
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int idx = tid + 512 * e;
        sm.dO[(idx >> 5) * kLdC + (idx & 31)] = dov[e];
      }
    }
    if (jc > 0) fetch(jc - 1);
    // dS before the update: the gradient w.r.t. the state leaving the chunk
    float* dhn = a.dhn + cm * (kDim * kDim);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * w + 4 * g + e, col = 16 * ct + l;
        sm.u.ds[row * kLdC + col] = dS[ct][e];
        dhn[(size_t)row * kDim + col0 + col] = dS[ct][e];
      }
    __syncthreads();

    // Wave w's 16 x 16 tile of the 64 x 32 results below: row block w % 4,
    // column block w / 4. Lane (g, l) supplies contraction slots
    // k0 + 4 g + ks (one per MFMA step) of its operand row or column.
    const int rt = w & 3, ctl = w >> 2;
    const int ia = 16 * rt + l, cb = 16 * ctl + l;

    // dV' = KG dS + Aqk^T dO (Aqk lower triangular with its diagonal:
    // contraction blocks kb >= rt, masked r >= i in the diagonal one)
    {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
      for (int k0 = 0; k0 < kDim; k0 += 16) {
        const float4 av = *reinterpret_cast<const float4*>(sm.kg + ia * kLdO + k0 + 4 * g);
        const float ava[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ava[ks], sm.u.ds[(k0 + 4 * g + ks) * kLdC + cb], acc, 0, 0, 0);
      }
      for (int kb = rt; kb < 4; ++kb) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int r = 16 * kb + 4 * g + ks;
          float pv = bf2f(sm.p[r * kLdM + ia]);
          if (kb == rt) pv = r >= ia ? pv : 0.0f;
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(pv, sm.dO[r * kLdC + cb], acc, 0, 0, 0);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * rt + 4 * g + e;
        sm.dv[row * kLdC + cb] = acc[e];
        a.dvn[cm * (kChunk * kDim) + (size_t)row * kDim + col0 + cb] = acc[e];
      }
    }
    __syncthreads();

    // Y = T^T dV' (T lower triangular: blocks kb >= rt, masked i >= j in the
    // diagonal one); Y takes the place of dS, whose readers are done
    {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int kb = rt; kb < 4; ++kb) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int i = 16 * kb + 4 * g + ks;
          float tv = sm.t[i * kLdM + ia];
          if (kb == rt) tv = i >= ia ? tv : 0.0f;
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(tv, sm.dv[i * kLdC + cb], acc, 0, 0, 0);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.u.y[(16 * rt + 4 * g + e) * kLdC + cb] = acc[e];
    }
    __syncthreads();

    // dS <- diag(2^G_last) dS + QD^T dO - KDB^T Y (wave w: rows 16 w ..)
    {
      f32x4 acc[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[ct][e] = sm.dec[16 * w + 4 * g + e] * dS[ct][e];
      const int d = 16 * w + l;
#pragma unroll 2
      for (int k0 = 0; k0 < kChunk; k0 += 16) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int i = k0 + 4 * g + ks;
          const float qa = sm.qd[i * kLdO + d], ka = -sm.kdb[i * kLdO + d];
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) {
            acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(qa, sm.dO[i * kLdC + 16 * ct + l], acc[ct], 0, 0, 0);
            acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(ka, sm.u.y[i * kLdC + 16 * ct + l], acc[ct], 0, 0, 0);
          }
        }
      }
      dS[0] = acc[0];
      dS[1] = acc[1];
    }
    __syncthreads();  // the next chunk rewrites the operands
  }
  if (a.ds0) {
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) a.ds0[sbase + (size_t)(16 * w + 4 * g + e) * kDim + col0 + 16 * ct + l] = dS[ct][e];
  }
}

// ---------------------------------------------------------------------------
// Per-chunk gradients of the KDA backward, the chunk-form reverse pass of
// one (chunk, head) given the state products E = dO S^T, F = dV' S^T,
// D = V' dS_next^T (the state-products kernel), dV' and dS_next (the reverse
// pass), the saved S and V' (the forward recompute):
//   mats: dP = scale (dO V'^T) on i >= j, dT = dV' (b v)^T - F (b KD)^T,
//         tU = T^T dV', tW = -T^T F, dv = b tU, db1 = rowsum(tU v + tW KD),
//         dKD = b tW, dA = (T^T dT T^T) on i > j;
//   gram: the terms of A and P with their per-channel decays, the chains
//         through KD = k^ 2^G, QD = q^ 2^G, KG = k^ 2^(G_last - G) and
//         2^G_last, the reverse cumulative sum of the gate gradient inside
//         the chunk, the L2-norm and sigmoid derivatives.
// k^ = k rk and q^ = q rq are the normalised rows; G the cumulative log2
// gate. Every exponent 2^(G_i - G_j) is taken with i >= j, so it is <= 0.
// fp32 throughout: the mats kernel's products on v_mfma_f32_16x16x4f32
// (exact fp32 operands); the gram kernel's pairs of rows in different 16-row
// blocks on the same instruction (decays split at a reference row), its
// pairs inside a block on the vector units. One workgroup per (chunk, head)
// (the kernels with 512 threads; the gram kernel's thread: row r, 16
// channels), heads fastest in dispatch order.
// ---------------------------------------------------------------------------
namespace {

constexpr int kLdR = kDim + 4;    // fp32 row stride of 64 x 128 arrays in LDS
constexpr int kLdB = kDim + 8;    // bf16 row stride

struct alignas(16) MatsSmem {
  union {
    struct {
      float dO[kChunk * kLdR];
      float vp[kChunk * kLdR];
    } p1;
    struct {
      float dv[kChunk * kLdR];
      float f[kChunk * kLdR];    // F, then X = T^T dT
      float kd[kChunk * kLdR];
      uint16_t v[kChunk * kLdB];
    } p2;
  } u;
  float t[kChunk * kLdM];
  float dt[kChunk * kLdM];
  float b[kChunk];
  float red[8][kChunk];          // per-wave partial row sums of d beta
};

__device__ __forceinline__ void chunk_of(const Geometry& geo, int bx, int H, int& c, int& h, ChunkInfo& ci) {
  c = bx / H;
  h = bx - (bx / H) * H;
  ci = geo.chunk(c);
}

// 64 x 128 fp32 rows (global, row stride 128) into LDS (row stride kLdR), 512 threads
__device__ __forceinline__ void rows_f32(float* dst, const float* src, int tid) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int idx = tid + 512 * e, r = idx >> 5, c4 = (idx & 31) * 4;
    *reinterpret_cast<float4*>(dst + r * kLdR + c4) = *reinterpret_cast<const float4*>(src + r * kDim + c4);
  }
}

// T = hi + lo from its stored permuted columns into LDS (row stride kLdM), 512 threads
__device__ __forceinline__ void load_t(float* dst, const uint16_t* tm, int tid) {
  const int r = tid >> 3, qq = tid & 7;
  const uint16_t* row = tm + r * (2 * kChunk) + 8 * qq;
  const uint4 h0 = *reinterpret_cast<const uint4*>(row);
  const uint4 l0 = *reinterpret_cast<const uint4*>(row + kChunk);
  const uint32_t hw[4] = {h0.x, h0.y, h0.z, h0.w};
  const uint32_t lw[4] = {l0.x, l0.y, l0.z, l0.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float hv = __uint_as_float((e & 1) ? (hw[e >> 1] & 0xFFFF0000u) : (hw[e >> 1] << 16));
    const float lv = __uint_as_float((e & 1) ? (lw[e >> 1] & 0xFFFF0000u) : (lw[e >> 1] << 16));
    dst[r * kLdM + unperm_col(8 * qq + e)] = hv + lv;
  }
}

// acc += the 16 x 16 tile (rows r0.., columns c0..) of A B^T over a
// contraction of 16 indices from k0, on v_mfma_f32_16x16x4f32 (exact fp32
// products, fp32 accumulation): A and B are fp32 rows in LDS (row stride
// kLdR, contraction index contiguous). Lane (g, l) takes contraction slots
// k0 + 4g .. k0 + 4g + 3, one per MFMA step, so each operand is one 16-byte
// read; it ends with C[r0 + 4g + e][c0 + l] in acc[e].
__device__ __forceinline__ f32x4 mma_rows(const float* A, const float* B, int r0, int c0, int k0, int l, int g,
                                          f32x4 acc) {
  const float4 x = *reinterpret_cast<const float4*>(A + (r0 + l) * kLdR + k0 + 4 * g);
  const float4 y = *reinterpret_cast<const float4*>(B + (c0 + l) * kLdR + k0 + 4 * g);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.x, y.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.y, y.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.z, y.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.w, y.w, acc, 0, 0, 0);
  return acc;
}

}  // namespace

__global__ __launch_bounds__(512) void kda_bwd_mats_kernel(KdaBwdArgs a) {
  __shared__ MatsSmem sm;
  const int tid = threadIdx.x;
  int c, h;
  ChunkInfo ci;
  chunk_of(a.geo, blockIdx.x, a.H, c, h, ci);
  const int L = ci.len, H = a.H, NT = a.geo.NT;
  const size_t cm = (size_t)h * NT + c;
  const size_t plane = (size_t)H * NT * kChunk * kDim;
  const float* vec = a.vec + cm * (kVecRows * kChunk);
  const int i = tid >> 3, q8 = tid & 7;   // row i; 8 columns from 8 q8 (64-wide) or 16 from 16 q8
  // the 64 x 64 products on the matrix unit: wave w takes the 16 x 16 tiles
  // (row block w % 4, column blocks 2 (w / 4) and 2 (w / 4) + 1)
  const int lane = tid & 63, ml = lane & 15, mg = lane >> 4;
  const int mrt = (tid >> 6) & 3, mct = 2 * (tid >> 8);

  // ---- dP = scale (dO V'^T), i >= j
  {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = tid + 512 * e, r = idx >> 5, c4 = (idx & 31) * 4;
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (r < L) {
        const uint2 w = *reinterpret_cast<const uint2*>(a.dout + ((size_t)(ci.tok0 + r) * H + h) * kDim + c4);
        x = make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                        __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u));
      }
      *reinterpret_cast<float4*>(sm.u.p1.dO + r * kLdR + c4) = x;
    }
    rows_f32(sm.u.p1.vp, a.vnew + cm * (kChunk * kDim), tid);
    load_t(sm.t, a.tmat + cm * (kChunk * 2 * kChunk), tid);
    if (tid < kChunk) sm.b[tid] = vec[tid];
    __syncthreads();
    // tiles above the diagonal are zero (a wave-uniform skip)
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    for (int k0 = 0; k0 < kDim; k0 += 16) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
        if (mct + t <= mrt) acc[t] = mma_rows(sm.u.p1.dO, sm.u.p1.vp, 16 * mrt, 16 * (mct + t), k0, ml, mg, acc[t]);
    }
    float* dP = a.dp + cm * (kChunk * kChunk);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ii = 16 * mrt + 4 * mg + e, j = 16 * (mct + t) + ml;
        dP[ii * kChunk + j] = ii >= j ? a.scale * acc[t][e] : 0.0f;
      }
    __syncthreads();
  }

  // ---- dT = dV' (b v)^T - F (b KD)^T
  {
    rows_f32(sm.u.p2.dv, a.dvn + cm * (kChunk * kDim), tid);
    rows_f32(sm.u.p2.f, a.efd + plane + cm * (kChunk * kDim), tid);
    const float* gk = a.gk + cm * (kChunk * kDim);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = tid + 512 * e, r = idx >> 5, c4 = (idx & 31) * 4;
      const float rk = vec[2 * kChunk + r];
      float4 kv = make_float4(0.f, 0.f, 0.f, 0.f);
      uint2 vv = make_uint2(0, 0);
      if (r < L) {
        const size_t off = ((size_t)(ci.tok0 + r) * H + h) * kDim + c4;
        const uint2 w = *reinterpret_cast<const uint2*>(a.k + off);
        vv = *reinterpret_cast<const uint2*>(a.v + off);
        kv = make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                         __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u));
      }
      const float4 g = *reinterpret_cast<const float4*>(gk + r * kDim + c4);
      *reinterpret_cast<float4*>(sm.u.p2.kd + r * kLdR + c4) =
          make_float4(kv.x * rk * exp2_hw(g.x), kv.y * rk * exp2_hw(g.y), kv.z * rk * exp2_hw(g.z),
                      kv.w * rk * exp2_hw(g.w));
      *reinterpret_cast<uint2*>(sm.u.p2.v + r * kLdB + c4) = vv;
    }
    __syncthreads();
    // dV' v^T and F KD^T, tile by tile; v is exact in bf16
    f32x4 au[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    f32x4 aw[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    for (int k0 = 0; k0 < kDim; k0 += 16) {
      const float4 x = *reinterpret_cast<const float4*>(sm.u.p2.dv + (16 * mrt + ml) * kLdR + k0 + 4 * mg);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint2 wv = *reinterpret_cast<const uint2*>(sm.u.p2.v + (16 * (mct + t) + ml) * kLdB + k0 + 4 * mg);
        au[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(x.x, __uint_as_float(wv.x << 16), au[t], 0, 0, 0);
        au[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(x.y, __uint_as_float(wv.x & 0xFFFF0000u), au[t], 0, 0, 0);
        au[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(x.z, __uint_as_float(wv.y << 16), au[t], 0, 0, 0);
        au[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(x.w, __uint_as_float(wv.y & 0xFFFF0000u), au[t], 0, 0, 0);
        aw[t] = mma_rows(sm.u.p2.f, sm.u.p2.kd, 16 * mrt, 16 * (mct + t), k0, ml, mg, aw[t]);
      }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ii = 16 * mrt + 4 * mg + e, j = 16 * (mct + t) + ml;
        sm.dt[ii * kLdM + j] = sm.b[j] * (au[t][e] - aw[t][e]);
      }
  }

  // ---- tU = T^T dV', tW = -T^T F: dv = b tU, db1 = rowsum(tU v + tW KD), dKD = b tW.
  // On the matrix unit: wave w takes value columns 16 w .. 16 w + 15 and
  // every row block; T is lower triangular, so row block rt takes the
  // contraction blocks kb >= rt, masked (r >= i) inside the diagonal block.
  {
    const int mw = tid >> 6, cc = 16 * mw + ml;
    f32x4 tu[4], tw[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      tu[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
      tw[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      float bu[4], bw[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int r = 16 * kb + 4 * mg + ks;
        bu[ks] = sm.u.p2.dv[r * kLdR + cc];
        bw[ks] = sm.u.p2.f[r * kLdR + cc];
      }
#pragma unroll
      for (int rt = 0; rt <= kb; ++rt) {
        const int ii = 16 * rt + ml;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int r = 16 * kb + 4 * mg + ks;
          float tv = sm.t[r * kLdM + ii];
          if (rt == kb) tv = r >= ii ? tv : 0.0f;
          tu[rt] = __builtin_amdgcn_mfma_f32_16x16x4f32(tv, bu[ks], tu[rt], 0, 0, 0);
          tw[rt] = __builtin_amdgcn_mfma_f32_16x16x4f32(-tv, bw[ks], tw[rt], 0, 0, 0);
        }
      }
    }
    float* dkd = a.dkd + cm * (kChunk * kDim);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ii = 16 * rt + 4 * mg + e;
        const float bi = sm.b[ii];
        const float vv = bf2f(sm.u.p2.v[ii * kLdB + cc]);
        float part = fmaf(tu[rt][e], vv, tw[rt][e] * sm.u.p2.kd[ii * kLdR + cc]);
        part += __shfl_xor(part, 1);
        part += __shfl_xor(part, 2);
        part += __shfl_xor(part, 4);
        part += __shfl_xor(part, 8);
        if (ml == 0) sm.red[mw][ii] = part;
        dkd[ii * kDim + cc] = bi * tw[rt][e];
        if (ii < L) a.dv[((size_t)(ci.tok0 + ii) * H + h) * kDim + cc] = bi * tu[rt][e];
      }
  }
  __syncthreads();
  if (tid < kChunk) {
    float s = 0.f;
#pragma unroll
    for (int w8 = 0; w8 < 8; ++w8) s += sm.red[w8][tid];
    a.db1[cm * kChunk + tid] = s;
  }

  // ---- dA = (T^T dT T^T) on i > j: X = T^T dT (into the F area), then
  // X T^T, both on the matrix unit. X: wave w takes column block w % 4 and
  // row blocks {0, 3} or {1, 2} (equal contraction lengths, T lower
  // triangular, masked r >= i inside the diagonal block).
  {
    const int xct = (tid >> 6) & 3, xsel = tid >> 8;
    f32x4 xa[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      float bx[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) bx[ks] = sm.dt[(16 * kb + 4 * mg + ks) * kLdM + 16 * xct + ml];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int rt = q == 0 ? xsel : 3 - xsel;
        if (kb < rt) continue;
        const int ii = 16 * rt + ml;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int r = 16 * kb + 4 * mg + ks;
          float tv = sm.t[r * kLdM + ii];
          if (kb == rt) tv = r >= ii ? tv : 0.0f;
          xa[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(tv, bx[ks], xa[q], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int rt = q == 0 ? xsel : 3 - xsel;
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.u.p2.f[(16 * rt + 4 * mg + e) * kLdR + 16 * xct + ml] = xa[q][e];
    }
  }
  __syncthreads();
  {
    // dA tile (rt, ct) = X T^T over k2 <= j, i.e. contraction blocks
    // kb <= ct, masked inside the diagonal one; tiles above the diagonal are
    // zero. Tiles per wave (row block, column block; -1: none), balanced at
    // four contraction blocks per computing wave.
    constexpr signed char kTr[8][3] = {{3, -1, -1}, {2, 0, -1}, {3, 1, -1}, {1, 2, -1},
                                       {3, 2, 3},   {0, 0, -1}, {0, 1, -1}, {1, 2, -1}};
    constexpr signed char kTc[8][3] = {{3, -1, -1}, {2, 0, -1}, {2, 0, -1}, {1, 1, -1},
                                       {1, 0, 0},   {1, 2, -1}, {3, 2, -1}, {3, 3, -1}};
    const int mw = __builtin_amdgcn_readfirstlane(tid >> 6);
    float* dA = a.da + cm * (kChunk * kChunk);
#pragma unroll
    for (int sl = 0; sl < 3; ++sl) {
      const int rt = kTr[mw][sl], ct = kTc[mw][sl];
      if (rt < 0) continue;
      const int jj = 16 * ct + ml;
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      if (rt >= ct) {
        for (int kb = 0; kb <= ct; ++kb) {
          const float4 xv = *reinterpret_cast<const float4*>(sm.u.p2.f + (16 * rt + ml) * kLdR + 16 * kb + 4 * mg);
          const float xs[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const int k2 = 16 * kb + 4 * mg + ks;
            float tb = sm.t[jj * kLdM + k2];
            if (kb == ct) tb = k2 <= jj ? tb : 0.0f;
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xs[ks], tb, acc, 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ii = 16 * rt + 4 * mg + e;
        dA[ii * kChunk + jj] = ii > jj ? acc[e] : 0.0f;
      }
    }
  }
}

namespace {

struct alignas(16) GramSmem {
  float g[kChunk * kLdR];     // G, then the gate gradient
  float kn[kChunk * kLdR];    // k^, then dKG * KG
  float qn[kChunk * kLdR];
  float da[kChunk * kLdM];
  float dp[kChunk * kLdM];
  float b[kChunk];
  float dgl[kDim];
  float stg[3][16 * kLdR];    // one row block's R1, R2, C1 (pairs across row blocks)
};

}  // namespace

__global__ __launch_bounds__(512) void kda_bwd_gram_kernel(KdaBwdArgs a) {
  __shared__ GramSmem sm;
  const int tid = threadIdx.x;
  int c, h;
  ChunkInfo ci;
  chunk_of(a.geo, blockIdx.x, a.H, c, h, ci);
  const int L = ci.len, H = a.H, NT = a.geo.NT;
  const size_t cm = (size_t)h * NT + c;
  const float* vec = a.vec + cm * (kVecRows * kChunk);
  const int r = tid >> 3, q8 = tid & 7, d0 = 16 * q8;

  // G, k^, q^ rows; dA, dP; beta
  {
    const float* gk = a.gk + cm * (kChunk * kDim);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = tid + 512 * e, rr = idx >> 5, c4 = (idx & 31) * 4;
      *reinterpret_cast<float4*>(sm.g + rr * kLdR + c4) = *reinterpret_cast<const float4*>(gk + rr * kDim + c4);
      float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), qv = kv;
      if (rr < L) {
        const size_t off = ((size_t)(ci.tok0 + rr) * H + h) * kDim + c4;
        const uint2 kw = *reinterpret_cast<const uint2*>(a.k + off);
        const uint2 qw = *reinterpret_cast<const uint2*>(a.q + off);
        const float rk = vec[6 * kChunk + rr], rq = vec[5 * kChunk + rr];
        kv = make_float4(rk * __uint_as_float(kw.x << 16), rk * __uint_as_float(kw.x & 0xFFFF0000u),
                         rk * __uint_as_float(kw.y << 16), rk * __uint_as_float(kw.y & 0xFFFF0000u));
        qv = make_float4(rq * __uint_as_float(qw.x << 16), rq * __uint_as_float(qw.x & 0xFFFF0000u),
                         rq * __uint_as_float(qw.y << 16), rq * __uint_as_float(qw.y & 0xFFFF0000u));
      }
      *reinterpret_cast<float4*>(sm.kn + rr * kLdR + c4) = kv;
      *reinterpret_cast<float4*>(sm.qn + rr * kLdR + c4) = qv;
    }
    const float* dA = a.da + cm * (kChunk * kChunk);
    const float* dP = a.dp + cm * (kChunk * kChunk);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int idx = tid + 512 * e, rr = idx >> 6, cc = idx & 63;
      sm.da[rr * kLdM + cc] = dA[idx];
      sm.dp[rr * kLdM + cc] = dP[idx];
    }
    if (tid < kChunk) sm.b[tid] = vec[tid];
  }
  __syncthreads();

  float knr[16], qnr[16], gr[16], dkn[16], dqn[16], dG[16];
#pragma unroll
  for (int e4 = 0; e4 < 4; ++e4) {
    const float4 k4 = *reinterpret_cast<const float4*>(sm.kn + r * kLdR + d0 + 4 * e4);
    const float4 q4v = *reinterpret_cast<const float4*>(sm.qn + r * kLdR + d0 + 4 * e4);
    const float4 g4 = *reinterpret_cast<const float4*>(sm.g + r * kLdR + d0 + 4 * e4);
    knr[4 * e4] = k4.x; knr[4 * e4 + 1] = k4.y; knr[4 * e4 + 2] = k4.z; knr[4 * e4 + 3] = k4.w;
    qnr[4 * e4] = q4v.x; qnr[4 * e4 + 1] = q4v.y; qnr[4 * e4 + 2] = q4v.z; qnr[4 * e4 + 3] = q4v.w;
    gr[4 * e4] = g4.x; gr[4 * e4 + 1] = g4.y; gr[4 * e4 + 2] = g4.z; gr[4 * e4 + 3] = g4.w;
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) { dkn[e] = 0.f; dqn[e] = 0.f; dG[e] = 0.f; }
  float dbp = 0.f;   // sum_j dA[r,j] sum_d k^_rd k^_jd 2^(G_rd - G_jd) over this thread's channels

  // Pairs inside row r's 16-row block here; pairs across blocks on the
  // matrix unit below. Row r as the later row i: j <= r
  const float br = sm.b[r];
  for (int j = r & ~15; j <= r; ++j) {
    const float dAr = j < r ? sm.da[r * kLdM + j] : 0.0f;
    const float wa = -br * dAr, dp = sm.dp[r * kLdM + j];
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const float4 kj = *reinterpret_cast<const float4*>(sm.kn + j * kLdR + d0 + 4 * e4);
      const float4 gj = *reinterpret_cast<const float4*>(sm.g + j * kLdR + d0 + 4 * e4);
      const float kja[4] = {kj.x, kj.y, kj.z, kj.w}, gja[4] = {gj.x, gj.y, gj.z, gj.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = 4 * e4 + e;
        const float ke = kja[e] * exp2_hw(gr[d] - gja[e]);
        const float t1 = wa * ke, t2 = dp * ke;
        dkn[d] += t1;
        dqn[d] += t2;
        dG[d] = fmaf(t1, knr[d], fmaf(t2, qnr[d], dG[d]));
        dbp = fmaf(dAr * knr[d], ke, dbp);
      }
    }
  }
  // row r as the earlier row j: i >= r
  for (int i2 = r; i2 <= (r | 15); ++i2) {
    const float wa = i2 > r ? -sm.b[i2] * sm.da[i2 * kLdM + r] : 0.0f;
    const float dp = sm.dp[i2 * kLdM + r];
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const float4 ki = *reinterpret_cast<const float4*>(sm.kn + i2 * kLdR + d0 + 4 * e4);
      const float4 qi = *reinterpret_cast<const float4*>(sm.qn + i2 * kLdR + d0 + 4 * e4);
      const float4 gi = *reinterpret_cast<const float4*>(sm.g + i2 * kLdR + d0 + 4 * e4);
      const float kia[4] = {ki.x, ki.y, ki.z, ki.w}, qia[4] = {qi.x, qi.y, qi.z, qi.w};
      const float gia[4] = {gi.x, gi.y, gi.z, gi.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = 4 * e4 + e;
        const float ex = exp2_hw(gia[e] - gr[d]);
        const float s = (wa * kia[e] + dp * qia[e]) * ex;
        dkn[d] += s;
        dG[d] = fmaf(-s, knr[d], dG[d]);
      }
    }
  }

  // Pairs (i, j) in different 16-row blocks, on v_mfma_f32_16x16x4f32, one
  // row block per round (wave w: channels 16 w .. 16 w + 15). Each decay is
  // split at a reference row between the two blocks, both factors <= 1:
  //   row side of block I (j < 16 I <= i): 2^(G_i - G_j) =
  //     2^(G_i - G_16I) 2^(G_16I - G_j), giving
  //     R1[i] = sum_j dA[i,j] k^_j 2^(..),  R2[i] = sum_j dP[i,j] k^_j 2^(..);
  //   column side of block J (j < rho = 16 (J + 1) <= i): 2^(G_i - G_j) =
  //     2^(G_i - G_rho) 2^(G_rho - G_j), giving
  //     C1[j] = sum_i (wA[i,j] k^_i + dP[i,j] q^_i) 2^(..), wA = -b_i dA[i,j].
  // The rows of the round's block then add them to their sums as the
  // in-block loops above do per pair.
  {
    const int lane = tid & 63, ml = lane & 15, mg = lane >> 4;
    const int dch = 16 * (tid >> 6) + ml;
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      f32x4 r1 = f32x4{0.f, 0.f, 0.f, 0.f}, r2 = r1, c1 = r1;
      if (I >= 1) {
        const float gref = sm.g[16 * I * kLdR + dch];
        const int i = 16 * I + ml;
        for (int k0 = 0; k0 < 16 * I; k0 += 16) {
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const int j = k0 + 4 * mg + ks;
            const float bv = sm.kn[j * kLdR + dch] * exp2_hw(gref - sm.g[j * kLdR + dch]);
            r1 = __builtin_amdgcn_mfma_f32_16x16x4f32(sm.da[i * kLdM + j], bv, r1, 0, 0, 0);
            r2 = __builtin_amdgcn_mfma_f32_16x16x4f32(sm.dp[i * kLdM + j], bv, r2, 0, 0, 0);
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float as = exp2_hw(sm.g[(16 * I + 4 * mg + e) * kLdR + dch] - gref);
          r1[e] *= as;
          r2[e] *= as;
        }
      }
      if (I <= 2) {
        const int rho = 16 * (I + 1);
        const float gref = sm.g[rho * kLdR + dch];
        const int j = 16 * I + ml;
        for (int k0 = rho; k0 < kChunk; k0 += 16) {
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const int i = k0 + 4 * mg + ks;
            const float ex = exp2_hw(sm.g[i * kLdR + dch] - gref);
            const float wa = -sm.b[i] * sm.da[i * kLdM + j];
            c1 = __builtin_amdgcn_mfma_f32_16x16x4f32(wa, sm.kn[i * kLdR + dch] * ex, c1, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_16x16x4f32(sm.dp[i * kLdM + j], sm.qn[i * kLdR + dch] * ex, c1, 0, 0, 0);
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) c1[e] *= exp2_hw(gref - sm.g[(16 * I + 4 * mg + e) * kLdR + dch]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int o = (4 * mg + e) * kLdR + dch;
        sm.stg[0][o] = r1[e];
        sm.stg[1][o] = r2[e];
        sm.stg[2][o] = c1[e];
      }
      __syncthreads();
      if ((r >> 4) == I) {
        const int o = (r & 15) * kLdR + d0;
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const float4 x1 = *reinterpret_cast<const float4*>(&sm.stg[0][o + 4 * e4]);
          const float4 x2 = *reinterpret_cast<const float4*>(&sm.stg[1][o + 4 * e4]);
          const float4 x3 = *reinterpret_cast<const float4*>(&sm.stg[2][o + 4 * e4]);
          const float a1[4] = {x1.x, x1.y, x1.z, x1.w}, a2[4] = {x2.x, x2.y, x2.z, x2.w};
          const float a3[4] = {x3.x, x3.y, x3.z, x3.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int d = 4 * e4 + e;
            const float dkr = -br * a1[e];
            dkn[d] += dkr + a3[e];
            dqn[d] += a2[e];
            dG[d] = fmaf(dkr - a3[e], knr[d], fmaf(a2[e], qnr[d], dG[d]));
            dbp = fmaf(a1[e], knr[d], dbp);
          }
        }
      }
      __syncthreads();
    }
  }

  // chains through KD, QD, KG and 2^G_last
  const size_t plane = (size_t)H * NT * kChunk * kDim;
  const float* Eo = a.efd + cm * (kChunk * kDim) + r * kDim + d0;
  const float* Do = a.efd + 2 * plane + cm * (kChunk * kDim) + r * kDim + d0;
  const float* dKD = a.dkd + cm * (kChunk * kDim) + r * kDim + d0;
  float wkg[16];
#pragma unroll
  for (int e4 = 0; e4 < 4; ++e4) {
    const float4 eo = *reinterpret_cast<const float4*>(Eo + 4 * e4);
    const float4 dd = *reinterpret_cast<const float4*>(Do + 4 * e4);
    const float4 dk4 = *reinterpret_cast<const float4*>(dKD + 4 * e4);
    const float4 gl = *reinterpret_cast<const float4*>(sm.g + (kChunk - 1) * kLdR + d0 + 4 * e4);
    const float eoa[4] = {eo.x, eo.y, eo.z, eo.w}, dda[4] = {dd.x, dd.y, dd.z, dd.w};
    const float dka[4] = {dk4.x, dk4.y, dk4.z, dk4.w}, gla[4] = {gl.x, gl.y, gl.z, gl.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int d = 4 * e4 + e;
      const float eg = exp2_hw(gr[d]), el = exp2_hw(gla[e] - gr[d]);
      const float dqd = a.scale * eoa[e];
      const float kg = knr[d] * el;
      dkn[d] = fmaf(dka[e], eg, fmaf(dda[e], el, dkn[d]));
      dqn[d] = fmaf(dqd, eg, dqn[d]);
      dG[d] += dka[e] * knr[d] * eg + dqd * qnr[d] * eg - dda[e] * kg;
      wkg[d] = dda[e] * kg;
    }
  }
  __syncthreads();  // every thread is done with G, k^, q^ in LDS
#pragma unroll
  for (int e4 = 0; e4 < 4; ++e4) {
    *reinterpret_cast<float4*>(sm.g + r * kLdR + d0 + 4 * e4) =
        make_float4(dG[4 * e4], dG[4 * e4 + 1], dG[4 * e4 + 2], dG[4 * e4 + 3]);
    *reinterpret_cast<float4*>(sm.kn + r * kLdR + d0 + 4 * e4) =
        make_float4(wkg[4 * e4], wkg[4 * e4 + 1], wkg[4 * e4 + 2], wkg[4 * e4 + 3]);
  }
  // gradient of G_last per channel: 2^G_last rowsum(S * dS_next) + sum_i dKG KG
  if (tid < kDim) {
    const int d = tid;
    const float* S = a.h + cm * (kDim * kDim) + (size_t)d * kDim;
    const float* dSn = a.dhn + cm * (kDim * kDim) + (size_t)d * kDim;
    float s = 0.f;
    for (int v4 = 0; v4 < kDim; v4 += 4) {
      const float4 x = *reinterpret_cast<const float4*>(S + v4), y = *reinterpret_cast<const float4*>(dSn + v4);
      s = fmaf(x.x, y.x, fmaf(x.y, y.y, fmaf(x.z, y.z, fmaf(x.w, y.w, s))));
    }
    sm.dgl[d] = exp2_hw(a.gk[cm * (kChunk * kDim) + (kChunk - 1) * kDim + d]) * s;
  }
  __syncthreads();
  // reverse cumulative sum of the gate gradient inside the chunk (channel d
  // per thread), G_last's gradient entering at the last row
  if (tid < kDim) {
    const int d = tid;
    float w = 0.f;
    for (int i2 = 0; i2 < kChunk; ++i2) w += sm.kn[i2 * kLdR + d];
    float run = sm.dgl[d] + w;
    for (int i2 = kChunk - 1; i2 >= 0; --i2) {
      run += sm.g[i2 * kLdR + d];
      sm.g[i2 * kLdR + d] = run;
    }
  }
  __syncthreads();

  // outputs of row r: L2-norm and sigmoid derivatives
  float qdot = 0.f, kdot = 0.f;
#pragma unroll
  for (int d = 0; d < 16; ++d) {
    qdot = fmaf(qnr[d], dqn[d], qdot);
    kdot = fmaf(knr[d], dkn[d], kdot);
  }
#pragma unroll
  for (int m = 1; m <= 4; m <<= 1) {
    qdot += __shfl_xor(qdot, m);
    kdot += __shfl_xor(kdot, m);
    dbp += __shfl_xor(dbp, m);
  }
  if (r < L) {
    const bool l2 = (a.flags & 1u) != 0;
    const float rq = vec[5 * kChunk + r], rk = vec[6 * kChunk + r];
    const size_t off = ((size_t)(ci.tok0 + r) * H + h) * kDim + d0;
    constexpr float kLn2 = 0.6931471805599453f;
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      float4 oq, ok, og;
      float* pq = &oq.x;
      float* pk = &ok.x;
      float* pg = &og.x;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = 4 * e4 + e;
        pq[e] = l2 ? rq * (dqn[d] - qnr[d] * qdot) : dqn[d];
        pk[e] = l2 ? rk * (dkn[d] - knr[d] * kdot) : dkn[d];
        pg[e] = kLn2 * sm.g[r * kLdR + d0 + d];
      }
      *reinterpret_cast<float4*>(a.dq + off + 4 * e4) = oq;
      *reinterpret_cast<float4*>(a.dk + off + 4 * e4) = ok;
      *reinterpret_cast<float4*>(a.dg + off + 4 * e4) = og;
    }
    if (q8 == 0) {
      const float db = a.db1[cm * kChunk + r] - dbp;
      a.dbeta[(size_t)(ci.tok0 + r) * H + h] = (a.flags & 2u) ? db * br * (1.0f - br) : db;
    }
  }
}

hipError_t launch_kda_bwd_chunks(const KdaBwdArgs& a, hipStream_t stream) {
  const unsigned grid = (unsigned)((size_t)a.geo.NT * a.H);
  hipLaunchKernelGGL(kda_bwd_mats_kernel, dim3(grid), dim3(512), 0, stream, a);
  hipLaunchKernelGGL(kda_bwd_gram_kernel, dim3(grid), dim3(512), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_kda_bwd_dh(const KdaBwdArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(kda_bwd_dh_kernel, dim3(state_grid(a.geo.N, a.H, kDim / kCols)), dim3(512), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gdn
