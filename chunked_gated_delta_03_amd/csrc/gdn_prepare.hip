// Prepare kernels: everything of one (chunk, head) that does not depend on
// the carried state. GDN: persistent workgroups of 4 waves (three per compute
// unit) looping over the (chunk, head) items; KDA: one workgroup of 4 waves
// per (chunk, head).
//
// Steps of the eager chunk algorithm on the hyper-parallel "Diff Coverage"
// page (gate build 2026-09-10; _prepare_gdn_chunks_for_summary), done here:
//   - optional L2 normalisation of q and k (the _l2norm helper, eps 1e-6
//     added to the sum of squares) -- kept as per-row factors rq, rk so the
//     bf16 inputs enter the MFMAs unrounded;
//   - optional sigmoid of beta;
//   - chunk-local cumulative sum G of the gate;
//   - A = -(beta k k^T * Gamma), strictly lower, Gamma[i,j] = exp(G_i - G_j)
//     with the mask applied before the exponential;
//   - T = (I - A)^-1 (the page's row-by-row forward substitution plus the
//     identity), computed blockwise: each 16x16 diagonal block as the
//     product (I + N)(I + N^2)(I + N^4)(I + N^8) of its strictly lower part N
//     (equal to the substitution result for a nilpotent N), then the
//     off-diagonal blocks T_ij = T_ii * sum_m A_im T_mj;
//   - the intra-chunk output matrix scale * (q k^T * Gamma), lower with the
//     diagonal (_run_prepared_gdn_chunks).
// The WY products U = T v_beta and W = T (k_beta e^G) are not formed here:
// the state kernel applies T to (beta v - c * (k S)) directly, which needs T
// and the per-row vectors only.
//
// Kimi Delta Attention (per-key-channel gate in log2 units; the chunk-local
// cumulative log2 decay gk of the KDA prepare stage on the coverage page of
// kimi_delta_attention_ascendc.py): Gamma carries a channel index inside the
// contraction, sum_d k_id k_jd 2^(G_id - G_jd). Between 16-row tiles I > J
// it is an MFMA product of rows scaled against the reference row r = 16 I:
// (k_i 2^(G_i - G_r)) . (k_j 2^(G_r - G_j)), both exponents <= 0 because
// r lies between j and i. Inside a diagonal tile no such reference is safe for
// an unbounded gate, so those pairs are summed elementwise with the mask
// applied before the power.
#include "gdn_kernels.h"

namespace gdn {

constexpr int kLdRow = kDim + 8;    // bf16 row stride of a 64 x 128 tile in LDS
constexpr int kLdF = kChunk + 1;    // fp32 row stride of a 64 x 64 matrix in LDS
constexpr int kLdQ = kChunk + 8;    // bf16 row stride of a 64 x 64 matrix in LDS
constexpr int kLdG = kDim + 4;      // fp32 row stride of the 64 x 128 KDA gate

// the 6 tiles below the diagonal (I > J), and the 6 pairs i > j of a 4 x 4 block
__constant__ int kOffI[6] = {1, 2, 2, 3, 3, 3};
__constant__ int kOffJ[6] = {0, 0, 1, 0, 1, 2};
__constant__ int kInI[6] = {1, 2, 2, 3, 3, 3};
__constant__ int kInJ[6] = {0, 0, 1, 0, 1, 2};

__device__ __forceinline__ float sumsq8(const uint4& v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float lo = __uint_as_float(w[i] << 16);
    float hi = __uint_as_float(w[i] & 0xFFFF0000u);
    s = fmaf(lo, lo, s);
    s = fmaf(hi, hi, s);
  }
  return s;
}

// The q, k rows of one (chunk, head) in registers, zero past the end.
struct QKRegs {
  u32x4 k[4], q[4];
};

__device__ __forceinline__ void fetch_qk(const PrepareArgs& a, const ChunkInfo& ci, int h, int tid, QKRegs& x) {
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int idx = pass * 256 + tid;
    const int r = idx >> 4;
    const int cc = (idx & 15) * 8;
    const size_t off = ((size_t)(ci.tok0 + r) * a.H + h) * kDim + cc;
    x.k[pass] = r < ci.len ? *reinterpret_cast<const u32x4*>(a.k + off) : u32x4{0, 0, 0, 0};
    x.q[pass] = r < ci.len ? *reinterpret_cast<const u32x4*>(a.q + off) : u32x4{0, 0, 0, 0};
  }
}

// q, k rows into LDS and their normalisation factors.
__device__ __forceinline__ void put_qk_norms(const PrepareArgs& a, const ChunkInfo& ci, int tid, const QKRegs& x,
                                             uint16_t* sk, uint16_t* sq, float* sRk, float* sRq) {
  const bool l2 = (a.flags & 1u) != 0;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int idx = pass * 256 + tid;
    const int r = idx >> 4;
    const int cc = (idx & 15) * 8;
    const uint4 kv = __builtin_bit_cast(uint4, x.k[pass]);
    const uint4 qv = __builtin_bit_cast(uint4, x.q[pass]);
    *reinterpret_cast<uint4*>(sk + r * kLdRow + cc) = kv;
    *reinterpret_cast<uint4*>(sq + r * kLdRow + cc) = qv;
    float ssk = sumsq8(kv), ssq = sumsq8(qv);
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) {
      ssk += __shfl_xor(ssk, m);
      ssq += __shfl_xor(ssq, m);
    }
    if ((tid & 15) == 0) {
      const bool valid = r < ci.len;
      sRk[r] = valid ? (l2 ? 1.0f / sqrtf(ssk + 1e-6f) : 1.0f) : 0.0f;
      sRq[r] = valid ? (l2 ? 1.0f / sqrtf(ssq + 1e-6f) : 1.0f) : 0.0f;
    }
  }
}

// beta (with the optional sigmoid) by wave 0; zero past the end.
__device__ __forceinline__ void load_beta(const PrepareArgs& a, const ChunkInfo& ci, int h, int lane,
                                          float* sBeta) {
  const bool valid = lane < ci.len;
  float b = valid ? bf2f(a.beta[(size_t)(ci.tok0 + lane) * a.H + h]) : 0.0f;
  if ((a.flags & 2u) && valid) b = 1.0f / (1.0f + expf(-b));
  sBeta[lane] = b;
}

// T (fp32) and Aqk (bf16) to global, zero above the diagonal blocks.
// T and Aqk to HBM in the layout the state kernel stages without arithmetic:
// T as a bf16 hi | lo pair per element (row r: 64 hi then 64 lo), Aqk as
// bf16, both with their columns permuted by perm_col. Thread item (r, m)
// forms output positions 8m .. 8m+7 of row r; blocks above the diagonal are
// zero.
__device__ __forceinline__ void store_t_aqk(const PrepareArgs& a, size_t cm, int tid, const float* sT,
                                            const uint16_t* sAqk) {
  uint16_t* tdst = a.tmat + cm * (kChunk * 2 * kChunk);
  uint16_t* qdst = a.aqk + cm * (kChunk * kChunk);
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int idx = pass * 256 + tid;
    const int r = idx >> 3, m = idx & 7;
    const int c0 = 32 * (m >> 2) + 4 * (m & 3);  // columns c0 + e and c0 + 16 + e
    const bool up0 = (c0 >> 4) > (r >> 4);
    const bool up1 = ((c0 + 16) >> 4) > (r >> 4);
    float x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = up0 ? 0.f : sT[r * kLdF + c0 + e];
      x[4 + e] = up1 ? 0.f : sT[r * kLdF + c0 + 16 + e];
    }
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) split2(x[2 * p], x[2 * p + 1], hi[p], lo[p]);
    *reinterpret_cast<uint4*>(tdst + r * (2 * kChunk) + 8 * m) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    *reinterpret_cast<uint4*>(tdst + r * (2 * kChunk) + kChunk + 8 * m) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    const u16x4 q0 = up0 ? u16x4{0, 0, 0, 0} : *reinterpret_cast<const u16x4*>(sAqk + r * kLdQ + c0);
    const u16x4 q1 = up1 ? u16x4{0, 0, 0, 0} : *reinterpret_cast<const u16x4*>(sAqk + r * kLdQ + c0 + 16);
    *reinterpret_cast<u16x8*>(qdst + r * kChunk + 8 * m) = cat4(q0, q1);
  }
}

// ===========================================================================
// GDN: scalar natural-log gate per (token, head)
// ===========================================================================
constexpr int kLdP = kChunk + 4;  // fp32 row stride (16-byte aligned rows) of A and T

// 16x16 fp32 product X Y on v_mfma_f32_16x16x4f32, both factors in the
// accumulator layout (lane (g, l) holds rows 4g..4g+3 of column l): xt holds
// X^T, y holds Y. The contraction slot of lane group g at step ks is 4g + ks,
// which is register ks of both operands.
__device__ __forceinline__ f32x4 mm16(const f32x4& xt, const f32x4& y, f32x4 acc) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xt[ks], y[ks], acc, 0, 0, 0);
  return acc;
}

// acc += A_IM T_MJ, both 16x16 blocks read from LDS (stride kLdP); the
// contraction slot of lane group g at step ks is 4g + ks, so the A fragment
// is one 16-byte read.
__device__ __forceinline__ f32x4 mm_lds(const float* sA, const float* sT, int I, int M, int J, int g, int l,
                                        f32x4 acc) {
  const float4 av = *reinterpret_cast<const float4*>(sA + (16 * I + l) * kLdP + 16 * M + 4 * g);
  const float ava[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ava[ks], sT[(16 * M + 4 * g + ks) * kLdP + 16 * J + l], acc, 0, 0, 0);
  return acc;
}

// inclusive prefix sum over the 64 lanes of a wave (DPP row shifts, then the
// row broadcasts of lanes 15 and 31)
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_or_zero(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWS, 0xF, false));
}
__device__ __forceinline__ float wave_inclusive_sum(float x) {
  x += dpp_or_zero<0x111, 0xF>(x);  // row_shr:1
  x += dpp_or_zero<0x112, 0xF>(x);  // row_shr:2
  x += dpp_or_zero<0x114, 0xF>(x);  // row_shr:4
  x += dpp_or_zero<0x118, 0xF>(x);  // row_shr:8
  x += dpp_or_zero<0x142, 0xA>(x);  // row_bcast:15 into rows 1 and 3
  x += dpp_or_zero<0x143, 0xC>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}

// Gram tiles per wave. Wave W loads the 16 rows of block W of k and q (MFMA
// operand order) and shares its k block with the other waves through LDS. It
// forms the q k^T tiles of block row W (its own q rows against k_J), the
// diagonal k k^T tile (W, W) and some of the six k k^T tiles below the
// diagonal:
//   wave 0: (2,0) (3,0) (3,1)    wave 1: (1,0) (2,1)    wave 2: (3,2)    wave 3: none
// Each wave then owns row block W: the norms of its rows, the inverse of its
// diagonal block and block row W of T.

struct PrepSmem {
  union {
    float A[kChunk * kLdP];   // off-diagonal blocks of A
    u16x8 kst[4][4][64];      // the k blocks in operand order, [block][step][lane]
  } u;
  float T[kChunk * kLdP];     // lower blocks of T
  float G[kChunk], beta[kChunk], rq[kChunk], rk[kChunk];
};

// One 16x128 block of q or k rows in MFMA operand order: lane (g, l) holds
// row 16R + l, columns 32s + 8g .. +7 in element s. Rows past the chunk end
// read the last valid row (finite data; their norm factors are zero).
__device__ __forceinline__ void fetch_block(const uint16_t* base, const PrepareArgs& a, const ChunkInfo& ci, int h,
                                            int R, int g, int l, u16x8 (&blk)[4]) {
  const int r = min(16 * R + l, ci.len - 1);
  const uint16_t* p = base + ((size_t)(ci.tok0 + r) * a.H + h) * kDim + 8 * g;
#pragma unroll
  for (int s = 0; s < 4; ++s) blk[s] = *reinterpret_cast<const u16x8*>(p + 32 * s);
}

__device__ __forceinline__ float sumsq_blk(const u16x8 (&blk)[4]) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    s += sumsq8(__builtin_bit_cast(uint4, blk[i]));
  return s;
}

__device__ __forceinline__ f32x4 gram_tile(const u16x8 (&x)[4], const u16x8 (&y)[4]) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = mfma16(x[s], y[s], acc);
  return acc;
}

// T (stride kLdP) of one item to HBM in the layout of store_t_aqk: row r
// holds 64 bf16 hi values, then the 64 lo values.
__device__ __forceinline__ void store_t_p(const PrepareArgs& a, size_t cm, int tid, const float* sT) {
  uint16_t* tdst = a.tmat + cm * (kChunk * 2 * kChunk);
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int idx = pass * 256 + tid;
    const int r = idx >> 3, m = idx & 7;
    const int c0 = 32 * (m >> 2) + 4 * (m & 3);  // columns c0 + e and c0 + 16 + e
    const bool up0 = (c0 >> 4) > (r >> 4);
    const bool up1 = ((c0 + 16) >> 4) > (r >> 4);
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    const float4 x0 = up0 ? z : *reinterpret_cast<const float4*>(sT + r * kLdP + c0);
    const float4 x1 = up1 ? z : *reinterpret_cast<const float4*>(sT + r * kLdP + c0 + 16);
    uint32_t hi[4], lo[4];
    split2(x0.x, x0.y, hi[0], lo[0]);
    split2(x0.z, x0.w, hi[1], lo[1]);
    split2(x1.x, x1.y, hi[2], lo[2]);
    split2(x1.z, x1.w, hi[3], lo[3]);
    *reinterpret_cast<uint4*>(tdst + r * (2 * kChunk) + 8 * m) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    *reinterpret_cast<uint4*>(tdst + r * (2 * kChunk) + kChunk + 8 * m) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  }
}

// The work of wave W over all items of the workgroup (persistent, items
// chunk-major). Per item: its k block to LDS, the Gram tiles that need only
// its own rows, the norms, gate scan and beta; after a barrier the tiles that
// need other k blocks, the previous item's T, Aqk and row vectors to HBM and
// the next item's loads; after a second barrier the scaling into A / Aqk, the
// diagonal block inverse in registers and the off-diagonal blocks of T, one
// block diagonal per barrier.
template <int W>
__device__ __forceinline__ void gdn_prepare_wave(const PrepareArgs& a, PrepSmem& sm) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int l = lane & 15;
  const int n_items = a.geo.NT * a.H;
  const bool l2 = (a.flags & 1u) != 0;

  // own rows of the item in flight, with the gate and beta (wave 0)
  u16x8 kw[4], qw[4];
  float graw = 0.f, ga = 0.f, gb = 0.f;
  uint16_t braw = 0;
  auto fetch = [&](int it) {
    const int c = it / a.H, h = it - (it / a.H) * a.H;
    const ChunkInfo ci = a.geo.chunk(c);
    fetch_block(a.k, a, ci, h, W, g, l, kw);
    fetch_block(a.q, a, ci, h, W, g, l, qw);
    if constexpr (W == 0) {
      const size_t off = (size_t)(ci.tok0 + min(lane, ci.len - 1)) * a.H + h;
      graw = a.g[off];
      braw = a.beta[off];
      if (a.a_log) {
        ga = a.a_log[h];
        gb = a.dt_bias[h];
      }
    }
  };
  auto kblk = [&](int J, u16x8 (&x)[4]) {
#pragma unroll
    for (int s = 0; s < 4; ++s) x[s] = sm.u.kst[J][s][lane];
  };

  int prev = -1;  // item whose T and Aqk are still in LDS
  float vrow0 = 0.f, vrow1 = 0.f;  // its row vectors W and W + 4
  auto store_prev = [&]() {
    const int c = prev / a.H, h = prev - (prev / a.H) * a.H;
    const size_t cm = (size_t)h * a.geo.NT + c;
    store_t_p(a, cm, tid, sm.T);
    float* vd = a.vec + cm * (kVecRows * kChunk);
    vd[W * 64 + lane] = vrow0;
    vd[(W + 4) * 64 + lane] = vrow1;
  };

  if ((int)blockIdx.x < n_items) fetch(blockIdx.x);
  for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
    const int c = it / a.H, hh = it - c * a.H;
    const ChunkInfo ci = a.geo.chunk(c);

    // own k block to LDS (the A area is free since the previous item's last
    // barrier); the tiles of own rows only
#pragma unroll
    for (int s = 0; s < 4; ++s) sm.u.kst[W][s][lane] = kw[s];
    const f32x4 kkD = gram_tile(kw, kw);
    const f32x4 qkD = gram_tile(kw, qw);  // transposed: lane (g, l) holds row l
    // norms of this wave's 16 rows; lanes l, l+16, l+32, l+48 share a row
    {
      float sk = sumsq_blk(kw), sq = sumsq_blk(qw);
      sk += __shfl_xor(sk, 16);
      sq += __shfl_xor(sq, 16);
      sk += __shfl_xor(sk, 32);
      sq += __shfl_xor(sq, 32);
      if (g == 0) {
        const int r = 16 * W + l;
        const bool valid = r < ci.len;
        sm.rk[r] = valid ? (l2 ? 1.0f / sqrtf(sk + 1e-6f) : 1.0f) : 0.0f;
        sm.rq[r] = valid ? (l2 ? 1.0f / sqrtf(sq + 1e-6f) : 1.0f) : 0.0f;
      }
    }
    if constexpr (W == 0) {
      const bool valid = lane < ci.len;
      const float gt = a.a_log ? gate_ln(graw, expf(ga), gb) : graw;
      sm.G[lane] = wave_inclusive_sum(valid ? gt : 0.0f);
      const float b = valid ? bf2f(braw) : 0.0f;
      sm.beta[lane] = ((a.flags & 2u) && valid) ? 1.0f / (1.0f + expf(-b)) : b;
    }
    __syncthreads();

    // tiles with other k blocks: kk* = k k^T (I, J), qk* = q_W k_J^T
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    f32x4 kk0 = z, kk1 = z, kk2 = z, qk0 = z, qk1 = z, qk2 = z;
    {
      u16x8 b0[4], b1[4], b2[4];
      if constexpr (W == 0) {
        kblk(2, b0); kblk(3, b1); kblk(1, b2);
        kk0 = gram_tile(b0, kw);  // (2,0)
        kk1 = gram_tile(b1, kw);  // (3,0)
        kk2 = gram_tile(b1, b2);  // (3,1)
      } else if constexpr (W == 1) {
        kblk(0, b0); kblk(2, b1);
        kk0 = gram_tile(kw, b0);  // (1,0)
        kk1 = gram_tile(b1, kw);  // (2,1)
        qk0 = gram_tile(b0, qw);  // q (1,0), transposed
      } else if constexpr (W == 2) {
        kblk(0, b0); kblk(1, b1); kblk(3, b2);
        kk0 = gram_tile(b2, kw);  // (3,2)
        qk0 = gram_tile(b0, qw);  // q (2,0)
        qk1 = gram_tile(b1, qw);  // q (2,1)
      } else {
        kblk(0, b0); kblk(1, b1); kblk(2, b2);
        qk0 = gram_tile(b0, qw);  // q (3,0)
        qk1 = gram_tile(b1, qw);  // q (3,1)
        qk2 = gram_tile(b2, qw);  // q (3,2)
      }
    }
    const int next = min(it + (int)gridDim.x, n_items - 1);
    if (prev >= 0) store_prev();
    prev = it;
    fetch(next);
    __syncthreads();

    // scaling: A_ij = -beta_i rk_i rk_j e^(G_i - G_j) (k_i . k_j), i > j;
    // Aqk_ij = scale rq_i rk_j e^(G_i - G_j) (q_i . k_j), i >= j. Off-diagonal
    // tiles need no mask; on the diagonal the mask zeroes the exponent first.
    auto put_kk = [&](int I, int J, const f32x4& kk) {
      const int i0 = 16 * I + 4 * g, j = 16 * J + l;
      const float4 gi = *reinterpret_cast<const float4*>(sm.G + i0);
      const float4 bi = *reinterpret_cast<const float4*>(sm.beta + i0);
      const float4 ki = *reinterpret_cast<const float4*>(sm.rk + i0);
      const float gj = sm.G[j], rj = sm.rk[j];
      const float gia[4] = {gi.x, gi.y, gi.z, gi.w}, bia[4] = {bi.x, bi.y, bi.z, bi.w};
      const float kia[4] = {ki.x, ki.y, ki.z, ki.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.u.A[(i0 + e) * kLdP + j] = -bia[e] * kia[e] * rj * __expf(gia[e] - gj) * kk[e];
    };
    // Aqk_ij = scale rq_i rk_j e^(G_i - G_j) (q_i . k_j), i >= j, for row
    // i = 16 W + l and columns 16 J + 4 g + e of the transposed tile, as four
    // bf16; the stored position 8 p of a row holds columns 4p..4p+3 and
    // 16+4p..16+4p+3 of its 32-column half (perm_col), so a lane's tiles
    // J = 0, 1 and J = 2, 3 make its two 16-byte pieces of the row
    auto aqk4 = [&](int J, const f32x4& qkt) {
      const int i = 16 * W + l, j0 = 16 * J + 4 * g;
      const float gi = sm.G[i], qi = sm.rq[i];
      const float4 gj = *reinterpret_cast<const float4*>(sm.G + j0);
      const float4 kj = *reinterpret_cast<const float4*>(sm.rk + j0);
      const float gja[4] = {gj.x, gj.y, gj.z, gj.w}, kja[4] = {kj.x, kj.y, kj.z, kj.w};
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float m = (J < W || l >= 4 * g + e) ? 1.0f : 0.0f;
        x[e] = m * qi * (kja[e] * a.scale) * __expf((gi - gja[e]) * m) * qkt[e];
      }
      return uint2{pack2(x[0], x[1]), pack2(x[2], x[3])};
    };
    {
      const uint2 zz = {0u, 0u};
      uint2 t0 = zz, t1 = zz, t2 = zz, t3 = zz;
      if constexpr (W == 0) {
        t0 = aqk4(0, qkD);
      } else if constexpr (W == 1) {
        t0 = aqk4(0, qk0); t1 = aqk4(1, qkD);
      } else if constexpr (W == 2) {
        t0 = aqk4(0, qk0); t1 = aqk4(1, qk1); t2 = aqk4(2, qkD);
      } else {
        t0 = aqk4(0, qk0); t1 = aqk4(1, qk1); t2 = aqk4(2, qk2); t3 = aqk4(3, qkD);
      }
      uint16_t* qrow = a.aqk + ((size_t)hh * a.geo.NT + c) * (kChunk * kChunk) + (16 * W + l) * kChunk;
      *reinterpret_cast<uint4*>(qrow + 8 * g) = make_uint4(t0.x, t0.y, t1.x, t1.y);
      *reinterpret_cast<uint4*>(qrow + 8 * (4 + g)) = make_uint4(t2.x, t2.y, t3.x, t3.y);
    }
    if constexpr (W == 0) {
      put_kk(2, 0, kk0);
      put_kk(3, 0, kk1);
      put_kk(3, 1, kk2);
    } else if constexpr (W == 1) {
      put_kk(1, 0, kk0);
      put_kk(2, 1, kk1);
    } else if constexpr (W == 2) {
      put_kk(3, 2, kk0);
    }

    // diagonal block W: N (strictly lower part of A's block) and N^T in the
    // accumulator layout from the symmetric k k^T tile
    f32x4 N, Nt, Y;
    {
      const int r0 = 16 * W + 4 * g, cc = 16 * W + l;
      const float4 gi = *reinterpret_cast<const float4*>(sm.G + r0);
      const float4 bi = *reinterpret_cast<const float4*>(sm.beta + r0);
      const float4 ki = *reinterpret_cast<const float4*>(sm.rk + r0);
      const float gc = sm.G[cc], bc = sm.beta[cc], kc = sm.rk[cc];
      const float gia[4] = {gi.x, gi.y, gi.z, gi.w}, bia[4] = {bi.x, bi.y, bi.z, bi.w};
      const float kia[4] = {ki.x, ki.y, ki.z, ki.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g + e;  // row inside the block; column l
        const float lower = r > l ? 1.0f : 0.0f, upper = r < l ? 1.0f : 0.0f;
        const float kk = kkD[e] * kia[e] * kc;
        N[e] = lower * -bia[e] * kk * __expf((gia[e] - gc) * lower);
        Nt[e] = upper * -bc * kk * __expf((gc - gia[e]) * upper);
        Y[e] = Nt[e] + (r == l ? 1.0f : 0.0f);
      }
    }
    // (I - N)^-1 = (I + N)(I + N^2)(I + N^4)(I + N^8) for the nilpotent N;
    // Y carries the transposed partial product, finally T_WW^T.
    {
      const f32x4 N2 = mm16(Nt, N, z), N2t = mm16(N, Nt, z);
      Y = mm16(N2, Y, Y);
      const f32x4 N4 = mm16(N2t, N2, z), N4t = mm16(N2, N2t, z);
      Y = mm16(N4, Y, Y);
      const f32x4 N8 = mm16(N4t, N4, z);
      Y = mm16(N8, Y, Y);
    }
    // lane (g, l) holds T_WW[l][4g + e]
    *reinterpret_cast<float4*>(sm.T + (16 * W + l) * kLdP + 16 * W + 4 * g) = make_float4(Y[0], Y[1], Y[2], Y[3]);
    __syncthreads();

    // off-diagonal blocks of block row W: T_WJ = T_WW sum_{J <= M < W} A_WM T_MJ,
    // partial sums formed as soon as their T blocks exist
    auto put_t = [&](int J, const f32x4& t) {
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.T[(16 * W + 4 * g + e) * kLdP + 16 * J + l] = t[e];
    };
    f32x4 p0 = z, p1 = z;
    if constexpr (W == 1) {
      put_t(0, mm16(Y, mm_lds(sm.u.A, sm.T, 1, 0, 0, g, l, z), z));
    } else if constexpr (W == 2) {
      put_t(1, mm16(Y, mm_lds(sm.u.A, sm.T, 2, 1, 1, g, l, z), z));
      p0 = mm_lds(sm.u.A, sm.T, 2, 0, 0, g, l, z);
    } else if constexpr (W == 3) {
      put_t(2, mm16(Y, mm_lds(sm.u.A, sm.T, 3, 2, 2, g, l, z), z));
      p1 = mm_lds(sm.u.A, sm.T, 3, 1, 1, g, l, z);
      p0 = mm_lds(sm.u.A, sm.T, 3, 0, 0, g, l, z);
    }
    __syncthreads();
    if constexpr (W == 2) {
      put_t(0, mm16(Y, mm_lds(sm.u.A, sm.T, 2, 1, 0, g, l, p0), z));
    } else if constexpr (W == 3) {
      put_t(1, mm16(Y, mm_lds(sm.u.A, sm.T, 3, 2, 1, g, l, p1), z));
      p0 = mm_lds(sm.u.A, sm.T, 3, 1, 0, g, l, p0);
    }
    __syncthreads();
    if constexpr (W == 3) put_t(0, mm16(Y, mm_lds(sm.u.A, sm.T, 3, 2, 0, g, l, p0), z));

    // row vectors W and W + 4 of this item (beta, c, d, r, G, rq, rk, e^G_last)
    {
      const int i = lane;
      const bool valid = i < ci.len;
      const float G = sm.G[i];
      if constexpr (W == 0) {
        vrow0 = valid ? sm.beta[i] : 0.f;
        vrow1 = G;
      } else if constexpr (W == 1) {
        vrow0 = valid ? sm.beta[i] * sm.rk[i] * expf(G) : 0.f;
        vrow1 = sm.rq[i];
      } else if constexpr (W == 2) {
        vrow0 = valid ? sm.rk[i] * expf(sm.G[63] - G) : 0.f;
        vrow1 = sm.rk[i];
      } else {
        vrow0 = valid ? a.scale * sm.rq[i] * expf(G) : 0.f;
        vrow1 = (i == 0) ? expf(sm.G[63]) : 0.f;
      }
    }
    __syncthreads();  // T complete; A, the k blocks and the vectors are rewritten by the next item
  }
  if (prev >= 0) store_prev();
}

// One workgroup (4 waves) per compute-unit slot (three fit), looping over
// the (chunk, head) items.
__global__ __launch_bounds__(256, 3) void gdn_prepare_kernel(PrepareArgs a) {
  __shared__ __attribute__((aligned(16))) PrepSmem sm;
  switch (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) {
    case 0: gdn_prepare_wave<0>(a, sm); break;
    case 1: gdn_prepare_wave<1>(a, sm); break;
    case 2: gdn_prepare_wave<2>(a, sm); break;
    default: gdn_prepare_wave<3>(a, sm); break;
  }
}

// T = (I - A)^-1 for strictly lower A (fp32 in LDS, row stride LD; only the
// strictly lower part of A is read), as in the GDN prepare: wave W inverts
// diagonal block W in registers by the nilpotent product formula on fp32
// MFMA, then forms block row W of T, T_WJ = T_WW sum_{J<=M<W} A_WM T_MJ, one
// block diagonal per barrier with the partial sums formed as soon as their
// T blocks exist. All 256 threads call it; it ends with a barrier. The wave
// index only selects straight-line branches (no register array is indexed
// by it).
template <int LD>
__device__ __forceinline__ void invert_unit_lower(const float* sA, float* sT, int wave, int lane) {
  const int W = __builtin_amdgcn_readfirstlane(wave);
  const int g = lane >> 4, l = lane & 15;
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  f32x4 N, Nt, Y;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r = 4 * g + e;  // row inside the block; column l
    N[e] = r > l ? sA[(16 * W + r) * LD + 16 * W + l] : 0.0f;
    Nt[e] = l > r ? sA[(16 * W + l) * LD + 16 * W + r] : 0.0f;
    Y[e] = Nt[e] + (r == l ? 1.0f : 0.0f);
  }
  {
    const f32x4 N2 = mm16(Nt, N, z), N2t = mm16(N, Nt, z);
    Y = mm16(N2, Y, Y);
    const f32x4 N4 = mm16(N2t, N2, z), N4t = mm16(N2, N2t, z);
    Y = mm16(N4, Y, Y);
    const f32x4 N8 = mm16(N4t, N4, z);
    Y = mm16(N8, Y, Y);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) sT[(16 * W + l) * LD + 16 * W + 4 * g + e] = Y[e];  // T_WW[l][4g+e]
  __syncthreads();
  // A_IM T_MJ + acc from LDS, contraction slot 4g + ks
  auto mml = [&](int I, int M, int J, f32x4 acc) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sA[(16 * I + l) * LD + 16 * M + 4 * g + ks],
                                                 sT[(16 * M + 4 * g + ks) * LD + 16 * J + l], acc, 0, 0, 0);
    return acc;
  };
  auto put_t = [&](int J, const f32x4& t) {
#pragma unroll
    for (int e = 0; e < 4; ++e) sT[(16 * W + 4 * g + e) * LD + 16 * J + l] = t[e];
  };
  f32x4 p0 = z, p1 = z;
  if (W == 1) {
    put_t(0, mm16(Y, mml(1, 0, 0, z), z));
  } else if (W == 2) {
    put_t(1, mm16(Y, mml(2, 1, 1, z), z));
    p0 = mml(2, 0, 0, z);
  } else if (W == 3) {
    put_t(2, mm16(Y, mml(3, 2, 2, z), z));
    p1 = mml(3, 1, 1, z);
    p0 = mml(3, 0, 0, z);
  }
  __syncthreads();
  if (W == 2) {
    put_t(0, mm16(Y, mml(2, 1, 0, p0), z));
  } else if (W == 3) {
    put_t(1, mm16(Y, mml(3, 2, 1, p1), z));
    p0 = mml(3, 1, 0, p0);
  }
  __syncthreads();
  if (W == 3) put_t(0, mm16(Y, mml(3, 2, 0, p0), z));
  __syncthreads();
}

// ===========================================================================
// KDA: per-key-channel log2 gate per (token, head, channel)
// ===========================================================================
__global__ __launch_bounds__(256) void kda_prepare_kernel(PrepareArgs a) {
  // 1-D grid over the (chunk, head) items, heads fastest in dispatch order
  // (neighbouring workgroups read the neighbouring head rows of the same
  // tokens)
  const int c = blockIdx.x / a.H;
  const int h = blockIdx.x - c * a.H;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g4 = lane >> 4;
  const int l16 = lane & 15;
  const ChunkInfo ci = a.geo.chunk(c);
  const size_t cm = (size_t)h * a.geo.NT + c;

  __shared__ union alignas(16) {
    struct {
      uint16_t k[kChunk * kLdRow];
      uint16_t q[kChunk * kLdRow];
      float G[kChunk * kLdG];
    } in;
    struct {
      float A[kChunk * kLdF];
      float T[kChunk * kLdF];
      uint16_t aqk[kChunk * kLdQ];
    } mat;
  } u;
  __shared__ float sBeta[kChunk], sRq[kChunk], sRk[kChunk];
  __shared__ __attribute__((aligned(16))) float sSeg[8 * kDim];  // gate segment totals
  uint16_t* sk = u.in.k;
  uint16_t* sq = u.in.q;
  float* sG = u.in.G;

  // all global loads (q, k rows, the gate block, beta) in flight together;
  // thread (channel quad cq, segment sg) holds rows 8 sg .. 8 sg + 7 of
  // channels 4 cq .. 4 cq + 3 of the gate
  const int cq = tid & 31, sg = tid >> 5;
  float4 gv[8];
  {
    QKRegs x;
    fetch_qk(a, ci, h, tid, x);
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const int r = 8 * sg + rr;
      gv[rr] = r < ci.len ? *reinterpret_cast<const float4*>(a.g + ((size_t)(ci.tok0 + r) * a.H + h) * kDim + 4 * cq)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (wave == 0) load_beta(a, ci, h, lane, sBeta);
    float ea = 0.f;
    float4 db = make_float4(0.f, 0.f, 0.f, 0.f);
    if (a.a_log) {
      ea = a.a_log[h];
      db = *reinterpret_cast<const float4*>(a.dt_bias + (size_t)h * kDim + 4 * cq);
    }
    put_qk_norms(a, ci, tid, x, sk, sq, sRk, sRq);
    // in-kernel gate, after the q, k work so that the gate loads have landed
    if (a.a_log) {
      ea = expf(ea);
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        if (8 * sg + rr < ci.len) {
          gv[rr].x = gate_log2(gv[rr].x, ea, db.x);
          gv[rr].y = gate_log2(gv[rr].y, ea, db.y);
          gv[rr].z = gate_log2(gv[rr].z, ea, db.z);
          gv[rr].w = gate_log2(gv[rr].w, ea, db.w);
        }
      }
    }
  }

  // per-channel cumulative gate: each thread scans its 8 rows in registers;
  // the segment totals go through LDS
  {
#pragma unroll
    for (int rr = 1; rr < 8; ++rr) {
      gv[rr].x += gv[rr - 1].x; gv[rr].y += gv[rr - 1].y; gv[rr].z += gv[rr - 1].z; gv[rr].w += gv[rr - 1].w;
    }
    reinterpret_cast<float4*>(sSeg)[sg * 32 + cq] = gv[7];
    __syncthreads();
    float4 base = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s2 = 0; s2 < sg; ++s2) {
      const float4 t = reinterpret_cast<const float4*>(sSeg)[s2 * 32 + cq];
      base.x += t.x; base.y += t.y; base.z += t.z; base.w += t.w;
    }
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const int r = 8 * sg + rr;
      const float4 G = make_float4(gv[rr].x + base.x, gv[rr].y + base.y, gv[rr].z + base.z, gv[rr].w + base.w);
      *reinterpret_cast<float4*>(sG + r * kLdG + 4 * cq) = G;
      if (a.gk) *reinterpret_cast<float4*>(a.gk + cm * (kChunk * kDim) + r * kDim + 4 * cq) = G;
    }
  }
  __syncthreads();

  // whole pass: the state kernel's decayed operands k 2^G and
  // k 2^(G_last - G) (bf16 hi + lo), q 2^G (bf16) and 2^G_last per channel.
  // Thread item (row r, 8 channels from 8 p) per pass, as the q, k loads.
  if (a.kdec) {
    uint16_t* kd = a.kdec + cm * kKdecElems;
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int idx = pass * 256 + tid, r = idx >> 4, c0 = (idx & 15) * 8;
      const uint4 kv = *reinterpret_cast<const uint4*>(sk + r * kLdRow + c0);
      const uint4 qv = *reinterpret_cast<const uint4*>(sq + r * kLdRow + c0);
      const float4 g0 = *reinterpret_cast<const float4*>(sG + r * kLdG + c0);
      const float4 g1 = *reinterpret_cast<const float4*>(sG + r * kLdG + c0 + 4);
      const float4 l0 = *reinterpret_cast<const float4*>(sG + 63 * kLdG + c0);
      const float4 l1 = *reinterpret_cast<const float4*>(sG + 63 * kLdG + c0 + 4);
      const float ga[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      const float la[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
      const uint32_t kw[4] = {kv.x, kv.y, kv.z, kv.w}, qw[4] = {qv.x, qv.y, qv.z, qv.w};
      uint32_t dh[4], dl[4], gh[4], gl[4], qq[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float k0 = __uint_as_float(kw[e] << 16), k1 = __uint_as_float(kw[e] & 0xFFFF0000u);
        const float q0 = __uint_as_float(qw[e] << 16), q1 = __uint_as_float(qw[e] & 0xFFFF0000u);
        const float f0 = exp2_hw(ga[2 * e]), f1 = exp2_hw(ga[2 * e + 1]);
        const float d0 = exp2_hw(la[2 * e] - ga[2 * e]), d1 = exp2_hw(la[2 * e + 1] - ga[2 * e + 1]);
        split2(k0 * f0, k1 * f1, dh[e], dl[e]);
        split2(k0 * d0, k1 * d1, gh[e], gl[e]);
        qq[e] = pack2(q0 * f0, q1 * f1);
      }
      const int off = r * kDim + c0;
      *reinterpret_cast<uint4*>(kd + kKdecKdh + off) = make_uint4(dh[0], dh[1], dh[2], dh[3]);
      *reinterpret_cast<uint4*>(kd + kKdecKdl + off) = make_uint4(dl[0], dl[1], dl[2], dl[3]);
      *reinterpret_cast<uint4*>(kd + kKdecKgh + off) = make_uint4(gh[0], gh[1], gh[2], gh[3]);
      *reinterpret_cast<uint4*>(kd + kKdecKgl + off) = make_uint4(gl[0], gl[1], gl[2], gl[3]);
      *reinterpret_cast<uint4*>(kd + kKdecQd + off) = make_uint4(qq[0], qq[1], qq[2], qq[3]);
    }
    if (tid < 32) {
      const float4 l = *reinterpret_cast<const float4*>(sG + 63 * kLdG + 4 * tid);
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(kd + kKdecDec) + 4 * tid) =
          make_float4(exp2_hw(l.x), exp2_hw(l.y), exp2_hw(l.z), exp2_hw(l.w));
    }
  }

  // Gram tiles. Lane (l16, g4) of an MFMA step s covers channels
  // 32 s + 8 g4 .. + 7 of operand row/column l16. Products of rows scaled
  // against a reference row r with j < r <= i have both exponents <= 0.
  auto g8 = [&](int row, int d0, float (&x)[8]) {
    const float4 x0 = *reinterpret_cast<const float4*>(sG + row * kLdG + d0);
    const float4 x1 = *reinterpret_cast<const float4*>(sG + row * kLdG + d0 + 4);
    x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w; x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
  };
  auto scale_split = [&](const u16x8& v, const float (&f)[8], u16x8& hi, u16x8& lo) {
    u32x4 hh, ll;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t x, y;
      split2(bf2f(v[2 * p]) * f[2 * p], bf2f(v[2 * p + 1]) * f[2 * p + 1], x, y);
      hh[p] = x;
      ll[p] = y;
    }
    hi = __builtin_bit_cast(u16x8, hh);
    lo = __builtin_bit_cast(u16x8, ll);
  };
  auto scale_pack = [&](const u16x8& v, const float (&f)[8]) {
    u32x4 pp;
#pragma unroll
    for (int p = 0; p < 4; ++p) pp[p] = pack2(bf2f(v[2 * p]) * f[2 * p], bf2f(v[2 * p + 1]) * f[2 * p + 1]);
    return __builtin_bit_cast(u16x8, pp);
  };
  auto row8 = [&](const uint16_t* base, int row, int d0) {
    return *reinterpret_cast<const u16x8*>(base + row * kLdRow + d0);
  };

  // off-diagonal tiles I > J (reference r = 16 I; k k^T with hi + lo
  // operands, q k^T with single bf16 operands). Wave w: jobs w and w + 4.
  f32x4 accA[2], accQ[2];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int job = wave + 4 * jj;
    accA[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
    accQ[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (job >= 6) continue;
    const int I = kOffI[job], J = kOffJ[job];
    const int i = 16 * I + l16, j = 16 * J + l16, r = 16 * I;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int d0 = 32 * s + 8 * g4;
      float gi[8], gr[8], gj[8], fi[8], fj[8];
      g8(i, d0, gi);
      g8(r, d0, gr);
      g8(j, d0, gj);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        fi[e] = exp2_hw(gi[e] - gr[e]);
        fj[e] = exp2_hw(gr[e] - gj[e]);
      }
      u16x8 ah, al, bh, bl;
      scale_split(row8(sk, i, d0), fi, ah, al);
      const u16x8 aq = scale_pack(row8(sq, i, d0), fi);
      scale_split(row8(sk, j, d0), fj, bh, bl);
      accA[jj] = mfma16(ah, bh, accA[jj]);
      accA[jj] = mfma16(ah, bl, accA[jj]);
      accA[jj] = mfma16(al, bh, accA[jj]);
      accQ[jj] = mfma16(aq, bh, accQ[jj]);
    }
  }

  // diagonal tile I = wave (rows/columns t0 .. t0+15), split into 4 x 4
  // sub-blocks p = l16 / 4. Pass P (reference t0 + 4P) takes A rows of
  // sub-block P and B columns of sub-blocks below P; together the passes
  // cover every pair of different sub-blocks exactly once. q k^T without
  // decay gives the diagonal of the output matrix.
  const int t0 = 16 * wave;
  const int psub = l16 >> 2;
  f32x4 dA = {0.f, 0.f, 0.f, 0.f}, dQ = {0.f, 0.f, 0.f, 0.f}, dQ0 = {0.f, 0.f, 0.f, 0.f};
  {
    const int i = t0 + l16;  // A row and B column of this lane
    const u16x8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int d0 = 32 * s + 8 * g4;
      float gi[8], gp[8], fa[8];
      g8(i, d0, gi);
      g8(t0 + 4 * psub, d0, gp);
#pragma unroll
      for (int e = 0; e < 8; ++e) fa[e] = exp2_hw(gi[e] - gp[e]);
      const u16x8 ki = row8(sk, i, d0), qi = row8(sq, i, d0);
      u16x8 ah, al;
      scale_split(ki, fa, ah, al);
      const u16x8 aq = scale_pack(qi, fa);
      dQ0 = mfma16(qi, ki, dQ0);
#pragma unroll
      for (int P = 1; P < 4; ++P) {
        float gr[8], fb[8];
        g8(t0 + 4 * P, d0, gr);
#pragma unroll
        for (int e = 0; e < 8; ++e) fb[e] = exp2_hw(psub < P ? gr[e] - gi[e] : -1000.0f);
        u16x8 bh, bl;
        scale_split(ki, fb, bh, bl);
        const bool rowP = psub == P;
        const u16x8 aph = rowP ? ah : zero8, apl = rowP ? al : zero8, apq = rowP ? aq : zero8;
        dA = mfma16(aph, bh, dA);
        dA = mfma16(aph, bl, dA);
        dA = mfma16(apl, bh, dA);
        dQ = mfma16(apq, bh, dQ);
      }
    }
  }
  // pairs inside a 4 x 4 sub-block (i > j), elementwise with the mask
  // before the power: lane < 48 takes pair lane / 2 and half the channels
  float ekk = 0.f, eqk = 0.f;
  int ei = 0, ej = 0;
  if (lane < 48) {
    const int pp = lane >> 1, half = lane & 1;
    const int sb = pp / 6, w6 = pp - 6 * (pp / 6);
    const int il = kInI[w6], jl = kInJ[w6];
    ei = t0 + 4 * sb + il;
    ej = t0 + 4 * sb + jl;
    for (int d = 64 * half; d < 64 * half + 64; d += 4) {
      const float4 gi = *reinterpret_cast<const float4*>(sG + ei * kLdG + d);
      const float4 gj = *reinterpret_cast<const float4*>(sG + ej * kLdG + d);
      const u16x4 ki = *reinterpret_cast<const u16x4*>(sk + ei * kLdRow + d);
      const u16x4 kj = *reinterpret_cast<const u16x4*>(sk + ej * kLdRow + d);
      const u16x4 qi = *reinterpret_cast<const u16x4*>(sq + ei * kLdRow + d);
      const float w0 = bf2f(kj[0]) * exp2_hw(gi.x - gj.x), w1 = bf2f(kj[1]) * exp2_hw(gi.y - gj.y);
      const float w2 = bf2f(kj[2]) * exp2_hw(gi.z - gj.z), w3 = bf2f(kj[3]) * exp2_hw(gi.w - gj.w);
      ekk = fmaf(bf2f(ki[0]), w0, ekk); ekk = fmaf(bf2f(ki[1]), w1, ekk);
      ekk = fmaf(bf2f(ki[2]), w2, ekk); ekk = fmaf(bf2f(ki[3]), w3, ekk);
      eqk = fmaf(bf2f(qi[0]), w0, eqk); eqk = fmaf(bf2f(qi[1]), w1, eqk);
      eqk = fmaf(bf2f(qi[2]), w2, eqk); eqk = fmaf(bf2f(qi[3]), w3, eqk);
    }
  }
  ekk += __shfl_xor(ekk, 1);
  eqk += __shfl_xor(eqk, 1);
  __syncthreads();

  // results into the reused LDS: A = -beta_i rk_i rk_j (k k^T)_ij (i > j),
  // Aqk = scale rq_i rk_j (q k^T)_ij (i >= j), zero above the diagonal
  // inside the diagonal tiles (the inverse and the stores ignore the blocks
  // above them)
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int job = wave + 4 * jj;
    if (job >= 6) continue;
    const int I = kOffI[job], J = kOffJ[job];
    const int jc = 16 * J + l16;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int ii = 16 * I + 4 * g4 + e;
      u.mat.A[ii * kLdF + jc] = -sBeta[ii] * sRk[ii] * sRk[jc] * accA[jj][e];
      u.mat.aqk[ii * kLdQ + jc] = f2bf(a.scale * sRq[ii] * sRk[jc] * accQ[jj][e]);
    }
  }
  {
    const int jc = t0 + l16;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int il = 4 * g4 + e, ii = t0 + il;
      if ((il >> 2) == psub && il > l16) continue;  // inside a sub-block: elementwise lanes
      const bool lower = il > l16;
      u.mat.A[ii * kLdF + jc] = lower ? -sBeta[ii] * sRk[ii] * sRk[jc] * dA[e] : 0.0f;
      const float qv = il == l16 ? dQ0[e] : dQ[e];
      u.mat.aqk[ii * kLdQ + jc] = il >= l16 ? f2bf(a.scale * sRq[ii] * sRk[jc] * qv) : (uint16_t)0;
    }
  }
  if (lane < 48 && (lane & 1) == 0) {
    u.mat.A[ei * kLdF + ej] = -sBeta[ei] * sRk[ei] * sRk[ej] * ekk;
    u.mat.aqk[ei * kLdQ + ej] = f2bf(a.scale * sRq[ei] * sRk[ej] * eqk);
  }
  __syncthreads();

  invert_unit_lower<kLdF>(u.mat.A, u.mat.T, wave, lane);

  store_t_aqk(a, cm, tid, u.mat.T, u.mat.aqk);
  if (tid < 64) {
    const int i = tid;
    const bool valid = i < ci.len;
    const float b = valid ? sBeta[i] : 0.f;
    const float rk = sRk[i], rq = sRq[i];
    float* vd = a.vec + cm * (kVecRows * kChunk);
    vd[0 * 64 + i] = b;
    vd[1 * 64 + i] = valid ? b * rk : 0.f;
    vd[2 * 64 + i] = valid ? rk : 0.f;
    vd[3 * 64 + i] = valid ? a.scale * rq : 0.f;
    vd[4 * 64 + i] = 0.f;
    vd[5 * 64 + i] = rq;
    vd[6 * 64 + i] = rk;
    vd[7 * 64 + i] = 0.f;
  }
}

hipError_t launch_prepare(bool kda, const PrepareArgs& a, hipStream_t stream) {
  const long items = (long)a.geo.NT * a.H;
  const int cus = a.cus > 0 ? a.cus : 256;
  if (kda) {
    hipLaunchKernelGGL(kda_prepare_kernel, dim3((unsigned)((size_t)a.geo.NT * a.H)), dim3(256), 0, stream, a);
  } else {
    // three workgroups fit a compute unit (43.5 KiB of LDS each)
    const long slots = 3L * cus;
    hipLaunchKernelGGL(gdn_prepare_kernel, dim3((unsigned)(items < slots ? items : slots)), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace gdn
