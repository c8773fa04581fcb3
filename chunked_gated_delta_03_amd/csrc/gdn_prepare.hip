// Prepare kernels: everything of one (chunk, head) that does not depend on
// the carried state. One workgroup of 4 waves per (chunk, head).
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
//     identity), computed blockwise: 16x16 diagonal blocks by substitution,
//     then the off-diagonal blocks T_ij = T_ii * sum_m A_im T_mj;
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

// the 10 lower 16x16 tiles (I >= J) of a 64 x 64 matrix
__constant__ int kTileI[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
__constant__ int kTileJ[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};

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

// q, k rows of the chunk into LDS (zero past the end), normalisation factors.
// All global loads are issued before the first LDS write.
__device__ __forceinline__ void load_qk_norms(const PrepareArgs& a, const ChunkInfo& ci, int h, int tid,
                                              uint16_t* sk, uint16_t* sq, float* sRk, float* sRq) {
  QKRegs x;
  fetch_qk(a, ci, h, tid, x);
  put_qk_norms(a, ci, tid, x, sk, sq, sRk, sRq);
}

// beta (with the optional sigmoid) by wave 0; zero past the end.
__device__ __forceinline__ void load_beta(const PrepareArgs& a, const ChunkInfo& ci, int h, int lane,
                                          float* sBeta) {
  const bool valid = lane < ci.len;
  float b = valid ? bf2f(a.beta[(size_t)(ci.tok0 + lane) * a.H + h]) : 0.0f;
  if ((a.flags & 2u) && valid) b = 1.0f / (1.0f + expf(-b));
  sBeta[lane] = b;
}

// T = (I - A)^-1 for strictly lower A (fp32, LDS), blockwise. All 256
// threads call it; it ends with a barrier. The diagonal 16x16 blocks are
// inverted by forward substitution (one block per wave); the off-diagonal
// blocks follow one block row at a time, T_ij = T_ii * (sum_m A_im T_mj),
// as 16x16x16 fp32 MFMA products. In the second product the contraction
// slot of lane group g at step ks is 4g + ks, so the first product's
// accumulator feeds it as the B operand without leaving registers.
__device__ __forceinline__ void invert_unit_lower(const float* sA, float* sT, int wave, int lane) {
  const int g4 = lane >> 4;
  const int l16 = lane & 15;
  if (lane < 16) {
    const int base = 16 * wave;
    float t[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float val = (i == lane) ? 1.0f : 0.0f;
#pragma unroll
      for (int m = 0; m < i; ++m) val = fmaf(sA[(base + i) * kLdF + base + m], t[m], val);
      t[i] = val;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sT[(base + i) * kLdF + base + lane] = t[i];
  }
  __syncthreads();
  for (int I = 1; I < 4; ++I) {
    const int J = wave;
    if (J < I) {
      f32x4 p = {0.f, 0.f, 0.f, 0.f};
      for (int M = J; M < I; ++M) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const float av = sA[(16 * I + l16) * kLdF + 16 * M + 4 * ks + g4];
          const float bv = sT[(16 * M + 4 * ks + g4) * kLdF + 16 * J + l16];
          p = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, p, 0, 0, 0);
        }
      }
      f32x4 r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const float av = sT[(16 * I + l16) * kLdF + 16 * I + 4 * g4 + ks];
        r = __builtin_amdgcn_mfma_f32_16x16x4f32(av, p[ks], r, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) sT[(16 * I + 4 * g4 + e) * kLdF + 16 * J + l16] = r[e];
    }
    __syncthreads();
  }
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
// One workgroup per compute-unit slot, looping over the (chunk, head) items
// (chunk-major, so neighbouring workgroups read neighbouring rows); the q, k,
// g and beta of the next item are loaded into registers while the current
// one is computed.
__global__ __launch_bounds__(256, 3) void gdn_prepare_kernel(PrepareArgs a) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g4 = lane >> 4;
  const int l16 = lane & 15;
  const int n_items = a.geo.NT * a.H;

  // q, k rows live only until the Gram tiles are in registers; A, T and Aqk
  // reuse their space afterwards.
  __shared__ union alignas(16) {
    struct {
      uint16_t k[kChunk * kLdRow];
      uint16_t q[kChunk * kLdRow];
    } in;
    struct {
      float A[kChunk * kLdF];
      float T[kChunk * kLdF];
      uint16_t aqk[kChunk * kLdQ];
    } mat;
  } u;
  __shared__ __attribute__((aligned(16))) float sG[kChunk], sBeta[kChunk], sRq[kChunk], sRk[kChunk];

  // registers of the next item: q, k rows (all threads), raw g and beta
  // (wave 0; masked when they are written to LDS, so nothing waits on them)
  QKRegs nx;
  float ngx = 0.0f;
  uint16_t nbx = 0;
  auto fetch = [&](int it) {
    const int c = it / a.H, h = it - (it / a.H) * a.H;
    const ChunkInfo ci = a.geo.chunk(c);
    fetch_qk(a, ci, h, tid, nx);
    if (wave == 0) {
      const size_t off = (size_t)(ci.tok0 + (lane < ci.len ? lane : 0)) * a.H + h;
      ngx = a.g[off];
      nbx = a.beta[off];
    }
  };
  if ((int)blockIdx.x < n_items) fetch(blockIdx.x);

  for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
    const int c = it / a.H;
    const int h = it - c * a.H;
    const ChunkInfo ci = a.geo.chunk(c);

    put_qk_norms(a, ci, tid, nx, u.in.k, u.in.q, sRk, sRq);
    if (wave == 0) {
      const bool valid = lane < ci.len;
      float gx = valid ? ngx : 0.0f;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const float y = __shfl_up(gx, o);
        if (lane >= o) gx += y;
      }
      sG[lane] = gx;
      const float b = valid ? bf2f(nbx) : 0.0f;
      sBeta[lane] = ((a.flags & 2u) && valid) ? 1.0f / (1.0f + expf(-b)) : b;
    }
    // the next item's loads (the last item's again past the end, harmlessly)
    fetch(min(it + (int)gridDim.x, n_items - 1));
    __syncthreads();

    // Gram tiles on MFMA: k k^T (strictly lower) by waves 0-1, q k^T (lower) by
    // waves 2-3; each wave takes 5 of the 10 lower 16x16 tiles.
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int kind = wv >> 1;
    const uint16_t* left = kind == 0 ? u.in.k : u.in.q;
    f32x4 acc[5];
#pragma unroll
    for (int jj = 0; jj < 5; ++jj) {
      const int t = (wv & 1) + 2 * jj;
      const int I = kTileI[t], J = kTileJ[t];
      u16x8 av[4], bv[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        av[s] = *reinterpret_cast<const u16x8*>(left + (16 * I + l16) * kLdRow + 32 * s + 8 * g4);
        bv[s] = *reinterpret_cast<const u16x8*>(u.in.k + (16 * J + l16) * kLdRow + 32 * s + 8 * g4);
      }
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) x = mfma16(av[s], bv[s], x);
      acc[jj] = x;
    }
    __syncthreads();
    // scale into A (fp32) or Aqk (bf16); the causal mask is applied to the
    // exponent before the exponential (masked entries use a large negative one)
    {
      const float* rrow = kind == 0 ? sRk : sRq;
      const float sgn = kind == 0 ? -1.0f : a.scale;
#pragma unroll
      for (int jj = 0; jj < 5; ++jj) {
        const int t = (wv & 1) + 2 * jj;
        const int I = kTileI[t], J = kTileJ[t];
        const int jc = 16 * J + l16;
        const int i0 = 16 * I + 4 * g4;
        const float4 gi = *reinterpret_cast<const float4*>(sG + i0);
        const float4 ri = *reinterpret_cast<const float4*>(rrow + i0);
        const float4 bi = kind == 0 ? *reinterpret_cast<const float4*>(sBeta + i0) : make_float4(1.f, 1.f, 1.f, 1.f);
        const float gj = sG[jc], rj = sRk[jc] * sgn;
        const float gia[4] = {gi.x, gi.y, gi.z, gi.w};
        const float ria[4] = {ri.x, ri.y, ri.z, ri.w};
        const float bia[4] = {bi.x, bi.y, bi.z, bi.w};
        float val[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float m = (i0 + e + kind > jc) ? 1.0f : 0.0f;  // i > j (k k^T) or i >= j (q k^T)
          const float ex = __expf((gia[e] - gj) * m);
          val[e] = m * bia[e] * ria[e] * rj * acc[jj][e] * ex;
        }
        if (kind == 0) {
#pragma unroll
          for (int e = 0; e < 4; ++e) u.mat.A[(i0 + e) * kLdF + jc] = val[e];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) u.mat.aqk[(i0 + e) * kLdQ + jc] = __builtin_bit_cast(uint16_t, (__bf16)val[e]);
        }
      }
    }
    __syncthreads();

    invert_unit_lower(u.mat.A, u.mat.T, wave, lane);

    const size_t cm = (size_t)h * a.geo.NT + c;
    store_t_aqk(a, cm, tid, u.mat.T, u.mat.aqk);
    if (tid < 64) {
      const int i = tid;
      const bool valid = i < ci.len;
      const float G = sG[i];
      const float Glast = sG[63];
      const float b = valid ? sBeta[i] : 0.f;
      const float rk = sRk[i], rq = sRq[i];
      float* vd = a.vec + cm * (kVecRows * kChunk);
      vd[0 * 64 + i] = b;
      vd[1 * 64 + i] = valid ? b * rk * expf(G) : 0.f;
      vd[2 * 64 + i] = valid ? rk * expf(Glast - G) : 0.f;
      vd[3 * 64 + i] = valid ? a.scale * rq * expf(G) : 0.f;
      vd[4 * 64 + i] = G;
      vd[5 * 64 + i] = rq;
      vd[6 * 64 + i] = rk;
      vd[7 * 64 + i] = (i == 0) ? expf(Glast) : 0.f;
    }
    __syncthreads();  // LDS is rewritten by the next item
  }
}

// ===========================================================================
// KDA: per-key-channel log2 gate per (token, head, channel)
// ===========================================================================
__global__ __launch_bounds__(256) void kda_prepare_kernel(PrepareArgs a) {
  const int c = blockIdx.x;
  const int h = blockIdx.y;
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
  uint16_t* sk = u.in.k;
  uint16_t* sq = u.in.q;
  float* sG = u.in.G;

  load_qk_norms(a, ci, h, tid, sk, sq, sRk, sRq);
  if (wave == 0) load_beta(a, ci, h, lane, sBeta);

  // per-channel cumulative gate: the 64 x 128 block is loaded with all its
  // vector loads in flight, then thread (d, half) scans 32 rows in LDS
  {
    float4 gv[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int idx = p * 256 + tid;
      const int r = idx >> 5, c4 = (idx & 31) * 4;
      gv[p] = r < ci.len ? *reinterpret_cast<const float4*>(a.g + ((size_t)(ci.tok0 + r) * a.H + h) * kDim + c4)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int idx = p * 256 + tid;
      const int r = idx >> 5, c4 = (idx & 31) * 4;
      *reinterpret_cast<float4*>(sG + r * kLdG + c4) = gv[p];
    }
  }
  __syncthreads();
  {
    const int d = tid & 127;
    const int half = tid >> 7;
    float run = 0.0f;
    for (int r = 32 * half; r < 32 * half + 32; ++r) {
      run += sG[r * kLdG + d];
      sG[r * kLdG + d] = run;
    }
  }
  __syncthreads();
  {
    const int d = tid & 127;
    const int half = tid >> 7;
    if (half == 1) {
      const float base = sG[31 * kLdG + d];
      for (int r = 32; r < 64; ++r) sG[r * kLdG + d] += base;
    }
  }
  __syncthreads();
  {
    float* gdst = a.gk + cm * (kChunk * kDim);
    for (int idx = tid; idx < kChunk * kDim / 4; idx += 256) {
      const int r = idx >> 5, c4 = (idx & 31) * 4;
      *reinterpret_cast<float4*>(gdst + r * kDim + c4) =
          make_float4(sG[r * kLdG + c4], sG[r * kLdG + c4 + 1], sG[r * kLdG + c4 + 2], sG[r * kLdG + c4 + 3]);
    }
  }

  // off-diagonal tiles I > J on MFMA, rows scaled against r = 16 I; the
  // k k^T product carries hi + lo operands (it feeds the inverse), the
  // q k^T product single bf16 operands. Wave w: jobs w and w + 4.
  f32x4 accA[2], accQ[2];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int job = wave + 4 * jj;
    accA[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
    accQ[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (job >= 6) continue;
    int t = job, I = 1;
    while (t >= I) { t -= I; ++I; }
    const int J = t;
    const int r = 16 * I;
    const int i = 16 * I + l16;   // A-operand row
    const int j = 16 * J + l16;   // B-operand row (column of the product)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u16x8 lk_hi, lk_lo, lq, rr_hi, rr_lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = 32 * s + 8 * g4 + e;
        const float gr = sG[r * kLdG + d];
        const float fi = exp2f(sG[i * kLdG + d] - gr);
        const float fj = exp2f(gr - sG[j * kLdG + d]);
        uint16_t hh, ll;
        split_bf(bf2f(sk[i * kLdRow + d]) * fi, hh, ll);
        lk_hi[e] = hh; lk_lo[e] = ll;
        lq[e] = f2bf(bf2f(sq[i * kLdRow + d]) * fi);
        split_bf(bf2f(sk[j * kLdRow + d]) * fj, hh, ll);
        rr_hi[e] = hh; rr_lo[e] = ll;
      }
      accA[jj] = mfma16(lk_hi, rr_hi, accA[jj]);
      accA[jj] = mfma16(lk_hi, rr_lo, accA[jj]);
      accA[jj] = mfma16(lk_lo, rr_hi, accA[jj]);
      accQ[jj] = mfma16(lq, rr_hi, accQ[jj]);
    }
  }

  // diagonal tiles: pairs i >= j of each 16-row block, elementwise
  float dkk[3], dqk[3];
#pragma unroll
  for (int pp = 0; pp < 3; ++pp) {
    const int p = tid + 256 * pp;
    dkk[pp] = 0.f;
    dqk[pp] = 0.f;
    if (p >= 4 * 136) continue;
    const int I = p / 136;
    int rem = p - I * 136, il = 0;
    while (rem > il) { rem -= il + 1; ++il; }
    const int i = 16 * I + il, j = 16 * I + rem;
    float skk = 0.f, sqk = 0.f;
    for (int d = 0; d < kDim; d += 4) {
      const float4 gi = *reinterpret_cast<const float4*>(sG + i * kLdG + d);
      const float4 gj = *reinterpret_cast<const float4*>(sG + j * kLdG + d);
      const u16x4 ki = *reinterpret_cast<const u16x4*>(sk + i * kLdRow + d);
      const u16x4 kj = *reinterpret_cast<const u16x4*>(sk + j * kLdRow + d);
      const u16x4 qi = *reinterpret_cast<const u16x4*>(sq + i * kLdRow + d);
      const float e0 = exp2f(gi.x - gj.x), e1 = exp2f(gi.y - gj.y);
      const float e2 = exp2f(gi.z - gj.z), e3 = exp2f(gi.w - gj.w);
      const float w0 = bf2f(kj[0]) * e0, w1 = bf2f(kj[1]) * e1, w2 = bf2f(kj[2]) * e2, w3 = bf2f(kj[3]) * e3;
      skk = fmaf(bf2f(ki[0]), w0, skk);
      skk = fmaf(bf2f(ki[1]), w1, skk);
      skk = fmaf(bf2f(ki[2]), w2, skk);
      skk = fmaf(bf2f(ki[3]), w3, skk);
      sqk = fmaf(bf2f(qi[0]), w0, sqk);
      sqk = fmaf(bf2f(qi[1]), w1, sqk);
      sqk = fmaf(bf2f(qi[2]), w2, sqk);
      sqk = fmaf(bf2f(qi[3]), w3, sqk);
    }
    dkk[pp] = skk;
    dqk[pp] = sqk;
  }
  __syncthreads();

  // results into the reused LDS
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int job = wave + 4 * jj;
    if (job >= 6) continue;
    int t = job, I = 1;
    while (t >= I) { t -= I; ++I; }
    const int J = t;
    const int jc = 16 * J + l16;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int ii = 16 * I + 4 * g4 + e;
      u.mat.A[ii * kLdF + jc] = -sBeta[ii] * sRk[ii] * sRk[jc] * accA[jj][e];
      u.mat.aqk[ii * kLdQ + jc] = f2bf(a.scale * sRq[ii] * sRk[jc] * accQ[jj][e]);
    }
  }
  for (int idx = tid; idx < 4 * 256; idx += 256) {
    const int I = idx >> 8, il = (idx >> 4) & 15, jl = idx & 15;
    if (il < jl) u.mat.aqk[(16 * I + il) * kLdQ + 16 * I + jl] = 0;
  }
#pragma unroll
  for (int pp = 0; pp < 3; ++pp) {
    const int p = tid + 256 * pp;
    if (p >= 4 * 136) continue;
    const int I = p / 136;
    int rem = p - I * 136, il = 0;
    while (rem > il) { rem -= il + 1; ++il; }
    const int i = 16 * I + il, j = 16 * I + rem;
    u.mat.A[i * kLdF + j] = (i > j) ? -sBeta[i] * sRk[i] * sRk[j] * dkk[pp] : 0.0f;
    u.mat.aqk[i * kLdQ + j] = f2bf(a.scale * sRq[i] * sRk[j] * dqk[pp]);
  }
  __syncthreads();

  invert_unit_lower(u.mat.A, u.mat.T, wave, lane);

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
  if (kda) {
    hipLaunchKernelGGL(kda_prepare_kernel, dim3(a.geo.NT, a.H), dim3(256), 0, stream, a);
  } else {
    // three workgroups fit a compute unit (43.5 KiB of LDS each)
    const long items = (long)a.geo.NT * a.H;
    const long slots = 3L * (a.cus > 0 ? a.cus : 256);
    hipLaunchKernelGGL(gdn_prepare_kernel, dim3((unsigned)(items < slots ? items : slots)), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace gdn
