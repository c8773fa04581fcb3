// Backward pass of the chunked gated delta rule, scalar (GDN) gate, on gfx950.
//
// The stage split of _GDNStateP2PTritonFunction.backward on the hyper-parallel
// "Diff Coverage" page of the 2026-09-10 gate build: recompute the forward
// intermediates (prepare + chunk_fwd_h, run by the caller with the forward
// kernels), then a reverse sequential pass over the chunks for the state
// gradient (bwd_state_saved), then the per-chunk input gradients
// (bwd_finish_saved). As the native backward of the 2026-11-06 gate build's
// GDN training function, the gate gradient returned is the one of the raw
// per-token gate g (the chunk-local cumulative sum differentiated back).
//
// Per chunk (K x V state S entering it, rows i of the chunk, G the chunk-local
// cumulative gate, G_L its last valid value, b = beta, qn/kn the normalised
// rows, T = (I - A)^-1 with A[i,j] = -b_i kn_i.kn_j e^(G_i - G_j) for i > j):
//   W = T diag(b e^G) Kn,  U = T diag(b) V,  V' = U - W S,
//   O = scale [diag(e^G) Qn S + (Qn Kn^T * Gamma) V'],
//   S_next = e^(G_L) S + Kn^T diag(e^(G_L - G)) V'.
// Given dO and dS_next (the gradient w.r.t. the state leaving the chunk):
//   dV' = diag(e^(G_L - G)) Kn dS_next + Aqk^T dO        (Aqk = scale Qn Kn^T * Gamma)
//   dS  = e^(G_L) dS_next + scale (diag(e^G) Qn)^T dO - W^T dV'
// run backwards over the chunks (kernel 1); then, chunk by chunk, with
// E = dO S^T, F = dV' S^T, D = V' dS_next^T (kernel 2):
//   dQn = scale [diag(e^G) E + (dO V'^T * Gamma) Kn]
//   dKn = diag(e^(G_L - G)) D + scale (dO V'^T * Gamma)^T Qn + b e^G dX
//         - diag(b) P Kn - P^T diag(b) Kn
//   dX = -T^T F,  dY = T^T dV',  dv = b dY,
//   dA = strictLower(T^T (-F X^T + dV' Y^T) T^T),  P = dA * Gamma,
// and the row sums that give d beta and dG; dg is the reverse cumulative sum
// of dG inside the chunk; the L2-norm and sigmoid are differentiated last
// (kernel 3).
//
// All products run on v_mfma_f32_16x16x4f32 (fp32 operands, fp32
// accumulation): the state and its gradient are never rounded to bf16.
#include "gdn_bwd.h"

namespace gdn {

namespace {

constexpr int kL128 = 132;  // fp32 LDS row stride of 64/128-row x 128 matrices
constexpr int kL64 = 68;    // fp32, 64 wide
constexpr int kL32 = 36;    // fp32, 32 wide
constexpr int kLb = 136;    // bf16, 128 wide
constexpr int kVecStride = kVecRows * kChunk;

__device__ __forceinline__ float ldv(const float* p) { return *p; }
__device__ __forceinline__ float ldv(const uint16_t* p) { return bf2f(*p); }

// One 16x16 output tile of C = op(A) op(B) on v_mfma_f32_16x16x4f32:
// acc (lane (g, l) holds C[r0 + 4g + e][c0 + l]) += sum_k A(r, k) B(k, c),
// k over [0, kd), kd a multiple of 16. A(r, k) is a[r * sar + k * sak] and
// B(k, c) is b[k * sbk + c * sbc] (LDS, fp32 or bf16), so transposed
// operands are a matter of strides. Contraction slot g at step ks is
// k0 + 4g + ks for both operands.
template <class TA, class TB>
__device__ __forceinline__ f32x4 tile_mm(const TA* a, int sar, int sak, const TB* b, int sbk, int sbc, int r0,
                                         int c0, int kd, int lane, f32x4 acc) {
  const int l = lane & 15, g = lane >> 4;
  const TA* ap = a + (r0 + l) * sar + 4 * g * sak;
  const TB* bp = b + (c0 + l) * sbc + 4 * g * sbk;
  for (int k0 = 0; k0 < kd; k0 += 16) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ldv(ap + (k0 + ks) * sak), ldv(bp + (k0 + ks) * sbk), acc, 0, 0, 0);
  }
  return acc;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// sum over the 16 lanes of a row group (lanes with the same lane / 16)
__device__ __forceinline__ float sum16(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  x += __shfl_xor(x, 8);
  return x;
}

// T (fp32, natural column order, stride kL64) from the prepare kernel's
// bf16 hi | lo rows with permuted columns
__device__ __forceinline__ void load_t(float* sT, const uint16_t* tm, int tid) {
  for (int idx = tid; idx < kChunk * kChunk; idx += 256) {
    const int r = idx >> 6, p = idx & 63;
    sT[r * kL64 + unperm_col(p)] = bf2f(tm[r * 128 + p]) + bf2f(tm[r * 128 + 64 + p]);
  }
}

// ===========================================================================
// Kernel 1: reverse state pass. One workgroup per (sequence, head, 32 value
// columns); the state gradient block (128 x 32) lives in registers, wave w
// holding rows 32w .. 32w+31.
// ===========================================================================
struct DhSmem {
  float k[kChunk * kL128];   // raw k
  float qg[kChunk * kL128];  // q scaled by scale rq e^G
  float aqk[kChunk * kL64];  // scale Qn Kn^T * Gamma (lower, with diagonal)
  float t[kChunk * kL64];
  float dO[kChunk * kL32];
  float dS[kDim * kL32];
  float z[kChunk * kL32];    // dV', then diag(b rk e^G) T^T dV'
  float kgs[kChunk], xs[kChunk];
};

__global__ __launch_bounds__(256, 1) void gdn_bwd_dh_kernel(BwdArgs a) {
  int n, h, vb;
  if (!state_unit(a.geo, a.H, 4, n, h, vb)) return;
  __shared__ DhSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l = lane & 15, g = lane >> 4;
  const int v0 = 32 * vb;
  const int H = a.H;
  const SeqInfo si = a.geo.seq(n);
  const size_t unit = (size_t)n * H + h;

  f32x4 ds[2][2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 32 * w + 16 * rt + 4 * g + e, col = v0 + 16 * ct + l;
        ds[rt][ct][e] = a.dsfinal ? a.dsfinal[(unit * kDim + row) * kDim + col] : 0.0f;
      }

  for (int jc = si.nch - 1; jc >= 0; --jc) {
    const int c = si.c0 + jc;
    const ChunkInfo ci = a.geo.chunk(c);
    const size_t cm = (size_t)h * a.geo.NT + c;
    const float* vec = a.vec + cm * kVecStride;
    // gradient w.r.t. the state leaving chunk c
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 32 * w + 16 * rt + 4 * g + e, col = 16 * ct + l;
          a.dhn[cm * (kDim * kDim) + row * kDim + v0 + col] = ds[rt][ct][e];
          sm.dS[row * kL32 + col] = ds[rt][ct][e];
        }
    for (int idx = tid; idx < kChunk * 16; idx += 256) {
      const int r = idx >> 4, cc = (idx & 15) * 8;
      u16x8 kv = u16x8{0, 0, 0, 0, 0, 0, 0, 0}, qv = kv;
      float qs = 0.0f;
      if (r < ci.len) {
        const size_t off = ((size_t)(ci.tok0 + r) * H + h) * kDim + cc;
        kv = *reinterpret_cast<const u16x8*>(a.k + off);
        qv = *reinterpret_cast<const u16x8*>(a.q + off);
        qs = vec[3 * kChunk + r];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sm.k[r * kL128 + cc + e] = bf2f(kv[e]);
        sm.qg[r * kL128 + cc + e] = bf2f(qv[e]) * qs;
      }
    }
    for (int idx = tid; idx < kChunk * kChunk; idx += 256) {
      const int r = idx >> 6, p = idx & 63;
      sm.aqk[r * kL64 + unperm_col(p)] = bf2f(a.aqk[cm * 4096 + idx]);
    }
    load_t(sm.t, a.tmat + cm * (kChunk * 128), tid);
    {
      const int r = tid >> 2, cc = (tid & 3) * 8;
      u16x8 dv = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
      if (r < ci.len) dv = *reinterpret_cast<const u16x8*>(a.dout + ((size_t)(ci.tok0 + r) * H + h) * kDim + v0 + cc);
#pragma unroll
      for (int e = 0; e < 8; ++e) sm.dO[r * kL32 + cc + e] = bf2f(dv[e]);
    }
    if (tid < kChunk) {
      const bool ok = tid < ci.len;
      sm.kgs[tid] = ok ? vec[2 * kChunk + tid] : 0.0f;
      sm.xs[tid] = ok ? vec[1 * kChunk + tid] : 0.0f;
    }
    const float eL = vec[7 * kChunk];
    __syncthreads();

    // dV' = diag(rk e^(G_L - G)) k dS + Aqk^T dO   (rows 16w .. 16w+15)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      f32x4 acc = tile_mm(sm.k, kL128, 1, sm.dS, kL32, 1, 16 * w, 16 * ct, kDim, lane, zero4());
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] *= sm.kgs[16 * w + 4 * g + e];
      acc = tile_mm(sm.aqk, 1, kL64, sm.dO, kL32, 1, 16 * w, 16 * ct, kChunk, lane, acc);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * w + 4 * g + e, col = 16 * ct + l;
        a.dvn[cm * (kChunk * kDim) + row * kDim + v0 + col] = acc[e];
        sm.z[row * kL32 + col] = acc[e];
      }
    }
    __syncthreads();
    // Z = diag(b rk e^G) T^T dV'
    f32x4 zz[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      zz[ct] = tile_mm(sm.t, 1, kL64, sm.z, kL32, 1, 16 * w, 16 * ct, kChunk, lane, zero4());
#pragma unroll
      for (int e = 0; e < 4; ++e) zz[ct][e] *= sm.xs[16 * w + 4 * g + e];
    }
    __syncthreads();
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.z[(16 * w + 4 * g + e) * kL32 + 16 * ct + l] = zz[ct][e];
    __syncthreads();
    // dS = e^(G_L) dS + qg^T dO - k^T Z   (W^T dV' = k^T Z)
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const int r0 = 32 * w + 16 * rt;
        f32x4 acc = ds[rt][ct] * eL;
        acc = tile_mm(sm.qg, 1, kL128, sm.dO, kL32, 1, r0, 16 * ct, kChunk, lane, acc);
        const f32x4 t = tile_mm(sm.k, 1, kL128, sm.z, kL32, 1, r0, 16 * ct, kChunk, lane, zero4());
        ds[rt][ct] = acc - t;
      }
    __syncthreads();
  }
  if (a.ds0) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 32 * w + 16 * rt + 4 * g + e, col = v0 + 16 * ct + l;
          a.ds0[(unit * kDim + row) * kDim + col] = ds[rt][ct][e];
        }
  }
}

// ===========================================================================
// Kernel 2: products with the chunk's state and state gradient, one
// workgroup per (chunk, head): E = dO S^T, F = dV' S^T, D = V' dS_next^T
// (64 x 128 each) and <dS_next, S>. Wave w computes rows 16w .. 16w+15.
// ===========================================================================
struct SpSmem {
  float s[kDim * kL128];     // S, then dS_next
  float x[kChunk * kL128];   // dO, then V'
  float y[kChunk * kL128];   // dV'
  float red[4];
};

__global__ __launch_bounds__(256, 1) void gdn_bwd_sprod_kernel(BwdArgs a) {
  __shared__ SpSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l = lane & 15, g = lane >> 4;
  const int NT = a.geo.NT;
  const size_t cm = blockIdx.x;
  const int h = (int)(cm / NT), c = (int)(cm % NT);
  const ChunkInfo ci = a.geo.chunk(c);
  const int H = a.H;
  const size_t plane = (size_t)a.H * NT * kChunk * kDim;

  const float* S = a.h + cm * (kDim * kDim);
  for (int idx = tid; idx < kDim * kDim / 4; idx += 256) {
    const int r = idx >> 5, cc = (idx & 31) * 4;
    *reinterpret_cast<float4*>(sm.s + r * kL128 + cc) = *reinterpret_cast<const float4*>(S + r * kDim + cc);
  }
  for (int idx = tid; idx < kChunk * 16; idx += 256) {
    const int r = idx >> 4, cc = (idx & 15) * 8;
    u16x8 dv = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
    if (r < ci.len) dv = *reinterpret_cast<const u16x8*>(a.dout + ((size_t)(ci.tok0 + r) * H + h) * kDim + cc);
#pragma unroll
    for (int e = 0; e < 8; ++e) sm.x[r * kL128 + cc + e] = bf2f(dv[e]);
  }
  const float* dvn = a.dvn + cm * (kChunk * kDim);
  for (int idx = tid; idx < kChunk * kDim / 4; idx += 256) {
    const int r = idx >> 5, cc = (idx & 31) * 4;
    *reinterpret_cast<float4*>(sm.y + r * kL128 + cc) = *reinterpret_cast<const float4*>(dvn + r * kDim + cc);
  }
  __syncthreads();

  float* E = a.efd + cm * (kChunk * kDim);
  float* F = E + plane;
  float* D = F + plane;
#pragma unroll 2
  for (int ct = 0; ct < 8; ++ct) {
    // B(v, kk) = S[kk][v]
    const f32x4 e4 = tile_mm(sm.x, kL128, 1, sm.s, 1, kL128, 16 * w, 16 * ct, kDim, lane, zero4());
    const f32x4 f4 = tile_mm(sm.y, kL128, 1, sm.s, 1, kL128, 16 * w, 16 * ct, kDim, lane, zero4());
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * w + 4 * g + e, col = 16 * ct + l;
      E[row * kDim + col] = e4[e];
      F[row * kDim + col] = f4[e];
    }
  }
  __syncthreads();

  const float* dSn = a.dhn + cm * (kDim * kDim);
  float part = 0.0f;
  for (int idx = tid; idx < kDim * kDim / 4; idx += 256) {
    const int r = idx >> 5, cc = (idx & 31) * 4;
    const float4 nv = *reinterpret_cast<const float4*>(dSn + r * kDim + cc);
    float4* dst = reinterpret_cast<float4*>(sm.s + r * kL128 + cc);
    const float4 ov = *dst;
    part += ov.x * nv.x + ov.y * nv.y + ov.z * nv.z + ov.w * nv.w;
    *dst = nv;
  }
  const float* vn = a.vnew + cm * (kChunk * kDim);
  for (int idx = tid; idx < kChunk * kDim / 4; idx += 256) {
    const int r = idx >> 5, cc = (idx & 31) * 4;
    *reinterpret_cast<float4*>(sm.x + r * kL128 + cc) = *reinterpret_cast<const float4*>(vn + r * kDim + cc);
  }
  part += __shfl_xor(part, 16);
  part += __shfl_xor(part, 32);
  part = sum16(part);
  if (lane == 0) sm.red[w] = part;
  __syncthreads();
  if (tid == 0) a.sdot[cm] = (sm.red[0] + sm.red[1]) + (sm.red[2] + sm.red[3]);
#pragma unroll 2
  for (int ct = 0; ct < 8; ++ct) {
    const f32x4 d4 = tile_mm(sm.x, kL128, 1, sm.s, 1, kL128, 16 * w, 16 * ct, kDim, lane, zero4());
#pragma unroll
    for (int e = 0; e < 4; ++e) D[(16 * w + 4 * g + e) * kDim + 16 * ct + l] = d4[e];
  }
}

// ===========================================================================
// Kernel 3: input gradients of one (chunk, head). Wave w owns rows
// 16w .. 16w+15 of every 64-row result; per-row sums (d beta, dG) are kept
// per lane and reduced at the end, column sums through LDS partials.
// ===========================================================================
struct InSmem {
  uint16_t q[kChunk * kLb], k[kChunk * kLb], v[kChunk * kLb], dO[kChunk * kLb];
  float t[kChunk * kL64];
  float m1[kChunk * kL64];
  float m2[kChunk * kL64];
  float x[kChunk * kL128];  // V', then F, then dV'
  float b[kChunk], G[kChunk], rq[kChunk], rk[kChunk];
  float colg[4][kChunk];
  float rowg[kChunk], rowb[kChunk];
  float red[4];
};

__device__ __forceinline__ void load_f32_rows(float* dst, const float* src, int tid) {
  for (int idx = tid; idx < kChunk * kDim / 4; idx += 256) {
    const int r = idx >> 5, cc = (idx & 31) * 4;
    *reinterpret_cast<float4*>(dst + r * kL128 + cc) = *reinterpret_cast<const float4*>(src + r * kDim + cc);
  }
}

__global__ __launch_bounds__(256, 1) void gdn_bwd_intra_kernel(BwdArgs a) {
  __shared__ InSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l = lane & 15, g = lane >> 4;
  const int NT = a.geo.NT;
  const size_t cm = blockIdx.x;
  const int h = (int)(cm / NT), c = (int)(cm % NT);
  const ChunkInfo ci = a.geo.chunk(c);
  const int L = ci.len;
  const int H = a.H;
  const float scale = a.scale;
  const size_t plane = (size_t)a.H * NT * kChunk * kDim;
  const float* vec = a.vec + cm * kVecStride;

  for (int idx = tid; idx < kChunk * 16; idx += 256) {
    const int r = idx >> 4, cc = (idx & 15) * 8;
    uint4 qv = make_uint4(0, 0, 0, 0), kv = qv, vv = qv, ov = qv;
    if (r < L) {
      const size_t off = ((size_t)(ci.tok0 + r) * H + h) * kDim + cc;
      qv = *reinterpret_cast<const uint4*>(a.q + off);
      kv = *reinterpret_cast<const uint4*>(a.k + off);
      vv = *reinterpret_cast<const uint4*>(a.v + off);
      ov = *reinterpret_cast<const uint4*>(a.dout + off);
    }
    *reinterpret_cast<uint4*>(sm.q + r * kLb + cc) = qv;
    *reinterpret_cast<uint4*>(sm.k + r * kLb + cc) = kv;
    *reinterpret_cast<uint4*>(sm.v + r * kLb + cc) = vv;
    *reinterpret_cast<uint4*>(sm.dO + r * kLb + cc) = ov;
  }
  load_t(sm.t, a.tmat + cm * (kChunk * 128), tid);
  load_f32_rows(sm.x, a.vnew + cm * (kChunk * kDim), tid);
  if (tid < kChunk) {
    const bool ok = tid < L;
    sm.b[tid] = ok ? vec[0 * kChunk + tid] : 0.0f;
    sm.G[tid] = ok ? vec[4 * kChunk + tid] : 0.0f;
    sm.rq[tid] = ok ? vec[5 * kChunk + tid] : 0.0f;
    sm.rk[tid] = ok ? vec[6 * kChunk + tid] : 0.0f;
  }
  __syncthreads();

  // this lane's rows i = 16w + 4g + e
  float rb_[4], rG[4], rq_[4], rk_[4], eG[4], er[4];
  bool okr[4];
  const float GL = sm.G[L - 1];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = 16 * w + 4 * g + e;
    okr[e] = i < L;
    rb_[e] = sm.b[i];
    rG[e] = sm.G[i];
    rq_[e] = sm.rq[i];
    rk_[e] = sm.rk[i];
    eG[e] = okr[e] ? __expf(rG[e]) : 0.0f;
    er[e] = okr[e] ? __expf(GL - rG[e]) : 0.0f;
  }
  float accG[4] = {0.f, 0.f, 0.f, 0.f}, accB[4] = {0.f, 0.f, 0.f, 0.f};
  float colG[4] = {0.f, 0.f, 0.f, 0.f};

  // ---- dO V'^T and Qn Kn^T on the lower tiles: the o-term gradients -----
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    f32x4 m1v = zero4(), m2v = zero4();
    if (ct <= w) {
      const f32x4 p1 = tile_mm(sm.dO, kLb, 1, sm.x, 1, kL128, 16 * w, 16 * ct, kDim, lane, zero4());
      const f32x4 mq = tile_mm(sm.q, kLb, 1, sm.k, 1, kLb, 16 * w, 16 * ct, kDim, lane, zero4());
      const int j = 16 * ct + l;
      const float Gj = sm.G[j], rkj = sm.rk[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * w + 4 * g + e;
        if (j <= i && okr[e]) {
          const float sp = scale * p1[e] * __expf(rG[e] - Gj);
          const float z = sp * rq_[e] * rkj * mq[e];
          accG[e] += z;
          colG[ct] -= z;
          m1v[e] = sp * rkj;
          m2v[e] = sp * rq_[e];
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sm.m1[(16 * w + 4 * g + e) * kL64 + 16 * ct + l] = m1v[e];
      sm.m2[(16 * w + 4 * g + e) * kL64 + 16 * ct + l] = m2v[e];
    }
  }
  __syncthreads();
  load_f32_rows(sm.x, a.efd + plane + cm * (kChunk * kDim), tid);  // F

  f32x4 dq[8], dk[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) {
    dq[ct] = tile_mm(sm.m1, kL64, 1, sm.k, kLb, 1, 16 * w, 16 * ct, kChunk, lane, zero4());
    dk[ct] = tile_mm(sm.m2, 1, kL64, sm.q, kLb, 1, 16 * w, 16 * ct, kChunk, lane, zero4());
  }
  __syncthreads();

  // ---- F: dX = -T^T F, and -F X^T into dT -------------------------------
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) {
    const f32x4 t = tile_mm(sm.t, 1, kL64, sm.x, kL128, 1, 16 * w, 16 * ct, kChunk, lane, zero4());
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * w + 4 * g + e;
      const float kv = bf2f(sm.k[i * kLb + 16 * ct + l]);
      dk[ct][e] -= rb_[e] * eG[e] * t[e];
      const float tk = -rk_[e] * eG[e] * t[e] * kv;  // e^G dX_i . kn_i, one column
      accB[e] += tk;
      accG[e] += rb_[e] * tk;
    }
  }
  f32x4 dT[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const f32x4 t = tile_mm(sm.x, kL128, 1, sm.k, 1, kLb, 16 * w, 16 * ct, kDim, lane, zero4());
    const int j = 16 * ct + l;
    const float xs = j < L ? sm.b[j] * sm.rk[j] * __expf(sm.G[j]) : 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) dT[ct][e] = -t[e] * xs;
  }
  __syncthreads();
  load_f32_rows(sm.x, a.dvn + cm * (kChunk * kDim), tid);  // dV'
  __syncthreads();

  // ---- dV': dY = T^T dV', dv = b dY, and dV' Y^T into dT -----------------
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) {
    const f32x4 t = tile_mm(sm.t, 1, kL64, sm.x, kL128, 1, 16 * w, 16 * ct, kChunk, lane, zero4());
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * w + 4 * g + e, col = 16 * ct + l;
      accB[e] += t[e] * bf2f(sm.v[i * kLb + col]);
      if (okr[e]) a.dv[((size_t)(ci.tok0 + i) * H + h) * kDim + col] = rb_[e] * t[e];
    }
  }
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const f32x4 t = tile_mm(sm.x, kL128, 1, sm.v, 1, kLb, 16 * w, 16 * ct, kDim, lane, zero4());
    const float bj = sm.b[16 * ct + l];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dT[ct][e] += t[e] * bj;
      sm.m1[(16 * w + 4 * g + e) * kL64 + 16 * ct + l] = dT[ct][e];
    }
  }
  __syncthreads();

  // ---- dA = strictLower(T^T dT T^T) ---------------------------------------
  f32x4 q1[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) q1[ct] = tile_mm(sm.t, 1, kL64, sm.m1, kL64, 1, 16 * w, 16 * ct, kChunk, lane, zero4());
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int e = 0; e < 4; ++e) sm.m2[(16 * w + 4 * g + e) * kL64 + 16 * ct + l] = q1[ct][e];
  __syncthreads();
  f32x4 pa[4], pb[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    pa[ct] = zero4();
    pb[ct] = zero4();
    if (ct <= w) {
      const f32x4 dA = tile_mm(sm.m2, kL64, 1, sm.t, 1, kL64, 16 * w, 16 * ct, kChunk, lane, zero4());
      const f32x4 mk = tile_mm(sm.k, kLb, 1, sm.k, 1, kLb, 16 * w, 16 * ct, kDim, lane, zero4());
      const int j = 16 * ct + l;
      const float Gj = sm.G[j], rkj = sm.rk[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * w + 4 * g + e;
        if (j < i && okr[e]) {
          const float gam = __expf(rG[e] - Gj);
          const float mkk = rk_[e] * rkj * mk[e];
          const float Aij = -rb_[e] * mkk * gam;
          const float z = dA[e] * Aij;
          accG[e] += z;
          colG[ct] -= z;
          const float P = dA[e] * gam;
          accB[e] -= P * mkk;
          pa[ct][e] = -rb_[e] * P * rkj;
          pb[ct][e] = -P * rb_[e] * rk_[e];
        }
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sm.m1[(16 * w + 4 * g + e) * kL64 + 16 * ct + l] = pa[ct][e];
      sm.m2[(16 * w + 4 * g + e) * kL64 + 16 * ct + l] = pb[ct][e];
    }
  __syncthreads();
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) {
    dk[ct] = tile_mm(sm.m1, kL64, 1, sm.k, kLb, 1, 16 * w, 16 * ct, kChunk, lane, dk[ct]);
    dk[ct] = tile_mm(sm.m2, 1, kL64, sm.k, kLb, 1, 16 * w, 16 * ct, kChunk, lane, dk[ct]);
  }

  // ---- E = dO S^T and D = V' dS_next^T -----------------------------------
  const float* E = a.efd + cm * (kChunk * kDim);
  const float* D = E + 2 * plane;
  float cl = 0.0f;
#pragma unroll
  for (int ct = 0; ct < 8; ++ct)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * w + 4 * g + e, col = 16 * ct + l;
      if (okr[e]) {
        const float Ev = E[i * kDim + col], Dv = D[i * kDim + col];
        dq[ct][e] += scale * eG[e] * Ev;
        accG[e] += scale * eG[e] * rq_[e] * Ev * bf2f(sm.q[i * kLb + col]);
        dk[ct][e] += er[e] * Dv;
        const float cc = er[e] * rk_[e] * Dv * bf2f(sm.k[i * kLb + col]);
        accG[e] -= cc;
        cl += cc;
      }
    }

  // ---- L2-norm backward, outputs dq, dk ------------------------------------
  const bool l2 = (a.flags & 1u) != 0;
  float sq[4] = {0.f, 0.f, 0.f, 0.f}, sk[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ct = 0; ct < 8; ++ct)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * w + 4 * g + e, col = 16 * ct + l;
      sq[e] += bf2f(sm.q[i * kLb + col]) * dq[ct][e];
      sk[e] += bf2f(sm.k[i * kLb + col]) * dk[ct][e];
    }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    sq[e] = sum16(sq[e]);
    sk[e] = sum16(sk[e]);
  }
#pragma unroll
  for (int ct = 0; ct < 8; ++ct)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * w + 4 * g + e, col = 16 * ct + l;
      if (!okr[e]) continue;
      float gq = dq[ct][e], gk = dk[ct][e];
      if (l2) {
        // d x = r (d xn - xn (xn . d xn)), xn = r x
        gq = rq_[e] * (gq - rq_[e] * rq_[e] * bf2f(sm.q[i * kLb + col]) * sq[e]);
        gk = rk_[e] * (gk - rk_[e] * rk_[e] * bf2f(sm.k[i * kLb + col]) * sk[e]);
      }
      const size_t off = ((size_t)(ci.tok0 + i) * H + h) * kDim + col;
      a.dq[off] = gq;
      a.dk[off] = gk;
    }

  // ---- row and column sums: d beta and dG, then dg ------------------------
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    accG[e] = sum16(accG[e]);
    accB[e] = sum16(accB[e]);
  }
  if (l == 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sm.rowg[16 * w + 4 * g + e] = accG[e];
      sm.rowb[16 * w + 4 * g + e] = accB[e];
    }
  }
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    float x = colG[ct];
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    if (g == 0) sm.colg[w][16 * ct + l] = x;
  }
  cl += __shfl_xor(cl, 16);
  cl += __shfl_xor(cl, 32);
  cl = sum16(cl);
  if (lane == 0) sm.red[w] = cl;
  __syncthreads();
  if (w == 0) {
    // lane r holds chunk row 63 - r, so the inclusive scan over lanes is the
    // reverse cumulative sum over rows
    const int i = 63 - lane;
    float dG = 0.0f;
    if (i < L) {
      dG = sm.rowg[i] + ((sm.colg[0][i] + sm.colg[1][i]) + (sm.colg[2][i] + sm.colg[3][i]));
      if (i == L - 1) {
        const float eL = vec[7 * kChunk];
        dG += eL * a.sdot[cm] + ((sm.red[0] + sm.red[1]) + (sm.red[2] + sm.red[3]));
      }
    }
    float x = dG;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (i < L) {
      const size_t tok = (size_t)(ci.tok0 + i) * H + h;
      a.dg[tok] = x;
      const float bi = sm.b[i];
      const float db = sm.rowb[i];
      a.dbeta[tok] = (a.flags & 2u) ? db * bi * (1.0f - bi) : db;
    }
  }
}

}  // namespace

hipError_t launch_gdn_bwd(const BwdArgs& a, hipStream_t stream) {
  const unsigned units = state_grid(a.geo.N, a.H, 4);
  hipLaunchKernelGGL(gdn_bwd_dh_kernel, dim3(units), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned cms = (unsigned)((size_t)a.H * a.geo.NT);
  hipLaunchKernelGGL(gdn_bwd_sprod_kernel, dim3(cms), dim3(256), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gdn_bwd_intra_kernel, dim3(cms), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gdn
