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

// Four consecutive contraction slots k .. k+3 of row (or column) rc of an
// operand stored at p[rc * SR + k * SK] (LDS): one 16-byte (fp32) or 8-byte
// (bf16) read when the contraction index is the contiguous one.
template <int SR, int SK>
__device__ __forceinline__ void fetch4(const float* p, int rc, int k, float (&v)[4]) {
  if constexpr (SK == 1) {
    const float4 t = *reinterpret_cast<const float4*>(p + rc * SR + k);
    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = p[rc * SR + (k + j) * SK];
  }
}
template <int SR, int SK>
__device__ __forceinline__ void fetch4(const uint16_t* p, int rc, int k, float (&v)[4]) {
  if constexpr (SK == 1) {
    const uint2 t = *reinterpret_cast<const uint2*>(p + rc * SR + k);
    v[0] = __uint_as_float(t.x << 16); v[1] = __uint_as_float(t.x & 0xFFFF0000u);
    v[2] = __uint_as_float(t.y << 16); v[3] = __uint_as_float(t.y & 0xFFFF0000u);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = bf2f(p[rc * SR + (k + j) * SK]);
  }
}

// An fp32 operand kept in LDS as a bf16 hi | lo pair (value = hi + lo).
struct HL {
  const uint16_t* h;
  const uint16_t* l;
};
template <int SR, int SK>
__device__ __forceinline__ void fetch4(const HL& p, int rc, int k, float (&v)[4]) {
  float a[4], b[4];
  fetch4<SR, SK>(p.h, rc, k, a);
  fetch4<SR, SK>(p.l, rc, k, b);
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = a[j] + b[j];
}

// One 16x16 output tile of C = op(A) op(B) on v_mfma_f32_16x16x4f32:
// acc (lane (g, l) holds C[r0 + 4g + e][c0 + l]) += sum_k A(r, k) B(k, c),
// k over [0, kd), kd a multiple of 16. A(r, k) is a[r * SAR + k * SAK] and
// B(k, c) is b[k * SBK + c * SBC] (LDS, fp32 or bf16), so transposed
// operands are a matter of strides. Lane group g takes the contraction slots
// k0 + 4g .. k0 + 4g + 3 (one per MFMA step) of both operands.
template <int SAR, int SAK, int SBK, int SBC, class PA, class PB>
__device__ __forceinline__ f32x4 tile_mm(PA a, PB b, int r0, int c0, int kd, int lane, f32x4 acc) {
  const int l = lane & 15, g = lane >> 4;
  for (int k0 = 0; k0 < kd; k0 += 16) {
    float av[4], bv[4];
    fetch4<SAR, SAK>(a, r0 + l, k0 + 4 * g, av);
    fetch4<SBC, SBK>(b, c0 + l, k0 + 4 * g, bv);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[ks], bv[ks], acc, 0, 0, 0);
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

// ===========================================================================
// Kernel 1: reverse state pass. One workgroup of 8 waves per (sequence,
// head, block of 32 or 16 value columns); the state gradient block lives in
// registers, wave w holding rows 16w .. 16w+15. Products on
// v_mfma_f32_16x16x32_bf16: the
// inputs k, q, dO and the stored Aqk are exact in bf16; T comes as the
// prepare kernel's bf16 hi + lo pair; fp32 operands (dS, dV', Z, dO scaled
// by scale rq e^G) are split into hi + lo in LDS and both halves multiplied
// (hi*hi + hi*lo + lo*hi where both sides are split). Every operand sits in
// LDS with its contraction index contiguous (transposed where a product
// contracts over the chunk rows), so each MFMA operand is one 16-byte read.
// The next chunk's inputs are fetched into registers while the current one
// computes.
// ===========================================================================
constexpr int kLh = 72;  // bf16 row stride of 64-wide operands

template <int NCT>  // 16-column tiles of the value block: 2 (32 columns) or 1 (16)
struct alignas(16) DhSmem {
  uint16_t k[kChunk * kLb];                       // k [i][kk]
  uint16_t kT[kDim * kLh];                        // k^T [kk][i]
  uint16_t qT[kDim * kLh];                        // q^T [kk][i]
  uint16_t aqkT[kChunk * kLh];                    // Aqk^T [i][j]
  uint16_t tTh[kChunk * kLh], tTl[kChunk * kLh];  // T^T [j][i], hi and lo
  uint16_t dSTh[16 * NCT * kLb], dSTl[16 * NCT * kLb];    // dS^T [c][kk]
  uint16_t dOT[16 * NCT * kLh];                           // dO^T [c][i]
  uint16_t dOsTh[16 * NCT * kLh], dOsTl[16 * NCT * kLh];  // (diag(scale rq e^G) dO)^T
  uint16_t zTh[16 * NCT * kLh], zTl[16 * NCT * kLh];      // dV'^T, then Z^T
  float kgs[kChunk], xs[kChunk];
};

// one chunk's inputs in flight, per thread (512 threads). k and q: rows 2j,
// 2j+1 at columns 8c .. 8c+7 (j = tid % 32, c = tid / 32), so that the
// transposed copies take one 4-byte store per column. Threads 0..255: Aqk and
// T, rows 2j, 2j+1 at positions 8c .. 8c+7 (j = tid % 32, c = tid / 32).
// Threads 256..: dO, row t % 64, value columns 8 (t / 64) .. +7 (t = tid - 256).
struct DhRegs {
  u16x8 k[2], q[2];
  u16x8 a[2], th[2], tl[2];
  u16x8 o;
  float qgs, kgs, xs;
};

template <int NCT>
__device__ __forceinline__ void dh_fetch(const BwdArgs& a, int h, int c, int v0, int tid, DhRegs& R) {
  const ChunkInfo ci = a.geo.chunk(c);
  const size_t cm = (size_t)h * a.geo.NT + c;
  const float* vec = a.vec + cm * kVecStride;
  const u16x8 z8 = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
  {
    const int r0 = 2 * (tid & 31), cc = 8 * (tid >> 5);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int r = r0 + m;
      R.k[m] = z8;
      R.q[m] = z8;
      if (r < ci.len) {
        const size_t off = ((size_t)(ci.tok0 + r) * a.H + h) * kDim + cc;
        R.k[m] = *reinterpret_cast<const u16x8*>(a.k + off);
        R.q[m] = *reinterpret_cast<const u16x8*>(a.q + off);
      }
    }
  }
  if (tid < 256) {
    const uint16_t* aq = a.aqk + cm * 4096;
    const uint16_t* tm = a.tmat + cm * (kChunk * 128);
    const int r0 = 2 * (tid & 31), p8 = 8 * (tid >> 5);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int r = r0 + m;
      R.a[m] = *reinterpret_cast<const u16x8*>(aq + r * 64 + p8);
      R.th[m] = *reinterpret_cast<const u16x8*>(tm + r * 128 + p8);
      R.tl[m] = *reinterpret_cast<const u16x8*>(tm + r * 128 + 64 + p8);
    }
  } else {
    const int t = tid - 256, r = t & 63, cc = (t >> 6) * 8;
    R.o = z8;
    R.qgs = 0.0f;
    if (r < ci.len && t < 128 * NCT) {
      R.o = *reinterpret_cast<const u16x8*>(a.dout + ((size_t)(ci.tok0 + r) * a.H + h) * kDim + v0 + cc);
      R.qgs = vec[3 * kChunk + r];
    }
  }
  R.kgs = 0.0f;
  R.xs = 0.0f;
  if (tid < kChunk && tid < ci.len) {
    R.kgs = vec[2 * kChunk + tid];
    R.xs = vec[1 * kChunk + tid];
  }
}

template <int NCT>
__device__ __forceinline__ void dh_put(DhSmem<NCT>& sm, const DhRegs& R, int tid) {
  {
    const int r0 = 2 * (tid & 31), cc = 8 * (tid >> 5);
#pragma unroll
    for (int m = 0; m < 2; ++m) *reinterpret_cast<u16x8*>(sm.k + (r0 + m) * kLb + cc) = R.k[m];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      *reinterpret_cast<uint32_t*>(sm.kT + (cc + e) * kLh + r0) = (uint32_t)R.k[0][e] | ((uint32_t)R.k[1][e] << 16);
      *reinterpret_cast<uint32_t*>(sm.qT + (cc + e) * kLh + r0) = (uint32_t)R.q[0][e] | ((uint32_t)R.q[1][e] << 16);
    }
  }
  if (tid < 256) {
    const int r0 = 2 * (tid & 31), p8 = 8 * (tid >> 5);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int off = unperm_col(p8 + e) * kLh + r0;
      *reinterpret_cast<uint32_t*>(sm.aqkT + off) = (uint32_t)R.a[0][e] | ((uint32_t)R.a[1][e] << 16);
      *reinterpret_cast<uint32_t*>(sm.tTh + off) = (uint32_t)R.th[0][e] | ((uint32_t)R.th[1][e] << 16);
      *reinterpret_cast<uint32_t*>(sm.tTl + off) = (uint32_t)R.tl[0][e] | ((uint32_t)R.tl[1][e] << 16);
    }
  } else if (tid - 256 < 128 * NCT) {
    const int t = tid - 256, r = t & 63, cc = (t >> 6) * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sm.dOT[(cc + e) * kLh + r] = R.o[e];
      uint16_t hi, lo;
      split_bf(bf2f(R.o[e]) * R.qgs, hi, lo);
      sm.dOsTh[(cc + e) * kLh + r] = hi;
      sm.dOsTl[(cc + e) * kLh + r] = lo;
    }
  }
  if (tid < kChunk) {
    sm.kgs[tid] = R.kgs;
    sm.xs[tid] = R.xs;
  }
}

__device__ __forceinline__ u16x8 ld8(const uint16_t* p) { return *reinterpret_cast<const u16x8*>(p); }

// four consecutive values of column c (rows r0 .. r0+3 of a C tile) into a
// transposed hi | lo pair: dst[c * ld + r0 ..]
__device__ __forceinline__ void put_split4(uint16_t* dh, uint16_t* dl, int off, const f32x4& v) {
  u16x4 h4, l4;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint16_t hi, lo;
    split_bf(v[e], hi, lo);
    h4[e] = hi;
    l4[e] = lo;
  }
  *reinterpret_cast<u16x4*>(dh + off) = h4;
  *reinterpret_cast<u16x4*>(dl + off) = l4;
}

// 8 waves. dV' and Z (64 x 16 NCT): wave w takes the tile of row block w % 4
// and column block w / 4 (with one column block, waves 4..7 sit out). dS
// (128 x 16 NCT): wave w holds rows 16w .. 16w+15, all column blocks, in
// registers.
template <int NCT>
__global__ __launch_bounds__(512, 1) void gdn_bwd_dh_kernel(BwdArgs a) {
  constexpr int VB = 8 / NCT;  // value blocks of 16 NCT columns
  int n, h, vb;
  if (!state_unit(a.geo, a.H, VB, n, h, vb)) return;
  __shared__ DhSmem<NCT> sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l = lane & 15, g = lane >> 4;
  const int v0 = 16 * NCT * vb;
  const int H = a.H;
  const SeqInfo si = a.geo.seq(n);
  const size_t unit = (size_t)n * H + h;
  const int vrt = w & 3, vct = w >> 2;      // dV' / Z tile of this wave
  const bool vact = vct < NCT;

  f32x4 ds[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * w + 4 * g + e, col = v0 + 16 * ct + l;
      ds[ct][e] = a.dsfinal ? a.dsfinal[(unit * kDim + row) * kDim + col] : 0.0f;
    }

  DhRegs R;
  dh_fetch<NCT>(a, h, si.c0 + si.nch - 1, v0, tid, R);
  for (int jc = si.nch - 1; jc >= 0; --jc) {
    const int c = si.c0 + jc;
    const size_t cm = (size_t)h * a.geo.NT + c;
    dh_put<NCT>(sm, R, tid);
    // gradient w.r.t. the state leaving chunk c: to memory, and to LDS as dS^T
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int row0 = 16 * w + 4 * g, col = 16 * ct + l;
#pragma unroll
      for (int e = 0; e < 4; ++e) a.dhn[cm * (kDim * kDim) + (row0 + e) * kDim + v0 + col] = ds[ct][e];
      put_split4(sm.dSTh, sm.dSTl, col * kLb + row0, ds[ct]);
    }
    const float eL = a.vec[cm * kVecStride + 7 * kChunk];
    __syncthreads();
    if (jc > 0) dh_fetch<NCT>(a, h, c - 1, v0, tid, R);

    // dV' = diag(rk e^(G_L - G)) k dS + Aqk^T dO   (tile (vrt, vct))
    if (vact) {
      f32x4 acc = zero4();
      const uint16_t* ap = sm.k + (16 * vrt + l) * kLb + 8 * g;
      const int bo = (16 * vct + l) * kLb + 8 * g;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u16x8 av = ld8(ap + 32 * ks);
        acc = mfma16(av, ld8(sm.dSTh + bo + 32 * ks), acc);
        acc = mfma16(av, ld8(sm.dSTl + bo + 32 * ks), acc);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] *= sm.kgs[16 * vrt + 4 * g + e];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        acc = mfma16(ld8(sm.aqkT + (16 * vrt + l) * kLh + 32 * ks + 8 * g),
                     ld8(sm.dOT + (16 * vct + l) * kLh + 32 * ks + 8 * g), acc);
      const int row0 = 16 * vrt + 4 * g, col = 16 * vct + l;
#pragma unroll
      for (int e = 0; e < 4; ++e) a.dvn[cm * (kChunk * kDim) + (row0 + e) * kDim + v0 + col] = acc[e];
      put_split4(sm.zTh, sm.zTl, col * kLh + row0, acc);
    }
    __syncthreads();
    // Z = diag(b rk e^G) T^T dV'
    f32x4 zz = zero4();
    if (vact) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int ao = (16 * vrt + l) * kLh + 32 * ks + 8 * g, bo = (16 * vct + l) * kLh + 32 * ks + 8 * g;
        const u16x8 ah = ld8(sm.tTh + ao), bh = ld8(sm.zTh + bo);
        zz = mfma16(ah, bh, zz);
        zz = mfma16(ah, ld8(sm.zTl + bo), zz);
        zz = mfma16(ld8(sm.tTl + ao), bh, zz);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) zz[e] *= sm.xs[16 * vrt + 4 * g + e];
    }
    __syncthreads();
    if (vact) put_split4(sm.zTh, sm.zTl, (16 * vct + l) * kLh + 16 * vrt + 4 * g, zz);
    __syncthreads();
    // dS = e^(G_L) dS + q^T diag(scale rq e^G) dO - k^T Z   (W^T dV' = k^T Z)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int ar = (16 * w + l) * kLh + 8 * g, bc = (16 * ct + l) * kLh + 8 * g;
      f32x4 acc = ds[ct] * eL;
      f32x4 t = zero4();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const u16x8 aq = ld8(sm.qT + ar + 32 * ks), ak = ld8(sm.kT + ar + 32 * ks);
        acc = mfma16(aq, ld8(sm.dOsTh + bc + 32 * ks), acc);
        acc = mfma16(aq, ld8(sm.dOsTl + bc + 32 * ks), acc);
        t = mfma16(ak, ld8(sm.zTh + bc + 32 * ks), t);
        t = mfma16(ak, ld8(sm.zTl + bc + 32 * ks), t);
      }
      ds[ct] = acc - t;
    }
    __syncthreads();
  }
  if (a.ds0) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * w + 4 * g + e, col = v0 + 16 * ct + l;
        a.ds0[(unit * kDim + row) * kDim + col] = ds[ct][e];
      }
  }
}

// ===========================================================================
// Kernel 2: products with the chunk's state and state gradient, one
// workgroup of 8 waves per (chunk, head): E = dO S^T, F = dV' S^T,
// D = V' dS_next^T (64 x 128 each) and <dS_next, S>. Wave w computes rows
// 16 (w % 4) .. +15, columns 64 (w / 4) .. +63. Both operands of every
// product are contiguous along the contraction (S is [kk][v], contracted
// over v), so all run on v_mfma_f32_16x16x32_bf16: dO is exact in bf16, the
// fp32 operands (S, dS_next, dV', V') sit in LDS as bf16 hi | lo pairs.
// ===========================================================================
struct alignas(16) SpSmem {
  uint16_t sh[kDim * kLb], sl[kDim * kLb];      // S, then dS_next [kk][v]
  uint16_t dO[kChunk * kLb];                    // dO [i][v]
  uint16_t yh[kChunk * kLb], yl[kChunk * kLb];  // dV', then V' [i][v]
  float red[8];
};

// n rows of 128 fp32 into a bf16 hi | lo pair (stride kLb), 512 threads;
// optionally the dot product with the pair already there (before it is
// overwritten)
template <int ROWS, bool DOT>
__device__ __forceinline__ float load_split_512(uint16_t* dh, uint16_t* dl, const float* src, int tid) {
  constexpr int M = ROWS * 32 / 512;
  float4 v[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int idx = tid + 512 * m, r = idx >> 5, cc = (idx & 31) * 4;
    v[m] = *reinterpret_cast<const float4*>(src + r * kDim + cc);
  }
  float dot = 0.0f;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int idx = tid + 512 * m, r = idx >> 5, cc = (idx & 31) * 4;
    const int off = r * kLb + cc;
    if constexpr (DOT) {
      const u16x4 oh = *reinterpret_cast<const u16x4*>(dh + off), ol = *reinterpret_cast<const u16x4*>(dl + off);
      dot += (bf2f(oh[0]) + bf2f(ol[0])) * v[m].x + (bf2f(oh[1]) + bf2f(ol[1])) * v[m].y +
             (bf2f(oh[2]) + bf2f(ol[2])) * v[m].z + (bf2f(oh[3]) + bf2f(ol[3])) * v[m].w;
    }
    u16x4 h4, l4;
    const float x[4] = {v[m].x, v[m].y, v[m].z, v[m].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint16_t hi, lo;
      split_bf(x[e], hi, lo);
      h4[e] = hi;
      l4[e] = lo;
    }
    *reinterpret_cast<u16x4*>(dh + off) = h4;
    *reinterpret_cast<u16x4*>(dl + off) = l4;
  }
  return dot;
}

__global__ __launch_bounds__(512, 1) void gdn_bwd_sprod_kernel(BwdArgs a) {
  __shared__ SpSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l = lane & 15, g = lane >> 4;
  const int rt = w & 3, ch = w >> 2;
  const int NT = a.geo.NT;
  // heads fastest in dispatch order: neighbouring workgroups read the
  // neighbouring head rows of the same tokens
  const int c = (int)(blockIdx.x / a.H), h = (int)(blockIdx.x % a.H);
  const size_t cm = (size_t)h * NT + c;
  const ChunkInfo ci = a.geo.chunk(c);
  const int H = a.H;
  const size_t plane = (size_t)a.H * NT * kChunk * kDim;

  load_split_512<kDim, false>(sm.sh, sm.sl, a.h + cm * (kDim * kDim), tid);
  load_split_512<kChunk, false>(sm.yh, sm.yl, a.dvn + cm * (kChunk * kDim), tid);
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int idx = tid + 512 * m, r = idx >> 4, cc = (idx & 15) * 8;
    u16x8 dv = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
    if (r < ci.len) dv = *reinterpret_cast<const u16x8*>(a.dout + ((size_t)(ci.tok0 + r) * H + h) * kDim + cc);
    *reinterpret_cast<u16x8*>(sm.dO + r * kLb + cc) = dv;
  }
  __syncthreads();

  float* E = a.efd + cm * (kChunk * kDim);
  float* F = E + plane;
  float* D = F + plane;
  const int ao = (16 * rt + l) * kLb + 8 * g;
#pragma unroll 2
  for (int j = 0; j < 4; ++j) {
    const int ct = 4 * ch + j;
    const int bo = (16 * ct + l) * kLb + 8 * g;  // B(v, kk) = S[kk][v]
    f32x4 e4 = zero4(), f4 = zero4();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int k0 = 32 * ks;
      const u16x8 bh = ld8(sm.sh + bo + k0), bl = ld8(sm.sl + bo + k0);
      const u16x8 ad = ld8(sm.dO + ao + k0);
      e4 = mfma16(ad, bh, e4);
      e4 = mfma16(ad, bl, e4);
      const u16x8 ah = ld8(sm.yh + ao + k0);
      f4 = mfma16(ah, bh, f4);
      f4 = mfma16(ah, bl, f4);
      f4 = mfma16(ld8(sm.yl + ao + k0), bh, f4);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * rt + 4 * g + e, col = 16 * ct + l;
      E[row * kDim + col] = e4[e];
      F[row * kDim + col] = f4[e];
    }
  }
  __syncthreads();

  float part = load_split_512<kDim, true>(sm.sh, sm.sl, a.dhn + cm * (kDim * kDim), tid);
  load_split_512<kChunk, false>(sm.yh, sm.yl, a.vnew + cm * (kChunk * kDim), tid);
  part += __shfl_xor(part, 16);
  part += __shfl_xor(part, 32);
  part = sum16(part);
  if (lane == 0) sm.red[w] = part;
  __syncthreads();
  if (tid == 0)
    a.sdot[cm] = ((sm.red[0] + sm.red[1]) + (sm.red[2] + sm.red[3])) +
                 ((sm.red[4] + sm.red[5]) + (sm.red[6] + sm.red[7]));
#pragma unroll 2
  for (int j = 0; j < 4; ++j) {
    const int ct = 4 * ch + j;
    const int bo = (16 * ct + l) * kLb + 8 * g;
    f32x4 d4 = zero4();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int k0 = 32 * ks;
      const u16x8 bh = ld8(sm.sh + bo + k0), ah = ld8(sm.yh + ao + k0);
      d4 = mfma16(ah, bh, d4);
      d4 = mfma16(ah, ld8(sm.sl + bo + k0), d4);
      d4 = mfma16(ld8(sm.yl + ao + k0), bh, d4);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) D[(16 * rt + 4 * g + e) * kDim + 16 * ct + l] = d4[e];
  }
}

// ===========================================================================
// Kernel 3: input gradients of one (chunk, head), 8 waves. Wave w owns rows
// 16 (w % 4) .. +15 of every 64-row result and half of its column tiles
// (h = w / 4); per-row sums (d beta, dG, the L2-norm dots) are kept per lane,
// reduced over the 16 lanes of a row group and combined over the two halves
// through LDS; column sums go through LDS partials.
//
// fp32 intermediates (V', F, dV', the o-term and dA-derived matrices, dT, Q1)
// sit in LDS as bf16 hi | lo pairs. A product with one exact bf16 operand
// (q, k, v, dO) whose contraction index is contiguous on both sides runs on
// v_mfma_f32_16x16x32_bf16 (hi and lo each against the exact operand); the
// others (contractions over the chunk rows of F, dV', dT, and those with T)
// run on v_mfma_f32_16x16x4f32 with hi + lo summed on read.
// ===========================================================================
constexpr int kLp = 72;  // bf16 row stride of 64-wide matrices and of k^T [kk][i]

struct alignas(16) InSmem {
  uint16_t q[kChunk * kLb], k[kChunk * kLb], v[kChunk * kLb];
  uint16_t okT[kDim * kLp];                      // dO [i][v] (stride kLb), then k^T [kk][i] (stride kLp)
  uint16_t xh[kChunk * kLb], xl[kChunk * kLb];  // V', then F, then dV' [i][*]
  uint16_t m1h[kChunk * kLp], m1l[kChunk * kLp];
  uint16_t m2h[kChunk * kLp], m2l[kChunk * kLp];
  union {
    float tT[kChunk * kL64];  // T^T [j][i], until the dA products
    struct {
      float colg[4][kChunk];
      float rowg[2][kChunk], rowb[2][kChunk], dotq[2][kChunk], dotk[2][kChunk];
      float red[8];
    } r;
  } u;
  float b[kChunk], G[kChunk], rq[kChunk], rk[kChunk];
};

// T^T (fp32, stride kL64) from the prepare kernel's bf16 hi | lo rows with
// permuted columns; 16-byte loads (512 threads, one row piece each)
__device__ __forceinline__ void load_tT(float* sT, const uint16_t* tm, int tid) {
  const int r = tid & 63, p8 = (tid >> 6) * 8;
  const u16x8 th = *reinterpret_cast<const u16x8*>(tm + r * 128 + p8);
  const u16x8 tl = *reinterpret_cast<const u16x8*>(tm + r * 128 + 64 + p8);
#pragma unroll
  for (int e = 0; e < 8; ++e) sT[unperm_col(p8 + e) * kL64 + r] = bf2f(th[e]) + bf2f(tl[e]);
}

// 64 x 128 fp32 rows into LDS as a bf16 hi | lo pair (stride kLb), 512
// threads, loads issued together
__device__ __forceinline__ void load_split_rows(uint16_t* dh, uint16_t* dl, const float* src, int tid) {
  float4 v[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int idx = tid + 512 * m, r = idx >> 5, cc = (idx & 31) * 4;
    v[m] = *reinterpret_cast<const float4*>(src + r * kDim + cc);
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int idx = tid + 512 * m, r = idx >> 5, cc = (idx & 31) * 4;
    put_split4(dh, dl, r * kLb + cc, f32x4{v[m].x, v[m].y, v[m].z, v[m].w});
  }
}

// a C tile (rows r0 + 4g + e, column c) into a row-major hi | lo pair
__device__ __forceinline__ void put_split_rows(uint16_t* dh, uint16_t* dl, int off, int ld, const f32x4& v) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint16_t hi, lo;
    split_bf(v[e], hi, lo);
    dh[off + e * ld] = hi;
    dl[off + e * ld] = lo;
  }
}

// 16x16 tiles on v_mfma_f32_16x16x32_bf16, contraction kd (a multiple of 32)
// contiguous in both operands: row r of A at a + r * SA, column c of B at
// b + c * SB. x = exact bf16 operand, p = hi | lo pair.
template <int SA, int SB>
__device__ __forceinline__ f32x4 bmm_xx(const uint16_t* a, const uint16_t* b, int r0, int c0, int kd, int lane,
                                        f32x4 acc) {
  const int l = lane & 15, g = lane >> 4;
  const uint16_t* ap = a + (r0 + l) * SA + 8 * g;
  const uint16_t* bp = b + (c0 + l) * SB + 8 * g;
  for (int k0 = 0; k0 < kd; k0 += 32) acc = mfma16(ld8(ap + k0), ld8(bp + k0), acc);
  return acc;
}
template <int SA, int SB>
__device__ __forceinline__ f32x4 bmm_px(const uint16_t* ah, const uint16_t* al, const uint16_t* b, int r0, int c0,
                                        int kd, int lane, f32x4 acc) {
  const int l = lane & 15, g = lane >> 4;
  const int ao = (r0 + l) * SA + 8 * g;
  const uint16_t* bp = b + (c0 + l) * SB + 8 * g;
  for (int k0 = 0; k0 < kd; k0 += 32) {
    const u16x8 bv = ld8(bp + k0);
    acc = mfma16(ld8(ah + ao + k0), bv, acc);
    acc = mfma16(ld8(al + ao + k0), bv, acc);
  }
  return acc;
}
template <int SA, int SB>
__device__ __forceinline__ f32x4 bmm_xp(const uint16_t* a, const uint16_t* bh, const uint16_t* bl, int r0, int c0,
                                        int kd, int lane, f32x4 acc) {
  const int l = lane & 15, g = lane >> 4;
  const uint16_t* ap = a + (r0 + l) * SA + 8 * g;
  const int bo = (c0 + l) * SB + 8 * g;
  for (int k0 = 0; k0 < kd; k0 += 32) {
    const u16x8 av = ld8(ap + k0);
    acc = mfma16(av, ld8(bh + bo + k0), acc);
    acc = mfma16(av, ld8(bl + bo + k0), acc);
  }
  return acc;
}

__global__ __launch_bounds__(512, 1) void gdn_bwd_intra_kernel(BwdArgs a) {
  __shared__ InSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l = lane & 15, g = lane >> 4;
  const int rt = w & 3, hf = w >> 2;  // row tile, column half
  const int NT = a.geo.NT;
  // heads fastest in dispatch order: neighbouring workgroups read the
  // neighbouring head rows of the same tokens
  const int c = (int)(blockIdx.x / a.H), h = (int)(blockIdx.x % a.H);
  const size_t cm = (size_t)h * NT + c;
  const ChunkInfo ci = a.geo.chunk(c);
  const int L = ci.len;
  const int H = a.H;
  const float scale = a.scale;
  const size_t plane = (size_t)a.H * NT * kChunk * kDim;
  const float* vec = a.vec + cm * kVecStride;
  uint16_t* const sdO = sm.okT;  // dO, stride kLb
  uint16_t* const skT = sm.okT;  // k^T, stride kLp (after the o-term products)

#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int idx = tid + 512 * m, r = idx >> 4, cc = (idx & 15) * 8;
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
    *reinterpret_cast<uint4*>(sdO + r * kLb + cc) = ov;
  }
  load_tT(sm.u.tT, a.tmat + cm * (kChunk * 128), tid);
  load_split_rows(sm.xh, sm.xl, a.vnew + cm * (kChunk * kDim), tid);  // V'
  if (tid < kChunk) {
    const bool ok = tid < L;
    sm.b[tid] = ok ? vec[0 * kChunk + tid] : 0.0f;
    sm.G[tid] = ok ? vec[4 * kChunk + tid] : 0.0f;
    sm.rq[tid] = ok ? vec[5 * kChunk + tid] : 0.0f;
    sm.rk[tid] = ok ? vec[6 * kChunk + tid] : 0.0f;
  }
  __syncthreads();

  // this lane's rows i = 16 rt + 4g + e
  const int r0 = 16 * rt;
  float rb_[4], rG[4], rq_[4], rk_[4], eG[4], er[4];
  bool okr[4];
  const float GL = sm.G[L - 1];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = r0 + 4 * g + e;
    okr[e] = i < L;
    rb_[e] = sm.b[i];
    rG[e] = sm.G[i];
    rq_[e] = sm.rq[i];
    rk_[e] = sm.rk[i];
    eG[e] = okr[e] ? __expf(rG[e]) : 0.0f;
    er[e] = okr[e] ? __expf(GL - rG[e]) : 0.0f;
  }
  float accG[4] = {0.f, 0.f, 0.f, 0.f}, accB[4] = {0.f, 0.f, 0.f, 0.f};
  float colG[2] = {0.f, 0.f};

  // ---- dO V'^T and Qn Kn^T on the lower tiles: the o-term gradients -----
#pragma unroll
  for (int jt = 0; jt < 2; ++jt) {
    const int ct = 2 * hf + jt;
    f32x4 m1v = zero4(), m2v = zero4();
    if (ct <= rt) {
      const f32x4 p1 = bmm_xp<kLb, kLb>(sdO, sm.xh, sm.xl, r0, 16 * ct, kDim, lane, zero4());
      const f32x4 mq = bmm_xx<kLb, kLb>(sm.q, sm.k, r0, 16 * ct, kDim, lane, zero4());
      const int j = 16 * ct + l;
      const float Gj = sm.G[j], rkj = sm.rk[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = r0 + 4 * g + e;
        if (j <= i && okr[e]) {
          const float sp = scale * p1[e] * __expf(rG[e] - Gj);
          const float z = sp * rq_[e] * rkj * mq[e];
          accG[e] += z;
          colG[jt] -= z;
          m1v[e] = sp * rkj;
          m2v[e] = sp * rq_[e];
        }
      }
    }
    put_split_rows(sm.m1h, sm.m1l, (r0 + 4 * g) * kLp + 16 * ct + l, kLp, m1v);  // M1a [i][j]
    put_split4(sm.m2h, sm.m2l, (16 * ct + l) * kLp + r0 + 4 * g, m2v);            // M1b^T [j][i]
  }
  __syncthreads();
  load_split_rows(sm.xh, sm.xl, a.efd + plane + cm * (kChunk * kDim), tid);  // F
  {
    // k^T into dO's place: rows 4j .. 4j+3 at columns 8c .. 8c+7 per thread
    const int rr = 4 * (tid & 15), cc = 8 * ((tid >> 4) & 15);
    if (tid < 256) {
      u16x8 kv[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) kv[m] = ld8(sm.k + (rr + m) * kLb + cc);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<u16x4*>(skT + (cc + e) * kLp + rr) = u16x4{kv[0][e], kv[1][e], kv[2][e], kv[3][e]};
    }
  }
  __syncthreads();

  // columns of this wave's 64 x 128 tiles: 16 (4 hf + j) + l
  f32x4 dq[4], dk[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ct = 4 * hf + j;
    dq[j] = bmm_px<kLp, kLp>(sm.m1h, sm.m1l, skT, r0, 16 * ct, kChunk, lane, zero4());
    dk[j] = tile_mm<kLp, 1, kLb, 1>(HL{sm.m2h, sm.m2l}, sm.q, r0, 16 * ct, kChunk, lane, zero4());
  }

  // ---- F: dX = -T^T F, and -F X^T into dT -------------------------------
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ct = 4 * hf + j;
    const f32x4 t = tile_mm<kL64, 1, kLb, 1>(sm.u.tT, HL{sm.xh, sm.xl}, r0, 16 * ct, kChunk, lane, zero4());
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = r0 + 4 * g + e;
      const float kv = bf2f(sm.k[i * kLb + 16 * ct + l]);
      dk[j][e] -= rb_[e] * eG[e] * t[e];
      const float tk = -rk_[e] * eG[e] * t[e] * kv;  // e^G dX_i . kn_i, one column
      accB[e] += tk;
      accG[e] += rb_[e] * tk;
    }
  }
  f32x4 dT[2];
#pragma unroll
  for (int jt = 0; jt < 2; ++jt) {
    const int ct = 2 * hf + jt;
    const f32x4 t = bmm_px<kLb, kLb>(sm.xh, sm.xl, sm.k, r0, 16 * ct, kDim, lane, zero4());
    const int j = 16 * ct + l;
    const float xs = j < L ? sm.b[j] * sm.rk[j] * __expf(sm.G[j]) : 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) dT[jt][e] = -t[e] * xs;
  }
  __syncthreads();
  load_split_rows(sm.xh, sm.xl, a.dvn + cm * (kChunk * kDim), tid);  // dV'
  __syncthreads();

  // ---- dV': dY = T^T dV', dv = b dY, and dV' Y^T into dT -----------------
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ct = 4 * hf + j;
    const f32x4 t = tile_mm<kL64, 1, kLb, 1>(sm.u.tT, HL{sm.xh, sm.xl}, r0, 16 * ct, kChunk, lane, zero4());
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = r0 + 4 * g + e, col = 16 * ct + l;
      accB[e] += t[e] * bf2f(sm.v[i * kLb + col]);
      if (okr[e]) a.dv[((size_t)(ci.tok0 + i) * H + h) * kDim + col] = rb_[e] * t[e];
    }
  }
#pragma unroll
  for (int jt = 0; jt < 2; ++jt) {
    const int ct = 2 * hf + jt;
    const f32x4 t = bmm_px<kLb, kLb>(sm.xh, sm.xl, sm.v, r0, 16 * ct, kDim, lane, zero4());
    const float bj = sm.b[16 * ct + l];
#pragma unroll
    for (int e = 0; e < 4; ++e) dT[jt][e] += t[e] * bj;
    put_split4(sm.m1h, sm.m1l, (16 * ct + l) * kLp + r0 + 4 * g, dT[jt]);  // dT^T [j][m]
  }
  __syncthreads();

  // ---- dA = strictLower(T^T dT T^T) ---------------------------------------
#pragma unroll
  for (int jt = 0; jt < 2; ++jt) {
    const int ct = 2 * hf + jt;
    const f32x4 q1 = tile_mm<kL64, 1, 1, kLp>(sm.u.tT, HL{sm.m1h, sm.m1l}, r0, 16 * ct, kChunk, lane, zero4());
    put_split_rows(sm.m2h, sm.m2l, (r0 + 4 * g) * kLp + 16 * ct + l, kLp, q1);  // Q1 [i][m]
  }
  __syncthreads();
  f32x4 pa[2], pb[2];
#pragma unroll
  for (int jt = 0; jt < 2; ++jt) {
    const int ct = 2 * hf + jt;
    pa[jt] = zero4();
    pb[jt] = zero4();
    if (ct <= rt) {
      const f32x4 dA = tile_mm<kLp, 1, kL64, 1>(HL{sm.m2h, sm.m2l}, sm.u.tT, r0, 16 * ct, kChunk, lane, zero4());
      const f32x4 mk = bmm_xx<kLb, kLb>(sm.k, sm.k, r0, 16 * ct, kDim, lane, zero4());
      const int j = 16 * ct + l;
      const float Gj = sm.G[j], rkj = sm.rk[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = r0 + 4 * g + e;
        if (j < i && okr[e]) {
          const float gam = __expf(rG[e] - Gj);
          const float mkk = rk_[e] * rkj * mk[e];
          const float Aij = -rb_[e] * mkk * gam;
          const float z = dA[e] * Aij;
          accG[e] += z;
          colG[jt] -= z;
          const float P = dA[e] * gam;
          accB[e] -= P * mkk;
          pa[jt][e] = -rb_[e] * P * rkj;
          pb[jt][e] = -P * rb_[e] * rk_[e];
        }
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int jt = 0; jt < 2; ++jt) {
    const int ct = 2 * hf + jt;
    put_split_rows(sm.m1h, sm.m1l, (r0 + 4 * g) * kLp + 16 * ct + l, kLp, pa[jt]);  // Pa [i][j]
    put_split4(sm.m2h, sm.m2l, (16 * ct + l) * kLp + r0 + 4 * g, pb[jt]);           // Pb^T [j][i]
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ct = 4 * hf + j;
    dk[j] = bmm_px<kLp, kLp>(sm.m1h, sm.m1l, skT, r0, 16 * ct, kChunk, lane, dk[j]);
    dk[j] = bmm_px<kLp, kLp>(sm.m2h, sm.m2l, skT, r0, 16 * ct, kChunk, lane, dk[j]);
  }

  // ---- E = dO S^T and D = V' dS_next^T -----------------------------------
  const float* E = a.efd + cm * (kChunk * kDim);
  const float* D = E + 2 * plane;
  // (all 64 rows of E and D exist, zero past the end: the loads need no guard
  // and are issued together)
  float cl = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ct = 4 * hf + j;
    float Ev[4], Dv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = r0 + 4 * g + e, col = 16 * ct + l;
      Ev[e] = E[i * kDim + col];
      Dv[e] = D[i * kDim + col];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = r0 + 4 * g + e, col = 16 * ct + l;
      const float sE = okr[e] ? scale * eG[e] : 0.0f;   // eG, er are 0 past the end
      dq[j][e] += sE * Ev[e];
      accG[e] += sE * rq_[e] * Ev[e] * bf2f(sm.q[i * kLb + col]);
      dk[j][e] += er[e] * Dv[e];
      const float cc = er[e] * rk_[e] * Dv[e] * bf2f(sm.k[i * kLb + col]);
      accG[e] -= cc;
      cl += cc;
    }
  }

  // ---- row dots of the L2-norm backward, combined over the two halves -----
  // (T^T is dead since the dA products: its LDS holds the reduction arrays)
  float sq[4] = {0.f, 0.f, 0.f, 0.f}, sk[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = r0 + 4 * g + e, col = 16 * (4 * hf + j) + l;
      sq[e] += bf2f(sm.q[i * kLb + col]) * dq[j][e];
      sk[e] += bf2f(sm.k[i * kLb + col]) * dk[j][e];
    }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    sq[e] = sum16(sq[e]);
    sk[e] = sum16(sk[e]);
    accG[e] = sum16(accG[e]);
    accB[e] = sum16(accB[e]);
  }
  if (l == 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = r0 + 4 * g + e;
      sm.u.r.dotq[hf][i] = sq[e];
      sm.u.r.dotk[hf][i] = sk[e];
      sm.u.r.rowg[hf][i] = accG[e];
      sm.u.r.rowb[hf][i] = accB[e];
    }
  }
#pragma unroll
  for (int jt = 0; jt < 2; ++jt) {
    float x = colG[jt];
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    if (g == 0) sm.u.r.colg[rt][16 * (2 * hf + jt) + l] = x;
  }
  cl += __shfl_xor(cl, 16);
  cl += __shfl_xor(cl, 32);
  cl = sum16(cl);
  if (lane == 0) sm.u.r.red[w] = cl;
  __syncthreads();

  // ---- L2-norm backward, outputs dq, dk ------------------------------------
  const bool l2 = (a.flags & 1u) != 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = r0 + 4 * g + e;
    sq[e] = sm.u.r.dotq[0][i] + sm.u.r.dotq[1][i];
    sk[e] = sm.u.r.dotk[0][i] + sm.u.r.dotk[1][i];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = r0 + 4 * g + e, col = 16 * (4 * hf + j) + l;
      if (!okr[e]) continue;
      float gq = dq[j][e], gk = dk[j][e];
      if (l2) {
        // d x = r (d xn - xn (xn . d xn)), xn = r x
        gq = rq_[e] * (gq - rq_[e] * rq_[e] * bf2f(sm.q[i * kLb + col]) * sq[e]);
        gk = rk_[e] * (gk - rk_[e] * rk_[e] * bf2f(sm.k[i * kLb + col]) * sk[e]);
      }
      const size_t off = ((size_t)(ci.tok0 + i) * H + h) * kDim + col;
      a.dq[off] = gq;
      a.dk[off] = gk;
    }

  // ---- d beta and dG, then dg ----------------------------------------------
  if (w == 0) {
    // lane r holds chunk row 63 - r, so the inclusive scan over lanes is the
    // reverse cumulative sum over rows
    const int i = 63 - lane;
    float dG = 0.0f;
    if (i < L) {
      dG = (sm.u.r.rowg[0][i] + sm.u.r.rowg[1][i]) +
           ((sm.u.r.colg[0][i] + sm.u.r.colg[1][i]) + (sm.u.r.colg[2][i] + sm.u.r.colg[3][i]));
      if (i == L - 1) {
        const float eL = vec[7 * kChunk];
        float cls = 0.0f;
#pragma unroll
        for (int ww = 0; ww < 8; ++ww) cls += sm.u.r.red[ww];
        dG += eL * a.sdot[cm] + cls;
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
      const float db = sm.u.r.rowb[0][i] + sm.u.r.rowb[1][i];
      a.dbeta[tok] = (a.flags & 2u) ? db * bi * (1.0f - bi) : db;
    }
  }
}

}  // namespace

hipError_t launch_gdn_bwd(const BwdArgs& a, int stage, hipStream_t stream) {
  const unsigned cms = (unsigned)((size_t)a.H * a.geo.NT);
  if (stage == 0) {
    // 32-column value blocks, or 16-column ones when that is still less than
    // one workgroup per compute unit of the device
    if ((long)a.geo.N * a.H * 8 <= a.cus)
      hipLaunchKernelGGL(gdn_bwd_dh_kernel<1>, dim3(state_grid(a.geo.N, a.H, 8)), dim3(512), 0, stream, a);
    else
      hipLaunchKernelGGL(gdn_bwd_dh_kernel<2>, dim3(state_grid(a.geo.N, a.H, 4)), dim3(512), 0, stream, a);
  }
  else if (stage == 1)
    hipLaunchKernelGGL(gdn_bwd_sprod_kernel, dim3(cms), dim3(512), 0, stream, a);
  else
    hipLaunchKernelGGL(gdn_bwd_intra_kernel, dim3(cms), dim3(512), 0, stream, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Backward of the in-kernel gate. Block (b, h) takes tokens
// b*kGateBwdTok .. +kGateBwdTok of head h, thread t the tokens t + 256 j,
// all eight loads of a thread issued before use. The sums are reduced in a
// fixed order (per thread in j, across the wave by xor shuffles, across the
// four waves in wave order), so results are bitwise reproducible.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum_fixed(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

__global__ __launch_bounds__(256) void gate_bwd_partial_kernel(GateBwdArgs a) {
  constexpr float kLog2e = 1.4426950408889634f;
  constexpr float kLn2 = 0.6931471805599453f;
  const int h = blockIdx.y, tid = threadIdx.x;
  const long t0 = (long)blockIdx.x * kGateBwdTok;
  const float ea = expf(a.a_log[h]), db = a.dt_bias[h];
  float xv[8], dv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const long t = t0 + tid + 256 * j;
    const bool in = t < a.ntok;
    xv[j] = in ? a.x[t * a.H + h] : 0.f;
    dv[j] = in ? a.dg[t * a.H + h] : 0.f;
  }
  float sa = 0.f, sb = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const long t = t0 + tid + 256 * j;
    const float y = xv[j] + db;
    const float g = -ea * kLn2 * softplus_log2(y);
    const float sig = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-y * kLog2e));
    const float dx = -ea * sig * dv[j];
    if (t < a.ntok) {
      a.dg[t * a.H + h] = dx;
      sa += dv[j] * g;
      sb += dx;
    }
  }
  __shared__ float red[2][4];
  sa = wave_sum_fixed(sa);
  sb = wave_sum_fixed(sb);
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = sa;
    red[1][tid >> 6] = sb;
  }
  __syncthreads();
  if (tid == 0) {
    a.part[(size_t)h * a.nblk + blockIdx.x] = ((red[0][0] + red[0][1]) + red[0][2]) + red[0][3];
    a.part[((size_t)a.H + h) * a.nblk + blockIdx.x] = ((red[1][0] + red[1][1]) + red[1][2]) + red[1][3];
  }
}

__global__ __launch_bounds__(64) void gate_bwd_final_kernel(GateBwdArgs a) {
  const int h = blockIdx.x, lane = threadIdx.x;
  float sa = 0.f, sb = 0.f;
  for (int b = lane; b < a.nblk; b += 64) {
    sa += a.part[(size_t)h * a.nblk + b];
    sb += a.part[((size_t)a.H + h) * a.nblk + b];
  }
  sa = wave_sum_fixed(sa);
  sb = wave_sum_fixed(sb);
  if (lane == 0) {
    a.da_log[h] = sa;
    a.ddt_bias[h] = sb;
  }
}

hipError_t launch_gate_bwd(const GateBwdArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(gate_bwd_partial_kernel, dim3(a.nblk, a.H), dim3(256), 0, stream, a);
  hipLaunchKernelGGL(gate_bwd_final_kernel, dim3(a.H), dim3(64), 0, stream, a);
  return hipGetLastError();
}

// KDA gate backward, per key channel. Partial sums per block of
// kKdaGateTok tokens and head: thread (channel d = tid % 128, token parity
// tid / 128) walks its tokens in order; dA_log's partial is reduced over the
// block in a fixed order (xor shuffles, then the four waves in order),
// dt_bias's per channel as (even tokens) + (odd tokens). The final kernel
// sums the blocks in order, so results are bitwise reproducible.
__global__ __launch_bounds__(256) void kda_gate_bwd_partial_kernel(KdaGateBwdArgs a) {
  constexpr float kLog2e = 1.4426950408889634f;
  const int h = blockIdx.y, tid = threadIdx.x, d = tid & 127, par = tid >> 7;
  const long t0 = (long)blockIdx.x * kKdaGateTok;
  const float ea = expf(a.a_log[h]), db = a.dt_bias[(size_t)h * kDim + d];
  const float c = -ea * kLog2e;
  float sa = 0.f, sb = 0.f;
  for (int j = 0; j < kKdaGateTok / 2; ++j) {
    const long t = t0 + par + 2 * j;
    if (t >= a.ntok) break;
    const size_t idx = ((size_t)t * a.H + h) * kDim + d;
    const float y = a.x[idx] + db;
    const float dgv = a.dg[idx];
    const float g = -ea * softplus_log2(y);
    const float sig = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-y * kLog2e));
    const float dx = dgv * c * sig;
    a.dg[idx] = dx;
    sa = fmaf(dgv, g, sa);
    sb += dx;
  }
  __shared__ float red[4];
  __shared__ float odd[kDim];
  sa = wave_sum_fixed(sa);
  if ((tid & 63) == 0) red[tid >> 6] = sa;
  if (par == 1) odd[d] = sb;
  __syncthreads();
  if (par == 0) a.part[(size_t)a.H * a.nblk + ((size_t)h * kDim + d) * a.nblk + blockIdx.x] = sb + odd[d];
  if (tid == 0) a.part[(size_t)h * a.nblk + blockIdx.x] = ((red[0] + red[1]) + red[2]) + red[3];
}

__global__ __launch_bounds__(128) void kda_gate_bwd_final_kernel(KdaGateBwdArgs a) {
  const int h = blockIdx.x, d = threadIdx.x;
  const float* pb = a.part + (size_t)a.H * a.nblk + ((size_t)h * kDim + d) * a.nblk;
  float sb = 0.f;
  for (int b = 0; b < a.nblk; ++b) sb += pb[b];
  a.ddt_bias[(size_t)h * kDim + d] = sb;
  if (d < 64) {
    float sa = 0.f;
    for (int b = d; b < a.nblk; b += 64) sa += a.part[(size_t)h * a.nblk + b];
    sa = wave_sum_fixed(sa);
    if (d == 0) a.da_log[h] = sa;
  }
}

hipError_t launch_kda_gate_bwd(const KdaGateBwdArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(kda_gate_bwd_partial_kernel, dim3(a.nblk, a.H), dim3(256), 0, stream, a);
  hipLaunchKernelGGL(kda_gate_bwd_final_kernel, dim3(a.H), dim3(128), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gdn
