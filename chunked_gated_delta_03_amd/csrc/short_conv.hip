// Causal depthwise Conv1d + SiLU (the ShortConv that forms q, k, v from the
// projections; _causal_conv1d_with_cp_halo on the hyper-parallel "Diff
// Coverage" page of the 2026-09-10 gate build): per channel c and token t,
//   y[t, c] = silu(bias[c] + sum_{j<W} w[c, j] x[t - (W-1-j) d, c]),
// rows before the start of the sequence taken from the halo (the preceding
// rows of a split sequence) or zero; packed documents are separate sequences,
// the halo preceding the first one only.
//
// HBM-bound: each thread owns 8 channels (one 16-byte piece of a token row)
// and walks a run of kRun consecutive tokens, so a wave's 64 lanes read and
// write 1 KiB of one row per step (fully coalesced); the taps of earlier rows
// are re-read from L1. All lanes of a wave see the same token, so the
// document-boundary and halo decisions are wave-uniform branches. Weights
// live in registers (W <= 8, a template parameter); accumulation in fp32,
// output bf16 round-to-nearest-even.
#include "gdn_kernels.h"

namespace gdn {

namespace {

constexpr int kRun = 32;  // tokens per thread

__device__ __forceinline__ void unpack8(const u16x8& v, float (&f)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = bf2f(v[e]);
}

// Sequence containing token t: [start, end) and whether it is the first one
// (the one the halo precedes). Dense: rows of T tokens; packed: binary search
// over the offsets (scalar loads: t is uniform).
struct SeqSpan {
  int start, end;
  bool first;
};
__device__ __forceinline__ SeqSpan seq_of(const ConvArgs& a, int t) {
  SeqSpan s;
  if (!a.cu) {
    const int b = t / a.T;
    s.start = b * a.T;
    s.end = s.start + a.T;
    s.first = true;  // every batch row has its own halo rows
    return s;
  }
  const __attribute__((address_space(4))) int* cu = (const __attribute__((address_space(4))) int*)a.cu;
  int lo = 0, hi = a.N;  // cu[lo] <= t < cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid;
    else hi = mid;
  }
  s.start = cu[lo];
  s.end = cu[lo + 1];
  s.first = lo == 0;
  return s;
}

template <int W>
__global__ __launch_bounds__(256) void short_conv_kernel(ConvArgs a) {
  const int cg = blockIdx.x * 256 + threadIdx.x;  // 8-channel group
  const int ngroups = a.D / 8;
  const int t0 = blockIdx.y * kRun;
  const int total = a.B * a.T;
  const bool active = cg < ngroups;
  const int c0 = 8 * (active ? cg : 0);
  const int dil = a.dilation;

  float w[W][8], bias[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
#pragma unroll
    for (int j = 0; j < W; ++j) w[j][e] = a.w[(size_t)(c0 + e) * W + j];
    bias[e] = a.bias ? a.bias[c0 + e] : 0.0f;
  }

  SeqSpan sp = seq_of(a, t0 < total ? t0 : total - 1);
  const int hw = (W - 1) * dil;
  for (int i = 0; i < kRun; ++i) {
    const int t = t0 + i;
    if (t >= total) break;
    if (t >= sp.end) sp = seq_of(a, t);
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = bias[e];
#pragma unroll
    for (int j = 0; j < W; ++j) {
      const int tt = t - (W - 1 - j) * dil;
      u16x8 xv = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
      if (tt >= sp.start) {
        xv = *reinterpret_cast<const u16x8*>(a.x + (size_t)tt * a.D + c0);
      } else if (a.halo && sp.first) {
        // halo row (hw - (sp.start - tt)) of this sequence's halo block
        const int hb = a.cu ? 0 : t / a.T;
        xv = *reinterpret_cast<const u16x8*>(a.halo + ((size_t)hb * hw + hw - (sp.start - tt)) * a.D + c0);
      }
      float xf[8];
      unpack8(xv, xf);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(w[j][e], xf[e], acc[e]);
    }
    if (a.silu) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = acc[e] / (1.0f + __expf(-acc[e]));
    }
    u32x4 out;
#pragma unroll
    for (int p = 0; p < 4; ++p) out[p] = pack2(acc[2 * p], acc[2 * p + 1]);
    if (active) *reinterpret_cast<u32x4*>(a.y + (size_t)t * a.D + c0) = out;
  }
}

// Dilation 1: rows are loaded eight at a time (eight 16-byte loads in
// flight per thread) and the W-1 rows before them are kept in registers, so
// every input row is read once. A group that a sequence boundary crosses (or
// that reaches past the end) goes through the per-token code above.
template <int W>
__global__ __launch_bounds__(256) void short_conv_d1_kernel(ConvArgs a) {
  constexpr int G = 8;
  constexpr int HW = W - 1;
  const int cg = blockIdx.x * 256 + threadIdx.x;
  const int ngroups = a.D / 8;
  const int t0 = blockIdx.y * kRun;
  const int total = a.B * a.T;
  const bool active = cg < ngroups;
  const int c0 = 8 * (active ? cg : 0);

  float w[W][8], bias[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
#pragma unroll
    for (int j = 0; j < W; ++j) w[j][e] = a.w[(size_t)(c0 + e) * W + j];
    bias[e] = a.bias ? a.bias[c0 + e] : 0.0f;
  }
  auto row_before = [&](const SeqSpan& sp, int t, int tt, float (&f)[8]) {  // tap row tt of token t
    u16x8 xv = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
    if (tt >= sp.start) {
      xv = *reinterpret_cast<const u16x8*>(a.x + (size_t)tt * a.D + c0);
    } else if (a.halo && sp.first) {
      const int hb = a.cu ? 0 : t / a.T;
      xv = *reinterpret_cast<const u16x8*>(a.halo + ((size_t)hb * HW + HW - (sp.start - tt)) * a.D + c0);
    }
    unpack8(xv, f);
  };
  auto finish = [&](float (&acc)[8], int t) {
    if (a.silu) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = acc[e] / (1.0f + __expf(-acc[e]));
    }
    u32x4 out;
#pragma unroll
    for (int p = 0; p < 4; ++p) out[p] = pack2(acc[2 * p], acc[2 * p + 1]);
    if (active) *reinterpret_cast<u32x4*>(a.y + (size_t)t * a.D + c0) = out;
  };

  SeqSpan sp = seq_of(a, t0);
  float hist[HW > 0 ? HW : 1][8];  // rows t-HW .. t-1 before the group
#pragma unroll
  for (int m = 0; m < HW; ++m) row_before(sp, t0, t0 - HW + m, hist[m]);
  for (int g = 0; g < kRun / G; ++g) {
    const int tg = t0 + G * g;
    if (tg >= total) break;
    if (tg + G <= total && tg + G <= sp.end) {
      // fast group: all G tokens in the current sequence
      u16x8 rv[G];
#pragma unroll
      for (int i = 0; i < G; ++i) rv[i] = *reinterpret_cast<const u16x8*>(a.x + (size_t)(tg + i) * a.D + c0);
      float rows[G][8];
#pragma unroll
      for (int i = 0; i < G; ++i) unpack8(rv[i], rows[i]);
#pragma unroll
      for (int i = 0; i < G; ++i) {
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = bias[e];
#pragma unroll
        for (int j = 0; j < W; ++j) {
          const int m = i - (W - 1 - j);  // row index relative to the group
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = fmaf(w[j][e], m >= 0 ? rows[m][e] : hist[HW + m][e], acc[e]);
        }
        finish(acc, tg + i);
      }
#pragma unroll
      for (int m = 0; m < HW; ++m) {
        const int src = G - HW + m;  // >= 0 since HW <= 7 < G
#pragma unroll
        for (int e = 0; e < 8; ++e) hist[m][e] = rows[src][e];
      }
    } else {
      // per token: a boundary or the end inside the group
      for (int i = 0; i < G; ++i) {
        const int t = tg + i;
        if (t >= total) break;
        if (t >= sp.end) sp = seq_of(a, t);
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = bias[e];
#pragma unroll
        for (int j = 0; j < W; ++j) {
          float f[8];
          row_before(sp, t, t - (W - 1 - j), f);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = fmaf(w[j][e], f[e], acc[e]);
        }
        finish(acc, t);
      }
      // history for the next group, from its first token's sequence
      const int tn = tg + G;
      if (tn < total) {
        if (tn >= sp.end) sp = seq_of(a, tn);
#pragma unroll
        for (int m = 0; m < HW; ++m) row_before(sp, tn, tn - HW + m, hist[m]);
      }
    }
  }
}

}  // namespace

hipError_t launch_short_conv(const ConvArgs& a, hipStream_t stream) {
  const int ngroups = a.D / 8;
  const dim3 grid((ngroups + 255) / 256, (a.B * a.T + kRun - 1) / kRun);
  if (a.dilation == 1) {
    switch (a.W) {
      case 1: hipLaunchKernelGGL(short_conv_d1_kernel<1>, grid, dim3(256), 0, stream, a); break;
      case 2: hipLaunchKernelGGL(short_conv_d1_kernel<2>, grid, dim3(256), 0, stream, a); break;
      case 3: hipLaunchKernelGGL(short_conv_d1_kernel<3>, grid, dim3(256), 0, stream, a); break;
      case 4: hipLaunchKernelGGL(short_conv_d1_kernel<4>, grid, dim3(256), 0, stream, a); break;
      case 5: hipLaunchKernelGGL(short_conv_d1_kernel<5>, grid, dim3(256), 0, stream, a); break;
      case 6: hipLaunchKernelGGL(short_conv_d1_kernel<6>, grid, dim3(256), 0, stream, a); break;
      case 7: hipLaunchKernelGGL(short_conv_d1_kernel<7>, grid, dim3(256), 0, stream, a); break;
      case 8: hipLaunchKernelGGL(short_conv_d1_kernel<8>, grid, dim3(256), 0, stream, a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch (a.W) {
    case 1: hipLaunchKernelGGL(short_conv_kernel<1>, grid, dim3(256), 0, stream, a); break;
    case 2: hipLaunchKernelGGL(short_conv_kernel<2>, grid, dim3(256), 0, stream, a); break;
    case 3: hipLaunchKernelGGL(short_conv_kernel<3>, grid, dim3(256), 0, stream, a); break;
    case 4: hipLaunchKernelGGL(short_conv_kernel<4>, grid, dim3(256), 0, stream, a); break;
    case 5: hipLaunchKernelGGL(short_conv_kernel<5>, grid, dim3(256), 0, stream, a); break;
    case 6: hipLaunchKernelGGL(short_conv_kernel<6>, grid, dim3(256), 0, stream, a); break;
    case 7: hipLaunchKernelGGL(short_conv_kernel<7>, grid, dim3(256), 0, stream, a); break;
    case 8: hipLaunchKernelGGL(short_conv_kernel<8>, grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gdn
