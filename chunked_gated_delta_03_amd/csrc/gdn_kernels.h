// Kernel argument blocks and launchers of the gfx950 kernels (host + device).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_common.h"

namespace gdn {

struct PrepareArgs {
  const uint16_t* q;
  const uint16_t* k;
  const float* g;
  const uint16_t* beta;
  uint16_t* tmat;  // [H,NT,64,128] bf16 hi | lo, permuted columns
  uint16_t* aqk;   // [H,NT,64,64] bf16, permuted columns
  float* vec;      // [H,NT,8,64]
  float* gk;       // [H,NT,64,128], KDA stage entry only
  uint16_t* kdec;  // [H,NT] blocks of kKdecElems, KDA whole pass only (see kda_kdec_*)
  // In-kernel gate: when a_log != nullptr, g holds the raw gate values x and
  // the gate is -exp(a_log[h]) softplus(x + dt_bias) (dt_bias [H] GDN,
  // [H,K] KDA), natural log for GDN, log2 for KDA.
  const float* a_log;
  const float* dt_bias;
  Geometry geo;
  int H;
  float scale;
  uint32_t flags;
  int cus;         // compute units of the device (grid size of persistent launches)
};

// KDA whole pass: the decayed operands of one (chunk, head), written by the
// prepare kernel and copied by the state kernel's loaders. bf16 arrays of
// 64 x 128 in natural column order, then 2^G_last per channel (fp32).
constexpr int kKdecKdh = 0;                       // k 2^G, hi
constexpr int kKdecKdl = 1 * kChunk * kDim;       // k 2^G, lo
constexpr int kKdecKgh = 2 * kChunk * kDim;       // k 2^(G_last - G), hi
constexpr int kKdecKgl = 3 * kChunk * kDim;       // k 2^(G_last - G), lo
constexpr int kKdecQd = 4 * kChunk * kDim;        // q 2^G
constexpr int kKdecDec = 5 * kChunk * kDim;       // 2^G_last, 128 fp32 (256 uint16 slots)
constexpr int kKdecElems = 5 * kChunk * kDim + 2 * kDim;

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* tmat;  // [H,NT,64,128] bf16 hi | lo, permuted columns
  const uint16_t* aqk;   // [H,NT,64,64] bf16, permuted columns
  const float* vec;
  const float* gk;       // KDA stage entry only
  const uint16_t* kdec;  // KDA whole pass only
  const float* s0;       // [N,H,K,V] or nullptr
  float* sfinal;         // [N,H,K,V] or nullptr
  uint16_t* o;           // [B*T,H,V]
  float* h_out;          // [H,NT,K,V]   (stage mode)
  float* vnew_out;       // [H,NT,64,V]  (stage mode)
  Geometry geo;
  int H;
  int s_identity;        // state summary transition: S0 = I and v taken as 0 (s0 ignored)
};

struct FinArgs {
  const uint16_t* q;
  const uint16_t* aqk;   // permuted columns
  const float* vec;
  const float* gk;       // KDA only
  const float* h;
  const float* vnew;
  uint16_t* o;
  Geometry geo;
  int H;
};

// All launchers enqueue on `stream` and return the launch status.
hipError_t launch_prepare(bool kda, const PrepareArgs& a, hipStream_t stream);
hipError_t launch_fwd(bool kda, bool store_h, bool compute_o, const FwdArgs& a, hipStream_t stream);
hipError_t launch_finalize(bool kda, const FinArgs& a, hipStream_t stream);
hipError_t launch_gdn_state(bool store_h, bool compute_o, const FwdArgs& a, hipStream_t stream);
hipError_t launch_kda_fwd(bool store_h, bool compute_o, const FwdArgs& a, hipStream_t stream);
hipError_t launch_kda_finalize(const FinArgs& a, hipStream_t stream);
// Causal depthwise Conv1d + SiLU over token-major rows of D channels.
struct ConvArgs {
  const uint16_t* x;     // [B*T, D] bf16
  const float* w;        // [D, W]
  const float* bias;     // [D] or nullptr
  const uint16_t* halo;  // [B or 1, (W-1)*dilation, D] bf16 or nullptr
  const int* cu;         // device offsets [N+1] (packed) or nullptr
  uint16_t* y;           // [B*T, D] bf16
  int B, T, D, W, dilation, N;
  int silu;
};
hipError_t launch_short_conv(const ConvArgs& a, hipStream_t stream);

hipError_t launch_summary_apply(const float* M, const float* S, const float* sin, float* sout, long units,
                                hipStream_t stream);

}  // namespace gdn
