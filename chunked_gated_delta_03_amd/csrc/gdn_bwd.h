// Argument block and launcher of the backward-pass kernels (host + device).
#pragma once

#include "gdn_kernels.h"

namespace gdn {

// Backward pass (GDN scalar gate): gradients of <dO, o> + <dS_final, S_final>.
struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;      // [B*T,H,V] bf16
  const uint16_t* tmat;      // prepare outputs, as FwdArgs
  const uint16_t* aqk;
  const float* vec;
  const float* h;            // [H,NT,K,V] state entering each chunk (forward stage)
  const float* vnew;         // [H,NT,64,V] U - W S (forward stage)
  const float* dsfinal;      // [N,H,K,V] or nullptr (zero)
  float* dhn;                // [H,NT,K,V] gradient w.r.t. the state leaving each chunk
  float* dvn;                // [H,NT,64,V] gradient w.r.t. v_new
  float* efd;                // [3][H,NT,64,K]: dO S^T, dv_new S^T, v_new dS_next^T
  float* sdot;               // [H,NT] <dS_next, S>
  float* ds0;                // [N,H,K,V] or nullptr
  float* dq;                 // [B*T,H,K] fp32
  float* dk;
  float* dv;
  float* dg;                 // [B*T,H] fp32
  float* dbeta;              // [B*T,H] fp32
  Geometry geo;
  int H;
  float scale;
  uint32_t flags;
  int cus;                   // compute units of the device (launch shape of the reverse pass)
};
// stage 0: reverse state pass, 1: state products, 2: per-chunk gradients
hipError_t launch_gdn_bwd(const BwdArgs& a, int stage, hipStream_t stream);

// Reverse state pass of the KDA backward (kda_bwd.hip).
struct KdaBwdArgs {
  const uint16_t* q;         // [B*T,H,K] bf16
  const uint16_t* k;
  const uint16_t* dout;      // [B*T,H,V] bf16
  const float* gk;           // [H,NT,64,K] cumulative log2 gate (prepare, stage mode)
  const float* vec;          // [H,NT,8,64] prepare row vectors
  const uint16_t* tmat;      // [H,NT,64,128] T, bf16 hi | lo, permuted columns
  const uint16_t* aqk;       // [H,NT,64,64] bf16, permuted columns
  const float* dsfinal;      // [N,H,K,V] or nullptr (zero)
  float* dhn;                // [H,NT,K,V] gradient w.r.t. the state leaving each chunk
  float* dvn;                // [H,NT,64,V] gradient w.r.t. v_new
  float* ds0;                // [N,H,K,V] or nullptr
  // per-chunk gradients (whole backward only)
  const uint16_t* v;         // [B*T,H,V] bf16
  const float* h;            // [H,NT,K,V] state entering each chunk
  const float* vnew;         // [H,NT,64,V] v_new
  const float* efd;          // [3][H,NT,64,K]: dO S^T, dV' S^T, V' dS_next^T
  float* dp;                 // [H,NT,64,64] workspace: dP
  float* da;                 // [H,NT,64,64] workspace: dA
  float* dkd;                // [H,NT,64,K] workspace: dKD
  float* db1;                // [H,NT,64] workspace: the T-term part of dbeta
  float* dq;                 // [B*T,H,K] fp32 outputs
  float* dk;
  float* dv;
  float* dg;                 // [B*T,H,K] w.r.t. the raw log2 gate
  float* dbeta;              // [B*T,H]
  float scale;
  uint32_t flags;
  Geometry geo;
  int H;
};
hipError_t launch_kda_bwd_dh(const KdaBwdArgs& a, hipStream_t stream);
// per-chunk gradients: the mats kernel, then the gram kernel
hipError_t launch_kda_bwd_chunks(const KdaBwdArgs& a, hipStream_t stream);

// Backward of the in-kernel gate g = -exp(A_log[h]) softplus(x + dt_bias[h])
// (GDN, natural log): dg (w.r.t. g) becomes dx = -exp(A_log) sigmoid(x +
// dt_bias) dg in place, and per head dA_log = sum dg g, ddt_bias = sum dx,
// summed in a fixed order (partial sums per block of kGateBwdTok tokens,
// then one pass over the blocks).
constexpr int kGateBwdTok = 2048;
struct GateBwdArgs {
  const float* x;        // [ntok,H] raw gate values
  const float* a_log;    // [H]
  const float* dt_bias;  // [H]
  float* dg;             // [ntok,H] in: w.r.t. g, out: w.r.t. x
  float* part;           // [2][H][nblk] workspace
  float* da_log;         // [H]
  float* ddt_bias;       // [H]
  long ntok;
  int H;
  int nblk;              // ceil(ntok / kGateBwdTok)
};
hipError_t launch_gate_bwd(const GateBwdArgs& a, hipStream_t stream);

// Backward of the KDA in-kernel gate, per key channel:
// g = -exp(A_log[h]) softplus(x + dt_bias[h,d]) / ln 2 (log2 units), so
// dx = dg (-exp(A_log) / ln 2) sigmoid(x + dt_bias), dA_log[h] = sum dg g
// over tokens and channels, ddt_bias[h,d] = sum of dx over tokens.
constexpr int kKdaGateTok = 256;  // tokens per block of the partial sums
struct KdaGateBwdArgs {
  const float* x;        // [ntok,H,128] raw gate values
  const float* a_log;    // [H]
  const float* dt_bias;  // [H,128]
  float* dg;             // [ntok,H,128] in: w.r.t. g, out: w.r.t. x
  float* part;           // [H][nblk] then [H][128][nblk] workspace
  float* da_log;         // [H]
  float* ddt_bias;       // [H,128]
  long ntok;
  int H;
  int nblk;              // ceil(ntok / kKdaGateTok)
};
hipError_t launch_kda_gate_bwd(const KdaGateBwdArgs& a, hipStream_t stream);

}  // namespace gdn
