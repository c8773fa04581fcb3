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
  float* gk;       // [H,NT,64,128], KDA only
  Geometry geo;
  int H;
  float scale;
  uint32_t flags;
  int cus;         // compute units of the device (grid size of persistent launches)
};

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* tmat;  // [H,NT,64,128] bf16 hi | lo, permuted columns
  const uint16_t* aqk;   // [H,NT,64,64] bf16, permuted columns
  const float* vec;
  const float* gk;       // KDA only
  const float* s0;       // [N,H,K,V] or nullptr
  float* sfinal;         // [N,H,K,V] or nullptr
  uint16_t* o;           // [B*T,H,V]
  float* h_out;          // [H,NT,K,V]   (stage mode)
  float* vnew_out;       // [H,NT,64,V]  (stage mode)
  Geometry geo;
  int H;
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

}  // namespace gdn
