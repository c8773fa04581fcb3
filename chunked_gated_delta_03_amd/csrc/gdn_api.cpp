// Host side of the C ABI declared in include/gdn.h: argument validation,
// chunk tables for packed input, workspace layout and kernel launches.
//
// Contract checks follow the pages' adapters (hyper-parallel "Diff Coverage"
// page of 2026-11-06: _packed_offsets and the Ascend C GDN entry; coverage
// page of kimi_delta_attention_ascendc.py: _packed_offsets, _packed_metadata,
// ascendc_chunk_kda): offsets strictly increasing from 0 to T, packed input
// only with B = 1, chunk size 64, head dimension 128.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/gdn.h"
#include "gdn_bwd.h"
#include "gdn_kernels.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(GDN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ---------------------------------------------------------------------------
// Problem description after validation.
struct Problem {
  bool kda = false;
  int B = 0, T = 0, H = 0, N = 0;
  bool packed = false;
  int64_t NT = 0;
  std::vector<int32_t> cu;  // snapshot of the offsets (packed)
};

constexpr uint32_t kKnownFlags = GDN_L2NORM_QK | GDN_BETA_SIGMOID | GDN_OUTPUT_FINAL_STATE;

int check_shape(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V, int32_t num_seqs,
                const int32_t* cu_seqlens, Problem& p) {
  if (B < 1 || T < 1 || H < 1)
    return fail(GDN_ERR_INVALID_ARGUMENT, "B, T and H must be >= 1 (got B=%d T=%d H=%d)", B, T, H);
  if (K != GDN_HEAD_DIM || V != GDN_HEAD_DIM)
    return fail(GDN_ERR_UNSUPPORTED, "only K = V = %d is supported (got K=%d V=%d)", GDN_HEAD_DIM, K, V);
  if (H > 65535)  // grid y of the stage finalize and gate-backward launches
    return fail(GDN_ERR_INVALID_ARGUMENT, "H = %d exceeds the supported range (at most 65535 heads)", H);
  if ((int64_t)B * T > INT32_MAX / 2)
    return fail(GDN_ERR_INVALID_ARGUMENT, "B*T = %lld tokens exceeds the supported range",
                (long long)B * T);
  p.B = B;
  p.T = T;
  p.H = H;
  if (cu_seqlens) {
    if (B != 1) return fail(GDN_ERR_INVALID_ARGUMENT, "packed input (cu_seqlens) requires B == 1 (got B=%d)", B);
    if (num_seqs < 1) return fail(GDN_ERR_INVALID_ARGUMENT, "num_seqs must be >= 1 with cu_seqlens");
    if (cu_seqlens[0] != 0)
      return fail(GDN_ERR_INVALID_ARGUMENT, "cu_seqlens[0] must be 0 (got %d)", cu_seqlens[0]);
    for (int i = 0; i < num_seqs; ++i)
      if (cu_seqlens[i + 1] <= cu_seqlens[i])
        return fail(GDN_ERR_INVALID_ARGUMENT,
                    "cu_seqlens must be strictly increasing (cu[%d]=%d, cu[%d]=%d)", i, cu_seqlens[i], i + 1,
                    cu_seqlens[i + 1]);
    if (cu_seqlens[num_seqs] != T)
      return fail(GDN_ERR_INVALID_ARGUMENT, "cu_seqlens[num_seqs] must equal T (got %d, T=%d)",
                  cu_seqlens[num_seqs], T);
    p.packed = true;
    p.N = num_seqs;
    p.cu.assign(cu_seqlens, cu_seqlens + num_seqs + 1);
    p.NT = 0;
    for (int i = 0; i < num_seqs; ++i) p.NT += (cu_seqlens[i + 1] - cu_seqlens[i] + GDN_CHUNK - 1) / GDN_CHUNK;
  } else {
    if (num_seqs != B)
      return fail(GDN_ERR_INVALID_ARGUMENT, "dense input needs num_seqs == B (got num_seqs=%d B=%d)", num_seqs, B);
    p.N = B;
    p.NT = (int64_t)B * ((T + GDN_CHUNK - 1) / GDN_CHUNK);
  }
  if ((int64_t)p.N * H > INT32_MAX || p.NT * H > INT32_MAX / 2)
    return fail(GDN_ERR_INVALID_ARGUMENT, "problem too large");
  return GDN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Device must be gfx950; result and compute-unit count cached per device id.
int check_device(int* cus) {
  static std::mutex mu;
  static std::vector<int> state;  // 0 unknown, 1 ok, 2 bad
  static std::vector<int> ncu;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(mu);
  if ((int)state.size() <= dev) {
    state.resize(dev + 1, 0);
    ncu.resize(dev + 1, 0);
  }
  if (state[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    state[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    ncu[dev] = prop.multiProcessorCount;
    if (state[dev] == 2)
      return fail(GDN_ERR_UNSUPPORTED, "device %d is %s; this library is built for gfx950 only", dev,
                  prop.gcnArchName);
  }
  if (state[dev] == 2) return fail(GDN_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
  if (cus) *cus = ncu[dev];
  return GDN_OK;
}

// ---------------------------------------------------------------------------
// Workspace layout: [tables | tmat | aqk | vec | kdec(KDA)], each 256-byte aligned.
// Packed tables: chunk table [NT] int4, sequence table [N] int4, sequence
// launch order [N] int (padded to whole int4).
struct Layout {
  size_t tab = 0, tmat = 0, aqk = 0, vec = 0, kdec = 0, total = 0;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// kda_gate: a KDA pass whose state kernel forms the decayed operands from the
// cumulative gate (state summary) instead of reading them from prepare.
Layout layout_for(const Problem& p, bool with_intermediates, bool kda_gate = false) {
  Layout L;
  size_t off = 0;
  L.tab = off;
  if (p.packed) off += align256(sizeof(int4) * ((size_t)p.NT + (size_t)p.N + ((size_t)p.N + 3) / 4));
  if (with_intermediates) {
    const size_t cmH = (size_t)p.NT * p.H;
    L.tmat = off;
    off += align256(cmH * GDN_CHUNK * 2 * GDN_CHUNK * sizeof(uint16_t));  // T, bf16 hi | lo
    L.aqk = off;
    off += align256(cmH * GDN_CHUNK * GDN_CHUNK * sizeof(uint16_t));
    L.vec = off;
    off += align256(cmH * GDN_VEC_ROWS * GDN_CHUNK * sizeof(float));
    if (p.kda) {
      L.kdec = off;
      off += align256(kda_gate ? cmH * GDN_CHUNK * GDN_HEAD_DIM * sizeof(float)
                               : cmH * gdn::kKdecElems * sizeof(uint16_t));
    }
  }
  L.total = off;
  return L;
}


// Pinned host staging for chunk tables: a small ring per process; a slot is
// reused only after the copy that last read it has completed.
struct StagingSlot {
  void* host = nullptr;
  size_t cap = 0;
  hipEvent_t done = nullptr;
  bool pending = false;
  int device = -1;
};

std::mutex g_stage_mu;
StagingSlot g_slots[8];
unsigned g_next_slot = 0;

int stage_upload(const void* src, size_t bytes, void* dst, hipStream_t stream);

int upload_tables(const Problem& p, void* dst, hipStream_t stream) {
  std::vector<int4> tab;
  tab.reserve((size_t)p.NT + p.N);
  std::vector<int4> seqs;
  seqs.reserve(p.N);
  int c = 0;
  for (int n = 0; n < p.N; ++n) {
    const int t0 = p.cu[n], len = p.cu[n + 1] - p.cu[n];
    const int nch = (len + GDN_CHUNK - 1) / GDN_CHUNK;
    seqs.push_back(make_int4(t0, len, c, nch));
    for (int j = 0; j < nch; ++j) {
      const int rem = len - j * GDN_CHUNK;
      tab.push_back(make_int4(t0 + j * GDN_CHUNK, rem < GDN_CHUNK ? rem : GDN_CHUNK, n, j));
    }
    c += nch;
  }
  tab.insert(tab.end(), seqs.begin(), seqs.end());
  // launch order of the sequential state pass: longest sequences first
  // (ties in sequence order)
  std::vector<int> order(p.N);
  for (int n = 0; n < p.N; ++n) order[n] = n;
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return seqs[x].w > seqs[y].w; });
  for (int n = 0; n < p.N; n += 4) {
    int4 e = make_int4(0, 0, 0, 0);
    e.x = order[n];
    if (n + 1 < p.N) e.y = order[n + 1];
    if (n + 2 < p.N) e.z = order[n + 2];
    if (n + 3 < p.N) e.w = order[n + 3];
    tab.push_back(e);
  }
  return stage_upload(tab.data(), tab.size() * sizeof(int4), dst, stream);
}

// Host data to device memory on `stream` through the pinned staging ring;
// the host buffer may be reused by the caller immediately.
int stage_upload(const void* src, size_t bytes, void* dst, hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_stage_mu);
  StagingSlot& s = g_slots[g_next_slot++ % 8];
  if (s.pending) {
    e = hipEventSynchronize(s.done);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize(staging)");
    s.pending = false;
  }
  if (s.device != dev && s.done) {
    (void)hipEventDestroy(s.done);
    s.done = nullptr;
  }
  if (!s.done) {
    e = hipEventCreateWithFlags(&s.done, hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
    s.device = dev;
  }
  if (s.cap < bytes) {
    if (s.host) (void)hipHostFree(s.host);
    s.host = nullptr;
    s.cap = 0;
    e = hipHostMalloc(&s.host, bytes, hipHostMallocDefault);
    if (e != hipSuccess) return hip_fail(e, "hipHostMalloc(staging)");
    s.cap = bytes;
  }
  std::memcpy(s.host, src, bytes);
  e = hipMemcpyAsync(dst, s.host, bytes, hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(tables)");
  e = hipEventRecord(s.done, stream);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord(staging)");
  s.pending = true;
  return GDN_OK;
}

gdn::Geometry make_geometry(const Problem& p, void* tab_dev) {
  gdn::Geometry g;
  g.T = p.T;
  g.ncb = (p.T + GDN_CHUNK - 1) / GDN_CHUNK;
  g.NT = (int)p.NT;
  g.N = p.N;
  if (p.packed) {
    g.ctab = static_cast<const int4*>(tab_dev);
    g.stab = static_cast<const int4*>(tab_dev) + p.NT;
    g.sorder = reinterpret_cast<const int*>(static_cast<const int4*>(tab_dev) + p.NT + p.N);
  } else {
    g.ctab = nullptr;
    g.stab = nullptr;
    g.sorder = nullptr;
  }
  return g;
}

// Workspace holder: caller's buffer, or a stream-ordered allocation.
struct Workspace {
  char* base = nullptr;
  bool owned = false;
  hipStream_t stream = nullptr;
  ~Workspace() {
    if (owned && base) (void)hipFreeAsync(base, stream);
  }
};

int acquire_workspace(void* ws, size_t ws_bytes, size_t need, hipStream_t stream, Workspace& W) {
  W.stream = stream;
  if (need == 0) return GDN_OK;
  if (ws) {
    if (ws_bytes < need)
      return fail(GDN_ERR_INVALID_ARGUMENT, "workspace too small: %zu bytes given, %zu needed", ws_bytes, need);
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
      return fail(GDN_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    W.base = static_cast<char*>(ws);
    return GDN_OK;
  }
  void* p = nullptr;
  hipError_t e = hipMallocAsync(&p, need, stream);
  if (e != hipSuccess) return hip_fail(e, "hipMallocAsync(workspace)");
  W.base = static_cast<char*>(p);
  W.owned = true;
  return GDN_OK;
}

// Optional per-kernel timing of the whole-pass entries (benchmarks): while
// enabled on the calling thread, each call records three events on its
// stream (before prepare, between the kernels, after the state kernel).
struct TimingRec {
  hipEvent_t ev[3];
};
thread_local bool g_timing = false;
thread_local std::vector<TimingRec> g_timing_recs;
thread_local std::vector<TimingRec> g_timing_pool;

int timing_mark(std::vector<TimingRec>& recs, int which, hipStream_t stream) {
  if (which == 0) {
    TimingRec r;
    if (!g_timing_pool.empty()) {
      r = g_timing_pool.back();
      g_timing_pool.pop_back();
    } else {
      for (int i = 0; i < 3; ++i) {
        hipError_t e = hipEventCreate(&r.ev[i]);
        if (e != hipSuccess) return hip_fail(e, "hipEventCreate(timing)");
      }
    }
    recs.push_back(r);
  }
  hipError_t e = hipEventRecord(recs.back().ev[which], stream);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord(timing)");
  return GDN_OK;
}

// The backward entry's marks: before prepare, after prepare, after the
// forward state pass, after each of the three backward kernels.
constexpr int kBwdMarks = 6;
struct BwdTimingRec {
  hipEvent_t ev[kBwdMarks];
};
thread_local std::vector<BwdTimingRec> g_bwd_recs;
thread_local std::vector<BwdTimingRec> g_bwd_pool;

int bwd_timing_mark(int which, hipStream_t stream) {
  if (which == 0) {
    BwdTimingRec r;
    if (!g_bwd_pool.empty()) {
      r = g_bwd_pool.back();
      g_bwd_pool.pop_back();
    } else {
      for (int i = 0; i < kBwdMarks; ++i) {
        hipError_t e = hipEventCreate(&r.ev[i]);
        if (e != hipSuccess) return hip_fail(e, "hipEventCreate(timing)");
      }
    }
    g_bwd_recs.push_back(r);
  }
  hipError_t e = hipEventRecord(g_bwd_recs.back().ev[which], stream);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord(timing)");
  return GDN_OK;
}

int check_common(const void* q, const void* k, const void* v, const float* g, const void* beta, float scale,
                 uint32_t flags) {
  if (!q || !k || !v || !g || !beta) return fail(GDN_ERR_INVALID_ARGUMENT, "q, k, v, g and beta must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v))
    return fail(GDN_ERR_INVALID_ARGUMENT, "q, k and v must be 16-byte aligned");
  if (!(std::isfinite(scale) && scale > 0.0f))
    return fail(GDN_ERR_INVALID_ARGUMENT, "scale must be finite and > 0 (got %g)", (double)scale);
  if (flags & ~kKnownFlags) return fail(GDN_ERR_INVALID_ARGUMENT, "unknown flag bits 0x%x", flags & ~kKnownFlags);
  return GDN_OK;
}

int chunk_fwd(bool kda, const void* q, const void* k, const void* v, const float* g, const void* beta,
              const float* initial_state, const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T,
              int32_t H, int32_t K, int32_t V, float scale, uint32_t flags, void* o, float* final_state,
              void* workspace, size_t workspace_bytes, void* stream_ptr, bool gated = false,
              const float* a_log = nullptr, const float* dt_bias = nullptr, bool timed = true) {
  g_last_error.clear();
  Problem p;
  p.kda = kda;
  int rc = check_shape(B, T, H, K, V, num_seqs, cu_seqlens, p);
  if (rc) return rc;
  rc = check_common(q, k, v, g, beta, scale, flags);
  if (rc) return rc;
  if (gated) {
    if (!a_log || !dt_bias) return fail(GDN_ERR_INVALID_ARGUMENT, "A_log and dt_bias must be non-NULL");
    if (kda && (!aligned16(dt_bias) || !aligned16(g)))
      return fail(GDN_ERR_INVALID_ARGUMENT, "KDA gate logits and dt_bias must be 16-byte aligned");
  }
  if (!o) return fail(GDN_ERR_INVALID_ARGUMENT, "o must be non-NULL");
  if (!aligned16(o)) return fail(GDN_ERR_INVALID_ARGUMENT, "o must be 16-byte aligned");
  if ((flags & GDN_OUTPUT_FINAL_STATE) && !final_state)
    return fail(GDN_ERR_INVALID_ARGUMENT, "GDN_OUTPUT_FINAL_STATE set but final_state is NULL");
  int cus = 0;
  rc = check_device(&cus);
  if (rc) return rc;

  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const Layout L = layout_for(p, true);
  Workspace W;
  rc = acquire_workspace(workspace, workspace_bytes, L.total, stream, W);
  if (rc) return rc;
  if (p.packed) {
    rc = upload_tables(p, W.base + L.tab, stream);
    if (rc) return rc;
  }
  const gdn::Geometry geo = make_geometry(p, W.base + L.tab);
  const bool timing = g_timing && timed;
  if (timing && (rc = timing_mark(g_timing_recs, 0, stream))) return rc;

  gdn::PrepareArgs pa{};
  pa.q = static_cast<const uint16_t*>(q);
  pa.k = static_cast<const uint16_t*>(k);
  pa.g = g;
  pa.beta = static_cast<const uint16_t*>(beta);
  pa.tmat = reinterpret_cast<uint16_t*>(W.base + L.tmat);
  pa.aqk = reinterpret_cast<uint16_t*>(W.base + L.aqk);
  pa.vec = reinterpret_cast<float*>(W.base + L.vec);
  pa.gk = nullptr;
  pa.kdec = kda ? reinterpret_cast<uint16_t*>(W.base + L.kdec) : nullptr;
  pa.a_log = gated ? a_log : nullptr;
  pa.dt_bias = gated ? dt_bias : nullptr;
  pa.geo = geo;
  pa.H = H;
  pa.scale = scale;
  pa.flags = flags;
  pa.cus = cus;
  hipError_t e = gdn::launch_prepare(kda, pa, stream);
  if (e != hipSuccess) return hip_fail(e, "prepare launch");
  if (timing && (rc = timing_mark(g_timing_recs, 1, stream))) return rc;

  gdn::FwdArgs fa{};
  fa.q = pa.q;
  fa.k = pa.k;
  fa.v = static_cast<const uint16_t*>(v);
  fa.tmat = pa.tmat;
  fa.aqk = pa.aqk;
  fa.vec = pa.vec;
  fa.gk = nullptr;
  fa.kdec = pa.kdec;
  fa.s0 = initial_state;
  fa.sfinal = (flags & GDN_OUTPUT_FINAL_STATE) ? final_state : nullptr;
  fa.o = static_cast<uint16_t*>(o);
  fa.geo = geo;
  fa.H = H;
  e = gdn::launch_fwd(kda, false, true, fa, stream);
  if (e != hipSuccess) return hip_fail(e, "state/output launch");
  if (timing && (rc = timing_mark(g_timing_recs, 2, stream))) return rc;
  return GDN_OK;
}

// ---------------------------------------------------------------------------
// The fixed scratch of gdn_chunk_fwd_noalloc: a file-scope device array in
// place of a workspace, so that a call allocates nothing. Every device the
// library runs on holds its own copy until the process ends. In host code
// the array's name is only a host-side stand-in: kernels get the device
// address that hipGetSymbolAddress returns for the current device, resolved
// once per device on the first call there and kept.
static __device__ __align__(256) unsigned char noalloc_scratch[GDN_NOALLOC_SCRATCH_BYTES];

int noalloc_scratch_address(void** out) {
  static std::mutex mu;
  static std::vector<void*> addr;  // per device id
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(mu);
  if ((int)addr.size() <= dev) addr.resize(dev + 1, nullptr);
  if (!addr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(noalloc_scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(noalloc scratch)");
    if (!ptr || (reinterpret_cast<uintptr_t>(ptr) & 255u) != 0)
      return fail(GDN_ERR_HIP, "the no-allocation scratch has no usable device address");
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return GDN_OK;
}

// State summary of every (sequence, head): prepare, then the state-only
// pass twice: from S0 = 0 with v (S), and from S0 = I with v = 0 (M).
int state_summary(bool kda, const void* q, const void* k, const void* v, const float* g, const void* beta,
                  const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t K,
                  int32_t V, uint32_t flags, float* transition, float* state_ext, void* workspace,
                  size_t workspace_bytes, void* stream_ptr, bool gated = false, const float* a_log = nullptr,
                  const float* dt_bias = nullptr) {
  g_last_error.clear();
  Problem p;
  p.kda = kda;
  int rc = check_shape(B, T, H, K, V, num_seqs, cu_seqlens, p);
  if (rc) return rc;
  rc = check_common(q ? q : k, k, v, g, beta, 1.0f, flags);
  if (rc) return rc;
  if (!transition || !state_ext) return fail(GDN_ERR_INVALID_ARGUMENT, "transition and state_ext must be non-NULL");
  if (gated) {
    if (!a_log || !dt_bias) return fail(GDN_ERR_INVALID_ARGUMENT, "A_log and dt_bias must be non-NULL");
    if (kda && (!aligned16(dt_bias) || !aligned16(g)))
      return fail(GDN_ERR_INVALID_ARGUMENT, "KDA gate logits and dt_bias must be 16-byte aligned");
  }
  int cus = 0;
  rc = check_device(&cus);
  if (rc) return rc;

  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const Layout L = layout_for(p, true, true);
  Workspace W;
  rc = acquire_workspace(workspace, workspace_bytes, L.total, stream, W);
  if (rc) return rc;
  if (p.packed) {
    rc = upload_tables(p, W.base + L.tab, stream);
    if (rc) return rc;
  }
  const gdn::Geometry geo = make_geometry(p, W.base + L.tab);

  gdn::PrepareArgs pa{};
  pa.q = static_cast<const uint16_t*>(q ? q : k);  // only the unused Aqk depends on q
  pa.k = static_cast<const uint16_t*>(k);
  pa.g = g;
  pa.beta = static_cast<const uint16_t*>(beta);
  pa.tmat = reinterpret_cast<uint16_t*>(W.base + L.tmat);
  pa.aqk = reinterpret_cast<uint16_t*>(W.base + L.aqk);
  pa.vec = reinterpret_cast<float*>(W.base + L.vec);
  pa.gk = kda ? reinterpret_cast<float*>(W.base + L.kdec) : nullptr;
  pa.kdec = nullptr;
  pa.a_log = gated ? a_log : nullptr;
  pa.dt_bias = gated ? dt_bias : nullptr;
  pa.geo = geo;
  pa.H = H;
  pa.scale = 1.0f;
  pa.flags = flags & ~(uint32_t)GDN_OUTPUT_FINAL_STATE;
  pa.cus = cus;
  hipError_t e = gdn::launch_prepare(kda, pa, stream);
  if (e != hipSuccess) return hip_fail(e, "prepare launch");

  gdn::FwdArgs fa{};
  fa.k = pa.k;
  fa.v = static_cast<const uint16_t*>(v);
  fa.tmat = pa.tmat;
  fa.aqk = pa.aqk;
  fa.vec = pa.vec;
  fa.gk = pa.gk;
  fa.s0 = nullptr;
  fa.sfinal = state_ext;
  fa.geo = geo;
  fa.H = H;
  fa.s_identity = 0;
  e = gdn::launch_fwd(kda, false, false, fa, stream);
  if (e != hipSuccess) return hip_fail(e, "state pass launch");
  fa.sfinal = transition;
  fa.s_identity = 1;
  e = gdn::launch_fwd(kda, false, false, fa, stream);
  if (e != hipSuccess) return hip_fail(e, "transition pass launch");
  return GDN_OK;
}

// Backward pass (GDN): workspace = forward layout | h | v_new | dS_next |
// dv_new | E, F, D | <dS_next, S>, each 256-byte aligned.
struct BwdLayout {
  Layout fwd;
  size_t h = 0, vnew = 0, dhn = 0, dvn = 0, efd = 0, sdot = 0, gpart = 0, total = 0;
  int gate_blocks = 0;  // token blocks of the gate backward
};

BwdLayout bwd_layout_for(const Problem& p) {
  BwdLayout L;
  L.fwd = layout_for(p, true);
  size_t off = L.fwd.total;
  const size_t cmH = (size_t)p.NT * p.H;
  const size_t state = cmH * GDN_HEAD_DIM * GDN_HEAD_DIM * sizeof(float);
  const size_t rows = cmH * GDN_CHUNK * GDN_HEAD_DIM * sizeof(float);
  L.h = off;
  off += align256(state);
  L.vnew = off;
  off += align256(rows);
  L.dhn = off;
  off += align256(state);
  L.dvn = off;
  off += align256(rows);
  L.efd = off;
  off += align256(3 * rows);
  L.sdot = off;
  off += align256(cmH * sizeof(float));
  L.gate_blocks = (int)(((long)p.B * p.T + gdn::kGateBwdTok - 1) / gdn::kGateBwdTok);
  L.gpart = off;
  off += align256((size_t)2 * p.H * L.gate_blocks * sizeof(float));
  L.total = off;
  return L;
}

// Recompute the forward intermediates (prepare; state pass storing the
// state entering every chunk and v_new), then the three backward kernels.
int chunk_bwd(const void* q, const void* k, const void* v, const float* g, const void* beta,
              const float* initial_state, const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T,
              int32_t H, int32_t K, int32_t V, float scale, uint32_t flags, const void* d_o,
              const float* d_final_state, float* dq, float* dk, float* dv, float* dg, float* dbeta,
              float* d_initial_state, void* workspace, size_t workspace_bytes, void* stream_ptr,
              bool gated = false, const float* a_log = nullptr, const float* dt_bias = nullptr,
              float* da_log = nullptr, float* ddt_bias = nullptr) {
  g_last_error.clear();
  Problem p;
  p.kda = false;
  int rc = check_shape(B, T, H, K, V, num_seqs, cu_seqlens, p);
  if (rc) return rc;
  rc = check_common(q, k, v, g, beta, scale, flags);
  if (rc) return rc;
  if (!d_o || !dq || !dk || !dv || !dg || !dbeta)
    return fail(GDN_ERR_INVALID_ARGUMENT, "d_o, dq, dk, dv, dg and dbeta must be non-NULL");
  if (gated && (!a_log || !dt_bias || !da_log || !ddt_bias))
    return fail(GDN_ERR_INVALID_ARGUMENT, "A_log, dt_bias, dA_log and ddt_bias must be non-NULL");
  if (!aligned16(d_o) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return fail(GDN_ERR_INVALID_ARGUMENT, "d_o, dq, dk and dv must be 16-byte aligned");
  int cus = 0;
  rc = check_device(&cus);
  if (rc) return rc;

  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const BwdLayout L = bwd_layout_for(p);
  Workspace W;
  rc = acquire_workspace(workspace, workspace_bytes, L.total, stream, W);
  if (rc) return rc;
  if (p.packed) {
    rc = upload_tables(p, W.base + L.fwd.tab, stream);
    if (rc) return rc;
  }
  const gdn::Geometry geo = make_geometry(p, W.base + L.fwd.tab);
  if (g_timing && (rc = bwd_timing_mark(0, stream))) return rc;

  gdn::PrepareArgs pa{};
  pa.q = static_cast<const uint16_t*>(q);
  pa.k = static_cast<const uint16_t*>(k);
  pa.g = g;
  pa.beta = static_cast<const uint16_t*>(beta);
  pa.tmat = reinterpret_cast<uint16_t*>(W.base + L.fwd.tmat);
  pa.aqk = reinterpret_cast<uint16_t*>(W.base + L.fwd.aqk);
  pa.vec = reinterpret_cast<float*>(W.base + L.fwd.vec);
  pa.geo = geo;
  pa.H = H;
  pa.scale = scale;
  pa.flags = flags & ~(uint32_t)GDN_OUTPUT_FINAL_STATE;
  pa.cus = cus;
  pa.a_log = gated ? a_log : nullptr;
  pa.dt_bias = gated ? dt_bias : nullptr;
  hipError_t e = gdn::launch_prepare(false, pa, stream);
  if (e != hipSuccess) return hip_fail(e, "prepare launch");

  gdn::FwdArgs fa{};
  fa.k = pa.k;
  fa.v = static_cast<const uint16_t*>(v);
  fa.tmat = pa.tmat;
  fa.aqk = pa.aqk;
  fa.vec = pa.vec;
  fa.s0 = initial_state;
  fa.sfinal = nullptr;
  fa.h_out = reinterpret_cast<float*>(W.base + L.h);
  fa.vnew_out = reinterpret_cast<float*>(W.base + L.vnew);
  fa.geo = geo;
  fa.H = H;
  if (g_timing && (rc = bwd_timing_mark(1, stream))) return rc;
  e = gdn::launch_fwd(false, true, false, fa, stream);
  if (e != hipSuccess) return hip_fail(e, "forward recompute launch");
  if (g_timing && (rc = bwd_timing_mark(2, stream))) return rc;

  gdn::BwdArgs ba{};
  ba.q = pa.q;
  ba.k = pa.k;
  ba.v = fa.v;
  ba.dout = static_cast<const uint16_t*>(d_o);
  ba.tmat = pa.tmat;
  ba.aqk = pa.aqk;
  ba.vec = pa.vec;
  ba.h = fa.h_out;
  ba.vnew = fa.vnew_out;
  ba.dsfinal = d_final_state;
  ba.dhn = reinterpret_cast<float*>(W.base + L.dhn);
  ba.dvn = reinterpret_cast<float*>(W.base + L.dvn);
  ba.efd = reinterpret_cast<float*>(W.base + L.efd);
  ba.sdot = reinterpret_cast<float*>(W.base + L.sdot);
  ba.ds0 = d_initial_state;
  ba.dq = dq;
  ba.dk = dk;
  ba.dv = dv;
  ba.dg = dg;
  ba.dbeta = dbeta;
  ba.geo = geo;
  ba.H = H;
  ba.scale = scale;
  ba.flags = flags;
  ba.cus = cus;
  for (int stage = 0; stage < 3; ++stage) {
    e = gdn::launch_gdn_bwd(ba, stage, stream);
    if (e != hipSuccess) return hip_fail(e, "backward launch");
    if (g_timing && (rc = bwd_timing_mark(3 + stage, stream))) return rc;
  }
  if (gated) {
    gdn::GateBwdArgs ga{};
    ga.x = g;
    ga.a_log = a_log;
    ga.dt_bias = dt_bias;
    ga.dg = dg;
    ga.part = reinterpret_cast<float*>(W.base + L.gpart);
    ga.da_log = da_log;
    ga.ddt_bias = ddt_bias;
    ga.ntok = (long)B * T;
    ga.H = H;
    ga.nblk = L.gate_blocks;
    e = gdn::launch_gate_bwd(ga, stream);
    if (e != hipSuccess) return hip_fail(e, "gate backward launch");
  }
  return GDN_OK;
}

// Shared front half of the stage entries: validation, tables, geometry.
struct StageCtx {
  Problem p;
  Workspace W;
  gdn::Geometry geo;
  int cus = 0;
};

int stage_begin(int32_t kda, const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H,
                int32_t K, int32_t V, hipStream_t stream, StageCtx& ctx) {
  g_last_error.clear();
  ctx.p.kda = kda != 0;
  int rc = check_shape(B, T, H, K, V, num_seqs, cu_seqlens, ctx.p);
  if (rc) return rc;
  rc = check_device(&ctx.cus);
  if (rc) return rc;
  const Layout L = layout_for(ctx.p, false);
  rc = acquire_workspace(nullptr, 0, L.total, stream, ctx.W);
  if (rc) return rc;
  if (ctx.p.packed) {
    rc = upload_tables(ctx.p, ctx.W.base + L.tab, stream);
    if (rc) return rc;
  }
  ctx.geo = make_geometry(ctx.p, ctx.W.base + L.tab);
  return GDN_OK;
}

}  // namespace

extern "C" {

const char* gdn_last_error(void) { return g_last_error.c_str(); }

int gdn_num_chunks(int32_t B, int32_t T, int32_t num_seqs, const int32_t* cu_seqlens, int64_t* num_chunks) {
  g_last_error.clear();
  if (!num_chunks) return fail(GDN_ERR_INVALID_ARGUMENT, "num_chunks must be non-NULL");
  Problem p;
  int rc = check_shape(B, T, 1, GDN_HEAD_DIM, GDN_HEAD_DIM, num_seqs, cu_seqlens, p);
  if (rc) return rc;
  *num_chunks = p.NT;
  return GDN_OK;
}

static size_t workspace_bytes(bool kda, int32_t B, int32_t T, int32_t H, int32_t K, int32_t V, int32_t num_seqs,
                              const int32_t* cu_seqlens, uint32_t flags) {
  g_last_error.clear();
  Problem p;
  p.kda = kda;
  if (check_shape(B, T, H, K, V, num_seqs, cu_seqlens, p)) return 0;
  if (flags & ~kKnownFlags) {
    fail(GDN_ERR_INVALID_ARGUMENT, "unknown flag bits 0x%x", flags & ~kKnownFlags);
    return 0;
  }
  return layout_for(p, true).total;
}

size_t gdn_chunk_fwd_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V, int32_t num_seqs,
                                     const int32_t* cu_seqlens, uint32_t flags) {
  return workspace_bytes(false, B, T, H, K, V, num_seqs, cu_seqlens, flags);
}

size_t kda_chunk_fwd_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V, int32_t num_seqs,
                                     const int32_t* cu_seqlens, uint32_t flags) {
  return workspace_bytes(true, B, T, H, K, V, num_seqs, cu_seqlens, flags);
}

int gdn_chunk_fwd(const void* q, const void* k, const void* v, const float* g, const void* beta,
                  const float* initial_state, const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T,
                  int32_t H, int32_t K, int32_t V, float scale, uint32_t flags, void* o, float* final_state,
                  void* workspace, size_t workspace_bytes, void* stream) {
  return chunk_fwd(false, q, k, v, g, beta, initial_state, cu_seqlens, num_seqs, B, T, H, K, V, scale, flags, o,
                   final_state, workspace, workspace_bytes, stream);
}

int gdn_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* g, const void* beta,
                          const float* initial_state, const int32_t* cu_seqlens, int32_t num_seqs, int32_t B,
                          int32_t T, int32_t H, int32_t K, int32_t V, float scale, uint32_t flags, void* o,
                          float* final_state, void* stream) {
  g_last_error.clear();
  if (cu_seqlens)
    return fail(GDN_ERR_UNSUPPORTED,
                "gdn_chunk_fwd_noalloc takes dense input only (the packed chunk table is staged through "
                "pinned host memory, which this entry does not allocate)");
  Problem p;
  int rc = check_shape(B, T, H, K, V, num_seqs, nullptr, p);
  if (rc) return rc;
  const size_t need = layout_for(p, true).total;
  if (need > (size_t)GDN_NOALLOC_SCRATCH_BYTES)
    return fail(GDN_ERR_INVALID_ARGUMENT,
                "problem needs %zu bytes of scratch, above the fixed %zu bytes of gdn_chunk_fwd_noalloc "
                "(B*ceil(T/64)*H = %lld chunk-heads; use gdn_chunk_fwd with a workspace)",
                need, (size_t)GDN_NOALLOC_SCRATCH_BYTES, (long long)(p.NT * p.H));
  rc = check_common(q, k, v, g, beta, scale, flags);
  if (rc) return rc;
  if (!o) return fail(GDN_ERR_INVALID_ARGUMENT, "o must be non-NULL");
  if ((flags & GDN_OUTPUT_FINAL_STATE) && !final_state)
    return fail(GDN_ERR_INVALID_ARGUMENT, "GDN_OUTPUT_FINAL_STATE set but final_state is NULL");
  rc = check_device(nullptr);
  if (rc) return rc;
  void* scratch = nullptr;
  rc = noalloc_scratch_address(&scratch);
  if (rc) return rc;
  return chunk_fwd(false, q, k, v, g, beta, initial_state, nullptr, num_seqs, B, T, H, K, V, scale, flags, o,
                   final_state, scratch, (size_t)GDN_NOALLOC_SCRATCH_BYTES, stream, false, nullptr, nullptr,
                   /*timed=*/false);
}

int kda_chunk_fwd(const void* q, const void* k, const void* v, const float* g, const void* beta,
                  const float* initial_state, const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T,
                  int32_t H, int32_t K, int32_t V, float scale, uint32_t flags, void* o, float* final_state,
                  void* workspace, size_t workspace_bytes, void* stream) {
  return chunk_fwd(true, q, k, v, g, beta, initial_state, cu_seqlens, num_seqs, B, T, H, K, V, scale, flags, o,
                   final_state, workspace, workspace_bytes, stream);
}

int gdn_chunk_fwd_gated(const void* q, const void* k, const void* v, const float* g_raw, const float* A_log,
                        const float* dt_bias, const void* beta, const float* initial_state,
                        const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t K,
                        int32_t V, float scale, uint32_t flags, void* o, float* final_state, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return chunk_fwd(false, q, k, v, g_raw, beta, initial_state, cu_seqlens, num_seqs, B, T, H, K, V, scale, flags,
                   o, final_state, workspace, workspace_bytes, stream, true, A_log, dt_bias);
}

int kda_chunk_fwd_gated(const void* q, const void* k, const void* v, const float* g_raw, const float* A_log,
                        const float* dt_bias, const void* beta, const float* initial_state,
                        const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t K,
                        int32_t V, float scale, uint32_t flags, void* o, float* final_state, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return chunk_fwd(true, q, k, v, g_raw, beta, initial_state, cu_seqlens, num_seqs, B, T, H, K, V, scale, flags,
                   o, final_state, workspace, workspace_bytes, stream, true, A_log, dt_bias);
}

size_t gdn_chunk_bwd_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V, int32_t num_seqs,
                                     const int32_t* cu_seqlens, uint32_t flags) {
  g_last_error.clear();
  Problem p;
  if (check_shape(B, T, H, K, V, num_seqs, cu_seqlens, p)) return 0;
  if (flags & ~kKnownFlags) {
    fail(GDN_ERR_INVALID_ARGUMENT, "unknown flag bits 0x%x", flags & ~kKnownFlags);
    return 0;
  }
  return bwd_layout_for(p).total;
}

int gdn_chunk_bwd(const void* q, const void* k, const void* v, const float* g, const void* beta,
                  const float* initial_state, const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T,
                  int32_t H, int32_t K, int32_t V, float scale, uint32_t flags, const void* d_o,
                  const float* d_final_state, float* dq, float* dk, float* dv, float* dg, float* dbeta,
                  float* d_initial_state, void* workspace, size_t workspace_bytes, void* stream) {
  return chunk_bwd(q, k, v, g, beta, initial_state, cu_seqlens, num_seqs, B, T, H, K, V, scale, flags, d_o,
                   d_final_state, dq, dk, dv, dg, dbeta, d_initial_state, workspace, workspace_bytes, stream);
}

int gdn_chunk_bwd_gated(const void* q, const void* k, const void* v, const float* g_raw, const float* A_log,
                        const float* dt_bias, const void* beta, const float* initial_state,
                        const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t K,
                        int32_t V, float scale, uint32_t flags, const void* d_o, const float* d_final_state,
                        float* dq, float* dk, float* dv, float* dg_raw, float* dA_log, float* ddt_bias,
                        float* dbeta, float* d_initial_state, void* workspace, size_t workspace_bytes,
                        void* stream) {
  return chunk_bwd(q, k, v, g_raw, beta, initial_state, cu_seqlens, num_seqs, B, T, H, K, V, scale, flags, d_o,
                   d_final_state, dq, dk, dv, dg_raw, dbeta, d_initial_state, workspace, workspace_bytes, stream,
                   true, A_log, dt_bias, dA_log, ddt_bias);
}

int gdn_state_summary(const void* q, const void* k, const void* v, const float* g, const void* beta,
                      const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t K,
                      int32_t V, uint32_t flags, float* transition, float* state_ext, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return state_summary(false, q, k, v, g, beta, cu_seqlens, num_seqs, B, T, H, K, V, flags, transition, state_ext,
                       workspace, workspace_bytes, stream);
}

int kda_state_summary(const void* q, const void* k, const void* v, const float* g, const void* beta,
                      const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t K,
                      int32_t V, uint32_t flags, float* transition, float* state_ext, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return state_summary(true, q, k, v, g, beta, cu_seqlens, num_seqs, B, T, H, K, V, flags, transition, state_ext,
                       workspace, workspace_bytes, stream);
}

int gdn_state_summary_gated(int32_t kda, const void* q, const void* k, const void* v, const float* g_raw,
                            const float* A_log, const float* dt_bias, const void* beta, const int32_t* cu_seqlens,
                            int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                            uint32_t flags, float* transition, float* state_ext, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return state_summary(kda != 0, q, k, v, g_raw, beta, cu_seqlens, num_seqs, B, T, H, K, V, flags, transition,
                       state_ext, workspace, workspace_bytes, stream, true, A_log, dt_bias);
}

size_t gdn_state_summary_workspace_bytes(int32_t kda, int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                                         int32_t num_seqs, const int32_t* cu_seqlens) {
  g_last_error.clear();
  Problem p;
  p.kda = kda != 0;
  if (check_shape(B, T, H, K, V, num_seqs, cu_seqlens, p)) return 0;
  return layout_for(p, true, true).total;
}

int gdn_state_summary_apply(const float* transition, const float* state_ext, const float* state_in,
                            float* state_out, int32_t N, int32_t H, int32_t K, int32_t V, void* stream) {
  g_last_error.clear();
  if (!transition || !state_ext || !state_out)
    return fail(GDN_ERR_INVALID_ARGUMENT, "transition, state_ext and state_out must be non-NULL");
  if (N <= 0 || H <= 0) return fail(GDN_ERR_INVALID_ARGUMENT, "N and H must be positive (got %d, %d)", N, H);
  if (K != GDN_HEAD_DIM || V != GDN_HEAD_DIM)
    return fail(GDN_ERR_UNSUPPORTED, "K and V must be %d (got %d, %d)", GDN_HEAD_DIM, K, V);
  if (!aligned16(transition) || !aligned16(state_ext) || !aligned16(state_out) || (state_in && !aligned16(state_in)))
    return fail(GDN_ERR_INVALID_ARGUMENT, "state arrays must be 16-byte aligned");
  if (state_out == transition || state_out == state_in)
    return fail(GDN_ERR_INVALID_ARGUMENT, "state_out must not alias transition or state_in");
  int rc = check_device(nullptr);
  if (rc) return rc;
  hipError_t e = gdn::launch_summary_apply(transition, state_ext, state_in, state_out, (long)N * H,
                                           static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "summary apply launch");
  return GDN_OK;
}

size_t gdn_short_conv_workspace_bytes(int32_t num_seqs, const int32_t* cu_seqlens) {
  g_last_error.clear();
  return cu_seqlens ? align256(sizeof(int32_t) * ((size_t)num_seqs + 1)) : 0;
}

int gdn_short_conv(const void* x, const float* weight, const float* bias, const void* halo,
                   const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t D, int32_t W,
                   int32_t dilation, int32_t silu, void* y, void* workspace, size_t workspace_bytes, void* stream_ptr) {
  g_last_error.clear();
  Problem p;
  int rc = check_shape(B, T, 1, GDN_HEAD_DIM, GDN_HEAD_DIM, num_seqs, cu_seqlens, p);
  if (rc) return rc;
  if (!x || !weight || !y) return fail(GDN_ERR_INVALID_ARGUMENT, "x, weight and y must be non-NULL");
  if (D < 8 || D % 8 != 0) return fail(GDN_ERR_UNSUPPORTED, "D must be a positive multiple of 8 (got %d)", D);
  if (W < 1 || W > 8) return fail(GDN_ERR_UNSUPPORTED, "kernel size W must be 1..8 (got %d)", W);
  if (dilation < 1 || (int64_t)(W - 1) * dilation > 4096)
    return fail(GDN_ERR_INVALID_ARGUMENT, "dilation must be >= 1 with (W-1)*dilation <= 4096 (got %d)", dilation);
  if ((int64_t)B * T * D > INT64_MAX / 4) return fail(GDN_ERR_INVALID_ARGUMENT, "problem too large");
  if (!aligned16(x) || !aligned16(y) || (halo && !aligned16(halo)))
    return fail(GDN_ERR_INVALID_ARGUMENT, "x, y and halo must be 16-byte aligned");
  if (x == y) return fail(GDN_ERR_INVALID_ARGUMENT, "y must not alias x");
  rc = check_device(nullptr);
  if (rc) return rc;
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  Workspace Wk;
  const size_t need = gdn_short_conv_workspace_bytes(num_seqs, cu_seqlens);
  rc = acquire_workspace(workspace, workspace_bytes, need, stream, Wk);
  if (rc) return rc;
  if (cu_seqlens) {
    rc = stage_upload(cu_seqlens, sizeof(int32_t) * ((size_t)num_seqs + 1), Wk.base, stream);
    if (rc) return rc;
  }
  gdn::ConvArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.w = weight;
  a.bias = bias;
  a.halo = static_cast<const uint16_t*>(halo);
  a.cu = cu_seqlens ? reinterpret_cast<const int*>(Wk.base) : nullptr;
  a.y = static_cast<uint16_t*>(y);
  a.B = B;
  a.T = T;
  a.D = D;
  a.W = W;
  a.dilation = dilation;
  a.N = p.N;
  a.silu = silu != 0;
  hipError_t e = gdn::launch_short_conv(a, stream);
  if (e != hipSuccess) return hip_fail(e, "short conv launch");
  return GDN_OK;
}

int gdn_timing_enable(int32_t enable) {
  g_last_error.clear();
  g_timing = enable != 0;
  return GDN_OK;
}

int gdn_timing_read(double* prepare_ms, double* state_ms, int64_t* calls) {
  g_last_error.clear();
  if (!prepare_ms || !state_ms || !calls) return fail(GDN_ERR_INVALID_ARGUMENT, "NULL output pointer");
  double a = 0.0, b = 0.0;
  for (TimingRec& r : g_timing_recs) {
    hipError_t e = hipEventSynchronize(r.ev[2]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize(timing)");
    float t0 = 0.f, t1 = 0.f;
    e = hipEventElapsedTime(&t0, r.ev[0], r.ev[1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    e = hipEventElapsedTime(&t1, r.ev[1], r.ev[2]);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    a += t0;
    b += t1;
  }
  *prepare_ms = a;
  *state_ms = b;
  *calls = (int64_t)g_timing_recs.size();
  g_timing_pool.insert(g_timing_pool.end(), g_timing_recs.begin(), g_timing_recs.end());
  g_timing_recs.clear();
  return GDN_OK;
}

int gdn_bwd_timing_read(double* ms, int64_t* calls) {
  g_last_error.clear();
  if (!ms || !calls) return fail(GDN_ERR_INVALID_ARGUMENT, "NULL output pointer");
  double acc[kBwdMarks - 1] = {0.0, 0.0, 0.0, 0.0, 0.0};
  for (BwdTimingRec& r : g_bwd_recs) {
    hipError_t e = hipEventSynchronize(r.ev[kBwdMarks - 1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize(timing)");
    for (int i = 0; i + 1 < kBwdMarks; ++i) {
      float t = 0.f;
      e = hipEventElapsedTime(&t, r.ev[i], r.ev[i + 1]);
      if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
      acc[i] += t;
    }
  }
  for (int i = 0; i + 1 < kBwdMarks; ++i) ms[i] = acc[i];
  *calls = (int64_t)g_bwd_recs.size();
  g_bwd_pool.insert(g_bwd_pool.end(), g_bwd_recs.begin(), g_bwd_recs.end());
  g_bwd_recs.clear();
  return GDN_OK;
}

int gdn_stage_prepare(int32_t kda, const void* q, const void* k, const float* g, const void* beta,
                      const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t K,
                      int32_t V, float scale, uint32_t flags, void* tmat, void* aqk, float* vec, float* gk,
                      void* stream_ptr) {
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  g_last_error.clear();
  int rc = check_common(q, k, q, g, beta, scale, flags);
  if (rc) return rc;
  if (!tmat || !aqk || !vec || (kda && !gk))
    return fail(GDN_ERR_INVALID_ARGUMENT, "tmat, aqk, vec (and gk for KDA) must be non-NULL");
  StageCtx ctx;
  rc = stage_begin(kda, cu_seqlens, num_seqs, B, T, H, K, V, stream, ctx);
  if (rc) return rc;
  gdn::PrepareArgs pa{};
  pa.q = static_cast<const uint16_t*>(q);
  pa.k = static_cast<const uint16_t*>(k);
  pa.g = g;
  pa.beta = static_cast<const uint16_t*>(beta);
  pa.tmat = static_cast<uint16_t*>(tmat);
  pa.aqk = static_cast<uint16_t*>(aqk);
  pa.vec = vec;
  pa.gk = gk;
  pa.geo = ctx.geo;
  pa.cus = ctx.cus;
  pa.H = H;
  pa.scale = scale;
  pa.flags = flags;
  hipError_t e = gdn::launch_prepare(kda != 0, pa, stream);
  if (e != hipSuccess) return hip_fail(e, "prepare launch");
  return GDN_OK;
}

// KDA backward workspace: the GDN backward's sections (the KDA decayed-operand
// area holds the cumulative gate) plus dP, dA (64 x 64), dKD (64 x 128) and
// the T-term part of dbeta per chunk-head, and the partial sums of the
// in-kernel gate's backward.
struct KdaBwdLayout {
  BwdLayout b;
  size_t dp = 0, da = 0, dkd = 0, db1 = 0, kgpart = 0, total = 0;
  int kgate_blocks = 0;
};

KdaBwdLayout kda_bwd_layout_for(const Problem& p) {
  KdaBwdLayout L;
  L.b = bwd_layout_for(p);
  size_t off = L.b.total;
  const size_t cmH = (size_t)p.NT * p.H;
  L.dp = off;
  off += align256(cmH * GDN_CHUNK * GDN_CHUNK * sizeof(float));
  L.da = off;
  off += align256(cmH * GDN_CHUNK * GDN_CHUNK * sizeof(float));
  L.dkd = off;
  off += align256(cmH * GDN_CHUNK * GDN_HEAD_DIM * sizeof(float));
  L.db1 = off;
  off += align256(cmH * GDN_CHUNK * sizeof(float));
  L.kgate_blocks = (int)(((long)p.B * p.T + gdn::kKdaGateTok - 1) / gdn::kKdaGateTok);
  L.kgpart = off;
  off += align256((size_t)p.H * (1 + GDN_HEAD_DIM) * L.kgate_blocks * sizeof(float));
  L.total = off;
  return L;
}

size_t kda_chunk_bwd_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V, int32_t num_seqs,
                                     const int32_t* cu_seqlens, uint32_t flags) {
  g_last_error.clear();
  Problem p;
  p.kda = true;
  if (check_shape(B, T, H, K, V, num_seqs, cu_seqlens, p)) return 0;
  if (flags & ~kKnownFlags) {
    fail(GDN_ERR_INVALID_ARGUMENT, "unknown flag bits 0x%x", flags & ~kKnownFlags);
    return 0;
  }
  return kda_bwd_layout_for(p).total;
}

static int kda_bwd_impl(const void* q, const void* k, const void* v, const float* g, const void* beta,
                        const float* initial_state, const int32_t* cu_seqlens, int32_t num_seqs, int32_t B,
                        int32_t T, int32_t H, int32_t K, int32_t V, float scale, uint32_t flags, const void* d_o,
                        const float* d_final_state, float* dq, float* dk, float* dv, float* dg, float* dbeta,
                        float* d_initial_state, void* workspace, size_t workspace_bytes, void* stream_ptr,
                        bool gated, const float* a_log, const float* dt_bias, float* da_log, float* ddt_bias) {
  g_last_error.clear();
  Problem p;
  p.kda = true;
  int rc = check_shape(B, T, H, K, V, num_seqs, cu_seqlens, p);
  if (rc) return rc;
  rc = check_common(q, k, v, g, beta, scale, flags);
  if (rc) return rc;
  if (!d_o || !dq || !dk || !dv || !dg || !dbeta)
    return fail(GDN_ERR_INVALID_ARGUMENT, "d_o, dq, dk, dv, dg and dbeta must be non-NULL");
  if (!aligned16(d_o) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(dg) || !aligned16(g))
    return fail(GDN_ERR_INVALID_ARGUMENT, "g, d_o, dq, dk, dv and dg must be 16-byte aligned");
  if (gated) {
    if (!a_log || !dt_bias || !da_log || !ddt_bias)
      return fail(GDN_ERR_INVALID_ARGUMENT, "A_log, dt_bias, dA_log and ddt_bias must be non-NULL");
    if (!aligned16(dt_bias)) return fail(GDN_ERR_INVALID_ARGUMENT, "dt_bias must be 16-byte aligned");
  }
  int cus = 0;
  rc = check_device(&cus);
  if (rc) return rc;

  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const KdaBwdLayout L = kda_bwd_layout_for(p);
  Workspace W;
  rc = acquire_workspace(workspace, workspace_bytes, L.total, stream, W);
  if (rc) return rc;
  if (p.packed) {
    rc = upload_tables(p, W.base + L.b.fwd.tab, stream);
    if (rc) return rc;
  }
  const gdn::Geometry geo = make_geometry(p, W.base + L.b.fwd.tab);
  auto ws = [&](size_t off) { return reinterpret_cast<float*>(W.base + off); };

  // forward recompute: T, Aqk, row vectors, cumulative gate; states and v_new
  gdn::PrepareArgs pa{};
  pa.q = static_cast<const uint16_t*>(q);
  pa.k = static_cast<const uint16_t*>(k);
  pa.g = g;
  pa.beta = static_cast<const uint16_t*>(beta);
  pa.tmat = reinterpret_cast<uint16_t*>(W.base + L.b.fwd.tmat);
  pa.aqk = reinterpret_cast<uint16_t*>(W.base + L.b.fwd.aqk);
  pa.vec = ws(L.b.fwd.vec);
  pa.gk = ws(L.b.fwd.kdec);
  pa.kdec = nullptr;
  pa.a_log = gated ? a_log : nullptr;
  pa.dt_bias = gated ? dt_bias : nullptr;
  pa.geo = geo;
  pa.H = H;
  pa.scale = scale;
  pa.flags = flags & ~(uint32_t)GDN_OUTPUT_FINAL_STATE;
  pa.cus = cus;
  hipError_t e = gdn::launch_prepare(true, pa, stream);
  if (e != hipSuccess) return hip_fail(e, "prepare launch");
  gdn::FwdArgs fa{};
  fa.k = pa.k;
  fa.v = static_cast<const uint16_t*>(v);
  fa.tmat = pa.tmat;
  fa.aqk = pa.aqk;
  fa.vec = pa.vec;
  fa.gk = pa.gk;
  fa.s0 = initial_state;
  fa.h_out = ws(L.b.h);
  fa.vnew_out = ws(L.b.vnew);
  fa.geo = geo;
  fa.H = H;
  e = gdn::launch_fwd(true, true, false, fa, stream);
  if (e != hipSuccess) return hip_fail(e, "forward recompute launch");

  // reverse state pass
  gdn::KdaBwdArgs ka{};
  ka.q = pa.q;
  ka.k = pa.k;
  ka.v = fa.v;
  ka.dout = static_cast<const uint16_t*>(d_o);
  ka.gk = pa.gk;
  ka.vec = pa.vec;
  ka.tmat = pa.tmat;
  ka.aqk = pa.aqk;
  ka.dsfinal = d_final_state;
  ka.dhn = ws(L.b.dhn);
  ka.dvn = ws(L.b.dvn);
  ka.ds0 = d_initial_state;
  ka.h = fa.h_out;
  ka.vnew = fa.vnew_out;
  ka.efd = ws(L.b.efd);
  ka.dp = ws(L.dp);
  ka.da = ws(L.da);
  ka.dkd = ws(L.dkd);
  ka.db1 = ws(L.db1);
  ka.dq = dq;
  ka.dk = dk;
  ka.dv = dv;
  ka.dg = dg;
  ka.dbeta = dbeta;
  ka.scale = scale;
  ka.flags = flags;
  ka.geo = geo;
  ka.H = H;
  e = gdn::launch_kda_bwd_dh(ka, stream);
  if (e != hipSuccess) return hip_fail(e, "reverse state pass launch");

  // products with the saved states (the gate does not enter them)
  gdn::BwdArgs ba{};
  ba.dout = ka.dout;
  ba.h = fa.h_out;
  ba.vnew = fa.vnew_out;
  ba.dhn = ka.dhn;
  ba.dvn = ka.dvn;
  ba.efd = ws(L.b.efd);
  ba.sdot = ws(L.b.sdot);
  ba.geo = geo;
  ba.H = H;
  ba.cus = cus;
  e = gdn::launch_gdn_bwd(ba, 1, stream);
  if (e != hipSuccess) return hip_fail(e, "state products launch");

  e = gdn::launch_kda_bwd_chunks(ka, stream);
  if (e != hipSuccess) return hip_fail(e, "per-chunk gradients launch");
  if (gated) {
    gdn::KdaGateBwdArgs ga{};
    ga.x = g;
    ga.a_log = a_log;
    ga.dt_bias = dt_bias;
    ga.dg = dg;
    ga.part = ws(L.kgpart);
    ga.da_log = da_log;
    ga.ddt_bias = ddt_bias;
    ga.ntok = (long)B * T;
    ga.H = H;
    ga.nblk = L.kgate_blocks;
    e = gdn::launch_kda_gate_bwd(ga, stream);
    if (e != hipSuccess) return hip_fail(e, "gate backward launch");
  }
  return GDN_OK;
}

int kda_chunk_bwd(const void* q, const void* k, const void* v, const float* g, const void* beta,
                  const float* initial_state, const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T,
                  int32_t H, int32_t K, int32_t V, float scale, uint32_t flags, const void* d_o,
                  const float* d_final_state, float* dq, float* dk, float* dv, float* dg, float* dbeta,
                  float* d_initial_state, void* workspace, size_t workspace_bytes, void* stream_ptr) {
  return kda_bwd_impl(q, k, v, g, beta, initial_state, cu_seqlens, num_seqs, B, T, H, K, V, scale, flags, d_o,
                      d_final_state, dq, dk, dv, dg, dbeta, d_initial_state, workspace, workspace_bytes, stream_ptr,
                      false, nullptr, nullptr, nullptr, nullptr);
}

int kda_chunk_bwd_gated(const void* q, const void* k, const void* v, const float* g_raw, const float* A_log,
                        const float* dt_bias, const void* beta, const float* initial_state,
                        const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t K,
                        int32_t V, float scale, uint32_t flags, const void* d_o, const float* d_final_state,
                        float* dq, float* dk, float* dv, float* dg_raw, float* dA_log, float* ddt_bias,
                        float* dbeta, float* d_initial_state, void* workspace, size_t workspace_bytes,
                        void* stream) {
  return kda_bwd_impl(q, k, v, g_raw, beta, initial_state, cu_seqlens, num_seqs, B, T, H, K, V, scale, flags, d_o,
                      d_final_state, dq, dk, dv, dg_raw, dbeta, d_initial_state, workspace, workspace_bytes, stream,
                      true, A_log, dt_bias, dA_log, ddt_bias);
}

size_t kda_bwd_state_pass_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V, int32_t num_seqs,
                                          const int32_t* cu_seqlens, uint32_t flags) {
  g_last_error.clear();
  Problem p;
  p.kda = true;
  if (check_shape(B, T, H, K, V, num_seqs, cu_seqlens, p)) return 0;
  if (flags & ~kKnownFlags) {
    fail(GDN_ERR_INVALID_ARGUMENT, "unknown flag bits 0x%x", flags & ~kKnownFlags);
    return 0;
  }
  return layout_for(p, true, true).total;
}

int kda_bwd_state_pass(const void* q, const void* k, const float* g, const void* beta, const int32_t* cu_seqlens,
                       int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t K, int32_t V, float scale,
                       uint32_t flags, const void* d_o, const float* d_final_state, float* dh_next, float* dv_new,
                       float* d_initial_state, void* workspace, size_t workspace_bytes, void* stream_ptr) {
  g_last_error.clear();
  Problem p;
  p.kda = true;
  int rc = check_shape(B, T, H, K, V, num_seqs, cu_seqlens, p);
  if (rc) return rc;
  rc = check_common(q, k, k, g, beta, scale, flags);
  if (rc) return rc;
  if (!d_o || !dh_next || !dv_new)
    return fail(GDN_ERR_INVALID_ARGUMENT, "d_o, dh_next and dv_new must be non-NULL");
  if (!aligned16(dv_new)) return fail(GDN_ERR_INVALID_ARGUMENT, "dv_new must be 16-byte aligned");
  int cus = 0;
  rc = check_device(&cus);
  if (rc) return rc;

  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const Layout L = layout_for(p, true, true);
  Workspace W;
  rc = acquire_workspace(workspace, workspace_bytes, L.total, stream, W);
  if (rc) return rc;
  if (p.packed) {
    rc = upload_tables(p, W.base + L.tab, stream);
    if (rc) return rc;
  }
  const gdn::Geometry geo = make_geometry(p, W.base + L.tab);

  gdn::PrepareArgs pa{};
  pa.q = static_cast<const uint16_t*>(q);
  pa.k = static_cast<const uint16_t*>(k);
  pa.g = g;
  pa.beta = static_cast<const uint16_t*>(beta);
  pa.tmat = reinterpret_cast<uint16_t*>(W.base + L.tmat);
  pa.aqk = reinterpret_cast<uint16_t*>(W.base + L.aqk);
  pa.vec = reinterpret_cast<float*>(W.base + L.vec);
  pa.gk = reinterpret_cast<float*>(W.base + L.kdec);
  pa.kdec = nullptr;
  pa.geo = geo;
  pa.H = H;
  pa.scale = scale;
  pa.flags = flags & ~(uint32_t)GDN_OUTPUT_FINAL_STATE;
  pa.cus = cus;
  hipError_t e = gdn::launch_prepare(true, pa, stream);
  if (e != hipSuccess) return hip_fail(e, "prepare launch");

  gdn::KdaBwdArgs ka{};
  ka.q = pa.q;
  ka.k = pa.k;
  ka.dout = static_cast<const uint16_t*>(d_o);
  ka.gk = pa.gk;
  ka.vec = pa.vec;
  ka.tmat = pa.tmat;
  ka.aqk = pa.aqk;
  ka.dsfinal = d_final_state;
  ka.dhn = dh_next;
  ka.dvn = dv_new;
  ka.ds0 = d_initial_state;
  ka.geo = geo;
  ka.H = H;
  e = gdn::launch_kda_bwd_dh(ka, stream);
  if (e != hipSuccess) return hip_fail(e, "reverse state pass launch");
  return GDN_OK;
}

int gdn_stage_fwd_h(int32_t kda, const void* k, const void* v, const void* tmat, const float* vec, const float* gk,
                    const float* initial_state, const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T,
                    int32_t H, int32_t K, int32_t V, uint32_t flags, float* h, float* v_new, float* final_state,
                    void* stream_ptr) {
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  g_last_error.clear();
  if (!k || !v || !tmat || !vec || !h || !v_new || (kda && !gk))
    return fail(GDN_ERR_INVALID_ARGUMENT, "k, v, tmat, vec, h, v_new (and gk for KDA) must be non-NULL");
  if (!aligned16(k) || !aligned16(v)) return fail(GDN_ERR_INVALID_ARGUMENT, "k and v must be 16-byte aligned");
  if (flags & ~kKnownFlags) return fail(GDN_ERR_INVALID_ARGUMENT, "unknown flag bits 0x%x", flags & ~kKnownFlags);
  if ((flags & GDN_OUTPUT_FINAL_STATE) && !final_state)
    return fail(GDN_ERR_INVALID_ARGUMENT, "GDN_OUTPUT_FINAL_STATE set but final_state is NULL");
  StageCtx ctx;
  int rc = stage_begin(kda, cu_seqlens, num_seqs, B, T, H, K, V, stream, ctx);
  if (rc) return rc;
  gdn::FwdArgs fa{};
  fa.k = static_cast<const uint16_t*>(k);
  fa.v = static_cast<const uint16_t*>(v);
  fa.tmat = static_cast<const uint16_t*>(tmat);
  fa.vec = vec;
  fa.gk = gk;
  fa.s0 = initial_state;
  fa.sfinal = (flags & GDN_OUTPUT_FINAL_STATE) ? final_state : nullptr;
  fa.h_out = h;
  fa.vnew_out = v_new;
  fa.geo = ctx.geo;
  fa.H = H;
  hipError_t e = gdn::launch_fwd(kda != 0, true, false, fa, stream);
  if (e != hipSuccess) return hip_fail(e, "chunk_fwd_h launch");
  return GDN_OK;
}

int gdn_stage_finalize(int32_t kda, const void* q, const void* aqk, const float* vec, const float* gk, const float* h,
                       const float* v_new, const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T,
                       int32_t H, int32_t K, int32_t V, void* o, void* stream_ptr) {
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  g_last_error.clear();
  if (!q || !aqk || !vec || !h || !v_new || !o || (kda && !gk))
    return fail(GDN_ERR_INVALID_ARGUMENT, "q, aqk, vec, h, v_new, o (and gk for KDA) must be non-NULL");
  if (!aligned16(q) || !aligned16(o)) return fail(GDN_ERR_INVALID_ARGUMENT, "q and o must be 16-byte aligned");
  StageCtx ctx;
  int rc = stage_begin(kda, cu_seqlens, num_seqs, B, T, H, K, V, stream, ctx);
  if (rc) return rc;
  gdn::FinArgs fa{};
  fa.q = static_cast<const uint16_t*>(q);
  fa.aqk = static_cast<const uint16_t*>(aqk);
  fa.vec = vec;
  fa.gk = gk;
  fa.h = h;
  fa.vnew = v_new;
  fa.o = static_cast<uint16_t*>(o);
  fa.geo = ctx.geo;
  fa.H = H;
  hipError_t e = gdn::launch_finalize(kda != 0, fa, stream);
  if (e != hipSuccess) return hip_fail(e, "finalize launch");
  return GDN_OK;
}

}  // extern "C"
