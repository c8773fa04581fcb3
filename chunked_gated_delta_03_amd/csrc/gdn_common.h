// Device-side helpers shared by the gfx950 kernels of the chunked
// gated-delta-rule forward pass: bf16 packing, MFMA wrappers, chunk geometry.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

constexpr int kChunk = 64;   // tokens per chunk
constexpr int kDim = 128;    // K == V
constexpr int kVecRows = 8;  // per-chunk vectors written by prepare

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint16_t u16x4;
typedef __attribute__((ext_vector_type(8))) uint16_t u16x8;

// ---- bf16 <-> fp32 -------------------------------------------------------
__device__ __forceinline__ float bf2f(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
// Round to nearest even. Inputs here are finite.
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
// hi = bf16(x), lo = bf16(x - hi): hi + lo carries ~16 significant bits.
__device__ __forceinline__ void split_bf(float x, uint16_t& hi, uint16_t& lo) {
  hi = f2bf(x);
  lo = f2bf(x - bf2f(hi));
}

// 2^x on v_exp_f32 alone. The library exp2f adds a range reduction and an
// ldexp (about seven instructions) to keep results below 2^-126 as
// denormals; the decays here only scale bf16 operands and states, where a
// factor below 2^-126 and zero are the same for every result. Results for
// normal outputs agree with exp2f to about one ulp.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- in-kernel gate --------------------------------------------------------
// softplus(y) / ln 2 = log2(1 + e^y) = max(y, 0) log2(e) + log2(1 + u) with
// u = e^-|y| in (0, 1]. log2(1 + u) by Goldberg's correction of the rounded
// sum ("What every computer scientist should know about floating-point
// arithmetic", Theorem 4): w = 1 + u, log2(1 + u) = log2(w) u / (w - 1), or
// u log2(e) when w rounds to 1 (w - 1 is exact). v_exp_f32, v_log_f32 and
// v_rcp_f32 directly: w is in [1, 2], so no denormal handling is needed, and
// a u that underflows gives l = 0. Relative error below 4e-6 for y > -80
// (most of it from rounding |y| log2(e) ahead of the exponential when |y|
// is large, where softplus(y) is below e^-10), a few ulp near y = 0.
__device__ __forceinline__ float softplus_log2(float y) {
  constexpr float kLog2e = 1.4426950408889634f;
  const float u = __builtin_amdgcn_exp2f(-fabsf(y) * kLog2e);
  const float w = 1.0f + u;
  const float d = w - 1.0f;
  const float l = (d == 0.0f) ? u * kLog2e : __builtin_amdgcn_logf(w) * (u * __builtin_amdgcn_rcpf(d));
  return fmaxf(y, 0.0f) * kLog2e + l;
}
// Gate from the raw per-token value x and the head's parameters:
// -exp(A_log) softplus(x + dt_bias), in log2 units (KDA) ...
__device__ __forceinline__ float gate_log2(float x, float exp_a_log, float dt_bias) {
  return -exp_a_log * softplus_log2(x + dt_bias);
}
// ... or in natural-log units (GDN).
__device__ __forceinline__ float gate_ln(float x, float exp_a_log, float dt_bias) {
  return -exp_a_log * 0.6931471805599453f * softplus_log2(x + dt_bias);
}

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// Two floats to one packed pair of bf16 (round to nearest even).
__device__ __forceinline__ uint32_t pack2(float x0, float x1) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x0, x1}, bf16x2));
}

// Two floats to packed bf16 hi and lo words: hi = bf16(x), lo = bf16(x - hi).
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  const uint32_t hp = pack2(x0, x1);
  const float h0 = __uint_as_float(hp << 16);
  const float h1 = __uint_as_float(hp & 0xFFFF0000u);
  hi = hp;
  lo = pack2(x0 - h0, x1 - h1);
}

// ---- permuted contraction columns ---------------------------------------------
// An MFMA 16x16x32 contraction step s takes, in lane group g (= lane / 16),
// contraction indices 32s + 4g + (0..3) and 32s + 16 + 4g + (0..3): the
// accumulator rows that a B operand built from two accumulator tiles holds.
// Matrices used as A operands against such B operands store their columns
// permuted so that these eight indices are adjacent (one 16-byte read):
//   column 32s + 16h + 4g + e  ->  position 32s + 8g + 4h + e.
__device__ __forceinline__ int perm_col(int c) {
  return (c & ~31) | ((c & 12) << 1) | ((c & 16) >> 2) | (c & 3);
}
// inverse: the column stored at position p
__device__ __forceinline__ int unperm_col(int p) {
  return (p & ~31) | ((p & 4) << 2) | ((p & 24) >> 1) | (p & 3);
}

// ---- MFMA ------------------------------------------------------------------
// v_mfma_f32_16x16x32_bf16, wave64. Lane l: A row (l % 16), B column (l % 16),
// both holding contraction slots 8*(l/16) .. 8*(l/16)+7; D column (l % 16),
// rows 4*(l/16) .. 4*(l/16)+3. Only the pairing of slots between A and B
// matters, so callers may map slots to any contraction indices as long as A
// and B agree.
__device__ __forceinline__ f32x4 mfma16(const u16x8& a, const u16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ u16x8 cat4(const u16x4& a, const u16x4& b) {
  return u16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// ---- chunk geometry ----------------------------------------------------------
// A chunk is at most 64 consecutive tokens of one sequence. Dense input:
// sequence n is batch row n and chunk j of it starts at token n*T + 64*j.
// Packed input: tables built on the host from cu_seqlens.
struct ChunkInfo {
  int tok0;  // first token (flat index into the [B*T] token axis)
  int len;   // valid rows, 1..64
  int seq;   // sequence index n
  int j;     // chunk index inside the sequence
};
struct SeqInfo {
  int tok0;
  int len;
  int c0;    // global index of the sequence's first chunk
  int nch;   // chunks in the sequence
};

struct Geometry {
  const int4* ctab;  // [NT] {tok0, len, seq, j} or nullptr (dense)
  const int4* stab;  // [N]  {tok0, len, c0, nch} or nullptr (dense)
  const int* sorder; // [N]  sequences by decreasing chunk count, or nullptr (dense: in order)
  int T;             // dense sequence length
  int ncb;           // dense chunks per sequence = ceil(T/64)
  int NT;            // total chunks
  int N;             // sequences

  // The tables are read-only for a kernel's lifetime: they are read through
  // the constant address space (scalar loads when the index is uniform, which
  // do not count against the vector-memory counter).
  __device__ __forceinline__ ChunkInfo chunk(int c) const {
    ChunkInfo ci;
    if (ctab) {
      const __attribute__((address_space(4))) int* e = (const __attribute__((address_space(4))) int*)ctab + 4 * c;
      ci.tok0 = e[0]; ci.len = e[1]; ci.seq = e[2]; ci.j = e[3];
    } else {
      int n = c / ncb, j = c - n * ncb;
      ci.seq = n; ci.j = j;
      ci.tok0 = n * T + j * kChunk;
      int rem = T - j * kChunk;
      ci.len = rem < kChunk ? rem : kChunk;
    }
    return ci;
  }
  __device__ __forceinline__ SeqInfo seq(int n) const {
    SeqInfo si;
    if (stab) {
      const __attribute__((address_space(4))) int* e = (const __attribute__((address_space(4))) int*)stab + 4 * n;
      si.tok0 = e[0]; si.len = e[1]; si.c0 = e[2]; si.nch = e[3];
    } else {
      si.tok0 = n * T; si.len = T; si.c0 = n * ncb; si.nch = ncb;
    }
    return si;
  }
  // sequence of rank r in the launch order
  __device__ __forceinline__ int seq_of_rank(int r) const {
    return sorder ? ((const __attribute__((address_space(4))) int*)sorder)[r] : r;
  }
};

// Workgroup -> (sequence, head, V-block) of the sequential state kernels,
// for a 1-D grid of ceil(N H / 8) * 8 * VB workgroups. Units (sequence,
// head) are taken in the order of geo.sorder (longest sequences first, so
// that the long ones start in the first dispatch round); the VB blocks of a
// unit get workgroup ids i, i + 8, i + 16, ..., which the dispatcher places
// on the same XCD (ids go round-robin over the 8 XCDs), so they share that
// XCD's L2 for the unit's k, q, T, Aqk rows. Returns false for the padding
// workgroups past the last unit.
__device__ __forceinline__ bool state_unit(const Geometry& geo, int H, int VB, int& n, int& h, int& vb) {
  const int i = blockIdx.x;
  const int uidx = (i / (8 * VB)) * 8 + (i & 7);
  vb = (i >> 3) % VB;
  if (uidx >= geo.N * H) return false;
  const int r = uidx / H;
  h = uidx - r * H;
  n = geo.seq_of_rank(r);
  return true;
}
__host__ inline unsigned state_grid(int N, int H, int VB) { return (unsigned)(((N * H + 7) / 8) * 8 * VB); }

}  // namespace gdn
