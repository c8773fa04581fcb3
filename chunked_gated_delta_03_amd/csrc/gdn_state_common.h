// Helpers shared by the state kernels: the transposing LDS read and bf16
// hi/lo splits of accumulator tiles.
#pragma once

#include "gdn_kernels.h"

namespace gdn {
namespace st {

// ds_read_b64_tr_b16: in each 16-lane group, lane i receives element (i % 4)
// of the 8-byte chunks read by lanes 4j + i/4, j = 0..3 (measured on gfx950).
__device__ __forceinline__ u16x4 tr_read(const uint16_t* p) {
  typedef __attribute__((ext_vector_type(4))) short s4;
  s4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(p));
  return __builtin_bit_cast(u16x4, r);
}


// Slot swizzle of the k (and q) rows: piece p of row r sits at slot
// p ^ kswz(r). Besides the 16-row fragment reads (any bijection of r & 15
// keeps those on distinct banks), the k rows are read transposed for the
// update: 16 lanes read the first 8 bytes of pieces P + j of rows x + i
// (i, j = 0..3, P and x multiples of 4). With p ^ (r & 15) those land in
// only 4 distinct slots (4 lanes per bank); folding the row's low bits into
// the slot's high bits spreads them over 16.
__device__ __forceinline__ int kswz(int r) { return (r & 15) ^ ((r & 3) << 2); }

// Slot swizzle of 32-column v rows (64 bytes, four 16-byte pieces): rows
// 4..7 of each group of 8 swap their halves, so that the transposing reads of
// lane groups 0 and 1 (rows 4 g4 + j) fall on different banks.
template <int BV>
__device__ __forceinline__ int vswz(int r) { return BV == 32 ? ((r >> 2) & 1) << 1 : 0; }

__device__ __forceinline__ uint16_t bfr(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

// B operand (8 contraction slots) from two accumulator tiles: slots 0..3 are
// rows 4g..4g+3 of tile a, slots 4..7 the same rows of tile b.
__device__ __forceinline__ void split_tiles(const f32x4& a, const f32x4& b, u16x8& hi, u16x8& lo) {
  uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
  split2(a[0], a[1], h0, l0);
  split2(a[2], a[3], h1, l1);
  split2(b[0], b[1], h2, l2);
  split2(b[2], b[3], h3, l3);
  hi = __builtin_bit_cast(u16x8, u32x4{h0, h1, h2, h3});
  lo = __builtin_bit_cast(u16x8, u32x4{l0, l1, l2, l3});
}

__device__ __forceinline__ u16x8 pack_tiles(const f32x4& a, const f32x4& b) {
  return __builtin_bit_cast(u16x8, u32x4{pack2(a[0], a[1]), pack2(a[2], a[3]), pack2(b[0], b[1]), pack2(b[2], b[3])});
}

}  // namespace st
}  // namespace gdn
