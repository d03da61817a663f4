// Device helpers shared by the HIP sources of libkvcache (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "kvc_internal.h"

namespace kvc {
namespace dev {

using bf16_t = uint16_t;

// ------------------------------------------------------------ conversions --

__device__ __forceinline__ float bf16_to_f32(bf16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Round-to-nearest-even float -> bfloat16, a NaN staying a NaN (gfx950
// converts two values per v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

template <typename T> struct Acc;
template <> struct Acc<double> { using type = double; };
template <> struct Acc<float> { using type = float; };
template <> struct Acc<bf16_t> { using type = float; };

template <typename A> __device__ __forceinline__ A to_acc(double v) { return A(v); }
template <typename A> __device__ __forceinline__ A to_acc(float v) { return A(v); }
template <typename A> __device__ __forceinline__ A to_acc(bf16_t v) { return A(bf16_to_f32(v)); }

template <typename T> __device__ __forceinline__ T from_acc(typename Acc<T>::type v);
template <> __device__ __forceinline__ double from_acc<double>(double v) { return v; }
template <> __device__ __forceinline__ float from_acc<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_acc<bf16_t>(float v) { return f32_to_bf16(v); }

__device__ __forceinline__ bool finite(double v) { return isfinite(v); }
__device__ __forceinline__ bool finite(float v) { return isfinite(v); }

__device__ __forceinline__ double fast_exp(double v) { return exp(v); }
__device__ __forceinline__ float fast_exp(float v) { return expf(v); }

// ------------------------------------------------------- vector row loads --

template <int BYTES> struct Raw;
template <> struct Raw<16> { using type = uint4; };
template <> struct Raw<8> { using type = uint2; };
template <> struct Raw<4> { using type = uint32_t; };
template <> struct Raw<2> { using type = uint16_t; };

// Loads VEC consecutive elements (VEC * sizeof(T) bytes, naturally aligned)
// and widens them to the accumulate type.
template <typename T, int VEC>
__device__ __forceinline__ void load_row_chunk(const T* __restrict__ p, typename Acc<T>::type (&out)[VEC]) {
  using R = typename Raw<VEC * sizeof(T)>::type;
  union {
    R raw;
    T e[VEC];
  } u;
  u.raw = *reinterpret_cast<const R*>(p);
#pragma unroll
  for (int i = 0; i < VEC; ++i) out[i] = to_acc<typename Acc<T>::type>(u.e[i]);
}

// Lane geometry of a row of DH elements of T: each lane reads one chunk of up
// to 16 bytes; G lanes cover a row; a wavefront of 64 covers RPW rows.
template <typename T, int DH>
struct RowGeo {
  static constexpr int VEC = (DH * int(sizeof(T)) >= 16) ? 16 / int(sizeof(T)) : DH;
  static constexpr int G = DH / VEC;
  static constexpr int RPW = 64 / G;
  static_assert(G >= 1 && G <= 64 && (G & (G - 1)) == 0, "unsupported head width");
};

template <int G, typename A>
__device__ __forceinline__ A group_sum(A v) {
#pragma unroll
  for (int off = G / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ void flag_min(unsigned long long* word, unsigned long long idx) {
  atomicMin(word, idx);
}

__device__ __forceinline__ bool any_error(const ErrWords* e) {
  return (e->key & e->value & e->query & e->position & e->output & e->token) != kErrClear;
}

// Element offset of row r of key/value lane (b, h), h < H_kv, in the K or V
// storage (contiguous [B, H_kv, C, d_h], or the block pool through the
// sequence's block table).
__device__ __forceinline__ size_t kv_offset(const DevState& s, int b, int h, int r) {
  const int dh = s.head_width;
  if (s.ring) return ((size_t(b) * s.kv_heads + h) * s.capacity + r % s.capacity) * dh;
  if (!s.paged) return ((size_t(b) * s.kv_heads + h) * s.capacity + r) * dh;
  const int lg = s.block_rows_log2;
  const int blk = s.block_table[size_t(b) * s.table_width + (r >> lg)];
  return (((size_t(blk) * s.kv_heads + h) << lg) + (r & ((1 << lg) - 1))) * dh;
}

// Element offset that row r0's block would have at row 0 of the same block:
// adding r * d_h addresses any row r of that block (paged), or of the lane
// (contiguous).  Used where a run of rows is known to lie in one block.
__device__ __forceinline__ ptrdiff_t kv_block_base(const DevState& s, int b, int h, int r0) {
  const int dh = s.head_width;
  // a ring's runs never cross a multiple of the capacity (a multiple of kMinBlockRows)
  if (s.ring) return ptrdiff_t((size_t(b) * s.kv_heads + h) * s.capacity) * dh - ptrdiff_t(r0 - r0 % s.capacity) * dh;
  if (!s.paged) return ptrdiff_t((size_t(b) * s.kv_heads + h) * s.capacity) * dh;
  const int lg = s.block_rows_log2;
  // an unassigned block (-1) is only reached by callers that read no cache row
  const int blk = max(s.block_table[size_t(b) * s.table_width + (r0 >> lg)], 0);
  return (ptrdiff_t(size_t(blk) * s.kv_heads + h) << lg) * dh - ptrdiff_t((r0 >> lg) << lg) * dh;
}

// Slot of row r in the per-sequence position table [B, C].
__device__ __forceinline__ int pos_slot(const DevState& s, int r) { return s.ring ? r % s.capacity : r; }

// First row a query at row r reads (sliding window), else 0.
__device__ __forceinline__ int window_start(const DevState& s, int r) {
  return s.window ? max(0, r - s.window + 1) : 0;
}

// The candidate row index (= committed rows) of sequence b in a decode call,
// clamped to what the storage can address.
__device__ __forceinline__ int decode_len(const DevState& s, int b) {
  const int len = max(s.len[b], 0);
  return s.ring ? len : min(len, s.capacity - 1);
}

// Rows a decode query at row len reads, [rs, len], in split-K tiles of
// tile_rows starting at base0 (rs rounded down to kDecodeTileRows).
struct DecodeSpan {
  int rs, base0, ntiles;
};
__device__ __forceinline__ DecodeSpan decode_span(const DevState& s, int len) {
  DecodeSpan d;
  d.rs = window_start(s, len);
  d.base0 = d.rs - d.rs % kDecodeTileRows;
  d.ntiles = (len + 1 - d.base0 + s.tile_rows - 1) / s.tile_rows;
  return d;
}

// True when a failure word of the cache's gate (its own words, or every layer
// of its session) is set: state-changing kernels then do nothing.
__device__ __forceinline__ bool gate_closed(const DevState& s) {
  for (int k = 0; k < s.gate_count; ++k)
    if (any_error(&s.gate[k])) return true;
  return false;
}



// ------------------------------------------------------------------ MFMA --
// Operand layouts of the gfx950 bf16 MFMAs used here (checked on the device):
//  32x32x16: A lane l = row l%32, k 8*(l/32)+e;  B lane l = k 8*(l/32)+e, col l%32;
//            C register r = row 8*(r/4)+4*(l/32)+(r%4), col l%32.
//  16x16x32: A lane l = row l%16, k 8*(l/16)+e;  B lane l = k 8*(l/16)+e, col l%16;
//            C register r = row 4*(l/16)+r, col l%16.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

union Frag8 {
  uint4 u;
  bf16x8_t v;
  bf16_t h[8];
};

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

}  // namespace dev
}  // namespace kvc
