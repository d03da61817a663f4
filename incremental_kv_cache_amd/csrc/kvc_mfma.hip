// bf16 matrix-core (MFMA) kernels of libkvcache for gfx950.
//
//  * project_skinny : the new rows (decode: M = B rows) through W_q, W_k, W_v.
//                     A [M, D] x [D, 3D] contraction whose time is the weight
//                     read from HBM; a workgroup owns a 32-row x 32-pair output
//                     tile, streams its 64 weight rows once and shares each
//                     input chunk between its four waves through LDS.
//  * project_tiled  : the same contraction for many rows (chunks, prefill):
//                     128 x 128 tiles staged through LDS, 2 x 2 waves.
//  * attend_flash   : causal chunk attention (prefix-reuse note: suffix row i
//                     reads the retained rows plus chunk rows 0..i) with the
//                     score and value contractions on MFMA and an online
//                     softmax in between.
//
// Rotary pairs: output columns are ordered so that feature f and f + d_h/2 of a
// head land in the same thread (tiled) or the same LDS row (skinny), so the
// rotation at position next_position + i is applied in the epilogue.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "kvc_dev_util.h"
#include "kvc_internal.h"

namespace kvc {

namespace {

using namespace dev;

__device__ __forceinline__ const bf16_t* weight_of(const DevState& s, int p) {
  return static_cast<const bf16_t*>(p == 0 ? s.wq : (p == 1 ? s.wk : (p == 2 ? s.wv : s.wo)));
}

// Heads of projection p: W_k and W_v may project to fewer (grouped) heads.
__device__ __forceinline__ int heads_of(const DevState& s, int p) { return (p == 1 || p == 2) ? s.kv_heads : s.heads; }

// Column tile t (tiles of `cols` output columns) of a launch over projections
// proj_first, proj_first + 1, ...: returns the projection and leaves in t the
// tile's index within it.
__device__ __forceinline__ int tile_proj(const DevState& s, int proj_first, int cols, int& t) {
  int p = proj_first;
  while (p < 3) {
    const int n = heads_of(s, p) * s.head_width / cols;
    if (t < n) break;
    t -= n;
    ++p;
  }
  return p;
}

// 16 input elements starting at p as two bf16x8 pieces (float input is rounded).
__device__ __forceinline__ void load16(const bf16_t* p, uint4& lo, uint4& hi) {
  lo = reinterpret_cast<const uint4*>(p)[0];
  hi = reinterpret_cast<const uint4*>(p)[1];
}
__device__ __forceinline__ uint4 pack8(const float4& a, const float4& b) {
  Frag8 f;
  f.v[0] = (__bf16)a.x;
  f.v[1] = (__bf16)a.y;
  f.v[2] = (__bf16)a.z;
  f.v[3] = (__bf16)a.w;
  f.v[4] = (__bf16)b.x;
  f.v[5] = (__bf16)b.y;
  f.v[6] = (__bf16)b.z;
  f.v[7] = (__bf16)b.w;
  return f.u;
}
__device__ __forceinline__ void load16(const float* p, uint4& lo, uint4& hi) {
  const float4* q = reinterpret_cast<const float4*>(p);
  lo = pack8(q[0], q[1]);
  hi = pack8(q[2], q[3]);
}

// Where output row m of a call lands: sequence b, chunk row i (i < 0: past M
// or past the sequence's rows, nothing stored) and, for rotated projections,
// the rotary position next_position + i.  A position past the rotary table is
// recorded in bad_pos (smallest sequence index) and rotates as position 0.
struct RowDst {
  int b, i, pos;
};
__device__ __forceinline__ RowDst row_dst(const DevState& s, int p, int m, int M, int n_max, int per_seq_rows,
                                          unsigned long long& bad_pos) {
  RowDst d{0, -1, 0};
  if (m >= M) return d;
  d.b = m / n_max;
  const int i = m - d.b * n_max;
  const int n_b = per_seq_rows ? s.rows[d.b] : n_max;
  if (i >= n_b) return d;
  d.i = i;
  if (p < 2 && s.rope) {
    d.pos = s.next_pos[d.b] + i;
    if (d.pos < 0 || d.pos >= s.max_positions) {
      bad_pos = min(bad_pos, (unsigned long long)d.b);
      d.pos = 0;
    }
  }
  return d;
}

// Rotates (if needed) and stores rotary pair `pair` (global pair index within
// projection p: head pair / half, feature pair % half) of a row; the smallest
// flat index of a non-finite stored value goes to `bad`.
__device__ __forceinline__ void put_pair(const DevState& s, int p, const RowDst& d, int pair, float lo, float hi,
                                         int n_max, unsigned long long& bad) {
  if (d.i < 0) return;
  const int dh = s.head_width;
  const int half = dh >> 1;
  const int h = pair / half;
  const int f = pair - h * half;
  if (p == 3) {  // output projection: plain columns h*d_h + f and + d_h/2 of the row
    const size_t flat = (size_t(d.b) * n_max + d.i) * s.model_width + size_t(h) * dh + f;
    float* o = static_cast<float*>(s.out_proj_dst) + flat;
    o[0] = lo;
    o[half] = hi;
    if (!isfinite(lo)) bad = min(bad, (unsigned long long)flat);
    if (!isfinite(hi)) bad = min(bad, (unsigned long long)(flat + half));
    return;
  }
  float r0 = lo, r1 = hi;
  if (p < 2 && s.rope) {
    const float c = static_cast<const float*>(s.rope_cos)[size_t(d.pos) * half + f];
    const float sn = static_cast<const float*>(s.rope_sin)[size_t(d.pos) * half + f];
    r0 = lo * c - hi * sn;
    r1 = hi * c + lo * sn;
  }
  const size_t flat0 = (size_t(d.b * heads_of(s, p) + h) * n_max + d.i) * dh + f;
  const size_t flat1 = flat0 + half;
  if (p == 0) {
    if (s.q_bf16) {
      const float sl2 = float(s.scale) * 1.4426950408889634f;
      bf16_t* q = static_cast<bf16_t*>(s.q);
      q[flat0] = f32_to_bf16(r0 * sl2);
      q[flat1] = f32_to_bf16(r1 * sl2);
    } else {
      float* q = static_cast<float*>(s.q);
      q[flat0] = r0;
      q[flat1] = r1;
    }
    if (!isfinite(r0)) bad = min(bad, (unsigned long long)flat0);
    if (!isfinite(r1)) bad = min(bad, (unsigned long long)flat1);
  } else {
    bf16_t* dst = static_cast<bf16_t*>(p == 1 ? s.cand_k : s.cand_v);
    const bf16_t t0 = f32_to_bf16(r0), t1 = f32_to_bf16(r1);
    dst[flat0] = t0;
    dst[flat1] = t1;
    if (!isfinite(bf16_to_f32(t0))) bad = min(bad, (unsigned long long)flat0);
    if (!isfinite(bf16_to_f32(t1))) bad = min(bad, (unsigned long long)flat1);
  }
}

// Publishes a thread's recorded failures to the projection's failure words.
__device__ __forceinline__ void flush_bad(const DevState& s, int p, unsigned long long bad,
                                          unsigned long long bad_pos) {
  if (bad_pos != kErrClear) flag_min(&s.err->position, bad_pos);
  if (bad != kErrClear)
    flag_min(p == 0 ? &s.err->query : (p == 1 ? &s.err->key : (p == 2 ? &s.err->value : &s.err->output)), bad);
}

// Rotary factors (cos, sin) of four consecutive pairs of a row, or (1, 0) when
// the projection is not rotated or the row is not stored.  Loaded apart from
// put_pairs4 so that a caller can issue the loads of several rows before any
// of their stores (the compiler may not move a load past a store it cannot
// prove disjoint).
struct Rope4 {
  float4 c, sn;
};
__device__ __forceinline__ Rope4 rope4(const DevState& s, int p, const RowDst& d, int pair0) {
  Rope4 r{make_float4(1.f, 1.f, 1.f, 1.f), make_float4(0.f, 0.f, 0.f, 0.f)};
  if (d.i < 0 || p >= 2 || !s.rope) return r;
  const int half = s.head_width >> 1;
  const int f = pair0 % half;
  r.c = *reinterpret_cast<const float4*>(static_cast<const float*>(s.rope_cos) + size_t(d.pos) * half + f);
  r.sn = *reinterpret_cast<const float4*>(static_cast<const float*>(s.rope_sin) + size_t(d.pos) * half + f);
  return r;
}

// Four consecutive pairs pair0 .. pair0 + 3 of one head (pair0 % 4 == 0 and
// d_h / 2 % 4 == 0): the same as four put_pair calls, with 16-byte (float) or
// 8-byte (bf16) stores, rotated by the factors from rope4.
__device__ __forceinline__ void put_pairs4(const DevState& s, int p, const RowDst& d, int pair0, float4 lo,
                                           float4 hi, const Rope4& rf, int n_max, unsigned long long& bad) {
  if (d.i < 0) return;
  const int dh = s.head_width;
  const int half = dh >> 1;
  const int h = pair0 / half;
  const int f = pair0 - h * half;
  // a non-finite value makes the sum non-finite (a sum that only overflows
  // sends the four values through the exact checks, which then find none)
  auto note = [&](const float4& v, size_t flat) {
    if (isfinite((v.x + v.y) + (v.z + v.w))) return;
    if (!isfinite(v.x)) bad = min(bad, (unsigned long long)flat);
    else if (!isfinite(v.y)) bad = min(bad, (unsigned long long)(flat + 1));
    else if (!isfinite(v.z)) bad = min(bad, (unsigned long long)(flat + 2));
    else if (!isfinite(v.w)) bad = min(bad, (unsigned long long)(flat + 3));
  };
  if (p == 3) {
    const size_t flat = (size_t(d.b) * n_max + d.i) * s.model_width + size_t(h) * dh + f;
    float* o = static_cast<float*>(s.out_proj_dst) + flat;
    *reinterpret_cast<float4*>(o) = lo;
    *reinterpret_cast<float4*>(o + half) = hi;
    note(lo, flat);
    note(hi, flat + half);
    return;
  }
  float4 r0 = lo, r1 = hi;
  if (p < 2 && s.rope) {
    const float4 c = rf.c, sn = rf.sn;
    r0 = make_float4(lo.x * c.x - hi.x * sn.x, lo.y * c.y - hi.y * sn.y, lo.z * c.z - hi.z * sn.z,
                     lo.w * c.w - hi.w * sn.w);
    r1 = make_float4(hi.x * c.x + lo.x * sn.x, hi.y * c.y + lo.y * sn.y, hi.z * c.z + lo.z * sn.z,
                     hi.w * c.w + lo.w * sn.w);
  }
  const size_t flat0 = (size_t(d.b * heads_of(s, p) + h) * n_max + d.i) * dh + f;
  if (p == 0) {
    if (s.q_bf16) {
      const float sl2 = float(s.scale) * 1.4426950408889634f;
      bf16_t* q = static_cast<bf16_t*>(s.q) + flat0;
      union {
        uint2 u;
        bf16_t e[4];
      } a, c;
      a.e[0] = f32_to_bf16(r0.x * sl2);
      a.e[1] = f32_to_bf16(r0.y * sl2);
      a.e[2] = f32_to_bf16(r0.z * sl2);
      a.e[3] = f32_to_bf16(r0.w * sl2);
      c.e[0] = f32_to_bf16(r1.x * sl2);
      c.e[1] = f32_to_bf16(r1.y * sl2);
      c.e[2] = f32_to_bf16(r1.z * sl2);
      c.e[3] = f32_to_bf16(r1.w * sl2);
      *reinterpret_cast<uint2*>(q) = a.u;
      *reinterpret_cast<uint2*>(q + half) = c.u;
    } else {
      float* q = static_cast<float*>(s.q) + flat0;
      *reinterpret_cast<float4*>(q) = r0;
      *reinterpret_cast<float4*>(q + half) = r1;
    }
    note(r0, flat0);
    note(r1, flat0 + half);
  } else {
    bf16_t* dst = static_cast<bf16_t*>(p == 1 ? s.cand_k : s.cand_v) + flat0;
    union {
      uint2 u;
      bf16_t e[4];
    } a, c;
    a.e[0] = f32_to_bf16(r0.x);
    a.e[1] = f32_to_bf16(r0.y);
    a.e[2] = f32_to_bf16(r0.z);
    a.e[3] = f32_to_bf16(r0.w);
    c.e[0] = f32_to_bf16(r1.x);
    c.e[1] = f32_to_bf16(r1.y);
    c.e[2] = f32_to_bf16(r1.z);
    c.e[3] = f32_to_bf16(r1.w);
    *reinterpret_cast<uint2*>(dst) = a.u;
    *reinterpret_cast<uint2*>(dst + half) = c.u;
    note(make_float4(bf16_to_f32(a.e[0]), bf16_to_f32(a.e[1]), bf16_to_f32(a.e[2]), bf16_to_f32(a.e[3])), flat0);
    note(make_float4(bf16_to_f32(c.e[0]), bf16_to_f32(c.e[1]), bf16_to_f32(c.e[2]), bf16_to_f32(c.e[3])),
         flat0 + half);
  }
}

// Rotary factors of eight consecutive pairs of a row (see rope4).
struct Rope8 {
  float4 c0, c1, s0, s1;
};
__device__ __forceinline__ Rope8 rope8(const DevState& s, int p, const RowDst& d, int pair0) {
  Rope8 r{make_float4(1.f, 1.f, 1.f, 1.f), make_float4(1.f, 1.f, 1.f, 1.f), make_float4(0.f, 0.f, 0.f, 0.f),
          make_float4(0.f, 0.f, 0.f, 0.f)};
  if (d.i < 0 || p >= 2 || !s.rope) return r;
  const int half = s.head_width >> 1;
  const int f = pair0 % half;
  const float4* cp = reinterpret_cast<const float4*>(static_cast<const float*>(s.rope_cos) + size_t(d.pos) * half + f);
  const float4* sp = reinterpret_cast<const float4*>(static_cast<const float*>(s.rope_sin) + size_t(d.pos) * half + f);
  r.c0 = cp[0];
  r.c1 = cp[1];
  r.s0 = sp[0];
  r.s1 = sp[1];
  return r;
}

// Eight consecutive pairs pair0 .. pair0 + 7 of one head (pair0 % 8 == 0 and
// d_h / 2 % 8 == 0): the same as two put_pairs4 calls, with 16-byte stores.
__device__ __forceinline__ void put_pairs8(const DevState& s, int p, const RowDst& d, int pair0, float4 lo0,
                                           float4 lo1, float4 hi0, float4 hi1, const Rope8& rf, int n_max,
                                           unsigned long long& bad) {
  if (d.i < 0) return;
  const int dh = s.head_width;
  const int half = dh >> 1;
  const int h = pair0 / half;
  const int f = pair0 - h * half;
  auto note = [&](const float4& v, size_t flat) {
    if (isfinite((v.x + v.y) + (v.z + v.w))) return;
    if (!isfinite(v.x)) bad = min(bad, (unsigned long long)flat);
    else if (!isfinite(v.y)) bad = min(bad, (unsigned long long)(flat + 1));
    else if (!isfinite(v.z)) bad = min(bad, (unsigned long long)(flat + 2));
    else if (!isfinite(v.w)) bad = min(bad, (unsigned long long)(flat + 3));
  };
  if (p == 3) {
    const size_t flat = (size_t(d.b) * n_max + d.i) * s.model_width + size_t(h) * dh + f;
    float* o = static_cast<float*>(s.out_proj_dst) + flat;
    reinterpret_cast<float4*>(o)[0] = lo0;
    reinterpret_cast<float4*>(o)[1] = lo1;
    reinterpret_cast<float4*>(o + half)[0] = hi0;
    reinterpret_cast<float4*>(o + half)[1] = hi1;
    note(lo0, flat);
    note(lo1, flat + 4);
    note(hi0, flat + half);
    note(hi1, flat + half + 4);
    return;
  }
  auto rot = [](float4 lo, float4 hi, float4 c, float4 sn, float4& r0, float4& r1) {
    r0 = make_float4(lo.x * c.x - hi.x * sn.x, lo.y * c.y - hi.y * sn.y, lo.z * c.z - hi.z * sn.z,
                     lo.w * c.w - hi.w * sn.w);
    r1 = make_float4(hi.x * c.x + lo.x * sn.x, hi.y * c.y + lo.y * sn.y, hi.z * c.z + lo.z * sn.z,
                     hi.w * c.w + lo.w * sn.w);
  };
  float4 a0 = lo0, a1 = lo1, b0 = hi0, b1 = hi1;
  if (p < 2 && s.rope) {
    rot(lo0, hi0, rf.c0, rf.s0, a0, b0);
    rot(lo1, hi1, rf.c1, rf.s1, a1, b1);
  }
  const size_t flat0 = (size_t(d.b * heads_of(s, p) + h) * n_max + d.i) * dh + f;
  union P8 {
    uint4 u;
    bf16_t e[8];
  };
  auto pack = [](float4 x, float4 y, float k) {
    P8 r;
    r.e[0] = f32_to_bf16(x.x * k);
    r.e[1] = f32_to_bf16(x.y * k);
    r.e[2] = f32_to_bf16(x.z * k);
    r.e[3] = f32_to_bf16(x.w * k);
    r.e[4] = f32_to_bf16(y.x * k);
    r.e[5] = f32_to_bf16(y.y * k);
    r.e[6] = f32_to_bf16(y.z * k);
    r.e[7] = f32_to_bf16(y.w * k);
    return r;
  };
  if (p == 0) {
    if (s.q_bf16) {
      const float sl2 = float(s.scale) * 1.4426950408889634f;
      bf16_t* q = static_cast<bf16_t*>(s.q) + flat0;
      *reinterpret_cast<uint4*>(q) = pack(a0, a1, sl2).u;
      *reinterpret_cast<uint4*>(q + half) = pack(b0, b1, sl2).u;
    } else {
      float* q = static_cast<float*>(s.q) + flat0;
      reinterpret_cast<float4*>(q)[0] = a0;
      reinterpret_cast<float4*>(q)[1] = a1;
      reinterpret_cast<float4*>(q + half)[0] = b0;
      reinterpret_cast<float4*>(q + half)[1] = b1;
    }
    note(a0, flat0);
    note(a1, flat0 + 4);
    note(b0, flat0 + half);
    note(b1, flat0 + half + 4);
  } else {
    bf16_t* dst = static_cast<bf16_t*>(p == 1 ? s.cand_k : s.cand_v) + flat0;
    const P8 x = pack(a0, a1, 1.f), y = pack(b0, b1, 1.f);
    *reinterpret_cast<uint4*>(dst) = x.u;
    *reinterpret_cast<uint4*>(dst + half) = y.u;
    auto back = [](const P8& v, int o) {
      return make_float4(bf16_to_f32(v.e[o]), bf16_to_f32(v.e[o + 1]), bf16_to_f32(v.e[o + 2]), bf16_to_f32(v.e[o + 3]));
    };
    note(back(x, 0), flat0);
    note(back(x, 4), flat0 + 4);
    note(back(y, 0), flat0 + half);
    note(back(y, 4), flat0 + half + 4);
  }
}

__device__ __forceinline__ void store_pair(const DevState& s, int p, int m, int pair, float lo, float hi, int M,
                                           int n_max, int per_seq_rows) {
  unsigned long long bad = kErrClear, bad_pos = kErrClear;
  put_pair(s, p, row_dst(s, p, m, M, n_max, per_seq_rows, bad_pos), pair, lo, hi, n_max, bad);
  flush_bad(s, p, bad, bad_pos);
}

// ------------------------------------------------------------ skinny GEMM --
// Block (t, mt): rows 32 mt .. +32 and 32 rotary pairs of projection
// p = t / (D/64).  Wave w owns 8 pairs: output column j < 8 of its 16 is the
// low feature of pair j, column j + 8 the high one.  Every wave runs the whole
// reduction axis over its 16 weight rows (16x16x32 MFMA, lane (c, g) reading
// 16 bytes at k = 128 c' + 32 u + 8 g of chunk c'); the 32 x 128 input chunk
// is loaded once per block into a double-buffered LDS tile and shared by the
// four waves, which is what keeps the small activation matrix from being
// re-read from L2 by every column tile.
constexpr int SKC = 128;           // k per chunk
constexpr int SLDX = SKC + 8;      // LDS row stride (bf16) of the input tile
constexpr int SUNROLL = 8;         // chunks per statically unrolled group
constexpr int SRING = 4;           // weight-fragment ring (chunks in flight + 1); divides SUNROLL

__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// NCH > 0: the reduction axis has exactly NCH chunks (fully unrolled); 0: any D.
// XT: input element type (bf16 rows, or the float32 merged heads for W_o).
// KSPLIT > 1: block z sums chunks z NCH/KSPLIT .. (z+1) NCH/KSPLIT - 1 only and
// stores its float32 partial sums at s.proj_partials[z][m][64 t + 16 w + c16]
// (tile t, wave w, MFMA column c16); skinny_reduce_kernel adds them in order z
// and runs the epilogue.  Splitting gives a 32-row projection (192 blocks at
// D = 4096) enough blocks and loads in flight to fill the chip.
template <int NCH, typename XT, int KSPLIT>
__global__ __launch_bounds__(256) void project_skinny_kernel(DevState s, const XT* __restrict__ x, int M,
                                                             int n_max, int per_seq_rows, int proj_first) {
  static_assert(KSPLIT == 1 || (NCH > 0 && NCH % KSPLIT == 0), "a split needs a fixed chunk count");
  __shared__ __attribute__((aligned(16))) bf16_t Xs[2][32 * SLDX];
  const int D = s.model_width;
  const int half = s.head_width >> 1;
  int tile = blockIdx.x;
  const int p = tile_proj(s, proj_first, 64, tile);
  const int pair_base = tile * 32;
  const int m0 = blockIdx.y * 32;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g4 = lane >> 4;
  const int c16 = lane & 15;

  const int pair = pair_base + wave * 8 + (c16 & 7);
  const int h = pair / half;
  const int f = pair - h * half;
  const int wrow = h * s.head_width + f + ((c16 >> 3) ? half : 0);
  constexpr int NCHK = NCH / KSPLIT;  // chunks of this block (split launches)
  const int k0 = KSPLIT > 1 ? int(blockIdx.z) * NCHK * SKC : 0;
  const bf16_t* wp = weight_of(s, p) + size_t(wrow) * D + 8 * g4 + k0;
  // input staging: thread copies 32 bytes of row tid/8
  const int xrow = tid >> 3;
  const int xseg = (tid & 7) * 16;
  const XT* xg = x + size_t(min(m0 + xrow, M - 1)) * D + xseg + k0;

  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  const int nch = NCH > 0 ? NCHK : D / SKC;
  // weight fragments and input chunks are loaded SRING - 1 chunks ahead of the
  // multiply, into rings indexed by chunk % SRING (static: chunks are unrolled
  // in groups of SUNROLL).  The two streams share the distance because vector
  // loads retire in order: waiting for an input chunk loaded later than the
  // weights would also wait for those weights.
  Frag8 b[SRING][4];
  uint4 xr[SRING][2];
  auto load_chunk = [&](int c, int slot) {
#pragma unroll
    for (int u = 0; u < 4; ++u) b[slot][u].u = *reinterpret_cast<const uint4*>(wp + c * SKC + 32 * u);
    uint4 lo, hi;
    load16(xg + c * SKC, lo, hi);
    xr[slot][0] = lo;
    xr[slot][1] = hi;
  };
  auto publish = [&](int slot, int buf) {
    *reinterpret_cast<uint4*>(&Xs[buf][xrow * SLDX + xseg]) = xr[slot][0];
    *reinterpret_cast<uint4*>(&Xs[buf][xrow * SLDX + xseg + 8]) = xr[slot][1];
  };
#pragma unroll
  for (int c = 0; c < SRING - 1; ++c)
    if (c < nch) load_chunk(c, c);
  publish(0, 0);
  __syncthreads();

  // one chunk: issue the loads SRING - 1 chunks ahead, multiply this chunk,
  // publish the next input chunk to the other LDS buffer
  auto step = [&](int c, int slot, int ahead_slot, int next_slot, int buf) {
    if (c + SRING - 1 < nch) load_chunk(c + SRING - 1, ahead_slot);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      Frag8 a0, a1;
      a0.u = *reinterpret_cast<const uint4*>(&Xs[buf][c16 * SLDX + 32 * u + 8 * g4]);
      a1.u = *reinterpret_cast<const uint4*>(&Xs[buf][(16 + c16) * SLDX + 32 * u + 8 * g4]);
      acc0 = mfma16(a0.v, b[slot][u].v, acc0);
      acc1 = mfma16(a1.v, b[slot][u].v, acc1);
    }
    if (c + 1 < nch) publish(next_slot, buf ^ 1);
    __syncthreads();
  };
  if constexpr (NCH > 0) {
#pragma unroll
    for (int c = 0; c < NCHK; ++c) step(c, c % SRING, (c + SRING - 1) % SRING, (c + 1) % SRING, c & 1);
  } else {
    int c = 0;
    for (; c + SUNROLL <= nch; c += SUNROLL) {
#pragma unroll
      for (int k = 0; k < SUNROLL; ++k) step(c + k, k % SRING, (k + SRING - 1) % SRING, (k + 1) % SRING, k & 1);
    }
#pragma unroll
    for (int k = 0; k < SUNROLL; ++k)
      if (c + k < nch) step(c + k, k % SRING, (k + SRING - 1) % SRING, (k + 1) % SRING, k & 1);
  }

  if constexpr (KSPLIT > 1) {
    const int cols = gridDim.x * 64;
    float* part = s.proj_partials + size_t(blockIdx.z) * 64 * cols + blockIdx.x * 64 + wave * 16 + c16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      part[size_t(4 * g4 + r) * cols] = acc0[r];
      part[size_t(16 + 4 * g4 + r) * cols] = acc1[r];
    }
    return;
  }
  // pairs: lanes with column j < 8 take the high feature from lane + 8
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float hi0 = __shfl_xor(acc0[r], 8, 64);
    const float hi1 = __shfl_xor(acc1[r], 8, 64);
    if (c16 < 8) {
      store_pair(s, p, m0 + 4 * g4 + r, pair, acc0[r], hi0, M, n_max, per_seq_rows);
      store_pair(s, p, m0 + 16 + 4 * g4 + r, pair, acc1[r], hi1, M, n_max, per_seq_rows);
    }
  }
}

// Sums the KSPLIT partials of a split skinny projection (in order z, so the
// result does not depend on scheduling) and runs its epilogue: thread
// (m, tile, wave, j < 8) owns rotary pair 32 tile + 8 wave + j of row m.
// Launched for M <= 32 rows (one row tile).
template <int KSPLIT>
__global__ __launch_bounds__(256) void skinny_reduce_kernel(DevState s, int M, int n_max, int per_seq_rows,
                                                            int proj_first, int tiles) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int per_row = tiles * 32;
  const int m = idx / per_row;
  if (m >= M) return;
  const int q = idx - m * per_row;
  int tile = q >> 5;
  const int w = (q >> 3) & 3, j = q & 7;
  const int cols = tiles * 64;
  const float* part = s.proj_partials + size_t(m) * cols + tile * 64 + w * 16 + j;
  float lo = 0.f, hi = 0.f;
#pragma unroll
  for (int z = 0; z < KSPLIT; ++z) {
    lo += part[size_t(z) * 64 * cols];
    hi += part[size_t(z) * 64 * cols + 8];
  }
  const int p = tile_proj(s, proj_first, 64, tile);
  store_pair(s, p, m, tile * 32 + w * 8 + j, lo, hi, M, n_max, per_seq_rows);
}

// ------------------------------------------------------------- tiled GEMM --
// Block (t, mt): rows 128 mt .. +128 and 64 rotary pairs of projection p.
// Wave (wm, wn) computes rows wm*64 .. +64 and pairs wn*32 .. +32: its
// n-subtile 0 holds their low features and n-subtile 1 their high features,
// so each thread owns both halves of its pairs.
constexpr int TBM = 128, TBN = 128, TBK = 64, TLD = TBK + 8;

template <typename XT>
__global__ __launch_bounds__(256) void project_tiled_kernel(DevState s, const XT* __restrict__ x, int M,
                                                            int n_max, int per_seq_rows, int proj_first) {
  __shared__ __attribute__((aligned(16))) bf16_t As[TBM * TLD];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[TBN * TLD];
  const int D = s.model_width;
  const int dh = s.head_width;
  const int half = dh >> 1;
  int tile = blockIdx.x;
  const int p = tile_proj(s, proj_first, TBN, tile);  // 64 pairs per tile
  const int pair_base = tile * 64;
  const int m0 = blockIdx.y * TBM;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 5;
  const int c32 = lane & 31;

  // global -> LDS assignment: thread loads 64 contiguous bytes of row tid/2
  const int lrow = tid >> 1;
  const int lk = (tid & 1) * 32;
  const XT* ag = x + size_t(min(m0 + lrow, M - 1)) * D + lk;
  const int v = lrow;  // virtual column of the B tile
  const int vpair = pair_base + (v >> 6) * 32 + (v & 31);
  const int vh = vpair / half;
  const int vf = vpair - vh * half;
  const int vrow = vh * dh + vf + (((v >> 5) & 1) ? half : 0);
  const bf16_t* bg = weight_of(s, p) + size_t(vrow) * D + lk;

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // register prefetch of the next K tile: 64 bytes of A and of B per thread,
  // kept in named registers (an indexed array here ends up in scratch memory)
  uint4 ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;
  auto fetch = [&](int kt) {
    const uint4* b4 = reinterpret_cast<const uint4*>(bg + kt * TBK);
    load16(ag + kt * TBK, ra0, ra1);
    load16(ag + kt * TBK + 16, ra2, ra3);
    rb0 = b4[0];
    rb1 = b4[1];
    rb2 = b4[2];
    rb3 = b4[3];
  };
  fetch(0);
  const int ktiles = D / TBK;
  for (int kt = 0; kt < ktiles; ++kt) {
    __syncthreads();
    uint4* as = reinterpret_cast<uint4*>(&As[lrow * TLD + lk]);
    uint4* bs = reinterpret_cast<uint4*>(&Bs[lrow * TLD + lk]);
    as[0] = ra0;
    as[1] = ra1;
    as[2] = ra2;
    as[3] = ra3;
    bs[0] = rb0;
    bs[1] = rb1;
    bs[2] = rb2;
    bs[3] = rb3;
    __syncthreads();
    if (kt + 1 < ktiles) fetch(kt + 1);
#pragma unroll
    for (int u = 0; u < TBK / 16; ++u) {
      Frag8 fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        fa[i].u = *reinterpret_cast<const uint4*>(&As[(wm * 64 + i * 32 + c32) * TLD + 16 * u + 8 * g]);
        fb[i].u = *reinterpret_cast<const uint4*>(&Bs[(wn * 64 + i * 32 + c32) * TLD + 16 * u + 8 * g]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(fa[i].v, fb[j].v, acc[i][j]);
    }
  }
  const int pair = pair_base + wn * 32 + c32;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
      store_pair(s, p, m, pair, acc[i][0][r], acc[i][1][r], M, n_max, per_seq_rows);
    }
}

// ------------------------------------------------------- wide tiled GEMM --
// Many bf16 rows (suffix chunks, prefill): 256 x 256 output tiles, one
// 512-thread workgroup per compute unit (two waves per SIMD, so one wave's
// waits and epilogue instructions overlap the other's MFMAs), each wave a
// 128 x 64 block held in eight 32x32 accumulators, so a 16-wide step reads 6
// fragments from LDS for 8 MFMAs.  The 64-wide K tiles of X and W are
// double-buffered in LDS (128 KB, unpadded rows with swizzled 16-byte slots)
// and go straight from global memory into their buffer by 16-byte direct
// loads while the tile before is multiplied, one wait and barrier per tile.
// Columns: block virtual column v holds pair pair_base + 32 (v / 64) + v % 32,
// low feature for (v / 32) even, high feature for odd, so the two 32-column
// subtiles of wave column wn (2 wn and 2 wn + 1) hold the two halves of the
// same 32 pairs.
// Tile order: consecutive tile ids run on one XCD (blocks are dealt to the
// eight XCDs in turn) and walk 4 row tiles per column step, so the 32 tiles an
// XCD runs at once share their X and W tiles through its L2.
constexpr int GBM = 256, GBN = 256, GBK = 64, GLD = GBK, GGROUP = 4, GWAVES = 8;

__global__ __launch_bounds__(64 * GWAVES) __attribute__((amdgpu_waves_per_eu(2, 2))) void project_wide_kernel(
    DevState s, const bf16_t* __restrict__ x, int M, int n_max, int per_seq_rows, int proj_first, int m_tiles,
    int n_tiles) {
  // two buffers each of the X and W tiles, as four arrays: the compiler tells
  // direct loads into one array from reads of another apart, so the fragment
  // reads of the current tiles do not wait for the loads into the next ones
  __shared__ __attribute__((aligned(16))) bf16_t X0[GBM * GLD];
  __shared__ __attribute__((aligned(16))) bf16_t X1[GBM * GLD];
  __shared__ __attribute__((aligned(16))) bf16_t W0[GBN * GLD];
  __shared__ __attribute__((aligned(16))) bf16_t W1[GBN * GLD];
  using Zero = std::integral_constant<int, 0>;
  using One = std::integral_constant<int, 1>;
  auto xbuf = [&](auto b) __attribute__((always_inline)) -> bf16_t* {
    if constexpr (decltype(b)::value == 0) return X0; else return X1;
  };
  auto wbuf = [&](auto b) __attribute__((always_inline)) -> bf16_t* {
    if constexpr (decltype(b)::value == 0) return W0; else return W1;
  };
  const int D = s.model_width;
  const int dh = s.head_width;
  const int half = dh >> 1;
  const int tiles = m_tiles * n_tiles;
  const int L = blockIdx.x;
  const int t = (tiles & 7) ? L : (L & 7) * (tiles >> 3) + (L >> 3);
  const int group = t / (GGROUP * n_tiles);
  const int within = t - group * GGROUP * n_tiles;
  const int rows_in_group = min(GGROUP, m_tiles - group * GGROUP);
  const int mt = group * GGROUP + within % rows_in_group;
  const int nt = within / rows_in_group;
  int ntp = nt;
  const int p = tile_proj(s, proj_first, GBN, ntp);  // 128 pairs per tile
  const int pair_base = ntp * 128;
  const int m0 = mt * GBM;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;  // rows 128 wm .., columns 64 wn ..
  const int g = lane >> 5;
  const int c32 = lane & 31;

  // global -> LDS with the 16-byte direct loads: a tile (256 rows of 64
  // elements, 128 bytes) is 2048 16-byte slots, slot 8 r + u (u < 8) of row r
  // holding elements 8 (u ^ f(r)) .. of the row, f(r) = (r / 2) mod 8, and one
  // wave instruction fills 64 consecutive slots, lane l slot 64 j + l (LDS byte
  // 16 (64 j + l)).  The swizzle puts the 16 rows a 16-lane fragment read takes
  // on distinct bank groups: row parity picks the half of the 64 banks, f(r)
  // the 16-byte group within it.  Waves 0-3 fill the X tile (32 instructions,
  // 8 each), waves 4-7 the W tile; element offsets are 32-bit (the dispatch
  // checks M * D and the weight rows times D against 2^31).
  // W tile row v = 32 i + c (c < 32) is virtual column v: pair pair_base +
  // 32 (i / 2) + c, its high feature (+ d_h / 2 rows) for odd i.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const bool fills_x = wave_u < 4;
  const bf16_t* gsrc = fills_x ? x : weight_of(s, p);
  constexpr int NDMA = 8;  // load instructions per wave and K tile
  int off[NDMA];
#pragma unroll
  for (int j = 0; j < NDMA; ++j) {
    const int q = (wave_u & 3) * NDMA + j;  // instruction within the tile
    const int slot = q * 64 + lane;
    const int r = slot >> 3, c = (slot & 7) ^ ((r >> 1) & 7);
    int row_off;
    if (fills_x) {
      row_off = min(m0 + r, M - 1) * D;
    } else {
      const int i = r >> 5;
      const int vpair = pair_base + 32 * (i >> 1) + (r & 31);
      const int vh = vpair / half;
      row_off = (vh * dh + (vpair - vh * half) + ((i & 1) ? half : 0)) * D;
    }
    off[j] = row_off + 8 * c;
  }
  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  typedef __attribute__((address_space(3))) void lds_void_t;
  // load instruction j of the K tile at k0 into buffer buf (completion: s_waitcnt vmcnt(0)), in
  // the buffer form: a descriptor over the wave's whole source matrix, the lane's row offset in
  // bytes as the vector offset and the K tile's as the scalar one.  (The global form is counted
  // as an LDS access as well, so each step's wait for its fragments would also wait for the
  // tile loads in flight, and it takes the issuing wave several times longer.)
  const uint32_t src_bytes = uint32_t(fills_x ? M : heads_of(s, p) * dh) * uint32_t(D) * 2u;
  const __amdgpu_buffer_rsrc_t src_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(gsrc), (short)0, src_bytes, 0x00020000);
  auto fetch_one = [&](int j, int k0, auto buf) __attribute__((always_inline)) {
    bf16_t* dst = (fills_x ? xbuf(buf) : wbuf(buf)) + (wave_u & 3) * NDMA * 64 * 8;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src_rsrc, (lds_void_t*)(dst + j * 64 * 8), 16, uint32_t(off[j]) * 2u,
                                             uint32_t(k0) * 2u, 0, 0);
  };
  auto fetch = [&](int k0, auto buf) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NDMA; ++j) fetch_one(j, k0, buf);
  };
  // fragments of one 16-wide step, double-buffered in registers: step ks + 1
  // is read from LDS while step ks's 16 MFMAs run
  Frag8 fa[2][4], fb[2][2];
  // (rows 32 i + c32 of either tile: f(row) = (c32 / 2) mod 8 for every i)
  const int fsw = (c32 >> 1) & 7;
  auto read_frags = [&](auto buf, int ks, int slot) __attribute__((always_inline)) {
    const int ps = 8 * (((2 * ks + g) ^ fsw) & 7);
    const bf16_t* ar = xbuf(buf) + (wm * 128 + c32) * GLD + ps;
    const bf16_t* br = wbuf(buf) + (wn * 64 + c32) * GLD + ps;
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[slot][i].u = *reinterpret_cast<const uint4*>(ar + i * 32 * GLD);
#pragma unroll
    for (int j = 0; j < 2; ++j) fb[slot][j].u = *reinterpret_cast<const uint4*>(br + j * 32 * GLD);
  };
  // One 16-wide step: an LDS-only wait (lgkmcnt(0), vmcnt and expcnt left
  // alone) for its operands in slot cur, two MFMAs, the next step's fragments
  // (K tile in buffer rbuf, step rks, into slot cur ^ 1), then the other six
  // MFMAs with up to six load instructions of a K tile (dma_first ..., at k0
  // into buffer dbuf) between them: the load path takes loads far slower than a
  // wave issues them, and a wave stuck issuing loads issues no MFMAs.
  auto step = [&](int cur, auto rbuf, int rks, int dma_first, int dma_count, int dk, auto dbuf)
                  __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0xC07F);
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[0][j] = mfma32(fa[cur][0].v, fb[cur][j].v, acc[0][j]);
    __builtin_amdgcn_sched_barrier(0);
    read_frags(rbuf, rks, cur ^ 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 1; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        acc[i][j] = mfma32(fa[cur][i].v, fb[cur][j].v, acc[i][j]);
        const int m = (i - 1) * 2 + j;
        if (m < dma_count) fetch_one(dma_first + m, dk, dbuf);
        __builtin_amdgcn_sched_barrier(0);
      }
  };
  // Steps 0-2 of K tile kt run before the tile's barrier and step 3 after it,
  // so the next tile's first fragments are read under step 3's MFMAs; tile
  // kt + 2 starts loading into tile kt's buffer in step 3 (6 instructions) and
  // step 0 of the next tile (2), and is waited for four steps later.  Past the
  // last tile the last one is loaded again (never read).
  const int ktiles = D / GBK;
  auto k_of = [&](int t) { return min(t, ktiles - 1) * GBK; };
  fetch(0, Zero());
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  read_frags(Zero(), 0, 0);
  // K tile kt in buffer B (the parity of kt), the next one in NB
  auto ktile = [&](auto B, int kt) __attribute__((always_inline)) {
    using NB = std::integral_constant<int, 1 - decltype(B)::value>;
    if (kt == 0) {
      step(0, B, 1, 0, 6, k_of(1), NB());
      step(1, B, 2, 6, 2, k_of(1), NB());
    } else {
      step(0, B, 1, 6, 2, k_of(kt + 1), NB());
      step(1, B, 2, 0, 0, 0, NB());
    }
    step(0, B, 3, 0, 0, 0, NB());
    // tile kt + 1 in LDS, and this wave's reads of tile kt done (its buffer is
    // reloaded after the barrier)
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __syncthreads();
    step(1, NB(), 0, 0, 6, k_of(kt + 2), B);
  };
  for (int kt = 0; kt < ktiles; kt += 2) {
    ktile(Zero(), kt);
    if (kt + 1 < ktiles) ktile(One(), kt + 1);
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __syncthreads();
  // epilogue, one 32-row quarter of the wave's block at a time, through LDS
  // (the K-tile buffers are free now: two waves stage into each).  The wave's 64 columns are the low and
  // high features of 32 pairs; lane (row r16, c8) then handles eight consecutive
  // pairs of rows r16, r16 + 16: 4 lanes cover one row's 32 pairs, with 16-byte
  // stores.  A wave reads back only the block it staged itself, and its LDS
  // operations complete in order, so the quarters need no barrier: the waves
  // stage, rotate and store independently, their stores left in flight.
  constexpr int EPS = 64 + 4;  // staging row stride (floats)
  static_assert(2 * 32 * EPS * 4 <= GBM * GLD * 2 && GBM == GBN, "staging of two waves fits one tile buffer");
  bf16_t* stage_base = X0;
  switch (wave_u >> 1) {
    case 0: break;
    case 1: stage_base = X1; break;
    case 2: stage_base = W0; break;
    default: stage_base = W1; break;
  }
  float* ep = reinterpret_cast<float*>(stage_base) + (wave_u & 1) * 32 * EPS;
  const int wrow0 = m0 + __builtin_amdgcn_readfirstlane(wm) * 128;
  const int r16 = lane >> 2;
  const int c8 = (lane & 3) * 8;
  const int pair0 = pair_base + __builtin_amdgcn_readfirstlane(wn) * 32 + c8;
  unsigned long long bad = kErrClear, bad_pos = kErrClear;
  // accumulators are only ever indexed by constants (a runtime index would move them to scratch)
  auto stage = [&](const f32x16_t (&q)[2]) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) ep[(8 * (r >> 2) + 4 * g + (r & 3)) * EPS + j * 32 + c32] = q[j][r];
  };
  // where each quarter's rows land (lane c32: row c32 of quarter i), all four at
  // once; the row's lanes fetch them by shuffle
  RowDst mine[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) mine[i] = row_dst(s, p, wrow0 + i * 32 + c32, M, n_max, per_seq_rows, bad_pos);
#pragma unroll 1
  for (int i = 0; i < 4; ++i) {
    // the quarter's rotary factors are loaded before it is staged
    RowDst d[2];
    Rope8 rf[2];
    RowDst mi = mine[0];
    switch (i) {
      case 0: break;
      case 1: mi = mine[1]; break;
      case 2: mi = mine[2]; break;
      default: mi = mine[3]; break;
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int row = 16 * k + r16;
      d[k] = RowDst{__shfl(mi.b, row, 64), __shfl(mi.i, row, 64), __shfl(mi.pos, row, 64)};
      rf[k] = rope8(s, p, d[k], pair0);
    }
    switch (i) {
      case 0: stage(acc[0]); break;
      case 1: stage(acc[1]); break;
      case 2: stage(acc[2]); break;
      default: stage(acc[3]); break;
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const float4* er = reinterpret_cast<const float4*>(ep + (16 * k + r16) * EPS + c8);
      put_pairs8(s, p, d[k], pair0, er[0], er[1], er[8], er[9], rf[k], n_max, bad);
    }
  }
  flush_bad(s, p, bad, bad_pos);
}

// ---------------------------------------------------------- flash attention --
// Block = one work item (sequence b, chunk queries QT qt .. +QT, QT =
// kChunkQueryTile = 256) of head h: eight waves of 32 queries, which share
// every K/V tile the block loads (twice the queries per loaded tile of a
// four-wave block, at the same two waves per SIMD).  Virtual key j < len is
// cache row j, else chunk row
// j - len; query i sees j <= len + i.  Scores are formed transposed
// (S^T = K Q^T) so that a lane holds every score of one query: the softmax
// scale factor is per lane, and the probabilities are already in the operand
// layout of O^T += V^T P^T.
//
// Keys and values pass through LDS in tiles of 128 rows, two buffers of each,
// filled by direct global-to-LDS loads (16 lanes per 256-byte row, so a load
// instruction covers whole rows) while the current tiles are multiplied
// (schedule below).  V stays
// row-major in LDS; the V^T operand comes from the transposing LDS read
// (ds_read_b64_tr_b16): within each 16-lane group, lane i receives element
// i % 4 of the 8-byte pieces addressed by lanes i / 4 + 4 m, m = 0..3, so
// lanes addressing (key kb + j / 4, features d0 + 4 (j % 4) ..) hand lane i
// feature d0 + i of keys kb .. kb + 3.
//
// Softmax: base 2 with the scale folded into q; the running maximum is only
// raised (and the accumulators rescaled) when a score exceeds it by more than
// 2^8, so probabilities stay below 256 and most tiles skip the rescale.  The
// maximum is kept as a bf16 value and subtracted by the score MFMAs (a 1 in
// the keys against -max in the queries), and the normaliser adds the
// probabilities as rounded to bf16 for P V, so numerator and denominator
// weight every key alike.
typedef short s16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint2 lds_read_tr16(const bf16_t* p) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(const_cast<bf16_t*>(p)));
  return __builtin_bit_cast(uint2, v);
}

// The larger of v in lanes l and l ^ 32, in every lane, by the vector unit's
// half-swap (v_permlane32_swap exchanges lanes 32-63 of the first register
// with lanes 0-31 of the second: copies of v become [lo, lo] and [hi, hi]),
// not through the LDS pipe as a cross-lane shuffle would be.  (Wait states
// around it: the compiler sees no hazard through inline asm.)
__device__ __forceinline__ float max_halves(float v) {
  float a = v, b = v;
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  return fmaxf(a, b);
}

// acc plus the eight bf16 values of f (packed dot products with ones)
__device__ __forceinline__ float add_bf16x8(const Frag8& f, float acc) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t one = {(__bf16)1.f, (__bf16)1.f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, f.u.x), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, f.u.y), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, f.u.z), one, acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, f.u.w), one, acc, false);
}

// WIN: sliding-window layer (ring storage, a lower key bound per query).
template <int DH, bool WIN>
__global__ __launch_bounds__(2 * kChunkQueryTile) __attribute__((amdgpu_waves_per_eu(2, 2))) void attend_flash_kernel(
    DevState s, int n_max, int per_seq_rows, ChunkOrder order, float* __restrict__ out,
    const int32_t* __restrict__ redo) {
  // after the role-split kernel: only the work items it handed back
  if (redo && redo[blockIdx.x] == 0) return;
  constexpr int KT = 128;  // keys per LDS tile (two buffers of K and V: 128 KB at d_h = 128)
  static_assert(kMinBlockRows % KT == 0, "a key tile must stay inside one block");
  constexpr int DSTEPS = DH / 16;
  constexpr int DTILES = DH / 32;
  constexpr int SPR = DH / 8;         // 16-byte slots per row
  constexpr int RPS = 16 / SPR;       // rows per 256-byte sweep of the 64 banks
  constexpr int RPL = 64 / SPR;       // rows filled by one wave's load instruction
  constexpr int NI = KT / RPL / 8;    // load instructions per eighth of a tile
  static_assert((NI == 2 || NI == 4) && NI * RPL * 8 == KT, "a tile is 16 or 32 load instructions");
  constexpr int QT = kChunkQueryTile;  // queries of the workgroup, 32 per wave
  constexpr float kRescale = 8.f;    // log2 of the largest probability kept unscaled
  // two buffers each of K and V, as four arrays: the compiler tells direct
  // loads into one array from reads of another apart, so the reads of the
  // current tiles do not wait for the loads into the next ones
  __shared__ __attribute__((aligned(16))) bf16_t K0[KT * DH];
  __shared__ __attribute__((aligned(16))) bf16_t K1[KT * DH];
  __shared__ __attribute__((aligned(16))) bf16_t V0[KT * DH];
  __shared__ __attribute__((aligned(16))) bf16_t V1[KT * DH];
  __shared__ int counters[6];  // waves seen per SIMD, leading and trailing waves seen
  using Zero = std::integral_constant<int, 0>;
  using One = std::integral_constant<int, 1>;
  auto kbuf = [&](auto p) __attribute__((always_inline)) -> bf16_t* {
    if constexpr (decltype(p)::value == 0) return K0; else return K1;
  };
  auto vbuf = [&](auto p) __attribute__((always_inline)) -> bf16_t* {
    if constexpr (decltype(p)::value == 0) return V0; else return V1;
  };

  const int H = s.heads;
  const int item = blockIdx.x / H;
  const int slot = blockIdx.x - item * H;
  // grouped layers: the query heads of one key/value head run on one XCD
  // (blocks are dealt to the eight XCDs in turn), so their shared K/V tiles
  // are fetched into one L2
  const int h = (s.kv_heads < H && (H & 7) == 0) ? (slot & 7) * (H >> 3) + (slot >> 3) : slot;
  int b, qt;
  if (order.count) {
    b = order.item[item] >> 16;
    qt = order.item[item] & 0xffff;
  } else {
    b = item / order.qtiles;
    qt = order.qtiles - 1 - (item - b * order.qtiles);
  }
  const int n_b = per_seq_rows ? s.rows[b] : n_max;
  if (qt * QT >= n_b) return;
  const int len = WIN ? max(s.len[b], 0) : min(max(s.len[b], 0), s.capacity);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;
  const int c32 = lane & 31;
  const int qi = qt * QT + wave * 32 + c32;
  const int qi_eff = min(qi, n_b - 1);
  const int limit = len + qi_eff;
  const int i_max = min(qt * QT + QT - 1, n_b - 1);
  const int total = len + i_max + 1;
  const int ntiles = (total + KT - 1) / KT;
  // sliding window: query qi reads keys lo .. limit; the block starts at the key
  // tile holding its first query's lowest key
  const int lo = WIN ? window_start(s, limit) : 0;
  const int it_first = WIN ? window_start(s, len + qt * QT) / KT : 0;
  const int n_it = ntiles - it_first;  // key tiles the block walks, >= 1
  const int wave_lo_max = WIN ? window_start(s, len + min(qt * QT + wave * 32 + 31, n_b - 1)) : 0;
  const size_t lane_id = size_t(b) * H + h;
  const int hk = h / (H / s.kv_heads);  // the key/value head this query head reads
  const size_t kv_lane = size_t(b) * s.kv_heads + hk;
  const bf16_t* kc = static_cast<const bf16_t*>(s.keys);  // rows through the block base
  const bf16_t* vc = static_cast<const bf16_t*>(s.values);
  const bf16_t* kn = static_cast<const bf16_t*>(s.cand_k) + kv_lane * n_max * DH;
  const bf16_t* vn = static_cast<const bf16_t*>(s.cand_v) + kv_lane * n_max * DH;

  // B operand of S^T: lane holds q[qi][16 u + 8 g + e] * scale * log2(e), rounded
  // to bf16, so scores come out of the MFMA already in base-2 softmax units.
  // (the projection of a chunk call stores q already scaled and rounded so,
  // s.q_bf16; otherwise q is float32 and is scaled and rounded here)
  const float sl2 = float(s.scale) * 1.4426950408889634f;
  Frag8 qf[DSTEPS];
  if (s.q_bf16) {
    const bf16_t* qp = static_cast<const bf16_t*>(s.q) + (lane_id * n_max + qi_eff) * DH;
#pragma unroll
    for (int u = 0; u < DSTEPS; ++u) qf[u].u = *reinterpret_cast<const uint4*>(qp + 16 * u + 8 * g);
  } else {
    const float* qp = static_cast<const float*>(s.q) + (lane_id * n_max + qi_eff) * DH;
#pragma unroll
    for (int u = 0; u < DSTEPS; ++u) {
      const float4 q0 = reinterpret_cast<const float4*>(qp + 16 * u + 8 * g)[0];
      const float4 q1 = reinterpret_cast<const float4*>(qp + 16 * u + 8 * g)[1];
      qf[u].v[0] = (__bf16)(q0.x * sl2);
      qf[u].v[1] = (__bf16)(q0.y * sl2);
      qf[u].v[2] = (__bf16)(q0.z * sl2);
      qf[u].v[3] = (__bf16)(q0.w * sl2);
      qf[u].v[4] = (__bf16)(q1.x * sl2);
      qf[u].v[5] = (__bf16)(q1.y * sl2);
      qf[u].v[6] = (__bf16)(q1.z * sl2);
      qf[u].v[7] = (__bf16)(q1.w * sl2);
    }
  }
  f32x16_t o[DTILES];
#pragma unroll
  for (int t = 0; t < DTILES; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  // Scores are taken against a reference maximum mref (0 until a key is seen,
  // else m_run, a bf16 value): the matrix core subtracts it as one more
  // 16-deep step with key feature 1 and query feature -mref.
  float mref = 0.f;
  Frag8 onek, mq;
  onek.u = make_uint4(g == 0 ? 0x3f80u : 0u, 0u, 0u, 0u);
  mq.u = make_uint4(0u, 0u, 0u, 0u);
  const int wave_limit_min = len + min(qt * QT + wave * 32, n_b - 1);  // smallest limit in the wave

  // Tiles are unpadded rows of d_h elements whose 16-byte slots are permuted
  // within each row (slot c of row r holds piece c ^ f(r)), so that the
  // fragment reads below hit every bank once per sweep: for K, f(r) =
  // (r / RPS) mod SPR (the 16 rows a 16-lane group reads start in different
  // banks); for V, f(r) = 4 ((r / RPS) mod (SPR / 4)) (the four rows a 32-lane
  // transposing read takes 16 bytes from fall in different bank quarters).
  // Global -> LDS with the 16-byte direct loads: one wave instruction fills
  // RPL whole rows (lane l: row l / SPR, slot l mod SPR), instruction q of a
  // tile rows RPL q ..; a tile is 8 NI instructions.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  auto kswz = [](int r) __attribute__((always_inline)) { return (r / RPS) & (SPR - 1); };
  auto vswz = [](int r) __attribute__((always_inline)) { return 4 * ((r / RPS) & (SPR / 4 - 1)); };
  typedef __attribute__((address_space(3))) void lds_void_t;
  typedef __attribute__((address_space(1))) void glb_void_t;
  // byte offset of this lane's slot within the rows of instruction q: V the
  // same for every q, K koff0 ^ 64 (q mod NI) (f(RPL q + l / SPR) differs from
  // f(l / SPR) in the slot bits worth 64 bytes, by 4 (q mod NI))
  const int lr = lane / SPR, lc = lane & (SPR - 1);
  const uint32_t voff = uint32_t(lr * DH + 8 * (lc ^ vswz(lr))) * 2u;
  const uint32_t koff0 = uint32_t(lr * DH + 8 * (lc ^ kswz(lr))) * 2u;
  // Block base (kv_block_base) of a run of rows starting at r0 of this lane's
  // cache, with the block table read through the scalar cache (it is not
  // written while the kernel runs), so no vector-memory wait orders it behind
  // the tile loads in flight.
  auto block_base = [&](int r0) __attribute__((always_inline)) -> ptrdiff_t {
    if (!s.paged) return kv_block_base(s, b, hk, r0);
    typedef const __attribute__((address_space(4))) int32_t* const_i32_t;
    const int lg = s.block_rows_log2;
    const int blk = max(((const_i32_t)s.block_table)[size_t(b) * s.table_width + (r0 >> lg)], 0);
    return (ptrdiff_t(size_t(blk) * s.kv_heads + hk) << lg) * DH - ptrdiff_t((r0 >> lg) << lg) * DH;
  };
  // Where tile t (absolute) of K or V comes from: a tile of contiguous rows
  // (all cache rows, or all chunk rows) from one base; otherwise row by row (a
  // tile across the cache end, or past the last key: rows after it repeat the
  // last key, which the mask hides).  A 128-row tile lies in one block of a
  // paged cache, so one block base serves all its cached rows.
  struct TileSrc {
    const char* base;       // contiguous: the tile's first row
    const bf16_t* cached;   // row by row: row j < len at cached + j d_h
    const bf16_t* chunk;    //             row j >= len at chunk + (j - len) d_h
    int j0;
    bool contiguous;
  };
  auto tile_src = [&](auto is_v, int t) __attribute__((always_inline)) {
    TileSrc src;
    const bf16_t* cache = is_v ? vc : kc;
    src.chunk = is_v ? vn : kn;
    src.j0 = t * KT;
    src.cached = cache + block_base(min(src.j0, max(len - 1, 0)));
    src.contiguous = src.j0 + KT <= len || (src.j0 >= len && src.j0 + KT <= total);
    src.base = reinterpret_cast<const char*>(src.j0 < len ? src.cached + ptrdiff_t(src.j0) * DH
                                                          : src.chunk + size_t(src.j0 - len) * DH);
    return src;
  };
  // Direct load of instruction q of a contiguous tile whose first row is at
  // `first`, in the buffer form: a buffer descriptor spanning the tile, the
  // lane's byte offset off and the instruction's rows as the scalar offset.
  // (The compiler counts the global form as an LDS access as well and then
  // waits for every LDS read in flight behind it; the buffer form counts as a
  // vector-memory load only.)
  auto dma_tile = [&](const char* first, bf16_t* tile, int q, uint32_t off) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(first), (short)0, KT * DH * 2, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(tile + q * RPL * DH), 16, off, q * (RPL * DH * 2), 0, 0);
  };
  // issues instruction q of the tile src into `tile`.  (The lane offsets are
  // copied opaquely here, so what they give for each q is formed per
  // instruction rather than held in registers across the loop.)
  auto load_one = [&](auto is_v, const TileSrc& src, bf16_t* tile, int q) __attribute__((always_inline)) {
    uint32_t off = is_v ? voff : koff0;
    asm volatile("" : "+v"(off));
    if (!is_v) off ^= 64u * uint32_t(q & (NI - 1));
    if (src.contiguous) {
      dma_tile(src.base, tile, q, off);
    } else {
      int row = lr;
      asm volatile("" : "+v"(row));
      const int j = min(src.j0 + RPL * q + row, total - 1);
      const int c = int(off & (DH * 2 - 1)) >> 1;  // element of the row
      const bf16_t* g_addr = (j < len ? src.cached + ptrdiff_t(j) * DH : src.chunk + size_t(j - len) * DH) + c;
      __builtin_amdgcn_global_load_lds((glb_void_t*)g_addr, (lds_void_t*)(tile + q * RPL * DH), 16, 0, 0);
    }
  };

  // Work of the block on key tile j (local index, tile it_first + j; buffers
  // by the parity of j):
  //   S_j  scores of tile j (matrix cores, K tile from LDS)
  //   X_j  mask, maximum, rescale, exponentials, bf16 probabilities (vector unit)
  //   P_j  O^T += V^T P^T (matrix cores, V tile from LDS)
  // A wave runs S_0, then X_j and [P_j, S_j+1] alternately, one barrier after
  // each.  One of the two waves on each SIMD (its second by an LDS ticket)
  // runs one segment behind the other, so on every SIMD one wave's
  // exponentials overlap the other wave's matrix products instead of both
  // waves switching between them together.  The pair (V_j, K_j+1) is read in
  // segments 2j+2 (leading waves) and 2j+3 (trailing waves).  Each wave loads
  // a quarter of every other tile, one load instruction after each step of
  // its S_j+1 (its P_j, the last read of the buffers it loads, done): the
  // leading waves K_j+2 in segment 2j+2, the trailing waves V_j+2 in segment
  // 2j+3; a leading wave waits for its loads at the end of its next X, a
  // trailing wave at the end of its next [P, S] (its V_j+2 is first read in
  // segment 2j+6), before the barrier that precedes the first reader.  (A load
  // instruction holds up the
  // wave that issues it for tens of cycles: spread this way, each wave loads
  // a quarter of a pair per tile.)  Should the tickets not come out as one
  // leading and one trailing wave per SIMD, every wave leads and loads an
  // eighth of K_j+2 and of V_j+1.
  f32x16_t st[KT / 32];
  Frag8 pb[KT / 32][2];
  const int kx = kswz(c32);  // the K rows this lane reads are c32 plus multiples of 32
  // S_j from the buffer `kt_tile`: the four 32-key blocks advance together one
  // 16-feature step at a time; the fragment of block kt for step u + 1 is read
  // right after the MFMA of step u that last used its registers, three MFMAs
  // ahead of its use; after step u, hook(u).  (The lane's swizzle is copied
  // opaquely per tile: the eight step offsets it gives are recomputed here
  // rather than held across the loop.)
  auto scores = [&](const bf16_t* kt_tile, auto&& hook) __attribute__((always_inline)) {
    kt_tile += c32 * DH;
    int kxo = kx;
    asm volatile("" : "+v"(kxo));
    Frag8 kf[KT / 32];
    auto read_k = [&](int u, int kt) __attribute__((always_inline)) {
      kf[kt].u = *reinterpret_cast<const uint4*>(&kt_tile[kt * 32 * DH + 8 * ((2 * u + g) ^ kxo)]);
    };
#pragma unroll
    for (int kt = 0; kt < KT / 32; ++kt) read_k(0, kt);
#pragma unroll
    for (int kt = 0; kt < KT / 32; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) st[kt][r] = 0.f;
      st[kt] = mfma32(onek.v, mq.v, st[kt]);
    }
#pragma unroll
    for (int u = 0; u < DSTEPS; ++u) {
#pragma unroll
      for (int kt = 0; kt < KT / 32; ++kt) {
        st[kt] = mfma32(kf[kt].v, qf[u].v, st[kt]);
        if (u + 1 < DSTEPS) read_k(u + 1, kt);
        // (kept in this order: the compiler would otherwise issue each read
        // just before its MFMA, too late to cover the LDS latency)
        __builtin_amdgcn_sched_barrier(0);
      }
      hook(u);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto softmax = [&](int j) __attribute__((always_inline)) {
    const int j0 = (it_first + j) * KT;
    // causal mask only where the tile reaches past the wave's first query, the
    // window's lower edge only where the tile starts below the wave's last one
    if (j0 + KT - 1 > wave_limit_min || (WIN && j0 < wave_lo_max)) {
#pragma unroll
      for (int kt = 0; kt < KT / 32; ++kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + kt * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (key > limit || (WIN && key < lo)) st[kt][r] = -INFINITY;
        }
        // (keeps the compiler from holding all 64 comparisons in scalar registers)
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // maximum: one chain per 32-key block, then across blocks and lane halves
    float bmax[KT / 32];
#pragma unroll
    for (int kt = 0; kt < KT / 32; ++kt) {
      bmax[kt] = st[kt][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) bmax[kt] = fmaxf(bmax[kt], st[kt][r]);
    }
    // (the maximum gates the exponentials: the LDS pipe, busy with the other
    // waves' fragment reads, would delay a shuffle)
    const float tmax = max_halves(fmaxf(fmaxf(bmax[0], bmax[1]), fmaxf(bmax[2], bmax[3])));
    // tmax is relative to mref
    if (__any(tmax + mref > m_run + kRescale)) {
      const float m_new = float((__bf16)fmaxf(m_run, tmax + mref));
      const float corr = m_new == -INFINITY ? 1.f : exp2f(m_run - m_new);
      l_run *= corr;
#pragma unroll
      for (int t = 0; t < DTILES; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[t][r] *= corr;
      m_run = m_new;
      // this tile's scores were taken against the old reference
      const float shift = (m_new == -INFINITY ? 0.f : m_new) - mref;
#pragma unroll
      for (int kt = 0; kt < KT / 32; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) st[kt][r] -= shift;
      mref += shift;
      mq.v[0] = g == 0 ? (__bf16)(-mref) : (__bf16)0.f;
    }
#pragma unroll
    for (int kt = 0; kt < KT / 32; ++kt)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // v_exp_f32 directly: probabilities below 2^-126 flush to zero
          pb[kt][u].v[e] = (__bf16)__builtin_amdgcn_exp2f(st[kt][8 * u + e]);
        }
        // the normaliser adds the probabilities as rounded for P V
        l_run = add_bf16x8(pb[kt][u], l_run);
      }
    // the probabilities and the normaliser are computed here, not moved past
    // the barrier into the matrix segment
#pragma unroll
    for (int kt = 0; kt < KT / 32; ++kt)
#pragma unroll
      for (int u = 0; u < 2; ++u) asm volatile("" : "+v"(pb[kt][u].v));
    asm volatile("" : "+v"(l_run));
  };
  // transposing-read address of this lane within a V tile (see above): key
  // row 4 g + li / 4 (+ 32 kt + 16 u, + 8), features 32 t + 16 ((lane >> 4) & 1)
  // + 4 (li & 3), whose slot lies in the slot quarter t ^ vq of the row
  const int li = lane & 15;
  const int vrow = 4 * g + (li >> 2);
  const int vq = vswz(vrow) >> 2;
  const int vlane = vrow * DH + 16 * ((lane >> 4) & 1) + 4 * (li & 3);
  // P_j from the buffer `v_tile`: eight groups of 16 keys (kt, u); the fragment
  // of feature tile t for group e + 1 is read right after the MFMA of group e
  // that last used its registers; after group e, hook(e)
  auto pv = [&](const bf16_t* v_tile, auto&& hook) __attribute__((always_inline)) {
    const bf16_t* vt = v_tile + vlane;
    union VFrag {
      uint2 h[2];
      bf16x8_t v;
    };
    VFrag vf[DTILES];
    int vqo = vq;
    asm volatile("" : "+v"(vqo));
    // keys 16 e + 4 g + {0..3} and + {8..11} of feature t*32 + c32
    auto read_v = [&](int e, int t) __attribute__((always_inline)) {
      const bf16_t* vtt = vt + 16 * e * DH + 32 * (t ^ vqo);
      vf[t].h[0] = lds_read_tr16(vtt);
      vf[t].h[1] = lds_read_tr16(vtt + 8 * DH);
    };
#pragma unroll
    for (int t = 0; t < DTILES; ++t) read_v(0, t);
#pragma unroll
    for (int e = 0; e < KT / 16; ++e) {
#pragma unroll
      for (int t = 0; t < DTILES; ++t) {
        o[t] = mfma32(vf[t].v, pb[e >> 1][e & 1].v, o[t]);
        if (e + 1 < KT / 16) read_v(e + 1, t);
        __builtin_amdgcn_sched_barrier(0);  // (order kept, as for the scores)
      }
      hook(e);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // completion of this wave's direct loads
  auto wait_loads = []() __attribute__((always_inline)) { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };
  // a workgroup barrier that waits for this wave's LDS reads but not for its
  // direct loads (__syncthreads' fence would wait for those too; their own
  // wait comes a segment later)
  auto barrier_lds = []() __attribute__((always_inline)) {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  auto no_hook = [](int) __attribute__((always_inline)) {};

  // prologue: every wave loads its eighth of K_0 and of (V_0, K_1)
  if (tid < 6) counters[tid] = 0;
  {
    const TileSrc k0 = tile_src(std::false_type(), it_first);
#pragma unroll
    for (int i = 0; i < NI; ++i) load_one(std::false_type(), k0, K0, NI * wave_u + i);
    if (n_it > 1) {
      const TileSrc v0 = tile_src(std::true_type(), it_first);
      const TileSrc k1 = tile_src(std::false_type(), it_first + 1);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        load_one(std::true_type(), v0, V0, NI * wave_u + i);
        load_one(std::false_type(), k1, K1, NI * wave_u + i);
      }
    } else {
      const TileSrc v0 = tile_src(std::true_type(), it_first);
#pragma unroll
      for (int i = 0; i < NI; ++i) load_one(std::true_type(), v0, V0, NI * wave_u + i);
    }
  }
  __syncthreads();
  // tickets: per SIMD (hardware register HW_ID, bits 5:4), then among the
  // SIMDs' first waves and among their second waves
  int ticket = 0, idx = 0;
  if (lane == 0) {
    ticket = atomicAdd(&counters[(__builtin_amdgcn_s_getreg(0xF804) >> 4) & 3], 1);
    idx = atomicAdd(&counters[ticket == 0 ? 4 : 5], 1);
  }
  ticket = __builtin_amdgcn_readfirstlane(ticket);
  idx = __builtin_amdgcn_readfirstlane(idx);
  wait_loads();  // this wave's eighths of K_0, V_0 and K_1
  __syncthreads();
  const bool paired = counters[4] == 4 && counters[5] == 4;  // one leading, one trailing wave on each SIMD
  const bool trail = paired && ticket != 0;
  // instructions of a tile this wave loads (a quarter paired, else an eighth)
  // and the first of them
  const int nq = paired ? 2 * NI : NI;
  const int q_first = paired ? 2 * NI * idx : NI * wave_u;
  // the loads of this wave in [P_j, S_j+1] (j = -1: the segment of S_0), one
  // instruction after each 16-feature step of S_j+1: paired, the leading waves
  // load K_j+2 and the trailing ones V_j+2; unpaired, every wave loads K_j+2
  // and V_j+1.  K_j+2 goes into the buffer of K_j, V_j+2 into that of V_j and
  // V_j+1 into that of V_j-1, each read for the last time by both halves in
  // or before this wave's P_j.
  struct Plan {
    TileSrc k, v;
    bf16_t* kdst;
    bf16_t* vdst;
    int nk, nv;
  };
  auto plan_for = [&](auto P, int j) __attribute__((always_inline)) {
    using Q = std::integral_constant<int, 1 - decltype(P)::value>;
    Plan pl;
    pl.nk = 0;
    pl.nv = 0;
    pl.kdst = kbuf(P);  // K_j+2: the buffer of K_j
    if (j >= 0 && (!paired || !trail) && j + 2 < n_it) {
      pl.nk = nq;
      pl.k = tile_src(std::false_type(), it_first + j + 2);
    }
    if (paired) {
      pl.vdst = vbuf(P);  // V_j+2: the buffer of V_j
      if (trail && j + 2 < n_it) {
        pl.nv = nq;
        pl.v = tile_src(std::true_type(), it_first + j + 2);
      }
    } else {
      pl.vdst = vbuf(Q());  // V_j+1: the buffer of V_j-1
      if (j >= 0 && j + 1 < n_it) {
        pl.nv = nq;
        pl.v = tile_src(std::true_type(), it_first + j + 1);
      }
    }
    return pl;
  };
  auto plan_hook = [&](const Plan& pl) __attribute__((always_inline)) {
    return [&pl, &load_one, q_first](int u) __attribute__((always_inline)) {
      if (u < pl.nk) load_one(std::false_type(), pl.k, pl.kdst, q_first + u);
      else if (u - pl.nk < pl.nv) load_one(std::true_type(), pl.v, pl.vdst, q_first + u - pl.nk);
    };
  };
  if (trail) barrier_lds();
  {
    // j = -1 (parity 1): the trailing waves load V_1 into the buffer of V_-1
    const Plan pl = plan_for(One(), -1);
    __builtin_amdgcn_s_setprio(1);
    scores(K0, plan_hook(pl));
    __builtin_amdgcn_s_setprio(0);
  }
  barrier_lds();
  // one tile: X_j, then [P_j, S_j+1] with this wave's loads; P the parity of j
  auto step = [&](auto P, int j) __attribute__((always_inline)) {
    using Q = std::integral_constant<int, 1 - decltype(P)::value>;
    // X_j; a leading wave's loads from its last [P, S] complete at its end
    __builtin_amdgcn_sched_barrier(0);
    softmax(j);
    if (!trail) wait_loads();
    __syncthreads();
    // [P_j, S_j+1], at raised priority: the SIMD's other wave is in its X,
    // whose vector instructions would otherwise be issued first whenever that
    // wave is the older one, leaving the matrix core waiting
    const bool more = j + 1 < n_it;
    __builtin_amdgcn_s_setprio(1);
    pv(vbuf(P), no_hook);
    __builtin_amdgcn_sched_barrier(0);
    bool just_issued = false;  // DSTEPS loads issued below, the newest in flight
    if (more) {
      const Plan pl = plan_for(P, j);
      const bool is_k = pl.nk > 0;
      const TileSrc& ts = is_k ? pl.k : pl.v;
      if (pl.nk + pl.nv == 0) {
        scores(kbuf(Q()), no_hook);
      } else if (pl.nk + pl.nv == DSTEPS && (pl.nk == 0 || pl.nv == 0) && ts.contiguous) {
        just_issued = true;
        // one contiguous tile, one instruction a step: no branch inside the
        // step sequence (a branch there costs the fragment reads' overlap)
        const char* base = ts.base;
        bf16_t* dst = is_k ? pl.kdst : pl.vdst;
        uint32_t ob = is_k ? koff0 : voff;
        asm volatile("" : "+v"(ob));
        scores(kbuf(Q()), [&](int u) __attribute__((always_inline)) {
          // q_first is a multiple of NI: q mod NI = u mod NI
          dma_tile(base, dst, q_first + u, ob ^ (is_k ? 64u * uint32_t(u & (NI - 1)) : 0u));
        });
      } else {
        scores(kbuf(Q()), plan_hook(pl));
      }
    }
    __builtin_amdgcn_s_setprio(0);
    // a trailing wave's loads from its last [P, S] complete here (those of
    // this one may stay in flight: they are read two segments later)
    if (trail) {
      if (just_issued) {
        if constexpr (DSTEPS == 8)
          asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        else
          asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      } else {
        wait_loads();
      }
    }
    // the trailing waves' last segment is the block's last: no barrier after it
    if (more || !trail) barrier_lds();
  };
  for (int j = 0; j < n_it; j += 2) {
    step(Zero(), j);
    if (j + 1 < n_it) step(One(), j + 1);
  }
  l_run += __shfl_xor(l_run, 32, 64);
  if (qi < n_b) {
    const float inv = 1.f / l_run;
    float* orow = out + (size_t(b) * n_max + qi) * s.model_width + size_t(h) * DH;
#pragma unroll
    for (int t = 0; t < DTILES; ++t)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        float4 w;
        w.x = o[t][4 * rr + 0] * inv;
        w.y = o[t][4 * rr + 1] * inv;
        w.z = o[t][4 * rr + 2] * inv;
        w.w = o[t][4 * rr + 3] * inv;
        const int d = t * 32 + 8 * rr + 4 * g;
        *reinterpret_cast<float4*>(orow + d) = w;
        if (!(isfinite(w.x) && isfinite(w.y) && isfinite(w.z) && isfinite(w.w)))
          flag_min(&s.err->output, (size_t(b) * n_max + qi) * s.model_width + size_t(h) * DH + d);
      }
  }
}

// Chunk attention with the two waves of each SIMD in different roles (bf16,
// d_h = 128, no window; the same work items and results as the general
// kernel).  The workgroup takes 256 queries in four groups of 64.  Wave p
// (p < 4) forms the scores and probabilities of group p, its two 32-query
// blocks sharing every K fragment read; wave p + 4 accumulates O^T += V^T P^T
// for the same queries, the two blocks sharing every V^T fragment read, and
// takes the probabilities through LDS, adding them up as it goes.  Per query
// and key, LDS carries half the fragment bytes of the general kernel's 32
// queries per wave, plus the probabilities.  Keys pass in 64-row tiles, three
// buffers each of K and V and two of probabilities (160 KB).  Step t: the
// scoring wave runs the scores of tile t's second 32 keys and of tile t + 1's
// first 32 keys, each interleaved with the exponentials of the 32 keys before
// (two register sets); the accumulating wave runs P V of tile t - 1 and loads
// K_t+2 and V_t+1; one barrier.  Each query keeps one fixed reference, the
// bf16-rounded maximum of its first 32 scores, and is never rescaled: the
// probabilities relative to it lose nothing in floating point unless a later
// score passes it by ~2^7 (base 2), which makes a sum or an accumulator
// non-finite; a work item whose sums pass 2^100 or whose outputs come out
// non-finite writes nothing, is marked in `redo` and is recomputed by the
// general kernel, which raises its reference as the scores rise.
template <int DH>
__global__ __launch_bounds__(2 * kChunkQueryTile) __attribute__((amdgpu_waves_per_eu(2, 2))) void attend_split_kernel(
    DevState s, int n_max, int per_seq_rows, ChunkOrder order, float* __restrict__ out) {
  static_assert(DH == 128, "the split path takes d_h = 128");
  constexpr int KT = 64;
  static_assert(kMinBlockRows % KT == 0, "a key tile must stay inside one block");
  constexpr int DSTEPS = DH / 16;
  constexpr int DTILES = DH / 32;
  constexpr int SPR = DH / 8;
  constexpr int RPS = 16 / SPR;
  constexpr int RPL = 64 / SPR;       // rows of one load instruction
  constexpr int NLD = KT / RPL / 4;   // load instructions of a tile per loading wave
  constexpr int QT = kChunkQueryTile;
  static_assert(QT == 256, "four groups of 64 queries");
  constexpr int TILE = KT * DH;
  constexpr int PFR = 4 * 8 * 64;     // 16-byte pieces of a probability buffer
  __shared__ __attribute__((aligned(16))) bf16_t K0[TILE];
  __shared__ __attribute__((aligned(16))) bf16_t K1[TILE];
  __shared__ __attribute__((aligned(16))) bf16_t K2[TILE];
  __shared__ __attribute__((aligned(16))) bf16_t V0[TILE];
  __shared__ __attribute__((aligned(16))) bf16_t V1[TILE];
  __shared__ __attribute__((aligned(16))) bf16_t V2[TILE];
  __shared__ __attribute__((aligned(16))) uint4 P0[PFR];
  __shared__ __attribute__((aligned(16))) uint4 P1[PFR];
  auto kbuf = [&](auto i) __attribute__((always_inline)) -> bf16_t* {
    constexpr int v = decltype(i)::value % 3;
    if constexpr (v == 0) return K0; else if constexpr (v == 1) return K1; else return K2;
  };
  auto vbuf = [&](auto i) __attribute__((always_inline)) -> bf16_t* {
    constexpr int v = decltype(i)::value % 3;
    if constexpr (v == 0) return V0; else if constexpr (v == 1) return V1; else return V2;
  };
  auto pbuf = [&](auto i) __attribute__((always_inline)) -> uint4* {
    if constexpr (decltype(i)::value % 2 == 0) return P0; else return P1;
  };

  const int H = s.heads;
  const int item = blockIdx.x / H;
  const int slot = blockIdx.x - item * H;
  const int h = (s.kv_heads < H && (H & 7) == 0) ? (slot & 7) * (H >> 3) + (slot >> 3) : slot;
  int b, qt;
  if (order.count) {
    b = order.item[item] >> 16;
    qt = order.item[item] & 0xffff;
  } else {
    b = item / order.qtiles;
    qt = order.qtiles - 1 - (item - b * order.qtiles);
  }
  const int tid = threadIdx.x;
  const int n_b = per_seq_rows ? s.rows[b] : n_max;
  if (qt * QT >= n_b) {
    if (tid == 0) s.redo[blockIdx.x] = 0;
    return;
  }
  const int len = min(max(s.len[b], 0), s.capacity);
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave & 3;
  const int g = lane >> 5;
  const int c32 = lane & 31;
  const int qbase = qt * QT + 64 * grp;
  const int i_max = min(qt * QT + QT - 1, n_b - 1);
  const int total = len + i_max + 1;
  const int n_it = (total + KT - 1) / KT;  // key tiles of the workgroup, >= 1
  // tiles holding a key that some query of the group sees (none when the
  // group starts past the chunk's last row)
  const int grp_tiles = qbase < n_b ? (len + min(qbase + 63, n_b - 1)) / KT + 1 : 0;
  const int grp_limit_min = len + min(qbase, n_b - 1);
  const size_t lane_id = size_t(b) * H + h;
  const int hk = h / (H / s.kv_heads);
  const size_t kv_lane = size_t(b) * s.kv_heads + hk;
  const bf16_t* kc = static_cast<const bf16_t*>(s.keys);
  const bf16_t* vc = static_cast<const bf16_t*>(s.values);
  const bf16_t* kn = static_cast<const bf16_t*>(s.cand_k) + kv_lane * n_max * DH;
  const bf16_t* vn = static_cast<const bf16_t*>(s.cand_v) + kv_lane * n_max * DH;

  // tiles: unpadded rows, 16-byte slots permuted as in the general kernel
  auto kswz = [](int r) __attribute__((always_inline)) { return (r / RPS) & (SPR - 1); };
  auto vswz = [](int r) __attribute__((always_inline)) { return 4 * ((r / RPS) & (SPR / 4 - 1)); };
  typedef __attribute__((address_space(3))) void lds_void_t;
  auto wait_loads = []() __attribute__((always_inline)) { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };
  auto barrier_lds = []() __attribute__((always_inline)) {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  using Z0 = std::integral_constant<int, 0>;
  using Z1 = std::integral_constant<int, 1>;
  using Z2 = std::integral_constant<int, 2>;
  using Z3 = std::integral_constant<int, 3>;
  using Z4 = std::integral_constant<int, 4>;
  using Z5 = std::integral_constant<int, 5>;
  // steps 0 .. n_it, each ending in the workgroup barrier; the step's index
  // modulo 6 as a type (it selects the buffers)
  auto run_steps = [&](auto&& step) __attribute__((always_inline)) {
    for (int t0 = 0;; t0 += 6) {
      step(Z0(), t0);
      if (t0 + 1 > n_it) break;
      step(Z1(), t0 + 1);
      if (t0 + 2 > n_it) break;
      step(Z2(), t0 + 2);
      if (t0 + 3 > n_it) break;
      step(Z3(), t0 + 3);
      if (t0 + 4 > n_it) break;
      step(Z4(), t0 + 4);
      if (t0 + 5 > n_it) break;
      step(Z5(), t0 + 5);
      if (t0 + 6 > n_it) break;
    }
  };

  if (wave < 4) {
    // ------------------------------------------------ scores and probabilities
    // The scores go by 32-key blocks (block 2 t + kb: keys 32 kb .. of tile
    // t): while one block's probabilities are formed (vector unit), the next
    // block's scores run (matrix cores), in two sets of registers by kb.  Step
    // t: [scores of block (t, 1) | probabilities of (t, 0)], then [scores of
    // (t + 1, 0) | probabilities of (t, 1)].
    Frag8 qf[2][DSTEPS];
    int limit[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qe = min(qbase + 32 * qb + c32, n_b - 1);
      limit[qb] = len + qe;
      const bf16_t* qp = static_cast<const bf16_t*>(s.q) + (lane_id * n_max + qe) * DH;
#pragma unroll
      for (int u = 0; u < DSTEPS; ++u) qf[qb][u].u = *reinterpret_cast<const uint4*>(qp + 16 * u + 8 * g);
    }
    float mref[2] = {0.f, 0.f};  // the fixed references, subtracted before the exponentials
    f32x16_t st[2][2];           // [kb][query block]
    const int kx = kswz(c32);
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    // S^T of the 32 keys at rows 32 KB .. of a K tile into set KB, each K
    // fragment read three 16-feature steps ahead; hook(u) after step u's MFMAs
    auto scores = [&](auto KB, const bf16_t* ktile, auto&& hook) __attribute__((always_inline)) {
      constexpr int kb = decltype(KB)::value;
      const bf16_t* kr = ktile + (32 * kb + c32) * DH;
      int kxo = kx;
      asm volatile("" : "+v"(kxo));
      Frag8 kf[3];
      auto read_k = [&](int u) __attribute__((always_inline)) {
        kf[u % 3].u = *reinterpret_cast<const uint4*>(&kr[8 * ((2 * u + g) ^ kxo)]);
      };
      read_k(0);
      read_k(1);
      read_k(2);
      f32x16_t z;
#pragma unroll
      for (int r = 0; r < 16; ++r) z[r] = 0.f;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < DSTEPS; ++u) {
        st[kb][0] = mfma32(kf[u % 3].v, qf[0][u].v, u == 0 ? z : st[kb][0]);
        st[kb][1] = mfma32(kf[u % 3].v, qf[1][u].v, u == 0 ? z : st[kb][1]);
        if (u + 3 < DSTEPS) read_k(u + 3);
        hook(u);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // keys past a query's last key, in set KB holding block (t, KB)
    auto mask = [&](auto KB, int t) __attribute__((always_inline)) {
      constexpr int kb = decltype(KB)::value;
      const int j0 = t * KT + 32 * kb;
      if (j0 + 31 > grp_limit_min) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = j0 + 8 * (r >> 2) + 4 * g + (r & 3);
            if (key > limit[qb]) st[kb][qb][r] = -INFINITY;
          }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // slice i (of 8) of the probabilities of set KB: four exponentials of
    // fragment f = (2 KB + qb) 2 + half, (qb, half) = (i / 4, (i / 2) mod 2);
    // a fragment complete goes to the group's slice of the P buffer at
    // f 64 + lane
    Frag8 pcur;
    auto prob_slice = [&](auto KB, uint4* pdst, int i) __attribute__((always_inline)) {
      constexpr int kb = decltype(KB)::value;
      const int qb = i >> 2, hf = (i >> 1) & 1, part = i & 1;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        pcur.v[4 * part + e] = (__bf16)__builtin_amdgcn_exp2f(st[kb][qb][8 * hf + 4 * part + e] - mref[qb]);
      if (part) pdst[grp * 8 * 64 + ((2 * kb + qb) * 2 + hf) * 64 + lane] = pcur.u;
    };
    barrier_lds();  // K_0, K_1 in LDS
    // block (0, 0) and the fixed references: maxima of its keys
    if (grp_tiles > 0) {
      scores(S0(), K0, [](int) {});
      mask(S0(), 0);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float m = st[0][qb][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) m = fmaxf(m, st[0][qb][r]);
        mref[qb] = float((__bf16)max_halves(m));
      }
    }
    run_steps([&](auto T, int t) __attribute__((always_inline)) {
      using TC = std::integral_constant<int, decltype(T)::value>;            // K_t
      using TN = std::integral_constant<int, (decltype(T)::value + 1) % 6>;  // K_t+1
      const int lim = min(n_it, grp_tiles);
      if (t < lim) {
        uint4* pdst = pbuf(T);
        // [scores of (t, 1) | probabilities of (t, 0)]
        __builtin_amdgcn_s_setprio(2);
        scores(S1(), kbuf(TC()), [&](int u) __attribute__((always_inline)) { prob_slice(S0(), pdst, u); });
        __builtin_amdgcn_s_setprio(0);
        mask(S1(), t);
        // [scores of (t + 1, 0) | probabilities of (t, 1)]
        if (t + 1 < lim) {
          __builtin_amdgcn_s_setprio(2);
          scores(S0(), kbuf(TN()), [&](int u) __attribute__((always_inline)) { prob_slice(S1(), pdst, u); });
          __builtin_amdgcn_s_setprio(0);
          mask(S0(), t + 1);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) prob_slice(S1(), pdst, i);
        }
      }
      barrier_lds();
    });
    barrier_lds();  // the accumulating waves' verdicts
    return;
  }

  // ----------------------------------------------------------- P V and loads
  const int lr = lane / SPR, lc = lane & (SPR - 1);
  const uint32_t voff = uint32_t(lr * DH + 8 * (lc ^ vswz(lr))) * 2u;
  const uint32_t koff0 = uint32_t(lr * DH + 8 * (lc ^ kswz(lr))) * 2u;
  auto block_base = [&](int r0) __attribute__((always_inline)) -> ptrdiff_t {
    if (!s.paged) return kv_block_base(s, b, hk, r0);
    typedef const __attribute__((address_space(4))) int32_t* const_i32_t;
    const int lg = s.block_rows_log2;
    const int blk = max(((const_i32_t)s.block_table)[size_t(b) * s.table_width + (r0 >> lg)], 0);
    return (ptrdiff_t(size_t(blk) * s.kv_heads + hk) << lg) * DH - ptrdiff_t((r0 >> lg) << lg) * DH;
  };
  struct TileSrc {
    const char* base;
    const bf16_t* cached;
    const bf16_t* chunk;
    int j0;
    bool contiguous;
  };
  auto tile_src = [&](auto is_v, int t) __attribute__((always_inline)) {
    TileSrc src;
    const bf16_t* cache = is_v ? vc : kc;
    src.chunk = is_v ? vn : kn;
    src.j0 = t * KT;
    src.cached = cache + block_base(min(src.j0, max(len - 1, 0)));
    src.contiguous = src.j0 + KT <= len || (src.j0 >= len && src.j0 + KT <= total);
    src.base = reinterpret_cast<const char*>(src.j0 < len ? src.cached + ptrdiff_t(src.j0) * DH
                                                          : src.chunk + size_t(src.j0 - len) * DH);
    return src;
  };
  auto dma_tile = [&](const char* first, bf16_t* tile, int q, uint32_t off) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(first), (short)0, KT * DH * 2, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(tile + q * RPL * DH), 16, off, q * (RPL * DH * 2), 0, 0);
  };
  // load instruction q (rows RPL q ..) of tile src into `tile`.  A tile that
  // is not one run of rows is loaded row by row, the lanes of cache rows and
  // those of chunk rows each through a descriptor of their own (rows past the
  // last key repeat it; the mask hides them).  (All loads take the buffer
  // form: the compiler counts the global form as an LDS access too, and then
  // waits for every LDS read in flight behind it.)
  auto load_one = [&](auto is_v, const TileSrc& src, bf16_t* tile, int q) __attribute__((always_inline)) {
    uint32_t off = is_v ? voff : koff0;
    asm volatile("" : "+v"(off));
    if (!is_v) off ^= 64u * uint32_t(q & 3);
    if (src.contiguous) {
      dma_tile(src.base, tile, q, off);
    } else {
      int row = lr;
      asm volatile("" : "+v"(row));
      const int j = min(src.j0 + RPL * q + row, total - 1);
      const uint32_t in_row = off & uint32_t(DH * 2 - 1);
      const uint32_t roff = uint32_t(j - src.j0) * uint32_t(DH * 2) + in_row;
      if (j < len) {
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<bf16_t*>(src.cached + ptrdiff_t(src.j0) * DH), (short)0, KT * DH * 2, 0x00020000);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(tile + q * RPL * DH), 16, roff, 0, 0, 0);
      } else {
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<bf16_t*>(src.chunk + (ptrdiff_t(src.j0) - len) * DH), (short)0, KT * DH * 2, 0x00020000);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(tile + q * RPL * DH), 16, roff, 0, 0, 0);
      }
    }
  };
  // this wave's quarter of the tiles: instructions NLD grp ..
  const int q0 = NLD * grp;
  {
    const TileSrc k0 = tile_src(std::false_type(), 0);
    const TileSrc v0 = tile_src(std::true_type(), 0);
#pragma unroll
    for (int i = 0; i < NLD; ++i) load_one(std::false_type(), k0, K0, q0 + i);
#pragma unroll
    for (int i = 0; i < NLD; ++i) load_one(std::true_type(), v0, V0, q0 + i);
    if (n_it > 1) {
      const TileSrc k1 = tile_src(std::false_type(), 1);
#pragma unroll
      for (int i = 0; i < NLD; ++i) load_one(std::false_type(), k1, K1, q0 + i);
    }
  }

  float l_run[2] = {0.f, 0.f};
  f32x16_t o[2][DTILES];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int t = 0; t < DTILES; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[qb][t][r] = 0.f;
  // transposing-read address of this lane within a V tile (as in the general
  // kernel): key row 4 g + li / 4 (+ 16 e, + 8), features 32 t + 16 ((lane >> 4)
  // & 1) + 4 (li & 3), in the slot quarter t ^ vq of the row
  const int li = lane & 15;
  const int vrow = 4 * g + (li >> 2);
  const int vq = vswz(vrow) >> 2;
  const int vlane = vrow * DH + 16 * ((lane >> 4) & 1) + 4 * (li & 3);
  union VFrag {
    uint2 hh[2];
    bf16x8_t v;
  };
  // O^T += V^T P^T over the 64 keys of a V tile: 16 steps k (16-key group
  // k / 4, feature tile k mod 4), V^T fragments read three steps ahead;
  // hook(k) after step k
  auto pv = [&](const bf16_t* vtile, const uint4* psrc, auto&& hook) __attribute__((always_inline)) {
    Frag8 pf[8];
    const uint4* pr = psrc + grp * 8 * 64 + lane;
#pragma unroll
    for (int f = 0; f < 8; ++f) pf[f].u = pr[f * 64];
    // the sums add the probabilities as rounded (fragment f: query block (f >> 1) & 1)
#pragma unroll
    for (int f = 0; f < 8; ++f) l_run[(f >> 1) & 1] = add_bf16x8(pf[f], l_run[(f >> 1) & 1]);
    const bf16_t* vt = vtile + vlane;
    int vqo = vq;
    asm volatile("" : "+v"(vqo));
    VFrag vf[4];
    auto read_v = [&](int k) __attribute__((always_inline)) {
      const bf16_t* vtt = vt + 16 * (k >> 2) * DH + 32 * ((k & 3) ^ vqo);
      vf[k & 3].hh[0] = lds_read_tr16(vtt);
      vf[k & 3].hh[1] = lds_read_tr16(vtt + 8 * DH);
    };
    read_v(0);
    read_v(1);
    read_v(2);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int e = k >> 2, t = k & 3;
      o[0][t] = mfma32(vf[k & 3].v, pf[(2 * (e >> 1) + 0) * 2 + (e & 1)].v, o[0][t]);
      o[1][t] = mfma32(vf[k & 3].v, pf[(2 * (e >> 1) + 1) * 2 + (e & 1)].v, o[1][t]);
      if (k + 3 < 16) read_v(k + 3);
      hook(k);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  wait_loads();
  barrier_lds();  // K_0, V_0, K_1 in LDS
  run_steps([&](auto T, int t) __attribute__((always_inline)) {
    using TK = std::integral_constant<int, (decltype(T)::value + 2) % 6>;  // K_t+2 (the buffer of K_t-1)
    using TV = std::integral_constant<int, (decltype(T)::value + 1) % 6>;  // V_t+1, and P_t-1
    using TR = std::integral_constant<int, (decltype(T)::value + 5) % 6>;  // V_t-1
    const bool lk = t + 2 < n_it, lv = t + 1 < n_it;
    TileSrc sk, sv;
    if (lk) sk = tile_src(std::false_type(), t + 2);
    if (lv) sv = tile_src(std::true_type(), t + 1);
    auto load_all = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < NLD; ++i)
        if (lk) load_one(std::false_type(), sk, kbuf(TK()), q0 + i);
#pragma unroll
      for (int i = 0; i < NLD; ++i)
        if (lv) load_one(std::true_type(), sv, vbuf(TV()), q0 + i);
    };
    // this step's loads: spread over the products when both tiles are one run
    // of rows, else issued before them
    const bool wk = t >= 1 && t - 1 < grp_tiles;
    const bool fast = lk && lv && sk.contiguous && sv.contiguous;
    if (!fast || !wk) load_all();
    if (wk) {
      const char* kbase = sk.base;
      const char* vbase = sv.base;
      uint32_t ko = koff0, vo = voff;
      asm volatile("" : "+v"(ko), "+v"(vo));
      pv(vbuf(TR()), pbuf(TV()), [&](int k) __attribute__((always_inline)) {
        if (fast) {
          if (k < NLD)
            dma_tile(kbase, kbuf(TK()), q0 + k, ko ^ (64u * uint32_t(k & 3)));
          else if (k < 2 * NLD)
            dma_tile(vbase, vbuf(TV()), q0 + k - NLD, vo);
        }
      });
    }
    // K_t+2 (first read in the next step) and V_t complete; V_t+1, loaded
    // after K_t+2, may stay in flight
    if (lv)
      asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else
      wait_loads();
    barrier_lds();
  });
  // the verdict of each group (in a P buffer no longer read)
  int* verdict = reinterpret_cast<int*>(P0);
  float inv[2];
  bool bad = false;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l = l_run[qb] + __shfl_xor(l_run[qb], 32, 64);
    bad |= !(l > 0.f && l < 0x1p100f);
    inv[qb] = 1.f / l;
#pragma unroll
    for (int t = 0; t < DTILES; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) bad |= !isfinite(o[qb][t][r]);
  }
  const bool wave_bad = __any(bad);
  if (lane == 0) verdict[grp] = (qbase < n_b && wave_bad) ? 1 : 0;
  barrier_lds();
  const bool redo_item = (verdict[0] | verdict[1] | verdict[2] | verdict[3]) != 0;
  if (grp == 0 && lane == 0) s.redo[blockIdx.x] = redo_item ? 1 : 0;
  if (redo_item) return;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qi = qbase + 32 * qb + c32;
    if (qi >= n_b) continue;
    float* orow = out + (size_t(b) * n_max + qi) * s.model_width + size_t(h) * DH;
#pragma unroll
    for (int t = 0; t < DTILES; ++t)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        float4 w;
        w.x = o[qb][t][4 * rr + 0] * inv[qb];
        w.y = o[qb][t][4 * rr + 1] * inv[qb];
        w.z = o[qb][t][4 * rr + 2] * inv[qb];
        w.w = o[qb][t][4 * rr + 3] * inv[qb];
        *reinterpret_cast<float4*>(orow + t * 32 + 8 * rr + 4 * g) = w;
      }
  }
}

inline hipStream_t st(void* p) { return static_cast<hipStream_t>(p); }

}  // namespace

// Projections proj_first .. proj_first + nproj - 1 (0 W_q, 1 W_k, 2 W_v, 3 W_o)
// of M = B * n_max rows of x.  Returns -1 when the shape has no MFMA kernel (the
// caller then uses the vector kernels), else 0 or a HIP error code.
template <typename XT>
int mfma_project_t(const DevState& s, const XT* xb, int n_max, int per_seq_rows, int proj_first, int nproj) {
  if (s.dtype != KVC_BF16 || s.model_width % 128 != 0) return -1;
  const int M = s.batch * n_max;
  // output columns of the launch: Q, K, V (K and V kv_width wide) or O
  const int cols = nproj == 3 ? s.model_width + 2 * s.kv_width : s.model_width;
  const int kv_cols = nproj == 3 ? s.kv_width : s.model_width;
  if (M <= 64) {
    if (kv_cols % 64 != 0) return -1;
    const int tiles = cols / 64;
    const int mtiles = (M + 31) / 32;
    // split the reduction axis until the launch has about 512 blocks (one row
    // tile and a fixed chunk count only: the partial buffer holds 32 rows)
    const int nch = s.model_width / SKC;
    int split = 1;
    if (s.proj_partials && mtiles == 1 && (nch == 16 || nch == 32 || nch == 64))
      while (split < kSkinnySplitMax && tiles * split < 512 && nch % (2 * split) == 0 && nch / (2 * split) >= SRING)
        split *= 2;
    dim3 grid(tiles, mtiles, split);
#define KVC_SKINNY(NCH_, SPLIT_)                                                                           \
  hipLaunchKernelGGL((project_skinny_kernel<NCH_, XT, SPLIT_>), grid, dim3(256), 0, st(s.stream), s, xb, M, n_max, \
                     per_seq_rows, proj_first)
#define KVC_SKINNY_SPLITS(NCH_)      \
  switch (split) {                   \
    case 1: KVC_SKINNY(NCH_, 1); break; \
    case 2: KVC_SKINNY(NCH_, 2); break; \
    case 4: KVC_SKINNY(NCH_, 4); break; \
    default: KVC_SKINNY(NCH_, 8); break; \
  }
    switch (s.model_width) {
      case 2048: KVC_SKINNY_SPLITS(16); break;
      case 4096: KVC_SKINNY_SPLITS(32); break;
      case 8192: KVC_SKINNY_SPLITS(64); break;
      default: KVC_SKINNY(0, 1);
    }
#undef KVC_SKINNY_SPLITS
#undef KVC_SKINNY
    if (split > 1) {
      const int rc = int(hipGetLastError());
      if (rc) return rc;
      const unsigned threads = unsigned(M) * unsigned(tiles) * 32u;
      const dim3 rgrid((threads + 255) / 256);
      switch (split) {
        case 2: hipLaunchKernelGGL(skinny_reduce_kernel<2>, rgrid, dim3(256), 0, st(s.stream), s, M, n_max,
                                   per_seq_rows, proj_first, tiles); break;
        case 4: hipLaunchKernelGGL(skinny_reduce_kernel<4>, rgrid, dim3(256), 0, st(s.stream), s, M, n_max,
                                   per_seq_rows, proj_first, tiles); break;
        default: hipLaunchKernelGGL(skinny_reduce_kernel<8>, rgrid, dim3(256), 0, st(s.stream), s, M, n_max,
                                    per_seq_rows, proj_first, tiles); break;
      }
    }
  } else if (std::is_same<XT, bf16_t>::value && M >= 2048 && s.model_width % GBN == 0 && kv_cols % GBN == 0 &&
             s.head_width % 64 == 0 && int64_t(M) * s.model_width < (int64_t(1) << 31) &&
             int64_t(std::max(s.heads, s.kv_heads)) * s.head_width * s.model_width < (int64_t(1) << 31)) {
    const int m_tiles = (M + GBM - 1) / GBM;
    const int n_tiles = cols / GBN;
    hipLaunchKernelGGL(project_wide_kernel, dim3(m_tiles * n_tiles), dim3(64 * GWAVES), 0, st(s.stream), s,
                       reinterpret_cast<const bf16_t*>(xb), M, n_max, per_seq_rows, proj_first, m_tiles, n_tiles);
  } else {
    if (kv_cols % TBN != 0) return -1;
    dim3 grid(cols / TBN, (M + TBM - 1) / TBM);
    hipLaunchKernelGGL((project_tiled_kernel<XT>), grid, dim3(256), 0, st(s.stream), s, xb, M, n_max,
                       per_seq_rows, proj_first);
  }
  return int(hipGetLastError());
}

int mfma_project(const DevState& s, const void* x, int n_max, int per_seq_rows) {
  return mfma_project_t(s, static_cast<const bf16_t*>(x), n_max, per_seq_rows, 0, 3);
}

int mfma_output_project(const DevState& s, int n_max, int per_seq_rows) {
  return mfma_project_t(s, static_cast<const float*>(s.merged), n_max, per_seq_rows, 3, 1);
}

int mfma_attend_chunk(const DevState& s, int n_max, int per_seq_rows, const ChunkOrder& order, void* out) {
  if (s.dtype != KVC_BF16) return -1;
  const int items = order.count ? order.count : s.batch * order.qtiles;
  if (items == 0) return 0;
  const dim3 grid(unsigned(items) * unsigned(s.heads));
#define KVC_FLASH_LAUNCH(DH_, WIN_, REDO_)                                                               \
  hipLaunchKernelGGL((attend_flash_kernel<DH_, WIN_>), grid, dim3(2 * kChunkQueryTile), 0, st(s.stream), s, n_max, \
                     per_seq_rows, order, static_cast<float*>(out), REDO_)
  if (s.head_width == 128) {
    if (s.window) {
      KVC_FLASH_LAUNCH(128, true, nullptr);
    } else if (s.redo && s.q_bf16) {
      // the role-split kernel, then the general one for the items it handed back
      hipLaunchKernelGGL((attend_split_kernel<128>), grid, dim3(2 * kChunkQueryTile), 0, st(s.stream), s, n_max,
                         per_seq_rows, order, static_cast<float*>(out));
      KVC_FLASH_LAUNCH(128, false, s.redo);
    } else {
      KVC_FLASH_LAUNCH(128, false, nullptr);
    }
  } else if (s.head_width == 64) {
    if (s.window)
      KVC_FLASH_LAUNCH(64, true, nullptr);
    else
      KVC_FLASH_LAUNCH(64, false, nullptr);
#undef KVC_FLASH_LAUNCH
  } else {
    return -1;
  }
  return int(hipGetLastError());
}

}  // namespace kvc
