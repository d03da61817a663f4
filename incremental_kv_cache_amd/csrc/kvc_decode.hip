// bf16 decode attention for gfx950: the HBM-bound core of the cached decode step.
//
// One new query per lane (b, h) reads all t_b = len_b + 1 rows: the len_b
// retained rows of the cache plus the candidate row (Chapter 37, the
// incremental-attention listing; "Count projection rows, not hardware time":
// the newest query still reads every retained row).  The position axis is
// split into tiles of 512 * 2^k rows, one workgroup each: the host picks the
// longest tile that still gives at least 1024 workgroups (512 when a
// workgroup serves several query heads), so a 4096-row lane of 32 x 32 lanes
// is one whole-lane tile and a 32768-row lane of 4 x 32 lanes is eight.
//
// Inside a workgroup a row is read by G = d_h / 8 lanes, one 16-byte load of
// K and one of V per lane; a wave covers 64 / G rows per load and issues U
// such row groups before using any of them, so each lane keeps 2 U loads in
// flight.  q . k is reduced over the G lanes with DPP row operations.  The
// softmax runs online in base 2 (q is pre-scaled by log2(e) / sqrt(d_h)), with
// one rescale per U rows.  Row groups are combined through LDS; then each tile
// either writes the output directly (a single-tile lane) or stores a partial
// (max, sum, weighted values) that a second, small kernel merges by
// log-sum-exp into the lane's head block of the output (merge_heads).  The
// merge stays a separate launch: a device-wide release inside the attention
// kernel would write back L2 once per workgroup on this multi-die part.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "kvc_dev_util.h"
#include "kvc_internal.h"

namespace kvc {

namespace {

using namespace dev;

template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  const int moved = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false);
  return v + __builtin_bit_cast(float, moved);
}

// Sum over aligned groups of G lanes (G = 4, 8 or 16), result in every lane.
template <int G>
__device__ __forceinline__ float group_sum_dpp(float v) {
  v = dpp_add<0xB1>(v);                     // quad_perm [1,0,3,2]
  v = dpp_add<0x4E>(v);                     // quad_perm [2,3,0,1]
  if constexpr (G >= 8) v = dpp_add<0x141>(v);   // row_half_mirror
  if constexpr (G >= 16) v = dpp_add<0x140>(v);  // row_mirror
  return v;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Dot product of 8 bf16 pairs held as 4 packed words, accumulated in float32
// (v_dot2c_f32_bf16: both products exact, summed in float32).
__device__ __forceinline__ float dot8_bf16(const uint32_t (&q)[4], const uint4& k) {
  float d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q[0]), __builtin_bit_cast(bf16x2_t, k.x), 0.f,
                                            false);
  d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q[1]), __builtin_bit_cast(bf16x2_t, k.y), d, false);
  d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q[2]), __builtin_bit_cast(bf16x2_t, k.z), d, false);
  d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q[3]), __builtin_bit_cast(bf16x2_t, k.w), d, false);
  return d;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(__builtin_bit_cast(uint16_t, (__bf16)lo)) | (uint32_t(__builtin_bit_cast(uint16_t, (__bf16)hi)) << 16);
}

__device__ __forceinline__ void unpack_bf16x8(const uint4& u, float (&f)[8]) {
  f[0] = __uint_as_float(u.x << 16);
  f[1] = __uint_as_float(u.x & 0xffff0000u);
  f[2] = __uint_as_float(u.y << 16);
  f[3] = __uint_as_float(u.y & 0xffff0000u);
  f[4] = __uint_as_float(u.z << 16);
  f[5] = __uint_as_float(u.z & 0xffff0000u);
  f[6] = __uint_as_float(u.w << 16);
  f[7] = __uint_as_float(u.w & 0xffff0000u);
}

constexpr int kWaves = 4;

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// K/V rows are read exactly once per step: non-temporal loads keep them from
// displacing reusable lines and measurably raise the streaming rate.
__device__ __forceinline__ uint4 load_stream(const bf16_t* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// QPW query heads (consecutive, sharing key/value head hk) per workgroup: every
// K/V row is loaded once and scored against all of them, so grouped layers read
// each retained row once per key/value head rather than once per query head.
// LAYOUT: 0 contiguous (one lane base), 1 block-paged, 2 windowed ring (row
// bases through kv_block_base; rows below the window start are masked).
template <int DH, int U, int LAYOUT, int QPW>
__global__ __launch_bounds__(64 * kWaves) void attend_decode_bf16_kernel(DevState s, SeqOrder order,
                                                                        float* __restrict__ out) {
  constexpr int G = DH / 8;
  constexpr int RPW = 64 / G;
  constexpr int GROUPS = kWaves * RPW;
  constexpr int STEP = GROUPS * U;
  static_assert(kMinBlockRows % STEP == 0 && kDecodeTileRows % STEP == 0, "a step must stay inside one block");
  __shared__ float sm_m[QPW][GROUPS], sm_l[QPW][GROUPS];
  __shared__ float sm_acc[QPW][GROUPS][DH + 4];

  // sequences with the most rows first (blocks are dispatched with z slowest)
  const int tile = blockIdx.x, h0 = blockIdx.y * QPW, b = order.count ? order.seq[blockIdx.z] : blockIdx.z;
  const int C = s.capacity;
  const int len = decode_len(s, b);
  const int t = len + 1;
  const int TR = s.tile_rows;
  const DecodeSpan span = decode_span(s, len);
  const int r0 = span.base0 + tile * TR;
  if (r0 >= t) return;
  const int r1 = min(t, r0 + TR);
  const int rs = span.rs;  // rows below rs lie outside the window (LAYOUT 2)
  const int ntiles = span.ntiles;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane % G;
  const int grp = wave * RPW + lane / G;
  const int hk = h0 / (s.heads / s.kv_heads);
  const size_t kv_lane = size_t(b) * s.kv_heads + hk;
  const size_t lane0 = size_t(b) * s.heads + h0;  // query lane of the first head
  const bf16_t* kpool = static_cast<const bf16_t*>(s.keys) + g * 8;
  const bf16_t* vpool = static_cast<const bf16_t*>(s.values) + g * 8;
  const bf16_t* kn = static_cast<const bf16_t*>(s.cand_k) + kv_lane * DH + g * 8;
  const bf16_t* vn = static_cast<const bf16_t*>(s.cand_v) + kv_lane * DH + g * 8;

  // one query: q in float32; several: q rounded to bf16 pairs (scaled first),
  // scored with packed bf16 dot products straight from the stored keys, which
  // keeps the vector work per K/V byte close to the one-query kernel's
  const float sl2 = float(s.scale) * 1.4426950408889634f;
  float qv[QPW == 1 ? 8 : 1];
  uint32_t qb[QPW][4];
#pragma unroll
  for (int qh = 0; qh < QPW; ++qh) {
    const float4* qp = reinterpret_cast<const float4*>(static_cast<const float*>(s.q) + (lane0 + qh) * DH + g * 8);
    const float4 a = qp[0], c = qp[1];
    if constexpr (QPW == 1) {
      qv[0] = a.x * sl2;
      qv[1] = a.y * sl2;
      qv[2] = a.z * sl2;
      qv[3] = a.w * sl2;
      qv[4] = c.x * sl2;
      qv[5] = c.y * sl2;
      qv[6] = c.z * sl2;
      qv[7] = c.w * sl2;
    } else {
      qb[qh][0] = pack_bf16x2(a.x * sl2, a.y * sl2);
      qb[qh][1] = pack_bf16x2(a.z * sl2, a.w * sl2);
      qb[qh][2] = pack_bf16x2(c.x * sl2, c.y * sl2);
      qb[qh][3] = pack_bf16x2(c.z * sl2, c.w * sl2);
    }
  }
  float m[QPW], l[QPW];
  float acc[QPW][8];
#pragma unroll
  for (int qh = 0; qh < QPW; ++qh) {
    m[qh] = -INFINITY;
    l[qh] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[qh][e] = 0.f;
  }

  for (int base = r0; base < r1; base += STEP) {
    // the STEP rows from base lie in one block of a paged cache (block rows are
    // a power-of-two multiple of STEP, tiles start on multiples of 512)
    const ptrdiff_t lane_base =
        LAYOUT ? kv_block_base(s, b, hk, min(base, max(len - 1, 0))) : ptrdiff_t(kv_lane * C) * DH;
    const bf16_t* kc = kpool + lane_base;
    const bf16_t* vc = vpool + lane_base;
    uint4 kr[U], vr[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = base + u * GROUPS + grp;
      ok[u] = r < r1 && (LAYOUT != 2 || r >= rs);
      const int rr = r < r1 ? r : r1 - 1;  // masked rows still load a held row
      const bf16_t* kp = rr < len ? kc + size_t(rr) * DH : kn;
      const bf16_t* vp = rr < len ? vc + size_t(rr) * DH : vn;
      kr[u] = load_stream(kp);
      vr[u] = load_stream(vp);
    }
    float sc[QPW][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (QPW == 1) {
        float kf[8];
        unpack_bf16x8(kr[u], kf);
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d = fmaf(qv[e], kf[e], d);
        sc[0][u] = d;
      } else {
#pragma unroll
        for (int qh = 0; qh < QPW; ++qh) sc[qh][u] = dot8_bf16(qb[qh], kr[u]);
      }
    }
#pragma unroll
    for (int qh = 0; qh < QPW; ++qh)
#pragma unroll
      for (int u = 0; u < U; ++u) sc[qh][u] = group_sum_dpp<G>(sc[qh][u]);
    float corr[QPW];
#pragma unroll
    for (int qh = 0; qh < QPW; ++qh) {
      float mx = m[qh];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        sc[qh][u] = ok[u] ? sc[qh][u] : -INFINITY;
        mx = fmaxf(mx, sc[qh][u]);
      }
      // a row group past the tile end sees only masked rows: keep its state at (-inf, 0, 0)
      corr[qh] = mx == -INFINITY ? 1.f : exp2f(m[qh] - mx);
      l[qh] *= corr[qh];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[qh][e] *= corr[qh];
#pragma unroll
      for (int u = 0; u < U; ++u) sc[qh][u] = ok[u] ? exp2f(sc[qh][u] - mx) : 0.f;
      m[qh] = mx;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vf[8];
      unpack_bf16x8(vr[u], vf);
#pragma unroll
      for (int qh = 0; qh < QPW; ++qh) {
        const float p = sc[qh][u];
        l[qh] += p;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[qh][e] = fmaf(p, vf[e], acc[qh][e]);
      }
    }
  }

#pragma unroll
  for (int qh = 0; qh < QPW; ++qh) {
    if (g == 0) {
      sm_m[qh][grp] = m[qh];
      sm_l[qh][grp] = l[qh];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) sm_acc[qh][grp][g * 8 + e] = acc[qh][e];
  }
  __syncthreads();

  const int j = threadIdx.x;  // output feature handled by this thread (j < DH)
#pragma unroll
  for (int qh = 0; qh < QPW; ++qh) {
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < GROUPS; ++k) M = fmaxf(M, sm_m[qh][k]);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int k = 0; k < GROUPS; ++k) {
      const float w = exp2f(sm_m[qh][k] - M);  // 0 for groups that saw no row
      L += sm_l[qh][k] * w;
      if (j < DH) A += sm_acc[qh][k][j] * w;
    }
    const size_t out_base = size_t(b) * s.model_width + size_t(h0 + qh) * DH;
    if (ntiles == 1) {
      if (j < DH) {
        const float o = A / L;
        out[out_base + j] = o;
        if (!isfinite(o)) flag_min(&s.err->output, out_base + j);
      }
      continue;
    }
    float* part = static_cast<float*>(s.partials) + ((lane0 + qh) * s.max_tiles + tile) * (DH + 2);
    if (j < DH) part[2 + j] = A;
    if (j == 0) {
      part[0] = M;
      part[1] = L;
    }
  }
}

// Log-sum-exp merge of a lane's tiles (lanes with one tile were written by the
// attention kernel).  Block = one lane, DH threads: the maximum and the
// weighted sum over tiles are block reductions, then thread j combines column j.
template <int DH>
__global__ __launch_bounds__(DH) void merge_decode_bf16_kernel(DevState s, float* __restrict__ out) {
  __shared__ float red[DH];
  const size_t lane_id = blockIdx.x;
  const int b = int(lane_id / s.heads);
  const int h = int(lane_id - size_t(b) * s.heads);
  const int ntiles = decode_span(s, decode_len(s, b)).ntiles;
  if (ntiles == 1) return;
  const int j = threadIdx.x;
  const float* p0 = static_cast<const float*>(s.partials) + lane_id * s.max_tiles * (DH + 2);
  float mx = -INFINITY;
  for (int k = j; k < ntiles; k += DH) mx = fmaxf(mx, p0[k * (DH + 2)]);
  red[j] = mx;
  __syncthreads();
  for (int w = DH / 2; w > 0; w >>= 1) {
    if (j < w) red[j] = fmaxf(red[j], red[j + w]);
    __syncthreads();
  }
  const float M = red[0];
  __syncthreads();
  float ls = 0.f;
  for (int k = j; k < ntiles; k += DH) ls += p0[k * (DH + 2) + 1] * exp2f(p0[k * (DH + 2)] - M);
  red[j] = ls;
  __syncthreads();
  for (int w = DH / 2; w > 0; w >>= 1) {
    if (j < w) red[j] += red[j + w];
    __syncthreads();
  }
  const float L = red[0];
  float A = 0.f;
#pragma unroll 8
  for (int k = 0; k < ntiles; ++k) A += p0[k * (DH + 2) + 2 + j] * exp2f(p0[k * (DH + 2)] - M);
  const float o = A / L;
  const size_t flat = size_t(b) * s.model_width + size_t(h) * DH + j;
  out[flat] = o;
  if (!isfinite(o)) flag_min(&s.err->output, flat);
}

inline hipStream_t st(void* p) { return static_cast<hipStream_t>(p); }

}  // namespace

// Split-K attention for bf16 storage with d_h in {64, 128}; returns -1 for
// other shapes (the vector kernels then run).
int fast_attend_decode(const DevState& s, const SeqOrder& order, void* out) {
  if (s.dtype != KVC_BF16) return -1;
  float* o = static_cast<float*>(out);
  const dim3 block(64 * kWaves);
  const int qpw = decode_heads_per_block(s.dtype, s.head_width, s.heads / s.kv_heads);
  const dim3 grid((s.span_rows + s.tile_rows - 1) / s.tile_rows, s.heads / qpw, s.batch);
#define KVC_DECODE_LAUNCH(DH_, U_, QPW_)                                                                    \
  do {                                                                                                   \
    if (s.ring)                                                                                          \
      hipLaunchKernelGGL((attend_decode_bf16_kernel<DH_, U_, 2, QPW_>), grid, block, 0, st(s.stream), s,   \
                         order, o);                                                                      \
    else if (s.paged)                                                                                    \
      hipLaunchKernelGGL((attend_decode_bf16_kernel<DH_, U_, 1, QPW_>), grid, block, 0, st(s.stream), s,   \
                         order, o);                                                                      \
    else                                                                                                 \
      hipLaunchKernelGGL((attend_decode_bf16_kernel<DH_, U_, 0, QPW_>), grid, block, 0, st(s.stream), s,   \
                         order, o);                                                                      \
  } while (0)
  // eight query heads per workgroup hold 8 x 16 accumulators per lane: half the
  // row groups in flight keeps them in registers
  if (s.head_width == 128) {
    switch (qpw) {
      case 1: KVC_DECODE_LAUNCH(128, 8, 1); break;
      case 2: KVC_DECODE_LAUNCH(128, 8, 2); break;
      case 4: KVC_DECODE_LAUNCH(128, 8, 4); break;
      default: KVC_DECODE_LAUNCH(128, 4, 8); break;
    }
  } else if (s.head_width == 64) {
    switch (qpw) {
      case 1: KVC_DECODE_LAUNCH(64, 4, 1); break;
      case 2: KVC_DECODE_LAUNCH(64, 4, 2); break;
      case 4: KVC_DECODE_LAUNCH(64, 4, 4); break;
      default: KVC_DECODE_LAUNCH(64, 2, 8); break;
    }
  } else {
    return -1;
  }
#undef KVC_DECODE_LAUNCH
  return int(hipGetLastError());
}

int fast_merge_decode(const DevState& s, void* out) {
  if (s.dtype != KVC_BF16) return -1;
  if (s.single_tile && (s.head_width == 128 || s.head_width == 64)) return 0;  // outputs already written
  const unsigned lanes = unsigned(s.batch) * unsigned(s.heads);
  if (s.head_width == 128) {
    hipLaunchKernelGGL(merge_decode_bf16_kernel<128>, dim3(lanes), dim3(128), 0, st(s.stream), s,
                       static_cast<float*>(out));
  } else if (s.head_width == 64) {
    hipLaunchKernelGGL(merge_decode_bf16_kernel<64>, dim3(lanes), dim3(64), 0, st(s.stream), s,
                       static_cast<float*>(out));
  } else {
    return -1;
  }
  return int(hipGetLastError());
}

}  // namespace kvc
