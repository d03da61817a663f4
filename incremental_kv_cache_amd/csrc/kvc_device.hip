// HIP kernels and device backend of libkvcache for gfx950 (MI355X, CDNA4).
//
// Pipeline of one call (Chapter 37, "Bind the state, calculate completely,
// then commit"; prefix-reuse note, "What must be trimmed together"):
//   project   : new rows through W_q, W_k, W_v, rotary at next_position + i,
//               candidate key/value rows and the query; non-finite checks.
//   attend    : decode -- split-K over the position axis, one partial
//               (max, sum, weighted values) per split-K tile of each lane
//               (512 * 2^k rows, chosen per call);
//               chunk  -- one workgroup per query row, causal over the
//               retained rows plus chunk rows 0..i.
//   merge     : log-sum-exp merge of a decode lane's partials into its head
//               block of the output (merge_heads).
//   commit    : candidate rows into slot len[b] (+ i), positions, then
//               len[b] and next_position[b] advance -- unless a failure word
//               is set, in which case nothing changes.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>
#include <utility>

#include "kvc_dev_util.h"
#include "kvc_internal.h"

namespace kvc {

namespace {

using namespace dev;

// --------------------------------------------------------------- project --

// One block = one input row m = (b, i) and one projection p; each thread
// produces one rotary pair (feature f and f + d_h/2 of head h), so the rotation
// needs no exchange.  The input row is staged through LDS in the accumulate
// type, in slices.
template <typename T, typename XT>
__global__ __launch_bounds__(256) void project_kernel(DevState s, const XT* __restrict__ x, int n_max,
                                                      int per_seq_rows, int proj_first) {
  using A = typename Acc<T>::type;
  constexpr int SLICE = 2048;
  __shared__ A xs[SLICE];
  const int m = blockIdx.y;
  const int p = proj_first + int(blockIdx.z);
  const int b = m / n_max;
  const int i = m - b * n_max;
  const int n_b = per_seq_rows ? s.rows[b] : n_max;
  if (i >= n_b) return;  // whole block leaves together

  const int D = s.model_width;
  const int dh = s.head_width;
  const int half = dh >> 1;
  const int pair = blockIdx.x * blockDim.x + threadIdx.x;
  const int heads_p = (p == 1 || p == 2) ? s.kv_heads : s.heads;  // K and V may have fewer heads
  const bool active = pair < heads_p * half;
  const int h = active ? pair / half : 0;
  const int f = active ? pair - h * half : 0;
  const T* W = static_cast<const T*>(p == 0 ? s.wq : (p == 1 ? s.wk : (p == 2 ? s.wv : s.wo)));
  const T* w0 = W + size_t(h * dh + f) * D;
  const T* w1 = W + size_t(h * dh + f + half) * D;
  const XT* xr = x + size_t(m) * D;

  A acc0 = 0, acc1 = 0;
  for (int k0 = 0; k0 < D; k0 += SLICE) {
    const int kn = min(SLICE, D - k0);
    __syncthreads();
    for (int k = threadIdx.x; k < kn; k += blockDim.x) xs[k] = to_acc<A>(xr[k0 + k]);
    __syncthreads();
    if (active) {
      for (int k = 0; k < kn; ++k) {
        const A xv = xs[k];
        acc0 += xv * to_acc<A>(w0[k0 + k]);
        acc1 += xv * to_acc<A>(w1[k0 + k]);
      }
    }
  }
  if (!active) return;

  if (p == 3) {  // output projection: plain columns of row m
    A* o = static_cast<A*>(s.out_proj_dst) + size_t(m) * D + size_t(h) * dh + f;
    o[0] = acc0;
    o[half] = acc1;
    if (!finite(acc0)) flag_min(&s.err->output, size_t(m) * D + size_t(h) * dh + f);
    if (!finite(acc1)) flag_min(&s.err->output, size_t(m) * D + size_t(h) * dh + f + half);
    return;
  }
  A r0 = acc0, r1 = acc1;
  if (p < 2 && s.rope) {
    int pos = s.next_pos[b] + i;
    if (pos < 0 || pos >= s.max_positions) {
      flag_min(&s.err->position, (unsigned long long)b);
      pos = 0;  // stay inside the table; the commit is suppressed
    }
    const A* ct = static_cast<const A*>(s.rope_cos);
    const A* st = static_cast<const A*>(s.rope_sin);
    const A c = ct[size_t(pos) * half + f];
    const A sn = st[size_t(pos) * half + f];
    r0 = acc0 * c - acc1 * sn;
    r1 = acc1 * c + acc0 * sn;
  }
  const size_t flat0 = (size_t(b * heads_p + h) * n_max + i) * dh + f;
  const size_t flat1 = flat0 + half;
  if (p == 0) {
    if (sizeof(T) == 2 && s.q_bf16) {  // bf16 layers: the flash kernel's operand (see DevState::q_bf16)
      const A sl2 = A(s.scale) * A(1.4426950408889634);
      bf16_t* q = static_cast<bf16_t*>(s.q);
      q[flat0] = f32_to_bf16(float(r0 * sl2));
      q[flat1] = f32_to_bf16(float(r1 * sl2));
    } else {
      A* q = static_cast<A*>(s.q);
      q[flat0] = r0;
      q[flat1] = r1;
    }
    if (!finite(r0)) flag_min(&s.err->query, flat0);
    if (!finite(r1)) flag_min(&s.err->query, flat1);
  } else {
    T* dst = static_cast<T*>(p == 1 ? s.cand_k : s.cand_v);
    const T t0 = from_acc<T>(r0), t1 = from_acc<T>(r1);
    dst[flat0] = t0;
    dst[flat1] = t1;
    unsigned long long* word = p == 1 ? &s.err->key : &s.err->value;
    if (!finite(to_acc<A>(t0))) flag_min(word, flat0);
    if (!finite(to_acc<A>(t1))) flag_min(word, flat1);
  }
}

// ------------------------------------------------------------ attention ----

// Online-softmax attention of one query over virtual rows [r0, r1) of a lane:
// virtual row r < len is cache row r, otherwise candidate row r - len.  Each
// group of G lanes owns one row at a time (its lanes hold one 16-byte chunk
// each); groups keep private (max, sum, weighted values) and are merged through
// LDS at the end.  Returns the tile's max and sum in M/L and the weighted
// values in acc_out[0..DH) (LDS), visible to the whole block after return.
// hk: the key/value head the query reads.
template <typename T, int DH, int NW>
__device__ __forceinline__ void attend_rows(const DevState& s, int b, int hk, const typename Acc<T>::type* __restrict__ q,
                                            const T* __restrict__ kc, const T* __restrict__ vc,
                                            const T* __restrict__ kn, const T* __restrict__ vn, int len,
                                            int r0, int r1, typename Acc<T>::type scale,
                                            typename Acc<T>::type* sm_m, typename Acc<T>::type* sm_l,
                                            typename Acc<T>::type* sm_acc, typename Acc<T>::type& M,
                                            typename Acc<T>::type& L, typename Acc<T>::type* acc_out) {
  using A = typename Acc<T>::type;
  using Geo = RowGeo<T, DH>;
  constexpr int VEC = Geo::VEC, G = Geo::G, RPW = Geo::RPW;
  constexpr int GROUPS = NW * RPW;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane % G;
  const int grp = wave * RPW + lane / G;

  A qv[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) qv[e] = q[g * VEC + e];

  A m = -INFINITY, l = 0;
  A acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0;

  for (int r = r0 + grp; r < r1; r += GROUPS) {
    const size_t off = r < len ? kv_offset(s, b, hk, r) : 0;
    const T* kr = (r < len) ? kc + off : kn + size_t(r - len) * DH;
    const T* vr = (r < len) ? vc + off : vn + size_t(r - len) * DH;
    A kv[VEC], vv[VEC];
    load_row_chunk<T, VEC>(kr + g * VEC, kv);
    load_row_chunk<T, VEC>(vr + g * VEC, vv);
    A dot = 0;
#pragma unroll
    for (int e = 0; e < VEC; ++e) dot += qv[e] * kv[e];
    dot = group_sum<G>(dot);
    const A sc = dot * scale;
    const A m_new = fmax(m, sc);
    const A corr = fast_exp(m - m_new);  // exp(-inf) = 0 on the first row
    const A pr = fast_exp(sc - m_new);
    l = l * corr + pr;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = acc[e] * corr + pr * vv[e];
    m = m_new;
  }

  if (g == 0) {
    sm_m[grp] = m;
    sm_l[grp] = l;
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) sm_acc[grp * DH + g * VEC + e] = acc[e];
  __syncthreads();
  A mx = -INFINITY;
  for (int k = 0; k < GROUPS; ++k) mx = fmax(mx, sm_m[k]);
  A sum = 0;
  for (int k = 0; k < GROUPS; ++k)
    if (sm_m[k] != -INFINITY) sum += sm_l[k] * fast_exp(sm_m[k] - mx);
  for (int j = threadIdx.x; j < DH; j += blockDim.x) {
    A a = 0;
    for (int k = 0; k < GROUPS; ++k)
      if (sm_m[k] != -INFINITY) a += sm_acc[k * DH + j] * fast_exp(sm_m[k] - mx);
    acc_out[j] = a;
  }
  M = mx;
  L = sum;
  __syncthreads();
}

constexpr int kAttendWaves = 4;

// Split-K decode attention: block (tile, h, b) handles rows
// [tile * 256, min(t_b, (tile + 1) * 256)) of lane (b, h), t_b = len[b] + 1.
template <typename T, int DH>
__global__ __launch_bounds__(64 * kAttendWaves) void attend_decode_kernel(DevState s) {
  using A = typename Acc<T>::type;
  using Geo = RowGeo<T, DH>;
  constexpr int GROUPS = kAttendWaves * Geo::RPW;
  __shared__ A sm_m[GROUPS], sm_l[GROUPS], sm_acc[GROUPS * DH], out_acc[DH];
  const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int len = decode_len(s, b);
  const int t = len + 1;
  const DecodeSpan span = decode_span(s, len);
  const int tile0 = span.base0 + tile * s.tile_rows;
  if (tile0 >= t) return;
  const int r0 = max(tile0, span.rs);
  const int r1 = min(t, tile0 + s.tile_rows);
  const size_t lane_id = size_t(b) * s.heads + h;
  const int hk = h / (s.heads / s.kv_heads);
  const size_t kv_lane = size_t(b) * s.kv_heads + hk;
  const T* kc = static_cast<const T*>(s.keys);
  const T* vc = static_cast<const T*>(s.values);
  const T* kn = static_cast<const T*>(s.cand_k) + kv_lane * DH;
  const T* vn = static_cast<const T*>(s.cand_v) + kv_lane * DH;
  const A* q = static_cast<const A*>(s.q) + lane_id * DH;
  A M, L;
  attend_rows<T, DH, kAttendWaves>(s, b, hk, q, kc, vc, kn, vn, len, r0, r1, A(s.scale), sm_m, sm_l, sm_acc, M, L,
                                   out_acc);
  A* part = static_cast<A*>(s.partials) + (lane_id * s.max_tiles + tile) * (DH + 2);
  if (threadIdx.x == 0) {
    part[0] = M;
    part[1] = L;
  }
  for (int j = threadIdx.x; j < DH; j += blockDim.x) part[2 + j] = out_acc[j];
}

// Log-sum-exp merge of the tiles of lane (b, h) into out[b, 0, h*d_h .. ].
template <typename T, int DH>
__global__ __launch_bounds__(64) void merge_decode_kernel(DevState s, typename Acc<T>::type* __restrict__ out) {
  using A = typename Acc<T>::type;
  const int h = blockIdx.x, b = blockIdx.y;
  const int ntiles = decode_span(s, decode_len(s, b)).ntiles;
  const size_t lane_id = size_t(b) * s.heads + h;
  const A* part = static_cast<const A*>(s.partials) + lane_id * s.max_tiles * (DH + 2);
  A mx = -INFINITY;
  for (int k = 0; k < ntiles; ++k) mx = fmax(mx, part[k * (DH + 2)]);
  A sum = 0;
  for (int k = 0; k < ntiles; ++k) sum += part[k * (DH + 2) + 1] * fast_exp(part[k * (DH + 2)] - mx);
  for (int j = threadIdx.x; j < DH; j += blockDim.x) {
    A a = 0;
    for (int k = 0; k < ntiles; ++k) a += part[k * (DH + 2) + 2 + j] * fast_exp(part[k * (DH + 2)] - mx);
    const A o = a / sum;
    const size_t flat = size_t(b) * s.model_width + size_t(h) * DH + j;
    out[flat] = o;
    if (!finite(o)) flag_min(&s.err->output, flat);
  }
}

// Chunk attention, one block per query row (i, h, b): rows [0, len[b] + i + 1).
template <typename T, int DH>
__global__ __launch_bounds__(64 * kAttendWaves) void attend_chunk_kernel(DevState s, int n_max, int per_seq_rows,
                                                                         typename Acc<T>::type* __restrict__ out) {
  using A = typename Acc<T>::type;
  using Geo = RowGeo<T, DH>;
  constexpr int GROUPS = kAttendWaves * Geo::RPW;
  __shared__ A sm_m[GROUPS], sm_l[GROUPS], sm_acc[GROUPS * DH], out_acc[DH];
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int n_b = per_seq_rows ? s.rows[b] : n_max;
  if (i >= n_b) return;
  const int len = s.ring ? max(s.len[b], 0) : min(max(s.len[b], 0), s.capacity);
  const size_t lane_id = size_t(b) * s.heads + h;
  const int hk = h / (s.heads / s.kv_heads);
  const size_t kv_lane = size_t(b) * s.kv_heads + hk;
  const T* kc = static_cast<const T*>(s.keys);
  const T* vc = static_cast<const T*>(s.values);
  const T* kn = static_cast<const T*>(s.cand_k) + kv_lane * n_max * DH;
  const T* vn = static_cast<const T*>(s.cand_v) + kv_lane * n_max * DH;
  const A* q = static_cast<const A*>(s.q) + (lane_id * n_max + i) * DH;
  A M, L;
  attend_rows<T, DH, kAttendWaves>(s, b, hk, q, kc, vc, kn, vn, len, window_start(s, len + i), len + i + 1,
                                   A(s.scale), sm_m, sm_l, sm_acc, M, L, out_acc);
  for (int j = threadIdx.x; j < DH; j += blockDim.x) {
    const A o = out_acc[j] / L;
    const size_t flat = (size_t(b) * n_max + i) * s.model_width + size_t(h) * DH + j;
    out[flat] = o;
    if (!finite(o)) flag_min(&s.err->output, flat);
  }
}

// --------------------------------------------------------------- commit ----

// Copies candidate rows 64 r .. 64 r + 63 of key/value lane (b, h) (block
// (r, h, b), h < H_kv) into rows len[b] + i of the cache.
constexpr int kCommitRows = 64;

template <typename T>
__global__ __launch_bounds__(256) void commit_copy_kernel(DevState s, int n_max, int per_seq_rows) {
  if (gate_closed(s)) return;
  const int r0 = blockIdx.x * kCommitRows, h = blockIdx.y, b = blockIdx.z;
  const int n_b = per_seq_rows ? s.rows[b] : n_max;
  const int len = s.len[b];
  const int C = s.capacity;
  // a ring takes any length (rows wrap; n_b <= C is checked on the host)
  if (r0 >= n_b || len < 0 || (!s.ring && len + n_b > C)) return;
  const int nr = min(kCommitRows, n_b - r0);
  const int dh = s.head_width;
  const size_t lane_id = size_t(b) * s.kv_heads + h;
  const T* sk = static_cast<const T*>(s.cand_k) + (lane_id * n_max + r0) * dh;
  const T* sv = static_cast<const T*>(s.cand_v) + (lane_id * n_max + r0) * dh;
  T* keys = static_cast<T*>(s.keys);
  T* values = static_cast<T*>(s.values);
  // row by row: in a paged cache consecutive rows may sit in different blocks
  if ((dh * sizeof(T)) % 16 == 0) {
    const int per_row = int(dh * sizeof(T) / 16);
    const int total = nr * per_row;
    // four 16-byte pieces of K and of V loaded before any is stored (the
    // compiler cannot move a load past a store to memory it cannot prove
    // disjoint, which would leave one load in flight per thread); past the end
    // a thread loads the last piece again and stores nothing
    constexpr int THREADS = 256;
    auto src = [&](int idx, const T* base) {
      const int i = min(idx, total - 1);
      const int k = i / per_row;
      return reinterpret_cast<const uint4*>(base + size_t(k) * dh)[i - k * per_row];
    };
    auto put = [&](int idx, const uint4 kk, const uint4 vv) {
      if (idx >= total) return;
      const int k = idx / per_row;
      const int c = idx - k * per_row;
      const size_t off = kv_offset(s, b, h, len + r0 + k);
      reinterpret_cast<uint4*>(keys + off)[c] = kk;
      reinterpret_cast<uint4*>(values + off)[c] = vv;
    };
    for (int i0 = threadIdx.x; i0 < total; i0 += 4 * THREADS) {
      const int i1 = i0 + THREADS, i2 = i1 + THREADS, i3 = i2 + THREADS;
      const uint4 k0 = src(i0, sk), v0 = src(i0, sv), k1 = src(i1, sk), v1 = src(i1, sv);
      const uint4 k2 = src(i2, sk), v2 = src(i2, sv), k3 = src(i3, sk), v3 = src(i3, sv);
      put(i0, k0, v0);
      put(i1, k1, v1);
      put(i2, k2, v2);
      put(i3, k3, v3);
    }
  } else {
    for (int idx = threadIdx.x; idx < nr * dh; idx += blockDim.x) {
      const int k = idx / dh;
      const int c = idx - k * dh;
      const size_t off = kv_offset(s, b, h, len + r0 + k);
      keys[off + c] = sk[size_t(k) * dh + c];
      values[off + c] = sv[size_t(k) * dh + c];
    }
  }
  if (h == 0) {
    const int np = s.next_pos[b];
    for (int k = threadIdx.x; k < nr; k += blockDim.x)
      s.positions[size_t(b) * C + pos_slot(s, len + r0 + k)] = np + r0 + k;
  }
}

// Decode commit in one launch: block b copies the H candidate rows of
// sequence b into row len[b], records the position, then advances len[b] and
// next_position[b]; no other block touches sequence b.
template <typename T>
__global__ __launch_bounds__(256) void commit_decode_kernel(DevState s) {
  if (gate_closed(s)) return;
  const int b = blockIdx.x;
  const int len = s.len[b];
  const int C = s.capacity;
  if (len < 0 || (!s.ring && len + 1 > C)) return;
  const int dh = s.head_width;
  const size_t row_bytes = size_t(dh) * sizeof(T);
  const size_t seq_rows = size_t(b) * s.kv_heads;
  if ((row_bytes & 15) == 0) {
    // two 16-byte pieces of K and of V per thread and pass, all four loaded
    // before any store (the stores may alias the loads as far as the compiler
    // knows, so it would not move a load past one)
    const int per_row = int(row_bytes / 16);
    const int n = s.kv_heads * per_row;
    auto src = [&](const void* cand, int idx) {
      const int h = idx / per_row;
      return reinterpret_cast<const uint4*>(static_cast<const T*>(cand) + (seq_rows + h) * dh)[idx - h * per_row];
    };
    auto put = [&](void* cache, int idx, uint4 v) {
      const int h = idx / per_row;
      reinterpret_cast<uint4*>(static_cast<T*>(cache) + kv_offset(s, b, h, len))[idx - h * per_row] = v;
    };
    for (int i0 = threadIdx.x; i0 < n; i0 += 2 * blockDim.x) {
      const int i1 = i0 + blockDim.x;
      const int i1c = min(i1, n - 1);
      const uint4 k0 = src(s.cand_k, i0), v0 = src(s.cand_v, i0);
      const uint4 k1 = src(s.cand_k, i1c), v1 = src(s.cand_v, i1c);
      put(s.keys, i0, k0);
      put(s.values, i0, v0);
      if (i1 < n) {
        put(s.keys, i1, k1);
        put(s.values, i1, v1);
      }
    }
  } else {
    for (int idx = threadIdx.x; idx < s.kv_heads * dh; idx += blockDim.x) {
      const int h = idx / dh;
      const int c = idx - h * dh;
      const size_t lane_id = seq_rows + h;
      const size_t off = kv_offset(s, b, h, len);
      static_cast<T*>(s.keys)[off + c] = static_cast<const T*>(s.cand_k)[lane_id * dh + c];
      static_cast<T*>(s.values)[off + c] = static_cast<const T*>(s.cand_v)[lane_id * dh + c];
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int np = s.next_pos[b];
    s.positions[size_t(b) * C + pos_slot(s, len)] = np;
    if (s.ring) s.held[b] = max(s.held[b], len + 1 - C);  // row len took the slot of row len - C
    s.len[b] = len + 1;
    s.next_pos[b] = np + 1;
  }
}

// Advances len[b] and next_position[b] by n_b (after every copy has read len[b]).
__global__ __launch_bounds__(256) void commit_advance_kernel(DevState s, int n_max, int per_seq_rows) {
  if (gate_closed(s)) return;
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= s.batch) return;
  const int n_b = per_seq_rows ? s.rows[b] : n_max;
  const int len = s.len[b];
  if (n_b <= 0 || len < 0 || (!s.ring && len + n_b > s.capacity)) return;
  if (s.ring) s.held[b] = max(s.held[b], len + n_b - s.capacity);
  s.len[b] = len + n_b;
  s.next_pos[b] = s.next_pos[b] + n_b;
}

// ------------------------------------------------------------ bookkeeping --

struct SetArgs {
  int32_t vals[kSetChunk];
  int first, count, mode;
  int held_src;  // dev_set_seq_length on a ring: sequence whose held row is copied (-1: 0)
};

__global__ __launch_bounds__(256) void set_lengths_kernel(DevState s, SetArgs a) {
  if (gate_closed(s)) return;
  for (int k = threadIdx.x; k < a.count; k += blockDim.x) {
    const int b = a.first + k;
    if (a.mode == 2) {
      s.len[b] = 0;
      s.next_pos[b] = 0;
      if (s.ring) s.held[b] = 0;
    } else if (a.mode == 3) {  // one sequence, after a fork
      s.len[b] = a.vals[k];
      s.next_pos[b] = a.vals[k];
      if (s.ring) s.held[b] = a.held_src >= 0 ? s.held[a.held_src] : 0;
    } else {
      s.len[b] = a.vals[k];
      if (a.mode == 0) s.next_pos[b] = a.vals[k];
      // a ring cut below its held rows (only a cut to 0 is allowed) starts afresh
      if (s.ring && a.vals[k] < s.held[b]) s.held[b] = a.vals[k];
    }
  }
}

__global__ __launch_bounds__(256) void set_rows_kernel(DevState s, SetArgs a) {
  for (int k = threadIdx.x; k < a.count; k += blockDim.x) s.rows[a.first + k] = a.vals[k];
}

struct TableArgs {
  int32_t idx[kSetChunk / 2];
  int32_t val[kSetChunk / 2];
  int count;
};

__global__ __launch_bounds__(256) void set_table_kernel(DevState s, TableArgs a) {
  if (gate_closed(s)) return;  // block moves are state changes like the length updates
  int32_t* table = const_cast<int32_t*>(s.block_table);
  for (int k = threadIdx.x; k < a.count; k += blockDim.x) table[a.idx[k]] = a.val[k];
}

// Rows [0, rows) of every head of block src into block dst, 16 bytes a thread.
__global__ __launch_bounds__(256) void clear_table_kernel(DevState s) {
  if (gate_closed(s)) return;
  int32_t* table = const_cast<int32_t*>(s.block_table);
  const size_t n = size_t(s.batch) * s.table_width;
  for (size_t k = size_t(blockIdx.x) * blockDim.x + threadIdx.x; k < n; k += size_t(gridDim.x) * blockDim.x)
    table[k] = -1;
}

// Grid-strided copy of `bytes` (a multiple of 4: rows are at least 4 bytes) in
// 16-byte units when both ends allow it, else in 4-byte units.
__device__ __forceinline__ void copy_span(char* to, const char* from, size_t bytes) {
  const size_t t = size_t(blockIdx.x) * blockDim.x + threadIdx.x, stride = size_t(gridDim.x) * blockDim.x;
  if (((reinterpret_cast<uintptr_t>(to) | reinterpret_cast<uintptr_t>(from) | bytes) & 15) == 0) {
    for (size_t k = t; k < bytes / 16; k += stride)
      reinterpret_cast<uint4*>(to)[k] = reinterpret_cast<const uint4*>(from)[k];
  } else {
    for (size_t k = t; k < bytes / 4; k += stride)
      reinterpret_cast<uint32_t*>(to)[k] = reinterpret_cast<const uint32_t*>(from)[k];
  }
}

// Paged caches: rows [0, rows) of head blockIdx.y, block src to block dst.
__global__ __launch_bounds__(256) void copy_block_rows_kernel(DevState s, int dst, int src, int rows, int es) {
  if (gate_closed(s)) return;
  const size_t row_bytes = size_t(s.head_width) * es;
  const size_t head_bytes = row_bytes << s.block_rows_log2;
  const int h = blockIdx.y;
  for (int part = 0; part < 2; ++part) {
    char* base = static_cast<char*>(part ? s.values : s.keys);
    copy_span(base + (size_t(dst) * s.kv_heads + h) * head_bytes, base + (size_t(src) * s.kv_heads + h) * head_bytes,
              size_t(rows) * row_bytes);
  }
}

__global__ __launch_bounds__(256) void copy_positions_kernel(DevState s, int dst_seq, int src_seq, int rows) {
  if (gate_closed(s)) return;
  for (int k = blockIdx.x * blockDim.x + threadIdx.x; k < rows; k += gridDim.x * blockDim.x)
    s.positions[size_t(dst_seq) * s.capacity + k] = s.positions[size_t(src_seq) * s.capacity + k];
}

// Contiguous caches: rows [0, rows) of head blockIdx.y, sequence src to dst.
__global__ __launch_bounds__(256) void copy_seq_rows_kernel(DevState s, int dst_seq, int src_seq, int rows, int es) {
  if (gate_closed(s)) return;
  const size_t row_bytes = size_t(s.head_width) * es;
  const size_t lane_bytes = size_t(s.capacity) * row_bytes;
  const int h = blockIdx.y;
  for (int part = 0; part < 2; ++part) {
    char* base = static_cast<char*>(part ? s.values : s.keys);
    copy_span(base + (size_t(dst_seq) * s.kv_heads + h) * lane_bytes,
              base + (size_t(src_seq) * s.kv_heads + h) * lane_bytes,
              size_t(rows) * row_bytes);
  }
}

__global__ void clear_err_kernel(ErrWords* e) {
  if (threadIdx.x < 8) reinterpret_cast<unsigned long long*>(e)[threadIdx.x] = kErrClear;
}

__global__ __launch_bounds__(256) void zero_kernel(uint4* p, size_t n16) {
  for (size_t k = size_t(blockIdx.x) * blockDim.x + threadIdx.x; k < n16; k += size_t(gridDim.x) * blockDim.x)
    p[k] = make_uint4(0, 0, 0, 0);
}

// ---------------------------------------------------------------- session ---
// Input rows of a model-wide step: token embedding plus the absolute sinusoidal
// encoding PE(p, 2i) = sin(p / 10000^(2i/D)), PE(p, 2i+1) = cos(same), with p =
// next_position + i (prefix-reuse note, "Work and error over 27 cases": the toy
// decoder's absolute sinusoidal positions; the angle is evaluated in double).
// Block = 256 columns of one row (b, i): blockIdx.x the row, blockIdx.y the columns.
template <typename A, typename W>
__global__ __launch_bounds__(256) void embed_kernel(DevState s, const int32_t* __restrict__ tokens,
                                                    const A* __restrict__ emb, int vocab, int sinusoidal, int n_max,
                                                    int per_seq_rows, A* __restrict__ h, W* __restrict__ x) {
  const int row = blockIdx.x;
  const int b = row / n_max;
  const int i = row - b * n_max;
  const int n_b = per_seq_rows ? s.rows[b] : n_max;
  if (i >= n_b) return;
  const int tok = tokens[row];
  if (tok < 0 || tok >= vocab) {
    if (threadIdx.x == 0 && blockIdx.y == 0) flag_min(&s.err->token, (unsigned long long)row);
    return;
  }
  const int D = s.model_width;
  const int j = blockIdx.y * blockDim.x + threadIdx.x;  // a row's columns are spread over blockIdx.y
  if (j >= D) return;
  const double p = double(s.next_pos[b] + i);
  A v = emb[size_t(tok) * D + j];
  if (sinusoidal) {
    const double ang = p / pow(10000.0, double(2 * (j >> 1)) / double(D));
    v += A((j & 1) ? cos(ang) : sin(ang));
  }
  h[size_t(row) * D + j] = v;
  if (x) x[size_t(row) * D + j] = from_acc<W>(v);
}

__device__ __forceinline__ double tanh_acc(double v) { return tanh(v); }
__device__ __forceinline__ float tanh_acc(float v) { return tanhf(v); }

// The tanh-residual block between layers: h_out = h_in + tanh(a).
template <typename A, typename W>
__global__ __launch_bounds__(256) void residual_kernel(DevState s, const A* __restrict__ h_in,
                                                       const A* __restrict__ a, A* h_out, W* __restrict__ x,
                                                       int n_max, int per_seq_rows) {
  const int row = blockIdx.x;
  const int b = row / n_max;
  const int i = row - b * n_max;
  const int n_b = per_seq_rows ? s.rows[b] : n_max;
  if (i >= n_b) return;
  const int D = s.model_width;
  const int j = blockIdx.y * blockDim.x + threadIdx.x;  // a row's columns are spread over blockIdx.y
  if (j >= D) return;
  const size_t k = size_t(row) * D + j;
  const A v = h_in[k] + tanh_acc(a[k]);
  h_out[k] = v;
  if (x) x[k] = from_acc<W>(v);
}

inline hipStream_t st(void* s) { return static_cast<hipStream_t>(s); }

inline int last_launch() { return int(hipGetLastError()); }

// Dispatch on (storage type, head width) to a template instance.
template <template <typename, int> class K, typename... Args>
int dispatch(int dtype, int dh, Args&&... args) {
#define KVC_DH_CASES(T)                                              \
  switch (dh) {                                                      \
    case 2: return K<T, 2>::run(std::forward<Args>(args)...);        \
    case 4: return K<T, 4>::run(std::forward<Args>(args)...);        \
    case 8: return K<T, 8>::run(std::forward<Args>(args)...);        \
    case 16: return K<T, 16>::run(std::forward<Args>(args)...);      \
    case 32: return K<T, 32>::run(std::forward<Args>(args)...);      \
    case 64: return K<T, 64>::run(std::forward<Args>(args)...);      \
    case 128: return K<T, 128>::run(std::forward<Args>(args)...);    \
    default: break;                                                  \
  }
  if (dtype == KVC_F64) {
    KVC_DH_CASES(double)
  } else if (dtype == KVC_F32) {
    KVC_DH_CASES(float)
    if (dh == 256) return K<float, 256>::run(std::forward<Args>(args)...);
  } else if (dtype == KVC_BF16) {
    KVC_DH_CASES(bf16_t)
    if (dh == 256) return K<bf16_t, 256>::run(std::forward<Args>(args)...);
    if (dh == 512) return K<bf16_t, 512>::run(std::forward<Args>(args)...);
  }
#undef KVC_DH_CASES
  return int(hipErrorInvalidValue);
}

template <typename T, int DH>
struct AttendDecode {
  static int run(const DevState& s) {
    dim3 grid((s.span_rows + s.tile_rows - 1) / s.tile_rows, s.heads, s.batch);
    hipLaunchKernelGGL((attend_decode_kernel<T, DH>), grid, dim3(64 * kAttendWaves), 0, st(s.stream), s);
    return last_launch();
  }
};

template <typename T, int DH>
struct MergeDecode {
  static int run(const DevState& s, void* out) {
    dim3 grid(s.heads, s.batch);
    hipLaunchKernelGGL((merge_decode_kernel<T, DH>), grid, dim3(64), 0, st(s.stream), s,
                       static_cast<typename Acc<T>::type*>(out));
    return last_launch();
  }
};

template <typename T, int DH>
struct AttendChunk {
  static int run(const DevState& s, int n_max, int per_seq_rows, void* out) {
    dim3 grid(n_max, s.heads, s.batch);
    hipLaunchKernelGGL((attend_chunk_kernel<T, DH>), grid, dim3(64 * kAttendWaves), 0, st(s.stream), s, n_max,
                       per_seq_rows, static_cast<typename Acc<T>::type*>(out));
    return last_launch();
  }
};

template <typename T, typename XT>
int project_t(const DevState& s, const XT* x, int n_max, int per_seq_rows, int proj_first, int nproj) {
  const int pairs = s.heads * (s.head_width / 2);
  dim3 grid((pairs + 255) / 256, s.batch * n_max, nproj);
  hipLaunchKernelGGL((project_kernel<T, XT>), grid, dim3(256), 0, st(s.stream), s, x, n_max, per_seq_rows,
                     proj_first);
  return last_launch();
}

// Readout of the newest query's softmax weights (Chapter 37 prints them for its
// worked trace): block = one head h of sequence b; q is the last decode call's
// rotated query, the rows r0 .. r0 + rows - 1 are the committed keys (the newest
// one included).  Scores q . k / sqrt(d_h), then a max-subtracted softmax, all
// in the accumulate type; one wave, each lane a strided subset of the rows.
template <typename T>
__global__ __launch_bounds__(64) void newest_weights_kernel(DevState s, int b, int r0, int rows,
                                                            typename Acc<T>::type* __restrict__ w) {
  using A = typename Acc<T>::type;
  const int h = blockIdx.x;
  const int hk = h / (s.heads / s.kv_heads);
  const int dh = s.head_width;
  const A* q = static_cast<const A*>(s.q) + (size_t(b) * s.heads + h) * dh;
  const T* keys = static_cast<const T*>(s.keys);
  const A scale = A(s.scale);
  A* wh = w + size_t(h) * rows;
  A mx = -INFINITY;
  for (int k = threadIdx.x; k < rows; k += 64) {
    const T* kr = keys + kv_offset(s, b, hk, r0 + k);
    A d = 0;
    for (int e = 0; e < dh; ++e) d += q[e] * to_acc<A>(kr[e]);
    d *= scale;
    wh[k] = d;
    mx = d > mx ? d : mx;
  }
  for (int o = 32; o > 0; o >>= 1) {
    const A other = __shfl_xor(mx, o, 64);
    mx = other > mx ? other : mx;
  }
  A sum = 0;
  for (int k = threadIdx.x; k < rows; k += 64) {
    const A e = exp(wh[k] - mx);
    wh[k] = e;
    sum += e;
  }
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
  for (int k = threadIdx.x; k < rows; k += 64) wh[k] /= sum;
}

template <typename T>
int commit_t(const DevState& s, int n_max, int per_seq_rows) {
  if (n_max == 1 && !per_seq_rows) {
    hipLaunchKernelGGL((commit_decode_kernel<T>), dim3(s.batch), dim3(256), 0, st(s.stream), s);
    return last_launch();
  }
  hipLaunchKernelGGL((commit_copy_kernel<T>), dim3((n_max + kCommitRows - 1) / kCommitRows, s.kv_heads, s.batch),
                     dim3(256), 0, st(s.stream), s, n_max, per_seq_rows);
  int rc = last_launch();
  if (rc) return rc;
  hipLaunchKernelGGL(commit_advance_kernel, dim3((s.batch + 255) / 256), dim3(256), 0, st(s.stream), s, n_max,
                     per_seq_rows);
  return last_launch();
}

}  // namespace

// ------------------------------------------------------------- backend API --

const char* dev_error_string(int code) { return hipGetErrorString(hipError_t(code)); }

int dev_current_device(int* device) { return int(hipGetDevice(device)); }

int dev_compute_units(int device, int* units) {
  return int(hipDeviceGetAttribute(units, hipDeviceAttributeMultiprocessorCount, device));
}

int dev_malloc(void** p, size_t bytes) { return int(hipMalloc(p, bytes ? bytes : 16)); }

void dev_free(void* p) {
  if (p) (void)hipFree(p);
}

int dev_host_malloc(void** p, size_t bytes) { return int(hipHostMalloc(p, bytes ? bytes : 16, hipHostMallocDefault)); }

void dev_host_free(void* p) {
  if (p) (void)hipHostFree(p);
}

int dev_copy_h2d_sync(void* dst, const void* src, size_t bytes, void* stream) {
  hipError_t e = hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, st(stream));
  if (e != hipSuccess) return int(e);
  return int(hipStreamSynchronize(st(stream)));
}

int dev_copy_d2h_sync(void* dst, const void* src, size_t bytes, void* stream) {
  hipError_t e = hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToHost, st(stream));
  if (e != hipSuccess) return int(e);
  return int(hipStreamSynchronize(st(stream)));
}

int dev_copy_d2h_2d_sync(void* dst, size_t dpitch, const void* src, size_t spitch, size_t width, size_t height,
                         void* stream) {
  if (width == 0 || height == 0) return int(hipStreamSynchronize(st(stream)));
  hipError_t e = hipMemcpy2DAsync(dst, dpitch, src, spitch, width, height, hipMemcpyDeviceToHost, st(stream));
  if (e != hipSuccess) return int(e);
  return int(hipStreamSynchronize(st(stream)));
}

int dev_sync(void* stream) { return int(hipStreamSynchronize(st(stream))); }

int dev_zero(void* p, size_t bytes, void* stream) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return 0;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(zero_kernel, dim3(unsigned(blocks)), dim3(256), 0, st(stream), static_cast<uint4*>(p), n16);
  return last_launch();
}

int dev_clear_err(ErrWords* err, void* stream) {
  hipLaunchKernelGGL(clear_err_kernel, dim3(1), dim3(64), 0, st(stream), err);
  return last_launch();
}

int dev_set_lengths(const DevState& s, const int32_t* vals, int mode) {
  for (int first = 0; first < s.batch; first += kSetChunk) {
    SetArgs a{};
    a.first = first;
    a.count = s.batch - first < kSetChunk ? s.batch - first : kSetChunk;
    a.mode = mode;
    if (mode != 2)
      for (int k = 0; k < a.count; ++k) a.vals[k] = vals[first + k];
    hipLaunchKernelGGL(set_lengths_kernel, dim3(1), dim3(256), 0, st(s.stream), s, a);
    int rc = last_launch();
    if (rc) return rc;
  }
  return 0;
}

int dev_set_rows(const DevState& s, const int32_t* vals) {
  for (int first = 0; first < s.batch; first += kSetChunk) {
    SetArgs a{};
    a.first = first;
    a.count = s.batch - first < kSetChunk ? s.batch - first : kSetChunk;
    for (int k = 0; k < a.count; ++k) a.vals[k] = vals[first + k];
    hipLaunchKernelGGL(set_rows_kernel, dim3(1), dim3(256), 0, st(s.stream), s, a);
    int rc = last_launch();
    if (rc) return rc;
  }
  return 0;
}

static int elem_bytes(int dtype) { return dtype == KVC_F64 ? 8 : (dtype == KVC_F32 ? 4 : 2); }

int dev_set_table(const DevState& s, const int32_t* idx, const int32_t* val, int count) {
  for (int first = 0; first < count; first += kSetChunk / 2) {
    TableArgs a{};
    a.count = count - first < kSetChunk / 2 ? count - first : kSetChunk / 2;
    for (int k = 0; k < a.count; ++k) {
      a.idx[k] = idx[first + k];
      a.val[k] = val[first + k];
    }
    hipLaunchKernelGGL(set_table_kernel, dim3(1), dim3(256), 0, st(s.stream), s, a);
    int rc = last_launch();
    if (rc) return rc;
  }
  return 0;
}

int dev_clear_table(const DevState& s) {
  const size_t n = size_t(s.batch) * s.table_width;
  const int blocks = int(n / 256 + 1 < 1024 ? n / 256 + 1 : 1024);
  hipLaunchKernelGGL(clear_table_kernel, dim3(blocks), dim3(256), 0, st(s.stream), s);
  return last_launch();
}

int dev_set_seq_length(const DevState& s, int seq, int32_t value, int held_src) {
  SetArgs a{};
  a.first = seq;
  a.count = 1;
  a.mode = 3;
  a.held_src = held_src;
  a.vals[0] = value;
  hipLaunchKernelGGL(set_lengths_kernel, dim3(1), dim3(256), 0, st(s.stream), s, a);
  return last_launch();
}

int dev_copy_block_rows(const DevState& s, int dst, int src, int rows) {
  if (rows <= 0) return 0;
  hipLaunchKernelGGL(copy_block_rows_kernel, dim3(8, s.kv_heads), dim3(256), 0, st(s.stream), s, dst, src, rows,
                     elem_bytes(s.dtype));
  return last_launch();
}

int dev_copy_positions(const DevState& s, int dst_seq, int src_seq, int rows) {
  if (rows <= 0) return 0;
  hipLaunchKernelGGL(copy_positions_kernel, dim3((rows + 255) / 256), dim3(256), 0, st(s.stream), s, dst_seq, src_seq,
                     rows);
  return last_launch();
}

int dev_copy_seq_rows(const DevState& s, int dst_seq, int src_seq, int rows) {
  if (rows <= 0) return 0;
  hipLaunchKernelGGL(copy_seq_rows_kernel, dim3(32, s.kv_heads), dim3(256), 0, st(s.stream), s, dst_seq, src_seq, rows,
                     elem_bytes(s.dtype));
  return last_launch();
}

int mfma_project(const DevState& s, const void* x, int n_max, int per_seq_rows);
int mfma_output_project(const DevState& s, int n_max, int per_seq_rows);
int mfma_attend_chunk(const DevState& s, int n_max, int per_seq_rows, const ChunkOrder& order, void* out);
int fast_attend_decode(const DevState& s, const SeqOrder& order, void* out);
int fast_merge_decode(const DevState& s, void* out);

int dev_project(const DevState& s, const void* x, int n_max, int per_seq_rows) {
  const int rc = mfma_project(s, x, n_max, per_seq_rows);
  if (rc >= 0) return rc;
  switch (s.dtype) {
    case KVC_F64: return project_t<double>(s, static_cast<const double*>(x), n_max, per_seq_rows, 0, 3);
    case KVC_F32: return project_t<float>(s, static_cast<const float*>(x), n_max, per_seq_rows, 0, 3);
    case KVC_BF16: return project_t<bf16_t>(s, static_cast<const bf16_t*>(x), n_max, per_seq_rows, 0, 3);
  }
  return int(hipErrorInvalidValue);
}

int dev_output_project(const DevState& state, int n_max, int per_seq_rows, void* out) {
  DevState s = state;
  s.out_proj_dst = out;
  const int rc = mfma_output_project(s, n_max, per_seq_rows);
  if (rc >= 0) return rc;
  switch (s.dtype) {
    case KVC_F64: return project_t<double>(s, static_cast<const double*>(s.merged), n_max, per_seq_rows, 3, 1);
    case KVC_F32: return project_t<float>(s, static_cast<const float*>(s.merged), n_max, per_seq_rows, 3, 1);
    case KVC_BF16: return project_t<bf16_t>(s, static_cast<const float*>(s.merged), n_max, per_seq_rows, 3, 1);
  }
  return int(hipErrorInvalidValue);
}

int dev_attend_decode(const DevState& s, const SeqOrder& order, void* out) {
  const int rc = fast_attend_decode(s, order, out);
  if (rc >= 0) return rc;
  return dispatch<AttendDecode>(s.dtype, s.head_width, s);
}

int dev_newest_weights(const DevState& s, int b, int r0, int rows, void* w) {
  switch (s.dtype) {
    case KVC_F64:
      hipLaunchKernelGGL(newest_weights_kernel<double>, dim3(s.heads), dim3(64), 0, st(s.stream), s, b, r0, rows,
                         static_cast<double*>(w));
      break;
    case KVC_F32:
      hipLaunchKernelGGL(newest_weights_kernel<float>, dim3(s.heads), dim3(64), 0, st(s.stream), s, b, r0, rows,
                         static_cast<float*>(w));
      break;
    default:
      hipLaunchKernelGGL(newest_weights_kernel<bf16_t>, dim3(s.heads), dim3(64), 0, st(s.stream), s, b, r0, rows,
                         static_cast<float*>(w));
      break;
  }
  return last_launch();
}

int dev_merge_decode(const DevState& s, void* out) {
  const int rc = fast_merge_decode(s, out);
  if (rc >= 0) return rc;
  return dispatch<MergeDecode>(s.dtype, s.head_width, s, out);
}

int dev_attend_chunk(const DevState& s, int n_max, int per_seq_rows, const ChunkOrder& order, void* out) {
  const int rc = mfma_attend_chunk(s, n_max, per_seq_rows, order, out);
  if (rc >= 0) return rc;
  return dispatch<AttendChunk>(s.dtype, s.head_width, s, n_max, per_seq_rows, out);
}

int dev_commit(const DevState& s, int n_max, int per_seq_rows) {
  switch (s.dtype) {
    case KVC_F64: return commit_t<double>(s, n_max, per_seq_rows);
    case KVC_F32: return commit_t<float>(s, n_max, per_seq_rows);
    case KVC_BF16: return commit_t<bf16_t>(s, n_max, per_seq_rows);
  }
  return int(hipErrorInvalidValue);
}

int dev_event_create(void** e) { return int(hipEventCreate(reinterpret_cast<hipEvent_t*>(e))); }

void dev_event_destroy(void* e) {
  if (e) (void)hipEventDestroy(static_cast<hipEvent_t>(e));
}

int dev_event_record(void* e, void* stream) { return int(hipEventRecord(static_cast<hipEvent_t>(e), st(stream))); }

int dev_event_elapsed(float* ms, void* start, void* stop) {
  hipError_t e = hipEventSynchronize(static_cast<hipEvent_t>(stop));
  if (e != hipSuccess) return int(e);
  return int(hipEventElapsedTime(ms, static_cast<hipEvent_t>(start), static_cast<hipEvent_t>(stop)));
}

bool dev_has_kernels() { return true; }

}  // namespace kvc

// Scratch of the entry point that allocates nothing (kvc_append_and_attend_static):
// the query, candidate rows, split-K partials and projection sums of one decode
// call live here instead of in the cache's own buffers.  Host code must never
// use this name as an address: it is a host-side stand-in, and only the address
// hipGetSymbolAddress returns for the current device is valid on that device.
static __device__ __align__(256) unsigned char scratch[kvc::kStaticScratchBytes];

namespace kvc {

int dev_static_scratch(int device, void** ptr, size_t* bytes) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices) return int(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[device]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != device) e = hipSetDevice(device);
    void* p = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != device) {
      const hipError_t back = hipSetDevice(cur);
      if (e == hipSuccess) e = back;
    }
    if (e != hipSuccess) return int(e);
    if (!p) return int(hipErrorInvalidSymbol);
    addr[device] = p;
  }
  *ptr = addr[device];
  *bytes = kStaticScratchBytes;
  return 0;
}

int dev_embed(const DevState& s, const int32_t* tokens, const void* embedding, int vocab, int sinusoidal,
              int n_max, int per_seq_rows, void* h, void* x) {
  const dim3 grid(unsigned(s.batch) * unsigned(n_max), unsigned(s.model_width + 255) / 256);
  switch (s.dtype) {
    case KVC_F64:
      hipLaunchKernelGGL((embed_kernel<double, double>), grid, dim3(256), 0, st(s.stream), s, tokens,
                         static_cast<const double*>(embedding), vocab, sinusoidal, n_max, per_seq_rows,
                         static_cast<double*>(h), static_cast<double*>(x));
      break;
    case KVC_F32:
      hipLaunchKernelGGL((embed_kernel<float, float>), grid, dim3(256), 0, st(s.stream), s, tokens,
                         static_cast<const float*>(embedding), vocab, sinusoidal, n_max, per_seq_rows,
                         static_cast<float*>(h), static_cast<float*>(x));
      break;
    case KVC_BF16:
      hipLaunchKernelGGL((embed_kernel<float, bf16_t>), grid, dim3(256), 0, st(s.stream), s, tokens,
                         static_cast<const float*>(embedding), vocab, sinusoidal, n_max, per_seq_rows,
                         static_cast<float*>(h), static_cast<bf16_t*>(x));
      break;
    default:
      return int(hipErrorInvalidValue);
  }
  return last_launch();
}

int dev_residual(const DevState& s, const void* h_in, const void* a, void* h_out, void* x, int n_max,
                 int per_seq_rows) {
  const dim3 grid(unsigned(s.batch) * unsigned(n_max), unsigned(s.model_width + 255) / 256);
  switch (s.dtype) {
    case KVC_F64:
      hipLaunchKernelGGL((residual_kernel<double, double>), grid, dim3(256), 0, st(s.stream), s,
                         static_cast<const double*>(h_in), static_cast<const double*>(a), static_cast<double*>(h_out),
                         static_cast<double*>(x), n_max, per_seq_rows);
      break;
    case KVC_F32:
      hipLaunchKernelGGL((residual_kernel<float, float>), grid, dim3(256), 0, st(s.stream), s,
                         static_cast<const float*>(h_in), static_cast<const float*>(a), static_cast<float*>(h_out),
                         static_cast<float*>(x), n_max, per_seq_rows);
      break;
    case KVC_BF16:
      hipLaunchKernelGGL((residual_kernel<float, bf16_t>), grid, dim3(256), 0, st(s.stream), s,
                         static_cast<const float*>(h_in), static_cast<const float*>(a), static_cast<float*>(h_out),
                         static_cast<bf16_t*>(x), n_max, per_seq_rows);
      break;
    default:
      return int(hipErrorInvalidValue);
  }
  return last_launch();
}

}  // namespace kvc
