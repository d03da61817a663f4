// CPU-only stand-in for the device backend, used to test the host cache
// manager (validation order, bookkeeping, snapshots of zeroed storage) on a
// machine without a GPU.  "Device" memory is host memory and no kernel can
// run: every compute launch reports an error, so nothing here computes
// attention.  Built by tests/test_host_manager.py; never shipped.
#include <cstdlib>
#include <cstring>
#include <initializer_list>

#include "../incremental_kv_cache_amd/csrc/kvc_internal.h"

namespace kvc {

const char* dev_error_string(int) { return "no device in the host-check build"; }
int dev_current_device(int* device) {
  *device = -1;
  return 0;
}
int dev_compute_units(int, int* units) {
  *units = 256;
  return 0;
}
int dev_malloc(void** p, size_t bytes) {
  *p = std::aligned_alloc(256, (bytes + 255) & ~size_t(255));
  return *p ? 0 : 2;
}
void dev_free(void* p) { std::free(p); }
int dev_host_malloc(void** p, size_t bytes) { return dev_malloc(p, bytes); }
void dev_host_free(void* p) { std::free(p); }
int dev_copy_h2d_sync(void* dst, const void* src, size_t bytes, void*) {
  std::memcpy(dst, src, bytes);
  return 0;
}
int dev_copy_d2h_sync(void* dst, const void* src, size_t bytes, void*) {
  std::memcpy(dst, src, bytes);
  return 0;
}
int dev_copy_d2h_2d_sync(void* dst, size_t dpitch, const void* src, size_t spitch, size_t width, size_t height,
                         void*) {
  for (size_t r = 0; r < height; ++r)
    std::memcpy(static_cast<char*>(dst) + r * dpitch, static_cast<const char*>(src) + r * spitch, width);
  return 0;
}
int dev_sync(void*) { return 0; }
int dev_zero(void* p, size_t bytes, void*) {
  std::memset(p, 0, bytes);
  return 0;
}
int dev_clear_err(ErrWords* err, void*) {
  std::memset(err, 0xff, sizeof(ErrWords));
  return 0;
}
static bool any_error(const ErrWords* e) {
  return (e->key & e->value & e->query & e->position & e->output & e->token) != kErrClear;
}
static bool gate_closed(const DevState& s) {
  for (int k = 0; k < s.gate_count; ++k)
    if (any_error(&s.gate[k])) return true;
  return false;
}
int dev_set_lengths(const DevState& s, const int32_t* vals, int mode) {
  if (gate_closed(s)) return 0;
  for (int b = 0; b < s.batch; ++b) {
    if (mode == 2) {
      s.len[b] = 0;
      s.next_pos[b] = 0;
      if (s.ring) s.held[b] = 0;
    } else {
      s.len[b] = vals[b];
      if (mode == 0) s.next_pos[b] = vals[b];
      if (s.ring && vals[b] < s.held[b]) s.held[b] = vals[b];
    }
  }
  return 0;
}
int dev_set_rows(const DevState& s, const int32_t* vals) {
  for (int b = 0; b < s.batch; ++b) s.rows[b] = vals[b];
  return 0;
}
// Block moves on host memory, with the device kernels' gating.
static int elem_bytes(int dtype) { return dtype == KVC_F64 ? 8 : (dtype == KVC_F32 ? 4 : 2); }
int dev_set_table(const DevState& s, const int32_t* idx, const int32_t* val, int count) {
  if (gate_closed(s)) return 0;
  for (int k = 0; k < count; ++k) const_cast<int32_t*>(s.block_table)[idx[k]] = val[k];
  return 0;
}
int dev_clear_table(const DevState& s) {
  if (gate_closed(s)) return 0;
  for (size_t k = 0; k < size_t(s.batch) * s.table_width; ++k) const_cast<int32_t*>(s.block_table)[k] = -1;
  return 0;
}
int dev_set_seq_length(const DevState& s, int seq, int32_t value, int held_src) {
  if (gate_closed(s)) return 0;
  s.len[seq] = value;
  s.next_pos[seq] = value;
  if (s.ring) s.held[seq] = held_src >= 0 ? s.held[held_src] : 0;
  return 0;
}
int dev_copy_block_rows(const DevState& s, int dst, int src, int rows) {
  if (gate_closed(s) || rows <= 0) return 0;
  const size_t row = size_t(s.head_width) * elem_bytes(s.dtype), head = row << s.block_rows_log2;
  for (int h = 0; h < s.kv_heads; ++h)
    for (void* base : {s.keys, s.values})
      std::memcpy(static_cast<char*>(base) + (size_t(dst) * s.kv_heads + h) * head,
                  static_cast<char*>(base) + (size_t(src) * s.kv_heads + h) * head, size_t(rows) * row);
  return 0;
}
int dev_copy_positions(const DevState& s, int dst_seq, int src_seq, int rows) {
  if (gate_closed(s)) return 0;
  for (int k = 0; k < rows; ++k)
    s.positions[size_t(dst_seq) * s.capacity + k] = s.positions[size_t(src_seq) * s.capacity + k];
  return 0;
}
int dev_copy_seq_rows(const DevState& s, int dst_seq, int src_seq, int rows) {
  if (gate_closed(s) || rows <= 0) return 0;
  const size_t row = size_t(s.head_width) * elem_bytes(s.dtype), lane = row * s.capacity;
  for (int h = 0; h < s.kv_heads; ++h)
    for (void* base : {s.keys, s.values})
      std::memcpy(static_cast<char*>(base) + (size_t(dst_seq) * s.kv_heads + h) * lane,
                  static_cast<char*>(base) + (size_t(src_seq) * s.kv_heads + h) * lane, size_t(rows) * row);
  return 0;
}
// Fake kernels (off by default; kvc_test_fake_kernels turns them on): no
// attention is computed, but the projection fills the candidate rows with a
// tag of (call, sequence, row, head, element) and the commit appends them
// through the block table, so the manager's block bookkeeping can be checked
// row by row.  kvc_test_fail_next makes the next projection set a failure
// word (a non-finite key at the given flat index).
static bool g_fake = false;
static int g_call = 0;
static long long g_fail_next = -1;
static size_t kv_off(const DevState& s, int b, int h, int r) {
  if (s.ring) r %= s.capacity;
  if (!s.paged) return ((size_t(b) * s.kv_heads + h) * s.capacity + r) * s.head_width;
  const int lg = s.block_rows_log2;
  const int blk = s.block_table[size_t(b) * s.table_width + (r >> lg)];
  return (((size_t(blk) * s.kv_heads + h) << lg) + (r & ((1 << lg) - 1))) * s.head_width;
}
int dev_project(const DevState& s, const void*, int n_max, int per_seq) {
  if (!g_fake) return 1;
  ++g_call;
  for (int b = 0; b < s.batch; ++b) {
    const int n = per_seq ? s.rows[b] : n_max;
    for (int h = 0; h < s.kv_heads; ++h)
      for (int i = 0; i < n; ++i)
        for (int e = 0; e < s.head_width; ++e) {
          const size_t at = ((size_t(b) * s.kv_heads + h) * n_max + i) * s.head_width + e;
          const double tag = g_call * 1e6 + b * 1e4 + i * 1e2 + h * 10 + e;
          static_cast<double*>(s.cand_k)[at] = tag;
          static_cast<double*>(s.cand_v)[at] = -tag;
        }
  }
  if (g_fail_next >= 0) {
    s.err->key = (unsigned long long)g_fail_next;
    g_fail_next = -1;
  }
  return 0;
}
int dev_attend_decode(const DevState&, const SeqOrder&, void*) { return g_fake ? 0 : 1; }
int dev_merge_decode(const DevState&, void*) { return g_fake ? 0 : 1; }
int dev_newest_weights(const DevState&, int, int, int, void*) { return 1; }
int dev_attend_chunk(const DevState&, int, int, const ChunkOrder&, void*) { return g_fake ? 0 : 1; }
int dev_output_project(const DevState&, int, int, void*) { return g_fake ? 0 : 1; }
int dev_commit(const DevState& s, int n_max, int per_seq) {
  if (!g_fake) return 1;
  if (gate_closed(s)) return 0;
  for (int b = 0; b < s.batch; ++b) {
    const int n = per_seq ? s.rows[b] : n_max;
    for (int i = 0; i < n; ++i) {
      const int r = s.len[b] + i;
      for (int h = 0; h < s.kv_heads; ++h) {
        const size_t src = ((size_t(b) * s.kv_heads + h) * n_max + i) * s.head_width;
        const size_t dst = kv_off(s, b, h, r);
        for (int e = 0; e < s.head_width; ++e) {
          static_cast<double*>(s.keys)[dst + e] = static_cast<const double*>(s.cand_k)[src + e];
          static_cast<double*>(s.values)[dst + e] = static_cast<const double*>(s.cand_v)[src + e];
        }
      }
      s.positions[size_t(b) * s.capacity + (s.ring ? r % s.capacity : r)] = s.next_pos[b] + i;
    }
    s.len[b] += n;
    s.next_pos[b] += n;
    if (s.ring && n > 0 && s.len[b] - s.capacity > s.held[b]) s.held[b] = s.len[b] - s.capacity;
  }
  return 0;
}
// The session's row kernels compute nothing here either; with the fake kernels on
// they succeed so that session calls reach the per-layer stages and commits.
int dev_embed(const DevState&, const int32_t*, const void*, int, int, int, int, void*, void*) { return g_fake ? 0 : 1; }
int dev_residual(const DevState&, const void*, const void*, void*, void*, int, int) { return g_fake ? 0 : 1; }
int dev_event_create(void** e) {
  *e = std::malloc(1);
  return 0;
}
void dev_event_destroy(void* e) { std::free(e); }
int dev_event_record(void*, void*) { return 0; }
int dev_event_elapsed(float* ms, void*, void*) {
  *ms = 0.f;
  return 0;
}
int dev_stream_read(const void*, int64_t, void*, void*) { return 1; }
int dev_mfma_rate(int64_t, void*, void*, double* flops) {
  *flops = 0;
  return 1;
}
bool dev_has_kernels() { return g_fake; }
// The no-allocation entry point's scratch: host memory here, and a smaller
// size (kvc_test_static_scratch_bytes) so that the size check can be tested.
static size_t g_static_bytes = kStaticScratchBytes;
int dev_static_scratch(int, void** ptr, size_t* bytes) {
  static void* mem = std::aligned_alloc(256, kStaticScratchBytes);
  if (!mem) return 2;
  *ptr = mem;
  *bytes = g_static_bytes;
  return 0;
}

}  // namespace kvc

// Test hooks (not part of the library ABI).
extern "C" void kvc_test_fake_kernels(int on) {
  kvc::g_fake = on != 0;
  kvc::g_call = 0;
  kvc::g_fail_next = -1;
}
extern "C" void kvc_test_fail_next(long long flat_index) { kvc::g_fail_next = flat_index; }
extern "C" void kvc_test_static_scratch_bytes(unsigned long long bytes) {
  kvc::g_static_bytes = bytes ? size_t(bytes) : kvc::kStaticScratchBytes;
}
extern "C" int kvc_test_chunk_order(int batch, int n_max, const int32_t* len, const int32_t* rows, int32_t* qtiles,
                                    int32_t* items) {
  kvc::ChunkOrder o;
  kvc::build_chunk_order(&o, batch, n_max, len, rows);
  *qtiles = o.qtiles;
  for (int k = 0; k < o.count; ++k) items[k] = o.item[k];
  return o.count;
}
extern "C" int kvc_test_seq_order(int batch, const int32_t* len, int per_round, int32_t* seq) {
  kvc::SeqOrder o;
  kvc::build_seq_order(&o, batch, len, per_round);
  for (int k = 0; k < o.count; ++k) seq[k] = o.seq[k];
  return o.count;
}
