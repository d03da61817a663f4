// CPU-only stand-in for the device backend, used to test the host cache
// manager (validation order, bookkeeping, snapshots of zeroed storage) on a
// machine without a GPU.  "Device" memory is host memory and no kernel can
// run: every compute launch reports an error, so nothing here computes
// attention.  Built by tests/test_host_manager.py; never shipped.
#include <cstdlib>
#include <cstring>

#include "../incremental_kv_cache_amd/csrc/kvc_internal.h"

namespace kvc {

const char* dev_error_string(int) { return "no device in the host-check build"; }
int dev_current_device(int* device) {
  *device = -1;
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
    } else {
      s.len[b] = vals[b];
      if (mode == 0) s.next_pos[b] = vals[b];
    }
  }
  return 0;
}
int dev_set_rows(const DevState& s, const int32_t* vals) {
  for (int b = 0; b < s.batch; ++b) s.rows[b] = vals[b];
  return 0;
}
int dev_project(const DevState&, const void*, int, int) { return 1; }
int dev_attend_decode(const DevState&, const SeqOrder&, void*) { return 1; }
int dev_merge_decode(const DevState&, void*) { return 1; }
int dev_attend_chunk(const DevState&, int, int, const ChunkOrder&, void*) { return 1; }
int dev_output_project(const DevState&, int, int, void*) { return 1; }
int dev_commit(const DevState&, int, int) { return 1; }
int dev_embed(const DevState&, const int32_t*, const void*, int, int, int, int, void*, void*) { return 1; }
int dev_residual(const DevState&, const void*, const void*, void*, void*, int, int) { return 1; }
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
bool dev_has_kernels() { return false; }

}  // namespace kvc

// Test hooks for the host-side work orders (not part of the library ABI).
extern "C" int kvc_test_chunk_order(int batch, int n_max, const int32_t* len, const int32_t* rows, int32_t* qtiles,
                                    int32_t* items) {
  kvc::ChunkOrder o;
  kvc::build_chunk_order(&o, batch, n_max, len, rows);
  *qtiles = o.qtiles;
  for (int k = 0; k < o.count; ++k) items[k] = o.item[k];
  return o.count;
}
extern "C" int kvc_test_seq_order(int batch, const int32_t* len, int32_t* seq) {
  kvc::SeqOrder o;
  kvc::build_seq_order(&o, batch, len);
  for (int k = 0; k < o.count; ++k) seq[k] = o.seq[k];
  return o.count;
}
