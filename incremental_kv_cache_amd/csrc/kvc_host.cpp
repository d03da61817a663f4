// Host side of libkvcache: handles, request validation in the order Chapter 37
// fixes, bookkeeping (lengths, next positions, binding), error reporting, and
// the C ABI declared in include/kvcache.h.  All device work goes through the
// backend interface in kvc_internal.h.
//
// Chapter 37 = "Keep the prefix, project only the new row" (incremental
// attention course chapter); prefix-reuse note = "LLM mechanism experiment
// (5): can only the changed suffix be recomputed?".
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "kvc_internal.h"

using namespace kvc;

struct kvc_params {
  int32_t model_width;
  int32_t kv_width;      // rows of W_k and W_v: H_kv * d_h (= model_width without grouping)
  kvc_dtype dtype;
  const void* w[4];      // W_q, W_k, W_v, W_o (W_o may be null)
  int32_t nweights;      // 3 without W_o, 4 with it
  uint64_t id;           // identity: unique per created parameter set
  uint64_t revision[4];  // value revision per weight
};

struct kvc_layer {
  const kvc_params* params;
  int32_t heads, head_width;
  int32_t kv_heads;  // key/value heads; query head h reads key/value head h / (heads / kv_heads)
  int32_t window;    // sliding window (rows a query reads, itself included); 0 = the whole prefix
  kvc_pos_mode pos_mode;
  double rope_base;
  int32_t rope_max_positions;
  int32_t rope_feature_width() const { return pos_mode == KVC_POS_ROPE ? head_width : 0; }
};

namespace {

struct Profile {
  int32_t slots = 0;
  int32_t used = 0;
  std::vector<void*> events;  // [slots][KVC_STAGES][2]
  std::vector<int8_t> recorded;
};

}  // namespace

struct kvc_cache {
  // geometry and binding (Chapter 37, layer-kv-cache listing: the cache struct)
  int32_t batch, heads, head_width, model_width, capacity, max_chunk_rows;
  int32_t kv_heads;
  int32_t window;  // sliding window of the bound layer (0: none); window caches are rings of `capacity` rows
  kvc_dtype dtype;
  uint64_t params_id;
  uint64_t revision[4];
  int32_t rope_feature_width, rope_max_positions;
  uint64_t rope_base_bits;
  double rope_base;
  kvc_pos_mode pos_mode;
  int device;
  int compute_units = 256;
  // host copy of the committed state
  std::vector<int32_t> len, next_pos;
  std::vector<int32_t> held;  // window (ring) caches: oldest row each sequence still holds
  bool pending_async = false;
  // device state
  DevState ds{};
  ErrWords* err_host = nullptr;  // pinned readback
  int64_t storage_bytes = 0;
  Profile prof;
  ChunkOrder order{};     // work order of the last chunk call
  SeqOrder seq_order{};   // sequence order of the last decode call
  bool session = false;   // a layer cache of a kvc_session: its failure words belong to the session
  // the query scratch holds the rotated queries of the newest committed rows
  // (set by a successful kvc_append_and_attend, cleared by every other call
  // that moves the cache)
  bool newest_q_valid = false;
  // block paging (paged caches only): host copy of the block table and the pool's bookkeeping
  bool paged = false;
  int32_t block_rows = 0, block_lg = 0, table_width = 0, pool_blocks = 0;
  std::vector<int32_t> table;        // [B * table_width], -1 = no block
  std::vector<int32_t> refcount;     // [pool_blocks]: table entries naming the block
  std::vector<int32_t> free_blocks;  // unreferenced blocks (a stack)
};

struct kvc_session {
  std::vector<const kvc_layer*> layers;
  std::vector<kvc_cache*> caches;  // one per layer, created and destroyed with the session
  int32_t batch = 0, max_chunk_rows = 0, model_width = 0, vocab = 0;
  kvc_dtype dtype = KVC_F64;
  int sinusoidal = 0;
  const void* embedding = nullptr;
  kvc::ErrWords* gate = nullptr;  // device: the layers' failure words, [L]
  void* h = nullptr;              // device [B, max_chunk_rows, D], accumulate type: the running rows
  void* a = nullptr;              // device [B, max_chunk_rows, D], accumulate type: a layer's attention
  void* x = nullptr;              // device [B, max_chunk_rows, D], weight type (bf16 sessions only)
  bool pending_async = false;
};

void kvc::build_chunk_order(ChunkOrder* o, int batch, int n_max, const int32_t* len, const int32_t* rows) {
  o->qtiles = (n_max + kChunkQueryTile - 1) / kChunkQueryTile;
  o->count = 0;
  if (int64_t(batch) * o->qtiles > kMaxChunkOrder) return;
  // (keys read by the tile's last query, item); a stable sort keeps equal
  // items in sequence order
  std::vector<std::pair<int64_t, int32_t>> w;
  for (int b = 0; b < batch; ++b) {
    const int n_b = rows ? rows[b] : n_max;
    for (int qt = 0; qt * kChunkQueryTile < n_b; ++qt) {
      const int64_t keys = int64_t(len[b]) + std::min(n_b, (qt + 1) * kChunkQueryTile);
      w.emplace_back(keys, (b << 16) | qt);
    }
  }
  std::stable_sort(w.begin(), w.end(), [](const auto& a, const auto& c) { return a.first > c.first; });
  for (size_t k = 0; k < w.size(); ++k) o->item[k] = w[k].second;
  o->count = int32_t(w.size());
}

void kvc::build_seq_order(SeqOrder* o, int batch, const int32_t* len, int per_round) {
  o->count = 0;
  if (batch > kMaxSeqOrder) return;
  for (int b = 0; b < batch; ++b) o->seq[b] = b;
  std::stable_sort(o->seq, o->seq + batch, [&](int32_t a, int32_t c) { return len[a] > len[c]; });
  per_round = std::max(per_round, 1);
  for (int r0 = per_round; r0 < batch; r0 += 2 * per_round)
    std::reverse(o->seq + r0, o->seq + std::min(batch, r0 + per_round));
  o->count = batch;
}

namespace {

std::atomic<uint64_t> g_next_params_id{1};
thread_local kvc_error_detail g_last;

size_t elem_size(kvc_dtype t) { return t == KVC_F64 ? 8 : (t == KVC_F32 ? 4 : 2); }
size_t acc_size(kvc_dtype t) { return t == KVC_F64 ? 8 : 4; }

void reset_detail() {
  std::memset(&g_last, 0, sizeof(g_last));
  g_last.parameter = -1;
  g_last.sequence = -1;
  g_last.layer = -1;
  g_last.flat_index = -1;
}

kvc_status fail(kvc_status st, const char* fmt, ...) {
  g_last.status = st;
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last.message, sizeof(g_last.message), fmt, ap);
  va_end(ap);
  return st;
}

kvc_status fail_ea(kvc_status st, int64_t expected, int64_t actual, const char* fmt, ...) {
  g_last.expected = expected;
  g_last.actual = actual;
  g_last.status = st;
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last.message, sizeof(g_last.message), fmt, ap);
  va_end(ap);
  return st;
}

kvc_status device_fail(int code, const char* what) {
  return fail(KVC_ERR_DEVICE, "%s failed: %s", what, dev_error_string(code));
}

bool checked_mul(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

int max_head_width(kvc_dtype t) { return t == KVC_F64 ? 128 : (t == KVC_F32 ? 256 : 512); }

// Request checks shared by both compute calls, from cache model width through
// the rotary configuration (Chapter 37, "Bind the state, calculate
// completely, then commit": the binding check).
kvc_status check_binding(const kvc_layer* layer, const kvc_cache* c) {
  const kvc_params* p = layer->params;
  if (c->model_width != p->model_width)
    return fail_ea(KVC_ERR_CACHE_MODEL_WIDTH_MISMATCH, p->model_width, c->model_width,
                   "cache model width %d does not match layer model width %d", c->model_width,
                   p->model_width);
  if (c->heads != layer->heads)
    return fail_ea(KVC_ERR_CACHE_HEAD_COUNT_MISMATCH, layer->heads, c->heads,
                   "cache head count %d does not match layer head count %d", c->heads, layer->heads);
  if (c->kv_heads != layer->kv_heads)
    return fail_ea(KVC_ERR_CACHE_HEAD_COUNT_MISMATCH, layer->kv_heads, c->kv_heads,
                   "cache key/value head count %d does not match layer key/value head count %d", c->kv_heads,
                   layer->kv_heads);
  if (c->head_width != layer->head_width)
    return fail_ea(KVC_ERR_CACHE_HEAD_WIDTH_MISMATCH, layer->head_width, c->head_width,
                   "cache head width %d does not match layer head width %d", c->head_width,
                   layer->head_width);
  if (c->params_id != p->id)
    return fail(KVC_ERR_CACHE_LAYER_MISMATCH,
                "cache was created for a different attention layer (parameter identity differs)");
  for (int k = 0; k < p->nweights; ++k) {
    if (c->revision[k] != p->revision[k]) {
      g_last.parameter = k;
      g_last.cache_revision = c->revision[k];
      g_last.layer_revision = p->revision[k];
      return fail(KVC_ERR_CACHE_LAYER_REVISION_MISMATCH,
                  "cache parameter %d was captured at value revision %llu, but the layer is at revision %llu",
                  k, (unsigned long long)c->revision[k], (unsigned long long)p->revision[k]);
    }
  }
  uint64_t base_bits;
  std::memcpy(&base_bits, &layer->rope_base, 8);
  if (c->rope_feature_width != layer->rope_feature_width() ||
      c->rope_max_positions != layer->rope_max_positions || c->rope_base_bits != base_bits) {
    g_last.rope_feature_width[0] = c->rope_feature_width;
    g_last.rope_feature_width[1] = layer->rope_feature_width();
    g_last.rope_max_positions[0] = c->rope_max_positions;
    g_last.rope_max_positions[1] = layer->rope_max_positions;
    g_last.rope_base[0] = c->rope_base;
    g_last.rope_base[1] = layer->rope_base;
    return fail(KVC_ERR_CACHE_ROPE_MISMATCH,
                "cache RoPE (feature width %d, max positions %d, base %g) does not match layer RoPE "
                "(feature width %d, max positions %d, base %g)",
                c->rope_feature_width, c->rope_max_positions, c->rope_base, layer->rope_feature_width(),
                layer->rope_max_positions, layer->rope_base);
  }
  if (c->window != layer->window)
    return fail_ea(KVC_ERR_CACHE_WINDOW_MISMATCH, layer->window, c->window,
                   "cache sliding window %d does not match layer window %d", c->window, layer->window);
  return KVC_OK;
}

// Whether sequence b of a window cache can continue from `cut`: cut 0 (a
// recompute), or every row the continuation's first row reads (cut - window + 1
// .. cut - 1) is still held, i.e. not older than the last `capacity` rows
// (prefix-reuse note, "Why a sliding-window partial hit must fall back").
bool window_continuable(const kvc_cache* c, int b, int64_t cut) {
  if (cut == 0) return true;
  if (cut < 0 || cut > c->len[b]) return false;
  return c->window == 0 || std::max<int64_t>(0, cut - c->window + 1) >= c->held[b];
}

// Smallest nonzero cut a window cache's sequence b can continue from.
int32_t window_min_cut(const kvc_cache* c, int b) {
  return std::max(1, c->window ? c->held[b] + c->window - 1 : 1);
}

// Reads the device failure words; on a failure fills the detail, clears the
// words and returns the failure's status (KVC_OK otherwise).  Stream must be idle.
kvc_status collect_device_error(kvc_cache* c, int64_t n_max_for_index) {
  int rc = dev_copy_d2h_sync(c->err_host, c->ds.err, sizeof(ErrWords), c->ds.stream);
  if (rc) return device_fail(rc, "reading the device error words");
  const ErrWords e = *c->err_host;
  kvc_status st = KVC_OK;
  unsigned long long idx = kErrClear;
  if (e.token != kErrClear) {
    st = KVC_ERR_TOKEN_RANGE;
    idx = e.token;
  } else if (e.key != kErrClear) {
    st = KVC_ERR_NONFINITE_KEY;
    idx = e.key;
  } else if (e.value != kErrClear) {
    st = KVC_ERR_NONFINITE_VALUE;
    idx = e.value;
  } else if (e.query != kErrClear) {
    st = KVC_ERR_NONFINITE_QUERY;
    idx = e.query;
  } else if (e.position != kErrClear) {
    st = KVC_ERR_ROTARY_POSITION;
    idx = e.position;
  } else if (e.output != kErrClear) {
    st = KVC_ERR_NONFINITE_OUTPUT;
    idx = e.output;
  }
  if (st == KVC_OK) return KVC_OK;
  (void)n_max_for_index;
  g_last.flat_index = int64_t(idx);
  if (st == KVC_ERR_NONFINITE_KEY || st == KVC_ERR_NONFINITE_VALUE) {
    // the offending element is still in the candidate buffer
    const void* src = static_cast<const char*>(st == KVC_ERR_NONFINITE_KEY ? c->ds.cand_k : c->ds.cand_v) +
                      idx * elem_size(c->dtype);
    uint64_t raw = 0;
    if (dev_copy_d2h_sync(&raw, src, elem_size(c->dtype), c->ds.stream) == 0) {
      if (c->dtype == KVC_F64) {
        std::memcpy(&g_last.value, &raw, 8);
      } else if (c->dtype == KVC_F32) {
        float f;
        std::memcpy(&f, &raw, 4);
        g_last.value = f;
      } else {
        uint32_t u = uint32_t(raw & 0xffff) << 16;
        float f;
        std::memcpy(&f, &u, 4);
        g_last.value = f;
      }
    }
  }
  if (st == KVC_ERR_ROTARY_POSITION) g_last.sequence = int32_t(idx);
  rc = dev_clear_err(c->ds.err, c->ds.stream);
  if (rc == 0) rc = dev_sync(c->ds.stream);
  if (rc) return device_fail(rc, "clearing the device error words");
  switch (st) {
    case KVC_ERR_NONFINITE_KEY:
      return fail(st, "candidate key element %llu is not finite (%g); nothing was appended", idx, g_last.value);
    case KVC_ERR_NONFINITE_VALUE:
      return fail(st, "candidate value element %llu is not finite (%g); nothing was appended", idx, g_last.value);
    case KVC_ERR_NONFINITE_QUERY:
      return fail(st, "rotated query at flat index %llu is not finite", idx);
    case KVC_ERR_ROTARY_POSITION:
      return fail(st, "sequence %llu reached the rotary position capacity %d", idx, c->rope_max_positions);
    case KVC_ERR_TOKEN_RANGE:
      return fail(st, "token at flat index %llu is outside the embedding", idx);
    default:
      return fail(st, "attention output at flat index %llu is not finite", idx);
  }
}

kvc_status resync_lengths(kvc_cache* c) {
  const size_t bytes = sizeof(int32_t) * size_t(c->batch);
  int rc = dev_copy_d2h_sync(c->len.data(), c->ds.len, bytes, c->ds.stream);
  if (rc == 0) rc = dev_copy_d2h_sync(c->next_pos.data(), c->ds.next_pos, bytes, c->ds.stream);
  if (rc == 0 && c->ds.ring) rc = dev_copy_d2h_sync(c->held.data(), c->ds.held, bytes, c->ds.stream);
  if (rc) return device_fail(rc, "reading lengths");
  return KVC_OK;
}

// ---- block paging ---------------------------------------------------------

// Sends table entries idx[k] = c->table[idx[k]] to the device (gated there like
// the length updates).
kvc_status upload_table(kvc_cache* c, const std::vector<int32_t>& idx) {
  if (idx.empty()) return KVC_OK;
  std::vector<int32_t> val(idx.size());
  for (size_t k = 0; k < idx.size(); ++k) val[k] = c->table[idx[k]];
  const int rc = dev_set_table(c->ds, idx.data(), val.data(), int(idx.size()));
  if (rc) return device_fail(rc, "block table update");
  return KVC_OK;
}

// Blocks holding rows [0, rows).
int blocks_for(const kvc_cache* c, int rows) { return (rows + c->block_rows - 1) >> c->block_lg; }

// Drops one reference to block `blk` (back to the free list at zero).
void release_block(kvc_cache* c, int32_t blk) {
  if (blk < 0) return;
  if (--c->refcount[blk] == 0) c->free_blocks.push_back(blk);
}

// Releases the blocks of sequence b from logical block `keep` on (host mirror);
// appends the changed table indices to `changed`.
void release_tail(kvc_cache* c, int b, int keep, std::vector<int32_t>& changed) {
  for (int j = keep; j < c->table_width; ++j) {
    const int idx = b * c->table_width + j;
    if (c->table[idx] < 0) continue;
    release_block(c, c->table[idx]);
    c->table[idx] = -1;
    changed.push_back(idx);
  }
}

// Rebuilds the host table, reference counts and free list from the device
// table (after a deferred failure suppressed table updates).  Stream idle.
kvc_status resync_paging(kvc_cache* c) {
  if (!c->paged) return KVC_OK;
  const int rc = dev_copy_d2h_sync(c->table.data(), c->ds.block_table, sizeof(int32_t) * c->table.size(),
                                   c->ds.stream);
  if (rc) return device_fail(rc, "reading the block table");
  std::fill(c->refcount.begin(), c->refcount.end(), 0);
  for (int32_t blk : c->table)
    if (blk >= 0) c->refcount[blk]++;
  c->free_blocks.clear();
  for (int blk = c->pool_blocks - 1; blk >= 0; --blk)
    if (c->refcount[blk] == 0) c->free_blocks.push_back(blk);
  // a failed call may have left blocks past the committed rows: give them back
  std::vector<int32_t> changed;
  for (int b = 0; b < c->batch; ++b) release_tail(c, b, blocks_for(c, c->len[b]), changed);
  return upload_table(c, changed);
}

// Blocks a call takes before it launches: fresh blocks for rows past the
// sequence's last block, and private copies of shared blocks the call appends
// into (copy-on-write).  Undone by revert_blocks when the call fails.
struct BlockReservation {
  std::vector<int32_t> idx, old_val;  // table entries changed, and their previous values
};

kvc_status reserve_blocks(kvc_cache* c, int n_max, const int32_t* n_rows, BlockReservation& r) {
  struct Need {
    int idx, old, copy_rows;
  };
  std::vector<Need> need;
  for (int b = 0; b < c->batch; ++b) {
    const int n = n_rows ? n_rows[b] : n_max;
    if (n <= 0) continue;
    const int len = c->len[b];
    const int first = len >> c->block_lg, last = (len + n - 1) >> c->block_lg;
    for (int j = first; j <= last; ++j) {
      const int idx = b * c->table_width + j;
      const int cur = c->table[idx];
      if (cur >= 0 && c->refcount[cur] == 1) continue;  // private block already in place
      const int copy_rows = cur >= 0 && j == first ? len - (j << c->block_lg) : 0;
      need.push_back({idx, cur, copy_rows});
    }
  }
  if (need.empty()) return KVC_OK;
  if (need.size() > c->free_blocks.size())
    return fail_ea(KVC_ERR_OUT_OF_BLOCKS, int64_t(need.size()), int64_t(c->free_blocks.size()),
                   "the block pool has %zu free blocks, the call needs %zu", c->free_blocks.size(), need.size());
  for (const Need& nd : need) {
    const int32_t blk = c->free_blocks.back();
    c->free_blocks.pop_back();
    c->refcount[blk] = 1;
    if (nd.old >= 0) c->refcount[nd.old]--;  // still referenced elsewhere: it was shared
    c->table[nd.idx] = blk;
    r.idx.push_back(nd.idx);
    r.old_val.push_back(nd.old);
    if (nd.old >= 0) {
      const int rc = dev_copy_block_rows(c->ds, blk, nd.old, nd.copy_rows);
      if (rc) return device_fail(rc, "copy-on-write of a shared block");
    }
  }
  return upload_table(c, r.idx);
}

void revert_blocks(kvc_cache* c, const BlockReservation& r) {
  for (size_t k = r.idx.size(); k-- > 0;) {
    const int idx = r.idx[k];
    release_block(c, c->table[idx]);
    if (r.old_val[k] >= 0) c->refcount[r.old_val[k]]++;
    c->table[idx] = r.old_val[k];
  }
  (void)upload_table(c, r.idx);
}

// Reports an error left by earlier KVC_ASYNC calls (synchronises).
kvc_status check_deferred(kvc_cache* c) {
  if (!c->pending_async) return KVC_OK;
  int rc = dev_sync(c->ds.stream);
  if (rc) return device_fail(rc, "stream synchronisation");
  c->pending_async = false;
  kvc_status st = collect_device_error(c, 0);
  if (st == KVC_ERR_DEVICE) return st;
  if (st != KVC_OK) {
    const kvc_status orig = st;
    const kvc_error_detail saved = g_last;
    kvc_status rs = resync_lengths(c);
    if (rs == KVC_OK) rs = resync_paging(c);
    if (rs != KVC_OK) return rs;
    g_last = saved;
    g_last.actual = orig;
    return fail(KVC_ERR_DEFERRED, "an earlier asynchronous call failed: %s (%s)", kvc_status_name(orig),
                std::string(g_last.message).c_str());
  }
  return KVC_OK;
}

void profile_mark(kvc_cache* c, int stage, int which) {
  Profile& p = c->prof;
  if (p.slots <= 0 || p.used >= p.slots) return;
  const size_t k = (size_t(p.used) * KVC_STAGES + stage) * 2 + which;
  if (dev_event_record(p.events[k], c->ds.stream) == 0 && which == 1) p.recorded[size_t(p.used) * KVC_STAGES + stage] = 1;
}

void profile_end_call(kvc_cache* c) {
  if (c->prof.slots > 0 && c->prof.used < c->prof.slots) c->prof.used++;
}

void free_cache(kvc_cache* c) {
  if (!c) return;
  dev_free(c->ds.keys);
  dev_free(c->ds.values);
  dev_free(c->ds.len);
  dev_free(c->ds.next_pos);
  dev_free(c->ds.positions);
  dev_free(c->ds.rows);
  dev_free(c->ds.held);
  dev_free(c->ds.cand_k);
  dev_free(c->ds.cand_v);
  dev_free(c->ds.q);
  dev_free(c->ds.partials);
  dev_free(c->ds.redo);
  dev_free(c->ds.rope_cos);
  dev_free(c->ds.rope_sin);
  if (!c->session) dev_free(c->ds.err);
  dev_free(const_cast<int32_t*>(c->ds.block_table));
  dev_free(c->ds.merged);
  dev_free(c->ds.proj_partials);
  dev_host_free(c->err_host);
  for (void* e : c->prof.events) dev_event_destroy(e);
  delete c;
}

// The compute stages of one call: projection, attention, split merge, output
// projection.  Merged heads (or W_o's result) go to `out`.
kvc_status compute_stages(kvc_cache* c, const void* x, int n_max, const int32_t* n_rows, void* out, bool decode) {
  DevState& s = c->ds;
  const int per_seq = n_rows != nullptr;
  int rc = 0;
  if (per_seq) {
    rc = dev_set_rows(s, n_rows);
    if (rc) return device_fail(rc, "chunk row upload");
  }
  // a chunk call's queries go to the flash kernel (bf16, d_h 64 or 128) as
  // its scaled bf16 operand; decode calls keep float32 queries
  s.q_bf16 = !decode && s.dtype == KVC_BF16 && (s.head_width == 64 || s.head_width == 128);
  profile_mark(c, KVC_STAGE_PROJECT, 0);
  rc = dev_project(s, x, n_max, per_seq);
  profile_mark(c, KVC_STAGE_PROJECT, 1);
  if (rc) return device_fail(rc, "projection launch");
  // merged heads go straight to the caller's output, or to scratch when the
  // output projection follows
  void* heads = s.wo ? s.merged : out;
  profile_mark(c, KVC_STAGE_ATTEND, 0);
  if (decode) {
    // one round: the sequences whose workgroups put one on every compute unit
    const int qpw = decode_heads_per_block(c->dtype, c->head_width, c->heads / c->kv_heads);
    build_seq_order(&c->seq_order, c->batch, c->len.data(), c->compute_units / (c->heads / qpw));
    rc = dev_attend_decode(s, c->seq_order, heads);
  } else {
    build_chunk_order(&c->order, c->batch, n_max, c->len.data(), per_seq ? n_rows : nullptr);
    rc = dev_attend_chunk(s, n_max, per_seq, c->order, heads);
  }
  profile_mark(c, KVC_STAGE_ATTEND, 1);
  if (rc) return device_fail(rc, "attention launch");
  if (decode) {
    profile_mark(c, KVC_STAGE_MERGE, 0);
    rc = dev_merge_decode(s, heads);
    profile_mark(c, KVC_STAGE_MERGE, 1);
    if (rc) return device_fail(rc, "merge launch");
  }
  if (s.wo) {
    profile_mark(c, KVC_STAGE_OUTPUT, 0);
    rc = dev_output_project(s, n_max, per_seq, out);
    profile_mark(c, KVC_STAGE_OUTPUT, 1);
    if (rc) return device_fail(rc, "output projection launch");
  }
  return KVC_OK;
}

// The predicated append (suppressed on the device while a gate word is set).
kvc_status commit_stage(kvc_cache* c, int n_max, const int32_t* n_rows) {
  profile_mark(c, KVC_STAGE_COMMIT, 0);
  const int rc = dev_commit(c->ds, n_max, n_rows != nullptr);
  profile_mark(c, KVC_STAGE_COMMIT, 1);
  profile_end_call(c);
  if (rc) return device_fail(rc, "commit launch");
  return KVC_OK;
}

void advance_mirror(kvc_cache* c, int n_max, const int32_t* n_rows) {
  for (int b = 0; b < c->batch; ++b) {
    const int n = n_rows ? n_rows[b] : n_max;
    if (n <= 0) continue;
    c->len[b] += n;
    c->next_pos[b] += n;
    if (c->window) c->held[b] = std::max(c->held[b], c->len[b] - c->capacity);  // slots reused
  }
}

// Runs the stages of one call and the sync-mode error collection.
// Paged caches first take the blocks the appended rows land in (and private
// copies of shared blocks they append into); a call that fails gives them back.
kvc_status run_call(kvc_cache* c, const void* x, int n_max, const int32_t* n_rows, void* out, int32_t flags,
                    bool decode) {
  BlockReservation r;
  kvc_status st = KVC_OK;
  if (c->paged) {
    st = reserve_blocks(c, n_max, n_rows, r);
    if (st != KVC_OK) {
      const kvc_error_detail saved = g_last;
      revert_blocks(c, r);
      g_last = saved;
      return st;
    }
  }
  st = compute_stages(c, x, n_max, n_rows, out, decode);
  if (st == KVC_OK) st = commit_stage(c, n_max, n_rows);
  if (st == KVC_OK && (flags & KVC_ASYNC)) {
    c->pending_async = true;
    advance_mirror(c, n_max, n_rows);
    return KVC_OK;
  }
  if (st == KVC_OK) {
    const int rc = dev_sync(c->ds.stream);
    st = rc ? device_fail(rc, "stream synchronisation") : collect_device_error(c, n_max);
  }
  if (st != KVC_OK) {
    const kvc_error_detail saved = g_last;
    revert_blocks(c, r);
    g_last = saved;
    return st;
  }
  advance_mirror(c, n_max, n_rows);
  return KVC_OK;
}

// Split-K tile of a decode call: the largest power-of-two multiple of 512
// rows that still gives at least 1024 workgroups (four per compute unit; 512
// when a workgroup serves several query heads);
// measured on the bench workloads, fewer and longer tiles stream faster than a
// finer split.
int64_t decode_span_rows(const kvc_cache* cache, int b) {
  // rows the newest query of sequence b reads from its tile-aligned start (the
  // whole prefix, or the window rounded down to a tile boundary)
  const int64_t len = cache->len[b];
  const int64_t rs = cache->window ? std::max<int64_t>(0, len - cache->window + 1) : 0;
  return len + 1 - (rs - rs % kDecodeTileRows);
}

void choose_decode_tiles(kvc_cache* cache) {
  int tile = kDecodeTileRows;
  int64_t max_len = 0;
  for (int b = 0; b < cache->batch; ++b) max_len = std::max(max_len, decode_span_rows(cache, b) - 1);
  // a workgroup serving several query heads does that many times the work per
  // row it reads: half as many (longer) tiles measured faster for them
  const int qpw = decode_heads_per_block(cache->dtype, cache->head_width, cache->heads / cache->kv_heads);
  const int64_t min_blocks = qpw > 1 ? 512 : 1024;
  for (int64_t cand = kDecodeTileRows; cand <= (int64_t(1) << 30); cand *= 2) {
    int64_t blocks = 0;
    for (int b = 0; b < cache->batch; ++b) blocks += (decode_span_rows(cache, b) - 1 + cand) / cand;
    if (blocks * (cache->heads / qpw) < min_blocks) break;
    tile = int(cand);
    if (cand > max_len) break;
  }
  cache->ds.tile_rows = tile;
  cache->ds.single_tile = tile > max_len;
}

kvc_status reject_session_cache(const char* what) {
  return fail(KVC_ERR_BAD_ARGUMENT, "%s: this cache is a layer of a session; use the kvc_session_* calls", what);
}

// The request checks of a decode call, in Chapter 37's order ("Bind the state,
// calculate completely, then commit": rank, one token, batch, width, binding,
// capacity), then the rotary position; fills the call's row counts.
kvc_status decode_checks(const char* what, const kvc_layer* layer, kvc_cache* cache, const void* x, int32_t rank,
                         const int64_t* shape, void* out, int32_t flags, kvc_work* w) {
  if (!layer || !cache || !x || !out || (rank > 0 && !shape))
    return fail(KVC_ERR_NULL_ARGUMENT, "null argument to %s", what);
  if (cache->session) return reject_session_cache(what);
  if (flags & ~int32_t(KVC_ASYNC)) return fail(KVC_ERR_BAD_ARGUMENT, "unknown flags %d", flags);
  if (!(flags & KVC_ASYNC)) {
    kvc_status d = check_deferred(cache);
    if (d != KVC_OK) return d;
  }
  if (rank != 3) return fail_ea(KVC_ERR_INPUT_RANK, 3, rank, "incremental input must have rank 3, got %d", rank);
  if (shape[1] != 1)
    return fail_ea(KVC_ERR_SINGLE_TOKEN_REQUIRED, 1, shape[1],
                   "incremental attention accepts exactly one token, got %lld", (long long)shape[1]);
  if (shape[0] != cache->batch)
    return fail_ea(KVC_ERR_INPUT_BATCH_MISMATCH, cache->batch, shape[0],
                   "incremental input batch %lld does not match cache batch %d", (long long)shape[0],
                   cache->batch);
  if (shape[2] != layer->params->model_width)
    return fail_ea(KVC_ERR_INPUT_WIDTH_MISMATCH, layer->params->model_width, shape[2],
                   "incremental input width %lld does not match model width %d", (long long)shape[2],
                   layer->params->model_width);
  kvc_status st = check_binding(layer, cache);
  if (st != KVC_OK) return st;
  for (int b = 0; b < cache->batch; ++b) {
    if (!cache->window && cache->len[b] >= cache->capacity) {  // a window cache is a ring
      g_last.sequence = b;
      return fail_ea(KVC_ERR_FULL, cache->capacity, cache->len[b],
                     "sequence %d already holds %d rows, all the cache has room for", b, cache->capacity);
    }
  }
  if (cache->ds.rope) {
    for (int b = 0; b < cache->batch; ++b) {
      if (cache->next_pos[b] >= cache->rope_max_positions) {
        g_last.sequence = b;
        return fail_ea(KVC_ERR_ROTARY_POSITION, cache->rope_max_positions, cache->next_pos[b],
                       "position %d of sequence %d reaches the rotary position capacity %d",
                       cache->next_pos[b], b, cache->rope_max_positions);
      }
    }
  }
  if (!dev_has_kernels()) return fail(KVC_ERR_DEVICE, "library built without device kernels");
  *w = kvc_work{};
  w->position_min = INT32_MAX;
  w->position_max = -1;
  for (int b = 0; b < cache->batch; ++b) {
    w->full_prefix_rows_per_projection += cache->len[b] + 1;
    w->incremental_rows_per_projection += 1;
    w->reused_key_value_rows += cache->len[b];
    w->position_min = std::min(w->position_min, cache->next_pos[b]);
    w->position_max = std::max(w->position_max, cache->next_pos[b]);
  }
  return KVC_OK;
}

// Byte offsets, inside one scratch region, of the buffers a decode call of a
// cache uses beyond its inputs and outputs: the rotated queries [B, H, d_h],
// the candidate key and value rows [B, H_kv, d_h], the split-K partials
// [B, H, max_tiles, d_h + 2], the skinny projection's split sums (when the
// cache has them) and the merged heads before W_o [B, D] (when it has W_o);
// each starts on a 256-byte boundary.  The sizes are those of the cache's own
// buffers at one row per sequence, so both entry points run the same kernels
// with the same launch shapes.
struct ScratchLayout {
  size_t q, cand_k, cand_v, partials, proj, merged, total;
};

ScratchLayout decode_scratch_layout(const kvc_cache* c) {
  auto r256 = [](size_t b) { return (b + 255) & ~size_t(255); };
  const size_t es = elem_size(c->dtype), as = acc_size(c->dtype);
  const size_t B = size_t(c->batch), H = size_t(c->heads), HK = size_t(c->kv_heads), dh = size_t(c->head_width);
  ScratchLayout L{};
  size_t at = 0;
  L.q = at;
  at += r256(B * H * dh * as);
  L.cand_k = at;
  at += r256(B * HK * dh * es);
  L.cand_v = at;
  at += r256(B * HK * dh * es);
  L.partials = at;
  at += r256(B * H * size_t(c->ds.max_tiles) * (dh + 2) * as);
  L.proj = at;
  if (c->ds.proj_partials)
    at += r256(sizeof(float) * kSkinnySplitMax * 64 * size_t(c->model_width + 2 * c->ds.kv_width));
  L.merged = at;
  if (c->ds.merged) at += r256(B * size_t(c->model_width) * as);
  L.total = at;
  return L;
}

// Cache construction.  shared_err: NULL for a standalone cache (it allocates
// its own failure words and gates on them); else this layer's failure words
// inside a session's block, and gate / gate_count the whole block.
kvc_status create_cache(const kvc_layer* layer, int32_t batch, int32_t capacity, int32_t max_chunk_rows,
                        void* hip_stream, ErrWords* shared_err, const ErrWords* gate, int gate_count,
                        kvc_cache** out, int32_t block_rows = 0, int32_t pool_blocks = 0) {
  *out = nullptr;
  // Chapter 37, layer-kv-cache listing: batch, capacity, position capacity,
  // element-count overflow, then allocation.
  if (batch <= 0)
    return fail_ea(KVC_ERR_ZERO_BATCH, 1, batch, "a cache needs at least one sequence, got %d", batch);
  if (capacity <= 0)
    return fail_ea(KVC_ERR_ZERO_CAPACITY, 1, capacity, "a cache needs room for at least one row, got %d", capacity);
  if (capacity > layer->rope_max_positions)
    return fail_ea(KVC_ERR_CAPACITY_EXCEEDS_POSITIONS, layer->rope_max_positions, capacity,
                   "%d rows per sequence need more rotary positions than the layer's %d", capacity,
                   layer->rope_max_positions);
  if (max_chunk_rows <= 0)
    return fail(KVC_ERR_BAD_ARGUMENT, "max_chunk_rows must be at least 1, got %d", max_chunk_rows);
  const bool paged = block_rows != 0;
  const int W = layer->window;
  if (W > 0) {
    // a window cache is a ring of `capacity` rows: it must hold a whole window,
    // whole 256-row runs (the fast kernels' aligned reads never wrap), and a
    // whole chunk (a chunk never overwrites its own rows)
    if (paged) return fail(KVC_ERR_BAD_ARGUMENT, "a sliding-window layer uses a contiguous (ring) cache");
    if (capacity < W || capacity % kMinBlockRows != 0 || max_chunk_rows > capacity)
      return fail_ea(KVC_ERR_BAD_ARGUMENT, W, capacity,
                     "a window cache needs capacity >= window %d, a multiple of %d, and >= max_chunk_rows %d "
                     "(capacity %d)",
                     W, kMinBlockRows, max_chunk_rows, capacity);
  }
  if (paged) {
    // Paged storage: a decode split-K step (at most 256 rows) and a 128-row
    // chunk-attention tile must each fall inside one block.
    if (!is_pow2(block_rows) || block_rows < kMinBlockRows || capacity % block_rows != 0)
      return fail_ea(KVC_ERR_BAD_ARGUMENT, kMinBlockRows, block_rows,
                     "block_rows %d must be a power of two >= %d that divides the capacity %d", block_rows,
                     kMinBlockRows, capacity);
    if (pool_blocks <= 0)
      return fail_ea(KVC_ERR_BAD_ARGUMENT, 1, pool_blocks, "the block pool needs at least one block, got %d",
                     pool_blocks);
  }
  const kvc_params* p = layer->params;
  const int H = layer->heads, HK = layer->kv_heads, dh = layer->head_width;
  int64_t elements = 0, cand = 0, qrows = 0, pos_elems = 0;
  if (!checked_mul(paged ? pool_blocks : batch, HK, &elements) ||
      !checked_mul(elements, paged ? block_rows : capacity, &elements) ||
      !checked_mul(elements, dh, &elements) || !checked_mul(int64_t(batch) * HK, int64_t(max_chunk_rows), &cand) ||
      !checked_mul(cand, dh, &cand) || !checked_mul(int64_t(batch) * H, int64_t(max_chunk_rows), &qrows) ||
      !checked_mul(qrows, dh, &qrows) || !checked_mul(batch, capacity, &pos_elems) ||
      elements > (INT64_MAX / 16) || cand > (INT64_MAX / 16)) {
    return fail(KVC_ERR_ELEMENT_COUNT_OVERFLOW,
                "storage of %d sequences x %d heads x %d rows x %d features is too large to index", batch,
                H, capacity, dh);
  }
  kvc_cache* c = new (std::nothrow) kvc_cache;
  if (!c) return fail(KVC_ERR_ALLOCATION_FAILED, "host allocation failed");
  c->batch = batch;
  c->heads = H;
  c->kv_heads = HK;
  c->window = W;
  c->head_width = dh;
  c->model_width = p->model_width;
  c->capacity = capacity;
  c->max_chunk_rows = max_chunk_rows;
  c->dtype = p->dtype;
  c->params_id = p->id;
  for (int k = 0; k < 4; ++k) c->revision[k] = p->revision[k];
  c->rope_feature_width = layer->rope_feature_width();
  c->rope_max_positions = layer->rope_max_positions;
  std::memcpy(&c->rope_base_bits, &layer->rope_base, 8);
  c->rope_base = layer->rope_base;
  c->pos_mode = layer->pos_mode;
  c->len.assign(batch, 0);
  c->next_pos.assign(batch, 0);
  c->held.assign(batch, 0);
  c->session = shared_err != nullptr;
  if (paged) {
    c->paged = true;
    c->block_rows = block_rows;
    while ((1 << c->block_lg) < block_rows) ++c->block_lg;
    c->table_width = capacity / block_rows;
    c->pool_blocks = pool_blocks;
    c->table.assign(size_t(batch) * c->table_width, -1);
    c->refcount.assign(pool_blocks, 0);
    for (int blk = pool_blocks - 1; blk >= 0; --blk) c->free_blocks.push_back(blk);
  }
  int rc = dev_current_device(&c->device);
  if (!rc) rc = dev_compute_units(c->device, &c->compute_units);
  if (rc) {
    free_cache(c);
    return device_fail(rc, "hipGetDevice");
  }

  const size_t es = elem_size(p->dtype), as = acc_size(p->dtype);
  // rows one decode query can read (a window, plus its start's misalignment)
  const int span_rows = W > 0 ? std::min(capacity, W) + kDecodeTileRows : capacity;
  const int max_tiles = (span_rows + kDecodeTileRows - 1) / kDecodeTileRows;
  auto round16 = [](size_t b) { return (b + 15) & ~size_t(15); };
  DevState& s = c->ds;
  s.dtype = p->dtype;
  s.batch = batch;
  s.heads = H;
  s.kv_heads = HK;
  s.head_width = dh;
  s.model_width = p->model_width;
  s.kv_width = p->kv_width;
  s.capacity = capacity;
  s.max_chunk_rows = max_chunk_rows;
  s.rope = layer->pos_mode == KVC_POS_ROPE;
  s.max_positions = layer->rope_max_positions;
  s.scale = 1.0 / std::sqrt(double(dh));
  s.wq = p->w[0];
  s.wk = p->w[1];
  s.wv = p->w[2];
  s.wo = p->w[3];
  s.max_tiles = max_tiles;
  s.tile_rows = kDecodeTileRows;
  s.stream = hip_stream;
  s.window = W;
  s.ring = W > 0;
  s.span_rows = span_rows;
  s.paged = paged;
  s.block_rows_log2 = c->block_lg;
  s.table_width = c->table_width;
  c->storage_bytes = int64_t(round16(size_t(elements) * es));
  struct Alloc {
    void** p;
    size_t bytes;
  } allocs[] = {
      {&s.keys, size_t(c->storage_bytes)},
      {&s.values, size_t(c->storage_bytes)},
      {reinterpret_cast<void**>(&s.len), round16(sizeof(int32_t) * batch)},
      {reinterpret_cast<void**>(&s.next_pos), round16(sizeof(int32_t) * batch)},
      {reinterpret_cast<void**>(&s.positions), round16(sizeof(int32_t) * size_t(pos_elems))},
      {reinterpret_cast<void**>(&s.rows), round16(sizeof(int32_t) * batch)},
      {reinterpret_cast<void**>(&s.held), W > 0 ? round16(sizeof(int32_t) * batch) : 0},
      {&s.cand_k, round16(size_t(cand) * es)},
      {&s.cand_v, round16(size_t(cand) * es)},
      {&s.q, round16(size_t(qrows) * as)},
      {&s.partials, round16(size_t(batch) * H * max_tiles * (dh + 2) * as)},
      // the role-split chunk attention's recompute flags, one per (work item, head)
      {reinterpret_cast<void**>(&s.redo),
       p->dtype == KVC_BF16 && dh == 128 && W == 0
           ? round16(sizeof(int32_t) * size_t(batch) * ((max_chunk_rows + kChunkQueryTile - 1) / kChunkQueryTile) * H)
           : 0},
      {reinterpret_cast<void**>(&s.err), shared_err ? 0 : round16(sizeof(ErrWords))},
      {&s.merged, p->w[3] ? round16(size_t(qrows) * as) : 0},  // [B, max_chunk_rows, D]
      // split-K partial sums of the bf16 decode projection (one 32-row tile)
      {reinterpret_cast<void**>(&s.proj_partials),
       p->dtype == KVC_BF16 && batch <= 32 && (p->model_width == 2048 || p->model_width == 4096 ||
                                               p->model_width == 8192)
           ? round16(sizeof(float) * kSkinnySplitMax * 64 * size_t(p->model_width + 2 * p->kv_width))
           : 0},
      {reinterpret_cast<void**>(const_cast<int32_t**>(&s.block_table)),
       paged ? round16(sizeof(int32_t) * c->table.size()) : 0},
  };
  for (auto& a : allocs) {
    if (a.bytes == 0) continue;
    rc = dev_malloc(a.p, a.bytes);
    if (rc) {
      *a.p = nullptr;
      free_cache(c);
      g_last.expected = int64_t(a.bytes);
      return fail(KVC_ERR_ALLOCATION_FAILED, "cannot allocate %zu bytes of KV cache storage", a.bytes);
    }
  }
  if (shared_err) {
    s.err = shared_err;
    s.gate = gate;
    s.gate_count = gate_count;
  } else {
    s.gate = s.err;
    s.gate_count = 1;
  }
  rc = dev_host_malloc(reinterpret_cast<void**>(&c->err_host), sizeof(ErrWords));
  if (rc) {
    c->err_host = nullptr;
    free_cache(c);
    return fail(KVC_ERR_ALLOCATION_FAILED, "cannot allocate pinned host memory");
  }
  // Zero-filled storage (Chapter 37: zeroed backing buffers), zero lengths;
  // an empty block table.
  for (auto& a : allocs) {
    if (*a.p == s.err || a.bytes == 0) continue;
    if (*a.p == s.block_table) {
      rc = dev_copy_h2d_sync(*a.p, c->table.data(), sizeof(int32_t) * c->table.size(), s.stream);
      if (rc) {
        free_cache(c);
        return device_fail(rc, "block table init");
      }
      continue;
    }
    rc = dev_zero(*a.p, a.bytes, s.stream);
    if (rc) {
      free_cache(c);
      return device_fail(rc, "zero fill");
    }
  }
  rc = dev_clear_err(s.err, s.stream);
  if (rc) {
    free_cache(c);
    return device_fail(rc, "error word init");
  }
  // Rotary table: cos/sin of p * base^(-2i/d_h), evaluated in double on the host.
  if (s.rope) {
    const int half = dh / 2;
    const size_t n = size_t(layer->rope_max_positions) * half;
    std::vector<double> cd(n), sd(n);
    for (int pos = 0; pos < layer->rope_max_positions; ++pos) {
      for (int i = 0; i < half; ++i) {
        const double inv = std::pow(layer->rope_base, -2.0 * double(i) / double(dh));
        const double ang = double(pos) * inv;
        cd[size_t(pos) * half + i] = std::cos(ang);
        sd[size_t(pos) * half + i] = std::sin(ang);
      }
    }
    const size_t bytes = n * as;
    rc = dev_malloc(&s.rope_cos, round16(bytes));
    if (rc == 0) rc = dev_malloc(&s.rope_sin, round16(bytes));
    if (rc) {
      free_cache(c);
      return fail(KVC_ERR_ALLOCATION_FAILED, "cannot allocate the rotary table");
    }
    if (as == 8) {
      rc = dev_copy_h2d_sync(s.rope_cos, cd.data(), bytes, s.stream);
      if (rc == 0) rc = dev_copy_h2d_sync(s.rope_sin, sd.data(), bytes, s.stream);
    } else {
      std::vector<float> cf(cd.begin(), cd.end()), sf(sd.begin(), sd.end());
      rc = dev_copy_h2d_sync(s.rope_cos, cf.data(), bytes, s.stream);
      if (rc == 0) rc = dev_copy_h2d_sync(s.rope_sin, sf.data(), bytes, s.stream);
    }
    if (rc) {
      free_cache(c);
      return device_fail(rc, "rotary table upload");
    }
  }
  rc = dev_sync(s.stream);
  if (rc) {
    free_cache(c);
    return device_fail(rc, "stream synchronisation");
  }
  *out = c;
  return KVC_OK;
}

void free_session(kvc_session* S) {
  if (!S) return;
  if (!S->caches.empty()) (void)dev_sync(S->caches[0]->ds.stream);
  for (kvc_cache* c : S->caches) free_cache(c);
  dev_free(S->gate);
  dev_free(S->h);
  dev_free(S->a);
  dev_free(S->x);
  delete S;
}

// Reads and clears every layer's failure words after the stream is idle; the
// first failing layer (in layer order) is reported, with detail.layer.
kvc_status collect_session_error(kvc_session* S) {
  kvc_status first = KVC_OK;
  kvc_error_detail saved{};
  for (size_t l = 0; l < S->caches.size(); ++l) {
    const kvc_status st = collect_device_error(S->caches[l], 0);
    if (st == KVC_ERR_DEVICE) return st;
    if (st != KVC_OK && first == KVC_OK) {
      first = st;
      g_last.layer = int32_t(l);
      saved = g_last;
    }
  }
  if (first != KVC_OK) g_last = saved;
  return first;
}

kvc_status check_deferred_session(kvc_session* S) {
  if (!S->pending_async) return KVC_OK;
  const int rc = dev_sync(S->caches[0]->ds.stream);
  if (rc) return device_fail(rc, "stream synchronisation");
  S->pending_async = false;
  for (kvc_cache* c : S->caches) c->pending_async = false;
  const kvc_status st = collect_session_error(S);
  if (st == KVC_ERR_DEVICE) return st;
  if (st != KVC_OK) {
    const kvc_error_detail saved = g_last;
    for (kvc_cache* c : S->caches) {
      const kvc_status rs = resync_lengths(c);
      if (rs != KVC_OK) return rs;
    }
    g_last = saved;
    g_last.actual = st;
    return fail(KVC_ERR_DEFERRED, "an earlier asynchronous session call failed: %s (%s)", kvc_status_name(st),
                std::string(saved.message).c_str());
  }
  return KVC_OK;
}

// One session call: every layer computes (embedding, then per layer the
// attention and the tanh residual), then every layer commits; the commits are
// suppressed on the device if any layer's failure word is set.
kvc_status session_call(kvc_session* S, const int32_t* tokens, int n_max, const int32_t* n_rows, void* out,
                        int32_t flags, kvc_work* work, bool decode) {
  const int L = int(S->layers.size());
  if (!(flags & KVC_ASYNC)) {
    kvc_status d = check_deferred_session(S);
    if (d != KVC_OK) return d;
  }
  for (int l = 0; l < L; ++l) {
    kvc_status st = check_binding(S->layers[l], S->caches[l]);
    if (st != KVC_OK) {
      g_last.layer = l;
      return st;
    }
  }
  for (int l = 0; l < L; ++l) {
    const kvc_cache* c = S->caches[l];
    for (int b = 0; b < c->batch; ++b) {
      const int n = n_rows ? n_rows[b] : n_max;
      if (!c->window && int64_t(c->len[b]) + n > c->capacity) {
        g_last.layer = l;
        g_last.sequence = b;
        return fail_ea(KVC_ERR_FULL, c->capacity, int64_t(c->len[b]) + n,
                       "layer %d: sequence %d holds %d of %d rows and cannot take %d more", l, b, c->len[b],
                       c->capacity, n);
      }
      if (c->ds.rope && n > 0 && int64_t(c->next_pos[b]) + n > c->rope_max_positions) {
        g_last.layer = l;
        g_last.sequence = b;
        return fail_ea(KVC_ERR_ROTARY_POSITION, c->rope_max_positions, int64_t(c->next_pos[b]) + n - 1,
                       "position %lld of sequence %d reaches the rotary position capacity %d of layer %d",
                       (long long)c->next_pos[b] + n - 1, b, c->rope_max_positions, l);
      }
    }
  }
  kvc_work w{};
  w.position_min = INT32_MAX;
  w.position_max = -1;
  int64_t total = 0;
  for (int l = 0; l < L; ++l) {
    const kvc_cache* c = S->caches[l];
    for (int b = 0; b < c->batch; ++b) {
      const int n = n_rows ? n_rows[b] : n_max;
      w.full_prefix_rows_per_projection += c->len[b] + n;
      w.incremental_rows_per_projection += n;
      w.reused_key_value_rows += c->len[b];
      total += n;
      if (n > 0) {
        w.position_min = std::min(w.position_min, c->next_pos[b]);
        w.position_max = std::max(w.position_max, c->next_pos[b] + n - 1);
      }
    }
  }
  if (total == 0) {
    w.position_min = w.position_max = -1;
    if (work) *work = w;
    return KVC_OK;
  }
  if (!dev_has_kernels()) return fail(KVC_ERR_DEVICE, "library built without device kernels");
  const int per_seq = n_rows != nullptr;
  DevState& s0 = S->caches[0]->ds;
  int rc = 0;
  if (per_seq) {
    rc = dev_set_rows(s0, n_rows);
    if (rc) return device_fail(rc, "chunk row upload");
  }
  rc = dev_embed(s0, tokens, S->embedding, S->vocab, S->sinusoidal, n_max, per_seq, S->h, S->x);
  if (rc) return device_fail(rc, "embedding launch");
  const void* xin = S->x ? S->x : S->h;
  for (int l = 0; l < L; ++l) {
    kvc_cache* c = S->caches[l];
    if (decode) choose_decode_tiles(c);
    kvc_status st = compute_stages(c, xin, n_max, n_rows, S->a, decode);
    if (st != KVC_OK) return st;
    const bool last = l == L - 1;
    rc = dev_residual(c->ds, S->h, S->a, last ? out : S->h, last ? nullptr : S->x, n_max, per_seq);
    if (rc) return device_fail(rc, "residual launch");
  }
  for (int l = 0; l < L; ++l) {
    kvc_status st = commit_stage(S->caches[l], n_max, n_rows);
    if (st != KVC_OK) return st;
  }
  if (flags & KVC_ASYNC) {
    S->pending_async = true;
    for (kvc_cache* c : S->caches) advance_mirror(c, n_max, n_rows);
    if (work) *work = w;
    return KVC_OK;
  }
  rc = dev_sync(s0.stream);
  if (rc) return device_fail(rc, "stream synchronisation");
  kvc_status st = collect_session_error(S);
  if (st != KVC_OK) return st;
  for (kvc_cache* c : S->caches) advance_mirror(c, n_max, n_rows);
  if (work) *work = w;
  return KVC_OK;
}

}  // namespace

extern "C" {

const char* kvc_status_name(kvc_status s) {
  switch (s) {
#define N(x) \
  case x: return #x;
    N(KVC_OK)
    N(KVC_ERR_ZERO_BATCH)
    N(KVC_ERR_ZERO_CAPACITY)
    N(KVC_ERR_CAPACITY_EXCEEDS_POSITIONS)
    N(KVC_ERR_ELEMENT_COUNT_OVERFLOW)
    N(KVC_ERR_ALLOCATION_FAILED)
    N(KVC_ERR_INPUT_RANK)
    N(KVC_ERR_SINGLE_TOKEN_REQUIRED)
    N(KVC_ERR_INPUT_BATCH_MISMATCH)
    N(KVC_ERR_INPUT_WIDTH_MISMATCH)
    N(KVC_ERR_CACHE_MODEL_WIDTH_MISMATCH)
    N(KVC_ERR_CACHE_HEAD_COUNT_MISMATCH)
    N(KVC_ERR_CACHE_HEAD_WIDTH_MISMATCH)
    N(KVC_ERR_CACHE_LAYER_MISMATCH)
    N(KVC_ERR_CACHE_LAYER_REVISION_MISMATCH)
    N(KVC_ERR_CACHE_ROPE_MISMATCH)
    N(KVC_ERR_FULL)
    N(KVC_ERR_OUT_OF_BLOCKS)
    N(KVC_ERR_CACHE_WINDOW_MISMATCH)
    N(KVC_ERR_NONFINITE_KEY)
    N(KVC_ERR_NONFINITE_VALUE)
    N(KVC_ERR_NONFINITE_QUERY)
    N(KVC_ERR_ROTARY_POSITION)
    N(KVC_ERR_NONFINITE_OUTPUT)
    N(KVC_ERR_TOKEN_RANGE)
    N(KVC_ERR_BAD_CUT)
    N(KVC_ERR_EMPTY_QUERY)
    N(KVC_ERR_CHUNK_ROWS)
    N(KVC_ERR_NULL_ARGUMENT)
    N(KVC_ERR_DTYPE_UNSUPPORTED)
    N(KVC_ERR_SHAPE_UNSUPPORTED)
    N(KVC_ERR_BAD_ARGUMENT)
    N(KVC_ERR_SCRATCH_EXCEEDED)
    N(KVC_ERR_DEVICE)
    N(KVC_ERR_DEFERRED)
    N(KVC_ERR_INTERNAL)
#undef N
  }
  return "KVC_ERR_UNKNOWN";
}

const kvc_error_detail* kvc_last_error(void) { return &g_last; }

kvc_status kvc_params_create(int32_t model_width, kvc_dtype dtype, const void* w_q, const void* w_k,
                             const void* w_v, const void* w_o, kvc_params** out) {
  return kvc_params_create_grouped(model_width, model_width, dtype, w_q, w_k, w_v, w_o, out);
}

kvc_status kvc_params_create_grouped(int32_t model_width, int32_t kv_width, kvc_dtype dtype, const void* w_q,
                                     const void* w_k, const void* w_v, const void* w_o, kvc_params** out) {
  reset_detail();
  if (!out || !w_q || !w_k || !w_v) return fail(KVC_ERR_NULL_ARGUMENT, "null argument to kvc_params_create");
  *out = nullptr;
  if (model_width <= 0) return fail(KVC_ERR_BAD_ARGUMENT, "model width must be positive, got %d", model_width);
  if (kv_width <= 0 || model_width % kv_width != 0)
    return fail_ea(KVC_ERR_BAD_ARGUMENT, model_width, kv_width,
                   "key/value width %d must be positive and divide the model width %d", kv_width, model_width);
  if (dtype != KVC_F64 && dtype != KVC_F32 && dtype != KVC_BF16)
    return fail(KVC_ERR_DTYPE_UNSUPPORTED, "unsupported weight type %d", int(dtype));
  kvc_params* p = new (std::nothrow) kvc_params;
  if (!p) return fail(KVC_ERR_ALLOCATION_FAILED, "host allocation failed");
  p->model_width = model_width;
  p->kv_width = kv_width;
  p->dtype = dtype;
  p->w[0] = w_q;
  p->w[1] = w_k;
  p->w[2] = w_v;
  p->w[3] = w_o;
  p->nweights = w_o ? 4 : 3;
  p->id = g_next_params_id.fetch_add(1);
  for (int k = 0; k < 4; ++k) p->revision[k] = 0;
  *out = p;
  return KVC_OK;
}

kvc_status kvc_params_mark_updated(kvc_params* params, int32_t which) {
  reset_detail();
  if (!params) return fail(KVC_ERR_NULL_ARGUMENT, "null parameter set");
  if (which < -1 || which >= params->nweights)
    return fail(KVC_ERR_BAD_ARGUMENT, "weight index %d out of range for %d weights", which, params->nweights);
  for (int k = 0; k < params->nweights; ++k)
    if (which == -1 || which == k) params->revision[k]++;
  return KVC_OK;
}

void kvc_params_destroy(kvc_params* params) { delete params; }

kvc_status kvc_layer_create(const kvc_params* params, int32_t heads, kvc_pos_mode pos_mode, double rope_base,
                            int32_t rope_max_positions, kvc_layer** out) {
  return kvc_layer_create_windowed(params, heads, pos_mode, rope_base, rope_max_positions, 0, out);
}

kvc_status kvc_layer_create_windowed(const kvc_params* params, int32_t heads, kvc_pos_mode pos_mode,
                                     double rope_base, int32_t rope_max_positions, int32_t window, kvc_layer** out) {
  reset_detail();
  if (!params || !out) return fail(KVC_ERR_NULL_ARGUMENT, "null argument to kvc_layer_create");
  *out = nullptr;
  if (heads <= 0 || params->model_width % heads != 0)
    return fail(KVC_ERR_BAD_ARGUMENT, "head count %d must divide model width %d", heads, params->model_width);
  if (pos_mode != KVC_POS_ROPE && pos_mode != KVC_POS_NONE)
    return fail(KVC_ERR_BAD_ARGUMENT, "unknown position mode %d", int(pos_mode));
  if (!(rope_base > 0.0) || !std::isfinite(rope_base) || rope_max_positions <= 0)
    return fail(KVC_ERR_BAD_ARGUMENT, "rotary base must be positive and finite and max positions positive");
  const int dh = params->model_width / heads;
  if (dh < 2 || !is_pow2(dh) || dh > max_head_width(params->dtype))
    return fail(KVC_ERR_SHAPE_UNSUPPORTED, "head width %d must be a power of two in [2, %d] for this type", dh,
                max_head_width(params->dtype));
  if (window < 0) return fail_ea(KVC_ERR_BAD_ARGUMENT, 0, window, "sliding window %d must be >= 0", window);
  if (params->kv_width % dh != 0 || heads % (params->kv_width / dh) != 0)
    return fail_ea(KVC_ERR_BAD_ARGUMENT, dh, params->kv_width,
                   "key/value width %d must be a whole number of %d-wide heads that divides the %d query heads",
                   params->kv_width, dh, heads);
  kvc_layer* l = new (std::nothrow) kvc_layer;
  if (!l) return fail(KVC_ERR_ALLOCATION_FAILED, "host allocation failed");
  l->params = params;
  l->heads = heads;
  l->kv_heads = params->kv_width / dh;
  l->window = window;
  l->head_width = dh;
  l->pos_mode = pos_mode;
  l->rope_base = rope_base;
  l->rope_max_positions = rope_max_positions;
  *out = l;
  return KVC_OK;
}

void kvc_layer_destroy(kvc_layer* layer) { delete layer; }

kvc_status kvc_cache_create(const kvc_layer* layer, int32_t batch, int32_t capacity, int32_t max_chunk_rows,
                            void* hip_stream, kvc_cache** out) {
  reset_detail();
  if (!layer || !out) return fail(KVC_ERR_NULL_ARGUMENT, "null argument to kvc_cache_create");
  return create_cache(layer, batch, capacity, max_chunk_rows, hip_stream, nullptr, nullptr, 0, out);
}

kvc_status kvc_cache_create_paged(const kvc_layer* layer, int32_t batch, int32_t capacity, int32_t max_chunk_rows,
                                  int32_t block_rows, int32_t pool_blocks, void* hip_stream, kvc_cache** out) {
  reset_detail();
  if (!layer || !out) return fail(KVC_ERR_NULL_ARGUMENT, "null argument to kvc_cache_create_paged");
  if (block_rows == 0) return fail(KVC_ERR_BAD_ARGUMENT, "block_rows must be nonzero");
  return create_cache(layer, batch, capacity, max_chunk_rows, hip_stream, nullptr, nullptr, 0, out, block_rows,
                      pool_blocks);
}

void kvc_cache_destroy(kvc_cache* cache) {
  if (!cache || cache->session) return;  // a session's layer caches go with the session
  (void)dev_sync(cache->ds.stream);
  free_cache(cache);
}

kvc_status kvc_append_and_attend(const kvc_layer* layer, kvc_cache* cache, const void* x, int32_t rank,
                                 const int64_t* shape, void* out, int32_t flags, kvc_work* work) {
  reset_detail();
  kvc_work w{};
  kvc_status st = decode_checks("kvc_append_and_attend", layer, cache, x, rank, shape, out, flags, &w);
  if (st != KVC_OK) return st;
  choose_decode_tiles(cache);
  cache->newest_q_valid = false;
  st = run_call(cache, x, 1, nullptr, out, flags, true);
  if (st == KVC_OK) cache->newest_q_valid = true;
  if (st == KVC_OK && work) *work = w;
  return st;
}

kvc_status kvc_append_and_attend_static(const kvc_layer* layer, kvc_cache* cache, const void* x, int32_t rank,
                                        const int64_t* shape, void* out, int32_t flags, kvc_work* work) {
  reset_detail();
  kvc_work w{};
  kvc_status st = decode_checks("kvc_append_and_attend_static", layer, cache, x, rank, shape, out, flags, &w);
  if (st != KVC_OK) return st;
  cache->newest_q_valid = false;  // this call's queries live in the static scratch
  void* base = nullptr;
  size_t cap = 0;
  const int rc = dev_static_scratch(cache->device, &base, &cap);
  if (rc) return device_fail(rc, "looking up the static scratch");
  const ScratchLayout L = decode_scratch_layout(cache);
  if (L.total > cap)
    return fail_ea(KVC_ERR_SCRATCH_EXCEEDED, int64_t(cap), int64_t(L.total),
                   "a decode step of this cache needs %zu bytes of scratch, the static scratch holds %zu", L.total,
                   cap);
  // the call's scratch pointers point into the static array for its duration
  DevState& s = cache->ds;
  void* const own[6] = {s.q, s.cand_k, s.cand_v, s.partials, s.proj_partials, s.merged};
  char* b = static_cast<char*>(base);
  s.q = b + L.q;
  s.cand_k = b + L.cand_k;
  s.cand_v = b + L.cand_v;
  s.partials = b + L.partials;
  s.proj_partials = s.proj_partials ? reinterpret_cast<float*>(b + L.proj) : nullptr;
  s.merged = s.merged ? b + L.merged : nullptr;
  choose_decode_tiles(cache);
  st = run_call(cache, x, 1, nullptr, out, flags, true);
  s.q = own[0];
  s.cand_k = own[1];
  s.cand_v = own[2];
  s.partials = own[3];
  s.proj_partials = static_cast<float*>(own[4]);
  s.merged = own[5];
  if (st == KVC_OK && work) *work = w;
  return st;
}

kvc_status kvc_newest_weights(kvc_cache* cache, int32_t seq, void* weights_out, int64_t rows_capacity,
                              int32_t* rows_out) {
  reset_detail();
  if (!cache || !rows_out) return fail(KVC_ERR_NULL_ARGUMENT, "null argument to kvc_newest_weights");
  if (seq < 0 || seq >= cache->batch)
    return fail_ea(KVC_ERR_BAD_ARGUMENT, cache->batch, seq, "sequence %d out of range", seq);
  kvc_status st = check_deferred(cache);
  if (st != KVC_OK) return st;
  if (!cache->newest_q_valid)
    return fail(KVC_ERR_BAD_ARGUMENT,
                "the cache has moved since its last kvc_append_and_attend: no newest query to read out");
  const int len = cache->len[seq];
  const int r0 = cache->window ? std::max(0, len - cache->window) : 0;
  const int rows = len - r0;
  *rows_out = rows;
  if (!weights_out) return KVC_OK;
  if (rows_capacity < rows)
    return fail_ea(KVC_ERR_BAD_ARGUMENT, rows, rows_capacity, "the weight buffer holds %lld of %d rows per head",
                   (long long)rows_capacity, rows);
  if (!dev_has_kernels()) return fail(KVC_ERR_DEVICE, "library built without device kernels");
  int rc = dev_newest_weights(cache->ds, seq, r0, rows, weights_out);
  if (rc == 0) rc = dev_sync(cache->ds.stream);
  if (rc) return device_fail(rc, "weight readout");
  return KVC_OK;
}

kvc_status kvc_continue_chunk(const kvc_layer* layer, kvc_cache* cache, const void* x, int32_t n_max,
                              const int32_t* n_rows, void* out, int32_t flags, kvc_work* work) {
  reset_detail();
  if (!layer || !cache || !x || !out) return fail(KVC_ERR_NULL_ARGUMENT, "null argument to kvc_continue_chunk");
  if (cache->session) return reject_session_cache("kvc_continue_chunk");
  if (flags & ~int32_t(KVC_ASYNC)) return fail(KVC_ERR_BAD_ARGUMENT, "unknown flags %d", flags);
  if (!(flags & KVC_ASYNC)) {
    kvc_status d = check_deferred(cache);
    if (d != KVC_OK) return d;
  }
  if (n_max < 1 || n_max > cache->max_chunk_rows)
    return fail_ea(KVC_ERR_CHUNK_ROWS, cache->max_chunk_rows, n_max, "chunk rows %d outside [1, %d]", n_max,
                   cache->max_chunk_rows);
  if (n_rows) {
    for (int b = 0; b < cache->batch; ++b) {
      if (n_rows[b] < 0 || n_rows[b] > n_max) {
        g_last.sequence = b;
        return fail_ea(KVC_ERR_CHUNK_ROWS, n_max, n_rows[b], "sequence %d has %d chunk rows, outside [0, %d]", b,
                       n_rows[b], n_max);
      }
    }
  }
  kvc_status st = check_binding(layer, cache);
  if (st != KVC_OK) return st;
  for (int b = 0; b < cache->batch; ++b) {
    const int n = n_rows ? n_rows[b] : n_max;
    if (!cache->window && int64_t(cache->len[b]) + n > cache->capacity) {
      g_last.sequence = b;
      return fail_ea(KVC_ERR_FULL, cache->capacity, int64_t(cache->len[b]) + n,
                     "sequence %d holds %d of %d rows and cannot take %d more", b, cache->len[b], cache->capacity, n);
    }
  }
  if (cache->ds.rope) {
    for (int b = 0; b < cache->batch; ++b) {
      const int n = n_rows ? n_rows[b] : n_max;
      if (n > 0 && int64_t(cache->next_pos[b]) + n > cache->rope_max_positions) {
        g_last.sequence = b;
        return fail_ea(KVC_ERR_ROTARY_POSITION, cache->rope_max_positions, int64_t(cache->next_pos[b]) + n - 1,
                       "position %lld of sequence %d reaches the rotary position capacity %d",
                       (long long)cache->next_pos[b] + n - 1, b, cache->rope_max_positions);
      }
    }
  }
  kvc_work w{};
  w.position_min = INT32_MAX;
  w.position_max = -1;
  int64_t total = 0;
  for (int b = 0; b < cache->batch; ++b) {
    const int n = n_rows ? n_rows[b] : n_max;
    w.full_prefix_rows_per_projection += cache->len[b] + n;
    w.incremental_rows_per_projection += n;
    w.reused_key_value_rows += cache->len[b];
    total += n;
    if (n > 0) {
      w.position_min = std::min(w.position_min, cache->next_pos[b]);
      w.position_max = std::max(w.position_max, cache->next_pos[b] + n - 1);
    }
  }
  if (total == 0) {
    w.position_min = w.position_max = -1;
    if (work) *work = w;
    return KVC_OK;
  }
  if (!dev_has_kernels()) return fail(KVC_ERR_DEVICE, "library built without device kernels");
  cache->newest_q_valid = false;
  st = run_call(cache, x, n_max, n_rows, out, flags, false);
  if (st == KVC_OK && work) *work = w;
  return st;
}

kvc_status kvc_truncate(kvc_cache* cache, const int32_t* cut, int32_t flags) {
  reset_detail();
  if (!cache || !cut) return fail(KVC_ERR_NULL_ARGUMENT, "null argument to kvc_truncate");
  if (cache->session) return reject_session_cache("kvc_truncate");
  if (flags & ~int32_t(KVC_TRUNCATE_KEEP_STALE_POSITION)) return fail(KVC_ERR_BAD_ARGUMENT, "unknown flags %d", flags);
  for (int b = 0; b < cache->batch; ++b) {
    if (cut[b] < 0 || cut[b] > cache->len[b]) {
      g_last.sequence = b;
      return fail_ea(KVC_ERR_BAD_CUT, cache->len[b], cut[b], "cut %d of sequence %d is outside [0, %d]", cut[b], b,
                     cache->len[b]);
    }
    if (!window_continuable(cache, b, cut[b])) {
      g_last.sequence = b;
      return fail_ea(KVC_ERR_BAD_CUT, window_min_cut(cache, b), cut[b],
                     "cut %d of sequence %d needs rows the window cache no longer holds (continue from 0 or from "
                     "%d .. %d)",
                     cut[b], b, window_min_cut(cache, b), cache->len[b]);
    }
  }
  const bool stale = flags & KVC_TRUNCATE_KEEP_STALE_POSITION;
  cache->newest_q_valid = false;
  int rc = dev_set_lengths(cache->ds, cut, stale ? 1 : 0);
  if (rc) return device_fail(rc, "length update");
  for (int b = 0; b < cache->batch; ++b) {
    cache->len[b] = cut[b];
    if (!stale) cache->next_pos[b] = cut[b];
    if (cut[b] < cache->held[b]) cache->held[b] = cut[b];
  }
  if (cache->paged) {
    // blocks wholly past the cut go back to the pool (a block other
    // sequences still name stays with them)
    std::vector<int32_t> changed;
    for (int b = 0; b < cache->batch; ++b) release_tail(cache, b, blocks_for(cache, cut[b]), changed);
    return upload_table(cache, changed);
  }
  return KVC_OK;
}

kvc_status kvc_reset(kvc_cache* cache) {
  reset_detail();
  if (!cache) return fail(KVC_ERR_NULL_ARGUMENT, "null cache");
  if (cache->session) return reject_session_cache("kvc_reset");
  cache->newest_q_valid = false;
  int rc = dev_set_lengths(cache->ds, nullptr, 2);
  if (rc) return device_fail(rc, "length reset");
  std::fill(cache->len.begin(), cache->len.end(), 0);
  std::fill(cache->next_pos.begin(), cache->next_pos.end(), 0);
  std::fill(cache->held.begin(), cache->held.end(), 0);
  if (cache->paged) {
    rc = dev_clear_table(cache->ds);
    if (rc) return device_fail(rc, "block table reset");
    std::fill(cache->table.begin(), cache->table.end(), -1);
    std::fill(cache->refcount.begin(), cache->refcount.end(), 0);
    cache->free_blocks.clear();
    for (int blk = cache->pool_blocks - 1; blk >= 0; --blk) cache->free_blocks.push_back(blk);
  }
  return KVC_OK;
}

kvc_status kvc_fork(kvc_cache* cache, int32_t src, int32_t dst, int32_t rows) {
  reset_detail();
  if (!cache) return fail(KVC_ERR_NULL_ARGUMENT, "null cache");
  if (cache->session) return reject_session_cache("kvc_fork");
  if (src < 0 || src >= cache->batch || dst < 0 || dst >= cache->batch || src == dst)
    return fail_ea(KVC_ERR_BAD_ARGUMENT, cache->batch, src == dst ? src : (src < 0 || src >= cache->batch ? src : dst),
                   "fork needs two different sequences in [0, %d), got %d -> %d", cache->batch, src, dst);
  if (rows < 0 || rows > cache->len[src]) {
    g_last.sequence = src;
    return fail_ea(KVC_ERR_BAD_CUT, cache->len[src], rows, "fork of %d rows outside [0, %d] of sequence %d", rows,
                   cache->len[src], src);
  }
  if (!window_continuable(cache, src, rows)) {
    g_last.sequence = src;
    return fail_ea(KVC_ERR_BAD_CUT, window_min_cut(cache, src), rows,
                   "fork of %d rows needs rows the window cache no longer holds", rows);
  }
  DevState& s = cache->ds;
  int rc = 0;
  cache->newest_q_valid = false;
  if (cache->paged) {
    // dst names src's blocks (shared, copied on a later append into them)
    const int nb = blocks_for(cache, rows);
    for (int j = 0; j < nb; ++j)
      if (cache->table[src * cache->table_width + j] < 0)
        return fail(KVC_ERR_INTERNAL, "sequence %d has no block for row %d", src, j * cache->block_rows);
    std::vector<int32_t> changed;
    release_tail(cache, dst, 0, changed);
    for (int j = 0; j < nb; ++j) {
      const int32_t blk = cache->table[src * cache->table_width + j];
      const int idx = dst * cache->table_width + j;
      cache->table[idx] = blk;
      cache->refcount[blk]++;
      if (std::find(changed.begin(), changed.end(), idx) == changed.end()) changed.push_back(idx);
    }
    kvc_status st = upload_table(cache, changed);
    if (st != KVC_OK) return st;
  } else {
    // a ring's rows sit in slots r % capacity: copy every slot
    rc = dev_copy_seq_rows(s, dst, src, cache->window ? cache->capacity : rows);
    if (rc) return device_fail(rc, "row copy");
  }
  rc = dev_copy_positions(s, dst, src, cache->window ? cache->capacity : rows);
  if (rc == 0) rc = dev_set_seq_length(s, dst, rows, rows > 0 ? src : -1);
  if (rc) return device_fail(rc, "fork bookkeeping");
  cache->len[dst] = rows;
  cache->next_pos[dst] = rows;
  cache->held[dst] = rows > 0 ? cache->held[src] : 0;
  return KVC_OK;
}

kvc_status kvc_pool_usage(kvc_cache* cache, int32_t* blocks_in_use, int32_t* blocks_free) {
  reset_detail();
  if (!cache) return fail(KVC_ERR_NULL_ARGUMENT, "null cache");
  if (!cache->paged) return fail(KVC_ERR_BAD_ARGUMENT, "the cache is not paged");
  kvc_status st = check_deferred(cache);
  if (st != KVC_OK) return st;
  if (blocks_in_use) *blocks_in_use = cache->pool_blocks - int32_t(cache->free_blocks.size());
  if (blocks_free) *blocks_free = int32_t(cache->free_blocks.size());
  return KVC_OK;
}

kvc_status kvc_sync(kvc_cache* cache) {
  reset_detail();
  if (!cache) return fail(KVC_ERR_NULL_ARGUMENT, "null cache");
  cache->pending_async = true;  // always look at the device words
  kvc_status st = check_deferred(cache);
  if (st != KVC_OK) return st;
  return resync_lengths(cache);
}

kvc_status kvc_lengths(kvc_cache* cache, int32_t* len_out, int32_t* next_position_out) {
  reset_detail();
  if (!cache) return fail(KVC_ERR_NULL_ARGUMENT, "null cache");
  kvc_status st = check_deferred(cache);
  if (st != KVC_OK) return st;
  st = resync_lengths(cache);
  if (st != KVC_OK) return st;
  if (len_out) std::memcpy(len_out, cache->len.data(), sizeof(int32_t) * cache->batch);
  if (next_position_out) std::memcpy(next_position_out, cache->next_pos.data(), sizeof(int32_t) * cache->batch);
  return KVC_OK;
}

kvc_status kvc_snapshot(kvc_cache* cache, int32_t seq, void* keys_out, void* values_out, int32_t* positions_out,
                        int64_t rows_capacity, int32_t* rows_out) {
  reset_detail();
  if (!cache) return fail(KVC_ERR_NULL_ARGUMENT, "null cache");
  if (seq < 0 || seq >= cache->batch)
    return fail_ea(KVC_ERR_BAD_ARGUMENT, cache->batch, seq, "sequence %d out of range", seq);
  kvc_status st = check_deferred(cache);
  if (st != KVC_OK) return st;
  st = resync_lengths(cache);
  if (st != KVC_OK) return st;
  const int len = cache->len[seq];
  // a window cache holds (and returns) rows held[seq] .. len - 1 only
  const int held = cache->window ? len - cache->held[seq] : len;
  if (rows_out) *rows_out = held;
  if ((keys_out || values_out || positions_out) && rows_capacity < held)
    return fail_ea(KVC_ERR_BAD_ARGUMENT, held, rows_capacity, "snapshot buffers hold %lld rows, need %d",
                   (long long)rows_capacity, held);
  const size_t es = elem_size(cache->dtype);
  const size_t row_bytes = size_t(cache->head_width) * es;
  int rc = 0;
  if (cache->window) {
    // rows len - held .. len - 1 sit in slots r % C: at most two runs
    const size_t lane_bytes = size_t(cache->capacity) * row_bytes;
    const size_t seq_off = size_t(seq) * cache->kv_heads * lane_bytes;
    int done = 0;
    while (done < held && rc == 0) {
      const int r = len - held + done;
      const int slot = r % cache->capacity;
      const int n = std::min(held - done, cache->capacity - slot);
      if (keys_out)
        rc = dev_copy_d2h_2d_sync(static_cast<char*>(keys_out) + done * row_bytes, size_t(held) * row_bytes,
                                  static_cast<char*>(cache->ds.keys) + seq_off + slot * row_bytes, lane_bytes,
                                  n * row_bytes, cache->kv_heads, cache->ds.stream);
      if (rc == 0 && values_out)
        rc = dev_copy_d2h_2d_sync(static_cast<char*>(values_out) + done * row_bytes, size_t(held) * row_bytes,
                                  static_cast<char*>(cache->ds.values) + seq_off + slot * row_bytes, lane_bytes,
                                  n * row_bytes, cache->kv_heads, cache->ds.stream);
      if (rc == 0 && positions_out)
        rc = dev_copy_d2h_sync(positions_out + done, cache->ds.positions + size_t(seq) * cache->capacity + slot,
                               sizeof(int32_t) * size_t(n), cache->ds.stream);
      done += n;
    }
    if (rc) return device_fail(rc, "snapshot copy");
    return KVC_OK;
  }
  if (cache->paged) {
    // [H, len, d_h] gathered block by block: [H, block rows, d_h] per block
    const size_t head_bytes = size_t(cache->block_rows) * row_bytes;
    for (int j = 0; j < blocks_for(cache, len) && rc == 0; ++j) {
      const int blk = cache->table[seq * cache->table_width + j];
      const int r0 = j * cache->block_rows, nr = std::min(len - r0, cache->block_rows);
      const size_t src_off = size_t(blk) * cache->kv_heads * head_bytes;
      if (keys_out)
        rc = dev_copy_d2h_2d_sync(static_cast<char*>(keys_out) + r0 * row_bytes, size_t(len) * row_bytes,
                                  static_cast<char*>(cache->ds.keys) + src_off, head_bytes, nr * row_bytes,
                                  cache->kv_heads, cache->ds.stream);
      if (rc == 0 && values_out)
        rc = dev_copy_d2h_2d_sync(static_cast<char*>(values_out) + r0 * row_bytes, size_t(len) * row_bytes,
                                  static_cast<char*>(cache->ds.values) + src_off, head_bytes, nr * row_bytes,
                                  cache->kv_heads, cache->ds.stream);
    }
    if (rc == 0 && positions_out && len > 0)
      rc = dev_copy_d2h_sync(positions_out, cache->ds.positions + size_t(seq) * cache->capacity,
                             sizeof(int32_t) * size_t(len), cache->ds.stream);
    if (rc) return device_fail(rc, "snapshot copy");
    return KVC_OK;
  }
  const size_t lane_bytes = size_t(cache->capacity) * row_bytes;
  const size_t seq_off = size_t(seq) * cache->kv_heads * lane_bytes;
  // [H, len, d_h] out of [H, C, d_h]: one strided copy per buffer.
  if (keys_out)
    rc = dev_copy_d2h_2d_sync(keys_out, size_t(len) * row_bytes, static_cast<char*>(cache->ds.keys) + seq_off,
                              lane_bytes, size_t(len) * row_bytes, cache->kv_heads, cache->ds.stream);
  if (rc == 0 && values_out)
    rc = dev_copy_d2h_2d_sync(values_out, size_t(len) * row_bytes, static_cast<char*>(cache->ds.values) + seq_off,
                              lane_bytes, size_t(len) * row_bytes, cache->kv_heads, cache->ds.stream);
  if (rc == 0 && positions_out && len > 0)
    rc = dev_copy_d2h_sync(positions_out, cache->ds.positions + size_t(seq) * cache->capacity,
                           sizeof(int32_t) * size_t(len), cache->ds.stream);
  if (rc) return device_fail(rc, "snapshot copy");
  return KVC_OK;
}

kvc_status kvc_lcp_cut(const int32_t* cached, int64_t n_cached, const int32_t* query, int64_t n_query,
                       int64_t* cut_out) {
  reset_detail();
  if (!cut_out || (n_cached > 0 && !cached) || (n_query > 0 && !query))
    return fail(KVC_ERR_NULL_ARGUMENT, "null argument to kvc_lcp_cut");
  if (n_cached < 0) return fail(KVC_ERR_BAD_ARGUMENT, "negative cached length");
  if (n_query <= 0) return fail(KVC_ERR_EMPTY_QUERY, "query token IDs must be non-empty");
  int64_t n = 0;
  const int64_t lim = std::min(n_cached, n_query);
  while (n < lim && cached[n] == query[n]) ++n;
  *cut_out = std::min(n, n_query - 1);
  return KVC_OK;
}

kvc_status kvc_reuse_cut(kvc_cache* cache, int32_t seq, int64_t lcp_cut, int64_t* cut_out) {
  reset_detail();
  if (!cache || !cut_out) return fail(KVC_ERR_NULL_ARGUMENT, "null argument to kvc_reuse_cut");
  if (seq < 0 || seq >= cache->batch)
    return fail_ea(KVC_ERR_BAD_ARGUMENT, cache->batch, seq, "sequence %d out of range", seq);
  kvc_status st = check_deferred(cache);
  if (st != KVC_OK) return st;
  if (lcp_cut < 0 || lcp_cut > cache->len[seq])
    return fail_ea(KVC_ERR_BAD_CUT, cache->len[seq], lcp_cut, "common prefix %lld outside [0, %d]",
                   (long long)lcp_cut, cache->len[seq]);
  *cut_out = window_continuable(cache, seq, lcp_cut) ? lcp_cut : 0;
  return KVC_OK;
}

kvc_status kvc_cache_describe(const kvc_cache* cache, kvc_cache_desc* out) {
  reset_detail();
  if (!cache || !out) return fail(KVC_ERR_NULL_ARGUMENT, "null argument to kvc_cache_describe");
  out->batch = cache->batch;
  out->heads = cache->heads;
  out->kv_heads = cache->kv_heads;
  out->head_width = cache->head_width;
  out->model_width = cache->model_width;
  out->capacity = cache->capacity;
  out->max_chunk_rows = cache->max_chunk_rows;
  out->kv_dtype = cache->dtype;
  out->pos_mode = cache->pos_mode;
  out->rope_max_positions = cache->rope_max_positions;
  out->device = cache->device;
  out->rope_base = cache->rope_base;
  out->block_rows = cache->block_rows;
  out->pool_blocks = cache->pool_blocks;
  out->window = cache->window;
  return KVC_OK;
}

kvc_status kvc_storage_pointers(const kvc_cache* cache, const void** keys, const void** values, int64_t* bytes_each) {
  reset_detail();
  if (!cache) return fail(KVC_ERR_NULL_ARGUMENT, "null cache");
  if (keys) *keys = cache->ds.keys;
  if (values) *values = cache->ds.values;
  if (bytes_each) *bytes_each = cache->storage_bytes;
  return KVC_OK;
}

kvc_status kvc_copy_storage(kvc_cache* cache, void* keys_out, void* values_out) {
  reset_detail();
  if (!cache) return fail(KVC_ERR_NULL_ARGUMENT, "null cache");
  int rc = dev_sync(cache->ds.stream);
  if (rc == 0 && keys_out) rc = dev_copy_d2h_sync(keys_out, cache->ds.keys, size_t(cache->storage_bytes), cache->ds.stream);
  if (rc == 0 && values_out)
    rc = dev_copy_d2h_sync(values_out, cache->ds.values, size_t(cache->storage_bytes), cache->ds.stream);
  if (rc) return device_fail(rc, "storage copy");
  return KVC_OK;
}

kvc_status kvc_profile_enable(kvc_cache* cache, int32_t slots) {
  reset_detail();
  if (!cache) return fail(KVC_ERR_NULL_ARGUMENT, "null cache");
  if (slots < 0) return fail(KVC_ERR_BAD_ARGUMENT, "negative slot count");
  int rc = dev_sync(cache->ds.stream);
  if (rc) return device_fail(rc, "stream synchronisation");
  for (void* e : cache->prof.events) dev_event_destroy(e);
  cache->prof = Profile{};
  if (slots == 0) return KVC_OK;
  const size_t n = size_t(slots) * KVC_STAGES * 2;
  cache->prof.events.assign(n, nullptr);
  for (size_t k = 0; k < n; ++k) {
    rc = dev_event_create(&cache->prof.events[k]);
    if (rc) {
      for (void* e : cache->prof.events) dev_event_destroy(e);
      cache->prof = Profile{};
      return device_fail(rc, "event creation");
    }
  }
  cache->prof.recorded.assign(size_t(slots) * KVC_STAGES, 0);
  cache->prof.slots = slots;
  return KVC_OK;
}

kvc_status kvc_profile_read(kvc_cache* cache, float* ms_out, int32_t* calls_out) {
  reset_detail();
  if (!cache || !ms_out || !calls_out) return fail(KVC_ERR_NULL_ARGUMENT, "null argument to kvc_profile_read");
  for (int s = 0; s < KVC_STAGES; ++s) {
    ms_out[s] = 0.f;
    calls_out[s] = 0;
  }
  const Profile& p = cache->prof;
  for (int call = 0; call < p.used; ++call) {
    for (int s = 0; s < KVC_STAGES; ++s) {
      if (!p.recorded[size_t(call) * KVC_STAGES + s]) continue;
      float ms = 0.f;
      const size_t k = (size_t(call) * KVC_STAGES + s) * 2;
      int rc = dev_event_elapsed(&ms, p.events[k], p.events[k + 1]);
      if (rc) return device_fail(rc, "event timing");
      ms_out[s] += ms;
      calls_out[s] += 1;
    }
  }
  return KVC_OK;
}

kvc_status kvc_stream_read(const void* buf, int64_t bytes, void* sink, void* hip_stream) {
  reset_detail();
  if (!buf || !sink) return fail(KVC_ERR_NULL_ARGUMENT, "null argument to kvc_stream_read");
  if (bytes <= 0 || bytes % kProbeUnitBytes != 0 || reinterpret_cast<uintptr_t>(buf) % 16 != 0)
    return fail_ea(KVC_ERR_BAD_ARGUMENT, kProbeUnitBytes, bytes,
                   "stream read needs a 16-byte aligned buffer and a positive multiple of %lld bytes",
                   static_cast<long long>(kProbeUnitBytes));
  if (!dev_has_kernels()) return fail(KVC_ERR_DEVICE, "library built without device kernels");
  const int rc = dev_stream_read(buf, bytes, sink, hip_stream);
  if (rc) return device_fail(rc, "stream read launch");
  return KVC_OK;
}

kvc_status kvc_mfma_rate(int64_t iterations, void* sink, void* hip_stream, double* flops_out) {
  reset_detail();
  if (!sink || !flops_out) return fail(KVC_ERR_NULL_ARGUMENT, "null argument to kvc_mfma_rate");
  if (iterations <= 0 || iterations > (int64_t(1) << 24))
    return fail_ea(KVC_ERR_BAD_ARGUMENT, int64_t(1) << 24, iterations, "iterations %lld outside [1, 2^24]",
                   (long long)iterations);
  if (!dev_has_kernels()) return fail(KVC_ERR_DEVICE, "library built without device kernels");
  const int rc = dev_mfma_rate(iterations, sink, hip_stream, flops_out);
  if (rc) return device_fail(rc, "matrix-core probe launch");
  return KVC_OK;
}

kvc_status kvc_session_create(const kvc_layer* const* layers, int32_t n_layers, const void* embedding,
                              int32_t vocab, int32_t position_encoding, int32_t batch, int32_t capacity,
                              int32_t max_chunk_rows, void* hip_stream, kvc_session** out) {
  reset_detail();
  if (!layers || !embedding || !out) return fail(KVC_ERR_NULL_ARGUMENT, "null argument to kvc_session_create");
  *out = nullptr;
  if (n_layers < 1) return fail_ea(KVC_ERR_BAD_ARGUMENT, 1, n_layers, "a session needs at least one layer");
  if (vocab < 1) return fail_ea(KVC_ERR_BAD_ARGUMENT, 1, vocab, "vocabulary size must be positive");
  if (position_encoding != KVC_PE_NONE && position_encoding != KVC_PE_SINUSOIDAL)
    return fail(KVC_ERR_BAD_ARGUMENT, "unknown position encoding %d", position_encoding);
  for (int l = 0; l < n_layers; ++l) {
    if (!layers[l]) {
      g_last.layer = l;
      return fail(KVC_ERR_NULL_ARGUMENT, "layer %d is null", l);
    }
  }
  const int D = layers[0]->params->model_width;
  const kvc_dtype dt = layers[0]->params->dtype;
  for (int l = 1; l < n_layers; ++l) {
    if (layers[l]->params->model_width != D || layers[l]->params->dtype != dt) {
      g_last.layer = l;
      return fail_ea(KVC_ERR_BAD_ARGUMENT, D, layers[l]->params->model_width,
                     "layer %d has model width %d and type %d, layer 0 has %d and %d", l,
                     layers[l]->params->model_width, int(layers[l]->params->dtype), D, int(dt));
    }
  }
  int64_t rows_elems = 0;
  if (batch > 0 && max_chunk_rows > 0 &&
      (!checked_mul(int64_t(batch) * max_chunk_rows, D, &rows_elems) || rows_elems > (INT64_MAX / 16)))
    return fail(KVC_ERR_ELEMENT_COUNT_OVERFLOW, "session row buffers overflow for batch %d, %d rows, width %d",
                batch, max_chunk_rows, D);
  kvc_session* S = new (std::nothrow) kvc_session;
  if (!S) return fail(KVC_ERR_ALLOCATION_FAILED, "host allocation failed");
  S->layers.assign(layers, layers + n_layers);
  S->batch = batch;
  S->max_chunk_rows = max_chunk_rows;
  S->model_width = D;
  S->vocab = vocab;
  S->dtype = dt;
  S->sinusoidal = position_encoding == KVC_PE_SINUSOIDAL;
  S->embedding = embedding;
  int rc = dev_malloc(reinterpret_cast<void**>(&S->gate), sizeof(ErrWords) * size_t(n_layers));
  if (rc) {
    S->gate = nullptr;
    free_session(S);
    return fail(KVC_ERR_ALLOCATION_FAILED, "cannot allocate the session's failure words");
  }
  for (int l = 0; l < n_layers; ++l) {
    kvc_cache* c = nullptr;
    const kvc_status st = create_cache(layers[l], batch, capacity, max_chunk_rows, hip_stream, &S->gate[l], S->gate,
                                       n_layers, &c);
    if (st != KVC_OK) {
      const kvc_error_detail saved = g_last;
      free_session(S);
      g_last = saved;
      g_last.layer = l;
      return st;
    }
    S->caches.push_back(c);
  }
  const size_t as = acc_size(dt), es = elem_size(dt);
  const size_t rows_bytes = (size_t(rows_elems) * as + 15) & ~size_t(15);
  rc = dev_malloc(&S->h, rows_bytes);
  if (rc == 0) rc = dev_malloc(&S->a, rows_bytes);
  if (rc == 0 && dt == KVC_BF16) rc = dev_malloc(&S->x, (size_t(rows_elems) * es + 15) & ~size_t(15));
  if (rc) {
    free_session(S);
    return fail(KVC_ERR_ALLOCATION_FAILED, "cannot allocate the session's row buffers");
  }
  *out = S;
  return KVC_OK;
}

void kvc_session_destroy(kvc_session* session) { free_session(session); }

kvc_status kvc_session_chunk(kvc_session* session, const int32_t* tokens, int32_t n_max, const int32_t* n_rows,
                             void* out, int32_t flags, kvc_work* work) {
  reset_detail();
  if (!session || !tokens || !out) return fail(KVC_ERR_NULL_ARGUMENT, "null argument to kvc_session_chunk");
  if (flags & ~int32_t(KVC_ASYNC)) return fail(KVC_ERR_BAD_ARGUMENT, "unknown flags %d", flags);
  if (n_max < 1 || n_max > session->max_chunk_rows)
    return fail_ea(KVC_ERR_CHUNK_ROWS, session->max_chunk_rows, n_max, "chunk rows %d outside [1, %d]", n_max,
                   session->max_chunk_rows);
  if (n_rows) {
    for (int b = 0; b < session->batch; ++b) {
      if (n_rows[b] < 0 || n_rows[b] > n_max) {
        g_last.sequence = b;
        return fail_ea(KVC_ERR_CHUNK_ROWS, n_max, n_rows[b], "sequence %d has %d chunk rows, outside [0, %d]", b,
                       n_rows[b], n_max);
      }
    }
  }
  return session_call(session, tokens, n_max, n_rows, out, flags, work, false);
}

kvc_status kvc_session_decode(kvc_session* session, const int32_t* tokens, void* out, int32_t flags,
                              kvc_work* work) {
  reset_detail();
  if (!session || !tokens || !out) return fail(KVC_ERR_NULL_ARGUMENT, "null argument to kvc_session_decode");
  if (flags & ~int32_t(KVC_ASYNC)) return fail(KVC_ERR_BAD_ARGUMENT, "unknown flags %d", flags);
  return session_call(session, tokens, 1, nullptr, out, flags, work, true);
}

kvc_status kvc_session_truncate(kvc_session* session, const int32_t* cut, int32_t flags) {
  reset_detail();
  if (!session || !cut) return fail(KVC_ERR_NULL_ARGUMENT, "null argument to kvc_session_truncate");
  if (flags & ~int32_t(KVC_TRUNCATE_KEEP_STALE_POSITION))
    return fail(KVC_ERR_BAD_ARGUMENT, "unknown flags %d", flags);
  for (size_t l = 0; l < session->caches.size(); ++l) {
    const kvc_cache* c = session->caches[l];
    for (int b = 0; b < c->batch; ++b) {
      if (cut[b] < 0 || cut[b] > c->len[b]) {
        g_last.layer = int32_t(l);
        g_last.sequence = b;
        return fail_ea(KVC_ERR_BAD_CUT, c->len[b], cut[b], "cut %d of sequence %d is outside [0, %d]", cut[b], b,
                       c->len[b]);
      }
      if (!window_continuable(c, b, cut[b])) {
        g_last.layer = int32_t(l);
        g_last.sequence = b;
        return fail_ea(KVC_ERR_BAD_CUT, window_min_cut(c, b), cut[b],
                       "cut %d of sequence %d needs rows layer %zu's window cache no longer holds", cut[b], b, l);
      }
    }
  }
  const bool stale = flags & KVC_TRUNCATE_KEEP_STALE_POSITION;
  for (kvc_cache* c : session->caches) {
    const int rc = dev_set_lengths(c->ds, cut, stale ? 1 : 0);
    if (rc) return device_fail(rc, "length update");
  }
  for (kvc_cache* c : session->caches) {
    for (int b = 0; b < c->batch; ++b) {
      c->len[b] = cut[b];
      if (!stale) c->next_pos[b] = cut[b];
      if (cut[b] < c->held[b]) c->held[b] = cut[b];  // as the device's length update does
    }
  }
  return KVC_OK;
}

kvc_status kvc_session_reset(kvc_session* session) {
  reset_detail();
  if (!session) return fail(KVC_ERR_NULL_ARGUMENT, "null session");
  for (kvc_cache* c : session->caches) {
    const int rc = dev_set_lengths(c->ds, nullptr, 2);
    if (rc) return device_fail(rc, "length reset");
  }
  for (kvc_cache* c : session->caches) {
    std::fill(c->len.begin(), c->len.end(), 0);
    std::fill(c->next_pos.begin(), c->next_pos.end(), 0);
    std::fill(c->held.begin(), c->held.end(), 0);
  }
  return KVC_OK;
}

kvc_status kvc_session_sync(kvc_session* session) {
  reset_detail();
  if (!session) return fail(KVC_ERR_NULL_ARGUMENT, "null session");
  session->pending_async = true;  // always look at the device words
  kvc_status st = check_deferred_session(session);
  if (st != KVC_OK) return st;
  for (kvc_cache* c : session->caches) {
    st = resync_lengths(c);
    if (st != KVC_OK) return st;
  }
  return KVC_OK;
}

kvc_status kvc_session_layer_cache(kvc_session* session, int32_t layer, kvc_cache** out) {
  reset_detail();
  if (!session || !out) return fail(KVC_ERR_NULL_ARGUMENT, "null argument to kvc_session_layer_cache");
  if (layer < 0 || layer >= int32_t(session->caches.size()))
    return fail_ea(KVC_ERR_BAD_ARGUMENT, int64_t(session->caches.size()), layer, "layer %d out of range", layer);
  *out = session->caches[layer];
  return KVC_OK;
}

}  // extern "C"
