// Interface between the host cache manager (kvc_host.cpp) and the device
// backend (kvc_device.hip).  The manager owns validation, bookkeeping and
// the C ABI; the backend owns allocation, copies and kernel launches.
#pragma once

#include <cstddef>
#include <cstdint>

#include "kvcache.h"

namespace kvc {

// Device-side failure words.  Each holds the smallest flat index at which the
// condition was seen (atomicMin), or ~0 when it was not.  While any word is
// set, every state-changing kernel of the cache is a no-op.
struct ErrWords {
  unsigned long long key;       // non-finite candidate key, flat index over [B,H,n,d_h]
  unsigned long long value;     // non-finite candidate value
  unsigned long long query;     // non-finite rotated query
  unsigned long long position;  // sequence index whose row position reached max positions
  unsigned long long output;    // non-finite attention output, flat index over [B,n,D]
  unsigned long long token;     // session calls: token id outside the embedding, flat index over [B,n]
  unsigned long long pad[2];
};
constexpr unsigned long long kErrClear = ~0ull;

// Smallest number of attention rows per split-K work item of the decode
// kernel (sizes the partial buffer); each call picks tile_rows >= this.
constexpr int kDecodeTileRows = 512;
// Smallest rows per block of a paged cache: every run of rows a kernel reads
// through one block base (a decode step, a 128-row chunk-attention tile) fits.
constexpr int kMinBlockRows = 256;
// Query heads that one bf16 decode workgroup serves from a single read of
// their shared key/value head: the largest power of two <= 8 dividing the
// group size heads / kv_heads (1 for the generic kernels).
inline int decode_heads_per_block(int dtype, int head_width, int group) {
  if (dtype != KVC_BF16 || (head_width != 64 && head_width != 128)) return 1;
  int q = 1;
  while (q < 8 && group % (2 * q) == 0) q *= 2;
  return q;
}
// Largest reduction-axis split of the skinny (at most 64-row) bf16 projection.
constexpr int kSkinnySplitMax = 8;
// Values per by-value length update (kernel-argument payload).
constexpr int kSetChunk = 480;

// Everything a launch needs about one cache.  Pointers are device memory.
struct DevState {
  int dtype;  // kvc_dtype of storage and weights
  int batch, heads, head_width, model_width, capacity, max_chunk_rows;
  int kv_heads;  // key/value heads H_kv (divides heads); query head h reads h / (heads / kv_heads)
  int kv_width;  // H_kv * d_h: rows of W_k and W_v
  int rope;           // 1: rotate q, k
  int max_positions;  // rotary table rows
  double scale;       // 1 / sqrt(d_h)
  const void* wq;
  const void* wk;
  const void* wv;
  const void* wo;      // output projection, or null
  void* keys;          // [B, H_kv, C, d_h] storage type
  void* values;        // [B, H_kv, C, d_h]
  int32_t* len;        // [B] committed rows
  int32_t* next_pos;   // [B] position of the next row
  int32_t* positions;  // [B, C] absolute position of each row
  int32_t* rows;       // [B] rows of the current chunk call
  int32_t* held;       // ring caches: [B] oldest row still held (older slots were written over)
  void* cand_k;        // [B, H_kv, n, d_h] storage type (n = rows of the call)
  void* cand_v;        // [B, H_kv, n, d_h]
  void* q;             // [B, H, n, d_h] accumulate type; with q_bf16, bf16 of q * scale * log2(e)
  // q_bf16 = 1 (chunk calls of bf16 layers whose attention is the matrix-core
  // flash kernel): the projection stores each rotated query already scaled to
  // base-2 softmax units and rounded to bf16, the flash kernel's operand type
  int q_bf16;
  void* merged;        // [B, n, D] accumulate type: merged heads before W_o (null without W_o)
  void* out_proj_dst;  // [B, n, D] accumulate type: destination of the W_o projection (per call)
  void* partials;      // [B, H, max_tiles, d_h + 2] accumulate type
  int32_t* redo;       // bf16 chunk calls at d_h = 128: per workgroup of the role-split attention, 1 = recompute
  float* proj_partials;  // bf16 caches: [kSkinnySplitMax, 64, D + 2 kv_width] float32 split-K sums of
                         // the skinny projection (null: that projection runs unsplit)
  int max_tiles;       // ceil(C / kDecodeTileRows)
  int tile_rows;       // split-K tile of the current decode call (multiple of kDecodeTileRows)
  int single_tile;     // 1 when every lane of the current decode call fits one tile
  void* rope_cos;  // [max_positions, d_h / 2] accumulate type (null without rotation)
  void* rope_sin;
  // Block-paged storage (paged = 1): keys and values are pools
  // [blocks, H_kv, block_rows, d_h] and row r of sequence b lives in block
  // block_table[b * table_width + (r >> block_rows_log2)] (capacity =
  // table_width << block_rows_log2).  paged = 0: [B, H, C, d_h].
  int paged;
  int block_rows_log2;
  int table_width;
  const int32_t* block_table;
  // Sliding window (window > 0): a query at row r reads rows r - window + 1 .. r,
  // and the contiguous storage is a ring: row r lives in slot r % capacity
  // (ring = 1), so lengths grow past the capacity while the last `capacity`
  // rows stay held.  window = 0: every row 0 .. r, no ring.
  int window;
  int ring;
  int span_rows;  // most rows one decode query reads, plus tile alignment (sizes the split-K grid)
  ErrWords* err;
  // The failure words every state-changing kernel checks before it writes:
  // the cache's own (gate_count 1), or those of every layer of a session, so
  // that one layer's failure keeps every layer unchanged.
  const ErrWords* gate;
  int gate_count;
  void* stream;  // hipStream_t
};

// ---- backend, implemented by kvc_device.hip (HIP) -------------------------
// Every function returns 0 on success or a nonzero backend error code;
// dev_error_string() describes the last one.
const char* dev_error_string(int code);
int dev_current_device(int* device);
int dev_compute_units(int device, int* units);
int dev_malloc(void** p, size_t bytes);
void dev_free(void* p);
int dev_host_malloc(void** p, size_t bytes);
void dev_host_free(void* p);
int dev_copy_h2d_sync(void* dst, const void* src, size_t bytes, void* stream);
int dev_copy_d2h_sync(void* dst, const void* src, size_t bytes, void* stream);
int dev_copy_d2h_2d_sync(void* dst, size_t dpitch, const void* src, size_t spitch, size_t width,
                         size_t height, void* stream);
int dev_sync(void* stream);
int dev_zero(void* p, size_t bytes, void* stream);  // bytes % 16 == 0, p 16-byte aligned
int dev_clear_err(ErrWords* err, void* stream);

// Length updates carried in kernel arguments (no host staging buffers).
// mode 0: len = np = vals; mode 1: len = vals (next position kept); mode 2: len = np = 0.
int dev_set_lengths(const DevState& s, const int32_t* vals, int mode);
// rows[b] = vals[b] for the next chunk call.
int dev_set_rows(const DevState& s, const int32_t* vals);
// Paged caches: table[idx[k]] = val[k] for k < count (kernel arguments).
int dev_set_table(const DevState& s, const int32_t* idx, const int32_t* val, int count);
// Paged caches: every table entry = -1 (no block).
int dev_clear_table(const DevState& s);
// len[seq] = next_pos[seq] = value (one sequence; the others unchanged); for a
// ring cache held[seq] = held[held_src] (a fork that copied every slot), or 0
// when held_src < 0.
int dev_set_seq_length(const DevState& s, int seq, int32_t value, int held_src);
// Paged caches: rows [0, rows) of every head of block `src` into block `dst`
// (copy-on-write of a shared block before an append into it).
int dev_copy_block_rows(const DevState& s, int dst, int src, int rows);
// positions[dst_seq, 0..rows) = positions[src_seq, 0..rows).
int dev_copy_positions(const DevState& s, int dst_seq, int src_seq, int rows);
// Contiguous caches: K/V rows [0, rows) of every head of src_seq into dst_seq.
int dev_copy_seq_rows(const DevState& s, int dst_seq, int src_seq, int rows);

// Pipeline stages.  n_max: rows per sequence of this call (1 for decode);
// per_seq_rows: 0 = every sequence has n_max rows, 1 = rows[] holds them.
int dev_project(const DevState& s, const void* x, int n_max, int per_seq_rows);
// Sequences of a decode call with the most retained rows first, dealt out in
// rounds of per_round sequences (as many as one workgroup per compute unit
// covers), every other round reversed: the bf16 split-K attention launches its
// workgroups in this order, so the longest lanes start early and a unit that
// takes a long lane in one round takes a short one in the next (ragged
// batches).  count is 0 when the batch exceeds the table (sequence order).
constexpr int kMaxSeqOrder = 256;
struct SeqOrder {
  int32_t count;
  int32_t seq[kMaxSeqOrder];
};
void build_seq_order(SeqOrder* o, int batch, const int32_t* len, int per_round);
int dev_attend_decode(const DevState& s, const SeqOrder& order, void* out);
int dev_merge_decode(const DevState& s, void* out);
// Softmax weights [H, rows] (accumulate type, device) of the last decode call's
// query of sequence b over its committed rows r0 .. r0 + rows - 1.
int dev_newest_weights(const DevState& s, int b, int r0, int rows, void* w);
// Work items of the bf16 chunk attention kernel: one per (sequence, tile of
// kChunkQueryTile chunk rows), listed with the most keys to read first, so
// that the longest items start early and the ragged tail is short.  With more
// items than the table holds, count is 0 and the kernel walks sequences in
// order (query tiles from the last one down).
constexpr int kChunkQueryTile = 256;
constexpr int kMaxChunkOrder = 256;
struct ChunkOrder {
  int32_t count;                 // items listed (0: natural order)
  int32_t qtiles;                // query tiles per sequence, ceil(n_max / kChunkQueryTile)
  int32_t item[kMaxChunkOrder];  // (sequence << 16) | query tile
};
// Fills `o` for a chunk call: rows[b] chunk rows and len[b] retained rows of
// sequence b (the work estimate only orders items; every item with rows is
// listed exactly once).
void build_chunk_order(ChunkOrder* o, int batch, int n_max, const int32_t* len, const int32_t* rows);
int dev_attend_chunk(const DevState& s, int n_max, int per_seq_rows, const ChunkOrder& order, void* out);
// out[b, i, :] = merged[b, i, :] x W_o (rows i < n_b).
int dev_output_project(const DevState& s, int n_max, int per_seq_rows, void* out);
int dev_commit(const DevState& s, int n_max, int per_seq_rows);

// Session stages (rows i < n_b of [B, n_max, D]; the first layer's DevState
// supplies geometry, next positions, rows and the token failure word).
// h[b, i] = embedding[tokens[b, i]] (+ sinusoidal encoding of next_position +
// i); x (non-null for bf16 sessions) receives h rounded to the weight type.
int dev_embed(const DevState& s, const int32_t* tokens, const void* embedding, int vocab, int sinusoidal,
              int n_max, int per_seq_rows, void* h, void* x);
// h_out = h_in + tanh(a) (the tanh-residual block); x as for dev_embed.
int dev_residual(const DevState& s, const void* h_in, const void* a, void* h_out, void* x, int n_max,
                 int per_seq_rows);

int dev_event_create(void** e);
void dev_event_destroy(void* e);
int dev_event_record(void* e, void* stream);
int dev_event_elapsed(float* ms, void* start, void* stop);

// Streaming read of `bytes` (a positive multiple of kProbeUnitBytes) at `buf`;
// `sink` receives a store only for one improbable xor of the data.
constexpr int64_t kProbeUnitBytes = 32768;
int dev_stream_read(const void* buf, int64_t bytes, void* sink, void* stream);
// Matrix-core rate probe: `iterations` rounds of independent bf16 32x32x16
// MFMAs per wave, two waves per SIMD on every compute unit; *flops receives the
// launch's floating-point operations.  `sink` receives a store only for one
// improbable sum.
int dev_mfma_rate(int64_t iterations, void* sink, void* stream, double* flops);

// True when the backend can run kernels (false in the CPU-only host-check build).
bool dev_has_kernels();

// Scratch of kvc_append_and_attend_static: a file-scope device array of this
// many bytes in the backend's code object (one copy per device, held until the
// process ends).  Its device address on `device` is looked up once per device,
// with that device current, and kept; later calls return the kept address.
constexpr size_t kStaticScratchBytes = KVC_STATIC_SCRATCH_BYTES;
int dev_static_scratch(int device, void** ptr, size_t* bytes);

}  // namespace kvc
