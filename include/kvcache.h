/*
 * kvcache.h -- C ABI of libkvcache.so: a layer-bound, fixed-capacity KV cache
 * with a cached decode step and a prefix-cut continuation, on AMD MI355X (gfx950).
 *
 * Sources.  "Chapter 37" is the incremental-attention course chapter "Keep the
 * prefix, project only the new row" (intale.github.io learn_llm).  "The
 * prefix-reuse note" is "LLM mechanism experiment (5): can only the changed
 * suffix be recomputed?" (huhohoo.com).  Each declaration names the passage
 * that defines its operation.
 *
 * Conventions for every call.
 *  - Every call returns kvc_status; KVC_OK is 0.  On any other status the
 *    cache's logical state (lengths, next positions, row positions, rows below
 *    the length) AND its whole physical storage are unchanged (Chapter 37,
 *    "Reset or reject without corrupting retained state"), and
 *    kvc_last_error() describes the failure.
 *  - Device pointers are HIP device memory on the cache's device.  Host
 *    pointers are ordinary host memory.  Each argument below says which.
 *  - All work of one cache is ordered on the HIP stream given at creation.  A
 *    handle is not thread-safe; use one cache from one thread at a time.
 *  - Weights, inputs and outputs are borrowed: the caller owns them and keeps
 *    them alive until the call (in KVC_ASYNC mode: the stream work) completes.
 *    The library owns the K/V storage, lengths, positions, candidate rows,
 *    scratch and the rotary table, allocated only in kvc_cache_create and
 *    freed only in kvc_cache_destroy.
 */
#ifndef KVCACHE_H
#define KVCACHE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t kvc_status;

enum {
  KVC_OK = 0,
  /* Cache construction, checked in this order (Chapter 37, layer-kv-cache
   * listing: the cache constructor and its error enum). */
  KVC_ERR_ZERO_BATCH = 1,
  KVC_ERR_ZERO_CAPACITY = 2,
  KVC_ERR_CAPACITY_EXCEEDS_POSITIONS = 3, /* capacity > rotary max positions          */
  KVC_ERR_ELEMENT_COUNT_OVERFLOW = 4,     /* B*H*C*d_h does not fit 64-bit indexing    */
  KVC_ERR_ALLOCATION_FAILED = 5,          /* device or pinned host allocation failed   */
  /* Request checks, in the order Chapter 37 gives under "Bind the state,
   * calculate completely, then commit": rank, one token, batch, width, cache
   * model width, heads, head width, parameter identity, parameter revision,
   * rotary configuration, remaining capacity. */
  KVC_ERR_INPUT_RANK = 10,
  KVC_ERR_SINGLE_TOKEN_REQUIRED = 11,
  KVC_ERR_INPUT_BATCH_MISMATCH = 12,
  KVC_ERR_INPUT_WIDTH_MISMATCH = 13,
  KVC_ERR_CACHE_MODEL_WIDTH_MISMATCH = 14,
  KVC_ERR_CACHE_HEAD_COUNT_MISMATCH = 15,
  KVC_ERR_CACHE_HEAD_WIDTH_MISMATCH = 16,
  KVC_ERR_CACHE_LAYER_MISMATCH = 17,          /* weights are not the bound parameter set */
  KVC_ERR_CACHE_LAYER_REVISION_MISMATCH = 18, /* bound weights were updated in place    */
  KVC_ERR_CACHE_ROPE_MISMATCH = 19,           /* feature width, max positions or base   */
  KVC_ERR_FULL = 20,                          /* a sequence has no room for the rows    */
  KVC_ERR_OUT_OF_BLOCKS = 21,                 /* paged cache: the pool has fewer free blocks
                                                 than the call needs (expected = needed,
                                                 actual = free)                          */
  KVC_ERR_CACHE_WINDOW_MISMATCH = 22,         /* the layer's sliding window differs from the
                                                 cache's (checked after the rotary setup)  */
  /* Found on the device before the commit; the commit is then suppressed.
   * Precedence when several hold: key, value, query, position, output. */
  KVC_ERR_NONFINITE_KEY = 30,    /* candidate rotated key has a NaN/Inf (first flat index
                                    over [B, H_kv, n, d_h])                                */
  KVC_ERR_NONFINITE_VALUE = 31,  /* candidate value has a NaN/Inf                          */
  KVC_ERR_NONFINITE_QUERY = 32,  /* rotated query has a NaN/Inf                            */
  KVC_ERR_ROTARY_POSITION = 33,  /* a row's position reaches the rotary max positions      */
  KVC_ERR_NONFINITE_OUTPUT = 34, /* softmax or mixture produced a NaN/Inf                  */
  KVC_ERR_TOKEN_RANGE = 35,      /* session call: a token id outside [0, vocab); reported
                                    before the others (flat index over [B, n])             */
  /* Continuation (prefix-reuse note). */
  KVC_ERR_BAD_CUT = 40,          /* cut < 0 or cut > current length                        */
  KVC_ERR_EMPTY_QUERY = 41,      /* lcp query with no tokens                               */
  KVC_ERR_CHUNK_ROWS = 42,       /* n_max outside [1, max_chunk_rows] or n_rows[b] outside [0, n_max] */
  /* Interface. */
  KVC_ERR_NULL_ARGUMENT = 50,
  KVC_ERR_DTYPE_UNSUPPORTED = 51,
  KVC_ERR_SHAPE_UNSUPPORTED = 52, /* head width not a power of two in [2, 16 B * 64 / elem] */
  KVC_ERR_BAD_ARGUMENT = 53,
  KVC_ERR_SCRATCH_EXCEEDED = 54, /* kvc_append_and_attend_static: the call needs more scratch
                                    than the static array holds (expected = its size in bytes,
                                    actual = bytes needed)                               */
  KVC_ERR_DEVICE = 60,           /* a HIP runtime call failed                              */
  KVC_ERR_DEFERRED = 61,         /* an earlier KVC_ASYNC call failed on the device         */
  KVC_ERR_INTERNAL = 62
};

/* Storage / arithmetic type.  A cache's K/V storage type must equal its
 * weights' type; F64 computes in double, F32 and BF16 accumulate in float. */
typedef enum { KVC_F64 = 0, KVC_F32 = 1, KVC_BF16 = 2 } kvc_dtype;

/* Position handling of a layer.  ROPE rotates q and k by rotate-half RoPE at
 * their absolute position (Chapter 37, "Append along the position axis").
 * NONE applies no rotation: the caller adds absolute position encodings to the
 * hidden rows itself, as the prefix-reuse note's toy decoder does. */
typedef enum { KVC_POS_ROPE = 0, KVC_POS_NONE = 1 } kvc_pos_mode;

/* Call flags. */
enum {
  KVC_SYNC = 0,  /* wait for the stream; device-found errors are returned directly */
  KVC_ASYNC = 1  /* return after enqueueing; a device-found error is sticky, every
                    later commit on the cache is suppressed, and the next KVC_SYNC
                    call or kvc_sync() returns KVC_ERR_DEFERRED with its detail.
                    Outputs of calls made after a failed one are undefined.
                    kvc_truncate, kvc_reset and kvc_fork never wait for the
                    stream: enqueued while such a failure is still unreported,
                    their device updates are suppressed like the commits (they
                    return KVC_OK); the DEFERRED report then restores the host's
                    lengths from the device and the caller repeats them. */
};

/* kvc_truncate flags. */
enum {
  KVC_TRUNCATE_KEEP_STALE_POSITION = 1 /* negative control of the prefix-reuse note
                                          ("What must be trimmed together"): trims the
                                          rows but leaves next_position unchanged.
                                          For tests; it produces wrong results. */
};

/* Payload of the last failure on the calling thread (Chapter 37 error enums). */
typedef struct {
  kvc_status status;
  int32_t parameter;        /* revision mismatch: first weight that differs (0 W_q .. 3 W_o) */
  int32_t sequence;         /* sequence index for FULL, BAD_CUT, CHUNK_ROWS, ROTARY_POSITION */
  int32_t layer;            /* session calls: index of the layer that failed; -1 otherwise   */
  int64_t expected, actual; /* rank, tokens, batch, width, heads, head width, capacity, ... */
  uint64_t cache_revision, layer_revision;
  int64_t flat_index;       /* NONFINITE_*: first flat index over the candidate [B,H,n,d_h]  */
  double value;             /* NONFINITE_KEY/VALUE: the offending element                    */
  int32_t rope_feature_width[2]; /* ROPE_MISMATCH: [cache, layer]                            */
  int32_t rope_max_positions[2];
  double rope_base[2];
  char message[256];
} kvc_error_detail;

/* Projection-row counts of one call, per Q, K or V projection, summed over
 * the batch (Chapter 37, "Count projection rows, not hardware time"):
 * decode: full = sum(len_b + 1), incremental = B, reused = sum(len_b);
 * chunk:  full = sum(len_b + n_b), incremental = sum(n_b), reused = sum(len_b).
 * position_min/max: smallest and largest absolute position computed. */
typedef struct {
  int64_t full_prefix_rows_per_projection;
  int64_t incremental_rows_per_projection;
  int64_t reused_key_value_rows;
  int32_t position_min, position_max;
} kvc_work;

/* Geometry of a cache, for callers that size buffers. */
typedef struct {
  int32_t batch, heads, head_width, model_width, capacity, max_chunk_rows;
  int32_t kv_dtype, pos_mode, rope_max_positions, device;
  double rope_base;
  int32_t block_rows, pool_blocks; /* paged caches; 0 for contiguous storage */
  int32_t kv_heads;                /* key/value heads H_kv (= heads without grouping) */
  int32_t window;                  /* sliding window (0: every row)                  */
} kvc_cache_desc;

typedef struct kvc_params kvc_params; /* W_q, W_k, W_v (, W_o) with an identity and revisions */
typedef struct kvc_layer kvc_layer;   /* parameters + head count + position handling           */
typedef struct kvc_cache kvc_cache;   /* one layer's fixed-capacity K/V state                  */

/* Registers a parameter set.  w_q, w_k, w_v: DEVICE, each [D, D] row-major as
 * [out, in] (a projected row is y[j] = sum_i x[i] W[j, i]), element type
 * `dtype`, borrowed.  w_o: the layer's output projection in the same layout,
 * or NULL for a layer whose calls return the merged heads (Chapter 37, "Bind
 * the state, calculate completely, then commit": the layer has four
 * parameters and the output projection is the last step before the commit).
 * Each call creates a new identity, so a rebuilt layer with equal shapes and
 * values is still a different parameter set.
 * Errors: NULL_ARGUMENT, BAD_ARGUMENT (D <= 0), DTYPE_UNSUPPORTED. */
kvc_status kvc_params_create(int32_t model_width, kvc_dtype dtype, const void* w_q,
                             const void* w_k, const void* w_v, const void* w_o,
                             kvc_params** out);

/* A parameter set with grouped key/value heads (Chapter 37, "From causal
 * attention to managed LLM inference state": Shazeer's analysis names the
 * repeated loading of the retained keys and values as the bandwidth bottleneck
 * and answers it with multi-query attention).  w_q and w_o are [D, D] as for
 * kvc_params_create; w_k and w_v are DEVICE [kv_width, D] row-major: they
 * project a row to H_kv = kv_width / d_h key/value heads, and query head h
 * reads key/value head h / (H / H_kv) (H_kv = 1: multi-query; kv_width = D:
 * the same as kvc_params_create).  A cache of such a layer stores
 * [B, H_kv, C, d_h], so every retained row is H / H_kv times smaller to keep
 * and to read.  kvc_layer_create checks that kv_width is a whole number of
 * head widths dividing the head count.  Errors: those of kvc_params_create,
 * and BAD_ARGUMENT (kv_width <= 0 or not dividing D). */
kvc_status kvc_params_create_grouped(int32_t model_width, int32_t kv_width, kvc_dtype dtype,
                                     const void* w_q, const void* w_k, const void* w_v,
                                     const void* w_o, kvc_params** out);

/* Records an in-place update of weight `which` (0 W_q, 1 W_k, 2 W_v, 3 W_o, -1
 * all): its value revision advances and caches bound to the old revision
 * reject further calls (Chapter 37: an optimiser step keeps the identity but
 * advances the revision).  Errors: NULL_ARGUMENT, BAD_ARGUMENT (index out of
 * range, or 3 without W_o). */
kvc_status kvc_params_mark_updated(kvc_params* params, int32_t which);
void kvc_params_destroy(kvc_params* params);

/* A layer view over a parameter set: `heads` divides D; d_h = D / heads must
 * be even and a power of two small enough for one wavefront (see
 * SHAPE_UNSUPPORTED).  Several layers may share one parameter set with
 * different rotary configurations (Chapter 37 error evidence: same parameters,
 * doubled base or one more max position).  rope_base > 0, rope_max_positions > 0.
 * With grouped parameters the layer has H_kv = kv_width / d_h key/value
 * heads, which must divide `heads`.  The params handle must outlive the layer.
 * Errors: NULL_ARGUMENT, BAD_ARGUMENT, SHAPE_UNSUPPORTED. */
kvc_status kvc_layer_create(const kvc_params* params, int32_t heads, kvc_pos_mode pos_mode,
                            double rope_base, int32_t rope_max_positions, kvc_layer** out);

/* A layer with sliding-window attention (prefix-reuse note, "Why a
 * sliding-window partial hit must fall back": the window is part of the
 * computation a cache is bound to): a query at row r reads rows
 * max(0, r - window + 1) .. r only; window 0 is kvc_layer_create.  Its cache
 * (contiguous only) is a ring of `capacity` rows: row r lives in slot
 * r % capacity, lengths and positions keep counting past the capacity (no
 * FULL; the rotary table still bounds positions), and only the last
 * `capacity` rows are held.  kvc_cache_create then requires capacity >=
 * window, capacity a multiple of 256 and max_chunk_rows <= capacity.  The
 * cache's binding includes the window (CACHE_WINDOW_MISMATCH).  A sequence
 * holds rows h .. len - 1, where h rises as appends write over the oldest
 * slots (a truncation keeps h; a cut to 0 or a reset clears it).  A cut
 * other than 0 must keep every row its continuation reads,
 * max(0, cut - window + 1) >= h; others are rejected (kvc_truncate,
 * kvc_fork: BAD_CUT with `expected` = the smallest nonzero cut allowed);
 * kvc_reuse_cut gives the cut to continue from.  kvc_snapshot returns the
 * held rows.  Errors: those of kvc_layer_create, BAD_ARGUMENT (window < 0). */
kvc_status kvc_layer_create_windowed(const kvc_params* params, int32_t heads, kvc_pos_mode pos_mode,
                                     double rope_base, int32_t rope_max_positions, int32_t window,
                                     kvc_layer** out);
void kvc_layer_destroy(kvc_layer* layer);

/* Creates an empty cache bound to `layer` (Chapter 37, the cache constructor):
 * K/V storage [B, H_kv, C, d_h] in the weights' type (H_kv = H unless the
 * parameter set groups its key/value heads), zero-filled; lengths and
 * next positions 0; binding = the layer's parameter identity and current
 * revisions and its rotary configuration.  max_chunk_rows (>= 1) bounds n_max
 * of kvc_continue_chunk and sizes its scratch.  hip_stream: a hipStream_t (or
 * NULL for the null stream) on the current device; all work of this cache runs
 * on it.  This is the only call that allocates.
 * Errors, in order: NULL_ARGUMENT, ZERO_BATCH, ZERO_CAPACITY,
 * CAPACITY_EXCEEDS_POSITIONS, BAD_ARGUMENT (max_chunk_rows < 1),
 * ELEMENT_COUNT_OVERFLOW, ALLOCATION_FAILED, DEVICE. */
kvc_status kvc_cache_create(const kvc_layer* layer, int32_t batch, int32_t capacity,
                            int32_t max_chunk_rows, void* hip_stream, kvc_cache** out);
void kvc_cache_destroy(kvc_cache* cache);

/* Block-paged cache (Chapter 37, "From causal attention to managed LLM
 * inference state": serving systems keep growing KV caches as logical blocks
 * mapped onto non-contiguous physical memory; the prefix-reuse note names
 * block storage as the next step after its copy-per-branch ownership, "Lookup
 * flow and cache ownership").  Same calls and results as kvc_cache_create,
 * with K and V held in one pool per tensor of `pool_blocks` blocks, each
 * [H, block_rows, d_h]: logical row r of sequence b is row r % block_rows of
 * the block that b's table names at r / block_rows.  block_rows is a power of
 * two >= 256 that divides `capacity`; the pool may hold fewer blocks than
 * B * capacity / block_rows (sequences share the pool).  Appends take free
 * blocks as rows cross a block boundary and fail with OUT_OF_BLOCKS (state
 * unchanged) when the pool runs out; kvc_truncate and kvc_reset return blocks
 * wholly past the cut; kvc_fork shares blocks, and an append into a block that
 * another sequence still names first copies it (copy-on-write).  Attention
 * results are bit-identical to a contiguous cache fed the same calls.
 * kvc_storage_pointers / kvc_copy_storage cover the pools
 * ([pool_blocks, H, block_rows, d_h] each).
 * Errors: those of kvc_cache_create, then BAD_ARGUMENT (block_rows or
 * pool_blocks invalid). */
kvc_status kvc_cache_create_paged(const kvc_layer* layer, int32_t batch, int32_t capacity,
                                  int32_t max_chunk_rows, int32_t block_rows, int32_t pool_blocks,
                                  void* hip_stream, kvc_cache** out);

/* Branches a sequence (prefix-reuse note, "Lookup flow and cache ownership":
 * a lookup that continues another branch's prefix must not modify that
 * branch): sequence dst becomes the first `rows` rows of sequence src (keys,
 * values and row positions) with next_position[dst] = rows, as if it were a
 * copy of src truncated at `rows`; src is unchanged.  A paged cache shares
 * src's blocks (no K/V data moves; a later append into a shared block copies
 * it first); a contiguous cache copies the rows.  Stream-ordered, no
 * allocation.  Errors: NULL_ARGUMENT, BAD_ARGUMENT (src or dst out of range,
 * or equal), BAD_CUT (rows outside [0, len[src]]), DEVICE. */
kvc_status kvc_fork(kvc_cache* cache, int32_t src, int32_t dst, int32_t rows);

/* Blocks of a paged cache's pool named by some sequence, and free ones (HOST,
 * each nullable).  Errors: NULL_ARGUMENT, BAD_ARGUMENT (not paged), DEFERRED. */
kvc_status kvc_pool_usage(kvc_cache* cache, int32_t* blocks_in_use, int32_t* blocks_free);

/* The cached decode step (Chapter 37, "Bind the state, calculate completely,
 * then commit", and the incremental-attention listing).  x: DEVICE, shape
 * `shape[0..rank-1]`, which must be [B, 1, D] in the weights' type.  For each
 * sequence b it projects only the new row, rotates q and k at position
 * next_position[b] (= the old length), scores q against the len[b] retained
 * keys plus the candidate key with scale 1/sqrt(d_h), applies a stable
 * softmax, mixes the retained values plus the candidate value, merges the
 * heads and, when the parameter set has W_o, applies it; the result goes to
 * out (DEVICE, [B, 1, D]; double for F64 caches, float otherwise).  Only then
 * does it append the rotated key and unrotated value at row len[b] and
 * advance len[b] and next_position[b] by one (cache transition, "Append along
 * the position axis").  work (HOST, nullable) receives the row counts.
 * Errors: the request checks above in their order, then the device-found
 * ones; DEFERRED. */
kvc_status kvc_append_and_attend(const kvc_layer* layer, kvc_cache* cache, const void* x,
                                 int32_t rank, const int64_t* shape, void* out, int32_t flags,
                                 kvc_work* work);

/* kvc_append_and_attend for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, checks, results and cache transition as
 * kvc_append_and_attend (the same kernels with the same launch shapes), but
 * the call's scratch -- rotated queries, candidate key/value rows, split-K
 * partials, the projection's split sums and, with W_o, the merged heads --
 * lives in one file-scope device array of KVC_STATIC_SCRATCH_BYTES per device
 * instead of the cache's own buffers.  The call allocates nothing (no
 * hipMalloc, hipFree or allocating library routine); the array is part of the
 * library's code object, each device holds its copy until the process ends,
 * and its address on a device is looked up on the first call there.  The
 * scratch a call needs, with a = 8 bytes for F64 caches and 4 otherwise and e
 * the storage element size: queries B * H * d_h * a, candidates
 * 2 * B * kv_width * e, partials B * H * T * (d_h + 2) * a with
 * T = ceil(C / 512) (a window cache: ceil((min(C, window) + 512) / 512)),
 * for bf16 caches of width 2048, 4096 or 8192 with B <= 32 the projection's
 * split sums 8 * 64 * (D + 2 * kv_width) * 4, and with W_o B * D * a; each
 * rounded up to 256 bytes.  A call needing more than the array holds (e.g. a
 * bf16 cache of B = 32, D = 8192, C = 512) fails with SCRATCH_EXCEEDED before
 * any work; the B = 32, H = 32, d_h = 128, C = 4096 bf16 layer needs 30.5 MB.
 * Every call on one device shares its array and keeps the previous call's
 * contents: calls whose stream work overlaps on one device (several threads,
 * or several streams in KVC_ASYNC mode) race and give undefined results;
 * serialise them.  In a DEFERRED report after KVC_ASYNC calls, `value` may
 * not be the offending element (the scratch has been reused).
 * Errors: those of kvc_append_and_attend, then SCRATCH_EXCEEDED. */
#define KVC_STATIC_SCRATCH_BYTES (32u << 20)
kvc_status kvc_append_and_attend_static(const kvc_layer* layer, kvc_cache* cache, const void* x,
                                        int32_t rank, const int64_t* shape, void* out, int32_t flags,
                                        kvc_work* work);

/* Readout of the newest query's attention weights, for small caches and tests
 * (Chapter 37, figure "Advance the layer cache one position at a time": the
 * trace prints, after each step, the softmax weights of the newest query of
 * each head over every retained row).  For sequence `seq`, right after a
 * successful kvc_append_and_attend on the cache (any call since that moves
 * the cache -- chunk, truncate, reset, fork, the static variant -- makes it
 * BAD_ARGUMENT): the weights softmax(q . k_j / sqrt(d_h)) of that call's
 * rotated query of each head over the committed rows j, the newest included
 * (a window cache: its last `window` rows), recomputed on the device from the
 * stored keys.  weights_out: DEVICE [H, rows] in the accumulate type (double
 * for F64 caches, float otherwise), or NULL to query `rows` only;
 * rows_capacity: rows per head the buffer holds; rows_out (HOST): rows.
 * Synchronises the stream.  Errors: NULL_ARGUMENT, BAD_ARGUMENT, DEFERRED,
 * DEVICE. */
kvc_status kvc_newest_weights(kvc_cache* cache, int32_t seq, void* weights_out, int64_t rows_capacity,
                              int32_t* rows_out);

/* Suffix-chunk continuation (prefix-reuse note, "What must be trimmed
 * together"): x DEVICE [B, n_max, D]; n_rows HOST int32[B] with 0 <= n_b <=
 * n_max (NULL: every n_b = n_max).  Row i < n_b of sequence b is projected,
 * rotated at next_position[b] + i, and attends causally to the len[b]
 * retained rows plus its chunk rows 0..i; merged heads (times W_o when the
 * parameter set has it) go to out DEVICE [B, n_max, D] (rows i >= n_b
 * untouched).  Then the n_b rows are appended and len[b] and
 * next_position[b] advance by n_b.  A prefill is this call on an empty cache.
 * Errors: NULL_ARGUMENT, CHUNK_ROWS, the binding checks (model width .. rotary
 * configuration), FULL (len[b] + n_b > C), ROTARY_POSITION, device-found
 * errors, DEFERRED. */
kvc_status kvc_continue_chunk(const kvc_layer* layer, kvc_cache* cache, const void* x,
                              int32_t n_max, const int32_t* n_rows, void* out, int32_t flags,
                              kvc_work* work);

/* Keeps rows 0..cut[b]-1 of every sequence and sets next_position[b] = cut[b]
 * (prefix-reuse note, "What must be trimmed together").  cut: HOST int32[B],
 * 0 <= cut[b] <= len[b].  Moves no K/V data and allocates nothing.
 * flags: 0 or KVC_TRUNCATE_KEEP_STALE_POSITION.  After a KVC_ASYNC call see
 * KVC_ASYNC (a pending device failure suppresses the update).  Errors:
 * NULL_ARGUMENT, BAD_CUT, BAD_ARGUMENT, DEVICE. */
kvc_status kvc_truncate(kvc_cache* cache, const int32_t* cut, int32_t flags);

/* Logical reset (Chapter 37, "Keep layer, logical length, and capacity
 * separate"): every length and next position becomes 0; capacity, storage
 * contents, allocation and the parameter binding are unchanged, so a cache
 * bound to updated weights stays rejected.  After a KVC_ASYNC call see
 * KVC_ASYNC.  Errors: NULL_ARGUMENT, DEVICE. */
kvc_status kvc_reset(kvc_cache* cache);

/* Logical snapshot of sequence `seq` (Chapter 37, logical key/value
 * accessors; a window cache gives the rows it still holds, h .. len - 1, and
 * `len` below means their count): keys_out, values_out HOST
 * [H_kv, len, d_h] in the storage type,
 * positions_out HOST int32[len] (each nullable).  rows_capacity: rows the
 * buffers hold; rows_out (HOST): len.  Synchronises the stream.  Errors:
 * NULL_ARGUMENT, BAD_ARGUMENT (seq out of range or rows_capacity < len),
 * DEFERRED, DEVICE. */
kvc_status kvc_snapshot(kvc_cache* cache, int32_t seq, void* keys_out, void* values_out,
                        int32_t* positions_out, int64_t rows_capacity, int32_t* rows_out);

/* Lengths and next positions as committed on the device (Chapter 37, "Keep
 * layer, logical length, and capacity separate": the cache's length accessors
 * report the logical rows apart from the capacity; per sequence here): HOST
 * int32[B] each (nullable).  Synchronises the stream.  Errors: NULL_ARGUMENT,
 * DEFERRED, DEVICE. */
kvc_status kvc_lengths(kvc_cache* cache, int32_t* len_out, int32_t* next_position_out);

/* Waits for the cache's stream and reports a deferred device-found error
 * (KVC_ERR_DEFERRED; kvc_last_error() then holds the original status in
 * `actual` and the original detail).  Clears the sticky error and resyncs
 * the host copy of the lengths.  The rejection it reports is the one Chapter
 * 37 requires under "Reset or reject without corrupting retained state": the
 * failed call and everything queued behind it left the cache unchanged. */
kvc_status kvc_sync(kvc_cache* cache);

/* Longest-common-prefix cut (prefix-reuse note, "First, one history edit" and
 * "Lookup flow and cache ownership"): the length of the contiguous common
 * prefix of `cached` and `query`, capped at n_query - 1 so the last query
 * token is always recomputed.  HOST arrays.  Errors: NULL_ARGUMENT (a NULL
 * pointer with a positive count), EMPTY_QUERY, BAD_ARGUMENT (n_cached < 0). */
kvc_status kvc_lcp_cut(const int32_t* cached, int64_t n_cached, const int32_t* query,
                       int64_t n_query, int64_t* cut_out);

/* The cut to continue sequence `seq` from, given the longest common prefix
 * `lcp_cut` of its cached tokens and a query (kvc_lcp_cut): lcp_cut itself
 * when every row the continuation reads is still held, else 0 -- a full
 * recompute (prefix-reuse note, "Why a sliding-window partial hit must fall
 * back": with window 4 a cache of positions 0..7 holds only 4..7, so an edit
 * at position 4 recomputes while an append reuses all 8 rows).  Caches
 * without a window return lcp_cut.  HOST cut_out.  Errors: NULL_ARGUMENT,
 * BAD_ARGUMENT (seq), BAD_CUT (lcp_cut outside [0, len]), DEFERRED. */
kvc_status kvc_reuse_cut(kvc_cache* cache, int32_t seq, int64_t lcp_cut, int64_t* cut_out);

/* Geometry of a cache.  Errors: NULL_ARGUMENT. */
kvc_status kvc_cache_describe(const kvc_cache* cache, kvc_cache_desc* out);

/* State audits (Chapter 37, "Reset or reject without corrupting retained
 * state": same allocation, storage unchanged).  kvc_storage_pointers returns
 * the DEVICE base addresses of the K and V storage and their size in bytes;
 * kvc_copy_storage copies the whole physical storage [B, H, C, d_h] of each
 * into HOST buffers of that size (either nullable) after synchronising. */
kvc_status kvc_storage_pointers(const kvc_cache* cache, const void** keys, const void** values,
                                int64_t* bytes_each);
kvc_status kvc_copy_storage(kvc_cache* cache, void* keys_out, void* values_out);

/* Per-stage kernel timing with HIP events on the cache's stream.
 * kvc_profile_enable(cache, slots): slots > 0 starts recording event pairs
 * around each stage of each call (at most `slots` calls, then recording
 * stops); 0 stops and frees them.  kvc_profile_read synchronises and writes
 * per-stage totals: ms_out[s] (HOST float[KVC_STAGES]) and calls_out[s]
 * (HOST int32[KVC_STAGES]).  Stages: 0 projection+rotary, 1 attention,
 * 2 split merge, 3 commit, 4 output projection. */
enum { KVC_STAGE_PROJECT = 0, KVC_STAGE_ATTEND = 1, KVC_STAGE_MERGE = 2, KVC_STAGE_COMMIT = 3,
       KVC_STAGE_OUTPUT = 4, KVC_STAGES = 5 };
kvc_status kvc_profile_enable(kvc_cache* cache, int32_t slots);
kvc_status kvc_profile_read(kvc_cache* cache, float* ms_out, int32_t* calls_out);

/* Measurement helper: reads `bytes` of DEVICE memory at `buf` once with the
 * decode attention's access shape (contiguous 32 KiB units, 16-byte
 * non-temporal loads) and discards it, so that timing it gives the
 * achievable streaming-read bandwidth the decode attention is bound by
 * (Chapter 37, "From causal attention to managed LLM inference state":
 * re-reading the retained keys and values is the bandwidth bottleneck).
 * Launched on `hip_stream` (NULL: the default stream); no synchronisation.
 * `buf`: 16-byte aligned, `bytes` a positive multiple of 32768; `sink`: DEVICE,
 * 16 writable bytes (written only for one improbable xor of the data).
 * Errors: NULL_ARGUMENT, BAD_ARGUMENT (size or alignment), DEVICE. */
kvc_status kvc_stream_read(const void* buf, int64_t bytes, void* sink, void* hip_stream);

/* Measurement helper: the achievable bf16 matrix-core rate, the yardstick of
 * the suffix chunk's projection and causal attention (prefix-reuse note, "What
 * must be trimmed together": the suffix rows go through the model as one
 * chunk, a dense contraction) besides the nominal peak.  Launches, on
 * `hip_stream` (NULL: the default stream), two waves per SIMD on every compute
 * unit, each issuing `iterations` rounds of eight independent 32x32x16 bf16
 * MFMAs on register operands with no memory traffic; *flops_out (HOST)
 * receives the launch's floating-point operations, so timing the launch gives
 * FLOP/s.  `sink`: DEVICE, 16 writable bytes (written only for one improbable
 * sum).  No synchronisation.  Errors: NULL_ARGUMENT, BAD_ARGUMENT (iterations
 * outside [1, 2^24]), DEVICE. */
kvc_status kvc_mfma_rate(int64_t iterations, void* sink, void* hip_stream, double* flops_out);

/* ---- Model-wide session ----------------------------------------------
 * Several layers behind one token stream, with one cache per layer (Chapter
 * 37, "Give every decoder block its own state next": a model-wide session
 * binds one cache per decoder block and threads them through prefill and
 * decode; "Bind the state, calculate completely, then commit", the
 * prepared-row listing: every block prepares its row and the stack is
 * committed only when all of them succeeded; prefix-reuse note, "What must be
 * trimmed together": every layer's K, V and row positions are trimmed with
 * next_position as one unit).  The block is the
 * note's toy decoder block: input rows h0 = E[token] (+ absolute sinusoidal
 * encoding PE(p, 2i) = sin(p / 10000^(2i/D)), PE(p, 2i+1) = cos(same) at p =
 * next_position + i), then per layer h <- h + tanh(layer attention of h)
 * (the layer's W_o applied first when it has one).  In a session call every
 * layer computes first; the appends of all layers are then made only if no
 * layer failed, so any failure leaves every layer unchanged. */
typedef struct kvc_session kvc_session;

enum { KVC_PE_NONE = 0, KVC_PE_SINUSOIDAL = 1 };

/* Creates a session over `layers` (HOST array of n_layers >= 1 layer handles,
 * borrowed; all with the same model width and type) and one empty cache per
 * layer (batch, capacity, max_chunk_rows as kvc_cache_create).  embedding:
 * DEVICE [vocab, D] row-major in the accumulate type (double for F64 layers,
 * float otherwise), borrowed.  position_encoding: KVC_PE_NONE or
 * KVC_PE_SINUSOIDAL.  Allocates the caches and the session's row buffers.
 * Errors: NULL_ARGUMENT, BAD_ARGUMENT (counts, encoding, layers of different
 * width or type), then kvc_cache_create's errors (detail.layer names the layer). */
kvc_status kvc_session_create(const kvc_layer* const* layers, int32_t n_layers, const void* embedding,
                              int32_t vocab, int32_t position_encoding, int32_t batch, int32_t capacity,
                              int32_t max_chunk_rows, void* hip_stream, kvc_session** out);
void kvc_session_destroy(kvc_session* session);

/* Suffix chunk through every layer (prefix-reuse note: model.chunk of the
 * suffix tokens after the cached prefix).  tokens: DEVICE int32 [B, n_max];
 * n_rows: HOST int32[B] (NULL: all n_max), as kvc_continue_chunk.  out: DEVICE
 * [B, n_max, D] accumulate type, the last layer's rows (rows i >= n_b
 * untouched).  work: projection rows summed over the batch and the layers.
 * Errors: as kvc_continue_chunk for each layer in order (detail.layer), then
 * TOKEN_RANGE and the device-found errors of any layer; DEFERRED. */
kvc_status kvc_session_chunk(kvc_session* session, const int32_t* tokens, int32_t n_max, const int32_t* n_rows,
                             void* out, int32_t flags, kvc_work* work);

/* One cached decode step of the whole stack: tokens DEVICE int32 [B]; out
 * DEVICE [B, 1, D] accumulate type.  Errors: as kvc_session_chunk, FULL when a
 * sequence has no room. */
kvc_status kvc_session_decode(kvc_session* session, const int32_t* tokens, void* out, int32_t flags,
                              kvc_work* work);

/* Trims every layer to cut[b] rows and sets next_position[b] = cut[b] in one
 * step (prefix-reuse note, "What must be trimmed together"); flags as
 * kvc_truncate (KVC_TRUNCATE_KEEP_STALE_POSITION: the note's negative
 * control).  Errors: NULL_ARGUMENT, BAD_CUT, BAD_ARGUMENT, DEVICE. */
kvc_status kvc_session_truncate(kvc_session* session, const int32_t* cut, int32_t flags);
/* Every layer's lengths and next positions to 0 (kvc_reset per layer).
 * After a KVC_ASYNC call, session truncations and resets behave as
 * kvc_truncate and kvc_reset do (see KVC_ASYNC). */
kvc_status kvc_session_reset(kvc_session* session);
/* Waits for the stream and reports a deferred failure of any layer, as kvc_sync. */
kvc_status kvc_session_sync(kvc_session* session);
/* The session's cache of layer `layer`, borrowed for the read-only calls
 * (kvc_snapshot, kvc_lengths, kvc_cache_describe, kvc_copy_storage, ...);
 * compute, truncate and reset calls on it return BAD_ARGUMENT and
 * kvc_cache_destroy ignores it.  Errors: NULL_ARGUMENT, BAD_ARGUMENT. */
kvc_status kvc_session_layer_cache(kvc_session* session, int32_t layer, kvc_cache** out);

/* Last failure on the calling thread; never NULL. */
const kvc_error_detail* kvc_last_error(void);
/* Symbolic name of a status ("KVC_ERR_FULL"); never NULL. */
const char* kvc_status_name(kvc_status status);

#ifdef __cplusplus
}
#endif

#endif /* KVCACHE_H */
