/*
 * embtab.h -- C ABI of the MI355X (gfx950) sparse embedding layer.
 *
 * What is computed (all pages are web articles; none gives code):
 *  - Embedding lookup: an id selects one row of a table; tables hold most of a
 *    recommender's parameters and lookups are memory bound ("NVIDIA Merlin
 *    Distributed Embeddings" page, introduction and section "Background").
 *  - Pooled lookup: the rows of one multi-hot feature are pooled (summed or
 *    averaged) into one vector ("Merlin HugeCTR interview" page, section three,
 *    technique (5), and section two: thousands of feature fields per sample).
 *  - Sparse Adagrad: only rows touched by the batch are updated, with the
 *    Adagrad optimizer of the synthetic DLRM benchmarks ("NVIDIA Merlin
 *    Distributed Embeddings", section "Performance", synthetic models; HugeCTR
 *    interview, section three, technique (1): memory-saving sparse optimizer).
 *  - Deduplication: repeated ids are merged so each touched row is read and
 *    written once per pass (DeepRec page, section "model quality",
 *    EmbeddingVariable item 2; EcoRec page, section "research method").
 *  - Dynamic keys: a GPU hash table maps raw feature keys to rows and inserts
 *    unseen keys on first sight (OneFlow OneEmbedding page, section "ease of
 *    use"; HugeCTR interview, section two and section three technique (1)).
 *
 * Conventions shared by every call
 *  - Pointers are DEVICE pointers unless marked HOST.  The library allocates
 *    no device memory: weights, accumulators, state, hash slots, workspaces and
 *    outputs all belong to the caller and must outlive the handle (or the call).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls enqueue
 *    work and return without waiting; results are ready when the stream is.
 *    A handle must not be used on two streams at the same time.
 *  - Batches are CSR and table-major: bag b = t*B + s (table t, sample s),
 *    bag b holds occurrences offsets[b] .. offsets[b+1]-1, offsets[0] = 0 and
 *    offsets[T*B] = nnz.  `ids` are table-local rows (int64).  Pooled outputs
 *    and upstream gradients are fp32 [B, T, D], row-major.
 *  - Argument errors found on the host (null pointers, sizes, workspace too
 *    small) return at once and enqueue nothing.  Data errors found on the
 *    device set bits of a sticky error word in the state buffer, read and
 *    cleared by emb_status_sync:
 *      EMB_FLAG_OUT_OF_RANGE  an id outside [0, rows of its table) other
 *                             than EMB_ID_ABSENT: that occurrence
 *                             contributes 0 and updates nothing;
 *      EMB_FLAG_BAD_OFFSETS   offsets not starting at 0, decreasing, or not
 *                             ending at nnz: outputs of that call are
 *                             unspecified, but no memory outside the given
 *                             arrays is touched;
 *      EMB_FLAG_RESERVED_KEY  a raw key equal to EMB_EMPTY_KEY (id -1);
 *      EMB_FLAG_TABLE_FULL    see emb_hash_find_or_insert;
 *      EMB_FLAG_CACHE_FULL    tiered tables: a cache set had no slot for a
 *                             missing row (see emb_table_create_tiered); the
 *                             outputs of that batch and the values of its
 *                             rows are unspecified, every other row keeps its
 *                             value and no memory outside the given arrays
 *                             is touched.
 */
#ifndef EMBTAB_H
#define EMBTAB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct emb_table_s* emb_table_t;

typedef enum {
  EMB_OK = 0,
  EMB_ERR_INVALID_ARG = 1,
  EMB_ERR_UNSUPPORTED = 2,
  EMB_ERR_WORKSPACE = 3,
  EMB_ERR_OUT_OF_RANGE = 4,
  EMB_ERR_BAD_OFFSETS = 5,
  EMB_ERR_RESERVED_KEY = 6,
  EMB_ERR_TABLE_FULL = 7,
  EMB_ERR_HIP = 8,
  EMB_ERR_CACHE_FULL = 9
} emb_status_t;

#define EMB_FLAG_OUT_OF_RANGE 1u
#define EMB_FLAG_BAD_OFFSETS 2u
#define EMB_FLAG_RESERVED_KEY 4u
#define EMB_FLAG_TABLE_FULL 8u
#define EMB_FLAG_CACHE_FULL 32u

/* The all-ones key marks an empty hash slot and may not be used as a key. */
#define EMB_EMPTY_KEY 0xFFFFFFFFFFFFFFFFull

typedef enum { EMB_POOL_SUM = 0, EMB_POOL_MEAN = 1 } emb_pool_t;

typedef struct {
  int32_t num_tables;             /* T >= 1 */
  int32_t dim;                    /* D: 4 <= D <= 1024, D % 4 == 0, same for all tables */
  const int64_t* rows_per_table;  /* HOST [T], each >= 1; sum < 2^32 - 1.  For hashed
                                     tables: the row capacity, <= max_load * hash_capacity */
  float* weights;                 /* [sum rows, D] fp32, row-major; table t starts at row
                                     off_t = sum_{t' < t} rows_per_table[t'] */
  float* accum;                   /* Adagrad accumulator, same shape as weights */
  void* state;                    /* emb_state_bytes(T) bytes, 256-byte aligned */
  int32_t hashed;                 /* 0: ids are rows; 1: every table is keyed by raw u64 keys */
  int64_t hash_capacity;          /* slots per table, a power of two >= 16 (hashed only) */
  float max_load;                 /* rows_per_table[t] <= max_load * capacity; max_load <= 0.9 */
  void* hash_slots;               /* emb_hash_bytes(T, capacity) bytes (hashed only) */
  uint64_t seed;                  /* seed of the counter-based initialiser */
  float init_lo, init_hi;         /* dense tables: W ~ U[init_lo, init_hi) */
  float init_std;                 /* hashed tables: a new key's row ~ N(0, init_std^2) */
  float accum_init;               /* initial Adagrad accumulator of every row */
  int32_t init_storage;           /* 1: initialise weights, accum, slots and state;
                                     0: attach to storage written by an earlier handle */
  uint32_t* free_rows;            /* hashed only, may be NULL: device uint32 [sum rows], the
                                     queue of rows freed by emb_hash_evict (needed for it) */
} emb_table_desc_t;

/* Bytes of the caller-owned state buffer for T tables (row offsets, row
 * capacities, live-row counters, free-row queue positions, error word). */
size_t emb_state_bytes(int32_t num_tables);

/* Bytes of the hash slot array: T * capacity slots of 16 bytes,
 * slot = { uint64 key; uint64 row } with key EMB_EMPTY_KEY when empty; the home
 * slot of a key is SplitMix64's finalizer of the key masked to capacity - 1
 * and collisions probe linearly.  Returns 0 on invalid arguments. */
size_t emb_hash_bytes(int32_t num_tables, int64_t capacity);

/* Workspace bytes that any call on handle h with `batch` samples and `nnz`
 * occurrences needs (the maximum over all calls).  0 on invalid arguments.
 *
 * Size limits shared by every call that takes a batch: nnz < 2^32 - 16 and
 * batch * T < 2^32 - 16, because sorted positions and bag indices are 32-bit on
 * the device with the top values kept as sentinels.  Outside them a call
 * returns EMB_ERR_UNSUPPORTED before it enqueues anything, and this function
 * returns 0. */
size_t emb_workspace_bytes(emb_table_t h, int64_t batch, int64_t nnz);

/* Create a handle over caller-owned storage.  With init_storage = 1 it enqueues
 * the initialisation on `stream`: dense rows W[off_t + r, d] = init_lo +
 * u * (init_hi - init_lo) with u the top 24 bits of
 * SM(SM(SM(SM(seed) ^ t) ^ r) ^ d) (SM = one SplitMix64 step, Steele, Lea and
 * Flood 2014), accum = accum_init, slots empty, live-row counters 0.  The
 * handle itself is host memory; emb_table_destroy frees it. */
emb_status_t emb_table_create(const emb_table_desc_t* desc, void* stream, emb_table_t* out);
emb_status_t emb_table_destroy(emb_table_t h);

/* Raw keys -> table-local rows, inserting unseen keys (OneFlow OneEmbedding
 * page, section "ease of use"; HugeCTR interview, section three, technique (1)).
 *   offsets [T*B+1] int64, keys [nnz] uint64 (CSR, table-major like ids),
 *   ids_out [nnz] int64.
 * A key already in table t's map gets its row.  A key not yet there gets row
 * n_live[t] + r, where r ranks its first occurrence among this call's new keys
 * of table t (in occurrence order); its weights are initialised to
 * init_std * z, z the Box-Muller normal of the draws SM-chain(seed, t, key,
 * 2d) and (.., 2d+1), and its accumulator to accum_init.  All-or-nothing: if
 * the new keys of any table would exceed rows_per_table, nothing is inserted,
 * new keys get id -1 and EMB_FLAG_TABLE_FULL is set.  Reserved keys get -1.
 * With eviction (emb_hash_evict) a new key takes a queued free row before
 * row n_live[t], and the call is full when the new keys outnumber the queued
 * rows plus the rows never used.
 * Row assignment is deterministic; slot positions are not (several layouts
 * are correct).  Needs a hashed handle. */
emb_status_t emb_hash_find_or_insert(emb_table_t h, const int64_t* offsets,
                                     const uint64_t* keys, int64_t batch, int64_t nnz,
                                     int64_t* ids_out, void* ws, size_t ws_bytes,
                                     void* stream);

/* ------------------------------------------------------------------------
 * The pooled embeddings' first consumer fused with the lookup: the DLRM dot
 * feature interaction (OneFlow OneEmbedding page, section "operator
 * optimisation": a fused dot-interaction operator for DLRM; HugeCTR
 * interview, section three, technique (5): pooling fused with the next
 * layer, so the pooled vectors do not go through device memory).  The pages
 * name the operator only; this is the DLRM model's definition.  Per sample s,
 * z_0 = dense[s, :] and z_{t+1} = the pooled bag (t, s) as emb_bag_forward
 * computes it; the output row is
 *   out[s] = [z_0 (D values), z_i . z_j for i = 1..T, j = 0..i-1]
 * (the strict lower triangle of Z Z^T in row-major order), of length
 * emb_interact_out_dim(h) = D + (T+1)T/2.  The [B, T, D] pooled tensor is not
 * written.  Needs T + 1 <= 32, D % 16 == 0 and D <= 256 (EMB_ERR_UNSUPPORTED
 * otherwise, and on tiered tables).  dense: [B, D] fp32, 16-byte aligned;
 * out: [B, D + (T+1)T/2] fp32.  Ids as for emb_bag_forward (EMB_ID_ABSENT is
 * a zero vector; out-of-range ids and bad offsets set the usual error bits).
 * Dot products accumulate in fp32 on the matrix cores. */
int64_t emb_interact_out_dim(emb_table_t h);
emb_status_t emb_bag_forward_interact(emb_table_t h, const int64_t* offsets, const int64_t* ids,
                                      int64_t batch, int64_t nnz, emb_pool_t pool,
                                      const float* dense, float* out, void* stream);
/* Backward of emb_bag_forward_interact for the same batch (the pooled vectors
 * are gathered again): with g_ij = g_ji = grad_out[s, pair (i, j)] and
 * g_ii = 0, dz_i = sum_j g_ij z_j;
 *   grad_dense[s] = grad_out[s, 0:D] + dz_0          [B, D]
 *   grad_pooled[s, t] = dz_{t+1}                      [B, T, D]
 * grad_pooled is the grad_out of emb_bag_backward_adagrad(_prepared). */
emb_status_t emb_interact_backward(emb_table_t h, const int64_t* offsets, const int64_t* ids,
                                   int64_t batch, int64_t nnz, emb_pool_t pool,
                                   const float* dense, const float* grad_out, float* grad_dense,
                                   float* grad_pooled, void* stream);

/* Eviction of hashed keys (DeepRec page, section "model quality",
 * EmbeddingVariable item 1: feature eviction policies; the page gives none).
 * The reading: every key whose row was last used before `before` leaves its
 * table and its row is freed.  Freed rows wait in a queue per table
 * (desc->free_rows; rows freed by one call in ascending order) and are handed
 * to new keys, oldest first, before rows never used; a reused row is
 * initialised like any new key's.  The slot arrays are rebuilt from the
 * remaining keys, and keys counted for admission but without a row are
 * dropped (pass the admission key_counts to have them cleared; NULL if
 * admission is not used).
 *   row_last_used: device uint32 [sum rows], by global row, the caller's
 *   record of each row's last use (for instance the row_periods written by
 *   emb_bag_backward_adagrad_decay_prepared with period = step; with rho = 1
 *   that is plain Adagrad).  Rows that hold no key are ignored.  Every row
 *   the call frees gets EMB_PERIOD_FRESH there, so that when it is the
 *   row_periods array the key that next receives the row starts from an
 *   undiscounted accumulator.
 *   ws: emb_hash_evict_workspace_bytes(h) bytes, 256-byte aligned (about
 *   16 bytes per slot plus one per row).
 * EMB_ERR_UNSUPPORTED on dense tables or without desc->free_rows. */
size_t emb_hash_evict_workspace_bytes(emb_table_t h);
emb_status_t emb_hash_evict(emb_table_t h, uint32_t* row_last_used, uint32_t before,
                            uint32_t* key_counts, void* ws, size_t ws_bytes, void* stream);
/* HOST out [T]: rows waiting in each table's free-row queue (waits for the stream). */
emb_status_t emb_hash_free_rows(emb_table_t h, void* stream, int64_t* queued_out);

/* An id that marks an absent feature: the forward treats it as a zero row
 * (counted in a mean bag's length), the backward updates nothing, and no
 * error bit is set.  emb_hash_find_or_insert_admit returns it for keys that
 * are not admitted yet. */
#define EMB_ID_ABSENT (-2)

/* emb_hash_find_or_insert with frequency admission (DeepRec page, section
 * "model quality", EmbeddingVariable item 1: features are admitted before
 * they get a row, so rare keys cost no row; the page gives no rule).  The
 * reading: a key without a row counts its occurrences over calls in
 * key_counts; in the call where its count reaches min_count it gets a row
 * (in order of its first occurrence in that call, initialised as a new key)
 * and every occurrence of it in that call gets the row.  Until then its
 * occurrences get EMB_ID_ABSENT.  A counted key holds a hash slot.  A call
 * that is full (rows or slots) admits nothing: keys that would have got a
 * row get -1, EMB_FLAG_TABLE_FULL is set, and their counts stay, so a later
 * call with room admits them at once; when slots run out, which keys got a
 * slot (and a count) is unspecified.
 *   key_counts: device uint32 [T * hash_capacity], caller-owned, 4-byte
 *   aligned, zero before the first call and kept between calls.
 *   min_count <= 1: same as emb_hash_find_or_insert (key_counts may be NULL).
 * EMB_ERR_INVALID_ARG for a null or misaligned key_counts with
 * min_count > 1; otherwise as emb_hash_find_or_insert. */
emb_status_t emb_hash_find_or_insert_admit(emb_table_t h, const int64_t* offsets,
                                           const uint64_t* keys, int64_t batch, int64_t nnz,
                                           int64_t* ids_out, uint32_t min_count,
                                           uint32_t* key_counts, void* ws, size_t ws_bytes,
                                           void* stream);

/* Pooled lookup ("Merlin Distributed Embeddings", introduction and
 * "Background"; HugeCTR interview, section three, technique (5)):
 *   out[s, t, :] = c_b * sum_{j in bag b} W[off_t + ids[j], :],  b = t*B + s,
 *   c_b = 1 (EMB_POOL_SUM) or 1 / (offsets[b+1] - offsets[b]) (EMB_POOL_MEAN);
 *   an empty bag gives 0.  fp32 accumulation.  `ws` may be NULL. */
emb_status_t emb_bag_forward(emb_table_t h, const int64_t* offsets, const int64_t* ids,
                             int64_t batch, int64_t nnz, emb_pool_t pool, float* out,
                             void* ws, size_t ws_bytes, void* stream);

/* Backward of emb_bag_forward fused with one element-wise Adagrad step on the
 * touched rows (Adagrad per the synthetic benchmarks of "Merlin Distributed
 * Embeddings", section "Performance"; textbook form of Duchi, Hazan and
 * Singer 2011):
 *   rows_j = off_t + ids[j]; stable sort by row; unique rows and inverse;
 *   g_u = sum over occurrences j of row u of c_b(j) * grad_out[s(j), t(j), :]
 *   G_u += g_u * g_u;   W_u -= lr * g_u / (sqrt(G_u) + eps)       (per element)
 * Each touched row gets exactly one step however often it occurs; rows not in
 * the batch are neither read nor written.  Deterministic: no float atomics.
 *   grad_out [B, T, D] fp32.  ws: emb_workspace_bytes(h, batch, nnz) bytes. */
emb_status_t emb_bag_backward_adagrad(emb_table_t h, const int64_t* offsets,
                                      const int64_t* ids, int64_t batch, int64_t nnz,
                                      emb_pool_t pool, const float* grad_out, float lr,
                                      float eps, void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * emb_bag_backward_adagrad with its workspace taken from a buffer of
 * EMB_NOALLOC_SCRATCH_BYTES bytes that the library holds on each device, from
 * its load onto that device until the process ends.  Same arguments, result
 * and errors as emb_bag_backward_adagrad, without ws and ws_bytes; it
 * allocates and frees nothing.  EMB_ERR_WORKSPACE (nothing enqueued) when
 * emb_workspace_bytes(h, batch, nnz) > EMB_NOALLOC_SCRATCH_BYTES; EMB_ERR_HIP
 * when the buffer's device address could not be resolved at handle creation.
 * Every call on one device shares that device's buffer, which keeps the last
 * call's contents (each call writes what it reads): calls ordered on one
 * stream are safe, calls that overlap in time on one device (other streams,
 * other threads, other handles) race and give undefined results. */
#define EMB_NOALLOC_SCRATCH_BYTES (64u << 20)
emb_status_t emb_bag_backward_adagrad_noalloc(emb_table_t h, const int64_t* offsets,
                                              const int64_t* ids, int64_t batch, int64_t nnz,
                                              emb_pool_t pool, const float* grad_out, float lr,
                                              float eps, void* stream);

/* The same backward split in two, so that the id-only stages can overlap the
 * forward gather (they need offsets and ids but not grad_out):
 *   emb_bag_prepare                    occurrence keys, stable sort, run
 *                                      heads and the unique rows, their
 *                                      segment offsets and the inverse map,
 *                                      left in `ws`;
 *   emb_bag_backward_adagrad_prepared  segmented reduction + Adagrad from a
 *                                      workspace prepared for the same batch,
 *                                      nnz and pool (same semantics as
 *                                      emb_bag_backward_adagrad).
 * Typical use: prepare on a second stream right after the ids are known, run
 * emb_bag_forward on the main stream, make the main stream wait for the second
 * one, then call the prepared backward.  Calling the prepared backward on a
 * workspace that was not prepared for this batch updates unspecified rows (no
 * memory outside W, G and ws is touched). */
emb_status_t emb_bag_prepare(emb_table_t h, const int64_t* offsets, const int64_t* ids,
                             int64_t batch, int64_t nnz, emb_pool_t pool, void* ws,
                             size_t ws_bytes, void* stream);
/* emb_bag_forward from a workspace prepared for this batch (same result).
 * When every bag holds exactly one id it gathers the rows in sorted order, so
 * a row shared by many bags is read once per reduction chunk and W is walked
 * in ascending order; otherwise it runs the same kernel as emb_bag_forward. */
emb_status_t emb_bag_forward_prepared(emb_table_t h, const int64_t* offsets, const int64_t* ids,
                                      int64_t batch, int64_t nnz, emb_pool_t pool, float* out,
                                      void* ws, size_t ws_bytes, void* stream);
/* emb_bag_forward_prepared writing the int8 exchange payload of a table-wise
 * split instead of fp32 rows: for every bag b' = s*T + t (the rows of `out`),
 * codes[b', :] and scales[b'] are what emb_quantize_rows_int8 gives for the
 * pooled row; the fp32 rows are never written (a quarter of the output bytes
 * plus 4 bytes per bag).  codes [B*T, D] int8 and scales [B*T] fp32, both
 * 4-byte aligned.  On one-hot batches the pooled row is the table row itself,
 * so the payload is exactly the quantized row; on multi-hot batches it is
 * quantized from the fp32 sum, whose rounding may move a code by one against
 * the quantized exact sum.  Errors as emb_bag_forward_prepared. */
emb_status_t emb_bag_forward_prepared_int8(emb_table_t h, const int64_t* offsets,
                                           const int64_t* ids, int64_t batch, int64_t nnz,
                                           emb_pool_t pool, int8_t* codes, float* scales,
                                           void* ws, size_t ws_bytes, void* stream);
/* emb_bag_backward_adagrad_prepared with the upstream gradient given as the
 * int8 exchange payload (what the table owner of a table-wise split receives):
 * grad_codes [B*T, D] int8 and grad_scales [B*T] fp32, both 4-byte aligned;
 * the gradient of bag b' is grad_codes[b', :] * grad_scales[b'] in fp32, so
 * the result equals emb_bag_backward_adagrad_prepared on the output of
 * emb_dequantize_rows_int8 bit for bit, reading a quarter of the bytes.
 * Errors as emb_bag_backward_adagrad_prepared. */
emb_status_t emb_bag_backward_adagrad_prepared_int8(emb_table_t h, int64_t batch, int64_t nnz,
                                                    emb_pool_t pool, const int8_t* grad_codes,
                                                    const float* grad_scales, float lr,
                                                    float eps, void* ws, size_t ws_bytes,
                                                    void* stream);
emb_status_t emb_bag_backward_adagrad_prepared(emb_table_t h, int64_t batch, int64_t nnz,
                                               emb_pool_t pool, const float* grad_out, float lr,
                                               float eps, void* ws, size_t ws_bytes,
                                               void* stream);

/* emb_bag_backward_adagrad_prepared with the Adagrad Decay optimizer (DeepRec
 * page, section "model quality", Adagrad Decay Optimizer: the accumulator is
 * discounted per period, every sample of one period alike, so that long
 * incremental training keeps learning).  The page gives no formula; this is
 * the reading: at every period boundary every accumulator is multiplied by
 * rho.  It is applied lazily, when a row is next updated:
 *   s = row_periods[row];  if (period > s) G_row *= rho^(period - s)
 *   then the Adagrad step of emb_bag_backward_adagrad;
 *   row_periods[row] = max(s, period).
 * row_periods: device uint32 [sum of rows], caller-owned, 4-byte aligned,
 * all 0 at the start of training for dense tables (rows start in period 0),
 * all EMB_PERIOD_FRESH for hashed tables; only touched rows are read and
 * written.  EMB_PERIOD_FRESH marks a row whose key is new (never updated, or
 * freed by emb_hash_evict and handed to another key): its accumulator is the
 * initial one, which the row's next update does not discount; that update
 * sets the row's period to `period`.  rho in (0, 1]; rho = 1 is plain Adagrad.  period:
 * the caller's step / period length.  rho^k is computed as
 * exp2f(k * log2(rho)) in fp32.  EMB_ERR_INVALID_ARG for a null or misaligned
 * row_periods or rho outside (0, 1]; EMB_ERR_UNSUPPORTED on tiered tables. */
#define EMB_PERIOD_FRESH 0xFFFFFFFFu
emb_status_t emb_bag_backward_adagrad_decay_prepared(emb_table_t h, int64_t batch, int64_t nnz,
                                                     emb_pool_t pool, const float* grad_out,
                                                     float lr, float eps, float rho,
                                                     uint32_t period, uint32_t* row_periods,
                                                     void* ws, size_t ws_bytes, void* stream);

/* Waits for `stream`, returns the highest-priority device error (TABLE_FULL,
 * CACHE_FULL, RESERVED_KEY, BAD_OFFSETS, OUT_OF_RANGE, in that order) or
 * EMB_OK, stores the raw EMB_FLAG_* bits in *flags_out (HOST, may be NULL)
 * and clears them. */
emb_status_t emb_status_sync(emb_table_t h, void* stream, uint32_t* flags_out);

/* HOST n_live_out[T]: rows handed out so far in each hashed table (waits for
 * the stream). */
emb_status_t emb_hash_n_live(emb_table_t h, void* stream, int64_t* n_live_out);

/* For table t: key_of_row[r] = the key mapped to row r, for r < n_live[t]
 * (the map is a bijection onto [0, n_live)); key_of_row [rows_per_table[t]]. */
emb_status_t emb_hash_export(emb_table_t h, int32_t table, uint64_t* key_of_row,
                             void* stream);

/* The sort / unique stage of emb_bag_backward_adagrad with its results copied
 * out (same kernels).  sorted_rows[nnz] (global rows; an out-of-range
 * occurrence has 0xFFFFFFFF and sorts last), perm[nnz] (occurrence index of
 * each sorted entry; stable), unique[nnz] (first num_unique used, ascending),
 * counts[nnz], seg_off[nnz+1] (first num_unique+1 used), inverse[nnz]
 * (unique index of each occurrence, 0xFFFFFFFF when out of range), num_unique
 * (device uint32).  Outputs other than num_unique may be NULL. */
emb_status_t emb_debug_sort_unique(emb_table_t h, const int64_t* offsets, const int64_t* ids,
                                   int64_t batch, int64_t nnz, uint32_t* sorted_rows,
                                   uint32_t* perm, uint32_t* unique, uint32_t* counts,
                                   uint32_t* seg_off, uint32_t* inverse, uint32_t* num_unique,
                                   void* ws, size_t ws_bytes, void* stream);

/* Measurement hook.  Phases of the calls, in launch order:
 *   EMB_PHASE_FORWARD  the pooled-gather kernel of emb_bag_forward;
 *   EMB_PHASE_KEYS     occurrence keys of emb_bag_backward_adagrad;
 *   EMB_PHASE_SORT     all radix passes;
 *   EMB_PHASE_UNIQUE   run heads, the unique index of each reduction chunk,
 *                      and unique / seg_off / inverse;
 *   EMB_PHASE_REDUCE   the fused segmented-reduction + Adagrad kernel (which
 *                      also finishes the rows whose occurrences span its
 *                      blocks);
 *   EMB_PHASE_FIXUP    reserved: no events are recorded for it (rows spanning
 *                      reduction blocks are finished inside the reduction);
 *   EMB_PHASE_HASH     all of emb_hash_find_or_insert;
 *   EMB_PHASE_CACHE    tiered tables: the kernel of emb_bag_prepare (or of
 *                      the one-call backward) that writes evicted rows back
 *                      to host memory and fetches the missing ones.
 * When `events` is not NULL, later calls on h record events[2p] (if not NULL)
 * just before phase p and events[2p+1] (if not NULL) just after it, with
 * hipEventRecord on the call's stream.  The array (2 * EMB_NUM_PHASES
 * hipEvent_t handles) is copied; the events stay the caller's.  NULL turns
 * recording off. */
typedef enum {
  EMB_PHASE_FORWARD = 0,
  EMB_PHASE_KEYS = 1,
  EMB_PHASE_SORT = 2,
  EMB_PHASE_UNIQUE = 3,
  EMB_PHASE_REDUCE = 4,
  EMB_PHASE_FIXUP = 5,
  EMB_PHASE_HASH = 6,
  EMB_PHASE_CACHE = 7,
  EMB_NUM_PHASES = 8
} emb_phase_t;
emb_status_t emb_set_phase_events(emb_table_t h, void* const* events);

/* Human-readable name of a status code (static string). */
const char* emb_status_string(emb_status_t s);

/* ------------------------------------------------------------------------
 * Tiered tables: weights and accumulators in host memory, an HBM cache of hot
 * rows (DeepRec page, section "deployment and serving", multi-level hybrid
 * embedding storage: frequently used features on fast memory, rarely used ones
 * on cheaper memory; OneFlow OneEmbedding page, closing section: layered
 * storage for tables beyond device memory).  Every result equals that of the
 * same table held wholly in device memory.
 *
 * The cache holds cache_rows rows in sets of EMB_CACHE_WAYS; a row's set is
 * SplitMix64's finalizer of the row modulo the number of sets (a power of
 * two).  emb_bag_prepare on a tiered table also looks every distinct row of
 * the batch up: a hit marks its slot used by this batch; a miss claims the
 * least recently used slot of its set that neither this batch nor the one
 * prepared just before it uses, writes that slot's row (weights and
 * accumulator) back to host memory and fetches the missing row into it.  So
 * the prepare of batch i+1 may run beside the forward and backward of batch
 * i on another stream, and must wait for the backward of batch i-1.  A set
 * has to hold the distinct rows that two consecutive batches place in it;
 * when it cannot, EMB_FLAG_CACHE_FULL is raised.  The forward and backward of
 * a batch run on the cache (emb_bag_forward_prepared,
 * emb_bag_backward_adagrad_prepared, or the one-call
 * emb_bag_backward_adagrad); emb_bag_forward without a prepared workspace,
 * hashed tiered tables and emb_hash_* are not supported.  Rows updated in the
 * cache reach host memory when evicted or at emb_cache_flush. */
#define EMB_CACHE_WAYS 16

typedef struct {
  float* host_weights;  /* [sum rows, D] fp32, host memory the device can read and write
                           (pinned: hipHostMalloc or torch pin_memory), 16-byte aligned */
  float* host_accum;    /* same shape */
  int64_t cache_rows;   /* C: EMB_CACHE_WAYS * 2^k, C <= sum rows */
  void* cache_state;    /* device, emb_cache_state_bytes(C) bytes, 256-byte aligned */
} emb_tier_desc_t;

/* Bytes of the cache state: per slot the row it holds and the step it was
 * last used at, plus counters.  0 if cache_rows is not EMB_CACHE_WAYS * 2^k. */
size_t emb_cache_state_bytes(int64_t cache_rows);

/* Like emb_table_create, with desc->weights / desc->accum the HBM cache
 * ([C, D] each) and the table itself in tier->host_weights / host_accum.
 * init_storage = 1 initialises the host rows exactly as a dense table's (same
 * counter-based values) and empties the cache.  init_storage = 0 attaches to
 * host rows and a state written by an earlier handle, which must have called
 * emb_cache_flush after its last backward (the cache is not carried over: it
 * starts empty).  desc->hashed must be 0 (else EMB_ERR_UNSUPPORTED).
 * EMB_ERR_INVALID_ARG for a null tier, null or misaligned pointers,
 * cache_rows that emb_cache_state_bytes rejects or above the table's total
 * rows. */
emb_status_t emb_table_create_tiered(const emb_table_desc_t* desc, const emb_tier_desc_t* tier,
                                     void* stream, emb_table_t* out);

/* Writes every row held in the cache back to host memory (the cache keeps
 * them).  Afterwards the host arrays hold the table's current values. */
emb_status_t emb_cache_flush(emb_table_t h, void* stream);

/* emb_bag_prepare in two parts, for tiered tables: emb_bag_prepare_ids runs
 * the id-only stages (keys, sort, run heads; no cache access) and
 * emb_cache_prepare the cache stages of the same workspace (lookup, claim,
 * write-back and fetch, slot keys).  emb_bag_prepare_ids followed by
 * emb_cache_prepare equals emb_bag_prepare.  Split, the id stages of batch
 * i+2, the cache stage of batch i+1 and the forward and backward of batch i
 * can run on three streams (three workspaces).  emb_cache_prepare calls come
 * in batch order, and each waits for the backward of the batch two before
 * it, as emb_bag_prepare does.  On a dense table emb_bag_prepare_ids is
 * emb_bag_prepare and emb_cache_prepare returns EMB_ERR_UNSUPPORTED. */
emb_status_t emb_bag_prepare_ids(emb_table_t h, const int64_t* offsets, const int64_t* ids,
                                 int64_t batch, int64_t nnz, emb_pool_t pool, void* ws,
                                 size_t ws_bytes, void* stream);
emb_status_t emb_cache_prepare(emb_table_t h, int64_t batch, int64_t nnz, void* ws,
                               size_t ws_bytes, void* stream);

/* HOST out: cumulative counts over all prepares of h (waits for the stream):
 * distinct rows looked up, misses (rows fetched from host memory) and
 * write-backs (evicted rows written to host memory; emb_cache_flush is not
 * counted). */
emb_status_t emb_cache_stats(emb_table_t h, void* stream, int64_t* lookups, int64_t* misses,
                             int64_t* writebacks);

/* ---------------------------------------------------------------- stream ceilings
 * What HBM sustains on this device for plain streams, the yardstick the
 * benchmark reports beside the published peak (every kernel of the path is
 * bound by HBM bandwidth: "NVIDIA Merlin Distributed Embeddings" page,
 * section "Background").  Hand-written dwordx4 kernels, one 16-byte item per
 * thread and one 256-thread block per 4 KiB (the fastest form measured on
 * MI355X); copy loads and stores are non-temporal, fill stores plain, read
 * loads non-temporal.  Asynchronous on `stream` (a hipStream_t; NULL is the
 * null stream).
 *   emb_stream_copy  dst[0, bytes) = src[0, bytes)   (bytes read + bytes written)
 *   emb_stream_fill  dst[0, bytes) = value, as fp32 words
 *   emb_stream_read  reads src[0, bytes), four items per thread; writes one
 *                    float per wave (a sum of its words) to sink, which must
 *                    hold emb_stream_read_sink_floats(bytes) floats
 * All pointers are device pointers, 16-byte aligned; bytes a multiple of 16
 * (0 launches nothing).  EMB_ERR_INVALID_ARG for null or misaligned pointers,
 * a bad size or a short sink; EMB_ERR_HIP if the launch fails.  The buffers
 * stay the caller's. */
emb_status_t emb_stream_copy(void* dst, const void* src, size_t bytes, void* stream);
emb_status_t emb_stream_fill(void* dst, float value, size_t bytes, void* stream);
size_t emb_stream_read_sink_floats(size_t bytes);
emb_status_t emb_stream_read(const void* src, size_t bytes, float* sink, size_t sink_floats,
                             void* stream);

/* ---------------------------------------------------------------- int8 exchange payload
 * A table-wise split over ranks exchanges the pooled embeddings [B, T, D]
 * (forward) and their gradients (backward); the OneFlow OneEmbedding page
 * (section "quantized compression") quantizes that payload from float to
 * int8 before the exchange and dequantizes it after.  The page gives no
 * scheme; this is the reading, per row of `dim` values (rows = B * T for a
 * pooled tensor), each step in fp32:
 *   amax = max_d |x_d|;  amax == 0: scale 0 and codes 0;
 *   otherwise code_d = round-to-nearest-even(x_d * (127 / amax)), clamped to
 *   [-127, 127], and scale = amax / 127;
 *   dequantized y_d = code_d * scale.
 * x: [rows, dim] fp32, 16-byte aligned; codes: [rows, dim] int8, 4-byte
 * aligned; scales: [rows] fp32, 4-byte aligned; y: [rows, dim] fp32, 16-byte
 * aligned.  dim a multiple of 4 in [4, 1024].  x must be finite.  Device
 * pointers, asynchronous on `stream`; rows = 0 launches nothing.
 * EMB_ERR_INVALID_ARG for bad sizes, null or misaligned pointers; EMB_ERR_HIP
 * if the launch fails.  The payload is 1/4 of the fp32 bytes plus 4 bytes
 * per row. */
emb_status_t emb_quantize_rows_int8(const float* x, int64_t rows, int32_t dim, int8_t* codes,
                                    float* scales, void* stream);
emb_status_t emb_dequantize_rows_int8(const int8_t* codes, const float* scales, int64_t rows,
                                      int32_t dim, float* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* EMBTAB_H */
