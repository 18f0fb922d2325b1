// Internal declarations of the gfx950 sparse embedding library: handle,
// state-buffer layout, workspace plan, device helpers and kernel launchers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <vector>

#include "embtab.h"

namespace embtab {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr uint64_t kEmptyKey = 0xFFFFFFFFFFFFFFFFull;
constexpr uint64_t kUnsetRow = 0xFFFFFFFFFFFFFFFFull;  // row word of an empty slot
constexpr uint64_t kPendingBit = 1ull << 62;           // row word = kPendingBit | first j
// row word of a key that is counted but not admitted yet (frequency admission);
// above every kPendingBit | j, so the first-occurrence atomicMin still works
constexpr uint64_t kCandRow = 0xFFFFFFFFFFFFFFFEull;
constexpr int64_t kAbsentId = -2;  // id of a feature without a row: looks up 0, no error
constexpr uint32_t kFreshPeriod = EMB_PERIOD_FRESH;  // Adagrad Decay: a row whose key is new
constexpr uint32_t kNoRow = 0xFFFFFFFFu;
constexpr int kMaxTables = 1024;

// Sort and unique tiles: 256 threads x 16 keys.
constexpr int kSortThreads = 256;
constexpr int kSortItems = 16;
constexpr int kSortTile = kSortThreads * kSortItems;
constexpr int kMaxDigitBits = 9;
constexpr int kMaxRadix = 1 << kMaxDigitBits;

// ---------------------------------------------------------------- state buffer
// [0, 256): uint32 error word (+ padding); then int64 row_off[T+1], rows[T],
// n_live[T], q_head[T], q_tail[T], slots_used[T].
struct StateView {
  uint32_t* flags;
  int64_t* row_off;
  int64_t* rows;
  int64_t* n_live;  // rows ever handed out (rows >= n_live were never used)
  // Free-row queue of table t (hashed tables with eviction): entries
  // q_head[t] .. q_tail[t] - 1, entry q stored at free_rows[row_off[t] + q % rows[t]]
  // (a ring: at most rows[t] rows are free at once).
  int64_t* q_head;
  int64_t* q_tail;
  // Hashed tables: slots holding a key (live keys and keys counted for
  // admission), bounded by kMaxSlotLoad of the capacity.
  int64_t* slots_used;
};

inline size_t state_bytes(int T) {
  size_t b = 256 + sizeof(int64_t) * (size_t)(6 * T + 1);
  return (b + 255) & ~(size_t)255;
}

inline StateView state_view(void* state, int T) {
  char* p = static_cast<char*>(state);
  StateView v;
  v.flags = reinterpret_cast<uint32_t*>(p);
  v.row_off = reinterpret_cast<int64_t*>(p + 256);
  v.rows = v.row_off + (T + 1);
  v.n_live = v.rows + T;
  v.q_head = v.n_live + T;
  v.q_tail = v.q_head + T;
  v.slots_used = v.q_tail + T;
  return v;
}

// ---------------------------------------------------------------- handle
struct Handle {
  int T = 0, D = 0;
  std::vector<int64_t> rows, row_off;  // host copies
  int64_t total_rows = 0;
  float* W = nullptr;
  float* G = nullptr;
  void* state = nullptr;
  StateView sv{};
  uint32_t* free_rows = nullptr;  // hashed tables with eviction
  bool hashed = false;
  int64_t capacity = 0;
  void* slots = nullptr;
  uint64_t seed = 0;
  float lo = 0, hi = 0, stdv = 0, accum0 = 0;
  bool timing = false;
  hipEvent_t events[2 * EMB_NUM_PHASES] = {};
  int cus = 256;  // compute units of the device current at creation
  int device = -1;  // the device current at creation (-1: none visible)
  // this device's copy of the library's own workspace, for callers that
  // cannot allocate one (null if its address could not be resolved)
  void* scratch = nullptr;
  // tiered tables: W / G above are the HBM cache, the table is in host memory
  bool tiered = false;
  float* hostW = nullptr;
  float* hostG = nullptr;
  int64_t cache_rows = 0;
  uint32_t cache_sets = 0;  // a power of two
  char* cache_state = nullptr;
  uint32_t step = 0;  // prepares so far (cache recency stamps)
};

// Cache state of a tiered table: counters, then per slot the row it holds
// (kNoRow when empty) and the step it was last used at (0: never).
struct CacheView {
  uint64_t* counters;  // [0] distinct rows looked up, [1] misses, [2] write-backs
  uint32_t* tag;
  uint32_t* stamp;
};
constexpr int kCacheWays = 16;
inline size_t cache_state_bytes(int64_t C) {
  auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
  return 256 + 2 * up(sizeof(uint32_t) * (size_t)C);
}
inline CacheView cache_view(char* st, int64_t C) {
  auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
  CacheView v;
  v.counters = reinterpret_cast<uint64_t*>(st);
  v.tag = reinterpret_cast<uint32_t*>(st + 256);
  v.stamp = reinterpret_cast<uint32_t*>(st + 256 + up(sizeof(uint32_t) * (size_t)C));
  return v;
}

// Measurement hook: events recorded around a phase when the caller set them.
inline void phase_mark(const Handle& h, int phase, bool end, hipStream_t s) {
  if (!h.timing) return;
  hipEvent_t e = h.events[2 * phase + (end ? 1 : 0)];
  if (e) (void)hipEventRecord(e, s);
}

// Lanes that share one embedding row (a power of two <= 64) and float4s per lane.
inline int subgroup_lanes(int D) {
  int v = D / 4;
  int sg = 1;
  while (sg < v && sg < 64) sg <<= 1;
  return sg;
}
inline int vec_per_lane(int D) {
  int sg = subgroup_lanes(D);
  return (D / 4 + sg - 1) / sg;
}
// Sorted occurrences per reduction chunk.
// Sorted positions per reduction chunk: at least kChunkMin, and a whole number
// of sub-group rounds (MPL metadata entries per lane).
#ifndef EMBTAB_CHUNK_MIN
#define EMBTAB_CHUNK_MIN 32
#endif
constexpr int kChunkMin = EMBTAB_CHUNK_MIN;
template <int SG>
constexpr int chunk_rounds() {
  return SG >= kChunkMin ? 1 : kChunkMin / SG;
}
inline int chunk_len(int D) {
  int sg = subgroup_lanes(D);
  return sg >= kChunkMin ? sg : kChunkMin;
}
// Sorted positions per reduction block (256 threads: 256 / SG chunks).
inline uint32_t reduce_block_positions(int D) {
  return (uint32_t)(chunk_len(D) * (256 / subgroup_lanes(D)));
}

// ---------------------------------------------------------------- workspace plan
struct Plan {
  int64_t nnz = 0, B = 0;
  int T = 0, D = 0;
  int passes = 0;
  int shift[4] = {0, 0, 0, 0};
  int dbits[4] = {0, 0, 0, 0};
  int64_t ntiles = 0;   // sort / unique tiles
  int64_t nchunks = 0;  // reduction chunks
  int chunk = 0;
  size_t keysA, valsA, keysB, valsB, gr;
  size_t kblk;  // per key block: 1 when every bag of the block holds its own occurrence
  size_t sgr, sscale;  // grad row and mean scale of each sorted occurrence
  size_t tile_hist, digit_tot;
  size_t unique, seg_off, counts, inverse;
  size_t misc;  // uint32[64 + 3T]
  size_t part_head, part_tail;
  // Runs crossing reduction blocks: span_u[b] = unique index of the run that
  // crosses the edge before block b (kNoRow: none), from the prepare;
  // span_cnt[b] = blocks arrived at the span that starts in block b (zeroed
  // by the prepare, left at zero by the block that finishes the span).
  size_t span_u, span_cnt;
  uint32_t bp = 0;  // sorted positions per reduction block
  size_t chunk_base;  // heads in the earlier chunks of the chunk's 256-position block
  size_t head_base;   // heads before each 256-position block (nnz / 256 + 1)
  size_t h_slot, h_first, h_tcnt, h_tb, h_fresh;  // hash find-or-insert
  size_t c_slot, c_miss, c_vict, c_mslot, c_rowmap;  // tiered: cache lookup
  size_t total = 0;
};

// misc[] words
enum : int {
  kMiscNumUnique = 0,
  kMiscNumValid = 1,
  kMiscHashAbort = 2,  // the hash call's offsets are invalid: it inserts nothing
  kMiscHashOverflow = 3,
  // some bag of the prepared batch does not hold exactly one id: this word
  // equals kMiscPrepareGen (the prepare's number, stored by its key build)
  kMiscNotOneHot = 5,
  kMiscPrepareGen = 6,
  kMiscCacheMiss = 7,  // tiered: misses of this prepare
  kMiscHashSlotFull = 4,  // the call's new keys would exceed a table's slot bound
  // per table: new keys [T], their base rank [T], block part [T + 1], then
  // the slots this call claimed [T] (at kMiscHashNew + 3T + 1)
  kMiscHashNew = 8,
};
inline size_t misc_words(int T) { return 64 + 4 * (size_t)T + 8; }

// A hashed table keeps at most this share of its slots holding keys (live or
// counted for admission); linear probes then stay short.
constexpr double kMaxSlotLoad = 0.9;
// Probes per occurrence before a call is declared full (reached only if the
// slot bound above failed to hold).
constexpr int64_t kMaxProbe = 8192;

bool make_plan(const Handle& h, int64_t B, int64_t nnz, Plan* p);

// ---------------------------------------------------------------- device helpers
__device__ inline uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Inclusive prefix sum over the 64 lanes of a wave (every lane active).
// Within each row of 16 lanes a Hillis-Steele scan on DPP row shifts by 1, 2,
// 4 and 8 (a lane whose source lies before its row adds nothing); then rows 1
// and 3 add the last lane of rows 0 and 2, and the upper half adds lane 31,
// both through readlane.  No LDS and no ds_bpermute.
template <int CTRL>
__device__ inline uint32_t dpp_shifted(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ inline uint32_t wave_incl_scan(uint32_t x) {
  const uint32_t lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const uint32_t r = lane & 15u;
  uint32_t t;
  t = dpp_shifted<0x111>(x);  // row_shr:1
  if (r >= 1u) x += t;
  t = dpp_shifted<0x112>(x);  // row_shr:2
  if (r >= 2u) x += t;
  t = dpp_shifted<0x114>(x);  // row_shr:4
  if (r >= 4u) x += t;
  t = dpp_shifted<0x118>(x);  // row_shr:8
  if (r >= 8u) x += t;
  const uint32_t row0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 15);
  const uint32_t row2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 47);
  if ((lane & 48u) == 16u) x += row0;
  if ((lane & 48u) == 48u) x += row2;
  const uint32_t half = (uint32_t)__builtin_amdgcn_readlane((int)x, 31);
  if (lane >= 32u) x += half;
  return x;
}

// Block index remapped so that each of the 8 XCDs (which take hardware blocks
// round-robin) works on one contiguous range of logical blocks, keeping the
// cache lines a range shares inside one XCD's L2.
__device__ inline uint32_t xcd_block() {
  const uint32_t nb = gridDim.x, b = blockIdx.x;
  const uint32_t q = nb >> 3, r = nb & 7u, x = b & 7u;
  return x * q + (x < r ? x : r) + (b >> 3);
}

// Row columns 4*d4 .. 4*d4+3 of `base`, or zeros when !ok.  The load is
// unconditional (from column 0 of row 0 when !ok), which keeps the code free
// of divergent branches around loads; `base` must hold at least 4 floats.
__device__ inline f4 load4_or_zero(const float* __restrict__ base, size_t row, uint32_t D,
                                   uint32_t d4, bool ok) {
  const size_t off = ok ? row * D + 4u * d4 : 0u;
  const f4 x = *reinterpret_cast<const f4*>(base + off);
  return ok ? x : f4{0.f, 0.f, 0.f, 0.f};
}

// Same, with a non-temporal load (data read once: keep it out of the way of
// rows that are reused).
__device__ inline f4 load4_nt_or_zero(const float* __restrict__ base, size_t row, uint32_t D,
                                      uint32_t d4, bool ok) {
  const size_t off = ok ? row * D + 4u * d4 : 0u;
  const f4 x = __builtin_nontemporal_load(reinterpret_cast<const f4*>(base + off));
  return ok ? x : f4{0.f, 0.f, 0.f, 0.f};
}

// Whether some bag of the prepared batch holds other than one id (the key
// build tags the flag word with its own number, so no clearing launch is
// needed; a stale tag can only select the general path, which is exact too).
__device__ inline bool batch_not_one_hot(const uint32_t* misc) {
  return misc[kMiscNotOneHot] == misc[kMiscPrepareGen];
}

// Grad row (= output row s*T + t) of occurrence j of a batch whose every bag
// holds just the occurrence with its own index (one-hot): its bag is j, the
// table j / B and the sample j % B.
__device__ inline uint32_t one_hot_grad_row(uint32_t j, uint32_t B, uint32_t T) {
  const uint32_t t = j / B;
  return (j - t * B) * T + t;
}

// One SplitMix64 step from `state` (Steele, Lea and Flood 2014).
__device__ inline uint64_t sm64(uint64_t state) {
  uint64_t z = state + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Home slot mixer of the hash table: SplitMix64's finalizer alone.
__device__ inline uint64_t slot_mix(uint64_t k) {
  k = (k ^ (k >> 30)) * 0xBF58476D1CE4E5B9ull;
  k = (k ^ (k >> 27)) * 0x94D049BB133111EBull;
  return k ^ (k >> 31);
}

// ---------------------------------------------------------------- launchers
hipError_t launch_init_dense(const Handle& h, hipStream_t s);
hipError_t launch_fill_u64(uint64_t* p, uint64_t v, size_t n, hipStream_t s);
hipError_t launch_fill_f32(float* p, float v, size_t n, hipStream_t s);
hipError_t launch_zero_words(uint32_t* p, int n, hipStream_t s);

hipError_t launch_forward(const Handle& h, const int64_t* offsets, const int64_t* ids,
                          int64_t B, int64_t nnz, bool mean, float* out, hipStream_t s);

// Keys, radix sort and unique (unique, seg_off, inverse, num_unique); results
// stay in the workspace.  *sorted_keys and *sorted_vals receive the workspace
// addresses of the sorted arrays.
hipError_t launch_sort_unique(const Handle& h, const Plan& p, const int64_t* offsets,
                              const int64_t* ids, bool mean, char* ws, uint32_t** sorted_keys,
                              uint32_t** sorted_vals, hipStream_t s);

// Segmented reduction + Adagrad over the sorted occurrences (grad_out must not
// be null).
// Adagrad Decay (stamps != NULL): before its step a row's accumulator is
// multiplied by 2^((period - stamp[row]) * log2_rho) when period > stamp[row],
// and stamp[row] becomes max(stamp[row], period).
struct DecayArgs {
  uint32_t* stamps = nullptr;
  float log2_rho = 0.0f;
  uint32_t period = 0;
};
// perm: the sorted occurrence indices (one-hot batches derive the grad row
// from them).
hipError_t launch_segment_adagrad(const Handle& h, const Plan& p, const uint32_t* keys,
                                  const uint32_t* perm, bool mean, const float* grad_out,
                                  float lr, float eps, char* ws, hipStream_t s,
                                  const DecayArgs& dec = DecayArgs());
// The same reduction with the gradient rows given as the int8 exchange payload
// (codes [bags, D], one scale per row; plain Adagrad).
hipError_t launch_segment_adagrad_int8(const Handle& h, const Plan& p, const uint32_t* keys,
                                       const uint32_t* perm, bool mean, const int8_t* codes,
                                       const float* scales, float lr, float eps, char* ws,
                                       hipStream_t s);

// Forward from a prepared workspace.  One-hot batches gather the rows in
// sorted order; otherwise (a device flag of the prepare) the same launch runs
// the pooled kernel.
// rowmap (tiered tables; NULL otherwise): the row of every occurrence, which
// the pooled kernel reads instead of computing it from the ids.
hipError_t launch_forward_sorted(const Handle& h, const Plan& p, const int64_t* offsets,
                                 const int64_t* ids, bool mean, const uint32_t* keys,
                                 const uint32_t* perm, float* out, char* ws,
                                 const uint32_t* rowmap, hipStream_t s);
// The pooled kernel alone (the ids and offsets are read directly).
// The prepared forward writing the int8 exchange payload (codes [B*T, D],
// one scale per row) instead of fp32 rows: the sorted one-hot kernel when
// maybe_one_hot (nnz == B * T), else the pooled one.
hipError_t launch_forward_prepared_int8(const Handle& h, const Plan& p, const int64_t* offsets,
                                        const int64_t* ids, bool mean, bool maybe_one_hot,
                                        const uint32_t* keys, const uint32_t* perm,
                                        int8_t* codes, float* scales, char* ws,
                                        const uint32_t* rowmap, hipStream_t s);
hipError_t launch_forward_bags(const Handle& h, const int64_t* offsets, const int64_t* ids,
                               int64_t B, int64_t nnz, bool mean, float* out,
                               const uint32_t* rowmap, hipStream_t s);

hipError_t launch_unique_counts(const Plan& p, char* ws, hipStream_t s);

// Tiered tables, after launch_sort_unique: look the batch's distinct rows up
// in the HBM cache, bring the missing ones in (writing evicted rows back to
// host memory), then write the cache slot of every sorted occurrence to
// *slot_keys (the sort's spare key buffer) and, when the batch is not
// one-hot, of every occurrence in input order to the workspace row map.
hipError_t launch_cache_prepare(Handle& h, const Plan& p, const uint32_t* sorted_keys,
                                const uint32_t* perm, uint32_t* slot_keys, char* ws,
                                hipStream_t s);
hipError_t launch_cache_flush(const Handle& h, hipStream_t s);
hipError_t launch_cache_init(const Handle& h, hipStream_t s);

// Frequency admission (counts != NULL and min_count > 1): counts[t * cap + slot]
// counts the occurrences of a key without a row; a key gets a row in the call
// where its count reaches min_count, else its ids are kAbsentId.
struct AdmitArgs {
  uint32_t* counts = nullptr;
  uint32_t min_count = 0;
};
hipError_t launch_hash_find_or_insert(const Handle& h, const Plan& p, const int64_t* offsets,
                                      const uint64_t* keys, int64_t* ids_out, char* ws,
                                      hipStream_t s, const AdmitArgs& adm = AdmitArgs());

hipError_t launch_hash_export(const Handle& h, int t, uint64_t* key_of_row, hipStream_t s);
size_t hash_evict_workspace_bytes(const Handle& h);
hipError_t launch_hash_evict(const Handle& h, uint32_t* last_used, uint32_t before,
                             uint32_t* key_counts, char* ws, hipStream_t s);

// Stream kernels (kind 0 copy, 1 fill, 2 read into one float per block).
size_t stream_read_sink_floats(size_t bytes);
hipError_t launch_stream(int kind, void* dst, const void* src, size_t bytes, float value,
                         hipStream_t s);

// int8 exchange payload, per row of D values: amax = max |x|, inv = 127 / amax
// (0 for a zero row), code = x * inv rounded to nearest with ties to even and
// clamped to +-127, scale = amax / 127; every step in fp32.  The quantize
// kernel and the fused forward share these two helpers.
__device__ inline float abs_max4(f4 v) {
  return __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(v[0]), __builtin_fabsf(v[1])),
                         __builtin_fmaxf(__builtin_fabsf(v[2]), __builtin_fabsf(v[3])));
}
// The four codes of one float4, packed little-endian in a word.
__device__ inline uint32_t int8_code_word(f4 v, float inv) {
  uint32_t w = 0u;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float q =
        __builtin_fminf(127.0f, __builtin_fmaxf(-127.0f, __builtin_rintf(v[e] * inv)));
    w |= (uint32_t)(uint8_t)(int8_t)(int)q << (8 * e);
  }
  return w;
}

// D % 4 == 0, D <= 1024; codes 4-byte aligned, x and y 16-byte aligned.
hipError_t launch_quantize_rows(const float* x, int64_t rows, int32_t D, int8_t* codes,
                                float* scales, hipStream_t s);
hipError_t launch_dequantize_rows(const int8_t* codes, const float* scales, int64_t rows,
                                  int32_t D, float* y, hipStream_t s);

hipError_t launch_debug_copy_sorted(const uint32_t* keys, uint32_t sentinel, uint32_t* out,
                                    int64_t n, hipStream_t s);

}  // namespace embtab
