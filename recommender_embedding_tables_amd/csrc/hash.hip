// Raw-key -> row hash table with dynamic insertion, for gfx950.
//
// Feature keys are mapped to rows by a GPU hash table that inserts keys it has
// not seen, so no capacity planning is needed (OneFlow OneEmbedding page,
// section "ease of use"; "Merlin HugeCTR interview", section two: a hash table
// identifies every input feature before the embedding layer, and section
// three, technique (1): GPU-accelerated hash table; DeepRec page, section
// "model quality": lock-free hash with one access per pass).
//
// Table t owns `cap` slots of 16 bytes {key, row}; an empty slot holds
// key = row = all ones.  The home slot of a key is SplitMix64's finalizer of
// the key masked to cap - 1; collisions probe linearly.  One call runs:
//   k_hash_probe   one thread per occurrence: look the key up (plain 16-byte
//                  slot loads first); a live key gives its row.  A missing key claims a slot with a 64-bit
//                  CAS on the key word (lock-free), and every occurrence of it
//                  lowers the slot's row word to (PENDING | j) with atomicMin,
//                  which leaves the first occurrence j in the slot.  A probe
//                  sequence is bounded by `cap`: running out marks the call
//                  full instead of looping.
//   k_hash_first   flags first occurrences; per-block counts, and per table
//                  the count before its first position inside its block.
//   k_hash_plan    one block: block bases (exclusive scan), per-table bases
//                  and new-key counts, and the call's capacity decision
//                  (all-or-nothing).
//   k_hash_assign  a first occurrence of table t with rank r (its order among
//                  table t's first occurrences) writes row n_live[t] + r into
//                  its slot and lists itself for initialisation; when the call
//                  is full it empties the claimed slot again instead, which
//                  restores the table exactly (the slot was empty before).
//   k_hash_finish  ids of new keys from their slots, live-row counters and,
//                  in the same launch, the new rows: W = init_std *
//                  Box-Muller normal of the counter draws (seed, t, key, 2d)
//                  and (.., 2d+1); G = accum_init.
// Row assignment follows first occurrence and is deterministic; which slot a
// key lands in depends on CAS order and is not part of the contract.
//
// Calls that cannot be kept are undone whole (all-or-nothing):
//   * rows: a table's new keys exceed its free rows (full);
//   * slots: the keys holding a table's slots (live keys and keys counted for
//     admission) would exceed kMaxSlotLoad of its capacity (full);
//   * offsets: the CSR offsets do not start at 0, end at nnz and rise (bad
//     offsets); such a call leaves even the admission counts as they were.
// Slots claimed by the call are emptied again, so probe sequences stay short:
// a probe walks at most kMaxProbe slots, and reaching that bound also makes
// the call full.
//
// Frequency admission (DeepRec page, section "model quality", EmbeddingVariable
// item 1: features are admitted before they get a row).  With a count array
// and min_count > 1, a key's slot also counts its occurrences (one atomicAdd
// per occurrence of a key without a row, in the probe); k_hash_first and
// k_hash_assign treat a first occurrence as new only when its key's count has
// reached min_count.  Other keys keep their slot with the row word kCandRow
// and get id -2 (absent).  A full call admits nothing: its would-be keys keep
// kCandRow (and their counts) instead of emptying their slots.
#include "embtab_internal.hpp"

namespace embtab {

namespace {

constexpr uint32_t kNoSlot = 0xFFFFFFFFu;
constexpr int64_t kFastProbes = 8;  // plain-load probes before the atomic path

__device__ inline int32_t table_of(const int64_t* tb, int32_t T, int64_t j) {
  // tb[t] = first occurrence of table t (T + 1 entries, non-decreasing).
  int32_t lo = 0, hi = T;  // answer in [0, T)
  while (hi - lo > 1) {
    const int32_t mid = (lo + hi) >> 1;
    if (tb[mid] <= j) lo = mid;
    else hi = mid;
  }
  return lo;
}

// First occurrence of every table (T + 1 entries), clamped to [0, nnz] and
// made non-decreasing (a running maximum), so that tables are contiguous
// ranges of occurrences even when the offsets are not valid.  Computed once
// per call by k_hash_start; the other kernels copy it to LDS.
__device__ inline void load_table_bounds(int64_t* tb, const int64_t* __restrict__ tbw, int32_t T) {
  for (int t = threadIdx.x; t <= T; t += blockDim.x) tb[t] = tbw[t];
  __syncthreads();
}

// Tables are the occurrence ranges [tb[t], tb[t+1]) with tb[0] = 0 and
// tb[T] = nnz, so every occurrence belongs to exactly one table whatever the
// offsets hold; offsets that do not start at 0, end at nnz and rise at the
// table starts mark the call aborted (k_hash_probe checks the other bags).
__global__ __launch_bounds__(256) void k_hash_start(const int64_t* __restrict__ offsets, int64_t B,
                                                    int32_t T, int64_t nnz,
                                                    int64_t* __restrict__ tbw,
                                                    uint32_t* __restrict__ misc, int32_t nzero,
                                                    uint32_t* __restrict__ flags) {
  extern __shared__ int64_t tb[];
  __shared__ uint32_t s_bad;
  if (threadIdx.x == 0) s_bad = 0u;
  for (int i = threadIdx.x; i < nzero; i += blockDim.x) misc[i] = 0u;
  __syncthreads();
  for (int t = threadIdx.x; t <= T; t += blockDim.x) {
    const int64_t v = offsets[(int64_t)t * B];
    if ((t == 0 && v != 0) || (t == T && v != nnz)) s_bad = 1u;
    tb[t] = v < 0 ? 0 : (v > nnz ? nnz : v);
  }
  __syncthreads();
  for (int t = threadIdx.x + 1; t <= T; t += blockDim.x)
    if (tb[t] < tb[t - 1]) s_bad = 1u;
  __syncthreads();
  if (threadIdx.x == 0) {
    tb[0] = 0;
    tb[T] = nnz;
  }
  __syncthreads();
  for (int o = 1; o <= T; o <<= 1) {  // running maximum, log-step (T + 1 <= 1025)
    int64_t mine[5];
    int k = 0;
    for (int t = threadIdx.x; t <= T; t += blockDim.x, ++k)
      mine[k] = (t >= o && tb[t - o] > tb[t]) ? tb[t - o] : tb[t];
    __syncthreads();
    k = 0;
    for (int t = threadIdx.x; t <= T; t += blockDim.x, ++k) tb[t] = mine[k];
    __syncthreads();
  }
  for (int t = threadIdx.x; t <= T; t += blockDim.x) tbw[t] = tb[t];
  if (threadIdx.x == 0 && s_bad) {
    misc[kMiscHashAbort] = 1u;
    atomicOr(flags, EMB_FLAG_BAD_OFFSETS);
  }
}

// misc word of the number of slots table t's keys claimed in this call.
__device__ inline uint32_t misc_fresh(int32_t T, int32_t t) {
  return (uint32_t)(kMiscHashNew + 3 * T + 1 + t);
}

struct Slot {
  uint64_t key;
  uint64_t row;
};

__global__ __launch_bounds__(256) void k_hash_probe(
    const int64_t* __restrict__ tbw, const uint64_t* __restrict__ keys, int64_t B, int32_t T,
    int64_t nnz, Slot* __restrict__ slots, int64_t cap, int64_t* __restrict__ ids_out,
    uint32_t* __restrict__ slot_of, uint32_t* __restrict__ flags, uint32_t* __restrict__ misc,
    uint32_t* __restrict__ counts, const int64_t* __restrict__ offsets,
    uint8_t* __restrict__ fresh_of) {
  extern __shared__ int64_t tb[];
  load_table_bounds(tb, tbw, T);
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  {
    // the bags' offsets rise (the ends and table starts are k_hash_start's)
    bool bad = false;
    const int64_t nbags = (int64_t)T * B, stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t b = j; b < nbags; b += stride) bad = bad || offsets[b + 1] < offsets[b];
    if (__ballot(bad) != 0ull && (threadIdx.x & 63u) == 0u) {
      misc[kMiscHashAbort] = 1u;
      atomicOr(flags, EMB_FLAG_BAD_OFFSETS);
    }
  }
  if (j >= nnz) return;
  fresh_of[j] = 0;
  const uint64_t key = keys[j];
  if (key == kEmptyKey) {
    ids_out[j] = -1;
    slot_of[j] = kNoSlot;
    atomicOr(flags, EMB_FLAG_RESERVED_KEY);
    return;
  }
  const int32_t t = table_of(tb, T, j);
  Slot* st = slots + (size_t)t * (size_t)cap;
  const uint64_t mask = (uint64_t)cap - 1u;
  const uint64_t pend = kPendingBit | (uint64_t)j;
  uint64_t s = slot_mix(key) & mask;
  int64_t probe = 0;
  // Keys inserted by earlier calls are found with plain 16-byte slot loads
  // (key and row together); an empty slot or a key still pending in this call
  // goes on with the atomic protocol below, from the same slot.
  for (; probe < kFastProbes && probe < cap; ++probe, s = (s + 1) & mask) {
    const Slot sl = st[s];
    if (sl.key == key && sl.row < kPendingBit) {
      ids_out[j] = (int64_t)sl.row;
      slot_of[j] = kNoSlot;
      return;
    }
    if (sl.key == kEmptyKey || sl.key == key) break;
  }
  for (; probe < cap && probe < kMaxProbe; ++probe, s = (s + 1) & mask) {
    uint64_t k = __hip_atomic_load(&st[s].key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (k == kEmptyKey) {
      const uint64_t old = atomicCAS((unsigned long long*)&st[s].key, (unsigned long long)kEmptyKey,
                                     (unsigned long long)key);
      k = (old == kEmptyKey) ? key : old;
      if (old == kEmptyKey) {  // this occurrence claimed the slot: one per new key
        fresh_of[j] = 1;
        atomicAdd(&misc[misc_fresh(T, t)], 1u);
      }
    }
    if (k != key) continue;
    const uint64_t r = __hip_atomic_load(&st[s].row, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (r < kPendingBit) {  // live key from an earlier call
      ids_out[j] = (int64_t)r;
      slot_of[j] = kNoSlot;
    } else {
      if (counts) atomicAdd(&counts[(size_t)t * (size_t)cap + s], 1u);  // not admitted yet
      if (pend < r) atomicMin((unsigned long long*)&st[s].row, (unsigned long long)pend);
      slot_of[j] = (uint32_t)s;
    }
    return;
  }
  // no free slot within kMaxProbe (or none at all): the call cannot insert
  slot_of[j] = kNoSlot;
  ids_out[j] = -1;
  misc[kMiscHashOverflow] = 1u;
}

__device__ inline bool is_first(const Slot* slots, int64_t cap, const uint32_t* slot_of,
                                int32_t t, int64_t j) {
  const uint32_t s = slot_of[j];
  if (s == kNoSlot) return false;
  return slots[(size_t)t * (size_t)cap + s].row == (kPendingBit | (uint64_t)j);
}

// A first occurrence whose key gets a row in this call: always without
// admission, else once the key's count has reached min_count.
__device__ inline bool admitted(const uint32_t* counts, uint32_t min_count, int64_t cap,
                                const uint32_t* slot_of, int32_t t, int64_t j) {
  return !counts || counts[(size_t)t * (size_t)cap + slot_of[j]] >= min_count;
}

// Per block: the number of first occurrences (bcnt) and, for every table
// whose first occurrence position tb[t] falls in this block, the number of
// first occurrences of the block before tb[t] (tpart[t]).  With the block
// bases these give each table's base rank without device atomics.
__global__ __launch_bounds__(256) void k_hash_first(const int64_t* __restrict__ tbw, int64_t B,
                                                    int32_t T, int64_t nnz,
                                                    const Slot* __restrict__ slots, int64_t cap,
                                                    const uint32_t* __restrict__ slot_of,
                                                    uint32_t* __restrict__ bcnt,
                                                    uint32_t* __restrict__ tpart,
                                                    const uint32_t* __restrict__ counts,
                                                    uint32_t min_count) {
  extern __shared__ int64_t tb[];
  __shared__ uint32_t lds4[4];
  load_table_bounds(tb, tbw, T);
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  bool f = false;
  int32_t t = 0;
  if (j < nnz) {
    t = table_of(tb, T, j);
    f = is_first(slots, cap, slot_of, t, j) && admitted(counts, min_count, cap, slot_of, t, j);
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint64_t m = __ballot(f);
  if (lane == 0) lds4[w] = (uint32_t)__popcll(m);
  __syncthreads();
  uint32_t before = 0;
  for (int i = 0; i < w; ++i) before += lds4[i];
  before += lanes_below(m);  // first occurrences of this block before j
  if (j < nnz) {
    // tables starting at j: t and the empty tables just before it
    for (int32_t u = t; u >= 0 && tb[u] == j; --u) tpart[u] = before;
  }
  if (threadIdx.x == 0) bcnt[blockIdx.x] = lds4[0] + lds4[1] + lds4[2] + lds4[3];
}

// One block of 1024 threads.  Exclusive scan of the block counts in place
// (each pass: 16 consecutive counts per thread, read and written as uint4).
__global__ __launch_bounds__(1024) void k_hash_plan(uint32_t* __restrict__ bcnt, uint32_t nblocks,
                                                    const int64_t* __restrict__ tbw, int32_t T,
                                                    int64_t nnz,
                                                    const uint32_t* __restrict__ tpart,
                                                    const int64_t* __restrict__ n_live,
                                                    const int64_t* __restrict__ rows,
                                                    const int64_t* __restrict__ q_head,
                                                    const int64_t* __restrict__ q_tail,
                                                    uint32_t* __restrict__ misc,
                                                    uint32_t* __restrict__ flags,
                                                    const int64_t* __restrict__ slots_used,
                                                    int64_t slot_limit) {
  constexpr uint32_t PER = 16;
  __shared__ uint32_t wsum[16];
  __shared__ uint32_t s_full, s_slot;
  uint32_t carry = 0;
  const uint32_t lane = threadIdx.x & 63u, w = threadIdx.x >> 6;
  for (uint32_t base = 0; base < nblocks; base += 1024u * PER) {
    const uint32_t lo = base + threadIdx.x * PER;
    uint32_t v[PER];
    if (lo + PER <= nblocks) {
#pragma unroll
      for (int q = 0; q < (int)PER / 4; ++q) {
        const uint4 x = reinterpret_cast<const uint4*>(bcnt + lo)[q];
        v[4 * q] = x.x;
        v[4 * q + 1] = x.y;
        v[4 * q + 2] = x.z;
        v[4 * q + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int q = 0; q < (int)PER; ++q) v[q] = lo + q < nblocks ? bcnt[lo + q] : 0u;
    }
    uint32_t sum = 0;
#pragma unroll
    for (int q = 0; q < (int)PER; ++q) sum += v[q];
    uint32_t x = sum;
    x = wave_incl_scan(x);
    if (lane == 63u) wsum[w] = x;
    __syncthreads();
    uint32_t before = 0, total = 0;
#pragma unroll
    for (uint32_t i = 0; i < 16u; ++i) {
      before += i < w ? wsum[i] : 0u;
      total += wsum[i];
    }
    __syncthreads();
    uint32_t run = carry + before + x - sum;
#pragma unroll
    for (int q = 0; q < (int)PER; ++q) {
      const uint32_t c = v[q];
      v[q] = run;
      run += c;
    }
    if (lo + PER <= nblocks) {
#pragma unroll
      for (int q = 0; q < (int)PER / 4; ++q)
        reinterpret_cast<uint4*>(bcnt + lo)[q] = make_uint4(v[4 * q], v[4 * q + 1], v[4 * q + 2],
                                                            v[4 * q + 3]);
    } else {
#pragma unroll
      for (int q = 0; q < (int)PER; ++q)
        if (lo + q < nblocks) bcnt[lo + q] = v[q];
    }
    carry += total;
  }
  __syncthreads();  // the bases written above are read back below
  if (threadIdx.x == 0) {
    s_full = misc[kMiscHashOverflow];
    s_slot = 0u;
  }
  __syncthreads();
  // table t's first occurrences have ranks [base_t, base_{t+1}) among this
  // call's first occurrences, in occurrence (and so table) order
  auto table_base = [&](int32_t t) -> uint32_t {
    const int64_t q = tbw[t];  // tbw[T] = nnz
    if (q >= nnz) return carry;
    return bcnt[q >> 8] + tpart[t];
  };
  for (int32_t t = threadIdx.x; t < T; t += blockDim.x) {
    const uint32_t b0 = table_base(t), b1 = table_base(t + 1);
    const uint32_t nw = b1 >= b0 ? b1 - b0 : 0u;
    misc[kMiscHashNew + t] = nw;
    misc[kMiscHashNew + T + t] = b0;
    // rows left: queued free rows, then rows never used
    if ((int64_t)nw > q_tail[t] - q_head[t] + rows[t] - n_live[t]) s_full = 1u;  // all store 1
    // slots: the keys already holding one, and the slots this call claimed
    if (slots_used[t] + (int64_t)misc[misc_fresh(T, t)] > slot_limit) s_slot = 1u;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t abort_call = misc[kMiscHashAbort];
    const uint32_t drop = s_slot | abort_call;  // keep none of the claimed slots
    misc[kMiscHashOverflow] = s_full | drop;
    misc[kMiscHashSlotFull] = drop;
    misc[kMiscNumUnique] = carry;  // new keys of this call (all tables)
    if ((s_full | s_slot) && !abort_call) atomicOr(flags, EMB_FLAG_TABLE_FULL);
  }
}

__global__ __launch_bounds__(256) void k_hash_assign(
    const int64_t* __restrict__ tbw, int64_t B, int32_t T, int64_t nnz,
    Slot* __restrict__ slots, int64_t cap, const uint32_t* __restrict__ slot_of,
    const uint32_t* __restrict__ bbase, const int64_t* __restrict__ n_live,
    const uint32_t* __restrict__ misc, uint32_t* __restrict__ newlist,
    const uint32_t* __restrict__ counts, uint32_t min_count,
    const uint32_t* __restrict__ free_rows, const int64_t* __restrict__ row_off,
    const int64_t* __restrict__ rows, const int64_t* __restrict__ q_head,
    const int64_t* __restrict__ q_tail) {
  extern __shared__ int64_t tb[];
  __shared__ uint32_t lds4[4];
  load_table_bounds(tb, tbw, T);
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  bool f = false, cand = false;
  int32_t t = 0;
  if (j < nnz) {
    t = table_of(tb, T, j);
    f = is_first(slots, cap, slot_of, t, j);
    if (f && !admitted(counts, min_count, cap, slot_of, t, j)) {
      f = false;  // counted, no row yet
      cand = true;
    }
  }
  if (cand) slots[(size_t)t * (size_t)cap + slot_of[j]].row = kCandRow;
  // block-wide exclusive count of first occurrences before this thread
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint64_t m = __ballot(f);
  if (lane == 0) lds4[w] = (uint32_t)__popcll(m);
  __syncthreads();
  uint32_t before = 0;
  for (int i = 0; i < w; ++i) before += lds4[i];
  if (!f) return;
  const uint32_t g = bbase[blockIdx.x] + before + lanes_below(m);
  const uint32_t full = misc[kMiscHashOverflow];
  Slot* sl = slots + (size_t)t * (size_t)cap + slot_of[j];
  if (full) {
    if (counts) {  // nothing is admitted; the key stays counted
      sl->row = kCandRow;
    } else {       // the slot was empty before this call
      sl->key = kEmptyKey;
      sl->row = kUnsetRow;
    }
    return;
  }
  const uint32_t rank = g - misc[kMiscHashNew + T + t];
  // queued free rows first (oldest first), then rows never used
  const int64_t queued = q_tail[t] - q_head[t];
  int64_t row;
  if ((int64_t)rank < queued)
    row = (int64_t)free_rows[row_off[t] + (q_head[t] + (int64_t)rank) % rows[t]];
  else
    row = n_live[t] + ((int64_t)rank - queued);
  sl->row = (uint64_t)row;
  newlist[g] = (uint32_t)j;
}

// Blocks [0, nfin) write the ids of this call's new keys (and block 0 the
// live-row counters); the blocks after them initialise the new rows:
// W = init_std * Box-Muller normal of the counter draws (seed, t, key, 2d) and
// (.., 2d+1), G = accum_init.  Nothing else reads n_live in this step.
__global__ __launch_bounds__(256) void k_hash_finish(
    const int64_t* __restrict__ tbw, const uint64_t* __restrict__ keys, int64_t B, int32_t T,
    int64_t nnz, const Slot* __restrict__ slots, int64_t cap, const uint32_t* __restrict__ slot_of,
    int64_t* __restrict__ ids_out, const uint32_t* __restrict__ newlist,
    const uint32_t* __restrict__ misc, int64_t* __restrict__ n_live,
    int64_t* __restrict__ q_head, const int64_t* __restrict__ q_tail,
    const uint32_t* __restrict__ counts, uint32_t min_count,
    const int64_t* __restrict__ row_off, const int64_t* __restrict__ rows, float* __restrict__ W,
    float* __restrict__ G, int32_t D,
    uint64_t seed, float stdv, float g0, uint32_t nfin, Slot* __restrict__ wslots,
    const uint8_t* __restrict__ fresh_of, int64_t* __restrict__ slots_used,
    uint32_t* __restrict__ wcounts) {
  extern __shared__ int64_t tb[];
  load_table_bounds(tb, tbw, T);
  const bool full = misc[kMiscHashOverflow] != 0u;
  // slot bound exceeded or bad offsets: none of the claimed slots is kept
  const bool drop = misc[kMiscHashSlotFull] != 0u;
  if (blockIdx.x < nfin) {
    if (blockIdx.x == 0) {
      for (int t = threadIdx.x; t < T; t += blockDim.x) {
        if (!full) {
          const int64_t nw = (int64_t)misc[kMiscHashNew + t];
          const int64_t queued = q_tail[t] - q_head[t];
          const int64_t take = nw < queued ? nw : queued;
          q_head[t] += take;
          n_live[t] += nw - take;
        }
        // the claimed slots stay: as rows, or as counted keys (a full call
        // with admission keeps its would-be keys counted)
        if (!drop && (!full || counts)) slots_used[t] += (int64_t)misc[misc_fresh(T, t)];
      }
    }
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= nnz) return;
    const uint32_t s = slot_of[j];
    if (s == kNoSlot) return;
    const int32_t t = table_of(tb, T, j);
    if (drop) {
      ids_out[j] = -1;
      const bool aborted = misc[kMiscHashAbort] != 0u;
      uint32_t* cnt = counts ? wcounts + (size_t)t * (size_t)cap + s : nullptr;
      // bad offsets: every occurrence takes back its count (a claimed slot's
      // count returns to 0); slot bound: only the claimed slots' counts go
      if (cnt && aborted) atomicSub(cnt, 1u);
      if (fresh_of[j]) {  // this occurrence claimed the slot: empty it again
        Slot* sl = wslots + (size_t)t * (size_t)cap + s;
        sl->key = kEmptyKey;
        sl->row = kUnsetRow;
        if (cnt && !aborted) *cnt = 0u;
      }
      return;
    }
    if (full) {  // keys that would have got a row: -1; keys still counted: absent
      ids_out[j] = admitted(counts, min_count, cap, slot_of, t, j) ? -1 : kAbsentId;
      return;
    }
    const uint64_t r = slots[(size_t)t * (size_t)cap + s].row;
    ids_out[j] = r < kPendingBit ? (int64_t)r : kAbsentId;
    return;
  }
  if (full) return;
  const uint32_t nnew = misc[kMiscNumUnique];
  const int32_t D4 = D >> 2;
  const uint64_t total = (uint64_t)nnew * (uint64_t)D4;
  const uint64_t s0 = sm64(seed);
  const uint32_t ib = blockIdx.x - nfin, nib = gridDim.x - nfin;
  for (uint64_t e = (uint64_t)ib * blockDim.x + threadIdx.x; e < total;
       e += (uint64_t)nib * blockDim.x) {
    const uint32_t g = (uint32_t)(e / D4);
    const int32_t d4 = (int32_t)(e - (uint64_t)g * D4);
    const uint32_t j = newlist[g];
    const int32_t t = table_of(tb, T, j);
    const uint64_t key = keys[j];
    const uint64_t row = slots[(size_t)t * (size_t)cap + slot_of[j]].row;
    if (row >= (uint64_t)rows[t]) continue;  // only with invalid offsets
    const uint64_t pre = sm64(sm64(s0 ^ (uint64_t)t) ^ key);
    f4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint64_t d = (uint64_t)(4 * d4 + i);
      const uint64_t h1 = sm64(pre ^ (2u * d)), h2 = sm64(pre ^ (2u * d + 1u));
      const double u1 = ((double)(h1 >> 40) + 0.5) * (1.0 / 16777216.0);
      const double u2 = (double)(h2 >> 40) * (1.0 / 16777216.0);
      const double z = sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925286766559 * u2);
      w[i] = (float)((double)stdv * z);
    }
    const size_t gi = (size_t)(row_off[t] + (int64_t)row) * D + 4 * d4;
    *reinterpret_cast<f4*>(W + gi) = w;
    *reinterpret_cast<f4*>(G + gi) = f4{g0, g0, g0, g0};
  }
}

__global__ __launch_bounds__(256) void k_hash_export(const Slot* __restrict__ st, int64_t cap,
                                                     uint64_t* __restrict__ key_of_row,
                                                     int64_t nrows) {
  for (int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x; s < cap;
       s += (int64_t)gridDim.x * 256) {
    const uint64_t k = st[s].key;
    const uint64_t r = st[s].row;
    if (k != kEmptyKey && r < kPendingBit && (int64_t)r < nrows) key_of_row[r] = k;
  }
}


// ------------------------------------------------------------------ eviction
// emb_hash_evict (DeepRec page, section "model quality", EmbeddingVariable
// item 1: eviction policies).  Keys whose row was last used before `before`
// leave their table and their rows join the table's free-row queue, in
// ascending order; the slot arrays are rebuilt from the other live keys, so
// probe sequences stay short and counted keys without a row are dropped.
//   (slot arrays copied to the workspace, then filled empty)
//   k_evict_rebuild  per slot of the copy: flag the row of an evicted key, or
//                    insert the live key again (lock-free, as the probe does)
//   k_evict_count    flagged rows per block of kEvictSpan rows
//   k_evict_scan     one block: exclusive scan of the block counts
//   k_evict_tables   per table boundary: the flags before it (global rank)
//   k_evict_scatter  a flagged row of table t with rank i (among t's flagged
//                    rows) goes to queue entry q_tail[t] + i
//   k_evict_finish   queue tails
constexpr int64_t kEvictSpan = 4096;  // rows per counting block: 256 threads x 16

// Slot (t, s) of the copy of the slot arrays: a live key whose row was last
// used before `before` flags its row; every other live key goes back into the
// (emptied) slot array of its table.  Counted keys without a row are dropped.
__global__ __launch_bounds__(256) void k_evict_rebuild(const Slot* __restrict__ old,
                                                       Slot* __restrict__ slots, int64_t cap,
                                                       const int64_t* __restrict__ row_off,
                                                       uint32_t* __restrict__ last_used,
                                                       uint32_t before,
                                                       uint8_t* __restrict__ flag) {
  const int32_t t = blockIdx.y;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= cap) return;
  const Slot sl = old[(size_t)t * (size_t)cap + i];
  const int64_t nrows = row_off[t + 1] - row_off[t];
  if (sl.key == kEmptyKey || sl.row >= (uint64_t)nrows) return;
  const int64_t g = row_off[t] + (int64_t)sl.row;
  if (last_used[g] < before) {
    flag[g] = 1u;
    last_used[g] = kFreshPeriod;  // the next key on this row starts undiscounted
    return;
  }
  Slot* st = slots + (size_t)t * (size_t)cap;
  const uint64_t mask = (uint64_t)cap - 1u;
  uint64_t s = slot_mix(sl.key) & mask;
  for (int64_t probe = 0; probe < cap; ++probe, s = (s + 1) & mask) {
    const uint64_t prev = atomicCAS((unsigned long long*)&st[s].key,
                                    (unsigned long long)kEmptyKey, (unsigned long long)sl.key);
    if (prev == kEmptyKey) {
      st[s].row = sl.row;
      return;
    }
  }
}

// Flags of rows [16 i, 16 i + 16) of this block's span, as a count.
__device__ inline uint32_t count16(const uint8_t* flag, int64_t lo, int64_t total) {
  uint32_t c = 0;
  if (lo + 16 <= total) {
    const uint4 x = *reinterpret_cast<const uint4*>(flag + lo);
    // each byte is 0 or 1
    c = (uint32_t)__popc(x.x) + (uint32_t)__popc(x.y) + (uint32_t)__popc(x.z) +
        (uint32_t)__popc(x.w);
  } else {
    for (int64_t r = lo; r < total; ++r) c += flag[r];
  }
  return c;
}

__global__ __launch_bounds__(256) void k_evict_count(const uint8_t* __restrict__ flag,
                                                     int64_t total, uint32_t* __restrict__ bcnt) {
  __shared__ uint32_t wsum[4];
  const int64_t lo = (int64_t)blockIdx.x * kEvictSpan + 16 * (int64_t)threadIdx.x;
  uint32_t c = count16(flag, lo, total);
  for (int o = 32; o > 0; o >>= 1) c += (uint32_t)__shfl_down((int)c, o, 64);
  if ((threadIdx.x & 63u) == 0) wsum[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) bcnt[blockIdx.x] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
}

// One block of 1024 threads: bcnt[0 .. n) -> exclusive prefix sums, bcnt[n] = total.
__global__ __launch_bounds__(1024) void k_evict_scan(uint32_t* __restrict__ bcnt, uint32_t n) {
  __shared__ uint32_t wsum[16];
  const uint32_t per = (n + 1023u) / 1024u;
  const uint32_t lo = threadIdx.x * per;
  const uint32_t hi = lo + per < n ? lo + per : n;
  uint32_t sum = 0;
  for (uint32_t i = lo; i < hi; ++i) sum += bcnt[i];
  uint32_t x = sum;
  const uint32_t lane = threadIdx.x & 63u, w = threadIdx.x >> 6;
  x = wave_incl_scan(x);
  if (lane == 63u) wsum[w] = x;
  __syncthreads();
  uint32_t before = 0, total = 0;
  for (uint32_t i = 0; i < 16u; ++i) {
    before += i < w ? wsum[i] : 0u;
    total += wsum[i];
  }
  uint32_t run = before + x - sum;
  for (uint32_t i = lo; i < hi; ++i) {
    const uint32_t c = bcnt[i];
    bcnt[i] = run;
    run += c;
  }
  if (threadIdx.x == 0) bcnt[n] = total;
}

// Block t (0 <= t <= T): the global rank of row row_off[t], i.e. the flags
// before it: its counting block's base plus the flags of that block before
// it, counted by the whole block (16 rows per thread).
__global__ __launch_bounds__(256) void k_evict_tables(const uint8_t* __restrict__ flag,
                                                      int64_t total,
                                                      const uint32_t* __restrict__ bbase,
                                                      const int64_t* __restrict__ row_off,
                                                      uint32_t* __restrict__ tbase) {
  __shared__ uint32_t wsum[4];
  const int64_t r = row_off[blockIdx.x];
  const int64_t b = r / kEvictSpan;
  const int64_t lo = b * kEvictSpan + 16 * (int64_t)threadIdx.x;
  uint32_t c = 0;
  if (lo + 16 <= r) c = count16(flag, lo, total);
  else
    for (int64_t q = lo; q < r; ++q) c += flag[q];
  for (int o = 32; o > 0; o >>= 1) c += (uint32_t)__shfl_down((int)c, o, 64);
  if ((threadIdx.x & 63u) == 0) wsum[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) tbase[blockIdx.x] = bbase[b] + wsum[0] + wsum[1] + wsum[2] + wsum[3];
}

__global__ __launch_bounds__(256) void k_evict_scatter(
    const uint8_t* __restrict__ flag, int64_t total, const uint32_t* __restrict__ bbase,
    const int64_t* __restrict__ row_off, const int64_t* __restrict__ rows, int32_t T,
    const uint32_t* __restrict__ tbase, const int64_t* __restrict__ q_tail,
    uint32_t* __restrict__ free_rows) {
  __shared__ uint32_t wsum[4];
  const int64_t lo = (int64_t)blockIdx.x * kEvictSpan + 16 * (int64_t)threadIdx.x;
  const uint32_t c = count16(flag, lo, total);
  // exclusive count of the block's flags before this thread's 16 rows
  uint32_t x = c;
  const uint32_t lane = threadIdx.x & 63u, w = threadIdx.x >> 6;
  x = wave_incl_scan(x);
  if (lane == 63u) wsum[w] = x;
  __syncthreads();
  uint32_t rank = bbase[blockIdx.x] + x - c;
  for (uint32_t i = 0; i < w; ++i) rank += wsum[i];
  if (c == 0) return;
  for (int64_t r = lo; r < lo + 16 && r < total; ++r) {
    if (!flag[r]) continue;
    int32_t a = 0, b = T;  // table of r: row_off[a] <= r < row_off[a + 1]
    while (b - a > 1) {
      const int32_t mid = (a + b) >> 1;
      if (row_off[mid] <= r) a = mid;
      else b = mid;
    }
    const int64_t q = q_tail[a] + (int64_t)(rank - tbase[a]);
    free_rows[row_off[a] + q % rows[a]] = (uint32_t)(r - row_off[a]);
    ++rank;
  }
}

__global__ __launch_bounds__(256) void k_evict_finish(const uint32_t* __restrict__ tbase,
                                                      int32_t T, int64_t* __restrict__ q_tail,
                                                      const int64_t* __restrict__ q_head,
                                                      const int64_t* __restrict__ n_live,
                                                      int64_t* __restrict__ slots_used) {
  for (int32_t t = threadIdx.x; t < T; t += 256) {
    q_tail[t] += (int64_t)(tbase[t + 1] - tbase[t]);
    // the slot arrays now hold the live keys only (counted keys were dropped)
    slots_used[t] = n_live[t] - (q_tail[t] - q_head[t]);
  }
}

}  // namespace

hipError_t launch_hash_find_or_insert(const Handle& h, const Plan& p, const int64_t* offsets,
                                      const uint64_t* keys, int64_t* ids_out, char* ws,
                                      hipStream_t s, const AdmitArgs& adm) {
  uint32_t* counts = adm.min_count > 1 ? adm.counts : nullptr;
  const int64_t nnz = p.nnz;
  uint32_t* misc = reinterpret_cast<uint32_t*>(ws + p.misc);
  uint32_t* slot_of = reinterpret_cast<uint32_t*>(ws + p.h_slot);
  uint32_t* bcnt = reinterpret_cast<uint32_t*>(ws + p.h_tcnt);
  uint32_t* newlist = reinterpret_cast<uint32_t*>(ws + p.h_first);
  Slot* slots = static_cast<Slot*>(h.slots);
  const size_t shm = sizeof(int64_t) * (size_t)(h.T + 1);
  const unsigned nb = (unsigned)((nnz + 255) / 256);
  const unsigned grid = nb > 0 ? nb : 1;
  phase_mark(h, EMB_PHASE_HASH, false, s);
  int64_t* tbw = reinterpret_cast<int64_t*>(ws + p.h_tb);
  uint8_t* fresh_of = reinterpret_cast<uint8_t*>(ws + p.h_fresh);
  hipLaunchKernelGGL(k_hash_start, dim3(1), dim3(256), shm, s, offsets, p.B, h.T, nnz, tbw, misc,
                     kMiscHashNew + 4 * h.T + 1, h.sv.flags);
  hipLaunchKernelGGL(k_hash_probe, dim3(grid), dim3(256), shm, s, tbw, keys, p.B, h.T, nnz,
                     slots, h.capacity, ids_out, slot_of, h.sv.flags, misc, counts, offsets,
                     fresh_of);
  uint32_t* tpart = misc + kMiscHashNew + 2 * h.T;
  hipLaunchKernelGGL(k_hash_first, dim3(grid), dim3(256), shm, s, tbw, p.B, h.T, nnz, slots,
                     h.capacity, slot_of, bcnt, tpart, counts, adm.min_count);
  const int64_t slot_limit = (int64_t)(kMaxSlotLoad * (double)h.capacity);
  hipLaunchKernelGGL(k_hash_plan, dim3(1), dim3(1024), 0, s, bcnt, nb, tbw, h.T, nnz, tpart,
                     h.sv.n_live, h.sv.rows, h.sv.q_head, h.sv.q_tail, misc, h.sv.flags,
                     h.sv.slots_used, slot_limit);
  hipLaunchKernelGGL(k_hash_assign, dim3(grid), dim3(256), shm, s, tbw, p.B, h.T, nnz, slots,
                     h.capacity, slot_of, bcnt, h.sv.n_live, misc, newlist, counts,
                     adm.min_count, h.free_rows, h.sv.row_off, h.sv.rows, h.sv.q_head,
                     h.sv.q_tail);
  // new rows: at most one per occurrence; enough blocks for a cold start
  int64_t igrid = (nnz * (h.D / 4) + 255) / 256;
  igrid = igrid < 1 ? 1 : (igrid > 2048 ? 2048 : igrid);
  hipLaunchKernelGGL(k_hash_finish, dim3(grid + (unsigned)igrid), dim3(256), shm, s, tbw,
                     keys, p.B, h.T, nnz, slots, h.capacity, slot_of, ids_out, newlist, misc,
                     h.sv.n_live, h.sv.q_head, h.sv.q_tail, counts, adm.min_count,
                     h.sv.row_off, h.sv.rows, h.W, h.G, h.D, h.seed, h.stdv,
                     h.accum0, grid, slots, fresh_of, h.sv.slots_used, counts);
  phase_mark(h, EMB_PHASE_HASH, true, s);
  return hipGetLastError();
}

// Workspace of emb_hash_evict: row flags, block counts, per-table ranks, and
// a copy of the slot arrays.
struct EvictPlan {
  size_t flag = 0, bcnt = 0, tbase = 0, copy = 0, total = 0;
  int64_t nblocks = 0;
};
static EvictPlan evict_plan(const Handle& h) {
  auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
  EvictPlan p;
  p.nblocks = (h.total_rows + kEvictSpan - 1) / kEvictSpan;
  size_t o = 0;
  p.flag = o;
  o += up((size_t)p.nblocks * kEvictSpan);  // whole blocks: 16-byte reads stay inside
  p.bcnt = o;
  o += up(sizeof(uint32_t) * (size_t)(p.nblocks + 1));
  p.tbase = o;
  o += up(sizeof(uint32_t) * (size_t)(h.T + 1));
  p.copy = o;
  o += up(sizeof(Slot) * (size_t)h.T * (size_t)h.capacity);
  p.total = o;
  return p;
}

size_t hash_evict_workspace_bytes(const Handle& h) {
  return h.hashed ? evict_plan(h).total : 0;
}

hipError_t launch_hash_evict(const Handle& h, uint32_t* last_used, uint32_t before,
                             uint32_t* key_counts, char* ws, hipStream_t s) {
  const EvictPlan p = evict_plan(h);
  uint8_t* flag = reinterpret_cast<uint8_t*>(ws + p.flag);
  uint32_t* bcnt = reinterpret_cast<uint32_t*>(ws + p.bcnt);
  uint32_t* tbase = reinterpret_cast<uint32_t*>(ws + p.tbase);
  Slot* copy = reinterpret_cast<Slot*>(ws + p.copy);
  Slot* slots = static_cast<Slot*>(h.slots);
  const size_t nslots = (size_t)h.T * (size_t)h.capacity;
  hipError_t e = launch_fill_u64(reinterpret_cast<uint64_t*>(flag), 0ull,
                                 (size_t)p.nblocks * kEvictSpan / 8, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(copy, slots, sizeof(Slot) * nslots, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess) e = launch_fill_u64(reinterpret_cast<uint64_t*>(slots), kEmptyKey, 2 * nslots, s);
  if (e != hipSuccess) return e;
  const dim3 sgrid((unsigned)((h.capacity + 255) / 256), (unsigned)h.T);
  hipLaunchKernelGGL(k_evict_rebuild, sgrid, dim3(256), 0, s, copy, slots, h.capacity,
                     h.sv.row_off, last_used, before, flag);
  hipLaunchKernelGGL(k_evict_count, dim3((unsigned)p.nblocks), dim3(256), 0, s, flag,
                     h.total_rows, bcnt);
  hipLaunchKernelGGL(k_evict_scan, dim3(1), dim3(1024), 0, s, bcnt, (uint32_t)p.nblocks);
  hipLaunchKernelGGL(k_evict_tables, dim3((unsigned)(h.T + 1)), dim3(256), 0, s, flag,
                     h.total_rows, bcnt, h.sv.row_off, tbase);
  hipLaunchKernelGGL(k_evict_scatter, dim3((unsigned)p.nblocks), dim3(256), 0, s, flag,
                     h.total_rows, bcnt, h.sv.row_off, h.sv.rows, h.T, tbase, h.sv.q_tail,
                     h.free_rows);
  hipLaunchKernelGGL(k_evict_finish, dim3(1), dim3(256), 0, s, tbase, h.T, h.sv.q_tail,
                     h.sv.q_head, h.sv.n_live, h.sv.slots_used);
  e = hipGetLastError();
  if (e == hipSuccess && key_counts)  // every counted key was dropped with its slot
    e = launch_fill_u64(reinterpret_cast<uint64_t*>(key_counts), 0ull, nslots / 2, s);
  return e;
}

hipError_t launch_hash_export(const Handle& h, int t, uint64_t* key_of_row, hipStream_t s) {
  const Slot* st = static_cast<const Slot*>(h.slots) + (size_t)t * (size_t)h.capacity;
  int64_t g = (h.capacity + 255) / 256;
  if (g > 8192) g = 8192;
  hipError_t e = launch_fill_u64(key_of_row, kEmptyKey, (size_t)h.rows[t], s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_hash_export, dim3((unsigned)g), dim3(256), 0, s, st, h.capacity, key_of_row,
                     h.rows[t]);
  return hipGetLastError();
}

}  // namespace embtab
