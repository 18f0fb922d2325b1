// HBM row cache of a tiered table (weights and accumulators in host memory),
// for gfx950.
//
// Tiered storage keeps every row in host memory and the rows a training step
// uses in device memory (DeepRec page, section "deployment and serving",
// multi-level hybrid embedding storage: frequently used features on fast
// memory, rarely used ones on cheaper memory; OneFlow OneEmbedding page,
// closing section: layered storage).  Here the device keeps C rows in sets of
// kCacheWays slots; the set of row r is SplitMix64's finalizer of r modulo
// the number of sets.  Per slot: the row it holds (kNoRow: empty) and the
// step it was last used at.
//
// After the sort of a batch, with the run heads of the sort (one per distinct
// row), one prepare runs:
//   k_cache_lookup  per sorted position; a run head searches its row's set.
//                   A hit stamps its slot with this step; a miss is listed
//                   (one device atomic per wave).
//   k_cache_claim   per miss: the slots of its set not used at this step or
//                   the previous one, in order of last use, are tried with a
//                   compare-and-swap of the stamp (so two misses never take
//                   one slot); the old row of the slot is the victim.  No such
//                   slot: the row gets none (EMB_FLAG_CACHE_FULL).
//   k_cache_move    per miss, one sub-group of lanes per row: the victim's
//                   weights and accumulator go back to host memory, then the
//                   missing row comes in.
//   k_cache_remap   per sorted position: the slot of its run, as the key the
//                   forward and the reduction use; for batches that are not
//                   one-hot also the slot of every occurrence in input order.
// The unique index of the run holding sorted position k is recomputed from
// the per-chunk run-head counts of the prepare (as the reduction does), so no
// kernel reads a key another kernel of the same launch is writing.  The cache
// is invisible in the results: the rows' values, and the reduction's
// summation order, do not depend on which slot holds a row.
#include "embtab_internal.hpp"

// Blocks of the row-move kernel per compute unit (see launch_move), as a
// fraction EMBTAB_MOVE_BLOCKS_PER_CU / EMBTAB_MOVE_CU_DIV.
#ifndef EMBTAB_MOVE_BLOCKS_PER_CU
#define EMBTAB_MOVE_BLOCKS_PER_CU 1
#endif
#ifndef EMBTAB_MOVE_CU_DIV
#define EMBTAB_MOVE_CU_DIV 2
#endif

namespace embtab {

namespace {

__device__ inline uint32_t set_of(uint32_t row, uint32_t nsets) {
  return (uint32_t)(slot_mix((uint64_t)row) & (uint64_t)(nsets - 1u));
}

// Unique index of the run holding sorted position k (valid keys only): the
// first run head of its chunk has index head_base[k / 256] + chunk_base[c];
// add the heads of the chunk at or before k, minus one.  `heads` is the
// wave's ballot of run heads; CH-position chunks are whole in one wave.
template <int CH>
__device__ inline uint32_t run_index(uint32_t k, uint64_t heads,
                                     const uint32_t* __restrict__ chunk_base,
                                     const uint32_t* __restrict__ head_base) {
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t first = lane - (lane % CH);  // first lane of the chunk
  const uint32_t upto = lane - first + 1u;     // lanes of the chunk up to k
  const uint64_t bits = (heads >> first) & (upto >= 64u ? ~0ull : ((1ull << upto) - 1ull));
  return head_base[k >> 8] + chunk_base[k / CH] + (uint32_t)__popcll(bits) - 1u;
}

template <int CH>
__global__ __launch_bounds__(256) void k_cache_lookup(
    const uint32_t* __restrict__ keys, uint32_t n, uint32_t sentinel,
    const uint32_t* __restrict__ chunk_base, const uint32_t* __restrict__ head_base,
    const uint32_t* __restrict__ tag, uint32_t* __restrict__ stamp, uint32_t nsets, uint32_t step,
    uint32_t* __restrict__ slot_of_u, uint32_t* __restrict__ miss_u,
    uint32_t* __restrict__ miss_row, uint32_t* __restrict__ misc) {
  const uint32_t k = blockIdx.x * 256u + threadIdx.x;
  uint32_t key = sentinel;
  bool head = false;
  if (k < n) {
    key = keys[k];
    head = key < sentinel && (k == 0 || keys[k - 1] != key);
  }
  const uint64_t heads = __ballot(head);
  bool miss = false;
  uint32_t u = 0;
  if (head) {
    u = run_index<CH>(k, heads, chunk_base, head_base);
    const uint32_t base = set_of(key, nsets) * kCacheWays;
    uint32_t slot = kNoRow;
    const uint4* t4 = reinterpret_cast<const uint4*>(tag + base);
#pragma unroll
    for (int q = 0; q < kCacheWays / 4; ++q) {
      const uint4 x = t4[q];
      if (x.x == key) slot = base + 4 * q;
      if (x.y == key) slot = base + 4 * q + 1;
      if (x.z == key) slot = base + 4 * q + 2;
      if (x.w == key) slot = base + 4 * q + 3;
    }
    if (slot != kNoRow) {
      stamp[slot] = step;
      slot_of_u[u] = slot;
    } else {
      miss = true;
    }
  }
  // list the misses: one device atomic per wave
  const uint64_t mm = __ballot(miss);
  if (mm) {
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t leader = (uint32_t)__ffsll((unsigned long long)mm) - 1u;
    uint32_t at = 0;
    if (lane == leader) at = atomicAdd(&misc[kMiscCacheMiss], (uint32_t)__popcll(mm));
    at = (uint32_t)__shfl((int)at, (int)leader, 64);
    if (miss) {
      const uint32_t i = at + lanes_below(mm);
      miss_u[i] = u;
      miss_row[i] = key;
    }
  }
}

__global__ __launch_bounds__(256) void k_cache_claim(
    const uint32_t* __restrict__ miss_u, const uint32_t* __restrict__ miss_row,
    const uint32_t* __restrict__ misc, uint32_t* __restrict__ tag, uint32_t* __restrict__ stamp,
    uint32_t nsets, uint32_t step, uint32_t* __restrict__ slot_of_u,
    uint32_t* __restrict__ victim, uint32_t* __restrict__ mslot, uint32_t* __restrict__ flags,
    uint64_t* __restrict__ counters, uint32_t n) {
  const uint32_t nm = misc[kMiscCacheMiss] < n ? misc[kMiscCacheMiss] : n;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    counters[0] += (uint64_t)misc[kMiscNumUnique];  // distinct rows looked up
    counters[1] += (uint64_t)nm;
  }
  const uint32_t m = blockIdx.x * 256u + threadIdx.x;
  if (m >= nm) return;
  const uint32_t row = miss_row[m];
  const uint32_t base = set_of(row, nsets) * kCacheWays;
  uint32_t seen[kCacheWays];
#pragma unroll
  for (int w = 0; w < kCacheWays; ++w) seen[w] = stamp[base + w];
  uint32_t tried = 0u, slot = kNoRow;
  // Least recently used first.  Slots used at this step or the previous one
  // are not candidates: the previous batch's forward and backward may still
  // be running on another stream (two-deep pipelining).
  for (int attempt = 0; attempt < kCacheWays && slot == kNoRow; ++attempt) {
    int best = -1;
    uint32_t bs = 0xFFFFFFFFu;
#pragma unroll
    for (int w = 0; w < kCacheWays; ++w) {
      const bool idle = seen[w] == 0u || seen[w] + 1u < step;
      const bool ok = ((tried >> w) & 1u) == 0u && idle;
      if (ok && (best < 0 || seen[w] < bs)) {
        best = w;
        bs = seen[w];
      }
    }
    if (best < 0) break;
    tried |= 1u << best;
    if (atomicCAS(&stamp[base + best], bs, step) == bs) slot = base + (uint32_t)best;
  }
  const uint32_t u = miss_u[m];
  uint32_t v = kNoRow;
  if (slot == kNoRow) {  // every slot of the set holds a row of this or the previous batch
    atomicOr(flags, EMB_FLAG_CACHE_FULL);
    slot_of_u[u] = kNoRow;
    mslot[m] = kNoRow;
  } else {
    v = tag[slot];
    victim[m] = v;
    tag[slot] = row;
    mslot[m] = slot;
    slot_of_u[u] = slot;
  }
  // count the write-backs: one device atomic per wave
  const uint64_t wb = __ballot(v != kNoRow);
  if (wb && (threadIdx.x & 63u) == (uint32_t)__ffsll((unsigned long long)wb) - 1u)
    atomicAdd(reinterpret_cast<unsigned long long*>(&counters[2]),
              (unsigned long long)__popcll(wb));
}

// One sub-group of SG lanes per miss, VEC float4 columns per lane.
template <int SG, int VEC>
__global__ __launch_bounds__(256) void k_cache_move(
    const uint32_t* __restrict__ miss_row, const uint32_t* __restrict__ victim,
    const uint32_t* __restrict__ mslot, const uint32_t* __restrict__ misc, float* __restrict__ W,
    float* __restrict__ G, float* __restrict__ hostW, float* __restrict__ hostG, int32_t D,
    uint32_t n) {
  constexpr int SGPB = 256 / SG;
  const uint32_t nm = misc[kMiscCacheMiss] < n ? misc[kMiscCacheMiss] : n;
  const uint32_t lane = threadIdx.x % SG;
  const uint32_t D4 = (uint32_t)D >> 2;
  for (uint32_t m = blockIdx.x * SGPB + threadIdx.x / SG; m < nm; m += gridDim.x * SGPB) {
    const uint32_t slot = mslot[m];
    if (slot == kNoRow) continue;
    const uint32_t v = victim[m], row = miss_row[m];
#pragma unroll
    for (int q = 0; q < VEC; ++q) {
      const uint32_t d4 = lane + q * SG;
      if (d4 >= D4) continue;
      f4* cw = reinterpret_cast<f4*>(W + (size_t)slot * D) + d4;
      f4* cg = reinterpret_cast<f4*>(G + (size_t)slot * D) + d4;
      // all four loads first: the host reads (the long ones) are in flight
      // together with the slot's old values
      const f4 nw = reinterpret_cast<const f4*>(hostW + (size_t)row * D)[d4];
      const f4 ng = reinterpret_cast<const f4*>(hostG + (size_t)row * D)[d4];
      const f4 ow = *cw, og = *cg;
      if (v != kNoRow) {  // write the evicted row back
        reinterpret_cast<f4*>(hostW + (size_t)v * D)[d4] = ow;
        reinterpret_cast<f4*>(hostG + (size_t)v * D)[d4] = og;
      }
      *cw = nw;
      *cg = ng;
    }
  }
}

template <int CH>
__global__ __launch_bounds__(256) void k_cache_remap(
    const uint32_t* __restrict__ keys, const uint32_t* __restrict__ perm, uint32_t n,
    uint32_t sentinel, const uint32_t* __restrict__ chunk_base,
    const uint32_t* __restrict__ head_base, const uint32_t* __restrict__ slot_of_u,
    uint32_t* __restrict__ slot_keys, uint32_t* __restrict__ rowmap,
    const uint32_t* __restrict__ misc) {
  const uint32_t k = blockIdx.x * 256u + threadIdx.x;
  uint32_t key = sentinel;
  bool head = false;
  if (k < n) {
    key = keys[k];
    head = key < sentinel && (k == 0 || keys[k - 1] != key);
  }
  const uint64_t heads = __ballot(head);
  if (k >= n) return;
  uint32_t out = sentinel;
  if (key < sentinel) {
    const uint32_t u = run_index<CH>(k, heads, chunk_base, head_base);
    const uint32_t slot = u < n ? slot_of_u[u] : kNoRow;
    if (slot != kNoRow) out = slot;
  }
  slot_keys[k] = out;
  if (batch_not_one_hot(misc)) {
    const uint32_t j = perm[k];
    if (j < n) rowmap[j] = out < sentinel ? out : kNoRow;
  }
}

__global__ __launch_bounds__(256) void k_cache_flush(const uint32_t* __restrict__ tag, int64_t C,
                                                     const float* __restrict__ W,
                                                     const float* __restrict__ G,
                                                     float* __restrict__ hostW,
                                                     float* __restrict__ hostG, int32_t D) {
  const int64_t D4 = D >> 2;
  const int64_t total = C * D4;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * 256) {
    const int64_t slot = e / D4, d4 = e - slot * D4;
    const uint32_t row = tag[slot];
    if (row == kNoRow) continue;
    reinterpret_cast<f4*>(hostW + (size_t)row * D)[d4] =
        reinterpret_cast<const f4*>(W + (size_t)slot * D)[d4];
    reinterpret_cast<f4*>(hostG + (size_t)row * D)[d4] =
        reinterpret_cast<const f4*>(G + (size_t)slot * D)[d4];
  }
}

__global__ __launch_bounds__(256) void k_cache_init(uint32_t* __restrict__ tag,
                                                    uint32_t* __restrict__ stamp, int64_t C,
                                                    uint64_t* __restrict__ counters) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < C;
       i += (int64_t)gridDim.x * 256) {
    tag[i] = kNoRow;
    stamp[i] = 0u;
  }
  if (blockIdx.x == 0 && threadIdx.x < 3) counters[threadIdx.x] = 0ull;
}

template <int SG, int VEC>
hipError_t launch_move(const Handle& h, const uint32_t* mrow, const uint32_t* vict,
                       const uint32_t* mslot, const uint32_t* misc, uint32_t n, hipStream_t s) {
  constexpr int SGPB = 256 / SG;
  // The host link, not the CUs, bounds this kernel: a block per two CUs
  // keeps megabytes of reads in flight (far above the link's bandwidth-latency
  // product) and leaves the CUs to the id stages and the forward and
  // backward of other batches, which run beside it on other streams.
  int64_t grid = ((int64_t)n + SGPB - 1) / SGPB;
  const int64_t cap =
      (int64_t)(h.cus > 0 ? h.cus : 256) * EMBTAB_MOVE_BLOCKS_PER_CU / EMBTAB_MOVE_CU_DIV;
  grid = grid < 1 ? 1 : (grid > cap ? cap : grid);
  hipLaunchKernelGGL((k_cache_move<SG, VEC>), dim3((unsigned)grid), dim3(256), 0, s, mrow, vict,
                     mslot, misc, h.W, h.G, h.hostW, h.hostG, h.D, n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_cache_prepare(Handle& h, const Plan& p, const uint32_t* sorted_keys,
                                const uint32_t* perm, uint32_t* slot_keys, char* ws,
                                hipStream_t s) {
  const uint32_t n = (uint32_t)p.nnz;
  ++h.step;
  if (h.step == 0) h.step = 1;  // 0 marks never-used slots
  if (n == 0) return hipSuccess;
  const uint32_t sentinel = (uint32_t)h.total_rows;
  CacheView cv = cache_view(h.cache_state, h.cache_rows);
  uint32_t* misc = reinterpret_cast<uint32_t*>(ws + p.misc);
  const uint32_t* cbase = reinterpret_cast<const uint32_t*>(ws + p.chunk_base);
  const uint32_t* hbase = reinterpret_cast<const uint32_t*>(ws + p.head_base);
  uint32_t* slot_of_u = reinterpret_cast<uint32_t*>(ws + p.c_slot);
  uint32_t* miss_u = reinterpret_cast<uint32_t*>(ws + p.c_miss);
  uint32_t* miss_row = reinterpret_cast<uint32_t*>(ws + p.c_miss) + n;
  uint32_t* vict = reinterpret_cast<uint32_t*>(ws + p.c_vict);
  uint32_t* mslot = reinterpret_cast<uint32_t*>(ws + p.c_mslot);
  uint32_t* rowmap = reinterpret_cast<uint32_t*>(ws + p.c_rowmap);
  const unsigned grid = (n + 255) / 256;
  if (p.chunk == 64)
    hipLaunchKernelGGL((k_cache_lookup<64>), dim3(grid), dim3(256), 0, s, sorted_keys, n, sentinel,
                       cbase, hbase, cv.tag, cv.stamp, h.cache_sets, h.step, slot_of_u, miss_u,
                       miss_row, misc);
  else
    hipLaunchKernelGGL((k_cache_lookup<32>), dim3(grid), dim3(256), 0, s, sorted_keys, n, sentinel,
                       cbase, hbase, cv.tag, cv.stamp, h.cache_sets, h.step, slot_of_u, miss_u,
                       miss_row, misc);
  hipLaunchKernelGGL(k_cache_claim, dim3(grid), dim3(256), 0, s, miss_u, miss_row, misc, cv.tag,
                     cv.stamp, h.cache_sets, h.step, slot_of_u, vict, mslot, h.sv.flags,
                     cv.counters, n);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int sg = subgroup_lanes(h.D), vec = vec_per_lane(h.D);
  phase_mark(h, EMB_PHASE_CACHE, false, s);
  switch (sg) {
    case 1: e = launch_move<1, 1>(h, miss_row, vict, mslot, misc, n, s); break;
    case 2: e = launch_move<2, 1>(h, miss_row, vict, mslot, misc, n, s); break;
    case 4: e = launch_move<4, 1>(h, miss_row, vict, mslot, misc, n, s); break;
    case 8: e = launch_move<8, 1>(h, miss_row, vict, mslot, misc, n, s); break;
    case 16: e = launch_move<16, 1>(h, miss_row, vict, mslot, misc, n, s); break;
    case 32: e = launch_move<32, 1>(h, miss_row, vict, mslot, misc, n, s); break;
    default:
      e = vec == 1   ? launch_move<64, 1>(h, miss_row, vict, mslot, misc, n, s)
          : vec == 2 ? launch_move<64, 2>(h, miss_row, vict, mslot, misc, n, s)
          : vec == 3 ? launch_move<64, 3>(h, miss_row, vict, mslot, misc, n, s)
                     : launch_move<64, 4>(h, miss_row, vict, mslot, misc, n, s);
  }
  phase_mark(h, EMB_PHASE_CACHE, true, s);
  if (e != hipSuccess) return e;
  if (p.chunk == 64)
    hipLaunchKernelGGL((k_cache_remap<64>), dim3(grid), dim3(256), 0, s, sorted_keys, perm, n,
                       sentinel, cbase, hbase, slot_of_u, slot_keys, rowmap, misc);
  else
    hipLaunchKernelGGL((k_cache_remap<32>), dim3(grid), dim3(256), 0, s, sorted_keys, perm, n,
                       sentinel, cbase, hbase, slot_of_u, slot_keys, rowmap, misc);
  return hipGetLastError();
}

hipError_t launch_cache_flush(const Handle& h, hipStream_t s) {
  CacheView cv = cache_view(h.cache_state, h.cache_rows);
  int64_t g = (h.cache_rows * (h.D / 4) + 255) / 256;
  g = g < 1 ? 1 : (g > 8192 ? 8192 : g);
  hipLaunchKernelGGL(k_cache_flush, dim3((unsigned)g), dim3(256), 0, s, cv.tag, h.cache_rows, h.W,
                     h.G, h.hostW, h.hostG, h.D);
  return hipGetLastError();
}

hipError_t launch_cache_init(const Handle& h, hipStream_t s) {
  CacheView cv = cache_view(h.cache_state, h.cache_rows);
  int64_t g = (h.cache_rows + 255) / 256;
  g = g < 1 ? 1 : (g > 4096 ? 4096 : g);
  hipLaunchKernelGGL(k_cache_init, dim3((unsigned)g), dim3(256), 0, s, cv.tag, cv.stamp,
                     h.cache_rows, cv.counters);
  return hipGetLastError();
}

}  // namespace embtab
