// Occurrence keys, LSD radix sort and run-length unique for gfx950.
//
// Deduplicating the ids of a batch so that every touched row is read and
// updated once follows the DeepRec page (section "model quality",
// EmbeddingVariable item 2: one table access per row per pass) and the EcoRec
// page (section "research method": merging work on identical indices, and
// reordering by index).  The sort is stable, so equal rows keep ascending
// occurrence order and the permutation is unique.
//
// Kernels, in launch order:
//   k_keys          per occurrence j: key = off_t + id (out-of-range ids get
//                   the sentinel key total_rows, which sorts last), grad row
//                   s*T + t and, for mean pooling, 1/L of its bag; flags the
//                   batch as not one-hot when a bag's length is not 1.  The
//                   sort's value of occurrence j is j itself (not stored).
//   k_sort_hist     per 4096-key tile, digit counts -> tile_hist[digit][tile].
//   k_sort_scan     one block per digit: exclusive scan over tiles, digit totals.
//   k_sort_scatter  per tile: stable rank of every key (per-wave ballot match
//                   of the digit, waves own contiguous quarters of the tile),
//                   staging of the tile in LDS in digit order, then writes in
//                   which consecutive lanes store consecutive addresses.
//   (hist / scan / scatter once per digit; digits of at most 9 bits cover
//    ceil(log2(total_rows + 1)) key bits, so three passes sort 2^27 rows.
//    A batch of at most one tile takes the scatter alone per digit.)
//   k_chunk_heads   run heads per reduction chunk (ballot), and the number of
//                   valid (in-range) occurrences.
//   k_chunk_scan    one block: exclusive scan of the chunk head counts, giving
//                   the unique index of each chunk's first run; num_unique and
//                   seg_off[num_unique].
//   k_materialize   unique[u], seg_off[u] and inverse[perm[k]] for every sorted
//                   position k (u = run heads at or before k, minus one).
// These kernels need only the ids, so a caller can run them for the next batch
// beside this batch's forward and backward; the scattered inverse stores then
// stay off the training kernels' stream.  counts[u] = seg_off[u+1] - seg_off[u]
// (k_unique_counts) is formed only for the sort / unique export, since no
// training step reads it.
#include <atomic>

#include "embtab_internal.hpp"

namespace embtab {

namespace {

// Number of this key build among all key builds of the process (never 0).
// It tags the one-hot flag word of the workspace; being unique per process
// rather than per handle, a workspace that several handles share cannot hold
// a stale tag equal to the current one.
uint32_t next_prepare_gen() {
  static std::atomic<uint32_t> n{0};
  uint32_t g = n.fetch_add(1u, std::memory_order_relaxed) + 1u;
  if (g == 0u) g = n.fetch_add(1u, std::memory_order_relaxed) + 1u;
  return g;
}

// Exclusive scan of one value per thread over a 256-thread block.
__device__ inline uint32_t block_excl_scan(uint32_t v, uint32_t* total, uint32_t* lds4) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t x = v;
  x = wave_incl_scan(x);
  if (lane == 63) lds4[w] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t s = lds4[i];
    before += (i < w) ? s : 0u;
    all += s;
  }
  __syncthreads();
  if (total) *total = all;
  return x - v + before;
}

// One block per `bpb` consecutive bags in CSR order (bpb <= 256, chosen so
// a block covers about 256 occurrences).  Thread i < bpb checks bag b0 + i.
// When every bag of the block holds exactly the occurrence with its own index
// (one-hot features), thread i writes occurrence b0 + i directly from loads it
// issued beside the offsets (the id at its own index, its table's bounds),
// and the block is marked in place (its grad rows are not stored: occurrence
// j's is s*T + t of bag j).
// Otherwise the bag offsets go to LDS, and the block walks the occurrences
// [offsets[b0], offsets[b0 + bpb]) with consecutive threads on consecutive
// occurrences (coalesced id loads and key stores, whatever the bag lengths),
// finding each occurrence's bag by binary search in LDS.  The value of
// occurrence j is j itself, so it is not stored.  T * B < 2^32 (grad rows are
// 32-bit).
__global__ __launch_bounds__(256) void k_keys(const int64_t* __restrict__ offsets,
                                              const int64_t* __restrict__ ids,
                                              const int64_t* __restrict__ row_off,
                                              const int64_t* __restrict__ rows,
                                              uint32_t* __restrict__ keys,
                                              uint32_t* __restrict__ gr,
                                              uint32_t* __restrict__ flags,
                                              uint32_t* __restrict__ misc, int64_t B, int32_t T,
                                              int64_t nnz, uint32_t sentinel, int32_t mean,
                                              int32_t bpb, uint8_t* __restrict__ in_place_blk,
                                              uint32_t gen, int32_t nmisc) {
  __shared__ int64_t s_off[257];
  __shared__ uint32_t s_bad;
  if (blockIdx.x == 0) {
    // the prepare's counters start at zero; the one-hot flag is tagged instead
    for (int i = threadIdx.x; i < nmisc; i += 256)
      if (i != kMiscNotOneHot) misc[i] = i == kMiscPrepareGen ? gen : 0u;
  }
  const int64_t nbags = B * (int64_t)T;
  const int64_t b0 = (int64_t)blockIdx.x * bpb;
  const int64_t b = b0 + threadIdx.x;
  const int64_t nb = (nbags - b0) < bpb ? (nbags - b0) : bpb;  // bags of this block
  if (nb <= 0) return;  // empty batch (the grid has one block)
  if (threadIdx.x == 0) s_bad = 0u;
  const bool mine = threadIdx.x < nb;
  int64_t o0 = 0, o1 = 1, own_id = 0, own_rows = 0, own_off = 0;
  uint32_t own_t = 0;
  if (mine) {
    o0 = offsets[b];
    o1 = offsets[b + 1];
    own_t = (uint32_t)b / (uint32_t)B;
    own_rows = rows[own_t];
    own_off = row_off[own_t];
    if (b < nnz) own_id = ids[b];  // the id of bag b if the bag is one-hot in place
  }
  {
    const uint64_t mm = __ballot(o1 - o0 != 1);
    // a plain store of the prepare's tag: device atomics on one word from
    // every block would serialise
    if ((threadIdx.x & 63u) == 0u && mm != 0ull) misc[kMiscNotOneHot] = gen;
  }
  uint32_t bad = 0;
  if (mine) {
    if ((b == 0 && o0 != 0) || (b == nbags - 1 && o1 != nnz) || o1 < o0 || o0 < 0 || o1 > nnz)
      bad |= EMB_FLAG_BAD_OFFSETS;
    // clamped to [0, nnz]: with offsets that are not monotone the search
    // below still lands on a bag of this block, and the batch is flagged
    s_off[threadIdx.x] = o0 < 0 ? 0 : (o0 > nnz ? nnz : o0);
    if (threadIdx.x == nb - 1) s_off[nb] = o1 < 0 ? 0 : (o1 > nnz ? nnz : o1);
  }
  const bool in_place = !mine || (o0 == b && o1 == b + 1 && o1 <= nnz);
  if (__syncthreads_and(in_place)) {
    // the grad row of these occurrences follows from their index: the block
    // is recorded as in place and writes none
    if (threadIdx.x == 0) in_place_blk[blockIdx.x] = 1;
    if (mine) {
      uint32_t key = sentinel;
      if (own_id >= 0 && own_id < own_rows) key = (uint32_t)own_off + (uint32_t)own_id;
      else if (own_id != kAbsentId) bad |= EMB_FLAG_OUT_OF_RANGE;
      keys[b] = key;
    }
  } else {
    if (threadIdx.x == 0) in_place_blk[blockIdx.x] = 0;
    const int64_t j0 = s_off[0], j1 = s_off[nb];
    for (int64_t j = j0 + threadIdx.x; j < j1; j += 256) {
      // last bag i of the block with s_off[i] <= j (bags of length 0 are skipped)
      int lo = 0, hi = (int)nb - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_off[mid] <= j) lo = mid;
        else hi = mid - 1;
      }
      const int64_t bag = b0 + lo;
      const int64_t t = bag / B, s = bag - t * B;
      const int64_t id = ids[j];
      uint32_t key = sentinel;
      if (id >= 0 && id < rows[t]) key = (uint32_t)row_off[t] + (uint32_t)id;
      else if (id != kAbsentId) bad |= EMB_FLAG_OUT_OF_RANGE;
      keys[j] = key;
      const uint32_t g = (uint32_t)(s * T + t);
      if (mean)  // grad row and scale side by side: one gather in the last pass
        reinterpret_cast<uint2*>(gr)[j] =
            make_uint2(g, __float_as_uint(1.0f / (float)(s_off[lo + 1] - s_off[lo])));
      else
        gr[j] = g;
    }
  }
  if (bad) atomicOr(&s_bad, bad);
  __syncthreads();
  if (threadIdx.x == 0 && s_bad) atomicOr(flags, s_bad);
}

// Per-wave stable digit ranking of 64 keys: returns the lanes of this wave that
// share the digit (mask) for valid lanes.
__device__ inline uint64_t match_digit(uint32_t d, bool valid, int nbits) {
  uint64_t m = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (d >> b) & 1u;
    const uint64_t bb = __ballot(bit);
    m &= bit ? bb : ~bb;
  }
  return m;
}

__global__ __launch_bounds__(256) void k_sort_hist(const uint32_t* __restrict__ keys, uint32_t n,
                                                   int shift, int nbits,
                                                   uint32_t* __restrict__ tile_hist,
                                                   uint32_t ntiles) {
  __shared__ uint32_t whist[4][kMaxRadix];
  const int radix = 1 << nbits;
  const uint32_t mask = (uint32_t)radix - 1u;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < 4 * kMaxRadix; i += 256) (&whist[0][0])[i] = 0u;
  // XCD-contiguous tiles: the per-digit counts of neighbouring tiles share
  // cache lines of tile_hist
  const uint32_t tile = xcd_block();
  const uint32_t base = tile * (uint32_t)kSortTile + (uint32_t)w * (kSortItems * 64);
  uint32_t kv[kSortItems];
#pragma unroll
  for (int r = 0; r < kSortItems; ++r) {
    const uint32_t idx = base + r * 64 + lane;
    kv[r] = idx < n ? keys[idx] : 0u;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kSortItems; ++r) {
    const uint32_t idx = base + r * 64 + lane;
    const bool valid = idx < n;
    const uint32_t d = (kv[r] >> shift) & mask;
    const uint64_t m = match_digit(d, valid, nbits);
    if (valid && lanes_below(m) == 0u) whist[w][d] += (uint32_t)__popcll(m);
  }
  __syncthreads();
  for (int d = threadIdx.x; d < radix; d += 256)
    tile_hist[(size_t)d * ntiles + tile] = whist[0][d] + whist[1][d] + whist[2][d] + whist[3][d];
}

__global__ __launch_bounds__(256) void k_sort_scan(uint32_t* __restrict__ tile_hist,
                                                   uint32_t ntiles,
                                                   uint32_t* __restrict__ digit_tot) {
  __shared__ uint32_t lds4[4];
  uint32_t* row = tile_hist + (size_t)blockIdx.x * ntiles;
  uint32_t carry = 0;
  for (uint32_t base = 0; base < ntiles; base += 256 * 4) {
    uint32_t v[4];
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t idx = base + threadIdx.x * 4 + i;
      v[i] = idx < ntiles ? row[idx] : 0u;
      sum += v[i];
    }
    uint32_t total;
    uint32_t ex = block_excl_scan(sum, &total, lds4) + carry;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t idx = base + threadIdx.x * 4 + i;
      if (idx < ntiles) row[idx] = ex;
      ex += v[i];
    }
    carry += total;
  }
  if (threadIdx.x == 0) digit_tot[blockIdx.x] = carry;
}

// FIRST: the values are the positions themselves (not read).  The last pass
// (gr_out != nullptr) also gathers each sorted occurrence's grad row (and
// mean scale) into sorted order, so the consumers of the sort read them with
// coalesced loads; a stale occurrence index gets the invalid grad row
// 0xFFFFFFFF.  When every bag holds one id (a flag of k_keys) the grad row
// follows from the occurrence index and the consumers compute it from perm.
template <bool FIRST>
__global__ __launch_bounds__(256) void k_sort_scatter(
    const uint32_t* __restrict__ keys_in, const uint32_t* __restrict__ vals_in,
    uint32_t* __restrict__ keys_out, uint32_t* __restrict__ vals_out, uint32_t n, int shift,
    int nbits, const uint32_t* __restrict__ tile_off, const uint32_t* __restrict__ digit_tot,
    uint32_t ntiles, const uint32_t* __restrict__ gr_in, uint32_t* __restrict__ gr_out,
    float* __restrict__ sc_out, const uint32_t* __restrict__ misc, uint32_t B, uint32_t T,
    const uint8_t* __restrict__ in_place_blk, uint32_t bpb, uint32_t nkblk) {
  __shared__ uint32_t whist[4][kMaxRadix];
  __shared__ uint32_t dstart[kMaxRadix];
  __shared__ uint32_t gbase[kMaxRadix];
  __shared__ uint32_t skeys[kSortTile];
  __shared__ uint32_t svals[kSortTile];
  __shared__ uint32_t lds4[4];
  const int radix = 1 << nbits;
  const uint32_t mask = (uint32_t)radix - 1u;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // XCD-contiguous tiles: a digit's runs from neighbouring tiles share cache
  // lines of the output, so their partial-line stores meet in one L2
  const uint32_t tile = xcd_block();
  for (int i = threadIdx.x; i < 4 * kMaxRadix; i += 256) (&whist[0][0])[i] = 0u;
  const uint32_t base = tile * (uint32_t)kSortTile + (uint32_t)w * (kSortItems * 64);
  uint32_t kv[kSortItems], vv[kSortItems], lr[kSortItems];
#pragma unroll
  for (int r = 0; r < kSortItems; ++r) {
    const uint32_t idx = base + r * 64 + lane;
    kv[r] = 0u;
    vv[r] = idx;
    if (idx < n) {
      kv[r] = keys_in[idx];
      if (!FIRST) vv[r] = vals_in[idx];
    }
  }
  __syncthreads();
  // Stable rank inside the wave's quarter: rounds go in position order.
#pragma unroll
  for (int r = 0; r < kSortItems; ++r) {
    const uint32_t idx = base + r * 64 + lane;
    const bool valid = idx < n;
    const uint32_t d = (kv[r] >> shift) & mask;
    const uint64_t m = match_digit(d, valid, nbits);
    const uint32_t below = lanes_below(m);
    uint32_t old = 0u;
    if (valid) old = whist[w][d];
    if (valid && below == 0u) whist[w][d] = old + (uint32_t)__popcll(m);
    lr[r] = old + below;
  }
  __syncthreads();
  // Per digit: exclusive prefix over waves; tile count into dstart.
  for (int d = threadIdx.x; d < radix; d += 256) {
    const uint32_t c0 = whist[0][d], c1 = whist[1][d], c2 = whist[2][d], c3 = whist[3][d];
    whist[0][d] = 0u;
    whist[1][d] = c0;
    whist[2][d] = c0 + c1;
    whist[3][d] = c0 + c1 + c2;
    dstart[d] = c0 + c1 + c2 + c3;
  }
  __syncthreads();
  {
    // Tile-local digit starts and global digit bases (radix <= 512: two per thread).
    // A single tile's own counts are the digit totals and its offsets are 0,
    // so the histogram and scan launches are skipped and nothing is read.
    const bool solo = ntiles == 1u;
    const int d0 = 2 * threadIdx.x, d1 = d0 + 1;
    const uint32_t a0 = d0 < radix ? dstart[d0] : 0u, a1 = d1 < radix ? dstart[d1] : 0u;
    const uint32_t t0 = solo ? a0 : (d0 < radix ? digit_tot[d0] : 0u);
    const uint32_t t1 = solo ? a1 : (d1 < radix ? digit_tot[d1] : 0u);
    const uint32_t ea = block_excl_scan(a0 + a1, nullptr, lds4);
    const uint32_t et = block_excl_scan(t0 + t1, nullptr, lds4);
    if (d0 < radix) {
      dstart[d0] = ea;
      gbase[d0] = et + (solo ? 0u : tile_off[(size_t)d0 * ntiles + tile]);
    }
    if (d1 < radix) {
      dstart[d1] = ea + a0;
      gbase[d1] = et + t0 + (solo ? 0u : tile_off[(size_t)d1 * ntiles + tile]);
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kSortItems; ++r) {
    const uint32_t idx = base + r * 64 + lane;
    if (idx < n) {
      const uint32_t d = (kv[r] >> shift) & mask;
      const uint32_t pos = dstart[d] + whist[w][d] + lr[r];
      skeys[pos] = kv[r];
      svals[pos] = vv[r];
    }
  }
  __syncthreads();
  const uint32_t tbase = tile * (uint32_t)kSortTile;
  const uint32_t tn = (n - tbase) < (uint32_t)kSortTile ? (n - tbase) : (uint32_t)kSortTile;
  const bool one_hot = gr_out && !batch_not_one_hot(misc);
  for (uint32_t i = threadIdx.x; i < tn; i += 256) {
    const uint32_t k = skeys[i];
    const uint32_t d = (k >> shift) & mask;
    const uint32_t g = gbase[d] + (i - dstart[d]);
    const uint32_t v = svals[i];
    keys_out[g] = k;
    vals_out[g] = v;
    // one-hot batches: the consumers take the grad row from the occurrence
    // index (perm) itself, so nothing more is written
    if (gr_out && !one_hot) {
      // occurrences of in-place key blocks: bag v, length 1 (key block v / bpb
      // holds exactly occurrences v of its own bags when it is in place)
      const bool ip = v < n && v / bpb < nkblk && in_place_blk[v / bpb] != 0;
      if (sc_out) {  // (grad row, scale) pairs
        const uint2 x = ip ? make_uint2(one_hot_grad_row(v, B, T), __float_as_uint(1.0f))
                           : (v < n ? reinterpret_cast<const uint2*>(gr_in)[v]
                                    : make_uint2(0xFFFFFFFFu, 0u));
        gr_out[g] = x.x;
        sc_out[g] = __uint_as_float(x.y);
      } else {
        gr_out[g] = ip ? one_hot_grad_row(v, B, T) : (v < n ? gr_in[v] : 0xFFFFFFFFu);
      }
    }
  }
}

// Run heads (first position of each distinct valid key) per reduction chunk
// of CH positions.  A block covers 256 positions = 256 / CH chunks: each
// chunk gets the number of heads in the block's earlier chunks (cloc) and
// the block its total (btot), which k_chunk_scan turns into block bases.
template <int CH>
__global__ __launch_bounds__(256) void k_chunk_heads(const uint32_t* __restrict__ keys, uint32_t n,
                                                     uint32_t sentinel,
                                                     uint32_t* __restrict__ cloc,
                                                     uint32_t* __restrict__ btot,
                                                     uint32_t* __restrict__ misc) {
  constexpr int CPB = 256 / CH;
  __shared__ uint32_t s_cnt[CPB];
  const uint32_t blk = xcd_block();  // neighbouring blocks' counts share cache lines
  const uint32_t k = blk * 256u + threadIdx.x;
  bool head = false;
  if (k < n) {
    const uint32_t key = keys[k];
    if (key < sentinel) {
      head = (k == 0) || keys[k - 1] != key;
      if (k + 1 == n || keys[k + 1] >= sentinel) misc[kMiscNumValid] = k + 1;
    }
  }
  const uint64_t m = __ballot(head);
  const uint32_t lane = threadIdx.x & 63u;
  if ((lane % CH) == 0u) {
    const uint64_t bits = CH == 64 ? m : (m >> lane) & ((1ull << CH) - 1ull);
    s_cnt[threadIdx.x / CH] = (uint32_t)__popcll(bits);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t nch = (n + CH - 1) / CH;
    uint32_t run = 0;
#pragma unroll
    for (int i = 0; i < CPB; ++i) {
      const uint32_t c = blk * CPB + i;
      if (c < nch) cloc[c] = run;
      run += s_cnt[i];
    }
    btot[blk] = run;
  }
}

// Exclusive scan of the per-block head totals in one block (in place): each
// pass covers 1024 threads x 32 consecutive counts, read and written with
// dwordx4 accesses.  The unique index of the first run head of reduction
// chunk c is then btot[c / (256 / CH)] + cloc[c].
__global__ __launch_bounds__(1024) void k_chunk_scan(uint32_t* __restrict__ hc, uint32_t nchunks,
                                                     uint32_t* __restrict__ misc,
                                                     uint32_t* __restrict__ seg_off) {
  constexpr uint32_t PER = 32;
  __shared__ uint32_t wsum[16];
  const uint32_t lane = threadIdx.x & 63u, w = threadIdx.x >> 6;
  uint32_t carry = 0;
  for (uint32_t base = 0; base < nchunks; base += 1024u * PER) {
    const uint32_t lo = base + threadIdx.x * PER;
    uint32_t v[PER];
    if (lo + PER <= nchunks) {
#pragma unroll
      for (int q = 0; q < (int)PER / 4; ++q) {
        const uint4 x = reinterpret_cast<const uint4*>(hc + lo)[q];
        v[4 * q] = x.x;
        v[4 * q + 1] = x.y;
        v[4 * q + 2] = x.z;
        v[4 * q + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int q = 0; q < (int)PER; ++q) v[q] = lo + q < nchunks ? hc[lo + q] : 0u;
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
    if (lo + PER <= nchunks) {
#pragma unroll
      for (int q = 0; q < (int)PER / 4; ++q)
        reinterpret_cast<uint4*>(hc + lo)[q] = make_uint4(v[4 * q], v[4 * q + 1], v[4 * q + 2],
                                                          v[4 * q + 3]);
    } else {
#pragma unroll
      for (int q = 0; q < (int)PER; ++q)
        if (lo + q < nchunks) hc[lo + q] = v[q];
    }
    carry += total;
  }
  if (threadIdx.x == 0) {
    hc[nchunks] = carry;
    misc[kMiscNumUnique] = carry;
    seg_off[carry] = misc[kMiscNumValid];
  }
}

__global__ __launch_bounds__(256) void k_unique_counts(const uint32_t* __restrict__ seg_off,
                                                       const uint32_t* __restrict__ misc,
                                                       uint32_t* __restrict__ counts, uint32_t n) {
  const uint32_t U = misc[kMiscNumUnique];
  for (uint32_t u = blockIdx.x * 256 + threadIdx.x; u < U && u < n; u += gridDim.x * 256)
    counts[u] = seg_off[u + 1] - seg_off[u];
}

__global__ __launch_bounds__(256) void k_copy_sorted(const uint32_t* __restrict__ keys,
                                                     uint32_t sentinel, uint32_t* __restrict__ out,
                                                     int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const uint32_t k = keys[i];
    out[i] = k >= sentinel ? kNoRow : k;
  }
}

// unique / seg_off / inverse from the sorted keys: position k's unique index
// is the number of run heads at or before k, minus one (block bases from the
// scanned head totals).  At the first position of every reduction block (bp
// positions each) it also records the run that crosses the block's leading
// edge (its unique index, or kNoRow) and zeroes the block's span counter.
__global__ __launch_bounds__(256) void k_materialize(const uint32_t* __restrict__ keys,
                                                     const uint32_t* __restrict__ perm, uint32_t n,
                                                     uint32_t sentinel,
                                                     const uint32_t* __restrict__ hbase,
                                                     uint32_t* __restrict__ unique,
                                                     uint32_t* __restrict__ seg_off,
                                                     uint32_t* __restrict__ inverse, uint32_t bp,
                                                     uint32_t* __restrict__ span_u,
                                                     uint32_t* __restrict__ span_cnt) {
  __shared__ uint32_t wcnt[4];
  // XCD-contiguous blocks: the inverse stores of neighbouring sorted positions
  // (one table's occurrences, a narrow range of inverse) meet in one L2
  const uint32_t blk = xcd_block();
  const uint32_t k = blk * 256u + threadIdx.x;
  const uint32_t lane = threadIdx.x & 63u, wv = threadIdx.x >> 6;
  uint32_t key = sentinel;
  bool head = false;
  if (k < n) {
    key = keys[k];
    head = key < sentinel && (k == 0 || keys[k - 1] != key);
  }
  const uint64_t m = __ballot(head);
  if (lane == 0) wcnt[wv] = (uint32_t)__popcll(m);
  __syncthreads();
  uint32_t before = hbase[blk];
  for (uint32_t i = 0; i < wv; ++i) before += wcnt[i];
  const uint32_t incl = before + lanes_below(m) + (head ? 1u : 0u);
  if (k < n) {
    const uint32_t j = perm[k];
    const uint32_t u = incl - 1u;
    if (j < n) inverse[j] = key < sentinel ? u : kNoRow;
    if (head) {
      unique[u] = key;
      seg_off[u] = k;
    }
    if (k % bp == 0u) {
      span_u[k / bp] = (key < sentinel && !head) ? u : kNoRow;
      span_cnt[k / bp] = 0u;
    }
  }
}

}  // namespace

hipError_t launch_sort_unique(
const Handle& h, const Plan& p, const int64_t* offsets,
                              const int64_t* ids, bool mean, char* ws, uint32_t** sorted_keys,
                              uint32_t** sorted_vals, hipStream_t s) {
  const uint32_t n = (uint32_t)p.nnz;
  const uint32_t sentinel = (uint32_t)h.total_rows;
  uint32_t* misc = reinterpret_cast<uint32_t*>(ws + p.misc);
  uint32_t* kA = reinterpret_cast<uint32_t*>(ws + p.keysA);
  uint32_t* vA = reinterpret_cast<uint32_t*>(ws + p.valsA);
  uint32_t* kB = reinterpret_cast<uint32_t*>(ws + p.keysB);
  uint32_t* vB = reinterpret_cast<uint32_t*>(ws + p.valsB);
  uint32_t* gr = reinterpret_cast<uint32_t*>(ws + p.gr);
  uint32_t* tile_hist = reinterpret_cast<uint32_t*>(ws + p.tile_hist);
  uint32_t* digit_tot = reinterpret_cast<uint32_t*>(ws + p.digit_tot);
  uint32_t* seg_off = reinterpret_cast<uint32_t*>(ws + p.seg_off);
  uint32_t* cbase = reinterpret_cast<uint32_t*>(ws + p.chunk_base);

  const int64_t nbags = p.B * (int64_t)h.T;
  // bags per key block: a power of two near 256 / (mean bag length)
  int bpb = 256;
  while (bpb > 1 && (int64_t)bpb * p.nnz > 256 * nbags * 2) bpb >>= 1;
  const unsigned kgrid = (unsigned)((nbags + bpb - 1) / bpb);
  phase_mark(h, EMB_PHASE_KEYS, false, s);
  uint8_t* in_place_blk = reinterpret_cast<uint8_t*>(ws + p.kblk);
  uint32_t gen = next_prepare_gen();
  hipLaunchKernelGGL(k_keys, dim3(kgrid > 0 ? kgrid : 1), dim3(256), 0, s, offsets, ids,
                     h.sv.row_off, h.sv.rows, kA, gr, h.sv.flags, misc, p.B, h.T,
                     p.nnz, sentinel, mean ? 1 : 0, bpb, in_place_blk, gen, 64 + 2 * h.T);
  hipError_t e;
  phase_mark(h, EMB_PHASE_KEYS, true, s);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint32_t ntiles = (uint32_t)p.ntiles;
  uint32_t* kin = kA;
  uint32_t* vin = vA;
  uint32_t* kout = kB;
  uint32_t* vout = vB;
  phase_mark(h, EMB_PHASE_SORT, false, s);
  if (n > 0) {
    for (int pass = 0; pass < p.passes; ++pass) {
      const int radix = 1 << p.dbits[pass];
      if (ntiles > 1) {  // a single tile ranks itself inside the scatter
        hipLaunchKernelGGL(k_sort_hist, dim3(ntiles), dim3(256), 0, s, kin, n, p.shift[pass],
                           p.dbits[pass], tile_hist, ntiles);
        hipLaunchKernelGGL(k_sort_scan, dim3(radix), dim3(256), 0, s, tile_hist, ntiles,
                           digit_tot);
      }
      const bool last = pass + 1 == p.passes;
      uint32_t* gro = last ? reinterpret_cast<uint32_t*>(ws + p.sgr) : nullptr;
      float* sco = (last && mean) ? reinterpret_cast<float*>(ws + p.sscale) : nullptr;
      if (pass == 0)
        hipLaunchKernelGGL(k_sort_scatter<true>, dim3(ntiles), dim3(256), 0, s, kin, vin, kout,
                           vout, n, p.shift[pass], p.dbits[pass], tile_hist, digit_tot, ntiles, gr,
                           gro, sco, misc, (uint32_t)p.B, (uint32_t)h.T, in_place_blk,
                           (uint32_t)bpb, kgrid);
      else
        hipLaunchKernelGGL(k_sort_scatter<false>, dim3(ntiles), dim3(256), 0, s, kin, vin, kout,
                           vout, n, p.shift[pass], p.dbits[pass], tile_hist, digit_tot, ntiles, gr,
                           gro, sco, misc, (uint32_t)p.B, (uint32_t)h.T, in_place_blk,
                           (uint32_t)bpb, kgrid);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      uint32_t* tk = kin;
      kin = kout;
      kout = tk;
      uint32_t* tv = vin;
      vin = vout;
      vout = tv;
    }
  }
  phase_mark(h, EMB_PHASE_SORT, true, s);
  phase_mark(h, EMB_PHASE_UNIQUE, false, s);
  const unsigned hgrid = (unsigned)((n + 255) / 256);
  uint32_t* btot = reinterpret_cast<uint32_t*>(ws + p.head_base);
  if (n > 0) {
    if (p.chunk == 64)
      hipLaunchKernelGGL((k_chunk_heads<64>), dim3(hgrid), dim3(256), 0, s, kin, n, sentinel,
                         cbase, btot, misc);
    else
      hipLaunchKernelGGL((k_chunk_heads<32>), dim3(hgrid), dim3(256), 0, s, kin, n, sentinel,
                         cbase, btot, misc);
  }
  hipLaunchKernelGGL(k_chunk_scan, dim3(1), dim3(1024), 0, s, btot, hgrid, misc, seg_off);
  if (n > 0)
    hipLaunchKernelGGL(k_materialize, dim3(hgrid), dim3(256), 0, s, kin, vin, n, sentinel, btot,
                       reinterpret_cast<uint32_t*>(ws + p.unique), seg_off,
                       reinterpret_cast<uint32_t*>(ws + p.inverse), p.bp,
                       reinterpret_cast<uint32_t*>(ws + p.span_u),
                       reinterpret_cast<uint32_t*>(ws + p.span_cnt));
  phase_mark(h, EMB_PHASE_UNIQUE, true, s);
  *sorted_keys = kin;
  *sorted_vals = vin;
  return hipGetLastError();
}

hipError_t launch_unique_counts(const Plan& p, char* ws, hipStream_t s) {
  const uint32_t n = (uint32_t)p.nnz;
  if (n == 0) return hipSuccess;
  const uint32_t* misc = reinterpret_cast<const uint32_t*>(ws + p.misc);
  const uint32_t* seg_off = reinterpret_cast<const uint32_t*>(ws + p.seg_off);
  uint32_t* counts = reinterpret_cast<uint32_t*>(ws + p.counts);
  const unsigned cgrid = (unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
  hipLaunchKernelGGL(k_unique_counts, dim3(cgrid), dim3(256), 0, s, seg_off, misc, counts, n);
  return hipGetLastError();
}

hipError_t launch_debug_copy_sorted(const uint32_t* keys, uint32_t sentinel, uint32_t* out,
                                    int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int64_t g = (n + 255) / 256;
  hipLaunchKernelGGL(k_copy_sorted, dim3((unsigned)(g < 4096 ? g : 4096)), dim3(256), 0, s, keys,
                     sentinel, out, n);
  return hipGetLastError();
}

}  // namespace embtab
