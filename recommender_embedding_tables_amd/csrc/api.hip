// C ABI of the sparse embedding library (declared in include/embtab.h):
// host-side validation, workspace planning and the launch sequence of each
// call on the caller's stream.  No device memory is allocated here.
#include <cmath>
#include <cstring>
#include <mutex>
#include <new>

#include "embtab_internal.hpp"
#include "interact.hpp"

// The workspace of emb_bag_backward_adagrad_noalloc: one copy per device,
// held from the library's load onto that device until the process ends.
// Host code never uses this name as an address (on the host it is only a
// stand-in); it uses the device address resolved for each device below.
static __device__ __align__(256) unsigned char scratch[EMB_NOALLOC_SCRATCH_BYTES];

namespace embtab {

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};  // address of `scratch` on each device

// Address of `dev`'s copy of `scratch`, resolved once per device; `dev` must
// be the current device.  Null when the runtime cannot give it.
void* device_scratch(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess && p != nullptr)
      g_scratch[dev] = p;
    else
      (void)hipGetLastError();
  }
  return g_scratch[dev];
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

int bit_width(uint64_t v) {
  int b = 0;
  while (v) {
    ++b;
    v >>= 1;
  }
  return b;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

emb_status_t hip_status(hipError_t e) { return e == hipSuccess ? EMB_OK : EMB_ERR_HIP; }

}  // namespace

bool make_plan(const Handle& h, int64_t B, int64_t nnz, Plan* p) {
  if (B < 0 || nnz < 0 || nnz >= 0xFFFFFFF0ll) return false;
  if (B * (int64_t)h.T >= 0xFFFFFFF0ll) return false;
  p->nnz = nnz;
  p->B = B;
  p->T = h.T;
  p->D = h.D;
  int bits = bit_width((uint64_t)h.total_rows);  // the sentinel total_rows must fit
  if (bits < 1) bits = 1;
  p->passes = (bits + kMaxDigitBits - 1) / kMaxDigitBits;
  int base = bits / p->passes, extra = bits % p->passes, sh = 0;
  for (int i = 0; i < p->passes; ++i) {
    p->dbits[i] = base + (i < extra ? 1 : 0);
    p->shift[i] = sh;
    sh += p->dbits[i];
  }
  p->ntiles = (nnz + kSortTile - 1) / kSortTile;
  p->chunk = chunk_len(h.D);
  p->nchunks = (nnz + p->chunk - 1) / p->chunk;
  const size_t n4 = sizeof(uint32_t) * (size_t)(nnz > 0 ? nnz : 1);
  const size_t nt = (size_t)(p->ntiles > 0 ? p->ntiles : 1);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o += align_up(bytes);
    return at;
  };
  p->misc = take(sizeof(uint32_t) * misc_words(h.T));
  p->keysA = take(n4);
  p->valsA = take(n4);
  p->keysB = take(n4);
  p->valsB = take(n4);
  p->gr = take(2 * n4);  // grad row, or (grad row, mean scale) pairs
  p->kblk = take((size_t)(B * (int64_t)h.T) + 1);  // at most one key block per bag
  p->sgr = take(n4);
  p->sscale = take(n4);
  p->tile_hist = take(sizeof(uint32_t) * kMaxRadix * nt);
  p->digit_tot = take(sizeof(uint32_t) * kMaxRadix);
  p->unique = take(n4);
  p->seg_off = take(n4 + sizeof(uint32_t));
  p->counts = take(n4);
  p->inverse = take(n4);
  const size_t nc = (size_t)(p->nchunks > 0 ? p->nchunks : 1);
  p->part_head = take(sizeof(float) * nc * (size_t)h.D);
  p->part_tail = take(sizeof(float) * nc * (size_t)h.D);
  p->span_u = take(sizeof(uint32_t) * (nc + 2));
  p->span_cnt = take(sizeof(uint32_t) * (nc + 2));
  p->bp = reduce_block_positions(h.D);
  p->chunk_base = take(sizeof(uint32_t) * (nc + 1));
  p->head_base = take(sizeof(uint32_t) * ((size_t)(nnz + 255) / 256 + 1));
  if (h.hashed) {
    p->h_slot = take(n4);
    p->h_first = take(n4);
    p->h_tcnt = take(sizeof(uint32_t) * (size_t)((nnz + 255) / 256 + 1));
    p->h_tb = take(sizeof(int64_t) * (size_t)(h.T + 1));
    p->h_fresh = take((size_t)(nnz > 0 ? nnz : 1));
  } else {
    p->h_slot = p->h_first = p->h_tcnt = p->h_tb = p->h_fresh = 0;
  }
  if (h.tiered) {
    p->c_slot = take(n4);       // cache slot of each distinct row
    p->c_miss = take(2 * n4);   // misses: unique index, then row
    p->c_vict = take(n4);       // evicted row of each miss
    p->c_mslot = take(n4);      // slot of each miss
    p->c_rowmap = take(n4);     // slot of each occurrence (batches that are not one-hot)
  } else {
    p->c_slot = p->c_miss = p->c_vict = p->c_mslot = p->c_rowmap = 0;
  }
  p->total = o;
  return true;
}

}  // namespace embtab

using namespace embtab;

struct emb_table_s {
  Handle h;
};

extern "C" {

size_t emb_state_bytes(int32_t num_tables) {
  if (num_tables < 1 || num_tables > (1 << 20)) return 0;
  return state_bytes(num_tables);
}

size_t emb_hash_bytes(int32_t num_tables, int64_t capacity) {
  if (num_tables < 1 || capacity < 16 || (capacity & (capacity - 1)) != 0 ||
      capacity > (1ll << 31))
    return 0;
  return (size_t)num_tables * (size_t)capacity * 16u;
}

size_t emb_workspace_bytes(emb_table_t t, int64_t batch, int64_t nnz) {
  if (!t) return 0;
  Plan p;
  if (!make_plan(t->h, batch, nnz, &p)) return 0;
  return p.total;
}

const char* emb_status_string(emb_status_t s) {
  switch (s) {
    case EMB_OK: return "ok";
    case EMB_ERR_INVALID_ARG: return "invalid argument";
    case EMB_ERR_UNSUPPORTED: return "unsupported";
    case EMB_ERR_WORKSPACE: return "workspace too small";
    case EMB_ERR_OUT_OF_RANGE: return "id out of range";
    case EMB_ERR_BAD_OFFSETS: return "bad offsets";
    case EMB_ERR_RESERVED_KEY: return "reserved key";
    case EMB_ERR_TABLE_FULL: return "table full";
    case EMB_ERR_HIP: return "HIP runtime error";
    case EMB_ERR_CACHE_FULL: return "cache set full";
  }
  return "unknown status";
}

static emb_status_t create_impl(const emb_table_desc_t* d, const emb_tier_desc_t* tier,
                                void* stream, emb_table_t* out) {
  if (!d || !out) return EMB_ERR_INVALID_ARG;
  *out = nullptr;
  if (d->num_tables < 1 || d->num_tables > 1024) return EMB_ERR_INVALID_ARG;
  if (d->dim < 4 || d->dim > 1024 || d->dim % 4 != 0) return EMB_ERR_INVALID_ARG;
  if (!d->rows_per_table || !d->weights || !d->accum || !d->state) return EMB_ERR_INVALID_ARG;
  if (!aligned16(d->weights) || !aligned16(d->accum) ||
      (reinterpret_cast<uintptr_t>(d->state) & 255u) != 0)
    return EMB_ERR_INVALID_ARG;
  int64_t total = 0;
  for (int t = 0; t < d->num_tables; ++t) {
    if (d->rows_per_table[t] < 1) return EMB_ERR_INVALID_ARG;
    total += d->rows_per_table[t];
    if (total >= 0xFFFFFFFFll) return EMB_ERR_UNSUPPORTED;  // rows are 32-bit inside
  }
  if (d->hashed) {
    if (emb_hash_bytes(d->num_tables, d->hash_capacity) == 0 || !d->hash_slots ||
        !aligned16(d->hash_slots) || (reinterpret_cast<uintptr_t>(d->free_rows) & 3u) != 0)
      return EMB_ERR_INVALID_ARG;
    if (!(d->max_load > 0.0f && d->max_load <= 0.9f)) return EMB_ERR_INVALID_ARG;
    for (int t = 0; t < d->num_tables; ++t)
      if ((double)d->rows_per_table[t] > (double)d->max_load * (double)d->hash_capacity)
        return EMB_ERR_INVALID_ARG;
  }
  if (tier) {
    if (d->hashed) return EMB_ERR_UNSUPPORTED;
    if (!tier->host_weights || !tier->host_accum || !tier->cache_state ||
        !aligned16(tier->host_weights) || !aligned16(tier->host_accum) ||
        (reinterpret_cast<uintptr_t>(tier->cache_state) & 255u) != 0)
      return EMB_ERR_INVALID_ARG;
    if (emb_cache_state_bytes(tier->cache_rows) == 0 || tier->cache_rows > total)
      return EMB_ERR_INVALID_ARG;
  }
  emb_table_s* tb = new (std::nothrow) emb_table_s();
  if (!tb) return EMB_ERR_INVALID_ARG;
  Handle& h = tb->h;
  if (tier) {
    h.tiered = true;
    h.hostW = tier->host_weights;
    h.hostG = tier->host_accum;
    h.cache_rows = tier->cache_rows;
    h.cache_sets = (uint32_t)(tier->cache_rows / kCacheWays);
    h.cache_state = static_cast<char*>(tier->cache_state);
  }
  h.T = d->num_tables;
  h.D = d->dim;
  h.rows.assign(d->rows_per_table, d->rows_per_table + h.T);
  h.row_off.assign(h.T + 1, 0);
  for (int t = 0; t < h.T; ++t) h.row_off[t + 1] = h.row_off[t] + h.rows[t];
  h.total_rows = h.row_off[h.T];
  h.W = d->weights;
  h.G = d->accum;
  h.state = d->state;
  h.sv = state_view(d->state, h.T);
  h.hashed = d->hashed != 0;
  h.capacity = h.hashed ? d->hash_capacity : 0;
  h.slots = h.hashed ? d->hash_slots : nullptr;
  h.free_rows = h.hashed ? d->free_rows : nullptr;
  h.seed = d->seed;
  h.lo = d->init_lo;
  h.hi = d->init_hi;
  h.stdv = d->init_std;
  h.accum0 = d->accum_init;
  {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        cus > 0) {
      h.cus = cus;
      h.device = dev;
      h.scratch = device_scratch(dev);
    } else {
      (void)hipGetLastError();  // no device visible: keep the default
    }
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (!d->init_storage && h.tiered) {
    // attach: the host arrays hold every row (the earlier handle flushed its
    // cache); the cache starts empty, its recency stamps with this handle
    e = launch_cache_init(h, s);
  }
  if (d->init_storage) {
    // state: flags 0, row offsets, capacities, live rows 0
    std::vector<int64_t> host(6 * (size_t)h.T + 1, 0);  // + free-row queues, slots: empty
    for (int t = 0; t <= h.T; ++t) host[t] = h.row_off[t];
    for (int t = 0; t < h.T; ++t) host[h.T + 1 + t] = h.rows[t];
    e = hipMemsetAsync(h.sv.flags, 0, 256, s);
    if (e == hipSuccess)
      e = hipMemcpyAsync(h.sv.row_off, host.data(), sizeof(int64_t) * host.size(),
                         hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);  // `host` goes out of scope
    if (e == hipSuccess && h.tiered) {
      // the table's rows live in host memory; the cache starts empty
      Handle hh = h;
      hh.W = h.hostW;
      hh.G = h.hostG;
      e = launch_init_dense(hh, s);
      if (e == hipSuccess) e = launch_cache_init(h, s);
    } else if (e == hipSuccess) {
      e = launch_init_dense(h, s);
    }
    if (e == hipSuccess && h.hashed)
      e = launch_fill_u64(static_cast<uint64_t*>(h.slots), kEmptyKey,
                          2 * (size_t)h.T * (size_t)h.capacity, s);
  }
  if (e != hipSuccess) {
    delete tb;
    return EMB_ERR_HIP;
  }
  *out = tb;
  return EMB_OK;
}

emb_status_t emb_table_create(const emb_table_desc_t* d, void* stream, emb_table_t* out) {
  return create_impl(d, nullptr, stream, out);
}

size_t emb_cache_state_bytes(int64_t cache_rows) {
  if (cache_rows < kCacheWays || cache_rows % kCacheWays != 0) return 0;
  const int64_t sets = cache_rows / kCacheWays;
  if ((sets & (sets - 1)) != 0 || cache_rows >= 0xFFFFFFFFll) return 0;
  return cache_state_bytes(cache_rows);
}

emb_status_t emb_table_create_tiered(const emb_table_desc_t* d, const emb_tier_desc_t* tier,
                                     void* stream, emb_table_t* out) {
  if (!tier) return EMB_ERR_INVALID_ARG;
  return create_impl(d, tier, stream, out);
}

emb_status_t emb_cache_flush(emb_table_t t, void* stream) {
  if (!t) return EMB_ERR_INVALID_ARG;
  if (!t->h.tiered) return EMB_ERR_UNSUPPORTED;
  return hip_status(launch_cache_flush(t->h, static_cast<hipStream_t>(stream)));
}

emb_status_t emb_cache_stats(emb_table_t t, void* stream, int64_t* lookups, int64_t* misses,
                             int64_t* writebacks) {
  if (!t || !lookups || !misses || !writebacks) return EMB_ERR_INVALID_ARG;
  if (!t->h.tiered) return EMB_ERR_UNSUPPORTED;
  uint64_t c[3] = {0, 0, 0};
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e == hipSuccess) e = hipMemcpy(c, t->h.cache_state, sizeof(c), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return EMB_ERR_HIP;
  *lookups = (int64_t)c[0];
  *misses = (int64_t)c[1];
  *writebacks = (int64_t)c[2];
  return EMB_OK;
}

emb_status_t emb_table_destroy(emb_table_t t) {
  delete t;
  return EMB_OK;
}

// The sort's key buffer that does not hold the final sorted keys.
static uint32_t* spare_keys(const Plan& p, char* w) {
  const bool in_b = p.nnz > 0 && (p.passes % 2) == 1;
  return reinterpret_cast<uint32_t*>(w + (in_b ? p.keysA : p.keysB));
}

static emb_status_t check_batch(const Handle& h, const int64_t* offsets, int64_t batch,
                                int64_t nnz) {
  if (!offsets || batch < 0 || nnz < 0) return EMB_ERR_INVALID_ARG;
  if (nnz >= 0xFFFFFFF0ll || batch * (int64_t)h.T >= 0xFFFFFFF0ll) return EMB_ERR_UNSUPPORTED;
  return EMB_OK;
}

emb_status_t emb_bag_forward(emb_table_t t, const int64_t* offsets, const int64_t* ids,
                             int64_t batch, int64_t nnz, emb_pool_t pool, float* out, void* ws,
                             size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  if (!t || !out || (nnz > 0 && !ids)) return EMB_ERR_INVALID_ARG;
  if (pool != EMB_POOL_SUM && pool != EMB_POOL_MEAN) return EMB_ERR_INVALID_ARG;
  emb_status_t st = check_batch(t->h, offsets, batch, nnz);
  if (st != EMB_OK) return st;
  if (!aligned16(out)) return EMB_ERR_INVALID_ARG;
  if (t->h.tiered) return EMB_ERR_UNSUPPORTED;  // rows are resolved by emb_bag_prepare
  if (batch == 0) return EMB_OK;
  return hip_status(launch_forward(t->h, offsets, ids, batch, nnz, pool == EMB_POOL_MEAN, out,
                                   static_cast<hipStream_t>(stream)));
}

emb_status_t emb_bag_backward_adagrad(emb_table_t t, const int64_t* offsets, const int64_t* ids,
                                      int64_t batch, int64_t nnz, emb_pool_t pool,
                                      const float* grad_out, float lr, float eps, void* ws,
                                      size_t ws_bytes, void* stream) {
  if (!t || !grad_out || (nnz > 0 && !ids)) return EMB_ERR_INVALID_ARG;
  if (pool != EMB_POOL_SUM && pool != EMB_POOL_MEAN) return EMB_ERR_INVALID_ARG;
  if (!std::isfinite(lr) || !std::isfinite(eps) || eps < 0.0f) return EMB_ERR_INVALID_ARG;
  emb_status_t st = check_batch(t->h, offsets, batch, nnz);
  if (st != EMB_OK) return st;
  if (!aligned16(grad_out)) return EMB_ERR_INVALID_ARG;
  Plan p;
  if (!make_plan(t->h, batch, nnz, &p)) return EMB_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < p.total || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return EMB_ERR_WORKSPACE;
  if (batch == 0) return EMB_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  uint32_t *keys = nullptr, *perm = nullptr;
  const bool mean = pool == EMB_POOL_MEAN;
  hipError_t e = launch_sort_unique(t->h, p, offsets, ids, mean, w, &keys, &perm, s);
  if (e == hipSuccess && t->h.tiered) {
    uint32_t* slot_keys = spare_keys(p, w);
    e = launch_cache_prepare(t->h, p, keys, perm, slot_keys, w, s);
    keys = slot_keys;
  }
  if (e == hipSuccess)
    e = launch_segment_adagrad(t->h, p, keys, perm, mean, grad_out, lr, eps, w, s);
  return hip_status(e);
}

emb_status_t emb_bag_backward_adagrad_noalloc(emb_table_t t, const int64_t* offsets,
                                              const int64_t* ids, int64_t batch, int64_t nnz,
                                              emb_pool_t pool, const float* grad_out, float lr,
                                              float eps, void* stream) {
  if (!t) return EMB_ERR_INVALID_ARG;
  // sizes that make no plan (need 0) and every other argument are judged by
  // emb_bag_backward_adagrad itself, before it enqueues anything
  const size_t need = emb_workspace_bytes(t, batch, nnz);
  if (need > (size_t)EMB_NOALLOC_SCRATCH_BYTES) return EMB_ERR_WORKSPACE;
  if (!t->h.scratch) {
    // without a workspace the call returns an argument error or, for
    // valid arguments, EMB_ERR_WORKSPACE: here that is the unresolved buffer
    const emb_status_t st = emb_bag_backward_adagrad(t, offsets, ids, batch, nnz, pool,
                                                     grad_out, lr, eps, nullptr, 0, stream);
    return st == EMB_ERR_WORKSPACE ? EMB_ERR_HIP : st;
  }
  return emb_bag_backward_adagrad(t, offsets, ids, batch, nnz, pool, grad_out, lr, eps,
                                  t->h.scratch, (size_t)EMB_NOALLOC_SCRATCH_BYTES, stream);
}

// launch_sort_unique ping-pongs A -> B -> A ... once per radix pass.  For a
// tiered table the prepare writes the cache slot keys to the other key buffer,
// and the prepared forward and backward use those.
static void sorted_arrays(const Handle& h, const Plan& p, char* w, uint32_t** keys,
                          uint32_t** vals) {
  const bool in_b = p.nnz > 0 && (p.passes % 2) == 1;
  const bool keys_b = h.tiered ? !in_b : in_b;
  *keys = reinterpret_cast<uint32_t*>(w + (keys_b ? p.keysB : p.keysA));
  *vals = reinterpret_cast<uint32_t*>(w + (in_b ? p.valsB : p.valsA));
}

static emb_status_t prepare_impl(emb_table_t t, const int64_t* offsets, const int64_t* ids,
                                 int64_t batch, int64_t nnz, emb_pool_t pool, void* ws,
                                 size_t ws_bytes, void* stream, bool with_cache) {
  if (!t || (nnz > 0 && !ids)) return EMB_ERR_INVALID_ARG;
  if (pool != EMB_POOL_SUM && pool != EMB_POOL_MEAN) return EMB_ERR_INVALID_ARG;
  emb_status_t st = check_batch(t->h, offsets, batch, nnz);
  if (st != EMB_OK) return st;
  Plan p;
  if (!make_plan(t->h, batch, nnz, &p)) return EMB_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < p.total || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return EMB_ERR_WORKSPACE;
  if (batch == 0) return EMB_OK;
  uint32_t *keys = nullptr, *vals = nullptr;
  char* w = static_cast<char*>(ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e =
      launch_sort_unique(t->h, p, offsets, ids, pool == EMB_POOL_MEAN, w, &keys, &vals, s);
  if (e == hipSuccess && t->h.tiered && with_cache)
    e = launch_cache_prepare(t->h, p, keys, vals, spare_keys(p, w), w, s);
  return hip_status(e);
}

emb_status_t emb_bag_prepare(emb_table_t t, const int64_t* offsets, const int64_t* ids,
                             int64_t batch, int64_t nnz, emb_pool_t pool, void* ws,
                             size_t ws_bytes, void* stream) {
  return prepare_impl(t, offsets, ids, batch, nnz, pool, ws, ws_bytes, stream, true);
}

emb_status_t emb_bag_prepare_ids(emb_table_t t, const int64_t* offsets, const int64_t* ids,
                                 int64_t batch, int64_t nnz, emb_pool_t pool, void* ws,
                                 size_t ws_bytes, void* stream) {
  return prepare_impl(t, offsets, ids, batch, nnz, pool, ws, ws_bytes, stream, false);
}

emb_status_t emb_cache_prepare(emb_table_t t, int64_t batch, int64_t nnz, void* ws,
                               size_t ws_bytes, void* stream) {
  if (!t || batch < 0 || nnz < 0) return EMB_ERR_INVALID_ARG;
  if (!t->h.tiered) return EMB_ERR_UNSUPPORTED;
  Plan p;
  if (!make_plan(t->h, batch, nnz, &p)) return EMB_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < p.total || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return EMB_ERR_WORKSPACE;
  if (batch == 0) return EMB_OK;
  char* w = static_cast<char*>(ws);
  // the sorted row keys and positions the id stages left (the buffer the last
  // radix pass wrote); the slot keys go to the other key buffer
  const bool in_b = p.nnz > 0 && (p.passes % 2) == 1;
  const uint32_t* keys = reinterpret_cast<const uint32_t*>(w + (in_b ? p.keysB : p.keysA));
  const uint32_t* vals = reinterpret_cast<const uint32_t*>(w + (in_b ? p.valsB : p.valsA));
  return hip_status(launch_cache_prepare(t->h, p, keys, vals, spare_keys(p, w), w,
                                         static_cast<hipStream_t>(stream)));
}

emb_status_t emb_bag_forward_prepared(emb_table_t t, const int64_t* offsets, const int64_t* ids,
                                      int64_t batch, int64_t nnz, emb_pool_t pool, float* out,
                                      void* ws, size_t ws_bytes, void* stream) {
  if (!t || !out || (nnz > 0 && !ids)) return EMB_ERR_INVALID_ARG;
  if (pool != EMB_POOL_SUM && pool != EMB_POOL_MEAN) return EMB_ERR_INVALID_ARG;
  emb_status_t st = check_batch(t->h, offsets, batch, nnz);
  if (st != EMB_OK) return st;
  if (!aligned16(out)) return EMB_ERR_INVALID_ARG;
  Plan p;
  if (!make_plan(t->h, batch, nnz, &p)) return EMB_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < p.total || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return EMB_ERR_WORKSPACE;
  if (batch == 0) return EMB_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  uint32_t *keys = nullptr, *vals = nullptr;
  sorted_arrays(t->h, p, w, &keys, &vals);
  phase_mark(t->h, EMB_PHASE_FORWARD, false, s);
  const bool mean = pool == EMB_POOL_MEAN;
  // As many ids as bags may be one-hot (a device flag decides inside the
  // launch); any other count is certainly not.
  const uint32_t* rowmap =
      t->h.tiered ? reinterpret_cast<const uint32_t*>(w + p.c_rowmap) : nullptr;
  hipError_t e =
      nnz == batch * (int64_t)t->h.T
          ? launch_forward_sorted(t->h, p, offsets, ids, mean, keys, vals, out, w, rowmap, s)
          : launch_forward_bags(t->h, offsets, ids, batch, nnz, mean, out, rowmap, s);
  phase_mark(t->h, EMB_PHASE_FORWARD, true, s);
  return hip_status(e);
}

static emb_status_t backward_prepared(emb_table_t t, int64_t batch, int64_t nnz,
                                      emb_pool_t pool, const float* grad_out, float lr,
                                      float eps, void* ws, size_t ws_bytes, void* stream,
                                      const DecayArgs& dec) {
  if (!t || !grad_out) return EMB_ERR_INVALID_ARG;
  if (pool != EMB_POOL_SUM && pool != EMB_POOL_MEAN) return EMB_ERR_INVALID_ARG;
  if (!std::isfinite(lr) || !std::isfinite(eps) || eps < 0.0f) return EMB_ERR_INVALID_ARG;
  if (batch < 0 || nnz < 0) return EMB_ERR_INVALID_ARG;
  if (!aligned16(grad_out)) return EMB_ERR_INVALID_ARG;
  Plan p;
  if (!make_plan(t->h, batch, nnz, &p)) return EMB_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < p.total || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return EMB_ERR_WORKSPACE;
  if (batch == 0) return EMB_OK;
  uint32_t *keys = nullptr, *vals = nullptr;
  char* w = static_cast<char*>(ws);
  sorted_arrays(t->h, p, w, &keys, &vals);
  return hip_status(launch_segment_adagrad(t->h, p, keys, vals, pool == EMB_POOL_MEAN, grad_out,
                                           lr, eps, w, static_cast<hipStream_t>(stream), dec));
}

emb_status_t emb_bag_backward_adagrad_prepared_int8(emb_table_t t, int64_t batch, int64_t nnz,
                                                    emb_pool_t pool, const int8_t* grad_codes,
                                                    const float* grad_scales, float lr,
                                                    float eps, void* ws, size_t ws_bytes,
                                                    void* stream) {
  if (!t || !grad_codes || !grad_scales) return EMB_ERR_INVALID_ARG;
  if (pool != EMB_POOL_SUM && pool != EMB_POOL_MEAN) return EMB_ERR_INVALID_ARG;
  if (!std::isfinite(lr) || !std::isfinite(eps) || eps < 0.0f) return EMB_ERR_INVALID_ARG;
  if (batch < 0 || nnz < 0) return EMB_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(grad_codes) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(grad_scales) & 3u) != 0)
    return EMB_ERR_INVALID_ARG;
  Plan p;
  if (!make_plan(t->h, batch, nnz, &p)) return EMB_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < p.total || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return EMB_ERR_WORKSPACE;
  if (batch == 0) return EMB_OK;
  uint32_t *keys = nullptr, *vals = nullptr;
  char* w = static_cast<char*>(ws);
  sorted_arrays(t->h, p, w, &keys, &vals);
  return hip_status(launch_segment_adagrad_int8(t->h, p, keys, vals, pool == EMB_POOL_MEAN,
                                                grad_codes, grad_scales, lr, eps, w,
                                                static_cast<hipStream_t>(stream)));
}

emb_status_t emb_bag_forward_prepared_int8(emb_table_t t, const int64_t* offsets,
                                           const int64_t* ids, int64_t batch, int64_t nnz,
                                           emb_pool_t pool, int8_t* codes, float* scales,
                                           void* ws, size_t ws_bytes, void* stream) {
  if (!t || !codes || !scales || (nnz > 0 && !ids)) return EMB_ERR_INVALID_ARG;
  if (pool != EMB_POOL_SUM && pool != EMB_POOL_MEAN) return EMB_ERR_INVALID_ARG;
  emb_status_t st = check_batch(t->h, offsets, batch, nnz);
  if (st != EMB_OK) return st;
  if ((reinterpret_cast<uintptr_t>(codes) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(scales) & 3u) != 0)
    return EMB_ERR_INVALID_ARG;
  Plan p;
  if (!make_plan(t->h, batch, nnz, &p)) return EMB_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < p.total || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return EMB_ERR_WORKSPACE;
  if (batch == 0) return EMB_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  uint32_t *keys = nullptr, *vals = nullptr;
  sorted_arrays(t->h, p, w, &keys, &vals);
  phase_mark(t->h, EMB_PHASE_FORWARD, false, s);
  const uint32_t* rowmap =
      t->h.tiered ? reinterpret_cast<const uint32_t*>(w + p.c_rowmap) : nullptr;
  hipError_t e = launch_forward_prepared_int8(t->h, p, offsets, ids, pool == EMB_POOL_MEAN,
                                              nnz == batch * (int64_t)t->h.T, keys, vals, codes,
                                              scales, w, rowmap, s);
  phase_mark(t->h, EMB_PHASE_FORWARD, true, s);
  return hip_status(e);
}

emb_status_t emb_bag_backward_adagrad_prepared(emb_table_t t, int64_t batch, int64_t nnz,
                                               emb_pool_t pool, const float* grad_out, float lr,
                                               float eps, void* ws, size_t ws_bytes,
                                               void* stream) {
  return backward_prepared(t, batch, nnz, pool, grad_out, lr, eps, ws, ws_bytes, stream,
                           DecayArgs());
}

emb_status_t emb_bag_backward_adagrad_decay_prepared(emb_table_t t, int64_t batch, int64_t nnz,
                                                     emb_pool_t pool, const float* grad_out,
                                                     float lr, float eps, float rho,
                                                     uint32_t period, uint32_t* row_periods,
                                                     void* ws, size_t ws_bytes, void* stream) {
  if (!t || !row_periods || (reinterpret_cast<uintptr_t>(row_periods) & 3u) != 0)
    return EMB_ERR_INVALID_ARG;
  if (!(rho > 0.0f && rho <= 1.0f)) return EMB_ERR_INVALID_ARG;
  if (t->h.tiered) return EMB_ERR_UNSUPPORTED;  // the periods are indexed by table row
  DecayArgs dec;
  dec.stamps = row_periods;
  dec.log2_rho = (float)std::log2((double)rho);
  dec.period = period;
  return backward_prepared(t, batch, nnz, pool, grad_out, lr, eps, ws, ws_bytes, stream, dec);
}

emb_status_t emb_debug_sort_unique(emb_table_t t, const int64_t* offsets, const int64_t* ids,
                                   int64_t batch, int64_t nnz, uint32_t* sorted_rows,
                                   uint32_t* perm, uint32_t* unique, uint32_t* counts,
                                   uint32_t* seg_off, uint32_t* inverse, uint32_t* num_unique,
                                   void* ws, size_t ws_bytes, void* stream) {
  if (!t || !num_unique || (nnz > 0 && !ids)) return EMB_ERR_INVALID_ARG;
  emb_status_t st = check_batch(t->h, offsets, batch, nnz);
  if (st != EMB_OK) return st;
  Plan p;
  if (!make_plan(t->h, batch, nnz, &p)) return EMB_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < p.total || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return EMB_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  uint32_t *keys = nullptr, *vals = nullptr;
  hipError_t e = launch_sort_unique(t->h, p, offsets, ids, false, w, &keys, &vals, s);
  if (e == hipSuccess)  // counts from seg_off; W and G untouched
    e = launch_unique_counts(p, w, s);
  const size_t nb = sizeof(uint32_t) * (size_t)nnz;
  if (e == hipSuccess && sorted_rows)
    e = launch_debug_copy_sorted(keys, (uint32_t)t->h.total_rows, sorted_rows, nnz, s);
  if (e == hipSuccess && perm && nb)
    e = hipMemcpyAsync(perm, vals, nb, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess && unique && nb)
    e = hipMemcpyAsync(unique, w + p.unique, nb, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess && counts && nb)
    e = hipMemcpyAsync(counts, w + p.counts, nb, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess && seg_off)
    e = hipMemcpyAsync(seg_off, w + p.seg_off, nb + sizeof(uint32_t), hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess && inverse && nb)
    e = hipMemcpyAsync(inverse, w + p.inverse, nb, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(num_unique, w + p.misc + sizeof(uint32_t) * kMiscNumUnique,
                       sizeof(uint32_t), hipMemcpyDeviceToDevice, s);
  return hip_status(e);
}

static emb_status_t find_or_insert(emb_table_t t, const int64_t* offsets, const uint64_t* keys,
                                   int64_t batch, int64_t nnz, int64_t* ids_out, void* ws,
                                   size_t ws_bytes, void* stream, const AdmitArgs& adm) {
  if (!t || (nnz > 0 && (!keys || !ids_out))) return EMB_ERR_INVALID_ARG;
  if (!t->h.hashed) return EMB_ERR_UNSUPPORTED;
  emb_status_t st = check_batch(t->h, offsets, batch, nnz);
  if (st != EMB_OK) return st;
  Plan p;
  if (!make_plan(t->h, batch, nnz, &p)) return EMB_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < p.total || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return EMB_ERR_WORKSPACE;
  if (nnz == 0) return EMB_OK;
  return hip_status(launch_hash_find_or_insert(t->h, p, offsets, keys, ids_out,
                                               static_cast<char*>(ws),
                                               static_cast<hipStream_t>(stream), adm));
}

emb_status_t emb_hash_find_or_insert(emb_table_t t, const int64_t* offsets, const uint64_t* keys,
                                     int64_t batch, int64_t nnz, int64_t* ids_out, void* ws,
                                     size_t ws_bytes, void* stream) {
  return find_or_insert(t, offsets, keys, batch, nnz, ids_out, ws, ws_bytes, stream,
                        AdmitArgs());
}

emb_status_t emb_hash_find_or_insert_admit(emb_table_t t, const int64_t* offsets,
                                           const uint64_t* keys, int64_t batch, int64_t nnz,
                                           int64_t* ids_out, uint32_t min_count,
                                           uint32_t* key_counts, void* ws, size_t ws_bytes,
                                           void* stream) {
  if (min_count > 1 && (!key_counts || (reinterpret_cast<uintptr_t>(key_counts) & 3u) != 0))
    return EMB_ERR_INVALID_ARG;
  AdmitArgs adm;
  adm.counts = key_counts;
  adm.min_count = min_count;
  return find_or_insert(t, offsets, keys, batch, nnz, ids_out, ws, ws_bytes, stream, adm);
}

int64_t emb_interact_out_dim(emb_table_t t) {
  if (!t) return 0;
  return (int64_t)t->h.D + (int64_t)(t->h.T + 1) * t->h.T / 2;
}

static emb_status_t interact_checks(emb_table_t t, const int64_t* offsets, const int64_t* ids,
                                    int64_t batch, int64_t nnz, emb_pool_t pool,
                                    const float* dense) {
  if (!t || !dense || (nnz > 0 && !ids)) return EMB_ERR_INVALID_ARG;
  if (pool != EMB_POOL_SUM && pool != EMB_POOL_MEAN) return EMB_ERR_INVALID_ARG;
  if (!aligned16(dense)) return EMB_ERR_INVALID_ARG;
  emb_status_t st = check_batch(t->h, offsets, batch, nnz);
  if (st != EMB_OK) return st;
  if (!interact_supported(t->h)) return EMB_ERR_UNSUPPORTED;
  return EMB_OK;
}

emb_status_t emb_bag_forward_interact(emb_table_t t, const int64_t* offsets, const int64_t* ids,
                                      int64_t batch, int64_t nnz, emb_pool_t pool,
                                      const float* dense, float* out, void* stream) {
  emb_status_t st = interact_checks(t, offsets, ids, batch, nnz, pool, dense);
  if (st != EMB_OK) return st;
  if (!out) return EMB_ERR_INVALID_ARG;
  if (batch == 0) return EMB_OK;
  return hip_status(launch_interact_forward(t->h, offsets, ids, batch, nnz,
                                            pool == EMB_POOL_MEAN, dense, out,
                                            static_cast<hipStream_t>(stream)));
}

emb_status_t emb_interact_backward(emb_table_t t, const int64_t* offsets, const int64_t* ids,
                                   int64_t batch, int64_t nnz, emb_pool_t pool,
                                   const float* dense, const float* grad_out, float* grad_dense,
                                   float* grad_pooled, void* stream) {
  emb_status_t st = interact_checks(t, offsets, ids, batch, nnz, pool, dense);
  if (st != EMB_OK) return st;
  if (!grad_out || !grad_dense || !grad_pooled) return EMB_ERR_INVALID_ARG;
  if (batch == 0) return EMB_OK;
  return hip_status(launch_interact_backward(t->h, offsets, ids, batch, nnz,
                                             pool == EMB_POOL_MEAN, dense, grad_out, grad_dense,
                                             grad_pooled, static_cast<hipStream_t>(stream)));
}

size_t emb_hash_evict_workspace_bytes(emb_table_t t) {
  if (!t || !t->h.hashed) return 0;
  return hash_evict_workspace_bytes(t->h);
}

emb_status_t emb_hash_evict(emb_table_t t, uint32_t* row_last_used, uint32_t before,
                            uint32_t* key_counts, void* ws, size_t ws_bytes, void* stream) {
  if (!t || !row_last_used || (reinterpret_cast<uintptr_t>(row_last_used) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(key_counts) & 3u) != 0)
    return EMB_ERR_INVALID_ARG;
  if (!t->h.hashed || !t->h.free_rows) return EMB_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < hash_evict_workspace_bytes(t->h) ||
      (reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return EMB_ERR_WORKSPACE;
  return hip_status(launch_hash_evict(t->h, row_last_used, before, key_counts,
                                      static_cast<char*>(ws), static_cast<hipStream_t>(stream)));
}

emb_status_t emb_hash_free_rows(emb_table_t t, void* stream, int64_t* queued_out) {
  if (!t || !queued_out) return EMB_ERR_INVALID_ARG;
  if (!t->h.hashed) return EMB_ERR_UNSUPPORTED;
  std::vector<int64_t> q(2 * (size_t)t->h.T);
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e == hipSuccess)  // q_head and q_tail are adjacent in the state
    e = hipMemcpy(q.data(), t->h.sv.q_head, sizeof(int64_t) * q.size(), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return EMB_ERR_HIP;
  for (int i = 0; i < t->h.T; ++i) queued_out[i] = q[t->h.T + i] - q[i];
  return EMB_OK;
}

emb_status_t emb_status_sync(emb_table_t t, void* stream, uint32_t* flags_out) {
  if (!t) return EMB_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t f = 0;
  hipError_t e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = hipMemcpy(&f, t->h.sv.flags, sizeof(f), hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemset(t->h.sv.flags, 0, sizeof(f));
  if (e != hipSuccess) return EMB_ERR_HIP;
  if (flags_out) *flags_out = f;
  if (f & EMB_FLAG_TABLE_FULL) return EMB_ERR_TABLE_FULL;
  if (f & EMB_FLAG_CACHE_FULL) return EMB_ERR_CACHE_FULL;
  if (f & EMB_FLAG_RESERVED_KEY) return EMB_ERR_RESERVED_KEY;
  if (f & EMB_FLAG_BAD_OFFSETS) return EMB_ERR_BAD_OFFSETS;
  if (f & EMB_FLAG_OUT_OF_RANGE) return EMB_ERR_OUT_OF_RANGE;
  return EMB_OK;
}

emb_status_t emb_hash_n_live(emb_table_t t, void* stream, int64_t* n_live_out) {
  if (!t || !n_live_out) return EMB_ERR_INVALID_ARG;
  if (!t->h.hashed) return EMB_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipStreamSynchronize(s);
  if (e == hipSuccess)
    e = hipMemcpy(n_live_out, t->h.sv.n_live, sizeof(int64_t) * t->h.T, hipMemcpyDeviceToHost);
  return hip_status(e);
}

emb_status_t emb_set_phase_events(emb_table_t t, void* const* events) {
  if (!t) return EMB_ERR_INVALID_ARG;
  t->h.timing = events != nullptr;
  for (int i = 0; i < 2 * EMB_NUM_PHASES; ++i)
    t->h.events[i] = events ? static_cast<hipEvent_t>(events[i]) : nullptr;
  return EMB_OK;
}

emb_status_t emb_hash_export(emb_table_t t, int32_t table, uint64_t* key_of_row, void* stream) {
  if (!t || !key_of_row || table < 0 || table >= t->h.T) return EMB_ERR_INVALID_ARG;
  if (!t->h.hashed) return EMB_ERR_UNSUPPORTED;
  return hip_status(launch_hash_export(t->h, table, key_of_row, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---------------------------------------------------------------- stream ceilings

static bool aligned16p(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

emb_status_t emb_stream_copy(void* dst, const void* src, size_t bytes, void* stream) {
  if (!dst || !src || bytes % 16 != 0 || !aligned16p(dst) || !aligned16p(src))
    return EMB_ERR_INVALID_ARG;
  return launch_stream(0, dst, src, bytes, 0.0f, static_cast<hipStream_t>(stream)) == hipSuccess
             ? EMB_OK
             : EMB_ERR_HIP;
}

emb_status_t emb_stream_fill(void* dst, float value, size_t bytes, void* stream) {
  if (!dst || bytes % 16 != 0 || !aligned16p(dst)) return EMB_ERR_INVALID_ARG;
  return launch_stream(1, dst, nullptr, bytes, value, static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? EMB_OK
             : EMB_ERR_HIP;
}

size_t emb_stream_read_sink_floats(size_t bytes) { return stream_read_sink_floats(bytes); }

// ---------------------------------------------------------------- int8 exchange payload

static bool aligned4p(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

static bool quant_dims_ok(int64_t rows, int32_t dim) {
  return rows >= 0 && dim >= 4 && dim % 4 == 0 && dim <= 1024;
}

emb_status_t emb_quantize_rows_int8(const float* x, int64_t rows, int32_t dim, int8_t* codes,
                                    float* scales, void* stream) {
  if (!quant_dims_ok(rows, dim)) return EMB_ERR_INVALID_ARG;
  if (rows == 0) return EMB_OK;
  if (!x || !codes || !scales || !aligned16p(x) || !aligned4p(codes) || !aligned4p(scales))
    return EMB_ERR_INVALID_ARG;
  return launch_quantize_rows(x, rows, dim, codes, scales, static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? EMB_OK
             : EMB_ERR_HIP;
}

emb_status_t emb_dequantize_rows_int8(const int8_t* codes, const float* scales, int64_t rows,
                                      int32_t dim, float* y, void* stream) {
  if (!quant_dims_ok(rows, dim)) return EMB_ERR_INVALID_ARG;
  if (rows == 0) return EMB_OK;
  if (!codes || !scales || !y || !aligned4p(codes) || !aligned4p(scales) || !aligned16p(y))
    return EMB_ERR_INVALID_ARG;
  return launch_dequantize_rows(codes, scales, rows, dim, y,
                                static_cast<hipStream_t>(stream)) == hipSuccess
             ? EMB_OK
             : EMB_ERR_HIP;
}

emb_status_t emb_stream_read(const void* src, size_t bytes, float* sink, size_t sink_floats,
                             void* stream) {
  if (!src || !sink || bytes % 16 != 0 || !aligned16p(src) ||
      sink_floats < emb_stream_read_sink_floats(bytes))
    return EMB_ERR_INVALID_ARG;
  return launch_stream(2, sink, src, bytes, 0.0f, static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? EMB_OK
             : EMB_ERR_HIP;
}
