// CPU oracle for the sparse embedding layer: multi-table EmbeddingBag forward,
// id sort/unique, segmented gradient reduction with element-wise Adagrad, and
// the raw-key to row map of dynamically inserted feature keys.
//
// TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
// benchmark's CPU-baseline leg may load this library.  It is a plain, slow,
// sequential definition of what the GPU path computes, written from the
// definitions directly: std::map for the key map, nested loops for gather and
// update, fp64 accumulation with one rounding to fp32 per stored value.  It
// shares no code, header, table or constant with the GPU library.
//
// Sources for what is computed (the pages are web articles; no code is given):
//  * Embedding lookup maps categorical ids to dense vectors and dominates the
//    parameters:  "NVIDIA Merlin Distributed Embeddings" page, introduction and
//    section "Background" (lookup is memory bound, HBM bandwidth is the lever).
//  * Pooling of several looked-up vectors per feature:  "Merlin HugeCTR
//    interview" page, section three, technique (5) (pooling fused with the
//    next layer) and section two (thousands of feature fields per sample).
//  * Sparse optimizer touching only the rows that were used:  HugeCTR
//    interview, section three, technique (1) ("memory-saving sparse
//    optimizer"); the optimizer is Adagrad in every synthetic benchmark of the
//    Merlin Distributed Embeddings page, section "Performance", synthetic
//    model benchmarks.
//  * Deduplicating repeated ids / one access per id per pass:  DeepRec page,
//    section "model quality", EmbeddingVariable item 2; EcoRec page, section
//    "research method" (merging redundant work on identical indices).
//  * Adagrad with a per-period discount of the accumulator, all samples of
//    one period discounted alike:  DeepRec page, section "model quality",
//    item "Adagrad Decay Optimizer".
//  * The first consumer of the pooled embeddings fused with the lookup: the
//    DLRM dot feature interaction (OneFlow OneEmbedding page, section
//    "operator optimisation": a fused dot-interaction operator for DLRM;
//    HugeCTR interview, section three, technique (5): pooling fused with the
//    next layer to save memory traffic).
//  * Feature admission (a key gets a row only once it is frequent enough):
//    DeepRec page, section "model quality", EmbeddingVariable item 1
//    (several admission methods; no formula is given).
//  * Quantized exchange of embeddings between ranks: floats are quantized to
//    int8 before the exchange and dequantized after (OneFlow OneEmbedding
//    page, section "quantized compression").
//  * Dynamic insertion of unseen feature keys, no capacity planning:
//    OneFlow OneEmbedding page, section "ease of use"; HugeCTR interview,
//    section two (a hash table identifies every input feature before the
//    embedding layer) and section three technique (1) (GPU hash table).
//
// Readings where the pages are silent (each is listed in the design notes):
//  * Adagrad is the textbook form (Duchi, Hazan and Singer, JMLR 2011):
//    G <- G + g*g (per element), w <- w - lr * g / (sqrt(G) + eps).
//  * Adagrad Decay (the page gives no formula): every accumulator is
//    multiplied by rho at each period boundary.  Done lazily, a row last
//    updated in period s and updated again in period p first takes
//    G <- rho^(p - s) * G (no discount when p <= s), then the Adagrad step;
//    its period becomes max(s, p).  Rows of dense tables start with period 0.
//    A row of a hashed table that has no key yet, or was freed by eviction,
//    is fresh (period all-ones): the key it next receives starts from the
//    initial accumulator, which the following update does not discount; that
//    update sets the row's period to p.  rho = 1 is Adagrad.
//  * Sum or mean pooling; mean divides by the bag length L (duplicates count,
//    out-of-range ids count in L but contribute nothing); an empty bag is 0.
//  * Bags are table-major (bag b = t*B + s); the output is [B, T, D].
//  * Duplicate ids in one batch: their gradients are summed and the row gets
//    one Adagrad step.  Accumulation is in ascending occurrence order.
//  * Sort is stable: equal rows keep ascending occurrence position.
//  * int8 exchange payload (the page gives no scheme): one symmetric scale per
//    row of D values, codes in [-127, 127].  amax = max |x|; a zero row has
//    scale 0 and codes 0; otherwise inv = 127 / amax, code = x * inv rounded
//    to nearest (ties to even), scale = amax / 127, each step in fp32 (a code
//    is an integer decided by floating point, so the oracle decides it in the
//    same precision as the kernel).  Dequantized value: code * scale in fp32.
//  * A key not yet in table t's map gets, in order of its first occurrence
//    among this call's new keys, the next free row (rows freed by eviction,
//    oldest eviction first), else row n_live[t] (rows never used, ascending);
//    the call is all-or-nothing when the new keys would exceed the rows left.
//  * Eviction (DeepRec page, section "model quality", EmbeddingVariable item 1
//    names eviction policies and gives none): keys whose row was last used
//    before a given step leave the map and free their rows; the caller keeps
//    the per-row last-use step.
//  * Initial values come from a counter-based generator built on SplitMix64
//    (Steele, Lea and Flood, OOPSLA 2014): uniform rows for dense tables and
//    Box-Muller (1958) normal rows for inserted keys.
//
//  * Admission (the page names the feature only): a key without a row counts
//    its occurrences over calls; in the call where its count reaches
//    min_count it gets a row, in order of its first occurrence in that call
//    (as a new key), and all its occurrences of that call see the row.  Until
//    then its occurrences get id -2, "absent": the lookup gives 0 (counted in
//    a mean bag's length) and the backward updates nothing, with no error
//    bit.  A full call admits nothing (keys that would have been admitted get
//    -1) but every count still advances.  min_count <= 1 is plain insertion.
//  * A table holds at most slot_limit keys, live or counted (the GPU table
//    keeps at most 0.9 of its slots in use, so that its probes stay short).
//    A call whose keys that are neither live nor counted would push a table
//    past it keeps none of them: it admits nothing, counts no new key, the
//    counts of already counted keys still advance, and every occurrence of a
//    key without a row gets -1 (full).  With plain insertion the bound is
//    never the binding one (rows <= slot_limit).
//
//  * Dot interaction (the pages name the operator only; this is the DLRM
//    model's definition, Naumov et al. 2019): per sample, z_0 = the dense
//    feature vector [D], z_{t+1} = the pooled embedding of table t; the
//    output is [z_0, z_i . z_j for i = 1..T, j = 0..i-1] (row-major order of
//    the strict lower triangle), D + (T+1)T/2 values.  Its backward gives
//    dz_i = sum_{j != i} g_ij z_j (g symmetric), the dense input's gradient
//    (the copied z_0 slot plus dz_0) and the pooled embeddings' ([B, T, D]).
//
// Adagrad Decay, admission and eviction are named by the DeepRec page but not
// defined there: the oracle follows the readings above, which the tests pin
// (worked cases, torch Adagrad at rho = 1, an eager discount model, counting
// and free-queue models); against the pages themselves parity is unpinned.
//
// Return values of the orc_* calls that check data: a bit mask,
//   1 = an id outside [0, rows of its table), other than -2 (contributes 0)
//   2 = offsets not starting at 0, decreasing, or not ending at nnz
//   4 = a key equal to the reserved all-ones value (id -1, nothing inserted)
//   8 = table full (nothing inserted, new keys get id -1)
//  -1 = bad arguments.

#include <cmath>
#include <cstdint>
#include <cstring>
#include <algorithm>
#include <deque>
#include <map>
#include <set>
#include <vector>
#include <algorithm>
#include <utility>

namespace {

const uint64_t kReservedKey = ~0ull;
const uint32_t kInvalidRow32 = 0xFFFFFFFFu;
const int64_t kAbsentId = -2;  // a feature without a row (not admitted yet)
const uint32_t kFreshPeriod = 0xFFFFFFFFu;  // Adagrad Decay: a row whose key is new

// SplitMix64, one output step: the state advances by the golden-ratio
// increment and the new state is passed through the variant-13 finalizer.
// Written from the published description of the generator.
uint64_t splitmix64(uint64_t state) {
  uint64_t z = state + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Counter-based draw for element i of row-or-key r of table t:
//   h = SM(SM(SM(SM(seed) ^ t) ^ r) ^ i)
uint64_t draw_bits(uint64_t seed, int64_t t, uint64_t r, uint64_t i) {
  uint64_t h = splitmix64(seed);
  h = splitmix64(h ^ (uint64_t)t);
  h = splitmix64(h ^ r);
  return splitmix64(h ^ i);
}

// Top 24 bits as a fraction in [0, 1).
double unit_from_bits(uint64_t h) { return (double)(h >> 40) * (1.0 / 16777216.0); }

float uniform_value(uint64_t seed, int64_t t, int64_t row, int64_t d, float lo, float hi) {
  float u = (float)unit_from_bits(draw_bits(seed, t, (uint64_t)row, (uint64_t)d));  // exact
  float span = hi - lo;
  return std::fmaf(u, span, lo);
}

float normal_value(uint64_t seed, int64_t t, uint64_t key, int64_t d, float stdv) {
  uint64_t h1 = draw_bits(seed, t, key, 2ull * (uint64_t)d);
  uint64_t h2 = draw_bits(seed, t, key, 2ull * (uint64_t)d + 1ull);
  double u1 = ((double)(h1 >> 40) + 0.5) * (1.0 / 16777216.0);  // (0, 1)
  double u2 = unit_from_bits(h2);                                // [0, 1)
  const double two_pi = 6.283185307179586476925286766559;
  double z = std::sqrt(-2.0 * std::log(u1)) * std::cos(two_pi * u2);
  return (float)((double)stdv * z);
}

struct RowState {
  std::vector<float> w, g;
};

struct Model {
  int64_t T = 0, D = 0;
  std::vector<int64_t> rows;     // capacity of each table
  std::vector<int64_t> row_off;  // T + 1 prefix sums
  bool hashed = false;
  uint64_t seed = 0;
  float lo = 0, hi = 0, stdv = 0, accum0 = 0;
  bool has_dense = false;
  std::vector<float> W0, G0;               // explicit initial table (small cases)
  std::map<int64_t, RowState> touched;     // rows written since creation
  // Adagrad Decay: period of each row's last update; rows not listed are in
  // period 0 (dense tables) or fresh (hashed tables)
  std::map<int64_t, uint32_t> period_of;
  uint32_t period_of_row(int64_t row) const {
    auto it = period_of.find(row);
    return it != period_of.end() ? it->second : (hashed ? kFreshPeriod : 0u);
  }
  std::vector<std::map<uint64_t, int64_t>> keymap;
  std::vector<std::map<uint64_t, uint64_t>> seen;  // admission: occurrences of keys without a row
  std::vector<int64_t> n_live;                    // rows ever handed out (high-water mark)
  int64_t slot_limit = INT64_MAX;                 // keys (live or counted) a table may hold
  std::vector<std::deque<int64_t>> free_rows;     // eviction: rows to hand out again, in order

  // Rows a call may still hand out in table t, and the next one.
  int64_t room(int64_t t) const { return (int64_t)free_rows[t].size() + rows[t] - n_live[t]; }
  int64_t next_row(int64_t t) {
    if (!free_rows[t].empty()) {
      const int64_t r = free_rows[t].front();
      free_rows[t].pop_front();
      return r;
    }
    return n_live[t]++;
  }

  int64_t table_of(int64_t grow) const {
    int64_t t = 0;
    while (t + 1 < T && row_off[t + 1] <= grow) ++t;
    return t;
  }

  // Current fp32 value of W and G for global row grow.
  void read(int64_t grow, float* w, float* g) const {
    auto it = touched.find(grow);
    if (it != touched.end()) {
      for (int64_t d = 0; d < D; ++d) { w[d] = it->second.w[d]; g[d] = it->second.g[d]; }
      return;
    }
    if (has_dense) {
      for (int64_t d = 0; d < D; ++d) { w[d] = W0[grow * D + d]; g[d] = G0[grow * D + d]; }
      return;
    }
    int64_t t = table_of(grow);
    int64_t local = grow - row_off[t];
    if (hashed) {  // a row that was never handed out holds no defined value
      for (int64_t d = 0; d < D; ++d) { w[d] = 0.0f; g[d] = 0.0f; }
      return;
    }
    for (int64_t d = 0; d < D; ++d) {
      w[d] = uniform_value(seed, t, local, d, lo, hi);
      g[d] = accum0;
    }
  }
};

bool offsets_ok(const int64_t* offsets, int64_t bags, int64_t nnz) {
  if (offsets[0] != 0 || offsets[bags] != nnz) return false;
  for (int64_t b = 0; b < bags; ++b)
    if (offsets[b + 1] < offsets[b]) return false;
  return true;
}

// Summed gradient of every touched global row, in ascending occurrence
// order (fp64): g_u = sum over occurrences of c_b * grad_out[s, t, :].
int32_t row_gradients(Model* m, const int64_t* offsets, const int64_t* ids, int64_t B,
                             int64_t nnz, int32_t pool_mean, const float* grad_out,
                             std::map<int64_t, std::vector<double>>& gsum) {
  const int64_t T = m->T, D = m->D, bags = T * B;
  if (!offsets_ok(offsets, bags, nnz)) return 2;
  int32_t flags = 0;
  for (int64_t b = 0; b < bags; ++b) {
    const int64_t t = b / B, s = b % B;
    const int64_t L = offsets[b + 1] - offsets[b];
    const double c = (pool_mean && L > 0) ? 1.0 / (double)L : 1.0;
    const float* go = grad_out + (s * T + t) * D;
    for (int64_t j = offsets[b]; j < offsets[b + 1]; ++j) {
      const int64_t id = ids[j];
      if (id < 0 || id >= m->rows[t]) { if (id != kAbsentId) flags |= 1; continue; }
      std::vector<double>& acc = gsum[m->row_off[t] + id];
      if (acc.empty()) acc.assign(D, 0.0);
      for (int64_t d = 0; d < D; ++d) acc[d] += c * (double)go[d];
    }
  }
  return flags;
}

// One Adagrad step on every touched row; the accumulator is first multiplied
// by `discount(row)` (1 for plain Adagrad).
template <class Discount>
void adagrad_rows(Model* m, const std::map<int64_t, std::vector<double>>& gsum, float lr,
                         float eps, Discount discount) {
  const int64_t D = m->D;
  const double dlr = (double)lr, deps = (double)eps;
  std::vector<float> w(D), g(D);
  for (auto& kv : gsum) {
    m->read(kv.first, w.data(), g.data());
    const double f = discount(kv.first);
    RowState next;
    next.w.resize(D);
    next.g.resize(D);
    for (int64_t d = 0; d < D; ++d) {
      const double gr = kv.second[d];
      const double G1 = f * (double)g[d] + gr * gr;
      const double w1 = (double)w[d] - dlr * gr / (std::sqrt(G1) + deps);
      next.g[d] = (float)G1;
      next.w[d] = (float)w1;
    }
    m->touched[kv.first] = std::move(next);
  }
}

}  // namespace

extern "C" {

uint64_t orc_splitmix64(uint64_t state) { return splitmix64(state); }
uint64_t orc_draw_bits(uint64_t seed, int64_t t, uint64_t r, uint64_t i) {
  return draw_bits(seed, t, r, i);
}
float orc_init_uniform(uint64_t seed, int64_t t, int64_t row, int64_t d, float lo, float hi) {
  return uniform_value(seed, t, row, d, lo, hi);
}
float orc_init_normal(uint64_t seed, int64_t t, uint64_t key, int64_t d, float stdv) {
  return normal_value(seed, t, key, d, stdv);
}

// Keys (live or counted for admission) each hashed table may hold.
int32_t orc_set_slot_limit(void* h, int64_t limit) {
  Model* m = static_cast<Model*>(h);
  if (!m || limit < 1) return -1;
  m->slot_limit = limit;
  return 0;
}

void* orc_create(int64_t T, int64_t D, const int64_t* rows, int32_t hashed, uint64_t seed,
                 float lo, float hi, float stdv, float accum0) {
  if (T < 1 || D < 1 || !rows) return nullptr;
  Model* m = new Model();
  m->T = T;
  m->D = D;
  m->rows.assign(rows, rows + T);
  m->row_off.assign(T + 1, 0);
  for (int64_t t = 0; t < T; ++t) m->row_off[t + 1] = m->row_off[t] + rows[t];
  m->hashed = hashed != 0;
  m->seed = seed;
  m->lo = lo;
  m->hi = hi;
  m->stdv = stdv;
  m->accum0 = accum0;
  m->keymap.resize(T);
  m->seen.resize(T);
  m->free_rows.resize(T);
  m->n_live.assign(T, 0);
  return m;
}

void orc_destroy(void* h) { delete static_cast<Model*>(h); }

// Replace the initial table with explicit values (all rows, row-major).
int32_t orc_set_dense(void* h, const float* W, const float* G) {
  Model* m = static_cast<Model*>(h);
  int64_t n = m->row_off[m->T] * m->D;
  m->W0.assign(W, W + n);
  m->G0.assign(G, G + n);
  m->has_dense = true;
  m->touched.clear();
  return 0;
}

// out[s, t, :] = c_b * sum_{j in bag b} W[row_off[t] + ids[j], :],  b = t*B + s.
int32_t orc_forward(void* h, const int64_t* offsets, const int64_t* ids, int64_t B,
                    int64_t nnz, int32_t pool_mean, float* out) {
  Model* m = static_cast<Model*>(h);
  const int64_t T = m->T, D = m->D, bags = T * B;
  if (!offsets_ok(offsets, bags, nnz)) return 2;
  int32_t flags = 0;
  std::vector<double> acc(D);
  std::vector<float> w(D), g(D);
  for (int64_t b = 0; b < bags; ++b) {
    const int64_t t = b / B, s = b % B;
    const int64_t L = offsets[b + 1] - offsets[b];
    std::fill(acc.begin(), acc.end(), 0.0);
    for (int64_t j = offsets[b]; j < offsets[b + 1]; ++j) {
      const int64_t id = ids[j];
      if (id < 0 || id >= m->rows[t]) { if (id != kAbsentId) flags |= 1; continue; }
      m->read(m->row_off[t] + id, w.data(), g.data());
      for (int64_t d = 0; d < D; ++d) acc[d] += (double)w[d];
    }
    const double c = (pool_mean && L > 0) ? 1.0 / (double)L : 1.0;
    float* o = out + (s * T + t) * D;
    for (int64_t d = 0; d < D; ++d) o[d] = (float)(c * acc[d]);
  }
  return flags;
}

// Row of every occurrence, a stable sort of (row, position) by row, and the
// run-length decomposition of the sorted rows.  An occurrence whose id is out
// of range gets the row 0xFFFFFFFF: it sorts last and belongs to no unique row
// (inverse = 0xFFFFFFFF).
int32_t orc_sort_unique(void* h, const int64_t* offsets, const int64_t* ids, int64_t B,
                        int64_t nnz, uint32_t* sorted_rows, uint32_t* perm, uint32_t* unique,
                        uint32_t* counts, uint32_t* seg_off, uint32_t* inverse,
                        int64_t* num_unique) {
  Model* m = static_cast<Model*>(h);
  const int64_t T = m->T, bags = T * B;
  if (!offsets_ok(offsets, bags, nnz)) return 2;
  int32_t flags = 0;
  std::vector<std::pair<uint32_t, uint32_t>> occ(nnz);
  for (int64_t b = 0; b < bags; ++b) {
    const int64_t t = b / B;
    for (int64_t j = offsets[b]; j < offsets[b + 1]; ++j) {
      const int64_t id = ids[j];
      uint32_t row = kInvalidRow32;
      if (id < 0 || id >= m->rows[t]) { if (id != kAbsentId) flags |= 1; }
      else row = (uint32_t)(m->row_off[t] + id);
      occ[j] = {row, (uint32_t)j};
    }
  }
  std::stable_sort(occ.begin(), occ.end(),
                   [](const std::pair<uint32_t, uint32_t>& a,
                      const std::pair<uint32_t, uint32_t>& b) { return a.first < b.first; });
  int64_t U = 0;
  for (int64_t k = 0; k < nnz; ++k) {
    sorted_rows[k] = occ[k].first;
    perm[k] = occ[k].second;
    if (occ[k].first == kInvalidRow32) {
      inverse[occ[k].second] = kInvalidRow32;
      continue;
    }
    if (k == 0 || occ[k].first != occ[k - 1].first) {
      unique[U] = occ[k].first;
      seg_off[U] = (uint32_t)k;
      counts[U] = 0;
      ++U;
    }
    counts[U - 1] += 1;
    inverse[occ[k].second] = (uint32_t)(U - 1);
  }
  int64_t valid = 0;
  for (int64_t u = 0; u < U; ++u) valid += counts[u];
  seg_off[U] = (uint32_t)valid;
  *num_unique = U;
  return flags;
}

// Gradient of the pooled lookup summed per row, then one Adagrad step on every
// row that occurs in the batch (and on no other row).
int32_t orc_backward_adagrad(void* h, const int64_t* offsets, const int64_t* ids, int64_t B,
                             int64_t nnz, int32_t pool_mean, const float* grad_out, float lr,
                             float eps) {
  Model* m = static_cast<Model*>(h);
  std::map<int64_t, std::vector<double>> gsum;
  const int32_t flags = row_gradients(m, offsets, ids, B, nnz, pool_mean, grad_out, gsum);
  if (flags & 2) return flags;
  adagrad_rows(m, gsum, lr, eps, [](int64_t) { return 1.0; });
  return flags;
}

// Adagrad Decay step in period `period` with discount rho per period.
int32_t orc_backward_adagrad_decay(void* h, const int64_t* offsets, const int64_t* ids,
                                   int64_t B, int64_t nnz, int32_t pool_mean,
                                   const float* grad_out, float lr, float eps, float rho,
                                   uint32_t period) {
  Model* m = static_cast<Model*>(h);
  if (!(rho > 0.0f && rho <= 1.0f)) return -1;
  std::map<int64_t, std::vector<double>> gsum;
  const int32_t flags = row_gradients(m, offsets, ids, B, nnz, pool_mean, grad_out, gsum);
  if (flags & 2) return flags;
  adagrad_rows(m, gsum, lr, eps, [&](int64_t row) {
    const uint32_t last = m->period_of_row(row);
    const double elapsed = (last != kFreshPeriod && period > last) ? (double)(period - last) : 0.0;
    return std::pow((double)rho, elapsed);
  });
  for (auto& kv : gsum) {
    const uint32_t last = m->period_of_row(kv.first);
    m->period_of[kv.first] = (last == kFreshPeriod || period > last) ? period : last;
  }
  return flags;
}

// Period of the last Adagrad Decay update of global rows grows[0..n) (0 if none).
int32_t orc_read_periods(void* h, const int64_t* grows, int64_t n, uint32_t* out) {
  Model* m = static_cast<Model*>(h);
  const int64_t total = m->row_off[m->T];
  for (int64_t i = 0; i < n; ++i) {
    if (grows[i] < 0 || grows[i] >= total) return -1;
    out[i] = m->period_of_row(grows[i]);
  }
  return 0;
}

// Pooled embedding of bag b = t*B + s in fp64 (sum or mean over its valid ids).
static void pooled_fp64(Model* m, const int64_t* offsets, const int64_t* ids, int64_t B,
                        int32_t pool_mean, int64_t t, int64_t s, double* z) {
  const int64_t D = m->D, b = t * B + s;
  std::vector<float> w(D), g(D);
  for (int64_t d = 0; d < D; ++d) z[d] = 0.0;
  const int64_t L = offsets[b + 1] - offsets[b];
  for (int64_t j = offsets[b]; j < offsets[b + 1]; ++j) {
    const int64_t id = ids[j];
    if (id < 0 || id >= m->rows[t]) continue;
    m->read(m->row_off[t] + id, w.data(), g.data());
    for (int64_t d = 0; d < D; ++d) z[d] += (double)w[d];
  }
  if (pool_mean && L > 0)
    for (int64_t d = 0; d < D; ++d) z[d] /= (double)L;
}

// The T + 1 vectors of sample s: z_0 = dense[s], z_{t+1} = pooled bag (t, s).
static void interaction_vectors(Model* m, const int64_t* offsets, const int64_t* ids, int64_t B,
                                int32_t pool_mean, const float* dense, int64_t s,
                                std::vector<double>& Z) {
  const int64_t T = m->T, D = m->D;
  Z.assign((size_t)(T + 1) * D, 0.0);
  for (int64_t d = 0; d < D; ++d) Z[d] = (double)dense[s * D + d];
  for (int64_t t = 0; t < T; ++t) pooled_fp64(m, offsets, ids, B, pool_mean, t, s, &Z[(t + 1) * D]);
}

// out [B, D + (T+1)T/2]: z_0, then z_i . z_j for i = 1..T, j < i.
int32_t orc_interact_forward(void* h, const int64_t* offsets, const int64_t* ids, int64_t B,
                             int64_t nnz, int32_t pool_mean, const float* dense, float* out) {
  Model* m = static_cast<Model*>(h);
  const int64_t T = m->T, D = m->D, P = (T + 1) * T / 2;
  if (!offsets_ok(offsets, T * B, nnz)) return 2;
  std::vector<double> Z;
  for (int64_t s = 0; s < B; ++s) {
    interaction_vectors(m, offsets, ids, B, pool_mean, dense, s, Z);
    float* o = out + s * (D + P);
    for (int64_t d = 0; d < D; ++d) o[d] = (float)Z[d];
    int64_t p = D;
    for (int64_t i = 1; i <= T; ++i)
      for (int64_t j = 0; j < i; ++j) {
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += Z[i * D + d] * Z[j * D + d];
        o[p++] = (float)dot;
      }
  }
  return 0;
}

// Backward of orc_interact_forward: grad_dense [B, D], grad_pooled [B, T, D].
int32_t orc_interact_backward(void* h, const int64_t* offsets, const int64_t* ids, int64_t B,
                              int64_t nnz, int32_t pool_mean, const float* dense,
                              const float* grad_out, float* grad_dense, float* grad_pooled) {
  Model* m = static_cast<Model*>(h);
  const int64_t T = m->T, D = m->D, P = (T + 1) * T / 2;
  if (!offsets_ok(offsets, T * B, nnz)) return 2;
  std::vector<double> Z, G((size_t)(T + 1) * (T + 1)), dZ;
  for (int64_t s = 0; s < B; ++s) {
    interaction_vectors(m, offsets, ids, B, pool_mean, dense, s, Z);
    const float* go = grad_out + s * (D + P);
    std::fill(G.begin(), G.end(), 0.0);
    int64_t p = D;
    for (int64_t i = 1; i <= T; ++i)
      for (int64_t j = 0; j < i; ++j, ++p) {
        G[i * (T + 1) + j] = (double)go[p];
        G[j * (T + 1) + i] = (double)go[p];
      }
    dZ.assign((size_t)(T + 1) * D, 0.0);
    for (int64_t i = 0; i <= T; ++i)
      for (int64_t j = 0; j <= T; ++j)
        for (int64_t d = 0; d < D; ++d) dZ[i * D + d] += G[i * (T + 1) + j] * Z[j * D + d];
    for (int64_t d = 0; d < D; ++d) grad_dense[s * D + d] = (float)((double)go[d] + dZ[d]);
    for (int64_t t = 0; t < T; ++t)
      for (int64_t d = 0; d < D; ++d)
        grad_pooled[(s * T + t) * D + d] = (float)dZ[(t + 1) * D + d];
  }
  return 0;
}

// Current values of global rows grows[0..n).
int32_t orc_read_rows(void* h, const int64_t* grows, int64_t n, float* W, float* G) {
  Model* m = static_cast<Model*>(h);
  const int64_t total = m->row_off[m->T];
  for (int64_t i = 0; i < n; ++i) {
    if (grows[i] < 0 || grows[i] >= total) return -1;
    m->read(grows[i], W + i * m->D, G + i * m->D);
  }
  return 0;
}

int64_t orc_touched_count(void* h) { return (int64_t) static_cast<Model*>(h)->touched.size(); }

int64_t orc_touched_rows(void* h, int64_t* out) {
  Model* m = static_cast<Model*>(h);
  int64_t i = 0;
  for (auto& kv : m->touched) out[i++] = kv.first;
  return i;
}

// keys (CSR, table-major like ids) -> table-local rows, inserting unseen keys.
int32_t orc_hash_find_or_insert(void* h, const int64_t* offsets, const uint64_t* keys,
                                int64_t B, int64_t nnz, int64_t* ids_out) {
  Model* m = static_cast<Model*>(h);
  const int64_t T = m->T, D = m->D, bags = T * B;
  if (!m->hashed) return -1;
  if (!offsets_ok(offsets, bags, nnz)) return 2;
  int32_t flags = 0;
  // Pass 1: would this call's distinct new keys fit in every table?
  bool full = false;
  for (int64_t t = 0; t < T; ++t) {
    std::set<uint64_t> fresh;
    for (int64_t j = offsets[t * B]; j < offsets[(t + 1) * B]; ++j) {
      if (keys[j] == kReservedKey) continue;
      if (m->keymap[t].find(keys[j]) == m->keymap[t].end()) fresh.insert(keys[j]);
    }
    if ((int64_t)fresh.size() > m->room(t)) full = true;
  }
  if (full) flags |= 8;
  // Pass 2: look up, inserting in order of first occurrence unless full.
  std::vector<float> w(D);
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t j = offsets[t * B]; j < offsets[(t + 1) * B]; ++j) {
      const uint64_t key = keys[j];
      if (key == kReservedKey) { flags |= 4; ids_out[j] = -1; continue; }
      auto it = m->keymap[t].find(key);
      if (it != m->keymap[t].end()) { ids_out[j] = it->second; continue; }
      if (full) { ids_out[j] = -1; continue; }
      const int64_t row = m->next_row(t);
      m->keymap[t][key] = row;
      RowState rs;
      rs.w.resize(D);
      rs.g.assign(D, m->accum0);
      for (int64_t d = 0; d < D; ++d) rs.w[d] = normal_value(m->seed, t, key, d, m->stdv);
      m->touched[m->row_off[t] + row] = std::move(rs);
      ids_out[j] = row;
    }
  }
  return flags;
}

// Find-or-insert with frequency admission (see the readings above).
int32_t orc_hash_find_or_insert_admit(void* h, const int64_t* offsets, const uint64_t* keys,
                                      int64_t B, int64_t nnz, int64_t* ids_out,
                                      uint32_t min_count) {
  Model* m = static_cast<Model*>(h);
  const int64_t T = m->T, D = m->D, bags = T * B;
  if (!m->hashed) return -1;
  if (!offsets_ok(offsets, bags, nnz)) return 2;
  int32_t flags = 0;
  // Pass 0: keys that are neither live nor counted; would they overfill a table?
  bool over = false;
  for (int64_t t = 0; t < T; ++t) {
    std::set<uint64_t> unknown;
    for (int64_t j = offsets[t * B]; j < offsets[(t + 1) * B]; ++j) {
      const uint64_t key = keys[j];
      if (key == kReservedKey || m->keymap[t].count(key) || m->seen[t].count(key)) continue;
      unknown.insert(key);
    }
    const int64_t held = (int64_t)(m->keymap[t].size() + m->seen[t].size());
    if (held + (int64_t)unknown.size() > m->slot_limit) over = true;
  }
  if (over) {
    for (int64_t t = 0; t < T; ++t)
      for (int64_t j = offsets[t * B]; j < offsets[(t + 1) * B]; ++j) {
        const uint64_t key = keys[j];
        if (key == kReservedKey) { flags |= 4; ids_out[j] = -1; continue; }
        auto it = m->keymap[t].find(key);
        if (it != m->keymap[t].end()) { ids_out[j] = it->second; continue; }
        auto c = m->seen[t].find(key);
        if (c != m->seen[t].end()) ++c->second;
        ids_out[j] = -1;
      }
    return flags | 8;
  }
  // Pass 1: counts of keys without a row advance; which of them reach min_count?
  std::vector<std::set<uint64_t>> admitted(T);
  bool full = false;
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t j = offsets[t * B]; j < offsets[(t + 1) * B]; ++j) {
      const uint64_t key = keys[j];
      if (key == kReservedKey || m->keymap[t].count(key)) continue;
      if (++m->seen[t][key] >= (uint64_t)(min_count > 0 ? min_count : 1)) admitted[t].insert(key);
    }
    if ((int64_t)admitted[t].size() > m->room(t)) full = true;
  }
  if (full) flags |= 8;
  // Pass 2: ids; admitted keys get rows in order of first occurrence.
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t j = offsets[t * B]; j < offsets[(t + 1) * B]; ++j) {
      const uint64_t key = keys[j];
      if (key == kReservedKey) { flags |= 4; ids_out[j] = -1; continue; }
      auto it = m->keymap[t].find(key);
      if (it != m->keymap[t].end()) { ids_out[j] = it->second; continue; }
      if (!admitted[t].count(key)) { ids_out[j] = kAbsentId; continue; }
      if (full) { ids_out[j] = -1; continue; }
      const int64_t row = m->next_row(t);
      m->keymap[t][key] = row;
      m->seen[t].erase(key);
      RowState rs;
      rs.w.resize(D);
      rs.g.assign(D, m->accum0);
      for (int64_t d = 0; d < D; ++d) rs.w[d] = normal_value(m->seed, t, key, d, m->stdv);
      m->touched[m->row_off[t] + row] = std::move(rs);
      ids_out[j] = row;
    }
  }
  return flags;
}

// Occurrences counted so far for a key of table t that has no row (0 if none).
uint64_t orc_admission_count(void* h, int64_t t, uint64_t key) {
  Model* m = static_cast<Model*>(h);
  auto it = m->seen[t].find(key);
  return it == m->seen[t].end() ? 0 : it->second;
}

// Eviction: every key of every table whose row was last used before `before`
// (last_used is indexed by global row) leaves the map; its row becomes free.
// Each table's freed rows join the end of its free list in ascending order.
// Counted keys without a row are forgotten.  Returns the number of evicted keys.
int64_t orc_hash_evict(void* h, const uint32_t* last_used, uint32_t before) {
  Model* m = static_cast<Model*>(h);
  if (!m->hashed) return -1;
  int64_t n = 0;
  for (int64_t t = 0; t < m->T; ++t) {
    std::vector<int64_t> freed;
    for (auto it = m->keymap[t].begin(); it != m->keymap[t].end();) {
      if (last_used[m->row_off[t] + it->second] < before) {
        freed.push_back(it->second);
        it = m->keymap[t].erase(it);
      } else {
        ++it;
      }
    }
    std::sort(freed.begin(), freed.end());
    for (int64_t r : freed) {
      m->free_rows[t].push_back(r);
      m->period_of.erase(m->row_off[t] + r);  // fresh for the key it receives next
    }
    n += (int64_t)freed.size();
    m->seen[t].clear();
  }
  return n;
}

int64_t orc_free_rows(void* h, int64_t t) {
  return (int64_t) static_cast<Model*>(h)->free_rows[t].size();
}

int64_t orc_n_live(void* h, int64_t t) { return static_cast<Model*>(h)->n_live[t]; }

// The key -> row map of table t in ascending key order; returns its size.
int64_t orc_hash_export(void* h, int64_t t, uint64_t* keys, int64_t* rows, int64_t cap) {
  Model* m = static_cast<Model*>(h);
  int64_t i = 0;
  for (auto& kv : m->keymap[t]) {
    if (i < cap) { keys[i] = kv.first; rows[i] = kv.second; }
    ++i;
  }
  return i;
}

// int8 exchange payload, row by row (the scheme is in the header notes).
int32_t orc_quantize_rows_int8(const float* x, int64_t rows, int64_t D, int8_t* codes,
                               float* scales) {
  if (rows < 0 || D < 1 || (rows > 0 && (!x || !codes || !scales))) return -1;
  for (int64_t r = 0; r < rows; ++r) {
    const float* xr = x + r * D;
    int8_t* cr = codes + r * D;
    float amax = 0.0f;
    for (int64_t d = 0; d < D; ++d) amax = std::max(amax, std::fabs(xr[d]));
    if (amax == 0.0f) {
      scales[r] = 0.0f;
      for (int64_t d = 0; d < D; ++d) cr[d] = 0;
      continue;
    }
    const float inv = 127.0f / amax;
    for (int64_t d = 0; d < D; ++d) {
      float v = std::nearbyint(xr[d] * inv);  // default rounding: to nearest, ties to even
      v = std::min(127.0f, std::max(-127.0f, v));
      cr[d] = (int8_t)v;
    }
    scales[r] = amax / 127.0f;
  }
  return 0;
}

int32_t orc_dequantize_rows_int8(const int8_t* codes, const float* scales, int64_t rows,
                                 int64_t D, float* y) {
  if (rows < 0 || D < 1 || (rows > 0 && (!codes || !scales || !y))) return -1;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t d = 0; d < D; ++d) y[r * D + d] = (float)codes[r * D + d] * scales[r];
  return 0;
}

}  // extern "C"
