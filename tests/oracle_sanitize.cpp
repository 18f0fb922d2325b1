// Drives every entry point of the CPU oracle (oracle/oracle.cpp) over random
// tiny batches, so that a build with AddressSanitizer and UndefinedBehavior-
// Sanitizer sees all of its code paths: dense lookups, sort/unique, Adagrad,
// Adagrad Decay, the dot interaction, invalid offsets, out-of-range and absent
// ids, hash insertion with duplicates and the reserved key, a full table,
// admission, a slot bound and eviction with row reuse.  Also checks a few
// invariants that hold for any batch; exits 1 with a message on a violation.
// Test infrastructure only (built by tests/test_oracle_sanitize.py with g++).
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

extern "C" {
uint64_t orc_splitmix64(uint64_t x);
uint64_t orc_draw_bits(uint64_t seed, int64_t t, uint64_t r, uint64_t i);
float orc_init_uniform(uint64_t seed, int64_t t, int64_t row, int64_t d, float lo, float hi);
float orc_init_normal(uint64_t seed, int64_t t, uint64_t key, int64_t d, float stdv);
void* orc_create(int64_t T, int64_t D, const int64_t* rows, int32_t hashed, uint64_t seed,
                 float lo, float hi, float stdv, float accum0);
void orc_destroy(void* h);
int32_t orc_set_slot_limit(void* h, int64_t limit);
int32_t orc_set_dense(void* h, const float* W, const float* G);
int32_t orc_forward(void* h, const int64_t* offsets, const int64_t* ids, int64_t B, int64_t nnz,
                    int32_t pool_mean, float* out);
int32_t orc_sort_unique(void* h, const int64_t* offsets, const int64_t* ids, int64_t B,
                        int64_t nnz, uint32_t* sorted_rows, uint32_t* perm, uint32_t* unique,
                        uint32_t* counts, uint32_t* seg_off, uint32_t* inverse,
                        int64_t* num_unique);
int32_t orc_backward_adagrad(void* h, const int64_t* offsets, const int64_t* ids, int64_t B,
                             int64_t nnz, int32_t pool_mean, const float* grad_out, float lr,
                             float eps);
int32_t orc_backward_adagrad_decay(void* h, const int64_t* offsets, const int64_t* ids,
                                   int64_t B, int64_t nnz, int32_t pool_mean,
                                   const float* grad_out, float lr, float eps, float rho,
                                   uint32_t period);
int32_t orc_read_periods(void* h, const int64_t* grows, int64_t n, uint32_t* out);
int32_t orc_interact_forward(void* h, const int64_t* offsets, const int64_t* ids, int64_t B,
                             int64_t nnz, int32_t pool_mean, const float* dense, float* out);
int32_t orc_interact_backward(void* h, const int64_t* offsets, const int64_t* ids, int64_t B,
                              int64_t nnz, int32_t pool_mean, const float* dense,
                              const float* grad_out, float* grad_dense, float* grad_pooled);
int32_t orc_read_rows(void* h, const int64_t* grows, int64_t n, float* W, float* G);
int64_t orc_touched_count(void* h);
int64_t orc_touched_rows(void* h, int64_t* out);
int32_t orc_hash_find_or_insert(void* h, const int64_t* offsets, const uint64_t* keys, int64_t B,
                                int64_t nnz, int64_t* ids_out);
int32_t orc_hash_find_or_insert_admit(void* h, const int64_t* offsets, const uint64_t* keys,
                                      int64_t B, int64_t nnz, int64_t* ids_out,
                                      uint32_t min_count);
uint64_t orc_admission_count(void* h, int64_t t, uint64_t key);
int64_t orc_hash_evict(void* h, const uint32_t* last_used, uint32_t before);
int64_t orc_free_rows(void* h, int64_t t);
int64_t orc_n_live(void* h, int64_t t);
int64_t orc_hash_export(void* h, int64_t t, uint64_t* keys, int64_t* rows, int64_t cap);
int32_t orc_quantize_rows_int8(const float* x, int64_t rows, int64_t D, int8_t* codes,
                               float* scales);
int32_t orc_dequantize_rows_int8(const int8_t* codes, const float* scales, int64_t rows,
                                 int64_t D, float* y);
}

namespace {

uint64_t g_state = 0x243F6A8885A308D3ull;
uint64_t next_u64() {
  g_state = orc_splitmix64(g_state);
  return g_state;
}
int64_t below(int64_t n) { return (int64_t)(next_u64() % (uint64_t)n); }
float unit_float() { return (float)(next_u64() >> 40) * (1.0f / 16777216.0f) - 0.5f; }

int g_fail = 0;
void check(bool ok, const char* what, int iter) {
  if (!ok) {
    std::fprintf(stderr, "iteration %d: %s\n", iter, what);
    g_fail = 1;
  }
}

struct Batch {
  int64_t B = 0, nnz = 0;
  std::vector<int64_t> offsets, ids;
};

// T*B bags; lengths 0..maxlen (some empty), ids with duplicates; a few ids
// out of range or absent (-2) when `dirty`.
Batch random_batch(int64_t T, int64_t B, const std::vector<int64_t>& rows, int64_t maxlen,
                   bool dirty) {
  Batch b;
  b.B = B;
  b.offsets.assign(T * B + 1, 0);
  for (int64_t i = 0; i < T * B; ++i) b.offsets[i + 1] = b.offsets[i] + below(maxlen + 1);
  b.nnz = b.offsets[T * B];
  b.ids.resize(b.nnz);
  for (int64_t t = 0; t < T; ++t)
    for (int64_t j = b.offsets[t * B]; j < b.offsets[(t + 1) * B]; ++j) {
      b.ids[j] = below(rows[t]);
      if (dirty && below(23) == 0) b.ids[j] = below(2) ? -2 : rows[t] + below(3);
    }
  return b;
}

void dense_round(int iter) {
  const int64_t T = 1 + below(3), D = 4 * (1 + below(3)), B = 1 + below(9);
  std::vector<int64_t> rows(T);
  int64_t total = 0;
  for (auto& r : rows) total += (r = 1 + below(12));
  void* h = orc_create(T, D, rows.data(), 0, (uint64_t)iter, -0.1f, 0.1f, 0.01f, 0.1f);
  check(h != nullptr, "create", iter);
  if (!h) return;
  if (below(2)) {
    std::vector<float> W(total * D), G(total * D);
    for (auto& x : W) x = unit_float();
    for (auto& x : G) x = 0.1f + 0.5f * (unit_float() + 0.5f);
    orc_set_dense(h, W.data(), G.data());
  }
  const bool dirty = below(3) == 0;
  const int32_t mean = (int32_t)below(2);
  Batch b = random_batch(T, B, rows, 1 + below(5), dirty);
  std::vector<float> out(B * T * D), grad(B * T * D), dense(B * D);
  for (auto& x : grad) x = unit_float();
  for (auto& x : dense) x = unit_float();
  const int32_t fl = orc_forward(h, b.offsets.data(), b.ids.data(), B, b.nnz, mean, out.data());
  check((fl & 2) == 0, "valid offsets flagged", iter);
  std::vector<uint32_t> sorted(b.nnz + 1), perm(b.nnz + 1), uniq(b.nnz + 1), cnt(b.nnz + 1),
      seg(b.nnz + 2), inv(b.nnz + 1);
  int64_t nu = -1;
  orc_sort_unique(h, b.offsets.data(), b.ids.data(), B, b.nnz, sorted.data(), perm.data(),
                  uniq.data(), cnt.data(), seg.data(), inv.data(), &nu);
  int64_t csum = 0;
  for (int64_t u = 0; u < nu; ++u) {
    csum += cnt[u];
    check(u == 0 || uniq[u - 1] < uniq[u], "unique ascending", iter);
    check(seg[u + 1] - seg[u] == cnt[u], "seg_off matches counts", iter);
  }
  int64_t valid = 0;
  for (int64_t t = 0; t < T; ++t)
    for (int64_t j = b.offsets[t * B]; j < b.offsets[(t + 1) * B]; ++j)
      valid += (b.ids[j] >= 0 && b.ids[j] < rows[t]) ? 1 : 0;
  check(csum == valid, "counts sum to the valid occurrences", iter);
  std::vector<char> seen(b.nnz + 1, 0);
  for (int64_t k = 0; k < valid; ++k) {
    check(perm[k] < (uint32_t)b.nnz && !seen[perm[k]], "perm is injective", iter);
    if (perm[k] < (uint32_t)b.nnz) seen[perm[k]] = 1;
    check(k == 0 || sorted[k - 1] <= sorted[k], "sorted rows ascending", iter);
    check(k == 0 || sorted[k - 1] != sorted[k] || perm[k - 1] < perm[k], "stable", iter);
    if (perm[k] < (uint32_t)b.nnz) check(uniq[inv[perm[k]]] == sorted[k], "inverse", iter);
  }
  const int mode = (int)below(3);
  if (mode == 0) {
    orc_backward_adagrad(h, b.offsets.data(), b.ids.data(), B, b.nnz, mean, grad.data(), 0.05f,
                         1e-6f);
  } else if (mode == 1) {
    orc_backward_adagrad_decay(h, b.offsets.data(), b.ids.data(), B, b.nnz, mean, grad.data(),
                               0.05f, 1e-6f, 0.9f, (uint32_t)below(4));
    std::vector<int64_t> all(total);
    for (int64_t r = 0; r < total; ++r) all[r] = r;
    std::vector<uint32_t> per(total);
    check(orc_read_periods(h, all.data(), total, per.data()) == 0, "read periods", iter);
  } else if (T + 1 <= 32 && D % 4 == 0) {
    std::vector<float> io(B * (D + (T + 1) * T / 2)), gi(io.size()), gd(B * D),
        gp(B * T * D);
    for (auto& x : gi) x = unit_float();
    orc_interact_forward(h, b.offsets.data(), b.ids.data(), B, b.nnz, mean, dense.data(),
                         io.data());
    orc_interact_backward(h, b.offsets.data(), b.ids.data(), B, b.nnz, mean, dense.data(),
                          gi.data(), gd.data(), gp.data());
  }
  std::vector<int64_t> touched(orc_touched_count(h) + 1);
  const int64_t nt = orc_touched_rows(h, touched.data());
  std::vector<float> w(D * (nt + 1)), g(D * (nt + 1));
  check(orc_read_rows(h, touched.data(), nt, w.data(), g.data()) == 0, "read rows", iter);
  // int8 exchange payload of the pooled output, and back
  {
    const int64_t nr = (int64_t)B * T;
    std::vector<int8_t> codes(nr * D + 1);
    std::vector<float> scales(nr + 1), back(nr * D + 1);
    check(orc_quantize_rows_int8(out.data(), nr, D, codes.data(), scales.data()) == 0,
          "quantize", iter);
    check(orc_dequantize_rows_int8(codes.data(), scales.data(), nr, D, back.data()) == 0,
          "dequantize", iter);
  }
  // invalid offsets: flagged, nothing written
  if (b.nnz > 0 && T * B > 1) {
    std::vector<int64_t> bad = b.offsets;
    bad[1] = b.nnz + 1;
    check((orc_forward(h, bad.data(), b.ids.data(), B, b.nnz, mean, out.data()) & 2) != 0,
          "bad offsets flagged", iter);
    orc_backward_adagrad(h, bad.data(), b.ids.data(), B, b.nnz, mean, grad.data(), 0.05f, 1e-6f);
  }
  orc_destroy(h);
}

void hash_round(int iter) {
  const int64_t T = 1 + below(3), D = 4, B = 1 + below(12);
  std::vector<int64_t> rows(T);
  for (auto& r : rows) r = 2 + below(10);
  void* h = orc_create(T, D, rows.data(), 1, 7u + (uint64_t)iter, 0.f, 0.f, 0.02f, 0.1f);
  check(h != nullptr, "create hashed", iter);
  if (!h) return;
  if (below(2)) orc_set_slot_limit(h, 4 + below(12));
  std::vector<int64_t> row_off(T + 1, 0);
  for (int64_t t = 0; t < T; ++t) row_off[t + 1] = row_off[t] + rows[t];
  std::vector<uint32_t> last(row_off[T], 0);  // last call that used each global row
  for (int call = 0; call < 6; ++call) {
    Batch b = random_batch(T, B, rows, 3, false);
    std::vector<uint64_t> keys(b.nnz + 1);
    for (int64_t j = 0; j < b.nnz; ++j) {
      keys[j] = 1000u + (uint64_t)below(25);
      if (below(40) == 0) keys[j] = ~0ull;  // the reserved key
    }
    std::vector<int64_t> ids(b.nnz + 1, 123);
    const uint32_t min_count = (uint32_t)below(3);
    if (min_count > 1)
      orc_hash_find_or_insert_admit(h, b.offsets.data(), keys.data(), B, b.nnz, ids.data(),
                                    min_count);
    else
      orc_hash_find_or_insert(h, b.offsets.data(), keys.data(), B, b.nnz, ids.data());
    for (int64_t t = 0; t < T; ++t) {
      check(orc_n_live(h, t) <= rows[t], "n_live within rows", iter);
      for (int64_t j = b.offsets[t * B]; j < b.offsets[(t + 1) * B]; ++j) {
        check(ids[j] >= -2 && ids[j] < rows[t], "id range", iter);
        if (ids[j] >= 0 && ids[j] < rows[t]) last[row_off[t] + ids[j]] = (uint32_t)call + 1u;
      }
      (void)orc_admission_count(h, t, 1000u);
      std::vector<uint64_t> ek(rows[t] + 1);
      std::vector<int64_t> er(rows[t] + 1);
      const int64_t n = orc_hash_export(h, t, ek.data(), er.data(), rows[t] + 1);
      check(n <= rows[t], "export size", iter);
      (void)orc_free_rows(h, t);
    }
    std::vector<float> grad(B * T * D, 0.25f);
    orc_backward_adagrad(h, b.offsets.data(), ids.data(), B, b.nnz, 0, grad.data(), 0.05f,
                         1e-6f);
    if (call % 2 == 1) orc_hash_evict(h, last.data(), (uint32_t)call);
  }
  orc_destroy(h);
}

}  // namespace

int main() {
  for (int64_t d = 0; d < 8; ++d) {
    (void)orc_draw_bits(1, 2, 3, (uint64_t)d);
    (void)orc_init_uniform(1, 0, 5, d, -1.f, 1.f);
    (void)orc_init_normal(1, 0, 5, d, 1.f);
  }
  for (int iter = 0; iter < 3000; ++iter) dense_round(iter);
  for (int iter = 0; iter < 2000; ++iter) hash_round(iter);
  if (g_fail) return 1;
  std::printf("ok\n");
  return 0;
}
