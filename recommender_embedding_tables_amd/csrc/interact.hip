// DLRM dot feature interaction fused with the pooled lookup, for gfx950.
//
// The pooled embeddings' first consumer in DLRM is the dot interaction:
// per sample the T + 1 vectors z_0 (the dense features) and z_1..z_T (the
// pooled bags) give [z_0, z_i . z_j for i > j] (OneFlow OneEmbedding page,
// section "operator optimisation": a fused dot-interaction operator;
// HugeCTR interview, section three, technique (5): pooling fused with the
// next layer so the pooled vectors never go through HBM).  The forward keeps
// a sample's vectors in LDS only: the [B, T, D] pooled tensor is neither
// written nor read back.
//
// One wave per sample.  The wave pools the T bags into rows 1..T of a
// (T + 1) x D matrix Z in its LDS (row 0: the dense input), padded to 32 rows
// with zeros in registers, then the Gram matrix Z Z^T comes from the matrix
// cores:
// v_mfma_f32_16x16x4_f32, lane l supplying A[l % 16][l / 16] and
// B[l / 16][l % 16] and holding D[4 (l / 16) + r][l % 16] in register r.
// Only the lower 16 x 16 blocks (0,0), (1,0), (1,1) are formed; both
// operands of a block are rows of Z, so the K-steps may take the columns in
// any order common to A and B: each 16-column step reads one float4 of each
// row block per lane and feeds four K-steps (twelve products).  Pairs are
// staged in LDS and written as one contiguous row per sample.
//
// The backward gathers Z again and forms dZ = G Z with G the symmetric
// matrix of the pair gradients (zero diagonal): M-blocks of 16 rows, N-blocks
// of 16 columns, K = 32 in steps of 4.  Row 0 of dZ (plus the copied slot's
// gradient) is the dense input's gradient, rows 1..T the pooled embeddings'
// ([B, T, D], the input of emb_bag_backward_adagrad).
#include "embtab_internal.hpp"
#include "interact.hpp"

namespace embtab {

namespace {

typedef float f4v __attribute__((ext_vector_type(4)));

constexpr int kZRows = 32;  // T + 1 <= 32

// LDS of one wave: Z [T + 1][D + 4] (the row stride D + 4 spreads the 16 rows
// of a K-step over the banks; rows T+1..31 are zeros supplied in registers),
// the symmetric pair matrix [32][kGStride] (backward; 16-byte rows),
// pair staging (forward) and the row of every table's current occurrence.
constexpr int kGStride = 36;
__host__ __device__ inline int z_stride(int D) { return D + 4; }
// Rows wider than 128 floats go through the pipeline in two column halves
// (widths multiples of 16, the first the wider): both kernels are separable
// over columns (the Gram matrix is a sum over them, dZ = G Z column by
// column), and a half keeps the registers and LDS of a 128-float row.  Z then
// holds one half.
__host__ __device__ inline int col_blocks(int D) { return D > 128 ? 2 : 1; }
__host__ __device__ inline int half_width(int D, int h) {  // columns of half h
  const int w0 = col_blocks(D) == 1 ? D : 16 * ((D / 16 + 1) / 2);
  return h == 0 ? w0 : D - w0;
}
__host__ __device__ inline size_t wave_lds_floats(int T, int D, bool bwd) {
  return (size_t)(T + 1) * z_stride(D) + (bwd ? 32 * kGStride : 512) + 32;
}

struct WaveLds {
  float* z;       // [T + 1][D + 4]
  float* g;       // [32][kGStride]  (backward)
  float* pairs;   // [<= 496]  (forward)
  uint32_t* row;  // [32]
};

__device__ inline WaveLds wave_lds(float* base, int T, int D, bool bwd, int w) {
  WaveLds l;
  float* p = base + (size_t)w * wave_lds_floats(T, D, bwd);
  l.z = p;
  l.g = p + (size_t)(T + 1) * z_stride(D);
  l.pairs = l.g;
  l.row = reinterpret_cast<uint32_t*>(l.g + (bwd ? 32 * kGStride : 512));
  return l;
}

__device__ inline void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The samples of one wave, software-pipelined so that no global load latency
// is exposed once per sample: while sample s's rows are in flight, the
// previous sample's Z (still in LDS) is consumed (matrix-core products and
// outputs), the first id of each bag of the next sample is fetched (its bag
// bounds were fetched one sample earlier) and so are the bag bounds of the
// sample after it.
//   Lane t < T owns bag (t, s): its bounds, and the row of its occurrence at
//   the current position, which it publishes in LDS; every lane then loads
//   its NQ items (table, float4 column) of that row.  Position 0 of the next
//   sample is resolved during this one; later positions of multi-hot bags are
//   walked in place.  Bags whose offsets lie outside [0, nnz] or decrease
//   count as empty and flag.  Rows of more than 128 floats go round in two
//   column halves (the bag bounds, ids and rows resolved once per sample);
//   consume(sp, hp) reads Z rows 0..T of half hp of sample sp;
//   issue(s) may start the consumer's own loads for sample s (it is consumed
//   in the next one or two iterations), and rotate() moves them to the
//   consumer's side after the sample's first half.
template <bool MEAN, int NQ, int NH, bool HOLD_ITEMS, class Issue, class Consume, class Rotate>
__device__ void pipelined_samples(const WaveLds& l, int64_t first, int64_t stride,
                                  const float* __restrict__ dense,
                                  const int64_t* __restrict__ offsets,
                                  const int64_t* __restrict__ ids,
                                  const int64_t* __restrict__ row_off,
                                  const int64_t* __restrict__ rows,
                                  const float* __restrict__ W, int64_t B, int32_t T, int32_t D,
                                  int64_t nnz, uint32_t& bad, Issue issue, Consume consume,
                                  Rotate rotate) {
  const int lane = threadIdx.x & 63;
  static_assert(NH == 1 || !HOLD_ITEMS, "held items assume one column block");
  const int zs = z_stride(half_width(D, 0));  // NH = col_blocks(D)
  int D4 = half_width(D, 0) >> 2;  // float4 columns of the current half
  // rows, global row offsets and valid offsets all fit 32 bits (the calls
  // reject nnz >= 2^32 - 16; global rows are 32-bit)
  const uint32_t nrows = lane < T ? (uint32_t)rows[lane] : 0u;
  const uint32_t roff = lane < T ? (uint32_t)row_off[lane] : 0u;
  // Item q of this lane is the flat (table, float4 column) index 64 q + lane:
  // table = index / D4, column = the rest.  HOLD_ITEMS keeps them packed in
  // NQ registers (table << 8 | column, -1 past the last item); otherwise they
  // are recomputed at each use from an opaque copy of the lane id (so that
  // the compiler does not hold them across the sample loop either), with the
  // quotient in fp32: for index < 2048 and D4 <= 64, (index + 1/2) / D4 lies
  // at least 1/128 from an integer, far beyond the rounding error.
  int nitems = T * D4;
  float rd4 = 1.0f / (float)D4;
  int tc[HOLD_ITEMS ? NQ : 1];
  if constexpr (HOLD_ITEMS) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int it = q * 64 + lane;
      const int t = it / D4;
      tc[q] = it < nitems ? (t << 8) | (it - t * D4) : -1;
    }
  }
  auto opaque_lane = [&]() {
    int v = lane;
    if constexpr (!HOLD_ITEMS) asm volatile("" : "+v"(v));
    return v;
  };
  auto item_of = [&](int ln, int q, int& t, int& c) -> bool {
    if constexpr (HOLD_ITEMS) {
      t = tc[q] >> 8;
      c = tc[q] & 255;
      return tc[q] >= 0;
    } else {
      const int it = q * 64 + ln;
      t = (int)(((float)it + 0.5f) * rd4);
      c = it - t * D4;
      return it < nitems;
    }
  };
  auto bag_of = [&](int64_t s, uint32_t& o0, uint32_t& len) {
    o0 = 0u;
    len = 0u;
    if (lane < T && s < B) {
      const int64_t b = (int64_t)lane * B + s;
      int64_t a = offsets[b], e = offsets[b + 1];
      if (a < 0 || e < a || e > nnz) {
        bad |= EMB_FLAG_BAD_OFFSETS;
        a = e = 0;
      }
      o0 = (uint32_t)a;
      len = (uint32_t)(e - a);
    }
  };
  // the row of id `id` at position j of a bag of `len` ids (lanes < T)
  auto row_of = [&](int64_t id, uint32_t len, uint32_t j) -> uint32_t {
    uint32_t r = kNoRow;
    if (lane < T && j < len) {
      if (id >= 0 && id < (int64_t)nrows) r = roff + (uint32_t)id;
      else if (id != kAbsentId) bad |= EMB_FLAG_OUT_OF_RANGE;
    }
    return r;
  };
  auto id_at = [&](uint32_t o0, uint32_t len, uint32_t j) -> int64_t {
    return (lane < T && j < len) ? ids[(size_t)o0 + j] : kAbsentId;
  };
  auto resolve = [&](uint32_t o0, uint32_t len, uint32_t j) -> uint32_t {
    return row_of(id_at(o0, len, j), len, j);
  };
  auto wave_max = [](uint32_t v) {
    for (int o = 32; o > 0; o >>= 1) {
      const uint32_t y = (uint32_t)__shfl_xor((int)v, o, 64);
      v = y > v ? y : v;
    }
    return (uint32_t)__builtin_amdgcn_readfirstlane(v);
  };
  auto load_item = [&](int ln, int q, int hcol) -> f4v {
    int t, c;
    const bool in = item_of(ln, q, t, c);
    const uint32_t r = in ? l.row[t] : kNoRow;
    const bool ok = r != kNoRow;
    const f4v v = *reinterpret_cast<const f4v*>(W + (ok ? (size_t)r * D + hcol + 4 * c : 0));
    return ok ? v : f4v{0.f, 0.f, 0.f, 0.f};
  };

  int64_t s = first;
  uint32_t o0, len, o0n, lenn;
  bag_of(s, o0, len);
  bag_of(s + stride, o0n, lenn);
  uint32_t maxlen = wave_max(len);
  if (lane < T) l.row[lane] = resolve(o0, len, 0);
  wave_sync();
  int64_t sp = -1;
  int hp = 0;
  while (s < B) {
    const int64_t sn = s + stride;
    // in flight during this sample's first half: the bag bounds of the sample
    // after the next one, and the first id of every bag of the next one
    uint32_t o0nn = 0u, lennn = 0u;
    int64_t idn = kAbsentId;
    for (int h = 0; h < NH; ++h) {
      const int hcol = h == 0 ? 0 : half_width(D, 0);
      if (NH > 1) {
        D4 = half_width(D, h) >> 2;
        nitems = T * D4;
        rd4 = 1.0f / (float)D4;
      }
      if (h == 0) {
        bag_of(sn + stride, o0nn, lennn);
        idn = id_at(o0n, lenn, 0);
      }
      f4v dv[(256 / 4 + 63) / 64];
  #pragma unroll
      for (int q = 0; q < (256 / 4 + 63) / 64; ++q) {
        const int c = lane + 64 * q;
        dv[q] = c < D4 ? *reinterpret_cast<const f4v*>(dense + (size_t)s * D + hcol + 4 * c)
                       : f4v{0.f, 0.f, 0.f, 0.f};
      }
      f4v acc[NQ];
      {
        const int ln = opaque_lane();
  #pragma unroll
        for (int q = 0; q < NQ; ++q) acc[q] = load_item(ln, q, hcol);  // position 0 of sample s
      }
      if (h == 0) issue(s);
      if (sp >= 0) consume(sp, hp);  // the previous half or sample, from LDS
      wave_sync();
      for (uint32_t j = 1; j < maxlen; ++j) {  // later positions of multi-hot bags
        if (lane < T) l.row[lane] = resolve(o0, len, j);
        wave_sync();
        const int ln = opaque_lane();
  #pragma unroll
        for (int q0 = 0; q0 < NQ; q0 += 4) {  // four loads in flight: few registers
          f4v x[4];
  #pragma unroll
          for (int q = 0; q < 4; ++q) x[q] = load_item(ln, q0 + q, hcol);
  #pragma unroll
          for (int q = 0; q < 4; ++q) acc[q0 + q] += x[q];
        }
        wave_sync();
      }
      // Z of sample s (this half): the dense row and the pooled bags
  #pragma unroll
      for (int q = 0; q < (256 / 4 + 63) / 64; ++q) {
        const int c = lane + 64 * q;
        if (c < D4) *reinterpret_cast<f4v*>(l.z + 4 * c) = dv[q];
      }
      {
        const int ln = opaque_lane();
  #pragma unroll
        for (int q = 0; q < NQ; ++q) {
          int t, c;
          const bool in = item_of(ln, q, t, c);
          const uint32_t lq = (uint32_t)__shfl((int)len, in ? t : 0, 64);
          if (!in) continue;
          f4v v = acc[q];
          if (MEAN && lq > 0) v *= 1.0f / (float)lq;
          *reinterpret_cast<f4v*>(l.z + (size_t)(t + 1) * zs + 4 * c) = v;
        }
      }
      if (h == NH - 1) {  // position 0 of the next sample
        if (lane < T) l.row[lane] = row_of(idn, lenn, 0);
        maxlen = wave_max(lenn);
        o0 = o0n;
        len = lenn;
        o0n = o0nn;
        lenn = lennn;
      } else if (maxlen > 1) {  // the walk moved on: position 0 again for the next half
        if (lane < T) l.row[lane] = resolve(o0, len, 0);
      }
      wave_sync();
      if (h == 0) rotate();
      sp = s;
      hp = h;
    }
    s = sn;
  }
  if (sp >= 0) consume(sp, hp);
  wave_sync();
}

template <bool MEAN, int NQ, int NH>
__global__ __launch_bounds__(256, 2) void k_interact_fwd(
    const float* __restrict__ dense, const int64_t* __restrict__ offsets,
    const int64_t* __restrict__ ids, const int64_t* __restrict__ row_off,
    const int64_t* __restrict__ rows, const float* __restrict__ W, int64_t B, int32_t T,
    int32_t D, int64_t nnz, float* __restrict__ out, uint32_t* __restrict__ flags) {
  extern __shared__ float lds[];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wpb = blockDim.x >> 6;
  const WaveLds l = wave_lds(lds, T, half_width(D, 0), false, w);
  const int zs = z_stride(half_width(D, 0));
  const int P = (T + 1) * T / 2;
  const int64_t ostride = (int64_t)D + P;
  uint32_t bad = 0;
  const int ri = lane & 15, kq = lane >> 4;
  // the Gram blocks, summed over the column halves of a sample
  f4v a00 = {0.f, 0.f, 0.f, 0.f}, a10 = a00, a11 = a00;
  auto consume = [&](int64_t s, int h) {
    const int hcol = h == 0 ? 0 : half_width(D, 0);
    const int Dh = half_width(D, h);
    // the copied dense slot (rows of D + P floats: not 16-byte aligned)
    for (int d = lane; d < Dh; d += 64) out[s * ostride + hcol + d] = l.z[d];
    // Gram blocks (0,0), (1,0), (1,1) of Z Z^T; rows past T are zero.  Both
    // operands are rows of Z, so the sum over k may visit the columns in any
    // order shared by A and B: in each 16-column step lane (ri, kq) supplies
    // the four adjacent columns 4 kq .. 4 kq + 3 (one 16-byte LDS read per
    // row) to four consecutive K-steps.  Rows past T read row T (in bounds)
    // and are replaced by zeros.
    const bool two = T + 1 > 16;
    const bool has0 = ri <= T, has1 = 16 + ri <= T;
    const f4v zero = {0.f, 0.f, 0.f, 0.f};
    if (h == 0) a00 = a10 = a11 = zero;
    const float* z0p = l.z + (size_t)(has0 ? ri : T) * zs + 4 * kq;
    const float* z1p = l.z + (size_t)(has1 ? 16 + ri : T) * zs + 4 * kq;
    if (two) {
      for (int k0 = 0; k0 < Dh; k0 += 16) {
        f4v x0 = *reinterpret_cast<const f4v*>(z0p + k0);
        f4v x1 = *reinterpret_cast<const f4v*>(z1p + k0);
        x0 = has0 ? x0 : zero;
        x1 = has1 ? x1 : zero;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          a00 = __builtin_amdgcn_mfma_f32_16x16x4f32(x0[m], x0[m], a00, 0, 0, 0);
          a10 = __builtin_amdgcn_mfma_f32_16x16x4f32(x1[m], x0[m], a10, 0, 0, 0);
          a11 = __builtin_amdgcn_mfma_f32_16x16x4f32(x1[m], x1[m], a11, 0, 0, 0);
        }
      }
    } else {
      for (int k0 = 0; k0 < Dh; k0 += 16) {
        f4v x0 = *reinterpret_cast<const f4v*>(z0p + k0);
        x0 = has0 ? x0 : zero;
#pragma unroll
        for (int m = 0; m < 4; ++m)
          a00 = __builtin_amdgcn_mfma_f32_16x16x4f32(x0[m], x0[m], a00, 0, 0, 0);
      }
    }
    if (h != NH - 1) return;
    // lane holds block[4 (l / 16) + r][l % 16]; pairs i > j go to staging
    const int j0 = lane & 15;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i0 = 4 * (lane >> 4) + r;
      if (i0 > j0 && i0 <= T) l.pairs[i0 * (i0 - 1) / 2 + j0] = a00[r];
      if (two) {
        const int i1 = 16 + i0;
        if (i1 <= T) {
          l.pairs[i1 * (i1 - 1) / 2 + j0] = a10[r];
          if (i0 > j0) l.pairs[i1 * (i1 - 1) / 2 + 16 + j0] = a11[r];
        }
      }
    }
    wave_sync();
    for (int p = lane; p < P; p += 64) out[s * ostride + D + p] = l.pairs[p];
  };
  // up to 16 items per lane stay in registers (sum pooling over whole rows;
  // with mean pooling, or with the Gram sums carried across column halves,
  // 16 held items spill)
  constexpr bool kHold = NQ <= 16 && !MEAN && NH == 1;
  pipelined_samples<MEAN, NQ, NH, kHold>(l, (int64_t)blockIdx.x * wpb + w,
                                         (int64_t)gridDim.x * wpb, dense, offsets, ids, row_off,
                                         rows, W, B, T, D, nnz, bad, [](int64_t) {}, consume,
                                         []() {});
  const uint32_t any = (uint32_t)(__ballot(bad != 0) != 0);
  if (any) {
    uint32_t all = bad;
    for (int o = 1; o < 64; o <<= 1) all |= (uint32_t)__shfl_xor((int)all, o, 64);
    if (lane == 0) atomicOr(flags, all);
  }
}

template <bool MEAN, int NQ, int NH>
__global__ __launch_bounds__(256, 2) void k_interact_bwd(
    const float* __restrict__ dense, const int64_t* __restrict__ offsets,
    const int64_t* __restrict__ ids, const int64_t* __restrict__ row_off,
    const int64_t* __restrict__ rows, const float* __restrict__ W, int64_t B, int32_t T,
    int32_t D, int64_t nnz, const float* __restrict__ grad_out, float* __restrict__ grad_dense,
    float* __restrict__ grad_pooled, uint32_t* __restrict__ flags) {
  extern __shared__ float lds[];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wpb = blockDim.x >> 6;
  const WaveLds l = wave_lds(lds, T, half_width(D, 0), true, w);
  const int zs = z_stride(half_width(D, 0));
  const int P = (T + 1) * T / 2;
  const int64_t gstride = (int64_t)D + P;
  uint32_t bad = 0;
  const int ri = lane & 15, kq = lane >> 4;
  // The symmetric pair-gradient matrix G: its diagonal and the entries past
  // row or column T stay zero for every sample; each sample rewrites the
  // pair entries only.
  for (int e = lane; e < 32 * kGStride; e += 64) l.g[e] = 0.0f;
  // The pair gradients of the sample being gathered are loaded with its rows
  // (issue) and written to G after the previous sample has been consumed
  // (rotate): pair p = (i, j), i > j, at p = i (i - 1) / 2 + j of the pair
  // row, goes to G[i][j] and G[j][i].
  constexpr int kPairIt = (kZRows * (kZRows - 1) / 2 + 63) / 64;
  float pr[kPairIt];
  auto issue = [&](int64_t s) {
    const float* gp = grad_out + s * gstride + D;
#pragma unroll
    for (int it = 0; it < kPairIt; ++it) {
      const int p = lane + 64 * it;
      pr[it] = p < P ? gp[p] : 0.0f;
    }
  };
  auto rotate = [&]() {
#pragma unroll
    for (int it = 0; it < kPairIt; ++it) {
      const int p = lane + 64 * it;
      if (p < P) {
        int i = (int)((1.0f + __builtin_sqrtf((float)(8 * p + 1))) * 0.5f);
        if (i * (i - 1) / 2 > p) --i;
        else if ((i + 1) * i / 2 <= p) ++i;
        const int j = p - i * (i - 1) / 2;
        l.g[i * kGStride + j] = pr[it];
        l.g[j * kGStride + i] = pr[it];
      }
    }
    wave_sync();
  };
  auto consume = [&](int64_t s, int h) {
    const int hcol = h == 0 ? 0 : half_width(D, 0);
    const int Dh = half_width(D, h);
    // the dense slot's upstream gradient, added to dz_0 once the products are
    // done (loaded now, used last)
    const float* go = grad_out + s * gstride + hcol;
    float gdn[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int d = lane + 64 * q;
      gdn[q] = d < Dh ? go[d] : 0.0f;
    }
    const bool two = T + 1 > 16;
    // K runs over the rows of Z in the order k = 8 kq + m (m = 0..7) for both
    // operands: lane (ri, kq) takes G[ri][8 kq .. 8 kq + 7] as two float4 and
    // Z[8 kq + m][n0 + ri] (zero past row T; rows past T read row T).
    const float* ga = l.g + ri * kGStride + 8 * kq;
    const float* gb = l.g + (16 + ri) * kGStride + 8 * kq;
    for (int n0 = 0; n0 < Dh; n0 += 16) {
      // both 16-row blocks of dZ for these 16 columns, side by side:
      // A[i][k] = G[16 mb + i][k], B[k][n] = Z[k][n0 + n].  G is read again
      // for every column block rather than held in registers.
      f4v acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {  // K-steps 4 h .. 4 h + 3: fewer registers live
        asm volatile("" ::: "memory");
        float bz[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int k = 8 * kq + 4 * h + m;
          const float v = l.z[(size_t)(k <= T ? k : T) * zs + n0 + ri];
          bz[m] = k <= T ? v : 0.0f;
        }
        const f4v g0 = *reinterpret_cast<const f4v*>(ga + 4 * h);
        if (two) {
          const f4v g1 = *reinterpret_cast<const f4v*>(gb + 4 * h);
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(g0[m], bz[m], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(g1[m], bz[m], acc1, 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int m = 0; m < 4; ++m)
            acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(g0[m], bz[m], acc0, 0, 0, 0);
        }
      }
      // lane holds dZ[16 mb + 4 (l / 16) + r][n0 + l % 16].  dz_0 goes to
      // Z's row 0, whose columns n0 .. n0 + 15 no later block reads.
      const int col = n0 + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * (lane >> 4) + r;
        if (row == 0)
          l.z[col] = acc0[r];
        else if (row <= T)
          grad_pooled[((size_t)s * T + (row - 1)) * D + hcol + col] = acc0[r];
        if (two && 16 + row <= T)
          grad_pooled[((size_t)s * T + (15 + row)) * D + hcol + col] = acc1[r];
      }
    }
    wave_sync();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int d = lane + 64 * q;
      if (d < Dh) grad_dense[s * D + hcol + d] = gdn[q] + l.z[d];
    }
  };
  // the backward's products need the registers: its items are recomputed
  pipelined_samples<MEAN, NQ, NH, false>(l, (int64_t)blockIdx.x * wpb + w,
                                     (int64_t)gridDim.x * wpb, dense, offsets, ids, row_off,
                                     rows, W, B, T, D, nnz, bad, issue, consume, rotate);
  const uint32_t any = (uint32_t)(__ballot(bad != 0) != 0);
  if (any) {
    uint32_t all = bad;
    for (int o = 1; o < 64; o <<= 1) all |= (uint32_t)__shfl_xor((int)all, o, 64);
    if (lane == 0) atomicOr(flags, all);
  }
}

int waves_per_block(int D) { return D <= 128 ? 4 : 2; }

// One round of resident blocks: each wave walks its samples with a stride of
// the grid, so a wave's pipeline fills once and drains once (four rounds of
// shorter walks: forward 0.247 -> 0.231 ms, backward 0.459 -> 0.452 ms on
// 26 one-hot tables, B = 65536, D = 128).
unsigned interact_grid(const Handle& h, const void* fn, int64_t B, int wpb, size_t shm) {
  const int64_t want = (B + wpb - 1) / wpb;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 64 * wpb, shm) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  const int64_t cap = (int64_t)(h.cus > 0 ? h.cus : 256) * per_cu;
  return (unsigned)(want < cap ? (want > 0 ? want : 1) : cap);
}

// Items (table, float4 column) per lane, rounded up to 4, 8 or 16.
int items_per_lane(const Handle& h) {
  const int n = (h.T * (half_width(h.D, 0) / 4) + 63) / 64;
  return n <= 4 ? 4 : n <= 8 ? 8 : 16;
}

template <bool BWD, bool MEAN, int NQ, int NH>
hipError_t launch_nq(const Handle& h, const int64_t* offsets, const int64_t* ids, int64_t B,
                     int64_t nnz, const float* dense, float* out, const float* grad_out,
                     float* grad_dense, float* grad_pooled, hipStream_t s) {
  const int Dh = half_width(h.D, 0);
  const int wpb = waves_per_block(Dh);
  const size_t shm = sizeof(float) * wave_lds_floats(h.T, Dh, BWD) * (size_t)wpb;
  // more than 64 KiB of dynamic LDS has to be allowed per kernel
  const void* fn = BWD ? reinterpret_cast<const void*>(&k_interact_bwd<MEAN, NQ, NH>)
                       : reinterpret_cast<const void*>(&k_interact_fwd<MEAN, NQ, NH>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  const unsigned grid = interact_grid(h, fn, B, wpb, shm);
  if (BWD)
    hipLaunchKernelGGL((k_interact_bwd<MEAN, NQ, NH>), dim3(grid), dim3(64 * wpb), shm, s, dense,
                       offsets, ids, h.sv.row_off, h.sv.rows, h.W, B, h.T, h.D, nnz, grad_out,
                       grad_dense, grad_pooled, h.sv.flags);
  else
    hipLaunchKernelGGL((k_interact_fwd<MEAN, NQ, NH>), dim3(grid), dim3(64 * wpb), shm, s, dense,
                       offsets, ids, h.sv.row_off, h.sv.rows, h.W, B, h.T, h.D, nnz, out,
                       h.sv.flags);
  return hipGetLastError();
}

template <bool BWD, bool MEAN>
hipError_t launch_mean(const Handle& h, const int64_t* offsets, const int64_t* ids, int64_t B,
                       int64_t nnz, const float* dense, float* out, const float* grad_out,
                       float* grad_dense, float* grad_pooled, hipStream_t s) {
#define EMB_IA(NQ, NH)                                                                     \
  return launch_nq<BWD, MEAN, NQ, NH>(h, offsets, ids, B, nnz, dense, out, grad_out, grad_dense, \
                                      grad_pooled, s)
  // a row or half of at most 128 floats has at most 31 x 32 items: 16 per lane
  if (col_blocks(h.D) == 2) {
    switch (items_per_lane(h)) {
      case 4: EMB_IA(4, 2);
      case 8: EMB_IA(8, 2);
      default: EMB_IA(16, 2);
    }
  }
  switch (items_per_lane(h)) {
    case 4: EMB_IA(4, 1);
    case 8: EMB_IA(8, 1);
    default: EMB_IA(16, 1);
  }
#undef EMB_IA
}

}  // namespace

bool interact_supported(const Handle& h) {
  return h.T + 1 <= kZRows && h.D % 16 == 0 && h.D <= 256 && !h.tiered;
}

hipError_t launch_interact_forward(const Handle& h, const int64_t* offsets, const int64_t* ids,
                                   int64_t B, int64_t nnz, bool mean, const float* dense,
                                   float* out, hipStream_t s) {
  return mean ? launch_mean<false, true>(h, offsets, ids, B, nnz, dense, out, nullptr, nullptr,
                                         nullptr, s)
              : launch_mean<false, false>(h, offsets, ids, B, nnz, dense, out, nullptr, nullptr,
                                          nullptr, s);
}

hipError_t launch_interact_backward(const Handle& h, const int64_t* offsets, const int64_t* ids,
                                    int64_t B, int64_t nnz, bool mean, const float* dense,
                                    const float* grad_out, float* grad_dense,
                                    float* grad_pooled, hipStream_t s) {
  return mean ? launch_mean<true, true>(h, offsets, ids, B, nnz, dense, nullptr, grad_out,
                                        grad_dense, grad_pooled, s)
              : launch_mean<true, false>(h, offsets, ids, B, nnz, dense, nullptr, grad_out,
                                         grad_dense, grad_pooled, s);
}

}  // namespace embtab
