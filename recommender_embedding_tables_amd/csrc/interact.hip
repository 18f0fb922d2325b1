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
// operands of a block are rows of Z, so each K-step loads two values per
// lane for three products.  Pairs are staged in LDS and written as one
// contiguous row per sample.
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
// the symmetric pair matrix [32][33] (backward), pair staging (forward) and
// the row of every table's current occurrence.
__host__ __device__ inline int z_stride(int D) { return D + 4; }
__host__ __device__ inline size_t wave_lds_floats(int T, int D, bool bwd) {
  return (size_t)(T + 1) * z_stride(D) + (bwd ? 32 * 33 : 512) + 32;
}

struct WaveLds {
  float* z;       // [T + 1][D + 4]
  float* g;       // [32][33]  (backward)
  float* pairs;   // [<= 496]  (forward)
  uint32_t* row;  // [32]
};

__device__ inline WaveLds wave_lds(float* base, int T, int D, bool bwd, int w) {
  WaveLds l;
  float* p = base + (size_t)w * wave_lds_floats(T, D, bwd);
  l.z = p;
  l.g = p + (size_t)(T + 1) * z_stride(D);
  l.pairs = l.g;
  l.row = reinterpret_cast<uint32_t*>(l.g + (bwd ? 32 * 33 : 512));
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
// outputs), and the next sample's bag bounds and first ids are fetched.
//   Lane t < T owns bag (t, s): its bounds, and the row of its occurrence at
//   the current position, which it publishes in LDS; every lane then loads
//   its NQ items (table, float4 column) of that row.  Position 0 of the next
//   sample is resolved during this one; later positions of multi-hot bags are
//   walked in place.  Bags whose offsets lie outside [0, nnz] or decrease
//   count as empty and flag.  consume(sp) reads Z rows 0..T of sample sp;
//   issue(s) may start the consumer's own loads for sample s (it is consumed
//   one iteration later), and rotate() moves them to the consumer's side.
template <bool MEAN, int NQ, class Issue, class Consume, class Rotate>
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
  const int D4 = D >> 2;
  const int zs = z_stride(D);
  const int64_t nrows = lane < T ? rows[lane] : 0, roff = lane < T ? row_off[lane] : 0;
  // item q of this lane: table (tc >> 8) and float4 column (tc & 255); -1: none
  int tc[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int it = q * 64 + lane;
    const int t = it / D4;
    tc[q] = it < T * D4 ? (t << 8) | (it - t * D4) : -1;
  }
  auto bag_of = [&](int64_t s, int64_t& o0, int64_t& len) {
    o0 = 0;
    len = 0;
    if (lane < T && s < B) {
      const int64_t b = (int64_t)lane * B + s;
      int64_t a = offsets[b], e = offsets[b + 1];
      if (a < 0 || e < a || e > nnz) {
        bad |= EMB_FLAG_BAD_OFFSETS;
        a = e = 0;
      }
      o0 = a;
      len = e - a;
    }
  };
  auto resolve = [&](int64_t o0, int64_t len, int64_t j) -> uint32_t {
    uint32_t r = kNoRow;
    if (lane < T && j < len) {
      const int64_t id = ids[o0 + j];
      if (id >= 0 && id < nrows) r = (uint32_t)(roff + id);
      else if (id != kAbsentId) bad |= EMB_FLAG_OUT_OF_RANGE;
    }
    return r;
  };
  auto wave_max = [](int64_t v) {
    for (int o = 32; o > 0; o >>= 1) {
      const int64_t y = __shfl_xor(v, o, 64);
      v = y > v ? y : v;
    }
    return v;
  };
  auto load_item = [&](int q) -> f4v {
    const uint32_t r = tc[q] >= 0 ? l.row[tc[q] >> 8] : kNoRow;
    const bool ok = r != kNoRow;
    const f4v v =
        *reinterpret_cast<const f4v*>(W + (ok ? (size_t)r * D + 4 * (tc[q] & 255) : 0));
    return ok ? v : f4v{0.f, 0.f, 0.f, 0.f};
  };

  int64_t s = first;
  int64_t o0, len;
  bag_of(s, o0, len);
  int64_t maxlen = wave_max(len);
  if (lane < T) l.row[lane] = resolve(o0, len, 0);
  wave_sync();
  int64_t sp = -1;
  while (s < B) {
    const int64_t sn = s + stride;
    int64_t o0n, lenn;
    bag_of(sn, o0n, lenn);  // in flight during this sample
    f4v dv[(256 / 4 + 63) / 64];
#pragma unroll
    for (int q = 0; q < (256 / 4 + 63) / 64; ++q) {
      const int c = lane + 64 * q;
      dv[q] = c < D4 ? *reinterpret_cast<const f4v*>(dense + (size_t)s * D + 4 * c)
                     : f4v{0.f, 0.f, 0.f, 0.f};
    }
    f4v acc[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) acc[q] = load_item(q);  // position 0 of sample s
    issue(s);
    if (sp >= 0) consume(sp);  // the previous sample, from LDS
    wave_sync();
    for (int64_t j = 1; j < maxlen; ++j) {  // later positions of multi-hot bags
      if (lane < T) l.row[lane] = resolve(o0, len, j);
      wave_sync();
#pragma unroll
      for (int q0 = 0; q0 < NQ; q0 += 4) {  // four loads in flight: few registers
        f4v x[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) x[q] = load_item(q0 + q);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q0 + q] += x[q];
      }
      wave_sync();
    }
    // Z of sample s: the dense row and the pooled bags
#pragma unroll
    for (int q = 0; q < (256 / 4 + 63) / 64; ++q) {
      const int c = lane + 64 * q;
      if (c < D4) *reinterpret_cast<f4v*>(l.z + 4 * c) = dv[q];
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int t = tc[q] >= 0 ? tc[q] >> 8 : 0;
      const int64_t lq = __shfl(len, t, 64);
      if (tc[q] < 0) continue;
      f4v v = acc[q];
      if (MEAN && lq > 0) v *= 1.0f / (float)lq;
      *reinterpret_cast<f4v*>(l.z + (size_t)(t + 1) * zs + 4 * (tc[q] & 255)) = v;
    }
    // position 0 of the next sample
    if (lane < T) l.row[lane] = resolve(o0n, lenn, 0);
    maxlen = wave_max(lenn);
    o0 = o0n;
    len = lenn;
    wave_sync();
    rotate();
    sp = s;
    s = sn;
  }
  if (sp >= 0) consume(sp);
  wave_sync();
}

template <bool MEAN, int NQ>
__global__ __launch_bounds__(256, 2) void k_interact_fwd(
    const float* __restrict__ dense, const int64_t* __restrict__ offsets,
    const int64_t* __restrict__ ids, const int64_t* __restrict__ row_off,
    const int64_t* __restrict__ rows, const float* __restrict__ W, int64_t B, int32_t T,
    int32_t D, int64_t nnz, float* __restrict__ out, uint32_t* __restrict__ flags) {
  extern __shared__ float lds[];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wpb = blockDim.x >> 6;
  const WaveLds l = wave_lds(lds, T, D, false, w);
  const int zs = z_stride(D);
  const int P = (T + 1) * T / 2;
  const int64_t ostride = (int64_t)D + P;
  uint32_t bad = 0;
  const int ri = lane & 15, kq = lane >> 4;
  auto consume = [&](int64_t s) {
    // the copied dense slot (rows of D + P floats: not 16-byte aligned)
    for (int d = lane; d < D; d += 64) out[s * ostride + d] = l.z[d];
    // Gram blocks (0,0), (1,0), (1,1) of Z Z^T; rows past T are zero
    f4v a00 = {0.f, 0.f, 0.f, 0.f}, a10 = a00, a11 = a00;
    const bool two = T + 1 > 16;
    const bool has0 = ri <= T, has1 = 16 + ri <= T;
    for (int k0 = 0; k0 < D; k0 += 4) {
      const float z0 = has0 ? l.z[(size_t)ri * zs + k0 + kq] : 0.0f;
      a00 = __builtin_amdgcn_mfma_f32_16x16x4f32(z0, z0, a00, 0, 0, 0);
      if (two) {
        const float z1 = has1 ? l.z[(size_t)(16 + ri) * zs + k0 + kq] : 0.0f;
        a10 = __builtin_amdgcn_mfma_f32_16x16x4f32(z1, z0, a10, 0, 0, 0);
        a11 = __builtin_amdgcn_mfma_f32_16x16x4f32(z1, z1, a11, 0, 0, 0);
      }
    }
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
  pipelined_samples<MEAN, NQ>(l, (int64_t)blockIdx.x * wpb + w, (int64_t)gridDim.x * wpb, dense,
                              offsets, ids, row_off, rows, W, B, T, D, nnz, bad,
                              [](int64_t) {}, consume, []() {});
  const uint32_t any = (uint32_t)(__ballot(bad != 0) != 0);
  if (any) {
    uint32_t all = bad;
    for (int o = 1; o < 64; o <<= 1) all |= (uint32_t)__shfl_xor((int)all, o, 64);
    if (lane == 0) atomicOr(flags, all);
  }
}

template <bool MEAN, int NQ>
__global__ __launch_bounds__(256, 2) void k_interact_bwd(
    const float* __restrict__ dense, const int64_t* __restrict__ offsets,
    const int64_t* __restrict__ ids, const int64_t* __restrict__ row_off,
    const int64_t* __restrict__ rows, const float* __restrict__ W, int64_t B, int32_t T,
    int32_t D, int64_t nnz, const float* __restrict__ grad_out, float* __restrict__ grad_dense,
    float* __restrict__ grad_pooled, uint32_t* __restrict__ flags) {
  extern __shared__ float lds[];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wpb = blockDim.x >> 6;
  const WaveLds l = wave_lds(lds, T, D, true, w);
  const int zs = z_stride(D);
  const int P = (T + 1) * T / 2;
  const int64_t gstride = (int64_t)D + P;
  uint32_t bad = 0;
  const int ri = lane & 15, kq = lane >> 4;
  auto consume = [&](int64_t s) {
    // symmetric pair-gradient matrix, zero diagonal and padding
    const float* go = grad_out + s * gstride;
    for (int e = lane; e < 32 * 32; e += 64) {
      const int i = e >> 5, j = e & 31;
      float v = 0.0f;
      if (i != j && i <= T && j <= T) {
        const int hi = i > j ? i : j, lo = i > j ? j : i;
        v = go[D + hi * (hi - 1) / 2 + lo];
      }
      l.g[i * 33 + j] = v;
    }
    wave_sync();
    const bool two = T + 1 > 16;
    for (int n0 = 0; n0 < D; n0 += 16) {
      // both 16-row blocks of dZ for these 16 columns, side by side:
      // A[i][k] = G[16 mb + i][k], B[k][n] = Z[k][n0 + n] (zero past row T)
      f4v acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll
      for (int k0 = 0; k0 < 32; k0 += 4) {
        const int k = k0 + kq;
        const float b = k <= T ? l.z[(size_t)k * zs + n0 + ri] : 0.0f;
        acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(l.g[ri * 33 + k], b, acc0, 0, 0, 0);
        if (two)
          acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(l.g[(16 + ri) * 33 + k], b, acc1, 0, 0, 0);
      }
      // lane holds dZ[16 mb + 4 (l / 16) + r][n0 + l % 16]
      const int col = n0 + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * (lane >> 4) + r;
        if (row == 0)
          grad_dense[s * D + col] = go[col] + acc0[r];
        else if (row <= T)
          grad_pooled[((size_t)s * T + (row - 1)) * D + col] = acc0[r];
        if (two && 16 + row <= T)
          grad_pooled[((size_t)s * T + (15 + row)) * D + col] = acc1[r];
      }
    }
  };
  pipelined_samples<MEAN, NQ>(l, (int64_t)blockIdx.x * wpb + w, (int64_t)gridDim.x * wpb, dense,
                              offsets, ids, row_off, rows, W, B, T, D, nnz, bad,
                              [](int64_t) {}, consume, []() {});
  const uint32_t any = (uint32_t)(__ballot(bad != 0) != 0);
  if (any) {
    uint32_t all = bad;
    for (int o = 1; o < 64; o <<= 1) all |= (uint32_t)__shfl_xor((int)all, o, 64);
    if (lane == 0) atomicOr(flags, all);
  }
}

int waves_per_block(int D) { return D <= 128 ? 4 : 2; }

unsigned interact_grid(const Handle& h, int64_t B, int wpb) {
  const int64_t want = (B + wpb - 1) / wpb;
  const int64_t cap = (int64_t)(h.cus > 0 ? h.cus : 256) * 8;
  return (unsigned)(want < cap ? (want > 0 ? want : 1) : cap);
}

// Items (table, float4 column) per lane, rounded up to 4, 8, 16 or 32.
int items_per_lane(const Handle& h) {
  const int n = (h.T * (h.D / 4) + 63) / 64;
  return n <= 4 ? 4 : n <= 8 ? 8 : n <= 16 ? 16 : 32;
}

template <bool BWD, bool MEAN, int NQ>
hipError_t launch_nq(const Handle& h, const int64_t* offsets, const int64_t* ids, int64_t B,
                     int64_t nnz, const float* dense, float* out, const float* grad_out,
                     float* grad_dense, float* grad_pooled, hipStream_t s) {
  const int wpb = waves_per_block(h.D);
  const size_t shm = sizeof(float) * wave_lds_floats(h.T, h.D, BWD) * (size_t)wpb;
  const unsigned grid = interact_grid(h, B, wpb);
  // more than 64 KiB of dynamic LDS has to be allowed per kernel
  const void* fn = BWD ? reinterpret_cast<const void*>(&k_interact_bwd<MEAN, NQ>)
                       : reinterpret_cast<const void*>(&k_interact_fwd<MEAN, NQ>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  if (BWD)
    hipLaunchKernelGGL((k_interact_bwd<MEAN, NQ>), dim3(grid), dim3(64 * wpb), shm, s, dense,
                       offsets, ids, h.sv.row_off, h.sv.rows, h.W, B, h.T, h.D, nnz, grad_out,
                       grad_dense, grad_pooled, h.sv.flags);
  else
    hipLaunchKernelGGL((k_interact_fwd<MEAN, NQ>), dim3(grid), dim3(64 * wpb), shm, s, dense,
                       offsets, ids, h.sv.row_off, h.sv.rows, h.W, B, h.T, h.D, nnz, out,
                       h.sv.flags);
  return hipGetLastError();
}

template <bool BWD, bool MEAN>
hipError_t launch_mean(const Handle& h, const int64_t* offsets, const int64_t* ids, int64_t B,
                       int64_t nnz, const float* dense, float* out, const float* grad_out,
                       float* grad_dense, float* grad_pooled, hipStream_t s) {
  switch (items_per_lane(h)) {
    case 4:
      return launch_nq<BWD, MEAN, 4>(h, offsets, ids, B, nnz, dense, out, grad_out, grad_dense,
                                     grad_pooled, s);
    case 8:
      return launch_nq<BWD, MEAN, 8>(h, offsets, ids, B, nnz, dense, out, grad_out, grad_dense,
                                     grad_pooled, s);
    case 16:
      return launch_nq<BWD, MEAN, 16>(h, offsets, ids, B, nnz, dense, out, grad_out, grad_dense,
                                      grad_pooled, s);
    default:
      return launch_nq<BWD, MEAN, 32>(h, offsets, ids, B, nnz, dense, out, grad_out, grad_dense,
                                      grad_pooled, s);
  }
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
