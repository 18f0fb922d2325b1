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

// Rows 0..T of Z for sample s: the dense input and the pooled bags.  Lane t
// (t < T) owns bag (t, s); per position j of the bags, lane t resolves its
// occurrence's row into LDS and every lane adds the rows of its NQ items
// (table, float4 column).  All of a sample's row loads of one position are in
// flight together.  Bags with offsets outside [0, nnz] or decreasing count as
// empty and flag.
template <bool MEAN, int NQ>
__device__ void gather_z(const WaveLds& l, int64_t s, const float* __restrict__ dense,
                         const int64_t* __restrict__ offsets, const int64_t* __restrict__ ids,
                         const int64_t* __restrict__ row_off, const int64_t* __restrict__ rows,
                         const float* __restrict__ W, int64_t B, int32_t T, int32_t D,
                         int64_t nnz, uint32_t& bad) {
  const int lane = threadIdx.x & 63;
  const int D4 = D >> 2;
  const int zs = z_stride(D);
  int64_t o0 = 0, o1 = 0;
  if (lane < T) {
    const int64_t b = (int64_t)lane * B + s;
    o0 = offsets[b];
    o1 = offsets[b + 1];
    if (o0 < 0 || o1 < o0 || o1 > nnz) {
      bad |= EMB_FLAG_BAD_OFFSETS;
      o0 = o1 = 0;
    }
  }
  const int64_t len = o1 - o0;
  const int64_t nrows = lane < T ? rows[lane] : 0, roff = lane < T ? row_off[lane] : 0;
  int64_t maxlen = len;
  for (int o = 32; o > 0; o >>= 1) {
    const int64_t y = __shfl_xor(maxlen, o, 64);
    maxlen = y > maxlen ? y : maxlen;
  }
  for (int c = lane; c < D4; c += 64)
    *reinterpret_cast<f4v*>(l.z + 4 * c) =
        *reinterpret_cast<const f4v*>(dense + (size_t)s * D + 4 * c);
  int tt[NQ], cc[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int it = q * 64 + lane;
    tt[q] = it < T * D4 ? it / D4 : -1;
    cc[q] = tt[q] >= 0 ? it - tt[q] * D4 : 0;
  }
  f4v acc[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) acc[q] = f4v{0.f, 0.f, 0.f, 0.f};
  for (int64_t j = 0; j < maxlen; ++j) {
    if (lane < T) {
      uint32_t r = kNoRow;
      if (j < len) {
        const int64_t id = ids[o0 + j];
        if (id >= 0 && id < nrows) r = (uint32_t)(roff + id);
        else if (id != kAbsentId) bad |= EMB_FLAG_OUT_OF_RANGE;
      }
      l.row[lane] = r;
    }
    wave_sync();
    f4v x[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const uint32_t r = tt[q] >= 0 ? l.row[tt[q]] : kNoRow;
      const bool ok = r != kNoRow;
      const f4v v = *reinterpret_cast<const f4v*>(W + (ok ? (size_t)r * D + 4 * cc[q] : 0));
      x[q] = ok ? v : f4v{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) acc[q] += x[q];
    wave_sync();  // l.row is rewritten by the next position
  }
  // every lane learns its items' bag lengths from the lanes that own them
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int64_t lq = __shfl(len, tt[q] >= 0 ? tt[q] : 0, 64);
    if (tt[q] < 0) continue;
    f4v v = acc[q];
    if (MEAN && lq > 0) v *= 1.0f / (float)lq;
    *reinterpret_cast<f4v*>(l.z + (size_t)(tt[q] + 1) * zs + 4 * cc[q]) = v;
  }
  wave_sync();
}

template <bool MEAN, int NQ>
__global__ __launch_bounds__(256) void k_interact_fwd(
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
  for (int64_t s = (int64_t)blockIdx.x * wpb + w; s < B; s += (int64_t)gridDim.x * wpb) {
    gather_z<MEAN, NQ>(l, s, dense, offsets, ids, row_off, rows, W, B, T, D, nnz, bad);
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
    wave_sync();
  }
  const uint32_t any = (uint32_t)(__ballot(bad != 0) != 0);
  if (any) {
    uint32_t all = bad;
    for (int o = 1; o < 64; o <<= 1) all |= (uint32_t)__shfl_xor((int)all, o, 64);
    if (lane == 0) atomicOr(flags, all);
  }
}

template <bool MEAN, int NQ>
__global__ __launch_bounds__(256) void k_interact_bwd(
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
  for (int64_t s = (int64_t)blockIdx.x * wpb + w; s < B; s += (int64_t)gridDim.x * wpb) {
    gather_z<MEAN, NQ>(l, s, dense, offsets, ids, row_off, rows, W, B, T, D, nnz, bad);
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
    const int mblocks = T + 1 > 16 ? 2 : 1;
    for (int n0 = 0; n0 < D; n0 += 16) {
      for (int mb = 0; mb < mblocks; ++mb) {
        f4v acc = {0.f, 0.f, 0.f, 0.f};
        // A[i][k] = G[16 mb + i][k], B[k][n] = Z[k][n0 + n] (zero past row T)
        for (int k0 = 0; k0 < 32; k0 += 4) {
          const int k = k0 + kq;
          const float a = l.g[(16 * mb + ri) * 33 + k];
          const float b = k <= T ? l.z[(size_t)k * zs + n0 + ri] : 0.0f;
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
        }
        // lane holds dZ[16 mb + 4 (l / 16) + r][n0 + l % 16]
        const int col = n0 + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * mb + 4 * (lane >> 4) + r;
          if (row == 0)
            grad_dense[s * D + col] = go[col] + acc[r];
          else if (row <= T)
            grad_pooled[((size_t)s * T + (row - 1)) * D + col] = acc[r];
        }
      }
    }
    wave_sync();
  }
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
