// Table initialisation and fill kernels.
//
// Dense rows are drawn from a counter-based generator so that any row of a
// table of any size has a fixed initial value without host traffic:
//   h = SM(SM(SM(SM(seed) ^ t) ^ r) ^ d),  SM = one SplitMix64 step
//   (Steele, Lea and Flood, OOPSLA 2014);  u = top 24 bits of h / 2^24;
//   W[off_t + r, d] = fmaf(u, hi - lo, lo);  G = accum_init.
// One thread writes one float4 column group; the row prefix (three SM steps)
// is shared by its four elements.  Fills use plain vector stores (no
// hipMemset nodes, so the same code can sit inside a captured graph).
#include "embtab_internal.hpp"

namespace embtab {

namespace {

__global__ __launch_bounds__(256) void k_init_dense(float* __restrict__ W, float* __restrict__ G,
                                                    const int64_t* __restrict__ row_off, int32_t T,
                                                    int32_t D, uint64_t seed, float lo, float hi,
                                                    float g0, int64_t total_rows, int32_t hashed) {
  const int64_t D4 = D >> 2;
  const int64_t n4 = total_rows * D4;
  const uint64_t s0 = sm64(seed);
  const float span = hi - lo;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n4;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = e / D4;
    const int64_t d4 = e - row * D4;
    f4 gv = f4{g0, g0, g0, g0};
    *reinterpret_cast<f4*>(G + (size_t)row * D + 4 * d4) = gv;
    if (hashed) continue;  // rows of hashed tables are written when a key is inserted
    int32_t t = 0;
    while (t + 1 < T && row_off[t + 1] <= row) ++t;
    const uint64_t local = (uint64_t)(row - row_off[t]);
    const uint64_t pre = sm64(sm64(s0 ^ (uint64_t)t) ^ local);
    f4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint64_t h = sm64(pre ^ (uint64_t)(4 * d4 + i));
      const float u = (float)(uint32_t)(h >> 40) * (1.0f / 16777216.0f);
      w[i] = __builtin_fmaf(u, span, lo);
    }
    *reinterpret_cast<f4*>(W + (size_t)row * D + 4 * d4) = w;
  }
}

__global__ __launch_bounds__(256) void k_fill_u64(uint64_t* __restrict__ p, uint64_t v, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

__global__ __launch_bounds__(256) void k_fill_f32(float* __restrict__ p, float v, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

__global__ void k_zero_words(uint32_t* __restrict__ p, int32_t n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

unsigned grid_for(size_t n) {
  size_t g = (n + 255) / 256;
  const size_t cap = 256 * 64;  // 64 blocks per CU, then grid-stride
  if (g > cap) g = cap;
  if (g == 0) g = 1;
  return (unsigned)g;
}

}  // namespace

hipError_t launch_init_dense(const Handle& h, hipStream_t s) {
  const size_t n4 = (size_t)h.total_rows * (size_t)(h.D / 4);
  hipLaunchKernelGGL(k_init_dense, dim3(grid_for(n4)), dim3(256), 0, s, h.W, h.G, h.sv.row_off,
                     h.T, h.D, h.seed, h.lo, h.hi, h.accum0, h.total_rows, h.hashed ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_fill_u64(uint64_t* p, uint64_t v, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_u64, dim3(grid_for(n)), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

hipError_t launch_zero_words(uint32_t* p, int n, hipStream_t s) {
  hipLaunchKernelGGL(k_zero_words, dim3(1), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* p, float v, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_f32, dim3(grid_for(n)), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

}  // namespace embtab
