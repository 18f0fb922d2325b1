// Stream kernels that measure what HBM sustains on this device, the yardstick
// beside the published peak for the path's kernels (which are all bound by
// HBM bandwidth, as the "NVIDIA Merlin Distributed Embeddings" page,
// section "Background", says of embedding lookups).
//
// Copy, fill and read of a contiguous buffer: each thread moves U dwordx4
// (16-byte) items per round, consecutive lanes on consecutive items, all U
// loads issued before any store; grid-stride rounds.  Loads and stores are
// non-temporal (the data is touched once).  The read kernel adds its items
// and writes one value per block, so the loads cannot be dropped.
#include "embtab_internal.hpp"

namespace embtab {

namespace {

constexpr int kMeasureUnroll = 4;

template <int U>
__global__ __launch_bounds__(256) void k_stream_copy(const f4* __restrict__ src,
                                                     f4* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * 256u * U;
  for (size_t i = (size_t)blockIdx.x * 256u * U + threadIdx.x; i < n; i += stride) {
    f4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t k = i + (size_t)u * 256u;
      v[u] = __builtin_nontemporal_load(src + (k < n ? k : 0));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t k = i + (size_t)u * 256u;
      if (k < n) __builtin_nontemporal_store(v[u], dst + k);
    }
  }
}

template <int U>
__global__ __launch_bounds__(256) void k_stream_fill(f4* __restrict__ dst, f4 value, size_t n) {
  const size_t stride = (size_t)gridDim.x * 256u * U;
  for (size_t i = (size_t)blockIdx.x * 256u * U + threadIdx.x; i < n; i += stride) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t k = i + (size_t)u * 256u;
      if (k < n) __builtin_nontemporal_store(value, dst + k);
    }
  }
}

template <int U>
__global__ __launch_bounds__(256) void k_stream_read(const f4* __restrict__ src,
                                                     float* __restrict__ sink, size_t n) {
  __shared__ float part[4];
  const size_t stride = (size_t)gridDim.x * 256u * U;
  f4 acc = f4{0.f, 0.f, 0.f, 0.f};
  for (size_t i = (size_t)blockIdx.x * 256u * U + threadIdx.x; i < n; i += stride) {
    f4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t k = i + (size_t)u * 256u;
      v[u] = __builtin_nontemporal_load(src + (k < n ? k : 0));
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (i + (size_t)u * 256u < n) acc += v[u];
  }
  float s = acc[0] + acc[1] + acc[2] + acc[3];
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  if ((threadIdx.x & 63u) == 0u) part[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] + part[1] + part[2] + part[3];
}

}  // namespace

// Blocks of a stream kernel over `bytes`: eight 256-thread blocks per
// compute unit of the current device (fewer for small buffers).
unsigned stream_blocks(size_t bytes) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0) {
    (void)hipGetLastError();
    cus = 256;
  }
  const size_t n = bytes / 16, per_block = 256u * kMeasureUnroll;
  const size_t g = (n + per_block - 1) / per_block, cap = (size_t)cus * 8u;
  return (unsigned)(g < cap ? (g > 0 ? g : 1) : cap);
}

hipError_t launch_stream(int kind, void* dst, const void* src, size_t bytes, float value,
                         hipStream_t s) {
  const size_t n = bytes / 16;
  if (n == 0) return hipSuccess;
  const unsigned grid = stream_blocks(bytes);
  switch (kind) {
    case 0:
      hipLaunchKernelGGL((k_stream_copy<kMeasureUnroll>), dim3(grid), dim3(256), 0, s,
                         static_cast<const f4*>(src), static_cast<f4*>(dst), n);
      break;
    case 1:
      hipLaunchKernelGGL((k_stream_fill<kMeasureUnroll>), dim3(grid), dim3(256), 0, s,
                         static_cast<f4*>(dst), f4{value, value, value, value}, n);
      break;
    default:
      hipLaunchKernelGGL((k_stream_read<kMeasureUnroll>), dim3(grid), dim3(256), 0, s,
                         static_cast<const f4*>(src), static_cast<float*>(dst), n);
      break;
  }
  return hipGetLastError();
}

}  // namespace embtab
