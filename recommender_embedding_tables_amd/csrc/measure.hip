// Stream kernels that measure what HBM sustains on this device, the yardstick
// beside the published peak for the path's kernels (which are all bound by
// HBM bandwidth, as the "NVIDIA Merlin Distributed Embeddings" page,
// section "Background", says of embedding lookups).
//
// Copy, fill and read of a contiguous buffer: thread i of block b moves the
// one 16-byte item b * 256 + i, so each block covers 4 KiB and retires (no
// grid-stride loop; the read kernel takes four items per thread).  On MI355X this one-shot form measured faster than
// persistent grid-stride forms (eight blocks per compute unit, 1 or 4 items per
// thread per round): fill 6.5-6.75 vs 4.1-5.7 TB/s, copy 6.5 vs 5.8-5.9 TB/s
// (each way counted), read equal at 6.9-7.0 TB/s.  Copy loads and stores are
// non-temporal (the data is touched once); fill uses plain stores (6.75 vs 6.5
// TB/s non-temporal); the read kernel adds its items and writes one value per
// wave, so the loads cannot be dropped.
#include "embtab_internal.hpp"

namespace embtab {

namespace {

constexpr unsigned kStreamItemsPerBlock = 256;

__global__ __launch_bounds__(256) void k_stream_copy(const f4* __restrict__ src,
                                                     f4* __restrict__ dst, size_t n) {
  const size_t k = (size_t)blockIdx.x * kStreamItemsPerBlock + threadIdx.x;
  if (k < n) __builtin_nontemporal_store(__builtin_nontemporal_load(src + k), dst + k);
}

__global__ __launch_bounds__(256) void k_stream_fill(f4* __restrict__ dst, f4 value, size_t n) {
  const size_t k = (size_t)blockIdx.x * kStreamItemsPerBlock + threadIdx.x;
  if (k < n) dst[k] = value;
}

// Four items per thread (16 KiB per block) and one sum per wave, so that no
// block barrier sits between a block's loads and its retirement.
constexpr unsigned kReadItemsPerThread = 4;

__global__ __launch_bounds__(256) void k_stream_read(const f4* __restrict__ src,
                                                     float* __restrict__ sink, size_t n) {
  const size_t base =
      (size_t)blockIdx.x * kStreamItemsPerBlock * kReadItemsPerThread + threadIdx.x;
  f4 v[kReadItemsPerThread];
#pragma unroll
  for (unsigned u = 0; u < kReadItemsPerThread; ++u) {
    const size_t k = base + (size_t)u * kStreamItemsPerBlock;
    v[u] = k < n ? __builtin_nontemporal_load(src + k) : f4{0.f, 0.f, 0.f, 0.f};
  }
  f4 acc = v[0];
#pragma unroll
  for (unsigned u = 1; u < kReadItemsPerThread; ++u) acc += v[u];
  float s = acc[0] + acc[1] + acc[2] + acc[3];
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  if ((threadIdx.x & 63u) == 0u) sink[(size_t)blockIdx.x * 4u + (threadIdx.x >> 6)] = s;
}

}  // namespace

// Blocks of a stream kernel over `bytes`: one per 256 16-byte items (copy,
// fill) or per 1024 (read, kind 2).
size_t stream_blocks(int kind, size_t bytes) {
  const size_t n = bytes / 16;
  const size_t per = kStreamItemsPerBlock * (kind == 2 ? kReadItemsPerThread : 1u);
  return (n + per - 1) / per;
}

// Floats the read kernel writes over `bytes`: one per wave.
size_t stream_read_sink_floats(size_t bytes) { return 4u * stream_blocks(2, bytes); }

hipError_t launch_stream(int kind, void* dst, const void* src, size_t bytes, float value,
                         hipStream_t s) {
  const size_t n = bytes / 16;
  if (n == 0) return hipSuccess;
  const size_t grid = stream_blocks(kind, bytes);
  if (grid > 0x7FFFFFFFu) return hipErrorInvalidValue;
  switch (kind) {
    case 0:
      hipLaunchKernelGGL(k_stream_copy, dim3((unsigned)grid), dim3(256), 0, s,
                         static_cast<const f4*>(src), static_cast<f4*>(dst), n);
      break;
    case 1:
      hipLaunchKernelGGL(k_stream_fill, dim3((unsigned)grid), dim3(256), 0, s,
                         static_cast<f4*>(dst), f4{value, value, value, value}, n);
      break;
    default:
      hipLaunchKernelGGL(k_stream_read, dim3((unsigned)grid), dim3(256), 0, s,
                         static_cast<const f4*>(src), static_cast<float*>(dst), n);
      break;
  }
  return hipGetLastError();
}

}  // namespace embtab
