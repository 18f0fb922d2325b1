// int8 payload of the embedding exchange between ranks, for gfx950.
//
// A table-wise split exchanges the pooled embeddings (forward) and their
// gradients (backward) between the ranks that own the tables and the ranks
// that own the samples.  The OneFlow OneEmbedding page (section "quantized
// compression") quantizes that payload from float to int8 before the
// exchange and dequantizes it after.  The page gives no scheme; the reading:
// one symmetric fp32 scale per row of D values, codes in [-127, 127]:
//   amax = max_d |x_d|;  amax == 0: scale 0, codes 0;
//   inv = 127 / amax;  code_d = x_d * inv rounded to nearest (ties to even),
//   clamped to +-127;  scale = amax / 127;  dequantized x_d = code_d * scale,
// every step in fp32 (correctly rounded division).  A code is an integer that
// fp32 arithmetic decides, so every step is written out as such.
//
// One sub-group of SG lanes per row (SG = D/4 rounded up to a power of two, at
// most 64), each lane VEC float4 columns: a row is one pass.  The row maximum
// is a shuffle reduction inside the sub-group; codes leave as one 4-byte word
// per float4 (consecutive across the sub-group), the scale from the
// sub-group's first lane.  The payload is streamed once: non-temporal loads
// and stores.
#include "embtab_internal.hpp"

namespace embtab {

namespace {

template <int SG, int VEC>
__global__ __launch_bounds__(256) void k_quantize_rows(const float* __restrict__ x, int64_t rows,
                                                       int32_t D, uint32_t* __restrict__ codes,
                                                       float* __restrict__ scales) {
  constexpr int RPB = 256 / SG;  // rows per block
  const int lane = threadIdx.x % SG;
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / SG;
  if (r >= rows) return;  // the whole sub-group: its shuffles stay inside it
  const int D4 = D >> 2;
  const f4* xr = reinterpret_cast<const f4*>(x + r * D);
  f4 v[VEC];
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < VEC; ++k) {
    const int c = lane + k * SG;
    v[k] = c < D4 ? __builtin_nontemporal_load(xr + c) : f4{0.f, 0.f, 0.f, 0.f};
    amax = __builtin_fmaxf(amax, abs_max4(v[k]));
  }
  for (int o = SG / 2; o > 0; o >>= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, o, SG));
  const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
  uint32_t* cr = codes + r * D4;
#pragma unroll
  for (int k = 0; k < VEC; ++k) {
    const int c = lane + k * SG;
    if (c < D4) {
      __builtin_nontemporal_store(int8_code_word(v[k], inv), cr + c);
    }
  }
  if (lane == 0) scales[r] = amax / 127.0f;
}

template <int SG, int VEC>
__global__ __launch_bounds__(256) void k_dequantize_rows(const uint32_t* __restrict__ codes,
                                                         const float* __restrict__ scales,
                                                         int64_t rows, int32_t D,
                                                         float* __restrict__ y) {
  constexpr int RPB = 256 / SG;
  const int lane = threadIdx.x % SG;
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / SG;
  if (r >= rows) return;
  const int D4 = D >> 2;
  const float s = scales[r];
  const uint32_t* cr = codes + r * D4;
  f4* yr = reinterpret_cast<f4*>(y + r * D);
#pragma unroll
  for (int k = 0; k < VEC; ++k) {
    const int c = lane + k * SG;
    if (c < D4) {
      const uint32_t w = __builtin_nontemporal_load(cr + c);
      const f4 o = {(float)(int8_t)(w & 0xFFu) * s, (float)(int8_t)((w >> 8) & 0xFFu) * s,
                    (float)(int8_t)((w >> 16) & 0xFFu) * s, (float)(int8_t)(w >> 24) * s};
      __builtin_nontemporal_store(o, yr + c);
    }
  }
}

template <bool DEQ, int SG, int VEC>
hipError_t launch_t(const float* x, const uint32_t* cin, uint32_t* cout, float* scales_out,
                    const float* scales_in, float* y, int64_t rows, int32_t D, hipStream_t s) {
  constexpr int RPB = 256 / SG;
  const int64_t grid = (rows + RPB - 1) / RPB;
  if (DEQ)
    hipLaunchKernelGGL((k_dequantize_rows<SG, VEC>), dim3((unsigned)grid), dim3(256), 0, s, cin,
                       scales_in, rows, D, y);
  else
    hipLaunchKernelGGL((k_quantize_rows<SG, VEC>), dim3((unsigned)grid), dim3(256), 0, s, x,
                       rows, D, cout, scales_out);
  return hipGetLastError();
}

template <bool DEQ>
hipError_t dispatch(const float* x, const uint32_t* cin, uint32_t* cout, float* scales_out,
                    const float* scales_in, float* y, int64_t rows, int32_t D, hipStream_t s) {
  const int sg = subgroup_lanes(D), vec = vec_per_lane(D);
#define EMBTAB_Q_LAUNCH(SG_, VEC_) \
  launch_t<DEQ, SG_, VEC_>(x, cin, cout, scales_out, scales_in, y, rows, D, s)
  switch (sg) {
    case 1: return EMBTAB_Q_LAUNCH(1, 1);
    case 2: return EMBTAB_Q_LAUNCH(2, 1);
    case 4: return EMBTAB_Q_LAUNCH(4, 1);
    case 8: return EMBTAB_Q_LAUNCH(8, 1);
    case 16: return EMBTAB_Q_LAUNCH(16, 1);
    case 32: return EMBTAB_Q_LAUNCH(32, 1);
    default:
      switch (vec) {
        case 1: return EMBTAB_Q_LAUNCH(64, 1);
        case 2: return EMBTAB_Q_LAUNCH(64, 2);
        case 3: return EMBTAB_Q_LAUNCH(64, 3);
        default: return EMBTAB_Q_LAUNCH(64, 4);
      }
  }
#undef EMBTAB_Q_LAUNCH
}

}  // namespace

hipError_t launch_quantize_rows(const float* x, int64_t rows, int32_t D, int8_t* codes,
                                float* scales, hipStream_t s) {
  return dispatch<false>(x, nullptr, reinterpret_cast<uint32_t*>(codes), scales, nullptr,
                         nullptr, rows, D, s);
}

hipError_t launch_dequantize_rows(const int8_t* codes, const float* scales, int64_t rows,
                                  int32_t D, float* y, hipStream_t s) {
  return dispatch<true>(nullptr, reinterpret_cast<const uint32_t*>(codes), nullptr, nullptr,
                        scales, y, rows, D, s);
}

}  // namespace embtab
