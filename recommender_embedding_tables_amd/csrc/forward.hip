// Pooled embedding lookup (EmbeddingBag forward) for gfx950.
//
// out[s, t, :] = c_b * sum_{j in bag b} W[off_t + ids[j], :],  b = t*B + s
// (lookup of encoded categorical ids, "NVIDIA Merlin Distributed Embeddings",
// introduction and "Background"; pooling of a feature's rows, "Merlin HugeCTR
// interview", section three, technique (5)).
//
// Layout and schedule: a sub-group of SG lanes (SG = D/4 rounded up to a power
// of two, at most 64) owns one bag; each lane holds VEC float4 columns, so a
// row is read with dwordx4 loads that cover it contiguously.  A sub-group keeps
// UNR bags in flight at once.  Bags are visited in output order (sample-major,
// q = s*T + t), so consecutive sub-groups write consecutive 16-byte columns of
// `out` and each store instruction of a wave covers one contiguous span.  The
// ids of a bag are fetched SG at a time with one coalesced load and broadcast
// by lane shuffles, so a multi-hot bag costs one id round trip per SG ids.
// Rows are gathered through the cache hierarchy (hot Zipf rows stay in L2 /
// MALL); `out` is written with non-temporal stores since it is streamed once.
#include "embtab_internal.hpp"

namespace embtab {

namespace {

template <int SG, int VEC, bool MEAN, int UNR>
__global__ __launch_bounds__(256) void k_bag_forward(
    const int64_t* __restrict__ offsets, const int64_t* __restrict__ ids,
    const float* __restrict__ W, const int64_t* __restrict__ row_off,
    const int64_t* __restrict__ rows, float* __restrict__ out, uint32_t* __restrict__ flags,
    int64_t B, int32_t T, int32_t D, int64_t nnz) {
  constexpr int SGPB = 256 / SG;
  const int lane = threadIdx.x % SG;
  const int sgb = threadIdx.x / SG;
  const int64_t nbags = B * (int64_t)T;
  const int64_t qbase = (int64_t)blockIdx.x * SGPB * UNR + sgb;
  const int D4 = D >> 2;

  int64_t start[UNR];
  int32_t len[UNR];
  uint32_t roff[UNR];
  int64_t nrows[UNR];
  uint32_t bad = 0;
  int32_t maxlen = 0;
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    const int64_t q = qbase + (int64_t)u * SGPB;
    start[u] = 0;
    len[u] = 0;
    roff[u] = 0;
    nrows[u] = 0;
    if (q < nbags) {
      const int64_t t = q % T;
      const int64_t s = q / T;
      const int64_t b = t * B + s;
      int64_t o0 = offsets[b], o1 = offsets[b + 1];
      if ((b == 0 && o0 != 0) || (b == nbags - 1 && o1 != nnz) || o1 < o0 || o0 < 0 || o1 > nnz)
        bad |= EMB_FLAG_BAD_OFFSETS;
      o0 = o0 < 0 ? 0 : (o0 > nnz ? nnz : o0);
      o1 = o1 < o0 ? o0 : (o1 > nnz ? nnz : o1);
      start[u] = o0;
      len[u] = (int32_t)(o1 - o0);
      roff[u] = (uint32_t)row_off[t];
      nrows[u] = rows[t];
      maxlen = len[u] > maxlen ? len[u] : maxlen;
    }
  }

  f4 acc[UNR][VEC];
#pragma unroll
  for (int u = 0; u < UNR; ++u)
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[u][v] = f4{0.f, 0.f, 0.f, 0.f};

  for (int32_t kb = 0; kb < maxlen; kb += SG) {
    // One coalesced id load per bag per SG occurrences; invalid -> kNoRow.
    uint32_t myrow[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      myrow[u] = kNoRow;
      if (kb + lane < len[u]) {
        const int64_t id = ids[start[u] + kb + lane];
        if (id >= 0 && id < nrows[u]) myrow[u] = roff[u] + (uint32_t)id;
        else bad |= EMB_FLAG_OUT_OF_RANGE;
      }
    }
    int32_t kend = maxlen - kb;
    kend = kend > SG ? SG : kend;
    for (int32_t kk = 0; kk < kend; ++kk) {
      uint32_t grow[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) grow[u] = (uint32_t)__shfl((int)myrow[u], kk, SG);
      f4 x[UNR][VEC];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          const int d4 = lane + v * SG;
          x[u][v] = f4{0.f, 0.f, 0.f, 0.f};
          if (grow[u] != kNoRow && d4 < D4)
            x[u][v] = *reinterpret_cast<const f4*>(W + (size_t)grow[u] * D + 4 * d4);
        }
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u)
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[u][v] += x[u][v];
    }
  }

#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    const int64_t q = qbase + (int64_t)u * SGPB;
    if (q >= nbags) continue;
    float c = 1.0f;
    if (MEAN && len[u] > 0) c = 1.0f / (float)len[u];
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      const int d4 = lane + v * SG;
      if (d4 < D4) {
        f4 r = MEAN ? acc[u][v] * c : acc[u][v];
        __builtin_nontemporal_store(r, reinterpret_cast<f4*>(out + (size_t)q * D + 4 * d4));
      }
    }
  }
  if (bad) atomicOr(flags, bad);
}

template <int SG, int VEC, bool MEAN>
hipError_t launch_t(const Handle& h, const int64_t* offsets, const int64_t* ids, int64_t B,
                    int64_t nnz, float* out, hipStream_t s) {
  constexpr int UNR = 4;
  constexpr int SGPB = 256 / SG;
  const int64_t nbags = B * (int64_t)h.T;
  const int64_t per_block = (int64_t)SGPB * UNR;
  const int64_t grid = (nbags + per_block - 1) / per_block;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((k_bag_forward<SG, VEC, MEAN, UNR>), dim3((unsigned)grid), dim3(256), 0, s,
                     offsets, ids, h.W, h.sv.row_off, h.sv.rows, out, h.sv.flags, B, h.T, h.D,
                     nnz);
  return hipGetLastError();
}

template <bool MEAN>
hipError_t dispatch(const Handle& h, const int64_t* offsets, const int64_t* ids, int64_t B,
                    int64_t nnz, float* out, hipStream_t s) {
  const int sg = subgroup_lanes(h.D), vec = vec_per_lane(h.D);
  switch (sg) {
    case 1: return launch_t<1, 1, MEAN>(h, offsets, ids, B, nnz, out, s);
    case 2: return launch_t<2, 1, MEAN>(h, offsets, ids, B, nnz, out, s);
    case 4: return launch_t<4, 1, MEAN>(h, offsets, ids, B, nnz, out, s);
    case 8: return launch_t<8, 1, MEAN>(h, offsets, ids, B, nnz, out, s);
    case 16: return launch_t<16, 1, MEAN>(h, offsets, ids, B, nnz, out, s);
    case 32: return launch_t<32, 1, MEAN>(h, offsets, ids, B, nnz, out, s);
    default:
      switch (vec) {
        case 1: return launch_t<64, 1, MEAN>(h, offsets, ids, B, nnz, out, s);
        case 2: return launch_t<64, 2, MEAN>(h, offsets, ids, B, nnz, out, s);
        case 3: return launch_t<64, 3, MEAN>(h, offsets, ids, B, nnz, out, s);
        default: return launch_t<64, 4, MEAN>(h, offsets, ids, B, nnz, out, s);
      }
  }
}

}  // namespace

hipError_t launch_forward(const Handle& h, const int64_t* offsets, const int64_t* ids,
                          int64_t B, int64_t nnz, bool mean, float* out, hipStream_t s) {
  phase_mark(h, EMB_PHASE_FORWARD, false, s);
  hipError_t e = mean ? dispatch<true>(h, offsets, ids, B, nnz, out, s)
                      : dispatch<false>(h, offsets, ids, B, nnz, out, s);
  phase_mark(h, EMB_PHASE_FORWARD, true, s);
  return e;
}

}  // namespace embtab
