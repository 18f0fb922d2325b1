// Pooled embedding lookup (EmbeddingBag forward) for gfx950.
//
// out[s, t, :] = c_b * sum_{j in bag b} W[off_t + ids[j], :],  b = t*B + s
// (lookup of encoded categorical ids, "NVIDIA Merlin Distributed Embeddings",
// introduction and "Background"; pooling of a feature's rows, "Merlin HugeCTR
// interview", section three, technique (5)).
//
// Layout and schedule: a sub-group of SG lanes (SG = D/4 rounded up to a power
// of two, at most 64) reads a row with one dwordx4 load per lane (VEC float4
// columns per lane when D > 256).  It owns SG consecutive bags in CSR
// (table-major) order, one per lane for metadata: their offsets come in with
// one coalesced load, and when every bag of the wave holds at most one id
// (one-hot features) their ids with a second one, so a bag costs no dependent
// metadata round trip of its own.  The sub-group then walks its bags UNR at a
// time, broadcasting each bag's row by lane shuffle, with UNR row loads in
// flight per lane.  Multi-hot bags fetch their ids SG at a time with one
// coalesced load and broadcast them the same way.  Rows go through the cache
// hierarchy (hot Zipf rows stay in L2 / MALL); `out` is written once with
// non-temporal stores.  Blocks are remapped so that each XCD covers one
// contiguous range of bags.
#include "embtab_internal.hpp"

namespace embtab {

namespace {

template <int SG, int VEC, bool MEAN, int UNR>
__global__ __launch_bounds__(256) void k_bag_forward(
    const int64_t* __restrict__ offsets, const int64_t* __restrict__ ids,
    const float* __restrict__ W, const int64_t* __restrict__ row_off,
    const int64_t* __restrict__ rows, float* __restrict__ out, uint32_t* __restrict__ flags,
    uint32_t B, uint32_t T, uint32_t D, uint32_t nnz) {
  constexpr int SGPB = 256 / SG;
  const uint32_t lane = threadIdx.x % SG;
  const uint32_t sgb = threadIdx.x / SG;
  const uint32_t nbags = B * T;
  const uint32_t b0 = (xcd_block() * SGPB + sgb) * (uint32_t)SG;  // first bag of the sub-group
  const uint32_t D4 = D >> 2;

  // Lane metadata: bag b0 + lane.
  const uint32_t b = b0 + lane;
  uint32_t start = 0u, len = 0u, t = 0u, s = 0u, bad = 0u;
  uint32_t roff = 0u, nrow = 0u;
  if (b < nbags) {
    t = b / B;
    s = b - t * B;
    int64_t o0 = offsets[b], o1 = offsets[b + 1];
    roff = (uint32_t)row_off[t];
    nrow = (uint32_t)rows[t];
    if ((b == 0 && o0 != 0) || (b == nbags - 1 && o1 != (int64_t)nnz) || o1 < o0 || o0 < 0 ||
        o1 > (int64_t)nnz)
      bad |= EMB_FLAG_BAD_OFFSETS;
    o0 = o0 < 0 ? 0 : (o0 > (int64_t)nnz ? (int64_t)nnz : o0);
    o1 = o1 < o0 ? o0 : (o1 > (int64_t)nnz ? (int64_t)nnz : o1);
    start = (uint32_t)o0;
    len = (uint32_t)(o1 - o0);
  }
  const bool onehot = __all(len <= 1u);
  uint32_t myrow = kNoRow;
  if (onehot && len == 1u) {
    const int64_t id = ids[start];
    if (id >= 0 && id < (int64_t)nrow) myrow = roff + (uint32_t)id;
    else bad |= EMB_FLAG_OUT_OF_RANGE;
  }

  if (onehot) {
#pragma unroll 1
    for (uint32_t i0 = 0; i0 < (uint32_t)SG; i0 += UNR) {
      if (b0 + i0 >= nbags) break;
      f4 acc[UNR][VEC];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const uint32_t grow = (uint32_t)__shfl((int)myrow, (int)(i0 + u), SG);
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          const uint32_t d4 = lane + v * SG;
          acc[u][v] = f4{0.f, 0.f, 0.f, 0.f};
          if (grow != kNoRow && d4 < D4)
            acc[u][v] = *reinterpret_cast<const f4*>(W + (size_t)grow * D + 4 * d4);
        }
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const uint32_t bt = (uint32_t)__shfl((int)t, (int)(i0 + u), SG);
        const uint32_t bs = (uint32_t)__shfl((int)s, (int)(i0 + u), SG);
        if (b0 + i0 + u >= nbags) continue;
        const size_t o = ((size_t)bs * T + bt) * D;
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          const uint32_t d4 = lane + v * SG;
          if (d4 < D4)
            __builtin_nontemporal_store(acc[u][v], reinterpret_cast<f4*>(out + o + 4 * d4));
        }
      }
    }
  } else {
    // Multi-hot: MU bags at a time, their ids SG at a time, KU rows in flight per bag.
    constexpr int MU = 2, KU = 4;
#pragma unroll 1
    for (uint32_t i0 = 0; i0 < (uint32_t)SG; i0 += MU) {
      if (b0 + i0 >= nbags) break;
      uint32_t bl[MU], bst[MU], broff[MU], bnr[MU];
      uint32_t maxlen = 0u;
      f4 acc[MU][VEC];
#pragma unroll
      for (int u = 0; u < MU; ++u) {
        bl[u] = (uint32_t)__shfl((int)len, (int)(i0 + u), SG);
        bst[u] = (uint32_t)__shfl((int)start, (int)(i0 + u), SG);
        broff[u] = (uint32_t)__shfl((int)roff, (int)(i0 + u), SG);
        bnr[u] = (uint32_t)__shfl((int)nrow, (int)(i0 + u), SG);
        maxlen = bl[u] > maxlen ? bl[u] : maxlen;
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[u][v] = f4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll 1
      for (uint32_t kb = 0; kb < maxlen; kb += SG) {
        uint32_t r[MU];
#pragma unroll
        for (int u = 0; u < MU; ++u) {
          r[u] = kNoRow;
          if (kb + lane < bl[u]) {
            const int64_t id = ids[bst[u] + kb + lane];
            if (id >= 0 && id < (int64_t)bnr[u]) r[u] = broff[u] + (uint32_t)id;
            else bad |= EMB_FLAG_OUT_OF_RANGE;
          }
        }
        const uint32_t kend = (maxlen - kb) < (uint32_t)SG ? (maxlen - kb) : (uint32_t)SG;
#pragma unroll 1
        for (uint32_t kk = 0; kk < kend; kk += KU) {
          f4 x[MU][KU][VEC];
#pragma unroll
          for (int u = 0; u < MU; ++u)
#pragma unroll
            for (int k = 0; k < KU; ++k) {
              // lanes past kend hold kNoRow, so the tail of the last group loads nothing
              const uint32_t src = kk + k < (uint32_t)SG ? kk + k : (uint32_t)SG - 1u;
              uint32_t grow = (uint32_t)__shfl((int)r[u], (int)src, SG);
              if (kk + k >= kend) grow = kNoRow;
#pragma unroll
              for (int v = 0; v < VEC; ++v) {
                const uint32_t d4 = lane + v * SG;
                x[u][k][v] = f4{0.f, 0.f, 0.f, 0.f};
                if (grow != kNoRow && d4 < D4)
                  x[u][k][v] = *reinterpret_cast<const f4*>(W + (size_t)grow * D + 4 * d4);
              }
            }
#pragma unroll
          for (int u = 0; u < MU; ++u)
#pragma unroll
            for (int k = 0; k < KU; ++k)
#pragma unroll
              for (int v = 0; v < VEC; ++v) acc[u][v] += x[u][k][v];
        }
      }
#pragma unroll
      for (int u = 0; u < MU; ++u) {
        const uint32_t bt = (uint32_t)__shfl((int)t, (int)(i0 + u), SG);
        const uint32_t bs = (uint32_t)__shfl((int)s, (int)(i0 + u), SG);
        if (b0 + i0 + u >= nbags) continue;
        float c = 1.0f;
        if (MEAN && bl[u] > 0) c = 1.0f / (float)bl[u];
        const size_t o = ((size_t)bs * T + bt) * D;
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          const uint32_t d4 = lane + v * SG;
          if (d4 < D4) {
            const f4 rr = MEAN ? acc[u][v] * c : acc[u][v];
            __builtin_nontemporal_store(rr, reinterpret_cast<f4*>(out + o + 4 * d4));
          }
        }
      }
    }
  }
  if (bad) atomicOr(flags, bad);
}

template <int SG, int VEC, bool MEAN>
hipError_t launch_t(const Handle& h, const int64_t* offsets, const int64_t* ids, int64_t B,
                    int64_t nnz, float* out, hipStream_t s) {
  constexpr int UNR = VEC == 1 ? (SG >= 8 ? 8 : SG) : (VEC == 2 ? 4 : 2);  // one-hot rows in flight
  constexpr int SGPB = 256 / SG;
  const int64_t nbags = B * (int64_t)h.T;
  const int64_t per_block = (int64_t)SGPB * SG;
  const int64_t grid = (nbags + per_block - 1) / per_block;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((k_bag_forward<SG, VEC, MEAN, UNR>), dim3((unsigned)grid), dim3(256), 0, s,
                     offsets, ids, h.W, h.sv.row_off, h.sv.rows, out, h.sv.flags, (uint32_t)B,
                     (uint32_t)h.T, (uint32_t)h.D, (uint32_t)nnz);
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
