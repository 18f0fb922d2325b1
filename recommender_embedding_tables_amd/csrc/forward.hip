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

// Sample tile staged through LDS: a block owns samples [s0, s0 + S) of every
// table, i.e. the contiguous output rows q = s0*T .. (s0+S)*T - 1.  Offsets of
// table t for those samples are contiguous (bag b = t*B + s), so they are
// staged with coalesced loads, and so are the ids of one-id bags.  Sub-groups
// then walk the tile in output order.
constexpr int kFwdTileBags = 1024;

// The staging arrays of one sample tile (LDS).
struct BagTileLds {
  uint32_t start[kFwdTileBags], len[kFwdTileBags], row[kFwdTileBags];
};

// Where a pooled row goes, written by all SG lanes of its sub-group at once:
// fp32 rows of `out` [bags, D], or the int8 exchange payload of a table-wise
// split (codes [bags, D] and one scale per row, quantized as
// emb_quantize_rows_int8 does it, so the fp32 rows are never written).
struct F32Rows {
  float* out;
  template <int SG, int VEC>
  __device__ __forceinline__ void put(size_t row, uint32_t D, uint32_t lane,
                                      const f4 (&v)[VEC]) const {
    const uint32_t D4 = D >> 2;
#pragma unroll
    for (int k = 0; k < VEC; ++k) {
      const uint32_t d4 = lane + k * SG;
      if (d4 < D4)
        __builtin_nontemporal_store(v[k], reinterpret_cast<f4*>(out + row * D + 4 * d4));
    }
  }
};
struct I8Rows {
  uint32_t* codes;  // four codes per word
  float* scales;
  template <int SG, int VEC>
  __device__ __forceinline__ void put(size_t row, uint32_t D, uint32_t lane,
                                      const f4 (&v)[VEC]) const {
    const uint32_t D4 = D >> 2;
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < VEC; ++k)
      if (lane + k * SG < D4) amax = __builtin_fmaxf(amax, abs_max4(v[k]));
    for (int o = SG / 2; o > 0; o >>= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, o, SG));
    const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
#pragma unroll
    for (int k = 0; k < VEC; ++k) {
      const uint32_t d4 = lane + k * SG;
      if (d4 < D4) __builtin_nontemporal_store(int8_code_word(v[k], inv), codes + row * D4 + d4);
    }
    if (lane == 0) scales[row] = amax / 127.0f;
  }
};

// Pools sample tile `tile` (samples tile*S .. tile*S + S - 1 of every table);
// returns the EMB_FLAG_* bits it found.  Called by all 256 threads of a block.
template <int SG, int VEC, bool MEAN, int UNR, class OUT>
__device__ __forceinline__ uint32_t bag_tile(
    uint32_t tile, const int64_t* __restrict__ offsets, const int64_t* __restrict__ ids,
    const float* __restrict__ W, const int64_t* __restrict__ row_off,
    const int64_t* __restrict__ rows, OUT out, uint32_t B, uint32_t T,
    uint32_t D, uint32_t nnz, uint32_t S, BagTileLds& lds, const uint32_t* __restrict__ rowmap) {
  constexpr int SGPB = 256 / SG;
  uint32_t* s_start = lds.start;
  uint32_t* s_len = lds.len;
  uint32_t* s_row = lds.row;
  const uint32_t lane = threadIdx.x % SG;
  const uint32_t sgb = threadIdx.x / SG;
  const uint32_t nbags = B * T;
  const uint32_t s0 = tile * S;
  if (s0 >= B) return 0u;
  const uint32_t Sl = (B - s0) < S ? (B - s0) : S;
  const uint32_t ntile = Sl * T;  // bags of the tile; tile bag i = t * Sl + sl
  const uint32_t D4 = D >> 2;
  uint32_t bad = 0u;

  // Stage offsets (coalesced per table), then the ids of one-id bags; each
  // thread owns tile bags tid + 256k, k < 4, with all their loads in flight.
  constexpr int NST = kFwdTileBags / 256;
  int64_t o0[NST], o1[NST];
#pragma unroll
  for (int k = 0; k < NST; ++k) {
    const uint32_t i = threadIdx.x + 256u * k;
    o0[k] = 0;
    o1[k] = 0;
    if (i < ntile) {
      const uint32_t t = i / Sl, sl = i - t * Sl;
      const uint32_t b = t * B + s0 + sl;
      o0[k] = offsets[b];
      o1[k] = offsets[b + 1];
      if ((b == 0 && o0[k] != 0) || (b == nbags - 1 && o1[k] != (int64_t)nnz))
        bad |= EMB_FLAG_BAD_OFFSETS;
    }
  }
  uint32_t tb[NST];
  int64_t idv[NST];
#pragma unroll
  for (int k = 0; k < NST; ++k) {
    const uint32_t i = threadIdx.x + 256u * k;
    tb[k] = i / Sl;
    idv[k] = -1;
    if (i < ntile) {
      if (o1[k] < o0[k] || o0[k] < 0 || o1[k] > (int64_t)nnz) bad |= EMB_FLAG_BAD_OFFSETS;
      const int64_t a = o0[k] < 0 ? 0 : (o0[k] > (int64_t)nnz ? (int64_t)nnz : o0[k]);
      const int64_t e = o1[k] < a ? a : (o1[k] > (int64_t)nnz ? (int64_t)nnz : o1[k]);
      s_start[i] = (uint32_t)a;
      s_len[i] = (uint32_t)(e - a);
      if (e - a == 1) idv[k] = ids[a];
    }
  }
#pragma unroll
  for (int k = 0; k < NST; ++k) {
    const uint32_t i = threadIdx.x + 256u * k;
    if (i < ntile) {
      uint32_t r = kNoRow;
      if (s_len[i] == 1u) {
        const int64_t id = idv[k];
        if (rowmap) r = rowmap[s_start[i]];  // resolved by the prepare (tiered tables)
        else if (id >= 0 && id < rows[tb[k]]) r = (uint32_t)row_off[tb[k]] + (uint32_t)id;
        else if (id != kAbsentId) bad |= EMB_FLAG_OUT_OF_RANGE;
      }
      s_row[i] = r;
    }
  }
  __syncthreads();

  // Output order: tile-local q = sl * T + t  ->  out row s0 * T + q.
  const size_t qbase = (size_t)s0 * T;
#pragma unroll 1
  for (uint32_t q0 = sgb * UNR; q0 < ntile; q0 += SGPB * UNR) {
    uint32_t bi[UNR];
    bool simple = true;
    uint32_t sl = q0 / T, t = q0 - (q0 / T) * T;  // walk (sample, table) in output order
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      bi[u] = 0u;
      if (q0 + u < ntile) {
        bi[u] = t * Sl + sl;
        simple = simple && s_len[bi[u]] <= 1u;
      }
      if (++t == T) {
        t = 0;
        ++sl;
      }
    }
    f4 acc[UNR][VEC];
#pragma unroll
    for (int u = 0; u < UNR; ++u)
#pragma unroll
      for (int v = 0; v < VEC; ++v) acc[u][v] = f4{0.f, 0.f, 0.f, 0.f};
    if (simple) {
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const uint32_t r = q0 + u < ntile ? s_row[bi[u]] : kNoRow;
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          const uint32_t d4 = lane + v * SG;
          acc[u][v] = load4_or_zero(W, r, D, d4, r != kNoRow && d4 < D4);
        }
      }
    } else {
      // Multi-hot bags: ids SG at a time (one coalesced load), KU rows in flight.
      constexpr int KU = 4;
      uint32_t msl = q0 / T, mt = q0 - (q0 / T) * T;
#pragma unroll 1
      for (int u = 0; u < UNR; ++u) {
        if (q0 + u >= ntile) break;
        const uint32_t i = mt * Sl + msl;
        if (++mt == T) {
          mt = 0;
          ++msl;
        }
        const uint32_t len = s_len[i], st = s_start[i];
        const uint32_t tt = i / Sl;
        const uint32_t roff = (uint32_t)row_off[tt];
        const int64_t nr = rows[tt];
        f4 a[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) a[v] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
        for (uint32_t kb = 0; kb < len; kb += SG) {
          uint32_t r = kNoRow;
          if (kb + lane < len) {
            if (rowmap) {
              r = rowmap[st + kb + lane];
            } else {
              const int64_t id = ids[st + kb + lane];
              if (id >= 0 && id < nr) r = roff + (uint32_t)id;
              else if (id != kAbsentId) bad |= EMB_FLAG_OUT_OF_RANGE;
            }
          }
          const uint32_t kend = (len - kb) < (uint32_t)SG ? (len - kb) : (uint32_t)SG;
#pragma unroll 1
          for (uint32_t kk = 0; kk < kend; kk += KU) {
            f4 x[KU][VEC];
#pragma unroll
            for (int k = 0; k < KU; ++k) {
              const uint32_t src = kk + k < (uint32_t)SG ? kk + k : (uint32_t)SG - 1u;
              uint32_t grow = (uint32_t)__shfl((int)r, (int)src, SG);
              if (kk + k >= kend) grow = kNoRow;
#pragma unroll
              for (int v = 0; v < VEC; ++v) {
                const uint32_t d4 = lane + v * SG;
                x[k][v] = load4_or_zero(W, grow, D, d4, grow != kNoRow && d4 < D4);
              }
            }
#pragma unroll
            for (int k = 0; k < KU; ++k)
#pragma unroll
              for (int v = 0; v < VEC; ++v) a[v] += x[k][v];
          }
        }
        const float c = (MEAN && len > 0u) ? 1.0f / (float)len : 1.0f;
        f4 rr[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) rr[v] = MEAN ? a[v] * c : a[v];
        out.template put<SG, VEC>(qbase + q0 + u, D, lane, rr);
      }
      continue;
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      if (q0 + u >= ntile) continue;
      out.template put<SG, VEC>(qbase + q0 + u, D, lane, acc[u]);
    }
  }
  return bad;
}

template <int SG, int VEC, bool MEAN, int UNR, class OUT>
__global__ __launch_bounds__(256) void k_bag_forward(
    const int64_t* __restrict__ offsets, const int64_t* __restrict__ ids,
    const float* __restrict__ W, const int64_t* __restrict__ row_off,
    const int64_t* __restrict__ rows, OUT out, uint32_t* __restrict__ flags,
    uint32_t B, uint32_t T, uint32_t D, uint32_t nnz, uint32_t S,
    const uint32_t* __restrict__ rowmap) {
  __shared__ BagTileLds lds;
  const uint32_t bad = bag_tile<SG, VEC, MEAN, UNR, OUT>(xcd_block(), offsets, ids, W, row_off,
                                                         rows, out, B, T, D, nnz, S, lds, rowmap);
  if (bad) atomicOr(flags, bad);
}

// Sorted positions per sub-group of the one-hot forward: kFwdChunk when the
// sub-group has that many lanes (one position in each of its first lanes),
// else the reduction's chunk.  Chunks of 8 measured faster than 32 (4 or 16
// slower than 8): more blocks keep more output rows in flight.
constexpr int kFwdChunk = 8;
template <int SG, int MPL>
constexpr int fwd_chunk() {
  return SG >= kFwdChunk ? kFwdChunk : SG * MPL;
}

// One-hot batches after the sort: every bag holds one id, so the output row of
// occurrence j is W[row_j] stored at out[grad_row(j)].  Walking the sorted
// occurrences, a Zipf-hot row is read once per chunk and then stored to each
// of its bags, and W is visited in ascending address order.  Sub-groups are
// those of the reduction kernel, chunks are fwd_chunk() positions.
//
// Whether the batch is one-hot is known only on the device (a flag set while
// the keys were built), so the same launch also holds the general pooled
// kernel: when the flag is set, block i pools sample tile i instead.
template <int SG, int VEC, int MPL, bool MEAN, int UNR, class OUT>
__global__ __launch_bounds__(256) void k_fwd_sorted(
    const uint32_t* __restrict__ keys, const uint32_t* __restrict__ perm,
    const uint32_t* __restrict__ gr, const float* __restrict__ W, OUT out,
    uint32_t n, uint32_t sentinel, uint32_t D, uint32_t nbags,
    const uint32_t* __restrict__ misc, const int64_t* __restrict__ offsets,
    const int64_t* __restrict__ ids, const int64_t* __restrict__ row_off,
    const int64_t* __restrict__ rows, uint32_t* __restrict__ flags, uint32_t B, uint32_t T,
    uint32_t S, const uint32_t* __restrict__ rowmap) {
  if (batch_not_one_hot(misc)) {
    __shared__ BagTileLds lds;
    const uint32_t bad = bag_tile<SG, VEC, MEAN, UNR, OUT>(xcd_block(), offsets, ids, W, row_off,
                                                           rows, out, B, T, D, n, S, lds, rowmap);
    if (bad) atomicOr(flags, bad);
    return;
  }
  constexpr int CH = fwd_chunk<SG, MPL>();
  constexpr int ML = CH < SG * MPL ? 1 : MPL;  // metadata entries per lane
  constexpr int LPR = CH < SG ? CH : SG;       // positions per metadata round
  constexpr int SGPB = 256 / SG;
  constexpr int UF = VEC > 1 ? 2 : (SG < 4 ? SG : 4);
  static_assert(LPR % UF == 0, "rows in flight must divide a round");
  const uint32_t lane = threadIdx.x % SG;
  // Chunks in launch order (no XCD remap): measured faster here, since the
  // row loads walk W in ascending order across the whole chip at once.
  const uint32_t c = blockIdx.x * SGPB + threadIdx.x / SG;
  const uint32_t k0 = c * CH;
  if (k0 >= n) return;
  const uint32_t D4 = D >> 2;
  uint32_t mkey[ML], mgr[ML];
#pragma unroll
  for (int i = 0; i < ML; ++i) {
    const uint32_t k = k0 + i * SG + lane;
    mkey[i] = kNoRow;
    mgr[i] = nbags;
    if (k < n && lane < (uint32_t)LPR) {
      mkey[i] = keys[k];
      const uint32_t v = perm[k];  // occurrence v is bag v: its output row
      mgr[i] = v < n ? one_hot_grad_row(v, B, T) : nbags;
    }
  }
  uint32_t prevkey = kNoRow;
  f4 prevrow[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) prevrow[v] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < ML; ++i) {
#pragma unroll 1
    for (int l0 = 0; l0 < LPR; l0 += UF) {
      uint32_t kk[UF], gg[UF];
#pragma unroll
      for (int u = 0; u < UF; ++u) {
        kk[u] = (uint32_t)__shfl((int)mkey[i], l0 + u, SG);
        gg[u] = (uint32_t)__shfl((int)mgr[i], l0 + u, SG);
      }
      f4 x[UF][VEC];
#pragma unroll
      for (int u = 0; u < UF; ++u) {
        const uint32_t pk = u == 0 ? prevkey : kk[u > 0 ? u - 1 : 0];
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          const uint32_t d4 = lane + v * SG;
          x[u][v] = load4_or_zero(W, kk[u], D, d4, kk[u] < sentinel && kk[u] != pk && d4 < D4);
        }
      }
#pragma unroll
      for (int u = 0; u < UF; ++u) {
        const uint32_t pk = u == 0 ? prevkey : kk[u > 0 ? u - 1 : 0];
        if (kk[u] < sentinel && kk[u] == pk) {
#pragma unroll
          for (int v = 0; v < VEC; ++v) x[u][v] = u == 0 ? prevrow[v] : x[u > 0 ? u - 1 : 0][v];
        }
        if (gg[u] < nbags) out.template put<SG, VEC>(gg[u], D, lane, x[u]);
      }
      prevkey = kk[UF - 1];
#pragma unroll
      for (int v = 0; v < VEC; ++v) prevrow[v] = x[UF - 1][v];
    }
  }
}

// Samples per tile of the pooled kernel: about kFwdTileBags bags of all
// tables, and about as many ids, so that long bags still give enough blocks.
int64_t tile_samples(int T, int64_t B, int64_t nnz) {
  const int64_t bags = B * (int64_t)T;
  const int64_t mean_len = bags > 0 ? (nnz + bags - 1) / bags : 1;
  int64_t S = kFwdTileBags / ((int64_t)T * (mean_len > 1 ? mean_len : 1));
  return S > 64 ? 64 : (S < 1 ? 1 : S);
}

template <int VEC>
constexpr int fwd_unroll() {
  return VEC == 1 ? 8 : (VEC == 2 ? 4 : 2);  // one-hot rows in flight per lane
}

template <int SG, int VEC, bool MEAN, class OUT>
hipError_t launch_t(const Handle& h, const int64_t* offsets, const int64_t* ids, int64_t B,
                    int64_t nnz, OUT out, const uint32_t* rowmap, hipStream_t s) {
  const int64_t S = tile_samples(h.T, B, nnz);
  const int64_t grid = (B + S - 1) / S;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((k_bag_forward<SG, VEC, MEAN, fwd_unroll<VEC>(), OUT>), dim3((unsigned)grid),
                     dim3(256), 0, s, offsets, ids, h.W, h.sv.row_off, h.sv.rows, out,
                     h.sv.flags, (uint32_t)B, (uint32_t)h.T, (uint32_t)h.D, (uint32_t)nnz,
                     (uint32_t)S, rowmap);
  return hipGetLastError();
}

template <bool MEAN, class OUT>
hipError_t dispatch(const Handle& h, const int64_t* offsets, const int64_t* ids, int64_t B,
                    int64_t nnz, OUT out, const uint32_t* rowmap, hipStream_t s) {
  const int sg = subgroup_lanes(h.D), vec = vec_per_lane(h.D);
  switch (sg) {
    case 1: return launch_t<1, 1, MEAN, OUT>(h, offsets, ids, B, nnz, out, rowmap, s);
    case 2: return launch_t<2, 1, MEAN, OUT>(h, offsets, ids, B, nnz, out, rowmap, s);
    case 4: return launch_t<4, 1, MEAN, OUT>(h, offsets, ids, B, nnz, out, rowmap, s);
    case 8: return launch_t<8, 1, MEAN, OUT>(h, offsets, ids, B, nnz, out, rowmap, s);
    case 16: return launch_t<16, 1, MEAN, OUT>(h, offsets, ids, B, nnz, out, rowmap, s);
    case 32: return launch_t<32, 1, MEAN, OUT>(h, offsets, ids, B, nnz, out, rowmap, s);
    default:
      switch (vec) {
        case 1: return launch_t<64, 1, MEAN, OUT>(h, offsets, ids, B, nnz, out, rowmap, s);
        case 2: return launch_t<64, 2, MEAN, OUT>(h, offsets, ids, B, nnz, out, rowmap, s);
        case 3: return launch_t<64, 3, MEAN, OUT>(h, offsets, ids, B, nnz, out, rowmap, s);
        default: return launch_t<64, 4, MEAN, OUT>(h, offsets, ids, B, nnz, out, rowmap, s);
      }
  }
}

}  // namespace

hipError_t launch_forward(const Handle& h, const int64_t* offsets, const int64_t* ids,
                          int64_t B, int64_t nnz, bool mean, float* out, hipStream_t s) {
  phase_mark(h, EMB_PHASE_FORWARD, false, s);
  const F32Rows o{out};
  hipError_t e = mean ? dispatch<true>(h, offsets, ids, B, nnz, o, nullptr, s)
                      : dispatch<false>(h, offsets, ids, B, nnz, o, nullptr, s);
  phase_mark(h, EMB_PHASE_FORWARD, true, s);
  return e;
}

hipError_t launch_forward_bags(const Handle& h, const int64_t* offsets, const int64_t* ids,
                               int64_t B, int64_t nnz, bool mean, float* out,
                               const uint32_t* rowmap, hipStream_t s) {
  const F32Rows o{out};
  return mean ? dispatch<true>(h, offsets, ids, B, nnz, o, rowmap, s)
              : dispatch<false>(h, offsets, ids, B, nnz, o, rowmap, s);
}

namespace {
template <int SG, int VEC, bool MEAN, class OUT>
hipError_t launch_sorted_t(const Handle& h, const Plan& p, const int64_t* offsets,
                           const int64_t* ids, const uint32_t* keys, const uint32_t* perm,
                           OUT out, char* ws, const uint32_t* rowmap, hipStream_t s) {
  constexpr int MPL = chunk_rounds<SG>();
  constexpr int SGPB = 256 / SG;
  constexpr int CH = fwd_chunk<SG, MPL>();
  const int64_t chunks = (p.nnz + CH - 1) / CH;
  const int64_t S = tile_samples(h.T, p.B, p.nnz);
  const int64_t tiles = (p.B + S - 1) / S;
  int64_t grid = (chunks + SGPB - 1) / SGPB;
  grid = grid > tiles ? grid : tiles;  // enough blocks for either path
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((k_fwd_sorted<SG, VEC, MPL, MEAN, fwd_unroll<VEC>(), OUT>),
                     dim3((unsigned)grid),
                     dim3(256), 0, s, keys, perm,
                     reinterpret_cast<const uint32_t*>(ws + p.sgr), h.W, out, (uint32_t)p.nnz,
                     (uint32_t)h.total_rows, (uint32_t)h.D, (uint32_t)(p.B * h.T),
                     reinterpret_cast<const uint32_t*>(ws + p.misc), offsets, ids, h.sv.row_off,
                     h.sv.rows, h.sv.flags, (uint32_t)p.B, (uint32_t)h.T, (uint32_t)S, rowmap);
  return hipGetLastError();
}

template <bool MEAN, class OUT>
hipError_t dispatch_sorted(const Handle& h, const Plan& p, const int64_t* offsets,
                           const int64_t* ids, const uint32_t* keys, const uint32_t* perm,
                           OUT out, char* ws, const uint32_t* rowmap, hipStream_t s) {
  const int sg = subgroup_lanes(h.D), vec = vec_per_lane(h.D);
#define EMB_SORTED(SG_, VEC_) \
  launch_sorted_t<SG_, VEC_, MEAN, OUT>(h, p, offsets, ids, keys, perm, out, ws, rowmap, s)
  switch (sg) {
    case 1: return EMB_SORTED(1, 1);
    case 2: return EMB_SORTED(2, 1);
    case 4: return EMB_SORTED(4, 1);
    case 8: return EMB_SORTED(8, 1);
    case 16: return EMB_SORTED(16, 1);
    case 32: return EMB_SORTED(32, 1);
    default:
      switch (vec) {
        case 1: return EMB_SORTED(64, 1);
        case 2: return EMB_SORTED(64, 2);
        case 3: return EMB_SORTED(64, 3);
        default: return EMB_SORTED(64, 4);
      }
  }
#undef EMB_SORTED
}
}  // namespace

hipError_t launch_forward_sorted(const Handle& h, const Plan& p, const int64_t* offsets,
                                 const int64_t* ids, bool mean, const uint32_t* keys,
                                 const uint32_t* perm, float* out, char* ws,
                                 const uint32_t* rowmap, hipStream_t s) {
  const F32Rows o{out};
  return mean ? dispatch_sorted<true>(h, p, offsets, ids, keys, perm, o, ws, rowmap, s)
              : dispatch_sorted<false>(h, p, offsets, ids, keys, perm, o, ws, rowmap, s);
}

hipError_t launch_forward_prepared_int8(const Handle& h, const Plan& p, const int64_t* offsets,
                                        const int64_t* ids, bool mean, bool maybe_one_hot,
                                        const uint32_t* keys, const uint32_t* perm,
                                        int8_t* codes, float* scales, char* ws,
                                        const uint32_t* rowmap, hipStream_t s) {
  const I8Rows o{reinterpret_cast<uint32_t*>(codes), scales};
  if (maybe_one_hot)
    return mean ? dispatch_sorted<true>(h, p, offsets, ids, keys, perm, o, ws, rowmap, s)
                : dispatch_sorted<false>(h, p, offsets, ids, keys, perm, o, ws, rowmap, s);
  return mean ? dispatch<true>(h, offsets, ids, p.B, p.nnz, o, rowmap, s)
              : dispatch<false>(h, offsets, ids, p.B, p.nnz, o, rowmap, s);
}

}  // namespace embtab
