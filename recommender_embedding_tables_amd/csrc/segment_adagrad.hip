// Segmented gradient reduction fused with element-wise Adagrad, for gfx950.
//
// After the stable sort, the occurrences of one row are contiguous.  For each
// touched row u:  g_u = sum_k c_b(k) * grad_out[s(k), t(k), :]  and
//   G_u += g_u * g_u;  W_u -= lr * g_u / (sqrt(G_u) + eps)   (per element),
// the sparse, memory-saving Adagrad of the "Merlin HugeCTR interview" page
// (section three, technique (1)) with the Adagrad optimizer of the synthetic
// benchmarks of "NVIDIA Merlin Distributed Embeddings" (section
// "Performance").  The form of the step is the textbook one (Duchi, Hazan and
// Singer 2011).
//
// Schedule.  The sorted occurrences are cut into fixed chunks of CH positions,
// one chunk per sub-group of SG lanes (a row is D/4 float4 columns spread over
// the lanes), so a Zipf-hot row with tens of thousands of occurrences is
// spread over many sub-groups instead of serialising one.  A sub-group loads
// the chunk's metadata once (sorted key, grad row, mean scale: one element
// per lane), then walks the positions UF at a time: it issues the UF
// gradient-row loads and, for every segment that ends inside the group and
// lies wholly in the chunk, the W and G rows, before accumulating in position
// order; a finished segment is updated in registers and written back once.
// A segment that crosses a chunk boundary leaves fp32 part sums in LDS.  If
// it lies wholly in the block, the chunk where it ends adds them and applies
// the step after the block barrier.  If it crosses a block edge ("span"), the
// block adds its chunks' parts and leaves one part per block in memory (the
// "tail" part in the block where it starts, a "head" part in each later
// block it covers), then counts itself on the span's counter; the last of the
// span's blocks to arrive adds the parts in block order and applies the step.
// The prepare has recorded, for every block edge that a run crosses, which
// run it is, so each block knows how many blocks share its spans.  Every sum
// has a fixed order, so the result is deterministic and no float atomics are
// used.
//
// The parts are the only data blocks exchange.  They are written through to
// memory and read past the L2 (agent-scope atomic stores and loads: each XCD
// has its own L2), and the writer waits for its stores to complete before it
// counts itself, so the block that finishes a span sees every part without a
// write-back of whole caches.  (A release/acquire fence per part, which
// writes back the XCD's L2, was measured to double the kernel's time.)
//
// Finishing such a segment inside this kernel, by the sub-group of the chunk
// where it starts reading on into the next one, was measured slower: the two
// sub-groups of a wave run in lockstep, so a wave whose one sub-group does
// extra rows holds the other idle for that time.
#include "embtab_internal.hpp"

#ifndef EMBTAB_SEG_UF
#define EMBTAB_SEG_UF 4
#endif

namespace embtab {

namespace {

// Sorted positions walked per group by one sub-group (rows in flight).
constexpr int kSegUF = EMBTAB_SEG_UF;

// The accumulator G is read and written once per touched row per step and
// read by nothing else, so its rows use non-temporal loads and stores: they
// would only evict the W rows and gradient metadata the step reuses from L2
// and MALL.  (Measured on 26 tables: 0.623 -> 0.600 ms per step; the same for
// W loads or stores, or for the forward's row loads, did not pay.)
__device__ inline void store4_nt(float* __restrict__ base, size_t row, uint32_t D, uint32_t d4,
                                 const f4 x) {
  __builtin_nontemporal_store(x, reinterpret_cast<f4*>(base + row * D + 4u * d4));
}

// A part of a span, stored and loaded coherently across XCDs (see above).
__device__ inline void store4_coherent(float* p, const f4 x) {
  __hip_atomic_store(p + 0, x[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(p + 1, x[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(p + 2, x[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(p + 3, x[3], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline f4 load4_coherent(const float* p) {
  float* q = const_cast<float*>(p);
  return f4{__hip_atomic_load(q + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
            __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
            __hip_atomic_load(q + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
            __hip_atomic_load(q + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)};
}

// One element-wise Adagrad step: G' = G + g^2, w' = w - lr * g / (sqrt(G') + eps).
// The square root and the reciprocal are the hardware instructions (each
// within 1 ulp), not the correctly rounded expansions: a third fewer
// instructions in the reduction kernel (reduction 112 -> 106 us on the hashed
// workload, 183 -> 179 us on the multi-hot one), and the step stays far inside
// the 1e-5 relative tolerance the results are held to.
__device__ inline void adagrad_step(f4& w, f4& g2, const f4 g, float lr, float eps) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float G1 = __builtin_fmaf(g[i], g[i], g2[i]);
    w[i] = w[i] - (lr * g[i]) * __builtin_amdgcn_rcpf(__builtin_amdgcn_sqrtf(G1) + eps);
    g2[i] = G1;
  }
}

// Adagrad Decay: the accumulator's discount for a row last updated in period
// `last` (DeepRec page, section "model quality", Adagrad Decay Optimizer:
// one discount per period).  rho^(period - last) as 2^(elapsed * log2 rho);
// none for a fresh row (a new key's initial accumulator).
__device__ inline float decay_factor(uint32_t last, uint32_t period, float log2_rho) {
  return (last != kFreshPeriod && period > last) ? exp2f((float)(period - last) * log2_rho)
                                                 : 1.0f;
}
// Whether an update in `period` moves the row's period stamp (to `period`).
__device__ inline bool period_advances(uint32_t last, uint32_t period) {
  return last == kFreshPeriod || period > last;
}

// Where the gradient rows come from: fp32 rows of grad_out [bags, D], or the
// int8 exchange payload as a table-wise split receives it (codes [bags, D]
// and one scale per row; a value is code * scale in fp32, the dequantized
// payload exactly).  Non-temporal loads for rows read once, cached loads for
// rows read once per occurrence of their bag (REUSE).
struct F32Grad {
  const float* g;
  template <bool REUSE>
  __device__ __forceinline__ f4 load(uint32_t row, uint32_t D, uint32_t d4, bool ok) const {
    return REUSE ? load4_or_zero(g, row, D, d4, ok) : load4_nt_or_zero(g, row, D, d4, ok);
  }
};
struct I8Grad {
  const uint32_t* codes;  // four codes per word
  const float* scales;
  template <bool REUSE>
  __device__ __forceinline__ f4 load(uint32_t row, uint32_t D, uint32_t d4, bool ok) const {
    const size_t off = ok ? (size_t)row * (D >> 2) + d4 : 0u;
    const uint32_t w = REUSE ? codes[off] : __builtin_nontemporal_load(codes + off);
    const float sc = scales[ok ? row : 0u];
    const f4 x = {(float)(int8_t)(w & 0xFFu) * sc, (float)(int8_t)((w >> 8) & 0xFFu) * sc,
                  (float)(int8_t)((w >> 16) & 0xFFu) * sc, (float)(int8_t)(w >> 24) * sc};
    return ok ? x : f4{0.f, 0.f, 0.f, 0.f};
  }
};

// A run that crosses chunk boundaries but neither enters the block from the
// previous one nor leaves it into the next is finished inside the block: the
// chunk where it ends keeps its own part sum and the row's W and G in
// registers, the earlier chunks leave their parts in LDS, and after the block
// barrier it adds them in chunk order and applies the step.  Only runs that
// cross a block boundary leave parts in memory.
template <int VEC>
struct BlockRun {
  uint32_t row = kNoRow;  // kNoRow: this chunk finishes no run of the block
  uint32_t last = 0u;     // Adagrad Decay: the row's period before this call
  f4 acc[VEC], w[VEC], g2[VEC];
};

// Walks chunk c (one sub-group).  key_bb / key_ba: the keys just before and
// just after the block.  A run continuing past the chunk and lying wholly in
// the block leaves its part in part_lds and its row in *slot_key.
template <int SG, int VEC, bool MEAN, int MPL, int UF, bool DECAY, bool REUSE, class GRAD>
__device__ __forceinline__ void seg_chunk(
    const uint32_t* __restrict__ keys, const uint32_t* __restrict__ sgr,
    const float* __restrict__ sscale, GRAD grad, float* __restrict__ W,
    float* __restrict__ G, uint32_t n, uint32_t sentinel, int32_t D, float lr, float eps,
    uint32_t nbags, uint32_t* __restrict__ stamps, float log2_rho, uint32_t period, uint32_t c,
    uint32_t key_bb, uint32_t key_ba, f4* part_lds,
    uint32_t* slot_key, f4* in_lds, uint32_t* in_key, f4* out_lds, uint32_t* out_key,
    BlockRun<VEC>& fin, const uint32_t* __restrict__ perm, bool one_hot, uint32_t B,
    uint32_t T) {
  constexpr int CH = SG * MPL;
  const int lane = threadIdx.x % SG;
  const uint32_t k0 = c * CH;
  if (k0 >= n) return;
  const uint32_t k1 = (k0 + CH < n) ? k0 + CH : n;
  const int D4 = D >> 2;
  const uint32_t key_prev = k0 > 0 ? keys[k0 - 1] : kNoRow;
  const uint32_t key_next = k1 < n ? keys[k1] : kNoRow;

  uint32_t mkey[MPL], mgr[MPL];
  float msc[MPL];
#pragma unroll
  for (int i = 0; i < MPL; ++i) {
    const uint32_t k = k0 + i * SG + lane;
    mkey[i] = kNoRow;
    mgr[i] = 0u;
    msc[i] = 1.0f;
    if (k < k1) mkey[i] = keys[k];
  }
#pragma unroll
  for (int i = 0; i < MPL; ++i) {
    const uint32_t k = k0 + i * SG + lane;
    if (k < k1) {
      // grad row and scale were gathered into sorted order by the last sort
      // pass (one-hot batches: computed from the occurrence index).  Positions
      // not written by any bag (offsets that do not tile [0, nnz)) may hold
      // stale values: such an occurrence is dropped.
      uint32_t g;
      if (one_hot) {
        const uint32_t v = perm[k];
        g = v < n ? one_hot_grad_row(v, B, T) : nbags;
      } else {
        g = sgr[k];
      }
      if (mkey[i] < sentinel) {
        if (g < nbags) {
          mgr[i] = g;
          if (MEAN && !one_hot) msc[i] = sscale[k];
        } else {
          mkey[i] = sentinel;
        }
      }
    }
  }

  f4 acc[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) acc[v] = f4{0.f, 0.f, 0.f, 0.f};
  bool first_seg = true;
  const uint32_t last = k1 - k0 - 1;  // last position of the chunk

#pragma unroll
  for (int i = 0; i < MPL; ++i) {
    for (int l0 = 0; l0 < SG; l0 += UF) {
      uint32_t kk[UF + 1], gg[UF];
      float cc[UF];
#pragma unroll
      for (int u = 0; u < UF; ++u) {
        kk[u] = (uint32_t)__shfl((int)mkey[i], l0 + u, SG);
        gg[u] = (uint32_t)__shfl((int)mgr[i], l0 + u, SG);
        cc[u] = MEAN ? __shfl(msc[i], l0 + u, SG) : 1.0f;
      }
      {
        // key of the position after the group
        uint32_t nx;
        if (l0 + UF < SG) nx = (uint32_t)__shfl((int)mkey[i], l0 + UF, SG);
        else if (i + 1 < MPL) nx = (uint32_t)__shfl((int)mkey[(i + 1) < MPL ? i + 1 : i], 0, SG);
        else nx = key_next;
        kk[UF] = nx;
      }
      bool vld[UF], endf[UF], startb[UF], cont[UF];
      bool fs = first_seg;
#pragma unroll
      for (int u = 0; u < UF; ++u) {
        const uint32_t p = (uint32_t)(i * SG + l0 + u);
        vld[u] = (p <= last) && kk[u] < sentinel;
        const uint32_t nxt = (p == last) ? key_next : kk[u + 1];
        endf[u] = vld[u] && nxt != kk[u];
        cont[u] = vld[u] && (p == last) && nxt == kk[u];
        startb[u] = fs && kk[u] == key_prev;
        if (endf[u]) fs = false;
      }
      if (!vld[0]) break;  // the rest of the chunk holds no valid keys
      f4 g[UF][VEC], wv[UF][VEC], gv[UF][VEC];
      uint32_t last[UF];  // Adagrad Decay: period of the row finished at u
#pragma unroll
      for (int u = 0; u < UF; ++u) {
        last[u] = 0u;
        // the row is updated by this sub-group: its run starts here, or it
        // started in an earlier chunk of this block
        const bool mine = endf[u] && (!startb[u] || kk[u] != key_bb);
        if (DECAY && mine) last[u] = stamps[kk[u]];
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          const uint32_t d4 = (uint32_t)(lane + v * SG);
          const bool own = mine && d4 < (uint32_t)D4;
          g[u][v] = grad.template load<REUSE>(gg[u], (uint32_t)D, d4,
                                              vld[u] && d4 < (uint32_t)D4);
          wv[u][v] = load4_or_zero(W, kk[u], (uint32_t)D, d4, own);
          gv[u][v] = load4_nt_or_zero(G, kk[u], (uint32_t)D, d4, own);
        }
      }
#pragma unroll
      for (int u = 0; u < UF; ++u) {
        if (!vld[u]) continue;
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[v] += MEAN ? g[u][v] * cc[u] : g[u][v];
        if (endf[u]) {
          if (!startb[u]) {
            float df = 1.0f;
            if (DECAY) {
              df = decay_factor(last[u], period, log2_rho);
              if (lane == 0 && period_advances(last[u], period)) stamps[kk[u]] = period;
            }
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
              const int d4 = lane + v * SG;
              if (d4 < D4) {
                if (DECAY) gv[u][v] *= df;
                adagrad_step(wv[u][v], gv[u][v], acc[v], lr, eps);
                *reinterpret_cast<f4*>(W + (size_t)kk[u] * D + 4 * d4) = wv[u][v];
                store4_nt(G, kk[u], (uint32_t)D, (uint32_t)d4, gv[u][v]);
              }
            }
          } else if (kk[u] != key_bb) {  // finished after the block barrier
            fin.row = kk[u];
            fin.last = last[u];
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
              fin.acc[v] = acc[v];
              fin.w[v] = wv[u][v];
              fin.g2[v] = gv[u][v];
            }
          } else {  // the run entered the block from the previous one
#pragma unroll
            for (int v = 0; v < VEC; ++v) in_lds[lane + v * SG] = acc[v];
            *in_key = kk[u];
          }
#pragma unroll
          for (int v = 0; v < VEC; ++v) acc[v] = f4{0.f, 0.f, 0.f, 0.f};
        } else if (cont[u] && kk[u] != key_bb && kk[u] != key_ba) {
#pragma unroll
          for (int v = 0; v < VEC; ++v) part_lds[lane + v * SG] = acc[v];
          *slot_key = kk[u];
        } else if (cont[u]) {  // the run crosses an edge of the block
          f4* dst = kk[u] == key_bb ? in_lds : out_lds;
#pragma unroll
          for (int v = 0; v < VEC; ++v) dst[lane + v * SG] = acc[v];
          *(kk[u] == key_bb ? in_key : out_key) = kk[u];
        }
      }
      first_seg = fs;
    }
  }
}


// One block's arrival at span [bs, be] of `row` (called by the sub-group
// that wrote the block's part, after its stores).  The counter of the span's
// first block counts arrivals; the last of the be - bs + 1 blocks resets it
// and finishes the row: tail part of bs, then the head parts of bs+1 .. be,
// added in block order, then the Adagrad step.
template <int SG, int VEC, bool DECAY>
__device__ __forceinline__ void span_arrive(
    uint32_t row, uint32_t bs, uint32_t be, const float* __restrict__ part_head,
    const float* __restrict__ part_tail, uint32_t* __restrict__ span_cnt, float* __restrict__ W,
    float* __restrict__ G, int32_t D, float lr, float eps, uint32_t* __restrict__ stamps,
    float log2_rho, uint32_t period) {
  const int lane = threadIdx.x % SG;
  const int D4 = D >> 2;
  // this wave's part stores have completed (they were written through)
  __builtin_amdgcn_s_waitcnt(0);
  uint32_t seen = 0u;
  if (lane == 0)
    seen = __hip_atomic_fetch_add(&span_cnt[bs], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  seen = (uint32_t)__shfl((int)seen, 0, SG);
  if (seen != be - bs) return;  // another block of the span arrives later
  if (lane == 0) __hip_atomic_store(&span_cnt[bs], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  uint32_t last = 0u;
  if (DECAY) last = stamps[row];
  f4 w[VEC], g2[VEC], tot[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
    const uint32_t d4 = (uint32_t)(lane + v * SG);
    const bool ok = d4 < (uint32_t)D4;
    w[v] = load4_or_zero(W, row, (uint32_t)D, d4, ok);
    g2[v] = load4_nt_or_zero(G, row, (uint32_t)D, d4, ok);
    tot[v] = ok ? load4_coherent(part_tail + (size_t)bs * D + 4 * d4) : f4{0.f, 0.f, 0.f, 0.f};
  }
  // head parts four blocks at a time, added in block order
  for (uint32_t c = bs + 1; c <= be; c += 4) {
    f4 x[4][VEC];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        const uint32_t d4 = (uint32_t)(lane + v * SG);
        x[q][v] = (c + q <= be && d4 < (uint32_t)D4)
                      ? load4_coherent(part_head + (size_t)(c + q) * D + 4 * d4)
                      : f4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int v = 0; v < VEC; ++v)
        if (c + q <= be) tot[v] += x[q][v];
  }
  float df = 1.0f;
  if (DECAY) {
    df = decay_factor(last, period, log2_rho);
    if (lane == 0 && period_advances(last, period)) stamps[row] = period;
  }
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
    const int d4 = lane + v * SG;
    if (d4 >= D4) continue;
    if (DECAY) g2[v] *= df;
    adagrad_step(w[v], g2[v], tot[v], lr, eps);
    *reinterpret_cast<f4*>(W + (size_t)row * D + 4 * d4) = w[v];
    store4_nt(G, row, (uint32_t)D, (uint32_t)d4, g2[v]);
  }
}

template <int SG, int VEC, bool MEAN, int MPL, int UF, bool DECAY, bool REUSE, class GRAD>
__global__ __launch_bounds__(256) void k_seg_adagrad(
    const uint32_t* __restrict__ keys, const uint32_t* __restrict__ sgr,
    const float* __restrict__ sscale, GRAD grad, float* __restrict__ W,
    float* __restrict__ G, uint32_t n, uint32_t sentinel, int32_t D, float lr, float eps,
    float* __restrict__ part_head, float* __restrict__ part_tail,
    const uint32_t* __restrict__ span_u, const uint32_t* __restrict__ seg_off,
    uint32_t* __restrict__ span_cnt, uint32_t nbags, uint32_t* __restrict__ stamps,
    float log2_rho, uint32_t period, const uint32_t* __restrict__ perm,
    const uint32_t* __restrict__ misc, uint32_t B, uint32_t T) {
  constexpr int CH = SG * MPL;
  constexpr int SGPB = 256 / SG;
  constexpr uint32_t BP = SGPB * CH;  // sorted positions per block
  __shared__ f4 s_part[SGPB][SG * VEC];
  __shared__ f4 s_in[SGPB][SG * VEC];
  __shared__ f4 s_out[SGPB][SG * VEC];
  __shared__ uint32_t s_key[SGPB], s_in_key[SGPB], s_out_key[SGPB];
  const int lane = threadIdx.x % SG;
  const int sgb = threadIdx.x / SG;
  const uint32_t blk = blockIdx.x;
  const uint32_t c = blk * SGPB + sgb;
  const uint64_t b0 = (uint64_t)blk * BP, b1 = b0 + (uint64_t)BP;
  const uint32_t key_bb = b0 > 0 ? keys[b0 - 1] : kNoRow;
  const uint32_t key_ba = b1 < n ? keys[b1] : kNoRow;
  // The runs crossing this block's edges (unique indices, kNoRow for none),
  // recorded by the prepare; loaded now, used after the block's walk.
  const uint32_t sp_in = b0 > 0 ? span_u[blk] : kNoRow;
  const uint32_t sp_out = b1 < n ? span_u[blk + 1] : kNoRow;
  BlockRun<VEC> fin;
  uint32_t slot_key = kNoRow, in_key = kNoRow, out_key = kNoRow;
  seg_chunk<SG, VEC, MEAN, MPL, UF, DECAY, REUSE, GRAD>(
      keys, sgr, sscale, grad, W, G, n, sentinel, D, lr, eps, nbags, stamps, log2_rho, period, c,
      key_bb, key_ba, s_part[sgb], &slot_key, s_in[sgb], &in_key, s_out[sgb], &out_key, fin, perm,
      !batch_not_one_hot(misc), B, T);
  if (lane == 0) {
    s_key[sgb] = slot_key;
    s_in_key[sgb] = in_key;
    s_out_key[sgb] = out_key;
  }
  __syncthreads();
  const int D4 = D >> 2;
  // Runs crossing the block's edges: the block adds its chunks' parts in chunk
  // order and leaves one part per run, indexed by block: part_head[blk] for
  // the run that entered from the previous block (the whole block's sum when
  // the run covers the block), part_tail[blk] for a run that starts here and
  // continues into the next block.  Then it counts itself on the counter of
  // the span's first block; the last of the span's blocks finishes the row.
  if (sgb == 0 && key_bb < sentinel && s_in_key[0] == key_bb && sp_in != kNoRow) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      const int d4 = lane + v * SG;
      if (d4 >= D4) continue;
      f4 tot = s_in[0][lane + v * SG];
      for (int i = 1; i < SGPB && s_in_key[i] == key_bb; ++i) tot += s_in[i][lane + v * SG];
      store4_coherent(part_head + (size_t)blk * D + 4 * d4, tot);
    }
    const uint32_t st = seg_off[sp_in], en = seg_off[sp_in + 1];
    span_arrive<SG, VEC, DECAY>(key_bb, st / BP, (en - 1) / BP, part_head, part_tail, span_cnt, W,
                                G, D, lr, eps, stamps, log2_rho, period);
  }
  if (sgb == SGPB - 1 && key_ba < sentinel && key_ba != key_bb &&
      s_out_key[SGPB - 1] == key_ba && sp_out != kNoRow) {
    int j = SGPB - 1;
    while (j > 0 && s_out_key[j - 1] == key_ba) --j;
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      const int d4 = lane + v * SG;
      if (d4 >= D4) continue;
      f4 tot = s_out[j][lane + v * SG];
      for (int i = j + 1; i < SGPB; ++i) tot += s_out[i][lane + v * SG];
      store4_coherent(part_tail + (size_t)blk * D + 4 * d4, tot);
    }
    const uint32_t en = seg_off[sp_out + 1];
    span_arrive<SG, VEC, DECAY>(key_ba, blk, (en - 1) / BP, part_head, part_tail, span_cnt, W, G,
                                D, lr, eps, stamps, log2_rho, period);
  }
  if (fin.row == kNoRow) return;
  // chunks c0 .. c-1 of this block hold the run's earlier parts
  int i0 = sgb;
  while (i0 > 0 && s_key[i0 - 1] == fin.row) --i0;
  const float df = DECAY ? decay_factor(fin.last, period, log2_rho) : 1.0f;
  if (DECAY && lane == 0 && period_advances(fin.last, period)) stamps[fin.row] = period;
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
    const int d4 = lane + v * SG;
    if (d4 >= D4) continue;
    f4 tot = s_part[i0][lane + v * SG];
    for (int i = i0 + 1; i < sgb; ++i) tot += s_part[i][lane + v * SG];
    tot += fin.acc[v];
    f4 g2 = fin.g2[v];
    if (DECAY) g2 *= df;
    adagrad_step(fin.w[v], g2, tot, lr, eps);
    *reinterpret_cast<f4*>(W + (size_t)fin.row * D + 4 * d4) = fin.w[v];
    store4_nt(G, fin.row, (uint32_t)D, (uint32_t)d4, g2);
  }
}

template <int SG, int VEC, bool MEAN, bool DECAY, bool REUSE, class GRAD>
hipError_t launch_t(const Handle& h, const Plan& p, const uint32_t* keys, const uint32_t* perm,
                    GRAD grad_out, float lr, float eps, char* ws, hipStream_t s,
                    const DecayArgs& dec) {
  constexpr int MPL = chunk_rounds<SG>();
  constexpr int UF = VEC > 1 ? 2 : (SG < kSegUF ? SG : kSegUF);
  constexpr int SGPB = 256 / SG;
  static_assert(SG * MPL >= kChunkMin, "chunk");
  const uint32_t n = (uint32_t)p.nnz;
  if (n == 0) return hipSuccess;
  const int64_t chunks = (p.nnz + SG * MPL - 1) / (SG * MPL);
  const int64_t grid = (chunks + SGPB - 1) / SGPB;
  uint32_t* gr = reinterpret_cast<uint32_t*>(ws + p.sgr);
  float* scale = reinterpret_cast<float*>(ws + p.sscale);
  float* ph = reinterpret_cast<float*>(ws + p.part_head);
  float* pt = reinterpret_cast<float*>(ws + p.part_tail);
  const uint32_t* span_u = reinterpret_cast<const uint32_t*>(ws + p.span_u);
  const uint32_t* seg_off = reinterpret_cast<const uint32_t*>(ws + p.seg_off);
  uint32_t* span_cnt = reinterpret_cast<uint32_t*>(ws + p.span_cnt);
  const uint32_t nbags = (uint32_t)(p.B * h.T);
  phase_mark(h, EMB_PHASE_REDUCE, false, s);
  hipLaunchKernelGGL((k_seg_adagrad<SG, VEC, MEAN, MPL, UF, DECAY, REUSE, GRAD>),
                     dim3((unsigned)grid),
                     dim3(256), 0, s, keys, gr, scale, grad_out, h.W, h.G, n,
                     (uint32_t)h.total_rows, h.D, lr, eps, ph, pt, span_u, seg_off, span_cnt,
                     nbags, dec.stamps, dec.log2_rho, dec.period, perm,
                     reinterpret_cast<const uint32_t*>(ws + p.misc), (uint32_t)p.B,
                     (uint32_t)h.T);
  phase_mark(h, EMB_PHASE_REDUCE, true, s);
  return hipGetLastError();
}

template <bool MEAN, bool DECAY, bool REUSE, class GRAD>
hipError_t dispatch(const Handle& h, const Plan& p, const uint32_t* keys, const uint32_t* perm,
                    GRAD grad_out, float lr, float eps, char* ws, hipStream_t s,
                    const DecayArgs& dec) {
  const int sg = subgroup_lanes(h.D), vec = vec_per_lane(h.D);
#define EMBTAB_SEG_LAUNCH(SG_, VEC_) \
  launch_t<SG_, VEC_, MEAN, DECAY, REUSE, GRAD>(h, p, keys, perm, grad_out, lr, eps, ws, s, dec)
  switch (sg) {
    case 1: return EMBTAB_SEG_LAUNCH(1, 1);
    case 2: return EMBTAB_SEG_LAUNCH(2, 1);
    case 4: return EMBTAB_SEG_LAUNCH(4, 1);
    case 8: return EMBTAB_SEG_LAUNCH(8, 1);
    case 16: return EMBTAB_SEG_LAUNCH(16, 1);
    case 32: return EMBTAB_SEG_LAUNCH(32, 1);
    default:
      switch (vec) {
        case 1: return EMBTAB_SEG_LAUNCH(64, 1);
        case 2: return EMBTAB_SEG_LAUNCH(64, 2);
        case 3: return EMBTAB_SEG_LAUNCH(64, 3);
        default: return EMBTAB_SEG_LAUNCH(64, 4);
      }
  }
#undef EMBTAB_SEG_LAUNCH
}

}  // namespace

hipError_t launch_segment_adagrad(const Handle& h, const Plan& p, const uint32_t* keys,
                                  const uint32_t* perm, bool mean, const float* grad_out,
                                  float lr, float eps, char* ws, hipStream_t s,
                                  const DecayArgs& dec) {
  if (!grad_out) return hipErrorInvalidValue;
  const F32Grad g{grad_out};
  // Whether a bag's gradient row is read by more than one occurrence: a cache
  // policy only (both forms give the same result).  nnz == B * T means one id
  // per bag as a rule (the kernel checks one-hot batches exactly where it
  // matters); mean pooling is taken as multi-hot.
  const bool reuse = mean || p.nnz != p.B * (int64_t)h.T;
  if (dec.stamps) {
    if (mean) return dispatch<true, true, true>(h, p, keys, perm, g, lr, eps, ws, s, dec);
    return reuse ? dispatch<false, true, true>(h, p, keys, perm, g, lr, eps, ws, s, dec)
                 : dispatch<false, true, false>(h, p, keys, perm, g, lr, eps, ws, s, dec);
  }
  if (mean) return dispatch<true, false, true>(h, p, keys, perm, g, lr, eps, ws, s, dec);
  return reuse ? dispatch<false, false, true>(h, p, keys, perm, g, lr, eps, ws, s, dec)
               : dispatch<false, false, false>(h, p, keys, perm, g, lr, eps, ws, s, dec);
}

hipError_t launch_segment_adagrad_int8(const Handle& h, const Plan& p, const uint32_t* keys,
                                       const uint32_t* perm, bool mean, const int8_t* codes,
                                       const float* scales, float lr, float eps, char* ws,
                                       hipStream_t s) {
  if (!codes || !scales) return hipErrorInvalidValue;
  const I8Grad g{reinterpret_cast<const uint32_t*>(codes), scales};
  const DecayArgs dec;
  const bool reuse = mean || p.nnz != p.B * (int64_t)h.T;
  if (mean) return dispatch<true, false, true>(h, p, keys, perm, g, lr, eps, ws, s, dec);
  return reuse ? dispatch<false, false, true>(h, p, keys, perm, g, lr, eps, ws, s, dec)
               : dispatch<false, false, false>(h, p, keys, perm, g, lr, eps, ws, s, dec);
}

}  // namespace embtab
