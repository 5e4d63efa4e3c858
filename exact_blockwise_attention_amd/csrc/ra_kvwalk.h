// ra_kvwalk.h — the walk of a query tile over the ring's KV blocks, shared by
// the forward and the dQ kernels (bf16, 8 waves, 256 query rows per
// workgroup).
//
// A workgroup owns rows a0 .. a0+255 of rank i's query block. It visits the
// KV blocks in ring order j = (i - k) mod P ("Ring Attention: Sequence
// Parallelism for Long Context", section "Ring Attention: Compute While You
// Communicate") and, in each block, the 64-key tiles that some row of the
// workgroup can see under the causal / striped mask ("Ring Attention 論文分析"
// (blog), section "Causal Masking の処理": later blocks skipped, the diagonal
// masked); a single-step launch visits one given block only. KV tiles are
// double-buffered in LDS, the next one travelling through registers while the
// current one is computed.
#ifndef RA_KVWALK_H_
#define RA_KVWALK_H_

#include "ra_internal.h"
#include "ra_lds.h"
#include "ra_schedule.h"

namespace ra {

constexpr int kQWaves = 8;
constexpr int kQThreads = 64 * kQWaves;
constexpr int kQTm = 32 * kQWaves;  // query rows per workgroup
constexpr int kKvTn = 64;           // keys per KV tile
constexpr int kBandAll = 1 << 30;

// LDS: two stages of (K tile, V tile), each [64][D] padded.
template <int D>
struct KvLds {
  static constexpr int RS = PadRow<D>::RS;
  static constexpr int TILE = kKvTn * RS;
  static constexpr int STAGE = 2 * TILE;
  static constexpr int BYTES = 2 * STAGE * 2;
};

// Work order: the heaviest query tiles are dispatched first. Contiguous
// causal work grows with the rank, striped and non-causal work with the row.
__device__ __forceinline__ void query_tile_of(int32_t causal, int32_t layout, int32_t n_ranks, int64_t ord,
                                              int32_t tiles, int32_t* rank_idx, int32_t* tile) {
  if (causal && layout == kContiguous) {
    *rank_idx = n_ranks - 1 - (int32_t)(ord / tiles);
    *tile = tiles - 1 - (int32_t)(ord % tiles);
  } else {
    *tile = tiles - 1 - (int32_t)(ord / n_ranks);
    *rank_idx = n_ranks - 1 - (int32_t)(ord % n_ranks);
  }
}

// The (block, tile) pairs a query tile visits, in ring order.
struct KvIter {
  int32_t kstep, nsteps, j, t, ntile, band;
  int32_t i, P, layout, causal, a_hi, Bb, single_block;
  // moves to the next block with a visible tile; false when the ring is done
  __device__ bool next_block() {
    while (++kstep < nsteps) {
      j = (single_block >= 0) ? single_block : ring_block(i, kstep, P);
      const BlockRel rel = block_relation(layout, causal, i, j);
      const int64_t extent = visible_key_extent(rel, a_hi, Bb);
      if (extent <= 0) continue;
      band = (rel.kind == kAll) ? kBandAll : rel.band;
      ntile = (int32_t)((extent + kKvTn - 1) / kKvTn);
      t = 0;
      return true;
    }
    return false;
  }
  __device__ bool next() { return (++t < ntile) ? true : next_block(); }
};

// One KV tile on its way from global memory to LDS.
template <int D>
struct KvRegs {
  static constexpr int CR = D / 8;
  static constexpr int RPP = kQThreads / CR;
  static constexpr int NP = kKvTn / RPP;
  u32x4 k[NP], v[NP];
};

template <int D>
__device__ __forceinline__ void load_kv(KvRegs<D>& r, const __bf16* kb, const __bf16* vb, int64_t ks_tok,
                                        int64_t vs_tok, int32_t b0, int32_t Bb, int tid) {
  using T = KvRegs<D>;
  const int c = tid % T::CR;
  const int r0 = tid / T::CR;
#pragma unroll
  for (int q = 0; q < T::NP; ++q) {
    const int32_t x = b0 + r0 + T::RPP * q;
    u32x4 vk = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
    if (x < Bb) {
      vk = *reinterpret_cast<const u32x4*>(kb + (int64_t)x * ks_tok + 8 * c);
      vv = *reinterpret_cast<const u32x4*>(vb + (int64_t)x * vs_tok + 8 * c);
    }
    r.k[q] = vk;
    r.v[q] = vv;
  }
}

template <int D>
__device__ __forceinline__ void store_kv(const KvRegs<D>& r, __bf16* stage, int tid) {
  using T = KvRegs<D>;
  using L = KvLds<D>;
  const int c = tid % T::CR;
  const int r0 = tid / T::CR;
#pragma unroll
  for (int q = 0; q < T::NP; ++q) {
    const int row = r0 + T::RPP * q;
    *reinterpret_cast<u32x4*>(stage + tile_off<D>(row, 8 * c)) = r.k[q];
    *reinterpret_cast<u32x4*>(stage + L::TILE + tile_off<D>(row, 8 * c)) = r.v[q];
  }
}

}  // namespace ra

#endif  // RA_KVWALK_H_
