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
// masked); a single-step launch visits one given block only. KV tiles go
// straight from global memory to a ring of LDS stages, requested a few tiles
// ahead of their use.
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

// LDS: four stages of (K tile, V tile), each [64][D] swizzled.
template <int D>
struct KvLds {
  static constexpr int TILE = kKvTn * D;
  static constexpr int STAGE = 2 * TILE;
  static constexpr int NSTAGE = 4;
  static constexpr int BYTES = NSTAGE * STAGE * 2;
};

// Workgroups are dealt to the 8 XCDs round-robin by linear id, and each XCD
// has its own L2. This maps the linear id to a logical index such that the
// workgroups of one XCD cover a contiguous range of logical indices (XCD x
// gets ids x, x+8, ... and the logical range that starts after the ranges of
// XCDs 0..x-1). A bijection for any grid size.
__device__ __forceinline__ int64_t xcd_logical(int64_t id, int64_t n) {
  const int64_t x = id % 8, s = id / 8;
  const int64_t q = n / 8, r = n % 8;
  return x * q + (x < r ? x : r) + s;
}

// Within an XCD, consecutive workgroups go to its 4 shader engines (8 CUs
// each) in turn, and an engine takes its next workgroup only in that turn.
// An engine therefore receives positions p, p + 4, ... of the XCD's work
// list; if those are always the lightest of a heaviest-first list, the
// engine idles while the others catch up. This maps position p of an item in
// its group (items ranked 0 = heaviest) to the rank it takes: runs of 4 go
// alternately forwards and backwards, so every engine takes one item of
// every run, alternately from its heavy and its light end, and the engines
// get equal work for weights linear in the rank. A last, partial run keeps
// its order. A permutation of 0 .. items - 1.
__device__ __forceinline__ uint32_t se_balanced_rank(uint32_t p, uint32_t items) {
  const uint32_t b = p / 4;
  if (4 * b + 4 > items || b % 2 == 0) return p;
  return 8 * b + 3 - p;
}

// Balanced totals still leave an engine waiting when the 4 workgroups of one
// turn differ in length: its turn comes round only after the others have
// taken theirs. Where the workgroups of a group drift apart anyway (their
// walks differ at every block, as the query tiles of a striped causal block
// do), the work order can instead make every turn's workgroups equal: runs of
// 4 groups listed item by item (item 0 of each, then item 1, ...), so that
// each engine takes whole groups, one item per turn. This splits a logical
// index L of groups x items that way. A bijection for any sizes.
__device__ __forceinline__ void turn_balanced_split(uint32_t L, uint32_t groups, uint32_t items, uint32_t* group,
                                                    uint32_t* item) {
  const uint32_t per = 4 * items;
  const uint32_t c = L / per, r = L % per;
  const uint32_t g0 = 4 * c;
  const uint32_t ce = (groups - g0 < 4) ? groups - g0 : 4;
  *item = r / ce;
  *group = g0 + r % ce;
}

// Query-tile workgroups: consecutive logical indices share (batch, K/V
// head, rank) and take its query tiles heaviest first (in the order of
// se_balanced_rank), with the G query heads that read one K/V head
// innermost, so the workgroups resident on one XCD walk the same KV tiles at
// about the same time and share them in L2; with `turns`, groups of tiles
// follow turn_balanced_split instead. Heavier ranks come first (contiguous
// causal work grows with the rank). bh = b * H + h, H = G * (K/V heads). The
// grid is below 2^31 workgroups.
__device__ __forceinline__ void query_work_of(int64_t id, int32_t BH, int32_t G, int32_t n_ranks,
                                              int32_t tiles, int32_t causal, int32_t layout, bool turns,
                                              int32_t* bh, int32_t* rank_idx, int32_t* tile) {
  const int64_t n = (int64_t)BH * n_ranks * tiles;
  const uint32_t L = (uint32_t)xcd_logical(id, n);
  const uint32_t gi = L % (uint32_t)G;
  const uint32_t L2 = L / (uint32_t)G;
  uint32_t g, it;
  if (turns) {
    turn_balanced_split(L2, (uint32_t)(BH / G) * (uint32_t)n_ranks, (uint32_t)tiles, &g, &it);
  } else {
    // when G is a multiple of 4, every turn holds the G query heads of one
    // tile, and the plain heaviest-first order already balances the engines
    g = L2 / (uint32_t)tiles;
    it = (G % 4 == 0) ? L2 % (uint32_t)tiles : se_balanced_rank(L2 % (uint32_t)tiles, (uint32_t)tiles);
  }
  *tile = tiles - 1 - (int32_t)it;
  *bh = (int32_t)(g / (uint32_t)n_ranks) * G + (int32_t)gi;
  const int32_t r = (int32_t)(g % (uint32_t)n_ranks);
  *rank_idx = (causal && layout == kContiguous) ? n_ranks - 1 - r : r;
}

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

// The (block, tile) pairs a query tile visits, in ring order. rel is the
// relation of the current block to the query block (row a sees its keys
// 0 .. row_extent32(rel, a) - 1).
struct KvIter {
  int32_t kstep, nsteps, j, t, ntile;
  BlockRel rel;
  int32_t i, P, layout, causal, a_hi, Bb, single_block;
  int32_t a_w, ext_w;  // a row of the caller's choice and its extent in the block
  // moves to the next block with a visible tile; false when the ring is done
  __device__ bool next_block() {
    while (++kstep < nsteps) {
      j = (single_block >= 0) ? single_block : ring_block(i, kstep, P);
      rel = block_relation(layout, causal, i, j, Bb);
      const int32_t extent = row_extent32(rel, a_hi);
      if (extent <= 0) continue;
      ntile = (extent + kKvTn - 1) / kKvTn;
      ext_w = row_extent32(rel, a_w);
      t = 0;
      return true;
    }
    return false;
  }
  __device__ bool next() { return (++t < ntile) ? true : next_block(); }
};

// The same tiles in two passes over the ring: first, in each block, the
// tiles that some row of the query tile sees only in part (the causal
// diagonal, and a last tile cut by the block's end), then the tiles that
// every row sees whole (key tile t < ext(a_lo) / 64: row extents grow with
// the row). A kernel runs its masking code in the first pass only.
struct KvPassIter {
  int32_t pass, kstep, nsteps, j, t, t_hi, t_lo;
  BlockRel rel;
  int32_t i, P, layout, causal, a_lo, a_hi, Bb, single_block;
  __device__ bool next_block() {
    for (;;) {
      while (++kstep < nsteps) {
        j = (single_block >= 0) ? single_block : ring_block(i, kstep, P);
        rel = block_relation(layout, causal, i, j, Bb);
        const int32_t extent = row_extent32(rel, a_hi);
        if (extent <= 0) continue;
        const int32_t ntile = (extent + kKvTn - 1) / kKvTn;
        int32_t t_full = row_extent32(rel, a_lo) / kKvTn;
        t_full = t_full < ntile ? t_full : ntile;
        t_lo = pass == 0 ? t_full : 0;
        t_hi = pass == 0 ? ntile : t_full;
        if (t_lo >= t_hi) continue;
        t = t_lo;
        return true;
      }
      if (pass == 1) return false;
      pass = 1;
      kstep = -1;
    }
  }
  __device__ bool next() { return (++t < t_hi) ? true : next_block(); }
};

// Direct global -> LDS copy (global_load_lds_dwordx4: lane l of a wave
// writes its 16 bytes at the wave's LDS base + 16 l) of rows
// [r_lo, r_lo + ROWS) of a strided [rows][D] tensor into a swizzled LDS tile,
// shared by the NW waves of the workgroup. Each lane fetches the logical
// chunk that belongs at its physical position. Rows at or beyond `nrows` read
// row nrows-1 instead (finite data; the kernels mask those rows). The copy is
// asynchronous: wait_dma() and a barrier make it visible.
template <int D, int ROWS, int NW>
__device__ __forceinline__ void dma_rows(__bf16* tile, const __bf16* base, int64_t s_tok, int32_t r_lo,
                                         int32_t nrows, int wave, int lane) {
  constexpr int RW = 1024 / (2 * D);  // rows per wave copy
  constexpr int CPR = D / 8;          // chunks per row
  constexpr int COPIES = ROWS / RW;
  static_assert(COPIES % NW == 0, "copies must split evenly over the waves");
#pragma unroll
  for (int k = 0; k < COPIES / NW; ++k) {
    const int q = wave + NW * k;
    const int row = q * RW + lane / CPR;
    const int c = (lane % CPR) ^ chunk_swz<D>(row);
    int32_t x = r_lo + row;
    if (x > nrows - 1) x = nrows - 1;
    const __bf16* g = base + (int64_t)x * s_tok + 8 * c;
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)(tile + q * RW * D), 16, 0, 0);
  }
}

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Waits until at most N vector-memory loads of this wave are outstanding
// (loads complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier without the implicit memory waits of __syncthreads
// (which drain every copy in flight, also those for later tiles): the kernel
// waits for exactly the copies it needs before it, and every LDS read before
// it has been consumed, so none is still pending.
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

}  // namespace ra

#endif  // RA_KVWALK_H_
