// ra_schedule.h — ring schedule, token layouts and causal block relations.
//
// Plain integer logic used by the host driver and by the kernels (marked
// host+device under hipcc; plain inline functions under a host compiler, so
// a g++-built unit test can check it on the CPU).
//
// Sources: "Ring Attention: Sequence Parallelism for Long Context" (book
// chapter), section "Ring Attention: Compute While You Communicate": at step
// k device i attends KV block (i - k) mod P; section "The Causal-Mask
// Problem: Striped Attention": token t goes to device t mod P. "Ring
// Attention 論文分析" (blog), section "Causal Masking の処理": a KV block
// later than the query block is skipped, the diagonal block gets the
// strictly-upper triangle masked, earlier blocks are computed in full.
#ifndef RA_SCHEDULE_H_
#define RA_SCHEDULE_H_

#include <stdint.h>

#if defined(__HIPCC__)
#define RA_HD __host__ __device__ __forceinline__
#else
#define RA_HD inline
#endif

namespace ra {

enum Layout : int32_t { kContiguous = 0, kStriped = 1 };

// KV block held by device i at ring step k (each device forwards its block
// to (i + 1) mod P and receives from (i - 1) mod P).
RA_HD int32_t ring_block(int32_t i, int32_t k, int32_t P) {
  int32_t j = (i - k) % P;
  return j < 0 ? j + P : j;
}

// Query block visited by KV block j at ring step k (the inverse map: the
// block that started on device j is on device (j + k) mod P).
RA_HD int32_t ring_rank(int32_t j, int32_t k, int32_t P) { return (j + k) % P; }

// Original token position of local row x of block s.
RA_HD int64_t token_position(int32_t layout, int32_t P, int64_t block_len, int32_t s, int64_t x) {
  return layout == kStriped ? x * (int64_t)P + s : (int64_t)s * block_len + x;
}

// Relation of KV block j to query block i. Kinds: kNone (every key masked:
// skip the block), kAll (every key visible), kBand (key b visible to query a
// iff b - a <= band, in local row indices).
enum RelKind : int32_t { kNone = 0, kAll = 1, kBand = 2 };

struct BlockRel {
  int32_t kind;
  int32_t band;
};

// Derivation, striped: key b of block j is token b*P + j, query a of block i
// is token a*P + i; b*P + j <= a*P + i  <=>  b - a <= (i - j) / P, and with
// |i - j| < P that is b - a <= 0 for j <= i and b - a <= -1 for j > i.
RA_HD BlockRel block_relation(int32_t layout, int32_t causal, int32_t i, int32_t j) {
  BlockRel r;
  if (!causal) {
    r.kind = kAll;
    r.band = 0;
    return r;
  }
  if (layout == kStriped) {
    r.kind = kBand;
    r.band = (j <= i) ? 0 : -1;
    return r;
  }
  if (j > i) {
    r.kind = kNone;
    r.band = 0;
  } else if (j == i) {
    r.kind = kBand;
    r.band = 0;
  } else {
    r.kind = kAll;
    r.band = 0;
  }
  return r;
}

// Number of keys of a block of `block_len` rows that any query row in
// [a_lo, a_hi] (inclusive, local) can see: keys 0 .. n-1 with
// n = min(block_len, a_hi + band + 1) for a band, all for kAll, none for kNone.
RA_HD int64_t visible_key_extent(BlockRel r, int64_t a_hi, int64_t block_len) {
  if (r.kind == kNone) return 0;
  if (r.kind == kAll) return block_len;
  int64_t n = a_hi + r.band + 1;
  if (n < 0) n = 0;
  return n < block_len ? n : block_len;
}

// Visible (query, key) pairs between query rows [a_lo, a_hi] and all keys of
// a block, exact.
RA_HD int64_t visible_pairs(BlockRel r, int64_t a_lo, int64_t a_hi, int64_t block_len) {
  if (r.kind == kNone || a_hi < a_lo) return 0;
  if (r.kind == kAll) return (a_hi - a_lo + 1) * block_len;
  int64_t total = 0;
  // rows where a + band + 1 <= 0 see nothing; rows where it is >= block_len see all
  for (int64_t a = a_lo; a <= a_hi; ++a) {
    int64_t n = a + r.band + 1;
    if (n < 0) n = 0;
    if (n > block_len) n = block_len;
    total += n;
  }
  return total;
}

// Unmasked pairs computed by device i over the whole ring (all P blocks).
inline int64_t rank_pairs(int32_t layout, int32_t causal, int32_t P, int64_t block_len, int32_t i) {
  int64_t total = 0;
  for (int32_t k = 0; k < P; ++k) {
    int32_t j = ring_block(i, k, P);
    total += visible_pairs(block_relation(layout, causal, i, j), 0, block_len - 1, block_len);
  }
  return total;
}

}  // namespace ra

#endif  // RA_SCHEDULE_H_
