// ra_schedule.h — ring schedule, token layouts and causal block relations.
//
// Plain integer logic used by the host driver and by the kernels (marked
// host+device under hipcc; plain inline functions under a host compiler, so
// a g++-built unit test can check it on the CPU).
//
// Sources: "Ring Attention: Sequence Parallelism for Long Context" (book
// chapter), section "Ring Attention: Compute While You Communicate": at step
// k device i attends KV block (i - k) mod P; section "The Causal-Mask
// Problem: Striped Attention": token t goes to device t mod P, and the
// zigzag variant gives each device two half-blocks placed symmetrically near
// the start and the end of the sequence. "Ring Attention 論文分析" (blog),
// section "Causal Masking の処理": a KV block later than the query block is
// skipped, the diagonal block gets the strictly-upper triangle masked,
// earlier blocks are computed in full.
#ifndef RA_SCHEDULE_H_
#define RA_SCHEDULE_H_

#include <stdint.h>

#if defined(__HIPCC__)
#define RA_HD __host__ __device__ __forceinline__
#else
#define RA_HD inline
#endif

namespace ra {

enum Layout : int32_t { kContiguous = 0, kStriped = 1, kZigzag = 2 };

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
//   contiguous: t = s Bb + x
//   striped:    t = x P + s
//   zigzag:     the sequence is cut into 2P chunks of Bb/2 tokens; block s
//               holds chunk s (rows 0 .. Bb/2-1) then chunk 2P-1-s.
RA_HD int64_t token_position(int32_t layout, int32_t P, int64_t block_len, int32_t s, int64_t x) {
  if (layout == kStriped) return x * (int64_t)P + s;
  if (layout == kZigzag) {
    const int64_t hb = block_len / 2;
    return x < hb ? (int64_t)s * hb + x : (int64_t)(2 * P - 1 - s) * hb + (x - hb);
  }
  return (int64_t)s * block_len + x;
}

// Relation of KV block j to query block i: query row a (local) sees exactly
// the keys 0 .. ext(a) - 1 of the block (local order), with
//   ext(a) = clamp(a + band + 1, 0, cap),
//   (band, cap) = (band, cap_lo) if a < split, else (band_hi, cap_hi).
// ext is non-decreasing in a for every layout, so the last row of a tile
// bounds the keys the tile needs and its first row decides whether every key
// of a key tile is visible. kind: kNone (no key visible to any row: skip),
// kAll (every key visible to every row), kBand (anything else).
enum RelKind : int32_t { kNone = 0, kAll = 1, kBand = 2 };
constexpr int32_t kBandInf = 1 << 30;  // a band no row/key difference reaches

struct BlockRel {
  int32_t kind;
  int32_t band;
  int32_t split;
  int32_t band_hi;
  int32_t cap_lo;
  int32_t cap_hi;
};

RA_HD BlockRel make_rel(int32_t kind, int32_t band, int32_t block_len) {
  BlockRel r;
  r.kind = kind;
  r.band = band;
  r.split = block_len;
  r.band_hi = band;
  r.cap_lo = block_len;
  r.cap_hi = block_len;
  return r;
}

// Derivations.
//  striped: key b of block j is token b*P + j, query a of block i is token
//    a*P + i; b*P + j <= a*P + i  <=>  b - a <= (i - j) / P, and with
//    |i - j| < P that is b - a <= 0 for j <= i and b - a <= -1 for j > i.
//  zigzag (h = Bb/2): query a < h is in chunk i, a >= h in chunk 2P-1-i;
//    key b < h is in chunk j, b >= h in chunk 2P-1-j. Chunk j < P <= 2P-1-i,
//    so every query row sees the whole first half of every block; chunk
//    2P-1-j > i, so rows a < h never see the second half. Hence j < i:
//    ext = h for all rows; j > i: ext = 0 for a < h, Bb for a >= h; j == i:
//    the chunks pair up diagonally, ext = a + 1.
RA_HD BlockRel block_relation(int32_t layout, int32_t causal, int32_t i, int32_t j, int32_t block_len) {
  if (!causal) return make_rel(kAll, kBandInf, block_len);
  if (layout == kStriped) return make_rel(kBand, (j <= i) ? 0 : -1, block_len);
  if (layout == kZigzag) {
    const int32_t hb = block_len / 2;
    if (j == i) return make_rel(kBand, 0, block_len);
    BlockRel r = make_rel(kBand, kBandInf, block_len);
    if (j < i) {
      r.cap_lo = hb;
      r.cap_hi = hb;
    } else {
      r.split = hb;
      r.cap_lo = 0;
      r.band_hi = kBandInf;
      r.cap_hi = block_len;
    }
    if (hb == 0 && j < i) r.kind = kNone;  // one-token blocks: no first half
    return r;
  }
  if (j > i) return make_rel(kNone, 0, block_len);
  if (j == i) return make_rel(kBand, 0, block_len);
  return make_rel(kAll, kBandInf, block_len);
}

// ext(a): the number of leading keys of the block that row a sees.
RA_HD int64_t row_extent(const BlockRel& r, int64_t a) {
  if (r.kind == kNone) return 0;
  const bool lo = a < r.split;
  const int64_t band = lo ? r.band : r.band_hi;
  const int64_t cap = lo ? r.cap_lo : r.cap_hi;
  int64_t n = a + band + 1;
  if (n < 0) n = 0;
  return n < cap ? n : cap;
}

// row_extent in 32-bit arithmetic, for the kernels (a < 2^30 and
// |band| <= 2^30, so a + band + 1 fits).
RA_HD int32_t row_extent32(const BlockRel& r, int32_t a) {
  const bool lo = a < r.split;
  int32_t n = a + (lo ? r.band : r.band_hi) + 1;
  const int32_t cap = lo ? r.cap_lo : r.cap_hi;
  n = n < 0 ? 0 : n;
  n = n < cap ? n : cap;
  return r.kind == kNone ? 0 : n;
}

// Number of keys of the block that any query row up to a_hi can see.
RA_HD int64_t visible_key_extent(const BlockRel& r, int64_t a_hi, int64_t block_len) {
  (void)block_len;
  return row_extent(r, a_hi);
}

// First query row that sees key b (block_len if none does).
RA_HD int64_t first_row_seeing(const BlockRel& r, int64_t b, int64_t block_len) {
  if (r.kind == kNone) return block_len;
  // lower rows: a in [0, split) see b iff b < min(a + band + 1, cap_lo)
  if (r.split > 0 && b < r.cap_lo) {
    int64_t a = b - r.band;
    if (a < 0) a = 0;
    if (a < r.split && a < block_len) return a;
  }
  if (r.split < block_len && b < r.cap_hi) {
    int64_t a = b - r.band_hi;
    if (a < r.split) a = r.split;
    if (a < block_len) return a;
  }
  return block_len;
}

// first_row_seeing in 32-bit arithmetic, for the kernels: row a sees key b
// iff first_row_seeing32(r, b, Bb) <= a (row extents grow with the row).
RA_HD int32_t first_row_seeing32(const BlockRel& r, int32_t b, int32_t block_len) {
  if (r.kind == kNone) return block_len;
  if (r.split > 0 && b < r.cap_lo) {
    int32_t a = b - r.band;
    a = a < 0 ? 0 : a;
    if (a < r.split && a < block_len) return a;
  }
  if (r.split < block_len && b < r.cap_hi) {
    int32_t a = b - r.band_hi;
    a = a < r.split ? r.split : a;
    if (a < block_len) return a;
  }
  return block_len;
}

// The backward's stored score gradients: dS of a block pair is kept as
// tiles of kDsRows query rows x kDsKeys keys, only the tiles the key-side
// walk computes: key tile kt meets the query tiles from the first one whose
// last row sees its first key (row extents grow with the row) to the last.
// A pair's tiles are stored key tile by key tile, and within a key tile by
// query tile, so that the key-side walk writes consecutive tiles.
// Blocks of at most kDsMaxBlock tokens store dS (longer ones would need
// terabytes).
constexpr int32_t kDsRows = 64;
constexpr int32_t kDsKeys = 128;
constexpr int32_t kDsMaxBlock = 1 << 18;

// Key tiles that query tile qt meets: 0 .. ds_key_tiles - 1 (those whose
// first key its last row sees).
RA_HD int32_t ds_key_tiles(const BlockRel& r, int32_t qt, int32_t block_len) {
  int32_t a_last = qt * kDsRows + kDsRows - 1;
  a_last = a_last < block_len - 1 ? a_last : block_len - 1;
  return (row_extent32(r, a_last) + kDsKeys - 1) / kDsKeys;
}

// First query tile that key tile kt meets (the number of query tiles when
// no row sees its first key).
RA_HD int32_t ds_first_qtile(const BlockRel& r, int32_t kt, int32_t block_len) {
  const int32_t a = first_row_seeing32(r, kt * kDsKeys, block_len);
  return a >= block_len ? (block_len + kDsRows - 1) / kDsRows : a / kDsRows;
}

// Position of key tile kt's first tile in its pair's run (the tiles of the
// key tiles before it); with kt = the number of key tiles, the pair's count.
// Tile (qt, kt) is at ds_key_tile_start(kt) + qt - ds_first_qtile(kt).
RA_HD int64_t ds_key_tile_start(const BlockRel& r, int32_t kt, int32_t block_len) {
  const int32_t qtiles = (block_len + kDsRows - 1) / kDsRows;
  int64_t n = 0;
  for (int32_t k = 0; k < kt; ++k) n += qtiles - ds_first_qtile(r, k, block_len);
  return n;
}

// Visible (query, key) pairs between query rows [a_lo, a_hi] and all keys of
// a block, exact.
RA_HD int64_t visible_pairs(const BlockRel& r, int64_t a_lo, int64_t a_hi, int64_t block_len) {
  (void)block_len;
  if (r.kind == kNone || a_hi < a_lo) return 0;
  int64_t total = 0;
  for (int64_t a = a_lo; a <= a_hi; ++a) total += row_extent(r, a);
  return total;
}

// Unmasked pairs computed by device i over the whole ring (all P blocks).
inline int64_t rank_pairs(int32_t layout, int32_t causal, int32_t P, int64_t block_len, int32_t i) {
  int64_t total = 0;
  for (int32_t k = 0; k < P; ++k) {
    int32_t j = ring_block(i, k, P);
    total += visible_pairs(block_relation(layout, causal, i, j, (int32_t)block_len), 0, block_len - 1, block_len);
  }
  return total;
}

}  // namespace ra

#endif  // RA_SCHEDULE_H_
