// ra_host.h — host-side argument validation and workspace layout of the C
// ABI (include/ra.h): everything an entry point checks and computes before
// it enqueues work. Plain C++ over the public structs, with no HIP calls, so
// that it also builds with g++ under the address and undefined-behaviour
// sanitizers for the CPU tests; ra_api.cpp performs exactly these checks.
#ifndef RA_HOST_H_
#define RA_HOST_H_

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "ra.h"
#include "ra_schedule.h"

namespace ra {
namespace host {

constexpr size_t kAlign = 256;

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

inline int32_t elem_bytes(int32_t dtype) { return dtype == RA_BF16 ? 2 : 4; }

inline bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

inline bool misaligned(const void* p, uintptr_t a) { return reinterpret_cast<uintptr_t>(p) % a != 0; }

inline int32_t kv_heads_of(const ra_problem* pb) { return pb->kv_heads == 0 ? pb->heads : pb->kv_heads; }

// The problem itself and the rank range [rb, re).
inline ra_status check_problem(const ra_problem* pb, int32_t rb, int32_t re) {
  if (!pb) return RA_ERR_NULL;
  if (pb->batch < 1 || pb->heads < 1 || pb->ring_size < 1 || pb->block_len < 1) return RA_ERR_SHAPE;
  if (kv_heads_of(pb) < 1 || pb->heads % kv_heads_of(pb)) return RA_ERR_SHAPE;
  if (pb->layout != RA_LAYOUT_CONTIGUOUS && pb->layout != RA_LAYOUT_STRIPED && pb->layout != RA_LAYOUT_ZIGZAG)
    return RA_ERR_SHAPE;
  if (pb->layout == RA_LAYOUT_ZIGZAG && pb->block_len % 2) return RA_ERR_SHAPE;  // two half-blocks
  if (pb->causal != 0 && pb->causal != 1) return RA_ERR_SHAPE;
  if (pb->dtype != RA_F32 && pb->dtype != RA_BF16) return RA_ERR_SHAPE;
  if (!(pb->scale == pb->scale) || isinf(pb->scale)) return RA_ERR_SHAPE;  // NaN / inf
  if (pb->head_dim != 64 && pb->head_dim != 128) return RA_ERR_UNSUPPORTED;
  if (pb->block_len > (int64_t)(INT32_MAX / 2)) return RA_ERR_SHAPE;  // local rows are 32-bit
  if (rb < 0 || re > pb->ring_size || rb >= re) return RA_ERR_SHAPE;
  // grid sizes must fit a 32-bit launch: rows * heads * batch * ranks / 64
  int64_t t1, t2, t3;
  if (!mul_ok(pb->block_len, pb->heads, &t1) || !mul_ok(t1, pb->batch, &t2) ||
      !mul_ok(t2, (int64_t)re - rb, &t3))
    return RA_ERR_SHAPE;
  if (t3 / 64 > (int64_t)INT32_MAX) return RA_ERR_SHAPE;
  return RA_OK;
}

constexpr int64_t kMaxTokStride = int64_t(1) << 25;     // elements
constexpr int64_t kMaxBwdTokStride = int64_t(1) << 24;  // elements, exclusive

inline ra_status check_seq(const ra_seq* s, int32_t es) {
  if (!s || !s->ptr) return RA_ERR_NULL;
  const int64_t st[4] = {s->s_blk, s->s_batch, s->s_tok, s->s_head};
  for (int64_t x : st)
    if (x < 0 || x > INT64_MAX / 16) return RA_ERR_SHAPE;  // byte offsets must not overflow
  if (misaligned(s->ptr, 16)) return RA_ERR_ALIGN;
  for (int64_t x : st)
    if ((x * es) % 16) return RA_ERR_ALIGN;
  return RA_OK;
}

inline float eff_scale(const ra_problem* pb) {
  return pb->scale > 0.0f ? pb->scale : 1.0f / sqrtf((float)pb->head_dim);
}

// ---------------------------------------------------------------- forward

struct FwdWs {
  size_t kbuf[2], vbuf[2], st_o, st_lse, total;
  int32_t n_split;  // runs of ring steps of a split launch (1: not split)
};

// One rank's share whose query tiles (256 rows per workgroup) cannot fill the
// chip's 256 CUs runs its P ring steps as this many parallel runs, merged by
// log-sum-exp: enough runs for one workgroup per CU (the forward holds one
// per CU), at most P. More runs, in two rounds, measured slower: each run
// pays its start-up and its partial state's write and merge.
inline int32_t split_runs(const ra_problem* pb, int32_t n_ranks) {
  if (pb->dtype != RA_BF16 || n_ranks != 1 || pb->ring_size < 2) return 1;
  const int64_t tiles = (pb->block_len + 255) / 256;
  const int64_t base = (int64_t)n_ranks * pb->batch * pb->heads * tiles;
  if (base >= 256) return 1;
  const int64_t want = (256 + base - 1) / base;
  return (int32_t)(want < pb->ring_size ? want : pb->ring_size);
}

inline FwdWs fwd_ws_layout(const ra_problem* pb, int32_t n_ranks, int32_t copy) {
  FwdWs w{};
  w.n_split = 1;
  if (!copy) {
    // split launch: n_split partial states (fp32 O and lse per query row)
    const int32_t ns = split_runs(pb, n_ranks);
    if (ns < 2) return w;
    const size_t rows = (size_t)ns * n_ranks * pb->batch * pb->heads * pb->block_len;
    w.n_split = ns;
    w.st_o = 0;
    w.st_lse = align_up(rows * pb->head_dim * sizeof(float));
    w.total = align_up(w.st_lse + rows * sizeof(float));
    return w;
  }
  const size_t es = elem_bytes(pb->dtype);
  const size_t blk = (size_t)pb->batch * pb->block_len * kv_heads_of(pb) * pb->head_dim * es;
  const size_t rows = (size_t)n_ranks * pb->batch * pb->heads * pb->block_len;
  size_t off = 0;
  for (int b = 0; b < 2; ++b) {
    w.kbuf[b] = off;
    off = align_up(off + blk);
    w.vbuf[b] = off;
    off = align_up(off + blk);
  }
  w.st_o = off;
  off = align_up(off + rows * pb->head_dim * sizeof(float));
  w.st_lse = off;
  off = align_up(off + rows * sizeof(float));
  w.total = off;
  return w;
}

// What ra_forward checks before its first enqueue, and how it will run.
struct FwdPlan {
  ra_status st;
  FwdWs ws;
  bool use_copy, split;
};

inline FwdPlan plan_forward(const ra_problem* pb, int32_t rb, int32_t re, const ra_seq* q, const ra_seq* k,
                            const ra_seq* v, const ra_seq* o, const float* lse, const void* workspace,
                            size_t workspace_bytes, bool use_copy) {
  FwdPlan pl{};
  pl.use_copy = use_copy;
  if ((pl.st = check_problem(pb, rb, re)) != RA_OK) return pl;
  const int32_t es = elem_bytes(pb->dtype);
  const ra_seq* seqs[4] = {q, k, v, o};
  for (const ra_seq* s : seqs)
    if ((pl.st = check_seq(s, es)) != RA_OK) return pl;
  if (!lse) return pl.st = RA_ERR_NULL, pl;
  if (misaligned(lse, 4)) return pl.st = RA_ERR_ALIGN, pl;
  // the bf16 forward addresses the rows of a 64-row K/V tile with 32-bit byte offsets
  if (pb->dtype == RA_BF16 && (k->s_tok > kMaxTokStride || v->s_tok > kMaxTokStride))
    return pl.st = RA_ERR_UNSUPPORTED, pl;
  const int32_t n = re - rb;
  if (use_copy && n != 1) return pl.st = RA_ERR_SHAPE, pl;
  pl.ws = fwd_ws_layout(pb, n, use_copy ? 1 : 0);
  // without the copy stream the workspace is optional: it enables the split
  // launch, and a call without it runs the whole ring in one unsplit launch
  pl.split = !use_copy && pl.ws.n_split > 1 && workspace && workspace_bytes >= pl.ws.total;
  if (use_copy || pl.split) {
    if (!workspace || workspace_bytes < pl.ws.total) return pl.st = RA_ERR_WORKSPACE, pl;
    if (misaligned(workspace, kAlign)) return pl.st = RA_ERR_ALIGN, pl;
  }
  pl.st = RA_OK;
  return pl;
}

// ---------------------------------------------------------------- backward

struct BwdWs {
  size_t dsum, lse2, small_total;  // D and lse in base-2 units: what every backward needs
  size_t kop, ds, total;           // + K in operand order and the stored dS tiles (bf16)
  int64_t ds_stride;               // dS tiles reserved per (rank, batch, head, block)
};

// The most dS tiles a block pair stores (kDsRows x kDsKeys each): relations
// depend only on whether the key block comes before, is, or comes after the
// query block, so three representative pairs cover every pair.
inline int64_t ds_pair_stride(const ra_problem* pb) {
  const int32_t Bb = (int32_t)pb->block_len;
  const int32_t ktiles = (Bb + kDsKeys - 1) / kDsKeys;
  const int32_t pairs[3][2] = {{1, 0}, {0, 0}, {0, 1}};
  int64_t best = 0;
  for (const auto& ij : pairs) {
    if (ij[0] >= pb->ring_size || ij[1] >= pb->ring_size) continue;
    const BlockRel r = block_relation(pb->layout, pb->causal, ij[0], ij[1], Bb);
    const int64_t n = ds_key_tile_start(r, ktiles, Bb);
    best = n > best ? n : best;
  }
  return best;
}

// The backward's workspace. [0, small_total): D = rowsum(dO * O) and lse in
// base-2 units, one fp32 per query row each: enough for the walk that
// recomputes the scores for dQ. Then, for the bf16 path that stores dS once:
// K in MFMA operand order (one 128-key tile of D features per (batch, K/V
// head, block, key tile)) and the dS tiles, kDsRows x kDsKeys bf16 each,
// ds_stride of them per (rank, batch, query head, key block).
inline BwdWs bwd_ws_layout(const ra_problem* pb, int32_t n_ranks) {
  BwdWs w{};
  const size_t rows = (size_t)n_ranks * pb->batch * pb->heads * pb->block_len;
  w.dsum = 0;
  w.lse2 = align_up(rows * sizeof(float));
  w.small_total = w.lse2 + align_up(rows * sizeof(float));
  w.total = w.small_total;
  if (pb->dtype != RA_BF16 || pb->block_len > kDsMaxBlock) return w;
  const size_t ktiles = (size_t)((pb->block_len + kDsKeys - 1) / kDsKeys);
  w.kop = w.small_total;
  const size_t kop_bytes = (size_t)pb->batch * kv_heads_of(pb) * pb->ring_size * ktiles * kDsKeys * pb->head_dim * 2;
  w.ds = w.kop + align_up(kop_bytes);
  w.ds_stride = ds_pair_stride(pb);
  const size_t tiles = (size_t)n_ranks * pb->batch * pb->heads * pb->ring_size * (size_t)w.ds_stride;
  if (tiles >= ((size_t)1 << 31)) {  // the kernels number the tiles in 32 bits
    w.ds_stride = 0;
    return w;
  }
  const size_t tile_bytes = (size_t)kDsRows * kDsKeys * 2;
  w.total = w.ds + align_up(tiles * tile_bytes);
  return w;
}

struct BwdPlan {
  ra_status st;
  BwdWs ws;
  bool store_ds;  // bf16 with the full workspace: dS stored once, dQ from it
};

inline BwdPlan plan_backward(const ra_problem* pb, int32_t rb, int32_t re, const ra_seq* q, const ra_seq* k,
                             const ra_seq* v, const ra_seq* o, const ra_seq* dout, const float* lse,
                             const ra_seq* dq, const ra_seq* dk, const ra_seq* dv, const void* workspace,
                             size_t workspace_bytes) {
  BwdPlan pl{};
  if ((pl.st = check_problem(pb, rb, re)) != RA_OK) return pl;
  const int32_t es = elem_bytes(pb->dtype);
  const ra_seq* seqs[8] = {q, k, v, o, dout, dq, dk, dv};
  for (const ra_seq* s : seqs)
    if ((pl.st = check_seq(s, es)) != RA_OK) return pl;
  if (!lse) return pl.st = RA_ERR_NULL, pl;
  if (misaligned(lse, 4)) return pl.st = RA_ERR_ALIGN, pl;
  // the bf16 dK/dV walk addresses a 64-row query tile of Q and dO through
  // signed 32-bit byte offsets
  if (pb->dtype == RA_BF16 && (q->s_tok >= kMaxBwdTokStride || dout->s_tok >= kMaxBwdTokStride))
    return pl.st = RA_ERR_UNSUPPORTED, pl;
  pl.ws = bwd_ws_layout(pb, re - rb);
  if (!workspace || workspace_bytes < pl.ws.small_total) return pl.st = RA_ERR_WORKSPACE, pl;
  if (misaligned(workspace, kAlign)) return pl.st = RA_ERR_ALIGN, pl;
  pl.store_ds = pb->dtype == RA_BF16 && pl.ws.total > pl.ws.small_total && workspace_bytes >= pl.ws.total;
  pl.st = RA_OK;
  return pl;
}

// ---------------------------------------------------------------- the other entry points

inline ra_status check_merge(int64_t rows, int32_t head_dim, const float* o_a, const float* lse_a,
                             const float* o_b, const float* lse_b, const float* o_out, const float* lse_out) {
  if (!o_a || !lse_a || !o_b || !lse_b || !o_out || !lse_out) return RA_ERR_NULL;
  if (rows < 0 || head_dim < 1 || head_dim > 1024) return RA_ERR_SHAPE;
  if (rows / 4 > (int64_t)INT32_MAX) return RA_ERR_SHAPE;
  const void* ptrs[6] = {o_a, lse_a, o_b, lse_b, o_out, lse_out};
  for (const void* ptr : ptrs)
    if (misaligned(ptr, 4)) return RA_ERR_ALIGN;
  if (head_dim % 4 == 0) {
    const void* optrs[3] = {o_a, o_b, o_out};
    for (const void* ptr : optrs)
      if (misaligned(ptr, 16)) return RA_ERR_ALIGN;
  }
  return RA_OK;
}

inline ra_status check_layout_copy(const ra_problem* pb, const void* src, const void* dst) {
  const ra_status st = check_problem(pb, 0, pb ? pb->ring_size : 1);
  if (st != RA_OK) return st;
  if (!src || !dst) return RA_ERR_NULL;
  if (misaligned(src, 16) || misaligned(dst, 16)) return RA_ERR_ALIGN;
  return RA_OK;
}

inline ra_status check_linear(int64_t m, int32_t n, int32_t k, const void* a, int64_t lda, const void* w,
                              int64_t ldw, const float* bias, const void* residual, int64_t ldr, const void* out,
                              int64_t ldo) {
  if (!a || !w || !out) return RA_ERR_NULL;
  if (m < 1 || n < 128 || n % 128 || k < 64 || k % 64) return RA_ERR_SHAPE;
  if (lda < k || ldw < k || ldo < n || (residual && ldr < n)) return RA_ERR_SHAPE;
  if ((m + 255) / 256 * (n / 128) > (int64_t)INT32_MAX) return RA_ERR_SHAPE;
  const void* ptrs[4] = {a, w, out, residual};
  for (const void* ptr : ptrs)
    if (misaligned(ptr, 16)) return RA_ERR_ALIGN;
  if (lda % 8 || ldw % 8 || (residual && ldr % 8) || ldo % 8) return RA_ERR_ALIGN;
  if (bias && misaligned(bias, 4)) return RA_ERR_ALIGN;
  return RA_OK;
}

inline ra_status check_layer_norm(int64_t rows, int32_t d, const float* z, const float* gamma, const float* beta,
                                  float eps, const void* out) {
  if (!z || !gamma || !beta || !out) return RA_ERR_NULL;
  if (rows < 0 || rows > (int64_t)INT32_MAX || d < 1 || d > 8192) return RA_ERR_SHAPE;
  if (!(eps == eps) || isinf(eps)) return RA_ERR_SHAPE;
  const void* ptrs[4] = {z, gamma, beta, out};
  for (const void* ptr : ptrs)
    if (misaligned(ptr, 4)) return RA_ERR_ALIGN;
  return RA_OK;
}

struct BptWs {
  size_t y, h, u, total;  // y (then z): fp32 [br][dm]; h: bf16 [br][dm]; u: bf16 [br][dff]
};

inline bool bpt_problem_ok(const ra_bpt_problem* pb) {
  return pb && pb->rows >= 1 && pb->d_model >= 128 && pb->d_model % 128 == 0 && pb->d_model <= 8192 &&
         pb->d_ff >= 128 && pb->d_ff % 128 == 0 && pb->block_rows >= 1 && pb->block_rows <= (int64_t)1 << 24 &&
         pb->ln_eps == pb->ln_eps && !isinf(pb->ln_eps);
}

inline BptWs bpt_ws_layout(const ra_bpt_problem* pb) {
  BptWs w{};
  const size_t br = (size_t)(pb->block_rows < pb->rows ? pb->block_rows : pb->rows);
  w.y = 0;
  w.h = align_up(br * pb->d_model * sizeof(float));
  w.u = w.h + align_up(br * pb->d_model * 2);
  w.total = w.u + align_up(br * (size_t)pb->d_ff * 2);
  return w;
}

inline ra_status check_bpt(const ra_bpt_problem* pb, const void* attn, const void* x, const ra_bpt_weights* wts,
                           const void* out, const void* workspace, size_t workspace_bytes) {
  if (!pb || !attn || !x || !wts || !out) return RA_ERR_NULL;
  if (!bpt_problem_ok(pb)) return RA_ERR_SHAPE;
  const void* wptrs[10] = {wts->w_o, wts->b_o, wts->ln1_g, wts->ln1_b, wts->w_1,
                           wts->b_1, wts->w_2, wts->b_2, wts->ln2_g, wts->ln2_b};
  for (const void* ptr : wptrs)
    if (!ptr) return RA_ERR_NULL;
  const void* big[6] = {attn, x, out, wts->w_o, wts->w_1, wts->w_2};
  for (const void* ptr : big)
    if (misaligned(ptr, 16)) return RA_ERR_ALIGN;
  for (int i : {1, 2, 3, 5, 7, 8, 9})
    if (misaligned(wptrs[i], 4)) return RA_ERR_ALIGN;
  const BptWs w = bpt_ws_layout(pb);
  if (!workspace || workspace_bytes < w.total) return RA_ERR_WORKSPACE;
  if (misaligned(workspace, kAlign)) return RA_ERR_ALIGN;
  return RA_OK;
}

}  // namespace host
}  // namespace ra

#endif  // RA_HOST_H_
