// ra_api.cpp — the C ABI: argument validation, workspace carving, and the
// stream/event choreography of the ring walk. Every check runs before the
// first enqueue; no device memory is allocated here.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ra.h"
#include "ra_internal.h"
#include "ra_schedule.h"

namespace {

constexpr size_t kAlign = 256;
constexpr float kLog2e = 1.44269504088896340736f;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int32_t elem_bytes(int32_t dtype) { return dtype == RA_BF16 ? 2 : 4; }

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

int32_t kv_heads_of(const ra_problem* pb) { return pb->kv_heads == 0 ? pb->heads : pb->kv_heads; }

ra_status check_problem(const ra_problem* pb, int32_t rb, int32_t re) {
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
      !mul_ok(t2, (int64_t)(re - rb), &t3))
    return RA_ERR_SHAPE;
  if (t3 / 64 > (int64_t)INT32_MAX) return RA_ERR_SHAPE;
  return RA_OK;
}

constexpr int64_t kMaxTokStride = int64_t(1) << 25;     // elements
constexpr int64_t kMaxBwdTokStride = int64_t(1) << 24;  // elements, exclusive

ra_status check_seq(const ra_seq* s, int32_t es) {
  if (!s || !s->ptr) return RA_ERR_NULL;
  if (s->s_blk < 0 || s->s_batch < 0 || s->s_tok < 0 || s->s_head < 0) return RA_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(s->ptr) % 16) return RA_ERR_ALIGN;
  if ((s->s_blk * es) % 16 || (s->s_batch * es) % 16 || (s->s_tok * es) % 16 || (s->s_head * es) % 16)
    return RA_ERR_ALIGN;
  return RA_OK;
}

ra::Seq to_seq(const ra_seq* s) { return ra::Seq{s->ptr, s->s_blk, s->s_batch, s->s_tok, s->s_head}; }

float eff_scale(const ra_problem* pb) {
  return pb->scale > 0.0f ? pb->scale : 1.0f / sqrtf((float)pb->head_dim);
}

struct FwdWs {
  size_t kbuf[2], vbuf[2], st_o, st_lse, total;
  int32_t n_split;  // runs of ring steps of a split launch (1: not split)
};

// One rank's share whose query tiles (256 rows per workgroup) cannot fill the
// chip's 256 CUs runs its P ring steps as this many parallel runs, merged by
// log-sum-exp: enough runs for one workgroup per CU (the forward holds one
// per CU), at most P. More runs, in two rounds, measured slower: each run
// pays its start-up and its partial state's write and merge.
int32_t split_runs(const ra_problem* pb, int32_t n_ranks) {
  if (pb->dtype != RA_BF16 || n_ranks != 1 || pb->ring_size < 2) return 1;
  const int64_t tiles = (pb->block_len + 255) / 256;
  const int64_t base = (int64_t)n_ranks * pb->batch * pb->heads * tiles;
  if (base >= 256) return 1;
  const int64_t want = (256 + base - 1) / base;
  return (int32_t)(want < pb->ring_size ? want : pb->ring_size);
}

FwdWs fwd_ws_layout(const ra_problem* pb, int32_t n_ranks, int32_t copy) {
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

struct BwdWs {
  size_t dsum, lse2, total;
};

// D = rowsum(dO * O) and lse in log2 units, one fp32 per query row each
BwdWs bwd_ws_layout(const ra_problem* pb, int32_t n_ranks) {
  BwdWs w{};
  const size_t rows = (size_t)n_ranks * pb->batch * pb->heads * pb->block_len;
  w.dsum = 0;
  w.lse2 = align_up(rows * sizeof(float));
  w.total = w.lse2 + align_up(rows * sizeof(float));
  return w;
}

struct BptWs {
  size_t y, h, u, total;  // y (then z): fp32 [br][dm]; h: bf16 [br][dm]; u: bf16 [br][dff]
};

bool bpt_problem_ok(const ra_bpt_problem* pb) {
  return pb && pb->rows >= 1 && pb->d_model >= 128 && pb->d_model % 128 == 0 && pb->d_model <= 8192 &&
         pb->d_ff >= 128 && pb->d_ff % 128 == 0 && pb->block_rows >= 1 && pb->block_rows <= (int64_t)1 << 24 &&
         pb->ln_eps == pb->ln_eps && !isinf(pb->ln_eps);
}

BptWs bpt_ws_layout(const ra_bpt_problem* pb) {
  BptWs w{};
  const size_t br = (size_t)(pb->block_rows < pb->rows ? pb->block_rows : pb->rows);
  w.y = 0;
  w.h = align_up(br * pb->d_model * sizeof(float));
  w.u = w.h + align_up(br * pb->d_model * 2);
  w.total = w.u + align_up(br * (size_t)pb->d_ff * 2);
  return w;
}

#define RA_HIP(call)                         \
  do {                                       \
    if ((call) != hipSuccess) {              \
      (void)hipGetLastError();               \
      return RA_ERR_HIP;                     \
    }                                        \
  } while (0)

// Destroys the transient events of one call on every exit path.
struct Events {
  hipEvent_t ev[5] = {nullptr, nullptr, nullptr, nullptr, nullptr};
  ~Events() {
    for (auto& e : ev)
      if (e) (void)hipEventDestroy(e);
  }
};

}  // namespace

extern "C" {

size_t ra_workspace_bytes(const ra_problem* pb, int32_t rank_begin, int32_t rank_end,
                          int32_t use_copy_stream, int32_t backward) {
  if (check_problem(pb, rank_begin, rank_end) != RA_OK) return 0;
  const int32_t n = rank_end - rank_begin;
  if (backward) return bwd_ws_layout(pb, n).total;
  return fwd_ws_layout(pb, n, use_copy_stream ? 1 : 0).total;
}

ra_status ra_forward(const ra_problem* pb, int32_t rank_begin, int32_t rank_end, const ra_seq* q,
                     const ra_seq* k, const ra_seq* v, const ra_seq* o, float* lse, void* workspace,
                     size_t workspace_bytes, hipStream_t compute, hipStream_t copy) {
  ra_status st = check_problem(pb, rank_begin, rank_end);
  if (st != RA_OK) return st;
  const int32_t es = elem_bytes(pb->dtype);
  const ra_seq* seqs[4] = {q, k, v, o};
  for (const ra_seq* s : seqs)
    if ((st = check_seq(s, es)) != RA_OK) return st;
  if (!lse) return RA_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(lse) % 4) return RA_ERR_ALIGN;
  // the bf16 forward addresses the rows of a 64-row K/V tile with 32-bit byte offsets
  if (pb->dtype == RA_BF16 && (k->s_tok > kMaxTokStride || v->s_tok > kMaxTokStride)) return RA_ERR_UNSUPPORTED;
  const int32_t n = rank_end - rank_begin;
  const bool use_copy = copy != nullptr;
  if (use_copy && n != 1) return RA_ERR_SHAPE;
  const FwdWs w = fwd_ws_layout(pb, n, use_copy ? 1 : 0);
  // without the copy stream the workspace is optional: it enables the split
  // launch, and a call without it runs the whole ring in one unsplit launch
  const bool split = !use_copy && w.n_split > 1 && workspace && workspace_bytes >= w.total;
  if (use_copy || split) {
    if (!workspace || workspace_bytes < w.total) return RA_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % kAlign) return RA_ERR_ALIGN;
  }

  ra::FwdParams p{};
  p.q = to_seq(q);
  p.k = to_seq(k);
  p.v = to_seq(v);
  p.o = to_seq(o);
  p.lse = lse;
  p.B = pb->batch;
  p.H = pb->heads;
  p.Hk = kv_heads_of(pb);
  p.G = pb->heads / p.Hk;
  p.D = pb->head_dim;
  p.P = pb->ring_size;
  p.Bb = pb->block_len;
  p.layout = pb->layout;
  p.causal = pb->causal;
  p.scale_log2 = eff_scale(pb) * kLog2e;
  p.rank_begin = rank_begin;
  p.n_ranks = n;
  auto launch = [&](const ra::FwdParams& pp) {
    return pb->dtype == RA_BF16 ? ra::launch_fwd_bf16(pp, compute) : ra::launch_fwd_f32(pp, compute);
  };

  if (split) {
    // the runs' partial states, then their log-sum-exp merge into O and lse
    char* ws = reinterpret_cast<char*>(workspace);
    p.mode = 2;
    p.n_split = w.n_split;
    p.first = 1;
    p.last = 0;
    p.st_o = reinterpret_cast<float*>(ws + w.st_o);
    p.st_lse = reinterpret_cast<float*>(ws + w.st_lse);
    RA_HIP(launch(p));
    RA_HIP(ra::launch_merge_splits(p, compute));
    return RA_OK;
  }
  if (!use_copy) {
    p.mode = 0;
    RA_HIP(launch(p));
    return RA_OK;
  }

  // Ring receive stand-in: block (i - k - 1) mod P is copied into the idle
  // half of a double buffer on `copy` while step k computes on `compute`.
  // RAW: compute waits for the copy of its block (ev_copy). WAR: a copy
  // into a buffer waits for the step that last read it (ev_comp).
  char* ws = reinterpret_cast<char*>(workspace);
  const int32_t i = rank_begin;
  const int32_t P = pb->ring_size;
  Events evs;
  hipEvent_t& ev_start = evs.ev[0];
  hipEvent_t* ev_copy = &evs.ev[1];
  hipEvent_t* ev_comp = &evs.ev[3];
  for (auto& e : evs.ev) RA_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming));
  RA_HIP(hipEventRecord(ev_start, compute));  // inputs are ready on `compute`
  RA_HIP(hipStreamWaitEvent(copy, ev_start, 0));

  const int64_t dense_tok = (int64_t)kv_heads_of(pb) * pb->head_dim;
  auto buf_seq = [&](size_t off) {
    return ra::Seq{ws + off, 0, (int64_t)pb->block_len * dense_tok, dense_tok, pb->head_dim};
  };
  auto copy_block = [&](int32_t step) -> hipError_t {
    const int32_t j = ra::ring_block(i, step, P);
    const int32_t bsel = step & 1;
    hipError_t e = ra::launch_gather_block(to_seq(k), j, ws + w.kbuf[bsel], pb->batch, kv_heads_of(pb),
                                           pb->head_dim, pb->block_len, es, copy);
    if (e != hipSuccess) return e;
    e = ra::launch_gather_block(to_seq(v), j, ws + w.vbuf[bsel], pb->batch, kv_heads_of(pb),
                                pb->head_dim, pb->block_len, es, copy);
    if (e != hipSuccess) return e;
    return hipEventRecord(ev_copy[bsel], copy);
  };

  RA_HIP(copy_block(0));
  p.mode = 1;
  p.st_o = reinterpret_cast<float*>(ws + w.st_o);
  p.st_lse = reinterpret_cast<float*>(ws + w.st_lse);
  for (int32_t kstep = 0; kstep < P; ++kstep) {
    const int32_t bsel = kstep & 1;
    if (kstep + 1 < P) {
      // the buffer (kstep+1)&1 was last read by step kstep-1
      if (kstep >= 1) RA_HIP(hipStreamWaitEvent(copy, ev_comp[(kstep + 1) & 1], 0));
      RA_HIP(copy_block(kstep + 1));
    }
    RA_HIP(hipStreamWaitEvent(compute, ev_copy[bsel], 0));
    p.step_block = ra::ring_block(i, kstep, P);
    p.first = kstep == 0;
    p.last = kstep == P - 1;
    p.k = buf_seq(w.kbuf[bsel]);
    p.v = buf_seq(w.vbuf[bsel]);
    RA_HIP(launch(p));
    RA_HIP(hipEventRecord(ev_comp[bsel], compute));
  }
  return RA_OK;
}

static ra_status backward_impl(int32_t first_stage, int32_t last_stage, const ra_problem* pb,
                               int32_t rank_begin, int32_t rank_end, const ra_seq* q,
                               const ra_seq* k, const ra_seq* v, const ra_seq* o,
                               const ra_seq* dout, const float* lse, const ra_seq* dq,
                               const ra_seq* dk, const ra_seq* dv, void* workspace,
                               size_t workspace_bytes, hipStream_t compute) {
  ra_status st = check_problem(pb, rank_begin, rank_end);
  if (st != RA_OK) return st;
  const int32_t es = elem_bytes(pb->dtype);
  const ra_seq* seqs[8] = {q, k, v, o, dout, dq, dk, dv};
  for (const ra_seq* s : seqs)
    if ((st = check_seq(s, es)) != RA_OK) return st;
  if (!lse) return RA_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(lse) % 4) return RA_ERR_ALIGN;
  // the bf16 dK/dV walk addresses a 64-row query tile of Q and dO through
  // signed 32-bit byte offsets
  if (pb->dtype == RA_BF16 && (q->s_tok >= kMaxBwdTokStride || dout->s_tok >= kMaxBwdTokStride))
    return RA_ERR_UNSUPPORTED;
  const int32_t n = rank_end - rank_begin;
  const BwdWs w = bwd_ws_layout(pb, n);
  if (!workspace || workspace_bytes < w.total) return RA_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign) return RA_ERR_ALIGN;

  char* ws = reinterpret_cast<char*>(workspace);
  ra::BwdParams p{};
  p.q = to_seq(q);
  p.k = to_seq(k);
  p.v = to_seq(v);
  p.o = to_seq(o);
  p.dout = to_seq(dout);
  p.dq = to_seq(dq);
  p.dk = to_seq(dk);
  p.dv = to_seq(dv);
  p.lse = lse;
  p.dsum = reinterpret_cast<float*>(ws + w.dsum);
  p.lse2 = reinterpret_cast<float*>(ws + w.lse2);
  p.B = pb->batch;
  p.H = pb->heads;
  p.Hk = kv_heads_of(pb);
  p.G = pb->heads / p.Hk;
  p.D = pb->head_dim;
  p.P = pb->ring_size;
  p.Bb = pb->block_len;
  p.layout = pb->layout;
  p.causal = pb->causal;
  p.scale = eff_scale(pb);
  p.scale_log2 = p.scale * kLog2e;
  p.rank_begin = rank_begin;
  p.n_ranks = n;
  const int32_t bf16 = pb->dtype == RA_BF16;
  if (first_stage <= 0 && last_stage >= 0) RA_HIP(ra::launch_bwd_preprocess(p, bf16, compute));
  if (first_stage <= 1 && last_stage >= 1)
    RA_HIP(bf16 ? ra::launch_dkdv_bf16(p, compute) : ra::launch_dkdv_f32(p, compute));
  if (first_stage <= 2 && last_stage >= 2)
    RA_HIP(bf16 ? ra::launch_dq_bf16(p, compute) : ra::launch_dq_f32(p, compute));
  return RA_OK;
}

ra_status ra_backward(const ra_problem* pb, int32_t rank_begin, int32_t rank_end, const ra_seq* q,
                      const ra_seq* k, const ra_seq* v, const ra_seq* o, const ra_seq* dout,
                      const float* lse, const ra_seq* dq, const ra_seq* dk, const ra_seq* dv,
                      void* workspace, size_t workspace_bytes, hipStream_t compute) {
  return backward_impl(0, 2, pb, rank_begin, rank_end, q, k, v, o, dout, lse, dq, dk, dv, workspace,
                       workspace_bytes, compute);
}

ra_status ra_backward_stage(int32_t stage, const ra_problem* pb, int32_t rank_begin,
                            int32_t rank_end, const ra_seq* q, const ra_seq* k, const ra_seq* v,
                            const ra_seq* o, const ra_seq* dout, const float* lse,
                            const ra_seq* dq, const ra_seq* dk, const ra_seq* dv, void* workspace,
                            size_t workspace_bytes, hipStream_t compute) {
  if (stage < 0 || stage > 2) return RA_ERR_SHAPE;
  return backward_impl(stage, stage, pb, rank_begin, rank_end, q, k, v, o, dout, lse, dq, dk, dv,
                       workspace, workspace_bytes, compute);
}

ra_status ra_merge_lse(int64_t rows, int32_t head_dim, const float* o_a, const float* lse_a,
                       const float* o_b, const float* lse_b, float* o_out, float* lse_out,
                       hipStream_t stream) {
  if (!o_a || !lse_a || !o_b || !lse_b || !o_out || !lse_out) return RA_ERR_NULL;
  if (rows < 0 || head_dim < 1 || head_dim > 1024) return RA_ERR_SHAPE;
  if (rows / 4 > (int64_t)INT32_MAX) return RA_ERR_SHAPE;
  const void* ptrs[6] = {o_a, lse_a, o_b, lse_b, o_out, lse_out};
  for (const void* ptr : ptrs)
    if (reinterpret_cast<uintptr_t>(ptr) % 4) return RA_ERR_ALIGN;
  if (head_dim % 4 == 0) {
    const void* optrs[3] = {o_a, o_b, o_out};
    for (const void* ptr : optrs)
      if (reinterpret_cast<uintptr_t>(ptr) % 16) return RA_ERR_ALIGN;
  }
  RA_HIP(ra::launch_merge_lse(rows, head_dim, o_a, lse_a, o_b, lse_b, o_out, lse_out, stream));
  return RA_OK;
}

ra_status ra_layout_copy(const ra_problem* pb, const void* src, void* dst, int32_t inverse,
                         hipStream_t stream) {
  ra_status st = check_problem(pb, 0, pb ? pb->ring_size : 1);
  if (st != RA_OK) return st;
  if (!src || !dst) return RA_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(src) % 16 || reinterpret_cast<uintptr_t>(dst) % 16) return RA_ERR_ALIGN;
  RA_HIP(ra::launch_layout_copy(src, dst, pb->batch, pb->heads, pb->head_dim, pb->ring_size,
                                pb->block_len, pb->layout, inverse ? 1 : 0, elem_bytes(pb->dtype),
                                stream));
  return RA_OK;
}

ra_status ra_linear(int64_t m, int32_t n, int32_t k, const void* a, int64_t lda, const void* w,
                    int64_t ldw, const float* bias, const void* residual, int64_t ldr, int32_t gelu,
                    void* out, int64_t ldo, int32_t out_f32, hipStream_t stream) {
  if (!a || !w || !out) return RA_ERR_NULL;
  if (m < 1 || n < 128 || n % 128 || k < 64 || k % 64) return RA_ERR_SHAPE;
  if (lda < k || ldw < k || ldo < n || (residual && ldr < n)) return RA_ERR_SHAPE;
  if ((m + 255) / 256 * (n / 128) > (int64_t)INT32_MAX) return RA_ERR_SHAPE;
  const void* ptrs[4] = {a, w, out, residual};
  for (const void* ptr : ptrs)
    if (reinterpret_cast<uintptr_t>(ptr) % 16) return RA_ERR_ALIGN;
  if (lda % 8 || ldw % 8 || (residual && ldr % 8) || ldo % 8) return RA_ERR_ALIGN;
  if (bias && reinterpret_cast<uintptr_t>(bias) % 4) return RA_ERR_ALIGN;
  ra::GemmParams p{};
  p.a = reinterpret_cast<const __bf16*>(a);
  p.lda = lda;
  p.w = reinterpret_cast<const __bf16*>(w);
  p.ldw = ldw;
  p.bias = bias;
  p.res = reinterpret_cast<const __bf16*>(residual);
  p.ldr = ldr;
  p.out = out;
  p.ldo = ldo;
  p.M = m;
  p.N = n;
  p.K = k;
  p.gelu = gelu ? 1 : 0;
  p.out_f32 = out_f32 ? 1 : 0;
  RA_HIP(ra::launch_gemm_bf16(p, stream));
  return RA_OK;
}

ra_status ra_layer_norm(int64_t rows, int32_t d, const float* z, const float* gamma, const float* beta,
                        float eps, void* out, hipStream_t stream) {
  if (!z || !gamma || !beta || !out) return RA_ERR_NULL;
  if (rows < 0 || rows > (int64_t)INT32_MAX || d < 1 || d > 8192) return RA_ERR_SHAPE;
  if (!(eps == eps) || isinf(eps)) return RA_ERR_SHAPE;
  const void* ptrs[4] = {z, gamma, beta, out};
  for (const void* ptr : ptrs)
    if (reinterpret_cast<uintptr_t>(ptr) % 4) return RA_ERR_ALIGN;
  RA_HIP(ra::launch_layer_norm(z, rows, d, gamma, beta, eps > 0.0f ? eps : 1e-5f,
                               reinterpret_cast<__bf16*>(out), stream));
  return RA_OK;
}

size_t ra_bpt_workspace_bytes(const ra_bpt_problem* pb) {
  if (!bpt_problem_ok(pb)) return 0;
  return bpt_ws_layout(pb).total;
}

ra_status ra_bpt_ffn(const ra_bpt_problem* pb, const void* attn, const void* x, const ra_bpt_weights* wts,
                     void* out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!pb || !attn || !x || !wts || !out) return RA_ERR_NULL;
  if (!bpt_problem_ok(pb)) return RA_ERR_SHAPE;
  const void* wptrs[10] = {wts->w_o, wts->b_o, wts->ln1_g, wts->ln1_b, wts->w_1,
                           wts->b_1, wts->w_2, wts->b_2, wts->ln2_g, wts->ln2_b};
  for (const void* ptr : wptrs)
    if (!ptr) return RA_ERR_NULL;
  const void* big[6] = {attn, x, out, wts->w_o, wts->w_1, wts->w_2};
  for (const void* ptr : big)
    if (reinterpret_cast<uintptr_t>(ptr) % 16) return RA_ERR_ALIGN;
  for (int i : {1, 2, 3, 5, 7, 8, 9})
    if (reinterpret_cast<uintptr_t>(wptrs[i]) % 4) return RA_ERR_ALIGN;
  const BptWs w = bpt_ws_layout(pb);
  if (!workspace || workspace_bytes < w.total) return RA_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign) return RA_ERR_ALIGN;
  char* ws = reinterpret_cast<char*>(workspace);
  float* yz = reinterpret_cast<float*>(ws + w.y);
  __bf16* h = reinterpret_cast<__bf16*>(ws + w.h);
  __bf16* u = reinterpret_cast<__bf16*>(ws + w.u);
  const int64_t dm = pb->d_model, dff = pb->d_ff;
  const float eps = pb->ln_eps > 0.0f ? pb->ln_eps : 1e-5f;
  auto gemm = [&](int64_t m, int32_t n, int32_t k, const void* a, int64_t lda, const void* wt, const float* bias,
                  const void* res, int64_t ldr, int32_t gelu, void* o, int64_t ldo, int32_t f32) {
    ra::GemmParams p{};
    p.a = reinterpret_cast<const __bf16*>(a);
    p.lda = lda;
    p.w = reinterpret_cast<const __bf16*>(wt);
    p.ldw = k;
    p.bias = bias;
    p.res = reinterpret_cast<const __bf16*>(res);
    p.ldr = ldr;
    p.out = o;
    p.ldo = ldo;
    p.M = m;
    p.N = n;
    p.K = k;
    p.gelu = gelu;
    p.out_f32 = f32;
    return ra::launch_gemm_bf16(p, stream);
  };
  for (int64_t r0 = 0; r0 < pb->rows; r0 += pb->block_rows) {
    const int64_t br = (pb->rows - r0 < pb->block_rows) ? pb->rows - r0 : pb->block_rows;
    const __bf16* ab = reinterpret_cast<const __bf16*>(attn) + r0 * dm;
    const __bf16* xb = reinterpret_cast<const __bf16*>(x) + r0 * dm;
    __bf16* ob = reinterpret_cast<__bf16*>(out) + r0 * dm;
    RA_HIP(gemm(br, (int32_t)dm, (int32_t)dm, ab, dm, wts->w_o, wts->b_o, xb, dm, 0, yz, dm, 1));
    RA_HIP(ra::launch_layer_norm(yz, br, (int32_t)dm, wts->ln1_g, wts->ln1_b, eps, h, stream));
    RA_HIP(gemm(br, (int32_t)dff, (int32_t)dm, h, dm, wts->w_1, wts->b_1, nullptr, 0, 1, u, dff, 0));
    RA_HIP(gemm(br, (int32_t)dm, (int32_t)dff, u, dff, wts->w_2, wts->b_2, h, dm, 0, yz, dm, 1));
    RA_HIP(ra::launch_layer_norm(yz, br, (int32_t)dm, wts->ln2_g, wts->ln2_b, eps, ob, stream));
  }
  return RA_OK;
}

const char* ra_status_string(int32_t status) {
  switch (status) {
    case RA_OK: return "ok";
    case RA_ERR_NULL: return "a required pointer is NULL";
    case RA_ERR_SHAPE: return "sizes, ranks, strides or layout out of range";
    case RA_ERR_UNSUPPORTED:
      return "valid but unsupported configuration (head_dim other than 64 or 128, a bf16 forward K/V "
             "token stride above 2^25 elements, or a bf16 backward Q/dO token stride of 2^24 or more)";
    case RA_ERR_WORKSPACE: return "workspace missing or too small";
    case RA_ERR_ALIGN: return "pointer or stride not 16-byte aligned";
    case RA_ERR_HIP: return "HIP runtime call failed";
    default: return "unknown status";
  }
}

int32_t ra_abi_version(void) { return 2; }

}  // extern "C"
