// ra_api.cpp — the C ABI: argument validation, workspace carving, and the
// stream/event choreography of the ring walk. Every check runs before the
// first enqueue; no device memory is allocated here.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "ra.h"
#include "ra_host.h"
#include "ra_internal.h"
#include "ra_schedule.h"

namespace {

using namespace ra::host;

constexpr float kLog2e = 1.44269504088896340736f;

ra::Seq to_seq(const ra_seq* s) { return ra::Seq{s->ptr, s->s_blk, s->s_batch, s->s_tok, s->s_head}; }

#define RA_HIP(call)                         \
  do {                                       \
    if ((call) != hipSuccess) {              \
      (void)hipGetLastError();               \
      return RA_ERR_HIP;                     \
    }                                        \
  } while (0)

// The no-allocation backward's scratch: D = rowsum(dO * O) and lse in base-2
// units for up to kScratchBytes / 8 query rows, one copy per GPU for the
// life of the process. In host code `scratch` only names the array; its
// device address on the current GPU comes from hipGetSymbolAddress, once per
// device, and only that address is handed to kernels.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The scratch array's address on the current device (looked up on the first
// call made with that device current).
hipError_t scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = ptr;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  if (!g_scratch_ptr[dev]) return hipErrorInvalidSymbol;
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

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
  if (backward) return backward == 2 ? bwd_ws_layout(pb, n).small_total : bwd_ws_layout(pb, n).total;
  return fwd_ws_layout(pb, n, use_copy_stream ? 1 : 0).total;
}

ra_status ra_forward(const ra_problem* pb, int32_t rank_begin, int32_t rank_end, const ra_seq* q,
                     const ra_seq* k, const ra_seq* v, const ra_seq* o, float* lse, void* workspace,
                     size_t workspace_bytes, hipStream_t compute, hipStream_t copy) {
  const FwdPlan plan = plan_forward(pb, rank_begin, rank_end, q, k, v, o, lse, workspace, workspace_bytes,
                                    copy != nullptr);
  if (plan.st != RA_OK) return plan.st;
  const int32_t es = elem_bytes(pb->dtype);
  const int32_t n = rank_end - rank_begin;
  const bool use_copy = plan.use_copy;
  const bool split = plan.split;
  const FwdWs& w = plan.ws;

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
                               size_t workspace_bytes, hipStream_t compute, bool allow_ds = true) {
  const BwdPlan plan = plan_backward(pb, rank_begin, rank_end, q, k, v, o, dout, lse, dq, dk, dv, workspace,
                                     workspace_bytes);
  if (plan.st != RA_OK) return plan.st;
  const int32_t n = rank_end - rank_begin;
  const BwdWs& w = plan.ws;

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
  const bool store_ds = plan.store_ds && allow_ds;
  if (store_ds) {
    p.kop = reinterpret_cast<__bf16*>(ws + w.kop);
    p.ds = reinterpret_cast<__bf16*>(ws + w.ds);
    p.ds_stride = w.ds_stride;
  }
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
  if (first_stage <= 0 && last_stage >= 0) {
    RA_HIP(ra::launch_bwd_preprocess(p, bf16, compute));
    if (store_ds) RA_HIP(ra::launch_kop_pack(p, compute));
  }
  if (first_stage <= 1 && last_stage >= 1)
    RA_HIP(bf16 ? ra::launch_dkdv_bf16(p, compute) : ra::launch_dkdv_f32(p, compute));
  if (first_stage <= 2 && last_stage >= 2) {
    if (store_ds) RA_HIP(ra::launch_dq_from_ds(p, compute));
    else RA_HIP(bf16 ? ra::launch_dq_bf16(p, compute) : ra::launch_dq_f32(p, compute));
  }
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

ra_status ra_backward_noalloc(const ra_problem* pb, int32_t rank_begin, int32_t rank_end, const ra_seq* q,
                              const ra_seq* k, const ra_seq* v, const ra_seq* o, const ra_seq* dout,
                              const float* lse, const ra_seq* dq, const ra_seq* dk, const ra_seq* dv,
                              hipStream_t compute) {
  // every argument check first, with a stand-in for the workspace, then the
  // size against the static scratch
  const BwdPlan plan = plan_backward(pb, rank_begin, rank_end, q, k, v, o, dout, lse, dq, dk, dv,
                                     reinterpret_cast<const void*>(kAlign), SIZE_MAX);
  if (plan.st != RA_OK) return plan.st;
  if (plan.ws.small_total > kScratchBytes) return RA_ERR_SCRATCH;
  void* ws = nullptr;
  RA_HIP(scratch_of_current_device(&ws));
  return backward_impl(0, 2, pb, rank_begin, rank_end, q, k, v, o, dout, lse, dq, dk, dv, ws, kScratchBytes,
                       compute, /*allow_ds=*/false);
}

size_t ra_backward_noalloc_max_bytes(void) { return kScratchBytes; }

ra_status ra_merge_lse(int64_t rows, int32_t head_dim, const float* o_a, const float* lse_a,
                       const float* o_b, const float* lse_b, float* o_out, float* lse_out,
                       hipStream_t stream) {
  const ra_status st = check_merge(rows, head_dim, o_a, lse_a, o_b, lse_b, o_out, lse_out);
  if (st != RA_OK) return st;
  RA_HIP(ra::launch_merge_lse(rows, head_dim, o_a, lse_a, o_b, lse_b, o_out, lse_out, stream));
  return RA_OK;
}

ra_status ra_layout_copy(const ra_problem* pb, const void* src, void* dst, int32_t inverse,
                         hipStream_t stream) {
  const ra_status st = check_layout_copy(pb, src, dst);
  if (st != RA_OK) return st;
  RA_HIP(ra::launch_layout_copy(src, dst, pb->batch, pb->heads, pb->head_dim, pb->ring_size,
                                pb->block_len, pb->layout, inverse ? 1 : 0, elem_bytes(pb->dtype),
                                stream));
  return RA_OK;
}

ra_status ra_linear(int64_t m, int32_t n, int32_t k, const void* a, int64_t lda, const void* w,
                    int64_t ldw, const float* bias, const void* residual, int64_t ldr, int32_t gelu,
                    void* out, int64_t ldo, int32_t out_f32, hipStream_t stream) {
  const ra_status st = check_linear(m, n, k, a, lda, w, ldw, bias, residual, ldr, out, ldo);
  if (st != RA_OK) return st;
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
  const ra_status st = check_layer_norm(rows, d, z, gamma, beta, eps, out);
  if (st != RA_OK) return st;
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
  const ra_status st = check_bpt(pb, attn, x, wts, out, workspace, workspace_bytes);
  if (st != RA_OK) return st;
  const BptWs w = bpt_ws_layout(pb);
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
    case RA_ERR_SCRATCH:
      return "problem needs more than the static scratch of the no-allocation entry point "
             "(ra_backward_noalloc_max_bytes)";
    default: return "unknown status";
  }
}

int32_t ra_abi_version(void) { return 3; }

}  // extern "C"
