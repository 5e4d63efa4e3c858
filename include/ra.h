/*
 * ra.h — C ABI of the MI355X (gfx950) exact blockwise ring-attention library.
 *
 * What it computes. Softmax attention O = softmax(scale * Q K^T) V, exactly
 * (up to floating-point rounding order), computed the way one device of a
 * ring computes it: the device keeps its query block Q_i resident and visits
 * the P key/value blocks in ring order j = (i - k) mod P, k = 0..P-1, merging
 * the partial results with an online softmax (running max, running sum of
 * exponentials, rescaled accumulator).
 *   Sources: "Ring Attention 論文分析" (blog), sections "ブロック単位の分割戦略"
 *   (blockwise online softmax), "リングトポロジーと KV の循環" (ring loop:
 *   send to rank+1, receive from rank-1), "Causal Masking の処理" (skip /
 *   diagonal / full blocks) and "逆伝播での KV 再循環" (backward from the
 *   saved log-sum-exp); "Ring Attention: Sequence Parallelism for Long
 *   Context" (book chapter), sections "Ring Attention: Compute While You
 *   Communicate" (step k attends KV block (i - k) mod P) and "The
 *   Causal-Mask Problem: Striped Attention" (token t goes to device t mod P).
 *
 * One GPU plays one device's share (a single rank) or every device of the
 * ring (a rank range); KV blocks are read in place, or, for a single rank,
 * "received" into a double buffer by a copy on a second stream that overlaps
 * the compute of the previous block.
 *
 * Conventions.
 *   - A sequence of L = P * block_len tokens is split into P equal blocks.
 *     Token positions (used by the causal mask) of local row x of block s:
 *       RA_LAYOUT_CONTIGUOUS: t = s * block_len + x
 *       RA_LAYOUT_STRIPED:    t = x * P + s   (ascending order within a block)
 *       RA_LAYOUT_ZIGZAG:     with h = block_len / 2 (block_len even): t = s*h + x
 *                             for x < h, t = (2P-1-s)*h + (x-h) for x >= h — the
 *                             chapter's zigzag variant (two half-blocks placed
 *                             symmetrically near the start and the end)
 *     Causal: key t' is visible to query t iff t' <= t. Non-causal: all keys.
 *   - scale > 0 is used as given; scale <= 0 selects 1 / sqrt(head_dim).
 *   - lse (log-sum-exp) is the natural log of sum over visible keys of
 *     exp(scale * q.k); fp32, laid out [rank - rank_begin][batch][head][row],
 *     contiguous (row fastest).
 *   - Accumulation is fp32 in every mode; outputs O, dQ, dK, dV are written
 *     in the problem dtype, rounded to nearest even.
 *
 * Ownership and synchronisation. The caller owns every buffer (device memory)
 * including the workspace, sized by ra_workspace_bytes(). The library never
 * allocates or frees device memory; it creates and destroys only transient
 * HIP events. Calls are asynchronous on the given stream(s); all work on the
 * copy stream is joined back into the compute stream before the call returns,
 * so outputs are ready when the compute stream reaches that point. Inputs must
 * stay unmodified until then. The library keeps no state between calls.
 *
 * Errors. Every argument is validated before anything is enqueued; on a
 * failed check the call returns a non-zero ra_status and launches nothing.
 * A failing HIP call returns RA_ERR_HIP (work enqueued before it may run).
 */
#ifndef RA_H_
#define RA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RA_LAYOUT_CONTIGUOUS = 0, /* device s owns tokens s*Bb .. s*Bb + Bb - 1 */
  RA_LAYOUT_STRIPED = 1,    /* token t belongs to device t mod P */
  RA_LAYOUT_ZIGZAG = 2      /* device s owns half-blocks s and 2P-1-s of 2P */
} ra_layout;

typedef enum {
  RA_F32 = 0,  /* Q, K, V, O, dO, dQ, dK, dV are float32 */
  RA_BF16 = 1  /* ... are bfloat16 (accumulation stays fp32) */
} ra_dtype;

typedef enum {
  RA_OK = 0,
  RA_ERR_NULL = 1,        /* a required pointer is NULL */
  RA_ERR_SHAPE = 2,       /* sizes, ranks, strides or layout out of range */
  RA_ERR_UNSUPPORTED = 3, /* valid but not implemented (e.g. head_dim) */
  RA_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than required */
  RA_ERR_ALIGN = 5,       /* a pointer or stride breaks 16-byte alignment */
  RA_ERR_HIP = 6,         /* a HIP runtime call failed */
  RA_ERR_SCRATCH = 7      /* ra_backward_noalloc: problem larger than its static scratch */
} ra_status;

/* The problem: batch B, heads H, head dim d (= value dim), ring of P blocks
 * of block_len tokens each. Supported: head_dim 64 or 128; any block_len >= 1
 * (ragged tiles are masked); causal 0/1; layout matters only when causal.
 * Grouped-query attention (blog, section "比較分析: Ring Attention vs
 * Sequence Parallelism vs Tensor Parallelism": ring attention works with
 * GQA/MQA unchanged): K, V, dK and dV have kv_heads heads, and query head h
 * reads K/V head h / (heads / kv_heads) — consecutive query heads share one
 * K/V head; dK/dV of a K/V head sum over the query heads that read it.
 * kv_heads = 0 means kv_heads = heads (multi-head); otherwise it must divide
 * heads (RA_ERR_SHAPE). lse, O, dQ and D have `heads` heads. */
typedef struct {
  int32_t batch;
  int32_t heads;
  int32_t head_dim;
  int32_t ring_size;  /* P >= 1 */
  int64_t block_len;  /* tokens per block, all blocks equal */
  int32_t layout;     /* ra_layout */
  int32_t causal;     /* 0 or 1 */
  float scale;        /* <= 0: 1/sqrt(head_dim) */
  int32_t dtype;      /* ra_dtype */
  int32_t kv_heads;   /* heads of K, V, dK, dV; 0: same as heads */
} ra_problem;

/* A sequence tensor seen as ring blocks. Element (blk, b, x, h, e) — block,
 * batch, local row, head, feature — is at
 *     ptr + blk*s_blk + b*s_batch + x*s_tok + h*s_head + e
 * counted in elements of the problem dtype (features are contiguous). An
 * original-order [B, L, H, d] tensor is described without copying by
 *     contiguous: s_blk = block_len*H*d, s_tok = H*d,   s_head = d, s_batch = L*H*d
 *     striped:    s_blk = H*d,           s_tok = P*H*d, s_head = d, s_batch = L*H*d
 * A zigzag block is not a strided slice of the original order: pass blocked
 * tensors ([P][B][block_len][H][d]: s_blk = B*block_len*H*d, s_batch =
 * block_len*H*d, s_tok = H*d, s_head = d), which ra_layout_copy produces.
 * ptr and every stride times the element size must be multiples of 16 bytes.
 * The bf16 forward needs the K and V token strides at most 2^25 elements,
 * the bf16 backward the Q and dO token strides below 2^24 elements
 * (RA_ERR_UNSUPPORTED otherwise). */
typedef struct {
  void* ptr;
  int64_t s_blk;
  int64_t s_batch;
  int64_t s_tok;
  int64_t s_head;
} ra_seq;

/* Bytes of workspace ra_forward (backward = 0) or ra_backward (backward = 1
 * or 2) needs for ranks [rank_begin, rank_end). use_copy_stream selects the
 * forward's double-buffered receive mode. Without it, a bf16 forward of a
 * single rank whose query block is too small to fill the GPU asks for the
 * partial states of its split launch (see ra_forward). For the backward,
 * backward = 2 gives the smallest workspace (8 bytes per query row: D and
 * lse), with which dQ recomputes the scores; backward = 1 the size with
 * which a bf16 backward also stores dS once (K in operand order and 2 bytes
 * per visible pair, in 64 x 128 tiles) and forms dQ from it, the faster path.
 * The two are equal when dS is not stored (fp32, block_len above 2^18).
 * Returns 0 for an invalid problem (and when no workspace is needed). */
size_t ra_workspace_bytes(const ra_problem* pb, int32_t rank_begin, int32_t rank_end,
                          int32_t use_copy_stream, int32_t backward);

/* Forward (blog: ring_attention_forward and the causal step; chapter: ring
 * step k attends KV block (i - k) mod P). For every rank i in
 * [rank_begin, rank_end): O_i and lse_i of query block i against all P KV
 * blocks, visited in ring order, with the causal/striped mask; fully masked
 * KV tiles are skipped.
 *   q, o : blocks indexed by i - rank_begin (o written, dtype of problem)
 *   k, v : blocks indexed by absolute block id 0..P-1
 *   lse  : fp32 output, [rank_end - rank_begin][B][H][block_len]
 *   copy : NULL -> one launch reads KV blocks in place, state stays on chip;
 *          non-NULL -> requires rank_end = rank_begin + 1: each ring step's
 *          KV block is gathered into a double buffer on `copy` while the
 *          previous step computes on `compute` (events order both hazards);
 *          the running state is merged between steps by log-sum-exp.
 *          The workspace then starts with the double buffer: K0, V0, K1,
 *          V1, each one dense [B][block_len][kv_heads][head_dim] block in
 *          the problem dtype at a 256-byte aligned offset; step k receives
 *          into pair k & 1, so after the call pair (P-1) & 1 holds the block
 *          of step P-1 and the other pair that of step P-2.
 *   workspace: ra_workspace_bytes(pb, rb, re, copy != NULL, 0) bytes.
 *          With copy = NULL it is optional. Given, and when the problem is
 *          bf16 with a single rank whose 256-row query tiles number fewer
 *          than 256 (one device's share with a short query block), the P ring
 *          steps are cut into contiguous runs computed in parallel, each
 *          leaving a partial (O, lse) in the workspace, and the partials are
 *          merged by log-sum-exp (the blog's online-softmax correction, as in
 *          ra_merge_lse). Without it, the same share runs in one launch, one
 *          workgroup per query tile. The two agree within rounding. */
ra_status ra_forward(const ra_problem* pb, int32_t rank_begin, int32_t rank_end,
                     const ra_seq* q, const ra_seq* k, const ra_seq* v, const ra_seq* o,
                     float* lse, void* workspace, size_t workspace_bytes,
                     hipStream_t compute, hipStream_t copy);

/* Backward (blog, section "逆伝播での KV 再循環"): recomputes P = exp(S - lse)
 * with the forward's mask and returns dQ, dK, dV of sum(dO * O). D =
 * rowsum(dO * O) is computed first from the given O (into the workspace).
 * Each KV block visits the query blocks of ranks [rank_begin, rank_end) in
 * ring order ((j + k) mod P at step k) carrying its dK/dV accumulators on
 * chip. With the workspace of ra_workspace_bytes(..., 1) (bf16) that walk
 * writes dS once and dQ = scale * dS K is formed from it, each query tile's
 * sum on chip over the KV blocks in ring order; with the smaller workspace
 * of ra_workspace_bytes(..., 2) each query block walks the KV blocks again
 * ((i - k) mod P), recomputing S and dP. No atomics on either path: the
 * result is deterministic, and dK, dV are the same bits on both.
 *   q, o, dout, dq, lse: indexed by i - rank_begin; k, v, dk, dv: absolute.
 *   dk, dv receive the contributions of the ranks in range (all P ranks:
 *   the full gradient). Blocks of dk/dv are written for every j.
 *   workspace: at least ra_workspace_bytes(pb, rb, re, 0, 2) bytes (else
 *   RA_ERR_WORKSPACE); ra_workspace_bytes(pb, rb, re, 0, 1) or more selects
 *   the stored-dS path. */
ra_status ra_backward(const ra_problem* pb, int32_t rank_begin, int32_t rank_end,
                      const ra_seq* q, const ra_seq* k, const ra_seq* v, const ra_seq* o,
                      const ra_seq* dout, const float* lse, const ra_seq* dq,
                      const ra_seq* dk, const ra_seq* dv, void* workspace,
                      size_t workspace_bytes, hipStream_t compute);

/* One stage of ra_backward, with the same arguments (ra_backward runs stages
 * 0, 1, 2 in order on `compute`): 0 = D = rowsum(dO * O), and lse in base-2
 * units, into the workspace (on the stored-dS path also K in operand order);
 * 1 = the key-side ring walk (recompute S and P, dP, dS; dV and dK; on the
 * stored-dS path dS is written);
 * 2 = dQ: from the stored dS, or by the query-side ring walk that recomputes
 * S, P, dP and dS. Each stage reads what the ones before it wrote, so they
 * must run in order; lets a caller time or interleave the stages. The
 * workspace size selects the path as in ra_backward and must be the same
 * for all three stages. Unknown stage: RA_ERR_SHAPE. */
ra_status ra_backward_stage(int32_t stage, const ra_problem* pb, int32_t rank_begin,
                            int32_t rank_end, const ra_seq* q, const ra_seq* k, const ra_seq* v,
                            const ra_seq* o, const ra_seq* dout, const float* lse,
                            const ra_seq* dq, const ra_seq* dk, const ra_seq* dv,
                            void* workspace, size_t workspace_bytes, hipStream_t compute);

/* ra_backward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the same computation and kernels as ra_backward
 * on its smallest workspace (dQ by the recomputing walk; dK, dV the same
 * bits as ra_backward's), with D and lse in base-2 units (8 bytes per query
 * row of the range) kept
 * in a static device array of ra_backward_noalloc_max_bytes() bytes (64 MiB:
 * 8M query rows, e.g. 8 ranks x 32 heads x 32768 rows), one per GPU, held
 * until the process ends. The array used is the current device's (the
 * compute stream must belong to it); its address is looked up on the first
 * call made with that device current. Nothing is allocated or freed, and
 * nothing in the array needs to start at zero: every call writes the rows it
 * reads. Calls that overlap on one GPU (concurrent streams, threads) share
 * the one array and race: serialise them. A problem whose rows need more
 * than the array returns RA_ERR_SCRATCH before anything is enqueued; other
 * errors as ra_backward. */
ra_status ra_backward_noalloc(const ra_problem* pb, int32_t rank_begin, int32_t rank_end,
                              const ra_seq* q, const ra_seq* k, const ra_seq* v, const ra_seq* o,
                              const ra_seq* dout, const float* lse, const ra_seq* dq,
                              const ra_seq* dk, const ra_seq* dv, hipStream_t compute);

/* Bytes of the static scratch ra_backward_noalloc uses on each GPU. */
size_t ra_backward_noalloc_max_bytes(void);

/* Merge two partial results over disjoint key sets (blog, section
 * "ブロック単位の分割戦略": the online-softmax correction; here in its
 * log-sum-exp form): lse = M + ln(e^(lse_a - M) + e^(lse_b - M)),
 * M = max(lse_a, lse_b); O = e^(lse_a - lse) O_a + e^(lse_b - lse) O_b.
 * A -inf partial has weight 0; two give lse = -inf, O = 0.
 * o_*: fp32 [rows][head_dim]; lse_*: fp32 [rows]. o_out/lse_out may alias
 * the a or b inputs exactly (in place). head_dim in 1..1024. */
ra_status ra_merge_lse(int64_t rows, int32_t head_dim, const float* o_a, const float* lse_a,
                       const float* o_b, const float* lse_b, float* o_out, float* lse_out,
                       hipStream_t stream);

/* Layout gather (chapter, section "The Causal-Mask Problem: Striped
 * Attention"): copy an original-order [B, L, H, d] tensor `src` into blocked
 * order `dst` ([P][B][block_len][H][d], block of rank 0 first) for the given
 * layout, or back when inverse != 0. Pure data movement: bit-exact. Uses the
 * problem's batch, heads, head_dim, ring_size, block_len, layout and dtype
 * (H = heads: to copy the K or V of a grouped-query problem, pass a problem
 * whose heads is its kv_heads). */
ra_status ra_layout_copy(const ra_problem* pb, const void* src, void* dst, int32_t inverse,
                         hipStream_t stream);

/* ---- The Blockwise Parallel Transformer layer around attention ("Ring
 * Attention 論文分析" (blog), section "BPT の Feedforward 融合": each query
 * block goes through attention, the output projection, residual + layer
 * norm, the feedforward network and residual + layer norm before the next
 * block starts, so intermediate results never exist for the whole sequence).
 * The Q/K/V projections are ra_linear calls and attention is ra_forward. */

/* A linear layer with fused epilogue: out[r][c] = sum_i a[r][i] w[c][i],
 * then + bias[c] (fp32, or NULL), then + residual[r][c] (bf16, row stride
 * ldr, or NULL), then the exact GELU 0.5 v (1 + erf(v / sqrt 2)) if gelu != 0.
 * a: bf16 [m][k] (row stride lda); w: bf16 [n][k] (row stride ldw), the
 * [out][in] weight of the layer; out: fp32 if out_f32 != 0 else bf16 (round
 * to nearest even), row stride ldo. fp32 accumulation. Requires m >= 1,
 * n % 128 == 0, k % 64 == 0, 16-byte aligned pointers and row strides
 * (RA_ERR_SHAPE / RA_ERR_ALIGN otherwise). */
ra_status ra_linear(int64_t m, int32_t n, int32_t k, const void* a, int64_t lda, const void* w,
                    int64_t ldw, const float* bias, const void* residual, int64_t ldr, int32_t gelu,
                    void* out, int64_t ldo, int32_t out_f32, hipStream_t stream);

/* Row layer normalisation: out[r] = (z[r] - mean) / sqrt(var + eps) * gamma
 * + beta, mean and biased variance over the d entries of the row. z: fp32
 * [rows][d]; gamma, beta: fp32 [d]; out: bf16 [rows][d]. eps <= 0 selects
 * 1e-5. d in 1..8192. */
ra_status ra_layer_norm(int64_t rows, int32_t d, const float* z, const float* gamma, const float* beta,
                        float eps, void* out, hipStream_t stream);

typedef struct {
  int64_t rows;       /* rows of the sequence (all blocks) */
  int32_t d_model;    /* multiple of 128, at most 8192 */
  int32_t d_ff;       /* multiple of 128 */
  int64_t block_rows; /* rows finished at a time; the workspace holds one block */
  float ln_eps;       /* <= 0: 1e-5 */
} ra_bpt_problem;

/* Weights in bf16 as [out][in], biases and normalisation gains/offsets in fp32. */
typedef struct {
  const void* w_o;    /* [d_model][d_model] */
  const float* b_o;   /* [d_model] */
  const float* ln1_g; /* [d_model] */
  const float* ln1_b;
  const void* w_1;    /* [d_ff][d_model] */
  const float* b_1;   /* [d_ff] */
  const void* w_2;    /* [d_model][d_ff] */
  const float* b_2;   /* [d_model] */
  const float* ln2_g;
  const float* ln2_b;
} ra_bpt_weights;

/* Workspace of ra_bpt_ffn: block_rows * (6 d_model + 2 d_ff) bytes (rounded
 * up per buffer); 0 for an invalid problem. */
size_t ra_bpt_workspace_bytes(const ra_bpt_problem* pb);

/* The layer after attention, block_rows rows at a time:
 *   y = attn W_o^T + b_o + x        h = LN1(y)
 *   u = GELU(h W_1^T + b_1)         z = u W_2^T + b_2 + h      out = LN2(z)
 * attn (the heads side by side), x and out: bf16 [rows][d_model],
 * contiguous. y and z are fp32; h and u are bf16 (the next product's
 * operands). */
ra_status ra_bpt_ffn(const ra_bpt_problem* pb, const void* attn, const void* x, const ra_bpt_weights* wts,
                     void* out, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Static description of a status code. */
const char* ra_status_string(int32_t status);

/* ABI version: increments when a signature or struct above changes. */
int32_t ra_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RA_H_ */
