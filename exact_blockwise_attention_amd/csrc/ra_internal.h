// ra_internal.h — kernel parameter blocks and launch entry points shared by
// the C ABI driver (ra_api.cpp) and the kernel translation units.
#ifndef RA_INTERNAL_H_
#define RA_INTERNAL_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

// A strided sequence tensor as ring blocks (element strides; features
// contiguous). Mirrors ra_seq from the public header.
struct Seq {
  void* ptr;
  int64_t s_blk, s_batch, s_tok, s_head;
};

// Forward launch. mode 0: every rank in [rank_begin, rank_begin + n_ranks)
// walks the whole ring inside one launch. mode 1: one ring step (block
// step_block) for a single rank, K/V read from a received buffer; the running
// state enters from / leaves to (st_o, st_lse) unless first / last. mode 2:
// the ring steps of every rank in range are cut into n_split contiguous runs
// (run s: steps s*P/n_split .. (s+1)*P/n_split - 1), one workgroup per (run,
// query tile), K/V read in place; run s leaves its partial state in slot s of
// (st_o, st_lse), and merge_splits combines the slots.
struct FwdParams {
  Seq q, k, v, o;
  float* lse;      // [n_ranks][B][H][Bb], natural log
  float* st_o;     // step mode: fp32 [n_ranks][B][H][Bb][D] normalised partial O
  float* st_lse;   // step mode: fp32 [n_ranks][B][H][Bb], log2 domain
  int32_t B, H, D, P;
  int32_t Hk, G;   // K/V heads; query heads per K/V head (H = G * Hk)
  int64_t Bb;
  int32_t layout, causal;
  float scale_log2;  // scale * log2(e)
  int32_t rank_begin, n_ranks;
  int32_t mode, step_block, first, last;
  int32_t n_split;  // mode 2: runs of ring steps per rank
};

// Backward launches (whole ring for ranks in range).
struct BwdParams {
  Seq q, k, v, o, dout, dq, dk, dv;
  const float* lse;  // [n_ranks][B][H][Bb]
  float* dsum;       // workspace: D = rowsum(dO * O), [n_ranks][B][H][Bb]
  float* lse2;       // workspace: lse * log2(e) (the exponent base the kernels use), same layout
  int32_t B, H, D, P;
  int32_t Hk, G;     // K/V heads; query heads per K/V head (H = G * Hk)
  int64_t Bb;
  int32_t layout, causal;
  float scale, scale_log2;
  int32_t rank_begin, n_ranks;
  // The backward that stores dS once (bf16; null ds: dQ recomputes S and
  // dP instead). ds: kDsRows x kDsKeys tiles, ds_stride per (rank - begin,
  // batch, query head, key block), the query tiles of a pair in order and
  // in each the key tiles its last row sees; kop: K of every (batch, K/V
  // head, block, 128-key tile) in the operand order of dQ = dS K.
  __bf16* ds;
  __bf16* kop;
  int64_t ds_stride;
};

// Dense product with fused epilogue: out[m][n] = sum_k a[m][k] w[n][k]
// (+ bias[n]) (+ res[m][n]) (then GELU), fp32 or bf16 out.
struct GemmParams {
  const __bf16* a;
  int64_t lda;
  const __bf16* w;
  int64_t ldw;
  const float* bias;  // [N] or null
  const __bf16* res;  // [M][ldr] or null
  int64_t ldr;
  void* out;
  int64_t ldo;
  int64_t M;
  int32_t N, K;
  int32_t gelu, out_f32;
};

hipError_t launch_gemm_bf16(const GemmParams& p, hipStream_t s);
hipError_t launch_layer_norm(const float* in, int64_t rows, int32_t d, const float* gamma, const float* beta,
                             float eps, __bf16* out, hipStream_t s);
hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t s);
hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t s);
hipError_t launch_merge_splits(const FwdParams& p, hipStream_t s);
hipError_t launch_bwd_preprocess(const BwdParams& p, int32_t bf16, hipStream_t s);
hipError_t launch_dkdv_bf16(const BwdParams& p, hipStream_t s);
hipError_t launch_dkdv_f32(const BwdParams& p, hipStream_t s);
hipError_t launch_dq_bf16(const BwdParams& p, hipStream_t s);
hipError_t launch_dq_f32(const BwdParams& p, hipStream_t s);
hipError_t launch_kop_pack(const BwdParams& p, hipStream_t s);
hipError_t launch_dq_from_ds(const BwdParams& p, hipStream_t s);
hipError_t launch_merge_lse(int64_t rows, int32_t d, const float* oa, const float* la,
                            const float* ob, const float* lb, float* oo, float* lo,
                            hipStream_t s);
// Copies block `blk` of a strided sequence into a dense [B][Bb][H][D] buffer.
hipError_t launch_gather_block(const Seq& src, int32_t blk, void* dst, int32_t B, int32_t H,
                               int32_t D, int64_t Bb, int32_t elem_bytes, hipStream_t s);
// Original order [B, L, H, D] <-> blocked [P][B][Bb][H][D] for a layout.
hipError_t launch_layout_copy(const void* src, void* dst, int32_t B, int32_t H, int32_t D,
                              int32_t P, int64_t Bb, int32_t layout, int32_t inverse,
                              int32_t elem_bytes, hipStream_t s);

}  // namespace ra

#endif  // RA_INTERNAL_H_
