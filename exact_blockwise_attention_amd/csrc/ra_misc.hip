// ra_misc.hip — memory-bound kernels: log-sum-exp merge of partial results,
// the KV block receive copy, layout gathers, and the backward's row sums.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ra_internal.h"
#include "ra_schedule.h"

namespace ra {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Merge rule ("Ring Attention 論文分析" (blog), section "ブロック
// 単位の分割戦略", the online-softmax correction in log-sum-exp form):
// lse = M + ln(e^(la-M) + e^(lb-M)), O = e^(la-lse) Oa + e^(lb-lse) Ob.
__device__ __forceinline__ void merge_weights(float xa, float xb, float* ca, float* cb, float* lo) {
  const float m = fmaxf(xa, xb);
  const float ms = (m == -INFINITY) ? 0.0f : m;
  const float wa = expf(xa - ms), wb = expf(xb - ms);
  const float tot = wa + wb;
  *ca = (tot > 0.0f) ? wa / tot : 0.0f;
  *cb = (tot > 0.0f) ? wb / tot : 0.0f;
  *lo = (tot > 0.0f) ? ms + logf(tot) : -INFINITY;
}

// Any head_dim: one wave per row. Every lane reads the row's two lse values
// before lane 0 writes the merged one, so lse_out may alias an input (a
// wave executes in lockstep).
__global__ __launch_bounds__(256) void merge_lse_kernel(int64_t rows, int32_t d, const float* oa,
                                                        const float* la, const float* ob,
                                                        const float* lb, float* oo, float* lo) {
  const int lane = threadIdx.x % 64;
  const int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;
  if (row >= rows) return;
  float ca, cb, l;
  merge_weights(la[row], lb[row], &ca, &cb, &l);
  const int64_t base = row * d;
  for (int e = lane; e < d; e += 64) oo[base + e] = ca * oa[base + e] + cb * ob[base + e];
  if (lane == 0) lo[row] = l;
}

// head_dim 64 or 128 (D): D / 4 lanes per row, 16 bytes each per input, and
// kRowsPerLane rows per lane group, all loads issued before any use so that
// enough bytes are in flight to keep HBM busy. The group's lanes read the
// row's lse values before its first lane writes the merged one (in place is
// allowed: a wave executes in lockstep).
constexpr int kMergeRows = 4;

template <int D>
__global__ __launch_bounds__(256) void merge_lse_vec_kernel(int64_t rows, const float* oa, const float* la,
                                                            const float* ob, const float* lb, float* oo,
                                                            float* lo) {
  constexpr int LPR = D / 4;
  constexpr int GROUPS = 256 / LPR;
  const int g = threadIdx.x / LPR, e = 4 * (threadIdx.x % LPR);
  const int64_t row0 = ((int64_t)blockIdx.x * GROUPS + g) * kMergeRows;
  float4 u[kMergeRows], w[kMergeRows];
  float xa[kMergeRows], xb[kMergeRows];
#pragma unroll
  for (int k = 0; k < kMergeRows; ++k) {
    const int64_t row = row0 + k < rows ? row0 + k : rows - 1;
    u[k] = *reinterpret_cast<const float4*>(oa + row * D + e);
    w[k] = *reinterpret_cast<const float4*>(ob + row * D + e);
    xa[k] = la[row];
    xb[k] = lb[row];
  }
#pragma unroll
  for (int k = 0; k < kMergeRows; ++k) {
    const int64_t row = row0 + k;
    if (row >= rows) break;
    float ca, cb, l;
    merge_weights(xa[k], xb[k], &ca, &cb, &l);
    float4 r;
    r.x = ca * u[k].x + cb * w[k].x;
    r.y = ca * u[k].y + cb * w[k].y;
    r.z = ca * u[k].z + cb * w[k].z;
    r.w = ca * u[k].w + cb * w[k].w;
    *reinterpret_cast<float4*>(oo + row * D + e) = r;
    if (e == 0) lo[row] = l;
  }
}

// Combines the partial states of the n_split runs of ring steps of a split
// forward launch into O (bf16) and lse (natural log): the same log-sum-exp
// correction as merge_lse_kernel, over n_split partials. Partial s of row r
// is the normalised O at st_o[(s * rows + r) * D] and its lse in log2 units
// at st_lse[s * rows + r]; a run that saw no key has lse -inf and weight 0.
// Row r = ((ri * B + b) * H + h) * Bb + a.
//
// The rows are few (a short query block), so the kernel is bound by load
// latency: one wave per row, split into G groups of D/8 lanes (8 features
// each). Group g takes partials g, g + G, ..., kMergeBatch at a time with
// all their loads in flight, keeps its own (max, sum, accumulator), and the
// groups combine by lane exchanges.
constexpr int kMergeBatch = 8;

template <int D, int WPB>
__global__ __launch_bounds__(64 * WPB) void merge_splits_kernel(FwdParams p) {
  constexpr int LPR = D / 8;    // lanes per copy of a row
  constexpr int G = 64 / LPR;   // partial groups per row
  const int64_t rows = (int64_t)p.n_ranks * p.B * p.H * p.Bb;
  const int64_t r = (int64_t)blockIdx.x * WPB + threadIdx.x / 64;  // uniform over the wave
  if (r >= rows) return;
  const int lane = threadIdx.x % 64;
  const int g = lane / LPR;
  const int e = 8 * (lane % LPR);
  float m = -INFINITY, l = 0.0f;  // group max and sum (log2 units, relative to m)
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.0f;
  for (int32_t s0 = g; s0 < p.n_split; s0 += kMergeBatch * G) {
    float lv[kMergeBatch];
    float4 u[kMergeBatch][2];
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      const int32_t sk = s0 + k * G;
      const bool ok = sk < p.n_split;
      const int64_t at = (int64_t)(ok ? sk : 0) * rows + r;
      lv[k] = ok ? p.st_lse[at] : -INFINITY;
      u[k][0] = *reinterpret_cast<const float4*>(p.st_o + at * D + e);
      u[k][1] = *reinterpret_cast<const float4*>(p.st_o + at * D + e + 4);
    }
    float mb = m;
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) mb = fmaxf(mb, lv[k]);
    const float ms = (mb == -INFINITY) ? 0.0f : mb;
    const float c = (m == -INFINITY) ? 0.0f : exp2f(m - ms);  // rescales what the group has
    l *= c;
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] *= c;
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      const float w = exp2f(lv[k] - ms);  // 0 for a run that saw no key (and past n_split)
      l += w;
      const float uv[8] = {u[k][0].x, u[k][0].y, u[k][0].z, u[k][0].w, u[k][1].x, u[k][1].y, u[k][1].z, u[k][1].w};
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] += w * uv[q];
    }
    m = mb;
  }
  // combine the G groups (lanes LPR apart)
#pragma unroll
  for (int off = LPR; off < 64; off *= 2) {
    const float mo = __shfl_xor(m, off);
    const float lo = __shfl_xor(l, off);
    const float mn = fmaxf(m, mo);
    const float ms = (mn == -INFINITY) ? 0.0f : mn;
    const float a = (m == -INFINITY) ? 0.0f : exp2f(m - ms);
    const float b = (mo == -INFINITY) ? 0.0f : exp2f(mo - ms);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float ao = __shfl_xor(acc[q], off);
      acc[q] = acc[q] * a + ao * b;
    }
    l = l * a + lo * b;
    m = mn;
  }
  if (g != 0) return;
  const float inv = (l > 0.0f) ? 1.0f / l : 0.0f;
  // (rows are below 2^31: the launcher checks)
  const uint32_t r32 = (uint32_t)r, Bb32 = (uint32_t)p.Bb;
  const int32_t a = (int32_t)(r32 % Bb32);
  const uint32_t t = r32 / Bb32;
  const int32_t h = (int32_t)(t % (uint32_t)p.H);
  const int32_t b = (int32_t)((t / (uint32_t)p.H) % (uint32_t)p.B);
  const int32_t ri = (int32_t)(t / (uint32_t)p.H / (uint32_t)p.B);
  __bf16* orow = reinterpret_cast<__bf16*>(p.o.ptr) + ri * p.o.s_blk + b * p.o.s_batch + (int64_t)a * p.o.s_tok +
                 h * p.o.s_head;
  typedef __bf16 b16x8 __attribute__((ext_vector_type(8)));
  b16x8 w8;
#pragma unroll
  for (int q = 0; q < 8; ++q) w8[q] = (__bf16)(acc[q] * inv);
  *reinterpret_cast<b16x8*>(orow + e) = w8;
  if (e == 0) {
    const float ms = (m == -INFINITY) ? 0.0f : m;
    p.lse[r] = (l > 0.0f) ? (ms + log2f(l)) * 0.69314718055994530942f : -INFINITY;
  }
}

// Copies 16-byte chunks of one ring block of a strided sequence tensor into
// a dense [B][Bb][H][D] buffer (the stand-in for a ring receive).
__global__ __launch_bounds__(256) void gather_block_kernel(const char* src, int64_t s_blk,
                                                           int64_t s_batch, int64_t s_tok,
                                                           int64_t s_head, int32_t blk, char* dst,
                                                           int32_t B, int32_t H, int64_t Bb,
                                                           int32_t chunks, int32_t es) {
  const int64_t total = (int64_t)B * Bb * H * chunks;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int32_t c = (int32_t)(idx % chunks);
    int64_t r = idx / chunks;
    const int32_t h = (int32_t)(r % H);
    r /= H;
    const int64_t x = r % Bb;
    const int32_t b = (int32_t)(r / Bb);
    const int64_t off = ((int64_t)blk * s_blk + (int64_t)b * s_batch + x * s_tok + (int64_t)h * s_head) * es;
    *reinterpret_cast<u32x4*>(dst + idx * 16) = *reinterpret_cast<const u32x4*>(src + off + 16 * c);
  }
}

// Original order [B][L][H][D] <-> blocked [P][B][Bb][H][D] (pure data movement).
__global__ __launch_bounds__(256) void layout_copy_kernel(const char* src, char* dst, int32_t B,
                                                          int32_t H, int32_t P, int64_t Bb,
                                                          int32_t layout, int32_t inverse,
                                                          int32_t chunks) {
  const int64_t L = (int64_t)P * Bb;
  const int64_t total = (int64_t)P * B * Bb * H * chunks;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int32_t c = (int32_t)(idx % chunks);
    int64_t r = idx / chunks;
    const int32_t h = (int32_t)(r % H);
    r /= H;
    const int64_t x = r % Bb;
    r /= Bb;
    const int32_t b = (int32_t)(r % B);
    const int32_t s = (int32_t)(r / B);
    const int64_t t = token_position(layout, P, Bb, s, x);
    const int64_t orig = (((int64_t)b * L + t) * H + h) * chunks + c;
    if (inverse)
      reinterpret_cast<u32x4*>(dst)[orig] = reinterpret_cast<const u32x4*>(src)[idx];
    else
      reinterpret_cast<u32x4*>(dst)[idx] = reinterpret_cast<const u32x4*>(src)[orig];
  }
}

// D = rowsum(dO * O) per (rank, batch, head, row) ("Ring Attention 論文分析"
// (blog), section "逆伝播での KV 再循環"). Each lane handles 8 features; TPR =
// D/8 lanes share a row, and a lane group takes ROWS consecutive rows (8 for
// bf16, kept as raw words until the sums; 4 for fp32), all their loads
// issued before the sums so that enough bytes are in flight. A workgroup
// covers the rows of one (rank, batch, head) run that its lane groups take
// together, decoding the run once; lanes 0 .. ROWS-1 of a group then write
// D and lse * log2(e) of the group's rows side by side.
template <bool BF16>
constexpr int pre_rows() { return BF16 ? 8 : 4; }

template <int TPR, bool BF16>
__global__ __launch_bounds__(256) void bwd_preprocess_kernel(BwdParams p, int32_t xblocks) {
  constexpr int ROWS = pre_rows<BF16>();
  constexpr int PER_BLK = 256 / TPR * ROWS;
  constexpr int W = BF16 ? 1 : 2;  // 16-byte words per 8 features
  static_assert(ROWS <= TPR, "one writing lane per row");
  const int32_t run = (int32_t)(blockIdx.x / (uint32_t)xblocks);  // (ri * B + b) * H + h
  const int32_t xb = (int32_t)(blockIdx.x % (uint32_t)xblocks);
  const int32_t h = run % p.H;
  const int32_t b = (run / p.H) % p.B;
  const int32_t ri = run / (p.H * p.B);
  const int part = threadIdx.x % TPR;
  const int64_t x0 = (int64_t)xb * PER_BLK + (threadIdx.x / TPR) * ROWS;
  constexpr int ES = BF16 ? 2 : 4;  // element bytes
  const char* ob = reinterpret_cast<const char*>(p.o.ptr) +
                   ES * (ri * p.o.s_blk + b * p.o.s_batch + h * p.o.s_head + 8 * part);
  const char* db = reinterpret_cast<const char*>(p.dout.ptr) +
                   ES * (ri * p.dout.s_blk + b * p.dout.s_batch + h * p.dout.s_head + 8 * part);
  u32x4 ow[ROWS][W], dw[ROWS][W];
#pragma unroll
  for (int k = 0; k < ROWS; ++k) {
    const int64_t x = x0 + k < p.Bb ? x0 + k : p.Bb - 1;  // a valid row; not written
#pragma unroll
    for (int w = 0; w < W; ++w) {
      ow[k][w] = *reinterpret_cast<const u32x4*>(ob + ES * x * p.o.s_tok + 16 * w);
      dw[k][w] = *reinterpret_cast<const u32x4*>(db + ES * x * p.dout.s_tok + 16 * w);
    }
  }
  float mine = 0.0f;  // D of row x0 + part (lanes part < ROWS)
#pragma unroll
  for (int k = 0; k < ROWS; ++k) {
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (BF16) {
          acc = fmaf(__uint_as_float(ow[k][w][q] << 16), __uint_as_float(dw[k][w][q] << 16), acc);
          acc = fmaf(__uint_as_float(ow[k][w][q] & 0xFFFF0000u), __uint_as_float(dw[k][w][q] & 0xFFFF0000u), acc);
        } else {
          acc = fmaf(__uint_as_float(ow[k][w][q]), __uint_as_float(dw[k][w][q]), acc);
        }
      }
#pragma unroll
    for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (part == k) mine = acc;
  }
  const int64_t x = x0 + part;
  if (part < ROWS && x < p.Bb) {
    const int64_t row = (int64_t)run * p.Bb + x;
    p.dsum[row] = mine;
    p.lse2[row] = p.lse[row] * 1.44269504088896340736f;  // log2(e): the walks use exp2
  }
}

inline uint32_t grid_for(int64_t items, int32_t per_block) {
  int64_t g = (items + per_block - 1) / per_block;
  if (g > 1048576) g = 1048576;  // grid-stride beyond this
  if (g < 1) g = 1;
  return (uint32_t)g;
}

}  // namespace

hipError_t launch_merge_lse(int64_t rows, int32_t d, const float* oa, const float* la,
                            const float* ob, const float* lb, float* oo, float* lo,
                            hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (d == 128 || d == 64) {
    // 16-byte aligned rows (the C ABI checks the O pointers for d % 4 == 0)
    const int64_t per_block = (256 / (d / 4)) * kMergeRows;
    const int64_t grid = (rows + per_block - 1) / per_block;
    if (d == 128)
      hipLaunchKernelGGL(merge_lse_vec_kernel<128>, dim3((uint32_t)grid), dim3(256), 0, s, rows, oa, la, ob, lb, oo, lo);
    else
      hipLaunchKernelGGL(merge_lse_vec_kernel<64>, dim3((uint32_t)grid), dim3(256), 0, s, rows, oa, la, ob, lb, oo, lo);
    return hipGetLastError();
  }
  const int64_t grid = (rows + 3) / 4;
  hipLaunchKernelGGL(merge_lse_kernel, dim3((uint32_t)grid), dim3(256), 0, s, rows, d, oa, la, ob, lb, oo, lo);
  return hipGetLastError();
}

hipError_t launch_merge_splits(const FwdParams& p, hipStream_t s) {
  const int64_t rows = (int64_t)p.n_ranks * p.B * p.H * p.Bb;
  if (rows <= 0) return hipSuccess;
  if (rows >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  // a wave per row; few rows (a short query block) get a workgroup each, so
  // that they spread over every CU
  if (rows <= 4096) {
    if (p.D == 128)
      hipLaunchKernelGGL((merge_splits_kernel<128, 1>), dim3((uint32_t)rows), dim3(64), 0, s, p);
    else
      hipLaunchKernelGGL((merge_splits_kernel<64, 1>), dim3((uint32_t)rows), dim3(64), 0, s, p);
    return hipGetLastError();
  }
  const int64_t grid = (rows + 3) / 4;
  if (p.D == 128)
    hipLaunchKernelGGL((merge_splits_kernel<128, 4>), dim3((uint32_t)grid), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((merge_splits_kernel<64, 4>), dim3((uint32_t)grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_gather_block(const Seq& src, int32_t blk, void* dst, int32_t B, int32_t H,
                               int32_t D, int64_t Bb, int32_t es, hipStream_t s) {
  const int32_t chunks = D * es / 16;
  const int64_t total = (int64_t)B * Bb * H * chunks;
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_block_kernel, dim3(grid_for(total, 256)), dim3(256), 0, s,
                     reinterpret_cast<const char*>(src.ptr), src.s_blk, src.s_batch, src.s_tok,
                     src.s_head, blk, reinterpret_cast<char*>(dst), B, H, Bb, chunks, es);
  return hipGetLastError();
}

hipError_t launch_layout_copy(const void* src, void* dst, int32_t B, int32_t H, int32_t D,
                              int32_t P, int64_t Bb, int32_t layout, int32_t inverse, int32_t es,
                              hipStream_t s) {
  const int32_t chunks = D * es / 16;
  const int64_t total = (int64_t)P * B * Bb * H * chunks;
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL(layout_copy_kernel, dim3(grid_for(total, 256)), dim3(256), 0, s,
                     reinterpret_cast<const char*>(src), reinterpret_cast<char*>(dst), B, H, P, Bb,
                     layout, inverse, chunks);
  return hipGetLastError();
}

hipError_t launch_bwd_preprocess(const BwdParams& p, int32_t bf16, hipStream_t s) {
  const int64_t rows = (int64_t)p.n_ranks * p.B * p.H * p.Bb;
  if (rows <= 0) return hipSuccess;
  const int32_t tpr = p.D / 8;  // 16 or 8 (head_dim 128 or 64)
  const int64_t per_blk = 256 / tpr * (bf16 ? pre_rows<true>() : pre_rows<false>());
  const int64_t xblocks = (p.Bb + per_blk - 1) / per_blk;
  const int64_t grid = (int64_t)p.n_ranks * p.B * p.H * xblocks;
  if (grid > 0xFFFFFFFFLL) return hipErrorInvalidValue;
  const dim3 g((uint32_t)grid), t(256);
  const int32_t xbl = (int32_t)xblocks;
  if (tpr == 16 && bf16) hipLaunchKernelGGL((bwd_preprocess_kernel<16, true>), g, t, 0, s, p, xbl);
  else if (tpr == 16) hipLaunchKernelGGL((bwd_preprocess_kernel<16, false>), g, t, 0, s, p, xbl);
  else if (bf16) hipLaunchKernelGGL((bwd_preprocess_kernel<8, true>), g, t, 0, s, p, xbl);
  else hipLaunchKernelGGL((bwd_preprocess_kernel<8, false>), g, t, 0, s, p, xbl);
  return hipGetLastError();
}

}  // namespace ra
