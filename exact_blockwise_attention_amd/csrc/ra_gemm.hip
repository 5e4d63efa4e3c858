// ra_gemm.hip — the dense layers around attention in a Blockwise Parallel
// Transformer layer ("Ring Attention 論文分析" (blog), section "BPT の
// Feedforward 融合"): the Q/K/V and output projections and the feedforward
// network as one bf16 matrix-product kernel with a fused epilogue, and the
// row layer normalisation.
//
// gemm_bf16_kernel: C[m][n] = epilogue(sum_k A[m][k] W[n][k]) for A [M][K]
// (rows at stride lda) and W [N][K] (the [out][in] weight of a linear layer),
// bf16 with fp32 accumulation on v_mfma_f32_32x32x16_bf16. The epilogue adds
// bias[n], then residual[m][n] (bf16), then applies the exact GELU, and stores
// fp32 or bf16 (rounded to nearest even).
//
// Tiling: a workgroup owns a 256 x 128 tile of C; its 8 waves each own 64 x 64
// (2 x 2 MFMA tiles). K advances 64 at a time through three LDS stages (a
// 256 x 64 A tile and a 128 x 64 W tile each, 48 KB), copied straight from
// global memory into LDS two steps ahead of their use. LDS rows are 128
// bytes; the 16-byte chunk c of row r sits at c ^ ((r >> 1) & 7), so that the
// 16 lanes of a read phase, on 16 consecutive rows at one chunk, hit all 64
// banks once.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ra_internal.h"
#include "ra_kvwalk.h"
#include "ra_lds.h"

namespace ra {
namespace {

constexpr int kBM = 256, kBN = 128, kBK = 64;
constexpr int kGWaves = 8;
constexpr int kGThreads = 64 * kGWaves;
constexpr int kNSt = 3;
constexpr int kATileB = kBM * kBK * 2;             // 32 KB
constexpr int kWTileB = kBN * kBK * 2;             // 16 KB
constexpr int kStageB = kATileB + kWTileB;         // 48 KB
constexpr int kGemmLds = kNSt * kStageB;           // 144 KB
constexpr int kACopies = kATileB / 1024 / kGWaves;  // 1 KB copies per wave per stage
constexpr int kWCopies = kWTileB / 1024 / kGWaves;
constexpr int kGNI = kACopies + kWCopies;

__device__ __forceinline__ int gswz(int r) { return (r >> 1) & 7; }

__global__ __launch_bounds__(kGThreads, 1) void gemm_bf16_kernel(GemmParams p) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64;
  const int n = lane % 32, hf = lane / 32;
  const int wm = wave % 4, wn = wave / 4;

  // tile order: consecutive workgroups (one XCD) share a row band of A and
  // walk the W column tiles, so a band is read from HBM about once
  const int32_t ntn = p.N / kBN;
  const int64_t ntm = (p.M + kBM - 1) / kBM;
  const int64_t lw = xcd_logical(blockIdx.x, ntm * ntn);
  const int64_t m0 = (lw / ntn) * kBM;
  const int32_t n0 = (int32_t)(lw % ntn) * kBN;

  // per-lane global sources of this wave's copies (row pointers; the logical
  // chunk that belongs at the lane's physical LDS position), rows past M read
  // row M - 1
  const __bf16* asrc[kACopies];
  const __bf16* wsrc[kWCopies];
#pragma unroll
  for (int c = 0; c < kACopies; ++c) {
    const int row = (wave + kGWaves * c) * 8 + lane / 8;
    int64_t gr = m0 + row;
    if (gr > p.M - 1) gr = p.M - 1;
    asrc[c] = p.a + gr * p.lda + 8 * ((lane % 8) ^ gswz(row));
  }
#pragma unroll
  for (int c = 0; c < kWCopies; ++c) {
    const int row = (wave + kGWaves * c) * 8 + lane / 8;
    wsrc[c] = p.w + (int64_t)(n0 + row) * p.ldw + 8 * ((lane % 8) ^ gswz(row));
  }
  auto copy = [&](int kt, int st) __attribute__((always_inline)) {
    unsigned char* sa = smem_raw + st * kStageB;
    unsigned char* sw = sa + kATileB;
#pragma unroll
    for (int c = 0; c < kACopies; ++c)
      __builtin_amdgcn_global_load_lds(asrc[c] + kt * kBK,
                                       (__attribute__((address_space(3))) void*)(sa + (wave + kGWaves * c) * 1024), 16, 0, 0);
#pragma unroll
    for (int c = 0; c < kWCopies; ++c)
      __builtin_amdgcn_global_load_lds(wsrc[c] + kt * kBK,
                                       (__attribute__((address_space(3))) void*)(sw + (wave + kGWaves * c) * 1024), 16, 0, 0);
  };

  // LDS byte addresses of this lane's operand reads in stage 0 for k-step ks:
  // A row 64wm + n (+32 for the second row tile), W row 64wn + n (+32),
  // logical chunk 2ks + hf
  uint32_t ra_[4], rw_[4];
  const uint32_t base = lds_addr(smem_raw);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int ar = 64 * wm + n, wr = 64 * wn + n;
    ra_[ks] = base + ar * 128 + 16 * ((2 * ks + hf) ^ gswz(ar));
    rw_[ks] = base + kATileB + wr * 128 + 16 * ((2 * ks + hf) ^ gswz(wr));
  }

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int32_t nk = p.K / kBK;
  copy(0, 0);
  if (nk > 1) copy(1, 1);
  for (int32_t kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) wait_vm<kGNI>();  // step kt has landed; kt + 1 may still be in flight
    else wait_vm<0>();
    wg_barrier();  // every wave's part of step kt is in LDS; stage (kt + 2) % 3 is free
    if (kt + 2 < nk) copy(kt + 2, (kt + 2) % kNSt);
    const uint32_t so = (uint32_t)((kt % kNSt) * kStageB);
    u32x4 fr[2][4];  // [slot][A0, A1, W0, W1]
    auto rd = [&](u32x4(&r)[4], int ks) __attribute__((always_inline)) {
      r[0] = lds_read16<0>(ra_[ks] + so);
      r[1] = lds_read16<32 * 128>(ra_[ks] + so);
      r[2] = lds_read16<0>(rw_[ks] + so);
      r[3] = lds_read16<32 * 128>(rw_[ks] + so);
    };
    rd(fr[0], 0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks + 1 < 4) {
        rd(fr[(ks + 1) & 1], ks + 1);
        lds_wait<4>(fr[ks & 1]);
      } else {
        lds_wait<0>(fr[ks & 1]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = mfma32(__builtin_bit_cast(bf16x8, fr[ks & 1][i]), __builtin_bit_cast(bf16x8, fr[ks & 1][2 + j]),
                             acc[i][j]);
    }
  }

  // epilogue: lane (hf, n) of tile (i, j) holds rows 8(e/4) + 4hf + e%4 of
  // column n
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int32_t col = n0 + 64 * wn + 32 * j + n;
    const float bj = p.bias ? p.bias[col] : 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + 64 * wm + 32 * i + 8 * (e / 4) + 4 * hf + (e % 4);
        if (row >= p.M) continue;
        float v = acc[i][j][e] + bj;
        if (p.res) v += (float)p.res[row * p.ldr + col];
        if (p.gelu) v = 0.5f * v * (1.0f + erff(v * 0.70710678118654752f));
        if (p.out_f32)
          reinterpret_cast<float*>(p.out)[row * p.ldo + col] = v;
        else
          reinterpret_cast<__bf16*>(p.out)[row * p.ldo + col] = (__bf16)v;
      }
  }
}

// Row layer normalisation of fp32 rows: (z - mean) / sqrt(var + eps) *
// gamma + beta with the biased variance, to bf16. One workgroup per row; the
// row stays in registers between the mean and the variance pass.
constexpr int kLnThreads = 256;
constexpr int kLnMaxPer = 32;  // elements per thread: d up to 8192

__device__ __forceinline__ float block_sum(float v, float* red) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  const int w = threadIdx.x / 64;
  __syncthreads();
  if (threadIdx.x % 64 == 0) red[w] = v;
  __syncthreads();
  float t = 0.0f;
#pragma unroll
  for (int i = 0; i < kLnThreads / 64; ++i) t += red[i];
  return t;
}

__global__ __launch_bounds__(kLnThreads) void layer_norm_kernel(const float* in, int64_t rows, int32_t d,
                                                                 const float* gamma, const float* beta, float eps,
                                                                 __bf16* out) {
  __shared__ float red[kLnThreads / 64];
  const int64_t row = blockIdx.x;
  if (row >= rows) return;
  const float* z = in + row * d;
  float v[kLnMaxPer];
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kLnMaxPer; ++i) {
    const int c = threadIdx.x + kLnThreads * i;
    v[i] = (c < d) ? z[c] : 0.0f;
    s += v[i];
  }
  const float mean = block_sum(s, red) / (float)d;
  float q = 0.0f;
#pragma unroll
  for (int i = 0; i < kLnMaxPer; ++i) {
    const int c = threadIdx.x + kLnThreads * i;
    const float t = (c < d) ? v[i] - mean : 0.0f;
    q = fmaf(t, t, q);
  }
  const float inv = 1.0f / sqrtf(block_sum(q, red) / (float)d + eps);
#pragma unroll
  for (int i = 0; i < kLnMaxPer; ++i) {
    const int c = threadIdx.x + kLnThreads * i;
    if (c < d) out[row * d + c] = (__bf16)((v[i] - mean) * inv * gamma[c] + beta[c]);
  }
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmParams& p, hipStream_t s) {
  const int64_t grid = ((p.M + kBM - 1) / kBM) * (p.N / kBN);
  if (grid <= 0) return hipSuccess;
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_bf16_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kGemmLds);
  hipLaunchKernelGGL(gemm_bf16_kernel, dim3((uint32_t)grid), dim3(kGThreads), kGemmLds, s, p);
  return hipGetLastError();
}

hipError_t launch_layer_norm(const float* in, int64_t rows, int32_t d, const float* gamma, const float* beta,
                             float eps, __bf16* out, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(layer_norm_kernel, dim3((uint32_t)rows), dim3(kLnThreads), 0, s, in, rows, d, gamma, beta,
                     eps, out);
  return hipGetLastError();
}

}  // namespace ra
