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
// Tiling: a workgroup owns a 256 x BN tile of C (BN = 256 when N allows,
// else 128); its 8 waves each own 64 x BN/2 (2 x BN/64 MFMA tiles). K advances
// 64 at a time through LDS stages of a 256 x 64 A tile and a BN x 64 W tile
// (two stages of 64 KB for BN = 256, three of 48 KB for BN = 128), copied
// straight from global memory into LDS ahead of their use. LDS rows are 128
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

constexpr int kBM = 256, kBK = 64;
constexpr int kGWaves = 8;
constexpr int kGThreads = 64 * kGWaves;
constexpr int kATileB = kBM * kBK * 2;  // 32 KB

template <int BN>
struct GemmCfg {
  static constexpr int NST = BN == 256 ? 2 : 3;
  static constexpr int WTILE_B = BN * kBK * 2;
  static constexpr int STAGE_B = kATileB + WTILE_B;
  static constexpr int LDS = NST * STAGE_B;
  static constexpr int ACOPIES = kATileB / 1024 / kGWaves;  // 1 KB copies per wave per stage
  static constexpr int WCOPIES = WTILE_B / 1024 / kGWaves;
  static constexpr int NI = ACOPIES + WCOPIES;
  static constexpr int NT = BN / 64;  // MFMA column tiles per wave
  static_assert(LDS <= 160 * 1024, "LDS");
};

__device__ __forceinline__ int gswz(int r) { return (r >> 1) & 7; }

// One K step's copies of this wave into the stage at `stage`: 1 KB (8 rows of
// 64 elements) per copy, A rows first, then W rows behind the A tile.
template <int AC, int WC>
__device__ __forceinline__ void copy_stage(const __bf16* const (&asrc)[AC], const __bf16* const (&wsrc)[WC], int32_t k0,
                                           unsigned char* stage, int wave) {
#pragma unroll
  for (int c = 0; c < AC; ++c)
    __builtin_amdgcn_global_load_lds(asrc[c] + k0, (__attribute__((address_space(3))) void*)(stage + (wave + kGWaves * c) * 1024),
                                     16, 0, 0);
#pragma unroll
  for (int c = 0; c < WC; ++c)
    __builtin_amdgcn_global_load_lds(wsrc[c] + k0,
                                     (__attribute__((address_space(3))) void*)(stage + kATileB + (wave + kGWaves * c) * 1024),
                                     16, 0, 0);
}

template <int BN>
__global__ __launch_bounds__(kGThreads, 1) void gemm_bf16_kernel(GemmParams p) {
  using C = GemmCfg<BN>;
  constexpr int kBN = BN;
  constexpr int kNSt = C::NST;
  constexpr int kStageB = C::STAGE_B;
  constexpr int kACopies = C::ACOPIES;
  constexpr int kWCopies = C::WCOPIES;
  constexpr int kGNI = C::NI;
  constexpr int NT = C::NT;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64;
  const int n = lane % 32, hf = lane / 32;
  const int wm = wave % 4, wn = wave / 4;

  // tile order: consecutive workgroups (one XCD) share a row band of A and
  // walk the W column tiles, so a band is read from HBM about once
  const int32_t ntn = (p.N + kBN - 1) / kBN;
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
    int32_t gr = n0 + row;
    if (gr > p.N - 1) gr = p.N - 1;  // a ragged last column tile reads a valid row
    wsrc[c] = p.w + (int64_t)gr * p.ldw + 8 * ((lane % 8) ^ gswz(row));
  }
  // the copy builtin sits in a function: written directly in a lambda of a
  // kernel template, it makes the host compilation drop the launch stub
  auto copy = [&](int kt, int st) __attribute__((always_inline)) {
    copy_stage<kACopies, kWCopies>(asrc, wsrc, kt * kBK, smem_raw + st * kStageB, wave);
  };

  // LDS byte addresses of this lane's operand reads in stage 0 for k-step ks:
  // A row 64wm + n (+32 for the second row tile), W row (BN/2) wn + n (+32j),
  // logical chunk 2ks + hf (rows 32 apart share the swizzle)
  uint32_t ra_[4], rw_[4];
  const uint32_t base = lds_addr(smem_raw);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int ar = 64 * wm + n, wr = (kBN / 2) * wn + n;
    ra_[ks] = base + ar * 128 + 16 * ((2 * ks + hf) ^ gswz(ar));
    rw_[ks] = base + kATileB + wr * 128 + 16 * ((2 * ks + hf) ^ gswz(wr));
  }

  f32x16 acc[2][NT];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x16{};

  // copies run DIST = NST - 1 steps ahead of the compute
  constexpr int DIST = kNSt - 1;
  const int32_t nk = p.K / kBK;
#pragma unroll
  for (int d = 0; d < DIST; ++d)
    if (d < nk) copy(d, d);
  for (int32_t kt = 0; kt < nk; ++kt) {
    // step kt has landed; the copies of steps kt+1 .. kt+DIST-1 may stay in flight
    if (DIST > 1 && kt + DIST - 1 < nk) wait_vm<(DIST - 1) * kGNI>();
    else wait_vm<0>();
    wg_barrier();  // every wave's part of step kt is in LDS; the stage of step kt-1 is free
    if (kt + DIST < nk) copy(kt + DIST, (kt + DIST) % kNSt);
    const uint32_t so = (uint32_t)((kt % kNSt) * kStageB);
    u32x4 fr[2][2 + NT];  // [slot][A0, A1, W0 .. W(NT-1)]
    auto rd = [&](u32x4(&r)[2 + NT], int ks) __attribute__((always_inline)) {
      const uint32_t a = ra_[ks] + so, w = rw_[ks] + so;
      r[0] = lds_read16<0>(a);
      r[1] = lds_read16<32 * 128>(a);
      r[2] = lds_read16<0>(w);
      r[3] = lds_read16<32 * 128>(w);
      if constexpr (NT == 4) {
        r[4] = lds_read16<64 * 128>(w);
        r[5] = lds_read16<96 * 128>(w);
      }
    };
    rd(fr[0], 0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks + 1 < 4) {
        rd(fr[(ks + 1) & 1], ks + 1);
        lds_wait<2 + NT>(fr[ks & 1]);
      } else {
        lds_wait<0>(fr[ks & 1]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
          acc[i][j] = mfma32(__builtin_bit_cast(bf16x8, fr[ks & 1][i]), __builtin_bit_cast(bf16x8, fr[ks & 1][2 + j]),
                             acc[i][j]);
    }
  }

  // epilogue: lane (hf, n) of tile (i, j) holds rows 8(e/4) + 4hf + e%4 of
  // column n
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int32_t col = n0 + (kBN / 2) * wn + 32 * j + n;
    if (col >= p.N) continue;
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
  const bool wide = p.N % 256 == 0;
  const int bn = wide ? 256 : 128;
  const int64_t grid = ((p.M + kBM - 1) / kBM) * ((p.N + bn - 1) / bn);
  if (grid <= 0) return hipSuccess;
  if (wide) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_bf16_kernel<256>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, GemmCfg<256>::LDS);
    hipLaunchKernelGGL(gemm_bf16_kernel<256>, dim3((uint32_t)grid), dim3(kGThreads), GemmCfg<256>::LDS, s, p);
  } else {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_bf16_kernel<128>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, GemmCfg<128>::LDS);
    hipLaunchKernelGGL(gemm_bf16_kernel<128>, dim3((uint32_t)grid), dim3(kGThreads), GemmCfg<128>::LDS, s, p);
  }
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
