// ra_bwd.hip — backward kernels of exact blockwise ring attention (gfx950).
//
// "Ring Attention 論文分析" (blog), section "逆伝播での KV 再循環": the
// backward walks the same ring, recomputes the probabilities from the saved
// log-sum-exp, P = exp(S - lse), and forms dV = P^T dO, dP = dO V^T,
// dS = P * (dP - D) with D = rowsum(dO * O), dQ = scale * dS K and
// dK = scale * dS^T Q; the dK/dV partials belong to the KV block's owner.
//
// Here one workgroup owns a tile of keys of KV block j for one (batch, head)
// and carries its dK/dV accumulators on chip while the block travels the
// ring: at step k it meets the query block of rank (j + k) mod P. Query
// tiles the causal/striped mask hides from every key of the tile are
// skipped. dQ of the met query rows is accumulated with fp32 atomics in a
// workspace and scaled/cast once at the end.
//
// bf16 path, per wave (32 keys of the tile's 128): K and V of the wave's keys
// live in registers as MFMA B operands; S = Q K^T and dP = dO V^T come out
// with lane (h, n) holding key n against 16 query rows, which is the operand
// layout the dV^T += dO^T P and dK^T += Q^T dS products need (contraction
// over query rows, whose order inside an MFMA is free). dS goes through LDS
// once, row-major, for dQ = dS K with K^T staged in LDS.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ra_internal.h"
#include "ra_schedule.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kKn = 128;  // keys per workgroup (32 per wave)
constexpr int kQm = 64;   // query rows per visited tile
constexpr int kBandAll = 1 << 30;
constexpr float kLog2e = 1.44269504088896340736f;

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int D>
struct BwdLds {
  static constexpr int RS = D + 8;     // [rows][D] row stride
  static constexpr int TS = kQm + 4;   // [D][64 rows] transposed stride
  static constexpr int KTS = kKn + 8;  // K^T [D][128 keys] stride
  static constexpr int DSS = kKn + 8;  // dS [64 rows][128 keys] stride
  static constexpr int Q_ROW = 0;
  static constexpr int DO_ROW = Q_ROW + kQm * RS;
  static constexpr int Q_T = DO_ROW + kQm * RS;
  static constexpr int DO_T = Q_T + D * TS;
  static constexpr int K_T = DO_T + D * TS;
  static constexpr int DS = K_T + D * KTS;
  static constexpr int BF16_ELEMS = DS + kQm * DSS;
  static constexpr int F32_OFF = (BF16_ELEMS * 2 + 15) / 16 * 16;  // bytes
  static constexpr int BYTES = F32_OFF + 2 * kQm * 4;
};

// Rows [r_lo, r_lo + ROWS) of a [rows][D] strided tensor into LDS, row-major.
template <int D, int ROWS>
__device__ __forceinline__ void stage_rows(__bf16* dst, int stride, const __bf16* base, int64_t s_tok,
                                           int64_t r_lo, int64_t nrows, int tid) {
  constexpr int CR = D / 8;
  constexpr int RPP = kThreads / CR;
  const int c = tid % CR;
  const int r0 = tid / CR;
#pragma unroll
  for (int p = 0; p < ROWS / RPP; ++p) {
    const int r = r0 + RPP * p;
    const int64_t x = r_lo + r;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (x < nrows) val = *reinterpret_cast<const u32x4*>(base + x * s_tok + 8 * c);
    *reinterpret_cast<u32x4*>(dst + r * stride + 8 * c) = val;
  }
}

// Same rows transposed: dst[e][r] (feature-major), written as 8-byte chunks.
template <int D, int ROWS>
__device__ __forceinline__ void stage_transposed(__bf16* dst, int stride, const __bf16* base,
                                                 int64_t s_tok, int64_t r_lo, int64_t nrows, int tid) {
  constexpr int NP = D / 2;
  constexpr int NG = kThreads / NP;
  constexpr int KG = ROWS / NG;
  const int pr = tid % NP;
  const int g = tid / NP;
  uint32_t w[KG];
#pragma unroll
  for (int q = 0; q < KG; ++q) {
    const int64_t x = r_lo + KG * g + q;
    w[q] = (x < nrows) ? *reinterpret_cast<const uint32_t*>(base + x * s_tok + 2 * pr) : 0u;
  }
  __bf16* even = dst + (2 * pr) * stride + KG * g;
  __bf16* odd = even + stride;
#pragma unroll
  for (int q = 0; q < KG; q += 4) {
    u32x2 e, o;
    e[0] = (w[q] & 0xFFFFu) | (w[q + 1] << 16);
    e[1] = (w[q + 2] & 0xFFFFu) | (w[q + 3] << 16);
    o[0] = (w[q] >> 16) | (w[q + 1] & 0xFFFF0000u);
    o[1] = (w[q + 2] >> 16) | (w[q + 3] & 0xFFFF0000u);
    *reinterpret_cast<u32x2*>(even + q) = e;
    *reinterpret_cast<u32x2*>(odd + q) = o;
  }
}

// Heaviest KV tiles first: early keys are seen by more query rows.
__device__ __forceinline__ void kv_tile_of(const BwdParams& p, int64_t ord, int32_t tiles, int32_t* j,
                                           int32_t* tile) {
  if (p.causal && p.layout == kContiguous) {
    *j = (int32_t)(ord / tiles);
    *tile = (int32_t)(ord % tiles);
  } else {
    *tile = (int32_t)(ord / p.P);
    *j = (int32_t)(ord % p.P);
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void bwd_bf16_kernel(BwdParams p) {
  using L = BwdLds<D>;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __bf16* lds = reinterpret_cast<__bf16*>(smem_raw);
  float* lse_s = reinterpret_cast<float*>(smem_raw + L::F32_OFF);
  float* dsum_s = lse_s + kQm;

  const int tid = threadIdx.x;
  const int wave = tid / 64;
  const int lane = tid % 64;
  const int n = lane % 32;
  const int hf = lane / 32;

  const int32_t BH = p.B * p.H;
  const int32_t tiles = (int32_t)((p.Bb + kKn - 1) / kKn);
  const int64_t id = blockIdx.x;
  const int32_t bh = (int32_t)(id % BH);
  const int32_t b = bh / p.H;
  const int32_t h = bh % p.H;
  int32_t j, tile;
  kv_tile_of(p, id / BH, tiles, &j, &tile);
  const int64_t kv0 = (int64_t)tile * kKn;
  const int64_t kw = kv0 + 32 * wave;  // the wave's first key
  const int64_t key = kw + n;          // this lane's key

  const __bf16* kbase = reinterpret_cast<const __bf16*>(p.k.ptr) + j * p.k.s_blk + b * p.k.s_batch +
                        h * p.k.s_head;
  const __bf16* vbase = reinterpret_cast<const __bf16*>(p.v.ptr) + j * p.v.s_blk + b * p.v.s_batch +
                        h * p.v.s_head;
  bf16x8 kreg[D / 16], vreg[D / 16];
#pragma unroll
  for (int ss = 0; ss < D / 16; ++ss) {
    u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
    if (key < p.Bb) {
      kv = *reinterpret_cast<const u32x4*>(kbase + key * p.k.s_tok + 16 * ss + 8 * hf);
      vv = *reinterpret_cast<const u32x4*>(vbase + key * p.v.s_tok + 16 * ss + 8 * hf);
    }
    kreg[ss] = __builtin_bit_cast(bf16x8, kv);
    vreg[ss] = __builtin_bit_cast(bf16x8, vv);
  }
  stage_transposed<D, kKn>(lds + L::K_T, L::KTS, kbase, p.k.s_tok, kv0, p.Bb, tid);

  f32x16 dk[D / 32], dv[D / 32];  // dK^T, dV^T: [dt][i] = feature 32dt + 8(i/4) + 4hf + i%4
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    f32x16 z = {};
    dk[dt] = z;
    dv[dt] = z;
  }
  const float c2 = p.scale_log2;
  const int32_t qtiles = (int32_t)((p.Bb + kQm - 1) / kQm);

  for (int32_t kstep = 0; kstep < p.P; ++kstep) {
    const int32_t i = ring_rank(j, kstep, p.P);
    if (i < p.rank_begin || i >= p.rank_begin + p.n_ranks) continue;
    const int32_t ri = i - p.rank_begin;
    const BlockRel rel = block_relation(p.layout, p.causal, i, j);
    if (rel.kind == kNone) continue;
    const int32_t band = (rel.kind == kAll) ? kBandAll : rel.band;
    // first query row any key of the tile can see: a >= kv0 - band
    int64_t a_first = (rel.kind == kAll) ? 0 : kv0 - band;
    if (a_first < 0) a_first = 0;
    const int32_t qt0 = (int32_t)(a_first / kQm);
    const __bf16* qbase = reinterpret_cast<const __bf16*>(p.q.ptr) + ri * p.q.s_blk + b * p.q.s_batch +
                          h * p.q.s_head;
    const __bf16* dobase = reinterpret_cast<const __bf16*>(p.dout.ptr) + ri * p.dout.s_blk +
                           b * p.dout.s_batch + h * p.dout.s_head;
    const int64_t srow = (((int64_t)ri * p.B + b) * p.H + h) * p.Bb;
    for (int32_t qt = qt0; qt < qtiles; ++qt) {
      const int64_t q0 = (int64_t)qt * kQm;
      __syncthreads();  // previous tile's LDS reads are done
      stage_rows<D, kQm>(lds + L::Q_ROW, L::RS, qbase, p.q.s_tok, q0, p.Bb, tid);
      stage_rows<D, kQm>(lds + L::DO_ROW, L::RS, dobase, p.dout.s_tok, q0, p.Bb, tid);
      stage_transposed<D, kQm>(lds + L::Q_T, L::TS, qbase, p.q.s_tok, q0, p.Bb, tid);
      stage_transposed<D, kQm>(lds + L::DO_T, L::TS, dobase, p.dout.s_tok, q0, p.Bb, tid);
      if (tid < kQm) {
        const int64_t a = q0 + tid;
        lse_s[tid] = (a < p.Bb) ? p.lse[srow + a] * kLog2e : 0.0f;
        dsum_s[tid] = (a < p.Bb) ? p.dsum[srow + a] : 0.0f;
      }
      __syncthreads();

      const bool wave_dead = (kw >= p.Bb) || (kw - (q0 + kQm - 1) > (int64_t)band);
      const bool need_mask = (kw + 31 - q0 > (int64_t)band) || (q0 + kQm > p.Bb) || (kw + 32 > p.Bb);
      __bf16* ds_s = lds + L::DS;
      if (wave_dead) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i4 = 0; i4 < 16; ++i4) {
            const int qr = 32 * mt + 8 * (i4 / 4) + 4 * hf + (i4 % 4);
            ds_s[qr * L::DSS + 32 * wave + n] = (__bf16)0.0f;
          }
      } else {
        f32x16 s[2], dp[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          f32x16 z = {};
          s[mt] = z;
          dp[mt] = z;
#pragma unroll
          for (int ss = 0; ss < D / 16; ++ss) {
            const bf16x8 qa = *reinterpret_cast<const bf16x8*>(lds + L::Q_ROW + (32 * mt + n) * L::RS + 16 * ss + 8 * hf);
            const bf16x8 oa = *reinterpret_cast<const bf16x8*>(lds + L::DO_ROW + (32 * mt + n) * L::RS + 16 * ss + 8 * hf);
            s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kreg[ss], s[mt], 0, 0, 0);
            dp[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, vreg[ss], dp[mt], 0, 0, 0);
          }
        }
        bf16x8 pb[4], dsb[4];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int qr0 = 32 * mt + 8 * g4 + 4 * hf;
            const float4 l4 = *reinterpret_cast<const float4*>(lse_s + qr0);
            const float4 d4 = *reinterpret_cast<const float4*>(dsum_s + qr0);
            const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
            const float dvv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int i4 = 4 * g4 + e;
              float pv = fexp2(fmaf(s[mt][i4], c2, -lv[e]));
              if (need_mask) {
                const int64_t a = q0 + qr0 + e;
                if (key - a > (int64_t)band || a >= p.Bb || key >= p.Bb) pv = 0.0f;
              }
              const float dsv = pv * (dp[mt][i4] - dvv[e]);
              pb[2 * mt + i4 / 8][i4 % 8] = (__bf16)pv;
              const __bf16 dsh = (__bf16)dsv;
              dsb[2 * mt + i4 / 8][i4 % 8] = dsh;
              ds_s[(qr0 + e) * L::DSS + 32 * wave + n] = dsh;
            }
          }
        // dV^T += dO^T P, dK^T += Q^T dS (contraction over the 64 query rows)
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int kq = 0; kq < 4; ++kq) {
            const __bf16* orow = lds + L::DO_T + (32 * dt + n) * L::TS + 16 * kq + 4 * hf;
            const __bf16* qrow = lds + L::Q_T + (32 * dt + n) * L::TS + 16 * kq + 4 * hf;
            const bf16x8 ot = __builtin_shufflevector(*reinterpret_cast<const bf16x4*>(orow),
                                                      *reinterpret_cast<const bf16x4*>(orow + 8), 0, 1, 2,
                                                      3, 4, 5, 6, 7);
            const bf16x8 qtv = __builtin_shufflevector(*reinterpret_cast<const bf16x4*>(qrow),
                                                       *reinterpret_cast<const bf16x4*>(qrow + 8), 0, 1, 2,
                                                       3, 4, 5, 6, 7);
            dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ot, pb[kq], dv[dt], 0, 0, 0);
            dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qtv, dsb[kq], dk[dt], 0, 0, 0);
          }
      }
      __syncthreads();  // dS of all 128 keys is in LDS

      // dQ[q][d] += sum over the tile's keys dS[q][key] K[key][d]
      constexpr int NT = 2 * (D / 32);  // 32x32 output tiles
      constexpr int PER_WAVE = NT / 4;
#pragma unroll
      for (int u = 0; u < PER_WAVE; ++u) {
        const int t = wave * PER_WAVE + u;
        const int mt = t / (D / 32);
        const int dt = t % (D / 32);
        f32x16 acc = {};
#pragma unroll
        for (int kk = 0; kk < kKn / 16; ++kk) {
          const bf16x8 da = *reinterpret_cast<const bf16x8*>(ds_s + (32 * mt + n) * L::DSS + 16 * kk + 8 * hf);
          const bf16x8 kt = *reinterpret_cast<const bf16x8*>(lds + L::K_T + (32 * dt + n) * L::KTS + 16 * kk + 8 * hf);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, kt, acc, 0, 0, 0);
        }
        // acc lane (hf, n): feature 32dt + n, query rows 32mt + 8(i/4) + 4hf + i%4
#pragma unroll
        for (int i4 = 0; i4 < 16; ++i4) {
          const int64_t a = q0 + 32 * mt + 8 * (i4 / 4) + 4 * hf + (i4 % 4);
          if (a < p.Bb) unsafeAtomicAdd(p.dq_acc + (srow + a) * D + 32 * dt + n, acc[i4]);
        }
      }
    }
  }

  // write dK = scale * dK^T^T and dV for this lane's key
  if (key >= p.Bb) return;
  __bf16* dkrow = reinterpret_cast<__bf16*>(p.dk.ptr) + j * p.dk.s_blk + b * p.dk.s_batch +
                  key * p.dk.s_tok + h * p.dk.s_head;
  __bf16* dvrow = reinterpret_cast<__bf16*>(p.dv.ptr) + j * p.dv.s_blk + b * p.dv.s_batch +
                  key * p.dv.s_tok + h * p.dv.s_head;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      bf16x4 wk, wv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        wk[e] = (__bf16)(dk[dt][4 * g4 + e] * p.scale);
        wv[e] = (__bf16)dv[dt][4 * g4 + e];
      }
      *reinterpret_cast<bf16x4*>(dkrow + 32 * dt + 8 * g4 + 4 * hf) = wk;
      *reinterpret_cast<bf16x4*>(dvrow + 32 * dt + 8 * g4 + 4 * hf) = wv;
    }
}

// ---------------------------------------------------------------- fp32 path
// Plain VALU kernel for float32: one lane per key (64 keys per workgroup),
// dK/dV of that key in registers, query tiles of 32 rows staged in LDS.
constexpr int kF32Keys = 64;
constexpr int kF32Rows = 32;

template <int D>
struct BwdF32Lds {
  static constexpr int S = D + 1;  // padded rows: per-lane own-row reads are conflict-free
  static constexpr int KS = 0;
  static constexpr int VS = KS + kF32Keys * S;
  static constexpr int QS = VS + kF32Keys * S;
  static constexpr int OS = QS + kF32Rows * S;
  static constexpr int DS = OS + kF32Rows * S;
  static constexpr int LSE = DS + kF32Rows * (kF32Keys + 1);
  static constexpr int DSUM = LSE + kF32Rows;
  static constexpr int FLOATS = DSUM + kF32Rows;
  static constexpr int BYTES = FLOATS * 4;
};

template <int D>
__global__ __launch_bounds__(kF32Keys) void bwd_f32_kernel(BwdParams p) {
  using L = BwdF32Lds<D>;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  float* sm = reinterpret_cast<float*>(smem_raw);
  float* ks = sm + L::KS;
  float* vs = sm + L::VS;
  float* qs = sm + L::QS;
  float* os = sm + L::OS;
  float* dss = sm + L::DS;
  float* lse_s = sm + L::LSE;
  float* dsum_s = sm + L::DSUM;
  const int tid = threadIdx.x;
  const int32_t BH = p.B * p.H;
  const int32_t tiles = (int32_t)((p.Bb + kF32Keys - 1) / kF32Keys);
  const int64_t id = blockIdx.x;
  const int32_t bh = (int32_t)(id % BH);
  const int32_t b = bh / p.H;
  const int32_t h = bh % p.H;
  int32_t j, tile;
  kv_tile_of(p, id / BH, tiles, &j, &tile);
  const int64_t kv0 = (int64_t)tile * kF32Keys;
  const int64_t key = kv0 + tid;
  const float* kbase = reinterpret_cast<const float*>(p.k.ptr) + j * p.k.s_blk + b * p.k.s_batch + h * p.k.s_head;
  const float* vbase = reinterpret_cast<const float*>(p.v.ptr) + j * p.v.s_blk + b * p.v.s_batch + h * p.v.s_head;
  for (int idx = tid; idx < kF32Keys * D; idx += kF32Keys) {
    const int r = idx / D, e = idx % D;
    const int64_t x = kv0 + r;
    ks[r * L::S + e] = (x < p.Bb) ? kbase[x * p.k.s_tok + e] : 0.0f;
    vs[r * L::S + e] = (x < p.Bb) ? vbase[x * p.v.s_tok + e] : 0.0f;
  }
  float dk[D], dv[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    dk[e] = 0.0f;
    dv[e] = 0.0f;
  }
  const float c2 = p.scale_log2;
  const int32_t qtiles = (int32_t)((p.Bb + kF32Rows - 1) / kF32Rows);
  for (int32_t kstep = 0; kstep < p.P; ++kstep) {
    const int32_t i = ring_rank(j, kstep, p.P);
    if (i < p.rank_begin || i >= p.rank_begin + p.n_ranks) continue;
    const int32_t ri = i - p.rank_begin;
    const BlockRel rel = block_relation(p.layout, p.causal, i, j);
    if (rel.kind == kNone) continue;
    const int32_t band = (rel.kind == kAll) ? kBandAll : rel.band;
    int64_t a_first = (rel.kind == kAll) ? 0 : kv0 - band;
    if (a_first < 0) a_first = 0;
    const float* qbase = reinterpret_cast<const float*>(p.q.ptr) + ri * p.q.s_blk + b * p.q.s_batch + h * p.q.s_head;
    const float* dobase = reinterpret_cast<const float*>(p.dout.ptr) + ri * p.dout.s_blk + b * p.dout.s_batch + h * p.dout.s_head;
    const int64_t srow = (((int64_t)ri * p.B + b) * p.H + h) * p.Bb;
    for (int32_t qt = (int32_t)(a_first / kF32Rows); qt < qtiles; ++qt) {
      const int64_t q0 = (int64_t)qt * kF32Rows;
      __syncthreads();
      for (int idx = tid; idx < kF32Rows * D; idx += kF32Keys) {
        const int r = idx / D, e = idx % D;
        const int64_t x = q0 + r;
        qs[r * L::S + e] = (x < p.Bb) ? qbase[x * p.q.s_tok + e] : 0.0f;
        os[r * L::S + e] = (x < p.Bb) ? dobase[x * p.dout.s_tok + e] : 0.0f;
      }
      if (tid < kF32Rows) {
        const int64_t x = q0 + tid;
        lse_s[tid] = (x < p.Bb) ? p.lse[srow + x] * kLog2e : 0.0f;
        dsum_s[tid] = (x < p.Bb) ? p.dsum[srow + x] : 0.0f;
      }
      __syncthreads();
      for (int r = 0; r < kF32Rows; ++r) {
        const int64_t a = q0 + r;
        const bool vis = key < p.Bb && a < p.Bb && key - a <= (int64_t)band;
        float s = 0.0f, dpv = 0.0f;
#pragma unroll
        for (int e = 0; e < D; ++e) {
          s = fmaf(qs[r * L::S + e], ks[tid * L::S + e], s);
          dpv = fmaf(os[r * L::S + e], vs[tid * L::S + e], dpv);
        }
        const float pv = vis ? fexp2(fmaf(s, c2, -lse_s[r])) : 0.0f;
        const float dsv = pv * (dpv - dsum_s[r]);
#pragma unroll
        for (int e = 0; e < D; ++e) {
          dv[e] = fmaf(pv, os[r * L::S + e], dv[e]);
          dk[e] = fmaf(dsv, qs[r * L::S + e], dk[e]);
        }
        dss[r * (kF32Keys + 1) + tid] = dsv;
      }
      __syncthreads();
      // dQ rows of the tile: lane -> (row tid % 32, half of the features)
      {
        const int r = tid % kF32Rows;
        const int half = tid / kF32Rows;
        const int64_t a = q0 + r;
        if (a < p.Bb) {
          for (int e = half * (D / 2); e < (half + 1) * (D / 2); ++e) {
            float acc = 0.0f;
            for (int kk = 0; kk < kF32Keys; ++kk) acc = fmaf(dss[r * (kF32Keys + 1) + kk], ks[kk * L::S + e], acc);
            unsafeAtomicAdd(p.dq_acc + (srow + a) * D + e, acc);
          }
        }
      }
    }
  }
  if (key >= p.Bb) return;
  float* dkrow = reinterpret_cast<float*>(p.dk.ptr) + j * p.dk.s_blk + b * p.dk.s_batch + key * p.dk.s_tok + h * p.dk.s_head;
  float* dvrow = reinterpret_cast<float*>(p.dv.ptr) + j * p.dv.s_blk + b * p.dv.s_batch + key * p.dv.s_tok + h * p.dv.s_head;
#pragma unroll
  for (int e = 0; e < D; ++e) {
    dkrow[e] = dk[e] * p.scale;
    dvrow[e] = dv[e];
  }
}

template <typename K>
hipError_t launch_dyn(K kernel, int64_t grid, int threads, int bytes, hipStream_t s, const BwdParams& p) {
  if (grid <= 0) return hipSuccess;
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  hipLaunchKernelGGL(kernel, dim3((uint32_t)grid), dim3(threads), bytes, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t s) {
  const int64_t grid = ((p.Bb + kKn - 1) / kKn) * (int64_t)p.P * p.B * p.H;
  if (p.D == 128) return launch_dyn(bwd_bf16_kernel<128>, grid, kThreads, BwdLds<128>::BYTES, s, p);
  return launch_dyn(bwd_bf16_kernel<64>, grid, kThreads, BwdLds<64>::BYTES, s, p);
}

hipError_t launch_bwd_f32(const BwdParams& p, hipStream_t s) {
  const int64_t grid = ((p.Bb + kF32Keys - 1) / kF32Keys) * (int64_t)p.P * p.B * p.H;
  if (p.D == 128) return launch_dyn(bwd_f32_kernel<128>, grid, kF32Keys, BwdF32Lds<128>::BYTES, s, p);
  return launch_dyn(bwd_f32_kernel<64>, grid, kF32Keys, BwdF32Lds<64>::BYTES, s, p);
}

}  // namespace ra
