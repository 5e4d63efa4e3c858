// ra_fwd.hip — forward kernels of exact blockwise ring attention (gfx950).
//
// One workgroup owns a tile of query rows of one rank's query block for one
// (batch, head). It visits KV blocks in ring order j = (i - k) mod P ("Ring
// Attention: Sequence Parallelism for Long Context", section "Ring
// Attention: Compute While You Communicate") and, inside a block, KV tiles of
// 64 keys, keeping the online-softmax state (running max m, running sum l,
// accumulator) on chip ("Ring Attention 論文分析" (blog), section "ブロック
// 単位の分割戦略": new max, correction exp(old - new), rescaled sum and
// accumulator). KV tiles that the causal/striped mask hides entirely are
// never loaded; tiles that cross the diagonal get the mask in registers.
//
// bf16 path, per wave (64 lanes, 32 query rows):
//   S^T = K Q^T on v_mfma_f32_32x32x16_bf16, so that lane (h, n) holds the
//   scores of query n against 16 keys: the row max needs one exchange with
//   lane n ^ 32 and the row sum none (each half keeps its own partial sum).
//   O^T += V^T P^T on the same MFMA; the probabilities stay in registers as
//   the B operand (the contraction order of keys inside an MFMA is free, so
//   the key order the score accumulators hold is used as is). K sits in LDS
//   row-major [key][d]; V is transposed to [d][key] while it is staged.
// Scores are scaled in the exponent: p = exp2(S * scale*log2(e) - m), with m
// kept in log2 units; lse is exported as a natural log.
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
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;  // 4 waves
constexpr int kTm = 128;       // query rows per workgroup, 32 per wave
constexpr int kTn = 64;        // keys per KV tile
constexpr int kBandAll = 1 << 30;
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Work order: the heaviest query tiles are dispatched first. Contiguous
// causal work grows with the rank, striped and non-causal work with the row.
__device__ __forceinline__ void tile_of(const FwdParams& p, int64_t ord, int32_t tiles,
                                        int32_t* rank_idx, int32_t* tile) {
  if (p.causal && p.layout == kContiguous) {
    *rank_idx = p.n_ranks - 1 - (int32_t)(ord / tiles);
    *tile = tiles - 1 - (int32_t)(ord % tiles);
  } else {
    *tile = tiles - 1 - (int32_t)(ord / p.n_ranks);
    *rank_idx = p.n_ranks - 1 - (int32_t)(ord % p.n_ranks);
  }
}

template <int D>
struct FwdLds {
  static constexpr int KS = D + 8;    // K row stride (elements): rows 16B-aligned
  static constexpr int VS = kTn + 4;  // V^T row stride (elements): 136 B rows
  static constexpr int K_ELEMS = kTn * KS;
  static constexpr int V_ELEMS = D * VS;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr int BYTES = 2 * STAGE * 2;  // two stages of bf16
};

// Registers holding one KV tile between its global load and its LDS store.
template <int D>
struct TileRegs {
  static constexpr int CR = D / 8;             // 16-byte chunks per K row
  static constexpr int RPP = kThreads / CR;    // K rows per pass
  static constexpr int KP = kTn / RPP;         // passes
  static constexpr int NP = D / 2;             // feature pairs of V
  static constexpr int NG = kThreads / NP;     // key groups of V
  static constexpr int KG = kTn / NG;          // keys per thread for V
  u32x4 k[KP];
  uint32_t v[KG];
};

template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D>& r, const __bf16* kbase, const __bf16* vbase,
                                          int64_t s_tok_k, int64_t s_tok_v, int32_t b0, int32_t Bb,
                                          int tid) {
  using T = TileRegs<D>;
  const int c = tid % T::CR;
  const int r0 = tid / T::CR;
#pragma unroll
  for (int p = 0; p < T::KP; ++p) {
    const int32_t x = b0 + r0 + T::RPP * p;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (x < Bb) val = *reinterpret_cast<const u32x4*>(kbase + (int64_t)x * s_tok_k + 8 * c);
    r.k[p] = val;
  }
  const int pr = tid % T::NP;
  const int g = tid / T::NP;
#pragma unroll
  for (int q = 0; q < T::KG; ++q) {
    const int32_t x = b0 + T::KG * g + q;
    uint32_t val = 0u;
    if (x < Bb) val = *reinterpret_cast<const uint32_t*>(vbase + (int64_t)x * s_tok_v + 2 * pr);
    r.v[q] = val;
  }
}

template <int D>
__device__ __forceinline__ void store_tile(const TileRegs<D>& r, __bf16* stage, int tid) {
  using T = TileRegs<D>;
  using L = FwdLds<D>;
  __bf16* ks = stage;
  __bf16* vt = stage + L::K_ELEMS;
  const int c = tid % T::CR;
  const int r0 = tid / T::CR;
#pragma unroll
  for (int p = 0; p < T::KP; ++p)
    *reinterpret_cast<u32x4*>(ks + (r0 + T::RPP * p) * L::KS + 8 * c) = r.k[p];
  // transpose: the thread holds features (2pr, 2pr+1) of KG consecutive keys
  const int pr = tid % T::NP;
  const int g = tid / T::NP;
  __bf16* even = vt + (2 * pr) * L::VS + T::KG * g;
  __bf16* odd = even + L::VS;
#pragma unroll
  for (int q = 0; q < T::KG; q += 4) {
    u32x2 e, o;
    e[0] = (r.v[q] & 0xFFFFu) | (r.v[q + 1] << 16);
    e[1] = (r.v[q + 2] & 0xFFFFu) | (r.v[q + 3] << 16);
    o[0] = (r.v[q] >> 16) | (r.v[q + 1] & 0xFFFF0000u);
    o[1] = (r.v[q + 2] >> 16) | (r.v[q + 3] & 0xFFFF0000u);
    *reinterpret_cast<u32x2*>(even + q) = e;
    *reinterpret_cast<u32x2*>(odd + q) = o;
  }
}

// Online-softmax state of one lane: query n of the wave, the half `hf` of
// the key rows of every score tile. m is shared by both halves; l is this
// half's partial sum.
template <int D>
struct RowState {
  f32x16 acc[D / 32];  // O^T: acc[dt][i] = feature 32dt + 8(i/4) + 4hf + i%4
  float m;             // log2 units, -inf before any visible key
  float l;
};

template <int D>
__device__ __forceinline__ void compute_tile(RowState<D>& st, const bf16x8* qreg, const __bf16* stage,
                                             int32_t b0, int32_t a, int32_t aw, int32_t band,
                                             int32_t Bb, float c2, int n, int hf) {
  using L = FwdLds<D>;
  const __bf16* ks = stage;
  const __bf16* vt = stage + L::K_ELEMS;
  f32x16 s[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    f32x16 z = {};
    s[t] = z;
#pragma unroll
    for (int ss = 0; ss < D / 16; ++ss) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(ks + (32 * t + n) * L::KS + 16 * ss + 8 * hf);
      s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qreg[ss], s[t], 0, 0, 0);
    }
  }
  // mask: only tiles that cross the band or the ragged end of the block
  const bool need_mask = (b0 + kTn - 1 - aw > band) || (b0 + kTn > Bb);
  if (need_mask) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int32_t b = b0 + 32 * t + 8 * (i / 4) + 4 * hf + (i % 4);
        if (b - a > band || b >= Bb) s[t][i] = -INFINITY;
      }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[t][i]);
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(st.m, mx * c2);
  const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
  const float alpha = fexp2(st.m - m_use);
  st.m = m_new;
  float lsum = 0.0f;
  bf16x8 pb[4];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float pv = fexp2(fmaf(s[t][i], c2, -m_use));
      lsum += pv;
      pb[2 * t + i / 8][i % 8] = (__bf16)pv;
    }
  st.l = fmaf(st.l, alpha, lsum);
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) st.acc[dt][i] *= alpha;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const __bf16* vr = vt + (32 * dt + n) * L::VS + 16 * kk + 4 * hf;
      const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vr);
      const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vr + 8);
      const bf16x8 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      st.acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[kk], st.acc[dt], 0, 0, 0);
    }
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(FwdParams p) {
  using L = FwdLds<D>;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __bf16* lds = reinterpret_cast<__bf16*>(smem_raw);

  const int tid = threadIdx.x;
  const int wave = tid / 64;
  const int lane = tid % 64;
  const int n = lane % 32;
  const int hf = lane / 32;

  const int32_t BH = p.B * p.H;
  const int32_t tiles = (int32_t)((p.Bb + kTm - 1) / kTm);
  const int64_t id = blockIdx.x;
  const int32_t bh = (int32_t)(id % BH);
  const int32_t b = bh / p.H;
  const int32_t h = bh % p.H;
  int32_t ri, tile;
  tile_of(p, id / BH, tiles, &ri, &tile);
  const int32_t i = p.rank_begin + ri;
  const int32_t Bb = (int32_t)p.Bb;
  const int32_t a0 = tile * kTm;
  const int32_t aw = a0 + 32 * wave;
  const int32_t a = aw + n;
  const int32_t a_hi = (a0 + kTm - 1 < Bb - 1) ? a0 + kTm - 1 : Bb - 1;

  // resident query rows, as the B operand of S^T = K Q^T
  const __bf16* qrow = reinterpret_cast<const __bf16*>(p.q.ptr) + ri * p.q.s_blk + b * p.q.s_batch +
                       (int64_t)a * p.q.s_tok + h * p.q.s_head;
  bf16x8 qreg[D / 16];
#pragma unroll
  for (int ss = 0; ss < D / 16; ++ss) {
    u32x4 val = {0u, 0u, 0u, 0u};
    if (a < Bb) val = *reinterpret_cast<const u32x4*>(qrow + 16 * ss + 8 * hf);
    qreg[ss] = __builtin_bit_cast(bf16x8, val);
  }

  RowState<D> st;
  const int64_t srow = (((int64_t)ri * p.B + b) * p.H + h) * p.Bb;  // state / lse row base
  if (p.mode == 1 && !p.first) {
    const float m_prev = (a < p.Bb) ? p.st_lse[srow + a] : -INFINITY;
    st.m = m_prev;
    st.l = (hf == 0) ? 1.0f : 0.0f;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        float4 v4 = make_float4(0.f, 0.f, 0.f, 0.f);
        if (a < p.Bb)
          v4 = *reinterpret_cast<const float4*>(p.st_o + (srow + a) * D + 32 * dt + 8 * g4 + 4 * hf);
        st.acc[dt][4 * g4 + 0] = v4.x;
        st.acc[dt][4 * g4 + 1] = v4.y;
        st.acc[dt][4 * g4 + 2] = v4.z;
        st.acc[dt][4 * g4 + 3] = v4.w;
      }
  } else {
    st.m = -INFINITY;
    st.l = 0.0f;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      f32x16 z = {};
      st.acc[dt] = z;
    }
  }

  const float c2 = p.scale_log2;
  int32_t it = 0;  // tile counter across blocks: selects the LDS stage
  const int32_t nsteps = (p.mode == 0) ? p.P : 1;
  for (int32_t kstep = 0; kstep < nsteps; ++kstep) {
    const int32_t j = (p.mode == 0) ? ring_block(i, kstep, p.P) : p.step_block;
    const BlockRel rel = block_relation(p.layout, p.causal, i, j);
    const int64_t extent = visible_key_extent(rel, a_hi, p.Bb);
    if (extent <= 0) continue;
    const int32_t band = (rel.kind == kAll) ? kBandAll : rel.band;
    const int64_t kblk = (p.mode == 0) ? (int64_t)j : 0;
    const __bf16* kbase = reinterpret_cast<const __bf16*>(p.k.ptr) + kblk * p.k.s_blk + b * p.k.s_batch +
                          h * p.k.s_head;
    const __bf16* vbase = reinterpret_cast<const __bf16*>(p.v.ptr) + kblk * p.v.s_blk + b * p.v.s_batch +
                          h * p.v.s_head;
    const int32_t ntile = (int32_t)((extent + kTn - 1) / kTn);
    TileRegs<D> regs;
    load_tile<D>(regs, kbase, vbase, p.k.s_tok, p.v.s_tok, 0, Bb, tid);
    for (int32_t t = 0; t < ntile; ++t, ++it) {
      __bf16* stage = lds + (it & 1) * L::STAGE;
      store_tile<D>(regs, stage, tid);
      __syncthreads();
      const int32_t b0 = t * kTn;
      if (t + 1 < ntile) load_tile<D>(regs, kbase, vbase, p.k.s_tok, p.v.s_tok, b0 + kTn, Bb, tid);
      // skip the MFMAs when the mask hides the whole tile from this wave
      const bool wave_dead = (aw >= Bb) || (b0 - (aw + 31) > band);
      if (!wave_dead) compute_tile<D>(st, qreg, stage, b0, a, aw, band, Bb, c2, n, hf);
    }
  }

  // finalise: combine the two halves' sums, normalise, export
  const float l_tot = st.l + __shfl_xor(st.l, 32);
  const float m_use = (st.m == -INFINITY) ? 0.0f : st.m;
  const float inv = (l_tot > 0.0f) ? 1.0f / l_tot : 0.0f;
  if (a >= p.Bb) return;
  if (p.mode == 0 || p.last) {
    __bf16* orow = reinterpret_cast<__bf16*>(p.o.ptr) + ri * p.o.s_blk + b * p.o.s_batch +
                   a * p.o.s_tok + h * p.o.s_head;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(st.acc[dt][4 * g4 + e] * inv);
        *reinterpret_cast<bf16x4*>(orow + 32 * dt + 8 * g4 + 4 * hf) = w;
      }
    if (hf == 0) p.lse[srow + a] = (l_tot > 0.0f) ? (m_use + log2f(l_tot)) * kLn2 : -INFINITY;
  } else {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        float4 v4 = make_float4(st.acc[dt][4 * g4] * inv, st.acc[dt][4 * g4 + 1] * inv,
                                st.acc[dt][4 * g4 + 2] * inv, st.acc[dt][4 * g4 + 3] * inv);
        *reinterpret_cast<float4*>(p.st_o + (srow + a) * D + 32 * dt + 8 * g4 + 4 * hf) = v4;
      }
    if (hf == 0) p.st_lse[srow + a] = (l_tot > 0.0f) ? m_use + log2f(l_tot) : -INFINITY;
  }
}

// ---------------------------------------------------------------- fp32 path
// Plain VALU kernel for float32 inputs: one lane per query row, KV tiles of
// 64 keys staged in LDS and read as broadcasts. Same ring walk, masks and
// state handling as the bf16 kernel.
constexpr int kF32Rows = 64;

template <int D>
__global__ __launch_bounds__(kF32Rows) void fwd_f32_kernel(FwdParams p) {
  constexpr int TN = 4096 / D;  // keys per staged tile: 32 KiB of LDS for K and V
  __shared__ float ks[TN][D];
  __shared__ float vs[TN][D];
  const int tid = threadIdx.x;
  const int32_t BH = p.B * p.H;
  const int32_t tiles = (int32_t)((p.Bb + kF32Rows - 1) / kF32Rows);
  const int64_t id = blockIdx.x;
  const int32_t bh = (int32_t)(id % BH);
  const int32_t b = bh / p.H;
  const int32_t h = bh % p.H;
  int32_t ri, tile;
  tile_of(p, id / BH, tiles, &ri, &tile);
  const int32_t i = p.rank_begin + ri;
  const int64_t a0 = (int64_t)tile * kF32Rows;
  const int64_t a = a0 + tid;
  const int64_t a_hi = (a0 + kF32Rows - 1 < p.Bb - 1) ? a0 + kF32Rows - 1 : p.Bb - 1;
  const bool live = a < p.Bb;

  float qv[D], acc[D];
  const float* qrow = reinterpret_cast<const float*>(p.q.ptr) + ri * p.q.s_blk + b * p.q.s_batch +
                      a * p.q.s_tok + h * p.q.s_head;
#pragma unroll
  for (int e = 0; e < D; ++e) qv[e] = live ? qrow[e] : 0.0f;
  const int64_t srow = (((int64_t)ri * p.B + b) * p.H + h) * p.Bb;
  float m, l;
  if (p.mode == 1 && !p.first) {
    m = live ? p.st_lse[srow + a] : -INFINITY;
    l = 1.0f;
#pragma unroll
    for (int e = 0; e < D; ++e) acc[e] = live ? p.st_o[(srow + a) * D + e] : 0.0f;
  } else {
    m = -INFINITY;
    l = 0.0f;
#pragma unroll
    for (int e = 0; e < D; ++e) acc[e] = 0.0f;
  }
  const float c2 = p.scale_log2;
  const int32_t nsteps = (p.mode == 0) ? p.P : 1;
  for (int32_t kstep = 0; kstep < nsteps; ++kstep) {
    const int32_t j = (p.mode == 0) ? ring_block(i, kstep, p.P) : p.step_block;
    const BlockRel rel = block_relation(p.layout, p.causal, i, j);
    const int64_t extent = visible_key_extent(rel, a_hi, p.Bb);
    if (extent <= 0) continue;
    const int32_t band = (rel.kind == kAll) ? kBandAll : rel.band;
    const int64_t kblk = (p.mode == 0) ? (int64_t)j : 0;
    const float* kbase = reinterpret_cast<const float*>(p.k.ptr) + kblk * p.k.s_blk + b * p.k.s_batch +
                         h * p.k.s_head;
    const float* vbase = reinterpret_cast<const float*>(p.v.ptr) + kblk * p.v.s_blk + b * p.v.s_batch +
                         h * p.v.s_head;
    for (int64_t b0 = 0; b0 < extent; b0 += TN) {
      __syncthreads();
      for (int idx = tid; idx < TN * D; idx += kF32Rows) {
        const int r = idx / D, e = idx % D;
        const int64_t x = b0 + r;
        ks[r][e] = (x < p.Bb) ? kbase[x * p.k.s_tok + e] : 0.0f;
        vs[r][e] = (x < p.Bb) ? vbase[x * p.v.s_tok + e] : 0.0f;
      }
      __syncthreads();
      if (!live) continue;
      for (int c0 = 0; c0 < TN; c0 += 16) {
        float sc[16];
        float mx = -INFINITY;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          float dot = 0.0f;
#pragma unroll
          for (int e = 0; e < D; ++e) dot = fmaf(qv[e], ks[c0 + u][e], dot);
          const int64_t kb = b0 + c0 + u;
          sc[u] = (kb - a > (int64_t)band || kb >= p.Bb) ? -INFINITY : dot;
          mx = fmaxf(mx, sc[u]);
        }
        const float m_new = fmaxf(m, mx * c2);
        const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
        const float alpha = fexp2(m - m_use);
        m = m_new;
        l *= alpha;
#pragma unroll
        for (int e = 0; e < D; ++e) acc[e] *= alpha;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const float pv = fexp2(fmaf(sc[u], c2, -m_use));
          l += pv;
#pragma unroll
          for (int e = 0; e < D; ++e) acc[e] = fmaf(pv, vs[c0 + u][e], acc[e]);
        }
      }
    }
  }
  if (!live) return;
  const float m_use = (m == -INFINITY) ? 0.0f : m;
  const float inv = (l > 0.0f) ? 1.0f / l : 0.0f;
  if (p.mode == 0 || p.last) {
    float* orow = reinterpret_cast<float*>(p.o.ptr) + ri * p.o.s_blk + b * p.o.s_batch + a * p.o.s_tok +
                  h * p.o.s_head;
#pragma unroll
    for (int e = 0; e < D; ++e) orow[e] = acc[e] * inv;
    p.lse[srow + a] = (l > 0.0f) ? (m_use + log2f(l)) * kLn2 : -INFINITY;
  } else {
#pragma unroll
    for (int e = 0; e < D; ++e) p.st_o[(srow + a) * D + e] = acc[e] * inv;
    p.st_lse[srow + a] = (l > 0.0f) ? m_use + log2f(l) : -INFINITY;
  }
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t s) {
  const int64_t tiles = (p.Bb + kTm - 1) / kTm;
  const int64_t grid = tiles * p.n_ranks * p.B * p.H;
  if (grid <= 0) return hipSuccess;
  if (p.D == 128) {
    hipLaunchKernelGGL(fwd_bf16_kernel<128>, dim3((uint32_t)grid), dim3(kThreads), FwdLds<128>::BYTES, s, p);
  } else {
    hipLaunchKernelGGL(fwd_bf16_kernel<64>, dim3((uint32_t)grid), dim3(kThreads), FwdLds<64>::BYTES, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t s) {
  const int64_t tiles = (p.Bb + kF32Rows - 1) / kF32Rows;
  const int64_t grid = tiles * p.n_ranks * p.B * p.H;
  if (grid <= 0) return hipSuccess;
  if (p.D == 128) {
    hipLaunchKernelGGL(fwd_f32_kernel<128>, dim3((uint32_t)grid), dim3(kF32Rows), 0, s, p);
  } else {
    hipLaunchKernelGGL(fwd_f32_kernel<64>, dim3((uint32_t)grid), dim3(kF32Rows), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace ra
