// ra_fwd.hip — forward kernels of exact blockwise ring attention (gfx950).
//
// A workgroup owns 256 query rows of one rank's query block for one
// (batch, head) and walks the KV blocks in ring order (ra_kvwalk.h), keeping
// the online-softmax state on chip ("Ring Attention 論文分析" (blog),
// section "ブロック単位の分割戦略": running max, correction exp(old - new),
// rescaled sum and accumulator).
//
// bf16 path, per wave (64 lanes, 32 query rows):
//   S^T = K Q^T on v_mfma_f32_32x32x16_bf16, so that lane (h, n) holds the
//   scores of query n against 16 keys: the row max needs one exchange with
//   lane n ^ 32 and the row sum none (each half keeps its own partial sum).
//   O^T += V^T P^T on the same MFMA; the probabilities stay in registers as
//   the B operand (the order of keys inside an MFMA contraction is free, so
//   the order the score accumulators hold is used), and V^T comes from
//   transposing reads of the row-major V tile.
// Scores are scaled in the exponent: p = exp2(S * scale*log2(e) - m), with m
// kept in log2 units. The reference max m is raised only when a tile's max
// exceeds it by more than 8 (then the accumulator is rescaled), so most
// tiles skip the rescale; probabilities then stay below 2^8, exact in the
// fp32 sums and representable in bf16. lse is exported as a natural log.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ra_internal.h"
#include "ra_kvwalk.h"
#include "ra_lds.h"
#include "ra_schedule.h"

namespace ra {
namespace {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescaleSlack = 8.0f;  // log2 units a tile max may exceed the reference max
// Instruction interleave requested from the scheduler for the block that
// issues the next tile's score MFMAs, this tile's exponentials and its P V
// MFMAs: 0 = compiler default, 1 = score MFMAs with 6 VALU each then the P V
// MFMAs with their reads, 2 = score MFMAs with 10 VALU each (fastest measured).
constexpr int kFwdInterleave = 2;

// Work order for the fp32 kernel (64-row tiles); same rule as query_tile_of.
__device__ __forceinline__ void tile_of(const FwdParams& p, int64_t ord, int32_t tiles, int32_t* rank_idx,
                                        int32_t* tile) {
  query_tile_of(p.causal, p.layout, p.n_ranks, ord, tiles, rank_idx, tile);
}

template <int D>
__global__ __launch_bounds__(kQThreads, 1) void fwd_bf16_kernel(FwdParams p) {
  using L = KvLds<D>;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __bf16* lds = reinterpret_cast<__bf16*>(smem_raw);

  const int tid = threadIdx.x;
  const int wave = tid / 64;
  const int lane = tid % 64;
  const int n = lane % 32;
  const int hf = lane / 32;
  const int grp = (lane / 16) % 2;
  const int j16 = lane % 16;

  const int32_t BH = p.B * p.H;
  const int32_t Bb = (int32_t)p.Bb;
  const int32_t tiles = (Bb + kQTm - 1) / kQTm;
  int32_t bh, ri, tile;
  query_work_of(blockIdx.x, BH, p.n_ranks, tiles, p.causal, p.layout, &bh, &ri, &tile);
  const int32_t b = bh / p.H;
  const int32_t h = bh % p.H;
  const int32_t i = p.rank_begin + ri;
  const int32_t a0 = tile * kQTm;
  const int32_t aw = a0 + 32 * wave;  // first row of this wave
  const int32_t a = aw + n;           // this lane's row
  const int32_t a_hi = (a0 + kQTm - 1 < Bb - 1) ? a0 + kQTm - 1 : Bb - 1;

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

  // online-softmax state: acc[dt][e] = O^T feature 32dt + 8(e/4) + 4hf + e%4
  f32x16 acc[D / 32];
  float m, l;
  const int64_t srow = (((int64_t)ri * p.B + b) * p.H + h) * p.Bb;  // state / lse row base
  if (p.mode == 1 && !p.first) {
    m = (a < Bb) ? p.st_lse[srow + a] : -INFINITY;
    l = (hf == 0) ? 1.0f : 0.0f;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        float4 v4 = make_float4(0.f, 0.f, 0.f, 0.f);
        if (a < Bb) v4 = *reinterpret_cast<const float4*>(p.st_o + (srow + a) * D + 32 * dt + 8 * g4 + 4 * hf);
        acc[dt][4 * g4 + 0] = v4.x;
        acc[dt][4 * g4 + 1] = v4.y;
        acc[dt][4 * g4 + 2] = v4.z;
        acc[dt][4 * g4 + 3] = v4.w;
      }
  } else {
    m = -INFINITY;
    l = 0.0f;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      f32x16 z = {};
      acc[dt] = z;
    }
  }

  // per-lane element offsets inside a tile: K rows n (+32t) at columns
  // 16ss + 8hf; V^T transposing reads at rows 4hf + j16/4 (+8) (+16kk) and
  // columns 32dt + 16grp + 4(j16%4)
  int koff[D / 16], voff[2][D / 32];
#pragma unroll
  for (int ss = 0; ss < D / 16; ++ss) koff[ss] = tile_off<D>(n, 16 * ss + 8 * hf);
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
      voff[h2][dt] = tile_off<D>(4 * hf + j16 / 4 + 8 * h2, 32 * dt + 16 * grp + 4 * (j16 % 4));

  KvIter c0;
  c0.kstep = -1;
  c0.nsteps = (p.mode == 0) ? p.P : 1;
  c0.single_block = (p.mode == 0) ? -1 : p.step_block;
  c0.i = i;
  c0.P = p.P;
  c0.layout = p.layout;
  c0.causal = p.causal;
  c0.a_hi = a_hi;
  c0.Bb = Bb;
  const int64_t kvblk_mul = (p.mode == 0) ? 1 : 0;  // the single-step buffer holds one block
  auto kv_base = [&](const Seq& sq, int32_t blk) {
    return reinterpret_cast<const __bf16*>(sq.ptr) + kvblk_mul * blk * sq.s_blk + b * sq.s_batch + h * sq.s_head;
  };
  auto dma_tile = [&](const KvIter& t, int stage) {
    __bf16* st = lds + stage * L::STAGE;
    dma_rows<D, kKvTn, kQWaves>(st, kv_base(p.k, t.j), p.k.s_tok, t.t * kKvTn, Bb, wave, lane);
    dma_rows<D, kKvTn, kQWaves>(st + L::TILE, kv_base(p.v, t.j), p.v.s_tok, t.t * kKvTn, Bb, wave, lane);
  };
  // S^T = K Q^T for the tile's 64 keys (two 32-key halves)
  auto scores = [&](int stage, f32x16* s) {
    const __bf16* ks = lds + stage * L::STAGE;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x16 z = {};
      s[t] = z;
#pragma unroll
      for (int ss = 0; ss < D / 16; ++ss) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(ks + koff[ss] + 32 * t * D);
        s[t] = mfma32(kf, qreg[ss], s[t]);
      }
    }
  };
  const float c2 = p.scale_log2;
  // Mask and running-max update of tile t (scores in s); returns the max to
  // subtract. Rows whose keys are all masked keep a zero weight.
  auto prepare = [&](const KvIter& t, f32x16* s) {
    const int32_t band = t.band;
    const int32_t b0 = t.t * kKvTn;
    if ((b0 + kKvTn - 1 - aw > band) || (b0 + kKvTn > Bb)) {
      // key b0 + off is visible iff off <= min(band + a - b0, Bb - 1 - b0)
      const int32_t lim0 = band + a - b0, lim1 = Bb - 1 - b0;
      const int32_t lim = lim0 < lim1 ? lim0 : lim1;
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int32_t off = 32 * t2 + 8 * (e / 4) + 4 * hf + (e % 4);
          if (off > lim) s[t2][e] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[t2][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mt = mx * c2;  // tile max, log2 units
    if (__builtin_amdgcn_ballot_w64(mt > m + kRescaleSlack) != 0) {
      const float m_new = fmaxf(m, mt);
      const float alpha = (m_new == -INFINITY) ? 1.0f : fexp2(m - m_new);
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[dt][e] *= alpha;
      m = m_new;
    }
    return (m == -INFINITY) ? 0.0f : m;
  };
  // One branch-free block: the next tile's scores (into s_next, from stage
  // s1), this tile's probabilities (from s_cur) and O^T += V^T P^T (stage sc).
  auto fused = [&](int sc, int s1, f32x16* s_cur, f32x16* s_next, float m_use) {
    scores(s1, s_next);
    const __bf16* vs = lds + sc * L::STAGE + L::TILE;
    bf16x8 pb[4];
    float lsum = 0.0f;
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pv = fexp2(fmaf(s_cur[t2][e], c2, -m_use));
        lsum += pv;
        pb[2 * t2 + e / 8][e % 8] = (__bf16)pv;
      }
    l += lsum;
    // P element e of k-step kk is key 16kk + 8(e/4) + 4hf + e%4
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 vf = cat(tr_read(vs + voff[0][dt] + 16 * kk * D), tr_read(vs + voff[1][dt] + 16 * kk * D));
        acc[dt] = mfma32(vf, pb[kk], acc[dt]);
      }
    if (kFwdInterleave == 2) {
#pragma unroll
      for (int k = 0; k < D / 8; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);
      }
    }
    if (kFwdInterleave == 1) {
      // 16 score MFMAs each followed by a K read and 6 VALU (exponentials),
      // then the 16 P V MFMAs with their V^T reads
#pragma unroll
      for (int k = 0; k < D / 8; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // VALU
      }
#pragma unroll
      for (int k = 0; k < D / 8; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
    }
  };

  if (c0.next_block()) {
    KvIter c1 = c0;
    bool v1 = c1.next();
    dma_tile(c0, 0);
    if (v1) dma_tile(c1, 1);
    wait_dma();
    __syncthreads();
    f32x16 sa[2], sb[2];
    scores(0, sa);
    int sc = 0;
    // Each half: this tile's softmax runs while the next tile's score MFMAs
    // are on the matrix pipe, and the tile after next is being copied. Two
    // halves per trip swap the score buffers without copies. Every wave does
    // every tile (a tile hidden from a wave by the mask is fully masked and
    // contributes zero), which keeps the block free of branches; the last
    // half computes scores of a stale stage and drops them.
    while (true) {
      {
        KvIter c2 = c1;
        const bool v2 = v1 && c2.next();
        const int s1 = (sc == 2) ? 0 : sc + 1;
        const int s2 = (s1 == 2) ? 0 : s1 + 1;
        if (v2) dma_tile(c2, s2);
        const float m_use = prepare(c0, sa);
        fused(sc, s1, sa, sb, m_use);
        if (!v1) break;
        wait_dma();
        __syncthreads();  // tile c2 is in LDS; stage sc is free
        c0 = c1;
        c1 = c2;
        v1 = v2;
        sc = s1;
      }
      {
        KvIter c2 = c1;
        const bool v2 = v1 && c2.next();
        const int s1 = (sc == 2) ? 0 : sc + 1;
        const int s2 = (s1 == 2) ? 0 : s1 + 1;
        if (v2) dma_tile(c2, s2);
        const float m_use = prepare(c0, sb);
        fused(sc, s1, sb, sa, m_use);
        if (!v1) break;
        wait_dma();
        __syncthreads();
        c0 = c1;
        c1 = c2;
        v1 = v2;
        sc = s1;
      }
    }
  }

  // finalise: combine the two halves' sums, normalise, export
  const float l_tot = l + __shfl_xor(l, 32);
  const float m_use = (m == -INFINITY) ? 0.0f : m;
  const float inv = (l_tot > 0.0f) ? 1.0f / l_tot : 0.0f;
  if (a >= Bb) return;
  if (p.mode == 0 || p.last) {
    __bf16* orow = reinterpret_cast<__bf16*>(p.o.ptr) + ri * p.o.s_blk + b * p.o.s_batch +
                   (int64_t)a * p.o.s_tok + h * p.o.s_head;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(acc[dt][4 * g4 + e] * inv);
        *reinterpret_cast<bf16x4*>(orow + 32 * dt + 8 * g4 + 4 * hf) = w;
      }
    if (hf == 0) p.lse[srow + a] = (l_tot > 0.0f) ? (m_use + log2f(l_tot)) * kLn2 : -INFINITY;
  } else {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const float4 v4 = make_float4(acc[dt][4 * g4] * inv, acc[dt][4 * g4 + 1] * inv,
                                      acc[dt][4 * g4 + 2] * inv, acc[dt][4 * g4 + 3] * inv);
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
  const int64_t tiles = (p.Bb + kQTm - 1) / kQTm;
  const int64_t grid = tiles * p.n_ranks * p.B * p.H;
  if (grid <= 0) return hipSuccess;
  if (p.D == 128) {
    hipLaunchKernelGGL(fwd_bf16_kernel<128>, dim3((uint32_t)grid), dim3(kQThreads), KvLds<128>::BYTES, s, p);
  } else {
    hipLaunchKernelGGL(fwd_bf16_kernel<64>, dim3((uint32_t)grid), dim3(kQThreads), KvLds<64>::BYTES, s, p);
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
