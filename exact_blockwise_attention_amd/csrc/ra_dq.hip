// ra_dq.hip — the dQ half of the backward (gfx950).
//
// "Ring Attention 論文分析" (blog), section "逆伝播での KV 再循環": with P
// recomputed from the saved log-sum-exp, dS = P * (dP - D), dP = dO V^T and
// D = rowsum(dO * O), the query gradient is dQ = scale * dS K. Here a
// workgroup owns 256 query rows and walks the KV blocks in ring order exactly
// as the forward does (ra_kvwalk.h), accumulating dQ of its rows on chip — no
// atomics, so the result does not depend on scheduling. The dK/dV half runs
// in ra_bwd.hip with the roles of queries and keys swapped.
//
// bf16 path, per wave (32 query rows): S^T = K Q^T and dP^T = V dO^T leave
// lane (h, n) with query n against 16 keys; dS^T stays in registers as the B
// operand of dQ^T += K^T dS^T, whose K^T operand comes from transposing reads
// of the row-major K tile.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "ra_internal.h"
#include "ra_kvwalk.h"
#include "ra_lds.h"
#include "ra_schedule.h"

namespace ra {
namespace {

template <int D>
__global__ __launch_bounds__(kQThreads, 1) void dq_bf16_kernel(BwdParams p) {
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
  // the tiles of a group share K/V tiles in L2 through the walk's second
  // pass: keep them together
  query_work_of(blockIdx.x, BH, p.G, p.n_ranks, tiles, p.causal, p.layout, false, &bh, &ri, &tile);
  const int32_t b = bh / p.H;
  const int32_t h = bh % p.H;
  const int32_t hk = h / p.G;  // the K/V head this query head reads
  const int32_t i = p.rank_begin + ri;
  const int32_t a0 = tile * kQTm;
  const int32_t aw = a0 + 32 * wave;
  const int32_t a = aw + n;
  const int32_t a_hi = (a0 + kQTm - 1 < Bb - 1) ? a0 + kQTm - 1 : Bb - 1;

  // this lane's query and output-gradient rows, as B operands
  const __bf16* qrow = reinterpret_cast<const __bf16*>(p.q.ptr) + ri * p.q.s_blk + b * p.q.s_batch +
                       (int64_t)a * p.q.s_tok + h * p.q.s_head;
  const __bf16* orow = reinterpret_cast<const __bf16*>(p.dout.ptr) + ri * p.dout.s_blk + b * p.dout.s_batch +
                       (int64_t)a * p.dout.s_tok + h * p.dout.s_head;
  bf16x8 qreg[D / 16], oreg[D / 16];
#pragma unroll
  for (int ss = 0; ss < D / 16; ++ss) {
    u32x4 vq = {0u, 0u, 0u, 0u}, vo = {0u, 0u, 0u, 0u};
    if (a < Bb) {
      vq = *reinterpret_cast<const u32x4*>(qrow + 16 * ss + 8 * hf);
      vo = *reinterpret_cast<const u32x4*>(orow + 16 * ss + 8 * hf);
    }
    qreg[ss] = __builtin_bit_cast(bf16x8, vq);
    oreg[ss] = __builtin_bit_cast(bf16x8, vo);
  }
  const int64_t srow = (((int64_t)ri * p.B + b) * p.H + h) * p.Bb;
  const float lse2 = (a < Bb) ? p.lse2[srow + a] : 0.0f;  // log2 units
  const float dsum = (a < Bb) ? p.dsum[srow + a] : 0.0f;

  f32x16 acc[D / 32];  // dQ^T: feature 32dt + 8(i/4) + 4hf + i%4, query n
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    f32x16 z = {};
    acc[dt] = z;
  }

  // per-lane element offsets inside a tile: K / V rows n (+32t) at columns
  // 16ss + 8hf; K^T transposing reads at rows 4hf + j16/4 (+8) (+16kk) and
  // columns 32dt + 16grp + 4(j16%4)
  int koff[D / 16], toff[2][D / 32];
#pragma unroll
  for (int ss = 0; ss < D / 16; ++ss) koff[ss] = tile_off<D>(n, 16 * ss + 8 * hf);
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
      toff[h2][dt] = tile_off<D>(4 * hf + j16 / 4 + 8 * h2, 32 * dt + 16 * grp + 4 * (j16 % 4));

  KvPassIter c0;
  c0.pass = 0;
  c0.kstep = -1;
  c0.nsteps = p.P;
  c0.single_block = -1;
  c0.i = i;
  c0.P = p.P;
  c0.layout = p.layout;
  c0.causal = p.causal;
  c0.a_lo = a0;
  c0.a_hi = a_hi;
  c0.Bb = Bb;
  auto kv_base = [&](const Seq& sq, int32_t blk) {
    return reinterpret_cast<const __bf16*>(sq.ptr) + (int64_t)blk * sq.s_blk + b * sq.s_batch + hk * sq.s_head;
  };
  auto dma_tile = [&](const KvPassIter& t, int stage) {
    __bf16* st = lds + stage * L::STAGE;
    dma_rows<D, kKvTn, kQWaves>(st, kv_base(p.k, t.j), p.k.s_tok, t.t * kKvTn, Bb, wave, lane);
    dma_rows<D, kKvTn, kQWaves>(st + L::TILE, kv_base(p.v, t.j), p.v.s_tok, t.t * kKvTn, Bb, wave, lane);
  };
  // no row of the wave sees the tile's first key (row extents grow with the row)
  auto dead = [&](const KvPassIter& t) { return (aw >= Bb) || (row_extent32(t.rel, aw + 31) <= t.t * kKvTn); };
  // S^T = K Q^T and dP^T = V dO^T for keys 32 half .. +31 of a tile; the K
  // and V fragments of feature step ss + 1 are requested before the
  // products of step ss
  const uint32_t lbase = lds_addr(smem_raw);
  auto produce = [&](int stage, auto HALFc, f32x16* sd) __attribute__((always_inline)) {
    constexpr int half = decltype(HALFc)::value;
    constexpr int NSS = D / 16;
    constexpr int KO = 32 * half * D * 2, VO = L::TILE * 2 + KO;  // bytes
    const uint32_t sb = lbase + stage * L::STAGE * 2;
    u32x4 f[2][2];  // [slot][K, V]
    {
      const uint32_t ad = sb + 2 * koff[0];
      f[0][0] = lds_read16<KO>(ad);
      f[0][1] = lds_read16<VO>(ad);
    }
    const f32x16 z = {};
#pragma unroll
    for (int ss = 0; ss < NSS; ++ss) {
      if (ss + 1 < NSS) {
        const uint32_t ad = sb + 2 * koff[ss + 1];
        f[(ss + 1) & 1][0] = lds_read16<KO>(ad);
        f[(ss + 1) & 1][1] = lds_read16<VO>(ad);
        lds_wait<2>(f[ss & 1]);
      } else {
        lds_wait<0>(f[ss & 1]);
      }
      sd[0] = mfma32(__builtin_bit_cast(bf16x8, f[ss & 1][0]), qreg[ss], ss == 0 ? z : sd[0]);
      sd[1] = mfma32(__builtin_bit_cast(bf16x8, f[ss & 1][1]), oreg[ss], ss == 0 ? z : sd[1]);
    }
  };
  const float c2 = p.scale_log2;
  // dS^T from the half's scores, then dQ^T += K^T dS^T (MASK: the tile is
  // one of the walk's first pass, which some rows see only in part)
  auto consume = [&](const KvPassIter& t, int stage, auto HALFc, f32x16* sd, auto MASKc) __attribute__((always_inline)) {
    constexpr int half = decltype(HALFc)::value;
    constexpr bool MASK = decltype(MASKc)::value != 0;
    const int32_t b0 = t.t * kKvTn + 32 * half;
    const uint32_t kb = lds_addr(lds + stage * L::STAGE);
    // the wave's first row sees the fewest keys; extents never exceed Bb
    const bool need_mask = MASK && row_extent32(t.rel, aw) < b0 + 32;
    const int32_t ext_a = MASK ? row_extent32(t.rel, a) : 0;
    bf16x8 dsb[2];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float pv = fexp2(fmaf(sd[0][e], c2, -lse2));
      if (MASK && need_mask) {
        const int32_t key = b0 + 8 * (e / 4) + 4 * hf + (e % 4);
        if (key >= ext_a) pv = 0.0f;
      }
      dsb[e / 8][e % 8] = (__bf16)(pv * (sd[1][e] - dsum));
    }
    // dS element e of k-step 2 half + u is key 16(2 half + u) + 8(e/4) + 4hf + e%4.
    // K^T fragments in groups of 4 reads (one 32-feature block)
    constexpr int R0 = 16 * (2 * half) * D * 2, R1 = 16 * (2 * half + 1) * D * 2;  // bytes
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      u32x2 g[2][2];
      const uint32_t a0 = kb + 2 * toff[0][dt], a1 = kb + 2 * toff[1][dt];
      g[0][0] = tr_read_at<R0>(a0);
      g[0][1] = tr_read_at<R0>(a1);
      g[1][0] = tr_read_at<R1>(a0);
      g[1][1] = tr_read_at<R1>(a1);
      lds_wait<0>(g);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8 kt = __builtin_bit_cast(bf16x8, __builtin_shufflevector(g[u][0], g[u][1], 0, 1, 2, 3));
        acc[dt] = mfma32(kt, dsb[u], acc[dt]);
      }
    }
  };

  // copies per K/V tile per wave (K and V), for the counted waits below
  constexpr int NI = 2 * (kKvTn / (1024 / (2 * D))) / kQWaves;
  if (c0.next_block()) {
    KvPassIter c1 = c0, c2;
    const bool v1 = c1.next();
    bool v2 = false;
    if (v1) {
      c2 = c1;
      v2 = c2.next();
    }
    dma_tile(c0, 0);
    if (v1) dma_tile(c1, 1);
    if (v2) dma_tile(c2, 2);
    if (v2) wait_vm<NI>();  // tiles c0 and c1 are needed now, c2 may stay in flight
    else wait_dma();
    __syncthreads();
    f32x16 sa[2], sb[2];  // scores of half 0 / half 1 of a tile
    bool da = dead(c0);
    if (!da) produce(0, ic<0>{}, sa);
    int sc = 0;
    bool w1 = v1, w2 = v2;
    // One tile (c0) per call; false once the walk is done. The MFMA pipe
    // gets the next half's products before the current half's exponentials
    // are computed; a ring of four stages holds the tile, the next one and
    // two more in flight. The walk's first pass (tiles some rows see only in
    // part) runs the masking copy of the step, the second pass the other.
    auto step = [&](auto MASKc) __attribute__((always_inline)) -> bool {
      KvPassIter c3 = c2;
      const bool v3 = w2 && c3.next();
      const int s1 = (sc + 1) & 3;
      if (v3) dma_tile(c3, (sc + 3) & 3);  // the stage the previous tile freed
      if (!da) {
        produce(sc, ic<1>{}, sb);
        consume(c0, sc, ic<0>{}, sa, MASKc);
      }
      bool db = true;
      if (w1) {
        db = dead(c1);
        if (!db) produce(s1, ic<0>{}, sa);
      }
      if (!da) consume(c0, sc, ic<1>{}, sb, MASKc);
      if (!w1) return false;
      if (v3) wait_vm<NI>();  // tile c2 (read from the next step on) is in LDS
      else wait_dma();
      wg_barrier();  // stage sc is free
      c0 = c1;
      c1 = c2;
      c2 = c3;
      w1 = w2;
      w2 = v3;
      da = db;
      sc = s1;
      return true;
    };
    bool more = true;
    while (more && c0.pass == 0) more = step(ic<1>{});
    while (more) more = step(ic<0>{});
  }

  if (a >= Bb) return;
  __bf16* drow = reinterpret_cast<__bf16*>(p.dq.ptr) + ri * p.dq.s_blk + b * p.dq.s_batch +
                 (int64_t)a * p.dq.s_tok + h * p.dq.s_head;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      bf16x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (__bf16)(acc[dt][4 * g4 + e] * p.scale);
      *reinterpret_cast<bf16x4*>(drow + 32 * dt + 8 * g4 + 4 * hf) = w;
    }
}

// ---------------------------------------------------------------- fp32 path
// Plain VALU kernel for float32: kF32Split lanes per query row, each holding
// a quarter of the row's features (Q, dO and the dQ accumulator); the S and
// dP dot products add the quarters with two lane exchanges. KV tiles are
// staged in LDS; same ring walk and masks as the forward.
constexpr int kF32Rows = 64;
constexpr int kF32Split = 4;  // lanes per row
constexpr int kF32Threads = kF32Rows * kF32Split;

template <int D>
__global__ __launch_bounds__(kF32Threads) void dq_f32_kernel(BwdParams p) {
  constexpr int TN = 2048 / D;  // keys per staged tile: 16 KiB of LDS for K and V
  constexpr int DQ = D / kF32Split;
  __shared__ float ks[TN][D];
  __shared__ float vs[TN][D];
  const int tid = threadIdx.x;
  const int f0 = (tid % kF32Split) * DQ;  // this lane's first feature
  const int32_t BH = p.B * p.H;
  const int32_t Bb = (int32_t)p.Bb;
  const int32_t tiles = (Bb + kF32Rows - 1) / kF32Rows;
  const int64_t id = blockIdx.x;
  const int32_t bh = (int32_t)(id % BH);
  const int32_t b = bh / p.H;
  const int32_t h = bh % p.H;
  int32_t ri, tile;
  query_tile_of(p.causal, p.layout, p.n_ranks, id / BH, tiles, &ri, &tile);
  const int32_t i = p.rank_begin + ri;
  const int32_t a0 = tile * kF32Rows;
  const int32_t a = a0 + tid / kF32Split;
  const int32_t a_hi = (a0 + kF32Rows - 1 < Bb - 1) ? a0 + kF32Rows - 1 : Bb - 1;
  const bool live = a < Bb;
  const float* qrow = reinterpret_cast<const float*>(p.q.ptr) + ri * p.q.s_blk + b * p.q.s_batch +
                      (int64_t)a * p.q.s_tok + h * p.q.s_head + f0;
  const float* orow = reinterpret_cast<const float*>(p.dout.ptr) + ri * p.dout.s_blk + b * p.dout.s_batch +
                      (int64_t)a * p.dout.s_tok + h * p.dout.s_head + f0;
  float qv[DQ], ov[DQ], dq[DQ];
#pragma unroll
  for (int e = 0; e < DQ; ++e) {
    qv[e] = live ? qrow[e] : 0.0f;
    ov[e] = live ? orow[e] : 0.0f;
    dq[e] = 0.0f;
  }
  const int64_t srow = (((int64_t)ri * p.B + b) * p.H + h) * p.Bb;
  const float lse2 = live ? p.lse2[srow + a] : 0.0f;
  const float dsum = live ? p.dsum[srow + a] : 0.0f;
  const float c2 = p.scale_log2;
  for (int32_t kstep = 0; kstep < p.P; ++kstep) {
    const int32_t j = ring_block(i, kstep, p.P);
    const BlockRel rel = block_relation(p.layout, p.causal, i, j, Bb);
    const int64_t extent = visible_key_extent(rel, a_hi, p.Bb);
    if (extent <= 0) continue;
    const int32_t ext_a = row_extent32(rel, a);  // this row sees keys 0 .. ext_a - 1
    const float* kbase = reinterpret_cast<const float*>(p.k.ptr) + (int64_t)j * p.k.s_blk + b * p.k.s_batch +
                         (h / p.G) * p.k.s_head;
    const float* vbase = reinterpret_cast<const float*>(p.v.ptr) + (int64_t)j * p.v.s_blk + b * p.v.s_batch +
                         (h / p.G) * p.v.s_head;
    for (int32_t b0 = 0; b0 < extent; b0 += TN) {
      __syncthreads();
      for (int idx = tid; idx < TN * D; idx += kF32Threads) {
        const int r = idx / D, e = idx % D;
        const int32_t x = b0 + r;
        ks[r][e] = (x < Bb) ? kbase[(int64_t)x * p.k.s_tok + e] : 0.0f;
        vs[r][e] = (x < Bb) ? vbase[(int64_t)x * p.v.s_tok + e] : 0.0f;
      }
      __syncthreads();
      if (!live) continue;  // the four lanes of a row leave together
      for (int u = 0; u < TN; ++u) {
        const int32_t kb = b0 + u;
        float s = 0.0f, dpv = 0.0f;
#pragma unroll
        for (int e = 0; e < DQ; ++e) {
          s = fmaf(qv[e], ks[u][f0 + e], s);
          dpv = fmaf(ov[e], vs[u][f0 + e], dpv);
        }
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        dpv += __shfl_xor(dpv, 1);
        dpv += __shfl_xor(dpv, 2);
        const bool vis = kb < ext_a;
        const float pv = vis ? fexp2(fmaf(s, c2, -lse2)) : 0.0f;
        const float dsv = pv * (dpv - dsum);
#pragma unroll
        for (int e = 0; e < DQ; ++e) dq[e] = fmaf(dsv, ks[u][f0 + e], dq[e]);
      }
    }
  }
  if (!live) return;
  float* drow = reinterpret_cast<float*>(p.dq.ptr) + ri * p.dq.s_blk + b * p.dq.s_batch + (int64_t)a * p.dq.s_tok +
                h * p.dq.s_head + f0;
#pragma unroll
  for (int e = 0; e < DQ; ++e) drow[e] = dq[e] * p.scale;
}

}  // namespace

hipError_t launch_dq_bf16(const BwdParams& p, hipStream_t s) {
  const int64_t grid = ((p.Bb + kQTm - 1) / kQTm) * (int64_t)p.n_ranks * p.B * p.H;
  if (grid <= 0) return hipSuccess;
  if (p.D == 128) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(dq_bf16_kernel<128>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, KvLds<128>::BYTES);
    hipLaunchKernelGGL(dq_bf16_kernel<128>, dim3((uint32_t)grid), dim3(kQThreads), KvLds<128>::BYTES, s, p);
  } else {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(dq_bf16_kernel<64>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, KvLds<64>::BYTES);
    hipLaunchKernelGGL(dq_bf16_kernel<64>, dim3((uint32_t)grid), dim3(kQThreads), KvLds<64>::BYTES, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_dq_f32(const BwdParams& p, hipStream_t s) {
  const int64_t grid = ((p.Bb + kF32Rows - 1) / kF32Rows) * (int64_t)p.n_ranks * p.B * p.H;
  if (grid <= 0) return hipSuccess;
  if (p.D == 128) {
    hipLaunchKernelGGL(dq_f32_kernel<128>, dim3((uint32_t)grid), dim3(kF32Threads), 0, s, p);
  } else {
    hipLaunchKernelGGL(dq_f32_kernel<64>, dim3((uint32_t)grid), dim3(kF32Threads), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace ra
