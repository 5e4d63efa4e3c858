// ra_bwd.hip — backward kernels of exact blockwise ring attention (gfx950).
//
// "Ring Attention 論文分析" (blog), section "逆伝播での KV 再循環": the
// backward walks the same ring, recomputes the probabilities from the saved
// log-sum-exp, P = exp(S - lse), and forms dV = P^T dO, dP = dO V^T,
// dS = P * (dP - D) with D = rowsum(dO * O), dQ = scale * dS K and
// dK = scale * dS^T Q; the dK/dV partials belong to the KV block's owner.
//
// This file holds the dK/dV half: one workgroup owns a tile of 128 keys of KV
// block j for one (batch, K/V head) and carries its dK/dV accumulators on
// chip while the block travels the ring: at step k it meets the query block
// of rank (j + k) mod P, once for each query head that reads this K/V head
// (grouped-query attention sums their contributions). Query tiles the
// causal/striped mask hides from every key of the tile are skipped. The dQ half (ra_dq.hip) walks the ring from
// the query side, so neither half needs atomics.
//
// bf16 path: 8 waves; wave w owns keys 32(w%4) .. +31 of the tile and query
// rows 32(w/4) .. +31 of each 64-row query tile (the two waves sharing keys
// add their dK/dV partials at the end). K and V of the tile and a double
// buffer of Q/dO tiles sit row-major in swizzled LDS, copied there directly
// from global memory; the next query tile is copied while the current one is
// computed. S = Q K^T and
// dP = dO V^T come out with lane (h, n) holding key n against 16 query rows —
// the operand layout dV^T += dO^T P and dK^T += Q^T dS need (contraction over
// query rows, whose order inside an MFMA is free); the dO^T and Q^T operands
// come from transposing LDS reads.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ra_internal.h"
#include "ra_kvwalk.h"
#include "ra_lds.h"
#include "ra_schedule.h"

namespace ra {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kKn = 128;  // keys per workgroup (32 per wave, two waves per key group)
constexpr int kQm = 64;   // query rows per visited tile (32 per wave)

template <int D>
struct BwdLds {
  static constexpr int K = 0;                  // [128][D] swizzled
  static constexpr int V = K + kKn * D;        // [128][D] swizzled
  static constexpr int Q = V + kKn * D;        // [2 stages][64][D] swizzled
  static constexpr int DO = Q + 2 * kQm * D;   // [2 stages][64][D] swizzled
  static constexpr int BF16_ELEMS = DO + 2 * kQm * D;
  static constexpr int F32_OFF = BF16_ELEMS * 2;       // bytes
  static constexpr int BYTES = F32_OFF + 4 * kQm * 4;  // lse2[2][64], dsum[2][64]
  static_assert(4 * ((D / 32) * 16) * 64 * 4 <= F32_OFF, "the dK (then dV) exchange must fit in the tile area");
};

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

// The (rank, query head, query tile) triples a KV tile meets: ranks in ring
// order, and at each rank the G query heads of its K/V head in turn (gi is
// the head's index within the group).
struct QTileIter {
  int32_t kstep, i, gi, qt, qtiles;
  int32_t j, P, G, rb, re, layout, causal, kv0, Bb;
  // the first row of rank i's block that sees the tile's first key, which is
  // the first row that sees any of its keys (Bb if none does)
  __device__ int32_t first_row() const {
    return first_row_seeing32(block_relation(layout, causal, i, j, Bb), kv0, Bb);
  }
  __device__ bool step_rank() {
    while (++kstep < P) {
      i = ring_rank(j, kstep, P);
      if (i < rb || i >= re) continue;
      const int32_t a_first = first_row();
      if (a_first >= Bb) continue;
      qt = a_first / kQm;
      gi = 0;
      return true;
    }
    return false;
  }
  __device__ bool next() {
    if (++qt < qtiles) return true;
    if (++gi < G) {
      qt = first_row() / kQm;
      return true;
    }
    return step_rank();
  }
};

// Copies query tile `it` (Q and dO rows, lse and D) into LDS stage `stage`
// (asynchronous; wait_dma() and a barrier make it visible).
template <int D>
__device__ __forceinline__ void dma_qtile(const BwdParams& p, const QTileIter& it, int32_t b, int32_t h,
                                          __bf16* lds, float* f32s, int stage, int wave, int lane) {
  using L = BwdLds<D>;
  const int32_t ri = it.i - p.rank_begin;
  const int32_t q0 = it.qt * kQm;
  const int32_t Bb = (int32_t)p.Bb;
  const __bf16* qb = reinterpret_cast<const __bf16*>(p.q.ptr) + ri * p.q.s_blk + b * p.q.s_batch + h * p.q.s_head;
  const __bf16* ob = reinterpret_cast<const __bf16*>(p.dout.ptr) + ri * p.dout.s_blk + b * p.dout.s_batch +
                     h * p.dout.s_head;
  // the 4-byte copies go first: issued after the 16-byte ones, they make the
  // compiler wait for those to land
  const int64_t srow = (((int64_t)ri * p.B + b) * p.H + h) * p.Bb;
  if (wave == 0) dma_f32_64(f32s + stage * kQm, p.lse2 + srow, q0, Bb, lane);
  if (wave == 1) dma_f32_64(f32s + 2 * kQm + stage * kQm, p.dsum + srow, q0, Bb, lane);
  dma_rows<D, kQm, kWaves>(lds + L::Q + stage * kQm * D, qb, p.q.s_tok, q0, Bb, wave, lane);
  dma_rows<D, kQm, kWaves>(lds + L::DO + stage * kQm * D, ob, p.dout.s_tok, q0, Bb, wave, lane);
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void dkdv_bf16_kernel(BwdParams p) {
  using L = BwdLds<D>;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __bf16* lds = reinterpret_cast<__bf16*>(smem_raw);
  float* f32s = reinterpret_cast<float*>(smem_raw + L::F32_OFF);  // lse2[2][64], dsum[2][64]

  const int tid = threadIdx.x;
  const int wave = tid / 64;
  const int lane = tid % 64;
  const int n = lane % 32;
  const int hf = lane / 32;
  const int grp = (lane / 16) % 2;
  const int j16 = lane % 16;
  const int kg = wave % 4;
  const int qh = wave / 4;

  const int32_t BHk = p.B * p.Hk;
  const int32_t tiles = (int32_t)((p.Bb + kKn - 1) / kKn);
  // consecutive logical indices share (batch, K/V head, block) and take its
  // key tiles in order (early keys are seen by more rows), so the workgroups
  // of one XCD walk the same query tiles together and share them in L2
  const int64_t lw = xcd_logical(blockIdx.x, (int64_t)BHk * p.P * tiles);
  const int32_t tile = (int32_t)(lw % tiles);
  const int64_t g = lw / tiles;
  const int32_t bhk = (int32_t)(g / p.P);
  const int32_t j = (int32_t)(g % p.P);
  const int32_t b = bhk / p.Hk;
  const int32_t hk = bhk % p.Hk;
  const int32_t Bb = (int32_t)p.Bb;
  const int32_t kv0 = tile * kKn;
  const int32_t kw = kv0 + 32 * kg;  // first key of this wave
  const int32_t key = kw + n;        // this lane's key

  // K and V of the tile, once
  {
    const __bf16* kb = reinterpret_cast<const __bf16*>(p.k.ptr) + j * p.k.s_blk + b * p.k.s_batch + hk * p.k.s_head;
    const __bf16* vb = reinterpret_cast<const __bf16*>(p.v.ptr) + j * p.v.s_blk + b * p.v.s_batch + hk * p.v.s_head;
    dma_rows<D, kKn, kWaves>(lds + L::K, kb, p.k.s_tok, kv0, Bb, wave, lane);
    dma_rows<D, kKn, kWaves>(lds + L::V, vb, p.v.s_tok, kv0, Bb, wave, lane);
  }

  f32x16 dk[D / 32], dv[D / 32];  // dK^T, dV^T: [dt][i] = feature 32dt + 8(i/4) + 4hf + i%4, key n
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    f32x16 z = {};
    dk[dt] = z;
    dv[dt] = z;
  }
  const float c2 = p.scale_log2;

  QTileIter cur;
  cur.kstep = -1;
  cur.qtiles = (Bb + kQm - 1) / kQm;
  cur.j = j;
  cur.P = p.P;
  cur.G = p.G;
  cur.rb = p.rank_begin;
  cur.re = p.rank_begin + p.n_ranks;
  cur.layout = p.layout;
  cur.causal = p.causal;
  cur.kv0 = kv0;
  cur.Bb = Bb;
  const bool any = cur.step_rank();
  if (any) dma_qtile<D>(p, cur, b, hk * p.G + cur.gi, lds, f32s, 0, wave, lane);
  wait_dma();  // K, V and the first query tile
  // LDS addresses (bytes) of this lane's reads, as per-lane bases plus
  // compile-time offsets, so that the walk spends no instructions on them:
  //   bkv[ss]: K row n of the wave's key group, columns 16ss + 8hf (V: + V_B)
  //   bq[ss]:  Q row n of the wave's row half, same columns (query stage ST:
  //            + ST * QST_B; dO: + DO_B)
  //   bt[h2][dt]: transposing reads of Q / dO at rows 4hf + j16/4 + 8h2
  //            (+16kq) of the row half, columns 32dt + 16grp + 4(j16%4)
  //   bl:      lse2 of rows 32qh + 4hf .. of stage 0 (D: + DS_B)
  constexpr int V_B = 2 * (L::V - L::K);
  constexpr int QST_B = 2 * kQm * D;
  constexpr int DO_B = 2 * (L::DO - L::Q);
  constexpr int DS_B = 4 * 2 * kQm;
  static_assert(V_B < 65536 && DO_B + 2 * QST_B <= 65536, "LDS read offsets must fit the 16-bit field");
  const uint32_t lbase = lds_addr(smem_raw);
  uint32_t bkv[D / 16], bq[D / 16], bt[2][D / 32];
#pragma unroll
  for (int ss = 0; ss < D / 16; ++ss) {
    const int c = tile_off<D>(n, 16 * ss + 8 * hf);
    bkv[ss] = lbase + 2 * (L::K + c + 32 * kg * D);
    bq[ss] = lbase + 2 * (L::Q + c + 32 * qh * D);
  }
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
      bt[h2][dt] = lbase + 2 * (L::Q + 32 * qh * D +
                                tile_off<D>(4 * hf + j16 / 4 + 8 * h2, 32 * dt + 16 * grp + 4 * (j16 % 4)));
  const uint32_t bl = lbase + L::F32_OFF + 4 * (32 * qh + 4 * hf);

  // One query tile in stage ST: recompute S and P, dP, dS; dV^T += dO^T P,
  // dK^T += Q^T dS. The next tile is copied into the other stage meanwhile.
  // Returns whether there is a next tile.
  auto step = [&](auto STc) __attribute__((always_inline)) -> bool {
    constexpr int ST = decltype(STc)::value;
    __syncthreads();  // this query stage is in LDS; the other one is no longer read
    QTileIter nx = cur;
    const bool more = nx.next();
    if (more) dma_qtile<D>(p, nx, b, hk * p.G + nx.gi, lds, f32s, ST ^ 1, wave, lane);  // lands during the compute below

    const BlockRel rel = block_relation(p.layout, p.causal, cur.i, j, Bb);
    const int32_t q0 = cur.qt * kQm;
    const int32_t qw = q0 + 32 * qh;  // first row of this wave
    // row extents grow with the row: the wave's last row sees the most keys,
    // its first row the fewest
    const bool dead = (kw >= Bb) || (qw >= Bb) || (row_extent32(rel, qw + 31) <= kw);
    if (!dead) {
      const bool need_mask = (row_extent32(rel, qw) < kw + 32) || (qw + 32 > Bb);
      // rows a >= a_min see this lane's key (only needed when masking)
      const int32_t a_min = need_mask ? first_row_seeing32(rel, key, Bb) : 0;
      // S = Q K^T and dP = dO V^T over the features: the Q, K, dO and V
      // fragments of one 16-feature step are read one step ahead of their
      // MFMAs
      f32x16 s = {}, dp = {};
      u32x4 rg[2][4];
      auto rd = [&](u32x4(&r)[4], int ss) __attribute__((always_inline)) {
        r[0] = lds_read16<ST * QST_B>(bq[ss]);
        r[1] = lds_read16<0>(bkv[ss]);
        r[2] = lds_read16<DO_B + ST * QST_B>(bq[ss]);
        r[3] = lds_read16<V_B>(bkv[ss]);
      };
      rd(rg[0], 0);
#pragma unroll
      for (int ss = 0; ss < D / 16; ++ss) {
        if (ss + 1 < D / 16) {
          rd(rg[(ss + 1) & 1], ss + 1);
          lds_wait<4>(rg[ss & 1]);
        } else {
          lds_wait<0>(rg[ss & 1]);
        }
        s = mfma32(__builtin_bit_cast(bf16x8, rg[ss & 1][0]), __builtin_bit_cast(bf16x8, rg[ss & 1][1]), s);
        dp = mfma32(__builtin_bit_cast(bf16x8, rg[ss & 1][2]), __builtin_bit_cast(bf16x8, rg[ss & 1][3]), dp);
      }
      // lane (hf, n): key n against rows 8(i/4) + 4hf + i%4 of the wave's 32.
      // lse2 and D of rows 8g + 4hf .. +3 are read one group ahead.
      bf16x8 pb[2], dsb[2];
      u32x4 ldr[2][2];  // [slot][lse2, D]
      auto ld_rows = [&](u32x4(&r)[2], int g) __attribute__((always_inline)) {
        switch (g) {
          case 0: r[0] = lds_read16<ST * 4 * kQm + 0>(bl); r[1] = lds_read16<DS_B + ST * 4 * kQm + 0>(bl); break;
          case 1: r[0] = lds_read16<ST * 4 * kQm + 32>(bl); r[1] = lds_read16<DS_B + ST * 4 * kQm + 32>(bl); break;
          case 2: r[0] = lds_read16<ST * 4 * kQm + 64>(bl); r[1] = lds_read16<DS_B + ST * 4 * kQm + 64>(bl); break;
          default: r[0] = lds_read16<ST * 4 * kQm + 96>(bl); r[1] = lds_read16<DS_B + ST * 4 * kQm + 96>(bl); break;
        }
      };
      ld_rows(ldr[0], 0);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (g + 1 < 4) {
          ld_rows(ldr[(g + 1) & 1], g + 1);
          lds_wait<2>(ldr[g & 1]);
        } else {
          lds_wait<0>(ldr[g & 1]);
        }
        const int qr0 = 32 * qh + 8 * g + 4 * hf;  // row within the 64-row tile
        const float4 l4 = __builtin_bit_cast(float4, ldr[g & 1][0]);
        const float4 d4 = __builtin_bit_cast(float4, ldr[g & 1][1]);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};  // lse in log2 units
        const float dd[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * g + e;
          float pv = fexp2(fmaf(s[i], c2, -lv[e]));
          if (need_mask) {
            const int32_t a = q0 + qr0 + e;
            if (a < a_min || a >= Bb) pv = 0.0f;
          }
          const float dsv = pv * (dp[i] - dd[e]);
          pb[g / 2][4 * (g % 2) + e] = (__bf16)pv;
          dsb[g / 2][4 * (g % 2) + e] = (__bf16)dsv;
        }
      }
      // dV^T += dO^T P, dK^T += Q^T dS: contraction over the wave's 32 rows.
      // The transposing reads of (dt, kq) come in groups of 4, one group
      // ahead of their MFMAs.
      auto tr_group = [&](u32x2(&r)[2][2], int idx) __attribute__((always_inline)) {
        const int dt = idx / 2;
        if (idx % 2 == 0) {
          r[0][0] = tr_read_at<DO_B + ST * QST_B>(bt[0][dt]);
          r[0][1] = tr_read_at<DO_B + ST * QST_B>(bt[1][dt]);
          r[1][0] = tr_read_at<ST * QST_B>(bt[0][dt]);
          r[1][1] = tr_read_at<ST * QST_B>(bt[1][dt]);
        } else {
          r[0][0] = tr_read_at<DO_B + ST * QST_B + 16 * D * 2>(bt[0][dt]);
          r[0][1] = tr_read_at<DO_B + ST * QST_B + 16 * D * 2>(bt[1][dt]);
          r[1][0] = tr_read_at<ST * QST_B + 16 * D * 2>(bt[0][dt]);
          r[1][1] = tr_read_at<ST * QST_B + 16 * D * 2>(bt[1][dt]);
        }
      };
      constexpr int NG = 2 * (D / 32);
      u32x2 trg[2][2][2];
      tr_group(trg[0], 0);
#pragma unroll
      for (int idx = 0; idx < NG; ++idx) {
        if (idx + 1 < NG) {
          tr_group(trg[(idx + 1) & 1], idx + 1);
          lds_wait<4>(trg[idx & 1]);
        } else {
          lds_wait<0>(trg[idx & 1]);
        }
        const int dt = idx / 2, kq = idx % 2;
        const bf16x8 ot = __builtin_bit_cast(bf16x8, __builtin_shufflevector(trg[idx & 1][0][0], trg[idx & 1][0][1], 0, 1, 2, 3));
        const bf16x8 qt = __builtin_bit_cast(bf16x8, __builtin_shufflevector(trg[idx & 1][1][0], trg[idx & 1][1][1], 0, 1, 2, 3));
        dv[dt] = mfma32(ot, pb[kq], dv[dt]);
        dk[dt] = mfma32(qt, dsb[kq], dk[dt]);
      }
    }
    if (!more) return false;
    wait_dma();
    cur = nx;
    return true;
  };
  if (any)
    while (step(ic<0>{}) && step(ic<1>{})) {
    }

  // the two waves of a key group add their partial dK^T, then dV^T
  float* red = reinterpret_cast<float*>(smem_raw);  // [4 key groups][D/32*16 values][64 lanes]
  constexpr int NV = (D / 32) * 16;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    f32x16* acc = which == 0 ? dk : dv;
    __syncthreads();  // the LDS area is free
    if (qh == 1) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) red[(kg * NV + dt * 16 + i) * 64 + lane] = acc[dt][i];
    }
    __syncthreads();
    if (qh == 0) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[dt][i] += red[(kg * NV + dt * 16 + i) * 64 + lane];
    }
  }
  if (qh == 1 || key >= Bb) return;
  __bf16* dkrow = reinterpret_cast<__bf16*>(p.dk.ptr) + j * p.dk.s_blk + b * p.dk.s_batch +
                  (int64_t)key * p.dk.s_tok + hk * p.dk.s_head;
  __bf16* dvrow = reinterpret_cast<__bf16*>(p.dv.ptr) + j * p.dv.s_blk + b * p.dv.s_batch +
                  (int64_t)key * p.dv.s_tok + hk * p.dv.s_head;
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
// dK/dV of that key in registers, query tiles of 32 rows staged in LDS (dQ:
// dq_f32_kernel).
constexpr int kF32Keys = 64;
constexpr int kF32Rows = 32;

template <int D>
struct BwdF32Lds {
  static constexpr int S = D + 1;  // padded rows: per-lane own-row reads are conflict-free
  static constexpr int KS = 0;
  static constexpr int VS = KS + kF32Keys * S;
  static constexpr int QS = VS + kF32Keys * S;
  static constexpr int OS = QS + kF32Rows * S;
  static constexpr int LSE = OS + kF32Rows * S;
  static constexpr int DSUM = LSE + kF32Rows;
  static constexpr int FLOATS = DSUM + kF32Rows;
  static constexpr int BYTES = FLOATS * 4;
};

template <int D>
__global__ __launch_bounds__(kF32Keys) void dkdv_f32_kernel(BwdParams p) {
  using L = BwdF32Lds<D>;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  float* sm = reinterpret_cast<float*>(smem_raw);
  float* ks = sm + L::KS;
  float* vs = sm + L::VS;
  float* qs = sm + L::QS;
  float* os = sm + L::OS;
  float* lse_s = sm + L::LSE;
  float* dsum_s = sm + L::DSUM;
  const int tid = threadIdx.x;
  const int32_t BHk = p.B * p.Hk;
  const int32_t tiles = (int32_t)((p.Bb + kF32Keys - 1) / kF32Keys);
  const int64_t id = blockIdx.x;
  const int32_t bhk = (int32_t)(id % BHk);
  const int32_t b = bhk / p.Hk;
  const int32_t hk = bhk % p.Hk;
  int32_t j, tile;
  kv_tile_of(p, id / BHk, tiles, &j, &tile);
  const int64_t kv0 = (int64_t)tile * kF32Keys;
  const int64_t key = kv0 + tid;
  const float* kbase = reinterpret_cast<const float*>(p.k.ptr) + j * p.k.s_blk + b * p.k.s_batch + hk * p.k.s_head;
  const float* vbase = reinterpret_cast<const float*>(p.v.ptr) + j * p.v.s_blk + b * p.v.s_batch + hk * p.v.s_head;
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
    const BlockRel rel = block_relation(p.layout, p.causal, i, j, (int32_t)p.Bb);
    if (rel.kind == kNone) continue;
    const int64_t a_first = first_row_seeing(rel, kv0, p.Bb);  // first row that sees the tile
    if (a_first >= p.Bb) continue;
    const int64_t a_min = first_row_seeing(rel, key, p.Bb);  // rows a >= a_min see this lane's key
    for (int32_t gi = 0; gi < p.G; ++gi) {  // the query heads that read this K/V head
      const int32_t h = hk * p.G + gi;
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
          lse_s[tid] = (x < p.Bb) ? p.lse2[srow + x] : 0.0f;
          dsum_s[tid] = (x < p.Bb) ? p.dsum[srow + x] : 0.0f;
        }
        __syncthreads();
        for (int r = 0; r < kF32Rows; ++r) {
          const int64_t a = q0 + r;
          const bool vis = key < p.Bb && a < p.Bb && a >= a_min;
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
        }
      }
    }
  }
  if (key >= p.Bb) return;
  float* dkrow = reinterpret_cast<float*>(p.dk.ptr) + j * p.dk.s_blk + b * p.dk.s_batch + key * p.dk.s_tok + hk * p.dk.s_head;
  float* dvrow = reinterpret_cast<float*>(p.dv.ptr) + j * p.dv.s_blk + b * p.dv.s_batch + key * p.dv.s_tok + hk * p.dv.s_head;
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

hipError_t launch_dkdv_bf16(const BwdParams& p, hipStream_t s) {
  const int64_t grid = ((p.Bb + kKn - 1) / kKn) * (int64_t)p.P * p.B * p.Hk;
  if (p.D == 128) return launch_dyn(dkdv_bf16_kernel<128>, grid, kThreads, BwdLds<128>::BYTES, s, p);
  return launch_dyn(dkdv_bf16_kernel<64>, grid, kThreads, BwdLds<64>::BYTES, s, p);
}

hipError_t launch_dkdv_f32(const BwdParams& p, hipStream_t s) {
  const int64_t grid = ((p.Bb + kF32Keys - 1) / kF32Keys) * (int64_t)p.P * p.B * p.Hk;
  if (p.D == 128) return launch_dyn(dkdv_f32_kernel<128>, grid, kF32Keys, BwdF32Lds<128>::BYTES, s, p);
  return launch_dyn(dkdv_f32_kernel<64>, grid, kF32Keys, BwdF32Lds<64>::BYTES, s, p);
}

}  // namespace ra
