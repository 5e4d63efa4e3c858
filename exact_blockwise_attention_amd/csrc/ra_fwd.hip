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
// fp32 sums and representable in bf16. The row sum adds the bf16-rounded
// probabilities, the same values the P V product uses. lse is exported as a
// natural log.
//
// Schedule. The 8 waves form two groups, waves 0-3 and 4-7; waves w and
// w + 4 share a SIMD. Each wave alternates a matrix phase (the next tile's
// scores and this tile's P V product: 32 MFMAs) and a vector phase (mask,
// max, exponentials of the next tile). Workgroup barriers separate the
// phases and group 1 runs one phase behind group 0, so on every SIMD one
// wave feeds the matrix core while the other does the softmax. KV tiles go
// straight from global memory to a ring of four LDS stages (K tiles in the
// lower half of LDS, V tiles in the upper half); each group copies its half
// of a tile between the products of its matrix phase, three (group 1) or
// four (group 0) phases before the tile's first use.
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

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescaleSlack = 8.0f;  // log2 units a tile max may exceed the reference max

// LDS of the bf16 forward: NST stages of a K tile and a V tile ([64][D],
// swizzled), K tiles first.
template <int D>
struct FwdLds {
  static constexpr int NST = 4;
  static constexpr int TILE_B = kKvTn * D * 2;  // bytes of one tile
  static constexpr int VBASE_B = NST * TILE_B;  // byte offset of the V tiles
  static constexpr int BYTES = 2 * NST * TILE_B;
};

// Direct copies of a 64-row tile: a wave instruction moves 1 KB (RW rows);
// each wave issues CPW of them per tensor.
template <int D>
struct FwdDma {
  static constexpr int RW = 1024 / (2 * D);
  static constexpr int CPR = D / 8;  // 16-byte chunks per row
  static constexpr int CPW = kKvTn / RW / kQWaves;
  static constexpr int NI = 2 * CPW;  // instructions per tile per wave (K and V)
  static_assert(CPW >= 1 && (kKvTn / RW) % kQWaves == 0, "tile copies must split over the waves");
  static_assert(NI == D / 32, "a matrix phase issues one copy per feature group");
};

// max over the two half-waves (lanes n and n ^ 32)
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <int D>
__global__ __launch_bounds__(kQThreads, 1) void fwd_bf16_kernel(FwdParams p) {
  using L = FwdLds<D>;
  using DM = FwdDma<D>;
  extern __shared__ __align__(16) unsigned char smem_raw[];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64;
  const int n = lane % 32;
  const int hf = lane / 32;
  const int grp = (lane / 16) % 2;
  const int j16 = lane % 16;
  const bool g1 = wave >= kQWaves / 2;  // second ping-pong group

  const int32_t BH = p.B * p.H;
  const int32_t Bb = (int32_t)p.Bb;
  const int32_t tiles = (Bb + kQTm - 1) / kQTm;
  int32_t bh, ri, tile;
  // striped causal query tiles drift apart at every block: equal turns
  // (when G is a multiple of 4, the G query heads of a tile already make
  // every turn's workgroups equal, and the tiles stay together)
  const bool turns = p.causal && p.layout == kStriped && p.G % 4 != 0;
  // split launch: workgroup id = run * (query tiles of the range) + tile id
  const int64_t per_run = (int64_t)BH * p.n_ranks * tiles;
  const int32_t run = (p.mode == 2) ? (int32_t)(blockIdx.x / per_run) : 0;
  const int64_t wid = (p.mode == 2) ? (int64_t)(blockIdx.x % per_run) : (int64_t)blockIdx.x;
  query_work_of(wid, BH, p.G, p.n_ranks, tiles, p.causal, p.layout, turns, &bh, &ri, &tile);
  const int32_t b = bh / p.H;
  const int32_t h = bh % p.H;
  const int32_t hk = h / p.G;  // the K/V head this query head reads
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
  // state slot of this workgroup's run (split launch), in rows
  const int64_t slot = (p.mode == 2) ? (int64_t)run * p.n_ranks * BH * p.Bb : 0;
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

  // per-lane byte offsets inside a stage: K rows n (+32t) at columns
  // 16ss + 8hf; V^T transposing reads (LDS addresses of stage 0) at rows
  // 4hf + j16/4 (+8) (+16kk) and columns 32dt + 16grp + 4(j16%4)
  uint32_t koff[D / 16], voff[2][D / 32];
#pragma unroll
  for (int ss = 0; ss < D / 16; ++ss) koff[ss] = lds_addr(smem_raw) + 2 * tile_off<D>(n, 16 * ss + 8 * hf);
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
      voff[h2][dt] = lds_addr(smem_raw) + L::VBASE_B +
                     2 * tile_off<D>(4 * hf + j16 / 4 + 8 * h2, 32 * dt + 16 * grp + 4 * (j16 % 4));

  // per-lane source offsets (bytes, from the tile's first row) of the rows
  // this wave copies, and their swizzled chunk
  // (crow: the row, c16: the chunk's byte offset, for the copies of a tile
  // cut by the block's end)
  uint32_t dk[DM::CPW], dv[DM::CPW];
  int32_t crow[DM::CPW];
  uint32_t c16[DM::CPW];
#pragma unroll
  for (int kc = 0; kc < DM::CPW; ++kc) {
    const int row = (wave + kQWaves * kc) * DM::RW + lane / DM::CPR;
    const int c = (lane % DM::CPR) ^ chunk_swz<D>(row);
    dk[kc] = (uint32_t)(2 * ((int64_t)row * p.k.s_tok + 8 * c));
    dv[kc] = (uint32_t)(2 * ((int64_t)row * p.v.s_tok + 8 * c));
    crow[kc] = row;
    c16[kc] = 16 * c;
  }
  const int64_t kvblk_mul = (p.mode == 1) ? 0 : 1;  // the single-step buffer holds one block
  auto kv_base = [&](const Seq& sq, int32_t blk, int32_t r_lo) __attribute__((always_inline)) {
    return reinterpret_cast<const char*>(reinterpret_cast<const __bf16*>(sq.ptr) + kvblk_mul * blk * sq.s_blk +
                                         b * sq.s_batch + hk * sq.s_head + (int64_t)r_lo * sq.s_tok);
  };
  // Requests tile t into stage ST: this wave's CPW row groups of K and of V.
  // Rows at or beyond Bb read row Bb - 1 (finite data; masked later).
  auto dma = [&](const KvIter& t, auto STc) __attribute__((always_inline)) {
    constexpr int ST = decltype(STc)::value;
    const int32_t r_lo = t.t * kKvTn;
    const char* kb = kv_base(p.k, t.j, r_lo);
    const char* vb = kv_base(p.v, t.j, r_lo);
    unsigned char* kd = smem_raw + ST * L::TILE_B;
    unsigned char* vd = smem_raw + L::VBASE_B + ST * L::TILE_B;
    if (r_lo + kKvTn <= Bb) {
#pragma unroll
      for (int kc = 0; kc < DM::CPW; ++kc) {
        const int q = wave + kQWaves * kc;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const __bf16*>(kb + dk[kc]), (__attribute__((address_space(3))) void*)(kd + q * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const __bf16*>(vb + dv[kc]), (__attribute__((address_space(3))) void*)(vd + q * 1024), 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int kc = 0; kc < DM::CPW; ++kc) {
        const int q = wave + kQWaves * kc;
        int row = q * DM::RW + lane / DM::CPR;
        const int c = (lane % DM::CPR) ^ chunk_swz<D>(row);
        if (row > Bb - 1 - r_lo) row = Bb - 1 - r_lo;
        const int64_t ko = 2 * ((int64_t)row * p.k.s_tok + 8 * c), vo = 2 * ((int64_t)row * p.v.s_tok + 8 * c);
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const __bf16*>(kb + ko), (__attribute__((address_space(3))) void*)(kd + q * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const __bf16*>(vb + vo), (__attribute__((address_space(3))) void*)(vd + q * 1024), 16, 0, 0);
      }
    }
  };
  // The same copies one at a time, so that a matrix phase can spread them
  // between its products: copy I < CPW is K row group I, the others V row
  // group I - CPW. CopySrc holds the tile's first source rows.
  struct CopySrc {
    const char *kb, *vb;
    int32_t lim;  // last row of the tile inside the block
  };
  auto copy_src = [&](const KvIter& t) __attribute__((always_inline)) {
    const int32_t r_lo = t.t * kKvTn;
    CopySrc c;
    c.kb = kv_base(p.k, t.j, r_lo);
    c.vb = kv_base(p.v, t.j, r_lo);
    c.lim = Bb - 1 - r_lo;
    return c;
  };
  // (no branch: the matrix phase has LDS reads in flight around the copies)
  auto copy_one = [&](const CopySrc& c, auto STc, int I) __attribute__((always_inline)) {
    constexpr int ST = decltype(STc)::value;
    const bool isv = I >= DM::CPW;
    const int kc = I % DM::CPW;
    const int q = wave + kQWaves * kc;
    // a tile cut by the block's end: rows past it read the last row
    const int32_t lim = c.lim < kKvTn - 1 ? c.lim : kKvTn - 1;
    const uint32_t last = (uint32_t)(2 * (int64_t)lim * (isv ? p.v.s_tok : p.k.s_tok)) + c16[kc];
    const uint32_t off = crow[kc] > lim ? last : (isv ? dv[kc] : dk[kc]);
    unsigned char* dst = smem_raw + (isv ? L::VBASE_B : 0) + ST * L::TILE_B + q * 1024;
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const __bf16*>((isv ? c.vb : c.kb) + off),
                                     (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
  };

  const float c2 = p.scale_log2;
  f32x16 s[2];    // S^T of the tile in flight (32 keys each)
  bf16x8 pb[4];   // its probabilities, B operand of the P V product
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  // S^T = K Q^T for the 64 keys in stage ST: the two 32-key halves take
  // turns on the MFMA pipe, and the K fragments of feature step ss + 1 are
  // requested before the products of step ss
  auto scores = [&](auto STc) __attribute__((always_inline)) {
    constexpr int ST = decltype(STc)::value;
    constexpr int NSS = D / 16;
    u32x4 kf[2][2];  // [slot][half]
    kf[0][0] = lds_read16<ST * L::TILE_B>(koff[0]);
    kf[0][1] = lds_read16<ST * L::TILE_B + 32 * D * 2>(koff[0]);
    const f32x16 z = {};
#pragma unroll
    for (int ss = 0; ss < NSS; ++ss) {
      if (ss + 1 < NSS) {
        kf[(ss + 1) & 1][0] = lds_read16<ST * L::TILE_B>(koff[ss + 1]);
        kf[(ss + 1) & 1][1] = lds_read16<ST * L::TILE_B + 32 * D * 2>(koff[ss + 1]);
        lds_wait<2>(kf[ss & 1]);
      } else {
        lds_wait<0>(kf[ss & 1]);
      }
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
        s[t2] = mfma32(__builtin_bit_cast(bf16x8, kf[ss & 1][t2]), qreg[ss], ss == 0 ? z : s[t2]);
    }
  };
  // Matrix phase: scores of the tile in stage SK (if any) and O^T += V^T P^T
  // with the V tile in stage SV. The V^T fragments of one 32-feature group
  // (4 k-steps x 2 halves) are requested one group ahead of their MFMAs.
  auto matrix = [&](auto SKc, auto SVc, const CopySrc& cs, auto SCc) __attribute__((always_inline)) {
    constexpr int SV = decltype(SVc)::value;
    u32x2 vf[2][4][2];
    auto request = [&](u32x2(&r)[4][2], int dt) __attribute__((always_inline)) {
      // the addresses are loop-invariant; computing them here keeps the
      // compiler from holding all of them in registers across the walk
      const uint32_t o0 = opaque(voff[0][dt]), o1 = opaque(voff[1][dt]);
      r[0][0] = tr_read_at<SV * L::TILE_B + 0 * 16 * D * 2>(o0);
      r[0][1] = tr_read_at<SV * L::TILE_B + 0 * 16 * D * 2>(o1);
      r[1][0] = tr_read_at<SV * L::TILE_B + 1 * 16 * D * 2>(o0);
      r[1][1] = tr_read_at<SV * L::TILE_B + 1 * 16 * D * 2>(o1);
      r[2][0] = tr_read_at<SV * L::TILE_B + 2 * 16 * D * 2>(o0);
      r[2][1] = tr_read_at<SV * L::TILE_B + 2 * 16 * D * 2>(o1);
      r[3][0] = tr_read_at<SV * L::TILE_B + 3 * 16 * D * 2>(o0);
      r[3][1] = tr_read_at<SV * L::TILE_B + 3 * 16 * D * 2>(o1);
    };
    request(vf[0], 0);
    scores(SKc);  // on the last tile: of the spare copy in stage SK (finite, unused)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      if (dt + 1 < D / 32) {
        request(vf[(dt + 1) & 1], dt + 1);
        lds_wait<8>(vf[dt & 1]);
      } else {
        lds_wait<0>(vf[dt & 1]);
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 a8 = __builtin_bit_cast(bf16x8, __builtin_shufflevector(vf[dt & 1][kk][0], vf[dt & 1][kk][1], 0, 1, 2, 3));
        acc[dt] = mfma32(a8, pb[kk], acc[dt]);
      }
      // one tile copy per feature group (D / 32 groups, as many copies)
      copy_one(cs, SCc, dt);
    }
  };
  // Vector phase of tile t (scores in s): mask, running max, probabilities,
  // row sums. Rows whose keys are all masked keep a zero weight.
  auto softmax = [&](const KvIter& t) __attribute__((always_inline)) {
    const int32_t b0 = t.t * kKvTn;
    // the wave's first row sees the fewest keys (row extents grow with the
    // row; they never exceed Bb, which covers the ragged last tile)
    if (t.ext_w < b0 + kKvTn) {
      // key b0 + off is visible iff off < ext(a) - b0
      const int32_t lim = row_extent32(t.rel, a) - 1 - b0;
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
    mx = halves_max(mx);
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
    const float m_use = (m == -INFINITY) ? 0.0f : m;
    // P element e of k-step kk is key 16kk + 8(e/4) + 4hf + e%4
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int e = 0; e < 16; ++e) pb[2 * t2 + e / 8][e % 8] = (__bf16)fexp2(fmaf(s[t2][e], c2, -m_use));
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2)
      {
        const bf16x2 pr = {pb[kk][2 * e2], pb[kk][2 * e2 + 1]};
        l = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l, false);
      }
  };

  KvIter first;
  // ring steps walked: all, one received block, or this run's steps
  first.kstep = (p.mode == 2) ? (int32_t)((int64_t)run * p.P / p.n_split) - 1 : -1;
  first.nsteps = (p.mode == 0) ? p.P : (p.mode == 1) ? 1 : (int32_t)((int64_t)(run + 1) * p.P / p.n_split);
  first.single_block = (p.mode == 1) ? p.step_block : -1;
  first.i = i;
  first.P = p.P;
  first.layout = p.layout;
  first.causal = p.causal;
  first.a_hi = a_hi;
  first.Bb = Bb;
  first.a_w = aw;
  if (first.next_block()) {
    // DMA walk: sticks at the last tile once the walk is done, so that the
    // copies issued for tiles past the end re-read valid rows into a free
    // stage and every wave issues the same number of loads per phase.
    KvIter itd = first;
    bool dvalid = true;
    // the copies' source rows follow the walk: one tile further down the
    // same block, or a new block's first tile
    CopySrc cur = copy_src(itd);
    const int64_t kadv = 2 * (int64_t)kKvTn * p.k.s_tok, vadv = 2 * (int64_t)kKvTn * p.v.s_tok;
    auto dadv = [&]() __attribute__((always_inline)) {
      if (dvalid) {
        KvIter nx = itd;
        if (nx.next()) {
          if (nx.t == 0) {
            cur = copy_src(nx);
          } else {
            cur.kb += kadv;
            cur.vb += vadv;
            cur.lim -= kKvTn;
          }
          itd = nx;
        } else {
          dvalid = false;
        }
      }
    };
    // prologue: tiles 0..2 (group 1 also tile 3, which group 0 requests in
    // its first phase); tile 0's scores and probabilities
    dma(itd, ic<0>{});
    dadv();
    dma(itd, ic<1>{});
    dadv();
    dma(itd, ic<2>{});
    dadv();
    wait_vm<2 * DM::NI>();  // tile 0
    wg_barrier();
    // a wave whose rows all lie past the block's end (a block shorter than
    // the workgroup's 256 rows) keeps to the copies and barriers only
    const bool busy = aw < Bb;
    KvIter its = first;  // the tile whose scores are in s
    if (busy) {
      scores(ic<0>{});
      softmax(its);
    }
    if (g1) {
      wait_vm<DM::NI>();  // tile 1: group 0 reads it in the next phase
      wg_barrier();
    }
    // Phase pair t: [matrix: scores of tile t+1, P V of tile t] then
    // [vector: softmax of tile t+1]. Stage of tile t is t % 4. Each group
    // copies its half of tile t+3 during its own matrix phase, into the
    // stage of tile t-1: group 1 read that stage last, before the barrier
    // that opens group 0's matrix phase. Every wave waits for its copies of
    // tile t+2 before the barrier that opens group 0's next matrix phase
    // (group 0 at the top of the next step, group 1 at the end of its own
    // matrix phase), so the one copy of a tile in flight is t+3's.
    auto step = [&](auto Uc) __attribute__((always_inline)) -> bool {
      constexpr int U = decltype(Uc)::value;
      KvIter nx = its;
      const bool has_next = nx.next();
      if (!g1) wait_vm<DM::NI>();  // tile t+1 (its K is read now)
      wg_barrier();
      // the matrix phase takes the SIMD's issue slots first: the hardware
      // otherwise favours the older waves (group 0) in both phases
      __builtin_amdgcn_s_setprio(1);
      const CopySrc cs = cur;  // tile t+3 into the stage tile t-1 freed
      if (busy) {
        matrix(ic<(U + 1) % 4>{}, ic<U>{}, cs, ic<(U + 3) % 4>{});
      } else {
#pragma unroll
        for (int c = 0; c < DM::NI; ++c) copy_one(cs, ic<(U + 3) % 4>{}, c);
      }
      dadv();
      if (g1) wait_vm<DM::NI>();  // tile t+2, read by group 0 in the next phase
      __builtin_amdgcn_s_setprio(0);
      wg_barrier();
      if (has_next) {
        its = nx;
        if (busy) softmax(its);
      }
      return has_next;
    };
    while (step(ic<0>{}) && step(ic<1>{}) && step(ic<2>{}) && step(ic<3>{})) {
    }
    if (!g1) wg_barrier();  // group 1 started one barrier ahead
    wait_vm<0>();           // no copy may land after the workgroup ends
  }

  // finalise: combine the two halves' sums, normalise, export
  const float l_tot = l + __shfl_xor(l, 32);
  const float m_use = (m == -INFINITY) ? 0.0f : m;
  const float inv = (l_tot > 0.0f) ? 1.0f / l_tot : 0.0f;
  if (a >= Bb) return;
  if (p.mode == 0 || (p.mode == 1 && p.last)) {
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
        *reinterpret_cast<float4*>(p.st_o + (slot + srow + a) * D + 32 * dt + 8 * g4 + 4 * hf) = v4;
      }
    if (hf == 0) p.st_lse[slot + srow + a] = (l_tot > 0.0f) ? m_use + log2f(l_tot) : -INFINITY;
  }
}

// Work order for the fp32 kernel (64-row tiles); same rule as query_tile_of.
__device__ __forceinline__ void tile_of(const FwdParams& p, int64_t ord, int32_t tiles, int32_t* rank_idx,
                                        int32_t* tile) {
  query_tile_of(p.causal, p.layout, p.n_ranks, ord, tiles, rank_idx, tile);
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
    const BlockRel rel = block_relation(p.layout, p.causal, i, j, (int32_t)p.Bb);
    const int64_t extent = visible_key_extent(rel, a_hi, p.Bb);
    if (extent <= 0) continue;
    const int64_t ext_a = row_extent(rel, a);  // this row sees keys 0 .. ext_a - 1
    const int64_t kblk = (p.mode == 0) ? (int64_t)j : 0;
    const float* kbase = reinterpret_cast<const float*>(p.k.ptr) + kblk * p.k.s_blk + b * p.k.s_batch +
                         (h / p.G) * p.k.s_head;
    const float* vbase = reinterpret_cast<const float*>(p.v.ptr) + kblk * p.v.s_blk + b * p.v.s_batch +
                         (h / p.G) * p.v.s_head;
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
          sc[u] = (kb >= ext_a) ? -INFINITY : dot;
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
  const int64_t grid = tiles * p.n_ranks * p.B * p.H * (p.mode == 2 ? p.n_split : 1);
  if (grid <= 0) return hipSuccess;
  if (p.D == 128) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(fwd_bf16_kernel<128>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, FwdLds<128>::BYTES);
    hipLaunchKernelGGL(fwd_bf16_kernel<128>, dim3((uint32_t)grid), dim3(kQThreads), FwdLds<128>::BYTES, s, p);
  } else {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(fwd_bf16_kernel<64>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, FwdLds<64>::BYTES);
    hipLaunchKernelGGL(fwd_bf16_kernel<64>, dim3((uint32_t)grid), dim3(kQThreads), FwdLds<64>::BYTES, s, p);
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
