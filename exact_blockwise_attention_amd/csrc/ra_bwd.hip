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
// causal / striped / zigzag mask hides from every key of the tile are
// skipped. The dQ half (ra_dq.hip) walks the ring from the query side, so
// neither half needs atomics.
//
// S = Q K^T and dP = dO V^T come out with lane (h, n) holding key n against
// 16 query rows: the operand layout dV^T += dO^T P and dK^T += Q^T dS need
// (contraction over query rows, whose order inside an MFMA is free); the
// dO^T and Q^T operands come from transposing LDS reads.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ra_internal.h"
#include "ra_kvwalk.h"
#include "ra_lds.h"
#include "ra_schedule.h"

namespace ra {
namespace {

constexpr int kKn = 128;  // keys per workgroup (32 per wave)
constexpr int kQm = 64;   // query rows per visited tile

// Heaviest KV tiles first: early keys are seen by more query rows.
__device__ __forceinline__ void kv_tile_of(const BwdParams& p, int64_t ord, int32_t tiles, int32_t* j,
                                           int32_t* tile) {
  // (selects on the values, not on where they go: the kernels keep j and
  // tile in registers)
  const bool by_block = p.causal && p.layout == kContiguous;
  const int64_t div = by_block ? tiles : p.P;
  const int32_t q = (int32_t)(ord / div), r = (int32_t)(ord % div);
  *j = by_block ? q : r;
  *tile = by_block ? r : q;
}

// ---------------------------------------------------------------- bf16 path
// 4 waves of 32 keys each, every wave taking all 64 rows
// of each query tile. A wave holds its K and V rows in registers for the
// whole walk (the B operands of S = Q K^T and dP = dO V^T), so only Q, dO,
// lse and D go through LDS, in a ring of four stages copied two tiles ahead.
// With a single wave per SIMD the matrix and vector work overlap inside the
// wave: a step is a two-phase software pipeline over 32-row blocks, every
// phase interleaving the S / dP products of one row block, the P / dS of
// the row block before it and the dV^T += dO^T P, dK^T += Q^T dS products
// of the row block before that, slot by slot.
//
// The copies are bounds-checked buffer loads whose range ends at the last
// row of the block, so rows past it arrive as zeros (Q = dO = lse = D = 0,
// hence dS = 0 and a zero dO row: they add nothing). Every step copies
// exactly one tile (the tile two steps ahead, or the last one again once
// the walk has no more), and every wave issues the same number of copies per
// tile (waves 2 and 3 copy a spare lse row), so a fixed count of outstanding
// copies tells each wave that its current tile has landed.
constexpr int kWaves = 4;          // waves
constexpr int kThreads = 64 * kWaves;   // threads
constexpr int kNst = 4;        // query-tile stages
constexpr int kRawRsrcWord3 = 0x00020000;  // untyped 32-bit data, bounds-checked raw buffer

template <int D>
struct BwdLds {
  static constexpr int QST_B = kQm * D * 2;         // one tile of Q (or dO), bytes
  static constexpr int DO0 = kNst * QST_B;          // the dO tiles of the stages, after their Q tiles
  static constexpr int F32_B = 2 * kNst * QST_B;    // lse2[4][64], then dsum[4][64], then 2 spare rows
  static constexpr int DS_B = kNst * kQm * 4;      // dsum after lse2
  static constexpr int SPARE_B = F32_B + 2 * DS_B;  // [2][64] floats, written by waves 2 and 3
  static constexpr int BYTES = SPARE_B + 2 * kQm * 4;
  static_assert(BYTES <= 160 * 1024, "LDS");
  // a read names its stage in the instruction's offset (from a Q or a dO base)
  static_assert((kNst - 1) * QST_B + 48 * D * 2 < 65536, "DS offsets are 16 bits");
};

// s_waitcnt lgkmcnt(N) with the registers of one read group tied to it.
template <int N, int A, int B>
__device__ __forceinline__ void lds_wait_grp(u32x4 (&r)[A], u32x2 (&t)[B]) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt range");
  if constexpr (A == 4 && B == 4) {
    asm volatile("s_waitcnt lgkmcnt(%8)"
                 : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(t[0]), "+v"(t[1]), "+v"(t[2]), "+v"(t[3])
                 : "n"(N));
  } else if constexpr (A == 2 && B == 4) {
    asm volatile("s_waitcnt lgkmcnt(%6)"
                 : "+v"(r[0]), "+v"(r[1]), "+v"(t[0]), "+v"(t[1]), "+v"(t[2]), "+v"(t[3])
                 : "n"(N));
  } else {
    static_assert(A == 0, "read group shape");
  }
}

template <int N>
__device__ __forceinline__ void lds_wait_grp2(u32x4 (&r)[2], u32x4 (&t)[2]) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(r[0]), "+v"(r[1]), "+v"(t[0]), "+v"(t[1]) : "n"(N));
}

// One query tile as its copies see it: the first byte of its Q and dO rows
// and of its lse2 and D entries, and how many of its rows lie in the block.
struct QTileSrc {
  const unsigned char *q, *o;
  const float *l, *d;
  int32_t rows;
};

// S / dP products with the accumulator in VGPRs and the K / V operand in
// AGPRs: the vector work reads the scores without copying them out of
// AGPRs first. The operands' producers are far from these products (LDS
// reads retired by an explicit wait; K and V loaded once), and their
// results are read in the next phase, hundreds of instructions later.
__device__ __forceinline__ void mfma_s(f32x16& acc, const u32x4& a, const bf16x8& b, bool zero) {
  if (zero) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(acc) : "v"(a), "a"(b));
  } else {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "a"(b));
  }
}

template <int D, bool STORE_DS>
__global__ __launch_bounds__(kThreads, 1) void dkdv_bf16_kernel(BwdParams p) {
  using L = BwdLds<D>;
  constexpr int NSS = D / 16;          // 16-feature steps of the S / dP products
  constexpr int NDT = D / 32;          // 32-feature tiles of dK^T / dV^T
  constexpr int RW = 1024 / (2 * D);   // rows per 1 KB copy
  constexpr int CPR = D / 8;           // 16-byte chunks per row
  constexpr int NCP = kQm / RW / kWaves;  // row copies per wave per tensor
  constexpr int NCOPY = 2 * NCP + 1;   // copies per wave per tile
  constexpr int kCopiesA = NCP + 1;    // of which phase A issues lse2 / D and Q
  static_assert(kCopiesA < NSS && NCOPY - kCopiesA < NSS, "one copy per slot");
  static_assert(2 * NDT == NSS, "one pair of dV products per feature step");
  extern __shared__ __align__(16) unsigned char smem_raw[];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64;
  const int n = lane % 32;
  const int hf = lane / 32;
  const int grp = (lane / 16) % 2;
  const int j16 = lane % 16;

  const int32_t BHk = p.B * p.Hk;
  const int32_t tiles = (int32_t)((p.Bb + kKn - 1) / kKn);
  const uint32_t lw = (uint32_t)xcd_logical(blockIdx.x, (int64_t)BHk * p.P * tiles);
  // key tiles of a block heaviest first (its first keys are seen by the most
  // query rows), ordered so that the shader engines get equal work; striped
  // causal key tiles drift apart at every rank, so there equal turns
  uint32_t g, wit;
  if (p.causal && p.layout == kStriped) {
    turn_balanced_split(lw, (uint32_t)(BHk * p.P), (uint32_t)tiles, &g, &wit);
  } else {
    g = lw / (uint32_t)tiles;
    wit = se_balanced_rank(lw % (uint32_t)tiles, (uint32_t)tiles);
  }
  const int32_t tile = (int32_t)wit;
  const int32_t bhk = (int32_t)(g / (uint32_t)p.P);
  const int32_t j = (int32_t)(g % (uint32_t)p.P);
  const int32_t b = bhk / p.Hk;
  const int32_t hk = bhk % p.Hk;
  const int32_t Bb = (int32_t)p.Bb;
  const int32_t kv0 = tile * kKn;
  const int32_t kw = kv0 + 32 * wave;  // first key of this wave
  const int32_t key = kw + n;          // this lane's key
  const int32_t qtiles = (Bb + kQm - 1) / kQm;

  f32x16 dk[NDT], dv[NDT];  // dK^T, dV^T: [dt][i] = feature 32dt + 8(i/4) + 4hf + i%4, key n
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    dk[dt] = f32x16{};
    dv[dt] = f32x16{};
  }

  // The walk, in two passes over the ranks (ring order) and, at each rank,
  // the G query heads of this K/V head: first the query tiles in which some
  // row does not see some key of the tile (the causal diagonal), then the
  // tiles every row of which sees every key. Row extents grow with the row,
  // so at each rank the first kind is a run of tiles [wq_first, wq_full)
  // and the second the rest up to the last tile; each pass runs its own copy
  // of the step, and only the first masks. (wc, wgi, wqt) is the tile to
  // copy next, wc numbering the (pass, ring step) pairs pass-major; per
  // pair: the rank, its relation to block j, the pass's tile range, and (per
  // lane) the first row that sees this lane's key.
  int32_t wpass = 0, wc = -1, wi = 0, wgi = 0, wqt = 0, wq_lo = 0, wq_hi = 0;
  BlockRel wrel = make_rel(kNone, 0, Bb);
  int32_t wfrs = Bb;
  // stored dS (p.ds): the walk position's tile is number wds + wqt (the
  // tiles of this key tile follow each other, one per query tile)
  // p.ds != nullptr; known when compiling, so is the count of stores in flight
  constexpr bool store_ds = STORE_DS;
  int32_t wds = 0;
  const int32_t klast = kv0 + kKn - 1 < Bb ? kv0 + kKn - 1 : Bb - 1;
  // The pairs' rank, tile range and first stored dS tile, 64 pairs at a
  // time from pair cbase on, one pair per lane (cmask: the pairs that have
  // tiles), so that moving to the next pair reads lanes instead of searching.
  int32_t cbase = 0, c_wi = 0, c_lo = 0, c_hi = 0, c_ds = 0;
  uint64_t cmask = 0;
  auto fill = [&](int32_t base) {
    cbase = base;
    const int32_t c = base + lane;
    const int32_t cpass = c >= p.P ? 1 : 0;
    const int32_t ck = c - cpass * p.P;
    const int32_t ci = j + ck < p.P ? j + ck : j + ck - p.P;  // ring_rank(j, ck, P), both below P
    const BlockRel r = block_relation(p.layout, p.causal, ci, j, Bb);
    const int32_t a_first = first_row_seeing32(r, kv0, Bb);
    const int32_t q_first = a_first / kQm;
    int32_t q_full = (first_row_seeing32(r, klast, Bb) + kQm - 1) / kQm;
    q_full = q_full < qtiles ? q_full : qtiles;
    c_lo = cpass == 0 ? q_first : (q_full > q_first ? q_full : q_first);
    c_hi = cpass == 0 ? q_full : qtiles;
    c_wi = ci;
    const bool ok = c < 2 * p.P && ci >= p.rank_begin && ci < p.rank_begin + p.n_ranks && a_first < Bb &&
                    c_lo < c_hi;
    c_ds = 0;
    if (store_ds && ok) {
      const int32_t run = ((ci - p.rank_begin) * p.B + b) * p.H * p.P + hk * p.G * p.P + j;
      c_ds = run * (int32_t)p.ds_stride + (int32_t)ds_key_tile_start(r, tile, Bb) - q_first;
    }
    cmask = __builtin_amdgcn_ballot_w64(ok);
  };
  fill(0);
  auto next_rank = [&]() -> bool {
    for (;;) {
      const int32_t nb = wc + 1 > cbase ? wc + 1 - cbase : 0;  // the next pair's lane
      const uint64_t rest = nb < 64 ? cmask & (~0ull << nb) : 0ull;
      if (rest != 0) {
        const int32_t l = (int32_t)__builtin_ctzll(rest);
        wc = cbase + l;
        wpass = wc >= p.P ? 1 : 0;
        wi = __builtin_amdgcn_readlane(c_wi, l);
        wq_lo = __builtin_amdgcn_readlane(c_lo, l);
        wq_hi = __builtin_amdgcn_readlane(c_hi, l);
        if (store_ds) wds = __builtin_amdgcn_readlane(c_ds, l);
        wrel = block_relation(p.layout, p.causal, wi, j, Bb);
        wqt = wq_lo;
        wgi = 0;
        wfrs = first_row_seeing32(wrel, key, Bb);
        return true;
      }
      if (cbase + 64 >= 2 * p.P) return false;
      fill(cbase + 64);
    }
  };
  // 0: no more tiles; 1: the next tile of the same head; 2: another head or rank
  auto next_tile = [&]() -> int {
    if (++wqt < wq_hi) return 1;
    if (++wgi < p.G) {
      wqt = wq_lo;
      if (store_ds) wds += p.P * (int32_t)p.ds_stride;  // the next query head's run
      return 2;
    }
    return next_rank() ? 2 : 0;
  };
  // the walk position's stored dS tile (the tiles number below 2^31), kept
  // in a vector register: the walk's scalar state already fills the scalar
  // registers
  auto ds_of_walk = [&]() -> int32_t {
    int32_t t = wds + wqt;
    asm volatile("" : "+v"(t));
    return t;
  };
  auto src_of_walk = [&]() {
    const int32_t ri = wi - p.rank_begin;
    const int32_t h = hk * p.G + wgi;
    const int32_t q0 = wqt * kQm;
    QTileSrc s;
    s.q = reinterpret_cast<const unsigned char*>(p.q.ptr) +
          2 * (ri * p.q.s_blk + b * p.q.s_batch + h * p.q.s_head + q0 * p.q.s_tok);
    s.o = reinterpret_cast<const unsigned char*>(p.dout.ptr) +
          2 * (ri * p.dout.s_blk + b * p.dout.s_batch + h * p.dout.s_head + q0 * p.dout.s_tok);
    const int64_t srow = (((int64_t)ri * p.B + b) * p.H + h) * p.Bb + q0;
    s.l = p.lse2 + srow;
    s.d = p.dsum + srow;
    s.rows = Bb - q0 < kQm ? Bb - q0 : kQm;
    return s;
  };
  // the tile after `s` in the same head: 64 rows on
  auto src_next_row_tile = [&](QTileSrc& s) {
    s.q += (int64_t)kQm * 2 * p.q.s_tok;
    s.o += (int64_t)kQm * 2 * p.dout.s_tok;
    s.l += kQm;
    s.d += kQm;
    const int32_t left = Bb - wqt * kQm;
    s.rows = left < kQm ? left : kQm;
  };
  // the first row of the walk's tile (less 4hf) that sees this lane's key
  auto lo_of_walk = [&]() { return wfrs - wqt * kQm - 4 * hf; };

  if (next_rank()) {
    // K and V of this lane's key (row Bb - 1 past the block: finite, and its
    // results are not stored) as the B operands of the feature steps:
    // kreg[ss] = K[key][16ss + 8hf .. +7]
    bf16x8 kreg[NSS], vreg[NSS];
    {
      const int32_t kr = key < Bb ? key : Bb - 1;
      const __bf16* kp = reinterpret_cast<const __bf16*>(p.k.ptr) + j * p.k.s_blk + b * p.k.s_batch +
                         (int64_t)kr * p.k.s_tok + hk * p.k.s_head + 8 * hf;
      const __bf16* vp = reinterpret_cast<const __bf16*>(p.v.ptr) + j * p.v.s_blk + b * p.v.s_batch +
                         (int64_t)kr * p.v.s_tok + hk * p.v.s_head + 8 * hf;
#pragma unroll
      for (int ss = 0; ss < NSS; ++ss) {
        kreg[ss] = *reinterpret_cast<const bf16x8*>(kp + 16 * ss);
        vreg[ss] = *reinterpret_cast<const bf16x8*>(vp + 16 * ss);
      }
    }
    // The first step finishes a "previous" tile of zero probabilities read
    // from stage 3: zero that stage's Q and dO, so that no stale LDS bits (a
    // NaN pattern) reach the accumulators.
    {
      const u32x4 z = {0u, 0u, 0u, 0u};
      constexpr int N16 = L::QST_B / 16;
#pragma unroll
      for (int k = 0; k < N16 / kThreads; ++k) {
        reinterpret_cast<u32x4*>(smem_raw + 3 * L::QST_B)[tid + k * kThreads] = z;
        reinterpret_cast<u32x4*>(smem_raw + L::DO0 + 3 * L::QST_B)[tid + k * kThreads] = z;
      }
    }

    // This lane's byte offsets in the row copies: copy k of the wave covers
    // tile rows (wave + 4k) RW .. +RW-1; the lane fetches the logical chunk
    // that belongs at its place in the swizzled row (the swizzle repeats
    // every 16 rows, and 4 RW is a multiple of 16).
    const int32_t crow = wave * RW + lane / CPR;
    const int32_t cchunk = (lane % CPR) ^ chunk_swz<D>(crow);
    const int32_t sq2 = (int32_t)(2 * p.q.s_tok), so2 = (int32_t)(2 * p.dout.s_tok);
    const int32_t vq = crow * sq2 + 16 * cchunk, vo = crow * so2 + 16 * cchunk;
    // The copies of one tile, one instruction each: I = 0 is the lse2 / D
    // row (wave 0: lse2, wave 1: D, waves 2 and 3 a spare row), 1 .. NCP
    // the Q rows, NCP + 1 .. 2 NCP the dO rows. A direct copy holds its wave
    // until the memory system takes the request, which takes longest when
    // the waves of a workgroup request together, so a step issues one copy
    // per slot of its phases.
    auto copy_one = [&](const QTileSrc& s, int32_t stage, auto Ic) __attribute__((always_inline)) {
      constexpr int I = decltype(Ic)::value;
      static_assert(I >= 0 && I < NCOPY, "copy index");
      if constexpr (I == 0) {
        const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(wave == 1 ? s.d : s.l), (short)0, 4 * s.rows, kRawRsrcWord3);
        const int32_t foff = wave < 2 ? L::F32_B + (wave * kNst + stage) * kQm * 4 : L::SPARE_B + (wave - 2) * kQm * 4;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (__attribute__((address_space(3))) void*)(smem_raw + foff), 4,
                                                4 * lane, 0, 0, 0);
      } else if constexpr (I <= NCP) {
        constexpr int k = I - 1;
        const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)s.q, (short)0, sq2 * s.rows,
                                                                            kRawRsrcWord3);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rq, (__attribute__((address_space(3))) void*)(smem_raw + stage * L::QST_B + (wave + kWaves * k) * 1024), 16,
            vq + k * kWaves * RW * sq2, 0, 0, 0);
      } else {
        constexpr int k = I - 1 - NCP;
        const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc((void*)s.o, (short)0, so2 * s.rows,
                                                                            kRawRsrcWord3);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ro,
            (__attribute__((address_space(3))) void*)(smem_raw + L::DO0 + stage * L::QST_B + (wave + kWaves * k) * 1024),
            16, vo + k * kWaves * RW * so2, 0, 0, 0);
      }
    };
    auto dma = [&](const QTileSrc& s, int32_t stage) __attribute__((always_inline)) {
      unroll<NCOPY>([&](auto Ic) __attribute__((always_inline)) { copy_one(s, stage, Ic); });
    };

    // Tiles t (current), t + 1 and t + 2 (the walk's position): whether they
    // exist, and the pass and mask data of t and t + 1. Tile t + 1 is in
    // flight or has landed while tile t is computed; the step copies tile
    // t + 2 into the stage of t - 2, which no wave reads any more.
    QTileSrc src = src_of_walk();
    int32_t pass0 = wpass, pass1 = 1;
    int32_t lo0 = lo_of_walk(), lo1 = 0;
    // stored dS tiles of tiles t and t + 1, and of the tile before t (whose
    // dS the step writes out)
    // (the first step writes the zero chunks of a "previous" tile over tile
    // 0's, which the next step writes again: every step stores the same)
    int32_t ds0 = store_ds ? ds_of_walk() : 0, ds1 = 0, dsprev = ds0;
    // moves the walk on and its copy source with it (the source stays on the
    // last tile once the walk is over: copies then repeat it)
    auto advance = [&]() -> bool {
      const int nt = next_tile();
      if (nt == 1) src_next_row_tile(src);
      else if (nt == 2) src = src_of_walk();
      return nt != 0;
    };
    dma(src, 0);
    bool v1 = advance();
    if (v1) {
      pass1 = wpass;
      lo1 = lo_of_walk();
      if (store_ds) ds1 = ds_of_walk();
    }
    dma(src, 1);
    bool v2 = v1 && advance();
    // the K / V registers are in (the compiler waits for them here, once)
#pragma unroll
    for (int ss = 0; ss < NSS; ++ss) asm volatile("" : "+a"(kreg[ss]), "+a"(vreg[ss]));
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the zeroed stage
    wait_vm<NCOPY>();  // tile 0 has landed
    wg_barrier();

    const float c2 = p.scale_log2;
    // LDS byte addresses of this lane's reads in stage 0; a read adds its
    // stage's offset (stage x QST_B, or x 256 for lse2 / D) in the
    // instruction:
    //   cq[ss] / co[ss]: Q / dO row n, columns 16ss + 8hf (row block 1: + 32
    //     rows)
    //   cl: lse2 of rows 4hf .. +3 (+ 8gg + 32rb; D: + DS_B)
    //   pq[h2][dt] / po[h2][dt]: transposing reads of Q / dO rows 4hf +
    //     j16/4 + 8h2 (chunk kc: + 16 rows), columns 32dt + 16grp + 4(j16%4)
    const uint32_t lbase = lds_addr(smem_raw);
    uint32_t cq[NSS], co[NSS], pq[2][NDT], po[2][NDT];
#pragma unroll
    for (int ss = 0; ss < NSS; ++ss) {
      const uint32_t c = 2 * tile_off<D>(n, 16 * ss + 8 * hf);
      cq[ss] = lbase + c;
      co[ss] = lbase + L::DO0 + c;
    }
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const uint32_t c = 2 * tile_off<D>(4 * hf + j16 / 4 + 8 * h2, 32 * dt + 16 * grp + 4 * (j16 % 4));
        pq[h2][dt] = lbase + c;
        po[h2][dt] = lbase + L::DO0 + c;
      }
    const uint32_t cl = lbase + L::F32_B + 4 * (4 * hf);

    // The step is a two-phase software pipeline over the tile's two row
    // blocks of 32 rows. Phase A: S / dP of row block 1 of tile t, P / dS
    // of its row block 0, and dV^T / dK^T of row block 1 of tile t - 1;
    // phase B: S / dP of row block 0 of tile t + 1, P / dS of row block 1 of
    // tile t, and dV^T / dK^T of its row block 0. Every phase thus holds 16
    // products that feed the vector work, 16 that consume it, and the vector
    // work of one row block, interleaved slot by slot.
    //   s0 / d0, s1 / d1: S and dP of row blocks 0 and 1 (element i of row
    //     block rb: row 32rb + 8(i/4) + 4hf + i%4, key n)
    //   pa / da, pb2 / db2: P and dS (bf16) of the 16-row chunks 0, 1 and
    //     2, 3 (chunk kc, element x: row 16kc + 8(x/4) + 4hf + x%4), the B
    //     operands of the dV^T / dK^T products
    f32x16 s0, d0, s1, d1;
    bf16x8 pa[2], da[2], pb2[2], db2[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      pa[c] = bf16x8{};
      da[c] = bf16x8{};
      pb2[c] = bf16x8{};
      db2[c] = bf16x8{};
    }

    // s_waitcnt lgkmcnt(N) tied to one slot's reads
    auto slot_wait = [&](auto Nc, u32x4(&ra)[2], u32x2(&ta)[4], u32x4(&rl)[2]) __attribute__((always_inline)) {
      constexpr int N = decltype(Nc)::value;
      static_assert(N >= 0 && N <= 15, "lgkmcnt range");
      asm volatile("s_waitcnt lgkmcnt(%8)"
                   : "+v"(ra[0]), "+v"(ra[1]), "+v"(ta[0]), "+v"(ta[1]), "+v"(ta[2]), "+v"(ta[3]), "+v"(rl[0]),
                     "+v"(rl[1])
                   : "n"(N));
    };

    // One phase, NSS slots. Slot SS: the S / dP products of feature step SS
    // of the row block at ROFF bytes of stage SC into (sx, dx); the dV^T and
    // dK^T products of pair SS (feature tile SS/2, chunk KC0 + SS%2) of
    // stage ST with B operands (pi, di); and EPS elements of P / dS of row
    // block RBP of the current tile from (sp, dp), lse2 / D rows at LOFF of
    // stage SL, into (pw, dw). The reads of slot SS + 1 go out before slot SS
    // waits for its own.
    constexpr int EPS = 16 / NSS;  // P / dS elements per slot
    static_assert(EPS * NSS == 16 && 4 * NDT == 2 * NSS, "slot shape");
    auto phase = [&](auto MASKc, auto RBPc, auto KC0c, auto ROFFc, auto LOFFc, auto SCc, auto STc, auto SLc,
                     f32x16& sx, f32x16& dx, const f32x16& sp, const f32x16& dp, bf16x8(&pw)[2], bf16x8(&dw)[2],
                     const bf16x8(&pi)[2], const bf16x8(&di)[2], int32_t clo,
                     auto&& at_slot) __attribute__((always_inline)) {
      constexpr bool MASK = decltype(MASKc)::value != 0;
      constexpr int RBP = decltype(RBPc)::value, KC0 = decltype(KC0c)::value;
      constexpr int ROFF = decltype(ROFFc)::value, LOFF = decltype(LOFFc)::value;
      constexpr int SQ = decltype(SCc)::value * L::QST_B + ROFF;  // S / dP reads
      constexpr int ST = decltype(STc)::value * L::QST_B;         // dV^T / dK^T reads
      constexpr int SL = decltype(SLc)::value * kQm * 4 + LOFF;   // lse2 / D reads
      u32x4 ra[2][2];
      u32x2 tr[2][4];
      u32x4 rl[2][2];
      // reads of slot SS (the lse2 / D group of its first element when it
      // starts a group of 4)
      auto reads = [&](auto SSc) __attribute__((always_inline)) {
        constexpr int SS = decltype(SSc)::value;
        constexpr int sl = SS & 1, dt = SS / 2, kc = KC0 + SS % 2;
        ra[sl][0] = lds_read16<SQ>(cq[SS]);
        ra[sl][1] = lds_read16<SQ>(co[SS]);
        tr[sl][0] = tr_read_at<ST + kc * 16 * D * 2>(po[0][dt]);
        tr[sl][1] = tr_read_at<ST + kc * 16 * D * 2>(po[1][dt]);
        tr[sl][2] = tr_read_at<ST + kc * 16 * D * 2>(pq[0][dt]);
        tr[sl][3] = tr_read_at<ST + kc * 16 * D * 2>(pq[1][dt]);
        if constexpr ((SS * EPS) % 4 == 0) {
          constexpr int gg = SS * EPS / 4;
          rl[gg & 1][0] = lds_read16<SL + gg * 32>(cl);
          rl[gg & 1][1] = lds_read16<L::DS_B + SL + gg * 32>(cl);
        }
      };
      constexpr auto nreads = [](int SS) { return 6 + ((SS * EPS) % 4 == 0 ? 2 : 0); };
      reads(ic<0>{});
      unroll<NSS>([&](auto SSc) __attribute__((always_inline)) {
        constexpr int SS = decltype(SSc)::value;
        constexpr int sl = SS & 1, dt = SS / 2, c = SS % 2;
        constexpr int g0 = SS * EPS / 4;  // the lse2 / D group of this slot
        if constexpr (SS + 1 < NSS) {
          reads(ic<SS + 1>{});
          slot_wait(ic<nreads(SS + 1)>{}, ra[sl], tr[sl], rl[g0 & 1]);
        } else {
          slot_wait(ic<0>{}, ra[sl], tr[sl], rl[g0 & 1]);
        }
        const float4 l4 = __builtin_bit_cast(float4, rl[g0 & 1][0]);
        const float4 d4 = __builtin_bit_cast(float4, rl[g0 & 1][1]);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};  // lse in log2 units
        const float dd[4] = {d4.x, d4.y, d4.z, d4.w};
        mfma_s(sx, ra[sl][0], kreg[SS], SS == 0);
        dv[dt] = mfma32(__builtin_bit_cast(bf16x8, __builtin_shufflevector(tr[sl][0], tr[sl][1], 0, 1, 2, 3)), pi[c],
                        dv[dt]);
        at_slot(SSc);
#pragma unroll
        for (int x = 0; x < EPS; ++x) {
          const int i = SS * EPS + x, gg = i / 4, e = i % 4;
          float pv = fexp2(fmaf(sp[i], c2, -lv[e]));
          if constexpr (MASK) {
            if (32 * RBP + 8 * gg + e < clo) pv = 0.0f;
          }
          const float dsv = pv * (dp[i] - dd[e]);
          pw[gg / 2][4 * (gg % 2) + e] = (__bf16)pv;
          dw[gg / 2][4 * (gg % 2) + e] = (__bf16)dsv;
        }
        mfma_s(dx, ra[sl][1], vreg[SS], SS == 0);
        dk[dt] = mfma32(__builtin_bit_cast(bf16x8, __builtin_shufflevector(tr[sl][2], tr[sl][3], 0, 1, 2, 3)), di[c],
                        dk[dt]);
        // keeps the conversions of a finished chunk where they are
        if constexpr (((SS + 1) * EPS) % 8 == 0) {
          constexpr int ch = ((SS + 1) * EPS) / 8 - 1;
          asm volatile("" : "+v"(pw[ch]), "+v"(dw[ch]));
        }
      });
    };

    int32_t st = 0;  // stage of the current tile
    bool v0 = true;
    unsigned char* const ds_lane = reinterpret_cast<unsigned char*>(p.ds) + (32 * wave + n) * 32 + hf * 16;
    // dS chunks C0, C0 + 1 of stored tile `tix`: lane (hf, n) writes its
    // rows of key n at ((kc * 128 + 32 wave + n) * 2 + hf) * 16 bytes of the
    // tile, kc the 16-row chunk
    auto store_ds2 = [&](const bf16x8(&v)[2], int32_t tix, auto C0c) __attribute__((always_inline)) {
      constexpr int C0 = decltype(C0c)::value;
      unsigned char* t = ds_lane + (uint64_t)(uint32_t)tix * (uint32_t)(kDsRows * kDsKeys * 2);
#pragma unroll
      for (int c = 0; c < 2; ++c)
        __builtin_nontemporal_store(v[c], reinterpret_cast<bf16x8*>(t + (C0 + c) * 4096));
    };

    // S / dP of row block 0 of tile 0 (stage 0)
    {
      u32x4 ra[2][2];
      ra[0][0] = lds_read16<0>(cq[0]);
      ra[0][1] = lds_read16<0>(co[0]);
      unroll<NSS>([&](auto SSc) __attribute__((always_inline)) {
        constexpr int SS = decltype(SSc)::value;
        constexpr int sl = SS & 1;
        if constexpr (SS + 1 < NSS) {
          ra[sl ^ 1][0] = lds_read16<0>(cq[SS + 1]);
          ra[sl ^ 1][1] = lds_read16<0>(co[SS + 1]);
          lds_wait<2>(ra[sl]);
        } else {
          lds_wait<0>(ra[sl]);
        }
        mfma_s(s0, ra[sl][0], kreg[SS], SS == 0);
        mfma_s(d0, ra[sl][1], vreg[SS], SS == 0);
      });
    }

    bool slow = false;  // the walk's next tile is in another run
    // one step with the current tile in stage U (the step loop runs four
    // steps per round, so that every stage is known when compiling)
    auto step = [&](auto MASKc, auto Uc) __attribute__((always_inline)) {
      constexpr int U = decltype(Uc)::value;
      const int32_t clo = lo0;
      // Phase A. The previous tile's dS chunks 2, 3 go out first, then
      // tile t + 2's lse2 / D and Q copies, one per slot from slot 1, into
      // the stage of t - 2, which no wave reads any more.
      if (store_ds) store_ds2(db2, dsprev, ic<2>{});
      phase(MASKc, ic<0>{}, ic<2>{}, ic<32 * D * 2>{}, ic<0>{}, ic<U>{}, ic<(U + 3) % kNst>{}, ic<U>{}, s1, d1,
            s0, d0, pa, da, pb2, db2, clo, [&](auto SSc) __attribute__((always_inline)) {
              constexpr int SS = decltype(SSc)::value;
              if constexpr (SS >= 1 && SS <= kCopiesA) copy_one(src, (U + 2) % kNst, ic<SS - 1>{});
            });
      __builtin_amdgcn_sched_barrier(0);
      // Tile t + 1 has landed: only this phase's stores and copies, issued
      // after its last copy, may still be in flight. Past the barrier every
      // wave is done with the stage of t - 1.
      wait_vm<kCopiesA + (store_ds ? 2 : 0)>();
      wg_barrier();
      // Phase B: this tile's dS chunks 0, 1, then tile t + 2's dO copies
      if (store_ds) store_ds2(da, ds0, ic<0>{});
      phase(MASKc, ic<1>{}, ic<0>{}, ic<0>{}, ic<32 * 4>{}, ic<(U + 1) % kNst>{}, ic<U>{}, ic<U>{}, s0, d0, s1,
            d1, pb2, db2, pa, da, clo, [&](auto SSc) __attribute__((always_inline)) {
              constexpr int SS = decltype(SSc)::value;
              if constexpr (SS >= 1 && SS <= NCOPY - kCopiesA) copy_one(src, (U + 2) % kNst, ic<SS - 1 + kCopiesA>{});
            });
      __builtin_amdgcn_sched_barrier(0);
      // t + 1 becomes current, the walk moves on to t + 3
      v0 = v1;
      v1 = v2;
      pass0 = pass1;
      lo0 = lo1;
      dsprev = ds0;
      ds0 = ds1;
      if (v2) {
        pass1 = wpass;
        lo1 = lo_of_walk();
        if (store_ds) ds1 = ds_of_walk();
        if (wqt + 1 < wq_hi) {  // the next query tile of the same (rank, head) run
          ++wqt;
          src_next_row_tile(src);
        } else {
          slow = true;  // another head or rank: the walk moves on outside the step loop
        }
      }
    };
    // steps while cont() holds, entering the four-step round at stage st
    auto run = [&](auto MASKc, auto&& cont) __attribute__((always_inline)) {
      while (cont()) {
        // a run change (rare) moves the walk on here, outside the steps
        if (slow) {
          slow = false;
          v2 = advance();
        }
        if (st == 0) {
          step(MASKc, ic<0>{});
          st = 1;
          if (slow || !cont()) continue;
        }
        if (st == 1) {
          step(MASKc, ic<1>{});
          st = 2;
          if (slow || !cont()) continue;
        }
        if (st == 2) {
          step(MASKc, ic<2>{});
          st = 3;
          if (slow || !cont()) continue;
        }
        step(MASKc, ic<3>{});
        st = 0;
      }
    };
    run(ic<1>{}, [&]() { return v0 && pass0 == 0; });
    run(ic<0>{}, [&]() { return v0; });

    // the last tile's dS chunks 2, 3, and its dV^T / dK^T products of them
    // (stage of the last tile: now st - 1)
    if (store_ds) store_ds2(db2, dsprev, ic<2>{});
    {
      const uint32_t so = (uint32_t)(((st + kNst - 1) % kNst) * L::QST_B);
      u32x2 t[4];
      unroll<2 * NDT>([&](auto Qc) __attribute__((always_inline)) {
        constexpr int Q = decltype(Qc)::value;
        constexpr int dt = Q / 2, c = Q % 2, kc = 2 + c;
        t[0] = tr_read_at<kc * 16 * D * 2>(po[0][dt] + so);
        t[1] = tr_read_at<kc * 16 * D * 2>(po[1][dt] + so);
        t[2] = tr_read_at<kc * 16 * D * 2>(pq[0][dt] + so);
        t[3] = tr_read_at<kc * 16 * D * 2>(pq[1][dt] + so);
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(t[0]), "+v"(t[1]), "+v"(t[2]), "+v"(t[3]));
        dv[dt] = mfma32(__builtin_bit_cast(bf16x8, __builtin_shufflevector(t[0], t[1], 0, 1, 2, 3)), pb2[c], dv[dt]);
        dk[dt] = mfma32(__builtin_bit_cast(bf16x8, __builtin_shufflevector(t[2], t[3], 0, 1, 2, 3)), db2[c], dk[dt]);
      });
    }
    wait_vm<0>();  // the repeated copies of the last steps
  }

  if (key >= Bb) return;
  __bf16* dkrow = reinterpret_cast<__bf16*>(p.dk.ptr) + j * p.dk.s_blk + b * p.dk.s_batch +
                  (int64_t)key * p.dk.s_tok + hk * p.dk.s_head;
  __bf16* dvrow = reinterpret_cast<__bf16*>(p.dv.ptr) + j * p.dv.s_blk + b * p.dv.s_batch +
                  (int64_t)key * p.dv.s_tok + hk * p.dv.s_head;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      bf16x4 wk4, wv4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        wk4[e] = (__bf16)(dk[dt][4 * g4 + e] * p.scale);
        wv4[e] = (__bf16)dv[dt][4 * g4 + e];
      }
      *reinterpret_cast<bf16x4*>(dkrow + 32 * dt + 8 * g4 + 4 * hf) = wk4;
      *reinterpret_cast<bf16x4*>(dvrow + 32 * dt + 8 * g4 + 4 * hf) = wv4;
    }
}

// ---------------------------------------------------------------- fp32 path
// Plain VALU kernel for float32: kF32Split lanes per key (64 keys per
// workgroup), each holding dK/dV of a quarter of the features in registers;
// the S and dP dot products add the quarters with two lane exchanges. Query
// tiles of 32 rows are staged in LDS (dQ: dq_f32_kernel).
constexpr int kF32Keys = 64;
constexpr int kF32Rows = 32;
constexpr int kF32Split = 4;  // lanes per key
constexpr int kF32Threads = kF32Keys * kF32Split;

template <int D>
struct BwdF32Lds {
  static constexpr int S = D + 1;  // padded rows
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
__global__ __launch_bounds__(kF32Threads) void dkdv_f32_kernel(BwdParams p) {
  using L = BwdF32Lds<D>;
  constexpr int DQ = D / kF32Split;  // features per lane
  extern __shared__ __align__(16) unsigned char smem_raw[];
  float* sm = reinterpret_cast<float*>(smem_raw);
  float* ks = sm + L::KS;
  float* vs = sm + L::VS;
  float* qs = sm + L::QS;
  float* os = sm + L::OS;
  float* lse_s = sm + L::LSE;
  float* dsum_s = sm + L::DSUM;
  const int tid = threadIdx.x;
  const int kl = tid / kF32Split;          // this lane's key in the tile
  const int f0 = (tid % kF32Split) * DQ;   // its first feature
  const int32_t BHk = p.B * p.Hk;
  const int32_t tiles = (int32_t)((p.Bb + kF32Keys - 1) / kF32Keys);
  const int64_t id = blockIdx.x;
  const int32_t bhk = (int32_t)(id % BHk);
  const int32_t b = bhk / p.Hk;
  const int32_t hk = bhk % p.Hk;
  int32_t j, tile;
  kv_tile_of(p, id / BHk, tiles, &j, &tile);
  const int64_t kv0 = (int64_t)tile * kF32Keys;
  const int64_t key = kv0 + kl;
  const float* kbase = reinterpret_cast<const float*>(p.k.ptr) + j * p.k.s_blk + b * p.k.s_batch + hk * p.k.s_head;
  const float* vbase = reinterpret_cast<const float*>(p.v.ptr) + j * p.v.s_blk + b * p.v.s_batch + hk * p.v.s_head;
  for (int idx = tid; idx < kF32Keys * D; idx += kF32Threads) {
    const int r = idx / D, e = idx % D;
    const int64_t x = kv0 + r;
    ks[r * L::S + e] = (x < p.Bb) ? kbase[x * p.k.s_tok + e] : 0.0f;
    vs[r * L::S + e] = (x < p.Bb) ? vbase[x * p.v.s_tok + e] : 0.0f;
  }
  float dk[DQ], dv[DQ];
#pragma unroll
  for (int e = 0; e < DQ; ++e) {
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
        for (int idx = tid; idx < kF32Rows * D; idx += kF32Threads) {
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
          for (int e = 0; e < DQ; ++e) {
            s = fmaf(qs[r * L::S + f0 + e], ks[kl * L::S + f0 + e], s);
            dpv = fmaf(os[r * L::S + f0 + e], vs[kl * L::S + f0 + e], dpv);
          }
          // the four quarters of this key's lanes (lanes 4k .. 4k+3)
          s += __shfl_xor(s, 1);
          s += __shfl_xor(s, 2);
          dpv += __shfl_xor(dpv, 1);
          dpv += __shfl_xor(dpv, 2);
          const float pv = vis ? fexp2(fmaf(s, c2, -lse_s[r])) : 0.0f;
          const float dsv = pv * (dpv - dsum_s[r]);
#pragma unroll
          for (int e = 0; e < DQ; ++e) {
            dv[e] = fmaf(pv, os[r * L::S + f0 + e], dv[e]);
            dk[e] = fmaf(dsv, qs[r * L::S + f0 + e], dk[e]);
          }
        }
      }
    }
  }
  if (key >= p.Bb) return;
  float* dkrow = reinterpret_cast<float*>(p.dk.ptr) + j * p.dk.s_blk + b * p.dk.s_batch + key * p.dk.s_tok + hk * p.dk.s_head;
  float* dvrow = reinterpret_cast<float*>(p.dv.ptr) + j * p.dv.s_blk + b * p.dv.s_batch + key * p.dv.s_tok + hk * p.dv.s_head;
#pragma unroll
  for (int e = 0; e < DQ; ++e) {
    dkrow[f0 + e] = dk[e] * p.scale;
    dvrow[f0 + e] = dv[e];
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
  const bool st = p.ds != nullptr;
  if (p.D == 128)
    return st ? launch_dyn(dkdv_bf16_kernel<128, true>, grid, kThreads, BwdLds<128>::BYTES, s, p)
              : launch_dyn(dkdv_bf16_kernel<128, false>, grid, kThreads, BwdLds<128>::BYTES, s, p);
  return st ? launch_dyn(dkdv_bf16_kernel<64, true>, grid, kThreads, BwdLds<64>::BYTES, s, p)
            : launch_dyn(dkdv_bf16_kernel<64, false>, grid, kThreads, BwdLds<64>::BYTES, s, p);
}

hipError_t launch_dkdv_f32(const BwdParams& p, hipStream_t s) {
  const int64_t grid = ((p.Bb + kF32Keys - 1) / kF32Keys) * (int64_t)p.P * p.B * p.Hk;
  if (p.D == 128) return launch_dyn(dkdv_f32_kernel<128>, grid, kF32Threads, BwdF32Lds<128>::BYTES, s, p);
  return launch_dyn(dkdv_f32_kernel<64>, grid, kF32Threads, BwdF32Lds<64>::BYTES, s, p);
}

}  // namespace ra
