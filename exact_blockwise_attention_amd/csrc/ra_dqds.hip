// ra_dqds.hip — the query gradient from stored score gradients (gfx950).
//
// "Ring Attention 論文分析" (blog), section "逆伝播での KV 再循環": the
// backward recomputes P = exp(S - lse) once, forms dS = P * (dP - D) and
// from it dK = scale dS^T Q and dQ = scale dS K. The key-side walk
// (ra_bwd.hip) computes every dS tile for dK and dV and also writes it out,
// so that dQ needs no second recompute of S and dP: here each workgroup sums
// dQ = scale sum_j dS_ij K_j over the stored tiles of its query rows. The
// walk is bound by reading the dS tiles (2 bytes per visible pair) from
// HBM.
//
// A stored dS tile covers kDsRows = 64 query rows and kDsKeys = 128 keys in
// the key-side walk's register order: element (kc, key, half, x) at
// ((kc * 128 + key) * 2 + half) * 8 + x, row 16 kc + 8 (x / 4) + 4 half + x % 4.
// Here it is read with transposing LDS reads (ds_read_b64_tr_b16), which
// give each lane 4 consecutive keys of one query row: the A operand of
// dQ = dS K. K comes pre-arranged in operand order (kop_pack_kernel).
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

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTileBytes = kDsRows * kDsKeys * 2;  // one stored dS tile: 16 KB

// ---------------------------------------------------------------- K in operand order
// One 128-key tile of block j as the B operands of dQ = dS K, unit (dt, kk)
// (32 features x 16 keys) holding lane l's 16 bytes at (unit * 64 + l) * 16:
// lane (hf, n) = (l / 32, l % 32) gets K[16 kk + 8 hf + e][32 dt + n], e =
// 0..7. Keys past the block are written as zeros, so that they add nothing
// to dQ whatever the stored dS holds there.
template <int D>
__global__ __launch_bounds__(kThreads) void kop_pack_kernel(BwdParams p) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __bf16* tile = reinterpret_cast<__bf16*>(smem_raw);  // [128][D], swizzled
  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64;
  const int32_t Bb = (int32_t)p.Bb;
  const int32_t ktiles = (Bb + kDsKeys - 1) / kDsKeys;
  const int64_t id = blockIdx.x;
  const int32_t kt = (int32_t)(id % ktiles);
  const int64_t r = id / ktiles;
  const int32_t j = (int32_t)(r % p.P);
  const int32_t bhk = (int32_t)(r / p.P);
  const int32_t b = bhk / p.Hk, hk = bhk % p.Hk;
  const __bf16* base = reinterpret_cast<const __bf16*>(p.k.ptr) + (int64_t)j * p.k.s_blk + b * p.k.s_batch +
                       hk * p.k.s_head;
  dma_rows<D, kDsKeys, kWaves>(tile, base, p.k.s_tok, kt * kDsKeys, Bb, wave, lane);
  wait_dma();
  __syncthreads();
  const int hf = lane / 32, g = (lane / 16) % 2, j16 = lane % 16;
  __bf16* out = p.kop + id * (int64_t)(kDsKeys * D);
  constexpr int NU = (D / 32) * 8;
  const uint32_t lb = lds_addr(tile);
  for (int u = wave; u < NU; u += kWaves) {
    const int dt = u / 8, kk = u % 8;
    // lane j16 of a 16-lane group reads key row 16 kk + 8 hf + j16 / 4 (+4),
    // features 32 dt + 16 g + 4 (j16 % 4) .. +3; lane i of the group then
    // holds feature 32 dt + 16 g + i of the four rows
    const int row = 16 * kk + 8 * hf + j16 / 4;
    const int col = 32 * dt + 16 * g + 4 * (j16 % 4);
    u32x2 lo = tr_read_at<0>(lb + 2 * tile_off<D>(row, col));
    u32x2 hi = tr_read_at<0>(lb + 2 * tile_off<D>(row + 4, col));
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(lo), "+v"(hi));
    bf16x8 v = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3));
    const int32_t key0 = kt * kDsKeys + 16 * kk + 8 * hf;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (key0 + e >= Bb) v[e] = (__bf16)0.0f;
    *reinterpret_cast<bf16x8*>(out + ((int64_t)u * 64 + lane) * 8) = v;
  }
}

// ---------------------------------------------------------------- dQ from the stored tiles
// A workgroup owns query tiles qt0 = 2 qp and qt1 = 2 qp + 1 (128 rows) of
// rank i for one (batch, query head). It visits the key blocks in block
// order (the sum does not depend on it) and in each the key tiles the tiles' last rows see (qt1's, a superset of
// qt0's), one step per key tile: the step's two stored dS tiles and its K
// operand tile go global -> LDS directly, the dS tiles two steps ahead and
// the K tile one step ahead. d = 128: wave w takes the 64 rows of tile
// qt(w / 2) against features 64 (w % 2) .. +63; d = 64: rows 32 w .. +31 of
// the pair against all 64 features.
template <int D>
struct DqLds {
  static constexpr int DS_STAGE = 2 * kTileBytes;          // two dS tiles
  static constexpr int NDS = 3;                            // dS stages
  static constexpr int KOP_STAGE = kDsKeys * D * 2;         // one K operand tile
  static constexpr int NKOP = 2;
  static constexpr int KOP0 = NDS * DS_STAGE;
  static constexpr int BYTES = KOP0 + NKOP * KOP_STAGE;
  static_assert(BYTES <= 160 * 1024, "LDS");
};

// One step of the walk: the stored tiles of the pair's two query tiles at
// one key tile (tile indices are below 2^31), the K operand tile, and which
// of the two query tiles meet the key tile (bit 0: qt0, bit 1: qt1).
struct DsStep {
  int32_t t0, t1, kop, meets;
};

// The walk of a query-tile pair over the key blocks (block order) and their
// key tiles; one position = one step. A pair's stored tiles go key tile by
// key tile, key tile kt holding query tiles first(kt) .. qtiles - 1, so the
// step's two tiles are at start(kt) + qt - first(kt).
struct DsWalk {
  int32_t k, P, i, layout, causal, Bb, qt0, qtiles;
  bool has1;
  int32_t region0, stride, kop_region0, ktiles;
  // current position
  BlockRel rel;
  int32_t j, kt, n0, n1, nsteps, first, start, run, kop;
  __device__ bool next_block() {
    while (++k < P) {
      j = k;  // every rank walks the blocks in the same order: workgroups share K tiles
      rel = block_relation(layout, causal, i, j, Bb);
      n0 = ds_key_tiles(rel, qt0, Bb);
      n1 = has1 ? ds_key_tiles(rel, qt0 + 1, Bb) : 0;
      nsteps = n0 > n1 ? n0 : n1;
      if (nsteps == 0) continue;
      run = (region0 + j) * stride;
      kop = (kop_region0 + j) * ktiles;
      kt = 0;
      start = 0;
      first = ds_first_qtile(rel, 0, Bb);
      return true;
    }
    return false;
  }
  // false once the walk is over (the position then stays on the last step)
  __device__ bool next() {
    if (kt + 1 < nsteps) {
      start += qtiles - first;
      ++kt;
      first = ds_first_qtile(rel, kt, Bb);
      return true;
    }
    const int32_t keep_k = k;
    if (next_block()) return true;
    k = keep_k;
    return false;
  }
  __device__ DsStep step() const {
    DsStep s;
    s.t0 = run + start + (qt0 - first);
    s.t1 = s.t0 + 1;
    s.kop = kop + kt;
    s.meets = (kt < n0 ? 1 : 0) | (kt < n1 ? 2 : 0);
    return s;
  }
};

template <int D>
__global__ __launch_bounds__(kThreads, 1) void dq_from_ds_kernel(BwdParams p) {
  using L = DqLds<D>;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  constexpr int RBW = D == 128 ? 2 : 1;  // 32-row blocks per wave
  constexpr int NDT = D / 32;            // 32-feature tiles of a K tile
  constexpr int KOP_LOADS = L::KOP_STAGE / 1024 / kWaves;
  constexpr int DS_LOADS = L::DS_STAGE / 1024 / kWaves;  // 8

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64;
  const int n = lane % 32, hf = lane / 32;

  const int32_t Bb = (int32_t)p.Bb;
  const int32_t qtiles = (Bb + kDsRows - 1) / kDsRows;
  const int32_t npairs = (qtiles + 1) / 2;
  const int32_t BH = p.B * p.H;
  // consecutive logical indices: the ranks of one (batch, head, query-tile
  // pair), pairs heaviest (latest rows) first. Every rank walks the key
  // blocks in the same order and a pair's walk hardly depends on the rank,
  // so an XCD's workgroups read the same K tiles at about the same time and
  // share them in L2
  const int64_t nwg = (int64_t)BH * p.n_ranks * npairs;
  const uint32_t L0 = (uint32_t)xcd_logical(blockIdx.x, nwg);
  const int32_t ri = (int32_t)(L0 % (uint32_t)p.n_ranks);
  const uint32_t g0 = L0 / (uint32_t)p.n_ranks;
  const int32_t qp = npairs - 1 - (int32_t)(g0 % (uint32_t)npairs);
  const int32_t bh = (int32_t)(g0 / (uint32_t)npairs);
  const int32_t b = bh / p.H, h = bh % p.H, hk = h / p.G;

  // this wave's rows: query tile qh of the pair, 32-row blocks rb0 .. rb0 + RBW - 1;
  // features: 32-feature tiles dt0, dt0 + 1
  const int qh = wave / 2;
  const int rb0 = D == 128 ? 0 : wave % 2;
  const int dt0 = D == 128 ? 2 * (wave % 2) : 0;

  DsWalk w0;
  w0.k = -1;
  w0.qtiles = qtiles;
  w0.P = p.P;
  w0.i = p.rank_begin + ri;
  w0.layout = p.layout;
  w0.causal = p.causal;
  w0.Bb = Bb;
  w0.qt0 = 2 * qp;
  w0.has1 = 2 * qp + 1 < qtiles;
  w0.region0 = ((ri * p.B + b) * p.H + h) * p.P;
  w0.stride = (int32_t)p.ds_stride;
  w0.kop_region0 = (b * p.Hk + hk) * p.P;
  w0.ktiles = (Bb + kDsKeys - 1) / kDsKeys;

  f32x16 acc[RBW][2];
#pragma unroll
  for (int r = 0; r < RBW; ++r) {
    acc[r][0] = f32x16{};
    acc[r][1] = f32x16{};
  }

  const unsigned char* dsb = reinterpret_cast<const unsigned char*>(p.ds);
  const unsigned char* kopb = reinterpret_cast<const unsigned char*>(p.kop);
  // Loads of one step, global -> LDS, 16 bytes per lane. dS: load m of the
  // wave is tile m / 4 of the pair, 1 KB unit (kc, key block) = (m % 4,
  // wave): the lane fetches the 16 bytes that belong at its place once keys
  // of odd kc are XOR-swizzled by 4 (so that the transposing reads of the two
  // 16-row halves of a 32-row block fall in different bank halves).
  uint32_t dsl[4];
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) {
    const int key = (32 * wave + lane / 2) ^ ((kc & 1) << 2);
    dsl[kc] = (uint32_t)(kc * 4096 + key * 32 + (lane % 2) * 16);
  }
  auto load_ds = [&](const DsStep& s, int stage) __attribute__((always_inline)) {
    // a query tile that does not meet the key tile loads the other's tile
    // (valid memory, unused data)
    const uint32_t tile0 = (uint32_t)((s.meets & 1) ? s.t0 : s.t1);
    const uint32_t tile1 = (uint32_t)((s.meets & 2) ? s.t1 : s.t0);
    unsigned char* st = smem_raw + stage * L::DS_STAGE;
    const unsigned char* src0 = dsb + (uint64_t)tile0 * kTileBytes;
    const unsigned char* src1 = dsb + (uint64_t)tile1 * kTileBytes;
#pragma unroll
    for (int m = 0; m < DS_LOADS; ++m) {
      const int half = m / 4, kc = m % 4;
      const unsigned char* src = (half ? src1 : src0) + dsl[kc];
      // non-temporal: the tiles are read once, and should not push the K
      // tiles, which the workgroups share, out of L2
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(st + half * kTileBytes +
                                                                                        kc * 4096 + wave * 1024),
                                       16, 0, 2);
    }
  };
  auto load_kop = [&](const DsStep& s, int stage) __attribute__((always_inline)) {
    const unsigned char* src = kopb + (uint64_t)(uint32_t)s.kop * L::KOP_STAGE + lane * 16;
    unsigned char* st = smem_raw + L::KOP0 + stage * L::KOP_STAGE;
#pragma unroll
    for (int m = 0; m < KOP_LOADS; ++m) {
      const int u = wave + kWaves * m;
      __builtin_amdgcn_global_load_lds(src + u * 1024, (__attribute__((address_space(3))) void*)(st + u * 1024), 16,
                                       0, 0);
    }
  };

  // LDS byte offsets of this lane's transposing A reads (rows of its 32-row
  // block, 4 keys each): group g = lane / 16 holds rows 16 (g % 2) + i, keys
  // 8 (g / 2) + 0..3 (first read) and + 4..7 (second)
  const int g = lane / 16, j16 = lane % 16;
  const int kcp = g % 2;
  const int keyA = 8 * (g / 2) + j16 / 4;
  const int sub = (j16 % 4) % 2 * 16 + (j16 % 4) / 2 * 8;
  const uint32_t lbase = lds_addr(smem_raw);
  const uint32_t a_off0 = (uint32_t)(qh * kTileBytes + rb0 * 8192 + kcp * 4096 + ((keyA ^ (kcp << 2)) * 32) + sub);
  const uint32_t a_off1 = (uint32_t)(qh * kTileBytes + rb0 * 8192 + kcp * 4096 + (((keyA + 4) ^ (kcp << 2)) * 32) + sub);
  const uint32_t b_off = (uint32_t)(L::KOP0 + dt0 * 8 * 1024 + lane * 16);

  // One step: dQ[rows] += dS[rows, 128 keys] K[128 keys, features] in 8
  // k-steps of 16 keys; operands of k-step kk + 1 are read during kk.
  auto compute = [&](int ds_stage, int kop_stage) __attribute__((always_inline)) {
    const uint32_t a0 = lbase + ds_stage * L::DS_STAGE + a_off0;
    const uint32_t a1 = lbase + ds_stage * L::DS_STAGE + a_off1;
    const uint32_t bb = lbase + kop_stage * L::KOP_STAGE + b_off;
    u32x2 ta[2][2][2];  // [slot][row block][read]
    u32x4 tb[2][2];     // [slot][feature tile]
    auto rd = [&](auto KKc) __attribute__((always_inline)) {
      constexpr int kk = decltype(KKc)::value;
      constexpr int s = kk & 1;
      unroll<RBW>([&](auto Rc) __attribute__((always_inline)) {
        constexpr int r = decltype(Rc)::value;
        ta[s][r][0] = tr_read_at<r * 8192 + kk * 512>(a0);
        ta[s][r][1] = tr_read_at<r * 8192 + kk * 512>(a1);
      });
      tb[s][0] = lds_read16<kk * 1024>(bb);
      tb[s][1] = lds_read16<(8 + kk) * 1024>(bb);
    };
    rd(ic<0>{});
    unroll<8>([&](auto KKc) __attribute__((always_inline)) {
      constexpr int kk = decltype(KKc)::value;
      constexpr int s = kk & 1;
      if constexpr (kk + 1 < 8) {
        rd(ic<kk + 1>{});
        // outstanding after this k-step's reads: the next k-step's
        if constexpr (RBW == 2) {
          asm volatile("s_waitcnt lgkmcnt(6)"
                       : "+v"(ta[s][0][0]), "+v"(ta[s][0][1]), "+v"(ta[s][1][0]), "+v"(ta[s][1][1]),
                         "+v"(tb[s][0]), "+v"(tb[s][1]));
        } else {
          asm volatile("s_waitcnt lgkmcnt(4)" : "+v"(ta[s][0][0]), "+v"(ta[s][0][1]), "+v"(tb[s][0]), "+v"(tb[s][1]));
        }
      } else {
        if constexpr (RBW == 2) {
          asm volatile("s_waitcnt lgkmcnt(0)"
                       : "+v"(ta[s][0][0]), "+v"(ta[s][0][1]), "+v"(ta[s][1][0]), "+v"(ta[s][1][1]),
                         "+v"(tb[s][0]), "+v"(tb[s][1]));
        } else {
          asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(ta[s][0][0]), "+v"(ta[s][0][1]), "+v"(tb[s][0]), "+v"(tb[s][1]));
        }
      }
#pragma unroll
      for (int r = 0; r < RBW; ++r) {
        const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(ta[s][r][0], ta[s][r][1], 0, 1, 2, 3));
#pragma unroll
        for (int d = 0; d < 2; ++d) acc[r][d] = mfma32(av, __builtin_bit_cast(bf16x8, tb[s][d]), acc[r][d]);
      }
    });
  };

  if (w0.next_block()) {
    // one walker, two steps ahead of the step computed: s0 is the step
    // computed, s1 the one whose K tile is loaded, s2 the one whose dS tiles
    // are loaded; past the end the loads repeat the last step (valid
    // addresses, unused data) so that every step issues the same loads
    DsStep s0 = w0.step(), s1 = s0, s2 = s0;
    bool a1 = w0.next();
    if (a1) s1 = w0.step();
    bool a2 = a1 && w0.next();
    s2 = a2 ? w0.step() : s1;
    load_ds(s0, 0);
    load_kop(s0, 0);
    load_ds(s1, 1);
    bool a0 = true;
    int32_t t = 0;
    while (a0) {
      // this step's dS tiles and K tile have landed (the loads issued after
      // the K tile: the dS tiles of step t + 1, one step's worth)
      wait_vm<DS_LOADS>();
      wg_barrier();
      load_kop(s1, (t + 1) & 1);
      load_ds(s2, (t + 2) % L::NDS);
      if (s0.meets & (1 << qh)) compute(t % L::NDS, t & 1);
      s0 = s1;
      s1 = s2;
      a0 = a1;
      a1 = a2;
      if (a2) {
        a2 = w0.next();
        if (a2) s2 = w0.step();
      }
      ++t;
    }
    wait_vm<0>();
  }

  // dQ = scale * acc: lane (hf, n) holds feature 32 (dt0 + d) + n of rows
  // 32 (rb0 + r) + 8 (e / 4) + 4 hf + e % 4 of tile 2 qp + qh
  const int32_t a_base = (2 * qp + qh) * kDsRows;
  __bf16* dqp = reinterpret_cast<__bf16*>(p.dq.ptr) + ri * p.dq.s_blk + b * p.dq.s_batch + h * p.dq.s_head;
#pragma unroll
  for (int r = 0; r < RBW; ++r)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int32_t a = a_base + 32 * (rb0 + r) + 8 * (e / 4) + 4 * hf + (e % 4);
      if (a < Bb) {
#pragma unroll
        for (int d = 0; d < 2; ++d) dqp[(int64_t)a * p.dq.s_tok + 32 * (dt0 + d) + n] = (__bf16)(acc[r][d][e] * p.scale);
      }
    }
}

template <typename K>
hipError_t launch_dyn(K kernel, int64_t grid, int bytes, hipStream_t s, const BwdParams& p) {
  if (grid <= 0) return hipSuccess;
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  hipLaunchKernelGGL(kernel, dim3((uint32_t)grid), dim3(kThreads), bytes, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kop_pack(const BwdParams& p, hipStream_t s) {
  const int64_t grid = (int64_t)p.B * p.Hk * p.P * ((p.Bb + kDsKeys - 1) / kDsKeys);
  if (p.D == 128) return launch_dyn(kop_pack_kernel<128>, grid, kDsKeys * 128 * 2, s, p);
  return launch_dyn(kop_pack_kernel<64>, grid, kDsKeys * 64 * 2, s, p);
}

hipError_t launch_dq_from_ds(const BwdParams& p, hipStream_t s) {
  const int64_t qtiles = (p.Bb + kDsRows - 1) / kDsRows;
  const int64_t grid = (int64_t)p.B * p.H * p.n_ranks * ((qtiles + 1) / 2);
  if (p.D == 128) return launch_dyn(dq_from_ds_kernel<128>, grid, DqLds<128>::BYTES, s, p);
  return launch_dyn(dq_from_ds_kernel<64>, grid, DqLds<64>::BYTES, s, p);
}

}  // namespace ra
