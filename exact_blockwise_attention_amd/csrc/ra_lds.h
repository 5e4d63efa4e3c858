// ra_lds.h — LDS tile layouts and operand helpers shared by the kernels.
//
// Tiles of bf16 rows live in LDS row-major, unpadded, with the 16-byte
// chunks of each row permuted by an XOR swizzle of the row index. On gfx950
// the LDS serves 256 bytes per clock (64 banks of 4 bytes): a 16-byte read
// is served 16 lanes at a time, an 8-byte read 32 lanes at a time. The
// swizzle makes both read patterns the kernels use conflict-free (measured
// with the SQ_LDS_BANK_CONFLICT counter):
//   * MFMA row operands: 16 consecutive lanes read the same logical chunk of
//     16 consecutive rows;
//   * transposing reads (ds_read_b64_tr_b16): 32 lanes read 4 consecutive
//     rows (starting at a multiple of 4) times 64 consecutive bytes.
// For 256-byte rows (d = 128) the chunk index is XORed with
// ((r & 3) << 2) | ((r >> 2) & 3); for 128-byte rows (d = 64) with
// r1 | r2 << 1 | (r1 ^ r3) << 2 (r_k = bit k of the row).
// A transposing read returns, to lane i of each 16-lane group, element i%4
// of the 8 bytes read by lane 4e + i/4, for e = 0..3: with lane j reading
// row r0 + j/4, columns c0 + 4(j%4) .. +3 of a row-major [k][m] tile, lane i
// receives the column c0 + i for the four rows r0 .. r0+3 — four consecutive
// k of one m, which is how an MFMA operand wants them.
#ifndef RA_LDS_H_
#define RA_LDS_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace ra {

// A compile-time index (an LDS stage, an offset) passed to a generic lambda.
template <int N>
using ic = std::integral_constant<int, N>;

template <typename F, int... I>
__device__ __forceinline__ void unroll_seq(F& f, std::integer_sequence<int, I...>) {
  (f(ic<I>{}), ...);
}

// f(ic<0>{}), ..., f(ic<N-1>{}): straight-line code whose steps see their
// index as a constant.
template <int N, typename F>
__device__ __forceinline__ void unroll(F&& f) {
  unroll_seq(f, std::make_integer_sequence<int, N>{});
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int D>
__device__ __forceinline__ int chunk_swz(int r) {
  if (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  return ((r >> 1) & 1) | (((r >> 2) & 1) << 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 2);
}

// Element offset of (row r, column c) in a swizzled [rows][D] bf16 tile.
template <int D>
__device__ __forceinline__ int tile_off(int r, int c) {
  return r * D + ((((c >> 3) ^ chunk_swz<D>(r)) << 3) | (c & 7));
}

// Hides a value from the optimizer so that addresses derived from it are
// recomputed where they are used instead of being kept live across a loop
// (the transposing reads take no immediate offset, so every one of them
// would otherwise pin a register of its own).
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Byte address in LDS of a pointer into shared memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// LDS reads issued as inline assembly, at LDS byte address addr + OFF. The
// compiler, which cannot tell that the direct global-to-LDS copies in flight
// target other buffers, would wait for all of them before the equivalent
// builtins; for these reads it does not know, so the caller waits for the
// results itself with lds_wait*(). LDS reads complete in issue order, so
// waiting until at most N are outstanding, with N the number of reads issued
// after the ones needed, is enough whatever else is in flight.
template <int OFF>
__device__ __forceinline__ u32x2 tr_read_at(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "DS offsets are 16 bits");
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}

template <int OFF>
__device__ __forceinline__ u32x4 lds_read16(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "DS offsets are 16 bits");
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}

// s_waitcnt lgkmcnt(N) with the registers about to be used tied to it, so
// that their uses stay after the wait.
template <int N>
__device__ __forceinline__ void lds_wait(u32x2 (&r)[4][2]) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%8)"
               : "+v"(r[0][0]), "+v"(r[0][1]), "+v"(r[1][0]), "+v"(r[1][1]), "+v"(r[2][0]), "+v"(r[2][1]),
                 "+v"(r[3][0]), "+v"(r[3][1])
               : "n"(N));
}

template <int N>
__device__ __forceinline__ void lds_wait(u32x2 (&r)[2][2]) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(r[0][0]), "+v"(r[0][1]), "+v"(r[1][0]), "+v"(r[1][1]) : "n"(N));
}

template <int N>
__device__ __forceinline__ void lds_wait(u32x4 (&r)[2]) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(r[0]), "+v"(r[1]) : "n"(N));
}

template <int N>
__device__ __forceinline__ void lds_wait(u32x4 (&r)[4]) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]) : "n"(N));
}

template <int N>
__device__ __forceinline__ void lds_wait(u32x4 (&r)[6]) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%6)"
               : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5])
               : "n"(N));
}

}  // namespace ra

#endif  // RA_LDS_H_
