// ra_lds.h — LDS tile layouts and operand helpers shared by the kernels.
//
// Tiles of bf16 rows live in LDS row-major with rows padded by 32 bytes
// (row stride = 8 banks mod 32), and the two 16-byte halves of every 32-byte
// piece swapped on rows whose bit 2 is set. Both read patterns the kernels
// use are then free of bank conflicts, and addresses stay affine in the
// unrolled loop indices (the swap only involves lane-dependent bits):
//   * MFMA row operands: 8 consecutive lanes read the same 16-byte chunk of 8
//     consecutive rows (rows 0..3 land 8 banks apart, rows 4..7 shifted by 4);
//   * transposing reads (ds_read_b64_tr_b16): 16 lanes read 8 bytes each
//     from 4 consecutive rows (starting at a multiple of 4) and one 32-byte
//     piece of each, 8 banks apart.
// A transposing read returns, to lane i of each 16-lane group, element i%4
// of the 8 bytes read by lane 4e + i/4, for e = 0..3: with lane j reading
// row r0 + j/4, columns c0 + 4(j%4) .. +3 of a row-major [k][m] tile, lane i
// receives the column c0 + i for the four rows r0 .. r0+3 — four consecutive
// k of one m, which is how an MFMA operand wants them.
#ifndef RA_LDS_H_
#define RA_LDS_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Row stride (elements) of a padded [rows][D] bf16 tile.
template <int D>
struct PadRow {
  static constexpr int RS = D + 16;
};

// Element offset of (row r, column c) in a padded [rows][D] bf16 tile.
template <int D>
__device__ __forceinline__ int tile_off(int r, int c) {
  return r * PadRow<D>::RS + ((((c >> 3) ^ ((r >> 2) & 1)) << 3) | (c & 7));
}

// 8-byte unit swizzle for [rows][64] bf16 tiles (128-byte rows) written in
// 8-byte pieces by 16 lanes on 16 consecutive rows and read by transposing
// reads on 4 consecutive rows and 4 consecutive units.
__device__ __forceinline__ int swz8(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

__device__ __forceinline__ int tile64_off(int r, int c) {
  return r * 64 + ((((c >> 2) ^ swz8(r)) << 2) | (c & 3));
}

__device__ __forceinline__ bf16x4 tr_read(const __bf16* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

// Hides a value from the optimizer so that addresses derived from it are
// recomputed where they are used instead of being kept live across a loop
// (the transposing reads take no immediate offset, so every one of them
// would otherwise pin a register of its own).
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ bf16x8 cat(bf16x4 lo, bf16x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace ra

#endif  // RA_LDS_H_
