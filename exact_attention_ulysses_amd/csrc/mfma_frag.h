// MFMA operand fetch for gfx950 v_mfma_f32_32x32x16_bf16 (internal).
//
// Register layouts of the instruction (64 lanes, l = lane):
//   A (32 x 16, bf16x8): lane l holds A[l % 32][8 * (l / 32) + i], i = 0..7
//   B (16 x 32, bf16x8): lane l holds B[8 * (l / 32) + i][l % 32]
//   C (32 x 32, f32x16): lane l holds C[8 * (e / 4) + 4 * (l / 32) + e % 4][l % 32]
// Only the pairing of A's and B's k slots matters to the product, so an
// operand may enumerate its 16 k values in any order as long as the other
// operand uses the same one. Tiles live row-major in LDS; an operand whose k
// runs along a row is one 16-byte read per lane, an operand whose k runs down
// a column uses two ds_read_b64_tr_b16 transposing reads and enumerates k in
// the order in which a converted 32x32 accumulator holds its rows.
#pragma once

#include "common.h"

namespace ulysses {

// LDS row strides (elements) by how a tile is read; gfx950 LDS has 64 banks of
// 4 bytes, serves 16-byte reads in passes of 16 lanes and the transposing
// 8-byte reads in passes of 32 lanes (measured). A stride of 4 banks mod 64
// keeps 16 consecutive rows apart for row reads; 16 banks mod 64 keeps the 4
// rows of a transposing read apart; 12 banks mod 64 is conflict-free for row
// reads and 2-way for transposing reads (tiles read both ways).
template <int D> struct Stride;
template <> struct Stride<128> { static constexpr int row = 136, col = 160, both = 152; };
template <> struct Stride<64> { static constexpr int row = 72, col = 96, both = 88; };

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Buffer resource over one head's rows [base, base + bytes): loads whose
// vector offset lies past the range return zero (hardware range check), so
// tiles that run past the end of the sequence need no guards. Callers put the
// whole offset in the vector operand (scalar offset 0) so that the checked
// offset is the full one. Word 3 = 0x00020000 is the raw 32-bit data format of
// gfx9-family buffer descriptors.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
}


// Instruction classes for __builtin_amdgcn_sched_group_barrier (LLVM AMDGPU
// scheduling-group mask bits): a kernel lists groups in the order the
// scheduler must emit them, e.g. LDS reads a few fragments ahead of the MFMAs
// that consume them instead of one read, one wait, one MFMA at a time.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// fp32 operands (v_mfma_f32_32x32x2_f32): lane l holds A[l % 32][l / 32] and
// B[l / 32][l % 32]; the accumulator layout is the one above. The fp32 kernels
// pair accumulator rows 8 * (j / 4) + j % 4 (lanes 0-31) and the same + 4
// (lanes 32-63) as the two k slots of step j, so that element j of a 32x32
// accumulator is a ready B operand; the A operand of that step reads the same
// two rows of its LDS tile (kslot_row).
__device__ __forceinline__ f32x16 mfma32_f32(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int kslot_row(int j, int lane) { return 8 * (j >> 2) + (j & 3) + 4 * (lane >> 5); }

// fp32 LDS tiles: rows of D + 2 floats, so that the 64 lanes of a read of two
// adjacent columns over 32 rows (an operand whose k runs along a row) fall in
// 64 different banks.
template <int D> struct StrideF32 { static constexpr int row = D + 2; };

// k along a row: lane l gets T[row0 + l % 32][col0 + 8 * (l / 32) + i].
template <int STRIDE>
__device__ __forceinline__ bf16x8 frag_row(const __bf16* t, int row0, int col0, int lane) {
  return *reinterpret_cast<const bf16x8*>(t + (row0 + (lane & 31)) * STRIDE + col0 + 8 * (lane >> 5));
}

// k down a column: lane l gets T[row0 + 8 * (i / 4) + 4 * (l / 32) + i % 4][col0 + l % 32].
// ds_read_b64_tr_b16 hands lane j of each 16-lane group element j % 4 of the
// 8-byte blocks addressed by lanes 4i + j / 4 of the group; so lane 4i + c
// addresses row (its 4-row group) + i, columns 4c .. 4c + 3 of its 16-column half.
template <int STRIDE>
__device__ __forceinline__ bf16x8 frag_col(const __bf16* t, int row0, int col0, int lane) {
  const int j = lane & 15;
  const int row = row0 + 4 * (lane >> 5) + (j >> 2);
  const int col = col0 + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
  __bf16* p = const_cast<__bf16*>(t) + row * STRIDE + col;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 8 * STRIDE));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, both);
}

// Elements 8c .. 8c+7 of a 32x32 accumulator, rounded to bf16, as an operand
// whose k slots are accumulator rows 16c + 8 * (i / 4) + 4 * (l / 32) + i % 4:
// the same k order frag_col produces for rows starting at 16c.
__device__ __forceinline__ bf16x8 acc_chunk_bf16(const f32x16& a, int c) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)a[8 * c + i];
  return r;
}

// Four consecutive accumulator elements 4a .. 4a+3 (rows 8a + 4 * (l / 32) + 0..3)
// as bf16, for an 8-byte store.
__device__ __forceinline__ bf16x4 acc_quad_bf16(const f32x16& a, int q, float scale) {
  bf16x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = (__bf16)(a[4 * q + i] * scale);
  return r;
}

}  // namespace ulysses
