// Device-side building blocks for gfx950 (CDNA4): bf16 packing, MFMA and
// transposing LDS reads, tile/group mapping.
//
// Verified lane layouts (gfx950, wave64):
//  * v_mfma_f32_16x16x32_bf16: operand A lane l holds A[l % 16][8*(l/16) + j],
//    operand B lane l holds B[8*(l/16) + j][l % 16] (j = 0..7); the result lane
//    l holds C[4*(l/16) + i][l % 16] (i = 0..3).
//  * ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives, for
//    t = 0..3, element (i % 4) of the 8-byte chunk addressed by lane
//    (i / 4 + 4 t) of the same group. If lane j of a group addresses row
//    (r0 + j / 4), columns (c0 + 4 (j % 4)) .. +3 of a row-major bf16 tile,
//    lane i receives column c0 + i of rows r0 .. r0 + 3: a transposed 4 x 16
//    block, which is exactly what an MFMA operand needs when the reduction
//    index runs along the tile's rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lora4 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// Two fp32 values -> one word of two bf16 (round to nearest even, the
// hardware v_cvt_pk_bf16_f32). Whole-vector bit casts only: element access on
// __bf16 vectors is avoided on purpose.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint16_t to_bf16(float x) {
  return (uint16_t)(pack_bf16x2(x, 0.0f) & 0xFFFFu);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __builtin_bit_cast(float, b16 << 16);
}

__device__ __forceinline__ f32x4_t mfma_16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// v_mfma_f32_32x32x16_bf16: operand A lane l holds A[l % 32][8*(l/32) + j],
// operand B lane l holds B[8*(l/32) + j][l % 32]; result register r of lane l
// holds C[8*(r/4) + 4*(l/32) + r%4][l % 32].
__device__ __forceinline__ f32x16_t mfma_32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Pins a value to this point of the instruction stream: an empty volatile asm
// that "redefines" it, so that work feeding it cannot sink below and work
// using it cannot rise above (the hand-built schedules fence their slices
// with it). No instruction is emitted.
__device__ __forceinline__ void pin(uint32_t &v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void pin(float &v) { asm volatile("" : "+v"(v)); }

// Transposing 64-bit LDS read (see the layout note above).
// The pointer is declared restrict so that, once inlined, the read carries
// alias-scope metadata: without it the compiler cannot tell the read from a
// direct-to-LDS load still in flight and drains every outstanding vector-memory
// load before it. Every kernel here orders its LDS tiles with explicit waits
// and barriers.
__device__ __forceinline__ u32x2_t lds_read_tr16(const uint16_t *__restrict__ p) {
  i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(p));
  return __builtin_bit_cast(u32x2_t, v);
}

// LDS layout of a [rows][64] bf16 tile (128-byte rows, eight 16-byte chunks):
// chunk c of row r is stored at position c ^ ((r >> 1) & 7). The LDS serves a
// 16-byte-per-lane read to 16 lanes at a time (256 bytes, 64 banks); the MFMA
// operand reads give those 16 lanes 16 consecutive rows at one logical chunk,
// which this places in 16 different bank groups (two rows per 128-byte
// position, with distinct positions for rows of equal parity).
__device__ __forceinline__ int tile64_swz(int row, int chunk) { return row * 64 + ((chunk ^ ((row >> 1) & 7)) << 3); }

// Direct-to-LDS loads write lane l's 16 bytes at position l of a 1 KB block;
// with block (4 c + w) holding rows 8 (4 c + w) .. +7 (c = 0..7, wave w), the
// logical chunk lane l must fetch for the layout above.
__device__ __forceinline__ int tile64_dma_chunk(int lane, int wave) {
  return (lane & 7) ^ (((wave & 1) << 2) | (lane >> 4));
}

__device__ __forceinline__ u32x4_t lds_read_b128(const uint16_t *p) {
  return *reinterpret_cast<const u32x4_t *>(p);
}

__device__ __forceinline__ void lds_write_b128(uint16_t *p, u32x4_t v) {
  *reinterpret_cast<u32x4_t *>(p) = v;
}

__device__ __forceinline__ u32x4_t ldg_b128(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
}

__device__ __forceinline__ u32x4_t ldg_b128_cached(const void *p) {
  return *reinterpret_cast<const u32x4_t *>(p);
}

// Row range of one row tile of a (possibly grouped) problem.
struct RowTile {
  int group;       // -1: this workgroup has no tile
  int64_t row0;    // first row of the tile (absolute)
  int64_t row_end; // one past the last valid row of the group
};

// Maps a row-tile slot to (group, tile). Groups are row ranges
// offsets[e] .. offsets[e+1]; each group is cut into ceil(rows / BM) tiles in
// order. With offsets == nullptr there is a single group [0, M).
__device__ __forceinline__ RowTile map_row_tile(int slot, int BM, const int64_t *offsets,
                                                int groups, int64_t M) {
  RowTile t;
  if (offsets == nullptr) {
    t.group = 0;
    t.row0 = (int64_t)slot * BM;
    t.row_end = M;
    if (t.row0 >= M) t.group = -1;
    return t;
  }
  int64_t s = slot;
  for (int e = 0; e < groups; ++e) {
    int64_t a = offsets[e], b = offsets[e + 1];
    int64_t nt = (b - a + BM - 1) / BM;
    if (s < nt) {
      t.group = e;
      t.row0 = a + s * BM;
      t.row_end = b;
      return t;
    }
    s -= nt;
  }
  t.group = -1;
  t.row0 = 0;
  t.row_end = 0;
  return t;
}

}  // namespace lora4
