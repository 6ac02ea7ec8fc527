// The 4-bit storage formats of the frozen base and their device decoders.
//
// NF4 ("Training LLMs on a Budget: LoRA, QLoRA, and LoftQ", section 3, trick
// 1): 16 levels at normal quantiles, normalised to [-1, 1], applied per block
// of 64 consecutive K-elements with an fp32 absmax scale (trick 2). The
// dequantized element is bf16(fp32(q[code] * scale)): one fp32 product, one
// round-to-nearest-even.
//
// NF4 double quantization (same section, trick 2): the per-64 scales are
// stored as OCP E4M3FN codes with one fp32 second-level scale per 256
// consecutive first-level scales; the rebuilt scale is
// fp32(E4M3(code) * scale2).
//
// MXFP4 ("Fine-Tuning 4-Bit Models", section "Case 2"): E2M1 codes with one
// E8M0 scale 2^(E-127) per 32 consecutive K-elements. gfx950's
// v_cvt_scalef32_pk_bf16_fp4 converts two codes and the scale to two bf16
// values; it agrees bit for bit with the exact product rounded to bf16 for
// all 16 x 16 code pairs and all finite scales (checked on the device).
//
// Packing: row-major (the oracle's bytes, lora4_import_rowmajor's input):
// byte j of a row holds element 2j in its low nibble and element 2j+1 in its
// high nibble. The tiled storage keeps that order for MXFP4 and NVFP4 (the
// hardware FP4 convert takes element pairs from one byte); for NF4 and
// NF4-DQ, byte j of each 32-bit word of codes (elements 8w .. 8w+7 of the
// row) holds element 8w + j in its low nibble and 8w + j + 4 in its high
// nibble, so the table lookups take both halves' indices straight from the
// word (nf4_nibble).
#pragma once

#include "common.hpp"

namespace lora4 {

enum Fmt : int { FMT_BF16 = 0, FMT_NF4 = 1, FMT_NF4_DQ = 2, FMT_MXFP4 = 3, FMT_NVFP4 = 4 };

// The NF4 levels (ascending) and the 15 decision thresholds of the encoder.
// thr[i] is the largest fp32 value not above the exact midpoint of levels i
// and i+1, so "x > thr[i]" holds exactly when x is strictly nearer level
// i+1: counting exceeded thresholds gives the nearest level, ties to the
// lower one. Both tables are built on the host (lora4_abi.cpp).
struct Nf4Table {
  float q[16];
  float thr[15];
};

// E4M3FN code -> float (exact). 0x7F / 0xFF are NaN.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t s = (c >> 7) & 1u, e = (c >> 3) & 15u, m = c & 7u;
  float mag;
  if ((c & 0x7Fu) == 0x7Fu) {
    mag = __builtin_nanf("");
  } else if (e == 0) {
    mag = (float)m * 0x1p-9f;
  } else {
    mag = __builtin_bit_cast(float, ((e + 120u) << 23) | (m << 20));
  }
  return s ? -mag : mag;
}

// E8M0 code -> the fp32 scale operand of v_cvt_scalef32_pk_bf16_fp4:
// 2^(E-127); E = 0 is the fp32 subnormal 2^-127; E = 255 is NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t E) {
  uint32_t bits = (E == 0u) ? 0x00400000u : (E == 255u ? 0x7FC00000u : (E << 23));
  return __builtin_bit_cast(float, bits);
}

// Bit offset of element i (0..7) within an NF4 code word of the tiled storage.
__host__ __device__ constexpr int nf4_nibble(int i) { return i < 4 ? 8 * i : 8 * (i - 4) + 4; }

// Dequantize 32 consecutive NF4 elements (16 code bytes, tiled storage)
// sharing one scale into 16 words of bf16 pairs (element 2j in the low half
// of word j).
// qlds: the 16 fp32 levels in LDS (each lane reads its own level; the 16
// entries sit in 16 different banks, so the reads never conflict).
__device__ __forceinline__ void dequant32_nf4(u32x4_t codes, float scale, const float *qlds,
                                              uint32_t out[16]) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t w = codes[d];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t lo = (w >> nf4_nibble(2 * p)) & 15u;
      uint32_t hi = (w >> nf4_nibble(2 * p + 1)) & 15u;
      float a = qlds[lo] * scale;
      float b = qlds[hi] * scale;
      out[4 * d + p] = pack_bf16x2(a, b);
    }
  }
}

// Dequantize 32 consecutive MXFP4 elements (16 code bytes) sharing one E8M0
// scale into 16 words of bf16 pairs.
// 8 E2M1 codes (one word) times an arbitrary fp32 scale into 4 bf16 pairs:
// the convert's own scale operand applies only its exponent, so the codes are
// converted to fp32 at scale 1 and multiplied by s (E2M1 x E4M3 has at most 6
// significant bits: exact, and so is the bf16 rounding).
template <int SEL>
__device__ __forceinline__ uint32_t nvfp4_pair_t(uint32_t c, float s) {
  const auto f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, SEL);
  return pack_bf16x2(f[0] * s, f[1] * s);
}
__device__ __forceinline__ u32x4_t decode8_nvfp4(uint32_t c, float s) {
  return u32x4_t{nvfp4_pair_t<0>(c, s), nvfp4_pair_t<1>(c, s), nvfp4_pair_t<2>(c, s), nvfp4_pair_t<3>(c, s)};
}

// Dequantize 32 consecutive NVFP4 elements (16 code bytes) with the scales
// s0 (elements 0..15) and s1 (16..31) into 16 words of bf16 pairs.
__device__ __forceinline__ void dequant32_nvfp4(u32x4_t codes, float s0, float s1, uint32_t out[16]) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const u32x4_t v = decode8_nvfp4(codes[d], d < 2 ? s0 : s1);
    out[4 * d + 0] = v[0];
    out[4 * d + 1] = v[1];
    out[4 * d + 2] = v[2];
    out[4 * d + 3] = v[3];
  }
}

__device__ __forceinline__ void dequant32_mxfp4(u32x4_t codes, float scale, uint32_t out[16]) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t w = codes[d];
    out[4 * d + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
    out[4 * d + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
    out[4 * d + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
    out[4 * d + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
  }
}

// Storage of a packed base: each group's [N, K] is cut into tiles of 64 rows
// by 64 elements (RB = ceil(N / 64) row blocks, KB = ceil(K / 64) k blocks;
// tile (rb, kb) is number rb KB + kb). A tile's codes are 2048 contiguous
// bytes, 32 per row (nibble order above); its scales are 64 contiguous entries (one per row, NF4 and
// NF4-DQ) or 128 (two per row, MXFP4). Rows past N and elements past K are
// zero. One step of either GEMM reads one tile per wave, so every global load
// of codes covers whole contiguous rows of a tile.
__host__ __device__ constexpr int64_t w_blocks(int64_t x) { return (x + 63) >> 6; }

// byte of the codes holding elements k, k + 1 (k even) of row n
__host__ __device__ constexpr int64_t w_code_off(int64_t KB, int64_t n, int64_t k) {
  return (((n >> 6) * KB + (k >> 6)) << 11) + ((n & 63) << 5) + ((k & 63) >> 1);
}
// scale entry of the 64-element block of (n, k) (NF4, NF4-DQ)
__host__ __device__ constexpr int64_t w_scale64_idx(int64_t KB, int64_t n, int64_t k) {
  return (((n >> 6) * KB + (k >> 6)) << 6) + (n & 63);
}
// scale entry of the 32-element block of (n, k) (MXFP4)
__host__ __device__ constexpr int64_t w_scale32_idx(int64_t KB, int64_t n, int64_t k) {
  return (((n >> 6) * KB + (k >> 6)) << 7) + ((n & 63) << 1) + ((k >> 5) & 1);
}
// scale entry of the 16-element block of (n, k) (NVFP4: 256 per tile, row i's
// four at 4 i)
__host__ __device__ constexpr int64_t w_scale16_idx(int64_t KB, int64_t n, int64_t k) {
  return (((n >> 6) * KB + (k >> 6)) << 8) + ((n & 63) << 2) + ((k >> 4) & 3);
}

// A packed base W as the kernels see it (one group; the kernels add the
// group offsets).
struct PackedW {
  const uint8_t *codes;   // [groups][RB KB tiles][64][32]
  const void *scales;     // fp32 (NF4), e4m3 u8 (NF4_DQ, NVFP4), e8m0 u8 (MXFP4), tiled
  const float *scales2;   // NF4_DQ second level, [groups][ceil(N*K/64/256)]
  int64_t N, K;
  int64_t KB;             // k blocks of 64
  int64_t g_codes;        // bytes per group
  int64_t g_scales;       // scale entries per group
  int64_t g_scales2;      // second-level entries per group
  int32_t shared;         // 1: one W for every row group (adapters over one base)
};

// group of W that row group g reads
__device__ __forceinline__ int w_group(const PackedW &w, int g) { return w.shared ? 0 : g; }

// Scale of the block holding (row n, element k) of group g, as the fp32
// operand the dequantizer needs (the E8M0 operand for MXFP4; for NVFP4 the
// 16-element block's E4M3 value).
template <int FMT>
__device__ __forceinline__ float block_scale(const PackedW &w, int g, int64_t n, int64_t k) {
  g = w_group(w, g);
  if constexpr (FMT == FMT_NF4) {
    const float *s = reinterpret_cast<const float *>(w.scales) + g * w.g_scales;
    return s[w_scale64_idx(w.KB, n, k)];
  } else if constexpr (FMT == FMT_NF4_DQ) {
    const uint8_t *s = reinterpret_cast<const uint8_t *>(w.scales) + g * w.g_scales;
    // the second-level groups run over the scales in row-major order
    const int64_t idx = n * (w.K >> 6) + (k >> 6);
    float c2 = w.scales2[g * w.g_scales2 + (idx >> 8)];
    return e4m3_to_f32(s[w_scale64_idx(w.KB, n, k)]) * c2;
  } else if constexpr (FMT == FMT_NVFP4) {
    const uint8_t *s = reinterpret_cast<const uint8_t *>(w.scales) + g * w.g_scales;
    return e4m3_to_f32(s[w_scale16_idx(w.KB, n, k)]);
  } else {
    const uint8_t *s = reinterpret_cast<const uint8_t *>(w.scales) + g * w.g_scales;
    return e8m0_to_f32(s[w_scale32_idx(w.KB, n, k)]);
  }
}

// Dequantize elements k .. k+31 of row n (k a multiple of 32) into 16 words.
template <int FMT>
__device__ __forceinline__ void dequant_row32(const PackedW &w, int g, int64_t n, int64_t k,
                                              const float *qlds, uint32_t out[16]) {
  const uint8_t *src = w.codes + w_group(w, g) * w.g_codes + w_code_off(w.KB, n, k);
  u32x4_t codes = ldg_b128_cached(src);
  float sc = block_scale<FMT>(w, g, n, k);
  if constexpr (FMT == FMT_NVFP4) {
    dequant32_nvfp4(codes, sc, block_scale<FMT>(w, g, n, k + 16), out);
  } else if constexpr (FMT == FMT_MXFP4) {
    dequant32_mxfp4(codes, sc, out);
  } else {
    dequant32_nf4(codes, sc, qlds, out);
  }
}

}  // namespace lora4
