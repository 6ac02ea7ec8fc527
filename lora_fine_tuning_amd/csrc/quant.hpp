// Packing a bf16 base into NF4 (optionally double-quantized) or MXFP4.
// One pass over W, run once per weight. HBM-bound.
//
// NF4 ("Training LLMs on a Budget", section 3, tricks 1-2): per block of 64
// consecutive K-elements, c = max |w| (exact in fp32), x = fp32(w / c)
// (correctly rounded division; x = 0 when c = 0), code = nearest NF4 level
// with ties to the lower level (count of thresholds strictly exceeded).
// Double quantization (trick 2): the scales of one matrix, in row-major
// order, form groups of 256 consecutive entries; c2 = group max; the stored
// scale code is E4M3(fp32(c / c2)), nearest with ties to even.
//
// MXFP4 ("Fine-Tuning 4-Bit Models", section "Case 2"; OCP MX conversion):
// per block of 32, X = floor(log2 amax) - 2 clamped to [-127, 127]
// (X = -127 for an all-zero block), E = X + 127, v = w * 2^-X, code = nearest
// E2M1 magnitude (ties to the even code, saturating at 6) with w's sign.
//
// Codes and first-level scales are written in the 64 x 64 tile order of the
// packed base (w_code_off, w_scale64_idx, w_scale32_idx); the caller clears
// the padding of the last row and k blocks beforehand.
#pragma once

#include "formats.hpp"

namespace lora4 {

// Nearest E4M3FN code to a finite x >= 0, ties to even, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_encode_rne(float x) {
  if (!(x > 0.0f)) return 0u;
  if (x >= 448.0f) return 0x7Eu;
  const uint32_t b = __builtin_bit_cast(uint32_t, x);
  const int e = (int)(b >> 23) - 127;
  if (e < -6) {
    // subnormal E4M3 range: multiples of 2^-9 (x * 512 is exact); 8 -> 2^-6
    return (uint32_t)__builtin_rintf(x * 512.0f);
  }
  const uint32_t mant = b & 0x7FFFFFu;
  uint32_t m3 = mant >> 20;
  const uint32_t rem = mant & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (m3 & 1u))) ++m3;
  uint32_t E = (uint32_t)(e + 7);
  if (m3 == 8u) {
    m3 = 0u;
    ++E;
  }
  uint32_t code = (E << 3) | m3;
  return code > 0x7Eu ? 0x7Eu : code;
}

__device__ __forceinline__ uint32_t nf4_encode(float x, const Nf4Table &tab) {
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < 15; ++i) c += (x > tab.thr[i]) ? 1u : 0u;
  return c;
}

// Load the 64 bf16 of block (row n, block b) as 32 words.
__device__ __forceinline__ void load_block64(const uint16_t *W, int64_t K, int64_t n, int64_t b,
                                             uint32_t w[32]) {
  const u32x4_t *src = reinterpret_cast<const u32x4_t *>(W + n * K + b * 64);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    u32x4_t v = src[q];
    w[4 * q] = v[0];
    w[4 * q + 1] = v[1];
    w[4 * q + 2] = v[2];
    w[4 * q + 3] = v[3];
  }
}

// Encode one 64-block with scale c, write its 32 code bytes.
__device__ __forceinline__ void nf4_encode_block(const uint32_t w[32], float c, const Nf4Table &tab,
                                                 uint8_t *dst) {
  uint32_t out[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    uint32_t word = 0;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      // elements 8d + 2h, 8d + 2h + 1 live in word 4d + h
      uint32_t pair = w[4 * d + h];
      float a = bf16_bits_to_f32(pair & 0xFFFFu);
      float bb = bf16_bits_to_f32(pair >> 16);
      float xa = (c == 0.0f) ? 0.0f : a / c;
      float xb = (c == 0.0f) ? 0.0f : bb / c;
      word |= (nf4_encode(xa, tab) | (nf4_encode(xb, tab) << 4)) << (8 * h);
    }
    out[d] = word;
  }
  u32x4_t *o = reinterpret_cast<u32x4_t *>(dst);
  o[0] = u32x4_t{out[0], out[1], out[2], out[3]};
  o[1] = u32x4_t{out[4], out[5], out[6], out[7]};
}

__device__ __forceinline__ float absmax64(const uint32_t w[32]) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    m = fmaxf(m, fabsf(bf16_bits_to_f32(w[i] & 0xFFFFu)));
    m = fmaxf(m, fabsf(bf16_bits_to_f32(w[i] >> 16)));
  }
  return m;
}

// NF4 without double quantization: one thread per 64-element block.
__global__ void k_quant_nf4(const uint16_t *W, int64_t N, int64_t K, uint8_t *codes, float *scales,
                            Nf4Table tab) {
  const int64_t nb = K >> 6;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N * nb) return;
  const int64_t n = i / nb, b = i - n * nb;
  uint32_t w[32];
  load_block64(W, K, n, b, w);
  const float c = absmax64(w);
  const int64_t KB = w_blocks(K);
  nf4_encode_block(w, c, tab, codes + w_code_off(KB, n, b * 64));
  scales[w_scale64_idx(KB, n, b * 64)] = c;
}

// NF4 with double quantization: one 256-thread workgroup per group of 256
// consecutive scales; thread t owns scale index 256 G + t.
__global__ __launch_bounds__(256) void k_quant_nf4_dq(const uint16_t *W, int64_t N, int64_t K,
                                                      uint8_t *codes, uint8_t *code8, float *scales2,
                                                      Nf4Table tab) {
  __shared__ float red[256];
  const int64_t nb = K >> 6;
  const int64_t total = N * nb;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  float c = 0.0f;
  uint32_t w[32];
  if (i < total) {
    const int64_t n = i / nb, b = i - n * nb;
    load_block64(W, K, n, b, w);
    c = absmax64(w);
    nf4_encode_block(w, c, tab, codes + w_code_off(w_blocks(K), n, b * 64));
  }
  red[threadIdx.x] = c;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  const float c2 = red[0];
  if (i < total) {
    const float ratio = (c2 == 0.0f) ? 0.0f : c / c2;
    const int64_t n = i / nb, b = i - n * nb;
    code8[w_scale64_idx(w_blocks(K), n, b * 64)] = (uint8_t)e4m3_encode_rne(ratio);
  }
  if (threadIdx.x == 0) scales2[blockIdx.x] = c2;
}

// E2M1 magnitude code of a >= 0: nearest of {0,.5,1,1.5,2,3,4,6}, ties to the
// even code, saturating at 6.
__device__ __forceinline__ uint32_t e2m1_mag_code(float a) {
  return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
         (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
}

// floor(log2 a) for a finite a > 0 (normal or subnormal fp32), from its bits.
__device__ __forceinline__ int floor_log2_f32(float a) {
  const uint32_t b = __builtin_bit_cast(uint32_t, a);
  const int ef = (int)(b >> 23);
  if (ef > 0) return ef - 127;
  const uint32_t m = b & 0x7FFFFFu;
  return (31 - __builtin_clz(m)) - 149;
}

// MXFP4: one thread per 32-element block.
__global__ void k_quant_mxfp4(const uint16_t *W, int64_t N, int64_t K, uint8_t *codes, uint8_t *e8m0) {
  const int64_t nb = K >> 5;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N * nb) return;
  const int64_t n = i / nb, b = i - n * nb;
  const u32x4_t *src = reinterpret_cast<const u32x4_t *>(W + n * K + b * 32);
  uint32_t w[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    u32x4_t v = src[q];
    w[4 * q] = v[0];
    w[4 * q + 1] = v[1];
    w[4 * q + 2] = v[2];
    w[4 * q + 3] = v[3];
  }
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    amax = fmaxf(amax, fabsf(bf16_bits_to_f32(w[j] & 0xFFFFu)));
    amax = fmaxf(amax, fabsf(bf16_bits_to_f32(w[j] >> 16)));
  }
  int X = (amax == 0.0f) ? -127 : floor_log2_f32(amax) - 2;
  X = X < -127 ? -127 : (X > 127 ? 127 : X);
  uint32_t out[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t word = 0;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      uint32_t pair = w[4 * d + h];
      uint32_t lo16 = pair & 0xFFFFu, hi16 = pair >> 16;
      float a = __builtin_ldexpf(fabsf(bf16_bits_to_f32(lo16)), -X);
      float bb = __builtin_ldexpf(fabsf(bf16_bits_to_f32(hi16)), -X);
      uint32_t ca = e2m1_mag_code(a) | ((lo16 >> 15) << 3);
      uint32_t cb = e2m1_mag_code(bb) | ((hi16 >> 15) << 3);
      word |= (ca | (cb << 4)) << (8 * h);
    }
    out[d] = word;
  }
  const int64_t KB = w_blocks(K);
  *reinterpret_cast<u32x4_t *>(codes + w_code_off(KB, n, b * 32)) = u32x4_t{out[0], out[1], out[2], out[3]};
  e8m0[w_scale32_idx(KB, n, b * 32)] = (uint8_t)(X + 127);
}

// NVFP4: one thread per 16-element block. Scale code = E4M3 of amax / 6
// (the division is correctly rounded; amax / 6 is either exact in fp32 or not
// an E4M3 midpoint, so rounding it once more is exact), s = its value; each
// element's magnitude code counts the E2M1 midpoints below |w| / s, compared
// as |w| against midpoint x s (exact products), ties to the even code,
// saturating at 6; s == 0 gives magnitude 0. Sign copied.
__device__ __forceinline__ uint32_t nvfp4_mag_code(float a, float s) {
  if (!(s > 0.0f)) return 0u;
  return (uint32_t)(a > 0.25f * s) + (uint32_t)(a >= 0.75f * s) + (uint32_t)(a > 1.25f * s) +
         (uint32_t)(a >= 1.75f * s) + (uint32_t)(a > 2.5f * s) + (uint32_t)(a >= 3.5f * s) + (uint32_t)(a > 5.0f * s);
}

__global__ void k_quant_nvfp4(const uint16_t *W, int64_t N, int64_t K, uint8_t *codes, uint8_t *e4m3) {
  const int64_t nb = K >> 4;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N * nb) return;
  const int64_t n = i / nb, b = i - n * nb;
  const u32x4_t *src = reinterpret_cast<const u32x4_t *>(W + n * K + b * 16);
  uint32_t w[8];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const u32x4_t v = src[q];
    w[4 * q] = v[0];
    w[4 * q + 1] = v[1];
    w[4 * q + 2] = v[2];
    w[4 * q + 3] = v[3];
  }
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    amax = fmaxf(amax, fabsf(bf16_bits_to_f32(w[j] & 0xFFFFu)));
    amax = fmaxf(amax, fabsf(bf16_bits_to_f32(w[j] >> 16)));
  }
  const uint32_t sc = e4m3_encode_rne(fminf(amax / 6.0f, 448.0f));
  const float sv = e4m3_to_f32(sc);
  uint32_t out[2];
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    uint32_t word = 0;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const uint32_t pair = w[4 * d + h];
      const uint32_t lo16 = pair & 0xFFFFu, hi16 = pair >> 16;
      const uint32_t ca = nvfp4_mag_code(fabsf(bf16_bits_to_f32(lo16)), sv) | ((lo16 >> 15) << 3);
      const uint32_t cb = nvfp4_mag_code(fabsf(bf16_bits_to_f32(hi16)), sv) | ((hi16 >> 15) << 3);
      word |= (ca | (cb << 4)) << (8 * h);
    }
    out[d] = word;
  }
  const int64_t KB = w_blocks(K);
  *reinterpret_cast<u32x2_t *>(codes + w_code_off(KB, n, b * 16)) = u32x2_t{out[0], out[1]};
  e4m3[w_scale16_idx(KB, n, b * 16)] = (uint8_t)sc;
}

}  // namespace lora4
