// Packing a bf16 base into NF4 (optionally double-quantized), MXFP4 or NVFP4.
// One pass over W, run once per weight. HBM-bound: a lane per 16 bytes of W,
// so each wave reads 1 KiB of contiguous W per load.
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

// The packers take one lane per 8 consecutive elements (16 bytes) of W in
// row-major order: the 64 lanes of a wave read 1 KiB of contiguous W per
// load. K is a multiple of the block size (16, 32 or 64), so each block lies
// in one row and is held by block / 8 neighbouring lanes of one wave, which
// find its maximum by exchanging values (lanes of a block are all active or
// all inactive). A lane writes the 4 code bytes of its 8 elements (one word of
// a tile row); the first lane of a block writes the block's scale.
constexpr int PACK_THREADS = 256;
constexpr int64_t PACK_MAX_BLOCKS = int64_t(1) << 20;   // grid-stride beyond this

__device__ __forceinline__ u32x4_t load_chunk8(const uint16_t *W, int64_t chunk) {
  return *reinterpret_cast<const u32x4_t *>(W + chunk * 8);
}

// max over the NL lanes of an aligned group of lanes (NL a power of two)
template <int NL>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = 1; o < NL; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float absmax8(const u32x4_t v) {
  float m = 0.0f;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    m = fmaxf(m, fabsf(bf16_bits_to_f32(v[h] & 0xFFFFu)));
    m = fmaxf(m, fabsf(bf16_bits_to_f32(v[h] >> 16)));
  }
  return m;
}

// NF4 codes of 8 elements with block scale c, as one word of the tiled
// storage (element i at bit nf4_nibble(i)).
__device__ __forceinline__ uint32_t nf4_encode8(const u32x4_t v, float c, const Nf4Table &tab) {
  uint32_t word = 0;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const float a = bf16_bits_to_f32(v[h] & 0xFFFFu);
    const float b = bf16_bits_to_f32(v[h] >> 16);
    const float xa = (c == 0.0f) ? 0.0f : a / c;
    const float xb = (c == 0.0f) ? 0.0f : b / c;
    word |= (nf4_encode(xa, tab) << nf4_nibble(2 * h)) | (nf4_encode(xb, tab) << nf4_nibble(2 * h + 1));
  }
  return word;
}

// NF4 without double quantization.
__global__ __launch_bounds__(PACK_THREADS) void k_quant_nf4(const uint16_t *W, int64_t N, int64_t K, uint8_t *codes,
                                                            float *scales, Nf4Table tab) {
  const int64_t chunks = N * (K >> 3), KB = w_blocks(K);
  for (int64_t c = (int64_t)blockIdx.x * PACK_THREADS + threadIdx.x; c < chunks;
       c += (int64_t)gridDim.x * PACK_THREADS) {
    const u32x4_t v = load_chunk8(W, c);
    const float amax = group_max<8>(absmax8(v));
    const int64_t n = (c * 8) / K, k = c * 8 - n * K;
    *reinterpret_cast<uint32_t *>(codes + w_code_off(KB, n, k)) = nf4_encode8(v, amax, tab);
    if ((k & 63) == 0) scales[w_scale64_idx(KB, n, k)] = amax;
  }
}

// NF4 with double quantization: workgroup G packs the 256 blocks of
// second-level group G (row-major block order), 8 rounds of 32 blocks, then
// stores their scales as E4M3 of c / c2 with c2 the group's maximum.
__global__ __launch_bounds__(PACK_THREADS) void k_quant_nf4_dq(const uint16_t *W, int64_t N, int64_t K,
                                                               uint8_t *codes, uint8_t *code8, float *scales2,
                                                               Nf4Table tab) {
  __shared__ float red[PACK_THREADS / 64];
  const int64_t chunks = N * (K >> 3), KB = w_blocks(K);
  const int64_t c0 = (int64_t)blockIdx.x * 2048 + threadIdx.x;
  float cs[8];
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t c = c0 + j * PACK_THREADS;
    cs[j] = 0.0f;
    if (c < chunks) {
      const u32x4_t v = load_chunk8(W, c);
      cs[j] = group_max<8>(absmax8(v));
      m = fmaxf(m, cs[j]);
      const int64_t n = (c * 8) / K, k = c * 8 - n * K;
      *reinterpret_cast<uint32_t *>(codes + w_code_off(KB, n, k)) = nf4_encode8(v, cs[j], tab);
    }
  }
  m = group_max<64>(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  float c2 = red[0];
#pragma unroll
  for (int w = 1; w < PACK_THREADS / 64; ++w) c2 = fmaxf(c2, red[w]);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t c = c0 + j * PACK_THREADS;
    if (c < chunks) {
      const int64_t n = (c * 8) / K, k = c * 8 - n * K;
      if ((k & 63) == 0) {
        const float ratio = (c2 == 0.0f) ? 0.0f : cs[j] / c2;
        code8[w_scale64_idx(KB, n, k)] = (uint8_t)e4m3_encode_rne(ratio);
      }
    }
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

// MXFP4: blocks of 32 (4 lanes).
__global__ __launch_bounds__(PACK_THREADS) void k_quant_mxfp4(const uint16_t *W, int64_t N, int64_t K,
                                                              uint8_t *codes, uint8_t *e8m0) {
  const int64_t chunks = N * (K >> 3), KB = w_blocks(K);
  for (int64_t c = (int64_t)blockIdx.x * PACK_THREADS + threadIdx.x; c < chunks;
       c += (int64_t)gridDim.x * PACK_THREADS) {
    const u32x4_t v = load_chunk8(W, c);
    const float amax = group_max<4>(absmax8(v));
    int X = (amax == 0.0f) ? -127 : floor_log2_f32(amax) - 2;
    X = X < -127 ? -127 : (X > 127 ? 127 : X);
    uint32_t word = 0;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const uint32_t lo16 = v[h] & 0xFFFFu, hi16 = v[h] >> 16;
      const float a = __builtin_ldexpf(fabsf(bf16_bits_to_f32(lo16)), -X);
      const float b = __builtin_ldexpf(fabsf(bf16_bits_to_f32(hi16)), -X);
      const uint32_t ca = e2m1_mag_code(a) | ((lo16 >> 15) << 3);
      const uint32_t cb = e2m1_mag_code(b) | ((hi16 >> 15) << 3);
      word |= (ca | (cb << 4)) << (8 * h);
    }
    const int64_t n = (c * 8) / K, k = c * 8 - n * K;
    *reinterpret_cast<uint32_t *>(codes + w_code_off(KB, n, k)) = word;
    if ((k & 31) == 0) e8m0[w_scale32_idx(KB, n, k)] = (uint8_t)(X + 127);
  }
}

// NVFP4: blocks of 16 (2 lanes). Scale code = E4M3 of amax / 6 (the division
// is correctly rounded; amax / 6 is either exact in fp32 or not an E4M3
// midpoint, so rounding it once more is exact), s = its value; each element's
// magnitude code counts the E2M1 midpoints below |w| / s, compared as |w|
// against midpoint x s (exact products), ties to the even code, saturating at
// 6; s == 0 gives magnitude 0. Sign copied.
__device__ __forceinline__ uint32_t nvfp4_mag_code(float a, float s) {
  if (!(s > 0.0f)) return 0u;
  return (uint32_t)(a > 0.25f * s) + (uint32_t)(a >= 0.75f * s) + (uint32_t)(a > 1.25f * s) +
         (uint32_t)(a >= 1.75f * s) + (uint32_t)(a > 2.5f * s) + (uint32_t)(a >= 3.5f * s) + (uint32_t)(a > 5.0f * s);
}

__global__ __launch_bounds__(PACK_THREADS) void k_quant_nvfp4(const uint16_t *W, int64_t N, int64_t K,
                                                              uint8_t *codes, uint8_t *e4m3) {
  const int64_t chunks = N * (K >> 3), KB = w_blocks(K);
  for (int64_t c = (int64_t)blockIdx.x * PACK_THREADS + threadIdx.x; c < chunks;
       c += (int64_t)gridDim.x * PACK_THREADS) {
    const u32x4_t v = load_chunk8(W, c);
    const float amax = group_max<2>(absmax8(v));
    const uint32_t sc = e4m3_encode_rne(fminf(amax / 6.0f, 448.0f));
    const float sv = e4m3_to_f32(sc);
    uint32_t word = 0;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const uint32_t lo16 = v[h] & 0xFFFFu, hi16 = v[h] >> 16;
      const uint32_t ca = nvfp4_mag_code(fabsf(bf16_bits_to_f32(lo16)), sv) | ((lo16 >> 15) << 3);
      const uint32_t cb = nvfp4_mag_code(fabsf(bf16_bits_to_f32(hi16)), sv) | ((hi16 >> 15) << 3);
      word |= (ca | (cb << 4)) << (8 * h);
    }
    const int64_t n = (c * 8) / K, k = c * 8 - n * K;
    *reinterpret_cast<uint32_t *>(codes + w_code_off(KB, n, k)) = word;
    if ((k & 15) == 0) e4m3[w_scale16_idx(KB, n, k)] = (uint8_t)sc;
  }
}

// ---------------------------------------------------------------------------
// A base that ships already packed, in row-major order, into the tiled
// storage: codes [groups][N][K/2] and first-level scales [groups][N][K/block]
// rearranged bit for bit (padding written as zero). K % 32 == 0, so a 16-byte
// piece of a row's codes is either whole inside the row or past its end.
// ---------------------------------------------------------------------------

// A row-major NF4 code word (element i at bits 4i) in the tiled storage's
// nibble order (element i at nf4_nibble(i)).
__device__ __forceinline__ uint32_t nf4_word_to_tiled(uint32_t w) {
  uint32_t t = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) t |= ((w >> (4 * i)) & 15u) << nf4_nibble(i);
  return t;
}

// One thread per 16-byte piece c of the output: tile c / 128, row (c / 2) % 64,
// half c % 2. nf4: reorder the nibbles of each word (NF4, NF4-DQ).
__global__ void k_retile_codes(const uint8_t *src, int64_t N, int64_t K, int64_t groups, int nf4, uint8_t *dst) {
  const int64_t KB = w_blocks(K);
  const int64_t per_group = w_blocks(N) * KB * 128;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= groups * per_group) return;
  const int64_t g = idx / per_group;
  const int64_t c = idx - g * per_group;
  const int64_t t = c >> 7;
  const int64_t rb = t / KB, kb = t - rb * KB;
  const int64_t n = rb * 64 + ((c >> 1) & 63);
  const int64_t byte0 = kb * 32 + (c & 1) * 16;
  const int64_t row_bytes = K >> 1;
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (n < N && byte0 < row_bytes) v = *reinterpret_cast<const u32x4_t *>(src + (g * N + n) * row_bytes + byte0);
  if (nf4) v = u32x4_t{nf4_word_to_tiled(v[0]), nf4_word_to_tiled(v[1]), nf4_word_to_tiled(v[2]), nf4_word_to_tiled(v[3])};
  *reinterpret_cast<u32x4_t *>(dst + idx * 16) = v;
}

// One thread per scale entry of the output; a tile holds epr entries per row
// (1: NF4 and NF4-DQ, 2: MXFP4, 4: NVFP4), row i's at epr i .. epr i + epr - 1,
// entry q of row n of tile (rb, kb) being row-major column kb epr + q.
template <typename T>
__global__ void k_retile_scales(const T *src, int64_t N, int64_t K, int64_t groups, int epr, T *dst) {
  const int64_t KB = w_blocks(K);
  const int64_t per_tile = 64 * epr;
  const int64_t per_group = w_blocks(N) * KB * per_tile;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= groups * per_group) return;
  const int64_t g = idx / per_group;
  const int64_t e = idx - g * per_group;
  const int64_t t = e / per_tile, within = e - t * per_tile;
  const int64_t rb = t / KB, kb = t - rb * KB;
  const int64_t n = rb * 64 + within / epr;
  const int64_t col = kb * epr + within % epr;
  const int64_t cols = K * epr / 64;
  dst[idx] = (n < N && col < cols) ? src[(g * N + n) * cols + col] : T(0);
}

}  // namespace lora4
