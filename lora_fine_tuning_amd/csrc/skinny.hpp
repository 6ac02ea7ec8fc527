// Rank-r products with a long reduction, one pass over the activations:
//
//   Z  = X  . A^T     out[M, r] = sum_k X[m, k]  A[j, k]      (A  [r, K], K-contiguous)
//   dZ = dY . B       out[M, r] = sum_n dY[m, n] B[n, j]      (B  [N, r], r-contiguous)
//
// These are HBM-bound (about r flops per byte of activations). A workgroup owns
// BM = 16 TM rows of the activations and all r output columns over one range
// of the reduction (blockIdx.z selects the range): the four waves share the
// range, accumulate with v_mfma_f32_16x16x32_bf16, and add their partial
// tiles through LDS at the end. Splitting the reduction gives the grid enough workgroups to keep HBM
// busy with BM large enough that the small operand (A or B, re-read once per
// row block) stays a minor share of the traffic. The four waves take the
// range's 32-wide chunks in turn (wave w: chunks w, w + 4, ..), so at any
// time they read neighbouring pieces of the same rows (measured: 5-9 % faster
// passes than contiguous quarters per wave). Operands are loaded straight
// into MFMA layout (16 bytes per lane); the r-contiguous B is staged per wave
// in LDS and read back transposed with ds_read_b64_tr_b16. Outputs: with one
// range, out1 = bf16(alpha1 acc), out2 = bf16(alpha2 acc); with several, fp32
// partials part[range][row][col], summed by the deterministic reduction.
#pragma once

#include "common.hpp"

namespace lora4 {
namespace skinny {

struct Params {
  const uint16_t *act;   // [M, R] activations (absolute rows)
  int64_t ld_act;
  const uint16_t *w;     // TRANSB 0: [r, R] per group; TRANSB 1: [R, r] per group
  int64_t ld_w;
  int64_t g_w;           // elements per group of w
  int64_t R, M;
  int r;
  const int64_t *offsets;
  int groups;
  uint16_t *out1;        // [M, r]
  float alpha1;
  uint16_t *out2;        // [M, r] or nullptr
  float alpha2;
  int64_t klen;          // reduction elements per range (multiple of 32)
  float *part;           // [ranges][M][r] fp32 when gridDim.z > 1
};

constexpr int THREADS = 256;

// 16 bytes of row `row` of a bf16 matrix at column k (zero past `kend`,
// element-wise when the 16-byte load would be misaligned or cross kend).
__device__ __forceinline__ u32x4_t load8(const uint16_t *base, int64_t ld, int64_t row, bool row_ok, int64_t k,
                                         int64_t kend, bool vec_ok) {
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (row_ok && k < kend) {
    const uint16_t *src = base + row * ld + k;
    if (vec_ok && k + 8 <= kend) {
      v = *reinterpret_cast<const u32x4_t *>(src);
    } else {
      uint32_t w4[4] = {0u, 0u, 0u, 0u};
      for (int j = 0; j < 8; ++j)
        if (k + j < kend) w4[j >> 1] |= (uint32_t)src[j] << (16 * (j & 1));
      v = u32x4_t{w4[0], w4[1], w4[2], w4[3]};
    }
  }
  return v;
}

template <int TM, int TJ, int TRANSB>
__global__ __launch_bounds__(THREADS) void k_rows_skinny(Params p) {
  constexpr int BM = 16 * TM, BN = 16 * TJ;
  // per-wave staging of the transposed operand: 32 reduction rows x BN (+pad)
  constexpr int LDS_T = BN + 16;
  __shared__ __attribute__((aligned(16))) uint16_t stage[TRANSB ? 4 * 32 * LDS_T : 8];
  // the four waves' partial tiles are added through LDS in rounds of RS
  // accumulator slots (at most 32 KB)
  constexpr int SLOTS = TM * TJ * 4;
  constexpr int RS = SLOTS < 32 ? SLOTS : 32;
  __shared__ __attribute__((aligned(16))) float red[4][RS][64];

  const RowTile rt = map_row_tile(blockIdx.x, BM, p.offsets, p.groups, p.M);
  if (rt.group < 0) return;
  const int g = rt.group;
  const int64_t row0 = rt.row0, row_end = rt.row_end;
  const int j0 = blockIdx.y * BN;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint16_t *w = p.w + g * p.g_w;

  // this wave's share of the workgroup's range, in 32-wide chunks: local
  // chunk i is chunk cmap(i), i < n_local
  const int64_t chunks = (p.R + 31) / 32;
  const int64_t r_begin = (int64_t)blockIdx.z * (p.klen / 32);
  const int64_t r_end = r_begin + p.klen / 32 < chunks ? r_begin + p.klen / 32 : chunks;
  // waves interleaved (wave w takes chunks w, w + 4, ..): the four waves read
  // neighbouring 64-byte pieces of each row at about the same time
  const int64_t n_local = r_end - r_begin > wave ? (r_end - r_begin - wave + 3) / 4 : 0;
  auto cmap = [&](int64_t i) { return r_begin + wave + 4 * i; };

  const bool act_vec = (p.ld_act % 8) == 0;
  const bool w_vec = (p.ld_w % 8) == 0;
  const int lr = lane & 15, lg = lane >> 4;

  f32x4_t acc[TM][TJ];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint16_t *st = stage + wave * 32 * LDS_T;

  auto load_chunk = [&](int64_t c, u32x4_t af[TM], u32x4_t bw[TJ]) {
    const int64_t k = c * 32 + lg * 8;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int64_t row = row0 + i * 16 + lr;
      af[i] = load8(p.act, p.ld_act, row, row < row_end, k, p.R, act_vec);
    }
    if constexpr (TRANSB == 0) {
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int64_t jr = j0 + j * 16 + lr;
        bw[j] = load8(w, p.ld_w, jr, jr < p.r, k, p.R, w_vec);
      }
    } else {
      // raw rows of w (reduction rows c*32 .. +31, columns j0 .. j0+BN-1):
      // BN/8 16-byte pieces per row, spread over the lanes
#pragma unroll
      for (int q = 0; q < TJ; ++q) {
        const int idx = lane + 64 * q;
        const int rr = idx / (BN / 8), cc = (idx % (BN / 8)) * 8;
        const int64_t kr = c * 32 + rr;
        bw[q] = load8(w, p.ld_w, kr, kr < p.R, j0 + cc, p.r, w_vec);
      }
    }
  };

  auto compute_chunk = [&](const u32x4_t af[TM], const u32x4_t bw[TJ]) {
    u32x4_t bf[TJ];
    if constexpr (TRANSB == 0) {
#pragma unroll
      for (int j = 0; j < TJ; ++j) bf[j] = bw[j];
    } else {
#pragma unroll
      for (int q = 0; q < TJ; ++q) {
        const int idx = lane + 64 * q;
        const int rr = idx / (BN / 8), cc = (idx % (BN / 8)) * 8;
        lds_write_b128(st + rr * LDS_T + cc, bw[q]);
      }
      // lane (column lr, group lg) gets reduction rows 8 lg .. 8 lg + 7
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const uint16_t *q0 = st + (lg * 8 + (lr >> 2)) * LDS_T + j * 16 + (lr & 3) * 4;
        const u32x2_t lo = lds_read_tr16(q0);
        const u32x2_t hi = lds_read_tr16(q0 + 4 * LDS_T);
        bf[j] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
      }
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) acc[i][j] = mfma_16x16x32(af[i], bf[j], acc[i][j]);
  };

  // TRANSB: the 32 x BN raw tile is 4 BN 16-byte pieces = TJ per lane.
  // UNR chunks are loaded per group and two groups are in flight, so every
  // lane keeps 2 UNR (TM + TJ) 16-byte loads outstanding (HBM-bound pass).
  constexpr int UNR = (TM + TJ) <= 2 ? 4 : (TM + TJ) <= 4 ? 2 : 1;
  u32x4_t af0[UNR][TM], bw0[UNR][TJ], af1[UNR][TM], bw1[UNR][TJ];
  auto load_group = [&](int64_t i, u32x4_t (*af)[TM], u32x4_t (*bw)[TJ]) {
#pragma unroll
    for (int u = 0; u < UNR; ++u)
      if (i + u < n_local) load_chunk(cmap(i + u), af[u], bw[u]);
  };
  auto compute_group = [&](int64_t i, u32x4_t (*af)[TM], u32x4_t (*bw)[TJ]) {
#pragma unroll
    for (int u = 0; u < UNR; ++u)
      if (i + u < n_local) compute_chunk(af[u], bw[u]);
  };
  if (n_local > 0) load_group(0, af0, bw0);
  for (int64_t i = 0; i < n_local; i += 2 * UNR) {
    if (i + UNR < n_local) load_group(i + UNR, af1, bw1);
    compute_group(i, af0, bw0);
    if (i + 2 * UNR < n_local) load_group(i + 2 * UNR, af0, bw0);
    if (i + UNR < n_local) compute_group(i + UNR, af1, bw1);
  }

  // add the four waves' partial tiles, RS slots at a time
#pragma unroll
  for (int r0 = 0; r0 < SLOTS; r0 += RS) {
    if (r0 > 0) __syncthreads();   // the previous round's reads are done
#pragma unroll
    for (int q = 0; q < RS; ++q) {
      const int slot = r0 + q;
      red[wave][q][lane] = acc[(slot / 4) / TJ][(slot / 4) % TJ][slot % 4];
    }
    __syncthreads();
    for (int o = threadIdx.x; o < RS * 64; o += THREADS) {
      const int q = o / 64, ln = o % 64;
      const int slot = r0 + q;
      const float v = red[0][q][ln] + red[1][q][ln] + red[2][q][ln] + red[3][q][ln];
      const int i = (slot / 4) / TJ, j = (slot / 4) % TJ, e = slot % 4;
      // 16x16 result layout: lane ln holds row 4 (ln / 16) + e, column ln % 16
      const int64_t row = row0 + i * 16 + (ln >> 4) * 4 + e;
      const int col = j0 + j * 16 + (ln & 15);
      if (gridDim.z > 1) {
        if (row < row_end && col < p.r) p.part[((int64_t)blockIdx.z * p.M + row) * p.r + col] = v;
        continue;
      }
      if (row < row_end && col < p.r) {
        p.out1[row * p.r + col] = to_bf16(v * p.alpha1);
        if (p.out2) p.out2[row * p.r + col] = to_bf16(v * p.alpha2);
      }
    }
  }
}

}  // namespace skinny
}  // namespace lora4
