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
#include "gemm_big.hpp"

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
  // side job of block (0, 0, 0): zero_n words at `zero` set to 0 (the
  // arrival counters of a later launch of the same backward), or none
  unsigned *zero;
  int64_t zero_n;
};

constexpr int THREADS = 256;

// The side job (Params::zero), written through to memory.
__device__ __forceinline__ void zero_side_job(const Params &p) {
  if (p.zero && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0)
    for (int64_t i = threadIdx.x; i < p.zero_n; i += THREADS)
      __hip_atomic_store(&p.zero[i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

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

  zero_side_job(p);
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

// The same products through an LDS ring, for whole 16-byte pieces (the
// reduction length, both leading dimensions and, for dZ, the rank multiples of
// 8). Every load is a direct-to-LDS load of one 16-byte piece per lane, eight
// lanes per 128-byte row segment, so each load instruction reads whole cache
// lines (the register path above reads 64 bytes of each of 16 rows, half
// lines, and measured 2-3 TB/s at ranks 64 and 128). A step is 64 deep: the
// activation tile [BM rows][64] in the conflict-free tile64 layout and the
// small operand's tile (A [BN rows][64] in the same layout, or B [64 rows][BN]
// with its 16-byte pieces XOR-swizzled per row for the transposing reads).
// The four waves split the rows (wave w: rows 16 TM w ..) and share the small
// operand's tile, so it is read once per workgroup and no partial sums cross
// waves. NS stages, loads issued NS - 1 steps ahead; the loads past the range
// are issued as out-of-range loads (zeros), so every wave has the same number
// of loads in flight per step.
template <int TM, int TJ, int TRANSB, int NS>
struct LdsRing {
  static constexpr int BM = 64 * TM, BN = 16 * TJ;
  static constexpr int XT = BM * 64;                      // activation stage, bf16 elements
  static constexpr int WB = BN / 8;                       // 1 KB blocks of the small operand's stage
  static constexpr int WPW = (WB + 3) / 4;                // of them per wave (padded with empty loads)
  static constexpr int ST = XT + WPW * 4 * 512;           // stage size, bf16 elements
  static constexpr int LPS = BM / 32 + WPW;               // loads per wave per step
  static constexpr int bytes() { return NS * ST * 2; }
};

// B stage [64][BN] (TRANSB 1): 16-byte piece q of row n stored at q ^ bsw(n),
// which spreads the four rows of a transposing read over different banks.
template <int BN>
__device__ __forceinline__ int bsw(int n) {
  return BN >= 64 ? (n & 3) << 1 : 0;
}

template <int TM, int TJ, int TRANSB, int NS>
__global__ __launch_bounds__(THREADS) void k_rows_lds(Params p) {
  using Ring = LdsRing<TM, TJ, TRANSB, NS>;
  constexpr int BM = Ring::BM, BN = Ring::BN, XT = Ring::XT, WB = Ring::WB, WPW = Ring::WPW, ST = Ring::ST;
  constexpr int PPR = BN / 8;   // 16-byte pieces per row of the B stage
  extern __shared__ __attribute__((aligned(16))) uint16_t ring[];

  zero_side_job(p);
  const RowTile rt = map_row_tile(blockIdx.x, BM, p.offsets, p.groups, p.M);
  if (rt.group < 0) return;
  const int g = rt.group;
  const int64_t row0 = rt.row0, row_end = rt.row_end;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  // this workgroup's rank columns: j0 .. j0 + BN - 1 (grid.y covers ranks
  // above BN)
  const int j0 = blockIdx.y * BN;

  // this workgroup's range of 64-deep steps, and where its loads stop
  const int64_t nsteps_all = (p.R + 63) / 64;
  const int64_t s_begin = (int64_t)blockIdx.z * (p.klen / 64);
  const int64_t s_end = s_begin + p.klen / 64 < nsteps_all ? s_begin + p.klen / 64 : nsteps_all;
  const int nsteps = s_end > s_begin ? (int)(s_end - s_begin) : 0;
  const int64_t k_lim = s_end * 64 < p.R ? s_end * 64 : p.R;

  // activations: rows of this tile, 8 (4 c + wave) + lane / 8 (c < BM / 32)
  const big::rsrc_t x_rsrc =
      big::make_rsrc(p.act + row0 * p.ld_act, big::clamp_bytes((row_end - row0) * p.ld_act * 2));
  const int x_kq = tile64_dma_chunk(lane, wave) * 8;
  const uint32_t x_voff0 = (uint32_t)(((wave * 8 + (lane >> 3)) * p.ld_act + x_kq) * 2);
  const uint32_t x_cstep = (uint32_t)(32 * p.ld_act * 2);

  // the small operand of this group: A [r][R] (TRANSB 0) or B [R][r] (TRANSB 1)
  const uint16_t *w = p.w + g * p.g_w;
  const big::rsrc_t w_rsrc = big::make_rsrc(
      w, big::clamp_bytes((TRANSB ? p.R * p.ld_w : (int64_t)p.r * p.ld_w) * 2));
  // per load i < WPW of this wave: the piece's offset at step 0 (or OOB) and
  // the element it covers along the reduction (to cut at k_lim)
  uint32_t w_voff[WPW];
  int w_k[WPW];
#pragma unroll
  for (int i = 0; i < WPW; ++i) {
    const int b = wave + 4 * i;   // 1 KB block of the stage
    w_voff[i] = big::OOB;
    w_k[i] = 0;
    if (b < WB) {
      if constexpr (TRANSB == 0) {
        const int j = j0 + 8 * b + (lane >> 3);                  // A row (rank index)
        const int kq = tile64_dma_chunk(lane, b) * 8;
        w_k[i] = kq;
        if (j < p.r) w_voff[i] = (uint32_t)((j * p.ld_w + kq) * 2);
      } else {
        const int P = b * 64 + lane;                             // flat piece of the [64][BN] stage
        const int n = P / PPR, q = (P % PPR) ^ bsw<BN>(n);
        w_k[i] = n;
        if (j0 + q * 8 < p.r) w_voff[i] = (uint32_t)((n * p.ld_w + j0 + q * 8) * 2);
      }
    }
  }

  auto issue = [&](int s) {
    uint16_t *st = ring + (s % NS) * ST;
    const int64_t k0 = (s_begin + s) * 64;
    const bool x_edge = k0 + x_kq >= k_lim;
#pragma unroll
    for (int c = 0; c < BM / 32; ++c)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(x_rsrc, (__attribute__((address_space(3))) void *)(st + (c * 4 + wave) * 512),
                                               16, x_edge ? big::OOB : x_voff0 + c * x_cstep, (int)(k0 * 2), 0, 0);
#pragma unroll
    for (int i = 0; i < WPW; ++i) {
      const uint32_t vo = w_voff[i];   // (the builtin's offset taken straight from the array
                                       // leaves the kernel without its host-side launch stub)
      const uint32_t off = vo == big::OOB || k0 + w_k[i] >= k_lim ? big::OOB : vo;
      const int so = TRANSB ? (int)(k0 * p.ld_w * 2) : (int)(k0 * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(w_rsrc, (__attribute__((address_space(3))) void *)(st + XT + (wave + 4 * i) * 512),
                                               16, off, so, 0, 0);
    }
  };

  f32x4_t acc[TM][TJ];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int s) {
    const uint16_t *xs = ring + (s % NS) * ST;
    const uint16_t *ws = xs + XT;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4_t af[TM], bf[TJ];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = lds_read_b128(xs + tile64_swz(16 * (TM * wave + i) + lr, ks * 4 + lg));
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        if constexpr (TRANSB == 0) {
          bf[j] = lds_read_b128(ws + tile64_swz(16 * j + lr, ks * 4 + lg));
        } else {
          // lane (column 16 j + lr, group lg): reduction rows 32 ks + 8 lg .. +7
          const int n = 32 * ks + 8 * lg + (lr >> 2), c = 16 * j + (lr & 3) * 4;
          const u32x2_t lo = lds_read_tr16(ws + n * BN + (((c >> 3) ^ bsw<BN>(n)) << 3) + (c & 7));
          const u32x2_t hi = lds_read_tr16(ws + (n + 4) * BN + (((c >> 3) ^ bsw<BN>(n + 4)) << 3) + (c & 7));
          bf[j] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
        }
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = mfma_16x16x32(af[i], bf[j], acc[i][j]);
    }
  };

  // every step, each wave waits for its own loads of that step (those of the
  // NS - 2 later steps may stay in flight), then meets the others: the step's
  // stage is complete and the stage read one step earlier is free again
  constexpr int VM = (NS - 2) * Ring::LPS;
  static_assert(VM < 64, "vmcnt field");
  constexpr int VMCNT = (VM & 15) | (7 << 4) | (0 << 8) | ((VM >> 4) << 14);
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) issue(s);
  for (int s = 0; s < nsteps; ++s) {
    __builtin_amdgcn_s_waitcnt(VMCNT);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue(s + NS - 1);
    compute(s);
  }
  // the loads past the range still land (zeros): drain them before the
  // workgroup's LDS can be handed to another
  __builtin_amdgcn_s_waitcnt(0);

  // lane holds rows 4 lg + e of each 16-row block, column lr of each 16-column block
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t row = row0 + 16 * (TM * wave + i) + 4 * lg + e;
        const int col = j0 + 16 * j + lr;
        if (row >= row_end || col >= p.r) continue;
        const float v = acc[i][j][e];
        if (gridDim.z > 1) {
          p.part[((int64_t)blockIdx.z * p.M + row) * p.r + col] = v;
        } else {
          p.out1[row * p.r + col] = to_bf16(v * p.alpha1);
          if (p.out2) p.out2[row * p.r + col] = to_bf16(v * p.alpha2);
        }
      }
}

}  // namespace skinny
}  // namespace lora4
