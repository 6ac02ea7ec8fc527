// Tiled bf16 MFMA GEMMs for the LoRA linear, with in-register dequant of the
// 4-bit base. Three operand forms cover every product of the layer:
//
//  NT : C[M, Nc] = A[M, R] . B[Nc, R]^T  (both operands contiguous along R)
//       forward  Y = X deq(W)^T (+ s Z B^T as a tail) ; Z = X A^T
//  NN : C[M, Nc] = A[M, R] . B[R, Nc]    (B contiguous along Nc)
//       dgrad    dX = dY deq(W) (+ dZ A as a tail)    ; dZ = dY B
//  TN : C[P, Q]  = U[Mr, P]^T . V[Mr, Q] (reduction over rows, split)
//       dA = dZ^T X ; dB^T = Z^T dY
//
// Every product accumulates in fp32 on v_mfma_f32_16x16x32_bf16. A workgroup
// is 256 threads (4 waves of 64) arranged WAVES_M x WAVES_N, each wave owning
// a (BM/WAVES_M) x (BN/WAVES_N) block of 16 x 16 MFMA tiles. The reduction
// advances 64 at a time: global loads for step s+1 are issued before the
// MFMAs of step s run, so memory latency overlaps compute.
//
// The 4-bit base is read as packed nibbles (16 bytes = 32 elements per
// thread and step), dequantized in registers to bf16 and written to LDS; the
// bf16 copy of W exists only there, one tile at a time. For NN the tile is
// stored as it lies in memory (rows = reduction index) and the MFMA operand
// is fetched with the transposing read ds_read_b64_tr_b16, so dgrad
// dequantizes along the same axis as its scale blocks.
#pragma once

#include "formats.hpp"

namespace lora4 {

constexpr int BK = 64;          // reduction step
constexpr int THREADS = 256;
constexpr int APAD = 8;         // bf16 padding per LDS row of K-contiguous tiles
constexpr int CPAD = 16;        // bf16 padding per LDS row of column-contiguous tiles

// --------------------------------------------------------------------------
// Operand descriptions
// --------------------------------------------------------------------------

// bf16 matrix, row-major with leading dimension ld (elements); per-group
// element offset gstride (0 when the operand is shared by all groups).
struct Mat {
  const uint16_t *p;
  int64_t ld;
  int64_t gstride;
};

struct GemmOut {
  uint16_t *C;        // bf16 output (or nullptr)
  int64_t ldc;
  float *part;        // fp32 split partials [split][rows][cols] (or nullptr)
  int64_t part_stride;// elements between splits
  float alpha;        // scale applied before rounding (bf16 output only)
};

struct NtParams {
  Mat A;              // [M, R] rows indexed absolutely (shared across groups)
  Mat B;              // FMT_BF16: [Nc, R] per group
  PackedW W;          // packed base (FMT != BF16)
  int64_t R;          // main reduction length
  Mat A2;             // tail A [M, r2] (absolute rows)
  Mat B2;             // tail B [Nc, r2] per group
  int r2;             // tail reduction length (0: no tail)
  int64_t M, Nc;
  const int64_t *offsets;
  int groups;
  int64_t Rsplit;     // reduction elements per split (multiple of 64); splits = gridDim.z
  GemmOut out;
  Nf4Table tab;
};

struct NnParams {
  Mat A;              // [M, R]
  Mat B;              // FMT_BF16: [R, Nc] per group
  PackedW W;          // packed base [R = N rows][Nc = K cols]
  int64_t R;
  Mat A2;             // tail A [M, r2]
  Mat B2;             // tail B [r2, Nc] per group
  int r2;
  int64_t M, Nc;
  const int64_t *offsets;
  int groups;
  int64_t Rsplit;
  GemmOut out;
  Nf4Table tab;
};

struct TnParams {
  Mat U;              // [Mrows, P] (absolute rows)
  Mat V;              // [Mrows, Q]
  int64_t P, Q, M;
  const int64_t *offsets;
  int groups;
  int splits;         // row splits per group (gridDim.z == splits)
  float *part;        // [splits][groups][P][Q]
  // In-launch reduction (cnt != nullptr): one arrival counter per output
  // tile, zero on entry and left zero. The block that arrives last at a tile
  // sums the tile's partials in split order and writes
  // out[g][p][q] = bf16(alpha sum) (transpose_out: out[g][q][p]).
  unsigned *cnt;
  uint16_t *out;
  float alpha;
  int transpose_out;
};

// --------------------------------------------------------------------------
// Tile loaders
// --------------------------------------------------------------------------

// Loads a rows x 64 bf16 slab (reduction contiguous) into registers:
// each thread holds NCH 16-byte chunks. Chunk c of thread t is
// idx = t + 256 c: row idx / 8, columns 8 (idx % 8) .. +7.
template <int ROWS>
struct SlabRegs {
  static constexpr int NCH = ROWS * 8 / THREADS > 0 ? ROWS * 8 / THREADS : 1;
  u32x4_t v[NCH];
};

template <int ROWS>
__device__ __forceinline__ void load_slab(SlabRegs<ROWS> &r, const uint16_t *base, int64_t ld,
                                          int64_t row0, int64_t row_end, int64_t k0, int64_t kend,
                                          bool vec_ok) {
  const int t = threadIdx.x;
#pragma unroll
  for (int c = 0; c < SlabRegs<ROWS>::NCH; ++c) {
    int idx = t + THREADS * c;
    int row = idx >> 3;
    int col = (idx & 7) * 8;
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (idx < ROWS * 8) {
      int64_t gr = row0 + row;
      int64_t gk = k0 + col;
      if (gr < row_end && gk < kend) {
        const uint16_t *src = base + gr * ld + gk;
        if (vec_ok && gk + 8 <= kend) {
          v = ldg_b128_cached(src);
        } else {
          uint32_t w[4] = {0u, 0u, 0u, 0u};
          for (int j = 0; j < 8; ++j) {
            if (gk + j < kend) w[j >> 1] |= (uint32_t)src[j] << (16 * (j & 1));
          }
          v = u32x4_t{w[0], w[1], w[2], w[3]};
        }
      }
    }
    r.v[c] = v;
  }
}

template <int ROWS>
__device__ __forceinline__ void store_slab(const SlabRegs<ROWS> &r, uint16_t *lds) {
  const int t = threadIdx.x;
#pragma unroll
  for (int c = 0; c < SlabRegs<ROWS>::NCH; ++c) {
    int idx = t + THREADS * c;
    if (idx < ROWS * 8) {
      int row = idx >> 3;
      int col = (idx & 7) * 8;
      lds_write_b128(lds + row * (BK + APAD) + col, r.v[c]);
    }
  }
}

// Packed slab: ROWS x 64 elements of W (NT: rows = output n, 64 along K).
// Task c of thread t: idx = t + 256 c covers row idx / 2, half idx % 2
// (32 elements). Holds the raw codes and the scale until the LDS store.
template <int ROWS>
struct PackedSlabRegs {
  static constexpr int NT = ROWS * 2 / THREADS > 0 ? ROWS * 2 / THREADS : 1;
  u32x4_t codes[NT];
  float scale[NT];
  float scale2[NT];   // NVFP4: elements 16..31 of the piece
};

// --------------------------------------------------------------------------
// NT kernel
// --------------------------------------------------------------------------

template <int FMT, int BM, int BN, int WAVES_M>
__global__ __launch_bounds__(THREADS) void k_gemm_nt(NtParams p) {
  constexpr int WAVES_N = 4 / WAVES_M;
  constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  static_assert(FM >= 1 && FN >= 1, "wave tile too small");

  __shared__ __attribute__((aligned(16))) uint16_t As[BM * (BK + APAD)];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * (BK + APAD)];
  __shared__ float qlds[16];

  const RowTile rt = map_row_tile(blockIdx.y, BM, p.offsets, p.groups, p.M);
  if (rt.group < 0) return;
  const int g = rt.group;
  const int64_t row0 = rt.row0, row_end = rt.row_end;
  const int64_t col0 = (int64_t)blockIdx.x * BN;
  const int split = blockIdx.z;

  if (threadIdx.x < 16) qlds[threadIdx.x] = p.tab.q[threadIdx.x];

  // reduction ranges: main [rb, re) of R, then the tail [0, r2) (last split only)
  const int64_t rb = (int64_t)split * p.Rsplit;
  const int64_t re = rb + p.Rsplit < p.R ? rb + p.Rsplit : p.R;
  const int main_steps = re > rb ? (int)((re - rb + BK - 1) / BK) : 0;
  const bool has_tail = p.r2 > 0 && split == (int)gridDim.z - 1;
  const int tail_steps = has_tail ? (p.r2 + BK - 1) / BK : 0;
  const int steps = main_steps + tail_steps;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm0 = (wave % WAVES_M) * WTM, wn0 = (wave / WAVES_M) * WTN;

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const bool a_vec = (p.A.ld % 8) == 0;
  const bool a2_vec = (p.A2.ld % 8) == 0;
  const bool b_vec = (p.B.ld % 8) == 0;
  const bool b2_vec = (p.B2.ld % 8) == 0;
  const uint16_t *Bg = p.B.p ? p.B.p + g * p.B.gstride : nullptr;
  const uint16_t *B2g = p.B2.p ? p.B2.p + g * p.B2.gstride : nullptr;

  SlabRegs<BM> ra;
  SlabRegs<BN> rb_bf;
  PackedSlabRegs<BN> rb_pk;

  auto issue = [&](int s) {
    if (s < main_steps) {
      const int64_t k0 = rb + (int64_t)s * BK;
      load_slab<BM>(ra, p.A.p, p.A.ld, row0, row_end, k0, re, a_vec);
      if constexpr (FMT == FMT_BF16) {
        load_slab<BN>(rb_bf, Bg, p.B.ld, col0, p.Nc, k0, re, b_vec);
      } else {
#pragma unroll
        for (int c = 0; c < PackedSlabRegs<BN>::NT; ++c) {
          int idx = threadIdx.x + THREADS * c;
          int row = idx >> 1, half = idx & 1;
          int64_t n = col0 + row, k = k0 + half * 32;
          u32x4_t cz = {0u, 0u, 0u, 0u};
          float sc = 0.f, sc2 = 0.f;
          if (idx < BN * 2 && n < p.Nc && k < re) {
            const uint8_t *src = p.W.codes + w_group(p.W, g) * p.W.g_codes + w_code_off(p.W.KB, n, k);
            cz = ldg_b128_cached(src);
            sc = block_scale<FMT>(p.W, g, n, k);
            if constexpr (FMT == FMT_NVFP4) sc2 = block_scale<FMT>(p.W, g, n, k + 16);
          }
          rb_pk.codes[c] = cz;
          rb_pk.scale[c] = sc;
          rb_pk.scale2[c] = sc2;
        }
      }
    } else {
      const int64_t k0 = (int64_t)(s - main_steps) * BK;
      load_slab<BM>(ra, p.A2.p, p.A2.ld, row0, row_end, k0, p.r2, a2_vec);
      load_slab<BN>(rb_bf, B2g, p.B2.ld, col0, p.Nc, k0, p.r2, b2_vec);
    }
  };

  auto commit = [&](int s) {
    store_slab<BM>(ra, As);
    if (FMT == FMT_BF16 || s >= main_steps) {
      store_slab<BN>(rb_bf, Bs);
    } else {
#pragma unroll
      for (int c = 0; c < PackedSlabRegs<BN>::NT; ++c) {
        int idx = threadIdx.x + THREADS * c;
        if (idx < BN * 2) {
          int row = idx >> 1, half = idx & 1;
          uint32_t w[16];
          if constexpr (FMT == FMT_NVFP4) {
            dequant32_nvfp4(rb_pk.codes[c], rb_pk.scale[c], rb_pk.scale2[c], w);
          } else if constexpr (FMT == FMT_MXFP4) {
            dequant32_mxfp4(rb_pk.codes[c], rb_pk.scale[c], w);
          } else if constexpr (FMT != FMT_BF16) {
            dequant32_nf4(rb_pk.codes[c], rb_pk.scale[c], qlds, w);
          }
          uint16_t *dst = Bs + row * (BK + APAD) + half * 32;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            lds_write_b128(dst + 8 * q, u32x4_t{w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]});
        }
      }
    }
  };

  __syncthreads();  // qlds visible
  if (steps > 0) issue(0);
  for (int s = 0; s < steps; ++s) {
    commit(s);
    __syncthreads();
    if (s + 1 < steps) issue(s + 1);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      u32x4_t af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = lds_read_b128(As + (wm0 + i * 16 + (lane & 15)) * (BK + APAD) + kk + (lane >> 4) * 8);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = lds_read_b128(Bs + (wn0 + j * 16 + (lane & 15)) * (BK + APAD) + kk + (lane >> 4) * 8);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma_16x16x32(af[i], bfr[j], acc[i][j]);
    }
    __syncthreads();
  }

  // epilogue: lane holds C[4*(lane/16) + e][lane % 16] of each 16x16 tile
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t col = col0 + wn0 + j * 16 + (lane & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t row = row0 + wm0 + i * 16 + (lane >> 4) * 4 + e;
        if (row < row_end && col < p.Nc) {
          if (p.out.part) {
            p.out.part[split * p.out.part_stride + row * p.Nc + col] = acc[i][j][e];
          } else {
            p.out.C[row * p.out.ldc + col] = to_bf16(acc[i][j][e] * p.out.alpha);
          }
        }
      }
    }
  }
}

// --------------------------------------------------------------------------
// NN kernel
// --------------------------------------------------------------------------

// Column slab: 64 rows (reduction) x COLS bf16, columns contiguous. Chunk c
// of thread t: idx = t + 256 c, row idx / (COLS/8), columns 8 (idx % (COLS/8)).
template <int COLS>
struct ColSlabRegs {
  static constexpr int CPR = COLS / 8;                       // chunks per row
  static constexpr int NCH = (BK * CPR + THREADS - 1) / THREADS;
  u32x4_t v[NCH];
};

template <int COLS>
__device__ __forceinline__ void load_colslab(ColSlabRegs<COLS> &r, const uint16_t *base, int64_t ld,
                                             int64_t r0, int64_t rend, int64_t c0, int64_t cend,
                                             bool vec_ok) {
  constexpr int CPR = ColSlabRegs<COLS>::CPR;
#pragma unroll
  for (int c = 0; c < ColSlabRegs<COLS>::NCH; ++c) {
    int idx = threadIdx.x + THREADS * c;
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (idx < BK * CPR) {
      int row = idx / CPR;
      int col = (idx % CPR) * 8;
      int64_t gr = r0 + row, gc = c0 + col;
      if (gr < rend && gc < cend) {
        const uint16_t *src = base + gr * ld + gc;
        if (vec_ok && gc + 8 <= cend) {
          v = ldg_b128_cached(src);
        } else {
          uint32_t w[4] = {0u, 0u, 0u, 0u};
          for (int j = 0; j < 8; ++j) {
            if (gc + j < cend) w[j >> 1] |= (uint32_t)src[j] << (16 * (j & 1));
          }
          v = u32x4_t{w[0], w[1], w[2], w[3]};
        }
      }
    }
    r.v[c] = v;
  }
}

template <int COLS>
__device__ __forceinline__ void store_colslab(const ColSlabRegs<COLS> &r, uint16_t *lds) {
  constexpr int CPR = ColSlabRegs<COLS>::CPR;
#pragma unroll
  for (int c = 0; c < ColSlabRegs<COLS>::NCH; ++c) {
    int idx = threadIdx.x + THREADS * c;
    if (idx < BK * CPR) {
      int row = idx / CPR;
      int col = (idx % CPR) * 8;
      lds_write_b128(lds + row * (COLS + CPAD) + col, r.v[c]);
    }
  }
}

// Packed column slab: 64 rows x COLS elements of W, 32-element tasks.
template <int COLS>
struct PackedColSlabRegs {
  static constexpr int TPR = COLS / 32;                       // tasks per row
  static constexpr int NT = (BK * TPR + THREADS - 1) / THREADS;
  u32x4_t codes[NT];
  float scale[NT];
  float scale2[NT];   // NVFP4: elements 16..31 of the piece
};

// Operand fetch for a column-contiguous LDS tile (rows = reduction): the
// 16 x 32 block (columns c0..c0+15, reduction rows k0..k0+31 of the tile)
// as the MFMA B operand (or the A operand of a transposed product).
__device__ __forceinline__ u32x4_t frag_tr(const uint16_t *lds, int ldr, int k0, int c0, int lane) {
  const int grp = lane >> 4, j = lane & 15;
  const uint16_t *p = lds + (k0 + grp * 8 + (j >> 2)) * ldr + c0 + (j & 3) * 4;
  u32x2_t lo = lds_read_tr16(p);
  u32x2_t hi = lds_read_tr16(p + 4 * ldr);
  return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
}

template <int FMT, int BM, int BN, int WAVES_M>
__global__ __launch_bounds__(THREADS) void k_gemm_nn(NnParams p) {
  constexpr int WAVES_N = 4 / WAVES_M;
  constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  static_assert(FM >= 1 && FN >= 1, "wave tile too small");
  static_assert(BN % 32 == 0 || FMT == FMT_BF16, "packed tiles need BN % 32 == 0");

  __shared__ __attribute__((aligned(16))) uint16_t As[BM * (BK + APAD)];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BK * (BN + CPAD)];
  __shared__ float qlds[16];

  const RowTile rt = map_row_tile(blockIdx.y, BM, p.offsets, p.groups, p.M);
  if (rt.group < 0) return;
  const int g = rt.group;
  const int64_t row0 = rt.row0, row_end = rt.row_end;
  const int64_t col0 = (int64_t)blockIdx.x * BN;
  const int split = blockIdx.z;

  if (threadIdx.x < 16) qlds[threadIdx.x] = p.tab.q[threadIdx.x];

  const int64_t rb = (int64_t)split * p.Rsplit;
  const int64_t re = rb + p.Rsplit < p.R ? rb + p.Rsplit : p.R;
  const int main_steps = re > rb ? (int)((re - rb + BK - 1) / BK) : 0;
  const bool has_tail = p.r2 > 0 && split == (int)gridDim.z - 1;
  const int tail_steps = has_tail ? (p.r2 + BK - 1) / BK : 0;
  const int steps = main_steps + tail_steps;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm0 = (wave % WAVES_M) * WTM, wn0 = (wave / WAVES_M) * WTN;

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const bool a_vec = (p.A.ld % 8) == 0;
  const bool a2_vec = (p.A2.ld % 8) == 0;
  const bool b_vec = (p.B.ld % 8) == 0;
  const bool b2_vec = (p.B2.ld % 8) == 0;
  const uint16_t *Bg = p.B.p ? p.B.p + g * p.B.gstride : nullptr;
  const uint16_t *B2g = p.B2.p ? p.B2.p + g * p.B2.gstride : nullptr;

  SlabRegs<BM> ra;
  ColSlabRegs<BN> rb_bf;
  PackedColSlabRegs<BN> rb_pk;

  auto issue = [&](int s) {
    if (s < main_steps) {
      const int64_t k0 = rb + (int64_t)s * BK;
      load_slab<BM>(ra, p.A.p, p.A.ld, row0, row_end, k0, re, a_vec);
      if constexpr (FMT == FMT_BF16) {
        load_colslab<BN>(rb_bf, Bg, p.B.ld, k0, re, col0, p.Nc, b_vec);
      } else {
        constexpr int TPR = PackedColSlabRegs<BN>::TPR;
#pragma unroll
        for (int c = 0; c < PackedColSlabRegs<BN>::NT; ++c) {
          int idx = threadIdx.x + THREADS * c;
          int row = idx / TPR, part = idx % TPR;
          int64_t n = k0 + row, k = col0 + part * 32;
          u32x4_t cz = {0u, 0u, 0u, 0u};
          float sc = 0.f, sc2 = 0.f;
          if (idx < BK * TPR && n < re && k < p.Nc) {
            const uint8_t *src = p.W.codes + w_group(p.W, g) * p.W.g_codes + w_code_off(p.W.KB, n, k);
            cz = ldg_b128_cached(src);
            sc = block_scale<FMT>(p.W, g, n, k);
            if constexpr (FMT == FMT_NVFP4) sc2 = block_scale<FMT>(p.W, g, n, k + 16);
          }
          rb_pk.codes[c] = cz;
          rb_pk.scale[c] = sc;
          rb_pk.scale2[c] = sc2;
        }
      }
    } else {
      const int64_t k0 = (int64_t)(s - main_steps) * BK;
      load_slab<BM>(ra, p.A2.p, p.A2.ld, row0, row_end, k0, p.r2, a2_vec);
      load_colslab<BN>(rb_bf, B2g, p.B2.ld, k0, p.r2, col0, p.Nc, b2_vec);
    }
  };

  auto commit = [&](int s) {
    store_slab<BM>(ra, As);
    if (FMT == FMT_BF16 || s >= main_steps) {
      store_colslab<BN>(rb_bf, Bs);
    } else {
      constexpr int TPR = PackedColSlabRegs<BN>::TPR;
#pragma unroll
      for (int c = 0; c < PackedColSlabRegs<BN>::NT; ++c) {
        int idx = threadIdx.x + THREADS * c;
        if (idx < BK * TPR) {
          int row = idx / TPR, part = idx % TPR;
          uint32_t w[16];
          if constexpr (FMT == FMT_NVFP4) {
            dequant32_nvfp4(rb_pk.codes[c], rb_pk.scale[c], rb_pk.scale2[c], w);
          } else if constexpr (FMT == FMT_MXFP4) {
            dequant32_mxfp4(rb_pk.codes[c], rb_pk.scale[c], w);
          } else if constexpr (FMT != FMT_BF16) {
            dequant32_nf4(rb_pk.codes[c], rb_pk.scale[c], qlds, w);
          }
          uint16_t *dst = Bs + row * (BN + CPAD) + part * 32;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            lds_write_b128(dst + 8 * q, u32x4_t{w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]});
        }
      }
    }
  };

  __syncthreads();
  if (steps > 0) issue(0);
  for (int s = 0; s < steps; ++s) {
    commit(s);
    __syncthreads();
    if (s + 1 < steps) issue(s + 1);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      u32x4_t af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = lds_read_b128(As + (wm0 + i * 16 + (lane & 15)) * (BK + APAD) + kk + (lane >> 4) * 8);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = frag_tr(Bs, BN + CPAD, kk, wn0 + j * 16, lane);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma_16x16x32(af[i], bfr[j], acc[i][j]);
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t col = col0 + wn0 + j * 16 + (lane & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t row = row0 + wm0 + i * 16 + (lane >> 4) * 4 + e;
        if (row < row_end && col < p.Nc) {
          if (p.out.part) {
            p.out.part[split * p.out.part_stride + row * p.Nc + col] = acc[i][j][e];
          } else {
            p.out.C[row * p.out.ldc + col] = to_bf16(acc[i][j][e] * p.out.alpha);
          }
        }
      }
    }
  }
}

// --------------------------------------------------------------------------
// TN kernel: partial[split][g][P][Q] = sum over the split's rows of U^T V
// --------------------------------------------------------------------------

// In-launch reduction of a TN tile's split partials (TnParams::cnt): every
// block's partials are written through to memory (system-scope stores, so no
// cache of any XCD holds them dirty) and acknowledged before the block
// counts itself in; the block that arrives last reads them back past the
// caches, sums them in split order from +0 (so the result does not depend on
// which block is last) and writes the bf16 tile, then resets the counter for
// the next launch. No block waits for another.
template <int BP, int BQ>
__device__ __forceinline__ void tn_reduce_last(const TnParams &p, int64_t p0, int64_t q0, int g, int64_t cnt_idx) {
  __shared__ int last;
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this thread's partial stores are acknowledged
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned arrived =
        __hip_atomic_fetch_add(&p.cnt[cnt_idx], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    last = arrived + 1 == (unsigned)p.splits;
    if (last) __hip_atomic_store(&p.cnt[cnt_idx], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
  __syncthreads();
  if (!last) return;
  const int64_t PQ = p.P * p.Q;
  const int64_t gstride = (int64_t)p.groups * PQ;   // one split's partials
  // the job's partials through a buffer descriptor, read with sc0 sc1 (past
  // every cache) 16 bytes per lane, the loads of up to 16 splits in flight
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      p.part, (short)0, (int)std::min<int64_t>((int64_t)p.splits * gstride * 4, 0x7FFFFFFF), 0x00020000);
  constexpr int SYS = 17;   // cache policy: sc0 | sc1
  const bool vec = (p.Q % 4) == 0 && (int64_t)p.splits * gstride * 4 <= 0x7FFFFFFF;
  // 4 consecutive q per thread and pass
  for (int idx = threadIdx.x * 4; idx < BP * BQ; idx += THREADS * 4) {
    const int64_t pp = p0 + idx / BQ, q = q0 + idx % BQ;
    if (pp >= p.P || q >= p.Q) continue;
    float sum[4] = {0.f, 0.f, 0.f, 0.f};
    const int64_t e0 = (int64_t)g * PQ + pp * p.Q + q;   // element offset in split 0
    if (vec) {
      for (int k0 = 0; k0 < p.splits; k0 += 16) {
        f32x4_t v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u)
          if (k0 + u < p.splits)
            v[u] = __builtin_bit_cast(
                f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)((e0 + (k0 + u) * gstride) * 4), 0, SYS));
#pragma unroll
        for (int u = 0; u < 16; ++u)
          if (k0 + u < p.splits)
#pragma unroll
            for (int e = 0; e < 4; ++e) sum[e] += v[u][e];
      }
    } else {
      for (int k = 0; k < p.splits; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (q + e < p.Q)
            sum[e] += __hip_atomic_load(p.part + e0 + k * gstride + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (q + e >= p.Q) break;
      const int64_t o = p.transpose_out ? (q + e) * p.P + pp : pp * p.Q + q + e;
      p.out[(int64_t)g * PQ + o] = to_bf16(sum[e] * p.alpha);
    }
  }
}

template <int BP, int BQ, int WAVES_P>
__device__ __forceinline__ void tn_tile(const TnParams &p, int bx, int by, int bz, int64_t cnt_idx) {
  constexpr int WAVES_Q = 4 / WAVES_P;
  constexpr int WTP = BP / WAVES_P, WTQ = BQ / WAVES_Q;
  constexpr int FM = WTP / 16, FN = WTQ / 16;
  static_assert(FM >= 1 && FN >= 1, "wave tile too small");

  __shared__ __attribute__((aligned(16))) uint16_t Us[BK * (BP + CPAD)];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[BK * (BQ + CPAD)];

  const int64_t p0 = (int64_t)bx * BP;
  const int64_t q0 = (int64_t)by * BQ;
  const int split = bz % p.splits;
  const int g = bz / p.splits;

  int64_t ga = 0, gb = p.M;
  if (p.offsets) {
    ga = p.offsets[g];
    gb = p.offsets[g + 1];
  }
  const int64_t rows = gb - ga;
  const int64_t per = ((rows + p.splits - 1) / p.splits + BK - 1) / BK * BK;
  const int64_t m0 = ga + (int64_t)split * per;
  const int64_t m1 = m0 + per < gb ? m0 + per : gb;
  const int steps = m1 > m0 ? (int)((m1 - m0 + BK - 1) / BK) : 0;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wp0 = (wave % WAVES_P) * WTP, wq0 = (wave / WAVES_P) * WTQ;

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const bool u_vec = (p.U.ld % 8) == 0;
  const bool v_vec = (p.V.ld % 8) == 0;
  ColSlabRegs<BP> ru;
  ColSlabRegs<BQ> rv;

  auto issue = [&](int s) {
    const int64_t r0 = m0 + (int64_t)s * BK;
    load_colslab<BP>(ru, p.U.p, p.U.ld, r0, m1, p0, p.P, u_vec);
    load_colslab<BQ>(rv, p.V.p, p.V.ld, r0, m1, q0, p.Q, v_vec);
  };

  if (steps > 0) issue(0);
  for (int s = 0; s < steps; ++s) {
    store_colslab<BP>(ru, Us);
    store_colslab<BQ>(rv, Vs);
    __syncthreads();
    if (s + 1 < steps) issue(s + 1);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      u32x4_t af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = frag_tr(Us, BP + CPAD, kk, wp0 + i * 16, lane);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = frag_tr(Vs, BQ + CPAD, kk, wq0 + j * 16, lane);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma_16x16x32(af[i], bfr[j], acc[i][j]);
    }
    __syncthreads();
  }

  float *out = p.part + ((int64_t)split * p.groups + g) * p.P * p.Q;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t q = q0 + wq0 + j * 16 + (lane & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t pp = p0 + wp0 + i * 16 + (lane >> 4) * 4 + e;
        if (pp < p.P && q < p.Q) {
          if (p.cnt)   // written through to memory: read by another block below
            __hip_atomic_store(&out[pp * p.Q + q], acc[i][j][e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
          else
            out[pp * p.Q + q] = acc[i][j][e];
        }
      }
    }
  }
  if (p.cnt) tn_reduce_last<BP, BQ>(p, p0, q0, g, cnt_idx);
}

// Two independent TN products with the same P tiling in one launch (the
// weight gradients dA and dB of one backward). Blocks [0, na) take job a and
// the rest job b; within a job the block index runs over P tiles fastest,
// then Q tiles, then split + group.
template <int BP, int BQ, int WAVES_P>
__global__ __launch_bounds__(THREADS) void k_gemm_tn2(TnParams a, TnParams b, int ptiles, int qa, int qb,
                                                       int64_t na) {
  int64_t id = blockIdx.x;
  const bool second = id >= na;
  if (second) id -= na;
  const TnParams p = second ? b : a;
  const int64_t qt = second ? qb : qa;
  const int bx = (int)(id % ptiles), by = (int)((id / ptiles) % qt), bz = (int)(id / (ptiles * qt));
  // arrival counter of the output tile (group bz / splits, Q tile by, P tile bx)
  const int64_t cnt_idx = ((int64_t)(bz / p.splits) * qt + by) * ptiles + bx;
  tn_tile<BP, BQ, WAVES_P>(p, bx, by, bz, cnt_idx);
}

// --------------------------------------------------------------------------
// Deterministic reductions of split partials
// --------------------------------------------------------------------------

// out1[i] = bf16(alpha1 * sum_s part[s][i]); out2 (optional) with alpha2.
// out = bf16(alpha * sum_k part[k][i]), summed in split order. Four elements
// per thread, and the loads of up to 16 splits issued before the adds.
__global__ void k_reduce_bf16(const float *part, int splits, int64_t stride, int64_t n,
                              uint16_t *out1, float alpha1, uint16_t *out2, float alpha2) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= n) return;
  const bool vec = (n % 4) == 0 && (stride % 4) == 0;
  if (!vec || i + 4 > n) {
    for (int64_t e = i; e < n && e < i + 4; ++e) {
      float s = 0.f;
      for (int k = 0; k < splits; ++k) s += part[k * stride + e];
      if (out1) out1[e] = to_bf16(s * alpha1);
      if (out2) out2[e] = to_bf16(s * alpha2);
    }
    return;
  }
  f32x4_t s = {0.f, 0.f, 0.f, 0.f};
  int k = 0;
  for (; k + 16 <= splits; k += 16) {
    f32x4_t v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = *reinterpret_cast<const f32x4_t *>(part + (k + u) * stride + i);
#pragma unroll
    for (int u = 0; u < 16; ++u) s += v[u];
  }
  if (k < splits) {
    f32x4_t v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (k + u < splits) v[u] = *reinterpret_cast<const f32x4_t *>(part + (k + u) * stride + i);
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (k + u < splits) s += v[u];
  }
  if (out1) {
    const u32x2_t w = {pack_bf16x2(s[0] * alpha1, s[1] * alpha1), pack_bf16x2(s[2] * alpha1, s[3] * alpha1)};
    *reinterpret_cast<u32x2_t *>(out1 + i) = w;
  }
  if (out2) {
    const u32x2_t w = {pack_bf16x2(s[0] * alpha2, s[1] * alpha2), pack_bf16x2(s[2] * alpha2, s[3] * alpha2)};
    *reinterpret_cast<u32x2_t *>(out2 + i) = w;
  }
}

__global__ void k_fill_u16(uint16_t *p, int64_t n, uint16_t v) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace lora4
