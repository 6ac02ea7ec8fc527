// MX-native forward of an MXFP4 base ("Quantized weights, full precision",
// section "Forward pass in inference": where the hardware has MXFP4-native
// operations, the base product of an MXFP4 base runs natively while the
// adapters stay in bf16; "Forward pass in training": the same in the training
// forward).
//
// The activations are quantized to MXFP8 (E4M3 elements, one E8M0 scale per
// 32 elements along K; the OCP MX v1.0 conversion) by k_quant_mxfp8, and
// Y = X8 W4^T + (s Z) B^T runs on v_mfma_scale_f32_32x32x64_f8f6f4, which
// applies both block scales itself: the MXFP4 codes and E8M0 scales go from
// memory straight into the MFMA operands, with no decode. Operand layout of
// one 64-deep step (measured on the device with one-hot operands): in the E2M1
// operand lane half h holds k = 32 h .. 32 h + 31 (16 bytes); in the E4M3
// operand it holds k = 16 h .. 16 h + 15 in its first four registers and
// k = 32 + 16 h .. 47 + 16 h in its last four; block b (k = 32 b .. 32 b + 31)
// of either operand is scaled by the E8M0 byte of lane half b.
#pragma once

#include "gemm_big.hpp"

namespace lora4 {
namespace mx {

using big::OOB;
using big::Params;
using big::rsrc_t;

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2v_t __attribute__((ext_vector_type(2)));

// X stages in the LDS ring; steps ahead that W and the X scales are loaded
constexpr int BM = 256, BN = 256, BKS = 64, THREADS = 256, STAGES = 5, AHEAD = 4;
constexpr int TILE8 = BM * BKS;        // one MXFP8 X stage, bytes
constexpr int ZTILE = BM * BKS * 2;    // bf16 staging tile of the rank-r product, bytes
constexpr int EPI = 4 * BM * 64 * 2;   // epilogue: each wave's 256 x 64 bf16 block

__host__ __device__ constexpr int lds_bytes() {
  return STAGES * TILE8 + ZTILE > EPI ? STAGES * TILE8 + ZTILE : EPI;
}

// ---------------------------------------------------------------------------
// MXFP8 quantizer
// ---------------------------------------------------------------------------

// Shared exponent of a block from its largest magnitude given as bf16 bits
// (sign cleared): floor(log2 amax) - 8 (8 = largest E4M3 exponent), clamped to
// [-127, 127]; -127 for an all-zero block.
__device__ __forceinline__ int mx8_exponent(uint32_t a) {
  if (a == 0) return -127;
  const int e = (int)(a >> 7);
  const int fl = e ? e - 127 : (31 - __builtin_clz(a & 0x7Fu)) - 133;
  const int x = fl - 8;
  return x < -127 ? -127 : (x > 127 ? 127 : x);
}

// E4M3FN codes of two bf16 elements (the low and high halves of u) times
// 2^-Xe: |x| 2^-Xe is exact in fp32 (a power-of-two scaling; Xe >= -127, so
// 2^-Xe is a normal float), clamped to 448 and converted by v_cvt_pk_fp8_f32
// (nearest, ties to even; every clamped value is in range); the sign bits are
// copied from x afterwards, so -0 and negative values too small for E4M3 keep
// their sign. Returns the two codes in the low 16 bits.
__device__ __forceinline__ uint32_t mx8_code2(uint32_t u, float scale) {
  const float f0 = fminf(fabsf(__uint_as_float(u << 16)) * scale, 448.0f);
  const float f1 = fminf(fabsf(__uint_as_float(u & 0xFFFF0000u)) * scale, 448.0f);
  const uint32_t c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f0, f1, 0, false) & 0xFFFFu;
  return c | ((u >> 8) & 0x80u) | ((u >> 16) & 0x8000u);
}

// X bf16 [M][ldx] -> E4M3 codes [Mp][ldc] and E8M0 scales (K % 32 == 0).
// One workgroup per 256 rows x 256 columns; per pass the 256 threads cover
// 8 rows x 256 columns, one thread per 8 elements, so every load instruction
// reads whole 512-byte row segments; the 4 lanes of a quad hold one 32-element
// block. Rows [0, Mp) x columns [0, Kp) are written; outside [0, M) x [0, K)
// the codes are 0 (and the GEMM-order scales 0). GEMM: scales in the GEMM's
// order (step s = k / 64, row tile T = row / 256, half h = k / 32 % 2, then 32
// rows of 8 bytes: row % 32, block (row % 256) / 32), gathered in LDS and
// written as whole 512-byte runs (Mp % 256 == 0); else row-major [M][K / 32].
template <bool GEMM>
__global__ __launch_bounds__(256) void k_quant_mxfp8(const uint16_t *X, int64_t ldx, int64_t M, int64_t K,
                                                     uint8_t *codes, int64_t ldc, int64_t Mp, int64_t Kp,
                                                     uint8_t *scales) {
  __shared__ uint8_t sc_lds[GEMM ? 4 * 512 : 4];
  const int64_t CB = (Kp + 255) >> 8;   // 256-column chunks
  const int64_t cb = blockIdx.x % CB, T = blockIdx.x / CB;
  const int t = threadIdx.x;
  const int64_t k = cb * 256 + (t & 31) * 8;
  const int hh = (int)((k >> 5) & 1), sl = (t & 31) >> 3;   // block half, step within the chunk
  for (int pass = 0; pass < 32; ++pass) {
    const int rl = pass * 8 + (t >> 5);   // row within the tile
    const int64_t row = T * 256 + rl;
    const bool row_ok = row < Mp, col_ok = k < Kp;
    const bool in = row < M && k < K;
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (in) v = *reinterpret_cast<const u32x4_t *>(X + row * ldx + k);
    uint32_t a = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a = max(a, v[e] & 0x7FFFu);
      a = max(a, (v[e] >> 16) & 0x7FFFu);
    }
    a = max(a, (uint32_t)__shfl_xor((int)a, 1));
    a = max(a, (uint32_t)__shfl_xor((int)a, 2));
    const int Xe = mx8_exponent(a);
    const float scale = __uint_as_float((uint32_t)(127 - Xe) << 23);   // 2^-Xe
    const uint32_t w0 = mx8_code2(v[0], scale) | (mx8_code2(v[1], scale) << 16);
    const uint32_t w1 = mx8_code2(v[2], scale) | (mx8_code2(v[3], scale) << 16);
    if (row_ok && col_ok) *reinterpret_cast<u32x2v_t *>(codes + row * ldc + k) = u32x2v_t{w0, w1};
    if ((t & 3) == 0) {
      const uint8_t E = (uint8_t)(Xe + 127);
      if constexpr (GEMM) {
        sc_lds[(sl * 2 + hh) * 256 + (rl & 31) * 8 + (rl >> 5)] = in ? E : (uint8_t)0;
      } else if (in) {
        scales[row * (K >> 5) + (k >> 5)] = E;
      }
    }
  }
  if constexpr (GEMM) {
    __syncthreads();
    // run s (4 per chunk) of 512 bytes: (h, row % 32, block) for step cb * 4 + s
    const int run = t >> 6;
    const int64_t s = cb * 4 + run;
    if (s * 64 < Kp) {
      const u32x2v_t q = *reinterpret_cast<const u32x2v_t *>(sc_lds + run * 512 + (t & 63) * 8);
      *reinterpret_cast<u32x2v_t *>(scales + (s * (Mp >> 8) + T) * 512 + (t & 63) * 8) = q;
    }
  }
}

// ---------------------------------------------------------------------------
// The GEMM
// ---------------------------------------------------------------------------

// X stage layout: row r (0..255) of 64 bytes as four 16-byte chunks, chunk c
// at slot 4 r + (c ^ ((r >> 2) & 3)). A lane's fragment of a 32-row block is
// chunks h and 2 + h of one row (the E4M3 operand layout); the 16 lanes of a
// read phase (16 consecutive rows, one chunk) then hit 16 different 16-byte
// bank groups.
__device__ __forceinline__ int x8_slot(int r, int c) { return r * 4 + (c ^ ((r >> 2) & 3)); }

__device__ __forceinline__ f32x16_t mfma_scale_fp4_fp8(i32x8_t w4, i32x8_t x8, f32x16_t c, int sw, int sx) {
  // A = W (format 4: E2M1), B = X (format 0: E4M3); the scales are the E8M0
  // bytes of each lane's block
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w4, x8, c, 4, 0, 0, sw, 0, sx);
}

// Register set of one step: this lane's two W rows (16 bytes of codes and the
// E8M0 byte each) and the E8M0 bytes of its 8 X rows.
struct MxRegs {
  u32x4_t c[2];
  uint32_t sc[2];
  u32x2v_t xs;
};

// One block per output tile (SPLIT: per reduction range of a tile, fp32
// partials), 4 waves; wave w owns output columns 64 w .. 64 w + 63 of the
// tile for all 256 rows. Plain layers only (one group).
template <bool SPLIT>
__global__ __launch_bounds__(THREADS, 1) void k_gemm_fwd_mx(Params p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem8[];

  int b = blockIdx.x, tile, split = 0;
  if constexpr (!SPLIT) {
    const int per = p.nblocks >> 3;   // XCD-aware order, as the bf16 forward
    if (b < per * 8) b = (b & 7) * per + (b >> 3);
    tile = b;
  } else {
    tile = b / p.ksplit;
    split = b % p.ksplit;
  }
  int tn, slot;
  if constexpr (!SPLIT) {
    big::grouped_tile(tile, p.tiles_n, p.nblocks / p.tiles_n, slot, tn);
  } else {
    tn = tile % p.tiles_n;   // (k_reduce_tiles uses this order)
    slot = tile / p.tiles_n;
  }
  const int64_t row0 = (int64_t)slot * BM;
  if (row0 >= p.M) return;
  const int64_t col0 = (int64_t)tn * BN;

  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63;
  const int l32 = lane & 31, h = lane >> 5;

  const int sb = SPLIT ? split * p.split_steps : 0;
  const int all_steps = (int)((p.R + BKS - 1) / BKS);
  const int steps = SPLIT ? min(all_steps - sb, p.split_steps) : all_steps;
  const int64_t MT = (p.M + BM - 1) / BM;

  // ---- X: direct loads into the LDS ring. Load q (0..3) of wave w covers
  // tile rows 64 q + 16 w .. +15; lane l fills slot 4 (row) + l % 4, i.e.
  // row + l / 4, chunk (l % 4) ^ ((l / 16) % 4).
  const rsrc_t x_rsrc = big::make_rsrc(p.X8 + row0 * p.ld8, big::clamp_bytes((int64_t)BM * p.ld8));
  const uint32_t x_voff0 = (uint32_t)((16 * wave + (lane >> 2)) * p.ld8 + 16 * ((lane & 3) ^ ((lane >> 4) & 3)));
  const uint32_t x_qstep = (uint32_t)(64 * p.ld8);
  auto issue_x = [&](int s, int stage) {
    const bool past = s >= steps;   // look-ahead past the range: zeros, no memory traffic
    const int k0 = (s + sb) * BKS;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          x_rsrc, (__attribute__((address_space(3))) void *)(smem8 + stage * TILE8 + (64 * q + 16 * wave) * 64), 16,
          past ? OOB : x_voff0 + q * x_qstep, k0, 0, 0);
  };

  // ---- W rows col0 + 64 wave + 32 j + l32 (one row block of the tiled base;
  // per step the tile (rb, k0 / 64): row i's 32 code bytes at 32 i, its two
  // E8M0 bytes at 2 i) and the X scales of this lane's rows
  const int64_t KB = p.W.KB;
  const int64_t rb = (col0 >> 6) + wave;
  const bool rb_ok = rb < w_blocks(p.W.N);
  const rsrc_t w_rsrc = big::make_rsrc(rb_ok ? p.W.codes + rb * KB * 2048 : p.W.codes,
                                       rb_ok ? big::clamp_bytes(KB * 2048) : 0u);
  const uint8_t *sbase = reinterpret_cast<const uint8_t *>(p.W.scales);
  const rsrc_t s_rsrc = big::make_rsrc(rb_ok ? sbase + rb * KB * 128 : sbase, rb_ok ? big::clamp_bytes(KB * 128) : 0u);
  const rsrc_t xs_rsrc = big::make_rsrc(p.X8s, big::clamp_bytes((int64_t)all_steps * MT * 512));
  uint32_t w_voff[2], s_voff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    w_voff[j] = (uint32_t)((j * 32 + l32) * 32 + h * 16);
    s_voff[j] = (uint32_t)((j * 32 + l32) * 2 + h);
  }
  const uint32_t xs_voff = (uint32_t)((slot * 2 + h) * 256 + l32 * 8);
  // 5 loads per step, always issued (past the end they return zeros)
  auto load_regs = [&](int s, MxRegs &g) {
    const int gs = s + sb;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      g.c[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, w_voff[j], gs << 11, 0));
      g.sc[j] = __builtin_amdgcn_raw_buffer_load_b8(s_rsrc, s_voff[j], gs * 128, 0);
    }
    g.xs = __builtin_bit_cast(u32x2v_t, __builtin_amdgcn_raw_buffer_load_b64(xs_rsrc, xs_voff,
                                                                             (int)((int64_t)gs * MT * 512), 0));
  };

  f32x16_t acc[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    acc[i][0] = f32x16_t{};
    acc[i][1] = f32x16_t{};
  }

#pragma unroll
  for (int s = 0; s < STAGES; ++s) issue_x(s, s);
  MxRegs g[AHEAD];
#pragma unroll
  for (int u = 0; u < AHEAD; ++u) load_regs(u, g[u]);

  // ---- rank-r product (s Z) B^T into the zeroed accumulators (split 0),
  // bf16 MFMAs: Z rows through the staging tile, B rows to registers; lane
  // half h holds k0 + 32 h + 8 kk .. +7 in sub-step kk
  if (p.r2 > 0 && split == 0) {
    uint16_t *Zs = reinterpret_cast<uint16_t *>(smem8 + STAGES * TILE8);
    const bool a_vec = (p.A2.ld % 8) == 0;
    const bool b_vec = (p.B2.ld % 8) == 0;
    for (int k0 = 0; k0 < p.r2; k0 += BKS) {
      const int nkk = min(4, (p.r2 - k0 + 7) / 8);
      u32x4_t bt[2][4];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t n = col0 + wave * 64 + j * 32 + l32;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int64_t k = k0 + 32 * h + 8 * kk;
          uint32_t w4[4] = {0u, 0u, 0u, 0u};
          if (kk < nkk && n < p.Nc && k < p.r2) {
            const uint16_t *src = p.B2.p + n * p.B2.ld + k;
            if (b_vec && k + 8 <= p.r2) {
              const u32x4_t v = *reinterpret_cast<const u32x4_t *>(src);
              w4[0] = v[0];
              w4[1] = v[1];
              w4[2] = v[2];
              w4[3] = v[3];
            } else {
              for (int e = 0; e < 8; ++e)
                if (k + e < p.r2) w4[e >> 1] |= (uint32_t)src[e] << (16 * (e & 1));
            }
          }
          bt[j][kk] = u32x4_t{w4[0], w4[1], w4[2], w4[3]};
        }
      }
      if (p.A2part) {
        big::a2_parts_to_lds<false>(p, Zs, [](int i, int c) { return tile64_swz(i, c); }, row0, p.M, k0, t,
                                    col0 == 0);
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int idx = t + THREADS * c;
          const int row = idx >> 3, chunk = idx & 7;
          u32x4_t v = {0u, 0u, 0u, 0u};
          const int64_t gr = row0 + row;
          const int64_t gk = k0 + chunk * 8;
          if (gr < p.M && gk < p.r2) {
            const uint16_t *src = p.A2.p + gr * p.A2.ld + gk;
            if (a_vec && gk + 8 <= p.r2) {
              v = *reinterpret_cast<const u32x4_t *>(src);
            } else {
              uint32_t w4[4] = {0u, 0u, 0u, 0u};
              for (int e = 0; e < 8; ++e)
                if (gk + e < p.r2) w4[e >> 1] |= (uint32_t)src[e] << (16 * (e & 1));
              v = u32x4_t{w4[0], w4[1], w4[2], w4[3]};
            }
          }
          lds_write_b128(Zs + tile64_swz(row, chunk), v);
        }
      }
      __syncthreads();
      for (int kk = 0; kk < nkk; ++kk) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const u32x4_t x = lds_read_b128(Zs + tile64_swz(i * 32 + l32, h * 4 + kk));
          acc[i][0] = mfma_32x32x16(bt[0][kk], x, acc[i][0]);
          acc[i][1] = mfma_32x32x16(bt[1][kk], x, acc[i][1]);
        }
      }
      __syncthreads();   // before the next chunk restages
    }
  }

  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  i32x8_t xf[8];
  auto read_x = [&](int stage, int i) {
    const uint8_t *base = smem8 + stage * TILE8;
    const int r = i * 32 + l32;
    const u32x4_t lo = *reinterpret_cast<const u32x4_t *>(base + 16 * x8_slot(r, h));
    const u32x4_t hi = *reinterpret_cast<const u32x4_t *>(base + 16 * x8_slot(r, 2 + h));
    xf[i] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
#pragma unroll
  for (int i = 0; i < 8; ++i) read_x(0, i);

  // At the start of step s the X of step s + 1 (issued during step
  // s + 1 - STAGES) and the registers of step s (issued at the end of step
  // s - AHEAD) must have landed; still in flight may be what the AHEAD - 1
  // steps after that issued: 4 X loads and 5 register loads each
  // (STAGES - 1 >= AHEAD, so the X of step s + 1 is older than those).
  // lgkmcnt 0: this wave's reads of the stage refilled below have returned.
  static_assert(STAGES - 1 >= AHEAD && AHEAD >= 2, "load distances");
  constexpr int VM_OUT = (AHEAD - 1) * 9;
  constexpr int VMCNT = (VM_OUT & 15) | (7 << 4) | (0 << 8) | ((VM_OUT >> 4) << 14);
  auto step = [&](int s, MxRegs &g) {
    __builtin_amdgcn_s_waitcnt(VMCNT);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // every wave has read stage s % 4 (during step s - 1): refill it
    issue_x(s + STAGES, s % STAGES);
    const int nxt = (s + 1) % STAGES;
    i32x8_t w[2];
    int sw[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      w[j] = i32x8_t{(int)g.c[j][0], (int)g.c[j][1], (int)g.c[j][2], (int)g.c[j][3], 0, 0, 0, 0};
      sw[j] = (int)g.sc[j];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int sx = (int)((g.xs[i >> 2] >> (8 * (i & 3))) & 0xFFu);
      acc[i][0] = mfma_scale_fp4_fp8(w[0], xf[i], acc[i][0], sw[0], sx);
      acc[i][1] = mfma_scale_fp4_fp8(w[1], xf[i], acc[i][1], sw[1], sx);
      read_x(nxt, i);
    }
    load_regs(s + AHEAD, g);
  };
  // AHEAD register sets in rotation (the loop is unrolled AHEAD times)
  int s = 0;
  for (; s + AHEAD <= steps; s += AHEAD) {
#pragma unroll
    for (int u = 0; u < AHEAD; ++u) step(s + u, g[u]);
  }
#pragma unroll
  for (int u = 0; u < AHEAD - 1; ++u)
    if (s + u < steps) step(s + u, g[u]);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // ---- epilogue: register e of acc[i][j] holds
  // Y[32 i + lane % 32][64 wave + 32 j + 8 (e / 4) + 4 (lane / 32) + e % 4]
  if constexpr (SPLIT) {
    float *pt = p.Cpart + ((int64_t)tile * p.ksplit + split) * (BM * BN);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float *prow = pt + (i * 32 + l32) * BN;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int col = wave * 64 + j * 32 + r4 * 8 + h * 4;
          *reinterpret_cast<f32x4_t *>(prow + col) =
              f32x4_t{acc[i][j][4 * r4], acc[i][j][4 * r4 + 1], acc[i][j][4 * r4 + 2], acc[i][j][4 * r4 + 3]};
        }
    }
    return;
  }
  // each wave stages its 256 x 64 bf16 block (tile64 layout) and writes whole
  // 128-byte row segments
  {
    uint16_t *stg = reinterpret_cast<uint16_t *>(smem8) + wave * (BM * 64);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const u32x2_t pk = {pack_bf16x2(acc[i][j][4 * r4], acc[i][j][4 * r4 + 1]),
                              pack_bf16x2(acc[i][j][4 * r4 + 2], acc[i][j][4 * r4 + 3])};
          *reinterpret_cast<u32x2_t *>(stg + tile64_swz(i * 32 + l32, 4 * j + r4) + 4 * h) = pk;
        }
    const bool vec16 = (p.ldc % 8) == 0;
#pragma unroll 4
    for (int q = 0; q < 32; ++q) {
      const int row = q * 8 + (lane >> 3), chunk = lane & 7;
      const u32x4_t v = lds_read_b128(stg + tile64_swz(row, chunk));
      const int64_t grow = row0 + row;
      const int64_t gcol = col0 + wave * 64 + chunk * 8;
      if (grow < p.M && gcol < p.Nc) {
        uint16_t *dst = p.C + grow * p.ldc + gcol;
        if (vec16 && gcol + 8 <= p.Nc) {
          *reinterpret_cast<u32x4_t *>(dst) = v;
        } else {
          for (int e = 0; e < 8 && gcol + e < p.Nc; ++e) dst[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
        }
      }
    }
  }
}

}  // namespace mx
}  // namespace lora4
