// Large-tile dequant-GEMM for the two dense contractions of the layer:
//
//   NT (forward): Y[M, N]  = X[M, K]  . deq(W)[N, K]^T  (+ (s Z) B^T tail)
//   NN (dgrad):   dX[M, K] = dY[M, N] . deq(W)[N, K]    (+ dZ A tail)
//
// One workgroup = 256 threads = 4 waves (2 x 2) computing a 256 x 256 output
// tile; each wave owns 128 x 128 (4 x 4 MFMA 32x32x16 tiles, 256 fp32
// accumulators per lane, held in the accumulation registers). The reduction
// advances 64 per step through two LDS buffers, one barrier per step.
//
// Data movement per step:
//  * the activation slab (256 rows x 64) goes from HBM/L2 straight into LDS
//    with buffer_load_dwordx4 ... lds (no staging registers); the buffer
//    descriptor's range check zero-fills rows past the tile's group and
//    columns past the reduction length;
//  * each thread loads one 64-element run of packed W (32 bytes + its scale)
//    into registers two steps ahead and dequantizes it into the other LDS
//    buffer while the MFMAs of the current step run;
//  * NT keeps deq(W) K-contiguous; NN keeps it as it lies in memory (rows =
//    reduction index) and feeds the MFMA with ds_read_b64_tr_b16.
//
// LDS layout of K-contiguous 256 x 64 tiles: rows of 128 bytes, the eight
// 16-byte chunks of row r stored at chunk position (chunk ^ (r & 7)), so the
// MFMA operand reads of 8 consecutive rows hit 8 different bank groups.
//
// NF4 runs are decoded through a 16-entry bf16 table bf16(q[i] * c) selected
// with v_perm_b32 (bit-identical to bf16(fp32(q[code] * c)) per element);
// MXFP4 uses v_cvt_scalef32_pk_bf16_fp4. The MFMA operands are swapped
// (deq(W) first) so each lane holds four consecutive output columns of one
// row, stored as one 8-byte write.
#pragma once

#include "formats.hpp"

#ifndef LORA4_SCHED_INTERLEAVE
#define LORA4_SCHED_INTERLEAVE 1
#endif
#ifndef LORA4_SCHED_VALU
#define LORA4_SCHED_VALU 5
#endif

namespace lora4 {
namespace big {

constexpr int BM = 256, BN = 256, BKS = 64;
constexpr int THREADS = 256;
constexpr int TILE64 = BM * BKS;        // 256 x 64 bf16, unpadded (swizzled)
constexpr int LDB_NN = BN + 16;         // NN: W~ tile [64][272]
constexpr int B_ELEMS_NN = BKS * LDB_NN;
constexpr uint32_t RSRC_WORD3 = 0x00020000u;   // raw 32-bit buffer, gfx9 family
constexpr uint32_t OOB = 0x80000000u;           // an offset past any range

__host__ __device__ constexpr int lds_bytes(int mode) {
  return 2 * (TILE64 + (mode == 0 ? TILE64 : B_ELEMS_NN)) * 2;
}

struct Params {
  Mat A;              // [M, R] activations (absolute rows), ld % 8 == 0
  PackedW W;          // packed base
  int64_t R;          // main reduction length (NT: K, NN: N)
  Mat A2;             // tail A [M, r2]
  Mat B2;             // tail B: NT [Nc, r2] per group, NN [r2, Nc] per group
  int r2;
  int64_t M, Nc;      // output rows, output columns
  const int64_t *offsets;
  int groups;
  uint16_t *C;
  int64_t ldc;
  int tiles_n;        // ceil(Nc / 256)
  int nblocks;        // gridDim.x
  Nf4Table tab;
  // split reduction (forward kernel only): every tile runs in ksplit blocks
  // of split_steps 64-deep steps, which write fp32 partials
  // Cpart[tile][split][256][256] instead of C (the rank-r tail goes into
  // split 0)
  int ksplit;
  int split_steps;
  float *Cpart;
  // rank-r tail operand given as fp32 partial sums over reduction ranges
  // (A2part[range][M][r2], absolute rows; A2 is then unused): the tail adds
  // the A2parts ranges in order and uses bf16(A2scale * sum). Blocks of
  // column tile 0 also store bf16(A2alpha1 * sum) to A2out1 and
  // bf16(A2alpha2 * sum) to A2out2 ([M, r2] each, either may be null) for the
  // passes that follow.
  const float *A2part;
  int A2parts;        // 1 .. A2_MAX_PARTS
  float A2scale;
  uint16_t *A2out1;
  float A2alpha1;
  uint16_t *A2out2;
  float A2alpha2;
};

constexpr int A2_MAX_PARTS = 4;

// Sum over the partial ranges (in range order, from +0) of the 8 tail
// operand values of row gr, columns gk .. gk + 7 (zero past r2).
__device__ __forceinline__ void a2_part_sum(const Params &p, int64_t gr, int64_t gk, float (&v)[8]) {
  float q[A2_MAX_PARTS][8];
  const int64_t stride = p.M * p.r2;
  const float *src = p.A2part + gr * p.r2 + gk;
  const bool vec = (p.r2 % 4) == 0 && gk + 8 <= p.r2;
#pragma unroll
  for (int r = 0; r < A2_MAX_PARTS; ++r) {
#pragma unroll
    for (int e = 0; e < 8; ++e) q[r][e] = 0.0f;
    if (r < p.A2parts) {
      const float *sr = src + r * stride;
      if (vec) {
        const f32x4_t lo = *reinterpret_cast<const f32x4_t *>(sr);
        const f32x4_t hi = *reinterpret_cast<const f32x4_t *>(sr + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          q[r][e] = lo[e];
          q[r][e + 4] = hi[e];
        }
      } else {
        for (int e = 0; e < 8; ++e)
          if (gk + e < p.r2) q[r][e] = sr[e];
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float t = 0.0f;
#pragma unroll
    for (int r = 0; r < A2_MAX_PARTS; ++r)
      if (r < p.A2parts) t += q[r][e];
    v[e] = t;
  }
}

__device__ __forceinline__ u32x4_t pack_scaled8(const float (&v)[8], float a) {
  return u32x4_t{pack_bf16x2(a * v[0], a * v[1]), pack_bf16x2(a * v[2], a * v[3]), pack_bf16x2(a * v[4], a * v[5]),
                 pack_bf16x2(a * v[6], a * v[7])};
}

// bf16 row piece [gr][gk .. gk + 7] of an [M, r2] output (elements past r2
// dropped; one 16-byte store when the row piece is whole and aligned).
__device__ __forceinline__ void store_a2_piece(uint16_t *out, int r2, int64_t gr, int64_t gk, u32x4_t v) {
  uint16_t *dst = out + gr * r2 + gk;
  if ((r2 % 8) == 0) {
    *reinterpret_cast<u32x4_t *>(dst) = v;
  } else {
    for (int e = 0; e < 8; ++e)
      if (gk + e < r2) dst[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
  }
}

// One 64-column step (k0 ..) of the tail operand from the partials into the
// LDS tile `As` (256 rows, bf16, 8-column chunk c of row i at
// As + lds_off(i, c)): thread t owns row t; chunks past r2 are zero.
template <typename Off>
__device__ __forceinline__ void a2_parts_to_lds(const Params &p, uint16_t *As, Off lds_off, int64_t row0,
                                                int64_t row_end, int k0, int t, bool store_out) {
  const int64_t gr = row0 + t;
  const bool row_ok = gr < row_end;
#pragma unroll 1
  for (int c0 = 0; c0 < 8; c0 += 2) {
    float v[2][8];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t gk = k0 + 8 * (c0 + u);
      if (row_ok && gk < p.r2) {
        a2_part_sum(p, gr, gk, v[u]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[u][e] = 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t gk = k0 + 8 * (c0 + u);
      lds_write_b128(As + lds_off(t, c0 + u), pack_scaled8(v[u], p.A2scale));
      if (store_out && row_ok && gk < p.r2) {
        if (p.A2out1) store_a2_piece(p.A2out1, p.r2, gr, gk, pack_scaled8(v[u], p.A2alpha1));
        if (p.A2out2) store_a2_piece(p.A2out2, p.r2, gr, gk, pack_scaled8(v[u], p.A2alpha2));
      }
    }
  }
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, (int)RSRC_WORD3);
}

__device__ __forceinline__ uint32_t clamp_bytes(int64_t b) {
  return b <= 0 ? 0u : (b >= (int64_t)0x7FFFFFFF ? 0x7FFFFFFFu : (uint32_t)b);
}

__device__ __forceinline__ int swz(int row, int chunk) { return row * BKS + ((chunk ^ (row & 7)) << 3); }

// ---------------------------------------------------------------------------
// NF4 dequant through a per-run bf16 table and byte permutes
// ---------------------------------------------------------------------------

struct RunTable {
  uint32_t lo[4], hi[4];   // byte planes of T[0..15]
  uint32_t sel;            // 0x03020100 in a vector register (see sel_base)
};

// The byte-select base 0x03020100 as an opaque vector register. The bit-3
// selector of lookup4 is (idx >> 1) & 0x04040404 | base: with the base in a
// vector register (and the mask in a scalar one) that is one v_and_or_b32;
// with two literal constants it takes three instructions.
__device__ __forceinline__ uint32_t sel_base() {
  uint32_t v;
  asm volatile("v_mov_b32 %0, 0x03020100" : "=v"(v));
  return v;
}

__device__ __forceinline__ uint32_t perm(uint32_t hi_src, uint32_t lo_src, uint32_t sel) {
  return __builtin_amdgcn_perm(hi_src, lo_src, sel);
}

// Byte planes of the table from its bf16 pairs t[j] = (T[2 j], T[2 j + 1]).
__device__ __forceinline__ RunTable table_from(const uint32_t t[8], uint32_t sel) {
  RunTable r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r.lo[i] = perm(t[2 * i + 1], t[2 * i], 0x06040200u);
    r.hi[i] = perm(t[2 * i + 1], t[2 * i], 0x07050301u);
  }
  r.sel = sel;
  return r;
}

__device__ __forceinline__ RunTable make_table(float c, const Nf4Table &tab, uint32_t sel) {
  uint32_t t[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) t[j] = pack_bf16x2(tab.q[2 * j] * c, tab.q[2 * j + 1] * c);
  return table_from(t, sel);
}

// Second stage of make_table_pair (below), from this lane's four bf16 pairs
// t[k] = (q[8 h + 2 k] c, q[8 h + 2 k + 1] c).
__device__ __forceinline__ RunTable table_pair_from(const uint32_t t[4], uint32_t sel) {
  const uint32_t l0 = perm(t[1], t[0], 0x06040200u), l1 = perm(t[3], t[2], 0x06040200u);
  const uint32_t h0 = perm(t[1], t[0], 0x07050301u), h1 = perm(t[3], t[2], 0x07050301u);
  const auto sl0 = __builtin_amdgcn_permlane32_swap(l0, l0, false, false);
  const auto sl1 = __builtin_amdgcn_permlane32_swap(l1, l1, false, false);
  const auto sh0 = __builtin_amdgcn_permlane32_swap(h0, h0, false, false);
  const auto sh1 = __builtin_amdgcn_permlane32_swap(h1, h1, false, false);
  RunTable r;
  r.lo[0] = sl0[0];
  r.lo[1] = sl1[0];
  r.lo[2] = sl0[1];
  r.lo[3] = sl1[1];
  r.hi[0] = sh0[0];
  r.hi[1] = sh1[0];
  r.hi[2] = sh0[1];
  r.hi[3] = sh1[1];
  r.sel = sel;
  return r;
}

// The same table for a run shared by lanes l and l + 32 (same row, same
// scale): lane half h builds entries 8 h .. 8 h + 7 (qh[i] = q[8 h + i]), and
// one v_permlane32_swap per byte-plane register gives every lane both
// halves (element 0: the lower lane's value, element 1: the upper lane's).
// 20 instructions instead of 32. All 64 lanes must be active.
__device__ __forceinline__ RunTable make_table_pair(float c, const float qh[8], uint32_t sel) {
  uint32_t t[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) t[k] = pack_bf16x2(qh[2 * k] * c, qh[2 * k + 1] * c);
  return table_pair_from(t, sel);
}

// 4 indices (bytes 0..15) -> low and high bytes of T[idx].
__device__ __forceinline__ void lookup4(const RunTable &T, uint32_t idx, uint32_t &L, uint32_t &H) {
  const uint32_t i7 = idx & 0x07070707u;
  const uint32_t s3 = ((idx >> 1) & 0x04040404u) | T.sel;   // byte j: j + 4 * bit3
  const uint32_t la = perm(T.lo[1], T.lo[0], i7);
  const uint32_t lb = perm(T.lo[3], T.lo[2], i7);
  const uint32_t ha = perm(T.hi[1], T.hi[0], i7);
  const uint32_t hb = perm(T.hi[3], T.hi[2], i7);
  L = perm(lb, la, s3);
  H = perm(hb, ha, s3);
}

// 8 codes (element i in bits 4i..4i+3) -> 4 words of bf16 pairs.
__device__ __forceinline__ u32x4_t decode8_nf4(const RunTable &T, uint32_t c) {
  const uint32_t ev = c & 0x0F0F0F0Fu;            // n0 n2 n4 n6
  const uint32_t od = (c >> 4) & 0x0F0F0F0Fu;     // n1 n3 n5 n7
  const uint32_t i0 = perm(od, ev, 0x05010400u);  // n0 n1 n2 n3
  const uint32_t i1 = perm(od, ev, 0x07030602u);  // n4 n5 n6 n7
  uint32_t L0, H0, L1, H1;
  lookup4(T, i0, L0, H0);
  lookup4(T, i1, L1, H1);
  return u32x4_t{perm(H0, L0, 0x05010400u), perm(H0, L0, 0x07030602u), perm(H1, L1, 0x05010400u),
                 perm(H1, L1, 0x07030602u)};
}

__device__ __forceinline__ u32x4_t decode8_mxfp4(uint32_t c, float s) {
  return u32x4_t{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, s, 0)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, s, 1)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, s, 2)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, s, 3))};
}

// MFMA 32x32x16 operand from a column-contiguous LDS tile (rows = reduction):
// lane l gets column c0 + l % 32 of reduction rows k0 + 8 (l / 32) .. +7,
// built from two transposing reads per 16-lane group.
__device__ __forceinline__ u32x4_t frag_tr32(const uint16_t *lds, int ldr, int k0, int c0, int lane) {
  const int grp = lane >> 4, j = lane & 15;
  const uint16_t *p = lds + (k0 + (grp >> 1) * 8 + (j >> 2)) * ldr + c0 + (grp & 1) * 16 + (j & 3) * 4;
  u32x2_t lo = lds_read_tr16(p);
  u32x2_t hi = lds_read_tr16(p + 4 * ldr);
  return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
}

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------

template <int MODE, int FMT>
__global__ __launch_bounds__(THREADS, 1) void k_gemm_big(Params p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  const uint32_t sel = sel_base();
  constexpr int B_ELEMS = MODE == 0 ? TILE64 : B_ELEMS_NN;
  uint16_t *const As0 = smem, *const As1 = smem + TILE64;
  uint16_t *const Bs0 = smem + 2 * TILE64, *const Bs1 = smem + 2 * TILE64 + B_ELEMS;

  // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs; renumber
  // so that each XCD walks a contiguous range of tiles (shared operands in
  // its own L2).
  int b = blockIdx.x;
  {
    const int per = p.nblocks >> 3;
    if (b < per * 8) b = (b & 7) * per + (b >> 3);
  }
  const int tn = b % p.tiles_n;
  const int slot = b / p.tiles_n;
  const RowTile rt = map_row_tile(slot, BM, p.offsets, p.groups, p.M);
  if (rt.group < 0) return;
  const int g = rt.group;
  const int64_t row0 = rt.row0, row_end = rt.row_end;
  const int64_t col0 = (int64_t)tn * BN;

  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int wm0 = (wave & 1) * 128, wn0 = (wave >> 1) * 128;

  // ---- activation slab: direct HBM/L2 -> LDS --------------------------------
  // wave w, chunk c covers tile rows 8 (4 c + w) .. +7; lane l: row + l / 8,
  // stored chunk l % 8 which holds logical chunk (l % 8) ^ (row % 8).
  const rsrc_t a_rsrc = make_rsrc(p.A.p + row0 * p.A.ld, clamp_bytes((row_end - row0) * p.A.ld * 2));
  uint32_t a_voff[8];
  int a_kq = ((lane & 7) ^ ((lane >> 3) & 7)) * 8;   // logical column of this lane's chunk
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int row = (c * 4 + wave) * 8 + (lane >> 3);
    a_voff[c] = (uint32_t)((row * p.A.ld + a_kq) * 2);
  }
  auto issue_a = [&](int s, uint16_t *As) {
    const int64_t k0 = (int64_t)s * BKS;
    const bool edge = k0 + a_kq >= p.R;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (__attribute__((address_space(3))) void *)(As + (c * 4 + wave) * 512),
                                               16, edge ? OOB : a_voff[c], (int)(k0 * 2), 0, 0);
    }
  };

  // ---- packed W run of this thread ---------------------------------------------
  // NT: row n = col0 + t, elements k0 .. k0+63 of step s.
  // NN: reduction row n = k0 + t / 4, output columns col0 + 64 (t % 4) .. +63.
  const int64_t Kw = p.W.K;
  const uint8_t *codes_g = p.W.codes + g * p.W.g_codes;
  rsrc_t w_rsrc, s_rsrc;
  uint32_t w_voff[2], s_voff;
  int64_t w_step, s_step;          // byte advance per step (NT: along K; NN: 64 rows)
  if constexpr (MODE == 0) {
    const int64_t rows = p.Nc - col0;
    w_rsrc = make_rsrc(codes_g + col0 * (Kw >> 1), clamp_bytes(rows * (Kw >> 1)));
    w_voff[0] = (uint32_t)(t * (Kw >> 1));
    w_voff[1] = w_voff[0] + 16;
    w_step = BKS / 2;
  } else {
    w_rsrc = make_rsrc(codes_g, clamp_bytes(p.W.N * (Kw >> 1)));
    const int64_t kc = col0 + (t & 3) * 64;
    const uint32_t base = (uint32_t)((t >> 2) * (Kw >> 1) + (kc >> 1));
    w_voff[0] = kc < p.Nc ? base : OOB;
    w_voff[1] = kc + 32 < p.Nc ? base + 16 : OOB;
    w_step = (int64_t)BKS * (Kw >> 1);
  }
  // scales: NF4 fp32 / NF4_DQ e4m3 byte / MXFP4 two e8m0 bytes per run
  const int sc_per_row = FMT == FMT_MXFP4 ? (int)(Kw >> 5) : (int)(Kw >> 6);
  const int sc_bytes = FMT == FMT_NF4 ? 4 : 1;
  {
    const uint8_t *sb = reinterpret_cast<const uint8_t *>(p.W.scales) + (g * p.W.g_scales) * sc_bytes;
    if constexpr (MODE == 0) {
      const int64_t rows = p.Nc - col0;
      s_rsrc = make_rsrc(sb + col0 * sc_per_row * sc_bytes, clamp_bytes(rows * sc_per_row * sc_bytes));
      s_voff = (uint32_t)(t * sc_per_row * sc_bytes);
      s_step = (FMT == FMT_MXFP4 ? 2 : 1) * sc_bytes;
    } else {
      s_rsrc = make_rsrc(sb, clamp_bytes(p.W.N * sc_per_row * sc_bytes));
      const int64_t kc = col0 + (t & 3) * 64;
      const int64_t blk = FMT == FMT_MXFP4 ? (kc >> 5) : (kc >> 6);
      s_voff = kc < p.Nc ? (uint32_t)(((t >> 2) * sc_per_row + blk) * sc_bytes) : OOB;
      s_step = (int64_t)BKS * sc_per_row * sc_bytes;
    }
  }
  const float *scales2_g = FMT == FMT_NF4_DQ ? p.W.scales2 + g * p.W.g_scales2 : nullptr;

  struct WR {
    u32x4_t c0, c1;
    uint32_t sc;       // raw scale bits (fp32 bits, or e4m3 / e8m0 codes)
    float c2;          // DQ second level
  };
  auto load_w = [&](int s, WR &w) {
    const int wo = (int)(w_step * s);
    // NT runs run along K: the second half of the last run lies past the row
    // when K % 64 == 32 (MXFP4), so it is masked rather than read from the
    // next row. NN masks its column halves once, in w_voff.
    const bool h1 = MODE == 1 || (int64_t)s * BKS + 32 < p.R;
    w.c0 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, w_voff[0], wo, 0));
    w.c1 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, h1 ? w_voff[1] : OOB, wo, 0));
    const int so = (int)(s_step * s);
    if constexpr (FMT == FMT_NF4) {
      w.sc = __builtin_amdgcn_raw_buffer_load_b32(s_rsrc, s_voff, so, 0);
    } else if constexpr (FMT == FMT_NF4_DQ) {
      w.sc = __builtin_amdgcn_raw_buffer_load_b8(s_rsrc, s_voff, so, 0);
      int64_t idx;
      if constexpr (MODE == 0)
        idx = (col0 + t) * sc_per_row + (int64_t)s;
      else
        idx = ((int64_t)s * BKS + (t >> 2)) * sc_per_row + ((col0 + (t & 3) * 64) >> 6);
      const int64_t ng = p.W.g_scales2;
      const int64_t gi = idx >> 8;
      w.c2 = gi < ng ? scales2_g[gi] : 0.0f;
    } else {
      // two E8M0 codes, loaded one byte at a time so that a range check on
      // the second never discards the first
      const bool s1 = MODE == 0 ? h1 : (col0 + (t & 3) * 64 + 32 < p.Nc);
      const uint32_t e0 = __builtin_amdgcn_raw_buffer_load_b8(s_rsrc, s_voff, so, 0);
      const uint32_t e1 = __builtin_amdgcn_raw_buffer_load_b8(s_rsrc, s1 ? s_voff + 1 : OOB, so, 0);
      w.sc = e0 | (e1 << 8);
    }
  };

  // Dequantize the run in w into B tile Bs, chunks [2 part, 2 part + 2) of 8:
  // called in four parts between the MFMA sub-steps so the VALU work
  // overlaps the matrix cores.
  auto dequant_part = [&](const WR &w, const RunTable &T, float s0, float s1, uint16_t *Bs, int part) {
    uint16_t *dst = MODE == 0 ? Bs : Bs + (t >> 2) * LDB_NN + (t & 3) * 64;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int q = 2 * part + h;
      const uint32_t code = q < 4 ? w.c0[q] : w.c1[q - 4];
      u32x4_t v;
      if constexpr (FMT == FMT_MXFP4)
        v = decode8_mxfp4(code, q < 4 ? s0 : s1);
      else
        v = decode8_nf4(T, code);
      if constexpr (MODE == 0)
        lds_write_b128(dst + swz(t, q), v);
      else
        lds_write_b128(dst + 8 * q, v);
    }
  };
  auto run_setup = [&](const WR &w, RunTable &T, float &s0, float &s1) {
    if constexpr (FMT == FMT_MXFP4) {
      s0 = e8m0_to_f32(w.sc & 0xFFu);
      s1 = e8m0_to_f32((w.sc >> 8) & 0xFFu);
    } else {
      float c;
      if constexpr (FMT == FMT_NF4) c = __builtin_bit_cast(float, w.sc);
      else c = e4m3_to_f32(w.sc & 0xFFu) * w.c2;
      T = make_table(c, p.tab, sel);
      s0 = s1 = 0.0f;
    }
  };
  auto dequant_store = [&](const WR &w, uint16_t *Bs) {
    RunTable T;
    float s0, s1;
    run_setup(w, T, s0, s1);
#pragma unroll
    for (int part = 0; part < 4; ++part) dequant_part(w, T, s0, s1, Bs, part);
  };

  // acc[j][i]: 32 x 32 block (n-block j, m-block i) of this wave's 128 x 128
  f32x16_t acc[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[j][i] = f32x16_t{};

  // One 64-deep step of MFMAs on tiles (As, Bs). The operand reads are
  // software-pipelined: the next B fragment, and at the start of each
  // 16-deep sub-step the next sub-step's A fragments, are requested before
  // the current MFMAs issue, so LDS latency overlaps the matrix cores.
  // hook(kk) runs after sub-step kk's MFMAs (used to interleave dequant).
  auto load_af = [&](const uint16_t *As, int kk, u32x4_t af[4]) {
    const int q = kk * 2 + (lane >> 5);
#pragma unroll
    for (int i = 0; i < 4; ++i) af[i] = lds_read_b128(As + swz(wm0 + i * 32 + (lane & 31), q));
  };
  auto load_bf = [&](const uint16_t *Bs, int kk, int j) -> u32x4_t {
    if constexpr (MODE == 0)
      return lds_read_b128(Bs + swz(wn0 + j * 32 + (lane & 31), kk * 2 + (lane >> 5)));
    else
      return frag_tr32(Bs, LDB_NN, kk * 16, wn0 + j * 32, lane);
  };
  auto compute_step = [&](const uint16_t *As, const uint16_t *Bs, auto &&hook) {
    u32x4_t af0[4], af1[4];
    load_af(As, 0, af0);
    u32x4_t bcur = load_bf(Bs, 0, 0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4_t *af = (kk & 1) ? af1 : af0;
      u32x4_t *afn = (kk & 1) ? af0 : af1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4_t bnext = bcur;
        if (j < 3)
          bnext = load_bf(Bs, kk, j + 1);
        else if (kk < 3)
          bnext = load_bf(Bs, kk + 1, 0);
        if (j == 0 && kk < 3) load_af(As, kk + 1, afn);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[j][i] = mfma_32x32x16(bcur, af[i], acc[j][i]);
        bcur = bnext;
      }
      hook(kk);
#if LORA4_SCHED_INTERLEAVE
      // ask the scheduler to thread the hook's VALU work between this
      // sub-step's 16 MFMAs (each MFMA leaves the VALU free for a while)
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, LORA4_SCHED_VALU, 0);   // VALU
      }
#endif
    }
  };
  auto compute = [&](const uint16_t *As, const uint16_t *Bs) {
    compute_step(As, Bs, [](int) {});
  };

  const int steps = (int)((p.R + BKS - 1) / BKS);
  WR wa, wb;   // W registers for steps s+1 (wa) and s+2 (wb)
  if (steps > 0) {
    issue_a(0, As0);
    load_w(0, wa);
    dequant_store(wa, Bs0);
    if (steps > 1) load_w(1, wa);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // loads in flight per thread from one load_w (codes + scale bytes)
  constexpr int W_LOADS = FMT == FMT_NF4 ? 3 : 4;
  // s_waitcnt that waits until at most W_LOADS vector-memory loads are
  // outstanding: the direct LDS loads of the next step, issued before
  // load_w, have then landed, while the W loads two steps ahead stay in
  // flight across the barrier
  // (lgkmcnt 0: this wave's LDS writes are done before the barrier).
  constexpr int VMCNT_W = (W_LOADS & 15) | (7 << 4) | (0 << 8) | ((W_LOADS >> 4) << 14);
  // all but the last step: compute step s while step s+1 is dequantized and
  // loaded (one code path, so the accumulators stay put across iterations)
  for (int s = 0; s + 1 < steps; ++s) {
    const bool odd = s & 1;
    uint16_t *Acur = odd ? As1 : As0, *Bcur = odd ? Bs1 : Bs0;
    uint16_t *Anxt = odd ? As0 : As1, *Bnxt = odd ? Bs0 : Bs1;
    issue_a(s + 1, Anxt);
    const bool w_ahead = s + 2 < steps;
    if (w_ahead) load_w(s + 2, wb);
    RunTable T;
    float s0, s1;
    run_setup(wa, T, s0, s1);
    compute_step(Acur, Bcur, [&](int kk) { dequant_part(wa, T, s0, s1, Bnxt, kk); });
    wa = wb;
    if (w_ahead)
      __builtin_amdgcn_s_waitcnt(VMCNT_W);
    else
      __builtin_amdgcn_s_waitcnt(0);
    // a bare barrier: the waits above are all this step needs, and a full
    // workgroup fence would also drain the W loads still in flight
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }
  if (steps > 0) {
    const bool odd = (steps - 1) & 1;
    compute(odd ? As1 : As0, odd ? Bs1 : Bs0);
    __syncthreads();
  }

  // ---- rank-r tail: (s Z) B^T (NT) or dZ A (NN), plain bf16 steps ------------
  if (p.r2 > 0) {
    const uint16_t *B2 = p.B2.p + g * p.B2.gstride;
    for (int k0 = 0; k0 < p.r2; k0 += BKS) {
      // activation tail [256 x 64] and the adapter tile, through registers
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int idx = t + THREADS * c;
        const int row = idx >> 3, chunk = idx & 7;
        uint32_t w4[4] = {0u, 0u, 0u, 0u};
        const int64_t gr = row0 + row;
        const int64_t gk = k0 + chunk * 8;
        if (gr < row_end) {
          const uint16_t *src = p.A2.p + gr * p.A2.ld + gk;
          for (int j = 0; j < 8; ++j)
            if (gk + j < p.r2) w4[j >> 1] |= (uint32_t)src[j] << (16 * (j & 1));
        }
        lds_write_b128(As0 + swz(row, chunk), u32x4_t{w4[0], w4[1], w4[2], w4[3]});
      }
      if constexpr (MODE == 0) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int idx = t + THREADS * c;
          const int row = idx >> 3, chunk = idx & 7;
          uint32_t w4[4] = {0u, 0u, 0u, 0u};
          const int64_t gn = col0 + row;
          const int64_t gk = k0 + chunk * 8;
          if (gn < p.Nc) {
            const uint16_t *src = B2 + gn * p.B2.ld + gk;
            for (int j = 0; j < 8; ++j)
              if (gk + j < p.r2) w4[j >> 1] |= (uint32_t)src[j] << (16 * (j & 1));
          }
          lds_write_b128(Bs0 + swz(row, chunk), u32x4_t{w4[0], w4[1], w4[2], w4[3]});
        }
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int idx = t + THREADS * c;
          const int row = idx >> 5, cc = (idx & 31) * 8;
          uint32_t w4[4] = {0u, 0u, 0u, 0u};
          const int64_t gr = k0 + row;
          const int64_t gc = col0 + cc;
          if (gr < p.r2) {
            const uint16_t *src = B2 + gr * p.B2.ld + gc;
            for (int j = 0; j < 8; ++j)
              if (gc + j < p.Nc) w4[j >> 1] |= (uint32_t)src[j] << (16 * (j & 1));
          }
          lds_write_b128(Bs0 + row * LDB_NN + cc, u32x4_t{w4[0], w4[1], w4[2], w4[3]});
        }
      }
      __syncthreads();
      compute(As0, Bs0);
      __syncthreads();
    }
  }

  // ---- epilogue: register r of acc[j][i] holds
  // C[wm0 + 32 i + lane % 32][wn0 + 32 j + 8 (r / 4) + 4 (lane / 32) + r % 4]
  const bool vec_out = (p.ldc % 4) == 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = row0 + wm0 + i * 32 + (lane & 31);
    if (row >= row_end) continue;
    uint16_t *crow = p.C + row * p.ldc;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int64_t col = col0 + wn0 + j * 32 + r4 * 8 + (lane >> 5) * 4;
        const float v0 = acc[j][i][4 * r4], v1 = acc[j][i][4 * r4 + 1];
        const float v2 = acc[j][i][4 * r4 + 2], v3 = acc[j][i][4 * r4 + 3];
        if (vec_out && col + 4 <= p.Nc) {
          u32x2_t pk = {pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
          *reinterpret_cast<u32x2_t *>(crow + col) = pk;
        } else {
          const float v[4] = {v0, v1, v2, v3};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (col + e < p.Nc) crow[col + e] = to_bf16(v[e]);
        }
      }
    }
  }
}

}  // namespace big
}  // namespace lora4
