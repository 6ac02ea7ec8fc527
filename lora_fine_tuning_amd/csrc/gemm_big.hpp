// Shared pieces of the two 256 x 256 dequant-GEMMs (gemm_fwd.hpp,
// gemm_dgrad.hpp): their parameter block, buffer descriptors for bounds-checked
// loads, the NF4 run tables (16-entry bf16 tables bf16(q[i] c) whose byte
// planes are selected with v_perm_b32, bit-identical to bf16(fp32(q[code] c))
// per element), the MXFP4 decode through v_cvt_scalef32_pk_bf16_fp4, and the
// rank-r tail operand taken from fp32 range partials.
#pragma once

#include "formats.hpp"

namespace lora4 {
namespace big {

// VALU instructions the scheduling hints place between the two MFMAs of a pair
// in the sub-steps without hand-dealt slices (the rank-r product).
constexpr int SCHED_VALU = 5;

constexpr int BM = 256, BN = 256, BKS = 64;   // tile of both GEMMs
constexpr uint32_t RSRC_WORD3 = 0x00020000u;   // raw 32-bit buffer, gfx9 family
constexpr uint32_t OOB = 0x80000000u;           // an offset past any range

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
  int tiles_n;        // output column tiles (ceil(Nc / 256); the forward's 128 x 128 kernel: ceil(Nc / 128))
  int nblocks;        // gridDim.x
  int nslots;         // row-tile slots (tiles_n x nslots tiles in grouped order)
  // forward, whole-tile launches: the first nfull tiles in grouped order run
  // whole, the ntail after them as two 256 x 128 halves (blocks nfull ..)
  int nfull, ntail;
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
  // 1: one W for every row group (adapters over one base): the output tiles
  // ignore the groups, and the rank-r part runs once per group that has rows
  // in the tile, with that group's B2 (forward) or A (dgrad). The kernels
  // take it as a template argument (SHARED) too, so that the per-group code
  // is compiled only where it runs.
  int shared_rows;
  // MX-native forward: X as MXFP8, E4M3 codes [rows padded to 256][ld8]
  // (zero padding; ld8 = K rounded up to 64) and E8M0 scales in the order
  // k_quant_mxfp8 writes for the GEMM
  const uint8_t *X8;
  const uint8_t *X8s;
  int64_t ld8;
};

// Row tile of block slot: per group (experts), or over all M rows when the
// groups share W.
template <bool SHARED>
__device__ __forceinline__ RowTile tile_rows(const Params &p, int slot, int BM) {
  return SHARED ? map_row_tile(slot, BM, nullptr, 1, p.M) : map_row_tile(slot, BM, p.offsets, p.groups, p.M);
}

// The group holding row `row` (offsets non-decreasing, [0] = 0, [groups] = M):
// the last g with offsets[g] <= row.
__device__ __forceinline__ int group_of_row(const int64_t *offsets, int groups, int64_t row) {
  int lo = 0, hi = groups - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offsets[mid] <= row) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// The groups of a tile that ignores the groups (offsets given: tiles ignore
// the groups only where there are several), from the one holding row0 to the
// one holding row_hi - 1 (those between may have no rows; cols_empty skips
// them): their tail products run as one product whose
// reduction puts the groups' rank columns side by side, group g0 + i at
// columns i rp .. i rp + r2 - 1 (rp = r2 rounded up to 8). A row's operand
// is zero outside its own group's columns and each group's B rows fill its
// columns, so the sum over the wider reduction is each row's own group's
// product (a block-diagonal operand), in one pass for all the groups.
struct TileGroups {
  int g0, n, rp;
};

__device__ __forceinline__ TileGroups tile_groups(const Params &p, int64_t row0, int64_t row_hi) {
  TileGroups tg;
  tg.g0 = group_of_row(p.offsets, p.groups, row0);
  tg.n = group_of_row(p.offsets, p.groups, row_hi - 1) - tg.g0 + 1;
  tg.rp = (p.r2 + 7) & ~7;
  return tg;
}

// Whether the reduction columns [k0, k0 + width) hold no row of the tile:
// every tile group they belong to has no rows in [row0, row_hi). (Empty
// groups between the tile's first and last would otherwise cost full steps
// of zeros.) Uniform across the workgroup.
__device__ __forceinline__ bool cols_empty(const Params &p, const TileGroups &tg, int k0, int width, int64_t row0,
                                           int64_t row_hi) {
  const int gi_lo = k0 / tg.rp;
  const int gi_hi = min((k0 + width - 1) / tg.rp, tg.n - 1);
  for (int gi = gi_lo; gi <= gi_hi; ++gi) {
    const int64_t a = max(p.offsets[tg.g0 + gi], row0), b = min(p.offsets[tg.g0 + gi + 1], row_hi);
    if (a < b) return false;
  }
  return true;
}

// Index within the tile's groups of the group holding row gr (-1 for a row
// past the tile's range).
__device__ __forceinline__ int row_group(const Params &p, const TileGroups &tg, int64_t gr, int64_t row_hi) {
  return gr < row_hi ? group_of_row(p.offsets + tg.g0, tg.n, gr) : -1;
}

constexpr int A2_MAX_PARTS = 4;

// Row tiles per group of the tile order below (2 and 8 measured slower).
constexpr int GROUP_M = 4;

// Tile t of a slots x tiles_n grid of output tiles in grouped order: runs of
// GROUP_M row tiles are walked column by column, so that the tiles one
// XCD runs at the same time (a contiguous range of t) share activation row
// tiles and W column tiles in its L2.
__device__ __forceinline__ void grouped_tile(int t, int tiles_n, int slots, int &slot, int &tn) {
  const int per_group = GROUP_M * tiles_n;
  const int gi = t / per_group;
  const int r = t - gi * per_group;
  const int g0 = gi * GROUP_M;
  const int rows = slots - g0 < GROUP_M ? slots - g0 : GROUP_M;
  tn = r / rows;
  slot = g0 + (r - tn * rows);
}

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
// LDS tile `As` (256 rows from row0, bf16, 8-column chunk c of row i at
// As + lds_off(i, c)): thread t owns row row0 + t; rows at or past rb and
// chunks past r2 are zero. SHARED: the columns are those of the tile's groups
// side by side (rp per group) and the row's own group is the tile's group
// `my` (-1: none), its other groups' columns zero.
template <bool SHARED, typename Off>
__device__ __forceinline__ void a2_parts_to_lds(const Params &p, uint16_t *As, Off lds_off, int64_t row0,
                                                int64_t rb, int k0, int t, bool store_out, int rp = 0, int my = 0) {
  const int64_t gr = row0 + t;
  const bool row_ok = gr < rb;
#pragma unroll 1
  for (int c0 = 0; c0 < 8; c0 += 2) {
    float v[2][8];
    bool ok[2];
    int64_t gk[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int kc = k0 + 8 * (c0 + u);
      int gi = 0;
      if constexpr (SHARED) gi = kc / rp;
      gk[u] = kc - gi * rp;
      ok[u] = row_ok && gi == my && gk[u] < p.r2;
      if (ok[u]) {
        a2_part_sum(p, gr, gk[u], v[u]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[u][e] = 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      lds_write_b128(As + lds_off(t, c0 + u), pack_scaled8(v[u], p.A2scale));
      if (store_out && ok[u]) {
        if (p.A2out1) store_a2_piece(p.A2out1, p.r2, gr, gk[u], pack_scaled8(v[u], p.A2alpha1));
        if (p.A2out2) store_a2_piece(p.A2out2, p.r2, gr, gk[u], pack_scaled8(v[u], p.A2alpha2));
      }
    }
  }
}

// The same step from the bf16 operand rows of A2, thread t owning row
// row0 + t (the SHARED layout of a2_parts_to_lds).
template <typename Off>
__device__ __forceinline__ void a2_rows_to_lds(const Params &p, uint16_t *As, Off lds_off, int64_t row0, int64_t rb,
                                               int k0, int t, int rp, int my) {
  const int64_t gr = row0 + t;
  const bool a_vec = (p.A2.ld % 8) == 0;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int kc = k0 + 8 * c;
    const int gi = kc / rp;
    const int64_t gk = kc - gi * rp;
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (gr < rb && gi == my && gk < p.r2) {
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
    lds_write_b128(As + lds_off(t, c), v);
  }
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, (int)RSRC_WORD3);
}

__device__ __forceinline__ uint32_t clamp_bytes(int64_t b) {
  return b <= 0 ? 0u : (b >= (int64_t)0x7FFFFFFF ? 0x7FFFFFFFu : (uint32_t)b);
}

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

// Lookup indices of the four elements in the low (HI = 0) or high nibbles of
// an NF4 code word (elements 0..3 or 4..7, nf4_nibble): i7 = the code's low
// three bits per byte, s3 = byte j: j + 4 * bit 3 (selects the table half).
template <int HI>
__device__ __forceinline__ void nf4_idx(const RunTable &T, uint32_t c, uint32_t &i7, uint32_t &s3) {
  i7 = (c >> (4 * HI)) & 0x07070707u;
  s3 = ((c >> (4 * HI + 1)) & 0x04040404u) | T.sel;
}

// Low and high bytes of T[index] for the four indices (i7, s3).
__device__ __forceinline__ void lookup4(const RunTable &T, uint32_t i7, uint32_t s3, uint32_t &L, uint32_t &H) {
  const uint32_t la = perm(T.lo[1], T.lo[0], i7);
  const uint32_t lb = perm(T.lo[3], T.lo[2], i7);
  const uint32_t ha = perm(T.hi[1], T.hi[0], i7);
  const uint32_t hb = perm(T.hi[3], T.hi[2], i7);
  L = perm(lb, la, s3);
  H = perm(hb, ha, s3);
}

// Elements 0..3 (low and high bytes L, H) -> 2 words of bf16 pairs.
__device__ __forceinline__ uint32_t pair_lo(uint32_t L, uint32_t H) { return perm(H, L, 0x05010400u); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t L, uint32_t H) { return perm(H, L, 0x07030602u); }

// 8 codes (one word of the tiled NF4 storage) -> 4 words of bf16 pairs:
// 23 VALU instructions.
__device__ __forceinline__ u32x4_t decode8_nf4(const RunTable &T, uint32_t c) {
  uint32_t i7, s3, L0, H0, L1, H1;
  nf4_idx<0>(T, c, i7, s3);
  lookup4(T, i7, s3, L0, H0);
  nf4_idx<1>(T, c, i7, s3);
  lookup4(T, i7, s3, L1, H1);
  return u32x4_t{pair_lo(L0, H0), pair_hi(L0, H0), pair_lo(L1, H1), pair_hi(L1, H1)};
}

__device__ __forceinline__ u32x4_t decode8_mxfp4(uint32_t c, float s) {
  return u32x4_t{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, s, 0)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, s, 1)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, s, 2)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, s, 3))};
}


}  // namespace big
}  // namespace lora4
