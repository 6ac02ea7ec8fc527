// Input-gradient dequant-GEMM:
//
//   dX[M, K] = dY[M, N] . deq(W)[N, K]   (+ dZ[M, r] . A[r, K] tail)
//
// The reduction runs over the rows of W, while the packed codes are contiguous
// along K (the output), so the MFMA operand (eight consecutive reduction
// elements per lane) needs a transpose: each thread decodes one 64-element run
// of a W row into an LDS tile [64 reduction rows][256 output columns] (lane =
// row, wave = 64-column block), and the waves read it back with
// ds_read_b64_tr_b16. Both tiles are swizzled so that every LDS access is free
// of bank conflicts.
//
// One workgroup = 4 waves (2 x 2) computing a 256 x 256 tile of dX; each wave
// owns 128 x 128 (4 x 4 blocks of v_mfma_f32_32x32x16_bf16, 256 fp32
// accumulators per lane). Per 64-deep step s:
//  * dY of step s+1 streams HBM/L2 -> LDS with bounds-checked direct loads
//    (two stages of 256 x 64, swizzled), issued in the first half of step s;
//  * the packed run of step s+2 is loaded into registers in sub-step 0 of
//    step s, and the run of step s+1 (loaded a step earlier) is decoded into
//    the other W tile over the step;
//  * one barrier, inside the last sub-step, after which the first operand
//    fragments of step s+1 are read behind the last MFMAs of step s.
// All look-ahead loads are issued unconditionally (past the end they are out
// of range and return zeros); the main loop is unrolled twice so the two sets
// of look-ahead registers swap roles instead of being copied. The schedule is
// built by hand, one slice of work per pair of MFMAs (see below).
#pragma once

#include <type_traits>

#include "gemm_big.hpp"

namespace lora4 {
namespace dgrad {

using big::OOB;
using big::Params;
using big::RunTable;
using big::rsrc_t;

// VALU instructions placed between the two MFMAs of a pair in the hand-dealt
// sub-steps.
constexpr int SLICE_V1 = 5;

constexpr int BM = 256, BN = 256, BKS = 64, THREADS = 256;
constexpr int TILE_A = BM * BKS;    // dY stage [256][64], tile64 layout
constexpr int TILE_W = BKS * BN;    // deq(W) tile [64][256]

__host__ __device__ constexpr int lds_bytes() { return 2 * (TILE_A + TILE_W) * 2; }

__device__ __forceinline__ int swz(int row, int chunk) { return tile64_swz(row, chunk); }

// deq(W) tile [64 reduction rows][256 output columns]: 512-byte rows of 32
// chunks of 16 bytes, chunk c of row n stored at c ^ wsw(n). LDS writes are
// served 128 bytes at a time (8 lanes = 8 consecutive rows at one chunk: 8
// distinct positions), reads 256 bytes at a time (32 lanes of a transposing
// read = 4 rows x 4 consecutive chunks, 8 bytes each: 64 distinct banks).
__device__ __forceinline__ int wsw(int n) { return ((n & 3) << 2) | ((n >> 1) & 3); }
__device__ __forceinline__ int wt_off(int n, int col) { return n * BN + (((col >> 3) ^ wsw(n)) << 3) + (col & 7); }

// MFMA 32x32x16 operand from the deq(W) tile: lane l gets column c0 + l % 32
// of reduction rows k0 + 8 (l / 32) .. +7 (two transposing reads per lane).
__device__ __forceinline__ u32x4_t frag_w(const uint16_t *Bs, int k0, int c0, int lane) {
  const int grp = lane >> 4, j = lane & 15;
  const int n = k0 + (grp >> 1) * 8 + (j >> 2);
  const int col = c0 + (grp & 1) * 16 + (j & 3) * 4;
  const u32x2_t lo = lds_read_tr16(Bs + wt_off(n, col));
  const u32x2_t hi = lds_read_tr16(Bs + wt_off(n + 4, col));
  return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
}

// Raw loads of one thread for one step: its 64-element run.
struct WRaw {
  u32x4_t c0, c1;
  uint32_t sc;   // NF4: fp32 bits; DQ: e4m3 code; MXFP4: two e8m0 codes; NVFP4: four e4m3 codes
  uint32_t c2;   // DQ second level (fp32 bits)
};

// SHARED: the row tiles ignore the groups (Params::shared_rows).
template <int FMT, bool SHARED>
__global__ __launch_bounds__(THREADS, 1) void k_gemm_dgrad(Params p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  const uint32_t sel = big::sel_base();
  uint16_t *const As0 = smem, *const As1 = smem + TILE_A;
  uint16_t *const Bs0 = smem + 2 * TILE_A, *const Bs1 = smem + 2 * TILE_A + TILE_W;

  int b = blockIdx.x;
  {
    const int per = p.nblocks >> 3;
    if (b < per * 8) b = (b & 7) * per + (b >> 3);
  }
  int tn, slot;
  big::grouped_tile(b, p.tiles_n, p.nblocks / p.tiles_n, slot, tn);
  const RowTile rt = big::tile_rows<SHARED>(p, slot, BM);
  if (rt.group < 0) return;
  const int g = rt.group;
  const int64_t row0 = rt.row0, row_end = rt.row_end;
  const int64_t col0 = (int64_t)tn * BN;

  const int t = threadIdx.x;
  // the wave index is uniform: keep it (and what derives from it) scalar
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63;
  const int l32 = lane & 31, h = lane >> 5;
  const int wm0 = (wave & 1) * 128, wn0 = (wave >> 1) * 128;

  // ---- dY: direct loads into LDS; wave w, chunk c covers rows 8 (4 c + w)..
  const rsrc_t a_rsrc = big::make_rsrc(p.A.p + row0 * p.A.ld, big::clamp_bytes((row_end - row0) * p.A.ld * 2));
  const int a_kq = tile64_dma_chunk(lane, wave) * 8;
  const uint32_t a_voff0 = (uint32_t)(((wave * 8 + (lane >> 3)) * p.A.ld + a_kq) * 2);
  const uint32_t a_cstep = (uint32_t)(32 * p.A.ld * 2);
  // dY of step s into stage As, chunks 4 half .. 4 half + 3
  auto issue_a = [&](int s, uint16_t *As, int half) {
    const int64_t k0 = (int64_t)s * BKS;
    const bool edge = k0 + a_kq >= p.R;
#pragma unroll
    for (int c = 4 * half; c < 4 * half + 4; ++c)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (__attribute__((address_space(3))) void *)(As + (c * 4 + wave) * 512),
                                               16, edge ? OOB : a_voff0 + c * a_cstep, (int)(k0 * 2), 0, 0);
  };

  // ---- this thread's run: reduction row k0 + lane, output columns
  // col0 + 64 wave .. +63 = row lane of tile (k0 / 64, kc / 64) of the tiled
  // base: its 32 bytes of codes at 32 lane, its scale entries contiguous
  const int64_t Kw = p.W.K;
  const int64_t KB = p.W.KB;
  const int gw = w_group(p.W, g);   // group of W
  const uint8_t *codes_g = p.W.codes + gw * p.W.g_codes;
  const rsrc_t w_rsrc = big::make_rsrc(codes_g, big::clamp_bytes(p.W.g_codes));
  const int64_t kc = col0 + wave * 64;
  const uint32_t w_base = (uint32_t)((kc >> 6) * 2048 + lane * 32);
  const uint32_t w_voff0 = kc < p.Nc ? w_base : OOB;
  const uint32_t w_voff1 = kc + 32 < p.Nc ? w_base + 16 : OOB;
  const int64_t w_step = KB * 2048;   // one row block of tiles per step
  const int sc_per_row = (int)(Kw >> 6);   // NF4-DQ: scales per row, row-major (second level)
  constexpr int sc_bytes = FMT == FMT_NF4 ? 4 : 1;
  constexpr int sc_tile = FMT == FMT_MXFP4 ? 128 : FMT == FMT_NVFP4 ? 256 : 64 * sc_bytes;   // scale bytes per tile
  const uint8_t *sbase = reinterpret_cast<const uint8_t *>(p.W.scales) + (gw * p.W.g_scales) * sc_bytes;
  const rsrc_t s_rsrc = big::make_rsrc(sbase, big::clamp_bytes(p.W.g_scales * sc_bytes));
  const uint32_t s_voff =
      kc < p.Nc ? (uint32_t)((kc >> 6) * sc_tile + (FMT == FMT_MXFP4   ? lane * 2
                                                   : FMT == FMT_NVFP4 ? lane * 4
                                                                      : lane * sc_bytes))
                : OOB;
  // MXFP4: second code; NVFP4: third and fourth codes (the run's second half)
  const uint32_t s_voff1 = kc + 32 < p.Nc ? s_voff + (FMT == FMT_NVFP4 ? 2 : 1) : OOB;
  const int64_t s_step = KB * sc_tile;
  const rsrc_t s2_rsrc = FMT == FMT_NF4_DQ
                             ? big::make_rsrc(p.W.scales2 + gw * p.W.g_scales2, big::clamp_bytes(p.W.g_scales2 * 4))
                             : big::make_rsrc(p.W.codes, 0u);

  auto load_w = [&](int s, WRaw &w) {
    const int wo = (int)(w_step * s);
    w.c0 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, w_voff0, wo, 0));
    w.c1 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, w_voff1, wo, 0));
    const int so = (int)(s_step * s);
    if constexpr (FMT == FMT_NF4) {
      w.sc = __builtin_amdgcn_raw_buffer_load_b32(s_rsrc, s_voff, so, 0);
    } else if constexpr (FMT == FMT_NF4_DQ) {
      w.sc = __builtin_amdgcn_raw_buffer_load_b8(s_rsrc, s_voff, so, 0);
      const int64_t idx = ((int64_t)s * BKS + lane) * sc_per_row + (kc >> 6);
      w.c2 = __builtin_amdgcn_raw_buffer_load_b32(s2_rsrc, kc < p.Nc ? (uint32_t)((idx >> 8) * 4) : OOB, 0, 0);
    } else if constexpr (FMT == FMT_NVFP4) {
      // two E4M3 codes per half of the run, loaded per half as for MXFP4
      const uint32_t e0 = __builtin_amdgcn_raw_buffer_load_b16(s_rsrc, s_voff, so, 0);
      const uint32_t e1 = __builtin_amdgcn_raw_buffer_load_b16(s_rsrc, s_voff1, so, 0);
      w.sc = e0 | (e1 << 16);
    } else {
      // two E8M0 codes, one byte each, so that a range check on the second
      // never discards the first
      const uint32_t e0 = __builtin_amdgcn_raw_buffer_load_b8(s_rsrc, s_voff, so, 0);
      const uint32_t e1 = __builtin_amdgcn_raw_buffer_load_b8(s_rsrc, s_voff1, so, 0);
      w.sc = e0 | (e1 << 8);
    }
  };

  // decode part `part` (0..3) of raw run w: elements 16 part .. +15 (code
  // words 2 part, 2 part + 1) into row `lane` of W tile Bs
  auto decode_part = [&](const WRaw &w, uint16_t *Bs, RunTable &T, float &s0, float &s1, int part) {
    if (part == 0) {
      if constexpr (FMT == FMT_MXFP4) {
        s0 = e8m0_to_f32(w.sc & 0xFFu);
        s1 = e8m0_to_f32((w.sc >> 8) & 0xFFu);
      } else if constexpr (FMT == FMT_NVFP4) {
        // (the scale of each 16-element block is decoded with its words)
      } else {
        float c;
        if constexpr (FMT == FMT_NF4) c = __builtin_bit_cast(float, w.sc);
        else c = e4m3_to_f32(w.sc & 0xFFu) * __builtin_bit_cast(float, w.c2);
        T = big::make_table(c, p.tab, sel);
      }
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int q = 2 * part + e;
      const uint32_t code = q < 4 ? w.c0[q] : w.c1[q - 4];
      u32x4_t v;
      if constexpr (FMT == FMT_MXFP4)
        v = big::decode8_mxfp4(code, q < 4 ? s0 : s1);
      else if constexpr (FMT == FMT_NVFP4)
        v = decode8_nvfp4(code, e4m3_to_f32((w.sc >> (8 * (q >> 1))) & 0xFFu));
      else
        v = big::decode8_nf4(T, code);
      lds_write_b128(Bs + wt_off(lane, wave * 64 + 8 * q), v);
    }
  };

  // acc[j][i]: output columns wn0 + 32 j .., rows wm0 + 32 i ..
  f32x16_t acc[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[j][i] = f32x16_t{};

  auto read_af = [&](const uint16_t *As, int kk, u32x4_t af[4], int nblk = 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i < nblk) af[i] = lds_read_b128(As + swz(wm0 + i * 32 + l32, kk * 2 + h));
  };
  auto read_bf = [&](const uint16_t *Bs, int kk, int j) -> u32x4_t {
    return frag_w(Bs, kk * 16, wn0 + j * 32, lane);
  };

  // The first nk sub-steps of a 64-deep step on (As, Bs), for the rank-r
  // tail. The A fragments of the next sub-step are requested at its start
  // (double-buffered), the B fragment j of the next sub-step right after its
  // four MFMAs; the first fragments are read at the start.
  auto compute_step = [&](const uint16_t *As, const uint16_t *Bs, int nk) {
    u32x4_t afa[4], afb[4], bf[4];
    read_af(As, 0, afa);
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = read_bf(Bs, 0, j);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk >= nk) break;
      u32x4_t *af = (kk & 1) ? afb : afa;
      u32x4_t *afn = (kk & 1) ? afa : afb;
      const bool more = kk < 3;
      if (more) read_af(As, kk + 1, afn);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[j][i] = mfma_32x32x16(bf[j], af[i], acc[j][i]);
        if (more) bf[j] = read_bf(Bs, kk + 1, j);
      }
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                         // MFMA
        if (more && m < 12) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // LDS read
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- the step dealt out by hand over its 32 MFMA pairs (slice G =
  // 8 kk + m = MFMAs of block row j = m / 2, columns 2 (m % 2) ..), fenced
  // per pair: slices 0-3 build the NF4 table of run rdec, then its eight code
  // words go through four stages each (unpack; low-index lookup; high-index
  // lookup; interleave + LDS write), word w in slices 3 + 3 w .. 6 + 3 w; the
  // dY chunks of step s+1 go out in slices 0-7 and the run of step s+2 in
  // slices 8-10. At slice 28 every wave waits for its dY chunks and LDS writes
  // and meets the others; the next step's first fragments are then read
  // behind the last MFMAs of this one.
  struct WordDec {
    uint32_t i0, i1, L0, H0, L1, H1;   // i0, i1: lookup indices of elements 0..3 (big::nf4_idx)
    float sc;   // NVFP4: the word's E4M3 block scale
  };
  struct TabBuild {
    float c;
    float pr[16];
    uint32_t t[8];
  };
  auto issue_a1 = [&](int s, uint16_t *As, int c) {
    const int64_t k0 = (int64_t)s * BKS;
    const bool edge = k0 + a_kq >= p.R;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (__attribute__((address_space(3))) void *)(As + (c * 4 + wave) * 512),
                                             16, edge ? OOB : a_voff0 + c * a_cstep, (int)(k0 * 2), 0, 0);
  };
  // global loads of run s after the dY chunks: codes 0..3, codes 4..7, scales
  constexpr int W_LOADS_D = FMT == FMT_NF4 ? 3 : 4;
  auto load_w1 = [&](int s, WRaw &w, int part) {
    const int wo = (int)(w_step * s);
    const int so = (int)(s_step * s);
    if (part == 0) {
      w.c0 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, w_voff0, wo, 0));
    } else if (part == 1) {
      w.c1 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, w_voff1, wo, 0));
    } else if constexpr (FMT == FMT_NF4) {
      w.sc = __builtin_amdgcn_raw_buffer_load_b32(s_rsrc, s_voff, so, 0);
    } else if constexpr (FMT == FMT_NF4_DQ) {
      w.sc = __builtin_amdgcn_raw_buffer_load_b8(s_rsrc, s_voff, so, 0);
      const int64_t idx = ((int64_t)s * BKS + lane) * sc_per_row + (kc >> 6);
      w.c2 = __builtin_amdgcn_raw_buffer_load_b32(s2_rsrc, kc < p.Nc ? (uint32_t)((idx >> 8) * 4) : OOB, 0, 0);
    } else if constexpr (FMT == FMT_NVFP4) {
      const uint32_t e0 = __builtin_amdgcn_raw_buffer_load_b16(s_rsrc, s_voff, so, 0);
      const uint32_t e1 = __builtin_amdgcn_raw_buffer_load_b16(s_rsrc, s_voff1, so, 0);
      w.sc = e0 | (e1 << 16);
    } else {
      const uint32_t e0 = __builtin_amdgcn_raw_buffer_load_b8(s_rsrc, s_voff, so, 0);
      const uint32_t e1 = __builtin_amdgcn_raw_buffer_load_b8(s_rsrc, s_voff1, so, 0);
      w.sc = e0 | (e1 << 8);
    }
  };
  auto tab_stage = [&](int st, const WRaw &w, TabBuild &tb, RunTable &T, float &s0, float &s1) {
    if constexpr (FMT == FMT_NVFP4) {
      // (no run state: each word decodes its own block scale)
    } else if constexpr (FMT == FMT_MXFP4) {
      if (st == 0) {
        s0 = e8m0_to_f32(w.sc & 0xFFu);
        s1 = e8m0_to_f32((w.sc >> 8) & 0xFFu);
      }
    } else if (st == 0) {
      if constexpr (FMT == FMT_NF4) tb.c = __builtin_bit_cast(float, w.sc);
      else tb.c = e4m3_to_f32(w.sc & 0xFFu) * __builtin_bit_cast(float, w.c2);
      pin(tb.c);
#pragma unroll
      for (int k = 0; k < 8; ++k) tb.pr[k] = p.tab.q[k] * tb.c;
    } else if (st == 1) {
      pin(tb.c);
#pragma unroll
      for (int k = 8; k < 16; ++k) tb.pr[k] = p.tab.q[k] * tb.c;
    } else if (st == 2) {
#pragma unroll
      for (int k = 0; k < 8; ++k) tb.t[k] = pack_bf16x2(tb.pr[2 * k], tb.pr[2 * k + 1]);
    } else {
      T = big::table_from(tb.t, sel);
    }
  };
  auto word_stage = [&](int st, const WRaw &w, int q, WordDec &o, const RunTable &T, float s0, float s1,
                        uint16_t *Bs) {
    uint32_t code = q < 4 ? w.c0[q] : w.c1[q - 4];
    if (st == 0) pin(code);
    if constexpr (FMT == FMT_NVFP4) {
      if (st == 0) {
        o.sc = e4m3_to_f32((w.sc >> (8 * (q >> 1))) & 0xFFu);
        o.L0 = nvfp4_pair_t<0>(code, o.sc);
        o.H0 = nvfp4_pair_t<1>(code, o.sc);
      } else if (st == 1) {
        o.L1 = nvfp4_pair_t<2>(code, o.sc);
        o.H1 = nvfp4_pair_t<3>(code, o.sc);
      } else if (st == 3) {
        lds_write_b128(Bs + wt_off(lane, wave * 64 + 8 * q), u32x4_t{o.L0, o.H0, o.L1, o.H1});
      }
    } else if constexpr (FMT == FMT_MXFP4) {
      const float sc = q < 4 ? s0 : s1;
      if (st == 0) {
        o.L0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(code, sc, 0));
        o.H0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(code, sc, 1));
      } else if (st == 1) {
        o.L1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(code, sc, 2));
        o.H1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(code, sc, 3));
      } else if (st == 3) {
        lds_write_b128(Bs + wt_off(lane, wave * 64 + 8 * q), u32x4_t{o.L0, o.H0, o.L1, o.H1});
      }
    } else {
      // indices of elements 0..3; their lookup; indices and lookup of
      // elements 4..7 (from the code word); interleave + LDS write
      if (st == 0) {
        big::nf4_idx<0>(T, code, o.i0, o.i1);
        pin(o.i0);
        pin(o.i1);
      } else if (st == 1) {
        big::lookup4(T, o.i0, o.i1, o.L0, o.H0);
      } else if (st == 2) {
        uint32_t i7, s3;
        big::nf4_idx<1>(T, code, i7, s3);
        big::lookup4(T, i7, s3, o.L1, o.H1);
      } else {
        lds_write_b128(Bs + wt_off(lane, wave * 64 + 8 * q),
                       u32x4_t{big::pair_lo(o.L0, o.H0), big::pair_hi(o.L0, o.H0), big::pair_lo(o.L1, o.H1),
                               big::pair_hi(o.L1, o.H1)});
      }
    }
  };
  // wait for this wave's dY chunks (the run loads issued after them may stay
  // in flight) and LDS accesses, then meet the other waves
  constexpr int VM_D = W_LOADS_D;
  constexpr int VMCNT_D = (VM_D & 15) | (7 << 4) | (0 << 8) | ((VM_D >> 4) << 14);
  u32x4_t afa[4], afb[4], bf[4];
  // IA (a std::integral_constant): how many of the wave's four 32-row blocks
  // hold rows of the tile; MFMAs and operand reads of the others are left out
  auto step_s = [&](auto ia, int s, const uint16_t *Acur, const uint16_t *Bcur, uint16_t *Anxt, uint16_t *Bnxt,
                    const WRaw &rdec, WRaw &rload) __attribute__((always_inline)) {
    constexpr int IA = decltype(ia)::value;
    RunTable T;
    float s0 = 0.0f, s1 = 0.0f;
    TabBuild tb;
    WordDec wd[2];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4_t *af = (kk & 1) ? afb : afa;
      u32x4_t *afn = (kk & 1) ? afa : afb;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int G = kk * 8 + m;
        const int j = m >> 1, i0 = (m & 1) * 2;
        if (i0 < IA) acc[j][i0] = mfma_32x32x16(bf[j], af[i0], acc[j][i0]);
        if (i0 + 1 < IA) acc[j][i0 + 1] = mfma_32x32x16(bf[j], af[i0 + 1], acc[j][i0 + 1]);
        if (kk < 3) {
          if (m < IA) afn[m] = lds_read_b128(Acur + swz(wm0 + m * 32 + l32, (kk + 1) * 2 + h));
          if (IA > 0 && (m & 1)) bf[j] = read_bf(Bcur, kk + 1, j);
        } else if (m == 4) {
          __builtin_amdgcn_s_waitcnt(VMCNT_D);
          asm volatile("" ::: "memory");
          __builtin_amdgcn_s_barrier();
          asm volatile("" ::: "memory");
          read_af(Anxt, 0, afa, IA);
          if (IA > 0) {
            bf[0] = read_bf(Bnxt, 0, 0);
            bf[1] = read_bf(Bnxt, 0, 1);
          }
        } else if (IA > 0 && (m == 5 || m == 7)) {
          bf[j] = read_bf(Bnxt, 0, j);
        }
        if (G < 4) tab_stage(G, rdec, tb, T, s0, s1);
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          const int st = G - (3 + 3 * w);
          if (st >= 0 && st < 4) word_stage(st, rdec, w, wd[w & 1], T, s0, s1, Bnxt);
        }
        if (G < 8) issue_a1(s + 1, Anxt, G);
        else if (G < 11) load_w1(s + 2, rload, G - 8);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, SLICE_V1, 0);    // VALU
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);                 // LDS read
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);                 // LDS write
        __builtin_amdgcn_sched_group_barrier(0x010, 2, 0);                 // global load
        __builtin_amdgcn_sched_group_barrier(0x002, 32, 0);                // VALU
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  const int steps = (int)((p.R + BKS - 1) / BKS);
  WRaw r0, r1;
  issue_a(0, As0, 0);
  issue_a(0, As0, 1);
  load_w(0, r0);
  {
    RunTable T;
    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
    for (int part = 0; part < 4; ++part) decode_part(r0, Bs0, T, s0, s1, part);
  }
  load_w(1, r1);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // the main loop with IA active row blocks (every wave meets the same
  // barriers whatever its IA)
  auto main_loop = [&](auto ia) __attribute__((always_inline)) {
    constexpr int IA = decltype(ia)::value;
    read_af(As0, 0, afa, IA);
    if (IA > 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) bf[j] = read_bf(Bs0, 0, j);
    }
    int s = 0;
    for (; s + 2 <= steps; s += 2) {
      step_s(ia, s, As0, Bs0, As1, Bs1, r1, r0);
      step_s(ia, s + 1, As1, Bs1, As0, Bs0, r0, r1);
    }
    if (s < steps) step_s(ia, s, As0, Bs0, As1, Bs1, r1, r0);
  };
  // A tile with at most 64 rows (the last tile of an expert's rows, or of M)
  // keeps the full-tile schedule, but only its first two row blocks compute:
  // the waves of rows 128.. skip every MFMA, those of rows 0.. skip half.
  if (row_end - row0 <= 64) {
    if (wm0 == 0) main_loop(std::integral_constant<int, 2>{});
    else main_loop(std::integral_constant<int, 0>{});
  } else {
    main_loop(std::integral_constant<int, 4>{});
  }
  // the look-ahead loads past the end still write (zeros) into the stages,
  // and the last step's prefetch reads the stage the tail reuses
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // ---- rank-r tail: dZ A, plain bf16 steps through LDS -----------------------
  // Where the row tiles ignore the groups (one base for several adapters),
  // the tile's groups run as one block-diagonal product (big::TileGroups):
  // reduction row k is row k - i rp of the tile's group i. Each step ends
  // with a barrier, so the stages are free again.
  if (p.r2 > 0) {
    const bool a_vec = (p.A2.ld % 8) == 0;
    const bool b_vec = (p.B2.ld % 8) == 0;
    const int64_t row_hi = min(row0 + BM, row_end);
    big::TileGroups tg{g, 1, p.r2};
    int my = 0;
    if constexpr (SHARED) {
      tg = big::tile_groups(p, row0, row_hi);
      my = big::row_group(p, tg, row0 + t, row_hi);
    }
    const int rc = tg.n * tg.rp;   // reduction length
    for (int k0 = 0; k0 < rc; k0 += BKS) {
      if constexpr (SHARED)
        if (big::cols_empty(p, tg, k0, BKS, row0, row_hi)) continue;
      if (p.A2part) {
        big::a2_parts_to_lds<SHARED>(p, As0, [](int i, int c) { return swz(i, c); }, row0, row_hi, k0, t, col0 == 0,
                                     tg.rp, my);
      } else if constexpr (SHARED) {
        big::a2_rows_to_lds(p, As0, [](int i, int c) { return swz(i, c); }, row0, row_hi, k0, t, tg.rp, my);
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int idx = t + THREADS * c;
          const int row = idx >> 3, chunk = idx & 7;
          u32x4_t v = {0u, 0u, 0u, 0u};
          const int64_t gr = row0 + row;
          const int64_t gk = k0 + chunk * 8;
          if (gr < row_end && gk < p.r2) {
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
          lds_write_b128(As0 + swz(row, chunk), v);
        }
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int idx = t + THREADS * c;
        const int row = idx >> 5, cc = (idx & 31) * 8;
        u32x4_t v = {0u, 0u, 0u, 0u};
        const int kr = k0 + row;
        int gi = 0;
        if constexpr (SHARED) gi = kr / tg.rp;
        const int64_t gr = kr - gi * tg.rp;
        const int64_t gc = col0 + cc;
        if (kr < rc && gr < p.r2 && gc < p.Nc) {
          const uint16_t *src = p.B2.p + (tg.g0 + gi) * p.B2.gstride + gr * p.B2.ld + gc;
          if (b_vec && gc + 8 <= p.Nc) {
            v = *reinterpret_cast<const u32x4_t *>(src);
          } else {
            uint32_t w4[4] = {0u, 0u, 0u, 0u};
            for (int e = 0; e < 8; ++e)
              if (gc + e < p.Nc) w4[e >> 1] |= (uint32_t)src[e] << (16 * (e & 1));
            v = u32x4_t{w4[0], w4[1], w4[2], w4[3]};
          }
        }
        lds_write_b128(Bs0 + wt_off(row, cc), v);
      }
      __syncthreads();
      // sub-step kk covers reduction rows k0 + 16 kk .. +15: only those below rc
      compute_step(As0, Bs0, min(4, (rc - k0 + 15) / 16));
      __syncthreads();
    }
  }

  // ---- epilogue: register e of acc[j][i] holds
  // dX[wm0 + 32 i + lane % 32][wn0 + 32 j + 8 (e / 4) + 4 (lane / 32) + e % 4].
  // Each wave stages its 128 x 128 bf16 block in LDS (free now; 32 KB per
  // wave, 256-byte rows, chunk c of row r at c ^ (r % 16)) and writes it back
  // as 4 whole 256-byte row segments per store instruction (element stores
  // where a segment is cut by the output's edge or rows are not 16-byte
  // aligned).
  {
    uint16_t *stg = smem + wave * (128 * 128);
    auto st_off = [](int row, int chunk) { return row * 128 + ((chunk ^ (row & 15)) << 3); };
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const u32x2_t pk = {pack_bf16x2(acc[j][i][4 * r4], acc[j][i][4 * r4 + 1]),
                              pack_bf16x2(acc[j][i][4 * r4 + 2], acc[j][i][4 * r4 + 3])};
          *reinterpret_cast<u32x2_t *>(stg + st_off(i * 32 + l32, 4 * j + r4) + 4 * h) = pk;
        }
    const bool vec16 = (p.ldc % 8) == 0;
#pragma unroll 4
    for (int q = 0; q < 32; ++q) {
      const int row = q * 4 + (lane >> 4), chunk = lane & 15;
      const u32x4_t v = lds_read_b128(stg + st_off(row, chunk));
      const int64_t grow = row0 + wm0 + row;
      const int64_t gcol = col0 + wn0 + chunk * 8;
      if (grow < row_end && gcol < p.Nc) {
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

}  // namespace dgrad
}  // namespace lora4
