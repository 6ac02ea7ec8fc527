// Forward dequant-GEMM with the base dequantized straight into MFMA registers:
//
//   Y[M, N] = X[M, K] . deq(W)[N, K]^T  (+ (s Z)[M, r] . B[N, r]^T tail)
//
// One workgroup = 4 waves computing a 256 x 256 tile of Y. Wave w owns output
// columns 64 w .. 64 w + 63 for all 256 rows (8 x 2 blocks of 32 x 32, 256
// fp32 accumulators per lane on v_mfma_f32_32x32x16_bf16), so every row of W
// in the tile is needed by exactly one wave and deq(W) never touches LDS: each
// lane loads 32 packed codes (16 bytes) of each of its two rows per step,
// decodes them one step ahead in registers, and feeds them to the MFMA as the
// first operand. The order of the reduction inside a 64-deep step is chosen so
// that this works: in sub-step kk (16 deep), lane half h (lanes 32 h ..)
// supplies elements k = 32 h + 8 kk .. +7 of its row, i.e. a lane's operands
// over a step are 32 consecutive elements of one row. X is read from LDS in
// the same order, so every product pairs the same k on both sides.
//
// Outputs with too few tiles to fill the GPU, and the tiles of an
// under-filled last round, split their reduction over several blocks (fp32
// partials per tile, summed by k_reduce_tiles in a fixed order).
//
// X streams HBM/L2 -> LDS (swizzled so the operand reads are free of bank
// conflicts) with bounds-checked direct loads into a ring of
// five buffers of 256 x 64 (the X of step s+3 and the W of step s+2 are
// loaded while step s computes, spread evenly over its sub-steps so that the
// address units never back up and stall the issuing wave); one bare barrier
// per step, in mid-step. All look-ahead loads are issued unconditionally
// (past the end they are out of range and return zeros), so the number of
// loads in flight at each wait is a constant. The main loop is unrolled twice
// so that the two sets of look-ahead registers swap roles instead of being
// copied (a copy would wait for loads still in flight). The work between the
// MFMAs (decode stages, table builds, global loads) is dealt to the MFMA pairs
// by hand, one slice per pair, fenced so the compiler keeps it there.
//
// NF4 runs decode through a 16-entry bf16 table bf16(q[i] * c) selected with
// v_perm_b32, MXFP4 through v_cvt_scalef32_pk_bf16_fp4; NF4-DQ rebuilds
// c = E4M3(code) * c2 first.
#pragma once

#include "gemm_big.hpp"

namespace lora4 {
namespace fwd {

using big::OOB;
using big::Params;
using big::RunTable;
using big::rsrc_t;

// VALU instructions placed between the two MFMAs of a pair in the hand-dealt
// sub-steps (the rest of the pair's slice follows its LDS read and loads).
constexpr int SLICE_V1 = 5;

constexpr int BM = 256, BN = 256, BKS = 64, THREADS = 256, STAGES = 5;
constexpr int TILE = BM * BKS;   // one X stage, bf16 elements

__host__ __device__ constexpr int lds_bytes() { return STAGES * TILE * 2; }

__device__ __forceinline__ int swz(int row, int chunk) { return tile64_swz(row, chunk); }

// Decoded operands of one lane for one step: row j (two 32-row blocks), four
// sub-steps of 8 bf16 (k = 32 h + 8 kk .. +7 of the lane's row).
struct WFrag {
  u32x4_t w[2][4];
};

// Raw loads of one lane for one step (two rows).
struct WRaw {
  u32x4_t c[2];
  uint32_t sc[2];   // NF4: fp32 bits; DQ: e4m3 code; MXFP4: e8m0 code
  uint32_t c2[2];   // DQ second level (fp32 bits)
};

// One output tile of TBM rows x 128 NJ columns: wave w owns the 32 NJ columns
// from col0 + 32 NJ w (NJ 32-column blocks) for all TBM rows (TBM / 32 row
// blocks). SPLIT (TBM 256, NJ 2 only): the block computes reduction range
// `split` of the tile and writes fp32 partials. SHARED: the row tiles ignore
// the groups (Params::shared_rows). `tile` is the tile's index in the split
// partials. rt: the tile's rows (from the slot's 256-row tile; a short last
// tile of a group runs with TBM 64 or 128 over the same rows).
template <int FMT, bool SPLIT, bool SHARED, int TBM, int NJ>
__device__ __forceinline__ void fwd_tile(const Params &p, uint16_t *smem, const RowTile &rt, int64_t col0, int tile,
                                         int split) {
  static_assert(!SPLIT || (TBM == BM && NJ == 2), "split partials are laid out for 256 x 256 tiles");
  constexpr int RB = TBM / 32;       // 32-row blocks: MFMA row blocks per wave, X chunks per step
  constexpr int WN = 32 * NJ;        // columns per wave
  constexpr int CPS = 8 / RB;        // hand-dealt slices per MFMA row block (8 slices per sub-step)
  constexpr bool is_split = SPLIT;
  if (rt.group < 0) return;
  const int g = rt.group;
  const int64_t row0 = rt.row0, row_end = rt.row_end;

  const int t = threadIdx.x;
  // the wave index is uniform: keep it (and the LDS addresses derived from
  // it) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63;
  const int l32 = lane & 31, h = lane >> 5;
  // NF4 table build: this lane's half of the levels (see make_table_pair)
  const uint32_t sel = big::sel_base();
  float qh[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) qh[i] = h ? p.tab.q[8 + i] : p.tab.q[i];

  // ---- X: direct loads into the LDS ring ------------------------------------
  // wave w, chunk c covers tile rows 8 (4 c + w) .. +7; lane l: row + l / 8,
  // stored chunk position l % 8 (tile64 layout).
  const rsrc_t a_rsrc = big::make_rsrc(p.A.p + row0 * p.A.ld, big::clamp_bytes((row_end - row0) * p.A.ld * 2));
  // chunk c is 32 rows below chunk 0: offsets a_voff0 + c * a_cstep
  const int a_kq = tile64_dma_chunk(lane, wave) * 8;
  const uint32_t a_voff0 = (uint32_t)(((wave * 8 + (lane >> 3)) * p.A.ld + a_kq) * 2);
  const uint32_t a_cstep = (uint32_t)(32 * p.A.ld * 2);
  // X of step s into stage As, chunks 2 part .. 2 part + 1 (part 0..3)
  // steps are numbered within this block's range, which starts at step sb
  const int sb = is_split ? split * p.split_steps : 0;
  const int Ri = (int)p.R;   // < 2^31 (the buffer offsets are 32-bit)
  auto issue_a = [&](int s, uint16_t *As, int part) {
    const int k0 = (s + sb) * BKS;
    const bool edge = k0 + a_kq >= Ri;
#pragma unroll
    for (int c = 2 * part; c < 2 * part + 2 && c < RB; ++c)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (__attribute__((address_space(3))) void *)(As + (c * 4 + wave) * 512),
                                               16, edge ? OOB : a_voff0 + c * a_cstep, (int)(k0 * 2), 0, 0);
  };

  // ---- this lane's W rows: n = wcol0 + 32 j + l32, k = 32 h + .. ----------
  // The wave's WN rows lie in one row block of the tiled base (from row i0 of
  // it): per step it reads tile (rb, k0 / 64), its rows' 32 contiguous bytes of
  // codes each (row i at 32 i) and their scale entries. Row blocks past the
  // base read nothing (out-of-range descriptor).
  const int64_t KB = p.W.KB;
  const int64_t wcol0 = col0 + (int64_t)wave * WN;
  const int64_t rb = wcol0 >> 6;
  const int i0 = (int)(wcol0 & 63);
  const bool rb_ok = rb < w_blocks(p.W.N);
  const int gw = w_group(p.W, g);   // group of W
  const uint8_t *codes_g = p.W.codes + gw * p.W.g_codes;
  const rsrc_t w_rsrc = big::make_rsrc(rb_ok ? codes_g + rb * KB * 2048 : codes_g,
                                       rb_ok ? big::clamp_bytes(KB * 2048) : 0u);
  constexpr int sc_bytes = FMT == FMT_NF4 ? 4 : 1;
  constexpr int sc_tile = FMT == FMT_MXFP4 ? 128 : FMT == FMT_NVFP4 ? 256 : 64 * sc_bytes;   // scale bytes per tile
  const uint8_t *sbase = reinterpret_cast<const uint8_t *>(p.W.scales) + (gw * p.W.g_scales) * sc_bytes;
  const rsrc_t s_rsrc = big::make_rsrc(rb_ok ? sbase + rb * KB * sc_tile : sbase,
                                       rb_ok ? big::clamp_bytes(KB * sc_tile) : 0u);
  const rsrc_t s2_rsrc = FMT == FMT_NF4_DQ
                             ? big::make_rsrc(p.W.scales2 + gw * p.W.g_scales2, big::clamp_bytes(p.W.g_scales2 * 4))
                             : big::make_rsrc(p.W.codes, 0u);
  uint32_t w_voff[2], s_voff[2];
  int64_t s_idx0[2];   // DQ: row-major index of the row's first 64-run scale
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int i = i0 + j * 32 + l32;   // row inside the row block
    w_voff[j] = (uint32_t)(i * 32 + h * 16);
    s_voff[j] = (uint32_t)(FMT == FMT_MXFP4 ? i * 2 + h : FMT == FMT_NVFP4 ? i * 4 + h * 2 : i * sc_bytes);
    s_idx0[j] = (wcol0 + j * 32 + l32) * (p.W.K >> 6);
  }
  // per-step offsets of tile (rb, k0 / 64)
  auto w_step_off = [](int k0) { return (int)((k0 >> 6) << 11); };
  auto s_step_off = [](int k0) { return (int)((k0 >> 6) * sc_tile); };

  // W of step s, part 0..3: part j < 2 loads row j's codes and scale (with
  // its second-level scale for NF4-DQ); parts 2 and 3 load nothing, so every
  // W load of a step is issued in its first half, a full step ahead of use
  auto load_w = [&](int s, WRaw &w, int part) {
    if (part >= NJ) return;
    const int k0 = (s + sb) * BKS;
    // this lane's half lies inside the row (MXFP4 rows may end at k % 64 == 32)
    const bool half_ok = k0 + 32 * h < Ri;
    const int j = part;
    w.c[j] = __builtin_bit_cast(
        u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, half_ok ? w_voff[j] : OOB, w_step_off(k0), 0));
    if constexpr (FMT == FMT_NF4) {
      w.sc[j] = __builtin_amdgcn_raw_buffer_load_b32(s_rsrc, half_ok ? s_voff[j] : OOB, s_step_off(k0), 0);
    } else if constexpr (FMT == FMT_NF4_DQ) {
      w.sc[j] = __builtin_amdgcn_raw_buffer_load_b8(s_rsrc, half_ok ? s_voff[j] : OOB, s_step_off(k0), 0);
      const int64_t gi = (s_idx0[j] + (int64_t)(k0 >> 6)) >> 8;
      w.c2[j] = __builtin_amdgcn_raw_buffer_load_b32(s2_rsrc, half_ok ? (uint32_t)(gi * 4) : OOB, 0, 0);
    } else if constexpr (FMT == FMT_NVFP4) {   // the lane half's two E4M3 scales
      w.sc[j] = __builtin_amdgcn_raw_buffer_load_b16(s_rsrc, half_ok ? s_voff[j] : OOB, s_step_off(k0), 0);
    } else {
      w.sc[j] = __builtin_amdgcn_raw_buffer_load_b8(s_rsrc, half_ok ? s_voff[j] : OOB, s_step_off(k0), 0);
    }
  };
  // loads issued by load_w over a whole step, all in parts 0 .. NJ - 1
  // (issued unconditionally, so the count is exact)
  constexpr int W_LOADS = (FMT == FMT_NF4_DQ ? 3 : 2) * NJ;

  // Decode state of one row's run for a step: the NF4 table (shared by the
  // lane pair, see make_table_pair) or the MXFP4 scale. It is built a
  // sub-step or more before the run's words are decoded, so that the decode
  // instructions never wait on the table's own chain.
  struct RunDec {
    RunTable T;
    float sc;
    float sc2;   // NVFP4: scale of code words 2, 3 (sc: words 0, 1)
  };
  auto make_run = [&](const WRaw &w, int j) -> RunDec {
    RunDec d{};
    if constexpr (FMT == FMT_MXFP4) {
      d.sc = e8m0_to_f32(w.sc[j] & 0xFFu);
    } else if constexpr (FMT == FMT_NVFP4) {
      d.sc = e4m3_to_f32(w.sc[j] & 0xFFu);
      d.sc2 = e4m3_to_f32((w.sc[j] >> 8) & 0xFFu);
    } else {
      float c;
      if constexpr (FMT == FMT_NF4) c = __builtin_bit_cast(float, w.sc[j]);
      else c = e4m3_to_f32(w.sc[j] & 0xFFu) * __builtin_bit_cast(float, w.c2[j]);
      d.T = big::make_table_pair(c, qh, sel);
    }
    return d;
  };
  // decode code words q0, q0 + 1 of row j of raw w into f
  auto decode_words = [&](const WRaw &w, WFrag &f, const RunDec &d, int j, int q0) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int q = q0 + e;
      if constexpr (FMT == FMT_MXFP4)
        f.w[j][q] = big::decode8_mxfp4(w.c[j][q], d.sc);
      else if constexpr (FMT == FMT_NVFP4)
        f.w[j][q] = decode8_nvfp4(w.c[j][q], q < 2 ? d.sc : d.sc2);
      else
        f.w[j][q] = big::decode8_nf4(d.T, w.c[j][q]);
    }
  };

  // acc[i][j]: rows 32 i .. +31, columns WN wave + 32 j .. +31
  f32x16_t acc[RB][NJ];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16_t{};

  // At the mid-step wait of step s, the X of step s+1 (issued during step
  // s-2) must have landed; still in flight may be everything issued during
  // step s-1 and during sub-steps 0 and 1 of step s (X chunks go out two per
  // sub-step from sub-step 0, W loads in sub-steps 0 .. NJ - 1). lgkmcnt 0 as
  // well.
  constexpr int VM_OUT = (RB + W_LOADS) + ((RB < 4 ? RB : 4) + W_LOADS);
  static_assert(VM_OUT < 64, "vmcnt field");
  constexpr int VMCNT = (VM_OUT & 15) | (7 << 4) | (0 << 8) | ((VM_OUT >> 4) << 14);

  // Sub-step kk of a step: 16 MFMAs on fragments x (chunk kk of the step's X
  // stage); fragment i is reloaded as soon as its two MFMAs have issued, from
  // chunk kk+1, or for kk == 3 from chunk 0 of the next step's stage, so the
  // LDS latency is always a sub-step ahead. hook() holds this sub-step's share
  // of the VALU work (decode) and of the global loads. The schedule is pinned:
  // MFMA pairs with the LDS read of the freed fragment, a global load every
  // other pair, and VALU work between them; nothing moves across sub-steps.
  auto sub_step = [&](const WFrag &cur, int kk, u32x4_t x[RB], const uint16_t *src, int chunk, bool reload,
                      auto &&hook) {
#pragma unroll
    for (int i = 0; i < RB; ++i) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = mfma_32x32x16(cur.w[j][kk], x[i], acc[i][j]);
      if (reload) x[i] = lds_read_b128(src + swz(i * 32 + l32, chunk));
    }
    hook();
#pragma unroll
    for (int i = 0; i < RB; ++i) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, big::SCHED_VALU, 0);   // VALU
      }
      if (reload) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // LDS read
      if (i & 1) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);       // global load
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- the same step with its VALU and load work dealt out by hand: every
  // MFMA pair of a sub-step gets one slice (a stage of a code word's decode,
  // of a table build, or one global load), fenced so that nothing moves
  // between pairs.
  struct WordDec {
    uint32_t i0, i1, L0, H0, L1, H1;   // i0, i1: lookup indices of elements 0..3 (big::nf4_idx)
  };
  struct RunBuild {
    float c;
    float pr[8];
  };
  // X of step s, chunk c (0..7) of stage As
  auto issue_a1 = [&](int s, uint16_t *As, int c) {
    const int k0 = (s + sb) * BKS;
    const bool edge = k0 + a_kq >= Ri;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (__attribute__((address_space(3))) void *)(As + (c * 4 + wave) * 512),
                                             16, edge ? OOB : a_voff0 + c * a_cstep, (int)(k0 * 2), 0, 0);
  };
  // W of step s, row j: scale (and NF4-DQ second-level scale), then codes
  auto load_w_scale = [&](int s, WRaw &w, int j) {
    const int k0 = (s + sb) * BKS;
    const bool half_ok = k0 + 32 * h < Ri;
    if constexpr (FMT == FMT_NF4) {
      w.sc[j] = __builtin_amdgcn_raw_buffer_load_b32(s_rsrc, half_ok ? s_voff[j] : OOB, s_step_off(k0), 0);
    } else if constexpr (FMT == FMT_NF4_DQ) {
      w.sc[j] = __builtin_amdgcn_raw_buffer_load_b8(s_rsrc, half_ok ? s_voff[j] : OOB, s_step_off(k0), 0);
      const int64_t gi = (s_idx0[j] + (int64_t)(k0 >> 6)) >> 8;
      w.c2[j] = __builtin_amdgcn_raw_buffer_load_b32(s2_rsrc, half_ok ? (uint32_t)(gi * 4) : OOB, 0, 0);
    } else if constexpr (FMT == FMT_NVFP4) {   // the lane half's two E4M3 scales
      w.sc[j] = __builtin_amdgcn_raw_buffer_load_b16(s_rsrc, half_ok ? s_voff[j] : OOB, s_step_off(k0), 0);
    } else {
      w.sc[j] = __builtin_amdgcn_raw_buffer_load_b8(s_rsrc, half_ok ? s_voff[j] : OOB, s_step_off(k0), 0);
    }
  };
  auto load_w_codes = [&](int s, WRaw &w, int j) {
    const int k0 = (s + sb) * BKS;
    const bool half_ok = k0 + 32 * h < Ri;
    w.c[j] = __builtin_bit_cast(
        u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, half_ok ? w_voff[j] : OOB, w_step_off(k0), 0));
  };
  // slice i of decoding words q0, q0 + 1 of row j of w into f
  auto dec_slice = [&](int i, const WRaw &w, WFrag &f, const RunDec &d, int j, int q0, WordDec (&wd)[2]) {
    if constexpr (FMT == FMT_NVFP4) {
      // one bf16 pair per slice: convert at scale 1, multiply by the E4M3 scale
      const int q = q0 + (i >> 2);
      const float sc = q0 == 0 ? d.sc : d.sc2;
      uint32_t v;
      switch (i & 3) {
        case 0: v = nvfp4_pair_t<0>(w.c[j][q], sc); break;
        case 1: v = nvfp4_pair_t<1>(w.c[j][q], sc); break;
        case 2: v = nvfp4_pair_t<2>(w.c[j][q], sc); break;
        default: v = nvfp4_pair_t<3>(w.c[j][q], sc); break;
      }
      f.w[j][q][i & 3] = v;
    } else if constexpr (FMT == FMT_MXFP4) {
      // one conversion (a bf16 pair) per slice
      const int q = q0 + (i >> 2);
      uint32_t v;
      switch (i & 3) {
        case 0: v = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w.c[j][q], d.sc, 0)); break;
        case 1: v = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w.c[j][q], d.sc, 1)); break;
        case 2: v = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w.c[j][q], d.sc, 2)); break;
        default: v = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w.c[j][q], d.sc, 3)); break;
      }
      f.w[j][q][i & 3] = v;
    } else {
      // stages of a word: indices of elements 0..3; their lookup; indices
      // and lookup of elements 4..7 (from the code word); the interleave
      auto hi_half = [&](uint32_t c, WordDec &o) {
        uint32_t i7, s3;
        big::nf4_idx<1>(d.T, c, i7, s3);
        big::lookup4(d.T, i7, s3, o.L1, o.H1);
      };
      auto fin = [](const WordDec &o) -> u32x4_t {
        return u32x4_t{big::pair_lo(o.L0, o.H0), big::pair_hi(o.L0, o.H0), big::pair_lo(o.L1, o.H1),
                       big::pair_hi(o.L1, o.H1)};
      };
      switch (i) {
        case 0: big::nf4_idx<0>(d.T, w.c[j][q0], wd[0].i0, wd[0].i1); break;
        case 1: big::lookup4(d.T, wd[0].i0, wd[0].i1, wd[0].L0, wd[0].H0); break;
        case 2: hi_half(w.c[j][q0], wd[0]); break;
        case 3:
          f.w[j][q0] = fin(wd[0]);
          big::nf4_idx<0>(d.T, w.c[j][q0 + 1], wd[1].i0, wd[1].i1);
          break;
        case 4: big::lookup4(d.T, wd[1].i0, wd[1].i1, wd[1].L0, wd[1].H0); break;
        case 5: hi_half(w.c[j][q0 + 1], wd[1]); break;
        case 6: f.w[j][q0 + 1] = fin(wd[1]); break;
        default: break;
      }
    }
  };
  // slice i of building the decode state of row j of w into out
  auto run_slice = [&](int i, const WRaw &w, int j, RunBuild &rb, RunDec &out) {
    if constexpr (FMT == FMT_MXFP4) {
      if (i == 7) out.sc = e8m0_to_f32(w.sc[j] & 0xFFu);
    } else if constexpr (FMT == FMT_NVFP4) {
      if (i == 6) out.sc = e4m3_to_f32(w.sc[j] & 0xFFu);
      if (i == 7) out.sc2 = e4m3_to_f32((w.sc[j] >> 8) & 0xFFu);
    } else {
      if (i == 0) {
        if constexpr (FMT == FMT_NF4) rb.c = __builtin_bit_cast(float, w.sc[j]);
        else rb.c = e4m3_to_f32(w.sc[j] & 0xFFu) * __builtin_bit_cast(float, w.c2[j]);
#pragma unroll
        for (int k = 0; k < 4; ++k) rb.pr[k] = qh[k] * rb.c;
      } else if (i == 6) {
#pragma unroll
        for (int k = 4; k < 8; ++k) rb.pr[k] = qh[k] * rb.c;
      } else if (i == 7) {
        uint32_t t4[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) t4[k] = pack_bf16x2(rb.pr[2 * k], rb.pr[2 * k + 1]);
        out.T = big::table_pair_from(t4, sel);
      }
    }
  };
  // (a row block's MFMAs carry CPS consecutive slices of the sub-step's 8,
  // so the work dealt per step is the same for every tile shape)
  auto sub_step_s = [&](const WFrag &cur, int kk, u32x4_t x[RB], const uint16_t *src, int chunk, auto &&slice) {
#pragma unroll
    for (int i = 0; i < RB; ++i) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = mfma_32x32x16(cur.w[j][kk], x[i], acc[i][j]);
      x[i] = lds_read_b128(src + swz(i * 32 + l32, chunk));
#pragma unroll
      for (int c = 0; c < CPS; ++c) slice(i * CPS + c);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, SLICE_V1, 0);          // VALU
      if (NJ > 1) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                 // LDS read
      __builtin_amdgcn_sched_group_barrier(0x010, 2 * CPS, 0);           // global load
      __builtin_amdgcn_sched_group_barrier(0x002, 32 * CPS, 0);          // VALU
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto body_s = [&](int s, const uint16_t *cur, const uint16_t *nxt, uint16_t *ahead, const WRaw &rdec,
                    WRaw &rload, const WFrag &fcur, WFrag &fnxt, u32x4_t x[RB], RunDec &d0) {
    RunDec d1{};
    RunBuild rb;
    WordDec wd[2];
    // X chunks c < RB of step s + 3 go out two per sub-step, from sub-step 0
    auto x_chunk = [&](int c) {
      if (c < RB) issue_a1(s + 3, ahead, c);
    };
    sub_step_s(fcur, 0, x, cur, h * 4 + 1, [&](int i) {
      dec_slice(i, rdec, fnxt, d0, 0, 0, wd);
      if (i == 0) load_w_scale(s + 2, rload, 0);
      if (i == 2) x_chunk(0);
      if (i == 4) load_w_codes(s + 2, rload, 0);
      if (i == 6) x_chunk(1);
    });
    sub_step_s(fcur, 1, x, cur, h * 4 + 2, [&](int i) {
      dec_slice(i, rdec, fnxt, d0, 0, 2, wd);
      if (NJ > 1) run_slice(i, rdec, 1, rb, d1);
      if (NJ > 1 && i == 0) load_w_scale(s + 2, rload, 1);
      if (i == 2) x_chunk(2);
      if (NJ > 1 && i == 4) load_w_codes(s + 2, rload, 1);
      if (i == 6) x_chunk(3);
    });
    __builtin_amdgcn_s_waitcnt(VMCNT);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    sub_step_s(fcur, 2, x, cur, h * 4 + 3, [&](int i) {
      if (NJ > 1) dec_slice(i, rdec, fnxt, d1, 1, 0, wd);
      if (i == 2) x_chunk(4);
      if (i == 6) x_chunk(5);
    });
    sub_step_s(fcur, 3, x, nxt, h * 4 + 0, [&](int i) {
      if (NJ > 1) dec_slice(i, rdec, fnxt, d1, 1, 2, wd);
      run_slice(i, rload, 0, rb, d0);
      if (i == 2) x_chunk(6);
      if (i == 6) x_chunk(7);
    });
  };

  const int all_steps = (int)((p.R + BKS - 1) / BKS);
  const int steps = is_split ? min(all_steps - sb, p.split_steps) : all_steps;
  WRaw r0, r1;
  WFrag f0, f1;
  u32x4_t x[RB];
  // ring of five stages; step s uses stage s % 5
  auto stage = [&](int i) -> uint16_t * { return smem + (i >= STAGES ? i - STAGES : i) * TILE; };
#pragma unroll
  for (int part = 0; part < 4; ++part) {
    issue_a(0, stage(0), part);
    issue_a(1, stage(1), part);
    issue_a(2, stage(2), part);
    load_w(0, r0, part);
  }
  // ---- rank-r product (s Z) B^T first, into the zeroed accumulators: Z rows
  // through LDS stage 4 (free until step 1 refills it), B rows to registers.
  // Its operand loads are issued right behind the first X and W loads, so
  // their latency overlaps. (Sub-steps whose reduction slots all lie past r2
  // are skipped: in sub-step kk lane half h holds k0 + 32 h + 8 kk ..)
  // Where the row tiles ignore the groups (one base for several adapters),
  // the tile's groups run as one block-diagonal product (big::TileGroups):
  // reduction column k is column k - i rp of the tile's group i.
  if (p.r2 > 0 && split == 0) {
    uint16_t *As = stage(4);
    const bool a_vec = (p.A2.ld % 8) == 0;
    const bool b_vec = (p.B2.ld % 8) == 0;
    const int64_t row_hi = min(row0 + TBM, row_end);
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
      const int nkk = min(4, (rc - k0 + 7) / 8);
      WFrag bt;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int64_t n = wcol0 + j * 32 + l32;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int kc = k0 + 32 * h + 8 * kk;
          int gi = 0;
          if constexpr (SHARED) gi = kc / tg.rp;
          const int64_t k = kc - gi * tg.rp;
          uint32_t w4[4] = {0u, 0u, 0u, 0u};
          if (kk < nkk && n < p.Nc && kc < rc && k < p.r2) {
            const uint16_t *src = p.B2.p + (tg.g0 + gi) * p.B2.gstride + n * p.B2.ld + k;
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
          bt.w[j][kk] = u32x4_t{w4[0], w4[1], w4[2], w4[3]};
        }
      }
      if (p.A2part) {
        if (t < TBM)
          big::a2_parts_to_lds<SHARED>(p, As, [](int i, int c) { return swz(i, c); }, row0, row_hi, k0, t,
                                       col0 == 0, tg.rp, my);
      } else if constexpr (SHARED) {
        if (t < TBM) big::a2_rows_to_lds(p, As, [](int i, int c) { return swz(i, c); }, row0, row_hi, k0, t, tg.rp, my);
      } else {
#pragma unroll
        for (int c = 0; c < RB; ++c) {
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
          lds_write_b128(As + swz(row, chunk), v);
        }
      }
      __syncthreads();
      u32x4_t xt[RB];
#pragma unroll
      for (int i = 0; i < RB; ++i) xt[i] = lds_read_b128(As + swz(i * 32 + l32, h * 4));
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        if (kk < nkk) sub_step(bt, kk, xt, As, h * 4 + kk + 1, kk < 3, [] {});
      if (k0 + BKS < rc) __syncthreads();   // before the next chunk restages
    }
  }

#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const RunDec d = make_run(r0, j);
    decode_words(r0, f0, d, j, 0);
    decode_words(r0, f0, d, j, 2);
  }
#pragma unroll
  for (int part = 0; part < 4; ++part) load_w(1, r1, part);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  RunDec d0 = make_run(r1, 0);
#pragma unroll
  for (int i = 0; i < RB; ++i) x[i] = lds_read_b128(stage(0) + swz(i * 32 + l32, h * 4));
  int s = 0, si = 0;   // si = s % 5
  for (; s + 2 <= steps; s += 2) {
    body_s(s, stage(si), stage(si + 1), stage(si + 3), r1, r0, f0, f1, x, d0);
    body_s(s + 1, stage(si + 1), stage(si + 2), stage(si + 4), r0, r1, f1, f0, x, d0);
    si = si + 2 >= STAGES ? si + 2 - STAGES : si + 2;
  }
  if (s < steps) body_s(s, stage(si), stage(si + 1), stage(si + 3), r1, r0, f0, f1, x, d0);
  // the look-ahead loads past the end still write (zeros) into the ring, which
  // the epilogue reuses
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // ---- epilogue: register e of acc[i][j] holds
  // Y[32 i + lane % 32][64 wave + 32 j + 8 (e / 4) + 4 (lane / 32) + e % 4]
  if constexpr (SPLIT) {
    // fp32 partial of this range, tile-local [256][256] (rows and columns past
    // the output are written too and ignored by the reduction)
    float *pt = p.Cpart + ((int64_t)tile * p.ksplit + split) * (BM * BN);
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      float *prow = pt + (i * 32 + l32) * BN;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int col = wave * 64 + j * 32 + r4 * 8 + h * 4;
          *reinterpret_cast<f32x4_t *>(prow + col) =
              f32x4_t{acc[i][j][4 * r4], acc[i][j][4 * r4 + 1], acc[i][j][4 * r4 + 2], acc[i][j][4 * r4 + 3]};
        }
      }
    }
    return;
  }
  // Each wave stages its TBM x WN bf16 block in LDS (free now; tile64 layout,
  // chunks 0 .. 4 NJ - 1 of each row) and writes it back as whole row
  // segments of 16 NJ lanes per store instruction (element stores where a
  // row segment is cut by the output's edge or the rows are not 16-byte
  // aligned).
  {
    constexpr int CH = 4 * NJ;           // 16-byte chunks per staged row
    constexpr int RPI = 64 / CH;         // rows per store instruction
    uint16_t *stg = smem + wave * (TBM * 64);
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const u32x2_t pk = {pack_bf16x2(acc[i][j][4 * r4], acc[i][j][4 * r4 + 1]),
                              pack_bf16x2(acc[i][j][4 * r4 + 2], acc[i][j][4 * r4 + 3])};
          *reinterpret_cast<u32x2_t *>(stg + tile64_swz(i * 32 + l32, 4 * j + r4) + 4 * h) = pk;
        }
    const bool vec16 = (p.ldc % 8) == 0;
#pragma unroll 4
    for (int q = 0; q < TBM / RPI; ++q) {
      const int row = q * RPI + lane / CH, chunk = lane % CH;
      const u32x4_t v = lds_read_b128(stg + tile64_swz(row, chunk));
      const int64_t grow = row0 + row;
      const int64_t gcol = wcol0 + chunk * 8;
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

// SHORT: a whole 256-row tile whose rows end within 64 (128) rows of its start
// runs with 64 (128) row tiles' code: 2 (4) of the 8 row blocks of MFMAs, the
// same W decode. (The last tile of an expert's rows is often short.) Only the
// grouped launches take it: the kernels sit at 254-255 of 256 VGPRs, and with
// the extra paths the MXFP4 one spills 3 registers.
template <int FMT, bool SHARED, bool SHORT>
__device__ __forceinline__ void fwd_whole_tile(const Params &p, uint16_t *smem, const RowTile &rt, int64_t col0,
                                               int tile) {
  if (rt.group < 0) return;
  const int64_t rows = rt.row_end - rt.row0;
  if (SHORT && rows <= 64) fwd_tile<FMT, false, SHARED, 64, 2>(p, smem, rt, col0, tile, 0);
  else if (SHORT && rows <= 128) fwd_tile<FMT, false, SHARED, 128, 2>(p, smem, rt, col0, tile, 0);
  else fwd_tile<FMT, false, SHARED, BM, 2>(p, smem, rt, col0, tile, 0);
}

// Full 256 x 256 tiles (blocks below p.nfull, in grouped tile order, each XCD
// walking a contiguous range of them) and, after them, the last p.ntail tiles
// of that order as two 256 x 128 halves each: when the full tiles leave a
// last round that fills half the GPU or less, its tiles run as twice as many
// half tiles, one round in about half the time. SPLIT: block b computes range
// b % ksplit of tile b / ksplit (no halves). SHORT: see fwd_whole_tile.
template <int FMT, bool SPLIT, bool SHARED, bool SHORT = false>
__global__ __launch_bounds__(THREADS, 1) void k_gemm_fwd(Params p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  int b = blockIdx.x;
  if constexpr (SPLIT) {
    const int tile = b / p.ksplit;
    const int tn = tile % p.tiles_n, slot = tile / p.tiles_n;   // (the reduction of the split tiles uses this order)
    const RowTile rt = big::tile_rows<SHARED>(p, slot, BM);
    fwd_tile<FMT, true, SHARED, BM, 2>(p, smem, rt, (int64_t)tn * BN, tile, b % p.ksplit);
  } else {
    int slot, tn;
    if (b < p.nfull) {
      const int per = p.nfull >> 3;
      if (b < per * 8) b = (b & 7) * per + (b >> 3);
      big::grouped_tile(b, p.tiles_n, p.nslots, slot, tn);
      fwd_whole_tile<FMT, SHARED, SHORT>(p, smem, big::tile_rows<SHARED>(p, slot, BM), (int64_t)tn * BN, b);
    } else {
      int u = b - p.nfull;
      const int per = (2 * p.ntail) >> 3;
      if (u < per * 8) u = (u & 7) * per + (u >> 3);
      big::grouped_tile(p.nfull + (u >> 1), p.tiles_n, p.nslots, slot, tn);
      fwd_tile<FMT, false, SHARED, BM, 1>(p, smem, big::tile_rows<SHARED>(p, slot, BM),
                                          (int64_t)tn * BN + (u & 1) * (BN / 2), 0, 0);
    }
  }
}

// 128 x 128 tiles, for outputs whose 256 x 256 tiles would fill too little of
// the GPU (e.g. 4096 x 1024: 64 tiles, 256 of these). p.tiles_n counts
// 128-column tiles and p.nslots 128-row slots.
template <int FMT, bool SHARED>
__global__ __launch_bounds__(THREADS, 1) void k_gemm_fwd_small(Params p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  int b = blockIdx.x;
  const int per = p.nblocks >> 3;
  if (b < per * 8) b = (b & 7) * per + (b >> 3);
  int slot, tn;
  big::grouped_tile(b, p.tiles_n, p.nslots, slot, tn);
  fwd_tile<FMT, false, SHARED, 128, 1>(p, smem, big::tile_rows<SHARED>(p, slot, 128), (int64_t)tn * 128, b, 0);
}

// C[tile rows][tile columns] = bf16(sum_k part[t][k][r][c]) for the split
// tiles t; four columns per thread, splits summed in order.
__global__ void k_reduce_tiles(Params p, int split_tiles) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_tile = (int64_t)BM * (BN / 4);
  if (idx >= (int64_t)split_tiles * per_tile) return;
  const int t = (int)(idx / per_tile);
  const int rem = (int)(idx - (int64_t)t * per_tile);
  const int r = rem / (BN / 4), c = (rem % (BN / 4)) * 4;
  const int tile = t;
  const int tn = tile % p.tiles_n, slot = tile / p.tiles_n;
  const RowTile rt = p.shared_rows ? big::tile_rows<true>(p, slot, BM) : big::tile_rows<false>(p, slot, BM);
  if (rt.group < 0) return;
  const int64_t row = rt.row0 + r;
  const int64_t col = (int64_t)tn * BN + c;
  if (row >= rt.row_end || col >= p.Nc) return;
  const float *src = p.Cpart + (int64_t)t * p.ksplit * (BM * BN) + r * BN + c;
  f32x4_t s = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < p.ksplit; ++k) s += *reinterpret_cast<const f32x4_t *>(src + (int64_t)k * (BM * BN));
  uint16_t *dst = p.C + row * p.ldc + col;
  if (col + 4 <= p.Nc && (p.ldc % 4) == 0) {
    *reinterpret_cast<u32x2_t *>(dst) = u32x2_t{pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])};
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (col + e < p.Nc) dst[e] = to_bf16(s[e]);
  }
}

}  // namespace fwd
}  // namespace lora4
