// liblora4: the C ABI (include/lora4.h) over the gfx950 kernels.
//
// Host responsibilities: validate every argument before any HIP call, plan
// the split factors and workspace layout, and sequence the kernels on the
// caller's stream:
//
//   forward : Z pass (X A^T, split over K) -> reduce (Z, s Z)
//             -> base GEMM X deq(W)^T with the rank-r tail (s Z) B^T -> Y
//   backward: [Z pass if Z is not given] -> dZ pass (dY B, split over N) ->
//             reduce (s dY B) -> dgrad dY deq(W) with tail dZ A -> dX
//             -> dA = dZ^T X and dB^T = Z^T dY (split over rows) -> reduces
//
// The NF4 codebook and the encoder thresholds are derived here from their
// definition ("Training LLMs on a Budget: LoRA, QLoRA, and LoftQ", section 3,
// trick 1: 16 normal quantiles, normalised by the largest), with a local
// inverse normal CDF.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "lora4.h"
#include "gemm.hpp"
#include "gemm_big.hpp"
#include "gemm_fwd.hpp"
#include "gemm_dgrad.hpp"
#include "mx.hpp"
#include "loftq.hpp"
#include "skinny.hpp"
#include "quant.hpp"

using namespace lora4;

namespace {

// ---------------------------------------------------------------------------
// NF4 codebook
// ---------------------------------------------------------------------------

double norm_cdf(double x) { return 0.5 * std::erfc(-x / std::sqrt(2.0)); }

// Inverse of the standard normal CDF: bisection to a bracket, then Newton.
double norm_ppf(double p) {
  double lo = -40.0, hi = 40.0;
  for (int i = 0; i < 200; ++i) {
    double mid = 0.5 * (lo + hi);
    if (norm_cdf(mid) < p) lo = mid; else hi = mid;
  }
  double x = 0.5 * (lo + hi);
  for (int i = 0; i < 4; ++i) {
    double f = norm_cdf(x) - p;
    double d = std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI);
    if (d == 0.0) break;
    x -= f / d;
  }
  return x;
}

// Evenly spaced points start..stop (num of them), as i * step + start.
std::vector<double> spaced(double start, double stop, int num) {
#pragma clang fp contract(off)
  std::vector<double> v(num);
  const double step = (stop - start) / (double)(num - 1);
  for (int i = 0; i < num; ++i) {
    double y = (double)i * step;
    y = y + start;
    v[i] = y;
  }
  v[num - 1] = stop;
  return v;
}

Nf4Table build_nf4_table() {
#pragma clang fp contract(off)
  // offset: mean of 1 - 1/30 and 1 - 1/32
  const double delta = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0));
  std::vector<double> lv;
  std::vector<double> pp = spaced(delta, 0.5, 9);
  for (int i = 0; i < 8; ++i) lv.push_back(norm_ppf(pp[i]));          // 8 positive levels
  std::vector<double> pn = spaced(delta, 0.5, 8);
  for (int i = 0; i < 7; ++i) lv.push_back(-norm_ppf(pn[i]));         // 7 negative levels
  lv.push_back(0.0);                                                   // exact zero
  std::sort(lv.begin(), lv.end());
  const double mx = lv.back();
  Nf4Table t;
  for (int i = 0; i < 16; ++i) t.q[i] = (float)(lv[i] / mx);
  for (int i = 0; i < 15; ++i) {
    const double mid = ((double)t.q[i] + (double)t.q[i + 1]) * 0.5;   // exact
    float th = (float)mid;
    if ((double)th > mid) th = std::nextafter(th, -INFINITY);
    t.thr[i] = th;
  }
  return t;
}

const Nf4Table &nf4_table() {
  static const Nf4Table t = build_nf4_table();
  return t;
}

// ---------------------------------------------------------------------------
// Kernel timing (profiling aid)
// ---------------------------------------------------------------------------

struct PendingTiming {
  const char *name;
  hipEvent_t a, b;
};

std::mutex g_tmu;
bool g_timing = false;
std::vector<PendingTiming> g_pending;
std::vector<hipEvent_t> g_free_events;

// Set while lora4_forward_noalloc runs on this thread: timing then takes
// events from the pool only and never creates one.
thread_local bool tl_no_alloc = false;

hipEvent_t take_event() {
  if (tl_no_alloc && g_free_events.empty()) return nullptr;
  if (!g_free_events.empty()) {
    hipEvent_t e = g_free_events.back();
    g_free_events.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Runs `go` (which enqueues one kernel on `stream`), bracketed by two timing
// events when timing is on. An error still pending from earlier work on the
// thread is reported before anything is launched (so it is not pinned on this
// kernel); on any failure the events go back to the pool.
template <typename Go>
lora4_status launch_timed(const char *name, hipStream_t stream, Go &&go) {
  if (hipPeekAtLastError() != hipSuccess) return LORA4_ERR_HIP;
  hipEvent_t ea = nullptr, eb = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_tmu);
    if (g_timing) {
      ea = take_event();
      eb = take_event();
    }
  }
  auto give_back = [&] {
    std::lock_guard<std::mutex> lk(g_tmu);
    if (ea) g_free_events.push_back(ea);
    if (eb) g_free_events.push_back(eb);
  };
  const bool timed = ea && eb;
  if (!timed && (ea || eb)) {   // only one event could be had: run untimed
    give_back();
    ea = eb = nullptr;
  }
  if (timed && hipEventRecord(ea, stream) != hipSuccess) {
    give_back();
    return LORA4_ERR_HIP;
  }
  go();
  if (hipGetLastError() != hipSuccess) {
    give_back();
    return LORA4_ERR_HIP;
  }
  if (timed) {
    if (hipEventRecord(eb, stream) != hipSuccess) {
      give_back();
      return LORA4_ERR_HIP;
    }
    std::lock_guard<std::mutex> lk(g_tmu);
    g_pending.push_back({name, ea, eb});
  }
  return LORA4_OK;
}

template <typename Kern, typename Params>
lora4_status launch(const char *name, Kern kernel, dim3 grid, dim3 block, const Params &params,
                    hipStream_t stream) {
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return LORA4_OK;
  return launch_timed(name, stream, [&] { hipLaunchKernelGGL(kernel, grid, block, 0, stream, params); });
}

template <typename Kern, typename... Args>
lora4_status launch_args(const char *name, Kern kernel, dim3 grid, dim3 block, hipStream_t stream,
                         Args... args) {
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return LORA4_OK;
  return launch_timed(name, stream, [&] { hipLaunchKernelGGL(kernel, grid, block, 0, stream, args...); });
}

// Raises a kernel's dynamic LDS limit, once per (device, kernel): the
// attribute belongs to the kernel object of the device that is current.
lora4_status set_lds_limit(const void *kernel, size_t lds) {
  static std::mutex mu;
  static std::map<std::pair<int, const void *>, bool> done;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LORA4_ERR_HIP;
  std::lock_guard<std::mutex> lk(mu);
  bool &d = done[{dev, kernel}];
  if (!d) {
    if (hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return LORA4_ERR_HIP;
    d = true;
  }
  return LORA4_OK;
}

template <typename Kern, typename Params>
lora4_status launch_lds(const char *name, Kern kernel, dim3 grid, dim3 block, size_t lds, const Params &params,
                        hipStream_t stream) {
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return LORA4_OK;
  const lora4_status st = set_lds_limit((const void *)kernel, lds);
  if (st != LORA4_OK) return st;
  return launch_timed(name, stream, [&] { hipLaunchKernelGGL(kernel, grid, block, lds, stream, params); });
}

#define TRY(x)                              \
  do {                                      \
    lora4_status st_ = (x);                 \
    if (st_ != LORA4_OK) return st_;        \
  } while (0)

// ---------------------------------------------------------------------------
// Validation helpers
// ---------------------------------------------------------------------------

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
// NF4-DQ second-level scales are read and written one float at a time; a
// group's slice of a stacked [groups][...] array starts at a multiple of 4
// bytes only (lora4_packed_bytes part 2 is 4 * ceil(N*K/64/256))
bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

lora4_status check_W(const lora4_W *W) {
  if (!W) return LORA4_ERR_NULL;
  if (W->format != LORA4_NF4 && W->format != LORA4_NF4_DQ && W->format != LORA4_MXFP4 && W->format != LORA4_NVFP4)
    return LORA4_ERR_FORMAT;
  const int want = W->format == LORA4_MXFP4 ? 32 : W->format == LORA4_NVFP4 ? 16 : 64;
  if (W->block != want) return LORA4_ERR_FORMAT;
  // K: whole blocks, and whole 32-element halves of a 64-deep step (NVFP4)
  const int kmul = want < 32 ? 32 : want;
  if (W->N < 1 || W->K < kmul || W->K % kmul != 0 || W->groups < 1) return LORA4_ERR_SHAPE;
  if (W->N > (int64_t(1) << 31) || W->K > (int64_t(1) << 31) || W->groups > 65535) return LORA4_ERR_SHAPE;
  if (!W->codes || !W->scales) return LORA4_ERR_NULL;
  if (W->format == LORA4_NF4_DQ && !W->scales2) return LORA4_ERR_NULL;
  if (!aligned16(W->codes) || !aligned16(W->scales)) return LORA4_ERR_ALIGN;
  if (W->format == LORA4_NF4_DQ && !aligned4(W->scales2)) return LORA4_ERR_ALIGN;
  return LORA4_OK;
}

// A base as the host plans for it: the ABI description, the number of row
// groups, and whether one W serves every group (several adapters over one
// base) instead of one W per group (experts).
struct Base {
  const lora4_W *W;
  int64_t E;
  bool shared;
};

PackedW packed_of(const Base &b) {
  const lora4_W *W = b.W;
  PackedW p;
  p.codes = W->codes;
  p.scales = W->scales;
  p.scales2 = W->scales2;
  p.N = W->N;
  p.K = W->K;
  p.KB = w_blocks(W->K);
  p.g_codes = w_blocks(W->N) * p.KB * 2048;
  p.g_scales = w_blocks(W->N) * p.KB * (W->format == LORA4_MXFP4 ? 128 : W->format == LORA4_NVFP4 ? 256 : 64);
  p.g_scales2 = W->format == LORA4_NF4_DQ ? ceil_div(W->N * (W->K / 64), 256) : 0;
  p.shared = b.shared ? 1 : 0;
  return p;
}

// ---------------------------------------------------------------------------
// Planning: split factors and workspace layout
// ---------------------------------------------------------------------------

// Workgroups wanted for the rank-r TN passes (dA, dB) at rank 16; wider
// rank tiles do more work per workgroup and take proportionally fewer row
// splits (fewer fp32 partials to write and reduce).
constexpr int TARGET_WG = 1024;

int skinny_tile(int r) { return r <= 16 ? 16 : r <= 32 ? 32 : r <= 64 ? 64 : 128; }

// Forward base GEMM schedule (defined with the large-tile dispatch below).
struct FwdSched {
  bool use;          // register-direct kernels (else the 128 x 128 LDS kernel)
  int whole_tiles;   // 256 x 256 tiles computed by one block each (the first ones)
  int split_tiles;   // or: tiles each split over ksplit blocks
  int ksplit;        // reduction splits of a split tile
  int split_steps;   // 64-deep steps per split
  int tail_tiles;    // 256 x 256 tiles after the whole ones, run as two 256 x 128 halves
  bool small;        // or: 128 x 128 tiles (k_gemm_fwd_small)
};
constexpr FwdSched FWD_LDS_KERNEL{false, 0, 0, 1, 1 << 30, 0, false};
FwdSched fwd_sched(int64_t M, int64_t N, int64_t K, int64_t E, const PackedW &W);
struct SkSched;
size_t sk_part_bytes_for(int64_t M, int64_t R, int r, int64_t E, int transb);
lora4_status reduce_bf16(const char *name, const float *part, int splits, int64_t stride, int64_t n,
                         uint16_t *out1, float a1, uint16_t *out2, float a2, hipStream_t st);

struct Plan {
  int64_t M, N, K, E;
  int r;
  int rt;             // skinny tile width (Z, dZ, TN P tile)
  int64_t row_slots;  // row-tile slots for BM = 128
  int tq_a, tq_b;     // TN Q tiles (dA over K, dB over N)
  int msplit_a, msplit_b;
  FwdSched fs;                // forward base GEMM schedule
  int lds_splits;             // reduction splits of the 128 x 128 base GEMM (forward or dgrad), 1: none
  // workspace offsets
  size_t off_sz, off_zw, off_dz, off_part, off_part_b, off_cnt, off_party, off_skpart, off_partx, bytes;
  int64_t ncnt;       // backward: arrival counters of the dA / dB tiles (TnParams::cnt)
};

constexpr int BM_MAIN = 128, BN_MAIN = 128;
constexpr int BM_SKINNY = 128;
constexpr int TN_BQ = 128;

int cu_count();
bool big_fits(int64_t ld_a, int64_t M, const PackedW &W);
bool use_big(int64_t M, int64_t Nc, int64_t E);

// Reduction splits for the 128 x 128 base GEMM on a grid of `blocks`
// workgroups (R: reduction length): when the grid fills less than half the
// CUs, the reduction is cut into ranges of at least two 64-deep steps so that
// the grid approaches one workgroup per CU (fp32 partials of at most 64 MiB,
// summed in range order by k_reduce_bf16). 1: no split.
constexpr int LDS_SPLIT_MIN_STEPS = 2;
constexpr int64_t LDS_SPLIT_MAX_BYTES = (int64_t)64 << 20;
int lds_splits_for(int64_t blocks, int64_t R, int64_t M, int64_t Nc) {
  const int64_t cus = cu_count();
  if (R <= 0 || blocks <= 0 || 2 * blocks > cus) return 1;
  const int64_t steps = ceil_div(R, BK);
  int64_t k = std::min<int64_t>(steps / LDS_SPLIT_MIN_STEPS, cus / blocks);
  k = std::min<int64_t>(k, LDS_SPLIT_MAX_BYTES / std::max<int64_t>(1, M * Nc * 4));
  if (k < 2) return 1;
  // equal ranges of whole steps; the count actually needed for them
  const int64_t per = ceil_div(steps, k);
  return (int)ceil_div(steps, per);
}
int64_t lds_split_len(int splits, int64_t R) { return ceil_div(ceil_div(R, BK), (int64_t)splits) * BK; }

// cap: the workspace there is (the allocation-free forward's fixed scratch);
// a forward whose split partials would not fit runs the tiles unsplit.
Plan make_plan(int which, const Base &b, int64_t M, int r, size_t cap = SIZE_MAX) {
  const lora4_W *W = b.W;
  Plan p{};
  p.M = M;
  p.N = W->N;
  p.K = W->K;
  p.E = b.E;
  p.r = r;
  p.rt = skinny_tile(r);
  p.row_slots = ceil_div(std::max<int64_t>(M, 1), BM_MAIN) + (p.E > 1 ? p.E : 0);
  const int64_t rtiles = ceil_div(r, p.rt);
  p.tq_a = (int)ceil_div(p.K, TN_BQ);
  p.tq_b = (int)ceil_div(p.N, TN_BQ);
  const int64_t mavg = std::max<int64_t>(1, M / p.E);
  auto msplit = [&](int64_t qtiles) {
    int64_t tiles = rtiles * qtiles * p.E;
    int64_t want = ceil_div(TARGET_WG * 16 / p.rt, std::max<int64_t>(tiles, 1));
    int64_t maxs = std::max<int64_t>(1, mavg / 256);
    return (int)std::max<int64_t>(1, std::min<int64_t>({want, maxs, 65535 / p.E}));
  };
  p.msplit_a = msplit(p.tq_a);
  p.msplit_b = msplit(p.tq_b);
  p.fs = fwd_sched(M, p.N, p.K, p.E, packed_of(b));
  p.lds_splits = 1;
  {
    const PackedW pw = packed_of(b);
    if (which == 0 && !p.fs.use)
      p.lds_splits = lds_splits_for(p.row_slots * ceil_div(p.N, BN_MAIN), p.K, M, p.N);
    if (which == 1 && !(big_fits(p.N, M, pw) && use_big(M, p.K, pw.shared ? 1 : p.E)))
      p.lds_splits = lds_splits_for(p.row_slots * ceil_div(p.K, BN_MAIN), p.N, M, p.K);
  }

  const size_t mr2 = align256((size_t)M * r * 2);
  size_t off = 0;
  p.off_sz = off;   // forward: s Z ; backward: dZ
  off += mr2;
  p.off_zw = off;   // backward: recomputed Z
  if (which == 1) off += mr2;
  p.off_dz = p.off_sz;
  p.off_skpart = off;  // fp32 partials of the rank-r passes (Z, then dZ)
  {
    size_t b = sk_part_bytes_for(M, p.K, r, p.E, 0);
    if (which == 1) b = std::max(b, sk_part_bytes_for(M, p.N, r, p.E, 1));
    off += b;
  }
  p.off_party = off;  // forward: fp32 partials of the split base GEMM
  if (which == 0 && p.fs.use && p.fs.split_tiles > 0)
    off += align256((size_t)p.fs.split_tiles * p.fs.ksplit * fwd::BM * fwd::BN * 4);
  p.off_part = off;  // backward: dA partials, then dB^T partials, then their tiles' counters
  p.ncnt = 0;
  if (which == 1) {
    p.off_part_b = off + align256((size_t)p.msplit_a * p.E * r * p.K * 4);
    off = p.off_part_b + align256((size_t)p.msplit_b * p.E * r * p.N * 4);
    p.off_cnt = off;
    p.ncnt = rtiles * (p.tq_a + p.tq_b) * p.E;
    off += align256((size_t)p.ncnt * 4);
  }
  p.off_partx = off;  // fp32 partials of the split 128 x 128 base GEMM
  if (p.lds_splits > 1) off += align256((size_t)p.lds_splits * M * (which == 0 ? p.N : p.K) * 4);
  p.bytes = std::max<size_t>(off, 256);   // never 0: 0 reports invalid arguments
  if (p.bytes > cap && which == 0 && p.fs.use && p.fs.split_tiles > 0) {
    p.bytes -= align256((size_t)p.fs.split_tiles * p.fs.ksplit * fwd::BM * fwd::BN * 4);
    p.off_part = p.off_party;
    p.off_partx = p.off_party;
    p.fs = FWD_LDS_KERNEL;   // the 128 x 128 kernel, no partials
  }
  if (p.bytes > cap && p.lds_splits > 1) {
    p.bytes -= align256((size_t)p.lds_splits * M * (which == 0 ? p.N : p.K) * 4);
    p.lds_splits = 1;        // unsplit, no partials
  }
  return p;
}

template <typename T>
T *ws_at(void *ws, size_t off) {
  return reinterpret_cast<T *>(reinterpret_cast<char *>(ws) + off);
}

// ---------------------------------------------------------------------------
// Kernel dispatch (template instantiations by runtime shape)
// ---------------------------------------------------------------------------

template <int FMT>
lora4_status run_nt_main(const NtParams &p, dim3 grid, hipStream_t st) {
  return launch("gemm_nt_base", k_gemm_nt<FMT, BM_MAIN, BN_MAIN, 2>, grid, dim3(THREADS), p, st);
}

// Large-tile path (256 x 256 tiles) for the base GEMMs when the grid fills
// the GPU; LORA4_BIG=0/1 in the environment forces the choice.
int big_policy() {
  const char *e = std::getenv("LORA4_BIG");
  return e ? std::atoi(e) : -1;
}

// The large-tile kernels address their operands through 32-bit buffer offsets
// and stream 16-byte activation chunks: they need rows that are multiples of
// 8 elements and per-group buffers below 2 GiB.
bool big_fits(int64_t ld_a, int64_t M, const PackedW &W) {
  const int64_t lim = (int64_t)1 << 31;
  // (look-ahead loads run up to four row blocks of tiles past the end of W)
  const int64_t ahead = 4 * W.KB * 2048;
  return ld_a % 8 == 0 && W.g_codes + ahead < lim && ld_a * 2 * 256 < lim && W.g_scales * 4 + ahead < lim &&
         W.g_scales2 * 4 < lim;
}

// Compute units of the current device (cached per device).
int cu_count() {
  // per device; concurrent first calls may both query, and store the same value
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (!n) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Forced forward tile shapes for tests and measurements (LORA4_FWD_TILES):
// "small" (128 x 128 tiles), "half" (every 256 x 256 tile as two halves),
// "mixed" (the second half of the tiles as halves), "whole" (256 x 256 tiles
// only, no halves), "noshort" (automatic, but short last row tiles run the
// 256-row code); anything else or unset: automatic.
int fwd_tiles_policy() {
  const char *e = std::getenv("LORA4_FWD_TILES");
  if (!e) return 0;
  const std::string v(e);
  return v == "small" ? 1 : v == "half" ? 2 : v == "mixed" ? 3 : v == "whole" ? 4 : v == "noshort" ? 5 : 0;
}

// The register-direct forward kernels run one tile per CU at a time:
// * enough 256 x 256 tiles for 3/4 of the CUs: whole tiles, except that when
//   the last round would fill half the CUs or less (e.g. 896 tiles on 256
//   CUs: 3.5 rounds), its tiles run as two 256 x 128 halves each, a full
//   round of half the length;
// * else, enough 128 x 128 tiles for 3/4 of the CUs (e.g. 4096 x 1024: 64 of
//   256 x 256, 256 of 128 x 128): those;
// * else the reduction of every 256 x 256 tile is split over several blocks
//   (fp32 partials, at least 8 steps per split, partials capped at 256 MiB),
//   summed by a deterministic reduction.
// The automatic policy keeps the 128 x 128 LDS kernel when even a split grid
// would leave most of the GPU idle.
FwdSched fwd_sched(int64_t M, int64_t N, int64_t K, int64_t E, const PackedW &W) {
  FwdSched f = FWD_LDS_KERNEL;
  if (K <= 0 || M <= 0 || !big_fits(K, M, W)) return f;
  const int pol = big_policy();
  if (pol == 0) return f;
  int force = fwd_tiles_policy();
  if (force == 5) force = 0;   // (short tiles: big_params)
  const int64_t cus = cu_count();
  const int64_t groups = E > 1 && !W.shared ? E : 0;
  const int64_t tiles = (ceil_div(M, fwd::BM) + groups) * ceil_div(N, fwd::BN);
  const int64_t tiles128 = (ceil_div(M, 128) + groups) * ceil_div(N, 128);
  f.use = true;
  if (force == 1 || (force == 0 && tiles < cus * 3 / 4 && tiles128 >= cus * 3 / 4)) {
    f.small = true;
    return f;
  }
  if (force >= 2 || tiles >= cus * 3 / 4) {
    const int64_t rem = tiles % cus;
    int64_t tail = 0;
    if (force == 2) tail = tiles;
    else if (force == 3) tail = tiles / 2;
    else if (force == 0 && tiles > cus && rem > 0 && rem <= cus / 2) tail = rem;
    f.whole_tiles = (int)(tiles - tail);
    f.tail_tiles = (int)tail;
    return f;
  }
  const int64_t steps = ceil_div(K, fwd::BKS);
  const int64_t max_ks = std::min<int64_t>(16, std::max<int64_t>(1, steps / 8));
  int64_t ks = std::min<int64_t>(cus / tiles, max_ks);
  const int64_t cap = ((int64_t)256 << 20) / ((int64_t)fwd::BM * fwd::BN * 4 * tiles);
  ks = std::max<int64_t>(1, std::min(ks, cap));
  if (pol < 0 && tiles * ks < cus * 3 / 4) return FWD_LDS_KERNEL;
  if (ks == 1) {
    f.whole_tiles = (int)tiles;
    return f;
  }
  f.split_tiles = (int)tiles;
  f.split_steps = (int)ceil_div(steps, ks);
  f.ksplit = (int)ceil_div(steps, f.split_steps);
  return f;
}

bool use_big(int64_t M, int64_t Nc, int64_t E) {
  const int pol = big_policy();
  if (pol >= 0) return pol != 0;
  const int64_t tiles = (ceil_div(M, big::BM) + (E > 1 ? E : 0)) * ceil_div(Nc, big::BN);
  return tiles >= 256;
}

// Forward base GEMM with deq(W) decoded straight into MFMA registers.
template <int FMT, bool SHARED>
lora4_status run_fwd(const big::Params &p, bool small, hipStream_t st) {
  if (small)
    return launch_lds("gemm_nt_base", fwd::k_gemm_fwd_small<FMT, SHARED>, dim3((unsigned)p.nblocks),
                      dim3(fwd::THREADS), (size_t)fwd::lds_bytes(), p, st);
  if (p.ksplit > 1)
    return launch_lds("gemm_nt_base", fwd::k_gemm_fwd<FMT, true, SHARED>, dim3((unsigned)p.nblocks),
                      dim3(fwd::THREADS), (size_t)fwd::lds_bytes(), p, st);
  if constexpr (!SHARED) {
    // per-expert row tiles: short last tiles of a group run shorter tiles' code
    if (p.groups > 1 && fwd_tiles_policy() != 5)
      return launch_lds("gemm_nt_base", fwd::k_gemm_fwd<FMT, false, false, true>, dim3((unsigned)p.nblocks),
                        dim3(fwd::THREADS), (size_t)fwd::lds_bytes(), p, st);
  }
  return launch_lds("gemm_nt_base", fwd::k_gemm_fwd<FMT, false, SHARED>, dim3((unsigned)p.nblocks),
                    dim3(fwd::THREADS), (size_t)fwd::lds_bytes(), p, st);
}

template <int FMT>
lora4_status run_fwd(const big::Params &p, bool small, hipStream_t st) {
  return p.shared_rows ? run_fwd<FMT, true>(p, small, st) : run_fwd<FMT, false>(p, small, st);
}

lora4_status run_fwd_fmt(int fmt, const big::Params &p, bool small, hipStream_t st) {
  switch (fmt) {
    case LORA4_NF4: return run_fwd<FMT_NF4>(p, small, st);
    case LORA4_NF4_DQ: return run_fwd<FMT_NF4_DQ>(p, small, st);
    case LORA4_MXFP4: return run_fwd<FMT_MXFP4>(p, small, st);
    case LORA4_NVFP4: return run_fwd<FMT_NVFP4>(p, small, st);
  }
  return LORA4_ERR_FORMAT;
}

// Input-gradient base GEMM (deq(W) through a transposed LDS tile).
template <int FMT>
lora4_status run_dgrad(const big::Params &p, hipStream_t st) {
  if (p.shared_rows)
    return launch_lds("gemm_nn_dgrad", dgrad::k_gemm_dgrad<FMT, true>, dim3((unsigned)p.nblocks),
                      dim3(dgrad::THREADS), (size_t)dgrad::lds_bytes(), p, st);
  return launch_lds("gemm_nn_dgrad", dgrad::k_gemm_dgrad<FMT, false>, dim3((unsigned)p.nblocks),
                    dim3(dgrad::THREADS), (size_t)dgrad::lds_bytes(), p, st);
}

lora4_status run_dgrad_fmt(int fmt, const big::Params &p, hipStream_t st) {
  switch (fmt) {
    case LORA4_NF4: return run_dgrad<FMT_NF4>(p, st);
    case LORA4_NF4_DQ: return run_dgrad<FMT_NF4_DQ>(p, st);
    case LORA4_MXFP4: return run_dgrad<FMT_MXFP4>(p, st);
    case LORA4_NVFP4: return run_dgrad<FMT_NVFP4>(p, st);
  }
  return LORA4_ERR_FORMAT;
}

big::Params big_params(const Mat &A, const PackedW &W, int64_t R, const Mat &A2, const Mat &B2, int r2,
                       int64_t M, int64_t Nc, const int64_t *offs, int64_t E, uint16_t *C, int64_t ldc) {
  big::Params p{};
  p.A = A;
  p.W = W;
  p.R = R;
  p.A2 = A2;
  p.B2 = B2;
  p.r2 = r2;
  p.M = M;
  p.Nc = Nc;
  p.offsets = offs;
  p.groups = (int)E;
  p.C = C;
  p.ldc = ldc;
  p.tiles_n = (int)ceil_div(Nc, big::BN);
  // one W for every group: the row tiles run over all M rows, regardless of
  // the groups (which then only select the rank-r operands)
  p.shared_rows = W.shared && E > 1 ? 1 : 0;
  p.nslots = (int)(ceil_div(std::max<int64_t>(M, 1), big::BM) + (E > 1 && !p.shared_rows ? E : 0));
  p.nblocks = p.nslots * p.tiles_n;
  p.nfull = p.nblocks;
  p.ntail = 0;
  p.tab = nf4_table();
  p.ksplit = 1;
  p.split_steps = 1 << 30;
  p.Cpart = nullptr;
  return p;
}

// Rank-r tail operand handed to a GEMM as fp32 partials of the skinny pass
// (the GEMM sums them; see big::Params::A2part).
struct TailParts {
  const float *part;
  int parts;
  float scale;
  uint16_t *out1;
  float alpha1;
  uint16_t *out2;
  float alpha2;
};

void apply_tail_parts(big::Params &q, const TailParts *tp) {
  if (!tp) return;
  q.A2part = tp->part;
  q.A2parts = tp->parts;
  q.A2scale = tp->scale;
  q.A2out1 = tp->out1;
  q.A2alpha1 = tp->alpha1;
  q.A2out2 = tp->out2;
  q.A2alpha2 = tp->alpha2;
}

// Whether the forward base pass runs the register-direct kernel, and the
// backward dgrad pass the 256 x 256 dgrad kernel (the kernels that can take
// their tail operand as partials).
bool fwd_regs_taken(int64_t R, const Plan &pl) { return R > 0 && pl.fs.use; }
bool dgrad_taken(int64_t R, int64_t ld_a, int64_t M, const PackedW &W, int64_t Nc, int64_t E) {
  return R > 0 && big_fits(ld_a, M, W) && use_big(M, Nc, W.shared ? 1 : E);
}

// Forward base GEMM: the register-direct kernel as the plan schedules it
// (split partials in `party`, then reduced into the output), else the
// 128 x 128 kernel.
lora4_status run_nt_main_fmt(int fmt, const NtParams &p, dim3 grid, const Plan &pl, float *party,
                             float *partx, const TailParts *tp, hipStream_t st) {
  if (fwd_regs_taken(p.R, pl)) {
    big::Params q = big_params(p.A, p.W, p.R, p.A2, p.B2, p.r2, p.M, p.Nc, p.offsets, p.groups, p.out.C,
                               p.out.ldc);
    apply_tail_parts(q, tp);
    q.ksplit = pl.fs.ksplit;
    q.split_steps = pl.fs.split_steps;
    if (pl.fs.small) {
      q.tiles_n = (int)ceil_div(q.Nc, 128);
      q.nslots = (int)(ceil_div(std::max<int64_t>(q.M, 1), 128) + (q.groups > 1 && !q.shared_rows ? q.groups : 0));
      q.nblocks = q.nslots * q.tiles_n;
    } else {
      q.nfull = pl.fs.whole_tiles;
      q.ntail = pl.fs.tail_tiles;
      q.nblocks = pl.fs.whole_tiles + 2 * pl.fs.tail_tiles + pl.fs.split_tiles * pl.fs.ksplit;
    }
    q.Cpart = party;
    TRY(run_fwd_fmt(fmt, q, pl.fs.small, st));
    if (pl.fs.split_tiles > 0) {
      const int64_t n = (int64_t)pl.fs.split_tiles * fwd::BM * (fwd::BN / 4);
      TRY(launch_args("reduce_y", fwd::k_reduce_tiles, dim3((unsigned)ceil_div(n, 256)), dim3(256), st, q,
                      pl.fs.split_tiles));
    }
    return LORA4_OK;
  }
  if (tp) return LORA4_ERR_UNIMPLEMENTED;   // (callers check the same predicates)
  NtParams q = p;
  const bool split = pl.lds_splits > 1 && p.R > 0 && partx && p.out.C && p.out.ldc == p.Nc;
  if (split) {
    q.Rsplit = lds_split_len(pl.lds_splits, p.R);
    q.out.part = partx;
    q.out.part_stride = p.M * p.Nc;
    grid.z = (unsigned)pl.lds_splits;
  }
  lora4_status r = LORA4_ERR_FORMAT;
  switch (fmt) {
    case LORA4_NF4: r = run_nt_main<FMT_NF4>(q, grid, st); break;
    case LORA4_NF4_DQ: r = run_nt_main<FMT_NF4_DQ>(q, grid, st); break;
    case LORA4_MXFP4: r = run_nt_main<FMT_MXFP4>(q, grid, st); break;
    case LORA4_NVFP4: r = run_nt_main<FMT_NVFP4>(q, grid, st); break;
  }
  TRY(r);
  if (split)
    TRY(reduce_bf16("reduce_y", partx, pl.lds_splits, p.M * p.Nc, p.M * p.Nc, p.out.C, p.out.alpha, nullptr, 0.0f,
                    st));
  return LORA4_OK;
}

template <int FMT>
lora4_status run_nn_main(const NnParams &p, dim3 grid, hipStream_t st) {
  return launch("gemm_nn_dgrad", k_gemm_nn<FMT, BM_MAIN, BN_MAIN, 2>, grid, dim3(THREADS), p, st);
}

lora4_status run_nn_main_fmt(int fmt, const NnParams &p, dim3 grid, const Plan &pl, float *partx,
                             const TailParts *tp, hipStream_t st) {
  if (dgrad_taken(p.R, p.A.ld, p.M, p.W, p.Nc, p.groups)) {
    big::Params q = big_params(p.A, p.W, p.R, p.A2, p.B2, p.r2, p.M, p.Nc, p.offsets, p.groups, p.out.C,
                               p.out.ldc);
    apply_tail_parts(q, tp);
    return run_dgrad_fmt(fmt, q, st);
  }
  if (tp) return LORA4_ERR_UNIMPLEMENTED;   // (callers check the same predicates)
  NnParams q = p;
  const bool split = pl.lds_splits > 1 && p.R > 0 && partx && p.out.C && p.out.ldc == p.Nc;
  if (split) {
    q.Rsplit = lds_split_len(pl.lds_splits, p.R);
    q.out.part = partx;
    q.out.part_stride = p.M * p.Nc;
    grid.z = (unsigned)pl.lds_splits;
  }
  lora4_status r = LORA4_ERR_FORMAT;
  switch (fmt) {
    case LORA4_NF4: r = run_nn_main<FMT_NF4>(q, grid, st); break;
    case LORA4_NF4_DQ: r = run_nn_main<FMT_NF4_DQ>(q, grid, st); break;
    case LORA4_MXFP4: r = run_nn_main<FMT_MXFP4>(q, grid, st); break;
    case LORA4_NVFP4: r = run_nn_main<FMT_NVFP4>(q, grid, st); break;
  }
  TRY(r);
  if (split)
    TRY(reduce_bf16("reduce_dx", partx, pl.lds_splits, p.M * p.Nc, p.M * p.Nc, p.out.C, p.out.alpha, nullptr, 0.0f,
                    st));
  return LORA4_OK;
}

// Both jobs share P (the rank) and so the P tiling; grid sizes of the two are
// pa x qa x za and pa x qb x zb blocks.
lora4_status run_tn2(const char *name, int rt, const TnParams &a, const TnParams &b, int qa, int za, int qb,
                     int zb, hipStream_t st) {
  const int pt = (int)ceil_div(a.P, rt);
  const int64_t na = (int64_t)pt * qa * za, nb = (int64_t)pt * qb * zb;
  if (na + nb > INT32_MAX) return LORA4_ERR_SHAPE;
  const dim3 grid((unsigned)(na + nb)), block(THREADS);
  switch (rt) {
    case 16: return launch_args(name, k_gemm_tn2<16, TN_BQ, 1>, grid, block, st, a, b, pt, qa, qb, na);
    case 32: return launch_args(name, k_gemm_tn2<32, TN_BQ, 1>, grid, block, st, a, b, pt, qa, qb, na);
    case 64: return launch_args(name, k_gemm_tn2<64, TN_BQ, 1>, grid, block, st, a, b, pt, qa, qb, na);
    default: return launch_args(name, k_gemm_tn2<128, TN_BQ, 2>, grid, block, st, a, b, pt, qa, qb, na);
  }
}

Mat mat(const uint16_t *p, int64_t ld, int64_t gstride = 0) { return Mat{p, ld, gstride}; }

lora4_status reduce_bf16(const char *name, const float *part, int splits, int64_t stride, int64_t n,
                         uint16_t *out1, float a1, uint16_t *out2, float a2, hipStream_t st) {
  dim3 grid((unsigned)ceil_div(ceil_div(n, 4), 256));   // four elements per thread
  return launch_args(name, k_reduce_bf16, grid, dim3(256), st, part, splits, stride, n, out1, a1, out2, a2);
}

// Row-block rank-r product (Z = X A^T with transb 0, dY B with transb 1):
// out1 = bf16(a1 acc), out2 = bf16(a2 acc). TJ 16-wide column blocks per
// workgroup (up to 128 columns; grid.y covers larger r), TM 16-row blocks.
template <int TM, int TJ>
lora4_status run_rows_tj(int transb, const skinny::Params &p, dim3 grid, hipStream_t st) {
  if (transb) return launch("rows_skinny_dz", skinny::k_rows_skinny<TM, TJ, 1>, grid, dim3(skinny::THREADS), p, st);
  return launch("rows_skinny_z", skinny::k_rows_skinny<TM, TJ, 0>, grid, dim3(skinny::THREADS), p, st);
}

// Rank-r row-block pass schedule. Two kernels:
// * k_rows_lds (whole 16-byte pieces: R % 8 == 0, and r % 8 == 0 for dZ, whose
//   small operand B is r-contiguous): 64 tm rows per workgroup, ns stages of
//   64 deep; the reduction split into at most 4 `ranges` so that about one
//   round of workgroups (as many as fit the CUs' LDS) covers the GPU, one range
//   at rank 128 (the GEMM tails then read bf16 Z instead of four fp32 partials
//   of 128 columns);
// * k_rows_skinny otherwise: 16 tm rows, the four waves taking the range's
//   32-wide chunks in turn, ranges so that the grid has about two workgroups
//   per CU. Rank 16 takes 32-row blocks (512 workgroups on 4096 rows; 64-row
//   blocks and 256 workgroups measured 0.3% slower on the 8B layer set).
// Columns: 16 tj per workgroup (grid.y covers larger r).
struct SkSched {
  int tm, tj, ranges;
  int64_t klen;
  bool lds;
};
constexpr int64_t SK_TARGET_WG = 512;   // workgroups wanted per pass
constexpr int64_t SK_MAX_RANGES = 4;    // (8 measured 0.5% slower on the 8B layer set)
// below this many bytes of activations one range: the pass is short, and its
// partials would cost a reduction launch of its own on the small grids
constexpr int64_t SK_SPLIT_MIN_BYTES = (int64_t)4 << 20;
constexpr int64_t LDS_PER_CU = 160 * 1024;

bool sk_lds_fits(int64_t R, int r, int transb) {
  const int64_t lim = (int64_t)1 << 31;
  return R % 8 == 0 && (!transb || r % 8 == 0) && R * 2 * 128 < lim && (int64_t)r * R * 2 < lim;
}

// LDS of the k_rows_lds instantiation for tj (the tm and ns go with it)
size_t sk_lds_bytes(int tj) {
  switch (tj) {
    case 1: return skinny::LdsRing<1, 1, 0, 6>::bytes();
    case 2: return skinny::LdsRing<1, 2, 0, 6>::bytes();
    case 4: return skinny::LdsRing<2, 4, 0, 4>::bytes();
    default: return skinny::LdsRing<2, 8, 0, 4>::bytes();
  }
}

SkSched sk_sched(int64_t M, int64_t R, int r, int64_t E, int transb) {
  SkSched f{};
  f.tj = r <= 16 ? 1 : r <= 32 ? 2 : r <= 64 ? 4 : 8;
  f.lds = sk_lds_fits(R, r, transb);
  const int64_t jt = ceil_div(r, 16 * f.tj);
  if (f.lds) {
    f.tm = f.tj >= 4 ? 2 : 1;   // (stages: 6 up to rank 32, 4 above, as rows_skinny instantiates them)
    const int64_t blocks = (ceil_div(std::max<int64_t>(M, 1), 64 * f.tm) + (E > 1 ? E : 0)) * jt;
    const int64_t steps = std::max<int64_t>(1, ceil_div(R, 64));
    const int64_t round = cu_count() * std::max<int64_t>(1, LDS_PER_CU / (int64_t)sk_lds_bytes(f.tj));
    int64_t want = std::max<int64_t>(1, round / blocks);
    want = std::max<int64_t>(1, std::min<int64_t>({want, steps / 4, SK_MAX_RANGES}));
    if (f.tj >= 8 || M * R * 2 < SK_SPLIT_MIN_BYTES) want = 1;
    f.klen = ceil_div(steps, want) * 64;
    f.ranges = (int)ceil_div(steps * 64, f.klen);
    return f;
  }
  // 64-row blocks from rank 17 on: every block re-reads the small operand
  // (A or B) over its range, so taller blocks cut that traffic (at rank 128,
  // 16-row blocks read A from L2 eight times as often as X itself)
  f.tm = f.tj == 1 ? 2 : 4;
  const int64_t blocks = (ceil_div(std::max<int64_t>(M, 1), 16 * f.tm) + (E > 1 ? E : 0)) * jt;
  const int64_t chunks = std::max<int64_t>(1, ceil_div(R, 32));
  int64_t want = ceil_div(SK_TARGET_WG, blocks);
  want = std::max<int64_t>(1, std::min<int64_t>({want, chunks / 8, SK_MAX_RANGES}));
  if (M * R * 2 < SK_SPLIT_MIN_BYTES) want = 1;
  f.klen = ceil_div(chunks, want) * 32;
  f.ranges = (int)ceil_div(chunks * 32, f.klen);
  return f;
}

size_t sk_part_bytes_for(int64_t M, int64_t R, int r, int64_t E, int transb) {
  const SkSched f = sk_sched(M, R, r, E, transb);
  return f.ranges > 1 ? align256((size_t)f.ranges * M * r * 4) : 0;
}

template <int TM, int TJ, int NS>
lora4_status run_rows_lds(int transb, const skinny::Params &p, dim3 grid, hipStream_t st) {
  const size_t lds = skinny::LdsRing<TM, TJ, 0, NS>::bytes();
  if (transb)
    return launch_lds("rows_skinny_dz", skinny::k_rows_lds<TM, TJ, 1, NS>, grid, dim3(skinny::THREADS), lds, p, st);
  return launch_lds("rows_skinny_z", skinny::k_rows_lds<TM, TJ, 0, NS>, grid, dim3(skinny::THREADS), lds, p, st);
}

lora4_status rows_skinny(int transb, const uint16_t *act, int64_t ld_act, const uint16_t *w, int64_t ld_w,
                         int64_t g_w, int64_t R, int64_t M, int r, const int64_t *offs, int64_t E, uint16_t *o1,
                         float a1, uint16_t *o2, float a2, float *part, bool defer_reduce, hipStream_t st,
                         unsigned *zero = nullptr, int64_t zero_n = 0) {
  const SkSched f = sk_sched(M, R, r, E, transb);
  skinny::Params p{};
  p.act = act;
  p.ld_act = ld_act;
  p.w = w;
  p.ld_w = ld_w;
  p.g_w = g_w;
  p.R = R;
  p.M = M;
  p.r = r;
  p.offsets = offs;
  p.groups = (int)E;
  p.out1 = o1;
  p.alpha1 = a1;
  p.out2 = o2;
  p.alpha2 = a2;
  p.klen = f.klen;
  p.part = part;
  p.zero = zero;
  p.zero_n = zero_n;
  const int64_t slots = ceil_div(std::max<int64_t>(M, 1), (f.lds ? 64 : 16) * f.tm) + (E > 1 ? E : 0);
  dim3 grid((unsigned)slots, (unsigned)ceil_div(r, 16 * f.tj), (unsigned)f.ranges);
  lora4_status st1 = LORA4_ERR_UNIMPLEMENTED;
  if (f.lds) {
    switch (f.tj) {
      case 1: st1 = run_rows_lds<1, 1, 6>(transb, p, grid, st); break;
      case 2: st1 = run_rows_lds<1, 2, 6>(transb, p, grid, st); break;
      case 4: st1 = run_rows_lds<2, 4, 4>(transb, p, grid, st); break;
      default: st1 = run_rows_lds<2, 8, 4>(transb, p, grid, st); break;
    }
  } else switch (f.tj) {
    case 1:
      st1 = f.tm == 2 ? run_rows_tj<2, 1>(transb, p, grid, st) : run_rows_tj<4, 1>(transb, p, grid, st);
      break;
    case 2: st1 = run_rows_tj<4, 2>(transb, p, grid, st); break;
    case 4: st1 = run_rows_tj<4, 4>(transb, p, grid, st); break;
    default: st1 = run_rows_tj<4, 8>(transb, p, grid, st); break;
  }
  TRY(st1);
  if (f.ranges > 1 && !defer_reduce) {
    const int64_t n = M * r;
    TRY(reduce_bf16(transb ? "reduce_dz" : "reduce_z", part, f.ranges, n, n, o1, a1, o2, a2, st));
  }
  return LORA4_OK;
}

lora4_status z_pass(const Plan &pl, const lora4_W *W, const uint16_t *X, const uint16_t *A,
                    const int64_t *offs, uint16_t *z1, float a1, uint16_t *z2, float a2, float *part,
                    bool defer_reduce, hipStream_t st) {
  if (!z1) {   // one output only
    z1 = z2;
    a1 = a2;
    z2 = nullptr;
  }
  return rows_skinny(0, X, pl.K, A, pl.K, (int64_t)pl.r * pl.K, pl.K, pl.M, pl.r, offs, pl.E, z1, a1, z2, a2, part, defer_reduce,
                     st);
}

lora4_status check_common(const Base &b, int64_t M, int32_t r, float s, const int64_t *offs) {
  TRY(check_W(b.W));
  if (b.shared && (b.W->groups != 1 || b.E < 1 || b.E > 65535)) return LORA4_ERR_SHAPE;
  if (M < 0 || M > (int64_t(1) << 31)) return LORA4_ERR_SHAPE;
  if (r < 1 || r > 256) return LORA4_ERR_SHAPE;
  if (!std::isfinite(s)) return LORA4_ERR_SHAPE;
  if (b.E > 1 && !offs) return LORA4_ERR_NULL;
  if (b.E == 1 && offs) return LORA4_ERR_SHAPE;
  return LORA4_OK;
}

// ---------------------------------------------------------------------------
// MX-native forward: MXFP8 activations times an MXFP4 base on the scaled MFMA
// ---------------------------------------------------------------------------

// Split schedule of the MX GEMM: the same rule as the bf16 forward's (few
// output tiles split the reduction), without its choice of tile path.
FwdSched mx_sched(int64_t M, int64_t N, int64_t K) {
  FwdSched f{true, 0, 0, 1, 1 << 30, 0, false};
  const int64_t cus = cu_count();
  const int64_t tiles = ceil_div(std::max<int64_t>(M, 1), mx::BM) * ceil_div(N, mx::BN);
  const int64_t steps = ceil_div(K, mx::BKS);
  const int64_t max_ks = std::min<int64_t>(16, std::max<int64_t>(1, steps / 8));
  int64_t ks = 1;
  if (tiles < cus * 3 / 4) {
    ks = std::min<int64_t>(cus / tiles, max_ks);
    const int64_t cap = ((int64_t)256 << 20) / ((int64_t)mx::BM * mx::BN * 4 * tiles);
    ks = std::max<int64_t>(1, std::min(ks, cap));
  }
  if (ks > 1) {
    f.split_tiles = (int)tiles;
    f.split_steps = (int)ceil_div(steps, ks);
    f.ksplit = (int)ceil_div(steps, f.split_steps);
  } else {
    f.whole_tiles = (int)tiles;
  }
  return f;
}

// Workspace of the MX forward: the plain forward's s Z and rank-r partials,
// then the split partials, the MXFP8 codes [Mp][Kp] and their scales.
struct MxPlan {
  Plan pl;
  FwdSched fs;
  int64_t Mp, Kp;
  size_t off_party, off_x8, off_xs, bytes;
};

MxPlan make_mx_plan(const lora4_W *W, int64_t M, int r) {
  MxPlan q;
  q.pl = make_plan(0, Base{W, 1, false}, M, r);
  q.fs = mx_sched(M, W->N, W->K);
  q.Mp = ceil_div(std::max<int64_t>(M, 1), mx::BM) * mx::BM;
  q.Kp = ceil_div(W->K, mx::BKS) * mx::BKS;
  size_t off = q.pl.off_party;
  q.off_party = off;
  if (q.fs.split_tiles > 0) off += align256((size_t)q.fs.split_tiles * q.fs.ksplit * mx::BM * mx::BN * 4);
  q.off_x8 = off;
  off += align256((size_t)q.Mp * q.Kp);
  q.off_xs = off;
  off += align256((size_t)(q.Kp / 64) * (q.Mp / 256) * 512);
  q.bytes = off;
  return q;
}

lora4_status check_mx(const lora4_W *W, int64_t M, int32_t r, float s) {
  TRY(check_common(Base{W, 1, false}, M, r, s, nullptr));
  if (W->format != LORA4_MXFP4) return LORA4_ERR_FORMAT;
  if (W->groups != 1) return LORA4_ERR_SHAPE;
  // 32-bit buffer offsets: one row tile of codes, the scale table, the base
  const int64_t Mp = ceil_div(std::max<int64_t>(M, 1), mx::BM) * mx::BM, Kp = ceil_div(W->K, mx::BKS) * mx::BKS;
  if ((int64_t)mx::BM * Kp > 0x7FFFFFFF || (Kp / 64) * (Mp / 256) * 512 > 0x7FFFFFFF) return LORA4_ERR_SHAPE;
  if (w_blocks(W->K) * 2048 > 0x7FFFFFFF) return LORA4_ERR_SHAPE;
  return LORA4_OK;
}

// ---------------------------------------------------------------------------
// LoftQ: host steps of the subspace iteration
// ---------------------------------------------------------------------------

constexpr int LOFTQ_OVERSAMPLE = 16;   // columns beyond r in the subspace
constexpr int LOFTQ_POWER = 8;         // power iterations (R R^T applied 8 times)

constexpr int LOFTQ_MAX_SPLIT = 64;             // reduction ranges of one product
constexpr int64_t LOFTQ_TARGET_WG = 1024;        // workgroups wanted per product
constexpr size_t LOFTQ_PART_BYTES = 64u << 20;   // fp32 partials of the split products

struct LoftqPlan {
  int c;
  size_t off_T, off_R, off_Y, off_Y2, off_Z, off_Z2, off_G, off_M, off_B, off_AT, off_P, part_bytes, bytes;
};

LoftqPlan make_loftq_plan(int64_t N, int64_t K, int r) {
  LoftqPlan p{};
  p.c = r + LOFTQ_OVERSAMPLE;
  size_t off = 0;
  auto take = [&](size_t b) {
    const size_t o = off;
    off += align256(b);
    return o;
  };
  p.off_T = take((size_t)N * K * 2);
  p.off_R = take((size_t)N * K * 4);
  p.off_Y = take((size_t)N * p.c * 4);
  p.off_Y2 = take((size_t)N * p.c * 4);
  p.off_Z = take((size_t)K * p.c * 4);
  p.off_Z2 = take((size_t)K * p.c * 4);
  p.off_G = take((size_t)p.c * p.c * 4);
  p.off_M = take((size_t)p.c * p.c * 4);
  p.off_B = take((size_t)N * r * 4);
  p.off_AT = take((size_t)K * r * 4);
  p.off_P = take(std::max(LOFTQ_PART_BYTES, (size_t)LOFTQ_MAX_SPLIT * p.c * p.c * 4));   // split partials
  p.part_bytes = std::max(LOFTQ_PART_BYTES, (size_t)LOFTQ_MAX_SPLIT * p.c * p.c * 4);
  p.bytes = off;
  return p;
}

// out = X M or X^T M (k_mat). The reduction is split over enough ranges to
// give the grid ~LOFTQ_TARGET_WG workgroups (at most LOFTQ_MAX_SPLIT, at
// least 256 reduction rows each, partials within `part_bytes` of `parts`),
// the fp32 partials summed in order afterwards.
lora4_status run_mat(bool trans, const float *X, int64_t ldx, int64_t rows, int64_t inner, const float *M, int c,
                     float *out, float *parts, size_t part_bytes, hipStream_t st) {
  const int64_t tiles = ceil_div(rows, loftq::MAT_ROWS), cblocks = ceil_div(c, loftq::MAT_COLS);
  int64_t S = std::min<int64_t>({ceil_div(LOFTQ_TARGET_WG, tiles * cblocks), LOFTQ_MAX_SPLIT,
                                 std::max<int64_t>(1, inner / 256),
                                 std::max<int64_t>(1, (int64_t)(part_bytes / ((size_t)rows * c * 4)))});
  S = std::max<int64_t>(1, S);
  const int64_t per = ceil_div(inner, S * loftq::MAT_CHUNK) * loftq::MAT_CHUNK;
  S = ceil_div(inner, per);
  const dim3 grid((unsigned)tiles, (unsigned)S, (unsigned)cblocks);
  float *dst = S > 1 ? parts : out;
  if (trans)
    TRY(launch_args("loftq_mat_tn", loftq::k_mat<true>, grid, dim3(256), st, X, ldx, rows, inner, M, c, dst, per));
  else
    TRY(launch_args("loftq_mat_nn", loftq::k_mat<false>, grid, dim3(256), st, X, ldx, rows, inner, M, c, dst, per));
  if (S == 1) return LORA4_OK;
  const int64_t n = rows * c;
  return launch_args("loftq_sum", loftq::k_sum_parts, dim3((unsigned)ceil_div(n, 256)), dim3(256), st,
                     (const float *)parts, (int)S, n, out);
}

// c x c Gram matrix of the columns of Y [rows][c] to the host (double).
lora4_status gram_to_host(const float *Y, int64_t rows, int c, float *G_dev, float *parts, size_t part_bytes,
                          std::vector<double> &G, hipStream_t st) {
  TRY(run_mat(true, Y, c, c, rows, Y, c, G_dev, parts, part_bytes, st));
  std::vector<float> g((size_t)c * c);
  if (hipMemcpyAsync(g.data(), G_dev, g.size() * 4, hipMemcpyDeviceToHost, st) != hipSuccess) return LORA4_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return LORA4_ERR_HIP;
  G.assign(g.begin(), g.end());
  return LORA4_OK;
}

lora4_status upload(const std::vector<double> &M, float *dst, hipStream_t st, std::vector<float> &stage) {
  stage.assign(M.begin(), M.end());
  if (hipMemcpyAsync(dst, stage.data(), stage.size() * 4, hipMemcpyHostToDevice, st) != hipSuccess)
    return LORA4_ERR_HIP;
  return hipStreamSynchronize(st) == hipSuccess ? LORA4_OK : LORA4_ERR_HIP;   // (stage is reused)
}

// Orthonormalize the columns of Y [rows][c] (CholeskyQR, twice): Y <- Y L^-T
// with Y^T Y = L L^T. A Gram matrix that is not positive definite (Y of lower
// rank) gets a small diagonal shift. The factor is computed on the device
// (k_chol_inv) where c <= CHOL_MAX_C, else on the host, by the same steps.
lora4_status orthonormalize(float *Y, float *tmp, int64_t rows, int c, float *G_dev, float *M_dev, float *parts,
                            size_t part_bytes, hipStream_t st) {
  if (c <= loftq::CHOL_MAX_C) {   // the factor on the device: no host round trip
    for (int pass = 0; pass < 2; ++pass) {
      TRY(run_mat(true, Y, c, c, rows, Y, c, G_dev, parts, part_bytes, st));
      TRY(launch_args("loftq_chol", loftq::k_chol_inv, dim3(1), dim3(256), st, (const float *)G_dev, c, M_dev));
      TRY(run_mat(false, Y, c, rows, c, M_dev, c, tmp, parts, part_bytes, st));
      if (hipMemcpyAsync(Y, tmp, (size_t)rows * c * 4, hipMemcpyDeviceToDevice, st) != hipSuccess)
        return LORA4_ERR_HIP;
    }
    return LORA4_OK;
  }
  std::vector<double> G, M((size_t)c * c), L((size_t)c * c);
  std::vector<float> stage;
  for (int pass = 0; pass < 2; ++pass) {
    TRY(gram_to_host(Y, rows, c, G_dev, parts, part_bytes, G, st));
    double tr = 0;
    for (int i = 0; i < c; ++i) tr += G[(size_t)i * c + i];
    const double eps = 1e-12 * (tr > 0 ? tr : 1.0);
    std::fill(L.begin(), L.end(), 0.0);
    for (int j = 0; j < c; ++j) {
      double d = G[(size_t)j * c + j] + eps;
      for (int k = 0; k < j; ++k) d -= L[(size_t)j * c + k] * L[(size_t)j * c + k];
      d = d > eps ? std::sqrt(d) : std::sqrt(eps);
      L[(size_t)j * c + j] = d;
      for (int i = j + 1; i < c; ++i) {
        double v = G[(size_t)i * c + j];
        for (int k = 0; k < j; ++k) v -= L[(size_t)i * c + k] * L[(size_t)j * c + k];
        L[(size_t)i * c + j] = v / d;
      }
    }
    // M = L^-T (upper triangular): solve L^T M = I column by column
    std::fill(M.begin(), M.end(), 0.0);
    for (int col = 0; col < c; ++col)
      for (int i = c - 1; i >= 0; --i) {
        double v = (i == col) ? 1.0 : 0.0;
        for (int k = c - 1; k > i; --k) v -= L[(size_t)k * c + i] * M[(size_t)k * c + col];
        M[(size_t)i * c + col] = v / L[(size_t)i * c + i];
      }
    TRY(upload(M, M_dev, st, stage));
    TRY(run_mat(false, Y, c, rows, c, M_dev, c, tmp, parts, part_bytes, st));
    if (hipMemcpyAsync(Y, tmp, (size_t)rows * c * 4, hipMemcpyDeviceToDevice, st) != hipSuccess) return LORA4_ERR_HIP;
  }
  return LORA4_OK;
}

// Eigen-decomposition of a symmetric c x c matrix (cyclic Jacobi): values in
// descending order, vectors as columns of V.
void jacobi_eigen(std::vector<double> A, int c, std::vector<double> &vals, std::vector<double> &V) {
  V.assign((size_t)c * c, 0.0);
  for (int i = 0; i < c; ++i) V[(size_t)i * c + i] = 1.0;
  for (int sweep = 0; sweep < 100; ++sweep) {
    double off = 0, tot = 0;
    for (int i = 0; i < c; ++i)
      for (int j = 0; j < c; ++j) {
        const double a = A[(size_t)i * c + j] * A[(size_t)i * c + j];
        tot += a;
        if (i != j) off += a;
      }
    if (off <= 1e-30 * (tot > 0 ? tot : 1.0)) break;
    for (int p = 0; p < c - 1; ++p)
      for (int q = p + 1; q < c; ++q) {
        const double apq = A[(size_t)p * c + q];
        if (apq == 0.0) continue;
        const double theta = (A[(size_t)q * c + q] - A[(size_t)p * c + p]) / (2 * apq);
        const double t = (theta >= 0 ? 1.0 : -1.0) / (std::fabs(theta) + std::sqrt(theta * theta + 1));
        const double cs = 1 / std::sqrt(t * t + 1), sn = t * cs;
        for (int k = 0; k < c; ++k) {   // A <- A J (columns p, q)
          const double akp = A[(size_t)k * c + p], akq = A[(size_t)k * c + q];
          A[(size_t)k * c + p] = cs * akp - sn * akq;
          A[(size_t)k * c + q] = sn * akp + cs * akq;
        }
        for (int k = 0; k < c; ++k) {   // A <- J^T A (rows p, q)
          const double apk = A[(size_t)p * c + k], aqk = A[(size_t)q * c + k];
          A[(size_t)p * c + k] = cs * apk - sn * aqk;
          A[(size_t)q * c + k] = sn * apk + cs * aqk;
        }
        for (int k = 0; k < c; ++k) {   // V <- V J
          const double vkp = V[(size_t)k * c + p], vkq = V[(size_t)k * c + q];
          V[(size_t)k * c + p] = cs * vkp - sn * vkq;
          V[(size_t)k * c + q] = sn * vkp + cs * vkq;
        }
      }
  }
  std::vector<int> idx(c);
  for (int i = 0; i < c; ++i) idx[i] = i;
  std::sort(idx.begin(), idx.end(), [&](int a, int b) { return A[(size_t)a * c + a] > A[(size_t)b * c + b]; });
  std::vector<double> V2((size_t)c * c);
  vals.resize(c);
  for (int j = 0; j < c; ++j) {
    vals[j] = A[(size_t)idx[j] * c + idx[j]];
    for (int i = 0; i < c; ++i) V2[(size_t)i * c + j] = V[(size_t)i * c + idx[j]];
  }
  V.swap(V2);
}

template <bool GEMM>
lora4_status run_quant_mxfp8(const uint16_t *X, int64_t ldx, int64_t M, int64_t K, uint8_t *codes, int64_t ldc,
                             int64_t Mp, int64_t Kp, uint8_t *scales, hipStream_t st) {
  const int64_t n = ceil_div(Mp, 256) * ceil_div(Kp, 256);   // one workgroup per 256 rows x 256 columns
  if (n > 0x7FFFFFFF) return LORA4_ERR_SHAPE;
  return launch_args("quant_mxfp8", mx::k_quant_mxfp8<GEMM>, dim3((unsigned)n), dim3(256), st, X, ldx, M, K, codes,
                     ldc, Mp, Kp, scales);
}

}  // namespace

// ---------------------------------------------------------------------------
// Scratch of the allocation-free forward: one static device array that every
// GPU the library runs on holds (its own copy) until the process ends. Host
// code never uses the array's name as an address: the device address is
// taken once per device with hipGetSymbolAddress, with that device current.
// ---------------------------------------------------------------------------

static __device__ __attribute__((aligned(256))) unsigned char scratch[LORA4_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[MAX_DEVICES] = {};

// The current device's copy of `scratch` (looked up on its first use there).
lora4_status scratch_for_current_device(void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return LORA4_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return LORA4_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return LORA4_OK;
}

// Grid of the packers that take one lane per 8 elements (grid-strided past
// PACK_MAX_BLOCKS workgroups).
dim3 pack_grid(int64_t N, int64_t K) {
  return dim3((unsigned)std::min<int64_t>(ceil_div(N * (K / 8), PACK_THREADS), PACK_MAX_BLOCKS));
}

}  // namespace

// ===========================================================================
// Exported C ABI
// ===========================================================================

#pragma GCC visibility push(default)
extern "C" {

const char *lora4_version(void) { return "lora4 0.1 (gfx950)"; }

const char *lora4_status_string(lora4_status s) {
  switch (s) {
    case LORA4_OK: return "ok";
    case LORA4_ERR_NULL: return "a required pointer is NULL";
    case LORA4_ERR_SHAPE: return "a size is out of range or inconsistent";
    case LORA4_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case LORA4_ERR_FORMAT: return "unknown format or block size";
    case LORA4_ERR_WORKSPACE: return "workspace missing or too small";
    case LORA4_ERR_HIP: return "a HIP call or kernel launch failed";
    case LORA4_ERR_UNIMPLEMENTED: return "not supported by the library";
    case LORA4_ERR_SCRATCH: return "request needs more than the allocation-free scratch holds";
  }
  return "unknown status";
}

static size_t workspace_bytes_of(int which, const Base &b, int64_t M, int32_t r) {
  if ((which != 0 && which != 1) || check_W(b.W) != LORA4_OK || M < 0 || r < 1 || r > 256) return 0;
  if (b.shared && (b.W->groups != 1 || b.E < 1 || b.E > 65535)) return 0;
  return make_plan(which, b, M, r).bytes;
}

size_t lora4_workspace_bytes(int which, const lora4_W *W, int64_t M, int32_t r) {
  if (!W) return 0;
  return workspace_bytes_of(which, Base{W, W->groups, false}, M, r);
}

size_t lora4_workspace_bytes_multi(int which, const lora4_W *W, int64_t adapters, int64_t M, int32_t r) {
  if (!W) return 0;
  return workspace_bytes_of(which, Base{W, adapters, true}, M, r);
}

static lora4_status forward_impl(const Base &bs, const uint16_t *X, int64_t M, const uint16_t *A,
                           const uint16_t *B, int32_t r, float s, const int64_t *group_offsets,
                           uint16_t *Y, uint16_t *Z, uint16_t *Y_base, uint16_t *Y_lora,
                           void *workspace, size_t workspace_bytes, void *stream, size_t cap = SIZE_MAX) {
  TRY(check_common(bs, M, r, s, group_offsets));
  const lora4_W *W = bs.W;
  if (!A || !B || (M > 0 && (!X || !Y))) return LORA4_ERR_NULL;
  for (const void *q : {(const void *)X, (const void *)A, (const void *)B, (const void *)Y, (const void *)Z,
                        (const void *)Y_base, (const void *)Y_lora, (const void *)group_offsets})
    if (q && !aligned16(q)) return LORA4_ERR_ALIGN;
  const Plan pl = make_plan(0, bs, M, r, cap);
  if (cap != SIZE_MAX && pl.bytes > cap) return LORA4_ERR_SCRATCH;
  if (!workspace) return LORA4_ERR_WORKSPACE;
  if (!aligned16(workspace)) return LORA4_ERR_ALIGN;
  if (workspace_bytes < pl.bytes) return LORA4_ERR_WORKSPACE;
  if (M == 0) return LORA4_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);

  // Z = X A^T. With the reduction split into ranges and the register-direct
  // base kernel, that kernel's tail adds the fp32 range partials itself (and
  // its column-tile-0 blocks store Z, and s Z for a Y_lora pass); otherwise
  // the partials are reduced into Z and s Z here.
  uint16_t *sZ = ws_at<uint16_t>(workspace, pl.off_sz);
  float *skpart = ws_at<float>(workspace, pl.off_skpart);
  const SkSched zs = sk_sched(M, pl.K, r, pl.E, 0);
  const bool z_tail = zs.ranges > 1 && zs.ranges <= big::A2_MAX_PARTS && fwd_regs_taken(pl.K, pl);
  const TailParts ztp{skpart, zs.ranges, s, Z, 1.0f, Y_lora ? sZ : nullptr, s};
  TRY(z_pass(pl, W, X, A, group_offsets, Z, 1.0f, sZ, s, skpart, z_tail, st));

  NtParams p{};
  p.A = mat(X, pl.K);
  p.W = packed_of(bs);
  p.R = pl.K;
  p.A2 = mat(sZ, r);
  p.B2 = mat(B, r, pl.N * r);
  p.r2 = r;
  p.M = M;
  p.Nc = pl.N;
  p.offsets = group_offsets;
  p.groups = (int)pl.E;
  p.Rsplit = pl.K;
  p.out = GemmOut{Y, pl.N, nullptr, 0, 1.0f};
  p.tab = nf4_table();
  dim3 grid((unsigned)ceil_div(pl.N, BN_MAIN), (unsigned)pl.row_slots, 1);
  float *party = ws_at<float>(workspace, pl.off_party);
  float *partx = ws_at<float>(workspace, pl.off_partx);
  TRY(run_nt_main_fmt(W->format, p, grid, pl, party, partx, z_tail ? &ztp : nullptr, st));
  if (Y_base) {
    NtParams q = p;
    q.r2 = 0;
    q.out.C = Y_base;
    TRY(run_nt_main_fmt(W->format, q, grid, pl, party, partx, nullptr, st));
  }
  if (Y_lora) {
    NtParams q = p;
    q.R = 0;
    q.Rsplit = 64;
    q.out.C = Y_lora;
    TRY(run_nt_main_fmt(W->format, q, grid, pl, party, partx, nullptr, st));
  }
  return LORA4_OK;
}

static lora4_status backward_impl(const Base &bs, const uint16_t *X, const uint16_t *dY, int64_t M,
                            const uint16_t *A, const uint16_t *B, int32_t r, float s,
                            const int64_t *group_offsets, const uint16_t *Z, uint16_t *dX,
                            uint16_t *dA, uint16_t *dB, void *workspace, size_t workspace_bytes,
                            void *stream) {
  TRY(check_common(bs, M, r, s, group_offsets));
  const lora4_W *W = bs.W;
  if (!A || !B || !dA || !dB || (M > 0 && (!X || !dY || !dX))) return LORA4_ERR_NULL;
  for (const void *q : {(const void *)X, (const void *)dY, (const void *)A, (const void *)B, (const void *)Z,
                        (const void *)dX, (const void *)dA, (const void *)dB, (const void *)group_offsets})
    if (q && !aligned16(q)) return LORA4_ERR_ALIGN;
  const Plan pl = make_plan(1, bs, M, r);
  if (!workspace) return LORA4_ERR_WORKSPACE;
  if (!aligned16(workspace)) return LORA4_ERR_ALIGN;
  if (workspace_bytes < pl.bytes) return LORA4_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (M == 0) {
    const int64_t na = pl.E * r * pl.K, nb = pl.E * pl.N * r;
    TRY(launch_args("fill_zero", k_fill_u16, dim3((unsigned)ceil_div(na, 256)), dim3(256), st, dA, na, (uint16_t)0));
    TRY(launch_args("fill_zero", k_fill_u16, dim3((unsigned)ceil_div(nb, 256)), dim3(256), st, dB, nb, (uint16_t)0));
    return LORA4_OK;
  }

  uint16_t *dZ = ws_at<uint16_t>(workspace, pl.off_dz);
  float *part = ws_at<float>(workspace, pl.off_part);
  const uint16_t *Zu = Z;
  if (!Zu) {
    uint16_t *Zw = ws_at<uint16_t>(workspace, pl.off_zw);
    TRY(z_pass(pl, W, X, A, group_offsets, Zw, 1.0f, nullptr, 0.0f, ws_at<float>(workspace, pl.off_skpart), false,
               st));
    Zu = Zw;
  }

  // dZ = s dY B  (row blocks, reduction over N). With the reduction split
  // into ranges and the 256 x 256 dgrad kernel, that kernel's tail adds the
  // fp32 range partials (its column-tile-0 blocks store dZ for the dA pass).
  float *skpart = ws_at<float>(workspace, pl.off_skpart);
  const SkSched dzs = sk_sched(M, pl.N, r, pl.E, 1);
  const bool dz_tail = dzs.ranges > 1 && dzs.ranges <= big::A2_MAX_PARTS &&
                       dgrad_taken(pl.N, pl.N, M, packed_of(bs), pl.K, pl.E);
  const TailParts dztp{skpart, dzs.ranges, s, dZ, s, nullptr, 0.0f};
  // (its first block also zeroes the dA / dB tiles' arrival counters)
  unsigned *cnt = ws_at<unsigned>(workspace, pl.off_cnt);
  TRY(rows_skinny(1, dY, pl.N, B, r, pl.N * r, pl.N, M, r, group_offsets, pl.E, dZ, s, nullptr, 0.0f, skpart,
                  dz_tail, st, cnt, pl.ncnt));

  // dX = dY deq(W) + dZ A
  {
    NnParams p{};
    p.A = mat(dY, pl.N);
    p.W = packed_of(bs);
    p.R = pl.N;
    p.A2 = mat(dZ, r);
    p.B2 = mat(A, pl.K, (int64_t)r * pl.K);
    p.r2 = r;
    p.M = M;
    p.Nc = pl.K;
    p.offsets = group_offsets;
    p.groups = (int)pl.E;
    p.Rsplit = pl.N;
    p.out = GemmOut{dX, pl.K, nullptr, 0, 1.0f};
    p.tab = nf4_table();
    dim3 grid((unsigned)ceil_div(pl.K, BN_MAIN), (unsigned)pl.row_slots, 1);
    TRY(run_nn_main_fmt(W->format, p, grid, pl, ws_at<float>(workspace, pl.off_partx), dz_tail ? &dztp : nullptr,
                        st));
  }

  // dA = dZ^T X and dB^T = Z^T dY, split over rows, in one launch; the last
  // block to finish each output tile reduces its splits (TnParams::cnt)
  float *part_b = ws_at<float>(workspace, pl.off_part_b);
  {
    TnParams pa{};
    pa.U = mat(dZ, r);
    pa.V = mat(X, pl.K);
    pa.P = r;
    pa.Q = pl.K;
    pa.M = M;
    pa.offsets = group_offsets;
    pa.groups = (int)pl.E;
    pa.splits = pl.msplit_a;
    pa.part = part;
    pa.cnt = cnt;
    pa.out = dA;
    pa.alpha = 1.0f;
    pa.transpose_out = 0;
    TnParams pb = pa;
    pb.U = mat(Zu, r);
    pb.V = mat(dY, pl.N);
    pb.Q = pl.N;
    pb.splits = pl.msplit_b;
    pb.part = part_b;
    pb.cnt = cnt + ceil_div(r, pl.rt) * pl.tq_a * pl.E;
    pb.out = dB;
    pb.alpha = s;
    pb.transpose_out = 1;
    TRY(run_tn2("gemm_tn_dA_dB", pl.rt, pa, pb, pl.tq_a, (int)(pl.msplit_a * pl.E), pl.tq_b,
                (int)(pl.msplit_b * pl.E), st));
  }
  return LORA4_OK;
}

lora4_status lora4_forward(const lora4_W *W, const uint16_t *X, int64_t M, const uint16_t *A,
                           const uint16_t *B, int32_t r, float s, const int64_t *group_offsets,
                           uint16_t *Y, uint16_t *Z, uint16_t *Y_base, uint16_t *Y_lora,
                           void *workspace, size_t workspace_bytes, void *stream) {
  if (!W) return LORA4_ERR_NULL;
  return forward_impl(Base{W, W->groups, false}, X, M, A, B, r, s, group_offsets, Y, Z, Y_base, Y_lora, workspace,
                      workspace_bytes, stream);
}

lora4_status lora4_forward_noalloc(const lora4_W *W, const uint16_t *X, int64_t M, const uint16_t *A,
                                   const uint16_t *B, int32_t r, float s, const int64_t *group_offsets,
                                   uint16_t *Y, uint16_t *Z, uint16_t *Y_base, uint16_t *Y_lora, void *stream) {
  if (!W) return LORA4_ERR_NULL;
  TRY(check_common(Base{W, W->groups, false}, M, r, s, group_offsets));
  void *ws = nullptr;
  TRY(scratch_for_current_device(&ws));
  struct Guard {
    Guard() { tl_no_alloc = true; }
    ~Guard() { tl_no_alloc = false; }
  } guard;
  return forward_impl(Base{W, W->groups, false}, X, M, A, B, r, s, group_offsets, Y, Z, Y_base, Y_lora, ws,
                      LORA4_NOALLOC_SCRATCH_BYTES, stream, LORA4_NOALLOC_SCRATCH_BYTES);
}

lora4_status lora4_backward(const lora4_W *W, const uint16_t *X, const uint16_t *dY, int64_t M,
                            const uint16_t *A, const uint16_t *B, int32_t r, float s,
                            const int64_t *group_offsets, const uint16_t *Z, uint16_t *dX,
                            uint16_t *dA, uint16_t *dB, void *workspace, size_t workspace_bytes,
                            void *stream) {
  if (!W) return LORA4_ERR_NULL;
  return backward_impl(Base{W, W->groups, false}, X, dY, M, A, B, r, s, group_offsets, Z, dX, dA, dB, workspace,
                       workspace_bytes, stream);
}

lora4_status lora4_forward_multi(const lora4_W *W, int64_t adapters, const uint16_t *X, int64_t M,
                                 const uint16_t *A, const uint16_t *B, int32_t r, float s,
                                 const int64_t *adapter_offsets, uint16_t *Y, uint16_t *Z, uint16_t *Y_base,
                                 uint16_t *Y_lora, void *workspace, size_t workspace_bytes, void *stream) {
  if (!W) return LORA4_ERR_NULL;
  return forward_impl(Base{W, adapters, true}, X, M, A, B, r, s, adapter_offsets, Y, Z, Y_base, Y_lora, workspace,
                      workspace_bytes, stream);
}

lora4_status lora4_backward_multi(const lora4_W *W, int64_t adapters, const uint16_t *X, const uint16_t *dY,
                                  int64_t M, const uint16_t *A, const uint16_t *B, int32_t r, float s,
                                  const int64_t *adapter_offsets, const uint16_t *Z, uint16_t *dX, uint16_t *dA,
                                  uint16_t *dB, void *workspace, size_t workspace_bytes, void *stream) {
  if (!W) return LORA4_ERR_NULL;
  return backward_impl(Base{W, adapters, true}, X, dY, M, A, B, r, s, adapter_offsets, Z, dX, dA, dB, workspace,
                       workspace_bytes, stream);
}

size_t lora4_packed_bytes(int32_t format, int64_t N, int64_t K, int32_t part) {
  // K granularity: the block (NF4: 64, MXFP4: 32); NVFP4 (16-element blocks) whole 32-element halves
  const int64_t block = format == LORA4_MXFP4 || format == LORA4_NVFP4 ? 32 : 64;
  if (format != LORA4_NF4 && format != LORA4_NF4_DQ && format != LORA4_MXFP4 && format != LORA4_NVFP4) return 0;
  if (N < 1 || K < block || K % block != 0 || N > (int64_t(1) << 31) || K > (int64_t(1) << 31)) return 0;
  const int64_t tiles = w_blocks(N) * w_blocks(K);
  switch (part) {
    case 0: return (size_t)(tiles * 2048);
    case 1:
      return (size_t)(tiles * (format == LORA4_MXFP4 ? 128 : format == LORA4_NF4 || format == LORA4_NVFP4 ? 256 : 64));
    case 2: return format == LORA4_NF4_DQ ? (size_t)(ceil_div(N * (K / 64), 256) * 4) : 0;
  }
  return 0;
}

// Clears a packed matrix's codes and scales when the tiles have padding (rows
// past N, elements past K), which the quant kernels do not write.
lora4_status clear_padding(int64_t N, int64_t K, int32_t format, uint8_t *codes, void *scales, hipStream_t st) {
  if (N % 64 == 0 && K % 64 == 0) return LORA4_OK;
  const int64_t nc = (int64_t)lora4_packed_bytes(format, N, K, 0) / 2;
  const int64_t ns = (int64_t)lora4_packed_bytes(format, N, K, 1) / 2;
  TRY(launch_args("fill_zero", k_fill_u16, dim3((unsigned)ceil_div(nc, 256)), dim3(256), st,
                  reinterpret_cast<uint16_t *>(codes), nc, (uint16_t)0));
  return launch_args("fill_zero", k_fill_u16, dim3((unsigned)ceil_div(ns, 256)), dim3(256), st,
                     reinterpret_cast<uint16_t *>(scales), ns, (uint16_t)0);
}

lora4_status quant_pack_nf4(const uint16_t *W_bf16, int64_t N, int64_t K, int32_t double_quant,
                            uint8_t *codes, void *scales, float *scales2, void *stream) {
  if (!W_bf16 || !codes || !scales) return LORA4_ERR_NULL;
  if (double_quant && !scales2) return LORA4_ERR_NULL;
  if (N < 1 || K < 64 || K % 64 != 0 || N > (int64_t(1) << 31) || K > (int64_t(1) << 31)) return LORA4_ERR_SHAPE;
  if (!aligned16(W_bf16) || !aligned16(codes) || !aligned16(scales) || (double_quant && !aligned4(scales2)))
    return LORA4_ERR_ALIGN;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  TRY(clear_padding(N, K, double_quant ? LORA4_NF4_DQ : LORA4_NF4, codes, scales, st));
  if (!double_quant) {
    return launch_args("quant_pack_nf4", k_quant_nf4, pack_grid(N, K), dim3(PACK_THREADS), st, W_bf16, N, K, codes,
                       reinterpret_cast<float *>(scales), nf4_table());
  }
  // one workgroup per second-level group of 256 blocks
  const int64_t nblk = N * (K / 64);
  return launch_args("quant_pack_nf4_dq", k_quant_nf4_dq, dim3((unsigned)ceil_div(nblk, 256)), dim3(PACK_THREADS),
                     st, W_bf16, N, K, codes, reinterpret_cast<uint8_t *>(scales), scales2, nf4_table());
}

lora4_status quant_pack_mxfp4(const uint16_t *W_bf16, int64_t N, int64_t K, uint8_t *codes,
                              uint8_t *scales_e8m0, void *stream) {
  if (!W_bf16 || !codes || !scales_e8m0) return LORA4_ERR_NULL;
  if (N < 1 || K < 32 || K % 32 != 0 || N > (int64_t(1) << 31) || K > (int64_t(1) << 31)) return LORA4_ERR_SHAPE;
  if (!aligned16(W_bf16) || !aligned16(codes) || !aligned16(scales_e8m0)) return LORA4_ERR_ALIGN;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  TRY(clear_padding(N, K, LORA4_MXFP4, codes, scales_e8m0, st));
  return launch_args("quant_pack_mxfp4", k_quant_mxfp4, pack_grid(N, K), dim3(PACK_THREADS), st, W_bf16, N, K,
                     codes, scales_e8m0);
}

lora4_status lora4_import_rowmajor(int32_t format, int64_t N, int64_t K, int64_t groups, const uint8_t *codes_rm,
                                   const void *scales_rm, uint8_t *codes, void *scales, void *stream) {
  if (format != LORA4_NF4 && format != LORA4_NF4_DQ && format != LORA4_MXFP4 && format != LORA4_NVFP4)
    return LORA4_ERR_FORMAT;
  const int64_t kmul = format == LORA4_NF4 || format == LORA4_NF4_DQ ? 64 : 32;
  if (N < 1 || K < kmul || K % kmul != 0 || groups < 1 || groups > 65535 || N > (int64_t(1) << 31) ||
      K > (int64_t(1) << 31))
    return LORA4_ERR_SHAPE;
  if (!codes_rm || !scales_rm || !codes || !scales) return LORA4_ERR_NULL;
  if (!aligned16(codes_rm) || !aligned16(scales_rm) || !aligned16(codes) || !aligned16(scales))
    return LORA4_ERR_ALIGN;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int64_t nc = groups * w_blocks(N) * w_blocks(K) * 128;   // 16-byte pieces of codes
  const int nf4 = format == LORA4_NF4 || format == LORA4_NF4_DQ ? 1 : 0;   // (nibble order of the storage)
  TRY(launch_args("import_codes", k_retile_codes, dim3((unsigned)ceil_div(nc, 256)), dim3(256), st, codes_rm, N,
                  K, groups, nf4, codes));
  const int epr = format == LORA4_MXFP4 ? 2 : format == LORA4_NVFP4 ? 4 : 1;
  const int64_t ns = groups * w_blocks(N) * w_blocks(K) * 64 * epr;
  const dim3 grid((unsigned)ceil_div(ns, 256));
  if (format == LORA4_NF4)
    return launch_args("import_scales", k_retile_scales<float>, grid, dim3(256), st,
                       reinterpret_cast<const float *>(scales_rm), N, K, groups, epr, reinterpret_cast<float *>(scales));
  return launch_args("import_scales", k_retile_scales<uint8_t>, grid, dim3(256), st,
                     reinterpret_cast<const uint8_t *>(scales_rm), N, K, groups, epr,
                     reinterpret_cast<uint8_t *>(scales));
}

lora4_status quant_pack_mxfp8(const uint16_t *X, int64_t M, int64_t K, uint8_t *codes, uint8_t *scales_e8m0,
                              void *stream) {
  if (M < 0 || K < 32 || K % 32 != 0 || M > (int64_t(1) << 31) || K > (int64_t(1) << 31)) return LORA4_ERR_SHAPE;
  if (M == 0) return LORA4_OK;
  if (!X || !codes || !scales_e8m0) return LORA4_ERR_NULL;
  if (!aligned16(X) || !aligned16(codes) || !aligned16(scales_e8m0)) return LORA4_ERR_ALIGN;
  return run_quant_mxfp8<false>(X, K, M, K, codes, K, M, K, scales_e8m0, reinterpret_cast<hipStream_t>(stream));
}

size_t lora4_workspace_bytes_mx(const lora4_W *W, int64_t M, int32_t r) {
  if (check_mx(W, M, r, 1.0f) != LORA4_OK) return 0;
  return make_mx_plan(W, M, r).bytes;
}

lora4_status lora4_forward_mx(const lora4_W *W, const uint16_t *X, int64_t M, const uint16_t *A, const uint16_t *B,
                              int32_t r, float s, uint16_t *Y, uint16_t *Z, void *workspace, size_t workspace_bytes,
                              void *stream) {
  TRY(check_mx(W, M, r, s));
  if (!A || !B || (M > 0 && (!X || !Y))) return LORA4_ERR_NULL;
  for (const void *q : {(const void *)X, (const void *)A, (const void *)B, (const void *)Y, (const void *)Z})
    if (q && !aligned16(q)) return LORA4_ERR_ALIGN;
  const MxPlan mp = make_mx_plan(W, M, r);
  const Plan &pl = mp.pl;
  if (!workspace) return LORA4_ERR_WORKSPACE;
  if (!aligned16(workspace)) return LORA4_ERR_ALIGN;
  if (workspace_bytes < mp.bytes) return LORA4_ERR_WORKSPACE;
  if (M == 0) return LORA4_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);

  uint8_t *x8 = ws_at<uint8_t>(workspace, mp.off_x8);
  uint8_t *xs = ws_at<uint8_t>(workspace, mp.off_xs);
  TRY(run_quant_mxfp8<true>(X, pl.K, M, pl.K, x8, mp.Kp, mp.Mp, mp.Kp, xs, st));

  // Z = X A^T from the bf16 X; the GEMM adds the range partials itself
  // where there are several (and its column-tile-0 blocks store Z)
  uint16_t *sZ = ws_at<uint16_t>(workspace, pl.off_sz);
  float *skpart = ws_at<float>(workspace, pl.off_skpart);
  const SkSched zs = sk_sched(M, pl.K, r, 1, 0);
  const bool z_tail = zs.ranges > 1 && zs.ranges <= big::A2_MAX_PARTS;
  const TailParts ztp{skpart, zs.ranges, s, Z, 1.0f, nullptr, 0.0f};
  TRY(z_pass(pl, W, X, A, nullptr, Z, 1.0f, sZ, s, skpart, z_tail, st));

  big::Params q = big_params(mat(X, pl.K), packed_of(Base{W, 1, false}), pl.K, mat(sZ, r), mat(B, r, pl.N * r), r, M,
                             pl.N, nullptr, 1, Y, pl.N);
  if (z_tail) apply_tail_parts(q, &ztp);
  q.X8 = x8;
  q.X8s = xs;
  q.ld8 = mp.Kp;
  q.ksplit = mp.fs.ksplit;
  q.split_steps = mp.fs.split_steps;
  q.nblocks = mp.fs.whole_tiles + mp.fs.split_tiles * mp.fs.ksplit;
  q.Cpart = ws_at<float>(workspace, mp.off_party);
  if (mp.fs.split_tiles > 0) {
    TRY(launch_lds("gemm_mx_base", mx::k_gemm_fwd_mx<true>, dim3((unsigned)q.nblocks), dim3(mx::THREADS),
                   (size_t)mx::lds_bytes(), q, st));
    const int64_t n = (int64_t)mp.fs.split_tiles * mx::BM * (mx::BN / 4);
    return launch_args("reduce_y", fwd::k_reduce_tiles, dim3((unsigned)ceil_div(n, 256)), dim3(256), st, q,
                       mp.fs.split_tiles);
  }
  return launch_lds("gemm_mx_base", mx::k_gemm_fwd_mx<false>, dim3((unsigned)q.nblocks), dim3(mx::THREADS),
                    (size_t)mx::lds_bytes(), q, st);
}

lora4_status quant_pack_nvfp4(const uint16_t *W_bf16, int64_t N, int64_t K, uint8_t *codes,
                              uint8_t *scales_e4m3, void *stream) {
  if (!W_bf16 || !codes || !scales_e4m3) return LORA4_ERR_NULL;
  if (N < 1 || K < 32 || K % 32 != 0 || N > (int64_t(1) << 31) || K > (int64_t(1) << 31)) return LORA4_ERR_SHAPE;
  if (!aligned16(W_bf16) || !aligned16(codes) || !aligned16(scales_e4m3)) return LORA4_ERR_ALIGN;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  TRY(clear_padding(N, K, LORA4_NVFP4, codes, scales_e4m3, st));
  return launch_args("quant_pack_nvfp4", k_quant_nvfp4, pack_grid(N, K), dim3(PACK_THREADS), st, W_bf16, N, K,
                     codes, scales_e4m3);
}

size_t lora4_loftq_workspace_bytes(int64_t N, int64_t K, int32_t r) {
  if (N < 1 || K < 64 || K % 64 != 0 || N > (int64_t(1) << 31) || K > (int64_t(1) << 31)) return 0;
  if (r < 1 || r > 128 || r + LOFTQ_OVERSAMPLE > N || r + LOFTQ_OVERSAMPLE > K) return 0;
  return make_loftq_plan(N, K, r).bytes;
}

lora4_status lora4_loftq_init(const uint16_t *W, int64_t N, int64_t K, int32_t r, int32_t iters, float s,
                              int32_t double_quant, uint8_t *codes, void *scales, float *scales2, uint16_t *A,
                              uint16_t *B, void *workspace, size_t workspace_bytes, void *stream) {
  if (!W || !codes || !scales || !A || !B || (double_quant && !scales2)) return LORA4_ERR_NULL;
  if (N < 1 || K < 64 || K % 64 != 0 || N > (int64_t(1) << 31) || K > (int64_t(1) << 31)) return LORA4_ERR_SHAPE;
  if (r < 1 || r > 128 || r + LOFTQ_OVERSAMPLE > N || r + LOFTQ_OVERSAMPLE > K) return LORA4_ERR_SHAPE;
  if (iters < 1 || iters > 64 || !std::isfinite(s) || s == 0.0f) return LORA4_ERR_SHAPE;
  for (const void *q : {(const void *)W, (const void *)codes, (const void *)scales, (const void *)A,
                        (const void *)B})
    if (!aligned16(q)) return LORA4_ERR_ALIGN;
  if (scales2 && !aligned4(scales2)) return LORA4_ERR_ALIGN;
  const LoftqPlan lp = make_loftq_plan(N, K, r);
  if (!workspace) return LORA4_ERR_WORKSPACE;
  if (!aligned16(workspace)) return LORA4_ERR_ALIGN;
  if (workspace_bytes < lp.bytes) return LORA4_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int c = lp.c;
  uint16_t *T = ws_at<uint16_t>(workspace, lp.off_T);
  float *R = ws_at<float>(workspace, lp.off_R), *Y = ws_at<float>(workspace, lp.off_Y);
  float *Y2 = ws_at<float>(workspace, lp.off_Y2), *Z = ws_at<float>(workspace, lp.off_Z);
  float *Z2 = ws_at<float>(workspace, lp.off_Z2), *G = ws_at<float>(workspace, lp.off_G);
  float *Md = ws_at<float>(workspace, lp.off_M), *Bf = ws_at<float>(workspace, lp.off_B);
  float *ATf = ws_at<float>(workspace, lp.off_AT);
  float *P = ws_at<float>(workspace, lp.off_P);
  const size_t PB = lp.part_bytes;
  const lora4_W Wq{double_quant ? LORA4_NF4_DQ : LORA4_NF4, 64, N, K, 1, codes, scales, scales2};
  const PackedW Qp = packed_of(Base{&Wq, 1, false});
  const int64_t nk = N * K;
  std::vector<double> Gh, vals, V, Mh;
  std::vector<float> stage;
  for (int it = 0; it < iters; ++it) {
    // Q_t = NF4(bf16(W - B_{t-1} A_{t-1})), R_t = W - Q_t
    TRY(launch_args("loftq_shift", loftq::k_shift, dim3((unsigned)ceil_div(nk / 8, 256)), dim3(256), st, W,
                    (const float *)Bf, (const float *)ATf, N, K, it == 0 ? 0 : (int)r, T));
    TRY(quant_pack_nf4(T, N, K, double_quant, codes, scales, scales2, stream));
    const dim3 rg((unsigned)ceil_div(N * (K / 32), 256));
    if (double_quant)
      TRY(launch_args("loftq_residual", loftq::k_residual<FMT_NF4_DQ>, rg, dim3(256), st, W, Qp, nf4_table(), R));
    else
      TRY(launch_args("loftq_residual", loftq::k_residual<FMT_NF4>, rg, dim3(256), st, W, Qp, nf4_table(), R));
    // top-r subspace of R: Y = orth(R Omega), then (R R^T) applied LOFTQ_POWER times
    TRY(launch_args("loftq_start", loftq::k_rademacher, dim3((unsigned)ceil_div(K * c, 256)), dim3(256), st, Z2,
                    K * c, (uint64_t)0x5EED0000u + (uint64_t)it));
    TRY(run_mat(false, R, K, N, K, Z2, c, Y, P, PB, st));
    TRY(orthonormalize(Y, Y2, N, c, G, Md, P, PB, st));
    for (int q = 0; q < LOFTQ_POWER; ++q) {
      TRY(run_mat(true, R, K, K, N, Y, c, Z, P, PB, st));
      TRY(orthonormalize(Z, Z2, K, c, G, Md, P, PB, st));
      TRY(run_mat(false, R, K, N, K, Z, c, Y, P, PB, st));
      TRY(orthonormalize(Y, Y2, N, c, G, Md, P, PB, st));
    }
    // R ~ Y Z^T with Z = R^T Y; Z^T = U S V^T from the eigenvectors of Z^T Z:
    // B = Y U_r S_r^(1/2), A^T = Z U_r S_r^(-1/2)
    TRY(run_mat(true, R, K, K, N, Y, c, Z, P, PB, st));
    TRY(gram_to_host(Z, K, c, G, P, PB, Gh, st));
    jacobi_eigen(Gh, c, vals, V);
    const double smax = vals[0] > 0 ? std::sqrt(vals[0]) : 0.0;
    Mh.assign((size_t)c * r, 0.0);
    for (int i = 0; i < c; ++i)
      for (int j = 0; j < r; ++j) {
        const double sg = vals[j] > 0 ? std::sqrt(vals[j]) : 0.0;
        Mh[(size_t)i * r + j] = V[(size_t)i * c + j] * std::sqrt(sg);
      }
    TRY(upload(Mh, Md, st, stage));
    TRY(run_mat(false, Y, c, N, c, Md, r, Bf, P, PB, st));
    for (int i = 0; i < c; ++i)
      for (int j = 0; j < r; ++j) {
        const double sg = vals[j] > 0 ? std::sqrt(vals[j]) : 0.0;
        Mh[(size_t)i * r + j] = sg > 1e-30 * (smax > 0 ? smax : 1.0) ? V[(size_t)i * c + j] / std::sqrt(sg) : 0.0;
      }
    TRY(upload(Mh, Md, st, stage));
    TRY(run_mat(false, Z, c, K, c, Md, r, ATf, P, PB, st));
  }
  TRY(launch_args("loftq_out", loftq::k_to_bf16, dim3((unsigned)ceil_div(N * r, 256)), dim3(256), st,
                  (const float *)Bf, N * r, 1.0f / s, B));
  return launch_args("loftq_out", loftq::k_to_bf16_t, dim3((unsigned)ceil_div(K * r, 256)), dim3(256), st,
                     (const float *)ATf, K, (int)r, 1.0f, A);
}

lora4_status lora4_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_tmu);
  g_timing = on != 0;
  return LORA4_OK;
}

int lora4_timing_collect(lora4_kernel_time *out, int max) {
  std::vector<PendingTiming> pend;
  {
    std::lock_guard<std::mutex> lk(g_tmu);
    pend.swap(g_pending);
  }
  std::map<std::string, std::pair<int64_t, double>> agg;
  std::vector<std::string> order;
  lora4_status st = LORA4_OK;
  for (auto &t : pend) {
    float ms = 0.f;
    if (hipEventSynchronize(t.b) != hipSuccess || hipEventElapsedTime(&ms, t.a, t.b) != hipSuccess) {
      st = LORA4_ERR_HIP;
    }
    auto it = agg.find(t.name);
    if (it == agg.end()) {
      order.push_back(t.name);
      agg[t.name] = {1, (double)ms};
    } else {
      it->second.first += 1;
      it->second.second += ms;
    }
  }
  {
    std::lock_guard<std::mutex> lk(g_tmu);
    for (auto &t : pend) {
      g_free_events.push_back(t.a);
      g_free_events.push_back(t.b);
    }
  }
  if (st != LORA4_OK) return (int)st;
  int n = 0;
  for (auto &name : order) {
    if (out && n < max) {
      std::memset(out[n].name, 0, sizeof(out[n].name));
      std::strncpy(out[n].name, name.c_str(), sizeof(out[n].name) - 1);
      out[n].launches = agg[name].first;
      out[n].total_ms = agg[name].second;
    }
    ++n;
  }
  return n;
}

}  // extern "C"
#pragma GCC visibility pop
