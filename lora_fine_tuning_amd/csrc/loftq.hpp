// Device pieces of the LoftQ initialisation ("Training LLMs on a Budget",
// section 4: alternate NF4 quantization of W - B A with the best rank-r
// approximation of the residual W - Q). The rank-r approximation is found by
// randomized subspace iteration on the fp32 residual: the products R M and
// R^T M run in k_mat (deterministic fp32 sums), the small c x c steps
// (Cholesky for the orthonormalization, the eigen-decomposition of the
// projected Gram matrix) on the host.
#pragma once

#include "formats.hpp"

namespace lora4 {
namespace loftq {

constexpr int MAT_ROWS = 256;   // output rows per workgroup of k_mat
constexpr int MAT_COLS = 32;    // output columns per workgroup (blockIdx.z: column block)
constexpr int MAT_CHUNK = 16;   // reduction rows per LDS stage

// Up to four consecutive floats at p (n valid, zero past them; one 16-byte
// load where vec and all four are valid).
__device__ __forceinline__ f32x4_t load4f(const float *p, int64_t n, bool vec) {
  f32x4_t v = {0.f, 0.f, 0.f, 0.f};
  if (vec && n >= 4) return *reinterpret_cast<const f32x4_t *>(p);
  for (int e = 0; e < 4; ++e)
    if (e < n) v[e] = p[e];
  return v;
}

// out[o][j] = sum_t X(o, t) M[t][j] for o < rows, j < c, t < inner, with
// X(o, t) = X[o][t] (TRANS = false, X is [rows][ldx]) or X[t][o] (TRANS =
// true, X is [inner][ldx]); M is [inner][c], out [rows][c], all fp32. A
// workgroup owns 256 output rows x 32 columns (blockIdx.x, blockIdx.z) over
// one reduction range (blockIdx.y: t in [y per_split, (y + 1) per_split),
// written to out + y rows c); thread i owns rows 4 (i / 4) .. +3 and columns
// 8 (i % 4) .. +7. The range streams through two LDS stages of 16 reduction
// rows (the next stage's loads in flight during this one's FMAs), and every
// output sums its range in order (deterministic).
template <bool TRANS>
__global__ __launch_bounds__(256) void k_mat(const float *X, int64_t ldx, int64_t rows, int64_t inner,
                                             const float *M, int c, float *out, int64_t per_split) {
  __shared__ __attribute__((aligned(16))) float xs[2][MAT_CHUNK][MAT_ROWS + 4];
  __shared__ __attribute__((aligned(16))) float ms[2][MAT_CHUNK][MAT_COLS];
  const int t = threadIdx.x;
  const int64_t o0 = (int64_t)blockIdx.x * MAT_ROWS;
  const int j0 = blockIdx.z * MAT_COLS;
  const int64_t t_lo = (int64_t)blockIdx.y * per_split;
  const int64_t t_hi = t_lo + per_split < inner ? t_lo + per_split : inner;
  out += (int64_t)blockIdx.y * rows * c;
  const bool vec = (ldx % 4) == 0;
  const int rg = t >> 2, cq = t & 3;

  float acc[4][8];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = 0.f;

  // one stage: X as xs[t - k0][o - o0], M as ms[t - k0][j - j0] (zero outside)
  f32x4_t xv[4];
  float mv[2];
  auto load = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (TRANS) {   // X rows are reduction rows: 256 consecutive outputs per row
        const int64_t gk = k0 + (t >> 6) + 4 * i, go = o0 + 4 * (t & 63);
        xv[i] = gk < t_hi && go < rows ? load4f(X + gk * ldx + go, rows - go, vec) : f32x4_t{0.f, 0.f, 0.f, 0.f};
      } else {       // X rows are output rows: 16 consecutive reduction elements per row
        const int64_t go = o0 + t, gk = k0 + 4 * i;
        xv[i] = go < rows && gk < t_hi ? load4f(X + go * ldx + gk, t_hi - gk, vec) : f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = 2 * t + u, kk = e >> 5, jj = e & 31;
      const int64_t gk = k0 + kk;
      mv[u] = gk < t_hi && j0 + jj < c ? M[gk * c + j0 + jj] : 0.f;
    }
  };
  auto store = [&](int b) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (TRANS) {
        *reinterpret_cast<f32x4_t *>(&xs[b][(t >> 6) + 4 * i][4 * (t & 63)]) = xv[i];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) xs[b][4 * i + e][t] = xv[i][e];
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) ms[b][(2 * t + u) >> 5][(2 * t + u) & 31] = mv[u];
  };

  const int64_t nch = t_hi > t_lo ? (t_hi - t_lo + MAT_CHUNK - 1) / MAT_CHUNK : 0;
  if (nch > 0) {
    load(t_lo);
    store(0);
  }
  __syncthreads();
  for (int64_t ci = 0; ci < nch; ++ci) {
    const int b = (int)(ci & 1);
    if (ci + 1 < nch) load(t_lo + (ci + 1) * MAT_CHUNK);
#pragma unroll 4
    for (int kk = 0; kk < MAT_CHUNK; ++kk) {
      const f32x4_t x = *reinterpret_cast<const f32x4_t *>(&xs[b][kk][4 * rg]);
      const f32x4_t m0 = *reinterpret_cast<const f32x4_t *>(&ms[b][kk][8 * cq]);
      const f32x4_t m1 = *reinterpret_cast<const f32x4_t *>(&ms[b][kk][8 * cq + 4]);
#pragma unroll
      for (int a = 0; a < 4; ++a) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[a][e] = fmaf(x[a], m0[e], acc[a][e]);
          acc[a][4 + e] = fmaf(x[a], m1[e], acc[a][4 + e]);
        }
      }
    }
    if (ci + 1 < nch) store(b ^ 1);   // the stage read one iteration ago
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int64_t o = o0 + 4 * rg + a;
    if (o >= rows) continue;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = j0 + 8 * cq + e;
      if (j < c) out[o * c + j] = acc[a][e];
    }
  }
}

constexpr int CHOL_MAX_C = 64;   // widest c whose factor fits the LDS in fp64 (2 c^2 doubles)

// The CholeskyQR factor on the device: M = L^-T with G + eps I = L L^T, G the
// c x c Gram matrix (fp32, symmetric), eps = 1e-12 trace(G) (1e-12 if the
// trace is not positive), a pivot not above eps taken as sqrt(eps); in
// double, M written as fp32 [c][c]. One workgroup, c <= CHOL_MAX_C. The
// factor is right-looking (after column j, every entry below and right of it
// subtracts its column-j product) and L^T M = I is solved from the last row
// up (after row i of M, every row above subtracts its row-i product), so each
// entry takes the same operations in the same order as the host's sums.
__global__ __launch_bounds__(256) void k_chol_inv(const float *G, int c, float *M) {
  __shared__ double A[CHOL_MAX_C * CHOL_MAX_C];   // G + eps I, its lower part becoming L
  __shared__ double R[CHOL_MAX_C * CHOL_MAX_C];   // I, becoming M
  const int t = threadIdx.x;
  double tr = 0.0;   // every thread sums the diagonal in the same order
  for (int i = 0; i < c; ++i) tr += (double)G[i * c + i];
  const double eps = 1e-12 * (tr > 0 ? tr : 1.0);
  for (int e = t; e < c * c; e += 256) {
    const int i = e / c, k = e - i * c;
    A[e] = i == k ? (double)G[e] + eps : (double)G[e];
    R[e] = i == k ? 1.0 : 0.0;
  }
  __syncthreads();
  for (int j = 0; j < c; ++j) {
    if (t == 0) {
      const double d = A[j * c + j];
      A[j * c + j] = d > eps ? sqrt(d) : sqrt(eps);
    }
    __syncthreads();
    const double d = A[j * c + j];
    for (int i = j + 1 + t; i < c; i += 256) A[i * c + j] = A[i * c + j] / d;
    __syncthreads();
    const int w = c - j - 1;   // trailing block rows/columns j + 1 .. c - 1
    for (int e = t; e < w * w; e += 256) {
      const int i = j + 1 + e / w, k = j + 1 + e % w;
      if (k <= i) A[i * c + k] -= A[i * c + j] * A[k * c + j];
    }
    __syncthreads();
  }
  for (int i = c - 1; i >= 0; --i) {
    for (int col = t; col < c; col += 256) R[i * c + col] = R[i * c + col] / A[i * c + i];
    __syncthreads();
    for (int e = t; e < i * c; e += 256) {   // rows 0 .. i - 1
      const int ii = e / c, col = e - ii * c;
      R[ii * c + col] -= A[i * c + ii] * R[i * c + col];
    }
    __syncthreads();
  }
  for (int e = t; e < c * c; e += 256) M[e] = (float)R[e];
}

// out[i] = sum over the S partials part[s][i], in order.
__global__ void k_sum_parts(const float *part, int S, int64_t n, float *out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float v = 0.0f;
  for (int s = 0; s < S; ++s) v += part[s * n + i];
  out[i] = v;
}

// T[n][k] = bf16(W[n][k] - sum_j B[n][j] AT[k][j]) (B [N][r], AT [K][r] fp32;
// r = 0 copies W), the sum over j in order. One thread per 8 consecutive
// elements of a row (K % 8 == 0): its B row is shared by the 8, and where r %
// 4 == 0 both operands come in 16-byte loads.
__global__ void k_shift(const uint16_t *W, const float *B, const float *AT, int64_t N, int64_t K, int r,
                        uint16_t *T) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (i >= N * K) return;
  const int64_t n = i / K, k = i - n * K;
  const u32x4_t w = *reinterpret_cast<const u32x4_t *>(W + i);
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = bf16_bits_to_f32((w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
  const float *b = B + n * r;
  const float *at = AT + k * r;
  if ((r % 4) == 0) {
    for (int j = 0; j < r; j += 4) {
      const f32x4_t b4 = *reinterpret_cast<const f32x4_t *>(b + j);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const f32x4_t a4 = *reinterpret_cast<const f32x4_t *>(at + e * r + j);
#pragma unroll
        for (int q = 0; q < 4; ++q) v[e] = fmaf(-b4[q], a4[q], v[e]);
      }
    }
  } else {
    for (int j = 0; j < r; ++j) {
      const float bj = b[j];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = fmaf(-bj, at[e * r + j], v[e]);
    }
  }
  uint32_t o[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) o[q] = (uint32_t)to_bf16(v[2 * q]) | ((uint32_t)to_bf16(v[2 * q + 1]) << 16);
  *reinterpret_cast<u32x4_t *>(T + i) = u32x4_t{o[0], o[1], o[2], o[3]};
}

// R[n][k] = W[n][k] - deq(Q)[n][k] in fp32, one thread per 32 elements of a row.
template <int FMT>
__global__ void k_residual(const uint16_t *W, PackedW Q, Nf4Table tab, float *R) {
  __shared__ float qlds[16];
  if (threadIdx.x < 16) qlds[threadIdx.x] = tab.q[threadIdx.x];
  __syncthreads();
  const int64_t pieces = Q.K >> 5;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= Q.N * pieces) return;
  const int64_t n = i / pieces, k = (i - n * pieces) * 32;
  uint32_t d[16];
  dequant_row32<FMT>(Q, 0, n, k, qlds, d);
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int64_t o = n * Q.K + k + 2 * e;
    R[o] = bf16_bits_to_f32(W[o]) - bf16_bits_to_f32(d[e] & 0xFFFFu);
    R[o + 1] = bf16_bits_to_f32(W[o + 1]) - bf16_bits_to_f32(d[e] >> 16);
  }
}

// M[k][j] = +-1 from a counter hash (splitmix64 of the index): the start block
// of the subspace iteration.
__global__ void k_rademacher(float *M, int64_t n, uint64_t seed) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  uint64_t z = seed + (uint64_t)i * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  M[i] = (z >> 63) ? 1.0f : -1.0f;
}

// Transposing conversion out[j][k] = bf16(f in[k][j]) (AT [K][r] fp32 to
// A [r][K] bf16); k_to_bf16 converts B [N][r] with a factor.
__global__ void k_to_bf16_t(const float *in, int64_t rows, int cols, float f, uint16_t *out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * cols) return;
  const int64_t j = i / rows, k = i - j * rows;   // out[j][k] = in[k][j]
  out[i] = to_bf16(in[k * cols + j] * f);
}

__global__ void k_to_bf16(const float *in, int64_t n, float f, uint16_t *out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  out[i] = to_bf16(in[i] * f);
}

}  // namespace loftq
}  // namespace lora4
