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

constexpr int MAT_ROWS = 32;    // output rows per workgroup of k_mat
constexpr int MAT_CHUNK = 32;   // reduction chunk staged in LDS
constexpr int MAX_C = 144;      // widest M (r + 16 for r <= 128)

// out[o][j] = sum_t X(o, t) M[t][j] for o < rows, j < c, t < inner, with
// X(o, t) = X[o][t] (TRANS = false, X is [rows][ldx]) or X[t][o] (TRANS =
// true, X is [inner][ldx]); M is [inner][c], out [rows][c], all fp32. One
// workgroup per 32 output rows and reduction range (blockIdx.y: t in
// [y per_split, (y + 1) per_split), written to out + y rows c); thread t
// owns row t % 32 and columns t / 32 + 8 u; the sum over t runs in order
// (deterministic).
template <bool TRANS>
__global__ __launch_bounds__(256) void k_mat(const float *X, int64_t ldx, int64_t rows, int64_t inner,
                                             const float *M, int c, float *out, int64_t per_split) {
  __shared__ float xs[MAT_CHUNK][MAT_ROWS + 1];
  __shared__ float ms[MAT_CHUNK][MAX_C];
  const int t = threadIdx.x;
  const int64_t o0 = (int64_t)blockIdx.x * MAT_ROWS;
  const int ro = t & 31, cg = t >> 5;
  constexpr int NU = (MAX_C + 7) / 8;
  float acc[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) acc[u] = 0.0f;
  const int64_t t_lo = (int64_t)blockIdx.y * per_split;
  const int64_t t_hi = t_lo + per_split < inner ? t_lo + per_split : inner;
  out += (int64_t)blockIdx.y * rows * c;
  for (int64_t t0 = t_lo; t0 < t_hi; t0 += MAT_CHUNK) {
    // stage X(o0 .. +31, t0 .. +31) as xs[t][o] and M(t0 .. +31, 0 .. c)
    for (int e = t; e < MAT_CHUNK * MAT_ROWS; e += 256) {
      int tt, oo;
      if (TRANS) {   // rows of X are reduction rows: read along o
        tt = e / MAT_ROWS;
        oo = e % MAT_ROWS;
      } else {       // rows of X are output rows: read along t
        oo = e / MAT_CHUNK;
        tt = e % MAT_CHUNK;
      }
      const int64_t gt = t0 + tt, go = o0 + oo;
      float v = 0.0f;
      if (gt < t_hi && go < rows) v = TRANS ? X[gt * ldx + go] : X[go * ldx + gt];
      xs[tt][oo] = v;
    }
    for (int e = t; e < MAT_CHUNK * c; e += 256) {
      const int tt = e / c, j = e % c;
      const int64_t gt = t0 + tt;
      ms[tt][j] = gt < t_hi ? M[gt * c + j] : 0.0f;
    }
    __syncthreads();
    for (int tt = 0; tt < MAT_CHUNK; ++tt) {
      const float x = xs[tt][ro];
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int j = cg + 8 * u;
        if (j < c) acc[u] = fmaf(x, ms[tt][j], acc[u]);
      }
    }
    __syncthreads();
  }
  const int64_t o = o0 + ro;
  if (o < rows) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int j = cg + 8 * u;
      if (j < c) out[o * c + j] = acc[u];
    }
  }
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
// r = 0 copies W).
__global__ void k_shift(const uint16_t *W, const float *B, const float *AT, int64_t N, int64_t K, int r,
                        uint16_t *T) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N * K) return;
  const int64_t n = i / K, k = i - n * K;
  float v = bf16_bits_to_f32(W[i]);
  for (int j = 0; j < r; ++j) v = fmaf(-B[n * r + j], AT[k * r + j], v);
  T[i] = to_bf16(v);
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
