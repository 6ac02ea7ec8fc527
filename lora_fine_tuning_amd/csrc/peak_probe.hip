// Measured roofline denominators of the device the library runs on: the
// dense bf16 MFMA rate (the instruction both dequant-GEMMs are built on,
// v_mfma_f32_32x32x16_bf16, with no other work between the products) and the
// HBM read bandwidth (16-byte loads streaming a buffer far larger than the
// caches). Measurement aids, not part of the layer's computation.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include "peak_probe.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int CHAINS = 8;   // independent accumulators per wave (covers the MFMA latency)

__global__ __launch_bounds__(256) void k_probe_mfma(int iters, float *out) {
  const uint32_t l = threadIdx.x & 63;
  // small, lane-dependent bf16 operands (values stay finite for any iters)
  const u32x4_t ua = {0x3C003C00u ^ l, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
  const u32x4_t ub = {0x3C003C00u, 0x3C003C00u ^ (l << 16), 0x3C003C00u, 0x3C003C00u};
  const bf16x8_t a = __builtin_bit_cast(bf16x8_t, ua), b = __builtin_bit_cast(bf16x8_t, ub);
  f32x16_t acc[CHAINS];
#pragma unroll
  for (int j = 0; j < CHAINS; ++j) acc[j] = f32x16_t{};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < CHAINS; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < CHAINS; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Sum of a buffer read once with 16-byte loads, grid-strided.
__global__ __launch_bounds__(256) void k_probe_read(const u32x4_t *src, size_t n16, float *out) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  float s = 0.0f;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4_t v0 = __builtin_nontemporal_load(src + i), v1 = __builtin_nontemporal_load(src + i + stride);
    const u32x4_t v2 = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4_t v3 = __builtin_nontemporal_load(src + i + 3 * stride);
    s += __builtin_bit_cast(float, v0[0] ^ v1[1] ^ v2[2] ^ v3[3]);
  }
  for (; i < n16; i += stride) s += __builtin_bit_cast(float, src[i][0]);
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

float elapsed(hipEvent_t a, hipEvent_t b) {
  float ms = -1.0f;
  if (hipEventSynchronize(b) != hipSuccess || hipEventElapsedTime(&ms, a, b) != hipSuccess) return -1.0f;
  return ms;
}

template <typename Go>
float timed(hipStream_t st, Go &&go) {
  hipEvent_t a = nullptr, b = nullptr;
  if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return -1.0f;
  float ms = -1.0f;
  if (hipEventRecord(a, st) == hipSuccess) {
    go();
    if (hipGetLastError() == hipSuccess && hipEventRecord(b, st) == hipSuccess) ms = elapsed(a, b);
  }
  hipEventDestroy(a);
  hipEventDestroy(b);
  return ms;
}

}  // namespace

extern "C" {

__attribute__((visibility("default"))) double peak_probe_mfma_flops(int blocks, int iters) {
  return (double)blocks * 4.0 * iters * CHAINS * 2.0 * 32 * 32 * 16;
}

__attribute__((visibility("default"))) float peak_probe_mfma(int blocks, int iters, float *out, void *stream) {
  if (blocks < 1 || iters < 1 || !out) return -1.0f;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return timed(st, [&] { hipLaunchKernelGGL(k_probe_mfma, dim3(blocks), dim3(256), 0, st, iters, out); });
}

__attribute__((visibility("default"))) float peak_probe_read(const void *src, size_t bytes, int blocks, float *out,
                                                             void *stream) {
  if (!src || !out || blocks < 1 || bytes < 16 || ((uintptr_t)src & 15u)) return -1.0f;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return timed(st, [&] {
    hipLaunchKernelGGL(k_probe_read, dim3(blocks), dim3(256), 0, st, reinterpret_cast<const u32x4_t *>(src),
                       bytes / 16, out);
  });
}

}  // extern "C"
