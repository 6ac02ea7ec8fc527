/*
 * peak_probe.h - measured roofline denominators (libpeakprobe.so), a
 * measurement aid beside liblora4: the rate at which the device runs the
 * dense bf16 MFMA instruction both dequant-GEMMs are built on, and its HBM
 * read bandwidth. Device pointers, caller-owned; `stream` is a hipStream_t
 * passed as void*. Each call synchronizes on its own events and returns the
 * kernel's elapsed milliseconds, or a negative value on a bad argument or a
 * failed HIP call.
 */
#ifndef PEAK_PROBE_H
#define PEAK_PROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Flops that peak_probe_mfma(blocks, iters, ...) performs: every wave of the
 * blocks x 256 threads issues iters x 8 independent
 * v_mfma_f32_32x32x16_bf16 (32 768 flops each). */
double peak_probe_mfma_flops(int blocks, int iters);

/* Runs those MFMAs with nothing else between them. out: float [blocks * 256]
 * (one checksum per thread, so nothing is optimized away). */
float peak_probe_mfma(int blocks, int iters, float *out, void *stream);

/* Reads `bytes` (a multiple of 16 is used; 16-byte aligned src) once with
 * 16-byte loads, grid-strided over blocks x 256 threads. out: float
 * [blocks * 256]. */
float peak_probe_read(const void *src, size_t bytes, int blocks, float *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PEAK_PROBE_H */
