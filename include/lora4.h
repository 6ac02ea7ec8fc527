/*
 * lora4.h - C ABI of liblora4: the unmerged-LoRA linear layer over a frozen
 * 4-bit base, forward and backward, for AMD Instinct MI355X (gfx950).
 *
 * What is computed (terminology of "Quantized weights, full precision: The
 * math behind 75% cheaper fine-tuning", section "Terminology": X input
 * activations, Y output split into Y^base and Y^LoRA, W base weights, A and B
 * the down and up LoRA matrices; shapes of "Training LLMs on a Budget: LoRA,
 * QLoRA, and LoftQ", section 2 "The math": W is [d_out, d_in], A is
 * [r, d_in], B is [d_out, r]). With tokens as rows, M tokens, K = d_in,
 * N = d_out and s = alpha / r:
 *
 *   forward : Z = X A^T                      [M, r]
 *             Y = X deq(W)^T + s Z B^T       [M, N]   (= Y^base + Y^LoRA)
 *   backward: dZ = s dY B                    [M, r]
 *             dX = dY deq(W) + dZ A          [M, K]
 *             dA = dZ^T X                    [r, K]
 *             dB = s dY^T Z                  [N, r]
 *
 * There is no dW: the base is frozen (Crusoe post, "Backward pass and
 * optimizer step in training"). deq(W) is formed in registers/LDS inside
 * the kernels and is never written to device memory (same post, "Forward
 * pass in training"; "Training LLMs on a Budget", section 3 "The setup").
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller. Tensors are
 *    dense, row-major and contiguous. bf16 values are passed as uint16_t bit
 *    patterns. 16-byte alignment is required for every tensor pointer except
 *    the NF4-DQ second-level scales (scales2), which need 4 bytes: a group's
 *    slice of a stacked [groups][...] array starts at a multiple of 4 bytes.
 *  - stream is a hipStream_t passed as void* (NULL = the null stream). Every
 *    call is asynchronous on that stream; nothing synchronizes the device.
 *    Pointers are borrowed until the stream work completes.
 *  - Outputs are overwritten, never accumulated.
 *  - Arguments are validated on the host before any HIP call; a negative
 *    status is returned and nothing is launched. Launch failures return
 *    LORA4_ERR_HIP. No C++ exception crosses this boundary.
 *  - The library allocates no device memory. Scratch space comes from the
 *    caller's workspace, sized by lora4_workspace_bytes().
 *  - Calls are re-entrant; two calls that share output or workspace buffers
 *    on different streams race.
 *  - State kept between calls (all of it guarded for concurrent callers):
 *    the NF4 table, built once and never changed; per device, the CU count
 *    and which kernels have had their LDS limit raised; the opt-in kernel
 *    timing record (lora4_timing_enable / lora4_timing_collect); the static
 *    scratch array of lora4_forward_noalloc, one per device. No other state
 *    outlives a call.
 */
#ifndef LORA4_H
#define LORA4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage formats of the frozen base.
 *  LORA4_NF4    : NF4 codes, one fp32 absmax scale per 64 consecutive
 *                 K-elements of a row ("Training LLMs on a Budget",
 *                 section 3, tricks 1 and 2).
 *  LORA4_NF4_DQ : NF4 codes whose per-64 scales are themselves stored as
 *                 E4M3 (OCP E4M3FN) codes with one fp32 second-level scale per
 *                 256 consecutive first-level scales (same section, trick 2,
 *                 double quantization).
 *  LORA4_MXFP4  : E2M1 codes with one E8M0 scale per 32 consecutive
 *                 K-elements ("Fine-Tuning 4-Bit Models", section "Case 2").
 *  LORA4_NVFP4  : E2M1 codes with one E4M3 (FP8) scale per 16 consecutive
 *                 K-elements, no per-tensor scale ("Fine-Tuning 4-Bit Models",
 *                 section "Case 2: An NVFP4 deployment checkpoint is what you
 *                 were handed"); K % 32 == 0.
 */
typedef enum {
  LORA4_NF4 = 1,
  LORA4_NF4_DQ = 2,
  LORA4_MXFP4 = 3,
  LORA4_NVFP4 = 4
} lora4_format;

typedef enum {
  LORA4_OK = 0,
  LORA4_ERR_NULL = -1,          /* a required pointer is NULL                    */
  LORA4_ERR_SHAPE = -2,         /* a size is out of range or inconsistent        */
  LORA4_ERR_ALIGN = -3,         /* a tensor pointer is not 16-byte aligned (scales2: 4) */
  LORA4_ERR_FORMAT = -4,        /* unknown format, or block does not match it    */
  LORA4_ERR_WORKSPACE = -5,     /* workspace NULL or smaller than required       */
  LORA4_ERR_HIP = -6,           /* a HIP call or kernel launch failed            */
  LORA4_ERR_UNIMPLEMENTED = -7, /* valid request the library does not support   */
  LORA4_ERR_SCRATCH = -8        /* request exceeds the allocation-free scratch   */
} lora4_status;

/* The frozen 4-bit base W, logically [N = d_out, K = d_in] per group.
 *  format, block : LORA4_NF4 / LORA4_NF4_DQ with block 64, LORA4_MXFP4 with 32,
 *                  LORA4_NVFP4 with 16.
 *  N, K          : rows and columns of one group; K % block == 0, K >= block
 *                  (NVFP4: K % 32 == 0).
 *  groups        : 1 for a plain linear; E for E experts stored back to back,
 *                  each taking lora4_packed_bytes(format, N, K, part) bytes
 *                  of codes (part 0), scales (1) and scales2 (2).
 * Each group's [N, K] is stored in tiles of 64 rows by 64 elements: RB =
 * ceil(N/64) row blocks, KB = ceil(K/64) k blocks, tile (rb, kb) is tile
 * number t = rb*KB + kb; row i of a tile is row 64*rb + i of W, element j of
 * it is element 64*kb + j. Rows past N and elements past K are zero padding.
 *  codes         : uint8, 2048 bytes per tile at 2048*t; row i at 32*i.
 *                  MXFP4, NVFP4: byte j of a row holds element 2j in its low
 *                  nibble and element 2j+1 in its high nibble. NF4, NF4_DQ:
 *                  in each 4-byte word (elements 8w .. 8w+7 of the row),
 *                  byte j holds element 8w+j in its low nibble and 8w+j+4 in
 *                  its high nibble (the decoder reads each half's indices
 *                  straight from the word).
 *  scales        : NF4    : float, 64 per tile at 64*t; entry i = the scale of
 *                           row i's 64 elements
 *                  NF4_DQ : uint8 E4M3 codes, 64 per tile at 64*t, as NF4
 *                  MXFP4  : uint8 E8M0 codes (value 2^(E-127)), 128 per tile
 *                           at 128*t; entry 2i+h = the scale of elements
 *                           32h .. 32h+31 of row i
 *                  NVFP4  : uint8 E4M3 codes, 256 per tile at 256*t; entry
 *                           4i+q = the scale of elements 16q .. 16q+15 of
 *                           row i
 *  scales2       : NF4_DQ only: float [groups][ceil(N*K/64 / 256)], the
 *                  second-level scale of each run of 256 consecutive
 *                  first-level scales of one group, counted in row-major
 *                  order (row n, block b: n*(K/64) + b); the rebuilt scale
 *                  is fp32(E4M3(code) * scales2). NULL otherwise.
 * The dequantized element is bf16(fp32(q[code] * scale)) for NF4 (q the
 * 16-level NF4 codebook), bf16(e2m1(code) * 2^(E-127)) for MXFP4 and
 * bf16(e2m1(code) * e4m3(scale)) (exact) for NVFP4. The
 * tiles let every global load of codes in the GEMMs cover whole contiguous
 * rows of a tile (the kernels read one tile per wave and step).
 */
typedef struct lora4_W {
  int32_t format;
  int32_t block;
  int64_t N;
  int64_t K;
  int64_t groups;
  const uint8_t *codes;
  const void *scales;
  const float *scales2;
} lora4_W;

/* Bytes of one packed [N, K] matrix (one group) in format: part 0 the codes,
 * 1 the first-level scales, 2 the NF4-DQ second-level scales (0 for the
 * other formats). Returns 0 for invalid arguments. */
size_t lora4_packed_bytes(int32_t format, int64_t N, int64_t K, int32_t part);

/* Workspace (bytes) that lora4_forward (which = 0) or lora4_backward
 * (which = 1) needs for this W, M tokens and rank r. Returns 0 for invalid
 * arguments. A caller may size once for the largest M and reuse it. */
size_t lora4_workspace_bytes(int which, const lora4_W *W, int64_t M, int32_t r);

/* Forward: Y = X deq(W)^T + s (X A^T) B^T.
 *  X      : bf16 [M, K]                      (input activations)
 *  A      : bf16 [groups][r, K]              (down projection)
 *  B      : bf16 [groups][N, r]              (up projection)
 *  r      : LoRA rank, 1 <= r <= 256
 *  s      : LoRA scale alpha / r (any finite float)
 *  group_offsets : groups == 1: NULL. Otherwise a DEVICE int64 array of
 *           groups+1 non-decreasing row offsets, [0] == 0, [groups] == M;
 *           rows offsets[e]..offsets[e+1]-1 of X and Y belong to expert e
 *           (rows are pre-sorted by expert; routing and gating are outside).
 *  Y      : bf16 [M, N] output, rounded once from the fp32 sum.
 *  Z      : bf16 [M, r] output Z = X A^T kept for the backward; may be NULL.
 *  Y_base, Y_lora : optional bf16 [M, N] outputs of the two terms; may be NULL.
 *  workspace, workspace_bytes : device scratch, >= lora4_workspace_bytes(0,...).
 * M may be 0: nothing is launched, and X, Y may then be NULL. */
lora4_status lora4_forward(const lora4_W *W, const uint16_t *X, int64_t M,
                           const uint16_t *A, const uint16_t *B, int32_t r, float s,
                           const int64_t *group_offsets,
                           uint16_t *Y, uint16_t *Z, uint16_t *Y_base, uint16_t *Y_lora,
                           void *workspace, size_t workspace_bytes, void *stream);

/* Backward: dX = dY deq(W) + dZ A, dA = dZ^T X, dB = s dY^T Z, dZ = s dY B.
 *  X, A, B, r, s, group_offsets : as for lora4_forward.
 *  dY     : bf16 [M, N] upstream gradient.
 *  Z      : bf16 [M, r] from lora4_forward, or NULL to recompute X A^T.
 *  dX     : bf16 [M, K] output.
 *  dA     : bf16 [groups][r, K] output (zero for an expert with no rows).
 *  dB     : bf16 [groups][N, r] output (zero for an expert with no rows).
 *  workspace, workspace_bytes : device scratch, >= lora4_workspace_bytes(1,...).
 * M may be 0: then dA and dB are set to zero, and X, dY, dX may be NULL. */
lora4_status lora4_backward(const lora4_W *W, const uint16_t *X, const uint16_t *dY, int64_t M,
                            const uint16_t *A, const uint16_t *B, int32_t r, float s,
                            const int64_t *group_offsets, const uint16_t *Z,
                            uint16_t *dX, uint16_t *dA, uint16_t *dB,
                            void *workspace, size_t workspace_bytes, void *stream);

/* Forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * arguments of lora4_forward without the workspace. Its scratch is a static
 * device array of LORA4_NOALLOC_SCRATCH_BYTES that the library holds on every
 * GPU it runs on until the process ends; no call allocates or frees device
 * memory (with kernel timing on, only events already pooled are used).
 * Every call on one GPU uses that GPU's array and leaves its contents behind
 * (nothing in it has to start at zero): calls that overlap on one GPU, e.g.
 * on two streams, race. A request whose forward needs more scratch returns
 * LORA4_ERR_SCRATCH before anything is launched; outputs whose split
 * reduction would not fit run unsplit instead. Results are those of
 * lora4_forward (bit for bit where both run the same schedule). */
#define LORA4_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
lora4_status lora4_forward_noalloc(const lora4_W *W, const uint16_t *X, int64_t M,
                                   const uint16_t *A, const uint16_t *B, int32_t r, float s,
                                   const int64_t *group_offsets,
                                   uint16_t *Y, uint16_t *Z, uint16_t *Y_base, uint16_t *Y_lora,
                                   void *stream);

/* Several LoRA adapters over one shared base: adapter a applies to rows
 * adapter_offsets[a] .. adapter_offsets[a+1]-1 of X, Y, dY and dX ("Fine-Tuning
 * 4-Bit Models", section "Case 3": adapters trained in BF16 over a native
 * 4-bit base are kept separate and served over it with multi-LoRA).
 *  W        : one group (W->groups == 1), read by every adapter.
 *  adapters : 1 .. 65535; A is bf16 [adapters][r, K], B [adapters][N, r], and
 *             dA, dB have the same shapes (zero for an adapter with no rows).
 *  adapter_offsets : adapters == 1: NULL. Otherwise a DEVICE int64 array of
 *             adapters+1 non-decreasing row offsets, [0] == 0, [adapters] == M
 *             (rows are pre-sorted by adapter).
 * Everything else as lora4_forward / lora4_backward; the workspace is sized by
 * lora4_workspace_bytes_multi (which = 0 forward, 1 backward; 0 returned for
 * invalid arguments). Validation errors: LORA4_ERR_SHAPE if W->groups != 1 or
 * adapters is out of range, LORA4_ERR_NULL if adapters > 1 without offsets. */
size_t lora4_workspace_bytes_multi(int which, const lora4_W *W, int64_t adapters, int64_t M, int32_t r);
lora4_status lora4_forward_multi(const lora4_W *W, int64_t adapters, const uint16_t *X, int64_t M,
                                 const uint16_t *A, const uint16_t *B, int32_t r, float s,
                                 const int64_t *adapter_offsets, uint16_t *Y, uint16_t *Z,
                                 uint16_t *Y_base, uint16_t *Y_lora,
                                 void *workspace, size_t workspace_bytes, void *stream);
lora4_status lora4_backward_multi(const lora4_W *W, int64_t adapters, const uint16_t *X,
                                  const uint16_t *dY, int64_t M, const uint16_t *A,
                                  const uint16_t *B, int32_t r, float s,
                                  const int64_t *adapter_offsets, const uint16_t *Z,
                                  uint16_t *dX, uint16_t *dA, uint16_t *dB,
                                  void *workspace, size_t workspace_bytes, void *stream);

/* Quantize a bf16 base W [N, K] (K % 64 == 0) to NF4 with per-64 fp32 absmax
 * scales ("Training LLMs on a Budget", section 3, tricks 1 and 2): code = the
 * NF4 level nearest to fp32(w / absmax), ties to the lower level; an
 * all-zero block encodes as the zero level.
 *  double_quant == 0: codes and float scales in the tiled layout of lora4_W,
 *    scales2 unused.
 *  double_quant != 0: codes as above; scales receives uint8 E4M3 codes
 *    (tiled) of scale / group max (nearest, ties to even); scales2 receives
 *    float [ceil(N*K/64/256)] group maxima (a group's code is 0 if its max is 0).
 * Codes are always chosen with the exact fp32 scale. Buffer sizes:
 * lora4_packed_bytes(format, N, K, 0..2); the padding is written as zero. */
lora4_status quant_pack_nf4(const uint16_t *W_bf16, int64_t N, int64_t K, int32_t double_quant,
                            uint8_t *codes, void *scales, float *scales2, void *stream);

/* Quantize a bf16 base W [N, K] (K % 32 == 0) to MXFP4 ("Fine-Tuning 4-Bit
 * Models", section "Case 2"): per 32-element block the E8M0 code
 * E = clamp(floor(log2 amax) - 2, -127, 127) + 127 (E = 0 for an all-zero
 * block), and each element's E2M1 code is the nearest value to w * 2^-(E-127),
 * ties to the even code, saturating at +-6, sign copied from w.
 *  codes, scales_e8m0 : the tiled layout of lora4_W, sized by
 *  lora4_packed_bytes(LORA4_MXFP4, N, K, 0 / 1); the padding is written as
 *  zero (E8M0 padding code 0). */
lora4_status quant_pack_mxfp4(const uint16_t *W_bf16, int64_t N, int64_t K,
                              uint8_t *codes, uint8_t *scales_e8m0, void *stream);

/* A base that ships only in 4 bits, packed row-major ("Fine-Tuning 4-Bit
 * Models", section "Case 3: Only a 4-bit-native checkpoint ships": the native
 * base is loaded as it is and adapted without a bf16 copy), rearranged into
 * the tiled storage of lora4_W, bit for bit, on the stream:
 *  codes_rm  : uint8 [groups][N][K/2]; byte j of a row holds element 2j in its
 *              low nibble and element 2j+1 in its high nibble.
 *  scales_rm : NF4    : float [groups][N][K/64] (absmax per 64 elements)
 *              NF4_DQ : uint8 E4M3 codes [groups][N][K/64]
 *              MXFP4  : uint8 E8M0 codes [groups][N][K/32]
 *              NVFP4  : uint8 E4M3 codes [groups][N][K/16]
 *  codes, scales : outputs, lora4_packed_bytes(format, N, K, 0 / 1) bytes per
 *              group, groups back to back; the padding is written as zero.
 * NF4-DQ second-level scales have the same order in both layouts: the
 * caller's float [groups][ceil(N*K/64/256)] array serves lora4_W.scales2 as
 * it is. K % 64 == 0 for NF4 / NF4-DQ, K % 32 == 0 for MXFP4 / NVFP4.
 * Device pointers, 16-byte aligned, input and output buffers distinct.
 * Errors: LORA4_ERR_FORMAT, LORA4_ERR_SHAPE, LORA4_ERR_NULL, LORA4_ERR_ALIGN
 * before anything is launched; LORA4_ERR_HIP for a failed launch. */
lora4_status lora4_import_rowmajor(int32_t format, int64_t N, int64_t K, int64_t groups,
                                   const uint8_t *codes_rm, const void *scales_rm,
                                   uint8_t *codes, void *scales, void *stream);

/* ---- MX-native forward of an MXFP4 base -------------------------------------
 * "Quantized weights, full precision", section "Forward pass in inference"
 * (and "Forward pass in training": the same operations in the training
 * forward): where the hardware has MXFP4-native operations the base product
 * of an MXFP4 base runs natively while the adapters stay in bf16. The pages
 * leave the activation format open; here X enters the base product as MXFP8
 * (OCP MX v1.0): per 32 consecutive elements of a row the E8M0 code
 * E = clamp(floor(log2 amax) - 8, -127, 127) + 127 (E = 0 for an all-zero
 * block), and each element's E4M3 code is the nearest value to
 * x * 2^-(E-127), ties to the even code, saturating at +-448, sign copied
 * from x (-0 gives 0x80).
 *
 * Quantize bf16 X [M, K] (K % 32 == 0) to MXFP8, row-major:
 *  codes       : uint8 [M, K] E4M3 codes.
 *  scales_e8m0 : uint8 [M, K / 32].
 * Device pointers, 16-byte aligned. M may be 0 (nothing is launched). */
lora4_status quant_pack_mxfp8(const uint16_t *X, int64_t M, int64_t K, uint8_t *codes,
                              uint8_t *scales_e8m0, void *stream);

/* Workspace (bytes) that lora4_forward_mx needs for this W, M tokens and rank
 * r (0 for invalid arguments). */
size_t lora4_workspace_bytes_mx(const lora4_W *W, int64_t M, int32_t r);

/* MX-native forward of one plain layer (W->format == LORA4_MXFP4,
 * W->groups == 1):
 *   Y = mxfp8(X) deq(W)^T + s (X A^T) B^T,  Z = X A^T
 * The base product runs on the block-scaled MFMA with X as MXFP8 (quantized
 * into the workspace) and W's E2M1 codes and E8M0 scales as stored; Z and the
 * LoRA term use the bf16 X. Accumulation in fp32; Y rounded once to bf16.
 *  X : bf16 [M, K]; A : bf16 [r, K]; B : bf16 [N, r]; 1 <= r <= 256; s finite.
 *  Y : bf16 [M, N] output. Z : bf16 [M, r] output, may be NULL.
 *  workspace, workspace_bytes : device scratch, >= lora4_workspace_bytes_mx.
 * Errors: LORA4_ERR_FORMAT if W is not MXFP4, LORA4_ERR_SHAPE for grouped W
 * or sizes past the 32-bit buffer offsets, and as lora4_forward otherwise.
 * M may be 0: nothing is launched, and X, Y may then be NULL. */
lora4_status lora4_forward_mx(const lora4_W *W, const uint16_t *X, int64_t M,
                              const uint16_t *A, const uint16_t *B, int32_t r, float s,
                              uint16_t *Y, uint16_t *Z, void *workspace, size_t workspace_bytes,
                              void *stream);

/* Quantize a bf16 base W [N, K] (K % 32 == 0) to NVFP4 ("Fine-Tuning 4-Bit
 * Models", section "Case 2: An NVFP4 deployment checkpoint is what you were
 * handed": an FP8 scale per 16-element micro-block). No per-tensor scale: per
 * 16-element block the E4M3 code of amax / 6 (nearest, ties to even,
 * saturating at 448; 0 for an all-zero block), and each element's E2M1 code
 * is the nearest value to w / s with s that code's value (ties to the even
 * code, saturating at +-6, sign copied; magnitude 0 where s == 0).
 *  codes, scales_e4m3 : the tiled layout of lora4_W (256 scale bytes per
 *  tile, row i's four at 4 i), sized by lora4_packed_bytes(LORA4_NVFP4, N,
 *  K, 0 / 1); the padding is written as zero. */
lora4_status quant_pack_nvfp4(const uint16_t *W_bf16, int64_t N, int64_t K,
                              uint8_t *codes, uint8_t *scales_e4m3, void *stream);

/* ---- LoftQ initialisation ----------------------------------------------------
 * "Training LLMs on a Budget", section 4: choose the NF4 base Q and the
 * adapter so that Q + s B A is close to W at step 0, by alternating
 * Q <- NF4(bf16(W - s B A)) with B A <- the best rank-r approximation of
 * W - Q (split as U sqrt(S), sqrt(S) V^T); iters SVD steps (the page's
 * default is 5), the last one after the last quantization, so the returned
 * Q and B A belong together. The rank-r approximation is computed by a
 * randomized subspace iteration on the fp32 residual (r + 16 columns, 8 power
 * iterations, orthonormalized by Cholesky QR), not by an exact SVD.
 * Synchronizes the stream (the small c x c steps run on the host).
 *  W        : bf16 [N, K], K % 64 == 0; 1 <= r <= 128, r + 16 <= min(N, K);
 *             1 <= iters <= 64; s the layer's adapter scale (finite, != 0).
 *  codes, scales, scales2 : the NF4 (double_quant == 0) or NF4-DQ packing of
 *             the last Q, as quant_pack_nf4 writes it.
 *  A        : bf16 [r, K] output; B : bf16 [N, r] output (divided by s).
 *  workspace, workspace_bytes : device scratch, >= lora4_loftq_workspace_bytes
 *             (which returns 0 for invalid sizes). */
size_t lora4_loftq_workspace_bytes(int64_t N, int64_t K, int32_t r);
lora4_status lora4_loftq_init(const uint16_t *W_bf16, int64_t N, int64_t K, int32_t r, int32_t iters,
                              float s, int32_t double_quant, uint8_t *codes, void *scales,
                              float *scales2, uint16_t *A, uint16_t *B, void *workspace,
                              size_t workspace_bytes, void *stream);

/* A static, human-readable name for a status code. */
const char *lora4_status_string(lora4_status status);

/* ---- Kernel timing (profiling aid) ------------------------------------------
 * When enabled, every kernel the library launches is bracketed by two HIP
 * events recorded on the caller's stream. lora4_timing_collect() waits for
 * the recorded events, sums the elapsed time per kernel name and clears the
 * record. Timing adds two event records per launch; it is off by default. */
typedef struct lora4_kernel_time {
  char name[48];
  int64_t launches;
  double total_ms;
} lora4_kernel_time;

lora4_status lora4_timing_enable(int on);
/* Writes up to max entries; returns the number of distinct kernels (may
 * exceed max), or a negative status. */
int lora4_timing_collect(lora4_kernel_time *out, int max);

/* Library version string. */
const char *lora4_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LORA4_H */
