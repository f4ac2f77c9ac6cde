/*
 * lowbit.h -- C ABI of liblowbit, weight-only low-bit round-to-nearest (RTN)
 * quantized linear layers for AMD MI355X (gfx950).
 *
 * The method (sources are the pages this library was written from):
 *  - Weights are quantized with "MinMax", i.e. round-to-nearest with no
 *    calibration data (BladeLLM model quantization, "Quantization
 *    algorithms", MinMax), on a uniform asymmetric min-max grid per output
 *    row (OPTQ reproducibility card, "Experiment Setup" row) or per block of
 *    consecutive input channels (BladeLLM model quantization,
 *    "block_wise_quant": S in R^{Ci/group x Co}).
 *  - For b bits, M = 2^b - 1, per group:  scale = (max - min) / M,
 *    zero = round(-min / scale), q = clamp(round(w / scale) + zero, 0, M),
 *    rounding half to even.
 *  - Several codes share one machine word ([Feature Request] 4bit and 2bit
 *    and 1bit quantization support: two 4-bit codes per byte, four 2-bit
 *    codes per uint8, sixteen 2-bit codes per int32).
 *  - Widths b = 2, 3, 4 and 8 (8 and 4 bits are BladeLLM's weight-only
 *    widths, "Quantization modes"; GGUF has 8-bit round-to-nearest block
 *    types beside the 4-bit ones).
 *  - The low-bit weights stay in GPU memory and are turned back into numbers
 *    by the GPU's own cores inside the matrix product (same feature request;
 *    "weight_only_quant" in BladeLLM model quantization, "Quantization modes",
 *    is the mode that pays off when memory bandwidth is the constraint).
 *
 * Exact arithmetic contract (identical in every entry point):
 *  - lo, hi = min, max of the group's fp16 weights (widened to fp32, exact);
 *    s32 = fl32(fl32(hi - lo) / M); the stored scale is s16 = fp16_rne(s32),
 *    replaced by 1.0 when it is zero; s = (float)s16.
 *  - zero = (int32) rint(fl32(-lo / s)), signed and not clamped.
 *  - q = clamp((int) rint(fl32(w / s)) + zero, 0, M); divisions are IEEE
 *    fp32 divisions, rint rounds half to even.
 *  - Packing: per row, code k occupies bits [bits*k, bits*k + bits) of a
 *    little-endian stream of 32-bit words; 3-bit codes straddle words; 8-bit
 *    code k is byte k of the row; every row starts on a word boundary.
 *  - deq(q) = (q - zero) * s, the exact value the code stands for (GGUF file
 *    format, quantization-type table: weight = code x block scale + block
 *    offset), not rounded to any format;  y[b][n] = fp16_rne( sum_k x[b][k] *
 *    deq[n][k] ), with fp32 accumulation (summation order unspecified): within
 *    1e-3 |y| + 1e-4 of the exact sum for inputs of the workloads' scale.
 *
 * Layouts (dense, row-major, no strides; every pointer is a DEVICE pointer
 * allocated and owned by the caller, 16-byte aligned):
 *    w       fp16   [N][K]          N = output features, K = input features
 *    codes   uint8  [N][K]
 *    packed  uint32 [N][K*bits/32]
 *    scales  fp16   [N][G]          G = K / group_size, or 1 when group_size == 0
 *    zeros   int32  [N][G]
 *    x       fp16   [B][K]
 *    y       fp16   [B][N]
 *  fp16 values are passed as their IEEE binary16 bit patterns.
 *
 * Shape rules (violations return LOWBIT_ERR_SHAPE):
 *    K > 0, K % 32 == 0, (K * bits) % 128 == 0  (every packed row is whole
 *    16-byte chunks); group_size == 0 or (group_size % 32 == 0 and
 *    K % group_size == 0).  lowbit_quantize_rtn additionally needs
 *    K <= LOWBIT_QUANTIZE_MAX_K.
 *
 * Errors: every entry point returns LOWBIT_OK (0) or a negative status.
 * Arguments are validated on the host before anything is launched, so an
 * error return means nothing was enqueued.  N == 0 (or B == 0) is a valid
 * empty problem: nothing is launched and LOWBIT_OK is returned.  Kernels run
 * asynchronously on hip_stream (a hipStream_t; NULL = the null stream); a
 * device-side fault surfaces at the caller's next synchronization.  Inputs
 * must be finite.  Outputs must not alias inputs.  The library allocates no
 * memory and keeps no per-call state: calls on different streams may run
 * concurrently as long as their output buffers do not overlap.  (The one
 * exception is lowbit_quantize_gptq_noalloc, whose workspace is a static
 * device array of the library: see there.)
 */
#ifndef LOWBIT_H
#define LOWBIT_H

#include <stdint.h>

#ifndef LOWBIT_API
#define LOWBIT_API __attribute__((visibility("default")))
#endif

#ifdef __cplusplus
extern "C" {
#endif

#define LOWBIT_OK 0
#define LOWBIT_ERR_ARG (-1)         /* null / misaligned pointer, negative size, B out of range */
#define LOWBIT_ERR_SHAPE (-2)       /* K or group_size break the shape rules */
#define LOWBIT_ERR_UNSUPPORTED (-3) /* bits not in {2, 3, 4, 8} */
#define LOWBIT_ERR_HIP (-4)         /* the HIP runtime refused a launch or query */
#define LOWBIT_ERR_SCRATCH (-5)     /* larger than lowbit_quantize_gptq_noalloc's static scratch */

#define LOWBIT_QUANTIZE_MAX_K 131072
#define LOWBIT_QGEMV_MAX_B 15
#define LOWBIT_GPTQ_NOALLOC_MAX_BYTES 75497472 /* 72 MiB */

/*
 * Quantize fp16 weights w[N][K] with min-max RTN (BladeLLM model
 * quantization, "Quantization algorithms", MinMax; OPTQ reproducibility
 * card, "Experiment Setup" row; groups along input channels per BladeLLM
 * "block_wise_quant").  Writes scales[N][G] and zeros[N][G], plus the codes
 * as bytes (codes_or_null) and/or packed words (packed_or_null); at least
 * one of the two must be non-null.  The packed words equal those that
 * lowbit_pack produces from the codes.
 */
LOWBIT_API int lowbit_quantize_rtn(const void* w_f16, int64_t N, int64_t K, int bits, int64_t group_size,
                        uint8_t* codes_or_null, uint32_t* packed_or_null, uint16_t* scales_f16,
                        int32_t* zeros, void* hip_stream);

/*
 * Quantize w[N][K] onto the signed symmetric grid, the other RTN mode
 * (BladeLLM model quantization, "Quantization modes": symmetric quantization
 * keeps no zero point; GGUF file format, the quantization-type table: the
 * "legacy" x = d*q types).  Per group, with qmax = 2^(bits-1) - 1:
 *    amax = max |w| (fp32, exact); s16 = fp16_rne(fl32(amax / qmax)),
 *    replaced by 1.0 when it is zero; s = (float)s16;
 *    q = clamp((int) rint(fl32(w / s)), -qmax, qmax), rint half to even.
 * The stored code is q + 2^(bits-1) and every zero is 2^(bits-1), so codes
 * lie in [1, 2^bits - 1] and the output (scales, zeros, codes, packed words)
 * feeds lowbit_qgemv and lowbit_qgemm unchanged: (code - zero) * s = q * s.
 * Arguments, layouts, shape rules, ownership and errors exactly as
 * lowbit_quantize_rtn.
 */
LOWBIT_API int lowbit_quantize_rtn_sym(const void* w_f16, int64_t N, int64_t K, int bits,
                            int64_t group_size, uint8_t* codes_or_null, uint32_t* packed_or_null,
                            uint16_t* scales_f16, int32_t* zeros, void* hip_stream);

/*
 * Pack byte codes[N][K] (each < 2^bits; higher bits are ignored) into
 * packed[N][K*bits/32] (the feature request's several-codes-per-word
 * storage; bit order as in the contract above).
 */
LOWBIT_API int lowbit_pack(const uint8_t* codes, int64_t N, int64_t K, int bits, uint32_t* packed,
                void* hip_stream);

/*
 * y[B][N] = x[B][K] * deq(packed)^T for 1 <= B <= LOWBIT_QGEMV_MAX_B: the
 * fused dequantize-and-multiply of the feature request (weights kept
 * low-bit in memory, turned back into numbers by the GPU at run time).  Bandwidth-
 * bound: reads each packed word once.  B outside [0, 15] returns
 * LOWBIT_ERR_ARG.
 */
LOWBIT_API int lowbit_qgemv(const void* x_f16, int64_t B, const uint32_t* packed, const uint16_t* scales_f16,
                 const int32_t* zeros, int64_t N, int64_t K, int bits, int64_t group_size,
                 void* y_f16, void* hip_stream);

/*
 * Same product for any B >= 0 through fp16 matrix-core (MFMA) tiles; meant
 * for B >= 16, correct for every B.  Same arguments and contract as
 * lowbit_qgemv.
 */
LOWBIT_API int lowbit_qgemm(const void* x_f16, int64_t B, const uint32_t* packed, const uint16_t* scales_f16,
                 const int32_t* zeros, int64_t N, int64_t K, int bits, int64_t group_size,
                 void* y_f16, void* hip_stream);

/*
 * Compact group metadata: one 32-bit word per group, the fp16 scale's bit
 * pattern in bits 0-15 and the zero point as a two's-complement 16-bit
 * integer in bits 16-31 (4 bytes per group instead of 6).  Block formats keep
 * such per-block parameters beside the codes (GGUF file format, quantization
 * type table: block scale, and block minimum for the "_1" types); this word
 * keeps the integer zero point, so the dequantized weights do not change.
 *
 * lowbit_pack_meta writes meta[N][G] from scales_f16[N][G] and zeros[N][G]
 * (device pointers, 16-byte aligned).  A zero point outside [-32768, 32767]
 * is saturated to the nearest end; the number of saturated groups is ADDED
 * to *saturated_or_null (a 4-byte aligned device int32 the caller
 * initialises; NULL: not counted).  For 2-, 3- and 4-bit groups with
 * max > min every zero point fits (|zero| <= M * 2^11 <= 30720); constant
 * groups of magnitude >= 32768 and far one-signed 8-bit groups may not.
 * N == 0 or G == 0 launches nothing.
 */
LOWBIT_API int lowbit_pack_meta(const uint16_t* scales_f16, const int32_t* zeros, int64_t N,
                                int64_t G, uint32_t* meta, int32_t* saturated_or_null,
                                void* hip_stream);

/*
 * lowbit_qgemv and lowbit_qgemm with the group parameters as compact words
 * meta[N][G] (from lowbit_pack_meta) instead of scales and zeros.  Same
 * arguments otherwise, same contract, same results whenever no zero point was
 * saturated.
 */
LOWBIT_API int lowbit_qgemv_meta(const void* x_f16, int64_t B, const uint32_t* packed,
                                 const uint32_t* meta, int64_t N, int64_t K, int bits,
                                 int64_t group_size, void* y_f16, void* hip_stream);
LOWBIT_API int lowbit_qgemm_meta(const void* x_f16, int64_t B, const uint32_t* packed,
                                 const uint32_t* meta, int64_t N, int64_t K, int bits,
                                 int64_t group_size, void* y_f16, void* hip_stream);

/*
 * Error-feedback quantization (GPTQ / OPTQ): the parameters of each output
 * row are quantized one input channel after another, and the inverse of the
 * Hessian built from the layer's input activations adjusts the parameters
 * not yet quantized (BladeLLM model quantization, "Quantization algorithms",
 * GPTQ; OPTQ reproducibility card, "Experiment Setup" row: Hessians from
 * calibration inputs, per-row asymmetric min-max grid).  Contract:
 *  - H = (2/n) X^T X over the calibration rows x_f16[n_samples][K] (fp16,
 *    device), in fp64, plus damp * mean(diag H) on the diagonal (damp > 0;
 *    0.01 is customary);
 *  - scales and zeros are exactly those of lowbit_quantize_rtn on w (the
 *    grid of the original weights, per row or per group);
 *  - columns are taken in order 0..K-1; column i's code is
 *    clamp(rint(t_i / s) + zero, 0, M) on the current fp64 weight t_i, its
 *    dequantized value deq_i = (q - zero) * s (exact), and the error
 *    (t_i - deq_i) / Hinv_ii is fed into the later columns of the row through
 *    row i of the inverse Hessian of the columns not yet quantized;
 *  - outputs as lowbit_quantize_rtn (codes and/or packed words, scales,
 *    zeros), same shape rules.
 * The computation runs in fp64 in the caller's device workspace of at least
 * lowbit_gptq_workspace_bytes(N, K) bytes (256-byte aligned; returns a
 * negative status for invalid sizes).  On return of the work its first int32
 * is 0, or has bit value 1 set when H was not positive definite (all
 * calibration inputs zero), in which case the codes are unspecified; bit
 * value 2 would report that the factorization stopped waiting for a tile
 * after its bound (not expected to occur; the codes are then unspecified as
 * well).  Calls on one workspace must not overlap.  The library allocates
 * nothing.
 */
LOWBIT_API int64_t lowbit_gptq_workspace_bytes(int64_t N, int64_t K);
LOWBIT_API int lowbit_quantize_gptq(const void* w_f16, int64_t N, int64_t K, const void* x_f16,
                                    int64_t n_samples, double damp, int bits,
                                    int64_t group_size, uint8_t* codes_or_null,
                                    uint32_t* packed_or_null, uint16_t* scales_f16,
                                    int32_t* zeros, void* workspace, int64_t workspace_bytes,
                                    void* hip_stream);

/*
 * lowbit_quantize_gptq on the signed symmetric grid of
 * lowbit_quantize_rtn_sym (BladeLLM model quantization, "Quantization modes":
 * the weight-only mode lists gptq among its algorithms and quantizes on the
 * signed symmetric grid unless told otherwise).  scales
 * and zeros are exactly those of lowbit_quantize_rtn_sym on w (every zero is
 * 2^(bits-1)); column i's code is clamp(rint(t_i / s) + zero, 1, M), so codes
 * lie in [1, M] as there.  Everything else, including the workspace and the
 * status word, exactly as lowbit_quantize_gptq.
 */
LOWBIT_API int lowbit_quantize_gptq_sym(const void* w_f16, int64_t N, int64_t K,
                                        const void* x_f16, int64_t n_samples, double damp,
                                        int bits, int64_t group_size, uint8_t* codes_or_null,
                                        uint32_t* packed_or_null, uint16_t* scales_f16,
                                        int32_t* zeros, void* workspace,
                                        int64_t workspace_bytes, void* hip_stream);

/*
 * lowbit_quantize_gptq without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same computation, arguments, layouts,
 * shape rules and outputs as lowbit_quantize_gptq on the min-max grid; the
 * fp64 workspace is instead a static device array inside the library, of
 * LOWBIT_GPTQ_NOALLOC_MAX_BYTES per GPU, held from the first call on that GPU
 * until the process ends.  A problem whose lowbit_gptq_workspace_bytes(N, K)
 * exceeds it returns LOWBIT_ERR_SCRATCH before anything is enqueued (e.g.
 * N = K = 2048 fits; N = 11008, K = 4096 does not).  The status word (as
 * for lowbit_quantize_gptq) is written to *status_or_null (a
 * 4-byte aligned device int32 owned by the caller; NULL: not reported).
 * This entry point allocates nothing and calls no allocating routine.  All
 * calls on one GPU share the array and each call overwrites what the
 * previous one left there: calls that overlap on one GPU (different streams
 * or host threads) race and must be serialized by the caller.
 */
LOWBIT_API int lowbit_quantize_gptq_noalloc(const void* w_f16, int64_t N, int64_t K,
                                            const void* x_f16, int64_t n_samples, double damp,
                                            int bits, int64_t group_size, uint8_t* codes_or_null,
                                            uint32_t* packed_or_null, uint16_t* scales_f16,
                                            int32_t* zeros, int32_t* status_or_null,
                                            void* hip_stream);

/* Static, human-readable text for a status code (never NULL). */
LOWBIT_API const char* lowbit_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* LOWBIT_H */
