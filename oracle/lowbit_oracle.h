/*
 * lowbit_oracle.h -- declarations of the CPU oracle for weight-only low-bit
 * round-to-nearest (RTN) quantization, bitstream packing, dequantization and
 * the fp64 reference product.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the
 * HIP library and its Python binding) never calls it and shares no code with
 * it.
 *
 * Conventions (all host pointers, dense row-major, caller-owned):
 *   W      fp16 bit patterns  [N][K]   (N = output features, K = input features)
 *   codes  uint8              [N][K]   values in [0, 2^bits - 1]
 *   packed uint32             [N][K*bits/32]  per-row little-endian bitstream
 *   scales fp16 bit patterns  [N][G]   G = K / group_size (group_size 0 = per-row)
 *   zeros  int32              [N][G]
 *   x      fp16 bit patterns  [B][K]
 *   deq    double             [N][K]   exact (q - zero) * scale, not rounded
 *   y      double             [B][N]
 * Every function returns 0 on success and -1 on a bad argument.
 */
#ifndef LOWBIT_ORACLE_H
#define LOWBIT_ORACLE_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

double   orc_f16_to_f64(uint16_t h);
uint16_t orc_f64_to_f16(double v);

int orc_quantize_rtn(const uint16_t* w, int64_t N, int64_t K, int bits, int64_t group_size,
                     uint8_t* codes, uint16_t* scales, int32_t* zeros);
int orc_quantize_rtn_sym(const uint16_t* w, int64_t N, int64_t K, int bits, int64_t group_size,
                         uint8_t* codes, uint16_t* scales, int32_t* zeros);
int orc_pack(const uint8_t* codes, int64_t N, int64_t K, int bits, uint32_t* packed);
int orc_unpack(const uint32_t* packed, int64_t N, int64_t K, int bits, uint8_t* codes);
int orc_dequant(const uint8_t* codes, const uint16_t* scales, const int32_t* zeros,
                int64_t N, int64_t K, int bits, int64_t group_size, double* deq);
int orc_matmul_f64(const uint16_t* x, const double* deq, int64_t B, int64_t N, int64_t K,
                   double* y);
/* Compact metadata words (fp16 scale | int16 zero << 16); orc_pack_meta
 * returns the number of zero points saturated to the int16 range (or -1). */
int64_t orc_pack_meta(const uint16_t* scales, const int32_t* zeros, int64_t count,
                      uint32_t* meta);
int orc_unpack_meta(const uint32_t* meta, int64_t count, uint16_t* scales, int32_t* zeros);

/* Error-feedback (GPTQ) quantization.  orc_hessian: H[K][K] = (2/n) X^T X
 * for x[n][K] (fp16) plus damp * mean(diag) on the diagonal.
 * orc_quantize_gptq: codes on the RTN grid of the original weights, chosen
 * column by column with inverse-Hessian error feedback; `work` holds
 * 3*K*K + N*K doubles. */
int orc_hessian(const uint16_t* x, int64_t n, int64_t K, double damp, double* H);
int orc_quantize_gptq(const uint16_t* w, int64_t N, int64_t K, const double* H, int bits,
                      int64_t group_size, uint8_t* codes, uint16_t* scales, int32_t* zeros,
                      double* work);
/* The same on the signed symmetric grid of orc_quantize_rtn_sym (codes from 1). */
int orc_quantize_gptq_sym(const uint16_t* w, int64_t N, int64_t K, const double* H, int bits,
                          int64_t group_size, uint8_t* codes, uint16_t* scales, int32_t* zeros,
                          double* work);

#ifdef __cplusplus
}
#endif
#endif
