/*
 * bsfp_oracle.h -- plain CPU oracle for block-scaled 4-bit quantization and
 * quantized matmul (NVFP4, MXFP4, affine 4-bit).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the GPU product path may include,
 * link or call this code; only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no code, header, table or
 * constant generator with the HIP library.
 *
 * Every array is a host array, row-major and contiguous.  bf16 values travel
 * as their uint16 bit patterns.  Packed codes: element k of a row is nibble
 * (k mod 8) of 32-bit word k/8, bits 4*(k mod 8) .. 4*(k mod 8)+3.
 *
 * Parity status per function is stated in bsfp_oracle.c beside each one.
 */
#ifndef BSFP_ORACLE_H
#define BSFP_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- scalar codecs ---------------------------------------------------- */
float    bo_bf16_to_f32(uint16_t h);
uint16_t bo_bf16_from_f32(float f);
uint16_t bo_bf16_from_f64(double d);
double   bo_e2m1_decode(int code);
int      bo_e2m1_encode(float v);
int      bo_e2m1_encode_sr(float v, uint32_t r);
double   bo_e4m3_decode(int code);
int      bo_e4m3_encode(float s); /* s >= 0 */
double   bo_e8m0_decode(int code);

/* array helpers for the Python side */
void bo_e2m1_encode_array(const float* v, int64_t n, uint8_t* out);
void bo_e4m3_encode_array(const float* v, int64_t n, uint8_t* out);
void bo_bf16_from_f32_array(const float* v, int64_t n, uint16_t* out);
void bo_bf16_from_f64_array(const double* v, int64_t n, uint16_t* out);

/* ---- tensor amax and NVFP4 global scale --------------------------------- */
float bo_amax(const uint16_t* x, int64_t n);
float bo_nvfp4_global_scale(float amax);       /* amax / (448*6) in fp32 */
float bo_alpha(float g_x, float g_w);          /* g_x * g_w in fp32 */

/* ---- quantize ------------------------------------------------------------ */
/* NVFP4, group 16.  g_given != NULL: use *g_given as the global scale.
 * Otherwise g = amax/2688 is computed from x.  use_global == 0 means no global
 * scale at all (g = 1).  Writes *g_out (may be NULL) and *amax_out (may be
 * NULL; written only when amax was computed). */
void bo_quantize_nvfp4(const uint16_t* x, int64_t rows, int64_t cols,
                       int use_global, const float* g_given,
                       uint32_t* codes, uint8_t* scales,
                       float* g_out, float* amax_out);
/* MXFP4, group 32, E8M0 scales. */
void bo_quantize_mxfp4(const uint16_t* x, int64_t rows, int64_t cols,
                       uint32_t* codes, uint8_t* scales);
void bo_quantize_nvfp4_sr(const uint16_t* x, int64_t rows, int64_t cols,
                          int use_global, const float* g_given, const uint32_t* rbits,
                          uint32_t* codes, uint8_t* scales,
                          float* g_out, float* amax_out);
void bo_quantize_mxfp4_sr(const uint16_t* x, int64_t rows, int64_t cols,
                          const uint32_t* rbits, uint32_t* codes, uint8_t* scales);
/* Affine 4-bit, group 64, bf16 scale and bias. */
void bo_quantize_affine(const uint16_t* x, int64_t rows, int64_t cols,
                        uint32_t* codes, uint16_t* scales, uint16_t* biases);

/* ---- format variants: affine b-bit group G, MXFP8 ------------------------- */
void bo_quantize_affine_g(const uint16_t* x, int64_t rows, int64_t cols, int bits, int G,
                          uint32_t* codes, uint16_t* scales, uint16_t* biases);
void bo_quantize_mxfp8(const uint16_t* x, int64_t rows, int64_t cols,
                       uint32_t* codes, uint8_t* scales);
void bo_dequantize_g(int mode, int bits, int G, const uint32_t* codes, const void* scales,
                     const uint16_t* biases, int64_t rows, int64_t cols, uint16_t* out);
void bo_dequant_exact_g(int mode, int bits, int G, const uint32_t* codes, const void* scales,
                        const uint16_t* biases, int64_t rows, int64_t cols, double* out);

/* ---- dequantize to bf16 --------------------------------------------------- */
void bo_dequantize_nvfp4(const uint32_t* codes, const uint8_t* scales,
                         const float* g /* NULL: no global scale */,
                         int64_t rows, int64_t cols, uint16_t* out);
void bo_dequantize_mxfp4(const uint32_t* codes, const uint8_t* scales,
                         int64_t rows, int64_t cols, uint16_t* out);
void bo_dequantize_affine(const uint32_t* codes, const uint16_t* scales,
                          const uint16_t* biases, int64_t rows, int64_t cols,
                          uint16_t* out);

/* ---- exact real dequantized values (fp64), the matmul operands ------------ */
/* mode: 0 affine, 1 mxfp4, 2 nvfp4.  For NVFP4, g == NULL leaves the global
 * scale out (the qq operand), otherwise it is multiplied in. */
void bo_dequant_exact(int mode, const uint32_t* codes, const void* scales,
                      const uint16_t* biases, const float* g,
                      int64_t rows, int64_t cols, double* out);

/* ---- matmul ---------------------------------------------------------------- */
/* y[m,n] = scale * sum_k A[m,k]*B[n,k] in fp64, denom[m,n] = |scale| *
 * sum_k |A[m,k]*B[n,k]|.  Either output pointer may be NULL. */
void bo_matmul_f64(const double* A, const double* B, int64_t M, int64_t N,
                   int64_t K, double scale, double* y, double* denom);
/* The same for selected (m,n) pairs only. */
void bo_matmul_f64_pairs(const double* A_rows, const double* B_rows, int64_t K,
                         const int64_t* ai, const int64_t* bi, int64_t count,
                         double scale, double* y, double* denom);
/* bf16 activations as fp64 */
void bo_bf16_to_f64_array(const uint16_t* x, int64_t n, double* out);

#ifdef __cplusplus
}
#endif
#endif
