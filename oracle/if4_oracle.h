/*
 * IF4 reference oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, scalar CPU statement of what the IF4 hot path computes.
 * Only the tests, the smoke check and the CPU-baseline leg of the benchmark
 * may load it.  It shares no code, header, table or constant with the HIP
 * library under adaptive_block_scaled_amd/csrc and never calls into it.
 *
 * Source pages (cited by title and section throughout):
 *   [gist]    "Adaptive Block-Scaled Data Types", gist.science structured
 *             summary (Portuguese): section 1 "O Problema" (Hadamard
 *             transforms make data uniform); section 2 "Metodologia" with the
 *             items "Mecanismo de Selecao", "Codificacao Eficiente",
 *             "Metodo 6/7".
 *   [card]    "Adaptive Block-Scaled Data Types", shd-paper.top paper card:
 *             "方法详解" (method details) -- technical framework steps 1-5,
 *             key design; and the English abstract.
 *   [podcast] "Adaptive Block-Scaled Data Types for FP4 Training", episode
 *             companion: "It Generalizes: IF3 and IF6", "One Group, Two
 *             Candidate Encodings", "The Free Bit:
 *             Scale Factor Sign", "MAC Unit: Decoding Two Formats from One
 *             Sign Bit", "Where the Gain Actually Comes From" (the
 *             Hadamard-transformed weight gradient).
 *   [fugumt]  "論文の概要: Adaptive Block-Scaled Data Types": related-paper
 *             entry "FP8 Formats for Deep Learning" (E4M3 has no infinities
 *             and a single NaN mantissa pattern).
 *
 * Readings where the pages are silent are listed in the repository's design
 * notes; each is restated next to the code that implements it.
 *
 * Pins: every function here is checked by the CPU tests against closed forms,
 * exhaustive brute force and an exact-rational re-implementation (see
 * tests/test_oracle_pins.py); the Hadamard rotation against scipy's Sylvester
 * matrix, its error bound and hand-worked fp32 groups (tests/test_oracle_rht.py);
 * IF3 / IF6 against their grids' bit layouts, exhaustive exact-rational
 * roundings and an independent exact statement of groups (tests/test_oracle_ifn.py).
 */
#ifndef IF4_ORACLE_H
#define IF4_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Selection modes.  ADAPTIVE is IF4 proper; the two forced modes keep the
 * same scale and encodings but never choose the other format (the NVFP4-style
 * and the 7/6-scaled INT4 baselines the pages compare against). */
enum { IF4O_ADAPTIVE = 0, IF4O_FORCE_FP4 = 1, IF4O_FORCE_INT4 = 2 };

/* Value of a 7-bit E4M3FN magnitude code (0x00..0x7E); NaN for 0x7F. */
double if4o_e4m3_value(unsigned code7);

/* E2M1 value of a 3-bit FP4 magnitude index (0..7). */
double if4o_e2m1_value(unsigned idx3);

/* 7-bit scale code: round-to-nearest-even of a_scaled/6 onto the
 * non-negative E4M3FN grid, saturating at 448. */
unsigned if4o_scale_code(double a_scaled);

/* FP4 magnitude index: RNE of ax/s onto {0,.5,1,1.5,2,3,4,6}, saturating. */
unsigned if4o_fp4_index(double ax, double s);

/* INT4 magnitude: RNE of 7*ax/(6*s), clamped to 7. */
unsigned if4o_int4_mag(double ax, double s);

/* Quantize one group of 16 values.  Outputs the 8 code bytes, the scale
 * byte, and the two fp32 error sums (in the x7 domain; both 0 for zero or
 * non-finite groups). */
void if4o_quantize_group(const float x[16], int32_t scale_exp, int mode,
                         uint8_t codes[8], uint8_t* scale_byte,
                         float* err_fp4, float* err_int4);

/* Quantize a row-major [rows, cols] fp32 tensor (bf16 inputs are widened
 * exactly to fp32 by the caller).  codes: [rows, cols/2], scales:
 * [rows, cols/16].  err_fp4/err_int4 may be NULL, else [rows, cols/16].
 * nthreads <= 0 uses OpenMP's default; results do not depend on it. */
void if4o_quantize(const float* x, int64_t rows, int64_t cols, int64_t ld_x,
                   int32_t scale_exp, int mode, uint8_t* codes, uint8_t* scales,
                   float* err_fp4, float* err_int4, int nthreads);

/* Dequantize to fp32: FP4 -> sign * c * s' * 2^E (exact); INT4 ->
 * sign * fl32(6*|q|*s'/7) * 2^E.  Output [rows, cols] with leading dim ld_y. */
void if4o_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                     int64_t cols, int32_t scale_exp, float* y, int64_t ld_y,
                     int nthreads);

/* Round fp32 values to bf16 bit patterns (round-to-nearest-even, NaN kept). */
void if4o_f32_to_bf16(const float* x, int64_t n, uint16_t* out);

/* Decode to fp64: INT4 values as 6*q*s'*2^E/7 rounded once to double. */
void if4o_decode_f64(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                     int64_t cols, int32_t scale_exp, double* y, int nthreads);

/* fp64 reference GEMM on decoded operands, on a sample of the output:
 * c[i, j] = sum_k A[row_idx[i], k] * W[col_idx[j], k], A [*, K] and W [*, K]
 * packed IF4 grouped along K.  c is [n_rows, n_cols] fp64. */
void if4o_gemm_sample_f64(const uint8_t* a_codes, const uint8_t* a_scales,
                          int32_t a_exp, const uint8_t* w_codes,
                          const uint8_t* w_scales, int32_t w_exp, int64_t K,
                          const int64_t* row_idx, int64_t n_rows,
                          const int64_t* col_idx, int64_t n_cols, double* c,
                          int nthreads);

/* Random-sign Hadamard rotation of each group of 16 along dim 1:
 * y = H16 (d .* x) / 4, d_i = -1 where bit i of sign_mask is set, computed in
 * fp32 butterflies of strides 1, 2, 4, 8 (see the .c file for the reading);
 * with round_to_bf16 each y is rounded to bf16 (kept as fp32). */
void if4o_rht16(const float* x, int64_t rows, int64_t cols, int64_t ld_x,
                uint32_t sign_mask, int round_to_bf16, float* y, int64_t ld_y,
                int nthreads);

/* IF4 of the rotated tensor: if4o_rht16 followed by if4o_quantize. */
void if4o_quantize_rht(const float* x, int64_t rows, int64_t cols, int64_t ld_x,
                       uint32_t sign_mask, int round_to_bf16, int32_t scale_exp,
                       int mode, uint8_t* codes, uint8_t* scales, int nthreads);

/* IF3 / IF6 (bits = 3 or 6; see the .c file for the readings).  Codes are
 * [rows, cols/16 * 2*bits] bytes (element i of a group at bits
 * [bits*i, bits*(i+1)) of its little-endian field), scales [rows, cols/16];
 * mode as for IF4 (FORCE_FP4 = force the float format, FORCE_INT4 = force
 * INT).  Return 0, or -1 for an unknown width or cols % 16 != 0. */
double if4o_ifn_fp_value(int bits, unsigned idx);
unsigned if4o_ifn_scale_code(int bits, double a_scaled);
unsigned if4o_ifn_fp_index(int bits, double ax, double s);
unsigned if4o_ifn_int_mag(int bits, double ax, double s);
int if4o_ifn_quantize(int bits, const float* x, int64_t rows, int64_t cols, int64_t ld_x,
                      int32_t scale_exp, int mode, uint8_t* codes, uint8_t* scales,
                      float* err_fp, float* err_int, int nthreads);
int if4o_ifn_dequantize(int bits, const uint8_t* codes, const uint8_t* scales, int64_t rows,
                        int64_t cols, int32_t scale_exp, float* y, int64_t ld_y, int nthreads);

#ifdef __cplusplus
}
#endif

#endif
