/*
 * libif4 -- IF4 (Int/Float 4) adaptive block-scaled quantization on AMD
 * MI355X (gfx950).  C ABI.
 *
 * The format ("Adaptive Block-Scaled Data Types", gist.science summary,
 * section 2 "Metodologia"; podcast.do-not-panic.com episode companion
 * "Adaptive Block-Scaled Data Types for FP4 Training", sections "One Group,
 * Two Candidate Encodings" and "The Free Bit: Scale Factor Sign"): every
 * group of 16 consecutive values along the contraction dimension gets one
 * E4M3 scale; the group is encoded both as FP4 (E2M1) and as INT4
 * pre-scaled by 7/6 (descaled by 6/7 on use); the encoding with the lower
 * squared error is kept and the choice is stored in the scale byte's sign
 * bit, which NVFP4 leaves unused (0 = FP4, 1 = INT4).  Storage is the same
 * 4.5 bits per value as NVFP4.
 *
 * Exact definition implemented here (where the pages are silent):
 *   scale     s' = E4M3 value nearest to amax * 2^-E / 6 (ties to even,
 *             saturating at 448; rounding to 0 makes a zero group);
 *             s = s' * 2^E, E = scale_exp, a per-tensor power of two.
 *   FP4       c_i = E2M1 value nearest to |x_i| / s (ties to even, max 6).
 *   INT4      q_i = integer nearest to 7|x_i| / (6 s) (ties to even),
 *             clamped to 7.
 *   error     fp32, in the x7 domain, index order i = 0..15 from +0:
 *             d = fma(|x_i|, 7, -c_i*7s), e_fp = fma(d, d, e_fp), and the
 *             same with q_i*6s for e_int.  INT4 iff e_int < e_fp.
 *   nibble    bit 3 = sign bit of x_i, bits 2..0 = E2M1 index or |q_i|.
 *   scale byte  bit 7 = 1 for INT4, bits 6..0 = E4M3 code of s';
 *             0x00 for a zero group (codes 0), 0x7F (NaN) when the group
 *             holds a NaN or infinity (codes 0).
 *
 * Layouts (row-major, little-endian):
 *   x       [rows, cols]   fp32 or bf16, leading dimension ld_x (elements)
 *   codes   [rows, cols/2] uint8, element 2j in the low nibble of byte j
 *   scales  [rows, cols/16] uint8
 *
 * Conventions for every entry point:
 *   * All data pointers are DEVICE pointers owned by the caller; the library
 *     allocates no memory and keeps no state, and is safe to call from
 *     several threads.
 *   * `stream` is a hipStream_t (NULL = the default stream).  Work is only
 *     enqueued; the call returns before it runs.  Faults inside a kernel
 *     surface at the caller's next synchronisation.
 *   * Arguments are validated on the host before anything is launched; a
 *     non-zero status means nothing was enqueued.  Zero rows (or zero
 *     M/N/K) is valid and enqueues nothing -- except if4_gemm with K == 0,
 *     which writes zeros to C.
 */
#ifndef IF4_H
#define IF4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    IF4_OK = 0,
    IF4_ERR_NULL = 1,  /* a required pointer is NULL                      */
    IF4_ERR_SHAPE = 2, /* negative size, cols/K not a multiple of 16, ld too small */
    IF4_ERR_ALIGN = 3, /* pointer or leading dimension misaligned         */
    IF4_ERR_DTYPE = 4, /* unknown dtype or mode                           */
    IF4_ERR_RANGE = 5, /* |scale_exp| > 64                                */
    IF4_ERR_HIP = 6    /* the HIP runtime refused the launch              */
};

enum { IF4_F32 = 0, IF4_BF16 = 1 };

enum {
    IF4_MODE_ADAPTIVE = 0,   /* IF4: per-group lower-error choice            */
    IF4_MODE_FORCE_FP4 = 1,  /* every group FP4 (an NVFP4-style baseline)    */
    IF4_MODE_FORCE_INT4 = 2  /* every group 7/6-scaled INT4                  */
};

/* Library version as 10000*major + 100*minor + patch. */
int if4_version(void);

/* Static string naming a status code. */
const char* if4_status_string(int status);

/*
 * Quantize x to IF4 (the five steps of the shd-paper.top card "Adaptive
 * Block-Scaled Data Types", method details: split into blocks of 16, encode
 * both ways, compare errors, keep the lower, flag it in the scale's sign
 * bit).
 *   x        device [rows, cols], dtype IF4_F32 or IF4_BF16, 16-byte aligned,
 *            ld_x >= cols with ld_x * sizeof(dtype) a multiple of 16.
 *   codes    device [rows, cols/2], 8-byte aligned.
 *   scales   device [rows, cols/16].
 *   scale_exp  E in [-64, 64].
 * cols must be a multiple of 16 (whole groups only).
 */
int if4_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols,
                 int64_t ld_x, uint8_t* codes, uint8_t* scales,
                 int32_t scale_exp, void* stream);

/* As if4_quantize, with the selection mode (IF4_MODE_*).  The forced modes
 * compute the same scale and write the flag of the forced format. */
int if4_quantize_mode(const void* x, int x_dtype, int64_t rows, int64_t cols,
                      int64_t ld_x, uint8_t* codes, uint8_t* scales,
                      int32_t scale_exp, int mode, void* stream);

/*
 * Rotate, then quantize: each group of 16 along dim 1 is first turned by a
 * random-sign 16-point Hadamard transform, the preprocessing the pages use to
 * smooth outliers so that groups look uniform and the INT4 encoding wins more
 * often ("Adaptive Block-Scaled Data Types", gist.science summary, section 1
 * "O Problema"; podcast companion, "Where the Gain Actually Comes From").
 * Per group, y = H16 (d .* x) / 4, with d_i = -1 where bit i of sign_mask is
 * set and H16 the Sylvester matrix H2 (x) H2 (x) H2 (x) H2 (orthonormal after
 * the 1/4).  Arithmetic: fp32, through the butterfly stages of that
 * factorisation, strides 1, 2, 4, 8 in that order, each pair (lo, hi) ->
 * (lo + hi, lo - hi) rounded to nearest even, then the exact quarter; for
 * bf16 input each y is rounded to bf16 (nearest even) before it is
 * quantized.  The result is bit for bit if4_quantize_mode of that rotated
 * tensor, with y never written to memory.  The same sign_mask applied to both
 * operands of a product along their contraction dim leaves the product
 * unchanged (H16/4 is orthogonal), so a GEMM of two rotated operands
 * approximates the unrotated one.
 *   sign_mask  bits 0..15 (higher bits set: IF4_ERR_RANGE)
 * Other arguments, alignment and errors as if4_quantize_mode.  scale_exp
 * refers to the rotated values, whose absmax is at most 4x that of x.
 */
int if4_quantize_rht(const void* x, int x_dtype, int64_t rows, int64_t cols,
                     int64_t ld_x, uint32_t sign_mask, uint8_t* codes,
                     uint8_t* scales, int32_t scale_exp, int mode, void* stream);

/*
 * IF3 and IF6: the adaptive per-group choice at 3 and 6 bits per value
 * ("Adaptive Block-Scaled Data Types for FP4 Training", podcast companion,
 * "It Generalizes: IF3 and IF6"; gist.science summary, section 2,
 * "Extensoes").  The pages name the formats without defining them; these
 * keep IF4's construction:
 *   bits = 6 (IF6): float candidate FP6 E2M3 (2 exponent bits, bias 1,
 *     3 mantissa bits, subnormals; top 7.5); INT candidate |q| <= 31,
 *     decoding to q * (15/62) * s so that 31 lands on 7.5.
 *   bits = 3 (IF3): float candidate FP3 E2M0 (magnitudes 0, 1, 2, 4);
 *     INT candidate |q| <= 3, decoding to q * (4/3) * s.
 * Per group of 16 along dim 1: scale s' = RNE_E4M3(amax * 2^-E / top) with
 * top = 7.5 or 4 (saturating at 448; 0 gives the zero group), s = s' 2^E;
 * float code = RNE index on the grid (ties to the even index, saturating);
 * INT |q| = min(RNE(|x| / (step s)), qmax) with step = top / qmax; squared
 * errors summed in fp32 in index order as e = fma(d, d, e), with
 * d = fma(|x|, dd, -c dd s) for the float code and fma(|x|, dd, -|q| dn s)
 * for INT, where top / qmax = dn / dd in lowest terms (15/62, 4/3); INT is
 * kept iff its sum is strictly lower (mode as for if4_quantize_mode); the
 * scale byte is s' | flag << 7, 0x7F for a group holding NaN or infinity.
 * Codes: bit (bits - 1) = sign of x, low bits = float index or |q|; element i
 * of a group occupies bits [bits*i, bits*(i+1)) of the group's
 * little-endian field of 2*bits bytes.
 *   codes   device [rows, cols/16 * 2*bits] bytes, 8-byte aligned
 *   scales  device [rows, cols/16]
 *   bits    3 or 6 (else IF4_ERR_DTYPE)
 * Other arguments, alignment and errors as if4_quantize_mode.
 */
int if4_quantize_ifn(int bits, const void* x, int x_dtype, int64_t rows, int64_t cols,
                     int64_t ld_x, uint8_t* codes, uint8_t* scales, int32_t scale_exp, int mode,
                     void* stream);

/* Dequantize IF3 / IF6 codes (layout as if4_quantize_ifn): float codes to
 * sign * grid value * s' * 2^E, INT codes to sign * (the fp32 nearest
 * |q| * dn * s' / dd) * 2^E; y as for if4_dequantize (fp32 or bf16, rounded
 * to nearest even).  codes 8-byte aligned; errors as if4_dequantize, plus
 * IF4_ERR_DTYPE for bits other than 3 and 6. */
int if4_dequantize_ifn(int bits, const uint8_t* codes, const uint8_t* scales, int64_t rows,
                       int64_t cols, int32_t scale_exp, void* y, int y_dtype, int64_t ld_y,
                       void* stream);

/*
 * Quantize x^T: the groups are 16 consecutive ROWS of each column of x, and
 * the result is bit for bit if4_quantize_mode applied to the transpose of x
 * (same rules, same mode).  This is the operand layout the backward products
 * of a W4A4G4 linear layer need, which contract over the other dimension
 * ("Adaptive Block-Scaled Data Types", shd-paper.top card, training setup:
 * weights, activations and gradients all in 4 bits): dgrad groups W along
 * N, wgrad groups dY and X along M.
 *   x       device [rows, cols] row-major, fp32 or bf16, aligned to its
 *           element size, leading dimension ld_x >= cols
 *   rows    multiple of 16 (else IF4_ERR_SHAPE); cols any
 *   codes   device [cols, rows/2], 8-byte aligned (row c = column c of x)
 *   scales  device [cols, rows/16]
 * Errors as if4_quantize.
 */
int if4_quantize_t(const void* x, int x_dtype, int64_t rows, int64_t cols,
                   int64_t ld_x, uint8_t* codes, uint8_t* scales,
                   int32_t scale_exp, int mode, void* stream);

/*
 * Dequantize IF4 to fp32 or bf16.  INT4 magnitudes are descaled by 6/7
 * (gist.science summary, section 2, "Metodo 6/7"):
 *   FP4   y = (+-) c * s' * 2^E             (exact in fp32)
 *   INT4  y = (+-) fl32(6 |q| s' / 7) * 2^E (fp32 round to nearest even)
 * bf16 output is the fp32 value rounded to nearest even.  A 0x7F/0xFF scale
 * byte decodes to NaN.
 *   codes  device [rows, cols/2], 8-byte aligned; scales device [rows, cols/16]
 *   y      device [rows, cols] of y_dtype, 16-byte aligned, ld_y >= cols
 *          with ld_y * sizeof(dtype) a multiple of 16.
 */
int if4_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                   int64_t cols, int32_t scale_exp, void* y, int y_dtype,
                   int64_t ld_y, void* stream);

/*
 * W4A4 product of two IF4 operands ("MAC Unit: Decoding Two Formats from
 * One Sign Bit" on the podcast companion page: both operands 4-bit, each
 * group decoded by its own scale's sign bit):
 *   C[m, n] = sum_k A[m, k] * W[n, k]       (C = A W^T, nn.Linear layout)
 * with A [M, K] and W [N, K] both IF4 grouped along K.  Each operand is
 * decoded to fp16 without its 2^E and with a uniform 2^-9: FP4 values
 * c s' 2^-9 exactly, INT4 values fl16(|q| sigma 2^-9) with
 * sigma = fl16(fl32(s' * fl32(6/7))), the fp16 rounding of |q| sigma
 * (below 2^-5 to a multiple of 2^-15).  Products are accumulated in fp32 on
 * the matrix cores, and each output sum is scaled by 2^(a_exp + w_exp + 18)
 * with one ldexp before the fp32 store: exact while the result is a normal
 * fp32 number, one rounding where it is subnormal, +-inf only where it
 * overflows, and a zero sum stays +0 at every exponent pair.
 *   a_codes [M, K/2], w_codes [N, K/2]: device, 8-byte aligned
 *   a_scales [M, K/16], w_scales [N, K/16]: device
 *   c       device fp32 [M, N] with leading dimension ldc >= N, 4-byte aligned
 * K must be a multiple of 16.
 */
int if4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, int32_t a_exp,
             const uint8_t* w_codes, const uint8_t* w_scales, int32_t w_exp,
             int64_t M, int64_t N, int64_t K, float* c, int64_t ldc,
             void* stream);

#ifdef __cplusplus
}
#endif

#endif /* IF4_H */
