/*
 * IF4 reference oracle -- TEST INFRASTRUCTURE ONLY (see if4_oracle.h).
 *
 * Plain scalar C.  Every rounding decision is taken by an exact comparison in
 * fp64 against the midpoint between two neighbouring grid values; the error
 * sums are fp32 with each operation written out (built with
 * -ffp-contract=off, no fast-math, so nothing is fused or reordered).
 *
 * Parity pinned by tests/test_oracle_pins.py: closed-form grids, exhaustive
 * brute force of the scale and code roundings, an exact-rational
 * re-implementation of whole groups, hand-worked groups and invariants.
 */
#include "if4_oracle.h"

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define GROUP 16

/* E2M1 magnitudes in code order (code = 2-bit exponent, 1-bit mantissa,
 * bias 1): the FP4 grid of [gist] section 2 ("FP4 ... ponto flutuante
 * (E2M1)") with the familiar values 0, 0.5, 1, 1.5, 2, 3, 4, 6; its top
 * value 6 is the "maximum representable value" the 6/7 method keeps for
 * INT4 ([gist] section 2, "Metodo 6/7"). */
static const double E2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* INT4 magnitudes 0..7: the symmetric range [-7, 7]; 7 * 6/7 = 6 is the same
 * top value as FP4 ([gist] section 2, "Metodo 6/7"). */
static const double INT4[8] = {0.0, 1.0, 2.0, 3.0, 4.0, 5.0, 6.0, 7.0};

double if4o_e4m3_value(unsigned code7) {
    /* E4M3 as in "FP8 Formats for Deep Learning" (cited on [fugumt]): 4
     * exponent bits with bias 7, 3 mantissa bits, no infinities, and one
     * NaN mantissa pattern (S.1111.111) -- so 0x7E = 1.75 * 2^8 = 448 is the
     * largest finite magnitude. */
    code7 &= 0x7Fu;
    if (code7 == 0x7Fu) return NAN;
    unsigned e = code7 >> 3, m = code7 & 7u;
    if (e == 0) return ldexp((double)m, -9); /* subnormal: m/8 * 2^(1-7) */
    return ldexp(1.0 + m / 8.0, (int)e - 7);
}

double if4o_e2m1_value(unsigned idx3) { return E2M1[idx3 & 7u]; }

/* Index of the grid value nearest to num/unit; an exact tie picks the even
 * index.  Values beyond the last midpoint land on the last index, which is
 * saturation.  The comparisons num <, == unit * midpoint are exact because
 * callers only pass operands whose products are exact in fp64. */
static unsigned rne_index(double num, double unit, const double* grid,
                          unsigned n) {
    unsigned k = 0;
    while (k + 1 < n) {
        double mid = unit * (0.5 * (grid[k] + grid[k + 1]));
        if (num < mid) return k;
        if (num == mid) return (k & 1u) ? k + 1 : k;
        k++;
    }
    return k;
}

/* The 127 finite non-negative E4M3 values in code order (ascending). */
static double E4M3_GRID[127];

__attribute__((constructor)) static void fill_e4m3_grid(void) {
    for (unsigned c = 0; c < 127; c++) E4M3_GRID[c] = if4o_e4m3_value(c);
}

static const double* e4m3_grid(void) { return E4M3_GRID; }

unsigned if4o_scale_code(double a_scaled) {
    /* One E4M3 scale per group of 16 "as is done with NVFP4" ([card]
     * abstract).  Reading: s' = RNE(amax / 6) on the E4M3 grid, so that
     * the group maximum lands on the common top value 6 of both encodings;
     * a/6 above 448 saturates to 448.  Comparing a with 6 * midpoint is
     * exact (a is an fp32 value, the midpoints have at most 5 bits). */
    return rne_index(a_scaled, 6.0, e4m3_grid(), 127);
}

unsigned if4o_fp4_index(double ax, double s) {
    /* RNE of |x|/s on the E2M1 grid; s * midpoint has at most 7 bits. */
    return rne_index(ax, s, E2M1, 8);
}

unsigned if4o_int4_mag(double ax, double s) {
    /* INT4 after the 7/6 pre-scale ([gist] section 2, "Metodo 6/7"):
     * q = RNE(7|x| / (6s)), clamped to 7.  Compare 7|x| with 6s * (k + 1/2),
     * both exact in fp64. */
    return rne_index(7.0 * ax, 6.0 * s, INT4, 8);
}

void if4o_quantize_group(const float x[16], int32_t scale_exp, int mode,
                         uint8_t codes[8], uint8_t* scale_byte,
                         float* err_fp4, float* err_int4) {
    memset(codes, 0, 8);
    *err_fp4 = 0.0f;
    *err_int4 = 0.0f;

    /* Non-finite input: the scale byte takes the E4M3 NaN pattern, codes 0. */
    for (int i = 0; i < GROUP; i++) {
        if (!isfinite(x[i])) {
            *scale_byte = 0x7F;
            return;
        }
    }

    /* Step 1 of [card]'s technical framework: the block of 16 values.
     * Group absolute maximum, then the per-tensor power-of-two exponent E
     * (scale = s' * 2^E); E = 0 is the plain per-group rule. */
    double a = 0.0;
    for (int i = 0; i < GROUP; i++) {
        double ax = fabs((double)x[i]);
        if (ax > a) a = ax;
    }
    unsigned sc = if4o_scale_code(ldexp(a, -scale_exp));
    if (sc == 0) { /* zero group or underflowed scale: byte 0, codes 0 */
        *scale_byte = 0;
        return;
    }
    double s = ldexp(if4o_e4m3_value(sc), scale_exp);

    /* Steps 2 and 3: encode the block both ways ([podcast] "One Group, Two
     * Candidate Encodings"; [gist] section 2, "Mecanismo de Selecao"). */
    unsigned fidx[GROUP], qmag[GROUP];
    for (int i = 0; i < GROUP; i++) {
        double ax = fabs((double)x[i]);
        fidx[i] = if4o_fp4_index(ax, s);
        qmag[i] = if4o_int4_mag(ax, s);
    }

    /* Step 4: squared error of each encoding, in fp32, in index order.
     * Reading: the error is taken in the x7 domain, so the 6/7 of INT4 stays
     * exact: d = 7|x| - c*7s (FP4) and d = 7|x| - q*6s (INT4), each rounded
     * once (fma); e = fma(d, d, e) for i = 0..15 starting from +0.  This is
     * 49 times the sum of squared errors, so "lower error" is unchanged. */
    float sf = (float)s; /* exact: 4 significant bits, within fp32 range */
    float s7 = 7.0f * sf;
    float s6 = 6.0f * sf;
    float ef = 0.0f, ei = 0.0f;
    for (int i = 0; i < GROUP; i++) {
        float ax = fabsf(x[i]);
        float cs7 = (float)E2M1[fidx[i]] * s7; /* exact */
        float qs6 = (float)INT4[qmag[i]] * s6; /* exact */
        float df = fmaf(ax, 7.0f, -cs7);
        float di = fmaf(ax, 7.0f, -qs6);
        ef = fmaf(df, df, ef);
        ei = fmaf(di, di, ei);
    }
    *err_fp4 = ef;
    *err_int4 = ei;

    /* Step 5: keep the lower-error encoding; an exact tie keeps FP4.  The
     * choice goes into the scale's otherwise unused sign bit: 0 = FP4,
     * 1 = INT4 ([gist] section 2, "Codificacao Eficiente"; [podcast] "The
     * Free Bit: Scale Factor Sign"). */
    int use_int4;
    if (mode == IF4O_FORCE_FP4)
        use_int4 = 0;
    else if (mode == IF4O_FORCE_INT4)
        use_int4 = 1;
    else
        use_int4 = ei < ef;
    *scale_byte = (uint8_t)(sc | (use_int4 ? 0x80u : 0u));

    /* Nibbles: bit 3 = sign of x (kept for zero magnitudes too), bits 0-2 =
     * the E2M1 index or the INT4 magnitude.  Element 2j goes to the low
     * nibble of byte j. */
    for (int i = 0; i < GROUP; i++) {
        unsigned mag = use_int4 ? qmag[i] : fidx[i];
        unsigned nib = (signbit(x[i]) ? 8u : 0u) | mag;
        codes[i / 2] |= (uint8_t)(nib << (4 * (i & 1)));
    }
}

void if4o_quantize(const float* x, int64_t rows, int64_t cols, int64_t ld_x,
                   int32_t scale_exp, int mode, uint8_t* codes, uint8_t* scales,
                   float* err_fp4, float* err_int4, int nthreads) {
    int64_t gpr = cols / GROUP;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t g = 0; g < gpr; g++) {
            float ef, ei;
            if4o_quantize_group(x + r * ld_x + g * GROUP, scale_exp, mode,
                                codes + r * (cols / 2) + g * 8,
                                scales + r * gpr + g, &ef, &ei);
            if (err_fp4) err_fp4[r * gpr + g] = ef;
            if (err_int4) err_int4[r * gpr + g] = ei;
        }
    }
}

/* Value of one nibble in a group with scale byte b, as fp32, before 2^E.
 * INT4 magnitudes are descaled by 6/7 ([gist] section 2, "Metodo 6/7"):
 * 6*q*s' is exact in fp64, the division by 7 rounds once to fp64 and the
 * cast rounds to fp32; 6*q*s' has at most 8 bits, so the quotient is never
 * within 2^-53 of an fp32 midpoint and the two roundings equal one. */
static float nibble_value_f32(unsigned nib, unsigned b) {
    double sp = if4o_e4m3_value(b & 0x7Fu);
    unsigned mag = nib & 7u;
    float v;
    if (b & 0x80u)
        v = (float)((6.0 * INT4[mag] * sp) / 7.0);
    else
        v = (float)(E2M1[mag] * sp);
    return (nib & 8u) ? -v : v;
}

void if4o_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                     int64_t cols, int32_t scale_exp, float* y, int64_t ld_y,
                     int nthreads) {
    int64_t gpr = cols / GROUP;
    float p2 = ldexpf(1.0f, scale_exp); /* exact for |E| <= 64 */
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t k = 0; k < cols; k++) {
            unsigned b = scales[r * gpr + k / GROUP];
            unsigned byte = codes[r * (cols / 2) + k / 2];
            unsigned nib = (k & 1) ? (byte >> 4) : (byte & 0xFu);
            y[r * ld_y + k] = nibble_value_f32(nib, b) * p2;
        }
    }
}

void if4o_f32_to_bf16(const float* x, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; i++) {
        uint32_t u;
        memcpy(&u, &x[i], 4);
        if (isnan(x[i])) {
            out[i] = (uint16_t)((u >> 16) | 0x0040u);
            continue;
        }
        uint32_t lsb = (u >> 16) & 1u;
        out[i] = (uint16_t)((u + 0x7FFFu + lsb) >> 16);
    }
}

static double nibble_value_f64(unsigned nib, unsigned b, int32_t scale_exp) {
    double sp = if4o_e4m3_value(b & 0x7Fu);
    unsigned mag = nib & 7u;
    double v;
    if (b & 0x80u)
        v = ldexp(6.0 * INT4[mag] * sp, scale_exp) / 7.0;
    else
        v = ldexp(E2M1[mag] * sp, scale_exp);
    return (nib & 8u) ? -v : v;
}

static void decode_row_f64(const uint8_t* codes, const uint8_t* scales,
                           int64_t cols, int32_t scale_exp, double* y) {
    for (int64_t k = 0; k < cols; k++) {
        unsigned b = scales[k / GROUP];
        unsigned byte = codes[k / 2];
        unsigned nib = (k & 1) ? (byte >> 4) : (byte & 0xFu);
        y[k] = nibble_value_f64(nib, b, scale_exp);
    }
}

void if4o_decode_f64(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                     int64_t cols, int32_t scale_exp, double* y, int nthreads) {
    int64_t gpr = cols / GROUP;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
    for (int64_t r = 0; r < rows; r++)
        decode_row_f64(codes + r * (cols / 2), scales + r * gpr, cols, scale_exp,
                       y + r * cols);
}

void if4o_gemm_sample_f64(const uint8_t* a_codes, const uint8_t* a_scales,
                          int32_t a_exp, const uint8_t* w_codes,
                          const uint8_t* w_scales, int32_t w_exp, int64_t K,
                          const int64_t* row_idx, int64_t n_rows,
                          const int64_t* col_idx, int64_t n_cols, double* c,
                          int nthreads) {
    /* C = A * W^T with both operands quantized along K: the W4A4 product of
     * [podcast] "MAC Unit: Decoding Two Formats from One Sign Bit", each
     * operand decoded by its own scale's sign bit, accumulated in fp64 in
     * index order. */
    int64_t gpr = K / GROUP;
    double* ad = (double*)malloc(sizeof(double) * (size_t)(n_rows * K));
    double* wd = (double*)malloc(sizeof(double) * (size_t)(n_cols * K));
    if (!ad || !wd) {
        free(ad);
        free(wd);
        for (int64_t i = 0; i < n_rows * n_cols; i++) c[i] = NAN;
        return;
    }
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
    for (int64_t i = 0; i < n_rows; i++)
        decode_row_f64(a_codes + row_idx[i] * (K / 2), a_scales + row_idx[i] * gpr,
                       K, a_exp, ad + i * K);
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (int64_t j = 0; j < n_cols; j++)
        decode_row_f64(w_codes + col_idx[j] * (K / 2), w_scales + col_idx[j] * gpr,
                       K, w_exp, wd + j * K);
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (int64_t i = 0; i < n_rows; i++) {
        for (int64_t j = 0; j < n_cols; j++) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; k++) acc += ad[i * K + k] * wd[j * K + k];
            c[i * n_cols + j] = acc;
        }
    }
    free(ad);
    free(wd);
}

/* ------------------------------------------------------------------------
 * Random-sign 16-point Hadamard rotation before quantization.  The pages
 * apply a Hadamard transform to smooth outliers, which makes groups more
 * uniform and favours INT4 ([gist] section 1 "O Problema"; [podcast] "Where
 * the Gain Actually Comes From", the Hadamard-transformed weight gradient).
 * They give neither its size nor its arithmetic.  Reading used here: per
 * group of 16, y = H16 (d .* x) / 4 with d the +-1 vector of sign_mask (bit i
 * set: element i negated) and H16 the Sylvester matrix H2 (x) H2 (x) H2 (x) H2,
 * so H16/4 is orthonormal.  In fp32 the product is taken through the butterfly
 * stages of that Kronecker factorisation, strides 1, 2, 4, 8 in that order,
 * each pair (lo, hi) becoming (lo + hi, lo - hi); the quarter is applied last.
 * The rotated tensor keeps its input's precision: for bf16 input each y is
 * rounded to bf16 (nearest even) before it is quantized, which is what the
 * unfused rotate-then-quantize pipeline on a bf16 tensor would produce. */
static float round_bf16(float v) {
    uint16_t h;
    if4o_f32_to_bf16(&v, 1, &h);
    uint32_t u = (uint32_t)h << 16;
    float r;
    memcpy(&r, &u, 4);
    return r;
}

static void rht16_group(const float* x, uint32_t sign_mask, int round_to_bf16, float y[16]) {
    float v[GROUP];
    for (int i = 0; i < GROUP; i++)
        v[i] = ((sign_mask >> i) & 1u) ? -x[i] : x[i];
    for (int h = 1; h < GROUP; h *= 2) {
        for (int i = 0; i < GROUP; i++) {
            if (i & h) continue;
            float lo = v[i], hi = v[i + h];
            v[i] = lo + hi;
            v[i + h] = lo - hi;
        }
    }
    for (int i = 0; i < GROUP; i++) {
        float t = v[i] * 0.25f;
        y[i] = round_to_bf16 ? round_bf16(t) : t;
    }
}

void if4o_rht16(const float* x, int64_t rows, int64_t cols, int64_t ld_x,
                uint32_t sign_mask, int round_to_bf16, float* y, int64_t ld_y,
                int nthreads) {
    int64_t gpr = cols / GROUP;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
    for (int64_t r = 0; r < rows; r++)
        for (int64_t g = 0; g < gpr; g++)
            rht16_group(x + r * ld_x + g * GROUP, sign_mask, round_to_bf16,
                        y + r * ld_y + g * GROUP);
}

void if4o_quantize_rht(const float* x, int64_t rows, int64_t cols, int64_t ld_x,
                       uint32_t sign_mask, int round_to_bf16, int32_t scale_exp,
                       int mode, uint8_t* codes, uint8_t* scales, int nthreads) {
    int64_t gpr = cols / GROUP;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t g = 0; g < gpr; g++) {
            float y[GROUP], ef, ei;
            rht16_group(x + r * ld_x + g * GROUP, sign_mask, round_to_bf16, y);
            if4o_quantize_group(y, scale_exp, mode, codes + r * (cols / 2) + g * 8,
                                scales + r * gpr + g, &ef, &ei);
        }
    }
}

/* ------------------------------------------------------------------------
 * IF3 and IF6: the same adaptive choice at 3 and 6 bits per value ([podcast]
 * "It Generalizes: IF3 and IF6"; [gist] section 2, "Extensoes").  The pages
 * name the formats but define neither grid; the readings here keep IF4's
 * construction -- sign-magnitude codes, one E4M3 scale per 16 values with the
 * choice in its sign bit, the INT range pre-scaled so that its top value
 * lands on the float grid's top value, scale = RNE_E4M3(amax / top), errors
 * compared in fp32 in a domain where the INT descale is exact:
 *   IF6: FP6 = E2M3 (2 exponent bits, bias 1, 3 mantissa bits; top 7.5), INT6
 *        magnitudes 0..31 decoding to q * 7.5/31 * s = q * 15/62 * s; errors
 *        in the x62 domain.
 *   IF3: FP3 = E2M0 (magnitudes 0, 1, 2, 4; top 4), INT3 magnitudes 0..3
 *        decoding to q * 4/3 * s; errors in the x3 domain.  (The other 2-bit
 *        float, E1M1 = {0, 0.5, 1, 1.5}, is the INT grid itself and would
 *        leave no choice.)
 * Codes: bit (bits - 1) = sign of x, the low bits = FP index or |q|; element i
 * of a group occupies bits [bits*i, bits*(i+1)) of the group's little-endian
 * 2*bits-byte field. */
typedef struct {
    int bits;
    const double* fp;
    unsigned nfp;   /* 2^(bits-1) float magnitudes */
    unsigned qmax;  /* 2^(bits-1) - 1 */
    double top;     /* fp[nfp - 1] */
    double dn, dd;  /* top / qmax = dn / dd in lowest terms */
} ifn_format;

static double E2M3[32];
static const double E2M0[4] = {0.0, 1.0, 2.0, 4.0};
static double INT_MAG[32];

__attribute__((constructor)) static void fill_ifn_grids(void) {
    for (unsigned c = 0; c < 32; c++) {
        unsigned e = c >> 3, m = c & 7u;
        E2M3[c] = e == 0 ? m / 8.0 : ldexp(1.0 + m / 8.0, (int)e - 1);
        INT_MAG[c] = (double)c;
    }
}

static int ifn_get(int bits, ifn_format* f) {
    if (bits == 6) {
        *f = (ifn_format){6, E2M3, 32, 31, 7.5, 15.0, 62.0};
        return 0;
    }
    if (bits == 3) {
        *f = (ifn_format){3, E2M0, 4, 3, 4.0, 4.0, 3.0};
        return 0;
    }
    return -1;
}

double if4o_ifn_fp_value(int bits, unsigned idx) {
    ifn_format f;
    if (ifn_get(bits, &f)) return NAN;
    return f.fp[idx % f.nfp];
}

unsigned if4o_ifn_scale_code(int bits, double a_scaled) {
    ifn_format f;
    if (ifn_get(bits, &f)) return 0;
    /* a vs top * midpoint: top has at most 4 bits, the midpoints 5 */
    return rne_index(a_scaled, f.top, e4m3_grid(), 127);
}

unsigned if4o_ifn_fp_index(int bits, double ax, double s) {
    ifn_format f;
    if (ifn_get(bits, &f)) return 0;
    return rne_index(ax, s, f.fp, f.nfp);
}

unsigned if4o_ifn_int_mag(int bits, double ax, double s) {
    ifn_format f;
    if (ifn_get(bits, &f)) return 0;
    /* q = RNE(dd |x| / (dn s)), clamped: dd |x| vs dn s (k + 1/2), exact */
    return rne_index(f.dd * ax, f.dn * s, INT_MAG, f.qmax + 1);
}

static void ifn_quantize_group(const ifn_format* f, const float x[16], int32_t scale_exp,
                               int mode, unsigned code[16], uint8_t* scale_byte, float* err_fp,
                               float* err_int) {
    for (int i = 0; i < GROUP; i++) code[i] = 0;
    *err_fp = 0.0f;
    *err_int = 0.0f;
    for (int i = 0; i < GROUP; i++) {
        if (!isfinite(x[i])) {
            *scale_byte = 0x7F;
            return;
        }
    }
    double a = 0.0;
    for (int i = 0; i < GROUP; i++) {
        double ax = fabs((double)x[i]);
        if (ax > a) a = ax;
    }
    unsigned sc = rne_index(ldexp(a, -scale_exp), f->top, e4m3_grid(), 127);
    if (sc == 0) {
        *scale_byte = 0;
        return;
    }
    double s = ldexp(if4o_e4m3_value(sc), scale_exp);
    unsigned fidx[GROUP], qmag[GROUP];
    for (int i = 0; i < GROUP; i++) {
        double ax = fabs((double)x[i]);
        fidx[i] = rne_index(ax, s, f->fp, f->nfp);
        qmag[i] = rne_index(f->dd * ax, f->dn * s, INT_MAG, f->qmax + 1);
    }
    /* errors in the x dd domain, fp32, index order, one fma per element:
     * d = fma(|x|, dd, -c dd s) and fma(|x|, dd, -|q| dn s); the products
     * c*dd*s and |q|*dn*s have at most 13 bits and are exact in fp32 */
    float sf = (float)s, fdd = (float)f->dd, fdn = (float)f->dn;
    float ef = 0.0f, ei = 0.0f;
    for (int i = 0; i < GROUP; i++) {
        float ax = fabsf(x[i]);
        float cs = (float)f->fp[fidx[i]] * fdd * sf;
        float qs = (float)qmag[i] * fdn * sf;
        float df = fmaf(ax, fdd, -cs);
        float di = fmaf(ax, fdd, -qs);
        ef = fmaf(df, df, ef);
        ei = fmaf(di, di, ei);
    }
    *err_fp = ef;
    *err_int = ei;
    int use_int = mode == IF4O_FORCE_INT4 ? 1 : (mode == IF4O_FORCE_FP4 ? 0 : ei < ef);
    *scale_byte = (uint8_t)(sc | (use_int ? 0x80u : 0u));
    for (int i = 0; i < GROUP; i++) {
        unsigned mag = use_int ? qmag[i] : fidx[i];
        code[i] = (signbit(x[i]) ? (1u << (f->bits - 1)) : 0u) | mag;
    }
}

static void ifn_pack(int bits, const unsigned code[16], uint8_t* out) {
    for (int b = 0; b < 2 * bits; b++) out[b] = 0;
    for (int i = 0; i < GROUP; i++)
        for (int k = 0; k < bits; k++)
            if ((code[i] >> k) & 1u) {
                int bit = bits * i + k;
                out[bit >> 3] |= (uint8_t)(1u << (bit & 7));
            }
}

static unsigned ifn_unpack(int bits, const uint8_t* in, int i) {
    unsigned v = 0;
    for (int k = 0; k < bits; k++) {
        int bit = bits * i + k;
        v |= (unsigned)((in[bit >> 3] >> (bit & 7)) & 1u) << k;
    }
    return v;
}

int if4o_ifn_quantize(int bits, const float* x, int64_t rows, int64_t cols, int64_t ld_x,
                      int32_t scale_exp, int mode, uint8_t* codes, uint8_t* scales,
                      float* err_fp, float* err_int, int nthreads) {
    ifn_format f;
    if (ifn_get(bits, &f) || cols % GROUP) return -1;
    int64_t gpr = cols / GROUP, cb = gpr * 2 * bits;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t g = 0; g < gpr; g++) {
            unsigned code[GROUP];
            float ef, ei;
            ifn_quantize_group(&f, x + r * ld_x + g * GROUP, scale_exp, mode, code,
                               scales + r * gpr + g, &ef, &ei);
            ifn_pack(bits, code, codes + r * cb + g * 2 * bits);
            if (err_fp) err_fp[r * gpr + g] = ef;
            if (err_int) err_int[r * gpr + g] = ei;
        }
    }
    return 0;
}

/* Dequantize: FP -> sign * fp[idx] * s' * 2^E (exact); INT -> sign *
 * fl32(|q| dn s' / dd) * 2^E: |q| dn s' has at most 13 bits, so the fp64
 * quotient is never within 2^-53 of an fp32 midpoint and the two roundings
 * equal one. */
int if4o_ifn_dequantize(int bits, const uint8_t* codes, const uint8_t* scales, int64_t rows,
                        int64_t cols, int32_t scale_exp, float* y, int64_t ld_y, int nthreads) {
    ifn_format f;
    if (ifn_get(bits, &f) || cols % GROUP) return -1;
    int64_t gpr = cols / GROUP, cb = gpr * 2 * bits;
    float p2 = ldexpf(1.0f, scale_exp);
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t k = 0; k < cols; k++) {
            int64_t g = k / GROUP;
            unsigned b = scales[r * gpr + g];
            unsigned code = ifn_unpack(bits, codes + r * cb + g * 2 * bits, (int)(k % GROUP));
            unsigned mag = code & ((1u << (bits - 1)) - 1u);
            double sp = if4o_e4m3_value(b & 0x7Fu);
            float v;
            if (b & 0x80u)
                v = (float)((mag * f.dn * sp) / f.dd);
            else
                v = (float)(f.fp[mag] * sp);
            if ((code >> (bits - 1)) & 1u) v = -v;
            y[r * ld_y + k] = v * p2;
        }
    }
    return 0;
}
