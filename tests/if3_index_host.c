/*
 * Host model of the IF3 bf16 fast path's float index (quantize_ifn_kernel,
 * fast_group_bf16), checked against the oracle's IF3 rounding
 * (if4o_ifn_fp_index / if4o_ifn_fp_value) for every non-negative finite bf16
 * |x|, every nonzero E4M3 scale code s' and a set of exponents E.
 *
 * The kernel's steps, with the host's correctly rounded fmaf / frexpf /
 * ldexpf standing in for v_fma_f32 / v_frexp_exp_i32_f32 / v_ldexp_f32
 * (each exact or correctly rounded on both):
 *   r   = rcp(s') refined by one Newton step; rcp is modelled as the
 *         correctly rounded 1/s' moved by -2..+2 ulp (v_rcp_f32 is within 1)
 *   rs  = r 2^-E,  rsk = rs 2^18,  ra = fl(rs * A),  A = fl32(4/3 - 2^-16)
 *   h   = clamp01(fma(|x|, rsk, -(2^17 + 2)))      (u > 0.5 + 2^-17)
 *   f   = med3(fma(|x|, ra, C), h, 7.99)           C = 2^-15 by default
 *   idx = max(frexp_exp(f), 0),  2 * value = ldexp(h, idx)
 * Usage: if3_index_host [C [cap [nE]]]: C the additive constant (a margin
 * that is too small or too large must fail), cap 0 to drop the cap below 8
 * (products that overflow must then fail), nE how many exponents of the list
 * to run.  Prints "checked N mismatches M" and exits 1 if M > 0.
 * Test infrastructure: links the oracle, which only tests may do.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "if4_oracle.h"

static float u2f(uint32_t u) {
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static float e4m3(unsigned c) { return c >= 8 ? u2f((c + 960u) << 20) : (float)c * 0.001953125f; }

int main(int argc, char** argv) {
    const float C = argc > 1 ? strtof(argv[1], NULL) : 0x1p-15f;
    const int cap = argc > 2 ? atoi(argv[2]) : 1;
    static const int kE[] = {0, 7, -9, 20, -20, 60, -60, 64, -64};
    const int nE = argc > 3 ? atoi(argv[3]) : 9;
    const float A = 1.33331811f;
    long n = 0, bad = 0;
    for (int ei = 0; ei < nE; ei++) {
        const int E = kE[ei];
        const float pneg = ldexpf(1.0f, -E);
        for (unsigned sc = 1; sc < 127; sc++) {
            const float sp = e4m3(sc);
            const double s = ldexp((double)sp, E);
            for (int k = -2; k <= 2; k++) {
                float r0 = 1.0f / sp;
                for (int j = 0; j < abs(k); j++) r0 = nextafterf(r0, k < 0 ? 0.0f : INFINITY);
                const float r = fmaf(r0, fmaf(-sp, r0, 1.0f), r0);
                const float rs = r * pneg, rsk = rs * 0x1p18f, ra = rs * A;
                for (uint32_t b = 0; b < 0x7F80u; b++) {
                    const float ax = u2f(b << 16);
                    const float h = fminf(fmaxf(fmaf(ax, rsk, -131074.0f), 0.0f), 1.0f);
                    float f = fmaf(ax, ra, C);
                    if (cap) f = fminf(f, 7.99f);
                    f = fmaxf(f, h);
                    int e = 0;
                    frexpf(f, &e);
                    if (isinf(f) || isnan(f)) e = 0; /* v_frexp_exp_i32_f32 of inf / NaN */
                    const int idx = e > 0 ? e : 0;
                    const float twice = ldexpf(h, idx);
                    const unsigned ref = if4o_ifn_fp_index(3, (double)ax, s);
                    const double refv = if4o_ifn_fp_value(3, ref);
                    n++;
                    if ((unsigned)idx != ref || (double)twice != 2.0 * refv || (h != 0.0f && h != 1.0f)) {
                        if (bad < 5)
                            printf("mismatch E=%d s'=%g rcp%+d |x|=%g index %d oracle %u\n", E, sp, k,
                                   ax, idx, ref);
                        bad++;
                    }
                }
            }
        }
    }
    printf("checked %ld mismatches %ld\n", n, bad);
    return bad != 0;
}
