// IF4 quantize for gfx950.
//
// Method ("Adaptive Block-Scaled Data Types": shd-paper.top card, method
// details, framework steps 1-5; gist.science summary, section 2
// "Metodologia"): per group of 16 values one E4M3 scale from the group
// absmax; encode as FP4 (E2M1) and as INT4 pre-scaled by 7/6; keep the
// encoding with the lower squared error; flag INT4 in the scale byte's sign
// bit.  The exact rules (roundings, ties, error order, bit layout) are stated
// in include/if4.h.
//
// Layout: one lane owns one whole group, so the amax, both encodings, both
// error sums, the selection and the nibble packing happen in that lane's
// registers with no cross-lane traffic.  A wave reads 64 consecutive groups
// (2 KB of bf16) and writes 512 B of codes and 64 B of scales, all
// contiguous.  The bf16 kernel is one-shot (one group per thread, its loads
// issued first); the exact fp32 kernel is a grid-stride loop.
//
// Every rounding decision is taken exactly, for any fp32 input: each code
// is the count of grid midpoints the value passes, compared against exactly
// representable thresholds (s * midpoint for FP4; 7|x| - 3s(2k+1) by fma for
// INT4), with ties resolved to the even code by using >= or > per midpoint.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "if4_internal.h"

namespace if4 {
namespace {

constexpr int kThreads = 256;

// E4M3 code (0..126) of RNE(a / 6), saturating at 448 (0x7E).  The fp32
// quotient is correctly rounded; rounding it again to 3 mantissa bits equals
// one rounding of the exact quotient because a/6 is never within half an
// fp32 ulp of an E4M3 midpoint M unless a = 6M exactly.
__device__ __forceinline__ uint32_t scale_code(float a_scaled) {
    float q = a_scaled / 6.0f;
    if (q < 0.015625f)  // below 2^-6: subnormal E4M3, spacing 2^-9
        return (uint32_t)__builtin_rintf(q * 512.0f);
    uint32_t b = __float_as_uint(q);
    b = b + 0x7FFFFu + ((b >> 20) & 1u);  // round the mantissa to 3 bits, ties even
    uint32_t code = (b >> 20) - 960u;     // (exponent + 120) << 3 | mantissa
    return code < 0x7Eu ? code : 0x7Eu;
}

__device__ __forceinline__ float e4m3_value(uint32_t code) {
    return code >= 8u ? __uint_as_float((code + 960u) << 20) : (float)code * 0.001953125f;
}

// E2M1 index of |x| / s (ties to the even index, saturating at 6).
__device__ __forceinline__ uint32_t fp4_index(float ax, float s) {
    uint32_t i = 0;
    i += ax > 0.25f * s;
    i += ax >= 0.75f * s;
    i += ax > 1.25f * s;
    i += ax >= 1.75f * s;
    i += ax > 2.5f * s;
    i += ax >= 3.5f * s;
    i += ax > 5.0f * s;
    return i;
}

// min(RNE(7|x| / (6s)), 7): count the half-integers 7|x|/(6s) passes;
// t3 = 3s, midpoint k + 1/2 <=> 7|x| = 3s(2k+1).
__device__ __forceinline__ uint32_t int4_mag(float ax, float t3) {
    uint32_t q = 0;
#pragma unroll
    for (int k = 0; k < 7; k++) {
        float d = __builtin_fmaf(ax, 7.0f, -(float)(2 * k + 1) * t3);
        q += (k & 1) ? (d >= 0.0f) : (d > 0.0f);
    }
    return q;
}

__device__ __forceinline__ float e2m1_value(uint32_t idx) {
    // 0, .5, 1, 1.5, 2, 3, 4, 6
    float m = (idx & 1u) ? 1.5f : 1.0f;
    uint32_t e = idx >> 1;
    return e == 0 ? (idx ? 0.5f : 0.0f) : m * (float)(1u << (e - 1));
}

template <bool kBf16>
__device__ __forceinline__ void load_group(const void* __restrict__ x, int64_t off,
                                           float (&v)[16]) {
    if constexpr (kBf16) {
        const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + off);
        uint4 a = *p;
        uint4 b = p[1];
        uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; i++) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    } else {
        const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + off);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            float4 t = p[i];
            v[4 * i] = t.x;
            v[4 * i + 1] = t.y;
            v[4 * i + 2] = t.z;
            v[4 * i + 3] = t.w;
        }
    }
}

// One group, exact rules for any fp32 values (x 2^-E): codes (element 2j in
// the low nibble of byte j of lo:hi) and the flagged scale byte.
template <int kMode>
__device__ __forceinline__ void exact_group(const float (&v)[16], float p_exp, float p_negexp,
                                            uint32_t& lo, uint32_t& hi, uint32_t& byte) {
    // group absmax; a NaN or infinity anywhere makes the group non-finite
    float a = 0.0f;
    bool finite = true;
#pragma unroll
    for (int i = 0; i < 16; i++) {
        float ax = __builtin_fabsf(v[i]);
        finite &= ax <= 3.40282347e38f;
        a = __builtin_fmaxf(a, ax);
    }
    uint32_t sc = scale_code(a * p_negexp);
    lo = 0, hi = 0, byte = 0;
    if (!finite) {
        byte = 0x7Fu;
    } else if (sc != 0) {
        const float s = e4m3_value(sc) * p_exp;
        const float s7 = 7.0f * s, s6 = 6.0f * s, t3 = 3.0f * s;
        float ef = 0.0f, ei = 0.0f;
        uint32_t fl = 0, fh = 0, il = 0, ih = 0;
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const float ax = __builtin_fabsf(v[i]);
            const uint32_t fi = fp4_index(ax, s);
            const uint32_t qi = int4_mag(ax, t3);
            const float df = __builtin_fmaf(ax, 7.0f, -(e2m1_value(fi) * s7));
            const float di = __builtin_fmaf(ax, 7.0f, -((float)qi * s6));
            ef = __builtin_fmaf(df, df, ef);
            ei = __builtin_fmaf(di, di, ei);
            const uint32_t sg = (__float_as_uint(v[i]) >> 28) & 8u;
            if (i < 8) {
                fl |= (sg | fi) << (4 * i);
                il |= (sg | qi) << (4 * i);
            } else {
                fh |= (sg | fi) << (4 * (i - 8));
                ih |= (sg | qi) << (4 * (i - 8));
            }
        }
        const bool use_int4 = kMode == 2 ? true : (kMode == 1 ? false : (ei < ef));
        lo = use_int4 ? il : fl;
        hi = use_int4 ? ih : fh;
        byte = sc | (use_int4 ? 0x80u : 0u);
    }
}

// Random-sign 16-point Hadamard rotation applied before quantization: the
// pages use a Hadamard transform to smooth outliers, which leaves groups more
// uniform and favours the INT4 encoding ("Adaptive Block-Scaled Data Types",
// gist.science summary, section 1 "O Problema"; podcast companion, "Where the
// Gain Actually Comes From").  Per group y = H16 (d .* x) / 4 with H16 the
// Sylvester matrix H2 (x) H2 (x) H2 (x) H2, taken in fp32 through its butterfly
// stages, strides 1, 2, 4, 8 in that order, each pair (lo, hi) becoming
// (lo + hi, lo - hi), then the exact quarter.  The caller has already applied
// the signs d (an xor of the input's sign bits, exact).
__device__ __forceinline__ void hadamard16(float (&v)[16]) {
#pragma clang fp contract(off)
#pragma unroll
    for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 16; i++) {
            if (i & h) continue;
            const float lo = v[i], hi = v[i + h];
            v[i] = lo + hi;
            v[i + h] = lo - hi;
        }
    }
#pragma unroll
    for (int i = 0; i < 16; i++) v[i] *= 0.25f;
}

// ---------------------------------------------------------------------------
// Exact reference path (any fp32 input): thresholds compared exactly.  One-wave
// workgroups, as for the bf16 kernel: a small tensor (the 256x256 one holds
// 4096 groups) then spreads over 64 CUs instead of 16.
constexpr int kExactThreads = 64;
template <bool kBf16, int kMode, bool kRotate>
__global__ void __launch_bounds__(kExactThreads)
quantize_exact_kernel(const void* __restrict__ x, int64_t rows, int64_t gpr, int64_t ld_x,
                      uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float p_exp,
                      float p_negexp, uint32_t sign_mask) {
    const int64_t ngroups = rows * gpr;
    const int64_t stride = (int64_t)gridDim.x * kExactThreads;
    for (int64_t g = (int64_t)blockIdx.x * kExactThreads + threadIdx.x; g < ngroups; g += stride) {
        const int64_t r = g / gpr;
        const int64_t cg = g - r * gpr;
        float v[16];
        load_group<kBf16>(x, r * ld_x + cg * 16, v);
        if constexpr (kRotate) {
#pragma unroll
            for (int i = 0; i < 16; i++)
                v[i] = __uint_as_float(__float_as_uint(v[i]) ^ (((sign_mask >> i) & 1u) << 31));
            hadamard16(v);
            if constexpr (kBf16) {  // the rotated tensor keeps bf16 precision
#pragma unroll
                for (int i = 0; i < 16; i++) v[i] = (float)(__bf16)v[i];
            }
        }

        uint32_t lo, hi, byte;
        exact_group<kMode>(v, p_exp, p_negexp, lo, hi, byte);
        *reinterpret_cast<uint2*>(codes + g * 8) = make_uint2(lo, hi);
        scales[g] = (uint8_t)byte;
    }
}

// ---------------------------------------------------------------------------
// Fast bf16 path.  Same results as the exact path for every bf16 input (the
// GPU tests sweep every (bf16 x, E4M3 s') pair), with cheaper arithmetic:
//
//  * scale: RNE_E4M3(a/6) from fl(a * fl(1/6)).  fl(1/6) is 1/6 (1 - e) with
//    e < 2^-25, so a tie a/6 = M (an E4M3 midpoint, 5 bits) rounds back to M
//    exactly, and a bf16 a (8 bits) is never within 2^-9 relative of any other
//    midpoint, far beyond the product's error.
//  * codes: u = |x|/s is approximated as |x| * r, r an approximation of 1/s
//    within 2.2 * 2^-24 relative, and snapped to a 2^-18 grid in the same fma
//    (adding 48 puts the sum in [32, 64), whose fp32 spacing is 2^-18); 7u/6
//    likewise with r7 ~ 7/(6s).  Every midpoint of either grid is a multiple
//    of 2^-18, and at the largest midpoint that matters (5 for u, 6.5 for
//    7u/6) the approximation error is below 6.5 * 2.2 * 2^-24 < 2^-20, well
//    inside half the grid spacing, so a value exactly on a midpoint snaps onto
//    it and every other value stays on its side (a bf16 x sits at least 2^-16
//    from any midpoint of u or 7u/6 that it does not hit).  r is v_rcp_f32 of
//    s' (within one ulp) refined by one Newton step (then within half an ulp
//    plus a 2^-46 relative term), r7 = r + r * fl(1/6) in one fma; the power
//    of two 2^-E is applied exactly after.  FP4: the snapped value carries x's
//    sign into the hardware E2M1
//    conversion (round to nearest even, saturating, signed zero kept), and
//    the same hardware decodes the codes back for the error.  INT4: adding
//    1.5 * 2^23 - 48 rounds the snapped 7|x|/(6s) to an integer (ties even),
//    min() clamps it to 7, and the low bits of the float are |q|.
//  * errors: for bf16 x every d = 7x - c*7s or 7|x| - |q|*6s is exact in
//    fp32, so fma(-c, 7s, 7x) equals the reference fma(|x|, 7, -|c|*7s).
//  * non-finite: a NaN reaches the FP4 error sum (NaN) and an infinity the
//    absmax; zero-scale groups use zero reciprocals so their sums stay finite.
// (An earlier version took r and r7 from a per-workgroup LDS table of
// correctly rounded reciprocals; computing them per group costs fewer
// instructions than filling the table, and drops its barrier.)

// One group of bf16-exact values, fast path (see above): codes and flagged
// scale byte, identical to exact_group for bf16 inputs.
template <int kMode, bool kElideClamp = false>
__device__ __forceinline__ void fast_group(const float (&v)[16],
                                           float p_exp, float p_negexp, uint32_t& lo,
                                           uint32_t& hi, uint32_t& byte) {
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; i++) a = __builtin_fmaxf(a, __builtin_fabsf(v[i]));

    // scale code: RNE_E4M3(a * 2^-E / 6), saturating at 448
    const float q6 = (a * p_negexp) * 0.16666667f;
    uint32_t sc;
    if (q6 < 0.015625f) {
        sc = (uint32_t)__builtin_rintf(q6 * 512.0f);
    } else {
        uint32_t b = __float_as_uint(q6);
        b = b + 0x7FFFFu + ((b >> 20) & 1u);
        sc = (b >> 20) - 960u;
        sc = sc < 0x7Eu ? sc : 0x7Eu;
    }
    const float sp = e4m3_value(sc);
    const float s = sp * p_exp;
    float r = __builtin_amdgcn_rcpf(sp);
    r = __builtin_fmaf(r, __builtin_fmaf(-sp, r, 1.0f), r);
    float r7 = __builtin_fmaf(r, 0.16666667f, r);
    r = sc != 0 ? r : 0.0f;  // (rcp(0) is infinite)
    r7 = sc != 0 ? r7 : 0.0f;
    const float inv_s = r * p_negexp, k7 = r7 * p_negexp;
    const float s7 = 7.0f * s, s6 = 6.0f * s;

    // FP4 codes via the hardware E2M1 conversion of the snapped quotients
    float us[16];
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const float t = __builtin_fmaf(__builtin_fabsf(v[i]), inv_s, 48.0f) - 48.0f;
        us[i] = __builtin_copysignf(t, v[i]);
    }
    uint32_t f0 = 0, f1 = 0;
    f0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(f0, us[0], us[1], 1.0f, 0);
    f0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(f0, us[2], us[3], 1.0f, 1);
    f0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(f0, us[4], us[5], 1.0f, 2);
    f0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(f0, us[6], us[7], 1.0f, 3);
    f1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(f1, us[8], us[9], 1.0f, 0);
    f1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(f1, us[10], us[11], 1.0f, 1);
    f1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(f1, us[12], us[13], 1.0f, 2);
    f1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(f1, us[14], us[15], 1.0f, 3);
    float c[16];
    {
        auto d0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(f0, 1.0f, 0);
        auto d1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(f0, 1.0f, 1);
        auto d2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(f0, 1.0f, 2);
        auto d3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(f0, 1.0f, 3);
        auto d4 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(f1, 1.0f, 0);
        auto d5 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(f1, 1.0f, 1);
        auto d6 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(f1, 1.0f, 2);
        auto d7 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(f1, 1.0f, 3);
        c[0] = d0[0]; c[1] = d0[1]; c[2] = d1[0]; c[3] = d1[1];
        c[4] = d2[0]; c[5] = d2[1]; c[6] = d3[0]; c[7] = d3[1];
        c[8] = d4[0]; c[9] = d4[1]; c[10] = d5[0]; c[11] = d5[1];
        c[12] = d6[0]; c[13] = d6[1]; c[14] = d7[0]; c[15] = d7[1];
    }

    // INT4 magnitudes and both error sums, index order 0..15.  The clamp
    // |q| <= 7 can only act when s' is an E4M3 subnormal (codes 1-7, spaced
    // 2^-9 apart, so s' may sit far below a'/6) or when a'/6 reaches 448 (the
    // scale saturates).  For every other scale s' >= (a'/6) / (1 + 2^-4) --
    // rounding to three mantissa bits moves a value down by at most 2^-4 of
    // its binade's base -- so 7|x|/(6s) <= 7 * 1.0625 = 7.4375 (plus the
    // snapped quotient's error, below 2^-20) rounds to at most 7 without it.
    // With kElideClamp the clamp is taken out of the loop when no lane of the
    // wave needs it, at the cost of a second copy of the loop: 16 fewer VALU
    // per group on the row kernel (3-5% faster on 86-470 MB tensors); the x^T
    // kernels gain nothing from it and the rotating kernel runs 1-2% slower.
    float ef = 0.0f, ei = 0.0f;
    uint32_t rq[16];
    auto int4_pass = [&](auto clamp_c) {
        constexpr bool kClamp = decltype(clamp_c)::value;
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const float xa = __builtin_fabsf(v[i]);
            const float X = 7.0f * v[i];
            const float t = __builtin_fmaf(xa, k7, 48.0f);
            // 1.5*2^23 + |q|, clamped to |q| <= 7 (positive floats order as
            // their bits)
            uint32_t rb = __float_as_uint(t + 12582864.0f);
            if constexpr (kClamp) rb = __builtin_elementwise_min(rb, 0x4B400007u);
            rq[i] = rb;
            const float q = __uint_as_float(rb) - 12582912.0f;
            const float df = __builtin_fmaf(-c[i], s7, X);
            const float di = __builtin_fmaf(-q, s6, __builtin_fabsf(X));
            ef = __builtin_fmaf(df, df, ef);
            ei = __builtin_fmaf(di, di, ei);
        }
    };
    const bool need_clamp = (sc - 1u < 7u) || (q6 >= 448.0f);
    if (!kElideClamp || __builtin_amdgcn_ballot_w64(need_clamp) != 0)
        int4_pass(std::true_type{});
    else
        int4_pass(std::false_type{});
    // gather |q| (low byte of each float) into nibbles: even elements in
    // bits 0-2, odd elements in bits 4-6 of each byte
    uint32_t i0, i1;
    {
        const uint32_t e0 = __builtin_amdgcn_perm(rq[2], rq[0], 0x0C0C0400u) |
                            __builtin_amdgcn_perm(rq[6], rq[4], 0x04000C0Cu);
        const uint32_t o0 = __builtin_amdgcn_perm(rq[3], rq[1], 0x0C0C0400u) |
                            __builtin_amdgcn_perm(rq[7], rq[5], 0x04000C0Cu);
        const uint32_t e1 = __builtin_amdgcn_perm(rq[10], rq[8], 0x0C0C0400u) |
                            __builtin_amdgcn_perm(rq[14], rq[12], 0x04000C0Cu);
        const uint32_t o1 = __builtin_amdgcn_perm(rq[11], rq[9], 0x0C0C0400u) |
                            __builtin_amdgcn_perm(rq[15], rq[13], 0x04000C0Cu);
        // sign bits are those of the FP4 codes (both take x's sign bit)
        i0 = (e0 | (o0 << 4)) | (f0 & 0x88888888u);
        i1 = (e1 | (o1 << 4)) | (f1 & 0x88888888u);
    }

    const bool use_int4 = kMode == 2 ? true : (kMode == 1 ? false : (ei < ef));
    lo = use_int4 ? i0 : f0;
    hi = use_int4 ? i1 : f1;
    byte = sc | (use_int4 ? 0x80u : 0u);
    if (sc == 0) {
        lo = hi = 0;
        byte = 0;
    }
    if (!(a <= 3.40282347e38f) || ef != ef) {  // infinity or NaN in the group
        lo = hi = 0;
        byte = 0x7Fu;
    }
}

// The bf16 kernel is one-shot: each thread quantizes kGPT groups, kRowThreads
// apart (a wave's loads stay contiguous: 64 lanes x 32 bytes), with all of its
// loads issued before the first group is quantized, and one workgroup per
// kRowThreads * kGPT groups.  Past the end a load re-reads the last group and
// its store is skipped, so no load sits behind a branch.  One group per
// thread: on the 470 MB weight one, two and four groups per thread run alike,
// and on 86-172 MB tensors one is 4-9% faster (more, smaller workgroups fill
// the chip sooner and leave a shorter tail); for the same reason workgroups of
// one wave run faster than two (1.5-4%) and two faster than four or eight
// (1-2%).  (A grid-stride loop over fewer workgroups, with the next group
// prefetched into a second register set, measured 8-11% slower on the weight.)
constexpr int kRowThreads = 64;
constexpr int kGPT = 1;

// The rotation's signs as xor words on the bf16 input words (element 2j in
// the low half of word j, element 2j + 1 in the high half), computed on the
// host so that each reaches the kernel as one scalar: a word split into its
// two sign bits makes the compiler fuse the xor into a three-operand
// instruction with two scalar operands, one of which then has to be copied
// to a vector register for every group.
struct SignWords {
    uint32_t w[8];
};

inline SignWords sign_words(uint32_t sign_mask) {
    SignWords f;
    for (int j = 0; j < 8; j++)
        f.w[j] = (((sign_mask >> (2 * j)) & 1u) << 15) | (((sign_mask >> (2 * j + 1)) & 1u) << 31);
    return f;
}

template <int kMode, bool kContig, bool kRotate>
__global__ void __launch_bounds__(kRowThreads)
quantize_bf16_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t gpr, int64_t ld_x,
                     uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float p_exp,
                     float p_negexp, SignWords flip) {
    const int64_t ngroups = rows * gpr, last = ngroups - 1;
    const int64_t g0 = (int64_t)blockIdx.x * (kRowThreads * kGPT) + threadIdx.x;
    uint4 a[kGPT], b[kGPT];
#pragma unroll
    for (int k = 0; k < kGPT; k++) {
        int64_t g = g0 + k * kRowThreads;
        g = g < last ? g : last;
        int64_t off;
        if constexpr (kContig) {
            off = g * 16;
        } else {
            const int64_t r = g / gpr;
            off = r * ld_x + (g - r * gpr) * 16;
        }
        const uint4* p = reinterpret_cast<const uint4*>(x + off);
        a[k] = p[0];
        b[k] = p[1];
    }
#pragma unroll
    for (int k = 0; k < kGPT; k++) {
        const int64_t g = g0 + k * kRowThreads;
        uint32_t w[8] = {a[k].x, a[k].y, a[k].z, a[k].w, b[k].x, b[k].y, b[k].z, b[k].w};
        if constexpr (kRotate) {
#pragma unroll
            for (int i = 0; i < 8; i++) w[i] ^= flip.w[i];
        }
        float v[16];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
        if constexpr (kRotate) {
            // rotate in fp32, then round back to bf16 (nearest even), two
            // values per conversion: the values the fast path needs are
            // bf16-exact
            hadamard16(v);
#pragma unroll
            for (int i = 0; i < 8; i++) {
                typedef float float2v __attribute__((ext_vector_type(2)));
                typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
                const float2v f = {v[2 * i], v[2 * i + 1]};
                const uint32_t u = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2v));
                v[2 * i] = __uint_as_float(u << 16);
                v[2 * i + 1] = __uint_as_float(u & 0xFFFF0000u);
            }
        }
        uint32_t lo, hi, byte;
        fast_group<kMode, !kRotate>(v, p_exp, p_negexp, lo, hi, byte);
        if (g < ngroups) {
            *reinterpret_cast<uint2*>(codes + g * 8) = make_uint2(lo, hi);
            scales[g] = (uint8_t)byte;
        }
    }
}

template <bool kBf16, int kMode, bool kRotate>
hipError_t launch(const void* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* codes,
                  uint8_t* scales, int32_t scale_exp, uint32_t sign_mask, hipStream_t stream) {
    const int64_t gpr = cols / 16;
    const int64_t ngroups = rows * gpr;
    const float pe = pow2f(scale_exp), pn = pow2f(-scale_exp);
    if constexpr (kBf16) {
        const int64_t blocks = (ngroups + kRowThreads * kGPT - 1) / (kRowThreads * kGPT);
        if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
        const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
        if (ld_x == cols)
            hipLaunchKernelGGL((quantize_bf16_kernel<kMode, true, kRotate>),
                               dim3((unsigned)blocks), dim3(kRowThreads), 0, stream, xb, rows, gpr,
                               ld_x, codes, scales, pe, pn, sign_words(sign_mask));
        else
            hipLaunchKernelGGL((quantize_bf16_kernel<kMode, false, kRotate>),
                               dim3((unsigned)blocks), dim3(kRowThreads), 0, stream, xb, rows, gpr,
                               ld_x, codes, scales, pe, pn, sign_words(sign_mask));
    } else {
        // the exact kernel: one group per thread where the grid allows (up to
        // 2^24 groups per pass, then a grid-stride loop)
        int64_t blocks = (ngroups + kExactThreads - 1) / kExactThreads;
        if (blocks > 262144) blocks = 262144;
        hipLaunchKernelGGL((quantize_exact_kernel<false, kMode, kRotate>), dim3((unsigned)blocks),
                           dim3(kExactThreads), 0, stream, x, rows, gpr, ld_x, codes, scales, pe,
                           pn, sign_mask);
    }
    return hipGetLastError();
}


// ---------------------------------------------------------------------------
// Quantize of x^T: groups are 16 consecutive rows of one column of x, and
// the output is the IF4 encoding of x^T ([cols, rows] row-major: codes
// [cols, rows/2], scales [cols, rows/16]) -- the operand layout the backward
// GEMMs of W4A4G4 training need (dgrad groups W along N, wgrad groups dY and
// X along M).  Same per-group arithmetic as the row kernels.  A workgroup
// owns 256 consecutive columns (one per lane) and a chunk of kTChunk
// row-groups: each of a group's 16 loads reads 64 consecutive columns of one
// row (coalesced), and each lane writes its column's codes for consecutive
// row-groups, filling whole 128-byte lines.  The next group's 16 values are
// loaded while the current one is quantized.
constexpr int kTChunk = 16;

template <bool kBf16, int kMode>
__global__ void __launch_bounds__(kThreads)
quantize_t_kernel(const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
                  uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float p_exp,
                  float p_negexp, int64_t col_blocks) {
    const int64_t cb = blockIdx.x % col_blocks, chunk = blockIdx.x / col_blocks;
    const int64_t col = cb * kThreads + threadIdx.x;
    const int64_t rgs = rows / 16;
    const int64_t rg0 = chunk * kTChunk;
    const int64_t rg1 = rg0 + kTChunk < rgs ? rg0 + kTChunk : rgs;
    if (col >= cols) return;

    uint32_t raw[16];
    auto load = [&](int64_t rg) {
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const int64_t off = (rg * 16 + i) * ld_x + col;
            if constexpr (kBf16)
                raw[i] = reinterpret_cast<const uint16_t*>(x)[off];
            else
                raw[i] = reinterpret_cast<const uint32_t*>(x)[off];
        }
    };
    load(rg0);
    for (int64_t rg = rg0; rg < rg1; rg++) {
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; i++) v[i] = __uint_as_float(kBf16 ? raw[i] << 16 : raw[i]);
        if (rg + 1 < rg1) load(rg + 1);
        uint32_t lo, hi, byte;
        if constexpr (kBf16)
            fast_group<kMode>(v, p_exp, p_negexp, lo, hi, byte);
        else
            exact_group<kMode>(v, p_exp, p_negexp, lo, hi, byte);
        *reinterpret_cast<uint2*>(codes + col * (rows / 2) + rg * 8) = make_uint2(lo, hi);
        scales[col * rgs + rg] = (uint8_t)byte;
    }
}

// Tiled form of the x^T quantize, for 16-byte aligned rows: a workgroup
// takes a tile of 128 rows x 128 columns of x.  Each lane takes a pair of
// adjacent columns and two consecutive row-groups (wave w: row-groups 2w,
// 2w+1 of the tile) and loads its 32 rows straight from memory, one word per
// row for both columns -- the 64 lanes of a wave read one contiguous 256-byte
// row segment (512 for fp32) per load -- and quantizes its four groups.  The
// results go through LDS (codes [128 columns][64 bytes], scales [128
// columns][8 bytes], at padded pitches) so that the workgroup writes each
// column's 64 code bytes and 8 scale bytes with neighbouring lanes on
// neighbouring bytes: written straight from the lanes, every store instruction
// touched 64 cache lines, one per column.  (Staging the input tile in LDS
// first, with 16-byte loads, measured slower: it costs 32 KB of LDS per
// workgroup and a full barrier before any group is quantized.)
constexpr int kTR = 128, kTC = 128;  // tile rows (8 row-groups) and columns
constexpr int kTRG = kTR / 16;       // row-groups per tile

template <bool kBf16, int kMode>
__global__ void __launch_bounds__(kThreads)
quantize_t_tile_kernel(const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
                       uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float p_exp,
                       float p_negexp, int64_t col_tiles, int wide_out) {
    constexpr int kElem = kBf16 ? 2 : 4;
    // results only: codes [kTC][kCodePitch], scales [kTC][kScalePitch]
    constexpr int kCodePitch = kTRG * 8 + 8;       // 64 code bytes per column
    constexpr int kScalePitch = kTRG + 4;          // 8 scale bytes per column
    __shared__ __attribute__((aligned(16))) uint8_t obuf[kTC * (kCodePitch + kScalePitch)];

    const int64_t ct = blockIdx.x % col_tiles, rt = blockIdx.x / col_tiles;
    const int64_t c0 = ct * kTC, r0 = rt * kTR;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint8_t* xb = reinterpret_cast<const uint8_t*>(x);

    // this lane: tile columns 2*lane, 2*lane + 1 (one word per row for bf16,
    // two for fp32); tile row-groups 2*wave, +1 (rows 32*wave .. +31).  The
    // 64 lanes of a wave read one contiguous 256-byte (512 for fp32) row
    // segment per load.  Out-of-range rows and columns read as zero (their
    // groups are never stored); interior tiles skip the checks.
    float ve[32], vo[32];
    const int64_t gc = c0 + 2 * lane, gr = r0 + 32 * wave;
    if (r0 + kTR <= rows && c0 + kTC <= cols) {
        const uint8_t* p = xb + (gr * ld_x + gc) * kElem;
        const uint32_t ld_bytes = (uint32_t)(ld_x * kElem);
        if constexpr (kBf16) {
            uint32_t wd[32];
#pragma unroll
            for (int rr = 0; rr < 32; rr++)
                wd[rr] = *reinterpret_cast<const uint32_t*>(p + rr * ld_bytes);
#pragma unroll
            for (int rr = 0; rr < 32; rr++) {
                ve[rr] = __uint_as_float(wd[rr] << 16);
                vo[rr] = __uint_as_float(wd[rr] & 0xFFFF0000u);
            }
        } else {
#pragma unroll
            for (int rr = 0; rr < 32; rr++) {
                const uint2 wd = *reinterpret_cast<const uint2*>(p + rr * ld_bytes);
                ve[rr] = __uint_as_float(wd.x);
                vo[rr] = __uint_as_float(wd.y);
            }
        }
    } else {
#pragma unroll
        for (int rr = 0; rr < 32; rr++) {
            const int64_t r = gr + rr;
            float e = 0.0f, o = 0.0f;
            if (r < rows) {
                const uint8_t* q = xb + (r * ld_x + gc) * kElem;
                if constexpr (kBf16) {
                    if (gc < cols) e = __uint_as_float((uint32_t)*reinterpret_cast<const uint16_t*>(q) << 16);
                    if (gc + 1 < cols)
                        o = __uint_as_float((uint32_t)*reinterpret_cast<const uint16_t*>(q + 2) << 16);
                } else {
                    if (gc < cols) e = *reinterpret_cast<const float*>(q);
                    if (gc + 1 < cols) o = *reinterpret_cast<const float*>(q + 4);
                }
            }
            ve[rr] = e;
            vo[rr] = o;
        }
    }
    auto group = [&](const float* src, uint32_t& lo, uint32_t& hi, uint32_t& byte) {
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; i++) v[i] = src[i];
        if constexpr (kBf16)
            fast_group<kMode>(v, p_exp, p_negexp, lo, hi, byte);
        else
            exact_group<kMode>(v, p_exp, p_negexp, lo, hi, byte);
    };
    uint32_t lo[2][2], hi[2][2], by[2][2];  // [column][row-group]
#pragma unroll
    for (int cj = 0; cj < 2; cj++) {
        group(cj == 0 ? ve : vo, lo[cj][0], hi[cj][0], by[cj][0]);
        group((cj == 0 ? ve : vo) + 16, lo[cj][1], hi[cj][1], by[cj][1]);
    }

    // results into LDS, then out column-wise: each column's 64 code bytes and
    // 8 scale bytes, at pitches of 72 and 12 bytes -- at 64 and 8, the lanes'
    // writes (two columns apart) all fell on the same LDS banks
    uint8_t* ocodes = obuf;
    uint8_t* oscales = obuf + kTC * kCodePitch;
#pragma unroll
    for (int cj = 0; cj < 2; cj++) {
        const int lc = 2 * lane + cj;
#pragma unroll
        for (int ri = 0; ri < 2; ri++)
            *reinterpret_cast<uint2*>(ocodes + lc * kCodePitch + (2 * wave + ri) * 8) =
                make_uint2(lo[cj][ri], hi[cj][ri]);
        *reinterpret_cast<uint16_t*>(oscales + lc * kScalePitch + 2 * wave) =
            (uint16_t)(by[cj][0] | (by[cj][1] << 8));
    }
    __syncthreads();
    const int64_t rgs = rows / 16, rgt = rt * kTRG;  // row-groups in all, first of the tile
    if (wide_out) {
        // whole tiles down every column and 16-byte aligned codes, 8-byte
        // aligned scales: each column's 64 code bytes and 8 scale bytes are
        // aligned too
#pragma unroll
        for (int k = 0; k < kTC * 4 / kThreads; k++) {
            const int i = k * kThreads + tid;
            const int lc = i / 4, part = i % 4;
            const int64_t c = c0 + lc;
            if (c < cols) {
                const uint2 a = *reinterpret_cast<const uint2*>(ocodes + lc * kCodePitch + part * 16);
                const uint2 b = *reinterpret_cast<const uint2*>(ocodes + lc * kCodePitch + part * 16 + 8);
                *reinterpret_cast<uint4*>(codes + c * (rows / 2) + rgt * 8 + part * 16) =
                    make_uint4(a.x, a.y, b.x, b.y);
            }
        }
        if (tid < kTC && c0 + tid < cols) {
            const uint32_t* sp = reinterpret_cast<const uint32_t*>(oscales + tid * kScalePitch);
            *reinterpret_cast<uint2*>(scales + (c0 + tid) * rgs + rgt) = make_uint2(sp[0], sp[1]);
        }
        return;
    }
    // codes: 8-byte pieces, 8 per column; scales: single bytes, 8 per column
#pragma unroll
    for (int k = 0; k < kTC * kTRG / kThreads; k++) {
        const int i = k * kThreads + tid;
        const int lc = i / kTRG, part = i % kTRG;
        const int64_t c = c0 + lc, rg = rgt + part;
        if (c < cols && rg < rgs) {
            *reinterpret_cast<uint2*>(codes + c * (rows / 2) + rg * 8) =
                *reinterpret_cast<const uint2*>(ocodes + lc * kCodePitch + part * 8);
            scales[c * rgs + rg] = oscales[lc * kScalePitch + part];
        }
    }
}

template <bool kBf16, int kMode>
hipError_t launch_t(const void* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* codes,
                    uint8_t* scales, int32_t scale_exp, hipStream_t stream) {
    const float pe = pow2f(scale_exp), pn = pow2f(-scale_exp);
    const int elem = kBf16 ? 2 : 4;
    // the tiled kernel: 16-byte aligned rows, row strides below 16 MB (its
    // interior tiles address with 32-bit offsets)
    if ((uintptr_t)x % 16 == 0 && (ld_x * elem) % 16 == 0 && ld_x * elem < (1 << 24)) {
        const int64_t col_tiles = (cols + kTC - 1) / kTC, row_tiles = (rows + kTR - 1) / kTR;
        if (col_tiles * row_tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
        const int wide_out =
            rows % kTR == 0 && (uintptr_t)codes % 16 == 0 && (uintptr_t)scales % 8 == 0;
        hipLaunchKernelGGL((quantize_t_tile_kernel<kBf16, kMode>),
                           dim3((unsigned)(col_tiles * row_tiles)), dim3(kThreads), 0, stream, x,
                           rows, cols, ld_x, codes, scales, pe, pn, col_tiles, wide_out);
        return hipGetLastError();
    }
    const int64_t col_blocks = (cols + kThreads - 1) / kThreads;
    const int64_t chunks = (rows / 16 + kTChunk - 1) / kTChunk;
    if (col_blocks * chunks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL((quantize_t_kernel<kBf16, kMode>), dim3((unsigned)(col_blocks * chunks)),
                       dim3(kThreads), 0, stream, x, rows, cols, ld_x, codes, scales, pe, pn,
                       col_blocks);
    return hipGetLastError();
}

template <bool kRotate>
hipError_t dispatch_quantize(const void* x, int bf16, int64_t rows, int64_t cols, int64_t ld_x,
                             uint8_t* codes, uint8_t* scales, int32_t scale_exp, int mode,
                             uint32_t sign_mask, hipStream_t stream) {
#define IF4_Q(B, M) \
    launch<B, M, kRotate>(x, rows, cols, ld_x, codes, scales, scale_exp, sign_mask, stream)
    if (bf16) {
        if (mode == 1) return IF4_Q(true, 1);
        if (mode == 2) return IF4_Q(true, 2);
        return IF4_Q(true, 0);
    }
    if (mode == 1) return IF4_Q(false, 1);
    if (mode == 2) return IF4_Q(false, 2);
    return IF4_Q(false, 0);
#undef IF4_Q
}

}  // namespace

hipError_t launch_quantize(const void* x, int bf16, int64_t rows, int64_t cols, int64_t ld_x,
                           uint8_t* codes, uint8_t* scales, int32_t scale_exp, int mode,
                           hipStream_t stream) {
    return dispatch_quantize<false>(x, bf16, rows, cols, ld_x, codes, scales, scale_exp, mode, 0u,
                                    stream);
}

hipError_t launch_quantize_rht(const void* x, int bf16, int64_t rows, int64_t cols, int64_t ld_x,
                               uint32_t sign_mask, uint8_t* codes, uint8_t* scales,
                               int32_t scale_exp, int mode, hipStream_t stream) {
    return dispatch_quantize<true>(x, bf16, rows, cols, ld_x, codes, scales, scale_exp, mode,
                                   sign_mask, stream);
}

hipError_t launch_quantize_t(const void* x, int bf16, int64_t rows, int64_t cols, int64_t ld_x,
                             uint8_t* codes, uint8_t* scales, int32_t scale_exp, int mode,
                             hipStream_t stream) {
    if (bf16) {
        if (mode == 1) return launch_t<true, 1>(x, rows, cols, ld_x, codes, scales, scale_exp, stream);
        if (mode == 2) return launch_t<true, 2>(x, rows, cols, ld_x, codes, scales, scale_exp, stream);
        return launch_t<true, 0>(x, rows, cols, ld_x, codes, scales, scale_exp, stream);
    }
    if (mode == 1) return launch_t<false, 1>(x, rows, cols, ld_x, codes, scales, scale_exp, stream);
    if (mode == 2) return launch_t<false, 2>(x, rows, cols, ld_x, codes, scales, scale_exp, stream);
    return launch_t<false, 0>(x, rows, cols, ld_x, codes, scales, scale_exp, stream);
}

}  // namespace if4
