// IF3 and IF6 quantize / dequantize for gfx950.
//
// The pages extend the adaptive per-group choice to 3 and 6 bits per value
// ("Adaptive Block-Scaled Data Types for FP4 Training", podcast companion,
// "It Generalizes: IF3 and IF6"; gist.science summary, section 2,
// "Extensoes") without defining the formats.  The formats here keep IF4's
// construction (include/if4.h states them in full): sign-magnitude codes,
// one E4M3 scale per 16 values with the choice in its sign bit, the INT range
// pre-scaled so that its top value lands on the float grid's top value,
// scale = RNE_E4M3(amax / top), fp32 squared errors in a domain where the INT
// descale is exact.
//   IF6: FP6 E2M3 (top 7.5) or INT6 |q| <= 31 decoding to q * 15/62 * s;
//        errors x62.
//   IF3: FP3 E2M0 {0, 1, 2, 4} or INT3 |q| <= 3 decoding to q * 4/3 * s;
//        errors x3.
// Element i of a group occupies bits [bits*i, bits*(i+1)) of the group's
// little-endian 2*bits-byte code field.
//
// One group per thread, one workgroup per 256 groups, the thread's loads
// issued first.  Every rounding is decided exactly (exact comparisons, or the
// exact sign of one fma), ties to the even index -- valid for any fp32 input
// -- in branch-free code.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "if4_internal.h"

namespace if4 {
namespace {

constexpr int kThreads = 256;

template <int kBits>
struct Fmt;

template <>
struct Fmt<6> {
    static constexpr float kTop = 7.5f;     // 32 float magnitudes, INT 0..31
    static constexpr float kDn = 15.0f, kDd = 62.0f;  // top / qmax = dn / dd
    // E2M3 magnitude of index i: 2 exponent bits (bias 1), 3 mantissa bits
    __device__ static float fp(int i) {
        const int e = i >> 3, m = i & 7;
        return e == 0 ? (float)m * 0.125f : (float)(8 + m) * __builtin_ldexpf(1.0f, e - 4);
    }
};

template <>
struct Fmt<3> {
    static constexpr float kTop = 4.0f;     // E2M0: 0, 1, 2, 4; INT 0..3
    static constexpr float kDn = 4.0f, kDd = 3.0f;
    __device__ static float fp(int i) { return i == 0 ? 0.0f : __builtin_ldexpf(1.0f, i - 1); }
};

__device__ __forceinline__ float e4m3_value(uint32_t code) {
    return code >= 8u ? __uint_as_float((code + 960u) << 20) : (float)code * 0.001953125f;
}

// 1 if a magnitude ax (>= 0) rounds above the boundary t of index k (the
// midpoint between grid values k and k + 1): ax > t, or ax == t for odd k,
// so that ties go to the even index.  Non-negative floats order as their bit
// patterns; a negative t is always passed and t = +inf never.
__device__ __forceinline__ int passes(float ax, float t, int k) {
    return (int)__float_as_uint(ax) + (k & 1) > (int)__float_as_uint(t) ? 1 : 0;
}
// the same given the difference d = ax - t from one fma (its sign is exact and
// an exact zero is +0): d > 0, or d == +0 for odd k -- the low bit or'ed into
// d's bit pattern leaves a negative d negative
__device__ __forceinline__ int passes_d(float d, int k) {
    return ((int)__float_as_uint(d) | (k & 1)) > 0 ? 1 : 0;
}

// E2M3 on fp32 bits: the index k = 8e + m (2 exponent bits with bias 1, 3
// mantissa bits) placed at bit 20, k << 20, is the fp32 pattern with exponent
// field e and mantissa m / 8 -- read as a float it equals the E2M3 magnitude
// of k times 2^-126 for all 32 indices, E2M3's subnormals (e = 0) landing on
// fp32's.  Setting bit 19 as well gives the midpoint between k and k + 1.
// Multiplying by 2^126 makes either an exact normal float.
__device__ __forceinline__ float e2m3_value(int k) {
    return __uint_as_float((uint32_t)k << 20) * 0x1p126f;
}
__device__ __forceinline__ float e2m3_mid(int k) {
    return __uint_as_float(((uint32_t)k << 20) | (1u << 19)) * 0x1p126f;
}

// The scale code and IF6's indices are "guess, then one exact check".  A
// guess truncates an approximate quotient (at most a part in 2^21 off) to the
// grid below it, which gives the correctly rounded index or the one below
// (the grids are at least 2^-4 apart, relative); comparing with the exact
// boundary above the guess decides between them -- directly for the scale
// (an fp32 product of at most 9 significant bits), by the sign of one fma
// for the elements.  IF3 compares every element with its six boundaries.
template <int kBits, int kMode>
__device__ __forceinline__ void quantize_group(const float (&v)[16], float p_exp, float p_negexp,
                                               uint32_t (&out)[3], uint32_t& byte) {
    using F = Fmt<kBits>;
    constexpr float kInf = __builtin_inff();
    // amax on the magnitudes' bit patterns, which order as the values do and
    // put inf and NaN above every finite value
    uint32_t abits = 0;
#pragma unroll
    for (int i = 0; i < 16; i++) abits = max(abits, __float_as_uint(v[i]) & 0x7FFFFFFFu);
    out[0] = out[1] = out[2] = 0;
    if (abits >= 0x7F800000u) {
        byte = 0x7Fu;
        return;
    }
    const float a = __uint_as_float(abits);
    // scale code RNE_E4M3(a 2^-E / top) over the 127 finite codes; the
    // boundary above code k is top (v_k + v_{k+1}) / 2 (4 + 5 bits, exact)
    const float ap = a * p_negexp;
    const float qg = ap * (1.0f / F::kTop);
    int sc = qg < 0.015625f ? (int)(qg * 512.0f) : (int)(__float_as_uint(qg) >> 20) - 960;
    sc = sc < 126 ? sc : 126;
    sc += passes(ap, sc < 126 ? F::kTop * (0.5f * (e4m3_value(sc) + e4m3_value(sc + 1))) : kInf,
                 sc);
    if (sc == 0) {
        byte = 0;
        return;
    }
    const float s = e4m3_value((uint32_t)sc) * p_exp;
    const float sdd = F::kDd * s, sdn = F::kDn * s;
    constexpr int kFMax = (1 << (kBits - 1)) - 1, kQMax = kFMax;
    // IF6: reciprocals for the guesses.  IF3: its three boundaries of each
    // kind as fp32 values that ax is compared with directly.  The FP ones,
    // s (fp(k) + fp(k + 1)) / 2, are exact; the INT ones, dn s (k + 1/2) / dd,
    // are taken rounded down (exact when representable, as 2s is for k = 1):
    // a float passes the rounded-down value exactly when it passes the true
    // one, so "ax > t" decides an even k (ties stay down) and "ax >= t" the
    // odd k = 1, whose boundaries are exact.
    const float r = __builtin_amdgcn_rcpf(s);
    const float rq = r * (F::kDd / F::kDn);
    const float sdn_half = 0.5f * sdn;
    float tf[3], tq[3];
    if constexpr (kBits == 3) {
#pragma unroll
        for (int k = 0; k < 3; k++) {
            tf[k] = s * (0.5f * (F::fp(k) + F::fp(k + 1)));
            // within an ulp of sdn (k + 1/2) / dd; one step down if above it
            const float num = sdn * ((float)k + 0.5f);
            const float w = num * (1.0f / F::kDd);
            tq[k] = __builtin_fmaf(w, F::kDd, -num) > 0.0f ? __uint_as_float(__float_as_uint(w) - 1u) : w;
        }
    }
    float ef = 0.0f, ei = 0.0f;
    // magnitude fields of both candidates and the sign field, kBits per element
    uint32_t mf[3] = {0, 0, 0}, mq[3] = {0, 0, 0}, sg[3] = {0, 0, 0};
    auto put = [](uint32_t(&f)[3], uint32_t c, int bit) {
        f[bit >> 5] |= c << (bit & 31);
        if ((bit & 31) + kBits > 32) f[(bit >> 5) + 1] |= c >> (32 - (bit & 31));
    };
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const float ax = __builtin_fabsf(v[i]);
        int fi, q;
        // the candidates' values times dd s and dd s dn / dd = dn s, exact
        // (at most 14 significant bits)
        float fvs, qsdn;
        if constexpr (kBits == 6) {
            // guess: the approximate quotient u = ax / s times 2^-126 (an
            // fp32 subnormal below 1) truncated to the E2M3 bits above bit
            // 20, clamped to 30 so that the boundary above it exists; a
            // guess is never above the correctly rounded index.  The check
            // takes the sign of ax - mid s from one fma.
            const float u = ax * r;
            const int g = min((int)(__float_as_uint(__builtin_ldexpf(u, -126)) >> 20), kFMax - 1);
            fi = g + passes_d(__builtin_fmaf(e2m3_mid(g), -s, ax), g);
            fvs = e2m3_value(fi) * sdd;
            // INT: |q| > k  <=>  dd |x| > dn s (k + 1/2), the threshold
            // dn s k + dn s / 2 exact in one fma
            const int h = (int)__builtin_fminf(ax * rq, (float)(kQMax - 1));
            q = h + passes_d(__builtin_fmaf(ax, F::kDd, -__builtin_fmaf((float)h, sdn, sdn_half)), h);
            qsdn = (float)q * sdn;
        } else {
            const bool f0 = ax > tf[0], f1 = ax >= tf[1], f2 = ax > tf[2];
            const bool q0 = ax > tq[0], q1 = ax >= tq[1], q2 = ax > tq[2];
            fi = (int)f0 + (int)f1 + (int)f2;
            q = (int)q0 + (int)q1 + (int)q2;
            // E2M0 on fp32 bits: index k << 23 read as a float is 0, 1, 2, 4
            // times 2^-126 (exponent field k, k = 0 the zero)
            fvs = (__uint_as_float((uint32_t)fi << 23) * 0x1p126f) * sdd;
            qsdn = (float)q * sdn;
        }
        const float df = __builtin_fmaf(ax, F::kDd, -fvs);
        const float di = __builtin_fmaf(ax, F::kDd, -qsdn);
        ef = __builtin_fmaf(df, df, ef);
        ei = __builtin_fmaf(di, di, ei);
        put(mf, (uint32_t)fi, kBits * i);
        put(mq, (uint32_t)q, kBits * i);
        put(sg, (__float_as_uint(v[i]) >> 31) << (kBits - 1), kBits * i);
    }
    const bool use_int = kMode == 2 ? true : (kMode == 1 ? false : (ei < ef));
#pragma unroll
    for (int w = 0; w < 3; w++) out[w] = (use_int ? mq[w] : mf[w]) | sg[w];
    byte = (uint32_t)sc | (use_int ? 0x80u : 0u);
}

// kContig: rows back to back (ld = cols), so a group's offset is 16 g with
// no division by the groups per row
template <int kBits, int kMode, bool kBf16, bool kContig>
__global__ void __launch_bounds__(kThreads)
quantize_ifn_kernel(const void* __restrict__ x, int64_t rows, int64_t gpr, int64_t ld_x,
                    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float p_exp,
                    float p_negexp) {
    const int64_t ngroups = rows * gpr;
    const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t g = gid < ngroups - 1 ? gid : ngroups - 1;
    int64_t off;
    if constexpr (kContig) {
        off = g * 16;
    } else {
        const int64_t r = g / gpr;
        off = r * ld_x + (g - r * gpr) * 16;
    }
    float v[16];
    if constexpr (kBf16) {
        const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + off);
        const uint4 a = p[0], b = p[1];
        const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; i++) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    } else {
        const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + off);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const float4 t = p[i];
            v[4 * i] = t.x;
            v[4 * i + 1] = t.y;
            v[4 * i + 2] = t.z;
            v[4 * i + 3] = t.w;
        }
    }
    uint32_t out[3], byte;
    quantize_group<kBits, kMode>(v, p_exp, p_negexp, out, byte);
    if (gid >= ngroups) return;
    if constexpr (kBits == 6) {
        uint32_t* c = reinterpret_cast<uint32_t*>(codes + gid * 12);
        c[0] = out[0];
        c[1] = out[1];
        c[2] = out[2];
    } else {
        uint16_t* c = reinterpret_cast<uint16_t*>(codes + gid * 6);
        c[0] = (uint16_t)out[0];
        c[1] = (uint16_t)(out[0] >> 16);
        c[2] = (uint16_t)out[1];
    }
    scales[gid] = (uint8_t)byte;
}

// Dequantize: FP codes decode to fp(idx) * s' * 2^E (exact); INT codes to
// the fp32 nearest |q| dn s' / dd (times 2^E), as fma(q, h, q * l) with h =
// dn s'/dd rounded toward zero and l = fl32((dn s' - dd h) * fl32(1/dd)) --
// correctly rounded for every E4M3 s' and |q| (checked exhaustively in exact
// arithmetic), with l >= 0 so that a zero magnitude keeps its sign.
//
// Both forms are one fma: every element is fma(A, HE, A * LE) with A the
// code's signed integer on its grid and (HE, LE) a per-scale-byte pair --
// INT: A = +-|q|, (HE, LE) = (h, l) 2^E; FP: A = +-fp(idx) * kFpDen (an
// integer), (HE, LE) = (s' 2^E / kFpDen, 0), whose product is exact.  Each
// workgroup tabulates A for the 2 x 2^bits (flag, code) pairs and (HE, LE)
// for the 256 scale bytes in LDS while its loads are in flight, so an element
// costs one LDS read, a multiply and an fma.  (A NaN scale byte gives NaN.)
template <int kBits>
struct Fp {
    static constexpr float kDen = kBits == 6 ? 8.0f : 1.0f;  // fp(idx) * kDen is an integer
};

template <int kBits, bool kBf16, bool kContig>
__global__ void __launch_bounds__(kThreads)
dequantize_ifn_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                      int64_t rows, int64_t gpr, void* __restrict__ y, int64_t ld_y, float p_exp) {
    using F = Fmt<kBits>;
    constexpr int kCodes = 1 << kBits;
    __shared__ float2 stab[256];
    __shared__ float ctab[2 * kCodes];
    const int64_t ngroups = rows * gpr;
    const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t g = gid < ngroups - 1 ? gid : ngroups - 1;
    uint32_t w[3];
    if constexpr (kBits == 6) {
        const uint32_t* c = reinterpret_cast<const uint32_t*>(codes + g * 12);
        w[0] = c[0];
        w[1] = c[1];
        w[2] = c[2];
    } else {
        const uint16_t* c = reinterpret_cast<const uint16_t*>(codes + g * 6);
        w[0] = (uint32_t)c[0] | ((uint32_t)c[1] << 16);
        w[1] = c[2];
        w[2] = 0;
    }
    const uint32_t b = scales[g];

    // the tables, while the loads are in flight
    {
        const uint32_t t = threadIdx.x;  // scale byte t
        const float sp =
            (t & 0x7Fu) == 0x7Fu ? __uint_as_float(0x7FC00000u) : e4m3_value(t & 0x7Fu);
        float2 e;
        if (t & 0x80u) {
            const float num = F::kDn * sp;  // exact
            float h = num / F::kDd;
            if (__builtin_fmaf(-h, F::kDd, num) < 0.0f) h = __uint_as_float(__float_as_uint(h) - 1u);
            const float l = __builtin_fmaf(-h, F::kDd, num) * (1.0f / F::kDd);
            e = make_float2(h * p_exp, l * p_exp);
        } else {
            e = make_float2(sp * p_exp * (1.0f / Fp<kBits>::kDen), 0.0f);
        }
        stab[t] = e;
        if (t < 2u * kCodes) {  // (flag, code) -> signed integer grid value
            const uint32_t c = t & (kCodes - 1u), mag = c & (kCodes / 2 - 1u);
            const float a = (t >= (uint32_t)kCodes) ? (float)mag : F::fp((int)mag) * Fp<kBits>::kDen;
            ctab[t] = (c >> (kBits - 1)) ? -a : a;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");

    const float2 e = stab[b];
    const uint32_t fbase = (b >> 7) << kBits;  // INT codes in the table's upper half
    float out[16];
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const int bit = kBits * i;
        uint32_t c = w[bit >> 5] >> (bit & 31);
        if ((bit & 31) + kBits > 32) c |= w[(bit >> 5) + 1] << (32 - (bit & 31));
        c &= (1u << kBits) - 1u;
        const float a = ctab[fbase + c];
        out[i] = __builtin_fmaf(a, e.x, a * e.y);
    }
    if (gid >= ngroups) return;
    int64_t off;
    if constexpr (kContig) {
        off = gid * 16;
    } else {
        const int64_t r = gid / gpr;
        off = r * ld_y + (gid - r * gpr) * 16;
    }
    if constexpr (kBf16) {
        uint32_t o[8];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
            bf16x2 t;
            t[0] = (__bf16)out[2 * i];
            t[1] = (__bf16)out[2 * i + 1];
            o[i] = __builtin_bit_cast(uint32_t, t);
        }
        uint4* p = reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(y) + off);
        p[0] = make_uint4(o[0], o[1], o[2], o[3]);
        p[1] = make_uint4(o[4], o[5], o[6], o[7]);
    } else {
        float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + off);
#pragma unroll
        for (int i = 0; i < 4; i++)
            p[i] = make_float4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
    }
}

template <int kBits, int kMode, bool kBf16>
hipError_t launch_q(const void* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* codes,
                    uint8_t* scales, int32_t scale_exp, hipStream_t stream) {
    const int64_t gpr = cols / 16;
    const int64_t blocks = (rows * gpr + kThreads - 1) / kThreads;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (ld_x == cols)
        hipLaunchKernelGGL((quantize_ifn_kernel<kBits, kMode, kBf16, true>), dim3((unsigned)blocks),
                           dim3(kThreads), 0, stream, x, rows, gpr, ld_x, codes, scales,
                           pow2f(scale_exp), pow2f(-scale_exp));
    else
        hipLaunchKernelGGL((quantize_ifn_kernel<kBits, kMode, kBf16, false>),
                           dim3((unsigned)blocks), dim3(kThreads), 0, stream, x, rows, gpr, ld_x,
                           codes, scales, pow2f(scale_exp), pow2f(-scale_exp));
    return hipGetLastError();
}

template <int kBits>
hipError_t dispatch_q(const void* x, int bf16, int64_t rows, int64_t cols, int64_t ld_x,
                      uint8_t* codes, uint8_t* scales, int32_t scale_exp, int mode,
                      hipStream_t stream) {
#define IF4_QN(M, B) launch_q<kBits, M, B>(x, rows, cols, ld_x, codes, scales, scale_exp, stream)
    if (bf16) {
        if (mode == 1) return IF4_QN(1, true);
        if (mode == 2) return IF4_QN(2, true);
        return IF4_QN(0, true);
    }
    if (mode == 1) return IF4_QN(1, false);
    if (mode == 2) return IF4_QN(2, false);
    return IF4_QN(0, false);
#undef IF4_QN
}

template <int kBits>
hipError_t dispatch_dq(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                       int32_t scale_exp, void* y, int bf16, int64_t ld_y, hipStream_t stream) {
    const int64_t gpr = cols / 16;
    const int64_t blocks = (rows * gpr + kThreads - 1) / kThreads;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
#define IF4_DQN(B, C)                                                                  \
    hipLaunchKernelGGL((dequantize_ifn_kernel<kBits, B, C>), dim3((unsigned)blocks),            \
                       dim3(kThreads), 0, stream, codes, scales, rows, gpr, y, ld_y,            \
                       pow2f(scale_exp))
    const bool contig = ld_y == cols;
    if (bf16) {
        if (contig) IF4_DQN(true, true);
        else IF4_DQN(true, false);
    } else {
        if (contig) IF4_DQN(false, true);
        else IF4_DQN(false, false);
    }
#undef IF4_DQN
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_ifn(int bits, const void* x, int bf16, int64_t rows, int64_t cols,
                               int64_t ld_x, uint8_t* codes, uint8_t* scales, int32_t scale_exp,
                               int mode, hipStream_t stream) {
    if (bits == 6)
        return dispatch_q<6>(x, bf16, rows, cols, ld_x, codes, scales, scale_exp, mode, stream);
    return dispatch_q<3>(x, bf16, rows, cols, ld_x, codes, scales, scale_exp, mode, stream);
}

hipError_t launch_dequantize_ifn(int bits, const uint8_t* codes, const uint8_t* scales,
                                 int64_t rows, int64_t cols, int32_t scale_exp, void* y, int bf16,
                                 int64_t ld_y, hipStream_t stream) {
    if (bits == 6)
        return dispatch_dq<6>(codes, scales, rows, cols, scale_exp, y, bf16, ld_y, stream);
    return dispatch_dq<3>(codes, scales, rows, cols, scale_exp, y, bf16, ld_y, stream);
}

}  // namespace if4
