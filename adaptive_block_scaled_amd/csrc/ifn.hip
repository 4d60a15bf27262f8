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
// issued first.  Every rounding is decided by exact comparisons against
// thresholds that are exact in fp32 (the grids' midpoints times the scale),
// in binary searches with ties to the even index -- valid for any fp32 input.
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
    static constexpr int kFpLog2 = 5;      // 32 float magnitudes
    static constexpr int kQLog2 = 5;       // INT magnitudes 0..31
    static constexpr float kTop = 7.5f;
    static constexpr float kDn = 15.0f, kDd = 62.0f;  // top / qmax = dn / dd
    // E2M3 magnitude of index i: 2 exponent bits (bias 1), 3 mantissa bits
    __device__ static float fp(int i) {
        const int e = i >> 3, m = i & 7;
        return e == 0 ? (float)m * 0.125f : (float)(8 + m) * __builtin_ldexpf(1.0f, e - 4);
    }
};

template <>
struct Fmt<3> {
    static constexpr int kFpLog2 = 2;      // E2M0: 0, 1, 2, 4
    static constexpr int kQLog2 = 2;       // INT magnitudes 0..3
    static constexpr float kTop = 4.0f;
    static constexpr float kDn = 4.0f, kDd = 3.0f;
    __device__ static float fp(int i) { return i == 0 ? 0.0f : __builtin_ldexpf(1.0f, i - 1); }
};

__device__ __forceinline__ float e4m3_value(uint32_t code) {
    return code >= 8u ? __uint_as_float((code + 960u) << 20) : (float)code * 0.001953125f;
}

// index of RNE(v / unit) on an ascending grid of 2^kLog2 values with
// midpoints mid(k) (exact products unit * mid(k)); ties -> even index;
// values past the last midpoint saturate
template <int kLog2, typename Mid>
__device__ __forceinline__ uint32_t rne_search(float v, Mid mid) {
    uint32_t lo = 0;
#pragma unroll
    for (int step = 1 << (kLog2 - 1); step >= 1; step >>= 1) {
        const uint32_t k = lo + step - 1;  // boundary between k and k + 1
        const float t = mid(k);
        const bool up = v > t || (v == t && (k & 1u));
        lo = up ? k + 1 : lo;
    }
    return lo;
}

template <int kBits, int kMode>
__device__ __forceinline__ void quantize_group(const float (&v)[16], float p_exp, float p_negexp,
                                               uint32_t (&out)[3], uint32_t& byte) {
    using F = Fmt<kBits>;
    float a = 0.0f;
    bool finite = true;
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const float ax = __builtin_fabsf(v[i]);
        finite &= ax <= 3.40282347e38f;
        a = __builtin_fmaxf(a, ax);
    }
    out[0] = out[1] = out[2] = 0;
    if (!finite) {
        byte = 0x7Fu;
        return;
    }
    // scale code: RNE_E4M3(a 2^-E / top) over the 127 finite codes: a' vs
    // top * (v_k + v_{k+1}) / 2, exact (4 + 5 bits); 7 binary-search steps
    // over the 126 midpoints (the 128th boundary is never reached)
    const float ap = a * p_negexp;
    uint32_t sc = 0;
#pragma unroll
    for (int step = 64; step >= 1; step >>= 1) {
        const uint32_t k = sc + step - 1;
        if (k < 126u) {
            const float t = F::kTop * (0.5f * (e4m3_value(k) + e4m3_value(k + 1)));
            const bool up = ap > t || (ap == t && (k & 1u));
            sc = up ? k + 1 : sc;
        }
    }
    if (sc == 0) {
        byte = 0;
        return;
    }
    const float s = e4m3_value(sc) * p_exp;
    const float sdd = F::kDd * s, sdn = F::kDn * s;
    float ef = 0.0f, ei = 0.0f;
    uint32_t cf[16], ci[16];
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const float ax = __builtin_fabsf(v[i]);
        const uint32_t fi = rne_search<F::kFpLog2>(
            ax, [&](uint32_t k) { return s * (0.5f * (F::fp(k) + F::fp(k + 1))); });
        // INT: |q| > k  <=>  dd |x| > dn s (k + 1/2); the sign of the fma is exact
        uint32_t q = 0;
#pragma unroll
        for (int step = 1 << (F::kQLog2 - 1); step >= 1; step >>= 1) {
            const uint32_t k = q + step - 1;
            const float d = __builtin_fmaf(ax, F::kDd, -sdn * ((float)k + 0.5f));
            const bool up = d > 0.0f || (d == 0.0f && (k & 1u));
            q = up ? k + 1 : q;
        }
        const float df = __builtin_fmaf(ax, F::kDd, -(F::fp(fi) * sdd));
        const float di = __builtin_fmaf(ax, F::kDd, -((float)q * sdn));
        ef = __builtin_fmaf(df, df, ef);
        ei = __builtin_fmaf(di, di, ei);
        const uint32_t sg = (__float_as_uint(v[i]) >> 31) << (kBits - 1);
        cf[i] = sg | fi;
        ci[i] = sg | q;
    }
    const bool use_int = kMode == 2 ? true : (kMode == 1 ? false : (ei < ef));
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const uint32_t c = use_int ? ci[i] : cf[i];
        const int bit = kBits * i;
        out[bit >> 5] |= c << (bit & 31);
        if ((bit & 31) + kBits > 32) out[(bit >> 5) + 1] |= c >> (32 - (bit & 31));
    }
    byte = sc | (use_int ? 0x80u : 0u);
}

template <int kBits, int kMode, bool kBf16>
__global__ void __launch_bounds__(kThreads)
quantize_ifn_kernel(const void* __restrict__ x, int64_t rows, int64_t gpr, int64_t ld_x,
                    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float p_exp,
                    float p_negexp) {
    const int64_t ngroups = rows * gpr;
    const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t g = gid < ngroups - 1 ? gid : ngroups - 1;
    const int64_t r = g / gpr;
    const int64_t off = r * ld_x + (g - r * gpr) * 16;
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
template <int kBits, bool kBf16>
__global__ void __launch_bounds__(kThreads)
dequantize_ifn_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                      int64_t rows, int64_t gpr, void* __restrict__ y, int64_t ld_y, float p_exp) {
    using F = Fmt<kBits>;
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
    const float sp = (b & 0x7Fu) == 0x7Fu ? __uint_as_float(0x7FC00000u) : e4m3_value(b & 0x7Fu);
    const bool is_int = (b & 0x80u) != 0;
    float h, l;
    {
        const float num = F::kDn * sp;  // exact
        h = num / F::kDd;
        if (__builtin_fmaf(-h, F::kDd, num) < 0.0f) h = __uint_as_float(__float_as_uint(h) - 1u);
        l = __builtin_fmaf(-h, F::kDd, num) * (1.0f / F::kDd);
    }
    const float he = h * p_exp, le = l * p_exp, se = sp * p_exp;
    float out[16];
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const int bit = kBits * i;
        uint32_t c = w[bit >> 5] >> (bit & 31);
        if ((bit & 31) + kBits > 32) c |= w[(bit >> 5) + 1] << (32 - (bit & 31));
        c &= (1u << kBits) - 1u;
        const uint32_t mag = c & ((1u << (kBits - 1)) - 1u);
        const float m = (float)mag;
        const float val = is_int ? __builtin_fmaf(m, he, m * le) : F::fp((int)mag) * se;
        out[i] = (c >> (kBits - 1)) ? -val : val;
    }
    if (gid >= ngroups) return;
    const int64_t r = gid / gpr;
    const int64_t off = r * ld_y + (gid - r * gpr) * 16;
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
    hipLaunchKernelGGL((quantize_ifn_kernel<kBits, kMode, kBf16>), dim3((unsigned)blocks),
                       dim3(kThreads), 0, stream, x, rows, gpr, ld_x, codes, scales,
                       pow2f(scale_exp), pow2f(-scale_exp));
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
    if (bf16)
        hipLaunchKernelGGL((dequantize_ifn_kernel<kBits, true>), dim3((unsigned)blocks),
                           dim3(kThreads), 0, stream, codes, scales, rows, gpr, y, ld_y,
                           pow2f(scale_exp));
    else
        hipLaunchKernelGGL((dequantize_ifn_kernel<kBits, false>), dim3((unsigned)blocks),
                           dim3(kThreads), 0, stream, codes, scales, rows, gpr, y, ld_y,
                           pow2f(scale_exp));
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
