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
// contiguous.  The kernel is a grid-stride loop over groups.
//
// Every rounding decision is taken exactly, for any fp32 input: each code
// is the count of grid midpoints the value passes, compared against exactly
// representable thresholds (s * midpoint for FP4; 7|x| - 3s(2k+1) by fma for
// INT4), with ties resolved to the even code by using >= or > per midpoint.
#include <hip/hip_runtime.h>
#include <stdint.h>

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

template <bool kBf16, int kMode>
__global__ void __launch_bounds__(kThreads)
quantize_kernel(const void* __restrict__ x, int64_t rows, int64_t gpr, int64_t ld_x,
                uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float p_exp,
                float p_negexp) {
    const int64_t ngroups = rows * gpr;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < ngroups; g += stride) {
        const int64_t r = g / gpr;
        const int64_t cg = g - r * gpr;
        float v[16];
        load_group<kBf16>(x, r * ld_x + cg * 16, v);

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
        uint32_t lo = 0, hi = 0, byte = 0;
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
        *reinterpret_cast<uint2*>(codes + g * 8) = make_uint2(lo, hi);
        scales[g] = (uint8_t)byte;
    }
}

template <bool kBf16, int kMode>
hipError_t launch(const void* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* codes,
                  uint8_t* scales, int32_t scale_exp, hipStream_t stream) {
    const int64_t gpr = cols / 16;
    const int64_t ngroups = rows * gpr;
    int64_t blocks = (ngroups + kThreads - 1) / kThreads;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL((quantize_kernel<kBf16, kMode>), dim3((unsigned)blocks), dim3(kThreads), 0,
                       stream, x, rows, gpr, ld_x, codes, scales, pow2f(scale_exp),
                       pow2f(-scale_exp));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const void* x, int bf16, int64_t rows, int64_t cols, int64_t ld_x,
                           uint8_t* codes, uint8_t* scales, int32_t scale_exp, int mode,
                           hipStream_t stream) {
    if (bf16) {
        if (mode == 1) return launch<true, 1>(x, rows, cols, ld_x, codes, scales, scale_exp, stream);
        if (mode == 2) return launch<true, 2>(x, rows, cols, ld_x, codes, scales, scale_exp, stream);
        return launch<true, 0>(x, rows, cols, ld_x, codes, scales, scale_exp, stream);
    }
    if (mode == 1) return launch<false, 1>(x, rows, cols, ld_x, codes, scales, scale_exp, stream);
    if (mode == 2) return launch<false, 2>(x, rows, cols, ld_x, codes, scales, scale_exp, stream);
    return launch<false, 0>(x, rows, cols, ld_x, codes, scales, scale_exp, stream);
}

}  // namespace if4
