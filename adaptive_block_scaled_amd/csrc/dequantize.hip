// IF4 dequantize for gfx950.
//
// Each group's scale byte selects the decode: FP4 nibbles decode to
// (+-) E2M1 * s', INT4 nibbles to (+-) |q| * s' descaled by 6/7
// ("Adaptive Block-Scaled Data Types", gist.science summary, section 2,
// "Metodo 6/7"), then times 2^E.  One lane per group (8 code bytes + 1 scale
// byte in, 16 values out), grid-stride loop; output stores are 16-byte
// vectors, contiguous across the wave.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "if4_internal.h"

namespace if4 {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float e4m3_value_or_nan(uint32_t code7) {
    if (code7 == 0x7Fu) return __uint_as_float(0x7FC00000u);
    return code7 >= 8u ? __uint_as_float((code7 + 960u) << 20) : (float)code7 * 0.001953125f;
}

__device__ __forceinline__ float e2m1_value(uint32_t idx) {
    float m = (idx & 1u) ? 1.5f : 1.0f;
    uint32_t e = idx >> 1;
    return e == 0 ? (idx ? 0.5f : 0.0f) : m * (float)(1u << (e - 1));
}

// RNE fp32 -> bf16 bits (NaN stays NaN).
__device__ __forceinline__ uint32_t bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <bool kBf16>
__global__ void __launch_bounds__(kThreads)
dequantize_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                  int64_t rows, int64_t gpr, void* __restrict__ y, int64_t ld_y, float p_exp) {
    const int64_t ngroups = rows * gpr;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < ngroups; g += stride) {
        const int64_t r = g / gpr;
        const int64_t cg = g - r * gpr;
        const uint2 cw = *reinterpret_cast<const uint2*>(codes + g * 8);
        const uint32_t b = scales[g];
        const float sp = e4m3_value_or_nan(b & 0x7Fu);
        const bool int4 = (b & 0x80u) != 0;
        const float sp6 = 6.0f * sp;  // exact
        float out[16];
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const uint32_t nib = ((i < 8 ? cw.x : cw.y) >> (4 * (i & 7))) & 0xFu;
            const uint32_t mag = nib & 7u;
            float v;
            if (int4)
                v = ((float)mag * sp6) / 7.0f;  // exact numerator, correctly rounded quotient
            else
                v = e2m1_value(mag) * sp;       // exact
            v = v * p_exp;
            out[i] = (nib & 8u) ? -v : v;
        }
        if constexpr (kBf16) {
            uint4* p = reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(y) + r * ld_y + cg * 16);
            uint32_t w[8];
#pragma unroll
            for (int i = 0; i < 8; i++) w[i] = bf16_bits(out[2 * i]) | (bf16_bits(out[2 * i + 1]) << 16);
            p[0] = make_uint4(w[0], w[1], w[2], w[3]);
            p[1] = make_uint4(w[4], w[5], w[6], w[7]);
        } else {
            float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + r * ld_y + cg * 16);
#pragma unroll
            for (int i = 0; i < 4; i++)
                p[i] = make_float4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
        }
    }
}

}  // namespace

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                             int64_t cols, int32_t scale_exp, void* y, int bf16, int64_t ld_y,
                             hipStream_t stream) {
    const int64_t gpr = cols / 16;
    const int64_t ngroups = rows * gpr;
    int64_t blocks = (ngroups + kThreads - 1) / kThreads;
    if (blocks > 65536) blocks = 65536;
    if (bf16)
        hipLaunchKernelGGL(dequantize_kernel<true>, dim3((unsigned)blocks), dim3(kThreads), 0,
                           stream, codes, scales, rows, gpr, y, ld_y, pow2f(scale_exp));
    else
        hipLaunchKernelGGL(dequantize_kernel<false>, dim3((unsigned)blocks), dim3(kThreads), 0,
                           stream, codes, scales, rows, gpr, y, ld_y, pow2f(scale_exp));
    return hipGetLastError();
}

}  // namespace if4
