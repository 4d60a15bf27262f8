// Internal launcher interface between the C-ABI front end (api.cpp) and the
// HIP kernel translation units.  Not installed; callers use include/if4.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace if4 {

// Power-of-two float 2^e for -126 <= e <= 127 (exact).
inline float pow2f(int e) {
    union {
        uint32_t u;
        float f;
    } v;
    v.u = (uint32_t)(e + 127) << 23;
    return v.f;
}

hipError_t launch_quantize(const void* x, int bf16, int64_t rows, int64_t cols,
                           int64_t ld_x, uint8_t* codes, uint8_t* scales,
                           int32_t scale_exp, int mode, hipStream_t stream);

hipError_t launch_quantize_rht(const void* x, int bf16, int64_t rows, int64_t cols,
                               int64_t ld_x, uint32_t sign_mask, uint8_t* codes,
                               uint8_t* scales, int32_t scale_exp, int mode,
                               hipStream_t stream);

hipError_t launch_quantize_t(const void* x, int bf16, int64_t rows, int64_t cols,
                             int64_t ld_x, uint8_t* codes, uint8_t* scales,
                             int32_t scale_exp, int mode, hipStream_t stream);

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales,
                             int64_t rows, int64_t cols, int32_t scale_exp,
                             void* y, int bf16, int64_t ld_y, hipStream_t stream);

hipError_t launch_quantize_ifn(int bits, const void* x, int bf16, int64_t rows, int64_t cols,
                               int64_t ld_x, uint8_t* codes, uint8_t* scales, int32_t scale_exp,
                               int mode, hipStream_t stream);

hipError_t launch_dequantize_ifn(int bits, const uint8_t* codes, const uint8_t* scales,
                                 int64_t rows, int64_t cols, int32_t scale_exp, void* y, int bf16,
                                 int64_t ld_y, hipStream_t stream);

hipError_t launch_gemm(const uint8_t* a_codes, const uint8_t* a_scales,
                       int32_t a_exp, const uint8_t* w_codes,
                       const uint8_t* w_scales, int32_t w_exp, int64_t M,
                       int64_t N, int64_t K, float* c, int64_t ldc,
                       hipStream_t stream);

}  // namespace if4
