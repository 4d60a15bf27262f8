// C-ABI front end of libif4: host-side validation, then one launch.
// Validation runs before any HIP call, so a bad argument never enqueues work.
#include "../../include/if4.h"

#include <stdint.h>

#include "if4_internal.h"

namespace {

constexpr int kMaxExp = 64;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

int elem_size(int dtype) { return dtype == IF4_F32 ? 4 : 2; }

int hip_status(hipError_t e) { return e == hipSuccess ? IF4_OK : IF4_ERR_HIP; }

int check_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols,
                   int64_t ld_x, const uint8_t* codes, const uint8_t* scales,
                   int32_t scale_exp, int mode) {
    if (x_dtype != IF4_F32 && x_dtype != IF4_BF16) return IF4_ERR_DTYPE;
    if (mode < IF4_MODE_ADAPTIVE || mode > IF4_MODE_FORCE_INT4) return IF4_ERR_DTYPE;
    if (rows < 0 || cols < 0 || cols % 16 != 0 || ld_x < cols) return IF4_ERR_SHAPE;
    if (scale_exp < -kMaxExp || scale_exp > kMaxExp) return IF4_ERR_RANGE;
    if (rows == 0 || cols == 0) return IF4_OK;
    if (!x || !codes || !scales) return IF4_ERR_NULL;
    if (!aligned(x, 16) || (ld_x * elem_size(x_dtype)) % 16 != 0 || !aligned(codes, 8))
        return IF4_ERR_ALIGN;
    return IF4_OK;
}

// x^T quantize: groups run along dim 0, so rows (not cols) must be whole
// groups; x needs only element alignment (each lane loads single elements).
int check_quantize_t(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                     const uint8_t* codes, const uint8_t* scales, int32_t scale_exp, int mode) {
    if (x_dtype != IF4_F32 && x_dtype != IF4_BF16) return IF4_ERR_DTYPE;
    if (mode < IF4_MODE_ADAPTIVE || mode > IF4_MODE_FORCE_INT4) return IF4_ERR_DTYPE;
    if (rows < 0 || cols < 0 || rows % 16 != 0 || ld_x < cols) return IF4_ERR_SHAPE;
    if (scale_exp < -kMaxExp || scale_exp > kMaxExp) return IF4_ERR_RANGE;
    if (rows == 0 || cols == 0) return IF4_OK;
    if (!x || !codes || !scales) return IF4_ERR_NULL;
    if (!aligned(x, elem_size(x_dtype)) || !aligned(codes, 8)) return IF4_ERR_ALIGN;
    return IF4_OK;
}

}  // namespace

extern "C" {

int if4_version(void) { return 100; }

const char* if4_status_string(int status) {
    switch (status) {
        case IF4_OK: return "ok";
        case IF4_ERR_NULL: return "null pointer";
        case IF4_ERR_SHAPE: return "bad shape (negative size, cols/K not a multiple of 16, or leading dimension too small)";
        case IF4_ERR_ALIGN: return "misaligned pointer or leading dimension";
        case IF4_ERR_DTYPE: return "unknown dtype or mode";
        case IF4_ERR_RANGE: return "scale exponent outside [-64, 64]";
        case IF4_ERR_HIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

int if4_quantize_mode(const void* x, int x_dtype, int64_t rows, int64_t cols,
                      int64_t ld_x, uint8_t* codes, uint8_t* scales,
                      int32_t scale_exp, int mode, void* stream) {
    int st = check_quantize(x, x_dtype, rows, cols, ld_x, codes, scales, scale_exp, mode);
    if (st != IF4_OK || rows == 0 || cols == 0) return st;
    return hip_status(if4::launch_quantize(x, x_dtype == IF4_BF16, rows, cols, ld_x, codes,
                                           scales, scale_exp, mode, (hipStream_t)stream));
}

int if4_quantize_rht(const void* x, int x_dtype, int64_t rows, int64_t cols,
                     int64_t ld_x, uint32_t sign_mask, uint8_t* codes, uint8_t* scales,
                     int32_t scale_exp, int mode, void* stream) {
    if (sign_mask > 0xFFFFu) return IF4_ERR_RANGE;
    int st = check_quantize(x, x_dtype, rows, cols, ld_x, codes, scales, scale_exp, mode);
    if (st != IF4_OK || rows == 0 || cols == 0) return st;
    return hip_status(if4::launch_quantize_rht(x, x_dtype == IF4_BF16, rows, cols, ld_x,
                                               sign_mask, codes, scales, scale_exp, mode,
                                               (hipStream_t)stream));
}

int if4_quantize_t(const void* x, int x_dtype, int64_t rows, int64_t cols,
                   int64_t ld_x, uint8_t* codes, uint8_t* scales,
                   int32_t scale_exp, int mode, void* stream) {
    int st = check_quantize_t(x, x_dtype, rows, cols, ld_x, codes, scales, scale_exp, mode);
    if (st != IF4_OK || rows == 0 || cols == 0) return st;
    return hip_status(if4::launch_quantize_t(x, x_dtype == IF4_BF16, rows, cols, ld_x, codes,
                                             scales, scale_exp, mode, (hipStream_t)stream));
}

int if4_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols,
                 int64_t ld_x, uint8_t* codes, uint8_t* scales,
                 int32_t scale_exp, void* stream) {
    return if4_quantize_mode(x, x_dtype, rows, cols, ld_x, codes, scales, scale_exp,
                             IF4_MODE_ADAPTIVE, stream);
}

int if4_quantize_ifn(int bits, const void* x, int x_dtype, int64_t rows, int64_t cols,
                     int64_t ld_x, uint8_t* codes, uint8_t* scales, int32_t scale_exp, int mode,
                     void* stream) {
    if (bits != 3 && bits != 6) return IF4_ERR_DTYPE;
    int st = check_quantize(x, x_dtype, rows, cols, ld_x, codes, scales, scale_exp, mode);
    if (st != IF4_OK || rows == 0 || cols == 0) return st;
    return hip_status(if4::launch_quantize_ifn(bits, x, x_dtype == IF4_BF16, rows, cols, ld_x,
                                               codes, scales, scale_exp, mode,
                                               (hipStream_t)stream));
}

int if4_dequantize_ifn(int bits, const uint8_t* codes, const uint8_t* scales, int64_t rows,
                       int64_t cols, int32_t scale_exp, void* y, int y_dtype, int64_t ld_y,
                       void* stream) {
    if (bits != 3 && bits != 6) return IF4_ERR_DTYPE;
    if (y_dtype != IF4_F32 && y_dtype != IF4_BF16) return IF4_ERR_DTYPE;
    if (rows < 0 || cols < 0 || cols % 16 != 0 || ld_y < cols) return IF4_ERR_SHAPE;
    if (scale_exp < -kMaxExp || scale_exp > kMaxExp) return IF4_ERR_RANGE;
    if (rows == 0 || cols == 0) return IF4_OK;
    if (!codes || !scales || !y) return IF4_ERR_NULL;
    if (!aligned(y, 16) || (ld_y * elem_size(y_dtype)) % 16 != 0 || !aligned(codes, 8))
        return IF4_ERR_ALIGN;
    return hip_status(if4::launch_dequantize_ifn(bits, codes, scales, rows, cols, scale_exp, y,
                                                 y_dtype == IF4_BF16, ld_y, (hipStream_t)stream));
}

int if4_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                   int64_t cols, int32_t scale_exp, void* y, int y_dtype,
                   int64_t ld_y, void* stream) {
    if (y_dtype != IF4_F32 && y_dtype != IF4_BF16) return IF4_ERR_DTYPE;
    if (rows < 0 || cols < 0 || cols % 16 != 0 || ld_y < cols) return IF4_ERR_SHAPE;
    if (scale_exp < -kMaxExp || scale_exp > kMaxExp) return IF4_ERR_RANGE;
    if (rows == 0 || cols == 0) return IF4_OK;
    if (!codes || !scales || !y) return IF4_ERR_NULL;
    if (!aligned(y, 16) || (ld_y * elem_size(y_dtype)) % 16 != 0 || !aligned(codes, 8))
        return IF4_ERR_ALIGN;
    return hip_status(if4::launch_dequantize(codes, scales, rows, cols, scale_exp, y,
                                             y_dtype == IF4_BF16, ld_y, (hipStream_t)stream));
}

int if4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, int32_t a_exp,
             const uint8_t* w_codes, const uint8_t* w_scales, int32_t w_exp,
             int64_t M, int64_t N, int64_t K, float* c, int64_t ldc,
             void* stream) {
    if (M < 0 || N < 0 || K < 0 || K % 16 != 0 || ldc < N) return IF4_ERR_SHAPE;
    if (a_exp < -kMaxExp || a_exp > kMaxExp || w_exp < -kMaxExp || w_exp > kMaxExp)
        return IF4_ERR_RANGE;
    if (M == 0 || N == 0) return IF4_OK;
    if (!c) return IF4_ERR_NULL;
    if (K > 0 && (!a_codes || !a_scales || !w_codes || !w_scales)) return IF4_ERR_NULL;
    if (!aligned(c, 4) || (K > 0 && (!aligned(a_codes, 8) || !aligned(w_codes, 8))))
        return IF4_ERR_ALIGN;
    return hip_status(if4::launch_gemm(a_codes, a_scales, a_exp, w_codes, w_scales, w_exp, M,
                                       N, K, c, ldc, (hipStream_t)stream));
}

}  // extern "C"
