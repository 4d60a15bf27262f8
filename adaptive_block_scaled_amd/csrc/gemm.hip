// IF4 x IF4 (W4A4) GEMM for gfx950: C[M,N] = A[M,K] * W[N,K]^T, fp32 out.
//
// Both operands arrive packed (4-bit codes + one flagged E4M3 scale byte per
// 16 values along K).  The pages' MAC unit ("MAC Unit: Decoding Two Formats
// from One Sign Bit", podcast companion page) routes each operand group by
// its scale's sign bit to an FP or an INT decode path, with INT4 descaled by
// 6/7 "during multiplication" (gist.science summary, section 2, "Metodo
// 6/7").  Here each workgroup decodes its A and W K-slab once into LDS as
// fp16 with the group scale folded in -- FP4 values c*s' exactly, INT4 values
// rounded once to fp16 -- and the wave tiles run v_mfma_f32_32x32x16_f16
// (one MFMA K-step = one IF4 group) with fp32 accumulation.  The per-tensor
// 2^(E_A + E_W) is applied in the epilogue, so every decoded value stays in
// fp16's normal range (2^-10 .. 2688).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "if4_internal.h"

namespace if4 {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kThreads = 256;
constexpr int LDS_STRIDE = BK + 8;  // halfs; 144 B rows spread ds_read_b128 over all banks

__device__ __forceinline__ float e4m3_value_or_nan(uint32_t code7) {
    if (code7 == 0x7Fu) return __uint_as_float(0x7FC00000u);
    return code7 >= 8u ? __uint_as_float((code7 + 960u) << 20) : (float)code7 * 0.001953125f;
}

__device__ __forceinline__ float e2m1_value(uint32_t idx) {
    float m = (idx & 1u) ? 1.5f : 1.0f;
    uint32_t e = idx >> 1;
    return e == 0 ? (idx ? 0.5f : 0.0f) : m * (float)(1u << (e - 1));
}

// Decode one group (8 code bytes, scale byte b) to 16 fp16 values.
__device__ __forceinline__ void decode_group(uint2 cw, uint32_t b, _Float16 (&h)[16]) {
    const float sp = e4m3_value_or_nan(b & 0x7Fu);
    const bool int4 = (b & 0x80u) != 0;
    const float sp6 = 6.0f * sp;
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const uint32_t nib = ((i < 8 ? cw.x : cw.y) >> (4 * (i & 7))) & 0xFu;
        const uint32_t mag = nib & 7u;
        float v = int4 ? ((float)mag * sp6) / 7.0f : e2m1_value(mag) * sp;
        v = (nib & 8u) ? -v : v;
        h[i] = (_Float16)v;
    }
}

__global__ void __launch_bounds__(kThreads)
gemm_kernel(const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
            const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales,
            int64_t M, int64_t N, int64_t K, float* __restrict__ c, int64_t ldc, float out_scale) {
    __shared__ _Float16 As[BM * LDS_STRIDE];
    __shared__ _Float16 Ws[BN * LDS_STRIDE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;  // 2 x 2 waves, 64 x 64 each
    const int64_t m0 = (int64_t)blockIdx.y * BM;
    const int64_t n0 = (int64_t)blockIdx.x * BN;
    const int64_t gpr = K / 16;

    float16v acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

    for (int64_t k0 = 0; k0 < K; k0 += BK) {
        // decode: (BM + BN) rows x 4 groups = 1024 groups, 4 per thread
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int gid = tid + kThreads * j;
            const bool is_w = gid >= BM * 4;
            const int lr = (gid & (BM * 4 - 1)) >> 2;  // local row
            const int kg = gid & 3;
            const int64_t row = (is_w ? n0 : m0) + lr;
            const int64_t rows = is_w ? N : M;
            const int64_t g = k0 / 16 + kg;
            uint2 cw = make_uint2(0u, 0u);
            uint32_t b = 0;
            if (row < rows && g < gpr) {
                const uint8_t* cp = (is_w ? w_codes : a_codes) + row * (K / 2) + g * 8;
                cw = *reinterpret_cast<const uint2*>(cp);
                b = (is_w ? w_scales : a_scales)[row * gpr + g];
            }
            _Float16 h[16];
            decode_group(cw, b, h);
            _Float16* dst = (is_w ? Ws : As) + lr * LDS_STRIDE + kg * 16;
            half8 h0, h1;
#pragma unroll
            for (int t = 0; t < 8; t++) {
                h0[t] = h[t];
                h1[t] = h[8 + t];
            }
            *reinterpret_cast<half8*>(dst) = h0;
            *reinterpret_cast<half8*>(dst + 8) = h1;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK / 16; kk++) {
            half8 a[2], bv[2];
#pragma unroll
            for (int i = 0; i < 2; i++) {
                const int r = wm * 64 + i * 32 + (lane & 31);
                a[i] = *reinterpret_cast<const half8*>(As + r * LDS_STRIDE + kk * 16 + (lane >> 5) * 8);
            }
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const int r = wn * 64 + j * 32 + (lane & 31);
                bv[j] = *reinterpret_cast<const half8*>(Ws + r * LDS_STRIDE + kk * 16 + (lane >> 5) * 8);
            }
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < 2; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], bv[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }

    // epilogue: lane holds column lane%32 of each 32x32 block, rows
    // 8*(r/4) + 4*(lane/32) + r%4 for accumulator register r
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int64_t row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const int64_t col = n0 + wn * 64 + j * 32 + (lane & 31);
                if (row < M && col < N) c[row * ldc + col] = acc[i][j][r] * out_scale;
            }
}

__global__ void zero_kernel(float* __restrict__ c, int64_t M, int64_t N, int64_t ldc) {
    const int64_t total = M * N;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x)
        c[(i / N) * ldc + (i % N)] = 0.0f;
}

}  // namespace

hipError_t launch_gemm(const uint8_t* a_codes, const uint8_t* a_scales, int32_t a_exp,
                       const uint8_t* w_codes, const uint8_t* w_scales, int32_t w_exp, int64_t M,
                       int64_t N, int64_t K, float* c, int64_t ldc, hipStream_t stream) {
    if (K == 0) {
        int64_t blocks = (M * N + 255) / 256;
        if (blocks > 65536) blocks = 65536;
        hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, c, M, N, ldc);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
    // 2^(a_exp + w_exp) as a float: exact for |a_exp + w_exp| <= 126, else
    // applied as two factors
    const int e = a_exp + w_exp;
    float out_scale = (e >= -126 && e <= 127) ? pow2f(e) : 0.0f;
    if (!(e >= -126 && e <= 127)) {
        // |e| up to 128: split; keeps the product exact where representable
        out_scale = pow2f(e / 2) * pow2f(e - e / 2);
    }
    hipLaunchKernelGGL(gemm_kernel, grid, dim3(kThreads), 0, stream, a_codes, a_scales, w_codes,
                       w_scales, M, N, K, c, ldc, out_scale);
    return hipGetLastError();
}

}  // namespace if4
