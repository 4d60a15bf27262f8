// IF4 dequantize for gfx950.
//
// Each group's scale byte selects the decode: FP4 nibbles decode to
// (+-) E2M1 * s', INT4 nibbles to (+-) |q| * s' descaled by 6/7
// ("Adaptive Block-Scaled Data Types", gist.science summary, section 2,
// "Metodo 6/7"), then times 2^E.  The INT4 value is the fp32 nearest to
// 6 |q| s' / 7 (times 2^E, which is exact: every result is fp32-normal).
//
// One lane per group (8 code bytes + 1 scale byte in, 16 values out), one
// wave (64 groups) per workgroup.
// The decode is branch-free and identical for both formats:
//  * each nibble becomes an E4M3 byte -- FP4 s.e1e0.m -> s.00e1e0.m00 (the
//    value c * 2^-6), INT4 s.mmm -> s.0000.mmm (the subnormal |q| * 2^-9) --
//    and the hardware fp8 conversion yields m = +-c 2^-6 or +-|q| 2^-9
//    exactly, sign and zero included;
//  * y = fma(m, H, m * L) with a pair computed from the scale byte:
//    FP4: H = s' 2^(E+6), L = 0, so y = c s' 2^E exactly; INT4:
//    H = H' 2^(E+9) and L = fl32((6 s' - 7 H') * fl32(1/7)) 2^(E+9), where
//    H' is 6 s'/7 rounded toward zero: a two-term split of 6 s'/7 whose fma
//    gives the correctly rounded fl32(6 |q| s'/7) 2^E for every E4M3 s' and
//    |q| = 1..7 (checked exhaustively in exact arithmetic), with L >= 0 so
//    that a zero magnitude keeps its sign; NaN scales give H = NaN.
// bf16 output rounds each fp32 value to nearest even (v_cvt_pk_bf16_f32).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "if4_internal.h"
#include "xcd_order.h"

namespace if4 {
namespace {

constexpr int kThreads = 64;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float e4m3_value_or_nan(uint32_t code7) {
    if (code7 == 0x7Fu) return __uint_as_float(0x7FC00000u);
    return code7 >= 8u ? __uint_as_float((code7 + 960u) << 20) : (float)code7 * 0.001953125f;
}

// Per-scale-byte decode constants: H, L, nibble shift (2 for FP4, 0 for INT4).
struct Entry {
    float h, l;
    uint32_t sh;
};

__device__ __forceinline__ Entry make_entry(uint32_t b, float p_exp) {
    const float sp = e4m3_value_or_nan(b & 0x7Fu);
    Entry e;
    if (b & 0x80u) {
        const float six = 6.0f * sp;  // exact
        // H = 6 s'/7 rounded toward zero, so the residual and L are >= 0 and
        // y keeps the sign of m for a zero magnitude (-0 stays -0)
        float h = six / 7.0f;
        if (__builtin_fmaf(-h, 7.0f, six) < 0.0f) h = __uint_as_float(__float_as_uint(h) - 1u);
        const float l = __builtin_fmaf(-h, 7.0f, six) * 0.142857149f;  // exact residual / 7
        const float k = p_exp * 512.0f;                       // 2^(E+9), exact
        e.h = h * k;
        e.l = l * k;
        e.sh = 0;
    } else {
        e.h = sp * (p_exp * 64.0f);                           // s' 2^(E+6)
        e.l = 0.0f;
        e.sh = 2;
    }
    return e;
}

// Decode the 8 nibbles of code word w (element 2j in the low nibble of byte
// j) into out[0..7] in element order.
__device__ __forceinline__ void decode_word(uint32_t w, const Entry& e, float* out) {
    const uint32_t mask = 0x07070707u << e.sh;
    // even nibbles (elements 0, 2, 4, 6) and odd ones (1, 3, 5, 7) as E4M3 bytes
    const uint32_t ev = ((w << 4) & 0x80808080u) | ((w << e.sh) & mask);
    const uint32_t od = (w & 0x80808080u) | ((w >> (4u - e.sh)) & mask);
    const auto e01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(ev, 1.0f, false);  // elements 0, 2
    const auto e23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(ev, 1.0f, true);   // 4, 6
    const auto o01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(od, 1.0f, false);  // 1, 3
    const auto o23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(od, 1.0f, true);   // 5, 7
    const float m[8] = {e01[0], o01[0], e01[1], o01[1], e23[0], o23[0], e23[1], o23[1]};
#pragma unroll
    for (int i = 0; i < 8; i++) out[i] = __builtin_fmaf(m[i], e.h, m[i] * e.l);
}

template <bool kBf16, bool kContig>
__global__ void __launch_bounds__(kThreads)
dequantize_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                  int64_t rows, int64_t gpr, void* __restrict__ y, int64_t ld_y, float p_exp) {
    const int64_t ngroups = rows * gpr;
    auto store = [&](int64_t g, const float* out) {
        int64_t off;
        if constexpr (kContig) {
            off = g * 16;
        } else {
            const int64_t r = g / gpr;
            off = r * ld_y + (g - r * gpr) * 16;
        }
        if constexpr (kBf16) {
            uint32_t w[8];
#pragma unroll
            for (int i = 0; i < 8; i++) {
                bf16x2 v;
                v[0] = (__bf16)out[2 * i];
                v[1] = (__bf16)out[2 * i + 1];
                w[i] = __builtin_bit_cast(uint32_t, v);
            }
            uint4* p = reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(y) + off);
            p[0] = make_uint4(w[0], w[1], w[2], w[3]);
            p[1] = make_uint4(w[4], w[5], w[6], w[7]);
        } else {
            float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + off);
#pragma unroll
            for (int i = 0; i < 4; i++)
                p[i] = make_float4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
        }
    };

    // One group per thread, one wave per workgroup: the thread's loads go
    // out first (past the end they re-read the last group, whose store is
    // then skipped, so no load sits behind a branch) and the scale byte's
    // decode constants are computed by the thread itself -- no LDS table, no
    // barrier (a per-workgroup table of 256 entries cost the same VALU work
    // plus a barrier, and 12% more time at 256 x 256).  (Grid-stride loops
    // over fewer workgroups, with the next group prefetched, measured up to
    // 33% slower on a 470 MB output: they keep far fewer loads in flight.)
    const int64_t gid = xcd_paired_block(blockIdx.x, gridDim.x) * kThreads + threadIdx.x;
    const int64_t g = gid < ngroups - 1 ? gid : ngroups - 1;
    const uint2 cw = *reinterpret_cast<const uint2*>(codes + g * 8);
    const uint32_t b = scales[g];
    const Entry e = make_entry(b, p_exp);
    float out[16];
    decode_word(cw.x, e, out);
    decode_word(cw.y, e, out + 8);
    if (gid < ngroups) store(gid, out);
}

template <bool kBf16>
void launch(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t gpr, void* y,
            int64_t ld_y, float p_exp, unsigned blocks, hipStream_t stream) {
    if (ld_y == gpr * 16)
        hipLaunchKernelGGL((dequantize_kernel<kBf16, true>), dim3(blocks), dim3(kThreads), 0,
                           stream, codes, scales, rows, gpr, y, ld_y, p_exp);
    else
        hipLaunchKernelGGL((dequantize_kernel<kBf16, false>), dim3(blocks), dim3(kThreads), 0,
                           stream, codes, scales, rows, gpr, y, ld_y, p_exp);
}

}  // namespace

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                             int64_t cols, int32_t scale_exp, void* y, int bf16, int64_t ld_y,
                             hipStream_t stream) {
    const int64_t gpr = cols / 16;
    const int64_t ngroups = rows * gpr;
    const int64_t blocks = (ngroups + kThreads - 1) / kThreads;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (bf16)
        launch<true>(codes, scales, rows, gpr, y, ld_y, pow2f(scale_exp), (unsigned)blocks, stream);
    else
        launch<false>(codes, scales, rows, gpr, y, ld_y, pow2f(scale_exp), (unsigned)blocks, stream);
    return hipGetLastError();
}

}  // namespace if4
