// IF4 x IF4 (W4A4) GEMM for gfx950: C[M,N] = A[M,K] * W[N,K]^T, fp32 out.
//
// Both operands arrive packed (4-bit codes + one flagged E4M3 scale byte per
// 16 values along K).  The pages' MAC unit ("MAC Unit: Decoding Two Formats
// from One Sign Bit", podcast companion page) routes each operand group by
// its scale's sign bit to an FP or an INT decode path, with INT4 descaled by
// 6/7 "during multiplication" (gist.science summary, section 2, "Metodo
// 6/7").  Here each workgroup decodes its A and W K-slab once into LDS as
// fp16 with the group scale folded in -- FP4 values c*s' exactly, INT4
// values |q| * fl16(6 s'/7) -- and the waves run v_mfma_f32_32x32x16_f16
// (one MFMA K-step = one IF4 group) with fp32 accumulation.  The per-tensor
// 2^(E_A + E_W) is applied in the epilogue, so every decoded value stays in
// fp16's normal range (2^-10 .. 2688).
//
// Tiling: 256x256 output tile per workgroup of 8 waves (2 x 4), each wave
// 128x64 (4 x 2 MFMA blocks of 32x32, 128 fp32 accumulators per lane).
// K advances in slabs of 64 (four groups): every thread loads one row's
// 32 code bytes and 4 scale bytes of the next slab while the waves run the
// current slab's MFMAs from the other LDS buffer, then decodes and stores
// them; one barrier per slab.  LDS: 2 buffers x 512 rows x 144 B (128 B of
// fp16 + 16 B pad, which spreads the ds_read_b128/ds_write_b128 of
// consecutive rows over all banks) + a 1 KB table of group scales.
//
// Decode of one group (branch-free; the flag only picks two table words and
// the scale): the nibble magnitudes index an 8-entry byte table with
// v_perm_b32 -- the table holds the fp16 high byte of each FP4 value
// (0, .5, 1, 1.5, 2, 3, 4, 6) or INT4 magnitude (0..7); all of them have a
// zero low byte -- the sign bit is moved to bit 15, and a packed fp16
// multiply applies the group scale.  Nibbles j and j+4 of a code word form
// one fp16 pair, so a group lands in LDS in the order
// 0,4,1,5,2,6,3,7 | 8,12,9,13,10,14,11,15; A and W use the same order, so
// the dot products are unchanged.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "if4_internal.h"

namespace if4 {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float16v __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int WAVES_M = 2, WAVES_N = 4;
constexpr int TM = BM / WAVES_M, TN = BN / WAVES_N;  // 128 x 64 per wave
constexpr int FM = TM / 32, FN = TN / 32;            // 4 x 2 MFMA blocks
constexpr int kThreads = 64 * WAVES_M * WAVES_N;     // 512
constexpr int ROW_BYTES = BK * 2 + 16;               // 144
constexpr int BUF_BYTES = (BM + BN) * ROW_BYTES;     // 73728
constexpr int SIGMA_OFF = 2 * BUF_BYTES;
constexpr int SMEM_BYTES = SIGMA_OFF + 256 * 4;      // 148480
static_assert(BM + BN == kThreads, "one thread per tile row");

// fp16 high bytes of the 8 magnitudes, packed as v_perm_b32 table words
// (bytes 0-3 from the low word, 4-7 from the high word).
constexpr uint32_t FP4_LO = 0x3E3C3800u;  // 0, .5, 1, 1.5
constexpr uint32_t FP4_HI = 0x46444240u;  // 2, 3, 4, 6
constexpr uint32_t INT_LO = 0x42403C00u;  // 0, 1, 2, 3
constexpr uint32_t INT_HI = 0x47464544u;  // 4, 5, 6, 7

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ uint32_t pk_mul(uint32_t a, uint32_t b) {
    half2v x = __builtin_bit_cast(half2v, a);
    half2v y = __builtin_bit_cast(half2v, b);
    return __builtin_bit_cast(uint32_t, x * y);
}

// Decode one code word (8 nibbles) of a group into 4 fp16 pairs.
__device__ __forceinline__ void decode_word(uint32_t w, uint32_t tlo, uint32_t thi,
                                            uint32_t sig2, uint32_t (&out)[4]) {
    const uint32_t w4 = w << 4, w8 = w << 8, w12 = w << 12, wr4 = w >> 4;
    const uint32_t m_sel = 0x07000700u, z_sel = 0x000C000Cu, sgn = 0x80008000u;
    // pair j = (nibble j, nibble j + 4): magnitudes to bytes 1 and 3 of the
    // selector (bytes 0 and 2 select zero), signs to bits 15 and 31
    out[0] = pk_mul(perm(thi, tlo, (w8 & m_sel) | z_sel) | (w12 & sgn), sig2);
    out[1] = pk_mul(perm(thi, tlo, (w4 & m_sel) | z_sel) | (w8 & sgn), sig2);
    out[2] = pk_mul(perm(thi, tlo, (w & m_sel) | z_sel) | (w4 & sgn), sig2);
    out[3] = pk_mul(perm(thi, tlo, (wr4 & m_sel) | z_sel) | (w & sgn), sig2);
}

__device__ __forceinline__ void decode_group(uint32_t w0, uint32_t w1, uint32_t b,
                                             const uint32_t* __restrict__ sigma,
                                             uint32_t (&h)[8]) {
    const bool int4 = (b & 0x80u) != 0;
    const uint32_t tlo = int4 ? INT_LO : FP4_LO;
    const uint32_t thi = int4 ? INT_HI : FP4_HI;
    const uint32_t sig2 = sigma[b];
    uint32_t a[4], c[4];
    decode_word(w0, tlo, thi, sig2, a);
    decode_word(w1, tlo, thi, sig2, c);
#pragma unroll
    for (int i = 0; i < 4; i++) {
        h[i] = a[i];
        h[4 + i] = c[i];
    }
}

struct Packed {
    uint4 c0, c1;  // 32 code bytes = 4 groups of one row
    uint32_t b;    // 4 scale bytes
};

// Codes are only guaranteed 8-byte aligned (rows are K/2 bytes, K a
// multiple of 16), so the 32 bytes of a row's slab are read as four 8-byte
// loads.
__device__ __forceinline__ void load_slab(const uint8_t* __restrict__ codes,
                                          const uint8_t* __restrict__ scales, int64_t row,
                                          int64_t rows, int64_t K, int64_t gpr, int64_t k0,
                                          Packed& p) {
    uint2 q0 = make_uint2(0u, 0u), q1 = q0, q2 = q0, q3 = q0;
    uint32_t b = 0;
    if (row < rows) {
        const int64_t g0 = k0 / 16;
        const int64_t ng = gpr - g0;  // >= 1
        const uint2* cp = reinterpret_cast<const uint2*>(codes + row * (K / 2) + k0 / 2);
        const uint8_t* sp = scales + row * gpr + g0;
        q0 = cp[0];
        b = sp[0];
        if (ng > 1) {
            q1 = cp[1];
            b |= (uint32_t)sp[1] << 8;
        }
        if (ng > 2) {
            q2 = cp[2];
            b |= (uint32_t)sp[2] << 16;
        }
        if (ng > 3) {  // a K tail leaves fewer than 4 groups; the rest decode to 0
            q3 = cp[3];
            b |= (uint32_t)sp[3] << 24;
        }
    }
    p.c0 = make_uint4(q0.x, q0.y, q1.x, q1.y);
    p.c1 = make_uint4(q2.x, q2.y, q3.x, q3.y);
    p.b = b;
}

__device__ __forceinline__ void store_slab(uint8_t* __restrict__ rowp, const Packed& p,
                                           const uint32_t* __restrict__ sigma) {
    const uint32_t w[8] = {p.c0.x, p.c0.y, p.c0.z, p.c0.w, p.c1.x, p.c1.y, p.c1.z, p.c1.w};
#pragma unroll
    for (int g = 0; g < 4; g++) {
        uint32_t h[8];
        decode_group(w[2 * g], w[2 * g + 1], (p.b >> (8 * g)) & 0xFFu, sigma, h);
        uint4* dst = reinterpret_cast<uint4*>(rowp + g * 32);
        dst[0] = make_uint4(h[0], h[1], h[2], h[3]);
        dst[1] = make_uint4(h[4], h[5], h[6], h[7]);
    }
}

__device__ __forceinline__ uint32_t sigma_entry(uint32_t b) {
    // fp16 group scale for scale byte b: s' for FP4, fl16(fl32(6 s'/7)) for
    // INT4; NaN for the 0x7F/0xFF pattern.  Duplicated into both halves.
    const uint32_t code = b & 0x7Fu;
    float sp = code >= 8u ? __uint_as_float((code + 960u) << 20) : (float)code * 0.001953125f;
    if (code == 0x7Fu) sp = __uint_as_float(0x7FC00000u);
    const float v = (b & 0x80u) ? (6.0f * sp) / 7.0f : sp;
    const _Float16 hv = (_Float16)v;
    const uint32_t u = __builtin_bit_cast(uint16_t, hv);
    return u | (u << 16);
}

__global__ void __launch_bounds__(kThreads)
gemm_kernel(const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
            const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales,
            int64_t M, int64_t N, int64_t K, float* __restrict__ c, int64_t ldc, float out_scale,
            int tiles_m, int tiles_n) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint32_t* sigma = reinterpret_cast<uint32_t*>(smem + SIGMA_OFF);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a
    // contiguous run of tiles, walking down M within a column of W tiles so
    // that concurrently running tiles share W rows in their XCD's L2.
    const int total = tiles_m * tiles_n;
    int bid = blockIdx.x;
    if (total % 8 == 0) bid = (bid % 8) * (total / 8) + bid / 8;
    const int tm = bid % tiles_m, tn = bid / tiles_m;
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int64_t gpr = K / 16;

    if (tid < 256) sigma[tid] = sigma_entry(tid);

    // this thread's load/decode row: A rows 0..255, then W rows 0..255
    const bool is_w = tid >= BM;
    const int lr = is_w ? tid - BM : tid;
    const uint8_t* codes = is_w ? w_codes : a_codes;
    const uint8_t* scales = is_w ? w_scales : a_scales;
    const int64_t grow = (is_w ? n0 : m0) + lr;
    const int64_t grows = is_w ? N : M;
    const int lds_row = tid;  // rows 0..255 = A tile, 256..511 = W tile

    float16v acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

    const int nslabs = (int)((K + BK - 1) / BK);
    Packed p;
    load_slab(codes, scales, grow, grows, K, gpr, 0, p);
    __syncthreads();  // sigma table ready
    store_slab(smem + lds_row * ROW_BYTES, p, sigma);
    __syncthreads();

    const int a_row0 = wm * TM + (lane & 31);
    const int w_row0 = BM + wn * TN + (lane & 31);
    const int koff = (lane >> 5) * 16;  // bytes: 8 halfs per lane half

    for (int s = 0; s < nslabs; s++) {
        const uint8_t* buf = smem + (s & 1) * BUF_BYTES;
        const bool more = s + 1 < nslabs;
        if (more) load_slab(codes, scales, grow, grows, K, gpr, (int64_t)(s + 1) * BK, p);
#pragma unroll
        for (int kk = 0; kk < BK / 16; kk++) {
            half8 av[FM], bv[FN];
#pragma unroll
            for (int i = 0; i < FM; i++)
                av[i] = *reinterpret_cast<const half8*>(buf + (a_row0 + 32 * i) * ROW_BYTES +
                                                        kk * 32 + koff);
#pragma unroll
            for (int j = 0; j < FN; j++)
                bv[j] = *reinterpret_cast<const half8*>(buf + (w_row0 + 32 * j) * ROW_BYTES +
                                                        kk * 32 + koff);
#pragma unroll
            for (int i = 0; i < FM; i++)
#pragma unroll
                for (int j = 0; j < FN; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j],
                                                                       0, 0, 0);
        }
        if (more)
            store_slab(smem + ((s + 1) & 1) * BUF_BYTES + lds_row * ROW_BYTES, p, sigma);
        __syncthreads();
    }

    // epilogue: lane holds column lane%32 of each 32x32 block, rows
    // 8*(r/4) + 4*(lane/32) + r%4 for accumulator register r
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++) {
            const int64_t col = n0 + wn * TN + j * 32 + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int64_t row =
                    m0 + wm * TM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (row < M && col < N) c[row * ldc + col] = acc[i][j][r] * out_scale;
            }
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
    // LDS above 64 KB must be requested per kernel (idempotent, any device)
    hipError_t err = hipFuncSetAttribute((const void*)gemm_kernel,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, SMEM_BYTES);
    if (err != hipSuccess) return err;
    const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    if (tiles_m * tiles_n > 0x7FFFFFFF) return hipErrorInvalidValue;
    // 2^(a_exp + w_exp), exact; |a_exp + w_exp| <= 128 is split in two factors
    const int e = a_exp + w_exp;
    const float out_scale = pow2f(e / 2) * pow2f(e - e / 2);
    hipLaunchKernelGGL(gemm_kernel, dim3((unsigned)(tiles_m * tiles_n)), dim3(kThreads),
                       SMEM_BYTES, stream, a_codes, a_scales, w_codes, w_scales, M, N, K, c, ldc,
                       out_scale, (int)tiles_m, (int)tiles_n);
    return hipGetLastError();
}

}  // namespace if4
