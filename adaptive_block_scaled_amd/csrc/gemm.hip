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
// Tiling: 256x256 output tile per workgroup of 4 waves (2 x 2), each wave
// 128x128 (4 x 4 MFMA blocks of 32x32, 256 fp32 accumulators per lane in
// AGPRs, one wave per SIMD).
// K advances in slabs of 64 (four groups).  While the waves run the 64
// MFMAs of slab s from one LDS buffer, every thread decodes its A row and
// W row of slab s+1 into the other buffer, one group per 16-deep MFMA step,
// and right after decoding a group reloads that group's registers with the
// same group of slab s+2 -- so each load has a whole slab of MFMA work to
// arrive in, with one register set and no copies.  One barrier per slab.
// LDS: 2 buffers x 512 rows x 144 B (128 B of fp16 + 16 B pad, which spreads
// the ds_read_b128/ds_write_b128 of consecutive rows over all banks).
// Rows past M or N and groups past K load an in-range neighbour and decode
// with a zero scale, so there are no branches around the loads.
//
// Decode of one group is branch-free (the flag only picks a shift, a mask
// and a power-of-two conversion scale): see decode_word.  A group lands in
// LDS in the order 0,2,4,6,1,3,5,7 | 8,10,12,14,9,11,13,15; A and W use the
// same order, so the dot products are unchanged.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "if4_internal.h"

namespace if4 {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float16v __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256, BK = 64;
// LDS tiles are stored in MFMA-fragment order: for each block of 32 rows,
// each 16-deep group and each half of it, the 32 rows' 16-byte pieces lie
// next to each other, so a wave reads a whole 32x16 fragment as one
// contiguous 1 KB ds_read_b128 and a decoding wave writes contiguous 512 B
// runs.  Offset of (row R, group g, half h) inside an operand tile:
constexpr int TILE_BYTES = 256 * BK * 2;             // 32 KB per operand
constexpr int BUF_BYTES = 2 * TILE_BYTES;            // A tile, then W tile
constexpr int SMEM_BYTES = 2 * BUF_BYTES;            // double-buffered: 128 KB
__device__ __forceinline__ int frag_off(int R, int g, int h) {
    return ((((R >> 5) * (BK / 16) + g) * 2 + h) * 32 + (R & 31)) * 16;
}

// Wave layout of a 256x256 tile: WM x WN waves, each (256/WM) x (256/WN).
// With 4 waves every thread owns one A row and one W row; with 8 waves one
// row of either.
template <int WM, int WN>
struct Layout {
    static constexpr int kWaves = WM * WN;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int FM = TM / 32, FN = TN / 32;
    static constexpr bool kTwoRows = kThreads == BM;
    static_assert(kThreads == BM || kThreads == BM + BN, "one or two rows per thread");
};

__device__ __forceinline__ uint32_t pk_mul(uint32_t a, uint32_t b) {
    half2v x = __builtin_bit_cast(half2v, a);
    half2v y = __builtin_bit_cast(half2v, b);
    return __builtin_bit_cast(uint32_t, x * y);
}

// One group's packed data in registers: 16 nibbles and the scale byte.  The
// loaded values are only consumed by the decode one slab later, so nothing
// may touch them right after the load (that would force a wait).
struct Group {
    uint32_t w0, w1;
    uint32_t b;
};

// Decode one code word (8 nibbles) into 4 fp16 pairs.  Each nibble becomes
// an E4M3 byte: FP4 s.e1e0.m -> s.00e1e0.m00, whose value is c * 2^-6; INT4
// s.mmm -> s.0000.mmm, an E4M3 subnormal worth |q| * 2^-9.  The hardware
// E4M3 -> fp16 conversion scales by 2^6 or 2^9 (exact), giving c or |q|, and
// a packed fp16 multiply applies the group scale.  The even nibbles' bytes
// and the odd nibbles' bytes are built in two words, so the pairs come out
// as (0,2) (4,6) (1,3) (5,7).
__device__ __forceinline__ void decode_word(uint32_t w, uint32_t sh, uint32_t rsh, uint32_t mask,
                                            float cvt_scale, uint32_t sig2, uint32_t* out) {
    const uint32_t ev = ((w << 4) & 0x80808080u) | ((w << sh) & mask);
    const uint32_t od = (w & 0x80808080u) | ((w >> rsh) & mask);
    out[0] = pk_mul(__builtin_bit_cast(uint32_t,
                    __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(ev, cvt_scale, false)), sig2);
    out[1] = pk_mul(__builtin_bit_cast(uint32_t,
                    __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(ev, cvt_scale, true)), sig2);
    out[2] = pk_mul(__builtin_bit_cast(uint32_t,
                    __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(od, cvt_scale, false)), sig2);
    out[3] = pk_mul(__builtin_bit_cast(uint32_t,
                    __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(od, cvt_scale, true)), sig2);
}

// Decode a group to 16 fp16 values and store them (32 bytes) at dst.  The
// group scale: s' from the E4M3 code by the hardware conversion (exact,
// NaN for 0x7F), times fl32(6/7) for INT4, rounded once to fp16.
__device__ __forceinline__ void decode_store(uint8_t* __restrict__ tile, int R, int gi,
                                             const Group& g, bool zero) {
    const uint32_t b = g.b;
    const float sp = __builtin_amdgcn_cvt_scalef32_f32_fp8(b & 0x7Fu, 1.0f, 0);
    const bool int4 = (b & 0x80u) != 0;
    float sig = int4 ? sp * 0.857142866f : sp;
    sig = zero ? 0.0f : sig;
    const uint32_t h16 = __builtin_bit_cast(uint16_t, (_Float16)sig);
    const uint32_t sig2 = h16 | (h16 << 16);
    const uint32_t sh = int4 ? 0u : 2u;
    const uint32_t mask = 0x07070707u << sh;
    const float cvt_scale = int4 ? 512.0f : 64.0f;
    uint32_t h[8];
    decode_word(g.w0, sh, 4u - sh, mask, cvt_scale, sig2, h);
    decode_word(g.w1, sh, 4u - sh, mask, cvt_scale, sig2, h + 4);
    *reinterpret_cast<uint4*>(tile + frag_off(R, gi, 0)) = make_uint4(h[0], h[1], h[2], h[3]);
    *reinterpret_cast<uint4*>(tile + frag_off(R, gi, 1)) = make_uint4(h[4], h[5], h[6], h[7]);
}

// Load group index gi (clamped into the row) of a row whose code and scale
// rows start at cp and sp.  A group past K (or a row past M/N) decodes with
// a zero scale, decided at decode time from the indices.
__device__ __forceinline__ void load_group(const uint8_t* __restrict__ cp,
                                           const uint8_t* __restrict__ sp, int64_t gi,
                                           int64_t gpr, Group& g) {
    const int64_t gc = gi < gpr ? gi : gpr - 1;
    const uint2 q = *reinterpret_cast<const uint2*>(cp + gc * 8);
    g.w0 = q.x;
    g.w1 = q.y;
    g.b = sp[gc];
}

// Slab register state of one row (A or W).  kWide: the slab's 32 code bytes
// as two 16-byte words (groups 0-1, 2-3) and the 4 scale bytes as one word,
// which needs 16-byte aligned code rows and K a multiple of 64; otherwise
// one 8-byte word and one byte per group, clamped into the row.
template <bool kWide>
struct RowSlab;

template <>
struct RowSlab<true> {
    uint4 c01, c23;
    uint32_t sw;
    uint32_t b[4];  // scale bytes of the slab being decoded
    __device__ __forceinline__ void start_decode() {
        // take the scale bytes out first, so the scale word can be reloaded
        // at once (it then has a whole slab to arrive)
#pragma unroll
        for (int g = 0; g < 4; g++) b[g] = (sw >> (8 * g)) & 0xFFu;
    }
    __device__ __forceinline__ Group group(int g) const {
        const uint4 c = g < 2 ? c01 : c23;
        Group r;
        r.w0 = (g & 1) ? c.z : c.x;
        r.w1 = (g & 1) ? c.w : c.y;
        r.b = b[g];
        return r;
    }
    // reload after group g of the current slab was decoded
    __device__ __forceinline__ void refill(const uint8_t* __restrict__ cp,
                                           const uint8_t* __restrict__ sp, int64_t slab, int g,
                                           int64_t gpr) {
        (void)gpr;
        if (g == 0) sw = *reinterpret_cast<const uint32_t*>(sp + slab * 4);
        if (g == 1) c01 = reinterpret_cast<const uint4*>(cp + slab * 32)[0];
        if (g == 3) c23 = reinterpret_cast<const uint4*>(cp + slab * 32)[1];
    }
    __device__ __forceinline__ void load_all(const uint8_t* __restrict__ cp,
                                             const uint8_t* __restrict__ sp, int64_t slab,
                                             int64_t gpr) {
        refill(cp, sp, slab, 0, gpr);
        refill(cp, sp, slab, 1, gpr);
        refill(cp, sp, slab, 3, gpr);
    }
};

template <>
struct RowSlab<false> {
    Group gr[4];
    __device__ __forceinline__ void start_decode() {}
    __device__ __forceinline__ Group group(int g) const { return gr[g]; }
    __device__ __forceinline__ void refill(const uint8_t* __restrict__ cp,
                                           const uint8_t* __restrict__ sp, int64_t slab, int g,
                                           int64_t gpr) {
        load_group(cp, sp, slab * 4 + g, gpr, gr[g]);
    }
    __device__ __forceinline__ void load_all(const uint8_t* __restrict__ cp,
                                             const uint8_t* __restrict__ sp, int64_t slab,
                                             int64_t gpr) {
#pragma unroll
        for (int g = 0; g < 4; g++) refill(cp, sp, slab, g, gpr);
    }
};

template <bool kWide, int WM, int WN>
__global__ void __launch_bounds__(64 * WM * WN)
gemm_kernel(const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
            const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales,
            int64_t M, int64_t N, int64_t K, float* __restrict__ c, int64_t ldc, float out_scale,
            int tiles_m, int tiles_n) {
    using LY = Layout<WM, WN>;
    constexpr int TM = LY::TM, TN = LY::TN, FM = LY::FM, FN = LY::FN;
    constexpr bool kTwo = LY::kTwoRows;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a
    // contiguous run of tiles, walking down M within a column of W tiles so
    // that concurrently running tiles share W rows in their XCD's L2.
    const int total = tiles_m * tiles_n;
    int bid = blockIdx.x;
    if (total % 8 == 0) bid = (bid % 8) * (total / 8) + bid / 8;
    const int tm = bid % tiles_m, tn = bid / tiles_m;
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int64_t gpr = K / 16;

    // Rows this thread loads and decodes (clamped in range; dead rows decode
    // to 0).  Row 0: A row tid (4 waves) or tile row tid of A-then-W (8
    // waves); row 1 (4 waves only): W row tid.
    const bool r0_is_w = !kTwo && tid >= BM;
    const int lr0 = r0_is_w ? tid - BM : tid;
    const int64_t g0row = (r0_is_w ? n0 : m0) + lr0;
    const int64_t lim0 = r0_is_w ? N : M;
    const bool dead0 = g0row >= lim0;
    const int64_t cr0 = dead0 ? lim0 - 1 : g0row;
    const uint8_t* const cp0 = (r0_is_w ? w_codes : a_codes) + cr0 * (K / 2);
    const uint8_t* const sp0 = (r0_is_w ? w_scales : a_scales) + cr0 * gpr;
    const int tile0 = r0_is_w ? TILE_BYTES : 0;  // operand tile of row 0
    const int64_t wrow = n0 + tid;
    const bool dead1 = wrow >= N;
    const int64_t cr1 = dead1 ? N - 1 : wrow;
    const uint8_t* const cp1 = w_codes + cr1 * (K / 2);
    const uint8_t* const sp1 = w_scales + cr1 * gpr;
    const int tile1 = TILE_BYTES;

    float16v acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

    const int nslabs = (int)((K + BK - 1) / BK);
    const int64_t last = nslabs - 1;
    RowSlab<kWide> r0, r1;
    r0.load_all(cp0, sp0, 0, gpr);
    if (kTwo) r1.load_all(cp1, sp1, 0, gpr);
    r0.start_decode();
    if (kTwo) r1.start_decode();
#pragma unroll
    for (int g = 0; g < 4; g++) {
        decode_store(smem + tile0, lr0, g, r0.group(g), dead0 || g >= gpr);
        if (kTwo) decode_store(smem + tile1, tid, g, r1.group(g), dead1 || g >= gpr);
    }
    r0.load_all(cp0, sp0, last < 1 ? last : 1, gpr);
    if (kTwo) r1.load_all(cp1, sp1, last < 1 ? last : 1, gpr);
    __syncthreads();

    // fragment (block i, group kk) of this wave: frag_off(first row, kk, 0) + lane * 16
    const int a_off = frag_off(wm * TM, 0, 0) + lane * 16;
    const int w_off = TILE_BYTES + frag_off(wn * TN, 0, 0) + lane * 16;
    constexpr int FRAG_BLOCK = (BK / 16) * 2 * 32 * 16;  // bytes between 32-row blocks
    constexpr int FRAG_GROUP = 2 * 32 * 16;              // bytes between groups

    // With two waves per SIMD (8 waves; waves w and w+4 share a SIMD) the
    // pair runs in opposite phases inside every slab: one wave issues its
    // MFMAs while its partner decodes, then they swap, so the matrix core
    // and the VALU work at the same time.  With one wave per SIMD the decode
    // is interleaved with the MFMAs instead.
    const bool mfma_first = kTwo || wave < 4;
    for (int s = 0; s < nslabs; s++) {
        const uint8_t* buf = smem + (s & 1) * BUF_BYTES;
        uint8_t* nbuf = smem + ((s + 1) & 1) * BUF_BYTES;
        // registers hold slab s+1 (decoded now) and are refilled with slab
        // s+2, clamped: past the end the loads repeat the last slab and the
        // decodes write a buffer nobody reads again
        const int64_t sl = (int64_t)s + 2 < last ? (int64_t)s + 2 : last;
        const int64_t gdec = (int64_t)(s + 1) * 4;  // first group decoded now
        r0.start_decode();
        if (kTwo) r1.start_decode();
        auto decode_group = [&](int kk) {
            const bool past = gdec + kk >= gpr;  // group of slab s+1 beyond K
            decode_store(nbuf + tile0, lr0, kk, r0.group(kk), dead0 || past);
            if (kTwo) decode_store(nbuf + tile1, tid, kk, r1.group(kk), dead1 || past);
            r0.refill(cp0, sp0, sl, kk, gpr);
            if (kTwo) r1.refill(cp1, sp1, sl, kk, gpr);
        };
        if (!mfma_first) {
#pragma unroll
            for (int kk = 0; kk < BK / 16; kk++) decode_group(kk);
        }
        half8 av[2][FM], bv[2][FN];
#pragma unroll
        for (int i = 0; i < FM; i++)
            av[0][i] = *reinterpret_cast<const half8*>(buf + a_off + i * FRAG_BLOCK);
#pragma unroll
        for (int j = 0; j < FN; j++)
            bv[0][j] = *reinterpret_cast<const half8*>(buf + w_off + j * FRAG_BLOCK);
#pragma unroll
        for (int kk = 0; kk < BK / 16; kk++) {
            const int cur = kk & 1;
            if (kk + 1 < BK / 16) {
#pragma unroll
                for (int i = 0; i < FM; i++)
                    av[cur ^ 1][i] = *reinterpret_cast<const half8*>(
                        buf + a_off + i * FRAG_BLOCK + (kk + 1) * FRAG_GROUP);
#pragma unroll
                for (int j = 0; j < FN; j++)
                    bv[cur ^ 1][j] = *reinterpret_cast<const half8*>(
                        buf + w_off + j * FRAG_BLOCK + (kk + 1) * FRAG_GROUP);
            }
#pragma unroll
            for (int i = 0; i < FM; i++)
#pragma unroll
                for (int j = 0; j < FN; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[cur][i], bv[cur][j],
                                                                       acc[i][j], 0, 0, 0);
            if (kTwo) {
                decode_group(kk);
                // One MFMA (32 cycles in the matrix core), then a handful of
                // VALU/LDS/global instructions.
#pragma unroll
                for (int i = 0; i < FM * FN; i++) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // VALU
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
                    __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // LDS write
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (!kTwo && mfma_first) {
#pragma unroll
            for (int kk = 0; kk < BK / 16; kk++) decode_group(kk);
        }
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


#ifndef IF4_GEMM_WM
#define IF4_GEMM_WM 4
#define IF4_GEMM_WN 2
#endif

template <bool kWide>
hipError_t launch_tile(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* w_codes,
                       const uint8_t* w_scales, int64_t M, int64_t N, int64_t K, float* c,
                       int64_t ldc, float out_scale, int64_t tiles_m, int64_t tiles_n,
                       hipStream_t stream) {
    constexpr int WM = IF4_GEMM_WM, WN = IF4_GEMM_WN;
    const void* fn = (const void*)gemm_kernel<kWide, WM, WN>;
    // LDS above 64 KB must be requested per kernel (idempotent, any device)
    hipError_t err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, SMEM_BYTES);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((gemm_kernel<kWide, WM, WN>), dim3((unsigned)(tiles_m * tiles_n)),
                       dim3(Layout<WM, WN>::kThreads), SMEM_BYTES, stream, a_codes, a_scales,
                       w_codes, w_scales, M, N, K, c, ldc, out_scale, (int)tiles_m, (int)tiles_n);
    return hipGetLastError();
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
    const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    if (tiles_m * tiles_n > 0x7FFFFFFF) return hipErrorInvalidValue;
    // 2^(a_exp + w_exp), exact; |a_exp + w_exp| <= 128 is split in two factors
    const int e = a_exp + w_exp;
    const float out_scale = pow2f(e / 2) * pow2f(e - e / 2);
    // Wide loads need 16-byte aligned code rows and 4-byte aligned scale rows
    // with whole 64-deep slabs.
    const bool wide = K % 64 == 0 && (uintptr_t)a_codes % 16 == 0 &&
                      (uintptr_t)w_codes % 16 == 0 && (uintptr_t)a_scales % 4 == 0 &&
                      (uintptr_t)w_scales % 4 == 0;
    return wide ? launch_tile<true>(a_codes, a_scales, w_codes, w_scales, M, N, K, c, ldc,
                                    out_scale, tiles_m, tiles_n, stream)
                : launch_tile<false>(a_codes, a_scales, w_codes, w_scales, M, N, K, c, ldc,
                                     out_scale, tiles_m, tiles_n, stream);
}

}  // namespace if4
