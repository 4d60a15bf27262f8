// IF4 x IF4 (W4A4) GEMM for gfx950: C[M,N] = A[M,K] * W[N,K]^T, fp32 out.
//
// Both operands arrive packed (4-bit codes + one flagged E4M3 scale byte per
// 16 values along K).  The pages' MAC unit ("MAC Unit: Decoding Two Formats
// from One Sign Bit", podcast companion page) routes each operand group by
// its scale's sign bit to an FP or an INT decode path, with INT4 descaled by
// 6/7 "during multiplication" (gist.science summary, section 2, "Metodo
// 6/7").  Here both operands are decoded to fp16 with the group scale folded
// in, and the waves run v_mfma_f32_32x32x16_f16 (one MFMA K-step = one IF4
// group) with fp32 accumulation.
//
// Decode (decode_half): a code nibble becomes the high byte of an fp16
// number by shifts and masks alone -- FP4 s.e1e0.m -> s.000e1e0.m (the fp16
// value c * 2^-14; e = 0 lands on the fp16 subnormals, which keeps it
// exact), INT4 s.mmm -> s.0000.mmm (|q| * 2^-16).  v_perm_b32 spreads four
// such bytes into two fp16 pairs per instruction, and one packed fp16
// multiply by the group multiplier -- s' * 2^5 for FP4, fl16(6 s' / 7) * 2^7
// for INT4 -- gives every operand as (decoded value) * 2^-9.  FP4 operands
// are exact; an INT4 operand is fl16(|q| * fl16(6 s'/7) * 2^-9), i.e. the
// fp16 rounding of |q| * fl16(6 s'/7), with a 2^-15 absolute floor below
// 2^-5.  The epilogue multiplies by 2^(E_A + E_W + 18).  fp16 subnormals
// pass exactly through v_pk_mul_f16 and the MFMA on gfx950.
//
// Tiling: one 256x256 output tile per workgroup of 4 waves (one per SIMD).
// Wave w owns A rows 64w..64w+63 of the tile and all 256 columns (2 x 8
// MFMA blocks of 32x32, 256 fp32 accumulators per lane).  Because no other
// wave needs those A rows, a wave decodes its A operand straight into MFMA
// registers: lane l holds row l%32 and K-half l/32 of a 16-group, so a lane
// loads 16 bytes of its row's 32-byte K slab and one v_permlane32_swap per
// register pair hands each half-group to the lane that multiplies it.  The W
// tile is shared by all four waves and goes through LDS: each thread decodes
// one W row, 64 K values per slab, into a double-buffered 2 x 32 KB tile
// laid out in MFMA fragment order (a wave reads a 32x16 fragment as one
// contiguous 1 KB ds_read_b128).  While the MFMAs of K-slab s run, every
// wave decodes slab s+1 (its A registers, one W row into the other LDS
// buffer) and refills its load registers with slab s+2.  One barrier per
// slab.  Rows past M or N load their nearest in-range row (those outputs
// are never stored); groups past K (only without whole 64-deep slabs)
// decode with a zero multiplier.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "if4_internal.h"

namespace if4 {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float16v __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kThreads = 256;
constexpr int kGroups = BK / 16;                  // IF4 groups per K slab
constexpr int TILE_BYTES = BN * BK * 2;           // decoded W slab: 32 KB
constexpr int SMEM_BYTES = 2 * TILE_BYTES;        // double-buffered: 64 KB
constexpr int FRAG_GROUP = 2 * 32 * 16;           // bytes between groups of a 32-row block
constexpr int FRAG_BLOCK = kGroups * FRAG_GROUP;  // bytes between 32-row blocks
// Offset of (row R, group g, half h) in the W tile: for each block of 32
// rows, each group and each 8-value half, the 32 rows' 16-byte pieces are
// contiguous.
__device__ __forceinline__ int frag_off(int R, int g, int h) {
    return (R >> 5) * FRAG_BLOCK + g * FRAG_GROUP + h * 512 + (R & 31) * 16;
}

__device__ __forceinline__ uint32_t pk_mul(uint32_t a, uint32_t b) {
    half2v x = __builtin_bit_cast(half2v, a);
    half2v y = __builtin_bit_cast(half2v, b);
    return __builtin_bit_cast(uint32_t, x * y);
}

// Group multiplier (both fp16 halves) and nibble shift from a scale byte.
struct GroupScale {
    uint32_t sig2;
    uint32_t sh;
};

// s' comes from the hardware E4M3 conversion (exact; NaN for 0x7F, which
// then poisons the group's products).  FP4: s' * 2^5 (exact in fp16);
// INT4: fl16(fl32(s' * fl32(6/7))) * 2^7, computed as one fp32 product
// (power-of-two factors do not change the roundings).
__device__ __forceinline__ GroupScale group_scale(uint32_t b, bool zero) {
    const float sp = __builtin_amdgcn_cvt_scalef32_f32_fp8(b & 0x7Fu, 1.0f, 0);
    const bool int4 = (b & 0x80u) != 0;
    float sig = sp * (int4 ? 0.857142866f * 128.0f : 32.0f);
    sig = zero ? 0.0f : sig;
    const uint32_t h16 = __builtin_bit_cast(uint16_t, (_Float16)sig);
    GroupScale s;
    s.sig2 = h16 | (h16 << 16);
    s.sh = int4 ? 0u : 1u;
    return s;
}

// Decode one code word (8 nibbles = half a group, element 2j in the low
// nibble of byte j) into 8 fp16 operands in K order.
__device__ __forceinline__ half8 decode_half(uint32_t w, GroupScale s) {
    const uint32_t he = ((w & 0x07070707u) << s.sh) | ((w << 4) & 0x80808080u);
    const uint32_t ho = (((w >> 4) & 0x07070707u) << s.sh) | (w & 0x80808080u);
    // v_perm: byte j of `he` -> bits 15:8, byte j of `ho` -> bits 31:24, zeros below
    uint4 o;
    o.x = pk_mul(__builtin_amdgcn_perm(ho, he, 0x040C000Cu), s.sig2);
    o.y = pk_mul(__builtin_amdgcn_perm(ho, he, 0x050C010Cu), s.sig2);
    o.z = pk_mul(__builtin_amdgcn_perm(ho, he, 0x060C020Cu), s.sig2);
    o.w = pk_mul(__builtin_amdgcn_perm(ho, he, 0x070C030Cu), s.sig2);
    return __builtin_bit_cast(half8, o);
}

// One group's packed data in registers: 16 nibbles and the scale byte.
struct Group {
    uint32_t w0, w1;
    uint32_t b;
};

__device__ __forceinline__ void decode_store(uint8_t* __restrict__ tile, int R, int gi,
                                             const Group& g, bool zero) {
    const GroupScale s = group_scale(g.b, zero);
    *reinterpret_cast<half8*>(tile + frag_off(R, gi, 0)) = decode_half(g.w0, s);
    *reinterpret_cast<half8*>(tile + frag_off(R, gi, 1)) = decode_half(g.w1, s);
}

// W row state: the raw codes and scales of one 64-deep slab.  The loaded
// values are only consumed one slab later, so nothing may touch them right
// after the load (that would force a wait).  kWide: the slab's 32 code
// bytes as two 16-byte words and the 4 scale bytes as one word (16-byte
// aligned code rows and 4-byte aligned scale rows, K a multiple of 64);
// otherwise one 8-byte word and one byte per group, clamped into the row.
template <bool kWide>
struct WRow;

template <>
struct WRow<true> {
    uint4 c01, c23;
    uint32_t sw;
    uint32_t b[4];  // scale bytes of the slab being decoded
    __device__ __forceinline__ void start_decode() {
        // take the scale bytes out first so the scale word can be reloaded
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
struct WRow<false> {
    Group gr[4];
    __device__ __forceinline__ void start_decode() {}
    __device__ __forceinline__ Group group(int g) const { return gr[g]; }
    __device__ __forceinline__ void refill(const uint8_t* __restrict__ cp,
                                           const uint8_t* __restrict__ sp, int64_t slab, int g,
                                           int64_t gpr) {
        const int64_t gi = slab * 4 + g;
        const int64_t gc = gi < gpr ? gi : gpr - 1;
        const uint2 q = *reinterpret_cast<const uint2*>(cp + gc * 8);
        gr[g].w0 = q.x;
        gr[g].w1 = q.y;
        gr[g].b = sp[gc];
    }
    __device__ __forceinline__ void load_all(const uint8_t* __restrict__ cp,
                                             const uint8_t* __restrict__ sp, int64_t slab,
                                             int64_t gpr) {
#pragma unroll
        for (int g = 0; g < 4; g++) refill(cp, sp, slab, g, gpr);
    }
};

// A state of one lane for its two 32-row blocks: the raw data of one slab,
// and after take() the code word (group g, half lane/32) of each block with
// the group's scale byte.
template <bool kWide>
struct ARows;

template <>
struct ARows<true> {
    // lane l < 32 loads bytes 0-15 (groups 0-1) of its row's slab, lane
    // l + 32 bytes 16-31 (groups 2-3); both load the slab's scale word
    uint4 raw[2];
    uint32_t rsw[2];
    uint32_t word[2][4];
    uint32_t sw[2];
    __device__ __forceinline__ void load(const uint8_t* const* cp, const uint8_t* const* sp,
                                         int64_t slab, int64_t gpr) {
        (void)gpr;
#pragma unroll
        for (int i = 0; i < 2; i++) {
            raw[i] = *reinterpret_cast<const uint4*>(cp[i] + slab * 32);
            rsw[i] = *reinterpret_cast<const uint32_t*>(sp[i] + slab * 4);
        }
    }
    // Lanes l and l + 32 trade halves: permlane32_swap(x, y) exchanges the
    // upper 32 lanes of x with the lower 32 lanes of y, so words (0,1) of
    // the 16 bytes become groups 0 and 2 and words (2,3) groups 1 and 3,
    // each in the half that this lane multiplies.
    __device__ __forceinline__ void take() {
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const auto p = __builtin_amdgcn_permlane32_swap(raw[i].x, raw[i].y, false, false);
            const auto q = __builtin_amdgcn_permlane32_swap(raw[i].z, raw[i].w, false, false);
            word[i][0] = p[0];
            word[i][2] = p[1];
            word[i][1] = q[0];
            word[i][3] = q[1];
            sw[i] = rsw[i];
        }
    }
    __device__ __forceinline__ uint32_t scale(int i, int g) const {
        return (sw[i] >> (8 * g)) & 0xFFu;
    }
};

template <>
struct ARows<false> {
    uint32_t raw[2][4];
    uint32_t rb[2][4];
    uint32_t word[2][4];
    uint32_t sb[2][4];
    int hoff;  // byte offset of this lane's half inside a group (0 or 4)
    __device__ __forceinline__ void load(const uint8_t* const* cp, const uint8_t* const* sp,
                                         int64_t slab, int64_t gpr) {
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const int64_t gi = slab * 4 + g;
                const int64_t gc = gi < gpr ? gi : gpr - 1;
                raw[i][g] = *reinterpret_cast<const uint32_t*>(cp[i] + gc * 8 + hoff);
                rb[i][g] = sp[i][gc];
            }
    }
    __device__ __forceinline__ void take() {
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int g = 0; g < 4; g++) {
                word[i][g] = raw[i][g];
                sb[i][g] = rb[i][g];
            }
    }
    __device__ __forceinline__ uint32_t scale(int i, int g) const { return sb[i][g]; }
};

template <bool kWide>
__global__ void __launch_bounds__(kThreads)
gemm_kernel(const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
            const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales,
            int64_t M, int64_t N, int64_t K, float* __restrict__ c, int64_t ldc, float out_scale,
            int tiles_m, int tiles_n) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a
    // contiguous run of tiles, walking down M within a column of W tiles so
    // that concurrently running tiles share W rows in their XCD's L2.
    const int total = tiles_m * tiles_n;
    int bid = blockIdx.x;
    if (total % 8 == 0) bid = (bid % 8) * (total / 8) + bid / 8;
    const int tm = bid % tiles_m, tn = bid / tiles_m;
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int64_t kb = K / 2, gpr = K / 16;

    // W row decoded by this thread (tile row tid)
    const int64_t wrow = n0 + tid < N ? n0 + tid : N - 1;
    const uint8_t* const wcp = w_codes + wrow * kb;
    const uint8_t* const wsp = w_scales + wrow * gpr;
    // A rows of this lane: row lane%32 of the wave's two 32-row blocks
    const int half = lane >> 5;
    const uint8_t* acp[2];
    const uint8_t* asp[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int64_t r = m0 + 64 * wave + 32 * i + (lane & 31);
        const int64_t rc = r < M ? r : M - 1;
        acp[i] = a_codes + rc * kb + (kWide ? 16 * half : 0);
        asp[i] = a_scales + rc * gpr;
    }

    float16v acc[2][8];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 8; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

    const int nslabs = (int)((K + BK - 1) / BK);
    const int64_t last = nslabs - 1;
    WRow<kWide> wr;
    ARows<kWide> ar;
    if constexpr (!kWide) ar.hoff = 4 * half;

    // prologue: slab 0 decoded (W into buffer 0, A into registers), slab 1 loaded
    wr.load_all(wcp, wsp, 0, gpr);
    ar.load(acp, asp, 0, gpr);
    wr.start_decode();
    ar.take();
    half8 a[2][kGroups];
#pragma unroll
    for (int g = 0; g < kGroups; g++) {
        const bool past = g >= gpr;
        decode_store(smem, tid, g, wr.group(g), past);
#pragma unroll
        for (int i = 0; i < 2; i++)
            a[i][g] = decode_half(ar.word[i][g], group_scale(ar.scale(i, g), past));
    }
    wr.load_all(wcp, wsp, last < 1 ? last : 1, gpr);
    ar.load(acp, asp, last < 1 ? last : 1, gpr);
    __syncthreads();

    const int w_off = lane * 16;  // fragment (block j, group g) at j * FRAG_BLOCK + g * FRAG_GROUP
    for (int s = 0; s < nslabs; s++) {
        const uint8_t* buf = smem + (s & 1) * TILE_BYTES;
        uint8_t* nbuf = smem + ((s + 1) & 1) * TILE_BYTES;
        // registers hold slab s+1 (decoded now) and are refilled with slab
        // s+2, clamped: past the end the loads repeat the last slab and the
        // decodes fill registers and a buffer that nobody reads again
        const int64_t sl = (int64_t)s + 2 < last ? (int64_t)s + 2 : last;
        const int64_t gdec = (int64_t)(s + 1) * kGroups;  // first group decoded now
        wr.start_decode();
        ar.take();
        ar.load(acp, asp, sl, gpr);

        half8 bv[2][8];
#pragma unroll
        for (int j = 0; j < 8; j++)
            bv[0][j] = *reinterpret_cast<const half8*>(buf + w_off + j * FRAG_BLOCK);
#pragma unroll
        for (int kk = 0; kk < kGroups; kk++) {
            const int cur = kk & 1;
            if (kk + 1 < kGroups) {
#pragma unroll
                for (int j = 0; j < 8; j++)
                    bv[cur ^ 1][j] = *reinterpret_cast<const half8*>(
                        buf + w_off + j * FRAG_BLOCK + (kk + 1) * FRAG_GROUP);
            }
#pragma unroll
            for (int j = 0; j < 8; j++)
#pragma unroll
                for (int i = 0; i < 2; i++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i][kk], bv[cur][j],
                                                                       acc[i][j], 0, 0, 0);
            // next slab, group kk: this wave's A operands and one W row
            const bool past = gdec + kk >= gpr;
#pragma unroll
            for (int i = 0; i < 2; i++)
                a[i][kk] = decode_half(ar.word[i][kk], group_scale(ar.scale(i, kk), past));
            decode_store(nbuf, tid, kk, wr.group(kk), past);
            wr.refill(wcp, wsp, sl, kk, gpr);
            // one MFMA (32 cycles in the matrix core), then a few VALU, LDS
            // and global instructions
#pragma unroll
            for (int m = 0; m < 16; m++) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // VALU
                if (m < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
                if (m == 4 || m == 12) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
                if (m == 6) __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);  // global load
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
    }

    // epilogue: lane holds column lane%32 of each 32x32 block, rows
    // 8*(r/4) + 4*(lane/32) + r%4 for accumulator register r
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const int64_t col = n0 + j * 32 + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int64_t row = m0 + 64 * wave + 32 * i + 8 * (r >> 2) + 4 * half + (r & 3);
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

template <bool kWide>
hipError_t launch_tile(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* w_codes,
                       const uint8_t* w_scales, int64_t M, int64_t N, int64_t K, float* c,
                       int64_t ldc, float out_scale, int64_t tiles_m, int64_t tiles_n,
                       hipStream_t stream) {
    // dynamic LDS limit for this kernel (idempotent, any device)
    hipError_t err = hipFuncSetAttribute((const void*)gemm_kernel<kWide>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, SMEM_BYTES);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(gemm_kernel<kWide>, dim3((unsigned)(tiles_m * tiles_n)), dim3(kThreads),
                       SMEM_BYTES, stream, a_codes, a_scales, w_codes, w_scales, M, N, K, c, ldc,
                       out_scale, (int)tiles_m, (int)tiles_n);
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
    // 2^(a_exp + w_exp + 18) (each decoded operand carries 2^-9), exact; the
    // exponent lies in [-110, 146] and is split into two factors
    const int e = a_exp + w_exp + 18;
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
