// IF4 x IF4 (W4A4) GEMM for gfx950: C[M,N] = A[M,K] * W[N,K]^T, fp32 out.
//
// (design notes: see the comment above gemm_kernel)
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "if4_internal.h"

namespace if4 {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float16v __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kThreads = 256;                     // 4 waves, one per SIMD
constexpr int kGroups = BK / 16;                  // IF4 groups per K slab
constexpr int kWin = 4;                           // slabs per scale window (16 scale bytes)
constexpr int kBandM = 4;                         // M-tiles per band of the tile order
constexpr int TILE_BYTES = BN * BK * 2;           // decoded W slab: 32 KB
constexpr int LUT_OFF = 2 * TILE_BYTES;           // double-buffered W tile: 64 KB, then
constexpr int LUT_ENTRIES = 257;                  // the scale table: 256 bytes + "zero"
constexpr int SMEM_BYTES = LUT_OFF + LUT_ENTRIES * 8 + 8;
constexpr int FRAG_STEP = 2 * 32 * 16;            // bytes between MFMA steps of a 32-row block
constexpr int FRAG_BLOCK = kGroups * FRAG_STEP;   // bytes between 32-row blocks
// MFMA step t (0..3) of a K slab multiplies, in lane half h (lanes 32h ..
// 32h+31), the 8 values of word (group 2h + t/2, half t%2) of each row --
// any assignment of the slab's 64 K indices to MFMA positions gives the same
// sums as long as A and W use the same one, and this one lets an A lane use
// the 16 bytes it loads (groups 2h, 2h+1) without trading data with other
// lanes.  W tile offset of (row R, group g, half hf): for each block of 32
// rows and each step, the fragment's 64 16-byte pieces are contiguous, so a
// wave reads a fragment as one 1 KB ds_read_b128.
__device__ __forceinline__ int frag_off(int R, int g, int hf) {
    return (R >> 5) * FRAG_BLOCK + (2 * (g & 1) + hf) * FRAG_STEP + (g >> 1) * 512 +
           (R & 31) * 16;
}

// Workgroup barrier that orders LDS only.  __syncthreads() also orders
// global memory, which makes every wave wait for its outstanding global
// loads -- the prefetches of the next slabs -- at each barrier.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
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
__device__ __forceinline__ GroupScale group_scale(uint32_t b) {
    const float sp = __builtin_amdgcn_cvt_scalef32_f32_fp8(b & 0x7Fu, 1.0f, 0);
    const bool int4 = (b & 0x80u) != 0;
    const float sig = sp * (int4 ? 0.857142866f * 128.0f : 32.0f);
    const uint32_t h16 = __builtin_bit_cast(uint16_t, (_Float16)sig);
    GroupScale s;
    s.sig2 = h16 | (h16 << 16);
    s.sh = int4 ? 0u : 1u;
    return s;
}

// Every workgroup tabulates group_scale for the 256 scale bytes, plus entry
// 256 = zero multiplier (groups past K), in LDS; a lookup is one
// ds_read_b64 instead of a dozen VALU instructions.
constexpr uint32_t kZeroScale = 256;
__device__ __forceinline__ void fill_scale_table(uint8_t* smem, int tid) {
    uint2* lut = reinterpret_cast<uint2*>(smem + LUT_OFF);
    const GroupScale g = group_scale((uint32_t)tid);
    lut[tid] = make_uint2(g.sig2, g.sh);
    if (tid == 0) lut[kZeroScale] = make_uint2(0u, 1u);
}
__device__ __forceinline__ GroupScale lookup_scale(const uint8_t* smem, uint32_t idx) {
    const uint2 v = reinterpret_cast<const uint2*>(smem + LUT_OFF)[idx];
    GroupScale s;
    s.sig2 = v.x;
    s.sh = v.y;
    return s;
}

// Decode the two code words of one group (w0: elements 0-7, w1: elements
// 8-15; element 2j in the low nibble of byte j) into 16 fp16 operands in K
// order.  Per word, two bytes hold the fp16 high bytes of its even and odd
// elements: he = [sign | magnitude << sh] of the low nibbles, ho the same
// for the high nibbles.  The magnitudes are shifted as one 64-bit word per
// group (the shift moves no bit across a nibble: bit 3 of every nibble is
// cleared first), and each byte is assembled by one bit-field insert under
// the mask 0x0F0F0F0F: the low half from the shifted magnitudes, the high
// half from the sign bits (moved up by 4 for the even elements; the bits a
// 64-bit shift carries across the word boundary land in masked-off
// positions).  27 VALU instructions per group.
// m ? a : b, bit by bit: one v_bitop3_b32 (truth table over (a, b, m)).
__device__ __forceinline__ uint32_t bit_select(uint32_t a, uint32_t b, uint32_t m) {
    return __builtin_amdgcn_bitop3_b32(a, b, m, 0xE4);
}
// 64-bit shifts by 4 as single instructions (full rate on gfx950).  The
// amount comes in as `four`, a value the compiler cannot fold: a constant
// amount makes it split each shift into two 32-bit operations, and writing the
// instruction as inline asm instead costs a hazard s_nop after every one.
__device__ __forceinline__ uint64_t shr64_by4(uint64_t x, uint32_t four) { return x >> four; }
__device__ __forceinline__ uint64_t shl64_by4(uint64_t x, uint32_t four) { return x << four; }
__device__ __forceinline__ void decode_group(uint32_t w0, uint32_t w1, GroupScale s, half8& o0,
                                             half8& o1, uint32_t four) {
    constexpr uint32_t kLo = 0x0F0F0F0Fu;  // low nibble of every byte
    const uint32_t m0 = w0 & 0x77777777u, m1 = w1 & 0x77777777u;
    const uint64_t ms = ((uint64_t)m1 << 32 | m0) << s.sh;
    const uint64_t mr = shr64_by4(ms, four);
    const uint32_t g0 = w0 ^ m0, g1 = w1 ^ m1;  // sign bits (bits 3 and 7 of each byte)
    const uint64_t g4 = shl64_by4((uint64_t)g1 << 32 | g0, four);
    const uint32_t he0 = bit_select((uint32_t)ms, (uint32_t)g4, kLo);
    const uint32_t he1 = bit_select((uint32_t)(ms >> 32), (uint32_t)(g4 >> 32), kLo);
    const uint32_t ho0 = bit_select((uint32_t)mr, g0, kLo);
    const uint32_t ho1 = bit_select((uint32_t)(mr >> 32), g1, kLo);
    // v_perm: byte j of he -> bits 15:8, byte j of ho -> bits 31:24, zeros below
    uint4 r0, r1;
    r0.x = pk_mul(__builtin_amdgcn_perm(ho0, he0, 0x040C000Cu), s.sig2);
    r0.y = pk_mul(__builtin_amdgcn_perm(ho0, he0, 0x050C010Cu), s.sig2);
    r0.z = pk_mul(__builtin_amdgcn_perm(ho0, he0, 0x060C020Cu), s.sig2);
    r0.w = pk_mul(__builtin_amdgcn_perm(ho0, he0, 0x070C030Cu), s.sig2);
    r1.x = pk_mul(__builtin_amdgcn_perm(ho1, he1, 0x040C000Cu), s.sig2);
    r1.y = pk_mul(__builtin_amdgcn_perm(ho1, he1, 0x050C010Cu), s.sig2);
    r1.z = pk_mul(__builtin_amdgcn_perm(ho1, he1, 0x060C020Cu), s.sig2);
    r1.w = pk_mul(__builtin_amdgcn_perm(ho1, he1, 0x070C030Cu), s.sig2);
    o0 = __builtin_bit_cast(half8, r0);
    o1 = __builtin_bit_cast(half8, r1);
}

// ---------------------------------------------------------------------------
// Operand fetch.  The vector memory path costs about one cycle per distinct
// cache line an instruction touches, so loads are shaped to touch few lines:
// the two lanes l and l+32 load the two 16-byte halves of one row's 32-byte
// slab (A and W alike, 32 lines per instruction), and scale bytes are
// fetched 16 at a time, four slabs' worth per row.
//
// kWide: 16-byte aligned code and scale rows, K a multiple of 256 (whole
// scale windows).  The wide path reads through buffer resources based at
// the tile's first row: each lane's row offset is fixed (rows past M or N
// take the last row's; those outputs are never stored) and the slab's
// offset is one scalar register, clamped to the last slab on the scalar
// unit, so a fetch costs no vector address arithmetic and every access stays
// inside its operand.  Otherwise every word and byte is fetched on its own,
// clamped into the row, and groups past K decode with a zero multiplier.

// Word 3 of a buffer resource for plain byte-addressed dword loads on gfx9
// class chips (no format conversion, no swizzle).
constexpr int kRawBufferFlags = 0x00020000;
// cache-policy operand of a buffer store: non-temporal (the nt bit)
constexpr int kNonTemporal = 2;

struct Operand {
    __amdgpu_buffer_rsrc_t codes, scales;
    uint32_t code_off[2], scale_off[2];  // this lane's two rows
};

// Codes of one slab for one lane: A blocks i = 0, 1 (row lane%32 of each,
// groups 2h, 2h+1 with h = lane/32) and W rows k = 0, 1 (groups 2q, 2q+1
// with q = lane/32).
template <bool kWide>
struct SlabCodes;

template <>
struct SlabCodes<true> {
    uint4 a[2], w[2];
    __device__ __forceinline__ void load(const Operand& A, const Operand& W, int64_t slab) {
        const int so = (int)slab * 32;
#pragma unroll
        for (int i = 0; i < 2; i++)
            a[i] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(A.codes, A.code_off[i], so, 0));
#pragma unroll
        for (int k = 0; k < 2; k++)
            w[k] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(W.codes, W.code_off[k], so, 0));
    }
    // A block i, word u = 2 * (group - 2h) + half
    __device__ __forceinline__ uint32_t aword(int i, int u) const {
        return u == 0 ? a[i].x : u == 1 ? a[i].y : u == 2 ? a[i].z : a[i].w;
    }
    // W row k, word u = 2 * (group - 2q) + half
    __device__ __forceinline__ uint32_t wword(int k, int u) const {
        return u == 0 ? w[k].x : u == 1 ? w[k].y : u == 2 ? w[k].z : w[k].w;
    }
};

template <>
struct SlabCodes<false> {
    uint32_t a[2][4], w[2][4];
    uint32_t ab[2][2], wb[2][2];  // scale bytes per row and group
    // acp/asp, wcp/wsp: code and scale rows of this lane (clamped into the
    // operand); gpr: groups per row
    __device__ __forceinline__ void load(const uint8_t* const* acp, const uint8_t* const* asp,
                                         const uint8_t* const* wcp, const uint8_t* const* wsp,
                                         int64_t slab, int h, int64_t gpr) {
#pragma unroll
        for (int k = 0; k < 2; k++)
#pragma unroll
            for (int gg = 0; gg < 2; gg++) {
                const int64_t g = slab * kGroups + 2 * h + gg;
                const int64_t gc = g < gpr ? g : gpr - 1;
                const uint2 va = *reinterpret_cast<const uint2*>(acp[k] + gc * 8);
                a[k][2 * gg] = va.x;
                a[k][2 * gg + 1] = va.y;
                ab[k][gg] = asp[k][gc];
                const uint2 vw = *reinterpret_cast<const uint2*>(wcp[k] + gc * 8);
                w[k][2 * gg] = vw.x;
                w[k][2 * gg + 1] = vw.y;
                wb[k][gg] = wsp[k][gc];
            }
    }
    __device__ __forceinline__ uint32_t aword(int i, int u) const { return a[i][u]; }
    __device__ __forceinline__ uint32_t wword(int k, int u) const { return w[k][u]; }
};

// Scale bytes of one 4-slab window (wide path): 16 bytes per A block row and
// per W row; word u holds slab u's four groups.
struct WinScales {
    uint4 a[2], w[2];
    __device__ __forceinline__ void load(const Operand& A, const Operand& W, int64_t win) {
        const int so = (int)win * 16;
#pragma unroll
        for (int i = 0; i < 2; i++)
            a[i] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(A.scales, A.scale_off[i], so, 0));
#pragma unroll
        for (int k = 0; k < 2; k++)
            w[k] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(W.scales, W.scale_off[k], so, 0));
    }
};

__device__ __forceinline__ uint32_t word_of(const uint4& v, int u) {
    return u == 0 ? v.x : u == 1 ? v.y : u == 2 ? v.z : v.w;
}

// IF4 x IF4 GEMM kernel.
//
// Decode (decode_group): a code nibble becomes the high byte of an fp16
// number by shifts and masks alone -- FP4 s.e1e0.m -> s.000e1e0.m (the fp16
// value c * 2^-14; e = 0 lands on the fp16 subnormals, which keeps it
// exact), INT4 s.mmm -> s.0000.mmm (|q| * 2^-16).  v_perm_b32 spreads four
// such bytes into two fp16 pairs per instruction, and one packed fp16
// multiply by the group multiplier -- s' * 2^5 for FP4, fl16(6 s' / 7) * 2^7
// for INT4, looked up in a per-workgroup LDS table -- gives every operand as
// (decoded value) * 2^-9.  FP4 operands are exact; an INT4 operand is
// fl16(|q| * fl16(6 s'/7) * 2^-9), i.e. the fp16 rounding of
// |q| * fl16(6 s'/7) with a 2^-15 absolute floor below 2^-5.  The epilogue
// multiplies by 2^(E_A + E_W + 18).  fp16 subnormals pass exactly through
// v_pk_mul_f16 and the MFMA on gfx950.  The scale's sign bit picks the
// format per group (the pages' MAC unit: "MAC Unit: Decoding Two Formats
// from One Sign Bit", podcast companion page; the 6/7 factor: gist.science
// summary, section 2).
//
// Tiling: one 256x256 output tile per workgroup of 4 waves (one per SIMD);
// wave w owns A rows 64w..64w+63 of the tile and all 256 columns (2 x 8
// blocks of v_mfma_f32_32x32x16_f16, one MFMA K-step = one IF4 group,
// 256 fp32 accumulators per lane).  No other wave needs those A rows, so a
// wave decodes its A operand straight into MFMA registers: lane l holds row
// l%32 and K-half l/32 of a 16-deep step.  MFMA step t (0..3) of a 64-deep K
// slab multiplies, in lane half h, the 8 values of word (group 2h + t/2,
// half t%2) of each row -- any assignment of the slab's 64 K indices to
// MFMA positions gives the same sums as long as A and W use the same one,
// and this one lets an A lane use the 16 bytes it loads as they are.  The W
// tile is shared by the four waves and goes through LDS: each thread decodes
// two groups of two W rows per slab into a double-buffered 2 x 32 KB tile
// in MFMA fragment order (frag_off), which a wave reads as contiguous 1 KB
// ds_read_b128s (its stores: 64 lanes on 1 KB of consecutive 16-byte
// pieces, no bank conflicts).
//
// Pipeline: while the MFMAs of K slab s run, each wave decodes slab s+1
// (its A registers, its W share into the other LDS buffer) and fetches the
// codes of slab s+2 into the register set that slab s used; scales arrive a
// window ahead.  The slab loop is unrolled by the 4-slab window so that all
// register sets are fixed and no loaded value is copied (a copy would wait
// for its load).  One LDS-only barrier per slab.  Each wave numbers the W
// blocks in its own order, its own two (the ones it decodes) first: their
// first-step fragments for the next slab are read before the barrier, the
// other six right after it, before any MFMA is issued, and step 0 opens with
// the four MFMAs on the own blocks while those six arrive.
// Within a slab, each MFMA step runs four sub-blocks of four MFMAs: (A block
// 0, W blocks 0..3), (1, 0..3), (0, 4..7), (1, 4..7) -- in step 0 the W
// blocks go in pairs, (0, 0..1) (1, 0..1), (0, 2..3) (1, 2..3), ...; the eight W fragments
// of the next step are read into a second register set at the start of the
// step, a whole step before their use.  Every step decodes two groups: one
// of W (row t/2, group 2q + t%2 of the next slab, stored in sub-blocks 1
// and 2), and one of A, as soon as both of its operand registers are free --
// A block 1's words 2-3 of the running slab in step 0 (kept across the
// barrier) and words 0-1 of the next slab in step 2 (sub-block 0, after
// their last use in steps 0 and 1), A block 0's words 0-1 and 2-3 of the
// next slab in steps 1 and 3 (sub-block 3, after their last use).  The
// scale-table lookups of a step's decodes are issued at the start of the step
// before (LDS operations complete in order, so a lookup issued after the
// fragment reads would make its consumer wait for them too).
template <bool kWide>
__global__ void __launch_bounds__(kThreads)
gemm_kernel(const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
            const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales,
            int64_t M, int64_t N, int64_t K, float* __restrict__ c, int64_t ldc, int out_exp,
            int tiles_m, int tiles_n) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a
    // contiguous run of tiles.  The run is ordered in bands of kBandM M-tiles:
    // down a band, then across N, so that the 32 tiles an XCD runs at once
    // (one per CU, in step along K) cover 4 x 8 tiles and share their A and
    // W rows in the XCD's L2 -- 3072 distinct rows instead of the 8448 of a
    // whole column of M-tiles.
    const int total = tiles_m * tiles_n;
    int bid = blockIdx.x;
    if (total % 8 == 0) bid = (bid % 8) * (total / 8) + bid / 8;
    const int band = bid / (kBandM * tiles_n);
    const int first_m = band * kBandM;
    const int band_m = tiles_m - first_m < kBandM ? tiles_m - first_m : kBandM;
    const int in_band = bid - band * kBandM * tiles_n;
    const int tm = first_m + in_band % band_m, tn = in_band / band_m;
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int64_t kb = K / 2, gpr = K / 16;
    const uint32_t four = 4u + (uint32_t)((uint64_t)K >> 63);  // 4 (K > 0), not foldable

    // rows of this lane: A rows 64w + 32i + lane%32 of the tile (i = 0, 1),
    // W rows 64w + 32k + lane%32 (k = 0, 1); K-half h = q = lane/32
    const int h = lane >> 5, hs = 16 * h;
    const int q = h, qs = hs;
    const int rl = lane & 31;
    int wr_row[2];
#pragma unroll
    for (int k = 0; k < 2; k++) wr_row[k] = 64 * wave + 32 * k + rl;

    Operand opA, opW;
    const uint8_t* acp[2];
    const uint8_t* asp[2];
    const uint8_t* wcp[2];
    const uint8_t* wsp[2];
    if constexpr (kWide) {
        // resources based at the tile's first row, sized to the tile's rows
        // that exist (offsets fit 31 bits: 256 rows of K/2 bytes, checked on
        // launch)
        const int64_t arows = M - m0 < BM ? M - m0 : BM, wrows = N - n0 < BN ? N - n0 : BN;
        opA.codes = __builtin_amdgcn_make_buffer_rsrc((void*)(a_codes + m0 * kb), 0,
                                                       (int)(arows * kb), kRawBufferFlags);
        opA.scales = __builtin_amdgcn_make_buffer_rsrc((void*)(a_scales + m0 * gpr), 0,
                                                        (int)(arows * gpr), kRawBufferFlags);
        opW.codes = __builtin_amdgcn_make_buffer_rsrc((void*)(w_codes + n0 * kb), 0,
                                                       (int)(wrows * kb), kRawBufferFlags);
        opW.scales = __builtin_amdgcn_make_buffer_rsrc((void*)(w_scales + n0 * gpr), 0,
                                                        (int)(wrows * gpr), kRawBufferFlags);
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int ra = 64 * wave + 32 * i + rl, rw = wr_row[i];
            const uint32_t rac = (uint32_t)(ra < arows ? ra : arows - 1);
            const uint32_t rwc = (uint32_t)(rw < wrows ? rw : wrows - 1);
            opA.code_off[i] = rac * (uint32_t)kb + 16 * h;
            opA.scale_off[i] = rac * (uint32_t)gpr;
            opW.code_off[i] = rwc * (uint32_t)kb + 16 * q;
            opW.scale_off[i] = rwc * (uint32_t)gpr;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int64_t r = m0 + 64 * wave + 32 * i + rl;
            const int64_t rc = r < M ? r : M - 1;
            acp[i] = a_codes + rc * kb;
            asp[i] = a_scales + rc * gpr;
            const int64_t rw = n0 + wr_row[i];
            const int64_t rwc = rw < N ? rw : N - 1;
            wcp[i] = w_codes + rwc * kb;
            wsp[i] = w_scales + rwc * gpr;
        }
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
    const int64_t nwin = (nslabs + kWin - 1) / kWin;

    fill_scale_table(smem, tid);
    lds_barrier();

    // Scale of A block i / W row k, group 2h + g / 2q + g, in slab `slab` =
    // window slot u of a window's scales (wide) or from the slab's own bytes;
    // groups past K exist only without whole slabs.
    auto a_scale = [&](const SlabCodes<kWide>& x, const WinScales& win, int u, int64_t slab,
                       int i, int g) {
        uint32_t b;
        if constexpr (kWide) {
            b = (word_of(win.a[i], u) >> (hs + 8 * g)) & 0xFFu;
        } else {
            const bool past = slab * kGroups + 2 * h + g >= gpr;
            b = past ? kZeroScale : x.ab[i][g];
        }
        return lookup_scale(smem, b);
    };
    auto w_scale = [&](const SlabCodes<kWide>& x, const WinScales& win, int u, int64_t slab,
                       int k, int g) {
        uint32_t b;
        if constexpr (kWide) {
            b = (word_of(win.w[k], u) >> (qs + 8 * g)) & 0xFFu;
        } else {
            const bool past = slab * kGroups + 2 * q + g >= gpr;
            b = past ? kZeroScale : x.wb[k][g];
        }
        return lookup_scale(smem, b);
    };
    // slabs past the end (the prefetches of the last two slabs) re-read the
    // last slab into registers that are never decoded for use
    auto load_codes = [&](SlabCodes<kWide>& x, int64_t slab) {
        const int64_t sc = slab < last ? slab : last;
        if constexpr (kWide)
            x.load(opA, opW, sc);
        else
            x.load(acp, asp, wcp, wsp, sc, h, gpr);
    };
    // A block i, group 2h + g of codes x into a[i][2g], a[i][2g + 1]
    half8 a[2][kGroups];  // decoded A operands [block][MFMA step] of the running slab
    auto a_decode = [&](uint32_t w0, uint32_t w1, GroupScale sc, int i, int g) {
        decode_group(w0, w1, sc, a[i][2 * g], a[i][2 * g + 1], four);
    };
    // W row k, group 2q + g of codes x: both halves decoded; half 0 stored
    // now, half 1 returned for a later store
    auto w_decode_store0 = [&](const SlabCodes<kWide>& x, GroupScale sc, int k, int g,
                               uint8_t* tile) {
        half8 o0, o1;
        decode_group(x.wword(k, 2 * g), x.wword(k, 2 * g + 1), sc, o0, o1, four);
        *reinterpret_cast<half8*>(tile + frag_off(wr_row[k], 2 * q + g, 0)) = o0;
        return o1;
    };
    auto w_store1 = [&](half8 o1, int k, int g, uint8_t* tile) {
        *reinterpret_cast<half8*>(tile + frag_off(wr_row[k], 2 * q + g, 1)) = o1;
    };

    // register sets: raw[p] holds the codes of a slab of parity p
    SlabCodes<kWide> raw[2];
    WinScales win[2];  // scale windows: the running one and the next
    uint32_t k12, k13;  // A block 1, words 2 and 3 of the running slab
    // Scale-table lookups run one MFMA step ahead of the decodes that use
    // them: issued before that step's fragment prefetches, a lookup can be
    // waited for (LDS operations complete in order) without waiting for the
    // prefetches too.  la / lw: the coming step's A and W groups.
    GroupScale la, lw;

    // prologue: slab 0 decoded (W into buffer 0; A into registers, except
    // block 1's words 2-3, decoded in slab 0's step 0), slab 1 fetched
    if constexpr (kWide) {
        win[0].load(opA, opW, 0);
        win[1].load(opA, opW, nwin > 1 ? 1 : 0);
    }
    load_codes(raw[0], 0);
    load_codes(raw[1], 1);
#pragma unroll
    for (int g = 0; g < 2; g++) {
        a_decode(raw[0].aword(0, 2 * g), raw[0].aword(0, 2 * g + 1),
                 a_scale(raw[0], win[0], 0, 0, 0, g), 0, g);
#pragma unroll
        for (int k = 0; k < 2; k++) {
            const half8 o1 = w_decode_store0(raw[0], w_scale(raw[0], win[0], 0, 0, k, g), k, g,
                                             smem);
            w_store1(o1, k, g, smem);
        }
    }
    a_decode(raw[0].aword(1, 0), raw[0].aword(1, 1), a_scale(raw[0], win[0], 0, 0, 1, 0), 1, 0);
    k12 = raw[0].aword(1, 2);
    k13 = raw[0].aword(1, 3);
    // lookups for step 0 of slab 0: A block 1 group 2h+1 of slab 0, W row 0
    // group 2q of slab 1
    la = a_scale(raw[0], win[0], 0, 0, 1, 1);
    lw = w_scale(raw[1], win[0], 1, 1, 0, 0);
    lds_barrier();

    // Block order per wave: the wave's logical W block j = 2m + b is the tile's
    // block 2 (m ^ wave) + b, so that its first two blocks are the two it
    // decodes itself (tile rows 64 wave .. 64 wave + 63).  Those it can read
    // for the next slab before the barrier (a wave's own LDS writes and
    // reads complete in order), and step 0 of each slab starts with the four
    // MFMAs on them while the other six fragments arrive.
    // fragment (logical block 2m + b, step t) at fb[m] + b * FRAG_BLOCK + t * FRAG_STEP
    int fb[4];
#pragma unroll
    for (int m = 0; m < 4; m++) fb[m] = lane * 16 + 2 * (m ^ wave) * FRAG_BLOCK;
    auto frag = [&](const uint8_t* b, int j, int t) {
        return *reinterpret_cast<const half8*>(b + fb[j >> 1] + (j & 1) * FRAG_BLOCK +
                                               t * FRAG_STEP);
    };
    half8 bv[2][8];  // fragments of even / odd steps
    // slab 0's first two (own) fragments
    bv[0][0] = frag(smem, 0, 0);
    bv[0][1] = frag(smem, 1, 0);

    // One slab s = s0 + U (s0 a multiple of 4): MFMAs of slab s from buffer
    // U%2 while slab s+1 (register set (U+1)%2) is decoded into the other
    // buffer and slab s+2 is fetched into set U%2.
    auto slab_step = [&](auto UC, int s0, const WinScales& wcur, const WinScales& wnxt) {
        constexpr int U = decltype(UC)::value;
        constexpr int P = U & 1, Q = P ^ 1;
        const int s = s0 + U;
        const uint8_t* buf = smem + P * TILE_BYTES;
        uint8_t* nbuf = smem + Q * TILE_BYTES;
        const int64_t sn = (int64_t)s + 1;
        // scales of slab s+1: slot U+1 of this window, or slot 0 of the next;
        // of slab s+2 (looked up in the last step): slot U+2 of either
        const WinScales& sw_win = U + 1 < kWin ? wcur : wnxt;
        constexpr int US = (U + 1) % kWin;
        const WinScales& sw2_win = U + 2 < kWin ? wcur : wnxt;
        constexpr int US2 = (U + 2) % kWin;
        const SlabCodes<kWide>& x = raw[Q];

        // step 0's other six fragments (logical blocks 2..7) before any MFMA;
        // blocks 0 and 1, the wave's own, were read before the barrier
#pragma unroll
        for (int j = 2; j < 8; j++) bv[0][j] = frag(buf, j, 0);
        load_codes(raw[P], (int64_t)s + 2);
#pragma unroll
        for (int t = 0; t < kGroups; t++) {
            const int k = t >> 1, gg = t & 1;
            const GroupScale sa = la, sw = lw;
            // lookups for step t+1's decodes (the schedule above): its A
            // group and its W group
            if (t == 0) {
                la = a_scale(x, sw_win, US, sn, 0, 0);
                lw = w_scale(x, sw_win, US, sn, 0, 1);
            } else if (t == 1) {
                la = a_scale(x, sw_win, US, sn, 1, 0);
                lw = w_scale(x, sw_win, US, sn, 1, 0);
            } else if (t == 2) {
                la = a_scale(x, sw_win, US, sn, 0, 1);
                lw = w_scale(x, sw_win, US, sn, 1, 1);
            } else {
                // step 0 of the next slab: A block 1 group 2h+1 of slab s+1,
                // W row 0 group 2q of slab s+2
                la = a_scale(x, sw_win, US, sn, 1, 1);
                lw = w_scale(raw[P], sw2_win, US2, sn + 1, 0, 0);
            }
            // the next step's eight fragments, a whole step ahead
            if (t + 1 < kGroups) {
#pragma unroll
                for (int j = 0; j < 8; j++)
                    bv[(t + 1) & 1][j] = frag(buf, j, t + 1);
            }
            half8 w1;
            // sub-blocks: (A block 0, W 0..3), (1, 0..3), (0, 4..7), (1, 4..7);
            // in step 0, W blocks in pairs, (0, 0..1) (1, 0..1), (0, 2..3)
            // (1, 2..3), ..., so that the four MFMAs on the wave's own blocks
            // come first
#pragma unroll
            for (int sb = 0; sb < 4; sb++) {
#pragma unroll
                for (int jj = 0; jj < 4; jj++) {
                    const int i = t == 0 ? (jj >> 1) : (sb & 1);  // A block
                    const int j = t == 0 ? 2 * sb + (jj & 1) : 4 * (sb >> 1) + jj;
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i][t], bv[t & 1][j],
                                                                       acc[i][j], 0, 0, 0);
                }
                if (sb == 0 && t == 0) {
                    a_decode(k12, k13, sa, 1, 1);  // block 1 words 2-3 of slab s
                } else if (sb == 0 && t == 2) {
                    a_decode(x.aword(1, 0), x.aword(1, 1), sa, 1, 0);  // slab s+1
                } else if (sb == 1) {
                    w1 = w_decode_store0(x, sw, k, gg, nbuf);
                } else if (sb == 2) {
                    w_store1(w1, k, gg, nbuf);
                    if (t == kGroups - 1) {
                        // the next slab's first two fragments: this wave's
                        // own blocks, all written by now (in program order)
                        bv[0][0] = frag(nbuf, 0, 0);
                        bv[0][1] = frag(nbuf, 1, 0);
                    }
                } else if (sb == 3 && t == 1) {
                    a_decode(x.aword(0, 0), x.aword(0, 1), sa, 0, 0);  // slab s+1
                } else if (sb == 3 && t == 3) {
                    a_decode(x.aword(0, 2), x.aword(0, 3), sa, 0, 1);  // slab s+1
                }
                // interleave: each MFMA followed by four VALU and up to two
                // LDS reads; no fence between sub-blocks, so the scheduler
                // may pull a later sub-block's independent work forward
#pragma unroll
                for (int m = 0; m < 4; m++) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS read
                    if (m == 2) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // LDS write
                    if (m == 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load
                }
            }
        }
        k12 = x.aword(1, 2);
        k13 = x.aword(1, 3);
        lds_barrier();
    };

    // One 4-slab window.  The scales of the window after next are fetched
    // at its start, so that moving them into place at its end does not wait.
    for (int s0 = 0; s0 < nslabs; s0 += kWin) {
        WinScales nn;
        if constexpr (kWide) {
            const int64_t nw = (int64_t)s0 / kWin + 2;
            nn.load(opA, opW, nw < nwin ? nw : nwin - 1);
        }
        slab_step(std::integral_constant<int, 0>{}, s0, win[0], win[1]);
        if (kWide || s0 + 1 < nslabs) slab_step(std::integral_constant<int, 1>{}, s0, win[0], win[1]);
        if (kWide || s0 + 2 < nslabs) slab_step(std::integral_constant<int, 2>{}, s0, win[0], win[1]);
        if (kWide || s0 + 3 < nslabs) slab_step(std::integral_constant<int, 3>{}, s0, win[0], win[1]);
        if constexpr (kWide) {
            win[0] = win[1];
            win[1] = nn;
        }
    }

    // epilogue: lane holds column lane%32 of each 32x32 block (logical block
    // 2m + b is the tile's column block 2 (m ^ wave) + b), rows
    // 8*(r/4) + 4*(lane/32) + r%4 for accumulator register r.  Each sum is
    // scaled by 2^out_exp with one v_ldexp_f32 (a single rounding, and only
    // where the result leaves the fp32 range: out_exp spans [-110, 146], more
    // than one fp32 power of two can hold).  C is written with non-temporal
    // stores: nothing here reads it again, and dirty C lines left in the
    // caches slow whatever kernel runs next (a 470 MB quantize launched after
    // this GEMM took 125 us instead of 101 us)
    // (the lane id recomputed, and the wave index read back from the
    // fragment base of logical block 0, lane * 16 + wave * 2 FRAG_BLOCK, so
    // that nothing computed before the K loop has to stay live across it
    // for the epilogue alone)
    const int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int eh = ln >> 5;
    const int wv = __builtin_amdgcn_readfirstlane(fb[0] / (2 * FRAG_BLOCK));
    // Stores go through a buffer resource based at the tile's first output
    // and sized to the tile's rows that exist (a store to a row past M falls
    // outside it and is dropped by the hardware): the lane's column and row
    // half are one vector offset, each row of the wave one scalar offset and
    // each 32-column block an immediate, with one lane test per block for
    // columns past N -- no 64-bit address arithmetic per store.  (Offsets
    // are 32-bit; a row stride beyond 2^21 floats takes the general path.)
    if ((uint64_t)ldc * (4 * BM) < (1ull << 31)) {
        const uint32_t ld4 = (uint32_t)ldc * 4;
        const int rows_valid = (int)(M - m0 < BM ? M - m0 : BM);
        const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(c + m0 * ldc + n0), 0, (int)((uint32_t)rows_valid * ld4), kRawBufferFlags);
        const int cl = ln & 31;
        const uint32_t vo = (uint32_t)cl * 4 + (uint32_t)(4 * eh) * ld4;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const int pj = 2 * ((j >> 1) ^ wv) + (j & 1);  // the tile's column block
            if (n0 + 32 * pj + cl < N) {
#pragma unroll
                for (int i = 0; i < 2; i++)
#pragma unroll
                    for (int r = 0; r < 16; r++) {
                        const int so = (64 * wv + 32 * i + 8 * (r >> 2) + (r & 3)) * (int)ld4;
                        __builtin_amdgcn_raw_buffer_store_b32(
                            __float_as_uint(__builtin_amdgcn_ldexpf(acc[i][j][r], out_exp)), crs,
                            vo, so + pj * 128, kNonTemporal);
                    }
            }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const int64_t col = n0 + (2 * ((j >> 1) ^ wv) + (j & 1)) * 32 + (ln & 31);
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int64_t row = m0 + 64 * wv + 32 * i + 8 * (r >> 2) + 4 * eh + (r & 3);
                if (row < M && col < N)
                    __builtin_nontemporal_store(__builtin_amdgcn_ldexpf(acc[i][j][r], out_exp),
                                                &c[row * ldc + col]);
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
                       int64_t ldc, int out_exp, int64_t tiles_m, int64_t tiles_n,
                       hipStream_t stream) {
    // dynamic LDS above 64 KB must be allowed per kernel (idempotent, any device)
    hipError_t err = hipFuncSetAttribute((const void*)gemm_kernel<kWide>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, SMEM_BYTES);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(gemm_kernel<kWide>, dim3((unsigned)(tiles_m * tiles_n)), dim3(kThreads),
                       SMEM_BYTES, stream, a_codes, a_scales, w_codes, w_scales, M, N, K, c, ldc,
                       out_exp, (int)tiles_m, (int)tiles_n);
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
    // C = sum * 2^(a_exp + w_exp + 18): each decoded operand carries 2^-9.
    // The exponent lies in [-110, 146], so it is applied per output in the
    // kernel (ldexp), never as one fp32 factor, which would overflow.
    const int out_exp = a_exp + w_exp + 18;
    // Wide fetches need 16-byte aligned code and scale rows and whole 4-slab
    // scale windows.
    // Buffer offsets are 32-bit: 257 code rows of K/2 bytes from the tile's
    // first row must fit.
    const bool wide = K % (BK * kWin) == 0 && (uintptr_t)a_codes % 16 == 0 &&
                      (uintptr_t)w_codes % 16 == 0 && (uintptr_t)a_scales % 16 == 0 &&
                      (uintptr_t)w_scales % 16 == 0 && (uint64_t)(BM + 1) * (K / 2) < (1ull << 31);
    return wide ? launch_tile<true>(a_codes, a_scales, w_codes, w_scales, M, N, K, c, ldc,
                                    out_exp, tiles_m, tiles_n, stream)
                : launch_tile<false>(a_codes, a_scales, w_codes, w_scales, M, N, K, c, ldc,
                                     out_exp, tiles_m, tiles_n, stream);
}

}  // namespace if4
