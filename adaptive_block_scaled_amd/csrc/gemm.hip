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

// ---------------------------------------------------------------------------
// Operand fetch.  The vector memory path costs about one cycle per distinct
// cache line an instruction touches, so loads are shaped to touch few lines:
// an A lane's 16 code bytes share their 32-byte row segment with its partner
// lane (32 lines per instruction), two W lanes load the two halves of one
// row's 32-byte slab (32 lines), and scale bytes are fetched 16 at a time,
// four slabs' worth per row.
//
// kWide: 16-byte aligned code and scale rows, K a multiple of 256 (whole
// scale windows).  Otherwise every word and byte is fetched on its own,
// clamped into the row, and groups past K decode with a zero multiplier.

// Codes of one slab for one lane: A blocks i = 0, 1 (row lane%32 of each,
// groups 2h, 2h+1 with h = lane/32) and W rows k = 0, 1 (groups 2q, 2q+1
// with q = lane%2).
template <bool kWide>
struct SlabCodes;

template <>
struct SlabCodes<true> {
    uint4 a[2], w[2];
    __device__ __forceinline__ void load(const uint8_t* const* acp, const uint8_t* const* asp,
                                         const uint8_t* const* wcp, const uint8_t* const* wsp,
                                         int64_t slab, int h, int q, int64_t gpr) {
        (void)asp, (void)wsp, (void)h, (void)q, (void)gpr;
#pragma unroll
        for (int i = 0; i < 2; i++) a[i] = *reinterpret_cast<const uint4*>(acp[i] + slab * 32);
#pragma unroll
        for (int k = 0; k < 2; k++) w[k] = *reinterpret_cast<const uint4*>(wcp[k] + slab * 32);
    }
    // A block i, MFMA step t: word (group 2h + t/2, half t%2)
    __device__ __forceinline__ uint32_t aword(int i, int t) const {
        return t == 0 ? a[i].x : t == 1 ? a[i].y : t == 2 ? a[i].z : a[i].w;
    }
    // W row k, word u = 2 * (group - 2q) + half
    __device__ __forceinline__ uint32_t wword(int k, int u) const {
        return u == 0 ? w[k].x : u == 1 ? w[k].y : u == 2 ? w[k].z : w[k].w;
    }
};

template <>
struct SlabCodes<false> {
    uint32_t a[2][4], w[2][4];
    uint32_t ab[2][4], wb[2][2];  // scale bytes
    __device__ __forceinline__ void load(const uint8_t* const* acp, const uint8_t* const* asp,
                                         const uint8_t* const* wcp, const uint8_t* const* wsp,
                                         int64_t slab, int h, int q, int64_t gpr) {
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const int64_t g = slab * kGroups + 2 * h + (t >> 1);
                const int64_t gc = g < gpr ? g : gpr - 1;
                a[i][t] = *reinterpret_cast<const uint32_t*>(acp[i] + gc * 8 + 4 * (t & 1));
                ab[i][t] = asp[i][gc];
            }
#pragma unroll
        for (int k = 0; k < 2; k++)
#pragma unroll
            for (int gg = 0; gg < 2; gg++) {
                const int64_t g = slab * kGroups + 2 * q + gg;
                const int64_t gc = g < gpr ? g : gpr - 1;
                const uint2 v = *reinterpret_cast<const uint2*>(wcp[k] + gc * 8);
                w[k][2 * gg] = v.x;
                w[k][2 * gg + 1] = v.y;
                wb[k][gg] = wsp[k][gc];
            }
    }
    __device__ __forceinline__ uint32_t aword(int i, int t) const { return a[i][t]; }
    __device__ __forceinline__ uint32_t wword(int k, int u) const { return w[k][u]; }
};

// Scale bytes of one 4-slab window (wide path): 16 bytes per A block row and
// per W row; word u holds slab u's four groups.
struct WinScales {
    uint4 a[2], w[2];
    __device__ __forceinline__ void load(const uint8_t* const* asp, const uint8_t* const* wsp,
                                         int64_t win) {
#pragma unroll
        for (int i = 0; i < 2; i++) a[i] = *reinterpret_cast<const uint4*>(asp[i] + win * 16);
#pragma unroll
        for (int k = 0; k < 2; k++) w[k] = *reinterpret_cast<const uint4*>(wsp[k] + win * 16);
    }
};

__device__ __forceinline__ uint32_t word_of(const uint4& v, int u) {
    return u == 0 ? v.x : u == 1 ? v.y : u == 2 ? v.z : v.w;
}

// IF4 x IF4 GEMM kernel.
//
// Decode (decode_half): a code nibble becomes the high byte of an fp16
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
// ds_read_b128s.
//
// Pipeline: while the MFMAs of K slab s run, each wave decodes slab s+1
// (its A registers, its W share into the other LDS buffer) and fetches the
// codes of slab s+2 into the register set that slab s used; scales arrive a
// window ahead.  The slab loop is unrolled by the 4-slab window so that all
// register sets are fixed and no loaded value is copied (a copy would wait
// for its load).  One LDS-only barrier per slab, after which the eight W
// fragments of the slab's first step are read before any MFMA is issued.
// Within a slab, each MFMA step runs four sub-blocks of four MFMAs: (A block
// 0, W blocks 0..3), (1, 0..3), (0, 4..7), (1, 4..7); the eight W fragments
// of the next step are read into a second register set at the start of the
// step, a whole step before their use.
// Each sub-block carries one code-word decode (about 16 VALU instructions):
// A block 1's operand of step t-1 in sub-block 0 (for step 0, from a word
// kept across the barrier), W words in sub-blocks 1 and 2, A block 0's
// operand of step t in sub-block 3.  The scale-table lookups of a step's
// decodes are issued at the start of the step before (LDS operations
// complete in order, so a lookup issued after the fragment reads would make
// its consumer wait for them too).  Rows past M or N load their nearest
// in-range row (those outputs are never stored).
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

    // A rows of this lane: row lane%32 of the wave's two 32-row blocks
    const int h = lane >> 5, hs = 16 * h;
    const uint8_t* acp[2];
    const uint8_t* asp[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int64_t r = m0 + 64 * wave + 32 * i + (lane & 31);
        const int64_t rc = r < M ? r : M - 1;
        acp[i] = a_codes + rc * kb + (kWide ? 16 * h : 0);
        asp[i] = a_scales + rc * gpr;
    }
    // W rows of this thread: tile rows 64w + 32k + lane/2, groups 2q, 2q+1
    const int q = lane & 1, qs = 16 * q;
    int wr_row[2];
    const uint8_t* wcp[2];
    const uint8_t* wsp[2];
#pragma unroll
    for (int k = 0; k < 2; k++) {
        wr_row[k] = 64 * wave + 32 * k + (lane >> 1);
        const int64_t r = n0 + wr_row[k];
        const int64_t rc = r < N ? r : N - 1;
        wcp[k] = w_codes + rc * kb + (kWide ? 16 * q : 0);
        wsp[k] = w_scales + rc * gpr;
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

    // Scale of A block i / W row k, group selected by t / gg, in slab
    // `slab` = window slot u of a window's scales (wide) or from the slab's
    // own bytes; groups past K exist only without whole slabs.
    auto a_scale = [&](const SlabCodes<kWide>& x, const WinScales& win, int u, int64_t slab,
                       int i, int t) {
        uint32_t b;
        if constexpr (kWide) {
            b = (word_of(win.a[i], u) >> (hs + 8 * (t >> 1))) & 0xFFu;
        } else {
            const bool past = slab * kGroups + 2 * h + (t >> 1) >= gpr;
            b = past ? kZeroScale : x.ab[i][t];
        }
        return lookup_scale(smem, b);
    };
    auto w_scale = [&](const SlabCodes<kWide>& x, const WinScales& win, int u, int64_t slab,
                       int k, int gg) {
        uint32_t b;
        if constexpr (kWide) {
            b = (word_of(win.w[k], u) >> (qs + 8 * gg)) & 0xFFu;
        } else {
            const bool past = slab * kGroups + 2 * q + gg >= gpr;
            b = past ? kZeroScale : x.wb[k][gg];
        }
        return lookup_scale(smem, b);
    };
    // W row k, group 2q + gg, half hf into `tile`
    auto w_store = [&](const SlabCodes<kWide>& x, GroupScale sc, int k, int gg, int hf,
                       uint8_t* tile) {
        *reinterpret_cast<half8*>(tile + frag_off(wr_row[k], 2 * q + gg, hf)) =
            decode_half(x.wword(k, 2 * gg + hf), sc);
    };

    // register sets: raw[p] holds the codes of a slab of parity p
    SlabCodes<kWide> raw[2];
    WinScales win[2];      // scale windows: the running one and the next
    half8 a[2][kGroups];   // decoded A operands [block][MFMA step] of the running slab
    uint32_t w13;          // A block 1, last step: word and scale of the running slab
    GroupScale s13;
    // Scale-table lookups run one MFMA step ahead of the decodes that use
    // them: issued before that step's fragment prefetches, a lookup can be
    // waited for (LDS operations complete in order) without waiting for the
    // prefetches too.  la1 / la0 / lw: A block 1 (previous step's word),
    // A block 0 and W of the coming step.
    GroupScale la1, la0, lw;

    // prologue: slab 0 decoded (W into buffer 0, A into registers), slab 1 fetched
    if constexpr (kWide) {
        win[0].load(asp, wsp, 0);
        win[1].load(asp, wsp, nwin > 1 ? 1 : 0);
    }
    raw[0].load(acp, asp, wcp, wsp, 0, h, q, gpr);
    raw[1].load(acp, asp, wcp, wsp, last < 1 ? last : 1, h, q, gpr);
#pragma unroll
    for (int t = 0; t < kGroups; t++) {
#pragma unroll
        for (int i = 0; i < 2; i++)
            a[i][t] = decode_half(raw[0].aword(i, t), a_scale(raw[0], win[0], 0, 0, i, t));
        const int k = t >> 1, gg = t & 1;
        const GroupScale sw = w_scale(raw[0], win[0], 0, 0, k, gg);
        w_store(raw[0], sw, k, gg, 0, smem);
        w_store(raw[0], sw, k, gg, 1, smem);
    }
    w13 = raw[0].aword(1, kGroups - 1);
    s13 = a_scale(raw[0], win[0], 0, 0, 1, kGroups - 1);
    // lookups for step 0 of slab 0, which decodes slab 1
    la1 = s13;
    la0 = a_scale(raw[1], win[0], 1, 1, 0, 0);
    lw = w_scale(raw[1], win[0], 1, 1, 0, 0);
    lds_barrier();

    const int w_off = lane * 16;  // fragment (block j, step t) at j * FRAG_BLOCK + t * FRAG_STEP

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
        // slab s+2, clamped: past the end the loads repeat the last slab and
        // the decodes fill registers and a buffer that nobody reads again
        const int64_t sl = (int64_t)s + 2 < last ? (int64_t)s + 2 : last;
        // scales of slab s+1: slot U+1 of this window, or slot 0 of the next;
        // of slab s+2 (looked up in the last step): slot U+2 of either
        const WinScales& sw_win = U + 1 < kWin ? wcur : wnxt;
        constexpr int US = (U + 1) % kWin;
        const WinScales& sw2_win = U + 2 < kWin ? wcur : wnxt;
        constexpr int US2 = (U + 2) % kWin;
        const SlabCodes<kWide>& x = raw[Q];

        // step 0's fragments first, all eight before any MFMA, so that only
        // the first read's latency is exposed after the barrier
        half8 bv[2][8];  // fragments of even / odd steps
#pragma unroll
        for (int j = 0; j < 8; j++)
            bv[0][j] = *reinterpret_cast<const half8*>(buf + w_off + j * FRAG_BLOCK);
        raw[P].load(acp, asp, wcp, wsp, sl, h, q, gpr);
#pragma unroll
        for (int t = 0; t < kGroups; t++) {
            const int k = t >> 1, gg = t & 1;
            const GroupScale sa1 = la1, sa0 = la0, sw = lw;
            if (t + 1 < kGroups) {
                la1 = a_scale(x, sw_win, US, sn, 1, t);
                la0 = a_scale(x, sw_win, US, sn, 0, t + 1);
                lw = w_scale(x, sw_win, US, sn, (t + 1) >> 1, (t + 1) & 1);
            } else {
                // step 0 of the next slab: A block 1's last word of slab s+1,
                // then A block 0 and W of slab s+2
                la1 = a_scale(x, sw_win, US, sn, 1, kGroups - 1);
                la0 = a_scale(raw[P], sw2_win, US2, sn + 1, 0, 0);
                lw = w_scale(raw[P], sw2_win, US2, sn + 1, 0, 0);
            }
            // the next step's eight fragments, a whole step ahead
            if (t + 1 < kGroups) {
#pragma unroll
                for (int j = 0; j < 8; j++)
                    bv[(t + 1) & 1][j] = *reinterpret_cast<const half8*>(
                        buf + w_off + j * FRAG_BLOCK + (t + 1) * FRAG_STEP);
            }
            // sub-blocks: (A block 0, W 0..3), (1, 0..3), (0, 4..7), (1, 4..7)
#pragma unroll
            for (int sb = 0; sb < 4; sb++) {
                const int i = sb & 1;  // A block of this sub-block's MFMAs
#pragma unroll
                for (int jj = 0; jj < 4; jj++) {
                    const int j = 4 * (sb >> 1) + jj;
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i][t], bv[t & 1][j],
                                                                       acc[i][j], 0, 0, 0);
                }
                if (sb == 0) {
                    // t = 0: the word kept from the previous slab (sa1 holds its scale)
                    a[1][t == 0 ? kGroups - 1 : t - 1] =
                        decode_half(t == 0 ? w13 : x.aword(1, t - 1), sa1);
                } else if (sb == 3) {
                    a[0][t] = decode_half(x.aword(0, t), sa0);  // its last use was sub-block 2
                } else {
                    w_store(x, sw, k, gg, sb == 1 ? 0 : 1, nbuf);
                }
                // interleave: each MFMA followed by five VALU and up to two
                // LDS reads; no fence between sub-blocks, so the scheduler
                // may pull a later sub-block's independent work forward
#pragma unroll
                for (int m = 0; m < 4; m++) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // VALU
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS read
                    if (m == 2) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // LDS write
                    if (m == 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load
                }
            }
        }
        w13 = x.aword(1, kGroups - 1);
        lds_barrier();
    };

    // One 4-slab window.  The scales of the window after next are fetched
    // at its start, so that moving them into place at its end does not wait.
    for (int s0 = 0; s0 < nslabs; s0 += kWin) {
        WinScales nn;
        if constexpr (kWide) {
            const int64_t nw = (int64_t)s0 / kWin + 2;
            nn.load(asp, wsp, nw < nwin ? nw : nwin - 1);
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

    // epilogue: lane holds column lane%32 of each 32x32 block, rows
    // 8*(r/4) + 4*(lane/32) + r%4 for accumulator register r.  Each sum is
    // scaled by 2^out_exp with one v_ldexp_f32 (a single rounding, and only
    // where the result leaves the fp32 range: out_exp spans [-110, 146], more
    // than one fp32 power of two can hold).  C is written
    // with non-temporal stores: nothing here reads it again, and dirty C
    // lines left in the caches slow whatever kernel runs next (a 470 MB
    // quantize launched after this GEMM took 125 us instead of 101 us)
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const int64_t col = n0 + j * 32 + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int64_t row = m0 + 64 * wave + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
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
    const bool wide = K % (BK * kWin) == 0 && (uintptr_t)a_codes % 16 == 0 &&
                      (uintptr_t)w_codes % 16 == 0 && (uintptr_t)a_scales % 16 == 0 &&
                      (uintptr_t)w_scales % 16 == 0;
    return wide ? launch_tile<true>(a_codes, a_scales, w_codes, w_scales, M, N, K, c, ldc,
                                    out_exp, tiles_m, tiles_n, stream)
                : launch_tile<false>(a_codes, a_scales, w_codes, w_scales, M, N, K, c, ldc,
                                     out_exp, tiles_m, tiles_n, stream);
}

}  // namespace if4
