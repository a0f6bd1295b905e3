// W4A8 on the fp8 matrix cores of gfx950 (groups of 128 k, or whole rows,
// K a multiple of 128, M above the mid-size range).
//
// Both operands of v_mfma_f32_16x16x128_f8f6f4 are E4M3: the activation codes
// of the row quantizer, and each weight as the exact integer u - z
// (|u - z| <= 15 is an E4M3 value).  One 128-k step is one group, so one MFMA
// gives a 16 x 16 output block's exact group sum T = sum_k xq (u - z), and the
// group scale is applied to it per output, acc += s T; the row scale comes in
// the epilogue (gowda.ai "LLM fast inference", "Achievement 2": FP8
// operands, FP32 accumulation, the row scale in the epilogue; here the weight
// codes stay exact instead of rounding (u - z) s to E4M3).
//
// Tile BM x BN (64 to 256 rows, 64 to 256 columns) of eight waves in a
// WR x WC grid: wave (wr, wc) owns BM / WR rows (row blocks of 16) by
// BN / WC columns (CB column blocks of 16).  The accumulators take VALU
// multiply-adds, so they live in ordinary VGPRs (the file is built with MFMA
// results in VGPRs); two waves share a SIMD and one wave's VALU work runs
// under the other's MFMAs.  Large products take 256 x 256 tiles; products of
// a few hundred rows or fewer take narrower or shorter tiles, which give
// enough workgroups without splitting K (f8_split).
//
// The E4M3 activations go straight from global memory into LDS
// (buffer_load_dwordx4 ... lds into three BM x 128-byte stages, two steps ahead; the
// 16-byte chunk c of stage row r sits at position c ^ ((r >> 1) & 7), so the
// 16 rows of a fragment read spread over all 64 banks).  The weights
// never pass through LDS: for a 16-column block, lane (c, q) loads the 16
// bytes of 32-k tile 4 kt + q of its column (the 64 lanes read one contiguous
// 1 KB of the blocked layout), two steps ahead, and converts them one step
// ahead into its 32 B-operand bytes: per pair of codes one AND-OR into fp16
// 1024 + u (or 1024 + 16 u), one packed fp16 add of -(1024 + z) (or
// multiply-add by 1/16 and -(64 + z)), exact, and one
// v_cvt_scalef32_pk_fp8_f16.  Lane (c, q) of the A operand holds bytes
// 32 q .. 32 q + 31 of its row's 128-k step, so both operands pair the same k.
// The group sums of a block are scaled two MFMA slots after their MFMA.
//
// A zero point outside 0..15 (possible only for a contracted range that
// excludes 0) is clamped to zc for the MFMA operand, and the difference is
// restored exactly: acc += s (zc - z) sum_k xq, with sum_k xq from one more
// MFMA against ones, only in steps where some column of the wave needs it.
#include <type_traits>
#include <utility>

#include "device.hpp"
#include "kernels.hpp"

namespace w4 {
namespace {

namespace f8 {
constexpr int BK = 128;
static_assert(BK == kF8StepK, "one K step of the fp8 kernel");
// BM x BN tile of WR x WC waves: wave (wr, wc) owns rows (BM / WR) wr ..
// and columns (BN / WC) wc ..
template <int BM_, int BN_, int WR_, int WC_>
struct Geom {
    static constexpr int BM = BM_, BN = BN_, WR = WR_, WC = WC_, NW = WR * WC, NT = 64 * NW;
    static constexpr int STAGE = BM * BK;                 // bytes of one activation stage
    static constexpr int ADMA = STAGE / (1024 * NW);      // direct-to-LDS loads per wave and step
    static constexpr int RB = BM / 16 / WR;               // 16-row blocks per wave
    static constexpr int WN = BN / WC;                    // columns per wave
    static constexpr int CB = WN / 16;                    // 16-column blocks per wave
    static constexpr int NSLOT = RB * CB;                 // MFMAs per wave and step
    static constexpr int NCONV = CB * 4;                  // code words converted per lane and step
    static constexpr int BLOAD = 2 * CB;                  // code and scale/zero loads per lane and step
    static_assert(ADMA >= 1 && CB >= 1 && NSLOT % BLOAD == 0 && NSLOT % ADMA == 0, "slot plan");
};
}  // namespace f8

typedef _Float16 half2v_t __attribute__((ext_vector_type(2)));

constexpr int gcd2(int a, int b) { return b == 0 ? a : gcd2(b, a % b); }
constexpr int lcm3(int a, int b, int c) {
    const int ab = a / gcd2(a, b) * b;
    return ab / gcd2(ab, c) * c;
}
// f(integral_constant<int, 0>) .. f(integral_constant<int, N - 1>), in order
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}
typedef short short2v_t __attribute__((ext_vector_type(2)));

// The work of one workgroup (1-D grid): workgroup b < split_t0 computes tile b
// whole; the rest compute K range z of tile split_t0 + (b - split_t0) /
// splits, z = (b - split_t0) % splits.  Tile numbers map to the grid by tile_rc.
struct F8Job {
    int64_t m_base, n_base;
    int kb, KT;        // first K step and number of K steps
    int64_t part;      // partial-tile index in ws, or -1: write Y
};
template <int BM, int BN>
__device__ __forceinline__ F8Job f8_job(const MulParams& p) {
    using namespace f8;
    const int64_t b = blockIdx.x;
    const int64_t nt = (p.N + BN - 1) / BN;     // BN: output columns of a tile
    const int KT_all = static_cast<int>(p.K / BK);
    F8Job t;
    int64_t tile;
    if (b < p.split_t0) {
        tile = xcd_tile(b, p.split_t0);
        t.kb = 0;
        t.KT = KT_all;
        t.part = -1;
    } else {
        const int64_t j = (b - p.split_t0) / p.splits;
        const int z = static_cast<int>((b - p.split_t0) % p.splits);
        tile = p.split_t0 + j;
        t.kb = z * KT_all / p.splits;
        t.KT = (z + 1) * KT_all / p.splits - t.kb;
        t.part = j * p.splits + z;
    }
    int64_t tr, tc;
    tile_rc(tile, (p.M + BM - 1) / BM, nt, tr, tc);
    t.m_base = tr * BM;
    t.n_base = tc * BN;
    return t;
}

// One code word (codes k = 8j .. 8j + 7 of a column) as eight E4M3 bytes of
// u - zc in k order, into o0 (k 0..3) and o1 (k 4..7).  nb = -(1024 + zc)
// and nb16 = -(64 + zc) as fp16 pairs; bias = two fp16 1024.0 in a register.
__device__ __forceinline__ void f8_word(uint32_t w, uint32_t bias, half2v_t nb, half2v_t nb16, uint32_t& o0,
                                        uint32_t& o1) {
    const half2v_t sixteenth = {static_cast<_Float16>(0.0625f), static_cast<_Float16>(0.0625f)};
    const uint32_t w8 = w >> 8;
    const half2v_t e0 = __builtin_bit_cast(half2v_t, (w & 0x000F000Fu) | bias);     // 1024 + u: k 0, 1
    const half2v_t e1 = __builtin_bit_cast(half2v_t, (w & 0x00F000F0u) | bias);     // 1024 + 16 u: k 2, 3
    const half2v_t e2 = __builtin_bit_cast(half2v_t, (w8 & 0x000F000Fu) | bias);    // k 4, 5
    const half2v_t e3 = __builtin_bit_cast(half2v_t, (w8 & 0x00F000F0u) | bias);    // k 6, 7
    const half2v_t d0 = e0 + nb;
    const half2v_t d1 = __builtin_elementwise_fma(e1, sixteenth, nb16);
    const half2v_t d2 = e2 + nb;
    const half2v_t d3 = __builtin_elementwise_fma(e3, sixteenth, nb16);
    short2v_t r0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(short2v_t{0, 0}, d0, 1.0f, false);
    r0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(r0, d1, 1.0f, true);
    short2v_t r1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(short2v_t{0, 0}, d2, 1.0f, false);
    r1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(r1, d3, 1.0f, true);
    o0 = __builtin_bit_cast(uint32_t, r0);
    o1 = __builtin_bit_cast(uint32_t, r1);
}

// A raw buffer descriptor (base, no stride, `bytes` records; reads past the
// end return zeros), kept in SGPRs: every word passes readfirstlane, since a
// size computed with a division comes from the VALU, and a descriptor the
// compiler cannot prove uniform wraps each load in a loop over its values.
__device__ __forceinline__ u32x4_t buffer_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return u32x4_t{static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a))),
                   static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32))) & 0xFFFFu,
                   static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(bytes)), 0x00020000u};
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t as_rsrc(const u32x4_t& r) {
    return __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void*>(static_cast<uint64_t>(r[0]) | (static_cast<uint64_t>(r[1]) << 32)), static_cast<short>(0),
        static_cast<int>(r[2]), static_cast<int>(r[3]));
}

__device__ __forceinline__ float4_t mfma_f8_16x16x128(const int8x_t& a, const int8x_t& b) {
    // formats 0 / 0: both operands E4M3; no block scales
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, float4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0, 0, 0, 0);
}

// PAIR: the gate and up projections in one pass (p.wq2 / p.sz2 the up
// weight): the tile holds BN / 2 output columns, waves wc < WC / 2 sum them
// over the gate weight and the others over the up weight; the epilogue
// combines the two through LDS into H = bf16(act(g) u) (both sums scaled by
// the row scale first) and, with p.amax_part, records each row's maximum |H|
// over the tile's columns.  Never split along K.
//
// SA activation stages and DW weight register sets: the activations of step
// kt go out SA - 1 steps ahead, its codes DW steps ahead (converted one step
// ahead).  A step ends waiting for the loads of all but its last SA - 2
// steps, so codes loaded further ahead than SA steps would be waited for
// early: DW <= SA.  Large tiles are compute-bound and take (3, 2); small ones
// stream their weights at a few hundred rows or fewer and take deeper pipelines.
//
// A16: W4A16 on the same tiles (groups of 128): bf16 activations (two bytes
// a k in the stages), the exact bf16 values 128 + u as the B operand of
// v_mfma_f32_16x16x32_bf16 (four per 16 x 16 block and step; MFMA j takes,
// from every quarter q, the 8 k at 32 q + 8 j, and the activation fragment
// the same k), the row sums of the step's activations from four more MFMAs
// against ones, and per group and output acc += s (T - (128 + z) X1): exact
// weights, any zero point.
template <int BM_, int BN_, int WR_, int WC_, bool PAIR = false, int SA_ = 3, int DW_ = 2, bool A16 = false>
__global__ void __launch_bounds__(64 * WR_ * WC_) gemm_f8_kernel(MulParams p) {
    using namespace f8;
    using Gm = Geom<BM_, BN_, WR_, WC_>;
    constexpr int AB = A16 ? 2 : 1;               // bytes per activation
    constexpr int BM = Gm::BM, BN = Gm::BN, WC = Gm::WC, STAGE = Gm::STAGE * AB, ADMA = Gm::ADMA * AB,
                  RB = Gm::RB, WN = Gm::WN, CB = Gm::CB, NSLOT = Gm::NSLOT, NCONV = Gm::NCONV, BLOAD = Gm::BLOAD;
    constexpr int SA = SA_, DW = DW_;
    static_assert(SA >= 3 && DW >= 2 && DW <= SA, "pipeline depths");
    static_assert(NSLOT % ADMA == 0, "slot plan");
    static_assert(!A16 || (WR_ == 1 && RB <= 8), "bf16 activations: one wave row of up to 8 row blocks");
    // one array per stage (as separate objects their addresses stay constants)
    __shared__ __attribute__((aligned(16))) uint8_t lds_a0[STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t lds_a1[STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t lds_a2[STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t lds_a3[SA > 3 ? STAGE : 1];
    __shared__ __attribute__((aligned(16))) uint8_t lds_a4[SA > 4 ? STAGE : 1];
    __shared__ __attribute__((aligned(16))) uint8_t lds_a5[SA > 5 ? STAGE : 1];
    static_assert(SA <= 6, "at most six stages");
    auto stage_a = [&](auto S) -> uint8_t* {
        constexpr int si = decltype(S)::value;
        if constexpr (si == 0) return lds_a0;
        else if constexpr (si == 1) return lds_a1;
        else if constexpr (si == 2) return lds_a2;
        else if constexpr (si == 3) return lds_a3;
        else if constexpr (si == 4) return lds_a4;
        else return lds_a5;
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int c = lane & 15, q = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wave / WC, wc = wave % WC;
    const int row0 = 16 * RB * wr;   // the wave's first tile row
    static_assert(!PAIR || (WR_ == 1 && WC_ % 2 == 0 && (BN_ / 2) % 64 == 0), "pair tiles");
    constexpr int BNO = PAIR ? BN / 2 : BN;      // output columns of the tile
    const F8Job job = f8_job<BM, BNO>(p);
    const int64_t m_base = job.m_base, n_base = job.n_base;
    const int64_t M = p.M, N = p.N, K = p.K;
    __shared__ float lds_xs[BM];
    const int kb = job.kb, KT = job.KT;
    const int g_shift = group_shift(p.G);

    float4_t acc[RB][CB];
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < CB; ++j) acc[i][j] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // activations: load `it` of this wave fills stage rows 8 (wave ADMA + it)
    // .. + 7; lane l writes row r = 8 (wave ADMA + it) + l / 8 at chunk
    // position l % 8, so it loads the chunk the swizzle puts there,
    // (l % 8) ^ ((r >> 1) & 7) = (l % 8) ^ (l / 16) ^ (4 if wave ADMA + it is
    // odd).  Buffer loads with a 32-bit lane offset: rows past M lie past the
    // buffer's end and read as zeros (their outputs are never stored).
    const int a_row0 = 8 * wave * ADMA + (lane >> 3);
    const int a_chunk = (lane & 7) ^ (lane >> 4) ^ ((wave * ADMA) & 1 ? 4 : 0);
    const u32x4_t a_rsrc = buffer_rsrc(p.X, static_cast<uint32_t>(M * K * AB));
    const uint32_t a_voff = static_cast<uint32_t>((m_base + a_row0) * K + a_chunk * 16);
    // A16: a 256-byte stage row of 16 chunks, chunk ch of row r at position
    // ch ^ (r & 15); load `it` fills rows 4 (wave ADMA + it) .. + 3, lane l
    // row 4 (wave ADMA + it) + l / 16 at position l % 16
    auto dma_item = [&](int kt, uint8_t* stage, int it) {
        kt = (kt < KT ? kt : KT - 1) + kb;
        uint32_t voff;
        if constexpr (A16) {
            const int r = 4 * (wave * ADMA + it) + (lane >> 4);
            voff = static_cast<uint32_t>((m_base + r) * (2 * K) + 16 * ((lane & 15) ^ (r & 15)));
        } else {
            voff = (a_voff ^ ((it & 1) ? 64u : 0u)) + static_cast<uint32_t>(8 * it * K);
        }
        const uint32_t soff = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(kt * BK * AB));
        // Issued as plain instructions: the compiler cannot tell the three
        // stages apart and would wait for every pending direct-to-LDS load
        // before any LDS read.  No register result (the data goes to LDS at
        // M0 + 16 lane); completion is covered by the wait at each step's end.
        // the LDS byte address, as a uniform value (scalar arithmetic on the
        // stage's constant address)
        typedef __attribute__((address_space(3))) uint8_t lds_u8;
        const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_u8*)stage)) +
                            static_cast<uint32_t>((wave * ADMA + it) * 1024);
        asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds"
                     ::"v"(voff), "s"(a_rsrc), "s"(m0), "s"(soff) : "memory", "m0");
    };

    // weights: column n_base + WN wc + 16 cb + c, 32-k tile 4 kt + q.  In
    // the blocked layout, block cb's 16 rows start at row r0 (uniform): the
    // lane's 16 bytes of tile t are at word 4 nr t + 4 cc of the block and its
    // scale/zero word of group g at nr g + cc (nr rows in the block, cc the
    // lane's row, clamped to the block: columns past N repeat the last one,
    // whose outputs are not stored).  Buffer loads: uniform block and step
    // offsets, one lane offset per block.
    // (PAIR: the up weight for waves wc >= WC / 2, at the same columns)
    const bool up_wave = PAIR && wc >= WC / 2;
    const int wcol = WN * (PAIR ? wc % (WC / 2) : wc);   // the wave's first column in the tile
    const u32x4_t q_rsrc = buffer_rsrc(up_wave ? p.wq2 : p.wq, static_cast<uint32_t>(N * K / 2));
    const u32x4_t s_rsrc = buffer_rsrc(up_wave ? p.sz2 : p.sz, static_cast<uint32_t>(N * (K / p.G) * 4));
    uint32_t qblk[CB], sblk[CB], nrb[CB];      // uniform: block byte offsets, rows in the block
    uint32_t qoff[CB], soff[CB];               // the lane's byte offsets in the block
    const int64_t nblk_last = ((N - 1) / 16) * 16;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        int64_t r0 = n_base + wcol + 16 * cb;
        r0 = r0 < N ? r0 : nblk_last;
        const int nr = static_cast<int>(N - r0 < 16 ? N - r0 : 16);
        const int cc = c < nr ? c : nr - 1;
        qblk[cb] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(r0 * (K / 2)));
        sblk[cb] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(r0 * (K / p.G) * 4));
        nrb[cb] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(nr));
        qoff[cb] = static_cast<uint32_t>(16 * nr * q + 16 * cc);
        soff[cb] = static_cast<uint32_t>(4 * cc);
    }
    struct Regs {
        u32x4_t q[CB];
        uint32_t s[CB];
    };
    auto load_item = [&](int kt, Regs& r, int it) {
        kt = (kt < KT ? kt : KT - 1) + kb;
        if (it < CB) {
            const uint32_t so = qblk[it] + static_cast<uint32_t>(kt) * (64u * nrb[it]);   // 4 tiles of 16 nr bytes
            r.q[it] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                      as_rsrc(q_rsrc), qoff[it], __builtin_amdgcn_readfirstlane(so), 0));
        } else {
            const int cb = it - CB;
            // a 128-k step lies in one group (G is a multiple of 128)
            const uint32_t g = static_cast<uint32_t>((static_cast<int64_t>(kt) * BK) >> g_shift);
            const uint32_t so = sblk[cb] + g * (4u * nrb[cb]);
            r.s[cb] = __builtin_amdgcn_raw_buffer_load_b32(as_rsrc(s_rsrc), soff[cb], __builtin_amdgcn_readfirstlane(so), 0);
        }
    };
    // converted operands of one step: E4M3 bytes of u - zc, the group scale,
    // and whether any column of the wave has zc != z
    struct BOps8 {
        int8x_t b[CB];
        float s[CB];
        uint32_t oor;
    };
    // A16: per block the four MFMA operands (bf16 pairs 128 + u), the group
    // scale and 128 + z
    struct BOps16 {
        u32x4_t b[CB][4];
        float s[CB];
        float zb[CB];
    };
    using BOps = std::conditional_t<A16, BOps16, BOps8>;
    [[maybe_unused]] uint32_t bias128 = 0;
    if constexpr (A16) bias128 = opaque_vgpr(kBf16Bias128x2);
    const uint32_t bias = opaque_vgpr(0x64006400u);   // two fp16 1024.0
    half2v_t nbv[CB], nb16v[CB];
    uint32_t oor_lane = 0;
    auto conv_item = [&](int it, const Regs& r, BOps& o) {
        const int cb = it >> 2, wi = it & 3;
        if constexpr (A16) {
            if (wi == 0) {
                const uint32_t szw = r.s[cb];
                o.s[cb] = half_bits_to_float(szw);
                o.zb[cb] = 128.0f + half_bits_to_float(szw >> 16);
            }
            const uint32_t w = r.q[cb][wi];
            uint32_t b0 = nibble_pair_bf16(w, 0, bias128), b1 = nibble_pair_bf16(w, 1, bias128),
                     b2 = nibble_pair_bf16(w, 2, bias128), b3 = nibble_pair_bf16(w, 3, bias128);
            asm volatile("" : "+v"(b0), "+v"(b1), "+v"(b2), "+v"(b3));
            o.b[cb][wi] = u32x4_t{b0, b1, b2, b3};
            return;
        } else {
        if (wi == 0) {
            const uint32_t szw = r.s[cb];
            const float s = half_bits_to_float(szw);
            const float z = half_bits_to_float(szw >> 16);
            const float zc = fminf(fmaxf(z, 0.0f), 15.0f);
            o.s[cb] = s;
            const _Float16 e = static_cast<_Float16>(-(1024.0f + zc));
            const _Float16 e16 = static_cast<_Float16>(-(64.0f + zc));
            nbv[cb] = half2v_t{e, e};
            nb16v[cb] = half2v_t{e16, e16};
            oor_lane = (cb == 0 ? 0u : oor_lane) | (zc != z ? 1u : 0u);
        }
        uint32_t o0, o1;
        f8_word(r.q[cb][wi], bias, nbv[cb], nb16v[cb], o0, o1);
        // pinned here: the optimizer would otherwise sink the conversion
        // (used only in the next step) past the MFMAs of this one
        asm volatile("" : "+v"(o0), "+v"(o1));
        o.b[cb][2 * wi] = static_cast<int>(o0);
        o.b[cb][2 * wi + 1] = static_cast<int>(o1);
        if (it == NCONV - 1)
            o.oor = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(__builtin_amdgcn_ballot_w64(oor_lane != 0) != 0));
        }
    };

    // A fragment of the wave's row block rb: stage row row0 + 16 rb + c,
    // chunks 2 q and 2 q + 1 (swizzle ((16 j + c) >> 1) & 7 = c >> 1, the same
    // for every 16-row block j)
    const uint32_t aoff0 = static_cast<uint32_t>((row0 + c) * BK + 16 * ((2 * q) ^ (c >> 1)));
    const uint32_t aoff1 = static_cast<uint32_t>((row0 + c) * BK + 16 * ((2 * q + 1) ^ (c >> 1)));
    auto frag_a = [&](const uint8_t* A, int rb) -> int8x_t {
        const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(A + rb * (16 * BK) + aoff0);
        const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(A + rb * (16 * BK) + aoff1);
        return int8x_t{static_cast<int>(lo[0]), static_cast<int>(lo[1]), static_cast<int>(lo[2]), static_cast<int>(lo[3]),
                       static_cast<int>(hi[0]), static_cast<int>(hi[1]), static_cast<int>(hi[2]), static_cast<int>(hi[3])};
    };

    // a step ends with the activations of the next one in LDS: all loads
    // done but those of the last SA - 2 steps (loads complete in order)
    constexpr int kStepLoads = ADMA + BLOAD;
    constexpr int kLeft = (SA - 2) * kStepLoads;
    static_assert(kLeft < 64, "vmcnt range");
    auto step_end = [&]() {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt((kLeft & 15) | (7 << 4) | ((kLeft >> 4) << 14));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    auto scale_add = [&](int v, const BOps& cur, const float4_t& t) {
        const float sv = cur.s[v % CB];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[v / CB][v % CB][e] = fmaf(sv, t[e], acc[v / CB][v % CB][e]);
    };
    // step kt: MFMAs on `cur` (converted during step kt - 1) and the A stage
    // of kt; `ready` (codes of step kt + 1) converted into `nxt`; the codes of
    // step kt + DW loaded into `next`, the activations of step kt + SA - 1
    // sent to LDS
#ifndef W4_F8_TROT
#define W4_F8_TROT 2
#endif
    constexpr int TROT = W4_F8_TROT;   // group sums in flight: a block is scaled TROT - 1 slots after its MFMA
#ifndef W4_F8_CONV0
#define W4_F8_CONV0 1
#endif
    // conversion items from slot CONV0 on, spread evenly over the rest of the
    // step (a later start leaves the codes loaded a step before more time to arrive)
    constexpr int CONV0 = NSLOT > 1 ? W4_F8_CONV0 : 0;
    constexpr int CONV_EVERY = (NSLOT - CONV0) / NCONV, LOAD_EVERY = NSLOT / BLOAD, DMA_EVERY = NSLOT / ADMA;
    // conversion item i goes to slot conv_slot(i); with fewer slots than
    // items, several share a slot
    auto conv_slot = [](int i) constexpr {
        return CONV_EVERY >= 1 ? CONV0 + i * CONV_EVERY : CONV0 + i * (NSLOT - CONV0) / NCONV;
    };
    // the conversions, code loads and activation loads of slot u (A16; the
    // fp8 step spells the same plan out)
    auto slot_work = [&](int u, int kt, Regs& next, const Regs& ready, BOps& nxt, uint8_t* Ad) __attribute__((always_inline)) {
        if constexpr (CONV_EVERY >= 1) {
            if (u >= CONV0 && (u - CONV0) % CONV_EVERY == 0 && (u - CONV0) / CONV_EVERY < NCONV)
                conv_item((u - CONV0) / CONV_EVERY, ready, nxt);
        } else {
#pragma unroll
            for (int i = 0; i < NCONV; ++i)
                if (conv_slot(i) == u) conv_item(i, ready, nxt);
        }
        if (u % LOAD_EVERY == LOAD_EVERY / 2 - 1) {
            load_item(kt + DW, next, u / LOAD_EVERY);
            asm volatile("" ::: "memory");
        }
        if (u % DMA_EVERY == DMA_EVERY - 1) dma_item(kt + SA - 1, Ad, u / DMA_EVERY);
    };
    // A16: fragment j of row block rb, stage row row0 + 16 rb + c (its low
    // four bits are c), chunk 4 q + j at position (4 q + j) ^ c
    auto frag_a16 = [&](const uint8_t* A, int rb, int j) -> bf16x8_t {
        return *reinterpret_cast<const bf16x8_t*>(A + (row0 + 16 * rb + c) * (2 * BK) + 16 * ((4 * q + j) ^ c));
    };
    auto step = [&](int kt, auto S, Regs& next, const Regs& ready, const BOps& cur, BOps& nxt) __attribute__((always_inline)) {
        constexpr int sa = decltype(S)::value;
        const uint8_t* As = stage_a(std::integral_constant<int, sa>{});
        uint8_t* Ad = stage_a(std::integral_constant<int, (sa + SA - 1) % SA>{});
        if constexpr (A16) {
            const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
            bf16x8_t fa[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) fa[j] = frag_a16(As, 0, j);
            float4_t X1[RB], T[TROT];
            auto scale_add16 = [&](int v, const float4_t& t) {
                const int rb = v / CB, cb = v % CB;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[rb][cb][e] = fmaf(cur.s[cb], fmaf(-cur.zb[cb], X1[rb][e], t[e]), acc[rb][cb][e]);
            };
#pragma unroll
            for (int u = 0; u < NSLOT; ++u) {
                const int rb = u / CB, cb = u % CB;
                __builtin_amdgcn_sched_barrier(0);
                if (cb == 0) {
                    // the step's row sums of the block's 16 rows (every column alike)
                    X1[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[0], ones, float4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
#pragma unroll
                    for (int j = 1; j < 4; ++j) X1[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[j], ones, X1[rb], 0, 0, 0);
                }
                T[u % TROT] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[0], __builtin_bit_cast(bf16x8_t, cur.b[cb][0]),
                                                                      float4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
#pragma unroll
                for (int j = 1; j < 4; ++j)
                    T[u % TROT] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[j], __builtin_bit_cast(bf16x8_t, cur.b[cb][j]),
                                                                          T[u % TROT], 0, 0, 0);
                if (cb == CB - 1 && rb + 1 < RB) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) fa[j] = frag_a16(As, rb + 1, j);
                }
                if (u >= TROT - 1) scale_add16(u - (TROT - 1), T[(u - (TROT - 1)) % TROT]);
                slot_work(u, kt, next, ready, nxt, Ad);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int v = NSLOT - (TROT - 1); v < NSLOT; ++v) scale_add16(v, T[v % TROT]);
            step_end();
            return;
        } else {
        int8x_t fa = frag_a(As, 0);
        float4_t T[TROT];
#pragma unroll
        for (int u = 0; u < NSLOT; ++u) {
            const int rb = u / CB, cb = u % CB;
            __builtin_amdgcn_sched_barrier(0);
            T[u % TROT] = mfma_f8_16x16x128(fa, cur.b[cb]);
            // the fragment is reloaded for the next row block right after its last use
            if (cb == CB - 1 && rb + 1 < RB) fa = frag_a(As, rb + 1);
            if (u >= TROT - 1) scale_add(u - (TROT - 1), cur, T[(u - (TROT - 1)) % TROT]);
            if constexpr (CONV_EVERY >= 1) {
                if (u >= CONV0 && (u - CONV0) % CONV_EVERY == 0 && (u - CONV0) / CONV_EVERY < NCONV)
                    conv_item((u - CONV0) / CONV_EVERY, ready, nxt);
            } else {
#pragma unroll
                for (int i = 0; i < NCONV; ++i)
                    if (conv_slot(i) == u) conv_item(i, ready, nxt);
            }
            if (u % LOAD_EVERY == LOAD_EVERY / 2 - 1) {
                load_item(kt + DW, next, u / LOAD_EVERY);
                asm volatile("" ::: "memory");
            }
            if (u % DMA_EVERY == DMA_EVERY - 1) dma_item(kt + SA - 1, Ad, u / DMA_EVERY);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int v = NSLOT - (TROT - 1); v < NSLOT; ++v) scale_add(v, cur, T[v % TROT]);
        if (cur.oor) {
            // some column's zero point lies outside 0..15: add s (zc - z) sum_k xq,
            // with the scale/zero words of this step read again
            Regs rz;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) load_item(kt, rz, CB + cb);
            // E4M3 1.0 in every byte, made here (kept out of the loop's registers)
            const int one = static_cast<int>(opaque_vgpr(0x38383838u));
            const int8x_t ones = {one, one, one, one, one, one, one, one};
            float corr[CB];
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const float sc = half_bits_to_float(rz.s[cb]);
                const float z = half_bits_to_float(rz.s[cb] >> 16);
                corr[cb] = sc * (fminf(fmaxf(z, 0.0f), 15.0f) - z);
            }
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const float4_t t1 = mfma_f8_16x16x128(frag_a(As, rb), ones);
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[rb][cb][e] = fmaf(corr[cb], t1[e], acc[rb][cb][e]);
            }
        }
        step_end();
        }
    };

    Regs rr[DW];
    BOps oo[2];
    static_for<SA - 1>([&](auto S) {
#pragma unroll
        for (int it = 0; it < ADMA; ++it) dma_item(decltype(S)::value, stage_a(S), it);
    });
#pragma unroll
    for (int st = 0; st < DW; ++st)
#pragma unroll
        for (int it = 0; it < BLOAD; ++it) load_item(st, rr[st], it);
#pragma unroll
    for (int it = 0; it < NCONV; ++it) conv_item(it, rr[0], oo[0]);
    // the tile's row scales for the epilogue of a whole tile (a partial tile
    // leaves them to the split sum), fetched under the first steps' loads
    for (int r = tid; r < BM; r += Gm::NT) lds_xs[r] = !A16 && job.part < 0 && m_base + r < M ? p.xscale[m_base + r] : 1.0f;
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // A stages cycle with period SA, code registers with period DW and
    // converted operands with period 2: the loop body is their common period.
    // Whole rounds of U steps run with no branch between the steps, then the
    // steps left over: with a branch around every step the compiler's waits
    // for the code loads follow the worst of the joined paths, and a wave
    // waited for every load in flight (those of the steps ahead included)
    // early in each step.
    constexpr int U = lcm3(SA, DW, 2);
    int kt = 0;
    for (; kt + U <= KT; kt += U) {
        static_for<U>([&](auto I) __attribute__((always_inline)) {
            constexpr int u = decltype(I)::value;
            step(kt + u, std::integral_constant<int, u % SA>{}, rr[u % DW], rr[(u + 1) % DW], oo[u % 2],
                 oo[(u + 1) % 2]);
        });
    }
    static_for<U - 1>([&](auto I) __attribute__((always_inline)) {
        constexpr int u = decltype(I)::value;
        if (kt + u < KT)
            step(kt + u, std::integral_constant<int, u % SA>{}, rr[u % DW], rr[(u + 1) % DW], oo[u % 2],
                 oo[(u + 1) % 2]);
    });
    __builtin_amdgcn_s_waitcnt(0);
    asm volatile("" ::: "memory");

    // epilogue: register e of lane (c, q) in block (rb, cb) holds row
    // row0 + 16 rb + 4 q + e, column wcol + 16 cb + c
    if constexpr (PAIR) {
        // In two halves of the tile's rows: the up waves store their sums
        // (fp32) in the free activation stages, 64 output columns to a stage
        // ([BM / 2][64] each), the gate waves combine them with their own.
        // A row's maximum |H| goes from 16 lanes to a wave, then through LDS
        // across the gate waves.
        __shared__ float lds_amax[WC / 2][BM];
        auto su = [&](int oc, int lr) -> float& {
            float* const st = reinterpret_cast<float*>(oc < 64 ? lds_a0 : lds_a1);
            return st[lr * 64 + (oc & 63)];
        };
        static_assert(BM / 2 * 64 * 4 <= STAGE, "a half of the up sums fits a stage");
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            __syncthreads();
            if (up_wave) {
#pragma unroll
                for (int rb = hh * RB / 2; rb < (hh + 1) * RB / 2; ++rb)
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) {
                        const int oc = wcol + 16 * cb + c;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int lr = 16 * rb + 4 * q + e - hh * (BM / 2);
                            su(oc, lr) = acc[rb][cb][e];
                        }
                    }
            }
            __syncthreads();
            if (!up_wave) {
#pragma unroll
                for (int rb = hh * RB / 2; rb < (hh + 1) * RB / 2; ++rb) {
                    float hmax[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) {
                        const int oc = wcol + 16 * cb + c;
                        const int64_t col = n_base + oc;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int lr = 16 * rb + 4 * q + e;
                            const int64_t row = m_base + lr;
                            const float r = lds_xs[lr];
                            const float u = su(oc, lr - hh * (BM / 2));
                            if (row < M && col < N) {
                                const uint16_t hb = float_to_bf16_bits(activation(p.act, acc[rb][cb][e] * r) * (u * r));
                                p.Y[row * N + col] = hb;
                                hmax[e] = fmaxf(hmax[e], fabsf(bf16_lo(hb)));
                            }
                        }
                    }
                    if (p.amax_part) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float v = max16(hmax[e]);
                            if (c == 0) lds_amax[wc][16 * rb + 4 * q + e] = v;
                        }
                    }
                }
            }
        }
        if (p.amax_part) {
            __syncthreads();
            const int64_t tcol = n_base / BNO;
            for (int r = tid; r < BM; r += Gm::NT) {
                float v = 0.0f;
#pragma unroll
                for (int w = 0; w < WC / 2; ++w) v = fmaxf(v, lds_amax[w][r]);
                if (m_base + r < M) p.amax_part[(m_base + r) * p.amax_tiles + tcol] = v;
            }
        }
        return;
    }
    const bool whole = job.part < 0;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        float rsc[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) rsc[e] = lds_xs[row0 + 16 * rb + 4 * q + e];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            const int lc = wcol + 16 * cb + c;
            const int64_t col = n_base + lc;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int lr = row0 + 16 * rb + 4 * q + e;
                const int64_t row = m_base + lr;
                if (!whole) p.ws[job.part * (BM * BN) + lr * BN + lc] = acc[rb][cb][e];
                else if (row < M && col < N) p.Y[row * N + col] = float_to_bf16_bits(acc[rb][cb][e] * rsc[e]);
            }
        }
    }
}

}  // namespace

// byte offsets of the operands fit the 31-bit buffer records
bool f8_fits_buffers(int64_t M, int64_t K, int64_t N) {
    constexpr int64_t kMax = (int64_t{1} << 31) - 1;
    return M * K <= kMax && N * K / 2 <= kMax && N * (K / f8::BK) * 4 <= kMax;
}

// Output tile and K split of the fp8 kernel for an [M, K] x [N, K] product.
// Each tile shape gets the split schedule of the bf16 GEMM (with fewer tiles
// than half the compute units every tile is split along K into as many
// ranges as keep about one workgroup per compute unit, otherwise the tiles
// of the last, partial round are split; at most 16 ranges of at least four
// 128-k steps), and the shape with the least estimated time is taken:
//   rounds of whole tiles x steps x the tile's time per step
//   + the split tiles' steps x the same + the fp32 partials written and read.
// The times per 128-k step are measured on one MI355X (one workgroup per
// compute unit, all compute units busy); the partials cost about one
// microsecond per 4 MB (written, then read by the split sum: fitted to every
// tile timed on the 12B shapes from 40 to 384 rows, where it picks the
// fastest tile or one within 0.6 us of it).
#ifndef W4_F8_TILE
#define W4_F8_TILE 0      // 0: chosen by the estimate; 1..6 forces one of the tiles
#endif
namespace {
#ifndef W4_F8_DS
#define W4_F8_DS 3        // pipeline depth (SA = DW) of the tiles of 64 or 128 rows
#endif
#ifndef W4_F8_DB
#define W4_F8_DB 3        // the same for the 256-row tiles narrower than 256 columns (LDS: at most 4)
#endif
struct F8Tile {
    int bm, bn, wr, wc;
    int sa, dw;          // activation stages, code register sets
    double step_us;
};
#ifndef W4_F8_DSW
#define W4_F8_DSW W4_F8_DS
#endif
#ifndef W4_F8_DBW
#define W4_F8_DBW W4_F8_DB
#endif
constexpr int kDs = W4_F8_DS, kDb = W4_F8_DB, kDsw = W4_F8_DSW, kDbw = W4_F8_DBW;
constexpr F8Tile kF8Tiles[] = {{256, 256, 1, 8, 3, 2, 2.22},         {128, 256, 1, 8, kDs, kDsw, 1.48},
                               {256, 128, 2, 4, kDb, kDbw, 1.46},    {256, 64, 2, 4, kDb, kDbw, 0.83},
                               {64, 128, 1, 8, kDs, kDsw, 0.59},     {128, 64, 2, 4, kDs, kDsw, 0.59}};
constexpr int kF8NTiles = sizeof(kF8Tiles) / sizeof(kF8Tiles[0]);

GemmSplit f8_schedule(int t, int64_t M, int64_t K, int64_t N) {
    constexpr int64_t kCUs = 256;
    GemmSplit g{1, 0, 0, kF8Tiles[t].bm, kF8Tiles[t].bn};
    g.tiles = ((M + g.bm - 1) / g.bm) * ((N + g.bn - 1) / g.bn);
    g.t0 = g.tiles;
    const int64_t rem = g.tiles < kCUs / 2 ? g.tiles : g.tiles % kCUs;
    if (rem == 0) return g;
    int64_t s = kCUs / rem;
    if (s > (K / f8::BK) / 4) s = (K / f8::BK) / 4;
    if (s > 16) s = 16;
    if (s < 2) return g;
    g.splits = static_cast<int>(s);
    g.t0 = g.tiles - rem;
    return g;
}

double f8_estimate_us(int t, const GemmSplit& g, int64_t K) {
    constexpr int64_t kCUs = 256;
    const int64_t KT = K / f8::BK;
    double us = static_cast<double>((g.t0 + kCUs - 1) / kCUs) * KT * kF8Tiles[t].step_us;
    if (g.splits > 1) {
        us += static_cast<double>((KT + g.splits - 1) / g.splits) * kF8Tiles[t].step_us;
        us += static_cast<double>(g.tiles - g.t0) * g.splits * g.bm * g.bn * 4 / 4.0e6 + 3.0;
    }
    return us;
}

int f8_tile(int64_t M, int64_t K, int64_t N) {
    if (W4_F8_TILE >= 1 && W4_F8_TILE <= kF8NTiles) return W4_F8_TILE - 1;
    int best = 0;
    double best_us = 0.0;
    for (int t = 0; t < kF8NTiles; ++t) {
        const double us = f8_estimate_us(t, f8_schedule(t, M, K, N), K);
        if (t == 0 || us < best_us) {
            best = t;
            best_us = us;
        }
    }
    return best;
}
}  // namespace

GemmSplit f8_split(int64_t M, int64_t K, int64_t N) {
    if (M <= 0 || N <= 0 || K % f8::BK != 0) return GemmSplit{1, 0, 0, 256, 256};
    return f8_schedule(f8_tile(M, K, N), M, K, N);
}

size_t f8_workspace_bytes(int64_t M, int64_t K, int64_t N) {
    const GemmSplit g = f8_split(M, K, N);
    if (g.splits == 1) return 0;
    return static_cast<size_t>(g.tiles - g.t0) * g.splits * g.bm * g.bn * sizeof(float);
}

// The product on the tile and split of f8_split (p.splits / p.split_t0 and
// the workspace p.ws sized by f8_workspace_bytes, or splits = 1: unsplit),
// then the split sum.
hipError_t launch_gemm_f8(const MulParams& p, hipStream_t stream) {
    if (p.K % f8::BK != 0 || p.G % f8::BK != 0 || !p.x_fp8 || !p.xscale || !f8_fits_buffers(p.M, p.K, p.N))
        return hipErrorInvalidValue;
    if (p.M == 0 || p.N == 0) return hipSuccess;
    const GemmSplit g = f8_split(p.M, p.K, p.N);
    MulParams q = p;
    if (q.splits <= 1) {
        q.splits = 1;
        q.split_t0 = g.tiles;
        q.ws = nullptr;
    } else if (q.splits != g.splits || q.split_t0 != g.t0 || !q.ws) {
        return hipErrorInvalidValue;
    }
    const dim3 grid(static_cast<unsigned>(q.split_t0 + (g.tiles - q.split_t0) * q.splits));
    const int t = f8_tile(p.M, p.K, p.N);
    const dim3 block(static_cast<unsigned>(64 * kF8Tiles[t].wr * kF8Tiles[t].wc));
    switch (t) {
        case 0: hipLaunchKernelGGL((gemm_f8_kernel<256, 256, 1, 8>), grid, block, 0, stream, q); break;
#define W4_F8_LAUNCH(T)                                                                                         \
    hipLaunchKernelGGL((gemm_f8_kernel<kF8Tiles[T].bm, kF8Tiles[T].bn, kF8Tiles[T].wr, kF8Tiles[T].wc, false,      \
                                       kF8Tiles[T].sa, kF8Tiles[T].dw>),                                           \
                       grid, block, 0, stream, q)
        case 1: W4_F8_LAUNCH(1); break;
        case 2: W4_F8_LAUNCH(2); break;
        case 3: W4_F8_LAUNCH(3); break;
        case 4: W4_F8_LAUNCH(4); break;
        default: W4_F8_LAUNCH(5); break;
#undef W4_F8_LAUNCH
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || q.splits == 1) return e;
    return launch_split_sum(q, g.bm, g.bn, g.tiles, stream);
}

// W4A16 with groups of 128 on the same kernel's 64 x 128 or 128 x 128 tiles
// (bf16 activations, A16), in place of the mid-size kernel for up to 128
// rows: its K split (fp32 partial tiles in the same layout, each range a
// whole number of 128-k steps) within its workspace.
bool a16_eligible(int64_t M, int64_t K, int64_t N, int G) {
    return M > 0 && M <= 128 && K % f8::BK == 0 && G % f8::BK == 0 && f8_fits_buffers(2 * M, K, N);
}
// 64-row tiles up to 64 rows, 128-row tiles above (each weight converted
// once per tile: 8B and 12B shapes at M = 96 / 128 1-2 us faster, 3-5%)
#ifndef W4_A16_BM128_FROM
#define W4_A16_BM128_FROM 64
#endif
int a16_tile_rows(int64_t M) { return M > W4_A16_BM128_FROM ? 128 : 64; }
hipError_t launch_gemm_a16(const MulParams& p, hipStream_t stream) {
    if (p.x_fp8 || !a16_eligible(p.M, p.K, p.N, p.G)) return hipErrorInvalidValue;
    const int BM = a16_tile_rows(p.M);
    constexpr int BN = 128;
    const int64_t tiles = ((p.N + BN - 1) / BN) * ((p.M + BM - 1) / BM);
    MulParams q = p;
    if (q.splits <= 1) {
        q.splits = 1;
        q.split_t0 = tiles;
        q.ws = nullptr;
    }
    if (q.splits > q.K / f8::BK || q.split_t0 < 0 || q.split_t0 > tiles || (q.splits > 1 && !q.ws))
        return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(q.split_t0 + (tiles - q.split_t0) * q.splits));
    if (BM == 128)
        hipLaunchKernelGGL((gemm_f8_kernel<128, BN, 1, 8, false, 3, 3, true>), grid, dim3(512), 0, stream, q);
    else
        hipLaunchKernelGGL((gemm_f8_kernel<64, BN, 1, 8, false, 3, 3, true>), grid, dim3(512), 0, stream, q);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || q.splits == 1) return e;
    return launch_split_sum(q, BM, BN, tiles, stream);
}

// W4A16 gate and up with groups of 128 from 33 to 256 rows on the
// bf16-activation form: tiles of 64 or 128 rows by 128 output columns (256
// weight columns, 128 of each weight), no K split, in place of the mid-size
// pair kernel.
bool a16_pair_eligible(int64_t M, int64_t K, int64_t N, int G) {
    return M > 0 && M <= 256 && K % f8::BK == 0 && G % f8::BK == 0 && f8_fits_buffers(2 * M, K, N);
}
hipError_t launch_gemm_a16_pair(const MulParams& p, hipStream_t stream) {
    if (p.x_fp8 || !p.wq2 || !p.sz2 || !a16_pair_eligible(p.M, p.K, p.N, p.G)) return hipErrorInvalidValue;
// 64-row tiles up to 128 rows, 128-row tiles above (8B shapes at M = 200 /
// 256: 87.7 / 91.5 -> 79.1 / 82.4 us; at 128 rows the 64-row tiles are
// faster, 50 against 75 us)
#ifndef W4_A16_PAIR_BM128_FROM
#define W4_A16_PAIR_BM128_FROM 128
#endif
    const int bm = p.M > W4_A16_PAIR_BM128_FROM ? 128 : 64;
    MulParams q = p;
    const int64_t tiles = ((p.N + 127) / 128) * ((p.M + bm - 1) / bm);
    q.splits = 1;
    q.split_t0 = tiles;
    q.ws = nullptr;
    if (bm == 128)
        hipLaunchKernelGGL((gemm_f8_kernel<128, 256, 1, 8, true, 3, 3, true>), dim3(static_cast<unsigned>(tiles)), dim3(512),
                           0, stream, q);
    else
        hipLaunchKernelGGL((gemm_f8_kernel<64, 256, 1, 8, true, 3, 3, true>), dim3(static_cast<unsigned>(tiles)), dim3(512),
                           0, stream, q);
    return hipGetLastError();
}

// Gate and up on the fp8 kernel: tiles of BM rows by 128 output columns
// (256 weight columns: 128 of each weight), the most rows that still give
// about one workgroup per compute unit; no K split.
hipError_t launch_gemm_f8_pair(const MulParams& p, hipStream_t stream) {
    if (p.K % f8::BK != 0 || p.G % f8::BK != 0 || !p.x_fp8 || !p.xscale || !p.wq2 || !p.sz2 ||
        !f8_fits_buffers(p.M, p.K, p.N))
        return hipErrorInvalidValue;
    if (p.M == 0 || p.N == 0) return hipSuccess;
    const int64_t nt = (p.N + 127) / 128;
    const int bm = ((p.M + 255) / 256) * nt >= 224 ? 256 : (((p.M + 127) / 128) * nt >= 224 ? 128 : 64);
    MulParams q = p;
    const int64_t tiles = ((p.M + bm - 1) / bm) * nt;
    q.splits = 1;
    q.split_t0 = tiles;
    q.ws = nullptr;
    const dim3 grid(static_cast<unsigned>(tiles));
    if (bm == 256)
        hipLaunchKernelGGL((gemm_f8_kernel<256, 256, 1, 8, true>), grid, dim3(512), 0, stream, q);
    else if (bm == 128)
        hipLaunchKernelGGL((gemm_f8_kernel<128, 256, 1, 8, true>), grid, dim3(512), 0, stream, q);
    else
        hipLaunchKernelGGL((gemm_f8_kernel<64, 256, 1, 8, true>), grid, dim3(512), 0, stream, q);
    return hipGetLastError();
}

}  // namespace w4
