// W4A16 / W4A8 products for small M (1 to 64 activation rows) on gfx950.
//
// With few activation rows the product is bound by streaming the packed
// weights from HBM (gsantana.dev "Quantizing LLMs Without Guesswork",
// "Production reality": small batches are memory-bound; decode reads every
// weight once).  One kernel family covers the range; it differs only in how a
// step is multiplied.
//
// Work decomposition.  A workgroup owns 16 * FJ output columns (FJ 16-row
// blocks of the blocked weight layout) and all M rows; its wk waves split K:
// wave w takes the 128-wide K steps w, w + wk, ...  No weight is shared
// between waves, so the weights go from global memory straight into
// registers: in a step, lane l (column c = l % 16 of a block, quarter
// h = l / 16) loads the 16 bytes holding k = 32h .. 32h + 31 of its column --
// in the blocked layout the 64 lanes' pieces are one contiguous 1 KB.  A wave
// issues the loads of kDepth steps together, then multiplies them; the other
// waves on the compute unit cover the latency.  At the end the wk partial
// sums are added through LDS in a fixed order.
//
// Multiplying a step:
//  * one or two rows (v_dot2_f32_bf16): the lane's codes become bf16 pairs
//    128 + u with one AND-OR and are dotted with its 32 activations; the
//    group's scale and zero are applied per lane (its 32 k lie in one group)
//    as s (sum x (128 + u) - (128 + z) sum x).  The activations and their
//    32-k sums are staged in LDS once per workgroup when they fit, else every
//    lane loads its own.
//  * more rows, groups of 128 (v_mfma_f32_16x16x32_bf16): the same exact
//    values 128 + u times the activations, plus an MFMA of the activations
//    against ones for sum x over the group, then the same correction per
//    output.  MFMA b of a step multiplies, from every quarter h, the 8 k at
//    32h + 8b, and the activation fragments use the same order.
//  * more rows, groups of 32 or 64: every weight dequantized, W' = (1024 + u)
//    s - (1024 + z) s (fp16 1024 + u by one AND-OR, two mixed-precision FMAs,
//    exact before one rounding to bf16), then the MFMA.
//
// W4A8 reads the E4M3 activation codes, widens them exactly to bf16 and
// applies the row scale at the end (gowda.ai "LLM fast inference",
// "Achievement 2").
#include <type_traits>

#include "device.hpp"
#include "kernels.hpp"

namespace w4 {
namespace {

typedef float float4_v __attribute__((ext_vector_type(4)));

constexpr int kStepK = 128;   // k per wave and step (4 quarters of 32)

// weight steps in flight per wave (fewer with more activation rows, whose
// fragments take the registers)
#ifndef W4_SK_DEPTH
#define W4_SK_DEPTH 2
#endif
#ifndef W4_DOT_DEPTH
#define W4_DOT_DEPTH 4
#endif
#ifndef W4_DOTL_DEPTH
#define W4_DOTL_DEPTH 2
#endif
template <int MB, int MODE>
constexpr int skinny_depth() {
    return MODE >= 3 ? W4_DOTL_DEPTH : (MODE == 2 ? W4_DOT_DEPTH : (MB == 1 ? W4_SK_DEPTH : 2));
}

// weights of one step: the lane's 16 bytes of codes and its scale/zero word,
// per 16-column block
template <int FJ>
struct SkinnyB {
    u32x4_t q[FJ];          // codes of k = 32h .. 32h + 31 of the lane's column
    uint32_t s[FJ];         // scale | zero << 16
};
// activations of one step: k = 32h .. 32h + 31 of the lane's row, per 16-row block
template <int MB, bool XF8>
struct SkinnyA {
    static constexpr int AL = XF8 ? 2 : 4;   // 16-byte loads per block
    u32x4_t a[MB][AL];
    bool valid;             // the lane's quarter lies inside K (else its products are dropped)
};

// how a step is multiplied
constexpr int kDeq = 0;    // dequantize every weight to bf16, MFMA (groups of 32 or 64)
constexpr int kCorr = 1;   // MFMA on 128 + u, per-group correction (groups of 128)
constexpr int kDot = 2;    // v_dot2 on 128 + u, per-group correction (one or two rows)
constexpr int kDotLds = 3; // the same, activations and their 32-k sums staged in LDS once
constexpr int kDotLdsQ = 4; // the same for W4A8, quantizing the bf16 rows to E4M3 while staging
constexpr int kDotMaxM = 2;

// up to 16 waves per workgroup for the one-row dot form (few registers), 8 otherwise
template <int MB, int MODE>
constexpr int skinny_max_threads() { return MODE == kDotLds || MODE == kDotLdsQ ? 1024 : 512; }

template <int MB, int FJ, bool XF8, int MODE>
__global__ void __launch_bounds__((skinny_max_threads<MB, MODE>())) gemm_skinny_kernel(MulParams p, int wk) {
    constexpr bool CORR = MODE == kCorr, QX = MODE == kDotLdsQ, DOTL = MODE == kDotLds || QX,
                   DOT = MODE == kDot || DOTL;
    static_assert(!QX || XF8, "in-kernel row quantization is the W4A8 product");
    using BStage = SkinnyB<FJ>;
    using AStage = SkinnyA<MB, XF8>;
    constexpr int AL = AStage::AL;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 15, h = lane >> 4;
    const int64_t M = p.M, N = p.N, K = p.K;
    // gate and up in one pass: both blocks cover the same 16 columns (FJ = 2)
    const bool pair = p.wq2 != nullptr;
    const int KS = static_cast<int>((K + kStepK - 1) / kStepK);
    // K split across workgroups (MFMA forms, p.splits > 1): workgroup b
    // covers column block b % nblk and the steps [ks0, ks1) of K range
    // b / nblk, and writes fp32 partial sums to ws [range][M][N]
    const int64_t cols = pair ? 16 : 16 * FJ;
    const int64_t nblk = (N + cols - 1) / cols;
    const bool ksplit = !DOT && p.splits > 1;
    const int kr = ksplit ? static_cast<int>(blockIdx.x / nblk) : 0;
    const int ks0 = ksplit ? kr * KS / p.splits : 0;
    const int ks1 = ksplit ? (kr + 1) * KS / p.splits : KS;
    const int64_t n0 = (ksplit ? blockIdx.x % nblk : static_cast<int64_t>(blockIdx.x)) * cols;
    const int64_t words_row = K / 8, groups_row = K / p.G;
    const int g_shift = group_shift(p.G);

    // lane's column in each block and row in each 16-row block (clamped:
    // columns past N and rows past M compute values that are never stored)
    // the lane's row c in each 16-row block of the blocked GPU layout: its
    // 16-byte piece of tile t is at word 4 c + 4 nr t of the block, its
    // scale/zero word of group g at c + nr g (nr = rows in the block; rows
    // past N read the block's last row and give values never stored)
    // (offsets within a block fit 32 bits; the per-step parts are uniform)
    const uint8_t* bblk[FJ];                           // block bases (uniform)
    const uint8_t* sblk[FJ];
    uint32_t qlane[FJ], slane[FJ];                     // the lane's byte offsets in a tile
    int bnr[FJ];
#pragma unroll
    for (int j = 0; j < FJ; ++j) {
        int64_t r0 = pair ? n0 : n0 + 16 * j;
        r0 = r0 < N ? r0 : ((N - 1) / 16) * 16;
        const int nr = static_cast<int>(N - r0 < 16 ? N - r0 : 16);
        const int cc = c < nr ? c : nr - 1;
        const uint32_t* wq = pair && j == 1 ? p.wq2 : p.wq;
        const uint32_t* szp = pair && j == 1 ? p.sz2 : p.sz;
        bblk[j] = reinterpret_cast<const uint8_t*>(wq + r0 * words_row);
        sblk[j] = reinterpret_cast<const uint8_t*>(szp + r0 * groups_row);
        qlane[j] = 16 * cc;
        slane[j] = 4 * cc;
        bnr[j] = __builtin_amdgcn_readfirstlane(nr);
    }
    const int KQ = static_cast<int>(K / 32);          // 32-k quarters (tiles) per row
    const int KQ4 = (KQ + 3) & ~3;                    // padded to whole steps (LDS staging)
    const int q_shift = g_shift - 5;                  // tile -> group
    // activation rows: the MFMA forms give lane (c, h) row c of every 16-row
    // block; the dot form gives every lane all MB rows
    const uint8_t* arow[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
        int64_t m = DOT ? i : 16 * i + c;
        m = m < M ? m : M - 1;
        arow[i] = static_cast<const uint8_t*>(p.X) + m * K * (XF8 ? 1 : 2);
    }

    auto load_b = [&](int step, BStage& st) {
        // the lane's tile; past K (a multiple of 32 but not of 128) the lane
        // reads the last tile, whose products meet zero activations
        const int t = 4 * step + h;
        const uint32_t tq = static_cast<uint32_t>(t < KQ ? t : KQ - 1);
        const uint32_t g = tq >> q_shift;
#pragma unroll
        for (int j = 0; j < FJ; ++j) {
            // 32-bit byte offsets from uniform bases (a block spans K nr / 2 bytes)
            st.q[j] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4_t*>(bblk[j] + (__umul24(tq, 16 * bnr[j]) + qlane[j])));
            st.s[j] = *reinterpret_cast<const uint32_t*>(sblk[j] + (__umul24(g, 4 * bnr[j]) + slane[j]));
        }
    };
    auto load_a = [&](int step, AStage& st) {
        const int tq0 = 4 * step + h;
        const bool valid = tq0 < KQ;
        const int tq = valid ? tq0 : 0;
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            const u32x4_t* ap = reinterpret_cast<const u32x4_t*>(arow[i] + tq * (XF8 ? 32 : 64));
#pragma unroll
            for (int t = 0; t < AL; ++t) st.a[i][t] = ap[t];
        }
        // applied when the step is multiplied: touching the loaded values
        // here would make the wave wait for the loads at once
        st.valid = valid;
    };

    float4_v acc[MB][FJ];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j) acc[i][j] = float4_v{0.0f, 0.0f, 0.0f, 0.0f};

    // Activation fragment b (8 k) of 16-row block i as bf16 (E4M3 codes are
    // widened exactly; a quarter outside K contributes zeros).
    auto a_frag = [&](const AStage& sa, int i, int b) -> bf16x8_t {
        if constexpr (!XF8) {
            return __builtin_bit_cast(bf16x8_t, sa.valid ? sa.a[i][b] : u32x4_t{0u, 0u, 0u, 0u});
        } else {
            const u32x4_t v = sa.valid ? sa.a[i][b / 2] : u32x4_t{0u, 0u, 0u, 0u};
            const uint32_t w0 = (b & 1) ? v[2] : v[0];
            const uint32_t w1 = (b & 1) ? v[3] : v[1];
            const float2_t f0 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w0), false);
            const float2_t f1 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w0), true);
            const float2_t f2 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w1), false);
            const float2_t f3 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w1), true);
            return __builtin_bit_cast(bf16x8_t, u32x4_t{pack_bf16x2(f0[0], f0[1]), pack_bf16x2(f1[0], f1[1]),
                                                        pack_bf16x2(f2[0], f2[1]), pack_bf16x2(f3[0], f3[1])});
        }
    };

    const uint32_t bias16 = opaque_vgpr(0x64006400u);   // two fp16 1024.0
    const uint32_t bias128 = opaque_vgpr(kBf16Bias128x2);
    // dot form with staged activations: LDS holds, per row, the activations
    // as bf16 pairs ([MB][16 KQ4] words) and the sum of every 32-k quarter
    // ([MB][KQ4] floats), both zero past K up to a whole step; the partial
    // sums of the final reduction follow
    extern __shared__ float red[];
    uint32_t* const lds_x = reinterpret_cast<uint32_t*>(red);
    float* const lds_xs = red + (DOTL ? MB * 16 * KQ4 : 0);
    float* const red_base = DOTL ? lds_xs + MB * KQ4 : red;
    float row_scale[MB];                    // in-kernel W4A8 row scales (QX)

    auto compute = [&](const BStage& st, const AStage& sa, int step) {
        if constexpr (DOT) {
            // the lane's 32 activations of every row as bf16 pairs in k order
            uint32_t xw[MB][16];
            float xs[MB];
            if constexpr (DOTL) {
                const int kq = 4 * step + h;          // the lane's 32-k quarter (zeros past K)
#pragma unroll
                for (int m = 0; m < MB; ++m) {
                    const u32x4_t* xp = reinterpret_cast<const u32x4_t*>(lds_x + m * (16 * KQ4) + kq * 16);
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const u32x4_t v = xp[t];
#pragma unroll
                        for (int e = 0; e < 4; ++e) xw[m][4 * t + e] = v[e];
                    }
                    xs[m] = lds_xs[m * KQ4 + kq];
                }
            }
#pragma unroll
            for (int m = 0; m < MB && !DOTL; ++m) {
                if constexpr (!XF8) {
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const u32x4_t v = sa.valid ? sa.a[m][t] : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
                        for (int e = 0; e < 4; ++e) xw[m][4 * t + e] = v[e];
                    }
                } else {
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const u32x4_t v = sa.valid ? sa.a[m][t] : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float2_t f0 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(v[e]), false);
                            const float2_t f1 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(v[e]), true);
                            xw[m][8 * t + 2 * e] = pack_bf16x2(f0[0], f0[1]);
                            xw[m][8 * t + 2 * e + 1] = pack_bf16x2(f1[0], f1[1]);
                        }
                    }
                }
            }
            // sum of the 32 activations of every row (the lane's 32 k lie in
            // one group); four partial sums per chain keep the dependent
            // dot products apart
#pragma unroll
            for (int m = 0; m < MB && !DOTL; ++m) {
                float t[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int w = 0; w < 16; ++w) t[w & 3] = dot2_bf16(xw[m][w], 0x3F803F80u, t[w & 3]);
                xs[m] = (t[0] + t[1]) + (t[2] + t[3]);
            }
            // one chain per output: it starts at -(128 + z) sum x and adds
            // the products of the 32 exact values 128 + u
#pragma unroll
            for (int j = 0; j < FJ; ++j) {
                const float sc = half_bits_to_float(st.s[j]);
                const float zc = 128.0f + half_bits_to_float(st.s[j] >> 16);
                float d[MB];
#pragma unroll
                for (int m = 0; m < MB; ++m) d[m] = -zc * xs[m];
#pragma unroll
                for (int b = 0; b < 4; ++b)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t pr = nibble_pair_bf16(st.q[j][b], i, bias128);
#pragma unroll
                        for (int m = 0; m < MB; ++m) d[m] = dot2_bf16(pr, xw[m][4 * b + i], d[m]);
                    }
#pragma unroll
                for (int m = 0; m < MB; ++m) acc[m][j][0] = fmaf(sc, d[m], acc[m][j][0]);
            }
        } else if constexpr (CORR) {
            // One group per step (G = 128): multiply the exact bf16 values
            // 128 + u, and the row sums of x over the group (an MFMA against
            // ones), then acc += s (P - (128 + z) sum x) for every output.
            const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
            float4_v ps[MB][FJ], xs[MB];
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                xs[i] = float4_v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int j = 0; j < FJ; ++j) ps[i][j] = float4_v{0.0f, 0.0f, 0.0f, 0.0f};
            }
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                bf16x8_t bp[FJ];
#pragma unroll
                for (int j = 0; j < FJ; ++j) {
                    const uint32_t w = st.q[j][b];
                    bp[j] = __builtin_bit_cast(bf16x8_t, u32x4_t{nibble_pair_bf16(w, 0, bias128), nibble_pair_bf16(w, 1, bias128),
                                                                 nibble_pair_bf16(w, 2, bias128), nibble_pair_bf16(w, 3, bias128)});
                }
#pragma unroll
                for (int i = 0; i < MB; ++i) {
                    const bf16x8_t ap = a_frag(sa, i, b);
                    xs[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ap, ones, xs[i], 0, 0, 0);
#pragma unroll
                    for (int j = 0; j < FJ; ++j)
                        ps[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ap, bp[j], ps[i][j], 0, 0, 0);
                }
            }
#pragma unroll
            for (int j = 0; j < FJ; ++j) {
                const float sc = half_bits_to_float(st.s[j]);
                const float zc = 128.0f + half_bits_to_float(st.s[j] >> 16);
#pragma unroll
                for (int i = 0; i < MB; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[i][j][e] = fmaf(sc, fmaf(-zc, xs[i][e], ps[i][j][e]), acc[i][j][e]);
            }
        } else {
            // Groups smaller than a step: dequantize every weight, W' =
            // (1024 + u) s - (1024 + z) s rounded once to bf16.
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                bf16x8_t bp[FJ];
#pragma unroll
                for (int j = 0; j < FJ; ++j) {
                    const float sc = half_bits_to_float(st.s[j]);
                    const float cs = -(1024.0f + half_bits_to_float(st.s[j] >> 16)) * sc;
                    const uint32_t w = st.q[j][b];
                    uint32_t o[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t hw = ((w >> (4 * i)) & 0x000F000Fu) | bias16;
                        const _Float16 lo = __builtin_bit_cast(_Float16, static_cast<uint16_t>(hw & 0xFFFFu));
                        const _Float16 hi = __builtin_bit_cast(_Float16, static_cast<uint16_t>(hw >> 16));
                        o[i] = pack_bf16x2(fmaf(static_cast<float>(lo), sc, cs), fmaf(static_cast<float>(hi), sc, cs));
                    }
                    bp[j] = __builtin_bit_cast(bf16x8_t, u32x4_t{o[0], o[1], o[2], o[3]});
                }
#pragma unroll
                for (int i = 0; i < MB; ++i) {
                    const bf16x8_t ap = a_frag(sa, i, b);
#pragma unroll
                    for (int j = 0; j < FJ; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ap, bp[j], acc[i][j], 0, 0, 0);
                }
            }
        }
    };

    // Steps wave, wave + wk, ... in rounds of kDepth: a round issues the
    // loads of its steps together (weights, and activations unless they are
    // staged in LDS), then multiplies them in order.  Nothing is loaded that
    // is not used, and the latency of one round is covered by the other waves
    // on the compute unit.  The empty asm with a memory clobber after the
    // loads keeps the optimizer from sinking them down to their use, and the
    // scheduling barrier keeps the multiplications after them.
    constexpr int kDepth = skinny_depth<MB, MODE>();
    BStage bq[kDepth];
    AStage aq[kDepth];
    auto issue = [&](int step) {
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
            const int st = step + d * wk;
            if constexpr (DOTL) {
                // unconditional, so that each multiplication waits only for
                // its own step: a step past K reloads the last one (a cache
                // hit) and is not multiplied
                load_b(st < KS ? st : KS - 1, bq[d]);
            } else if (st < ks1) {
                load_b(st, bq[d]);
                load_a(st, aq[d]);
            }
        }
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };
    int step = ks0 + wave;               // every wave has at least one step
    // With staged activations their first loads go out before the weights':
    // loads return in order, so the staging below waits for these alone and
    // not for the weights in flight.  A thread's first quarter of each row
    // (W4A8 with the rows quantized here: its first kPreQ 16-byte units).
    constexpr int kPreQ = 2;
    constexpr int kPre = QX ? kPreQ : (XF8 ? 2 : 4);
    u32x4_t xpre[MB][kPre];
    if constexpr (DOTL) {
#pragma unroll
        for (int m = 0; m < MB; ++m) {
            const int64_t row = m < M ? m : M - 1;
#pragma unroll
            for (int i = 0; i < kPre; ++i) {
                // unconditional (a piece past the row reloads its last one and
                // is not used): a select would make the staging wait for the
                // weights as well
                int64_t piece = QX ? static_cast<int64_t>(threadIdx.x) + static_cast<int64_t>(i) * blockDim.x
                                   : static_cast<int64_t>(threadIdx.x < static_cast<unsigned>(KQ) ? threadIdx.x : KQ - 1) * kPre + i;
                if (QX && piece >= 4 * static_cast<int64_t>(KQ)) piece = 4 * static_cast<int64_t>(KQ) - 1;
                xpre[m][i] = reinterpret_cast<const u32x4_t*>(static_cast<const uint8_t*>(p.X) + row * K * (XF8 && !QX ? 1 : 2))[piece];
            }
        }
    }
    issue(step);
    if constexpr (DOTL) {
        // stage the activations while the first weights are in flight:
        // unit u = one 32-k quarter of one row (64 bytes of bf16 or 32 of
        // E4M3, widened exactly), stored as 16 bf16 pairs with its sum
        if constexpr (QX) {
            // W4A8 rows quantized here, with the arithmetic of the row
            // quantizer: scale = max(max |x| / 448, 1e-8), codes =
            // e4m3(clamp(x / scale, +-448)) (round to nearest even; the
            // quotient from e4m3_quotient, whose codes are those of the
            // correctly rounded one); the codes, widened exactly to bf16, are
            // what the products use.  Workgroup 0 also writes the codes and
            // scales out.  A lane takes one 16-byte unit (eight values)
            // at a time; the four units of a quarter sit in four neighbouring
            // lanes, which add their sums of the widened codes.  Those sums
            // are exact in any order: 32 E4M3 values are multiples of 2^-9
            // below 2^14 in magnitude, which fp32 holds exactly.
            __shared__ float wave_amax[kDotMaxM][16];
            const int KU = 4 * KQ;                    // 16-byte units per row
            float amax[MB];
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                amax[m] = 0.0f;
                auto take = [&](int u, const u32x4_t& v) {
                    *reinterpret_cast<u32x4_t*>(lds_x + m * (16 * KQ4) + 4 * u) = v;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        amax[m] = fmaxf(fmaxf(amax[m], fabsf(bf16_lo(v[e]))), fabsf(bf16_hi(v[e])));
                };
#pragma unroll
                for (int i = 0; i < kPreQ; ++i) {
                    const int u = threadIdx.x + i * blockDim.x;
                    if (u < KU) take(u, xpre[m][i]);
                }
                for (int u = threadIdx.x + kPreQ * blockDim.x; u < KU; u += blockDim.x)
                    take(u, *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(p.X) + static_cast<int64_t>(m) * K + 8 * u));
                amax[m] = wave_max(amax[m]);
                if (lane == 0) wave_amax[m][wave] = amax[m];
            }
            __syncthreads();
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                float a = 0.0f;
                for (int w = 0; w < wk; ++w) a = fmaxf(a, wave_amax[m][w]);
                float sc = a / 448.0f;
                sc = fmaxf(sc, 1e-8f);
                row_scale[m] = sc;
                const float rsc = 1.0f / sc;
                if (blockIdx.x == 0 && threadIdx.x == 0) p.xscale_out[m] = sc;
                // KU is a multiple of 4 and the stride a multiple of 64, so
                // the four lanes of a quarter enter and leave together
                for (int u = threadIdx.x; u < KU; u += blockDim.x) {
                    u32x4_t* buf = reinterpret_cast<u32x4_t*>(lds_x + m * (16 * KQ4) + 4 * u);
                    const u32x4_t v = *buf;
                    u32x4_t wv;
                    uint32_t codes[2];
                    float t2[2] = {0.0f, 0.0f};
#pragma unroll
                    for (int e = 0; e < 4; e += 2) {
                        const float f0 = fminf(fmaxf(e4m3_quotient(bf16_lo(v[e]), sc, rsc), -448.0f), 448.0f);
                        const float f1 = fminf(fmaxf(e4m3_quotient(bf16_hi(v[e]), sc, rsc), -448.0f), 448.0f);
                        const float f2 = fminf(fmaxf(e4m3_quotient(bf16_lo(v[e + 1]), sc, rsc), -448.0f), 448.0f);
                        const float f3 = fminf(fmaxf(e4m3_quotient(bf16_hi(v[e + 1]), sc, rsc), -448.0f), 448.0f);
                        int c4 = __builtin_amdgcn_cvt_pk_fp8_f32(f0, f1, 0, false);
                        c4 = __builtin_amdgcn_cvt_pk_fp8_f32(f2, f3, c4, true);
                        codes[e / 2] = static_cast<uint32_t>(c4);
                        const float2_t g0 = __builtin_amdgcn_cvt_pk_f32_fp8(c4, false);
                        const float2_t g1 = __builtin_amdgcn_cvt_pk_f32_fp8(c4, true);
                        wv[e] = pack_bf16x2(g0[0], g0[1]);
                        wv[e + 1] = pack_bf16x2(g1[0], g1[1]);
                        t2[0] = dot2_bf16(wv[e], 0x3F803F80u, t2[0]);
                        t2[1] = dot2_bf16(wv[e + 1], 0x3F803F80u, t2[1]);
                    }
                    *buf = wv;
                    float qs = t2[0] + t2[1];
                    qs += __shfl_xor(qs, 1, kWave);
                    qs += __shfl_xor(qs, 2, kWave);
                    if ((u & 3) == 0) lds_xs[m * KQ4 + (u >> 2)] = qs;
                    if (blockIdx.x == 0)
                        *reinterpret_cast<u32x2_t*>(p.xq_out + static_cast<int64_t>(m) * K + 8 * u) = u32x2_t{codes[0], codes[1]};
                }
            }
        } else {
            // quarter q of row m from its 16-byte pieces (4 of bf16, 2 of E4M3)
            auto stage = [&](int m, int q, const u32x4_t* vs) {
                uint32_t w[16];
                if constexpr (!XF8) {
#pragma unroll
                    for (int t = 0; t < 4; ++t)
#pragma unroll
                        for (int e = 0; e < 4; ++e) w[4 * t + e] = vs[t][e];
                } else {
#pragma unroll
                    for (int t = 0; t < 2; ++t)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float2_t f0 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(vs[t][e]), false);
                            const float2_t f1 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(vs[t][e]), true);
                            w[8 * t + 2 * e] = pack_bf16x2(f0[0], f0[1]);
                            w[8 * t + 2 * e + 1] = pack_bf16x2(f1[0], f1[1]);
                        }
                }
                float t4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int i = 0; i < 16; ++i) t4[i & 3] = dot2_bf16(w[i], 0x3F803F80u, t4[i & 3]);
                u32x4_t* dst = reinterpret_cast<u32x4_t*>(lds_x + m * (16 * KQ4) + 16 * q);
#pragma unroll
                for (int t = 0; t < 4; ++t) dst[t] = u32x4_t{w[4 * t], w[4 * t + 1], w[4 * t + 2], w[4 * t + 3]};
                lds_xs[m * KQ4 + q] = (t4[0] + t4[1]) + (t4[2] + t4[3]);
            };
            // the thread's first quarter, loaded before the weights, on its
            // own (a later quarter's load waits for the weights in flight)
#pragma unroll
            for (int m = 0; m < MB; ++m)
                if (static_cast<int>(threadIdx.x) < KQ) stage(m, threadIdx.x, xpre[m]);
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                const int64_t row = m < M ? m : M - 1;
                for (int q = threadIdx.x + blockDim.x; q < KQ; q += blockDim.x) {
                    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(static_cast<const uint8_t*>(p.X) +
                                                                          (row * K + 32 * q) * (XF8 ? 1 : 2));
                    u32x4_t vs[kPre];
#pragma unroll
                    for (int t = 0; t < kPre; ++t) vs[t] = src[t];
                    stage(m, q, vs);
                }
            }
        }
        // zero quarters past K up to a whole step
#pragma unroll
        for (int m = 0; m < MB; ++m)
            for (int q = KQ + static_cast<int>(threadIdx.x); q < KQ4; q += blockDim.x) {
                u32x4_t* dst = reinterpret_cast<u32x4_t*>(lds_x + m * (16 * KQ4) + 16 * q);
#pragma unroll
                for (int t = 0; t < 4; ++t) dst[t] = u32x4_t{0u, 0u, 0u, 0u};
                lds_xs[m * KQ4 + q] = 0.0f;
            }
        __syncthreads();
    }
    if constexpr (DOTL) {
        // Rolling pipeline: each buffer is refilled with the step kDepth
        // ahead as soon as it has been multiplied, so kDepth steps stay in
        // flight.  While every refill is a real step the loads are
        // unconditional (each multiplication waits only for its own step);
        // the last two rounds guard them.
        const int n = (KS - wave + wk - 1) / wk;      // steps of this wave
        int i = 0;
        for (; i + 2 * kDepth <= n; i += kDepth) {
#pragma unroll
            for (int d = 0; d < kDepth; ++d) {
                compute(bq[d], aq[d], step + d * wk);
                load_b(step + (kDepth + d) * wk, bq[d]);
                asm volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
            }
            step += kDepth * wk;
        }
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
            if (i + d < n) compute(bq[d], aq[d], step + d * wk);
            if (i + kDepth + d < n) load_b(step + (kDepth + d) * wk, bq[d]);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
        }
        step += kDepth * wk;
        i += kDepth;
#pragma unroll
        for (int d = 0; d < kDepth; ++d)
            if (i + d < n) compute(bq[d], aq[d], step + d * wk);
    } else {
        while (true) {
#pragma unroll
            for (int d = 0; d < kDepth; ++d)
                if (step + d * wk < ks1) compute(bq[d], aq[d], step + d * wk);
            step += kDepth * wk;
            if (step >= ks1) break;
            issue(step);
        }
    }

    if constexpr (DOT) {
        // sum the four quarters of every column (lanes c, c + 16, c + 32,
        // c + 48), then the wk waves through LDS ([wk][MB][16 FJ]) in wave order
        constexpr int TILE = 16 * MB * FJ;
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int j = 0; j < FJ; ++j) {
                float v = acc[m][j][0];
                v += __shfl_xor(v, 16, kWave);
                v += __shfl_xor(v, 32, kWave);
                if (h == 0) red_base[wave * TILE + m * 16 * FJ + 16 * j + c] = v;
            }
        __syncthreads();
        auto row_factor = [&](int row) -> float {
            if constexpr (QX) return row == 0 ? row_scale[0] : row_scale[MB - 1];
            else if constexpr (XF8) return p.xscale[row];
            else return 1.0f;
        };
        if (pair) {
            // output (row, c): act(gate) * up from blocks 0 and 1
            for (int o = threadIdx.x; o < 16 * MB; o += blockDim.x) {
                const int row = o / 16, cc = o % 16;
                float g = 0.0f, u = 0.0f;
                for (int w = 0; w < wk; ++w) {
                    g += red_base[w * TILE + row * 16 * FJ + cc];
                    u += red_base[w * TILE + row * 16 * FJ + 16 + cc];
                }
                const int64_t n = n0 + cc;
                float hv = 0.0f;
                if (row < M && n < N) {
                    const float r = row_factor(row);
                    const uint16_t hb = float_to_bf16_bits(activation(p.act, g * r) * (u * r));
                    p.Y[static_cast<int64_t>(row) * N + n] = hb;
                    hv = fabsf(bf16_lo(hb));
                }
                if (p.amax_part) {
                    // the row's maximum |H| over this workgroup's 16 columns
                    // (16 consecutive threads hold one row)
                    hv = max16(hv);
                    if (cc == 0 && row < M) p.amax_part[static_cast<int64_t>(row) * p.amax_tiles + blockIdx.x] = hv;
                }
            }
            return;
        }
        for (int o = threadIdx.x; o < TILE; o += blockDim.x) {
            const int row = o / (16 * FJ), col = o % (16 * FJ);
            float y = 0.0f;
            for (int w = 0; w < wk; ++w) y += red_base[w * TILE + o];
            const int64_t n = n0 + col;
            if (row < M && n < N) {
                if constexpr (QX || XF8) y *= row_factor(row);
                p.Y[static_cast<int64_t>(row) * N + n] = float_to_bf16_bits(y);
            }
        }
        return;
    }
    // Sum the wk partial tiles in LDS: wave w stores its [16 MB][16 FJ] tile
    // (register e of lane l holds row 4 (l / 16) + e of its 16-row block and
    // column l % 16 of its 16-column block), then each thread adds the wk
    // values of some outputs in wave order.
    constexpr int TILE = 256 * MB * FJ;
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                red[wave * TILE + (16 * i + 4 * h + e) * (16 * FJ) + 16 * j + c] = acc[i][j][e];
    __syncthreads();
    if (pair) {
        for (int o = threadIdx.x; o < 256 * MB; o += blockDim.x) {
            const int row = o / 16, cc = o % 16;
            float g = 0.0f, u = 0.0f;
            for (int w = 0; w < wk; ++w) {
                g += red[w * TILE + row * 16 * FJ + cc];
                u += red[w * TILE + row * 16 * FJ + 16 + cc];
            }
            const int64_t n = n0 + cc;
            float hv = 0.0f;
            if (row < M && n < N) {
                const float r = XF8 ? p.xscale[row] : 1.0f;
                const uint16_t hb = float_to_bf16_bits(activation(p.act, g * r) * (u * r));
                p.Y[static_cast<int64_t>(row) * N + n] = hb;
                hv = fabsf(bf16_lo(hb));
            }
            if (p.amax_part) {
                hv = max16(hv);
                if (cc == 0 && row < M) p.amax_part[static_cast<int64_t>(row) * p.amax_tiles + blockIdx.x] = hv;
            }
        }
        return;
    }
    for (int o = threadIdx.x; o < TILE; o += blockDim.x) {
        const int row = o / (16 * FJ), col = o % (16 * FJ);
        float y = 0.0f;
        for (int w = 0; w < wk; ++w) y += red[w * TILE + o];
        const int64_t n = n0 + col;
        if (row < M && n < N) {
            if (ksplit) {
                p.ws[(static_cast<int64_t>(kr) * M + row) * N + n] = y;
            } else {
                if constexpr (XF8) y *= p.xscale[row];
                p.Y[static_cast<int64_t>(row) * N + n] = float_to_bf16_bits(y);
            }
        }
    }
}

// Sum of the K-split partials of the streaming kernel: Y = bf16(sum over the
// ranges in order, times the row scale for W4A8).
__global__ void __launch_bounds__(256) skinny_reduce_kernel(MulParams p) {
    const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t mn = p.M * p.N;
    if (e >= mn) return;
    float y = p.ws[e];
    for (int z = 1; z < p.splits; ++z) y += p.ws[z * mn + e];
    if (p.x_fp8) y *= p.xscale[e / p.N];
    p.Y[e] = float_to_bf16_bits(y);
}

// LDS words of one staged activation row: 16 bf16 pairs and one sum per
// 32-k quarter, quarters padded to a whole 128-k step
int64_t staged_words_row(int64_t K) { return 17 * (((K / 32) + 3) & ~int64_t{3}); }

template <int MB, int FJ, bool XF8, int MODE>
hipError_t launch_skinny_c(const MulParams& p, int wk, hipStream_t stream) {
    const int64_t cols = p.wq2 ? 16 : 16 * FJ;       // output columns per workgroup
    if (p.wq2 && FJ != 2) return hipErrorInvalidValue;
    const bool split = MODE < kDot && p.splits > 1;
    const int64_t blocks = (p.N + cols - 1) / cols * (split ? p.splits : 1);
    size_t lds = static_cast<size_t>(wk) * (MODE >= kDot ? 16 : 256) * MB * FJ * sizeof(float);
    if (MODE == kDotLds || MODE == kDotLdsQ) lds += static_cast<size_t>(MB) * staged_words_row(p.K) * sizeof(uint32_t);
    hipLaunchKernelGGL((gemm_skinny_kernel<MB, FJ, XF8, MODE>), dim3(static_cast<unsigned>(blocks)), dim3(64 * wk), lds,
                       stream, p, wk);
    if (split) {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(skinny_reduce_kernel, dim3(static_cast<unsigned>((p.M * p.N + 255) / 256)), dim3(256), 0,
                           stream, p);
    }
    return hipGetLastError();
}

// groups of 128 or more (a K step lies in one group; per-channel included)
// use the exact correction form, smaller groups dequantize every weight
template <int MB, int FJ, bool XF8>
hipError_t launch_skinny_t(const MulParams& p, int wk, hipStream_t stream) {
    if (p.G % kStepK == 0) {
        // four bf16 row blocks with two column blocks would not fit the registers
        if constexpr (MB == 4 && FJ > 1 && !XF8) return launch_skinny_c<MB, 1, XF8, kCorr>(p, wk, stream);
        else return launch_skinny_c<MB, FJ, XF8, kCorr>(p, wk, stream);
    }
    return launch_skinny_c<MB, FJ, XF8, kDeq>(p, wk, stream);
}

template <int MB, bool XF8>
hipError_t launch_skinny_m(const MulParams& p, int fj, int wk, hipStream_t stream) {
    // four 16-row blocks by four 16-column blocks would not fit the registers
    if constexpr (MB < 4) {
        if (fj == 4) return launch_skinny_t<MB, 4, XF8>(p, wk, stream);
    }
    if (fj >= 2) return launch_skinny_t<MB, 2, XF8>(p, wk, stream);
    return launch_skinny_t<MB, 1, XF8>(p, wk, stream);
}

}  // namespace

#ifndef W4_SK_FJMAX
#define W4_SK_FJMAX 4
#endif
#ifndef W4_SK_MINBLK
#define W4_SK_MINBLK 240
#endif
#ifndef W4_SK_SPLIT_MINSTEPS
#define W4_SK_SPLIT_MINSTEPS 4
#endif
#ifndef W4_SK_SPLIT_MINWG
#define W4_SK_SPLIT_MINWG 120
#endif

// K split of the MFMA forms (3 <= M <= 64).  Every workgroup reads the whole
// activation block [M, K] from L2, once per column block; the unsplit
// schedule narrows the blocks until there are about as many as compute
// units, so its activation reads come to M x (bytes per activation) / (8 FJ)
// times the weight bytes.  Where that reaches four, K is cut into ranges
// instead: the widest column blocks the registers allow (64 columns, 32 for
// four row blocks), one workgroup per (block, range), at most 16 ranges of
// at least four 128-k steps, and a second kernel sums the ranges (below
// that ratio its launch costs more than the reads save).  A split that the
// four-step minimum keeps below 120 workgroups is dropped: there the unsplit
// schedule's several waves per workgroup do better than fewer one-wave
// workgroups and a second launch (SmolLM2-sized down projection, K = 1536,
// N = 576, at M = 16 / 32: 10.7 / 14.4 -> 4.4 / 5.9 us).  The ranges depend
// on the shape and the activation width; the workspace is sized for bf16,
// the wider.
int skinny_splits(int64_t M, int64_t K, int64_t N, int xbytes) {
    if (M < 3 || M > kSkinnyMaxM || K <= 0 || N <= 0) return 1;
    const int mb = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    const int fj = mb == 4 ? 2 : W4_SK_FJMAX;
    int fju = fj;                                    // the unsplit schedule's column blocks
    while (fju > 1 && (N + 16 * fju - 1) / (16 * fju) < W4_SK_MINBLK) fju /= 2;
    if (M * xbytes < 32 * fju) return 1;
    const int64_t nblk = (N + 16 * fj - 1) / (16 * fj);
    if (nblk >= W4_SK_MINBLK) return 1;
    const int64_t ks = (K + kStepK - 1) / kStepK;
    int64_t s = (W4_SK_MINBLK + nblk - 1) / nblk;
    if (s > ks / W4_SK_SPLIT_MINSTEPS) s = ks / W4_SK_SPLIT_MINSTEPS;
    if (s > 16) s = 16;
    // too few steps to reach the workgroup count: the split would leave
    // fewer, one-wave workgroups and a second launch
    if (nblk * s < W4_SK_SPLIT_MINWG) return 1;
    return s < 2 ? 1 : static_cast<int>(s);
}

size_t skinny_workspace_bytes(int64_t M, int64_t K, int64_t N) {
    const int s = skinny_splits(M, K, N, 2);
    return s > 1 ? static_cast<size_t>(s) * M * N * sizeof(float) : 0;
}

bool skinny_quantizes_rows(int64_t M, int64_t K) {
#ifndef W4_DOT_LDS_MAX
#define W4_DOT_LDS_MAX 65536
#endif
    return M >= 1 && M <= kDotMaxM && M * staged_words_row(K) * 4 <= W4_DOT_LDS_MAX;
}

// Launch shape: the widest column tile (16, 32 or 64 columns; 32 at most for
// 64 rows) that still gives at least 240 workgroups (one per compute unit,
// nearly), then K-splitting waves per workgroup: with one or two rows, about
// 32 waves per compute unit in all, at most 16 per workgroup (8 unless the
// rows are staged in LDS) with at least four 128-wide K steps each; with more
// rows about 16 waves per compute unit, at most 8 per workgroup, with at
// least three steps each (8B up at M = 4 / 16: 9.9 / 13.0 -> 9.4 / 12.6 us;
// 12B W4A8 up at M = 16, K = 3840: 17.8 -> 13.4 us, where eight steps a wave
// had left three waves to a workgroup).
hipError_t launch_skinny(const MulParams& p, hipStream_t stream) {
    if (p.M == 0 || p.N == 0) return hipSuccess;
#ifndef W4_SK_WKMAX
#define W4_SK_WKMAX 8
#endif
#ifndef W4_SK_MINSTEPS
#define W4_SK_MINSTEPS 3
#endif
#ifndef W4_DOT_FJMAX
#define W4_DOT_FJMAX 4
#endif
#ifndef W4_DOT_MINBLK
#define W4_DOT_MINBLK 240
#endif
#ifndef W4_DOT_MINSTEPS
#define W4_DOT_MINSTEPS 4
#endif
#ifndef W4_DOT_WAVES
#define W4_DOT_WAVES 8192
#endif
    const bool dotm = p.M <= kDotMaxM;
    const int mb = p.M <= 16 ? 1 : (p.M <= 32 ? 2 : 4);
    // two rows with four column blocks would not fit 128 registers a lane
    int fj = dotm ? (p.M == 2 && W4_DOT_FJMAX > 2 ? 2 : W4_DOT_FJMAX) : (mb == 4 ? 2 : W4_SK_FJMAX);
    const int minblk = dotm ? W4_DOT_MINBLK : W4_SK_MINBLK;
    // a K split (workspace given) keeps the widest blocks; otherwise narrower
    // blocks give enough workgroups
    const bool split = !dotm && !p.wq2 && p.splits > 1;
    if (!split)
        while (fj > 1 && (p.N + 16 * fj - 1) / (16 * fj) < minblk) fj /= 2;
    if (p.wq2) {
        // gate and up: two blocks over the same 16 columns (at most 32 rows)
        if (mb > 2) return hipErrorInvalidValue;
        fj = 2;
    }
    const int64_t blocks = (p.wq2 ? (p.N + 15) / 16 : (p.N + 16 * fj - 1) / (16 * fj)) * (split ? p.splits : 1);
    const int64_t ks = (p.K + kStepK - 1) / kStepK / (split ? p.splits : 1);
    const int64_t minsteps = dotm ? W4_DOT_MINSTEPS : (split ? W4_SK_SPLIT_MINSTEPS : W4_SK_MINSTEPS);
    int64_t wk = ((dotm ? W4_DOT_WAVES : 4096) + blocks - 1) / blocks;
    if (wk > ks / minsteps) wk = ks / minsteps;
#ifndef W4_DOT_WKMAX
#define W4_DOT_WKMAX 16
#endif
    // up to 16 waves where the activations are staged in LDS (1024-thread
    // workgroups, 128 registers a lane), else up to 8
    const bool lds_x = dotm && skinny_quantizes_rows(p.M, p.K);
    const int64_t wk_max = lds_x ? W4_DOT_WKMAX : W4_SK_WKMAX;
    if (wk > wk_max) wk = wk_max;
    if (wk < 1) wk = 1;
    // the LDS for the final sum: wk x 1 KB per 16 x 16 block of the tile
    while (wk > 1 && wk * mb * fj > 128) --wk;
    const int w = static_cast<int>(wk);
    if (p.M <= kDotMaxM) {
        // activations staged in LDS when they fit (up to 64 KB per workgroup)
        auto dot = [&](auto mt, auto xf8) -> hipError_t {
            constexpr int MT = decltype(mt)::value;
            constexpr bool X8 = decltype(xf8)::value;
            if (X8 && p.xq_out) {
                if constexpr (MT == 1)
                    if (fj == 4) return launch_skinny_c<MT, 4, true, kDotLdsQ>(p, w, stream);
                if (fj >= 2) return launch_skinny_c<MT, 2, true, kDotLdsQ>(p, w, stream);
                return launch_skinny_c<MT, 1, true, kDotLdsQ>(p, w, stream);
            }
            if (lds_x) {
                if constexpr (MT == 1)
                    if (fj == 4) return launch_skinny_c<MT, 4, X8, kDotLds>(p, w, stream);
                if (fj >= 2) return launch_skinny_c<MT, 2, X8, kDotLds>(p, w, stream);
                return launch_skinny_c<MT, 1, X8, kDotLds>(p, w, stream);
            }
            if (fj == 4) return launch_skinny_c<MT, 4, X8, kDot>(p, w, stream);
            if (fj == 2) return launch_skinny_c<MT, 2, X8, kDot>(p, w, stream);
            return launch_skinny_c<MT, 1, X8, kDot>(p, w, stream);
        };
        using one = std::integral_constant<int, 1>;
        using two = std::integral_constant<int, 2>;
        if (p.x_fp8) return p.M == 1 ? dot(one{}, std::true_type{}) : dot(two{}, std::true_type{});
        return p.M == 1 ? dot(one{}, std::false_type{}) : dot(two{}, std::false_type{});
    }
    if (p.x_fp8) {
        switch (mb) {
            case 1: return launch_skinny_m<1, true>(p, fj, w, stream);
            case 2: return launch_skinny_m<2, true>(p, fj, w, stream);
            default: return launch_skinny_m<4, true>(p, fj, w, stream);
        }
    }
    switch (mb) {
        case 1: return launch_skinny_m<1, false>(p, fj, w, stream);
        case 2: return launch_skinny_m<2, false>(p, fj, w, stream);
        default: return launch_skinny_m<4, false>(p, fj, w, stream);
    }
}

}  // namespace w4
