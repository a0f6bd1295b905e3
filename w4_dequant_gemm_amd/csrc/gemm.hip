// W4A16 / W4A8 GEMM for M > 16 on gfx950 bf16 MFMA.
//
// At prefill sizes the products are compute bound and the dequantization work
// shows (gsantana.dev "Quantizing LLMs Without Guesswork", "Production
// reality"), so each packed weight tile is dequantized once per workgroup into
// LDS and then reused by every activation row of the workgroup tile:
//
//   global (4-bit GPU layout) -> registers: fp16 1024 + u (or 1024 + 16 u)
//   via AND-OR, W' = (1024 + u) s - (1024 + z) s by mixed-precision FMAs
//   (exact in fp32; PairDequant below), rounded to bf16 (RNE)
//   -> LDS -> v_mfma_f32_32x32x16_bf16 with fp32 accumulation -> bf16 out.
//
// W4A8 reads the E4M3 activations produced by the row quantizer, widens them
// exactly to bf16 and multiplies by the row scale in the epilogue.
//
// Kernels, by M (K a multiple of 64 unless noted):
//   64 < M <= 128    gemm_mid_kernel, 64 x 128 tiles, K split towards 512 workgroups
//   M > 128, W4A16   gemm256_breg_kernel, 256 x 256 tiles, activations direct to
//                    LDS, weights dequantized straight into MFMA operands
//   M > 128, W4A8    gemm256_kernel, 256 x 256 tiles, activations through registers
//   K % 64 != 0      gemm_kernel, 128 x 128 tiles, K step 32
// and the gate + up pair (above 32 rows) on gemm_mid_kernel (64- or 128-row
// tiles, a B tile that interleaves the two weights) or, W4A16 above 256 rows,
// gemm256_breg_kernel (two waves on each weight).  Rows of X beyond M and rows of W beyond
// N are clamped or read as zero; the epilogues store only in-range outputs.
#include <type_traits>

#include "device.hpp"
#include "kernels.hpp"

namespace w4 {
namespace {

// Dequantization of one code word (8 consecutive k of one row: code 2i at
// bits 4i, code 2i + 1 at bits 16 + 4i) into four bf16 pairs.  Pairs 0 and 2
// take one AND-OR with 0x000F000F (of the word, and of the word >> 8) into
// the low mantissa bits of fp16 1024, giving 1024 + u (unit in the last
// place 1); pairs 1 and 3 take an AND-OR with 0x00F000F0 of the same
// operands, giving 1024 + 16 u (still inside the 10-bit mantissa).  Then
// W' = (1024 + u) s - (1024 + z) s, or (1024 + 16 u) (s / 16) - (64 + z) s,
// by two mixed-precision FMAs per pair (fp16 operands, fp32 result; exact:
// s / 16 is exact and every product and sum has at most 23 significant
// bits), and one rounding to a bf16 pair.  Both forms give the same value.
struct PairDequant {
    uint32_t bias;                 // two fp16 1024.0 (0x64006400), in a register
    float sc = 0.0f, cs = 0.0f, sc16 = 0.0f, cs16 = 0.0f;
    // the scale / zero word of the group: fp16 s in bits 0-15, z in 16-31
    __device__ __forceinline__ void group(uint32_t sz) {
        const float z = half_bits_to_float(sz >> 16);
        sc = half_bits_to_float(sz);
        cs = -(1024.0f + z) * sc;
        sc16 = sc * 0.0625f;
        cs16 = -(64.0f + z) * sc;
    }
    __device__ __forceinline__ uint32_t pair(uint32_t w, int i) const {
        const uint32_t src = i < 2 ? w : w >> 8;
        const uint32_t h = (src & ((i & 1) ? 0x00F000F0u : 0x000F000Fu)) | bias;
        const _Float16 lo = __builtin_bit_cast(_Float16, static_cast<uint16_t>(h & 0xFFFFu));
        const _Float16 hi = __builtin_bit_cast(_Float16, static_cast<uint16_t>(h >> 16));
        const float s = (i & 1) ? sc16 : sc, c = (i & 1) ? cs16 : cs;
        return pack_bf16x2(fmaf(static_cast<float>(lo), s, c), fmaf(static_cast<float>(hi), s, c));
    }
};

namespace small {
constexpr int BM = 128, BN = 128, BK = 32;
constexpr int LDS_STRIDE = BK + 8;   // bf16 elements per LDS row (16 bytes of padding)
}  // namespace small

template <bool XF8>
__global__ void __launch_bounds__(256) gemm_kernel(MulParams p) {
    using namespace small;
    __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDS_STRIDE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;    // wave position in the 2 x 2 grid
    const int64_t m_base = static_cast<int64_t>(blockIdx.y) * BM;
    const int64_t n_base = static_cast<int64_t>(blockIdx.x) * BN;
    const int64_t M = p.M, N = p.N, K = p.K;
    const uint32_t bias = opaque_vgpr(kBf16Bias128x2);

    float16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // A tile loader: thread -> (row tid/2, k half (tid%2)*16)
    const int a_row = tid >> 1;
    const int a_k = (tid & 1) * 16;
    // B tile loader: thread -> (row tid/2, words 2*(tid%2), +1)
    const int b_row = tid >> 1;
    const int b_w = (tid & 1) * 2;

    for (int64_t k0 = 0; k0 < K; k0 += BK) {
        // ---- A: 16 activations per thread
        {
            const int64_t m = m_base + a_row;
            uint32_t v[8];
            if (m < M) {
                if constexpr (!XF8) {
                    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.X) + m * K + k0 + a_k);
                    uint4 t0 = src[0], t1 = src[1];
                    v[0] = t0.x; v[1] = t0.y; v[2] = t0.z; v[3] = t0.w;
                    v[4] = t1.x; v[5] = t1.y; v[6] = t1.z; v[7] = t1.w;
                } else {
                    const uint4 b = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(p.X) + m * K + k0 + a_k);
                    const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        float2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(bw[j]), false);
                        float2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(bw[j]), true);
                        v[2 * j] = pack_bf16x2(lo[0], lo[1]);
                        v[2 * j + 1] = pack_bf16x2(hi[0], hi[1]);
                    }
                }
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) v[j] = 0u;
            }
            uint4* dst = reinterpret_cast<uint4*>(&As[a_row * LDS_STRIDE + a_k]);
            dst[0] = make_uint4(v[0], v[1], v[2], v[3]);
            dst[1] = make_uint4(v[4], v[5], v[6], v[7]);
        }
        // ---- B: 2 code words (16 weights) per thread, dequantized to bf16
        {
            const int64_t n = n_base + b_row;
            uint32_t out[8];
            if (n < N) {
                const TiledRow tr = tiled_row(p.wq, p.sz, n, N, K, p.G);
                const uint2 w = *reinterpret_cast<const uint2*>(tr.tile_ptr(k0 / 32) + b_w);
                const uint32_t szw = tr.group((k0 + 8 * b_w) / p.G);
                const float s = half_bits_to_float(szw);
                const float cs = (128.0f + half_bits_to_float(szw >> 16)) * s;
                const uint32_t ws[2] = {w.x, w.y};
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t pr = nibble_pair_bf16(ws[j], i, bias);
                        out[4 * j + i] = pack_bf16x2(fmaf(bf16_lo(pr), s, -cs), fmaf(bf16_hi(pr), s, -cs));
                    }
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) out[j] = 0u;
            }
            uint4* dst = reinterpret_cast<uint4*>(&Bs[b_row * LDS_STRIDE + 8 * b_w]);
            dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
            dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
        }
        __syncthreads();

#pragma unroll
        for (int kk = 0; kk < BK; kk += 16) {
            bf16x8_t a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = wm * 64 + i * 32 + (lane & 31);
                a[i] = *reinterpret_cast<const bf16x8_t*>(&As[row * LDS_STRIDE + kk + 8 * (lane >> 5)]);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int col = wn * 64 + j * 32 + (lane & 31);
                b[j] = *reinterpret_cast<const bf16x8_t*>(&Bs[col * LDS_STRIDE + kk + 8 * (lane >> 5)]);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }

    // epilogue: register r of lane l holds row (r%4) + 4(l/32) + 8(r/4), column l%32
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t col = n_base + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m_base + wm * 64 + i * 32 + (r & 3) + 4 * (lane >> 5) + 8 * (r >> 2);
                if (row < M && col < N) {
                    float y = acc[i][j][r];
                    if constexpr (XF8) y *= p.xscale[row];
                    p.Y[row * N + col] = float_to_bf16_bits(y);
                }
            }
        }
}


// ------------------------------------------------------------------ 256 x 256
//
// Large-M kernel.  A 512-thread workgroup (4 x 2 waves of 64 x 128 outputs,
// 2 x 4 MFMA 32x32x16 tiles each) owns a 256 x 256 output tile and walks K in
// steps of 64 through two LDS stages of bf16 operands (2 x 64 KB).  Global
// loads run two steps ahead of the MFMAs, which hides their latency (about
// one step of MFMA work):
//   * each thread owns half a row of the activation tile (32 values) and
//     half a row of the weight tile (32 codes plus the group's scale/zero
//     word), loaded into one of two register buffers;
//   * a step issues the loads of step k + 2, runs the 64 MFMAs of step k per
//     wave, converts step k + 1 (activations copied or widened from E4M3,
//     weights dequantized to bf16) into the idle LDS stage, waits until only
//     step k + 2's loads are outstanding, and synchronizes the workgroup.
// LDS rows are 128 bytes (64 bf16); the 16-byte chunk c of row r is stored at
// position c ^ ((r >> 1) & 7), spreading the row stores and the MFMA operand
// reads over the banks (the fastest of the XOR forms measured for this kernel).
namespace big {
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int STAGE = 256 * BK;          // bf16 elements per operand and stage

// Chunk swizzles of 128-byte LDS operand rows: the 16-byte chunk c of row
// `row` sits at position c ^ swizzle(row).  Variants (chosen by measurement):
__device__ __forceinline__ int swizzle_fn(int f, int row) {
    switch (f) {
        case 1: return (row >> 1) & 7;
        case 2: return (row >> 2) & 7;
        case 3: return (row ^ (row >> 3)) & 7;
        case 4: return ((row >> 1) ^ (row >> 4)) & 7;
        case 5: return ((row >> 2) ^ (row << 2)) & 7;
        default: return row & 7;
    }
}
#ifndef W4_RSWZ
#define W4_RSWZ 1
#endif
// bf16 offset of 16-byte chunk c (8 k) of operand row `row` in one 256 x 64
// stage: rows are 128 bytes; the chunk index is XORed with row bits so that
// both the row-wise stores and the MFMA fragment reads spread over the banks
__device__ __forceinline__ int lds_off(int row, int c) { return row * BK + ((c ^ swizzle_fn(W4_RSWZ, row)) << 3); }

// The work of one workgroup of the 256 x 256 kernels (1-D grid): workgroup
// b < split_t0 computes tile b whole; the rest compute K range z of tile
// split_t0 + (b - split_t0) / splits, z = (b - split_t0) % splits.  Tile
// numbers map to the grid by tile_rc.
struct TileJob {
    int64_t m_base, n_base;
    int kb, KT;        // first K step and number of K steps
    int64_t part;      // partial-tile index in ws, or -1: write Y
};
__device__ __forceinline__ TileJob tile_job(const MulParams& p) {
    const int64_t b = blockIdx.x;
    const int64_t nt = (p.N + BN - 1) / BN;
    const int KT_all = static_cast<int>(p.K / BK);
    TileJob t;
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
}  // namespace big

template <int WM, int WN, bool XF8>
__global__ void __launch_bounds__(64 * WM * WN) gemm256_kernel(MulParams p) {
    using namespace big;
    constexpr int NT = 64 * WM * WN;         // threads
    constexpr int TM = BM / WM, TN = BN / WN; // wave tile
    constexpr int FI = TM / 32, FJ = TN / 32; // 32 x 32 MFMA tiles per wave
    constexpr int TPR = NT / 256;             // threads per operand row
    constexpr int CPT = (BK / 8) / TPR;       // 16-byte bf16 chunks (8 k) per thread and row
    constexpr int XB = XF8 ? 1 : 2;           // activation bytes per element in global memory
    constexpr int ALD = CPT * 8 * XB / 16;    // 16-byte activation loads per thread and step
    static_assert(CPT % 4 == 0 && ALD >= 1, "operand split");
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * 2 * STAGE];   // [stage][A, B][256 x 64]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const TileJob job = tile_job(p);
    const int64_t m_base = job.m_base, n_base = job.n_base;
    const int64_t M = p.M, N = p.N, K = p.K;
    const int kb = job.kb, KT = job.KT;      // this workgroup's K steps
    const int g_shift = group_shift(p.G);
    const uint32_t bias = opaque_vgpr(kBf16Bias128x2);

    float16_t acc[FI][FJ];
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // operand row of this thread and its first 8-k chunk within a K step
    const int o_row = tid / TPR;
    const int o_c0 = (tid % TPR) * CPT;
    int64_t bn = n_base + o_row;
    bn = bn < N ? bn : N - 1;              // rows past N or M compute garbage that is never stored
    int64_t am = m_base + o_row;
    am = am < M ? am : M - 1;
    const TiledRow brow = tiled_row(p.wq, p.sz, bn, N, K, p.G);
    // Activation row address with its provenance hidden (an empty asm): loads
    // through it are then not known to be invariant, so the register
    // allocator cannot re-issue them at their use a step later instead of
    // keeping the prefetched values.  Re-cast to the global address space so
    // that they stay global (not flat) loads.
    uint64_t arow_addr = reinterpret_cast<uint64_t>(static_cast<const uint8_t*>(p.X) + (am * K + o_c0 * 8) * XB);
    asm volatile("" : "+v"(arow_addr));
    typedef const u32x4_t __attribute__((address_space(1))) global_u4;
    const global_u4* arow = (const global_u4*)arow_addr;

    // scale/zero words per thread and step: one per 32 k (the smallest group)
    constexpr int SZN = CPT / 4;
    struct Regs {
        uint4 a[ALD];
        u32x4_t q[CPT / 4];   // code words, kept as 16-byte vectors (no register copies)
        uint32_t s[SZN];
    };
    Regs r0, r1;

    // The global loads of one step: ALD activation loads, CPT / 4 code loads
    // and SZN scale/zero loads, issued one item at a time.
    constexpr int NLOAD = ALD + CPT / 4 + SZN;
    auto issue_load_item = [&](int kt, Regs& r, int it) {
        kt = (kt < KT ? kt : KT - 1) + kb;  // past the end: reload the last step (never used)
        if (it < ALD) {
            const u32x4_t t = arow[static_cast<int64_t>(kt) * (BK * XB / 16) + it];
            r.a[it] = make_uint4(t[0], t[1], t[2], t[3]);
        } else if (it < ALD + CPT / 4) {
            // words o_c0 + 4i .. + 3 of the step: one 32-k tile of the row
            const int i = it - ALD;
            r.q[i] = *reinterpret_cast<const u32x4_t*>(brow.tile_ptr(static_cast<int64_t>(kt) * (BK / 32) + o_c0 / 4 + i));
        } else {
            // words 4t .. 4t + 3 (32 k) of the thread lie in one group for every G
            const int t = it - ALD - CPT / 4;
            r.s[t] = brow.group((kt * BK + o_c0 * 8 + 32 * t) >> g_shift);
        }
    };
    auto issue_loads = [&](int kt, Regs& r) {
#pragma unroll
        for (int it = 0; it < NLOAD; ++it) issue_load_item(kt, r, it);
    };

    // ---- operand conversion, split into small work items -------------------
    // B: code word j (8 k) of the thread's row holds four pairs of codes,
    // each dequantized to a bf16 pair by PairDequant; the fourth pair of a
    // word completes a 16-byte LDS row chunk.
    const uint32_t bias16 = opaque_vgpr(0x64006400u);   // two fp16 1024.0
    PairDequant dq{bias16};
    uint32_t b_out[4];
    auto b_pair = [&](int pr, const Regs& r, uint16_t* B) {
        const int j = pr / 4, i = pr % 4;
        if (i == 0 && j % 4 == 0) dq.group(r.s[j / 4]);
        b_out[i] = dq.pair(r.q[j / 4][j % 4], i);
        if (i == 3)
            *reinterpret_cast<uint4*>(B + lds_off(o_row, o_c0 + j)) = make_uint4(b_out[0], b_out[1], b_out[2], b_out[3]);
    };
    // A: bf16 activations are copied (ALD items of 16 bytes); E4M3 ones are
    // widened exactly to bf16, each 16-byte load in two halves of 8 values.
    constexpr int A_ITEMS = XF8 ? 2 * ALD : ALD;
    auto a_item = [&](int it, const Regs& r, uint16_t* A) {
        if constexpr (!XF8) {
            // the empty asm keeps the wait for this load here, not earlier
            uint4 v = r.a[it];
            asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
            *reinterpret_cast<uint4*>(A + lds_off(o_row, o_c0 + it)) = v;
        } else {
            const uint4 src = r.a[it / 2];
            const uint32_t w0 = (it & 1) ? src.z : src.x;
            const uint32_t w1 = (it & 1) ? src.w : src.y;
            uint32_t o[4];
            const uint32_t bw[2] = {w0, w1};
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                float2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(bw[jj]), false);
                float2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(bw[jj]), true);
                o[2 * jj] = pack_bf16x2(lo[0], lo[1]);
                o[2 * jj + 1] = pack_bf16x2(hi[0], hi[1]);
            }
            *reinterpret_cast<uint4*>(A + lds_off(o_row, o_c0 + it)) = make_uint4(o[0], o[1], o[2], o[3]);
        }
    };
    // all conversion of one step at once (prologue)
    auto store_operands = [&](int stage, const Regs& r) {
        uint16_t* A = lds + stage * 2 * STAGE;
#pragma unroll
        for (int it = 0; it < A_ITEMS; ++it) a_item(it, r, A);
#pragma unroll
        for (int pr = 0; pr < 4 * CPT; ++pr) b_pair(pr, r, A + STAGE);
    };

    auto load_frags = [&](const uint16_t* A, const uint16_t* B, int kk, bf16x8_t (&a)[FI], bf16x8_t (&b)[FJ]) {
        const int ch = 2 * kk + (lane >> 5);
#pragma unroll
        for (int i = 0; i < FI; ++i)
            a[i] = *reinterpret_cast<const bf16x8_t*>(A + lds_off(wm * TM + i * 32 + (lane & 31), ch));
#pragma unroll
        for (int j = 0; j < FJ; ++j)
            b[j] = *reinterpret_cast<const bf16x8_t*>(B + lds_off(wn * TN + j * 32 + (lane & 31), ch));
    };

    // One K step: global loads for kt + 2 into `next` (its previous contents,
    // step kt, were converted during step kt - 1); the MFMAs of step kt from
    // one LDS stage; the conversion of step kt + 1 from `ready` into the other
    // stage; then a barrier.
    // The loads must stay in flight across the MFMAs.  An activation load
    // whose value is only copied to LDS a step later would otherwise be sunk
    // next to that copy by the optimizer (nothing in between writes global
    // memory); the empty asm with a memory clobber pins the loads here without
    // emitting code, and the scheduling barrier keeps them ahead of the rest.
    // The MFMAs and the conversion work are laid out by hand: MFMA slot u
    // (of FI * FJ * BK / 16 per step) is followed by B pair (u - 1) / 2 when
    // u is odd and by A item u / 4 when u is a multiple of 4, and a
    // scheduling barrier after every slot keeps that order, so the matrix
    // cores run while the VALU converts.  Fragments for the next 16 k are
    // read from LDS at the start of each 16-k sub-step.
    constexpr int NSLOT = FI * FJ * (BK / 16);
    static_assert(NSLOT >= 2 * 4 * CPT && NSLOT >= 4 * A_ITEMS, "conversion work must fit the MFMA slots");
    constexpr int LOAD_EVERY = NSLOT / NLOAD;
    auto step = [&](int kt, Regs& next, const Regs& ready) {
        __builtin_amdgcn_sched_barrier(0);
        const uint16_t* As = lds + (kt & 1) * 2 * STAGE;
        const uint16_t* Bs = As + STAGE;
        uint16_t* Ad = lds + ((kt + 1) & 1) * 2 * STAGE;   // past the end this refills an idle stage
        uint16_t* Bd = Ad + STAGE;
        bf16x8_t fa[2][FI], fb[2][FJ];
        load_frags(As, Bs, 0, fa[0], fb[0]);
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            if (kk + 1 < BK / 16) load_frags(As, Bs, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < FI * FJ; ++t) {
                const int u = kk * FI * FJ + t;
                const int i = t / FJ, j = t % FJ;
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk & 1][i], fb[kk & 1][j], acc[i][j], 0, 0, 0);
                if (u % 2 == 1 && u / 2 < 4 * CPT) b_pair(u / 2, ready, Bd);
                if (u % 4 == 0 && u / 4 < A_ITEMS) a_item(u / 4, ready, Ad);
                if (u % LOAD_EVERY == 0 && u / LOAD_EVERY < NLOAD) {
                    issue_load_item(kt + 2, next, u / LOAD_EVERY);
                    asm volatile("" ::: "memory");
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        __syncthreads();
    };

    issue_loads(0, r0);
    issue_loads(1, r1);
    store_operands(0, r0);
    __syncthreads();
    int kt = 0;
    for (; kt + 2 <= KT; kt += 2) {
        step(kt, r0, r1);
        step(kt + 1, r1, r0);
    }
    if (kt < KT) step(kt, r0, r1);

    // epilogue: register r of lane l holds row (r%4) + 4(l/32) + 8(r/4), column l%32
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j) {
            const int lc = wn * TN + j * 32 + (lane & 31);
            const int64_t col = n_base + lc;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int lr = wm * TM + i * 32 + (r & 3) + 4 * (lane >> 5) + 8 * (r >> 2);
                const int64_t row = m_base + lr;
                if (job.part >= 0) {
                    p.ws[job.part * (BM * BN) + lr * BN + lc] = acc[i][j][r];   // partial tile of a K split
                } else if (row < M && col < N) {
                    float y = acc[i][j][r];
                    if constexpr (XF8) y *= p.xscale[row];
                    p.Y[row * N + col] = float_to_bf16_bits(y);
                }
            }
        }
}


// ---------------------------------------------------------------------------
// Mid-size M (a few hundred rows at most): the register-path kernel above
// with a smaller output tile, TBM x TBN = 64 x 128 or 128 x 128, so that the
// 12B-class shapes give hundreds of tiles instead of 15-60 and the K split
// (and its fp32 partial tiles) stays small.  About 48-64 KB of LDS and few
// registers let two or three workgroups share a compute unit, so one
// workgroup's conversion work runs while another's MFMAs do.  A and B have
// their own thread-to-row maps (TBM and TBN rows); the conversion items of a
// step are spread evenly over its MFMA slots.

// The work of one workgroup of the TBM x TBN kernels (same scheme as
// big::tile_job).
template <int TBM, int TBN>
__device__ __forceinline__ big::TileJob tile_job_t(const MulParams& p) {
    const int64_t b = blockIdx.x;
    const int64_t nt = (p.N + TBN - 1) / TBN;
    const int KT_all = static_cast<int>(p.K / big::BK);
    big::TileJob t;
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
    tile_rc(tile, (p.M + TBM - 1) / TBM, nt, tr, tc);
    t.m_base = tr * TBM;
    t.n_base = tc * TBN;
    return t;
}

// PAIR: the gated MLP front half.  The B tile holds TBN / 2 columns of the
// gate weight (rows 0 .. TBN/2 - 1) and the same columns of the up weight
// (rows TBN/2 ..), so with two wave columns the waves of column 0 sum
// gate products and those of column 1 up products for the same outputs; at
// the end the up sums go through LDS and H = bf16(act(gate) * up).
template <int TBM, int TBN, int WM, int WN, bool XF8, bool PAIR = false>
__global__ void __launch_bounds__(64 * WM * WN) gemm_mid_kernel(MulParams p) {
    using big::BK;
    using big::lds_off;
    constexpr int NT = 64 * WM * WN;
    constexpr int TM = TBM / WM, TN = TBN / WN;
    constexpr int FI = TM / 32, FJ = TN / 32;
    constexpr int TPRA = NT / TBM, CPTA = (BK / 8) / TPRA;   // A: threads per row, 8-k chunks per thread
    constexpr int TPRB = NT / TBN, CPTB = (BK / 8) / TPRB;   // B: threads per row, code words per thread
    constexpr int XB = XF8 ? 1 : 2;
    constexpr int ALD = CPTA * 8 * XB / 16;                  // 16-byte activation loads per thread and step
    constexpr int SZN = CPTB / 4;
    static_assert(FI >= 1 && FJ >= 1 && TPRA >= 1 && TPRB >= 1 && ALD >= 1 && CPTB % 4 == 0, "tile split");
    static_assert(!PAIR || (WN == 2 && TN == TBN / 2), "pair tiles: one wave column per weight");
    constexpr int OUTN = PAIR ? TBN / 2 : TBN;                 // output columns per tile
    constexpr int SA = TBM * BK, SB = TBN * BK;               // bf16 elements per stage and operand
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * (SA + SB)];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const big::TileJob job = tile_job_t<TBM, OUTN>(p);
    const int64_t m_base = job.m_base, n_base = job.n_base;
    const int64_t M = p.M, N = p.N, K = p.K;
    const int kb = job.kb, KT = job.KT;
    const int g_shift = group_shift(p.G);

    float16_t acc[FI][FJ];
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int a_row = tid / TPRA, a_c0 = (tid % TPRA) * CPTA;
    const int b_row = tid / TPRB, b_c0 = (tid % TPRB) * CPTB;
    const bool b_up = PAIR && b_row >= OUTN;
    int64_t bn = n_base + (PAIR ? b_row % OUTN : b_row);
    bn = bn < N ? bn : N - 1;               // rows past N or M compute values never stored
    int64_t am = m_base + a_row;
    am = am < M ? am : M - 1;
    const TiledRow brow = tiled_row(b_up ? p.wq2 : p.wq, b_up ? p.sz2 : p.sz, bn, N, K, p.G);
    // activation row address with its provenance hidden (see gemm256_kernel)
    uint64_t arow_addr = reinterpret_cast<uint64_t>(static_cast<const uint8_t*>(p.X) + (am * K + a_c0 * 8) * XB);
    asm volatile("" : "+v"(arow_addr));
    typedef const u32x4_t __attribute__((address_space(1))) global_u4;
    const global_u4* arow = (const global_u4*)arow_addr;

    struct Regs {
        uint4 a[ALD];
        u32x4_t q[CPTB / 4];
        uint32_t s[SZN];
    };
    Regs r0, r1;
    constexpr int NLOAD = ALD + CPTB / 4 + SZN;
    auto issue_load_item = [&](int kt, Regs& r, int it) {
        kt = (kt < KT ? kt : KT - 1) + kb;
        if (it < ALD) {
            const u32x4_t t = arow[static_cast<int64_t>(kt) * (BK * XB / 16) + it];
            r.a[it] = make_uint4(t[0], t[1], t[2], t[3]);
        } else if (it < ALD + CPTB / 4) {
            const int i = it - ALD;
            r.q[i] = *reinterpret_cast<const u32x4_t*>(brow.tile_ptr(static_cast<int64_t>(kt) * (BK / 32) + b_c0 / 4 + i));
        } else {
            const int t = it - ALD - CPTB / 4;
            r.s[t] = brow.group((kt * BK + b_c0 * 8 + 32 * t) >> g_shift);
        }
    };

    // conversion items (as in gemm256_kernel)
    const uint32_t bias16 = opaque_vgpr(0x64006400u);
    PairDequant dq{bias16};
    uint32_t b_out[4];
    auto b_pair = [&](int pr, const Regs& r, uint16_t* B) {
        const int j = pr / 4, i = pr % 4;
        if (i == 0 && j % 4 == 0) dq.group(r.s[j / 4]);
        b_out[i] = dq.pair(r.q[j / 4][j % 4], i);
        if (i == 3)
            *reinterpret_cast<uint4*>(B + lds_off(b_row, b_c0 + j)) = make_uint4(b_out[0], b_out[1], b_out[2], b_out[3]);
    };
    constexpr int A_ITEMS = XF8 ? 2 * ALD : ALD;
    auto a_item = [&](int it, const Regs& r, uint16_t* A) {
        if constexpr (!XF8) {
            uint4 v = r.a[it];
            asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
            *reinterpret_cast<uint4*>(A + lds_off(a_row, a_c0 + it)) = v;
        } else {
            const uint4 src = r.a[it / 2];
            const uint32_t bw[2] = {(it & 1) ? src.z : src.x, (it & 1) ? src.w : src.y};
            uint32_t o[4];
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                float2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(bw[jj]), false);
                float2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(bw[jj]), true);
                o[2 * jj] = pack_bf16x2(lo[0], lo[1]);
                o[2 * jj + 1] = pack_bf16x2(hi[0], hi[1]);
            }
            *reinterpret_cast<uint4*>(A + lds_off(a_row, a_c0 + it)) = make_uint4(o[0], o[1], o[2], o[3]);
        }
    };
    auto load_frags = [&](const uint16_t* A, const uint16_t* B, int kk, bf16x8_t (&a)[FI], bf16x8_t (&b)[FJ]) {
        const int ch = 2 * kk + (lane >> 5);
#pragma unroll
        for (int i = 0; i < FI; ++i)
            a[i] = *reinterpret_cast<const bf16x8_t*>(A + lds_off(wm * TM + i * 32 + (lane & 31), ch));
#pragma unroll
        for (int j = 0; j < FJ; ++j)
            b[j] = *reinterpret_cast<const bf16x8_t*>(B + lds_off(wn * TN + j * 32 + (lane & 31), ch));
    };

    // One K step: MFMAs of step kt from one stage; the conversion of step
    // kt + 1 from `ready` into the other stage and the loads of step kt + 2
    // into `next`, spread evenly over the MFMA slots; then a barrier.
    constexpr int NSLOT = FI * FJ * (BK / 16);
    constexpr int BP = 4 * CPTB;
    auto step = [&](int kt, Regs& next, const Regs& ready) {
        __builtin_amdgcn_sched_barrier(0);
        const uint16_t* As = lds + (kt & 1) * (SA + SB);
        const uint16_t* Bs = As + SA;
        uint16_t* Ad = lds + ((kt + 1) & 1) * (SA + SB);
        uint16_t* Bd = Ad + SA;
        bf16x8_t fa[2][FI], fb[2][FJ];
        load_frags(As, Bs, 0, fa[0], fb[0]);
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            if (kk + 1 < BK / 16) load_frags(As, Bs, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < FI * FJ; ++t) {
                const int u = kk * FI * FJ + t;
                const int i = t / FJ, j = t % FJ;
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk & 1][i], fb[kk & 1][j], acc[i][j], 0, 0, 0);
#pragma unroll
                for (int l = u * NLOAD / NSLOT; l < (u + 1) * NLOAD / NSLOT; ++l) {
                    issue_load_item(kt + 2, next, l);
                    asm volatile("" ::: "memory");
                }
#pragma unroll
                for (int pr = u * BP / NSLOT; pr < (u + 1) * BP / NSLOT; ++pr) b_pair(pr, ready, Bd);
#pragma unroll
                for (int ai = u * A_ITEMS / NSLOT; ai < (u + 1) * A_ITEMS / NSLOT; ++ai) a_item(ai, ready, Ad);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        __syncthreads();
    };

#pragma unroll
    for (int it = 0; it < NLOAD; ++it) issue_load_item(0, r0, it);
#pragma unroll
    for (int it = 0; it < NLOAD; ++it) issue_load_item(1, r1, it);
#pragma unroll
    for (int ai = 0; ai < A_ITEMS; ++ai) a_item(ai, r0, lds);
#pragma unroll
    for (int pr = 0; pr < BP; ++pr) b_pair(pr, r0, lds + SA);
    __syncthreads();
    int kt = 0;
    for (; kt + 2 <= KT; kt += 2) {
        step(kt, r0, r1);
        step(kt + 1, r1, r0);
    }
    if (kt < KT) step(kt, r0, r1);

    if constexpr (PAIR) {
        // up sums of wave (wm, 1) to LDS in register order, read back by wave
        // (wm, 0), whose registers hold the gate sums of the same outputs
        static_assert(TBM * TN * 4 <= 2 * (SA + SB) * 2, "the up sums fit the operand stages");
        float* up = reinterpret_cast<float*>(lds) + wm * (FI * FJ * 16 * 64);
        __syncthreads();
        if (wn == 1) {
#pragma unroll
            for (int i = 0; i < FI; ++i)
#pragma unroll
                for (int j = 0; j < FJ; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) up[((i * FJ + j) * 16 + r) * 64 + lane] = acc[i][j][r];
        }
        __syncthreads();
        if (wn == 0) {
#pragma unroll
            for (int i = 0; i < FI; ++i) {
                float hmax[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) hmax[r] = 0.0f;
#pragma unroll
                for (int j = 0; j < FJ; ++j) {
                    const int64_t col = n_base + j * 32 + (lane & 31);
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int64_t row = m_base + wm * TM + i * 32 + (r & 3) + 4 * (lane >> 5) + 8 * (r >> 2);
                        if (row < M && col < N) {
                            const float rs = XF8 ? p.xscale[row] : 1.0f;
                            const float g = acc[i][j][r] * rs;
                            const float u = up[((i * FJ + j) * 16 + r) * 64 + lane] * rs;
                            const uint16_t hb = float_to_bf16_bits(activation(p.act, g) * u);
                            p.Y[row * N + col] = hb;
                            hmax[r] = fmaxf(hmax[r], fabsf(bf16_lo(hb)));
                        }
                    }
                }
                if (p.amax_part) {
                    // each row's maximum |H| over the tile's columns: the
                    // 32 lanes of a half hold one row's columns
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float hv = max32(hmax[r]);
                        const int64_t row = m_base + wm * TM + i * 32 + (r & 3) + 4 * (lane >> 5) + 8 * (r >> 2);
                        if ((lane & 31) == 0 && row < M) p.amax_part[row * p.amax_tiles + n_base / OUTN] = hv;
                    }
                }
            }
        }
        return;
    }

#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j) {
            const int lc = wn * TN + j * 32 + (lane & 31);
            const int64_t col = n_base + lc;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int lr = wm * TM + i * 32 + (r & 3) + 4 * (lane >> 5) + 8 * (r >> 2);
                const int64_t row = m_base + lr;
                if (job.part >= 0) {
                    p.ws[job.part * (TBM * TBN) + lr * TBN + lc] = acc[i][j][r];
                } else if (row < M && col < N) {
                    float y = acc[i][j][r];
                    if constexpr (XF8) y *= p.xscale[row];
                    p.Y[row * N + col] = float_to_bf16_bits(y);
                }
            }
        }
}

// ---------------------------------------------------------------------------
// W4A16, M > 128: activations straight from global memory into LDS, weights
// dequantized straight into MFMA operands.
//
// 256 x 256 tile, K step 64, NW waves side by side: wave w owns output
// columns 256 / NW of all 256 rows (NW = 4: 8 x 2 blocks of
// v_mfma_f32_32x32x16_bf16, 256 accumulators, one wave per SIMD; NW = 8:
// 8 x 1 blocks, 128 accumulators, two waves per SIMD).  The bf16 activations never
// pass through registers: each wave issues global_load_lds_dwordx4 (lane l's
// 16 bytes land at the instruction's LDS base + 16 l) two K steps ahead into
// the free one of three 32 KB activation stages (chunk swizzle (row ^ row >>
// 3) & 7), separate arrays so that with the loop unrolled by six every access
// names its stage statically.  No two waves share a weight column, so the
// weights never pass through LDS: lane (c, h) loads the 16 bytes of codes of
// its column c in the 32-k chunk h of a step two steps ahead and
// dequantizes them one step ahead into operand registers.  Inside a 64-k
// step the k order is permuted the same way for A and B: lane half h of
// k-step kk holds k = 32 h + 8 kk .. + 7.  Against a 2 x 2 wave grid sharing
// a dequantized B tile in LDS this reads as many fragment bytes from LDS and
// writes none for the weights (160 KB of LDS traffic per step and compute
// unit instead of 192 KB), with the same dequantization work per lane.
//
// The compiler does not order direct-to-LDS writes against the LDS reads of
// later steps, so every step ends with an explicit wait for all loads issued
// before it, then the workgroup barrier.  Loads past the last step are
// clamped to it (same count every step), and the loop ends with a full wait
// so that nothing writes LDS after the workgroup has finished.
//
// PAIR: the gated MLP front half on 256 x 128 output tiles.  Waves 0 and 1
// sum gate products of output columns 0 .. 63 and 64 .. 127, waves 2 and 3
// up products of the same columns, so wave 2 + w holds the up sums of wave
// w's gate sums register for register; after the loop both pass through LDS
// in register order and H = bf16(act(gate) * up).  No K split.
namespace breg {
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int STAGE = BM * BK;                    // bf16 elements per activation stage
// NW waves side by side, each owning BN / NW columns (FJ 32-column blocks):
// four waves of 64 columns (one per SIMD, 256 accumulators), or eight of 32
// (two per SIMD, 128 accumulators: one wave's dequantization runs while the
// other's MFMAs do)
template <int NW>
struct Geom {
    static constexpr int NT = 64 * NW;
    static constexpr int ADMA = BM * BK * 2 / (1024 * NW);   // direct-to-LDS loads per wave and step
    static constexpr int FJ = BN / (32 * NW);                 // 32-column blocks per wave
    static constexpr int BLOAD = 2 * FJ;                      // code and scale/zero loads per lane and step
};
#ifndef W4_DSWZ
#define W4_DSWZ 3
#endif
__device__ __forceinline__ int swz(int row) { return big::swizzle_fn(W4_DSWZ, row); }
}  // namespace breg

template <bool PAIR, int NW = 4>
__global__ void __launch_bounds__(64 * NW) gemm256_breg_kernel(MulParams p) {
    using namespace breg;
    static_assert(!PAIR || NW % 2 == 0, "the pair form pairs waves w and w + NW / 2");
    constexpr int NT = Geom<NW>::NT, ADMA = Geom<NW>::ADMA, FJ = Geom<NW>::FJ, BLOAD = Geom<NW>::BLOAD;
    constexpr int WNC = BN / NW;                      // columns per wave
    constexpr int FI = 8;
    __shared__ __attribute__((aligned(16))) uint16_t lds_a0[STAGE];
    __shared__ __attribute__((aligned(16))) uint16_t lds_a1[STAGE];
    __shared__ __attribute__((aligned(16))) uint16_t lds_a2[STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int h = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const big::TileJob job = PAIR ? tile_job_t<BM, BN / 2>(p) : big::tile_job(p);
    const int64_t m_base = job.m_base, n_base = job.n_base;
    const int64_t M = p.M, N = p.N, K = p.K;
    const int kb = job.kb, KT = job.KT;
    const int g_shift = group_shift(p.G);

    float16_t acc[FI][FJ];
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // activations: load i of this wave fills LDS rows 8 (wave * ADMA + i) ..
    // + 7 of a stage; lane l writes row + l / 8 at chunk position l % 8, so
    // it loads the chunk that the swizzle puts there, (l % 8) ^ swz(row).
    // Rows past M read row M - 1 and compute outputs that are never stored.
    const int a_row0 = 8 * wave * ADMA + (lane >> 3);
    const int64_t a_m = m_base + a_row0;
    const int64_t a_last = M - 1;
    const uint16_t* a_src = static_cast<const uint16_t*>(p.X);
    auto dma_item = [&](int kt, uint16_t* stage, int it) {
        kt = (kt < KT ? kt : KT - 1) + kb;
        int64_t m = a_m + 8 * it;
        m = m < a_last ? m : a_last;
        const int chunk = (lane & 7) ^ swz(a_row0 + 8 * it);
        const uint16_t* src = a_src + chunk * 8 + m * K + static_cast<int64_t>(kt) * BK;
        // Issued as plain instructions: the compiler cannot tell the three
        // activation stages apart and would otherwise wait for every pending
        // direct-to-LDS load before any LDS read.  There is no register
        // result (the data goes to LDS at M0 + 16 lane), and completion is
        // covered by the explicit wait at the end of each step.  Loads the
        // compiler does not know of only make its own vmcnt waits stricter.
        const uint32_t m0 = __builtin_amdgcn_readfirstlane(
            static_cast<uint32_t>(reinterpret_cast<uintptr_t>(stage + (wave * ADMA + it) * 512)));
        asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m0) : "memory", "m0");
    };

    // weights: column n_base + 64 wave + 32 jb + lane % 32 (PAIR: of the
    // gate weight for waves 0 and 1, of the up weight at 64 (wave - 2) for
    // waves 2 and 3), clamped to N - 1 (its outputs are not stored); 32-k
    // chunk 2 kt + h of step kt
    const bool b_up = PAIR && wave >= NW / 2;
    const int wcol = PAIR ? WNC * (wave % (NW / 2)) : WNC * wave;
    TiledRow brow[FJ];
#pragma unroll
    for (int jb = 0; jb < FJ; ++jb) {
        int64_t bn = n_base + wcol + 32 * jb + (lane & 31);
        bn = bn < N ? bn : N - 1;
        brow[jb] = tiled_row(b_up ? p.wq2 : p.wq, b_up ? p.sz2 : p.sz, bn, N, K, p.G);
    }
    struct Regs {
        u32x4_t q[FJ];
        uint32_t s[FJ];
    };
    auto load_item = [&](int kt, Regs& r, int it) {
        kt = (kt < KT ? kt : KT - 1) + kb;
        if (it < FJ) r.q[it] = *reinterpret_cast<const u32x4_t*>(brow[it].tile_ptr(static_cast<int64_t>(kt) * 2 + h));
        else r.s[it - FJ] = brow[it - FJ].group((kt * BK + 32 * h) >> g_shift);
    };
    // dequantized operands of one step: [kk][jb], word kk of the chunk
    struct BOps {
        u32x4_t b[BK / 16][FJ];
    };
    const uint32_t bias16 = opaque_vgpr(0x64006400u);
    PairDequant dq[FJ];
#pragma unroll
    for (int jb = 0; jb < FJ; ++jb) dq[jb] = PairDequant{bias16};
    // The loaded words are taken in their slots (the scale word with the first
    // pair, each code word with its first pair): the empty asm keeps the
    // compiler from hoisting their conversion, and with it the wait for their
    // loads, to the top of the step.
    uint32_t qpin[FJ];
    auto b_pair = [&](int pr, const Regs& r, BOps& o) {
        const int kk = pr / (4 * FJ), jb = (pr / 4) % FJ, i = pr % 4;
        if (kk == 0 && i == 0) {
            uint32_t sw = r.s[jb];
            asm volatile("" : "+v"(sw));
            dq[jb].group(sw);
        }
        if (i == 0) {
            qpin[jb] = r.q[jb][kk];
            asm volatile("" : "+v"(qpin[jb]));
        }
        o.b[kk][jb][i] = dq[jb].pair(qpin[jb], i);
    };
    // LDS byte offset of the lane's A fragment in row block i (rows 32 i +
    // lane % 32) at k-step kk: 4096 i + aoff[kk][i % 2], since the chunk
    // swizzle of row 32 i + r depends on i only through i % 2 (for swizzle 3,
    // (row ^ row >> 3) & 7, it is swz(r) ^ 4 (i % 2))
    uint32_t aoff[BK / 16][2];
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk)
#pragma unroll
        for (int ip = 0; ip < 2; ++ip) {
            const int r = lane & 31;
            aoff[kk][ip] = static_cast<uint32_t>(r * (BK * 2) + (((4 * h + kk) ^ swz(32 * ip + r)) << 4));
        }
    auto frag_a = [&](const uint16_t* A, int kk, int i) -> bf16x8_t {
        return *reinterpret_cast<const bf16x8_t*>(reinterpret_cast<const char*>(A) + i * 4096 + aoff[kk][i & 1]);
    };
    auto load_a = [&](const uint16_t* A, int kk, bf16x8_t (&a)[FI]) {
#pragma unroll
        for (int i = 0; i < FI; ++i) a[i] = frag_a(A, kk, i);
    };
    constexpr int NSLOT = FI * FJ * (BK / 16);
#ifndef W4_BREG_CONV0
#define W4_BREG_CONV0 4     // in eighths of a step
#endif
    constexpr int BREG_CONV0 = NSLOT * W4_BREG_CONV0 / 8;
    static_assert(BREG_CONV0 < NSLOT, "conversion slots");
    static_assert(4 * ADMA <= NSLOT && 4 * BLOAD <= NSLOT && NSLOT / 2 == 4 * FJ * (BK / 16), "slot plan");

    constexpr int kStepLoads = ADMA + BLOAD;
    auto step_end3 = [&]() {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt((kStepLoads & 15) | (7 << 4) | ((kStepLoads >> 4) << 14));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    auto stage_a = [&](auto S) -> uint16_t* {
        constexpr int s3 = decltype(S)::value;
        return s3 == 0 ? lds_a0 : (s3 == 1 ? lds_a1 : lds_a2);
    };
    // step kt: MFMAs on the operands `cur` (dequantized during step kt - 1);
    // the codes `ready` (step kt + 1) are dequantized into `nxt`, and the
    // weights of step kt + 2 load into `next`
    auto step3 = [&](int kt, auto SA, Regs& next, const Regs& ready, const BOps& cur, BOps& nxt) {
        constexpr int sa = decltype(SA)::value;
        const uint16_t* As = stage_a(std::integral_constant<int, sa>{});
        uint16_t* Ad = stage_a(std::integral_constant<int, (sa + 2) % 3>{});
        // one set of A fragments: fragment i is reloaded for k-step kk + 1
        // right after its last use in k-step kk
        bf16x8_t fa[FI];
        load_a(As, 0, fa);
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < FI * FJ; ++t) {
                const int u = kk * FI * FJ + t;
                const int i = t / FJ, j = t % FJ;
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], __builtin_bit_cast(bf16x8_t, cur.b[kk][j]),
                                                                    acc[i][j], 0, 0, 0);
                if (j == FJ - 1 && kk + 1 < BK / 16) fa[i] = frag_a(As, kk + 1, i);
                if (u % 4 == 0 && u / 4 < BLOAD) {
                    load_item(kt + 2, next, u / 4);
                    asm volatile("" ::: "memory");
                }
                if (u % 4 == 2 && u / 4 < ADMA) dma_item(kt + 2, Ad, u / 4);
                // dequantization of the NSLOT / 2 pairs spread over the
                // second half of the step's slots, which gives the codes
                // loaded during the step before half a step more to arrive
                // (70B shape: 0.844 against 0.851 ms starting at slot 0,
                // 0.847 from a quarter of the step)
#pragma unroll
                for (int pr = 0; pr < NSLOT / 2; ++pr)
                    if (BREG_CONV0 + pr * (NSLOT - BREG_CONV0) / (NSLOT / 2) == u) b_pair(pr, ready, nxt);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        step_end3();
    };
    Regs r0, r1;
    BOps o0, o1;
#pragma unroll
    for (int it = 0; it < ADMA; ++it) dma_item(0, lds_a0, it);
#pragma unroll
    for (int it = 0; it < ADMA; ++it) dma_item(1, lds_a1, it);
#pragma unroll
    for (int it = 0; it < BLOAD; ++it) load_item(0, r0, it);
#pragma unroll
    for (int it = 0; it < BLOAD; ++it) load_item(1, r1, it);
#pragma unroll
    for (int pr = 0; pr < NSLOT / 2; ++pr) b_pair(pr, r0, o0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    // A stages cycle with period 3, code registers and operands with period 2:
    // whole rounds of six steps with no branch between them (the compiler's
    // waits for the loads are then those of one straight path: 812 against
    // 824 us on the 70B shape), then the rest
    int kt0 = 0;
    for (; kt0 + 6 <= KT; kt0 += 6) {
        step3(kt0, I0{}, r0, r1, o0, o1);
        step3(kt0 + 1, I1{}, r1, r0, o1, o0);
        step3(kt0 + 2, I2{}, r0, r1, o0, o1);
        step3(kt0 + 3, I0{}, r1, r0, o1, o0);
        step3(kt0 + 4, I1{}, r0, r1, o0, o1);
        step3(kt0 + 5, I2{}, r1, r0, o1, o0);
    }
    for (int kt = kt0; kt < KT; kt += 6) {
        step3(kt, I0{}, r0, r1, o0, o1);
        if (kt + 1 < KT) step3(kt + 1, I1{}, r1, r0, o1, o0);
        if (kt + 2 < KT) step3(kt + 2, I2{}, r0, r1, o0, o1);
        if (kt + 3 < KT) step3(kt + 3, I0{}, r1, r0, o1, o0);
        if (kt + 4 < KT) step3(kt + 4, I1{}, r0, r1, o0, o1);
        if (kt + 5 < KT) step3(kt + 5, I2{}, r1, r0, o1, o0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    asm volatile("" ::: "memory");

    // epilogue: register r of lane l holds row (r%4) + 4(l/32) + 8(r/4), column l%32
    if (PAIR && job.part >= 0) {
        // a K range of a split pair tile: the fp32 sums of both weights as one
        // 256 x 256 partial tile, gate columns 0..127 and up columns 128..255
#pragma unroll
        for (int i = 0; i < FI; ++i)
#pragma unroll
            for (int j = 0; j < FJ; ++j) {
                const int lc = (b_up ? BN / 2 : 0) + wcol + 32 * j + (lane & 31);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int lr = i * 32 + (r & 3) + 4 * (lane >> 5) + 8 * (r >> 2);
                    p.ws[job.part * (BM * BN) + lr * BN + lc] = acc[i][j][r];
                }
            }
        return;
    }
    if constexpr (PAIR) {
        // rounds (w, hh): gate wave w and up wave NW / 2 + w put the sums of
        // their row blocks 4 hh .. 4 hh + 3 (16 KB per 32 columns, register
        // order) in lds_a0 and lds_a1; then all threads form the 128 x WNC
        // outputs of the round row by row (coalesced stores, one copy of the
        // activation code)
        constexpr int kQ = 4 * FJ * 16 * 64;      // floats per wave and round
        float* const g_l = reinterpret_cast<float*>(lds_a0);
        float* const u_l = reinterpret_cast<float*>(lds_a1);
#pragma unroll
        for (int w = 0; w < NW / 2; ++w)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                __syncthreads();
                if (wave == w || wave == NW / 2 + w) {
                    float* dst = wave == w ? g_l : u_l;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < FJ; ++j)
#pragma unroll
                            for (int r = 0; r < 16; ++r) dst[((i * FJ + j) * 16 + r) * 64 + lane] = acc[4 * hh + i][j][r];
                }
                __syncthreads();
                for (int o = tid; o < kQ; o += NT) {
                    const int lr = o / WNC, lc = o % WNC;        // row in the round's 128, column in the wave's WNC
                    const int64_t row = m_base + 128 * hh + lr, col = n_base + WNC * w + lc;
                    if (row >= M || col >= N) continue;
                    // register order of (lr, lc): block (lr / 32, lc / 32), register
                    // (rr / 8) 4 + rr % 4 of lane ((rr / 4) % 2) 32 + lc % 32, rr = lr % 32
                    const int rr = lr & 31;
                    const int e = ((((lr >> 5) * FJ + (lc >> 5)) * 16 + (rr >> 3) * 4 + (rr & 3)) * 64) +
                                  ((rr >> 2) & 1) * 32 + (lc & 31);
                    p.Y[row * N + col] = float_to_bf16_bits(activation(p.act, g_l[e]) * u_l[e]);
                }
            }
        return;
    }
    // W4A8 (widened E4M3 activations, whole tiles): the row scales of a row
    // block are loaded together before its stores
    const bool scale_rows = p.x_fp8 && job.part < 0;
#pragma unroll
    for (int i = 0; i < FI; ++i) {
        float rsc[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t row = m_base + i * 32 + (r & 3) + 4 * (lane >> 5) + 8 * (r >> 2);
            rsc[r] = scale_rows && row < M ? p.xscale[row] : 1.0f;
        }
#pragma unroll
        for (int j = 0; j < FJ; ++j) {
            const int lc = WNC * wave + 32 * j + (lane & 31);
            const int64_t col = n_base + lc;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int lr = i * 32 + (r & 3) + 4 * (lane >> 5) + 8 * (r >> 2);
                const int64_t row = m_base + lr;
                if (job.part >= 0) p.ws[job.part * (BM * BN) + lr * BN + lc] = acc[i][j][r];   // partial tile of a K split
                else if (row < M && col < N) p.Y[row * N + col] = float_to_bf16_bits(acc[i][j][r] * rsc[r]);
            }
        }
    }
}

// Sum of the K-split partial tiles: output (r, c) of split tile j is the
// fp32 sum of its `splits` partials in split order, times the row scale
// (W4A8), rounded to bf16.  A thread takes four consecutive columns of one
// tile row (16-byte loads; consecutive lanes read consecutive addresses).
template <int BM, int BN>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(MulParams p) {
    const int64_t e4 = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;   // element of the split tiles
    const int64_t j = e4 / (BM * BN);
    const int lr = static_cast<int>((e4 % (BM * BN)) / BN), lc = static_cast<int>(e4 % BN);
    const int64_t nt = (p.N + BN - 1) / BN;
    const int64_t tile = p.split_t0 + j;
    int64_t tr, tc;
    tile_rc(tile, (p.M + BM - 1) / BM, nt, tr, tc);
    const int64_t row = tr * BM + lr, col = tc * BN + lc;
    if (row >= p.M || col >= p.N) return;
    const float* src = p.ws + j * p.splits * (BM * BN) + lr * BN + lc;
    float4 y = *reinterpret_cast<const float4*>(src);
    for (int z = 1; z < p.splits; ++z) {
        const float4 v = *reinterpret_cast<const float4*>(src + z * (BM * BN));
        y.x += v.x; y.y += v.y; y.z += v.z; y.w += v.w;
    }
    if (p.x_fp8) {
        const float r = p.xscale[row];
        y.x *= r; y.y *= r; y.z *= r; y.w *= r;
    }
    const float yv[4] = {y.x, y.y, y.z, y.w};
    uint16_t* dst = p.Y + row * p.N + col;
    if (col + 3 < p.N && p.N % 4 == 0) {
        *reinterpret_cast<uint2*>(dst) = make_uint2(
            float_to_bf16_bits(yv[0]) | (static_cast<uint32_t>(float_to_bf16_bits(yv[1])) << 16),
            float_to_bf16_bits(yv[2]) | (static_cast<uint32_t>(float_to_bf16_bits(yv[3])) << 16));
    } else {
        for (int e = 0; e < 4 && col + e < p.N; ++e) dst[e] = float_to_bf16_bits(yv[e]);
    }
}

// Sum of the K-split partials of the W4A16 gate and up pair on 256 x 128
// output tiles: partial tile [256][256] holds the gate sums in columns
// 0..127 and the up sums in 128..255; H = bf16(act(g) u) with g and u added
// in split order.  A thread takes four consecutive output columns of a row.
__global__ void __launch_bounds__(256) splitk_reduce_pair_kernel(MulParams p) {
    constexpr int BM = big::BM, BN = big::BN, BNO = BN / 2;
    const int64_t e4 = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;   // output of the split tiles
    const int64_t j = e4 / (BM * BNO);
    const int lr = static_cast<int>((e4 % (BM * BNO)) / BNO), lc = static_cast<int>(e4 % BNO);
    const int64_t nt = (p.N + BNO - 1) / BNO;
    int64_t tr, tc;
    tile_rc(p.split_t0 + j, (p.M + BM - 1) / BM, nt, tr, tc);
    const int64_t row = tr * BM + lr, col = tc * BNO + lc;
    if (row >= p.M || col >= p.N) return;
    const float* src = p.ws + j * p.splits * (BM * BN) + lr * BN + lc;
    float4 g = *reinterpret_cast<const float4*>(src);
    float4 u = *reinterpret_cast<const float4*>(src + BNO);
    for (int z = 1; z < p.splits; ++z) {
        const float4 gv = *reinterpret_cast<const float4*>(src + z * (BM * BN));
        const float4 uv = *reinterpret_cast<const float4*>(src + z * (BM * BN) + BNO);
        g.x += gv.x; g.y += gv.y; g.z += gv.z; g.w += gv.w;
        u.x += uv.x; u.y += uv.y; u.z += uv.z; u.w += uv.w;
    }
    const float gs[4] = {g.x, g.y, g.z, g.w}, us[4] = {u.x, u.y, u.z, u.w};
    uint16_t* dst = p.Y + row * p.N + col;
    for (int e = 0; e < 4 && col + e < p.N; ++e) dst[e] = float_to_bf16_bits(activation(p.act, gs[e]) * us[e]);
}

}  // namespace

// K-split schedule of the 256 x 256 GEMM (workgroups run about one per
// compute unit at a time):
//  * fewer tiles than half the compute units: every tile is split, into as
//    many K ranges as keep about one workgroup per compute unit;
//  * otherwise the tiles of the last, partial round are split, so that the
//    round uses every compute unit and takes a fraction of a tile's time.
// At most 16 splits, each of at least 8 K steps of 64.
#ifndef W4_MID_MAXM
#define W4_MID_MAXM 128     // the mid-size tiles serve M up to this (above the streaming kernel's range)
#endif
#ifndef W4_MID_BM
#define W4_MID_BM 64        // tile rows of the mid-size kernel (64 or 128)
#endif
#ifndef W4_MID_WGS
#define W4_MID_WGS 512      // workgroups the mid-size K split aims for (two or three share a compute unit)
#endif
bool use_mid(int64_t M, int64_t K) { return M <= W4_MID_MAXM && K % big::BK == 0; }

// The fp8-MFMA W4A8 kernel takes 128-k steps that each lie in one group:
// groups of 128 (or per-channel rows) and K a multiple of 128; it serves
// every M above kF8MinM.
#ifndef W4_F8_GEMM
#define W4_F8_GEMM 1
#endif
bool f8_eligible(int64_t M, int64_t K, int G) {
    return W4_F8_GEMM && M > kF8MinM && K % kF8StepK == 0 && G % kF8StepK == 0;
}
bool use_f8(const MulParams& p) { return p.x_fp8 && f8_eligible(p.M, p.K, p.G) && f8_fits_buffers(p.M, p.K, p.N); }

// Mid-size tiles: when there are fewer tiles than the target, every tile is
// split along K (at most 16 ways, each of at least 4 steps of 64).  The
// mid-size kernel takes the split count rounded up (more workgroups than the
// target: two or three share a compute unit); the bf16-activation form of
// the fp8 kernel (two 512-thread workgroups a compute unit) rounded down, so
// that its workgroups fit one round (8B up at M = 64: 112 tiles in 4 ranges,
// 448 workgroups, 27.3 -> 23.3 us; with 5 ranges 560 left a second round).
// The workspace is sized for the larger, rounded-up split.
namespace {
GemmSplit mid_or_big_split(int64_t M, int64_t K, int64_t N, bool round_down) {
    constexpr int64_t kCUs = 256;
    GemmSplit g{1, 0, 0, big::BM, big::BN};
    if (N <= 0 || K % big::BK != 0) return g;
    if (use_mid(M, K)) {
        g.bm = W4_MID_BM;
        g.bn = 128;
        g.tiles = ((N + g.bn - 1) / g.bn) * ((M + g.bm - 1) / g.bm);
        g.t0 = g.tiles;
        int64_t s = round_down ? W4_MID_WGS / g.tiles : (W4_MID_WGS + g.tiles - 1) / g.tiles;
        if (s > (K / big::BK) / 4) s = (K / big::BK) / 4;
        if (s > 16) s = 16;
        if (s < 2) return g;
        g.splits = static_cast<int>(s);
        g.t0 = 0;
        return g;
    }
    if (M < 128) return g;
    g.tiles = ((N + big::BN - 1) / big::BN) * ((M + big::BM - 1) / big::BM);
    g.t0 = g.tiles;
#ifndef W4_TAIL_SPLIT
#define W4_TAIL_SPLIT 1
#endif
    const int64_t rem = g.tiles < kCUs / 2 ? g.tiles : (W4_TAIL_SPLIT ? g.tiles % kCUs : 0);
    if (rem == 0) return g;
    int64_t s = kCUs / rem;
    if (s > (K / big::BK) / 8) s = (K / big::BK) / 8;
    if (s > 16) s = 16;
    if (s < 2) return g;
    g.splits = static_cast<int>(s);
    g.t0 = g.tiles - rem;
    return g;
}
}  // namespace
GemmSplit gemm_split(int64_t M, int64_t K, int64_t N) { return mid_or_big_split(M, K, N, false); }

#ifndef W4_A16_MID
#define W4_A16_MID 1
#endif
bool a16_runs(int64_t M, int64_t K, int64_t N, int G, bool x_fp8) {
    return W4_A16_MID && W4_MID_BM == 64 && !x_fp8 && use_mid(M, K) && a16_eligible(M, K, N, G);
}
GemmSplit a16_split(int64_t M, int64_t K, int64_t N) {
    GemmSplit g = mid_or_big_split(M, K, N, true);
    const int bm = a16_tile_rows(M);
    if (bm == g.bm || g.tiles == 0) return g;
    // taller tiles: their own count and split, within the workspace sized
    // for the 64-row tiles' rounded-up split
    const size_t ws = gemm_workspace_bytes(M, K, N);
    GemmSplit t{1, 0, 0, bm, 128};
    t.tiles = ((N + 127) / 128) * ((M + bm - 1) / bm);
    t.t0 = t.tiles;
    int64_t s = (W4_MID_WGS / 2) / t.tiles;   // one such workgroup a compute unit (twice the LDS)
    if (s > (K / big::BK) / 4) s = (K / big::BK) / 4;
    if (s > 16) s = 16;
    const int64_t fit = static_cast<int64_t>(ws / (static_cast<size_t>(t.tiles) * bm * 128 * sizeof(float)));
    if (s > fit) s = fit;
    if (s < 2) return t;
    t.splits = static_cast<int>(s);
    t.t0 = 0;
    return t;
}

size_t gemm_workspace_bytes(int64_t M, int64_t K, int64_t N) {
    const GemmSplit g = gemm_split(M, K, N);
    if (g.splits == 1) return 0;
    return static_cast<size_t>(g.tiles - g.t0) * g.splits * g.bm * g.bn * sizeof(float);
}

size_t gemm_xw_offset(int64_t M, int64_t K, int64_t N) { return (gemm_workspace_bytes(M, K, N) + 255) & ~size_t{255}; }

// The widened activations pay from a whole round of 256 x 256 tiles over the
// 256 compute units: on the 70B shape (896 tiles, M = 2048) the bf16 kernel
// with them takes 0.83 ms against 0.87 ms for the E4M3 kernel, while on the
// 12B shapes at M = 256 (15 or 60 tiles, every one split 16 or 4 ways) it
// takes 67-69 us against 57-61 us, the extra row-quantizer writes included.
size_t gemm_xw_bytes(int64_t M, int64_t K, int64_t N) {
    if (M <= 0 || K <= 0 || N <= 0 || use_mid(M, K) || M < 128 || K % big::BK != 0) return 0;
    const int64_t tiles = ((M + big::BM - 1) / big::BM) * ((N + big::BN - 1) / big::BN);
    if (tiles < 256) return 0;
    return static_cast<size_t>(M) * static_cast<size_t>(K) * sizeof(uint16_t);
}

// wave grid of the register-path kernel (used for E4M3 activations): 4 x 2
// waves of 64 x 128 outputs measured faster than 2 x 2 of 128 x 128
#ifndef W4_BIG_WM
#define W4_BIG_WM 4
#define W4_BIG_WN 2
#endif
constexpr int kBigWM = W4_BIG_WM, kBigWN = W4_BIG_WN;
// Waves of the W4A16 256 x 256 kernel: eight of 32 columns, two per SIMD, so
// that one wave's dequantization and waits run under the other's MFMAs.
// Measured on one MI355X against four of 64 columns (one per SIMD): 12B up
// at M = 1024 (240 tiles) 118 against 126 us; the 70B shape at M = 2048
// (896 tiles) 810-812 against 832 us (with the dequantization in the second
// half of each step; 823 against 817 us before it).

template <int TBM, bool XF8>
hipError_t launch_mid(const MulParams& p, hipStream_t stream) {
    constexpr int TBN = 128;
    const int64_t tiles = ((p.N + TBN - 1) / TBN) * ((p.M + TBM - 1) / TBM);
    MulParams q = p;
    if (q.splits <= 1) {
        q.splits = 1;
        q.split_t0 = tiles;
        q.ws = nullptr;
    }
    if (q.splits > q.K / big::BK || q.split_t0 < 0 || q.split_t0 > tiles || (q.splits > 1 && !q.ws))
        return hipErrorInvalidValue;
    const int64_t wgs = q.split_t0 + (tiles - q.split_t0) * q.splits;
    hipLaunchKernelGGL((gemm_mid_kernel<TBM, TBN, 2, 2, XF8>), dim3(static_cast<unsigned>(wgs)), dim3(256), 0, stream, q);
    if (q.splits > 1 && q.split_t0 < tiles) {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t blocks = (tiles - q.split_t0) * (TBM * TBN / 1024);
        hipLaunchKernelGGL((splitk_reduce_kernel<TBM, TBN>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, q);
    }
    return hipGetLastError();
}

template <int TBM, bool XF8>
hipError_t launch_pair_t(const MulParams& p, hipStream_t stream) {
    constexpr int OUTN = 128;
    const int64_t tiles = ((p.N + OUTN - 1) / OUTN) * ((p.M + TBM - 1) / TBM);
    MulParams q = p;
    q.splits = 1;
    q.split_t0 = tiles;
    q.ws = nullptr;
    hipLaunchKernelGGL((gemm_mid_kernel<TBM, 2 * OUTN, 2, 2, XF8, true>), dim3(static_cast<unsigned>(tiles)), dim3(256), 0,
                       stream, q);
    return hipGetLastError();
}

// Gate and up GEMM (M above the streaming kernel's pair range), no K split:
// W4A8 with groups of 128 on the fp8 kernel's pair form; W4A16 above 256
// rows on 256 x 128 output tiles of the direct-to-LDS kernel (eight waves,
// four per weight); otherwise
// output tiles of 64 (M <= 64) or 128 rows by 128 columns.
// Measured on the 8B gate / up shapes (two 14336 x 4096): at M = 256 the
// 128-row tiles take 98 us against 138 us for one row of 256-row tiles (224
// workgroups against 112); from M = 384 the 256-row kernel is ahead
// (151 / 179 us).  A 256-row form of the 128-row kernel spilled and ran
// tens of times slower.
// waves of the W4A16 pair kernel: eight (four per weight, two per SIMD);
// 8B gate + up at M = 2048: 471-475 us against 516 us with four
#ifndef W4_BREG_PAIR_NW
#define W4_BREG_PAIR_NW 8
#endif
hipError_t launch_gemm_pair(const MulParams& p, hipStream_t stream) {
    if (p.M == 0 || p.N == 0) return hipSuccess;
    if (p.K % big::BK != 0 || !p.wq2 || !p.sz2) return hipErrorInvalidValue;
    // W4A8 with groups of 128 (or whole rows): the fp8 kernel's pair form
    if (use_f8(p)) return launch_gemm_f8_pair(p, stream);
    if (!p.x_fp8 && p.M > 256) {
        // W4A16: gemm256_breg_kernel on 256 x 128 output tiles, the tiles of
        // the last, partial round split along K when the caller gave the
        // workspace of pair_split (p.splits and p.split_t0 from it)
        const GemmSplit g = pair_split(p.M, p.K, p.N);
        MulParams q = p;
        if (q.splits <= 1 || !q.ws) {
            q.splits = 1;
            q.split_t0 = g.tiles;
            q.ws = nullptr;
        } else if (q.splits != g.splits || q.split_t0 != g.t0) {
            return hipErrorInvalidValue;
        }
        const int64_t wgs = q.split_t0 + (g.tiles - q.split_t0) * q.splits;
        hipLaunchKernelGGL((gemm256_breg_kernel<true, W4_BREG_PAIR_NW>), dim3(static_cast<unsigned>(wgs)),
                           dim3(breg::Geom<W4_BREG_PAIR_NW>::NT), 0, stream, q);
        if (q.splits > 1) {
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            const int64_t blocks = (g.tiles - q.split_t0) * (big::BM * big::BN / 2 / 1024);
            hipLaunchKernelGGL(splitk_reduce_pair_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, q);
        }
        return hipGetLastError();
    }
#ifndef W4_A16_PAIR
#define W4_A16_PAIR 1
#endif
    if (W4_A16_PAIR && !p.x_fp8 && a16_pair_eligible(p.M, p.K, p.N, p.G)) return launch_gemm_a16_pair(p, stream);
    if (p.M <= 64) return p.x_fp8 ? launch_pair_t<64, true>(p, stream) : launch_pair_t<64, false>(p, stream);
    return p.x_fp8 ? launch_pair_t<128, true>(p, stream) : launch_pair_t<128, false>(p, stream);
}

// K split of the W4A16 pair kernel (above 256 rows, K a multiple of 64):
// the tiles of the last, partial round over the compute units in as many K
// ranges as fill it (at most 16, each of at least 8 steps of 64), as for the
// 256 x 256 GEMM; tiles of 256 x 128 outputs.
GemmSplit pair_split(int64_t M, int64_t K, int64_t N) {
    constexpr int64_t kCUs = 256;
    GemmSplit g{1, 0, 0, big::BM, big::BN / 2};
    if (M <= 256 || N <= 0 || K % big::BK != 0) return g;
    g.tiles = ((N + big::BN / 2 - 1) / (big::BN / 2)) * ((M + big::BM - 1) / big::BM);
    g.t0 = g.tiles;
    const int64_t rem = g.tiles < kCUs / 2 ? g.tiles : g.tiles % kCUs;
    if (rem == 0) return g;
    int64_t s = kCUs / rem;
    if (s > (K / big::BK) / 8) s = (K / big::BK) / 8;
    if (s > 16) s = 16;
    if (s < 2) return g;
    g.splits = static_cast<int>(s);
    g.t0 = g.tiles - rem;
    return g;
}

size_t pair_workspace_bytes(int64_t M, int64_t K, int64_t N) {
    const GemmSplit g = pair_split(M, K, N);
    if (g.splits == 1) return 0;
    return static_cast<size_t>(g.tiles - g.t0) * g.splits * big::BM * big::BN * sizeof(float);
}

int64_t gate_up_amax_tiles(int64_t M, int64_t N) { return M <= kGateUpMaxM ? (N + 15) / 16 : (N + 127) / 128; }

hipError_t launch_split_sum(const MulParams& q, int bm, int bn, int64_t tiles, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>((tiles - q.split_t0) * (static_cast<int64_t>(bm) * bn / 1024)));
    if (bm == 256 && bn == 256)
        hipLaunchKernelGGL((splitk_reduce_kernel<256, 256>), grid, dim3(256), 0, stream, q);
    else if (bm == 128 && bn == 256)
        hipLaunchKernelGGL((splitk_reduce_kernel<128, 256>), grid, dim3(256), 0, stream, q);
    else if (bm == 64 && bn == 256)
        hipLaunchKernelGGL((splitk_reduce_kernel<64, 256>), grid, dim3(256), 0, stream, q);
    else if (bm == 64 && bn == 128)
        hipLaunchKernelGGL((splitk_reduce_kernel<64, 128>), grid, dim3(256), 0, stream, q);
    else if (bm == 256 && bn == 128)
        hipLaunchKernelGGL((splitk_reduce_kernel<256, 128>), grid, dim3(256), 0, stream, q);
    else if (bm == 256 && bn == 64)
        hipLaunchKernelGGL((splitk_reduce_kernel<256, 64>), grid, dim3(256), 0, stream, q);
    else if (bm == 128 && bn == 128)
        hipLaunchKernelGGL((splitk_reduce_kernel<128, 128>), grid, dim3(256), 0, stream, q);
    else if (bm == 64 && bn == 64)
        hipLaunchKernelGGL((splitk_reduce_kernel<64, 64>), grid, dim3(256), 0, stream, q);
    else if (bm == 128 && bn == 64)
        hipLaunchKernelGGL((splitk_reduce_kernel<128, 64>), grid, dim3(256), 0, stream, q);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_gemm(const MulParams& p, hipStream_t stream) {
    if (p.M == 0 || p.N == 0) return hipSuccess;
    // W4A8 on the fp8 matrix cores (groups of 128 or whole rows), on its own
    // tiles and split schedule
    if (use_f8(p)) return launch_gemm_f8(p, stream);
    if (use_mid(p.M, p.K)) {
        if (a16_runs(p.M, p.K, p.N, p.G, p.x_fp8)) return launch_gemm_a16(p, stream);
        constexpr int bm = W4_MID_BM;
        return p.x_fp8 ? launch_mid<bm, true>(p, stream) : launch_mid<bm, false>(p, stream);
    }
    if (p.M >= 128 && p.K % big::BK == 0) {
        // the split schedule the workspace was sized for; every split keeps
        // at least one K step
        const int64_t tiles = ((p.N + big::BN - 1) / big::BN) * ((p.M + big::BM - 1) / big::BM);
        MulParams q = p;
        if (q.splits <= 1) {
            q.splits = 1;
            q.split_t0 = tiles;
            q.ws = nullptr;
        }
        if (q.splits > q.K / big::BK || q.split_t0 < 0 || q.split_t0 > tiles || (q.splits > 1 && !q.ws))
            return hipErrorInvalidValue;
        const int64_t wgs = q.split_t0 + (tiles - q.split_t0) * q.splits;
        const dim3 grid(static_cast<unsigned>(wgs));
        if (q.x_fp8 && q.xw) {
            // W4A8 on the widened activations: the bf16 kernel, row scales in
            // its epilogue (or in the split sum)
            q.X = q.xw;
            hipLaunchKernelGGL((gemm256_breg_kernel<false, 8>), grid, dim3(breg::Geom<8>::NT), 0, stream, q);
        } else if (q.x_fp8) {
            hipLaunchKernelGGL((gemm256_kernel<kBigWM, kBigWN, true>), grid, dim3(64 * kBigWM * kBigWN), 0, stream, q);
        } else {
            hipLaunchKernelGGL((gemm256_breg_kernel<false, 8>), grid, dim3(breg::Geom<8>::NT), 0, stream, q);
        }
        if (q.splits > 1 && q.split_t0 < tiles) {
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            const int64_t blocks = (tiles - q.split_t0) * (big::BM * big::BN / 1024);
            hipLaunchKernelGGL((splitk_reduce_kernel<big::BM, big::BN>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, q);
        }
        return hipGetLastError();
    }
    const dim3 grid(static_cast<unsigned>((p.N + small::BN - 1) / small::BN),
                    static_cast<unsigned>((p.M + small::BM - 1) / small::BM));
    if (p.x_fp8)
        hipLaunchKernelGGL((gemm_kernel<true>), grid, dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL((gemm_kernel<false>), grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace w4
