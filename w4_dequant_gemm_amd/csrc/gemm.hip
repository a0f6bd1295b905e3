// W4A16 / W4A8 GEMM for M > 16 on gfx950 bf16 MFMA.
//
// At prefill sizes the products are compute bound and the dequantization work
// shows (gsantana.dev "Quantizing LLMs Without Guesswork", "Production
// reality"), so each packed weight tile is dequantized once per workgroup into
// LDS and then reused by every activation row of the workgroup tile:
//
//   global (4-bit GPU layout) -> registers: (128 + u) as bf16 via AND-OR,
//   widened to fp32, W' = (128 + u) s - (128 + z) s (exact in fp32: every
//   product has fewer than 24 significant bits), rounded to bf16 (RNE)
//   -> LDS -> v_mfma_f32_32x32x16_bf16 with fp32 accumulation -> bf16 out.
//
// W4A8 reads the E4M3 activations produced by the row quantizer, widens them
// exactly to bf16 and multiplies by the row scale in the epilogue.
//
// Tile: 128 x 128 outputs per 256-thread workgroup (2 x 2 waves of 64 x 64),
// K step 32.  Rows of X beyond M and rows of W beyond N read as zero; the
// epilogue stores only in-range outputs.
#include "device.hpp"
#include "kernels.hpp"

namespace w4 {
namespace {

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
    const int64_t words_row = K / 8, groups_row = K / p.G;
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
                const uint2 w = *reinterpret_cast<const uint2*>(p.wq + n * words_row + k0 / 8 + b_w);
                const uint32_t szw = p.sz[n * groups_row + (k0 + 8 * b_w) / p.G];
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
// position c ^ ((r >> 1) & 7), spreading an MFMA operand read over the banks.
namespace big {
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int STAGE = 256 * BK;          // bf16 elements per operand and stage

__device__ __forceinline__ int lds_off(int row, int c) { return row * BK + ((c ^ ((row >> 1) & 7)) << 3); }
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
    // dequantization VALU work per MFMA in one step (about 6 instructions per
    // bf16 pair, 4 pairs per chunk; E4M3 widening adds 3 per pair)
    constexpr int VALU_PER_MFMA = XF8 ? 5 : 3;
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * 2 * STAGE];   // [stage][A, B][256 x 64]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int64_t m_base = static_cast<int64_t>(blockIdx.y) * BM;
    const int64_t n_base = static_cast<int64_t>(blockIdx.x) * BN;
    const int64_t M = p.M, N = p.N, K = p.K;
    const int64_t words_row = K / 8, groups_row = K / p.G;
    const int KT = static_cast<int>(K / BK);
    const int g_shift = __builtin_ctz(static_cast<unsigned>(p.G));   // G is a power of two
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
    const uint32_t* brow = p.wq + bn * words_row + o_c0;
    const uint32_t* bsz = p.sz + bn * groups_row;
    // Activation row address with its provenance hidden (an empty asm): loads
    // through it are then not known to be invariant, so the register
    // allocator cannot re-issue them at their use a step later instead of
    // keeping the prefetched values.  Re-cast to the global address space so
    // that they stay global (not flat) loads.
    uint64_t arow_addr = reinterpret_cast<uint64_t>(static_cast<const uint8_t*>(p.X) + (am * K + o_c0 * 8) * XB);
    asm volatile("" : "+v"(arow_addr));
    typedef const u32x4_t __attribute__((address_space(1))) global_u4;
    const global_u4* arow = (const global_u4*)arow_addr;

    struct Regs {
        uint4 a[ALD];
        uint32_t q[CPT];
        uint32_t s;
    };
    Regs r0, r1;

    auto issue_loads = [&](int kt, Regs& r) {
        kt = kt < KT ? kt : KT - 1;         // past the end: reload the last step (never used)
        const global_u4* ga = arow + static_cast<int64_t>(kt) * (BK * XB / 16);
#pragma unroll
        for (int i = 0; i < ALD; ++i) {
            const u32x4_t t = ga[i];
            r.a[i] = make_uint4(t[0], t[1], t[2], t[3]);
        }
        const uint32_t* w = brow + static_cast<int64_t>(kt) * (BK / 8);
#pragma unroll
        for (int i = 0; i < CPT; i += 4) {
            const uint4 t = *reinterpret_cast<const uint4*>(w + i);
            r.q[i] = t.x; r.q[i + 1] = t.y; r.q[i + 2] = t.z; r.q[i + 3] = t.w;
        }
        // the thread's CPT words (8 * CPT k) lie in one group when G >= 8 * CPT
        r.s = bsz[(kt * BK + o_c0 * 8) >> g_shift];
    };

    auto store_operands = [&](int stage, const Regs& r) {
        uint16_t* A = lds + stage * 2 * STAGE;
        uint16_t* B = A + STAGE;
        if constexpr (!XF8) {
#pragma unroll
            for (int i = 0; i < ALD; ++i) {
                // pass through an empty asm at this point, so the copy (and the
                // wait for its load) is not scheduled ahead of the MFMA phase
                uint4 v = r.a[i];
                asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
                *reinterpret_cast<uint4*>(A + lds_off(o_row, o_c0 + i)) = v;
            }
        } else {
#pragma unroll
            for (int i = 0; i < ALD; ++i) {
                const uint32_t bw[4] = {r.a[i].x, r.a[i].y, r.a[i].z, r.a[i].w};
                uint32_t o[8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(bw[j]), false);
                    float2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(bw[j]), true);
                    o[2 * j] = pack_bf16x2(lo[0], lo[1]);
                    o[2 * j + 1] = pack_bf16x2(hi[0], hi[1]);
                }
                *reinterpret_cast<uint4*>(A + lds_off(o_row, o_c0 + 2 * i)) = make_uint4(o[0], o[1], o[2], o[3]);
                *reinterpret_cast<uint4*>(A + lds_off(o_row, o_c0 + 2 * i + 1)) = make_uint4(o[4], o[5], o[6], o[7]);
            }
        }
        const float sc = half_bits_to_float(r.s);
        const float cs = (128.0f + half_bits_to_float(r.s >> 16)) * sc;
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            uint32_t o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t pr = nibble_pair_bf16(r.q[j], i, bias);
                o[i] = pack_bf16x2(fmaf(bf16_lo(pr), sc, -cs), fmaf(bf16_hi(pr), sc, -cs));
            }
            *reinterpret_cast<uint4*>(B + lds_off(o_row, o_c0 + j)) = make_uint4(o[0], o[1], o[2], o[3]);
        }
    };

    auto compute = [&](int stage) {
        const uint16_t* A = lds + stage * 2 * STAGE;
        const uint16_t* B = A + STAGE;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int ch = 2 * kk + (lane >> 5);
            bf16x8_t a[FI], b[FJ];
#pragma unroll
            for (int i = 0; i < FI; ++i)
                a[i] = *reinterpret_cast<const bf16x8_t*>(A + lds_off(wm * TM + i * 32 + (lane & 31), ch));
#pragma unroll
            for (int j = 0; j < FJ; ++j)
                b[j] = *reinterpret_cast<const bf16x8_t*>(B + lds_off(wn * TN + j * 32 + (lane & 31), ch));
#pragma unroll
            for (int i = 0; i < FI; ++i)
#pragma unroll
                for (int j = 0; j < FJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    };

    // One K step: loads for kt + 2 into `next` (its previous contents, step
    // kt, were converted during step kt - 1), MFMAs of kt, convert kt + 1
    // from `ready` into the idle stage, then synchronize.
    // The loads must stay in flight across the MFMAs.  An activation load
    // whose value is only copied to LDS a step later would otherwise be sunk
    // next to that copy by the optimizer (nothing in between writes global
    // memory); the empty asm with a memory clobber pins the loads here without
    // emitting code, and the scheduling barrier keeps them ahead of the rest.
    // The MFMAs of step kt and the conversion of step kt + 1 (different LDS
    // stages) are then interleaved: one MFMA, then a few VALU instructions,
    // so the matrix cores keep running while the dequantization executes.
    auto step = [&](int kt, Regs& next, const Regs& ready) {
        issue_loads(kt + 2, next);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        compute(kt & 1);
        store_operands((kt + 1) & 1, ready);   // past the end this refills an idle stage
#pragma unroll
        for (int i = 0; i < FI * FJ * (BK / 16); ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, VALU_PER_MFMA, 0);   // VALU
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
            const int64_t col = n_base + wn * TN + j * 32 + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m_base + wm * TM + i * 32 + (r & 3) + 4 * (lane >> 5) + 8 * (r >> 2);
                if (row < M && col < N) {
                    float y = acc[i][j][r];
                    if constexpr (XF8) y *= p.xscale[row];
                    p.Y[row * N + col] = float_to_bf16_bits(y);
                }
            }
        }
}

}  // namespace

hipError_t launch_gemm(const MulParams& p, hipStream_t stream) {
    if (p.M == 0 || p.N == 0) return hipSuccess;
    if (p.M >= 128 && p.K % big::BK == 0) {
        const dim3 grid(static_cast<unsigned>((p.N + big::BN - 1) / big::BN),
                        static_cast<unsigned>((p.M + big::BM - 1) / big::BM));
        if (p.x_fp8)
            hipLaunchKernelGGL((gemm256_kernel<4, 2, true>), grid, dim3(512), 0, stream, p);
        else
            hipLaunchKernelGGL((gemm256_kernel<4, 2, false>), grid, dim3(512), 0, stream, p);
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
