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
// Large-M kernel.  A 256-thread workgroup (2 x 2 waves of 128 x 128 outputs,
// 4 x 4 MFMA 32x32x16 tiles each) owns a 256 x 256 output tile and walks K in
// steps of 64 with two LDS stages (128 KB):
//   * activations go from global memory straight into LDS
//     (global_load_lds_dwordx4: lane l's 16 bytes land at the instruction's
//     LDS base + 16 l), so they never occupy registers;
//   * each thread owns one weight row of the tile: 32 code bytes and its
//     scale/zero word per K step, dequantized to bf16 and stored to LDS;
//   * the next step's loads are in flight while the current step's 64 MFMAs
//     per wave run, and its dequantization follows them.
// LDS rows are 128 bytes (64 bf16); the 16-byte chunk c of row r is stored at
// position c ^ ((r >> 1) & 7), which spreads the 32 rows an MFMA operand read
// touches over all banks.
namespace big {
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int STAGE = 256 * BK;          // bf16 elements per operand and stage

__device__ __forceinline__ int lds_off(int row, int c) { return row * BK + ((c ^ ((row >> 1) & 7)) << 3); }

typedef uint32_t __attribute__((address_space(1))) global_u32;
typedef uint32_t __attribute__((address_space(3))) lds_u32;
}  // namespace big

template <int WM, int WN, bool XF8>
__global__ void __launch_bounds__(64 * WM * WN) gemm256_kernel(MulParams p) {
    using namespace big;
    constexpr int NT = 64 * WM * WN;         // threads
    constexpr int TM = BM / WM, TN = BN / WN; // wave tile
    constexpr int FI = TM / 32, FJ = TN / 32; // 32 x 32 MFMA tiles per wave
    constexpr int TPR = NT / 256;             // threads per weight row
    constexpr int WPT = (BK / 8) / TPR;       // code words per thread and K step
    constexpr int AINS = 32 / (NT / 64);      // direct-to-LDS instructions per wave and K step
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
    const uint32_t bias = opaque_vgpr(kBf16Bias128x2);

    float16_t acc[FI][FJ];
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // weight row of this thread and its first code word within a K step
    const int b_row = tid / TPR;
    const int b_w0 = (tid % TPR) * WPT;
    int64_t bn = n_base + b_row;
    bn = bn < N ? bn : N - 1;              // rows past N compute garbage that is never stored
    const uint32_t* brow = p.wq + bn * words_row + b_w0;
    const uint32_t* bsz = p.sz + bn * groups_row;
    // activation row of this thread (W4A8 path: bytes converted through registers)
    constexpr int A8_CH = (BK / 16) / TPR;  // 16-byte chunks of E4M3 activations per thread and K step
    static_assert(A8_CH >= 1 && A8_CH * TPR * 16 == BK, "E4M3 row split");
    int64_t am = m_base + b_row;
    am = am < M ? am : M - 1;

    uint32_t bq[WPT];
    uint32_t bs;
    uint4 aq[A8_CH];

    auto issue_loads = [&](int kt, int stage) {
        if constexpr (!XF8) {
            // activations: instruction i of wave w fills LDS slots (w * AINS + i) *
            // 64 + lane, slot s = row * 8 + position, position = chunk ^ ((row >> 1) & 7)
            const uint16_t* X = static_cast<const uint16_t*>(p.X);
#pragma unroll
            for (int i = 0; i < AINS; ++i) {
                const int slot0 = (wave * AINS + i) * 64;
                const int s = slot0 + lane;
                const int row = s >> 3;
                const int c = (s & 7) ^ ((row >> 1) & 7);
                int64_t m = m_base + row;
                m = m < M ? m : M - 1;
                const uint16_t* g = X + m * K + static_cast<int64_t>(kt) * BK + c * 8;
                __builtin_amdgcn_global_load_lds((const global_u32*)(const void*)g,
                                                 (lds_u32*)(void*)(lds + stage * 2 * STAGE + slot0 * 8), 16, 0, 0);
            }
        } else {
            // E4M3 activations: each thread A8_CH 16-byte chunks (64 / TPR bytes) of its row
            const uint4* g = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(p.X) + am * K +
                                                            static_cast<int64_t>(kt) * BK) + (tid % TPR) * A8_CH;
#pragma unroll
            for (int i = 0; i < A8_CH; ++i) aq[i] = g[i];
        }
        const uint32_t* w = brow + static_cast<int64_t>(kt) * (BK / 8);
#pragma unroll
        for (int i = 0; i < WPT; i += 4) {
            const uint4 t = *reinterpret_cast<const uint4*>(w + i);
            bq[i] = t.x; bq[i + 1] = t.y; bq[i + 2] = t.z; bq[i + 3] = t.w;
        }
        // the thread's WPT words (8 * WPT k) lie in one group when G >= 8 * WPT
        bs = bsz[(static_cast<int64_t>(kt) * BK + b_w0 * 8) / p.G];
    };

    auto store_operands = [&](int stage) {
        uint16_t* B = lds + stage * 2 * STAGE + STAGE;
        const float sc = half_bits_to_float(bs);
        const float cs = (128.0f + half_bits_to_float(bs >> 16)) * sc;
#pragma unroll
        for (int j = 0; j < WPT; ++j) {
            uint32_t o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t pr = nibble_pair_bf16(bq[j], i, bias);
                o[i] = pack_bf16x2(fmaf(bf16_lo(pr), sc, -cs), fmaf(bf16_hi(pr), sc, -cs));
            }
            *reinterpret_cast<uint4*>(B + lds_off(b_row, b_w0 + j)) = make_uint4(o[0], o[1], o[2], o[3]);
        }
        if constexpr (XF8) {
            uint16_t* A = lds + stage * 2 * STAGE;
#pragma unroll
            for (int i = 0; i < A8_CH; ++i) {
                const uint32_t bw[4] = {aq[i].x, aq[i].y, aq[i].z, aq[i].w};
                uint32_t o[8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(bw[j]), false);
                    float2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(bw[j]), true);
                    o[2 * j] = pack_bf16x2(lo[0], lo[1]);
                    o[2 * j + 1] = pack_bf16x2(hi[0], hi[1]);
                }
                const int c0 = ((tid % TPR) * A8_CH + i) * 2;
                *reinterpret_cast<uint4*>(A + lds_off(b_row, c0)) = make_uint4(o[0], o[1], o[2], o[3]);
                *reinterpret_cast<uint4*>(A + lds_off(b_row, c0 + 1)) = make_uint4(o[4], o[5], o[6], o[7]);
            }
        }
    };

    auto compute = [&](int stage) {
        const uint16_t* A = lds + stage * 2 * STAGE;
        const uint16_t* B = A + STAGE;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int c = 2 * kk + (lane >> 5);
            bf16x8_t a[FI], b[FJ];
#pragma unroll
            for (int i = 0; i < FI; ++i)
                a[i] = *reinterpret_cast<const bf16x8_t*>(A + lds_off(wm * TM + i * 32 + (lane & 31), c));
#pragma unroll
            for (int j = 0; j < FJ; ++j)
                b[j] = *reinterpret_cast<const bf16x8_t*>(B + lds_off(wn * TN + j * 32 + (lane & 31), c));
#pragma unroll
            for (int i = 0; i < FI; ++i)
#pragma unroll
                for (int j = 0; j < FJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    };

    issue_loads(0, 0);
    store_operands(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int stage = kt & 1;
        // branch free: the last step reloads its own data into the idle stage
        const int kn = kt + 1 < KT ? kt + 1 : kt;
        issue_loads(kn, stage ^ 1);
        compute(stage);
        store_operands(stage ^ 1);
        __builtin_amdgcn_s_waitcnt(0);     // direct-to-LDS loads and LDS stores of the next stage
        __syncthreads();
    }

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
