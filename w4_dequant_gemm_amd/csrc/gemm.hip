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

constexpr int BM = 128, BN = 128, BK = 32;
constexpr int LDS_STRIDE = BK + 8;   // bf16 elements per LDS row (16 bytes of padding)

template <bool XF8>
__global__ void __launch_bounds__(256) gemm_kernel(MulParams p) {
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

}  // namespace

hipError_t launch_gemm(const MulParams& p, hipStream_t stream) {
    if (p.M == 0 || p.N == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>((p.N + BN - 1) / BN), static_cast<unsigned>((p.M + BM - 1) / BM));
    if (p.x_fp8)
        hipLaunchKernelGGL((gemm_kernel<true>), grid, dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL((gemm_kernel<false>), grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace w4
