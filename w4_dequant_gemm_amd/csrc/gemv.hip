// W4A16 / W4A8 decode GEMV for M <= 16 rows of activations, gfx950.
//
// At batch 1 decoding reads every weight once and that read sets the pace
// (gsantana.dev "Quantizing LLMs Without Guesswork", "The Problem & Context";
// W4A16 dequantizes inside the matmul and computes in 16-bit, section
// "Weight-only methods").  So this kernel streams the packed codes from HBM
// exactly once, 16/8/4 contiguous bytes per lane, and keeps the arithmetic per
// weight to about one VALU op:
//
//   * a code word holds pairs (u[2i], u[2i+1]) in the low nibbles of its two
//     halves (GPU layout, see prepack.hip); one AND-OR with 0x43004300 turns a
//     pair into two exact bf16 values 128 + u;
//   * v_dot2_f32_bf16 multiplies that pair with the matching bf16 activation
//     pair and accumulates in fp32;
//   * the scale and zero point are applied once per lane and group:
//       sum_k (u - z) s x = s * (sum_k (128 + u) x - (128 + z) * sum_k x),
//     where sum_k x over the lane's k range is computed once per chunk and
//     reused for every row.
//
// Mapping: a wave owns R consecutive output rows; lane l covers KL
// consecutive k of each 64*KL-wide chunk of the row (KL = 32, 16 or 8 as M
// grows, to bound the activation registers); partial sums per (row, m) are
// reduced across the wave with a reduce-scatter butterfly, after which every
// lane holds one finished output.  W4A8 reads E4M3 activations, widens them
// exactly to bf16 and applies the row scale at the end (gowda.ai "LLM fast
// inference", "Achievement 2": FP32 accumulation, row scale in the epilogue,
// BF16 output).
#include "device.hpp"
#include "kernels.hpp"

namespace w4 {
namespace {

// Sum V values held by every lane of a wave; afterwards lane L holds the total
// of value index `idx`.  V is a power of two <= 64.  Each step halves the
// values a lane keeps (exchanging the other half with its partner), so the
// cost is about V shuffles instead of 6V.
template <int V>
__device__ __forceinline__ float wave_reduce_scatter(float (&a)[V], int lane, int& idx) {
    static_assert(V >= 1 && V <= 64 && (V & (V - 1)) == 0, "V must be a power of two <= 64");
    idx = 0;
    int off = 32;
#pragma unroll
    for (int h = V / 2; h >= 1; h /= 2, off /= 2) {
        const bool upper = (lane & off) != 0;
#pragma unroll
        for (int i = 0; i < h; ++i) {
            const float send = upper ? a[i] : a[h + i];
            const float keep = upper ? a[h + i] : a[i];
            a[i] = keep + __shfl_xor(send, off, kWave);
        }
        if (upper) idx += h;
    }
    float v = a[0];
    for (; off >= 1; off /= 2) v += __shfl_xor(v, off, kWave);
    return v;
}

template <int MT, int KL, int R, bool XF8>
__global__ void __launch_bounds__(256) gemv_kernel(MulParams p) {
    constexpr int XW = KL / 2;   // bf16 activation pairs per lane and row of X
    constexpr int WW = KL / 8;   // code words per lane and weight row
    const int lane = threadIdx.x & 63;
    const int64_t wave = static_cast<int64_t>(blockIdx.x) * (blockDim.x / 64) + (threadIdx.x >> 6);
    const int64_t n0 = wave * R;
    if (n0 >= p.N) return;
    const int64_t K = p.K, N = p.N;
    const int M = static_cast<int>(p.M);
    const int64_t words_row = K / 8;
    const int64_t groups_row = K / p.G;

    float acc[R * MT];
#pragma unroll
    for (int i = 0; i < R * MT; ++i) acc[i] = 0.0f;

    for (int64_t kc = 0; kc < K; kc += 64 * KL) {
        const int64_t k0 = kc + static_cast<int64_t>(lane) * KL;
        const bool active = k0 < K;

        // weights first, so their HBM latency overlaps the activation work
        uint32_t wv[R][WW];
        uint32_t szv[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t n = n0 + r;
            const bool ok = active && n < N;
            const uint32_t* src = p.wq + n * words_row + k0 / 8;
            if constexpr (WW == 4) {
                uint4 t = ok ? *reinterpret_cast<const uint4*>(src) : make_uint4(0, 0, 0, 0);
                wv[r][0] = t.x; wv[r][1] = t.y; wv[r][2] = t.z; wv[r][3] = t.w;
            } else if constexpr (WW == 2) {
                uint2 t = ok ? *reinterpret_cast<const uint2*>(src) : make_uint2(0, 0);
                wv[r][0] = t.x; wv[r][1] = t.y;
            } else {
                wv[r][0] = ok ? *src : 0u;
            }
            szv[r] = ok ? p.sz[n * groups_row + k0 / p.G] : 0u;
        }

        uint32_t xw[MT][XW];
        float xs[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const bool ok = active && m < M;
            if constexpr (!XF8) {
                const uint16_t* xr = static_cast<const uint16_t*>(p.X) + static_cast<int64_t>(m) * K + k0;
#pragma unroll
                for (int j = 0; j < XW; j += 4) {
                    uint4 t = ok ? *reinterpret_cast<const uint4*>(xr + 2 * j) : make_uint4(0, 0, 0, 0);
                    xw[m][j] = t.x; xw[m][j + 1] = t.y; xw[m][j + 2] = t.z; xw[m][j + 3] = t.w;
                }
            } else {
                // E4M3 -> fp32 (exact) -> bf16 pair (exact: 3 mantissa bits fit)
                const uint8_t* xr = static_cast<const uint8_t*>(p.X) + static_cast<int64_t>(m) * K + k0;
#pragma unroll
                for (int j = 0; j < XW; j += 2) {
                    const uint32_t b4 = ok ? *reinterpret_cast<const uint32_t*>(xr + 2 * j) : 0u;
                    float2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(b4), false);
                    float2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(b4), true);
                    xw[m][j] = pack_bf16x2(lo[0], lo[1]);
                    xw[m][j + 1] = pack_bf16x2(hi[0], hi[1]);
                }
            }
            float s = 0.0f;
#pragma unroll
            for (int j = 0; j < XW; ++j) s += bf16_lo(xw[m][j]) + bf16_hi(xw[m][j]);
            xs[m] = s;
        }

#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float sc = half_bits_to_float(szv[r]);
            const float cz = 128.0f + half_bits_to_float(szv[r] >> 16);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                float d = 0.0f;
#pragma unroll
                for (int ww = 0; ww < WW; ++ww)
#pragma unroll
                    for (int i = 0; i < 4; ++i) d = dot2_bf16(nibble_pair_bf16(wv[r][ww], i), xw[m][4 * ww + i], d);
                acc[r * MT + m] = fmaf(sc, d - cz * xs[m], acc[r * MT + m]);
            }
        }
    }

    constexpr int V = R * MT;
    int idx;
    if constexpr (V <= 64) {
        const float v = wave_reduce_scatter<V>(acc, lane, idx);
        // lanes whose bits below the scatter level are zero hold distinct totals
        constexpr int lanes_per = 64 / V;
        if ((lane & (lanes_per - 1)) == 0) {
            const int r = idx / MT, m = idx % MT;
            const int64_t n = n0 + r;
            if (n < N && m < M) {
                float y = v;
                if constexpr (XF8) y *= p.xscale[m];
                p.Y[static_cast<int64_t>(m) * N + n] = float_to_bf16_bits(y);
            }
        }
    }
}

template <int MT, int KL, int R, bool XF8>
hipError_t launch_t(const MulParams& p, hipStream_t stream) {
    const int waves_per_block = 4;
    const int64_t waves = (p.N + R - 1) / R;
    const int64_t blocks = (waves + waves_per_block - 1) / waves_per_block;
    hipLaunchKernelGGL((gemv_kernel<MT, KL, R, XF8>), dim3(static_cast<unsigned>(blocks)),
                       dim3(64 * waves_per_block), 0, stream, p);
    return hipGetLastError();
}

template <int MT, int KL, bool XF8>
hipError_t launch_r(const MulParams& p, hipStream_t stream) {
    // enough waves to cover the 256 CUs several times over, few enough rows
    // per wave that each keeps several loads in flight
    if (p.N >= 8192) return launch_t<MT, KL, 4, XF8>(p, stream);
    if (p.N >= 2048) return launch_t<MT, KL, 2, XF8>(p, stream);
    return launch_t<MT, KL, 1, XF8>(p, stream);
}

template <bool XF8>
hipError_t launch_m(const MulParams& p, hipStream_t stream) {
    if (p.M <= 1) return launch_r<1, 32, XF8>(p, stream);
    if (p.M <= 2) return launch_r<2, 32, XF8>(p, stream);
    if (p.M <= 4) return launch_r<4, 16, XF8>(p, stream);
    if (p.M <= 8) return launch_r<8, 8, XF8>(p, stream);
    return launch_r<16, 8, XF8>(p, stream);
}

}  // namespace

hipError_t launch_gemv(const MulParams& p, hipStream_t stream) {
    if (p.M == 0 || p.N == 0) return hipSuccess;
    if (p.M > kGemvMaxM) return hipErrorInvalidValue;
    return p.x_fp8 ? launch_m<true>(p, stream) : launch_m<false>(p, stream);
}

}  // namespace w4
