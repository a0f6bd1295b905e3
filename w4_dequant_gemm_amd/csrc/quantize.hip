// Blockwise INT4 quantizer with the data-free MSE clip search, for gfx950.
//
// What is computed (gowda.ai "LLM fast inference", sections "Achievement 1"
// and "MSE clipping"; gsantana.dev "Quantizing LLMs Without Guesswork",
// "Scale and zero point" and "Quantize, then dequantize"): for every group of G
// consecutive weights of a row, each clip fraction f gives a candidate range
// (asym: [min, max] at f = 1, else [mid - f h, mid + f h] about the observed
// midpoint; sym: [-f amax, f amax]); its fp16-rounded scale, integer zero
// point and codes; and its squared reconstruction error, clipped values
// included.  The first candidate is kept unless a later one is strictly
// better; the winner's codes are packed two per byte.
//
// Bit-exactness: every float operation is one IEEE binary32 operation with
// round-to-nearest-even in a fixed order -- no contraction into FMA (this file
// is built with -ffp-contract=off and the pragma below), correctly rounded
// division, v_rndne for half-to-even rounding, v_cvt_f16_f32 for the fp16
// scale.  The error of a group is added by a fixed pairwise halving tree:
// a[j] += a[j + len] for len = G/2, G/4, ..., 1.  In the search, rne(w / s)
// comes from w times the correctly rounded 1/s, which rounds to the same
// integer except within 2^-22 |w/s| of a half-integer; a candidate with any
// weight that close is recomputed with divisions (err2_fast).
//
// Mapping: one lane owns one group; its G weights stay in registers for the
// whole search, so the tree runs inside the lane with no cross-lane traffic
// and the per-candidate scale/zero arithmetic is done once per lane.  A wave
// covers 64 consecutive groups, i.e. a contiguous 64*G*4-byte span of W.
#include "device.hpp"
#include "kernels.hpp"

#pragma clang fp contract(off)

namespace w4 {
namespace {

template <bool ASYM>
struct Grid {
    static constexpr float lo = ASYM ? 0.0f : -8.0f;
    static constexpr float hi = ASYM ? 15.0f : 7.0f;
};

// Squared error of one weight under (s, zf): w - (clamp(rne(w/s) + zf) - zf) * s.
template <bool ASYM>
__device__ __forceinline__ float err2(float w, float s, float zf) {
    float t = rintf(w / s);
    float q = fminf(fmaxf(t + zf, Grid<ASYM>::lo), Grid<ASYM>::hi);
    float xr = (q - zf) * s;
    float e = w - xr;
    return e * e;
}

// The same with rne(w/s) taken from t = w * inv, inv = 1/s correctly
// rounded: t is within 2^-22 |t| of the correctly rounded quotient (two
// roundings of 2^-24 each), so both round to the same integer unless t lies
// within that distance of a half-integer.  Such a weight (a margin of
// 2^-20 |t| is used, or a NaN) sets `near`, and the caller redoes the
// candidate with exact divisions; otherwise the result is the same bits.
template <bool ASYM>
__device__ __forceinline__ float err2_fast(float w, float s, float zf, float inv, bool& near) {
    const float tq = w * inv;
    const float t = rintf(tq);
    near |= !(fabsf(fabsf(tq - t) - 0.5f) > fabsf(tq) * 0x1p-20f);
    float q = fminf(fmaxf(t + zf, Grid<ASYM>::lo), Grid<ASYM>::hi);
    float xr = (q - zf) * s;
    float e = w - xr;
    return e * e;
}

// Node (J, LEN) of the halving tree: after the passes for lengths G/2 .. LEN,
// a[J] = node(J, 2 LEN) + node(J + LEN, 2 LEN); the leaves of the first pass
// are e2[J] + e2[J + G/2].  Evaluated depth first to keep few partials live.
template <int G, int J, int LEN, bool ASYM>
struct Tree {
    static __device__ __forceinline__ float eval(const float* v, float s, float zf) {
        if constexpr (LEN == G / 2) {
            return err2<ASYM>(v[J], s, zf) + err2<ASYM>(v[J + G / 2], s, zf);
        } else {
            float a = Tree<G, J, 2 * LEN, ASYM>::eval(v, s, zf);
            float b = Tree<G, J + LEN, 2 * LEN, ASYM>::eval(v, s, zf);
            return a + b;
        }
    }
    static __device__ __forceinline__ float eval_fast(const float* v, float s, float zf, float inv, bool& near) {
        if constexpr (LEN == G / 2) {
            return err2_fast<ASYM>(v[J], s, zf, inv, near) + err2_fast<ASYM>(v[J + G / 2], s, zf, inv, near);
        } else {
            float a = Tree<G, J, 2 * LEN, ASYM>::eval_fast(v, s, zf, inv, near);
            float b = Tree<G, J + LEN, 2 * LEN, ASYM>::eval_fast(v, s, zf, inv, near);
            return a + b;
        }
    }
};

template <int G, bool ASYM>
__global__ void __launch_bounds__(256) quantize_kernel(QuantizeParams p) {
    const int64_t grp = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (grp >= p.n_groups) return;

    float v[G];
    const float4* src = reinterpret_cast<const float4*>(p.W + grp * G);
#pragma unroll
    for (int i = 0; i < G / 4; ++i) {
        float4 t = src[i];
        v[4 * i + 0] = t.x;
        v[4 * i + 1] = t.y;
        v[4 * i + 2] = t.z;
        v[4 * i + 3] = t.w;
    }
    float wmin = v[0], wmax = v[0], amax = fabsf(v[0]);
#pragma unroll
    for (int j = 1; j < G; ++j) {
        wmin = fminf(wmin, v[j]);
        wmax = fmaxf(wmax, v[j]);
        amax = fmaxf(amax, fabsf(v[j]));
    }

    int best = 0;
    float best_err = 0.0f, best_s = 1.0f, best_z = 0.0f;
    uint32_t best_sb = 0x3C00u;
    for (int i = 0; i < p.n_fracs; ++i) {
        const float f = p.fracs[i];
        float s32;
        float lo = 0.0f;
        if constexpr (ASYM) {
            float hi;
            if (f == 1.0f) {
                lo = wmin;
                hi = wmax;
            } else {
                float mid = (wmax + wmin) * 0.5f;
                float h = (wmax - wmin) * 0.5f;
                float fh = f * h;
                lo = mid - fh;
                hi = mid + fh;
            }
            s32 = (hi - lo) / 15.0f;
        } else {
            s32 = (f * amax) / 7.0f;
        }
        uint32_t sb = float_to_half_bits(s32);
        float s = half_bits_to_float(sb);
        if (s == 0.0f) {
            s = 1.0f;
            sb = 0x3C00u;
        }
        const float zf = ASYM ? rintf(-lo / s) : 0.0f;
        bool near = false;
        float e = Tree<G, 0, 1, ASYM>::eval_fast(v, s, zf, 1.0f / s, near);
        if (near) e = Tree<G, 0, 1, ASYM>::eval(v, s, zf);   // rare: some w / s next to a half-integer
        if (p.sse) p.sse[grp * p.n_fracs + i] = e;
        if (i == 0 || e < best_err) {
            best = i;
            best_err = e;
            best_s = s;
            best_z = zf;
            best_sb = sb;
        }
    }

    if (p.clip) p.clip[grp] = static_cast<uint8_t>(best);
    if (!p.encode) return;

    p.scale[grp] = static_cast<uint16_t>(best_sb);
    if constexpr (ASYM) p.zero[grp] = static_cast<uint16_t>(float_to_half_bits(best_z + 0.0f));

    // Canonical packing: byte b holds code 2b (low nibble) and 2b+1 (high);
    // 32 codes make one 16-byte store.
    uint4* dst = reinterpret_cast<uint4*>(p.packed + grp * (G / 2));
#pragma unroll
    for (int c = 0; c < G / 32; ++c) {
        uint32_t words[4];
#pragma unroll
        for (int wi = 0; wi < 4; ++wi) {
            uint32_t word = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float w = v[32 * c + 8 * wi + i];
                float q = fminf(fmaxf(rintf(w / best_s) + best_z, Grid<ASYM>::lo), Grid<ASYM>::hi);
                uint32_t nib = static_cast<uint32_t>(static_cast<int>(q)) & 0xFu;
                word |= nib << (4 * i);
            }
            words[wi] = word;
        }
        dst[c] = make_uint4(words[0], words[1], words[2], words[3]);
    }
}

// ------------------------------------------------------------ per-channel
//
// One group per row (G = K, the per-channel granularity of gsantana.dev
// "Granularity: who shares a scale"): one 1024-thread workgroup per row.  The
// halving tree of a group whose size is not a power of two runs over the
// errors padded with zeros to the next power of two P (zeros change no sum),
// and a tree over max(P, 1024) values gives the same sums (the extra first
// levels add zeros).  Thread t holds elements t + 1024 i, i < RPT: the levels
// with length >= 1024 pair elements of one thread, the rest go through LDS
// (lengths 512 .. 64) and wave shuffles (32 .. 1), each level computing
// a[j] = a[j] + a[j + len] exactly as the group kernel does in registers.
constexpr int kRowThreads = 1024;

template <int RPT, bool ASYM>
__global__ void __launch_bounds__(kRowThreads) quantize_row_kernel(QuantizeParams p, int64_t K) {
    __shared__ float red[kRowThreads];
    __shared__ float wstat[3][kRowThreads / 64];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int64_t row = blockIdx.x;
    const float* w_row = p.W + row * K;
    // element t + 1024 i is in the row when i < n_in
    const int n_in = static_cast<int>((K - t + kRowThreads - 1) / kRowThreads);
    float v[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) v[i] = i < n_in ? w_row[t + static_cast<int64_t>(kRowThreads) * i] : 0.0f;
    // statistics of the row (order-free: min, max, max |w|)
    float wmin = INFINITY, wmax = -INFINITY, amax = 0.0f;
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        if (i < n_in) {
            wmin = fminf(wmin, v[i]);
            wmax = fmaxf(wmax, v[i]);
            amax = fmaxf(amax, fabsf(v[i]));
        }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        wmin = fminf(wmin, __shfl_xor(wmin, o, 64));
        wmax = fmaxf(wmax, __shfl_xor(wmax, o, 64));
        amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    }
    if (lane == 0) {
        wstat[0][wave] = wmin;
        wstat[1][wave] = wmax;
        wstat[2][wave] = amax;
    }
    __syncthreads();
    wmin = wstat[0][0];
    wmax = wstat[1][0];
    amax = wstat[2][0];
    for (int w = 1; w < kRowThreads / 64; ++w) {
        wmin = fminf(wmin, wstat[0][w]);
        wmax = fmaxf(wmax, wstat[1][w]);
        amax = fmaxf(amax, wstat[2][w]);
    }

    int best = 0;
    float best_err = 0.0f, best_s = 1.0f, best_z = 0.0f;
    uint32_t best_sb = 0x3C00u;
    for (int c = 0; c < p.n_fracs; ++c) {
        const float f = p.fracs[c];
        float s32;
        float lo = 0.0f;
        if constexpr (ASYM) {
            float hi;
            if (f == 1.0f) {
                lo = wmin;
                hi = wmax;
            } else {
                float mid = (wmax + wmin) * 0.5f;
                float h = (wmax - wmin) * 0.5f;
                float fh = f * h;
                lo = mid - fh;
                hi = mid + fh;
            }
            s32 = (hi - lo) / 15.0f;
        } else {
            s32 = (f * amax) / 7.0f;
        }
        uint32_t sb = float_to_half_bits(s32);
        float s = half_bits_to_float(sb);
        if (s == 0.0f) {
            s = 1.0f;
            sb = 0x3C00u;
        }
        const float zf = ASYM ? rintf(-lo / s) : 0.0f;
        // the tree: levels inside the thread, then LDS, then shuffles
        float a[RPT];
        bool near = false;
        const float inv = 1.0f / s;
#pragma unroll
        for (int i = 0; i < RPT; ++i) a[i] = i < n_in ? err2_fast<ASYM>(v[i], s, zf, inv, near) : 0.0f;
        if (near) {                          // rare: some w / s next to a half-integer
#pragma unroll
            for (int i = 0; i < RPT; ++i) a[i] = i < n_in ? err2<ASYM>(v[i], s, zf) : 0.0f;
        }
#pragma unroll
        for (int len = RPT / 2; len >= 1; len /= 2)
#pragma unroll
            for (int i = 0; i < len; ++i) a[i] = a[i] + a[i + len];
        __syncthreads();                     // the previous candidate's reads of red are done
        red[t] = a[0];
        __syncthreads();
#pragma unroll
        for (int len = kRowThreads / 2; len >= 64; len /= 2) {
            if (t < len) red[t] = red[t] + red[t + len];
            __syncthreads();
        }
        if (wave == 0) {
            float x = red[t];
#pragma unroll
            for (int len = 32; len >= 1; len /= 2) {
                const float y = __shfl_down(x, len, 64);
                if (t < len) x = x + y;
            }
            if (t == 0) red[0] = x;
        }
        __syncthreads();
        const float e = red[0];
        if (p.sse && t == 0) p.sse[row * p.n_fracs + c] = e;
        if (c == 0 || e < best_err) {
            best = c;
            best_err = e;
            best_s = s;
            best_z = zf;
            best_sb = sb;
        }
    }

    if (t == 0) {
        if (p.clip) p.clip[row] = static_cast<uint8_t>(best);
        if (p.encode) {
            p.scale[row] = static_cast<uint16_t>(best_sb);
            if constexpr (ASYM) p.zero[row] = static_cast<uint16_t>(float_to_half_bits(best_z + 0.0f));
        }
    }
    if (!p.encode) return;
    // canonical packing: element j = t + 1024 i pairs with j + 1 in lane t + 1
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const float q = fminf(fmaxf(rintf(v[i] / best_s) + best_z, Grid<ASYM>::lo), Grid<ASYM>::hi);
        const uint32_t nib = static_cast<uint32_t>(static_cast<int>(q)) & 0xFu;
        const uint32_t hi_nib = __shfl_down(nib, 1, 64);
        const int64_t j = t + static_cast<int64_t>(kRowThreads) * i;
        if ((t & 1) == 0 && i < n_in) p.packed[(row * K + j) / 2] = static_cast<uint8_t>(nib | (hi_nib << 4));
    }
}

template <int RPT, bool ASYM>
hipError_t launch_row(const QuantizeParams& p, int64_t K, hipStream_t stream) {
    hipLaunchKernelGGL((quantize_row_kernel<RPT, ASYM>), dim3(static_cast<unsigned>(p.n_groups)), dim3(kRowThreads), 0,
                       stream, p, K);
    return hipGetLastError();
}

template <bool ASYM>
hipError_t launch_per_channel(const QuantizeParams& p, hipStream_t stream) {
    const int64_t K = p.G;
    int64_t P = kRowThreads;
    while (P < K) P *= 2;
    switch (P / kRowThreads) {
        case 1: return launch_row<1, ASYM>(p, K, stream);
        case 2: return launch_row<2, ASYM>(p, K, stream);
        case 4: return launch_row<4, ASYM>(p, K, stream);
        case 8: return launch_row<8, ASYM>(p, K, stream);
        case 16: return launch_row<16, ASYM>(p, K, stream);
        case 32: return launch_row<32, ASYM>(p, K, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int G, bool ASYM>
hipError_t launch(const QuantizeParams& p, hipStream_t stream) {
    const int threads = 256;
    const int64_t blocks = (p.n_groups + threads - 1) / threads;
    hipLaunchKernelGGL((quantize_kernel<G, ASYM>), dim3(static_cast<unsigned>(blocks)), dim3(threads), 0,
                       stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const QuantizeParams& p, hipStream_t stream) {
    if (p.n_groups == 0) return hipSuccess;
    switch (p.G) {
        case 32: return p.asym ? launch<32, true>(p, stream) : launch<32, false>(p, stream);
        case 64: return p.asym ? launch<64, true>(p, stream) : launch<64, false>(p, stream);
        case 128: return p.asym ? launch<128, true>(p, stream) : launch<128, false>(p, stream);
        default:
            // any other size is one group per row (per-channel, G = K <= 32768)
            if (p.G > kMaxPerChannelK || p.G % 32 != 0) return hipErrorInvalidValue;
            return p.asym ? launch_per_channel<true>(p, stream) : launch_per_channel<false>(p, stream);
    }
}

}  // namespace w4
