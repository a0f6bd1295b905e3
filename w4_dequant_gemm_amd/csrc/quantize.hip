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
// a[j] += a[j + len] for len = G/2, G/4, ..., 1.
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
        const float e = Tree<G, 0, 1, ASYM>::eval(v, s, zf);
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
        default: return hipErrorInvalidValue;
    }
}

}  // namespace w4
