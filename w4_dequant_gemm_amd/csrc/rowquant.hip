// Dynamic per-row FP8 E4M3 quantization of bf16 activations (gowda.ai "LLM
// fast inference", "Achievement 2"): for each row m,
//   xscale[m] = max(amax_m / 448, 1e-8)      (448 = largest finite E4M3)
//   xq[m, k]  = e4m3(fl32(x[m, k] / xscale[m])), round to nearest even,
//               saturating at +-448.
// The scale is recomputed on every call, so one row's outlier never costs
// another row resolution, and an all-zero row stays exactly zero.
//
// One block per row (256 threads, 1024 for rows of 12288 or more values): a
// max reduction (wavefront butterfly, then LDS across the waves) over the row, or over the partial row maxima its
// producer left (the fused gate and up pass), then a pass over the row that
// divides (a reciprocal product with one exact-residual correction, which
// gives the codes of the correctly rounded quotient: e4m3_quotient), clamps
// to +-448 and converts pairs with
// v_cvt_pk_fp8_f32 (OCP E4M3 on gfx950).  Rows are read 16 bytes per lane,
// once (kept in registers between the two passes) up to 32768 per row.
#include "device.hpp"
#include "kernels.hpp"

#pragma clang fp contract(off)

namespace w4 {
namespace {

// Row of up to REG * NT 16-byte pieces (K <= 32768 for both block sizes):
// each thread keeps its pieces in registers between the maximum and the
// quantizing pass, so the row is read once; longer rows are read twice.

__device__ __forceinline__ float amax8(uint4 v, float amax) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        amax = fmaxf(amax, fabsf(bf16_lo(w[j])));
        amax = fmaxf(amax, fabsf(bf16_hi(w[j])));
    }
    return amax;
}

__device__ __forceinline__ void quant8(const RowQuantParams& p, int64_t m, int64_t i, uint4 v, float s, float r) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float f[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f[2 * j] = fminf(fmaxf(e4m3_quotient(bf16_lo(w[j]), s, r), -448.0f), 448.0f);
        f[2 * j + 1] = fminf(fmaxf(e4m3_quotient(bf16_hi(w[j]), s, r), -448.0f), 448.0f);
    }
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], hi, true);
    reinterpret_cast<uint2*>(p.xq + m * p.K)[i] = make_uint2(static_cast<uint32_t>(lo), static_cast<uint32_t>(hi));
    if (p.xw) {
        // the same codes widened to bf16 (exact: every finite E4M3 value is a
        // bf16 value), two per conversion with scale 1
        const uint32_t c[2] = {static_cast<uint32_t>(lo), static_cast<uint32_t>(hi)};
        uint32_t wv[4];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            wv[2 * j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[j], 1.0f, false));
            wv[2 * j + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[j], 1.0f, true));
        }
        reinterpret_cast<uint4*>(p.xw + m * p.K)[i] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    }
}

template <int NT, int REG>
__global__ void __launch_bounds__(NT) rowquant_kernel(RowQuantParams p) {
    constexpr int NWV = NT / 64;
    __shared__ float red[NWV];
    const int64_t m = blockIdx.x;
    const int64_t K8 = p.K / 8;
    const uint4* x = reinterpret_cast<const uint4*>(p.X + m * p.K);
    const int tid = threadIdx.x;
    const bool in_regs = K8 <= REG * NT;

    float amax = 0.0f;
    uint4 v[REG];
    if (in_regs) {
#pragma unroll
        for (int r = 0; r < REG; ++r) {
            const int64_t i = tid + NT * r;
            v[r] = i < K8 ? x[i] : make_uint4(0u, 0u, 0u, 0u);
        }
    }
    if (p.amax_part) {
        // the producer of X left the row's maximum in partial maxima
        const float* part = p.amax_part + m * p.amax_tiles;
        for (int64_t i = tid; i < p.amax_tiles; i += NT) amax = fmaxf(amax, part[i]);
    } else if (in_regs) {
#pragma unroll
        for (int r = 0; r < REG; ++r) amax = amax8(v[r], amax);
    } else {
        for (int64_t i = tid; i < K8; i += NT) amax = amax8(x[i], amax);
    }
    amax = wave_max(amax);
    if ((tid & 63) == 0) red[tid >> 6] = amax;
    __syncthreads();
    amax = red[0];
#pragma unroll
    for (int w = 1; w < NWV; ++w) amax = fmaxf(amax, red[w]);

    float s = amax / 448.0f;
    s = fmaxf(s, 1e-8f);
    if (tid == 0) p.xscale[m] = s;
    const float rs = 1.0f / s;

    if (in_regs) {
#pragma unroll
        for (int r = 0; r < REG; ++r) {
            const int64_t i = tid + NT * r;
            if (i < K8) quant8(p, m, i, v[r], s, rs);
        }
    } else {
        for (int64_t i = tid; i < K8; i += NT) quant8(p, m, i, x[i], s, rs);
    }
}

}  // namespace

hipError_t launch_rowquant(const RowQuantParams& p, hipStream_t stream) {
    if (p.M == 0) return hipSuccess;
#ifndef W4_RQ_WIDE_K
#define W4_RQ_WIDE_K 12288
#endif
    // long rows: four times the threads, so that the quantizing pass of one
    // row (all on one compute unit) takes a quarter of the time (M = 2048:
    // K = 28672 38.2 -> 32.9 us; at K = 8192 the 256-thread blocks are 4%
    // faster)
    if (p.K >= W4_RQ_WIDE_K)
        hipLaunchKernelGGL((rowquant_kernel<1024, 4>), dim3(static_cast<unsigned>(p.M)), dim3(1024), 0, stream, p);
    else
        hipLaunchKernelGGL((rowquant_kernel<256, 16>), dim3(static_cast<unsigned>(p.M)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace w4
