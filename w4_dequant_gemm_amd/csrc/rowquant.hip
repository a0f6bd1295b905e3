// Dynamic per-row FP8 E4M3 quantization of bf16 activations (gowda.ai "LLM
// fast inference", "Achievement 2"): for each row m,
//   xscale[m] = max(amax_m / 448, 1e-8)      (448 = largest finite E4M3)
//   xq[m, k]  = e4m3(fl32(x[m, k] / xscale[m])), round to nearest even,
//               saturating at +-448.
// The scale is recomputed on every call, so one row's outlier never costs
// another row resolution, and an all-zero row stays exactly zero.
//
// One 256-thread block per row: a max reduction (wavefront butterfly, then
// LDS across the 4 waves), then a second pass over the row that divides
// (IEEE, correctly rounded), clamps to +-448 and converts pairs with
// v_cvt_pk_fp8_f32 (OCP E4M3 on gfx950).  Rows are read 16 bytes per lane.
#include "device.hpp"
#include "kernels.hpp"

#pragma clang fp contract(off)

namespace w4 {
namespace {

__global__ void __launch_bounds__(256) rowquant_kernel(RowQuantParams p) {
    __shared__ float red[4];
    const int64_t m = blockIdx.x;
    const int64_t K8 = p.K / 8;
    const uint4* x = reinterpret_cast<const uint4*>(p.X + m * p.K);

    float amax = 0.0f;
    for (int64_t i = threadIdx.x; i < K8; i += blockDim.x) {
        const uint4 v = x[i];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            amax = fmaxf(amax, fabsf(bf16_lo(w[j])));
            amax = fmaxf(amax, fabsf(bf16_hi(w[j])));
        }
    }
    amax = wave_max(amax);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

    float s = amax / 448.0f;
    s = fmaxf(s, 1e-8f);
    if (threadIdx.x == 0) p.xscale[m] = s;

    uint2* out = reinterpret_cast<uint2*>(p.xq + m * p.K);
    for (int64_t i = threadIdx.x; i < K8; i += blockDim.x) {
        const uint4 v = x[i];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        float f[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f[2 * j] = fminf(fmaxf(bf16_lo(w[j]) / s, -448.0f), 448.0f);
            f[2 * j + 1] = fminf(fmaxf(bf16_hi(w[j]) / s, -448.0f), 448.0f);
        }
        int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
        lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], lo, true);
        int hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
        hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], hi, true);
        out[i] = make_uint2(static_cast<uint32_t>(lo), static_cast<uint32_t>(hi));
        if (p.xw) {
            // the same codes widened to bf16 (exact: every finite E4M3 value
            // is a bf16 value), two per conversion with scale 1
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
}

}  // namespace

hipError_t launch_rowquant(const RowQuantParams& p, hipStream_t stream) {
    if (p.M == 0) return hipSuccess;
    hipLaunchKernelGGL(rowquant_kernel, dim3(static_cast<unsigned>(p.M)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace w4
