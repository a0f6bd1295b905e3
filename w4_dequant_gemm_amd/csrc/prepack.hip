// Portable packing -> GPU layout, once per weight, without requantizing
// (gowda.ai "LLM fast inference", "MSE clipping": the portable packed codes,
// scales and zero terms are rearranged into a GPU-specific layout).
//
// GPU layout, per 32-bit word of 8 codes (k = 8j .. 8j+7):
//   * codes become unsigned: u = q (asymmetric) or u = q + 8 (symmetric, two's
//     complement -> offset binary, i.e. the nibble XOR 8), with zero = 8;
//   * code 8j + 2i goes to bits 4i..4i+3, code 8j + 2i + 1 to bits 16+4i..;
//     so (w >> 4i) & 0x000F000F yields the pair (u[2i], u[2i+1]) in the low
//     bits of the two 16-bit halves -- one AND-OR with a bf16 constant turns it
//     into two bf16 values in natural k order, matching bf16 activation pairs.
// Scale and zero are interleaved into one 32-bit word per group so a kernel
// fetches both with one load.
#include "device.hpp"
#include "kernels.hpp"

namespace w4 {
namespace {

__global__ void __launch_bounds__(256) prepack_kernel(PrepackParams p) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t n_words = p.N * (p.K / 8);
    const int64_t n_groups = p.N * (p.K / p.G);
    if (idx < n_words) {
        uint32_t c = reinterpret_cast<const uint32_t*>(p.packed)[idx];
        if (!p.asym) c ^= 0x88888888u;
        uint32_t out = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t nib = (c >> (4 * i)) & 0xFu;
            const int dst = (i & 1) ? 16 + 4 * (i >> 1) : 4 * (i >> 1);
            out |= nib << dst;
        }
        p.wq[idx] = out;
    }
    if (idx < n_groups) {
        const uint32_t z = p.asym ? p.zero[idx] : 0x4800u;  // fp16 8.0
        p.sz[idx] = static_cast<uint32_t>(p.scale[idx]) | (z << 16);
    }
}

}  // namespace

hipError_t launch_prepack(const PrepackParams& p, hipStream_t stream) {
    const int64_t n_words = p.N * (p.K / 8);
    if (n_words == 0) return hipSuccess;
    const int threads = 256;
    const int64_t blocks = (n_words + threads - 1) / threads;
    hipLaunchKernelGGL(prepack_kernel, dim3(static_cast<unsigned>(blocks)), dim3(threads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace w4
