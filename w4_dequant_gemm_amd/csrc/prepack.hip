// Portable packing -> GPU layout, once per weight, without requantizing
// (gowda.ai "LLM fast inference", "MSE clipping": the portable packed codes,
// scales and zero terms are rearranged into a GPU-specific layout).
//
// Codes: every group of 8 codes (k = 8j .. 8j+7 of one row) becomes one
// 32-bit word:
//   * codes become unsigned: u = q (asymmetric) or u = q + 8 (symmetric, two's
//     complement -> offset binary, i.e. the nibble XOR 8), with zero = 8;
//   * code 8j + 2i goes to bits 4i..4i+3, code 8j + 2i + 1 to bits 16+4i..;
//     so (w >> 4i) & 0x000F000F yields the pair (u[2i], u[2i+1]) in the low
//     bits of the two 16-bit halves -- one AND-OR with a bf16 constant turns it
//     into two bf16 values in natural k order, matching bf16 activation pairs.
// Words are stored in 16-row blocks of 32-k tiles: for rows r0 .. r0 + nr - 1
// (r0 a multiple of 16, nr = min(16, N - r0)), tile t (k = 32t .. 32t + 31)
// holds the four words of each row in turn, row c of the block at words
// r0 K/8 + t 4 nr + 4c .. + 3.  A wavefront reading 1 KB contiguously thus
// receives, in lane c + 16h, the 32 codes of row c in tile 4s + h: exactly
// the operand fragments of a 16-column matrix-core product, with plain
// 128-byte-line reads.
// Scale and zero are interleaved into one 32-bit word per group (fp16 scale
// in the low half, fp16 zero in the high half) and blocked the same way:
// group g of row r0 + c at r0 (K/G) + g nr + c.
#include "device.hpp"
#include "kernels.hpp"

namespace w4 {
namespace {

// Position of row n's item i (word or group index within the row, `per_row`
// items per row, `per_tile` items per row and tile) in the blocked layout.
__device__ __forceinline__ int64_t blocked_index(int64_t n, int64_t i, int64_t N, int64_t per_row, int64_t per_tile) {
    const int64_t r0 = n & ~static_cast<int64_t>(15);
    const int64_t nr = N - r0 < 16 ? N - r0 : 16;
    const int64_t c = n - r0;
    const int64_t t = i / per_tile, w = i % per_tile;
    return r0 * per_row + t * per_tile * nr + c * per_tile + w;
}

// one thread per canonical 32-bit word (8 codes) and per group
__global__ void __launch_bounds__(256) prepack_kernel(PrepackParams p) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t words_row = p.K / 8, groups_row = p.K / p.G;
    const int64_t n_words = p.N * words_row;
    const int64_t n_groups = p.N * groups_row;
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
        p.wq[blocked_index(idx / words_row, idx % words_row, p.N, words_row, 4)] = out;
    }
    if (idx < n_groups) {
        const uint32_t z = p.asym ? p.zero[idx] : 0x4800u;  // fp16 8.0
        p.sz[blocked_index(idx / groups_row, idx % groups_row, p.N, groups_row, 1)] =
            static_cast<uint32_t>(p.scale[idx]) | (z << 16);
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
