// Plain streaming read, for measurement only: the HBM read rate that one
// launch reaches over a buffer the size of one decode product's weights,
// recorded beside the products' own rates as the achievable ceiling.  Built
// into libw4probe.so, apart from the product library; the products never
// call it.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Thread t reads 16-byte words t, t + T, t + 2T, ... (T threads in the grid),
// four of them in flight per iteration, with non-temporal loads as the
// products use for their weights.  Every index is checked against n.  The
// XOR of all words is stored only if it equals a fixed constant, which keeps
// the loads without writing anything in practice.
__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4* __restrict__ p, int64_t n, uint32_t* sink) {
    const int64_t nth = static_cast<int64_t>(gridDim.x) * blockDim.x;
    uint32_t acc = 0;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; base < n; base += 4 * nth) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t i = base + u * nth;
            v[u] = i < n ? __builtin_nontemporal_load(p + i) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

// launches reads of bufs[i % nbufs] for i = 0 .. launches - 1 back to back on
// the stream, each over `bytes` bytes (a positive multiple of 16) with
// `blocks` workgroups of 256 threads; sink: one device uint32.  Returns 0, or
// 1 for bad arguments, 2 for a launch error.
extern "C" __attribute__((visibility("default"))) int w4probe_stream_read(const void* const* bufs, int nbufs, int64_t bytes,
                                                                          int launches, int blocks, uint32_t* sink,
                                                                          hipStream_t stream) {
    if (!bufs || nbufs <= 0 || bytes <= 0 || bytes % 16 != 0 || launches < 0 || blocks <= 0 || !sink) return 1;
    for (int i = 0; i < nbufs; ++i)
        if (!bufs[i]) return 1;
    for (int i = 0; i < launches; ++i)
        hipLaunchKernelGGL(stream_read_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                           static_cast<const u32x4*>(bufs[i % nbufs]), bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
