// W4A16 / W4A8 decode GEMV for M <= 16 rows of activations, gfx950.
//
// At batch 1 decoding reads every weight once and that read sets the pace
// (gsantana.dev "Quantizing LLMs Without Guesswork", "The Problem & Context";
// W4A16 dequantizes inside the matmul and computes in 16-bit, section
// "Weight-only methods").  So this kernel streams the packed codes from HBM
// exactly once and keeps the arithmetic per weight to about one VALU op:
//
//   * a code word holds pairs (u[2i], u[2i+1]) in the low nibbles of its two
//     halves (GPU layout, see prepack.hip); one AND-OR with 0x43004300 turns a
//     pair into two exact bf16 values 128 + u;
//   * v_dot2_f32_bf16 multiplies that pair with the matching bf16 activation
//     pair and accumulates in fp32;
//   * the scale and zero point are applied once per lane and group:
//       sum_k (u - z) s x = s * (sum_k (128 + u) x - (128 + z) * sum_k x),
//     where sum_k x over the lane's k range is computed once and reused for
//     every row.
//
// Work split (M <= 4): K is cut into chunks of 2048 (32 k = 16 code bytes per
// lane).  A workgroup holds CW "chunk waves" x RG row groups; chunk wave c of a
// row group owns chunks c, c + CW, ... of RPW rows, spaced one grid-width of
// rows apart.  A wave issues the loads of all its rows for one chunk before
// the first use and keeps the next chunk's loads in flight while it
// multiplies the current one; the scale/zero words of a chunk come in one
// load per lane and reach their lanes by shuffles.  Per-row partial sums are
// reduced across the wave with a reduce-scatter butterfly and across chunk
// waves through LDS.
//
// M = 5..16: one wave per R rows, lanes stride over 512-wide chunks (8 k per
// lane), reduce-scatter at the end (VALU bound: every weight meets M
// activations).
//
// W4A8 reads E4M3 activations, widens them exactly to bf16 and applies the row
// scale at the end (gowda.ai "LLM fast inference", "Achievement 2": FP32
// accumulation, row scale in the epilogue, BF16 output).
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

constexpr int pow2_ceil(int v) { return v <= 1 ? 1 : 2 * pow2_ceil((v + 1) / 2); }

// Activation fragment of one lane: KL consecutive k of MT rows, as bf16 pairs,
// plus the per-row sum of those KL values.
template <int MT, int KL, bool XF8>
__device__ __forceinline__ void load_x(const MulParams& p, int M, int64_t k0, bool active,
                                       uint32_t (&xw)[MT][KL / 2], float (&xs)[MT]) {
    constexpr int XW = KL / 2;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const bool ok = active && m < M;
        if constexpr (!XF8) {
            const uint16_t* xr = static_cast<const uint16_t*>(p.X) + static_cast<int64_t>(m) * p.K + k0;
#pragma unroll
            for (int j = 0; j < XW; j += 4) {
                uint4 t = ok ? *reinterpret_cast<const uint4*>(xr + 2 * j) : make_uint4(0, 0, 0, 0);
                xw[m][j] = t.x; xw[m][j + 1] = t.y; xw[m][j + 2] = t.z; xw[m][j + 3] = t.w;
            }
        } else {
            // E4M3 -> fp32 (exact) -> bf16 pair (exact: 3 mantissa bits fit)
            const uint8_t* xr = static_cast<const uint8_t*>(p.X) + static_cast<int64_t>(m) * p.K + k0;
#pragma unroll
            for (int j = 0; j < XW; j += 2) {
                const uint32_t b4 = ok ? *reinterpret_cast<const uint32_t*>(xr + 2 * j) : 0u;
                float2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(b4), false);
                float2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(b4), true);
                xw[m][j] = pack_bf16x2(lo[0], lo[1]);
                xw[m][j + 1] = pack_bf16x2(hi[0], hi[1]);
            }
        }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        float s = 0.0f;
#pragma unroll
        for (int j = 0; j < XW; ++j) s += bf16_lo(xw[m][j]) + bf16_hi(xw[m][j]);
        xs[m] = s;
    }
}

// One lane's contribution of WW code words of one row to MT outputs.
template <int MT, int WW>
__device__ __forceinline__ void tile_dot(const uint32_t (&wv)[WW], uint32_t szw, const uint32_t (&xw)[MT][4 * WW],
                                         const float (&xs)[MT], float* acc, uint32_t bias) {
    const float sc = half_bits_to_float(szw);
    const float cz = 128.0f + half_bits_to_float(szw >> 16);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        float d = 0.0f;
#pragma unroll
        for (int ww = 0; ww < WW; ++ww)
#pragma unroll
            for (int i = 0; i < 4; ++i) d = dot2_bf16(nibble_pair_bf16(wv[ww], i, bias), xw[m][4 * ww + i], d);
        acc[m] = fmaf(sc, d - cz * xs[m], acc[m]);
    }
}

// ---------------------------------------------------------------- M <= 4

struct SplitShape {
    int cw;      // chunk waves per row group
    int rg;      // row groups per workgroup
    int rpw;     // rows per wave
};

template <int MT, int RPW, int G, bool XF8>
struct SplitChunk {
    static constexpr int KL = 32;                  // k per lane per chunk
    static constexpr int CHUNK = 64 * KL;          // 2048
    static constexpr int GPC = CHUNK / G;          // groups per row and chunk
    static constexpr int SZL = (RPW * GPC + 63) / 64;   // scale/zero loads per lane

    uint4 wv[RPW];
    uint32_t szl[SZL];
    uint32_t xw[MT][KL / 2];
    float xs[MT];

    // Issue the loads of chunk kc for the RPW rows n = r * row_stride + row_base:
    // one 16-byte code load per row and lane (non-temporal: read once), and the
    // chunk's scale/zero words for all rows, one word per lane and load (word
    // j = lane + 64 t is row j / GPC, group j % GPC of the chunk).
    __device__ __forceinline__ void load(const MulParams& p, int64_t kc, int lane, int64_t row_stride,
                                         int64_t row_base, int M) {
        const int64_t K = p.K, N = p.N;
        const int64_t words_row = K / 8, groups_row = K / G;
        const int64_t k0 = kc + static_cast<int64_t>(lane) * KL;
        const int64_t kk = k0 < K ? k0 : 0;        // lanes past K load valid words; their x is 0
        const int64_t g0 = kc / G;
        // activations first: with in-order load completion, the first row's
        // product then waits only for its own code load
        load_x<MT, KL, XF8>(p, M, k0, k0 < K, xw, xs);
#pragma unroll
        for (int t = 0; t < SZL; ++t) {
            const int j = lane + 64 * t;
            const int r = j / GPC;
            int64_t n = static_cast<int64_t>(r < RPW ? r : RPW - 1) * row_stride + row_base;
            n = n < N ? n : N - 1;
            int64_t g = g0 + j % GPC;
            g = g < groups_row ? g : groups_row - 1;
            szl[t] = p.sz[n * groups_row + g];
        }
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            int64_t n = r * row_stride + row_base;
            n = n < N ? n : N - 1;                 // rows past N are computed and dropped
            wv[r] = load_nt_16(p.wq + n * words_row + kk / 8);
        }
    }

    __device__ __forceinline__ void compute(int lane, float* acc, uint32_t bias) const {
        const int lane_group = lane / (G / KL);     // this lane's group within the chunk
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            const int j = r * GPC + lane_group;
            const uint32_t szw = __shfl(szl[(r * GPC) / 64], j % 64, kWave);
            const uint32_t w[4] = {wv[r].x, wv[r].y, wv[r].z, wv[r].w};
            tile_dot<MT, 4>(w, szw, xw, xs, &acc[r * MT], bias);
        }
    }
};

template <int MT, int RPW, int G, bool XF8, int DEPTH>
__global__ void __launch_bounds__(512) gemv_split_kernel(MulParams p, int cw, int rg) {
    using Chunk = SplitChunk<MT, RPW, G, XF8>;
    constexpr int V = pow2_ceil(RPW * MT);
    __shared__ float red[512 / 64][V];   // [wave][value] partial sums

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int cwi = wave % cw;             // chunk wave index
    const int rgi = wave / cw;             // row group in the workgroup
    const int64_t K = p.K, N = p.N;
    const int M = static_cast<int>(p.M);
    // Row r of this row group is n = r * row_stride + row_base: at every issue
    // step the whole grid reads one contiguous span of rows.
    const int64_t row_stride = static_cast<int64_t>(gridDim.x) * rg;
    const int64_t row_base = static_cast<int64_t>(blockIdx.x) * rg + rgi;
    const uint32_t bias = opaque_vgpr(kBf16Bias128x2);

    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.0f;

    // chunks cwi, cwi + cw, ... of every row; with DEPTH 2 the next chunk's
    // loads are in flight while the current one is multiplied
    const int64_t step = static_cast<int64_t>(cw) * Chunk::CHUNK;
    int64_t kc = static_cast<int64_t>(cwi) * Chunk::CHUNK;
    if constexpr (DEPTH == 1) {
        for (; kc < K; kc += step) {
            Chunk a;
            a.load(p, kc, lane, row_stride, row_base, M);
            __builtin_amdgcn_sched_barrier(0);
            a.compute(lane, acc, bias);
        }
    } else {
        Chunk a, b;
        a.load(p, kc, lane, row_stride, row_base, M);
        while (true) {
            const int64_t kn = kc + step;
            const bool more = kn < K;
            if (more) b.load(p, kn, lane, row_stride, row_base, M);
            __builtin_amdgcn_sched_barrier(0);
            a.compute(lane, acc, bias);
            if (!more) break;
            kc = kn;
            const int64_t kn2 = kc + step;
            const bool more2 = kn2 < K;
            if (more2) a.load(p, kn2, lane, row_stride, row_base, M);
            __builtin_amdgcn_sched_barrier(0);
            b.compute(lane, acc, bias);
            if (!more2) break;
            kc = kn2;
        }
    }

    int idx;
    const float v = wave_reduce_scatter<V>(acc, lane, idx);
    constexpr int lanes_per = 64 / V;
    if ((lane & (lanes_per - 1)) == 0) red[wave][idx] = v;
    __syncthreads();
    // one thread per (row, m) of the row group sums the chunk waves
    const int t = threadIdx.x;
    if (t < rg * RPW * MT) {
        const int g = t / (RPW * MT);
        const int rm = t % (RPW * MT);
        float y = 0.0f;
        for (int c = 0; c < cw; ++c) y += red[g * cw + c][rm];
        const int r = rm / MT, m = rm % MT;
        const int64_t n = r * (static_cast<int64_t>(gridDim.x) * rg) + static_cast<int64_t>(blockIdx.x) * rg + g;
        if (n < N && m < M) {
            if constexpr (XF8) y *= p.xscale[m];
            p.Y[static_cast<int64_t>(m) * N + n] = float_to_bf16_bits(y);
        }
    }
}

template <int MT, int RPW, int G, bool XF8>
hipError_t launch_split_t(const MulParams& p, const SplitShape& s, hipStream_t stream) {
    const int64_t rows_per_block = static_cast<int64_t>(s.rg) * RPW;
    const int64_t blocks = (p.N + rows_per_block - 1) / rows_per_block;
    hipLaunchKernelGGL((gemv_split_kernel<MT, RPW, G, XF8, 1>), dim3(static_cast<unsigned>(blocks)),
                       dim3(64 * s.cw * s.rg), 0, stream, p, s.cw, s.rg);
    return hipGetLastError();
}

template <int MT, int RPW, bool XF8>
hipError_t launch_split_g(const MulParams& p, const SplitShape& s, hipStream_t stream) {
    switch (p.G) {
        case 32: return launch_split_t<MT, RPW, 32, XF8>(p, s, stream);
        case 64: return launch_split_t<MT, RPW, 64, XF8>(p, s, stream);
        default: return launch_split_t<MT, RPW, 128, XF8>(p, s, stream);
    }
}

// Launch shape (swept on the 8B MLP shapes, up 14336 x 4096 and down
// 4096 x 14336): two chunk waves per row group, each walking every other
// 2048-wide chunk; two row groups per workgroup when a row has at most two
// chunks, one otherwise; four rows per wave while that keeps at least ~512
// workgroups, fewer for short matrices.  Pipelining the next chunk's loads
// measured slower than this single-buffered form.
template <int MT, bool XF8>
hipError_t launch_split(const MulParams& p, hipStream_t stream) {
    constexpr int64_t kChunk = 2048;
    const int64_t chunks = (p.K + kChunk - 1) / kChunk;
    SplitShape s;
    s.cw = chunks >= 2 ? 2 : 1;
    s.rg = chunks <= 2 ? 2 : 1;
    const int max_rpw = 16 / MT < 4 ? 16 / MT : 4;
    int rpw = max_rpw;
    while (rpw > 1 && (p.N + s.rg * rpw - 1) / (s.rg * rpw) < 512) rpw /= 2;
    s.rpw = rpw;
    switch (rpw) {
        case 1: return launch_split_g<MT, 1, XF8>(p, s, stream);
        case 2: return launch_split_g<MT, 2, XF8>(p, s, stream);
        case 4: return launch_split_g<MT, 4, XF8>(p, s, stream);
        default: break;
    }
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- M <= 16

template <int MT, int KL, int R, bool XF8>
__global__ void __launch_bounds__(256) gemv_rows_kernel(MulParams p) {
    constexpr int WW = KL / 8;   // code words per lane and weight row
    const int lane = threadIdx.x & 63;
    const int64_t wave = static_cast<int64_t>(blockIdx.x) * (blockDim.x / 64) +
                         __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t n0 = wave * R;
    if (n0 >= p.N) return;
    const uint32_t bias = opaque_vgpr(kBf16Bias128x2);
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

        uint32_t xw[MT][KL / 2];
        float xs[MT];
        load_x<MT, KL, XF8>(p, M, k0, active, xw, xs);
#pragma unroll
        for (int r = 0; r < R; ++r) tile_dot<MT, WW>(wv[r], szv[r], xw, xs, &acc[r * MT], bias);
    }

    constexpr int V = R * MT;
    int idx;
    const float v = wave_reduce_scatter<V>(acc, lane, idx);
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

template <int MT, int KL, int R, bool XF8>
hipError_t launch_rows_t(const MulParams& p, hipStream_t stream) {
    const int waves_per_block = 4;
    const int64_t waves = (p.N + R - 1) / R;
    const int64_t blocks = (waves + waves_per_block - 1) / waves_per_block;
    hipLaunchKernelGGL((gemv_rows_kernel<MT, KL, R, XF8>), dim3(static_cast<unsigned>(blocks)),
                       dim3(64 * waves_per_block), 0, stream, p);
    return hipGetLastError();
}

template <int MT, bool XF8>
hipError_t launch_rows(const MulParams& p, hipStream_t stream) {
    if (p.N >= 8192) return launch_rows_t<MT, 8, 4, XF8>(p, stream);
    if (p.N >= 2048) return launch_rows_t<MT, 8, 2, XF8>(p, stream);
    return launch_rows_t<MT, 8, 1, XF8>(p, stream);
}

template <bool XF8>
hipError_t launch_m(const MulParams& p, hipStream_t stream) {
    if (p.M <= 1) return launch_split<1, XF8>(p, stream);
    if (p.M <= 2) return launch_split<2, XF8>(p, stream);
    if (p.M <= 4) return launch_split<4, XF8>(p, stream);
    if (p.M <= 8) return launch_rows<8, XF8>(p, stream);
    return launch_rows<16, XF8>(p, stream);
}

}  // namespace

hipError_t launch_gemv(const MulParams& p, hipStream_t stream) {
    if (p.M == 0 || p.N == 0) return hipSuccess;
    if (p.M > kGemvMaxM) return hipErrorInvalidValue;
    return p.x_fp8 ? launch_m<true>(p, stream) : launch_m<false>(p, stream);
}

}  // namespace w4
