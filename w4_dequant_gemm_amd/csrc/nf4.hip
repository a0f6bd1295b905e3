// NF4 comparator: the normal-quantile 4-bit format and its decode GEMV.
//
// gsantana.dev "Quantizing LLMs Without Guesswork", "Weight-only methods: GPTQ,
// AWQ and the file formats" (the NF4 paragraph): 16 levels that are quantiles
// of a normal distribution (QLoRA's construction), blocks of 64 weights with
// an absmax scale, and double quantization of those scales (8-bit codes and
// one fp32 constant per 256 scales: 0.127 bits per weight).  It is the pages'
// throughput comparison point, so the product here is the same decode GEMV
// as the W4A16 one, run on the same hardware.
//
// Quantizer: one workgroup of 256 threads per group of 256 consecutive blocks
// (flattened row-major), one thread per block of 64 weights: absmax, then the
// group maximum for the second level (c2 = max / 255, codes rne(absmax / c2)),
// then every weight's nearest level to fp32(w / absmax) (fp32 distances, the
// lower index on ties).  Plain fp32 operations in a fixed order (built without
// contraction), so the result is bit-reproducible.
//
// GEMV: the levels enter as bf16 (one rounding, as for the W4A16 weights).  A
// 256-entry table in LDS turns a byte of two codes (k even in the low nibble)
// into a bf16 pair for v_dot2_f32_bf16 against the activation pair; the table
// is replicated once per lane (entry e of lane l at word 64 e + l), so the
// data-dependent reads of a wave never share a bank, and v_perm_b32 forms the
// byte address (code byte above the lane's offset) in one instruction.  The
// activation row is staged in LDS once per workgroup as [4][K/32][4] words,
// so lanes reading consecutive 32-k chunks read consecutive 16-byte pieces.
// A wave owns whole rows (a contiguous run of them, the same count for every
// wave) and works on R of them at once: lane l takes the chunks l, l + 64, ...
// PU at a time (an item), reads each activation chunk from LDS once for the R
// rows, and keeps D items in flight, so at the decode shapes every code byte
// of the launch is requested before the first product is formed and the
// products follow the data as it arrives.  A butterfly sum ends each row; the
// loop has no barrier.
#include "device.hpp"
#include "kernels.hpp"

#pragma clang fp contract(off)

namespace w4 {
namespace {

constexpr int kNf4Block = 64;
constexpr int kNf4Group = 256;

__global__ void __launch_bounds__(kNf4Group) nf4_quantize_kernel(Nf4QuantParams p) {
    __shared__ float wmax[kNf4Group / 64];
    const int t = threadIdx.x;
    const int64_t blk = static_cast<int64_t>(blockIdx.x) * kNf4Group + t;
    const bool live = blk < p.n_blocks;
    float v[kNf4Block];
    float amax = 0.0f;
    if (live) {
        const float4* src = reinterpret_cast<const float4*>(p.W + blk * kNf4Block);
#pragma unroll
        for (int i = 0; i < kNf4Block / 4; ++i) {
            const float4 f = src[i];
            v[4 * i] = f.x;
            v[4 * i + 1] = f.y;
            v[4 * i + 2] = f.z;
            v[4 * i + 3] = f.w;
        }
#pragma unroll
        for (int i = 0; i < kNf4Block; ++i) amax = fmaxf(amax, fabsf(v[i]));
    }
    // the group's largest block absmax
    float g = wave_max(amax);
    if ((t & 63) == 0) wmax[t >> 6] = g;
    __syncthreads();
    g = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    float c2 = g / 255.0f;
    if (c2 == 0.0f) c2 = 1.0f;
    if (t == 0) p.c2[blockIdx.x] = c2;
    if (!live) return;
    p.absmax_q[blk] = static_cast<uint8_t>(fminf(fmaxf(rintf(amax / c2), 0.0f), 255.0f));

    const float a = amax == 0.0f ? 1.0f : amax;
    uint32_t words[kNf4Block / 8];
#pragma unroll
    for (int w = 0; w < kNf4Block / 8; ++w) {
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float x = v[8 * w + i] / a;
            int best = 0;
            float bd = fabsf(x - p.levels[0]);
#pragma unroll
            for (int l = 1; l < 16; ++l) {
                const float d = fabsf(x - p.levels[l]);
                if (d < bd) {
                    bd = d;
                    best = l;
                }
            }
            word |= static_cast<uint32_t>(best) << (4 * i);   // k even: low nibble of its byte
        }
        words[w] = word;
    }
    uint4* dst = reinterpret_cast<uint4*>(p.packed + blk * (kNf4Block / 2));
    dst[0] = make_uint4(words[0], words[1], words[2], words[3]);
    dst[1] = make_uint4(words[4], words[5], words[6], words[7]);
}

constexpr int kGemvThreads = 1024;
constexpr int kGemvWaves = kGemvThreads / 64;
constexpr int kLutWords = 256 * 64;

// One item: PU chunks (32 k each) of R rows for every lane of a wave.
template <int R, int PU>
struct Nf4Item {
    uint4 q[R][PU];      // 32 codes per chunk
    uint32_t a[R][PU];   // the chunk's 8-bit block scale
    float c2[R][PU];     // its second-level constant
};

template <int R, int PU, int D>
__global__ void __launch_bounds__(kGemvThreads) nf4_gemv_kernel(Nf4GemvParams p, int64_t rows_per_wave,
                                                                int items_per_group) {
    __shared__ uint32_t lds[kLutWords + kNf4MaxK / 2];   // table [256][64], activations [4][K/32][4]
    uint32_t* xs = lds + kLutWords;
    const int t = threadIdx.x, lane = t & 63;
    const int64_t K = p.K;
    const int nch = static_cast<int>(K / 32);
    const int64_t nb = K / kNf4Block;
    const int64_t wave_id = static_cast<int64_t>(blockIdx.x) * kGemvWaves + (t >> 6);
    const int64_t row0 = wave_id * rows_per_wave;
    const int64_t row_end = row0 + rows_per_wave < p.N ? row0 + rows_per_wave : p.N;
    const int64_t n_items = row_end > row0 ? (row_end - row0 + R - 1) / R * items_per_group : 0;

    // item loads: lane chunks piece * 64 PU + 64 u + lane of rows row .. row + R - 1;
    // past the row or past the wave's rows, zeros and no memory access
    auto load = [&](int64_t row, int piece, Nf4Item<R, PU>& it) {
#pragma unroll
        for (int i = 0; i < R; ++i) {
#pragma unroll
            for (int u = 0; u < PU; ++u) {
                const int c = piece * 64 * PU + 64 * u + lane;
                if (row + i < row_end && c < nch) {
                    const int64_t bi = (row + i) * nb + (c >> 1);
                    it.q[i][u] = load_nt_16(reinterpret_cast<const uint32_t*>(p.packed + (row + i) * (K / 2)) + 4 * c);
                    it.a[i][u] = p.absmax_q[bi];
                    it.c2[i][u] = p.c2[bi >> 8];
                } else {
                    it.q[i][u] = make_uint4(0u, 0u, 0u, 0u);
                    it.a[i][u] = 0u;
                    it.c2[i][u] = 0.0f;
                }
            }
        }
    };

    Nf4Item<R, PU> st[D];
    int64_t lrow = row0;
    int lpiece = 0;
#pragma unroll
    for (int d = 0; d < D; ++d) {
        load(lrow, lpiece, st[d]);
        if (++lpiece == items_per_group) {
            lpiece = 0;
            lrow += R;
        }
    }

    // activations: 16-byte piece i of the row holds pairs 4i .. 4i + 3, word i % 4 of chunk i / 4
    const uint4* x4 = reinterpret_cast<const uint4*>(p.x);
    for (int i = t; i < nch * 4; i += kGemvThreads)
        *reinterpret_cast<uint4*>(xs + (i & 3) * (4 * nch) + 4 * (i >> 2)) = x4[i];
    // table word t + 1024 k holds entry 16 k + wave: low code the wave's level, high code level k
    static_assert(kGemvThreads == 1024 && kLutWords == 16 * kGemvThreads, "table fill assumes 16 waves");
    const float lo = p.levels[__builtin_amdgcn_readfirstlane(t >> 6)];
#pragma unroll
    for (int k2 = 0; k2 < 16; ++k2) lds[t + kGemvThreads * k2] = pack_bf16x2(lo, p.levels[k2]);
    __syncthreads();

    const uint32_t lane4 = static_cast<uint32_t>(lane) * 4u;
    const char* lut = reinterpret_cast<const char*>(lds);
    int64_t crow = row0;
    int cpiece = 0;
    float acc[R];
#pragma unroll
    for (int i = 0; i < R; ++i) acc[i] = 0.0f;
    for (int64_t j = 0; j < n_items; j += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if (j + d < n_items) {
#pragma unroll
                for (int u = 0; u < PU; ++u) {
                    const int c = cpiece * 64 * PU + 64 * u + lane;
                    if (c < nch) {
                        float dd[R];
#pragma unroll
                        for (int i = 0; i < R; ++i) dd[i] = 0.0f;
#pragma unroll
                        for (int w = 0; w < 4; ++w) {
                            // one read of the activation pairs for all R rows
                            const uint4 xv = *reinterpret_cast<const uint4*>(xs + w * (4 * nch) + 4 * c);
                            const uint32_t xp[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                            for (int i = 0; i < R; ++i) {
                                const uint32_t qw = w == 0 ? st[d].q[i][u].x : w == 1 ? st[d].q[i][u].y
                                                  : w == 2 ? st[d].q[i][u].z : st[d].q[i][u].w;
#pragma unroll
                                for (int b = 0; b < 4; ++b) {
                                    // byte address 256 * (byte b of the word) + 4 * lane
                                    const uint32_t sel = 0x0C0C0000u | (static_cast<uint32_t>(4 + b) << 8);
                                    const uint32_t addr = __builtin_amdgcn_perm(qw, lane4, sel);
                                    dd[i] = dot2_bf16(*reinterpret_cast<const uint32_t*>(lut + addr), xp[b], dd[i]);
                                }
                            }
                        }
#pragma unroll
                        for (int i = 0; i < R; ++i)
                            acc[i] = fmaf(static_cast<float>(st[d].a[i][u]) * st[d].c2[i][u], dd[i], acc[i]);
                    }
                }
                if (++cpiece == items_per_group) {
#pragma unroll
                    for (int i = 0; i < R; ++i) {
                        const float v = wave_sum(acc[i]);
                        if (lane == 0 && crow + i < row_end) p.y[crow + i] = float_to_bf16_bits(v);
                        acc[i] = 0.0f;
                    }
                    cpiece = 0;
                    crow += R;
                }
                load(lrow, lpiece, st[d]);
                if (++lpiece == items_per_group) {
                    lpiece = 0;
                    lrow += R;
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_nf4_quantize(const Nf4QuantParams& p, hipStream_t stream) {
    if (p.n_blocks == 0) return hipSuccess;
    const int64_t groups = (p.n_blocks + kNf4Group - 1) / kNf4Group;
    hipLaunchKernelGGL(nf4_quantize_kernel, dim3(static_cast<unsigned>(groups)), dim3(kNf4Group), 0, stream, p);
    return hipGetLastError();
}

template <int R, int PU>
hipError_t launch_nf4_gemv_rp(const Nf4GemvParams& p, int64_t rows_per_wave, hipStream_t stream) {
    constexpr int D = 8 / (R * PU) > 0 ? 8 / (R * PU) : 1;     // eight chunks per lane in flight
    const int64_t nch = p.K / 32;
    const int items_per_group = static_cast<int>((nch + 64 * PU - 1) / (64 * PU));
    const int64_t waves = (p.N + rows_per_wave - 1) / rows_per_wave;
    const int64_t wgs = (waves + kGemvWaves - 1) / kGemvWaves;
    hipLaunchKernelGGL((nf4_gemv_kernel<R, PU, D>), dim3(static_cast<unsigned>(wgs)), dim3(kGemvThreads), 0, stream,
                       p, rows_per_wave, items_per_group);
    return hipGetLastError();
}

template <int R>
hipError_t launch_nf4_gemv_r(const Nf4GemvParams& p, int64_t rows_per_wave, hipStream_t stream) {
    const int64_t nch = p.K / 32;
    if (nch <= 64) return launch_nf4_gemv_rp<R, 1>(p, rows_per_wave, stream);
    if constexpr (R == 4) {
        return launch_nf4_gemv_rp<R, 2>(p, rows_per_wave, stream);
    } else {
        if (nch <= 128) return launch_nf4_gemv_rp<R, 2>(p, rows_per_wave, stream);
        return launch_nf4_gemv_rp<R, 4>(p, rows_per_wave, stream);
    }
}

hipError_t launch_nf4_gemv(const Nf4GemvParams& p, hipStream_t stream) {
    if (p.N == 0) return hipSuccess;
    if (p.K % kNf4Block != 0 || p.K > kNf4MaxK || p.K <= 0) return hipErrorInvalidValue;
    // rows per wave: the fewest that fit the rows on one resident workgroup per
    // compute unit; a wave takes up to four of them at a time (one read of each
    // activation chunk for all of them)
    const int64_t slots = int64_t{256} * kGemvWaves;
    const int64_t rows_per_wave = (p.N + slots - 1) / slots;
    if (rows_per_wave >= 4) return launch_nf4_gemv_r<4>(p, rows_per_wave, stream);
    if (rows_per_wave >= 2) return launch_nf4_gemv_r<2>(p, rows_per_wave, stream);
    return launch_nf4_gemv_r<1>(p, rows_per_wave, stream);
}

}  // namespace w4
