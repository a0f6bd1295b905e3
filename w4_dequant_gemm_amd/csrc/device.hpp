// Device-side helpers shared by the gfx950 kernels of the W4 library.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4 {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef int int8x_t __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// fp16 bits <-> float
__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
    return __half2float(__ushort_as_half(static_cast<unsigned short>(h & 0xFFFFu)));
}
__device__ __forceinline__ uint32_t float_to_half_bits(float f) {
    return __half_as_ushort(__float2half_rn(f));
}

// bf16 halves of a 32-bit word -> float (exact)
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    float2_t v = {lo, hi};
    bf16x2_t r = __builtin_convertvector(v, bf16x2_t);
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
    return static_cast<uint16_t>(pack_bf16x2(f, 0.0f) & 0xFFFFu);
}

// x / s for the E4M3 row quantization, without a division: with r = fl(1/s),
// the product q1 = fl(x r) corrected once by its exact residual,
// fl(q1 + fl(x - q1 s) r), with the sign of x (so that -0 stays -0).  For
// every bf16 x and every row scale s = max(fl(a / 448), 1e-8) of a bf16
// a >= |x|, clamping this to +-448 and rounding it to E4M3 (nearest even)
// gives the same code as the correctly rounded fl(x / s) does; that was
// checked on the host over all such pairs (tests/row_quotient_check.c).
__device__ __forceinline__ float e4m3_quotient(float x, float s, float r) {
#pragma clang fp contract(off)
    const float q1 = x * r;
    const float e = __builtin_fmaf(-q1, s, x);
    return __builtin_copysignf(__builtin_fmaf(e, r, q1), x);
}

// sum_i a.bf16[i] * b.bf16[i] + c  (v_dot2_f32_bf16)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// 16-byte load marked non-temporal: streamed weights are read exactly once, so
// they should not displace reused data (activations, scales) in the caches.
__device__ __forceinline__ uint4 load_nt_16(const uint32_t* p) {
    const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(t[0], t[1], t[2], t[3]);
}

// A value the optimizer cannot see through, held in a VGPR.  Used for the
// bf16 bias constant below: with it in a register, (x & mask) | bias becomes
// one v_and_or_b32 (gfx9 VOP3 encodings take no literal, so two literal
// operands would split it into an AND and an OR).
__device__ __forceinline__ uint32_t opaque_vgpr(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}

constexpr uint32_t kBf16Bias128x2 = 0x43004300u;   // two bf16 128.0

// Nibble pair i (0..3) of a GPU-layout code word as two bf16 values 128 + u:
// the nibbles at bits 4i and 16 + 4i land in the low mantissa bits of the
// bf16 constant 128.0 (0x4300), whose unit in the last place is exactly 1.
// `bias` is kBf16Bias128x2, passed in a register (see opaque_vgpr).
__device__ __forceinline__ uint32_t nibble_pair_bf16(uint32_t w, int i, uint32_t bias) {
    return ((w >> (4 * i)) & 0x000F000Fu) | bias;
}

// Row n of a weight in the blocked GPU layout (16-row blocks of 32-k tiles,
// as written by the prepack kernel): code word j of the row is
// words[(j / 4) * tile + j % 4] and its scale/zero word of group g is
// sz[g * nr], where nr is the number of rows in the row's block.
// Shift that maps a k index to its group: log2 G for the power-of-two group
// sizes; a group that is not a power of two is a whole row (per-channel,
// G = K), whose only group is 0 = k >> 31 for every k < K < 2^31.
__device__ __forceinline__ int group_shift(int G) {
    return (G & (G - 1)) == 0 ? __builtin_ctz(static_cast<unsigned>(G)) : 31;
}

struct TiledRow {
    const uint32_t* words;
    const uint32_t* sz;
    int64_t nr;
    int64_t tile;            // words between consecutive tiles of the row (4 nr)
    __device__ __forceinline__ const uint32_t* tile_ptr(int64_t t) const { return words + t * tile; }
    __device__ __forceinline__ uint32_t group(int64_t g) const { return sz[g * nr]; }
};
__device__ __forceinline__ TiledRow tiled_row(const uint32_t* wq, const uint32_t* sz, int64_t n, int64_t N,
                                              int64_t K, int G) {
    const int64_t r0 = n & ~static_cast<int64_t>(15);
    const int64_t nr = N - r0 < 16 ? N - r0 : 16;
    TiledRow r;
    r.words = wq + r0 * (K / 8) + 4 * (n - r0);
    r.sz = sz + r0 * (K / G) + (n - r0);
    r.nr = nr;
    r.tile = 4 * nr;
    return r;
}

// XCD-aware order of whole output tiles.  Workgroups are handed to the 8
// XCDs (each with its own L2) round-robin by workgroup index, so workgroup b
// runs on XCD b % 8.  Of T tiles, the first T8 = 8 floor(T / 8) are dealt as
// tile = (b % 8) (T8 / 8) + b / 8, which gives each XCD one contiguous range
// of tile numbers (tile_rc below places them on the grid); the last T - T8
// keep their index.  A bijection on 0 .. T - 1.
#ifndef W4_XCD_RASTER
#define W4_XCD_RASTER 1
#endif
__device__ __forceinline__ int64_t xcd_tile(int64_t b, int64_t T) {
    const int64_t T8 = T & ~int64_t{7};
    if (!W4_XCD_RASTER || b >= T8) return b;
    return (b & 7) * (T8 >> 3) + (b >> 3);
}

// Position of output tile t in an mt x nt tile grid.  Tiles are numbered
// super-row by super-row (kTileGroup row tiles each), column by column inside
// a super-row: a run of consecutive tiles (one XCD's range above, or the
// tiles in flight on it at one time) covers a few row tiles by many column
// tiles, so its workgroups share activation row panels and weight column
// panels in L2 instead of each reading a weight panel of its own.  A
// bijection from 0 .. mt nt - 1 onto the grid.
#ifndef W4_TILE_GROUP
#define W4_TILE_GROUP 4
#endif
constexpr int64_t kTileGroup = W4_TILE_GROUP;
__device__ __forceinline__ void tile_rc(int64_t t, int64_t mt, int64_t nt, int64_t& r, int64_t& c) {
    const int64_t g = t / (kTileGroup * nt);
    const int64_t j = t - g * (kTileGroup * nt);
    const int64_t rows = mt - g * kTileGroup < kTileGroup ? mt - g * kTileGroup : kTileGroup;
    c = j / rows;
    r = g * kTileGroup + (j - c * rows);
}

// Activation of the gate projection in a gated MLP: SiLU x / (1 + e^-x)
// (SwiGLU) or the tanh form of GELU, 0.5 x (1 + tanh(sqrt(2/pi) (x +
// 0.044715 x^3))) (GeGLU), in fp32.
__device__ __forceinline__ float activation(int act, float x) {
    if (act == 1) return x / (1.0f + expf(-x));
    const float t = 0.7978845608028654f * (x + 0.044715f * x * x * x);
    return 0.5f * x * (1.0f + tanhf(t));
}

// Butterfly sum over the 64 lanes of a wavefront; every lane gets the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// Maximum over each aligned group of 16 lanes; every lane gets its group's.
__device__ __forceinline__ float max16(float v) {
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 16));
    return v;
}

// Maximum over each half (32 lanes) of the wavefront.
__device__ __forceinline__ float max32(float v) {
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 32));
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

}  // namespace w4
