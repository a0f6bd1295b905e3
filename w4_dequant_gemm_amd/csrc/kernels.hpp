// Host-side launch interface of the gfx950 kernels (used by api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4 {

constexpr int kMaxFracs = 32;
// largest K of a per-channel weight (one group of G = K per row)
constexpr int64_t kMaxPerChannelK = 32768;

struct QuantizeParams {
    const float* W;          // [n_groups * G] fp32: groups are consecutive runs of G weights
    int64_t n_groups;
    int G;                   // 32, 64, 128, or K of the rows (per-channel)
    int asym;                // 0 symmetric, 1 asymmetric
    int n_fracs;
    float fracs[kMaxFracs];
    bool encode;             // false: search only (clip index and errors)
    uint8_t* packed;         // [n_groups * G / 2] canonical nibbles (encode)
    uint16_t* scale;         // [n_groups] fp16 (encode)
    uint16_t* zero;          // [n_groups] fp16 (encode, asym)
    uint8_t* clip;           // [n_groups] or null
    float* sse;              // [n_groups * n_fracs] or null
};
hipError_t launch_quantize(const QuantizeParams& p, hipStream_t stream);

struct PrepackParams {
    const uint8_t* packed;   // [N, K/2]
    const uint16_t* scale;   // [N, K/G]
    const uint16_t* zero;    // [N, K/G] or null (sym)
    int64_t N, K;
    int G;
    int asym;
    uint32_t* wq;            // [N, K/8]
    uint32_t* sz;            // [N, K/G]
};
hipError_t launch_prepack(const PrepackParams& p, hipStream_t stream);

struct RowQuantParams {
    const uint16_t* X;       // [M, K] bf16
    int64_t M, K;
    uint8_t* xq;             // [M, K] e4m3
    float* xscale;           // [M]
    uint16_t* xw = nullptr;  // [M, K] the same codes widened exactly to bf16, or null
    // the rows' maxima of |x| already known as partial maxima [M][amax_tiles]
    // (written by the product that produced X), or null: scan X for them
    const float* amax_part = nullptr;
    int64_t amax_tiles = 0;
};
hipError_t launch_rowquant(const RowQuantParams& p, hipStream_t stream);

struct MulParams {
    const void* X;           // [M, K]: bf16 bits (W4A16) or e4m3 bytes (W4A8)
    const float* xscale;     // [M] row scales (W4A8) or null
    int64_t M, K, N;
    int G;
    const uint32_t* wq;      // [N, K/8] GPU-layout codes
    const uint32_t* sz;      // [N, K/G] fp16 scale | fp16 zero << 16
    uint16_t* Y;             // [M, N] bf16
    bool x_fp8;
    // W4A8 with the row quantization done inside the product (see
    // skinny_quantizes_rows): X is then the bf16 input, and the kernel also
    // writes the E4M3 codes and row scales here
    uint8_t* xq_out = nullptr;
    float* xscale_out = nullptr;
    // W4A8 above 128 rows: the E4M3 activations widened exactly to bf16 (the
    // row quantizer writes them into the caller's workspace when it is large
    // enough); the tiled product then runs the bf16 kernel on them and scales
    // rows in its epilogue or split sum.  Null: the E4M3 kernel.
    const uint16_t* xw = nullptr;
    // K split across workgroups.  Streaming kernel (splits > 1, M >= 3): K
    // ranges of whole steps, partial sums in ws [range][M][N].  The 64 x 128
    // and 256 x 256 GEMMs: output
    // tiles split_t0 .. tiles - 1 (numbered as tile_rc places them) are each
    // computed by `splits` workgroups over consecutive K ranges, which write
    // fp32 partial tiles to ws [tile - split_t0][split][tile rows x columns];
    // a second kernel adds them in split order, applies the row scale and
    // rounds to bf16.  Tiles before split_t0 are computed whole.
    int splits = 1;
    int64_t split_t0 = 0;
    float* ws = nullptr;
    // gate and up projections in one pass (streaming kernel, two column
    // blocks): block 0 reads wq/sz (gate), block 1 wq2/sz2 (up) at the same 16
    // output columns, and Y = bf16(act(gate) * up); act 1 = SiLU, 2 = GELU
    // (tanh form)
    const uint32_t* wq2 = nullptr;
    const uint32_t* sz2 = nullptr;
    int act = 0;
    // gate and up (W4A8): each workgroup also writes the maximum of |H| over
    // its columns of every row to amax_part [M][amax_tiles] (tile = its
    // column tile), for the row quantization of H that follows
    float* amax_part = nullptr;
    int64_t amax_tiles = 0;
};
// largest M of the streaming kernel's gate and up pass; above it the tiled
// pair GEMM (K a multiple of 64) takes the fused product
constexpr int64_t kGateUpMaxM = 32;
// column tiles of the W4A8 gate and up pass (the partial row maxima of H it
// writes per row): 16 columns in the streaming kernel, 128 in the tiled ones
int64_t gate_up_amax_tiles(int64_t M, int64_t N);
// Which kernel runs a product: M <= kSkinnyMaxM: the weight-streaming
// kernels (dot form for one or two rows, MFMA form above); larger M: the
// tiled MFMA GEMM (64 x 128 tiles up to 128 rows, 256 x 256 above; 128 x 128
// tiles when K is not a multiple of 64).
#ifndef W4_SKINNY_MAX
#define W4_SKINNY_MAX 64
#endif
constexpr int64_t kSkinnyMaxM = W4_SKINNY_MAX;
// W4A16 from this many rows up to kSkinnyMaxM: the tiled kernel's 64 x 128
// tiles (activations read once per 128 columns, against once per 32 in the
// streaming kernel's four row blocks) when K is a multiple of 64 and the
// caller's workspace holds their K split; otherwise the streaming kernel
#ifndef W4_TILED_FROM_M
#define W4_TILED_FROM_M 33
#endif
constexpr int64_t kTiledFromM = W4_TILED_FROM_M;
// the 64 x 128-tile kernel serves this shape (M up to 128, K a multiple of 64)
bool use_mid(int64_t M, int64_t K);
hipError_t launch_skinny(const MulParams& p, hipStream_t stream);
// K ranges of the streaming kernel's split for this shape and activation
// width in bytes (1: no split), and the fp32 partial sums it needs (sized for
// bf16): an optional workspace (without one the product runs unsplit)
int skinny_splits(int64_t M, int64_t K, int64_t N, int xbytes);
size_t skinny_workspace_bytes(int64_t M, int64_t K, int64_t N);
// true when a W4A8 product of M rows quantizes its activation rows itself
// (one or two rows whose bf16 activations fit the kernel's LDS staging)
bool skinny_quantizes_rows(int64_t M, int64_t K);
hipError_t launch_gemm(const MulParams& p, hipStream_t stream);
// gate and up in one tiled GEMM (p.wq2 / p.sz2 / p.act set; K a multiple of 64)
hipError_t launch_gemm_pair(const MulParams& p, hipStream_t stream);
// K-split schedule of the tiled GEMM for an [M, K] x [N, K] product
// (splits = 1: none) and the fp32 workspace bytes it needs
struct GemmSplit {
    int splits;
    int64_t t0;        // first split tile
    int64_t tiles;     // all output tiles
    int bm, bn;        // output tile of the kernel the schedule is for
};
GemmSplit gemm_split(int64_t M, int64_t K, int64_t N);
size_t gemm_workspace_bytes(int64_t M, int64_t K, int64_t N);
// K split of the W4A16 gate and up pair kernel (above 256 rows): its last
// partial round of 256 x 128 output tiles, and the fp32 workspace it needs
// (partial tiles of 256 x 256: the gate and up sums side by side)
GemmSplit pair_split(int64_t M, int64_t K, int64_t N);
size_t pair_workspace_bytes(int64_t M, int64_t K, int64_t N);
// W4A8 tiled product above 128 rows with at least 256 output tiles: byte
// offset (after the split partials, 256-byte aligned) and size of the
// widened activations in the workspace; gemm_xw_bytes is 0 where the product
// takes none
size_t gemm_xw_offset(int64_t M, int64_t K, int64_t N);
size_t gemm_xw_bytes(int64_t M, int64_t K, int64_t N);
// true when a W4A8 product of this shape and group size runs on the fp8
// matrix cores (M above kF8MinM, K and G multiples of 128); it takes the
// E4M3 activations as they are, never the widened copy.  Up to kF8MinM rows
// the weight-streaming kernel is faster.
#ifndef W4_F8_MINM
#define W4_F8_MINM 32
#endif
constexpr int64_t kF8MinM = W4_F8_MINM;
bool f8_eligible(int64_t M, int64_t K, int G);
// W4A16 with groups of 128 (K a multiple of 128) up to 128 rows: the fp8
// kernel's structure on bf16 activations, 64 x 128 tiles with the mid-size
// K split (gemm_split)
bool a16_eligible(int64_t M, int64_t K, int64_t N, int G);
hipError_t launch_gemm_a16(const MulParams& p, hipStream_t stream);
// true when the tiled W4A16 product of this shape runs that form, and its K
// split (gemm_split's rounded down: it fits the workspace gemm_split sizes)
bool a16_runs(int64_t M, int64_t K, int64_t N, int G, bool x_fp8);
// the W4A16 gate and up pair on that form (33 to 256 rows, groups of 128)
bool a16_pair_eligible(int64_t M, int64_t K, int64_t N, int G);
hipError_t launch_gemm_a16_pair(const MulParams& p, hipStream_t stream);
GemmSplit a16_split(int64_t M, int64_t K, int64_t N);
int a16_tile_rows(int64_t M);   // 64, or 128 from the rows it is set for
// K step of the fp8 kernel (one group of 128 k)
constexpr int kF8StepK = 128;
// the fp8 kernel addresses its operands with 31-bit byte offsets
bool f8_fits_buffers(int64_t M, int64_t K, int64_t N);
// output tile (bm x bn) and K split of the fp8 kernel for this shape, and the
// fp32 workspace bytes of its split partials
GemmSplit f8_split(int64_t M, int64_t K, int64_t N);
size_t f8_workspace_bytes(int64_t M, int64_t K, int64_t N);
// the fp8 W4A8 tiled kernel on the schedule of f8_split (p.splits and
// p.split_t0 from it, or splits = 1), then its split sum
hipError_t launch_gemm_f8(const MulParams& p, hipStream_t stream);
// gate and up (p.wq2 / p.sz2 / p.act set) on the fp8 kernel: W4A8 with
// groups of 128 (or whole rows), K a multiple of 128; no K split
hipError_t launch_gemm_f8_pair(const MulParams& p, hipStream_t stream);
// the sum of K-split partial tiles (bm x bn of p.ws, p.splits per tile, from
// tile p.split_t0 of `tiles` on), row scales applied for W4A8, into p.Y;
// bm x bn one of 256 x 256, 128 x 256, 64 x 256, 64 x 128, 256 x 128, 256 x 64
hipError_t launch_split_sum(const MulParams& p, int bm, int bn, int64_t tiles, hipStream_t stream);

// Library-held scratch of w4a16_gemm_noalloc: 64 MiB per GPU, the largest
// K-split workspace any shape of the tiled GEMM takes (at most 256 partial
// tiles of 256 x 256 fp32).  noalloc_scratch returns this GPU's address of it
// (looked up once per device).
constexpr size_t kNoAllocScratchBytes = size_t{64} << 20;
hipError_t noalloc_scratch(void** out);

// NF4 comparator (normal-quantile levels, blocks of 64, double-quantized scales)
constexpr int64_t kNf4MaxK = 32768;             // one 32-k chunk per lane of a 1024-lane workgroup
struct Nf4QuantParams {
    const float* W;          // [n_blocks * 64] fp32
    int64_t n_blocks;
    float levels[16];
    uint8_t* packed;         // [n_blocks * 32] codes, k even in the low nibble
    uint8_t* absmax_q;       // [n_blocks] 8-bit block scales
    float* c2;               // [ceil(n_blocks / 256)] second-level constants
};
hipError_t launch_nf4_quantize(const Nf4QuantParams& p, hipStream_t stream);
struct Nf4GemvParams {
    const uint16_t* x;       // [K] bf16
    int64_t K, N;
    const uint8_t* packed;   // [N, K/2]
    const uint8_t* absmax_q; // [N * K / 64]
    const float* c2;
    uint16_t* y;             // [N] bf16
    float levels[16];
};
hipError_t launch_nf4_gemv(const Nf4GemvParams& p, hipStream_t stream);

}  // namespace w4
