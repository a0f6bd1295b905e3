/*
 * w4.h -- C ABI of the MI355X (gfx950) library for blockwise 4-bit weight
 * quantization and the fused dequantize-and-multiply that consumes it.
 *
 * What the operations compute (the pages this follows):
 *  - gsantana.dev, "Quantizing LLMs Without Guesswork: What 4 Bits Really
 *    Cost": "Scale and zero point" (the symmetric and asymmetric formulas),
 *    "Granularity: who shares a scale" (a group is a run of G consecutive
 *    weights inside one output row), "Quantize, then dequantize" (half-to-even
 *    rounding, a zero scale replaced by 1), "Weight-only methods" (W4A16:
 *    dequantize inside the matmul, compute in 16-bit).
 *  - gowda.ai, "LLM fast inference" (Tahoma): "Achievement 1" (unsigned codes
 *    0..15, integer zero point, 16-bit scale and zero per group along K),
 *    "MSE clipping" (a data-free search over contracted ranges about the
 *    observed midpoint; a candidate replaces the plain quantizer only if its
 *    block error is strictly lower; clipped values count in the error; the
 *    portable packed form is rearranged into a GPU layout without requantizing),
 *    "Achievement 2" (each activation row quantized to FP8 E4M3 with a scale
 *    from its maximum over 448, floored at 1e-8; FP32 accumulation; the row
 *    scale applied in the epilogue; BF16 output).
 *
 * Conventions shared by every entry point:
 *  - Matrices are row-major and contiguous.  A weight W is [N, K]: row n is
 *    output channel n, K is the reduction (input) dimension.  Products are
 *    Y[M, N] = X[M, K] . W'^T.
 *  - Every pointer argument is a DEVICE pointer on the current HIP device,
 *    owned by the caller, except where a parameter says "host".  The library
 *    allocates no memory.  Its state is a thread-local message for the last
 *    failed call, the NF4 level table, and one fixed scratch array per GPU
 *    used only by w4a16_gemm_noalloc; the other products take their scratch
 *    memory from the caller (w4_gemm_workspace_bytes).
 *  - Device pointers must be 16-byte aligned.
 *  - Every call is asynchronous on `stream` (0 = the null stream).  Arguments
 *    are checked on the host before any launch: a violated precondition
 *    returns W4_EINVAL (or W4_EUNSUPPORTED for a valid but unsupported
 *    configuration) and launches nothing.  There is no fallback path: an
 *    unsupported shape is an error, never a slow or dense substitute.
 *    W4_EHIP reports a launch failure; faults during execution surface at the
 *    caller's next synchronization.
 *  - Weights must be finite with |w| <= 65504; activations must be finite.
 *  - fp16 values are passed as uint16_t bit patterns, bf16 as uint16_t bit
 *    patterns, FP8 E4M3 (OCP "fn" variant: max 448, no infinities) as bytes.
 */
#ifndef W4_H
#define W4_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
#define W4_OK 0
#define W4_EINVAL 1        /* a precondition on the arguments is violated */
#define W4_EUNSUPPORTED 2  /* well-formed, but not a configuration the library runs */
#define W4_EHIP 3          /* the HIP runtime reported an error at launch */

/* Quantizer modes. */
#define W4_SYM 0   /* codes -8..7, scale = f * amax / 7, no zero point */
#define W4_ASYM 1  /* codes 0..15, scale = (hi - lo) / 15, integer zero point */

/* Largest number of clip fractions one call accepts. */
#define W4_MAX_FRACS 32

/*
 * w4_quantize_blockwise -- quantize W[N, K] (fp32) in groups of G consecutive
 * weights along K, with an optional MSE clip search.
 * Follows gsantana.dev "Quantizing LLMs Without Guesswork", "Scale and zero
 * point" (both formulas) and "Granularity: who shares a scale"; gowda.ai "LLM
 * fast inference", "Achievement 1" (unsigned codes 0..15 with an integer zero
 * point, 16-bit scale and zero) and "MSE clipping" (the candidate search).
 *
 * For every group the candidate ranges are, for each fraction f in `fracs`:
 *   asym: f == 1 -> [min, max]; f < 1 -> [mid - f*h, mid + f*h] with
 *         mid = (max + min) * 0.5, h = (max - min) * 0.5;
 *   sym : [-f*amax, f*amax].
 * Each candidate's scale is rounded to fp16 (a zero scale becomes 1.0), the
 * asymmetric zero point is round_half_even(-lo / s) (an integer, not clamped),
 * codes are clamp(round_half_even(w / s) + z, 0, 15) or
 * clamp(round_half_even(w / s), -8, 7), and the candidate's error is the sum
 * over the group of (w - (q - z) * s)^2, added by a fixed pairwise halving
 * tree (a[j] += a[j + len], len = P/2 ... 1, over the errors padded with
 * zeros to the next power of two P).  The first candidate is kept unless a later one has a strictly lower
 * error.  All arithmetic is IEEE fp32 with round-to-nearest-even, so the
 * result is bit-for-bit reproducible.
 *
 *   W        [N, K] fp32, device.
 *   N, K     N >= 0, K > 0, K % G == 0.
 *   G        32, 64 or 128; or G == K: one group per row, the per-channel
 *            granularity (gsantana.dev "Granularity: who shares a scale"),
 *            for K a multiple of 32 up to 32768.  Every other value is
 *            W4_EUNSUPPORTED.  The products take the same G.
 *   mode     W4_SYM or W4_ASYM.
 *   fracs    HOST pointer to n_fracs fp32 fractions, 1 <= n_fracs <= 32,
 *            fracs[0] == 1.0f, every fraction in (0, 1].  n_fracs == 1 is the
 *            plain quantizer (no search).
 *   packed   [N, K/2] bytes out, the portable ("canonical") packing: byte
 *            [n, k/2] holds code k (k even) in its low nibble and code k+1 in
 *            its high nibble; symmetric codes as two's-complement nibbles.
 *   scale    [N, K/G] fp16 out.
 *   zero     [N, K/G] fp16 out: the integer zero point (exact for |z| <= 2048,
 *            which holds for every group whose range contains 0).  Required
 *            for W4_ASYM; must be NULL for W4_SYM.
 *   clip_idx [N, K/G] bytes out, index of the chosen fraction; may be NULL.
 */
int w4_quantize_blockwise(const float* W, int64_t N, int64_t K, int G, int mode,
                          const float* fracs, int n_fracs, uint8_t* packed, uint16_t* scale,
                          uint16_t* zero, uint8_t* clip_idx, hipStream_t stream);

/*
 * w4_mse_clip_search -- the search of w4_quantize_blockwise alone: for every
 * group, the index of the chosen fraction and optionally every candidate's
 * error.  Follows gowda.ai "LLM fast inference", "MSE clipping" (ranges
 * contracted about the observed midpoint, the block error including clipped
 * values, the plain quantizer kept unless a candidate is strictly better).
 * Arguments as for w4_quantize_blockwise, plus:
 *   clip_idx [N, K/G] bytes out (required).
 *   sse      [N, K/G, n_fracs] fp32 out, the candidates' squared-error sums
 *            exactly as compared by the search; may be NULL.
 */
int w4_mse_clip_search(const float* W, int64_t N, int64_t K, int G, int mode,
                       const float* fracs, int n_fracs, uint8_t* clip_idx, float* sse,
                       hipStream_t stream);

/*
 * w4_prepack -- rearrange the portable packing into the layout the multiply
 * kernels read ("GPU layout"), once per weight, without requantizing.
 * Follows gowda.ai "LLM fast inference", "MSE clipping" (last paragraph: the
 * portable packed codes, scales and zero terms are rearranged into a
 * GPU-specific layout without dequantizing) and "Runtime" (load-time
 * specialization of the checkpoint for the kernel).
 *   packed  [N, K/2] canonical bytes in (as written by w4_quantize_blockwise).
 *   scale   [N, K/G] fp16 in;  zero [N, K/G] fp16 in (W4_ASYM), NULL (W4_SYM).
 *   wq      N*K/8 uint32 out.  The 8 codes of row n, k = 8j..8j+7, form one
 *           word as unsigned 4-bit values u, with u = q (asym) or u = q + 8
 *           (sym); code k = 8j + 2i sits in bits 4i..4i+3 and code
 *           k = 8j + 2i + 1 in bits 16+4i..16+4i+3 (i = 0..3).  Words are
 *           stored in blocks of 16 rows and tiles of 32 k: with r0 = n - n % 16
 *           and nr = min(16, N - r0), word j of row n is at
 *             r0*K/8 + (j/4)*4*nr + 4*(n - r0) + j%4,
 *           so one 1 KB read holds a 16-row by 128-k fragment.
 *   sz      N*K/G uint32 out: per (row, group) the fp16 scale in the low half
 *           and the fp16 zero (8.0 for W4_SYM) in the high half, so that
 *           W'[n, k] = (u - zero) * scale; group g of row n is at
 *             r0*K/G + g*nr + (n - r0).
 *   N >= 0, K > 0, K % G == 0, G in {32, 64, 128} or G == K (per-channel).
 */
int w4_prepack(const uint8_t* packed, const uint16_t* scale, const uint16_t* zero, int64_t N,
               int64_t K, int G, int mode, uint32_t* wq, uint32_t* sz, hipStream_t stream);

/*
 * w4_quantize_rows_e4m3 -- dynamic per-row FP8 quantization of activations
 * (gowda.ai "LLM fast inference", "Achievement 2"; gsantana.dev "Number
 * formats: what the bits buy" for E4M3):
 *   xscale[m] = max(max_k |x[m, k]| / 448, 1e-8)   (fp32)
 *   xq[m, k]  = e4m3(fl32(x[m, k] / xscale[m]))      (round to nearest even,
 *                                                     saturating to +-448)
 *   X [M, K] bf16 in;  xq [M, K] bytes out;  xscale [M] fp32 out.
 *   M >= 0, K > 0, K % 8 == 0.  An all-zero row gives xscale = 1e-8 and codes 0.
 */
int w4_quantize_rows_e4m3(const uint16_t* X, int64_t M, int64_t K, uint8_t* xq, float* xscale,
                          hipStream_t stream);

/*
 * w4_gemm_workspace_bytes -- bytes of device workspace for the fastest
 * schedule of w4a16_gemm on a product of M rows, reduction K and N outputs
 * (the scratch of the products that gowda.ai "LLM fast inference",
 * "Achievement 2", defines; FP32 partial sums of one output are added in a
 * fixed order): splits * M * N * 4 bytes of fp32 partial sums when the
 * product splits K across workgroups, else 0.  Above 64 rows the tiled GEMM
 * needs it (a product with few output tiles splits K).  From 3 to 64 rows it
 * is optional.  From 33 to 64 rows with K a multiple of 64 it is the K split
 * of the tiled GEMM's 64 x 128 tiles, which then take the product (they read
 * the activations a quarter as often as the weight-streaming kernel).  Below
 * 33 rows (or with K not a multiple of 64) the weight-streaming kernel splits
 * K with it when its widest column blocks are fewer than the compute units.
 * Without it (NULL or fewer bytes) the product runs unsplit on the
 * weight-streaming kernel.  1 or 2 rows never use one.  Depends on the shape
 * only; 0 for shapes the products reject.
 */
size_t w4_gemm_workspace_bytes(int64_t M, int64_t K, int64_t N);

/*
 * w4a8_gemm_workspace_bytes -- bytes of device workspace for the fastest
 * schedule of w4a8_gemm and w4a8_gemm_e4m3 with any group size (gowda.ai
 * "LLM fast inference", "Achievement 2"), the larger of:
 *  - groups of 128 or whole rows, K a multiple of 128, more than 32 rows: the
 *    product runs on the fp8 matrix cores, on output tiles and a K split of
 *    its own (the fp32 partial tiles of the split; 0 when it does not split);
 *    this much is then required;
 *  - other groups: w4_gemm_workspace_bytes, and above 128 rows (K a multiple
 *    of 64, at least 256 output tiles of 256 x 256, i.e. a whole round over
 *    the compute units) also room for the row-quantized activations widened
 *    exactly to bf16 (M * K * 2 bytes after the split partials, at a 256-byte
 *    aligned offset).  With that much, w4a8_gemm runs the bf16 tiled kernel
 *    on the widened codes (same products: every finite E4M3 value is a bf16
 *    value); with only w4_gemm_workspace_bytes it runs a kernel that widens
 *    the E4M3 codes itself.  Both are exact widenings of the same
 *    activations; results may differ in the fp32 summation order only.
 */
size_t w4a8_gemm_workspace_bytes(int64_t M, int64_t K, int64_t N);

/*
 * w4a16_gemm -- W4A16: Y = bf16(X . W'^T) with W'[n, k] = (u - zero) * scale
 * from the GPU layout, fp32 accumulation, bf16 output (round to nearest
 * even).  Follows gsantana.dev "Quantizing LLMs Without Guesswork",
 * "Weight-only methods: GPTQ, AWQ and the file formats" (weights dequantized
 * inside the matmul, arithmetic in 16-bit), "Scale and zero point" (the
 * reconstruction (q - z) s) and "The Problem & Context" (decode reads every
 * weight once).  One entry point for every M: up to 32 rows run a kernel that
 * streams the weights once (bandwidth bound), larger M a tiled bf16-MFMA
 * GEMM; from 33 to 64 rows the tiled GEMM runs when the workspace holds its
 * K split (K a multiple of 64), else the streaming kernel.
 *   X  [M, K] bf16 in;  wq, sz as written by w4_prepack;  Y [M, N] bf16 out.
 *   workspace: device memory of workspace_bytes >= w4_gemm_workspace_bytes(M,
 *      K, N) bytes, 16-byte aligned, owned by the caller; its contents on
 *      entry do not matter and are overwritten.  May be NULL when that size
 *      is 0, or when M <= 64 (the streaming kernel then runs unsplit).  Calls
 *      in flight at the same time need separate workspaces.
 *      Too small or NULL when needed: W4_EINVAL.
 *   With a split K the partial sums are added in a fixed order: results do
 *   not depend on timing.
 */
int w4a16_gemm(const uint16_t* X, int64_t M, int64_t K, const uint32_t* wq, const uint32_t* sz,
               int64_t N, int G, uint16_t* Y, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * w4a16_gemm_noalloc -- w4a16_gemm for callers that cannot allocate device
 * memory (code under HIP graph capture, serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, with the scratch memory of a K
 * split taken from an array the library holds on each GPU
 * (W4_NOALLOC_SCRATCH_BYTES, kept until the process ends) instead of a
 * caller workspace.  The call allocates nothing; the caller passes X, the
 * weights and Y as for w4a16_gemm.
 *   A shape whose w4_gemm_workspace_bytes exceeds W4_NOALLOC_SCRATCH_BYTES
 *   returns W4_EINVAL (64 MiB covers every shape: a K split never needs more
 *   than 256 partial tiles of 256 x 256 fp32).
 *   Every call on one GPU uses that GPU's one array: calls that can overlap
 *   on a GPU (different streams or threads) race and must not be issued
 *   together; calls in order on one stream are safe.
 */
#define W4_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int w4a16_gemm_noalloc(const uint16_t* X, int64_t M, int64_t K, const uint32_t* wq, const uint32_t* sz,
                       int64_t N, int G, uint16_t* Y, hipStream_t stream);

/*
 * w4a8_gemm -- W4A8: each activation row is quantized to E4M3 exactly as by
 * w4_quantize_rows_e4m3, then Y = bf16(xscale[m] * sum_k e4m3(xq[m, k]) *
 * W'[n, k]) with fp32 accumulation.  Follows gowda.ai "LLM fast inference",
 * "Achievement 2: 8-bit activations without a calibration set" (per-row
 * dynamic E4M3, FP32 accumulation, the row scale in the epilogue, BF16
 * result).  With groups of 128 (or whole rows), K a multiple of 128 and more
 * than 32 rows the product runs on the fp8 matrix cores: both MFMA operands
 * E4M3, each weight as the exact integer u - z, one group per 128-k MFMA
 * step, its sum scaled by the group scale in fp32.  Otherwise up to 64 rows
 * the weight-streaming kernel and above them a tiled bf16-MFMA GEMM run on
 * the E4M3 codes widened exactly to bf16.
 *   X  [M, K] bf16 in.
 *   xq [M, K] bytes and xscale [M] fp32: device buffers the call fills (they
 *      are the operands of the multiply and are left for the caller to read).
 *   workspace: w4a8_gemm_workspace_bytes(M, K, N) bytes always suffice.
 *      The least accepted is the fp32 partials of the kernel that runs: on
 *      the fp8 kernel (groups of 128 or whole rows, K a multiple of 128, more
 *      than 32 rows) those of its own K split, otherwise
 *      w4_gemm_workspace_bytes(M, K, N) where that is required.  Too small or
 *      NULL when needed: W4_EINVAL.
 *   Other arguments as for w4a16_gemm.
 */
int w4a8_gemm(const uint16_t* X, int64_t M, int64_t K, const uint32_t* wq, const uint32_t* sz,
              int64_t N, int G, uint16_t* Y, uint8_t* xq, float* xscale, void* workspace,
              size_t workspace_bytes, hipStream_t stream);

/*
 * w4a16_gate_up / w4a8_gate_up -- the gate and up projections of a gated MLP
 * block in one pass, with the activation-and-multiply epilogue (gowda.ai "LLM
 * fast inference", "Machete, with credit where it is due": the speed comes
 * from a stack that includes model-specific fused paths):
 *   H = bf16(act(X . Wg'^T) * (X . Wu'^T)),
 * each product with fp32 accumulation (W4A8: the row-quantized E4M3
 * activations and their row scale, exactly as w4a8_gemm), the activation and
 * product in fp32, one rounding to bf16.  act: W4_ACT_SILU, x / (1 + e^-x)
 * (SwiGLU blocks), or W4_ACT_GELU_TANH, 0.5 x (1 + tanh(sqrt(2/pi) (x +
 * 0.044715 x^3))) (GeGLU blocks).  Up to 32 rows the weight-streaming
 * kernel reads both matrices at the same 16 output columns per workgroup;
 * above, a tiled MFMA GEMM holds 128 columns of each weight per workgroup
 * (some of its waves sum the gate products, the others the up products of
 * the same outputs) and needs K to be a multiple of 64 (else W4_EUNSUPPORTED).
 * W4A8 with groups of 128 runs it on the fp8 matrix cores.
 *   X            [M, K] bf16 in, M >= 0.
 *   wq_gate, sz_gate, wq_up, sz_up: two [N, K] weights in the GPU layout of
 *                w4_prepack, with the same G.
 *   H            [M, N] bf16 out.
 *   xq, xscale   (W4A8) as for w4a8_gemm.
 * W4A8 only -- the down projection's input in the same pass (gowda.ai "LLM
 * fast inference", "Machete, with credit where it is due", and "Achievement
 * 2": per-row E4M3 activations at the input of the next FP8 product):
 *   hq, hscale   [M, N] E4M3 bytes and [M] fp32 out, or both NULL: H's rows
 *                quantized exactly as w4_quantize_rows_e4m3(H) would (same
 *                codes and scales, bit for bit), for w4a8_gemm_e4m3 of the
 *                down projection.  Each workgroup of the pass also records
 *                the maximum |H| of every row over its columns, so the
 *                quantization reads H once instead of twice.  Needs N a
 *                multiple of 8.
 *   workspace    with hq: at least w4a8_gate_up_workspace_bytes(M, K, N)
 *                bytes, 16-byte aligned (the partial row maxima); else
 *                ignored (may be NULL).
 * W4A16 only -- an optional workspace (caller-owned, 16-byte aligned, its
 * contents on entry irrelevant) of w4a16_gate_up_workspace_bytes(M, K, N)
 * bytes lets the tiled form above 256 rows split the K range of the tiles of
 * its last, partial round over the compute units (fp32 partial sums of both
 * products, added in a fixed order by a second kernel that applies the
 * activation); NULL or fewer bytes: the same outputs unsplit.  Calls in
 * flight at the same time need separate workspaces.
 */
#define W4_ACT_SILU 1
#define W4_ACT_GELU_TANH 2
int w4a16_gate_up(const uint16_t* X, int64_t M, int64_t K, const uint32_t* wq_gate, const uint32_t* sz_gate,
                  const uint32_t* wq_up, const uint32_t* sz_up, int64_t N, int G, int act, uint16_t* H,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);
size_t w4a16_gate_up_workspace_bytes(int64_t M, int64_t K, int64_t N);
int w4a8_gate_up(const uint16_t* X, int64_t M, int64_t K, const uint32_t* wq_gate, const uint32_t* sz_gate,
                 const uint32_t* wq_up, const uint32_t* sz_up, int64_t N, int G, int act, uint16_t* H, uint8_t* xq,
                 float* xscale, uint8_t* hq, float* hscale, void* workspace, size_t workspace_bytes,
                 hipStream_t stream);
/* Bytes of workspace w4a8_gate_up needs to emit hq, the down projection's
 * per-row E4M3 input (gowda.ai "LLM fast inference", "Achievement 2": each
 * activation row is scaled by its own maximum before the FP8 product): M *
 * tiles * 4, the partial row maxima of H (16-column tiles up to 32 rows,
 * 128-column tiles above); 0 for empty shapes. */
size_t w4a8_gate_up_workspace_bytes(int64_t M, int64_t K, int64_t N);

/*
 * w4a8_gemm_e4m3 -- the W4A8 product on activations already quantized per
 * row (the hq / hscale of w4a8_gate_up, or w4_quantize_rows_e4m3):
 *   Y = bf16(xscale[m] * sum_k e4m3(xq[m, k]) * W'[n, k]), fp32 accumulation
 * (gowda.ai "LLM fast inference", "Achievement 2").  Same kernels and result
 * as w4a8_gemm after its row quantization.
 *   xq [M, K] E4M3 bytes in;  xscale [M] fp32 in;  K a multiple of 16.
 *   workspace: as for w4a8_gemm.
 *   Other arguments as for w4a8_gemm.
 */
int w4a8_gemm_e4m3(const uint8_t* xq, const float* xscale, int64_t M, int64_t K, const uint32_t* wq,
                   const uint32_t* sz, int64_t N, int G, uint16_t* Y, void* workspace, size_t workspace_bytes,
                   hipStream_t stream);

/*
 * NF4 comparator (gsantana.dev "Quantizing LLMs Without Guesswork",
 * "Weight-only methods: GPTQ, AWQ and the file formats", the NF4 paragraph):
 * 16 levels that are normal quantiles (QLoRA's construction: 8 positive and 7
 * negative quantiles at evenly spaced probabilities from delta = (1 - 1/30 +
 * 1 - 1/32) / 2 down to 1/2, an exact zero, scaled to [-1, 1]), blocks of 64
 * weights with an absmax scale, and double quantization of the scales: per
 * group of 256 consecutive block scales (flattened row-major) an fp32
 * constant c2 = max / 255 and 8-bit codes round_half_even(absmax / c2), 4.127
 * bits per weight in all.  It is the pages' comparison point, multiplied here
 * by the same kind of decode GEMV as W4A16.
 *
 * w4_nf4_levels: the 16 levels (fp32, ascending) into a HOST array.
 * w4_nf4_quantize: W [N, K] fp32 (K a multiple of 64) -> packed [N, K/2]
 *   (code of k even in the low nibble), absmax_q [N*K/64] bytes, absmax_c2
 *   [ceil(N*K/64/256)] fp32.  A weight's code is the level nearest to
 *   fp32(w / absmax) of its block (fp32 distances, the lower index on ties; a
 *   zero block gets the zero level); the codes use the unquantized absmax.
 *   Bit-reproducible (plain fp32 operations in a fixed order).
 * w4_nf4_gemv: y [N] = bf16(W' . x) for one bf16 row x [K] (K <= 32768),
 *   W'[n, k] = bf16(level[code]) * absmax_q * c2 of its block, fp32
 *   accumulation.
 * Device pointers, asynchronous on `stream`; W, packed, x and y 16-byte
 * aligned.
 */
int w4_nf4_levels(float* levels);
int w4_nf4_quantize(const float* W, int64_t N, int64_t K, uint8_t* packed, uint8_t* absmax_q, float* absmax_c2,
                    hipStream_t stream);
int w4_nf4_gemv(const uint16_t* x, int64_t K, const uint8_t* packed, const uint8_t* absmax_q, const float* absmax_c2,
                int64_t N, uint16_t* y, hipStream_t stream);

/*
 * Portable on-disk form of a quantized weight (gowda.ai "LLM fast inference",
 * "MSE clipping", last paragraph: the packed codes, scales and zero terms are
 * exported once in a portable representation and rearranged into the GPU
 * layout at load, without dequantizing and requantizing; "What the WMT26
 * paper finds": portable int4 codes are specialized for the kernel once).
 * The file holds exactly the canonical arrays of w4_quantize_blockwise, with
 * a header (shape, group size, mode, the clip fractions) and a 64-bit FNV-1a
 * hash of the payload.  Loading reads them into host memory; the caller
 * uploads them and runs w4_prepack (the Python binding's w4_portable_load
 * does both).  These three calls take HOST pointers, do file I/O only and
 * never touch the GPU.  Errors (unopenable, short, corrupted or foreign
 * files, inconsistent shapes) return W4_EINVAL, an unknown file version
 * W4_EUNSUPPORTED; w4_last_error says which.
 */
#define W4_PORTABLE_MAX_FRACS 32
typedef struct {
    int64_t N, K;            /* weight shape [N, K] */
    int32_t G;               /* group size (32, 64, 128, or K: per-channel) */
    int32_t mode;            /* W4_SYM or W4_ASYM */
    int32_t n_fracs;         /* clip fractions used by the quantizer (1 = plain) */
    int32_t has_clip;        /* 1 if the file holds the clip index of every group */
    uint64_t payload_bytes;  /* bytes after the header */
    float fracs[W4_PORTABLE_MAX_FRACS];
} w4_portable_info;

/* Writes packed [N, K/2], scale [N, K/G], zero [N, K/G] (W4_ASYM only; NULL
 * for W4_SYM) and clip_idx [N, K/G] (or NULL) to `path` (through a temporary
 * file renamed into place).  fracs: the n_fracs clip fractions of the search. */
int w4_portable_save(const char* path, int64_t N, int64_t K, int G, int mode, const float* fracs, int n_fracs,
                     const uint8_t* packed, const uint16_t* scale, const uint16_t* zero, const uint8_t* clip_idx);

/* Reads and checks the header of `path` into *info. */
int w4_portable_info_read(const char* path, w4_portable_info* info);

/* Reads the arrays of `path` into host buffers sized from its header (zero
 * may be NULL for W4_SYM; clip_idx may be NULL, and is zero-filled when the
 * file has none).  The payload hash is checked before anything is copied. */
int w4_portable_load(const char* path, uint8_t* packed, uint16_t* scale, uint16_t* zero, uint8_t* clip_idx);

/* Short text for a status code (static storage). */
const char* w4_status_string(int status);

/* Message of the last call on this thread that did not return W4_OK
 * (thread-local storage, valid until the next failing call). */
const char* w4_last_error(void);

/* Version of this ABI, currently 4 (4: w4a16_gate_up takes an optional
 * workspace, w4a16_gate_up_workspace_bytes; 3: w4a8_gate_up emits the down
 * projection's E4M3 input; w4a8_gemm_e4m3; w4a16_gemm_noalloc). */
int w4_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* W4_H */
