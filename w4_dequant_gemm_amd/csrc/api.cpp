// C ABI of the W4 library: argument checks, then the launches of the call on
// the caller's stream (one kernel, or two where a row quantization or a split
// sum goes with it).  No allocation, no state beyond a thread-local error
// message, the NF4 level table (computed once) and the per-device address of
// the no-alloc product's scratch array; no fallback: anything the kernels do
// not run is rejected before launch.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/w4.h"
#include "kernels.hpp"
#include "status.hpp"

namespace {
thread_local char g_last_error[512] = "";
}  // namespace

int w4::fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return status;
}

namespace {
using w4::fail;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return W4_OK;
    return fail(W4_EHIP, "%s: %s", what, hipGetErrorString(e));
}

int check_group(const char* fn, int64_t N, int64_t K, int G) {
    if (N < 0) return fail(W4_EINVAL, "%s: N = %lld must be >= 0", fn, static_cast<long long>(N));
    if (K <= 0) return fail(W4_EINVAL, "%s: K = %lld must be > 0", fn, static_cast<long long>(K));
    if (G == 32 || G == 64 || G == 128) {
        if (K % G != 0)
            return fail(W4_EINVAL, "%s: K = %lld is not a multiple of the group size %d", fn,
                        static_cast<long long>(K), G);
        return W4_OK;
    }
    if (G == K) {   // per-channel: one group per row
        if (K % 32 != 0 || K > w4::kMaxPerChannelK)
            return fail(W4_EUNSUPPORTED, "%s: per-channel groups (G = K = %lld) need K a multiple of 32, at most %lld",
                        fn, static_cast<long long>(K), static_cast<long long>(w4::kMaxPerChannelK));
        return W4_OK;
    }
    return fail(W4_EUNSUPPORTED, "%s: group size %d is not one of 32, 64, 128, or K (per-channel)", fn, G);
}

int check_fracs(const char* fn, const float* fracs, int n_fracs) {
    if (!fracs) return fail(W4_EINVAL, "%s: fracs is NULL", fn);
    if (n_fracs < 1 || n_fracs > W4_MAX_FRACS)
        return fail(W4_EINVAL, "%s: n_fracs = %d outside 1..%d", fn, n_fracs, W4_MAX_FRACS);
    if (fracs[0] != 1.0f) return fail(W4_EINVAL, "%s: fracs[0] must be 1.0 (the plain quantizer)", fn);
    for (int i = 0; i < n_fracs; ++i)
        if (!(fracs[i] > 0.0f && fracs[i] <= 1.0f))
            return fail(W4_EINVAL, "%s: fracs[%d] = %g outside (0, 1]", fn, i, static_cast<double>(fracs[i]));
    return W4_OK;
}

int check_mode(const char* fn, int mode) {
    if (mode != W4_SYM && mode != W4_ASYM) return fail(W4_EINVAL, "%s: mode %d is neither W4_SYM nor W4_ASYM", fn, mode);
    return W4_OK;
}

#define W4_REQUIRE_PTR(fn, p)                                                        \
    do {                                                                             \
        if (!(p)) return fail(W4_EINVAL, "%s: %s is NULL", fn, #p);                  \
        if (!aligned16(p)) return fail(W4_EINVAL, "%s: %s is not 16-byte aligned", fn, #p); \
    } while (0)

int quantize_common(const char* fn, const float* W, int64_t N, int64_t K, int G, int mode,
                    const float* fracs, int n_fracs, bool encode, uint8_t* packed, uint16_t* scale,
                    uint16_t* zero, uint8_t* clip, float* sse, hipStream_t stream) {
    W4_TRY(check_group(fn, N, K, G));
    W4_TRY(check_mode(fn, mode));
    W4_TRY(check_fracs(fn, fracs, n_fracs));
    if (N == 0) return W4_OK;
    W4_REQUIRE_PTR(fn, W);
    if (encode) {
        W4_REQUIRE_PTR(fn, packed);
        if (!scale) return fail(W4_EINVAL, "%s: scale is NULL", fn);
        if (mode == W4_ASYM && !zero) return fail(W4_EINVAL, "%s: zero is NULL for W4_ASYM", fn);
        if (mode == W4_SYM && zero) return fail(W4_EINVAL, "%s: zero must be NULL for W4_SYM", fn);
    } else if (!clip) {
        return fail(W4_EINVAL, "%s: clip_idx is NULL", fn);
    }
    w4::QuantizeParams p{};
    p.W = W;
    p.n_groups = N * (K / G);
    p.G = G;
    p.asym = mode == W4_ASYM;
    p.n_fracs = n_fracs;
    for (int i = 0; i < n_fracs; ++i) p.fracs[i] = fracs[i];
    p.encode = encode;
    p.packed = packed;
    p.scale = scale;
    p.zero = zero;
    p.clip = clip;
    p.sse = sse;
    return hip_status(w4::launch_quantize(p, stream), fn);
}

// true when a W4A8 product of this shape runs on the fp8 kernel (its own
// tiles and split schedule)
bool f8_product(int64_t M, int64_t K, int64_t N, int G) {
    return w4::f8_eligible(M, K, G) && w4::f8_fits_buffers(M, K, N);
}

// workspace the product's schedule needs (0: none)
size_t split_bytes(int64_t M, int64_t K, int64_t N, int G, bool fp8) {
    if (fp8 && f8_product(M, K, N, G)) return w4::f8_workspace_bytes(M, K, N);
    return M <= w4::kSkinnyMaxM ? 0 : w4::gemm_workspace_bytes(M, K, N);
}

int mul_common(const char* fn, const uint16_t* X, int64_t M, int64_t K, const uint32_t* wq,
               const uint32_t* sz, int64_t N, int G, uint16_t* Y, void* workspace, size_t workspace_bytes,
               bool fp8) {
    W4_TRY(check_group(fn, N, K, G));
    if (M < 0) return fail(W4_EINVAL, "%s: M = %lld must be >= 0", fn, static_cast<long long>(M));
    if (M == 0 || N == 0) return W4_OK;
    W4_REQUIRE_PTR(fn, X);
    W4_REQUIRE_PTR(fn, wq);
    W4_REQUIRE_PTR(fn, sz);
    W4_REQUIRE_PTR(fn, Y);
    // any workspace given is checked, whether or not this shape splits K: the
    // row quantizer of W4A8 may also place the widened activations there
    if (workspace && !aligned16(workspace)) return fail(W4_EINVAL, "%s: workspace is not 16-byte aligned", fn);
    const size_t need = split_bytes(M, K, N, G, fp8);
    if (need > 0) {
        if (!workspace)
            return fail(W4_EINVAL, "%s: this shape needs a workspace of %zu bytes (w4_gemm_workspace_bytes)", fn, need);
        if (workspace_bytes < need)
            return fail(W4_EINVAL, "%s: workspace of %zu bytes, this shape needs %zu", fn, workspace_bytes, need);
    }
    return W4_OK;
}

// the streaming kernel's K split when the caller gave a workspace large enough
// for it (optional: without one the product runs unsplit)
w4::MulParams with_skinny_split(w4::MulParams p, void* workspace, size_t workspace_bytes) {
    const int s = w4::skinny_splits(p.M, p.K, p.N, p.x_fp8 ? 1 : 2);
    if (s > 1 && workspace && aligned16(workspace) &&
        workspace_bytes >= w4::skinny_workspace_bytes(p.M, p.K, p.N)) {
        p.splits = s;
        p.ws = static_cast<float*>(workspace);
    }
    return p;
}

// the tiled-GEMM launch of a product, with the K split that its workspace was sized for
w4::MulParams with_split(w4::MulParams p, void* workspace) {
    const w4::GemmSplit g = p.x_fp8 && f8_product(p.M, p.K, p.N, p.G) ? w4::f8_split(p.M, p.K, p.N)
                            : w4::a16_runs(p.M, p.K, p.N, p.G, p.x_fp8) ? w4::a16_split(p.M, p.K, p.N)
                                                                          : w4::gemm_split(p.M, p.K, p.N);
    p.splits = g.splits;
    p.split_t0 = g.t0;
    p.ws = g.splits > 1 ? static_cast<float*>(workspace) : nullptr;
    return p;
}

}  // namespace

namespace {
// The 16 NF4 levels (QLoRA's construction): normal quantiles at 8 evenly
// spaced probabilities from delta down to 1/2 (exclusive) for the positive
// side and 7 for the negative side, delta = (1 - 1/30 + 1 - 1/32) / 2, and
// an exact zero, divided by the largest and rounded once to fp32.  The
// inverse normal CDF is found by bisection on Phi(x) = erfc(-x / sqrt 2) / 2
// in double precision (to the last bit of the bracket).
double inv_normal_cdf(double p) {
    double lo = -10.0, hi = 10.0;
    for (int i = 0; i < 200; ++i) {
        const double mid = 0.5 * (lo + hi);
        if (mid == lo || mid == hi) break;
        if (0.5 * std::erfc(-mid / std::sqrt(2.0)) < p) lo = mid;
        else hi = mid;
    }
    return 0.5 * (lo + hi);
}

void nf4_levels_compute(float* out) {
    const double delta = 0.5 * (1.0 - 1.0 / 30.0) + 0.5 * (1.0 - 1.0 / 32.0);
    double v[16];
    int n = 0;
    for (int i = 0; i < 7; ++i) v[n++] = -inv_normal_cdf(delta + (0.5 - delta) * i / 7.0);
    v[n++] = 0.0;
    for (int i = 0; i < 8; ++i) v[n++] = inv_normal_cdf(delta + (0.5 - delta) * i / 8.0);
    double vmax = 0.0;
    for (int i = 0; i < 16; ++i) vmax = v[i] > vmax ? v[i] : vmax;
    // ascending: the negative side from -1 up to 0, then the positive side from 0 up to 1
    float sorted[16];
    for (int i = 0; i < 7; ++i) sorted[i] = static_cast<float>(v[i] / vmax);
    sorted[7] = 0.0f;
    for (int i = 0; i < 8; ++i) sorted[15 - i] = static_cast<float>(v[8 + i] / vmax);
    for (int i = 0; i < 16; ++i) out[i] = sorted[i];
}

// The table, computed once (the bisection costs tens of microseconds, more
// than a decode product).
struct Nf4Table {
    float v[16];
    Nf4Table() { nf4_levels_compute(v); }
};

void nf4_levels(float* out) {
    static const Nf4Table table;
    for (int i = 0; i < 16; ++i) out[i] = table.v[i];
}

int check_nf4_shape(const char* fn, int64_t N, int64_t K) {
    if (N < 0) return fail(W4_EINVAL, "%s: N = %lld must be >= 0", fn, static_cast<long long>(N));
    if (K <= 0 || K % 64 != 0)
        return fail(W4_EINVAL, "%s: K = %lld must be a positive multiple of the NF4 block (64)", fn,
                    static_cast<long long>(K));
    return W4_OK;
}

// shared checks of the gate and up product
int gate_up_common(const char* fn, const uint16_t* X, int64_t M, int64_t K, const uint32_t* wq_gate,
                   const uint32_t* sz_gate, const uint32_t* wq_up, const uint32_t* sz_up, int64_t N, int G, int act,
                   uint16_t* H) {
    W4_TRY(check_group(fn, N, K, G));
    if (M < 0) return fail(W4_EINVAL, "%s: M = %lld must be >= 0", fn, static_cast<long long>(M));
    if (M > 0 && N > 0) {
        W4_REQUIRE_PTR(fn, X);
        W4_REQUIRE_PTR(fn, wq_gate);
        W4_REQUIRE_PTR(fn, sz_gate);
        W4_REQUIRE_PTR(fn, H);
    }
    if (M > w4::kGateUpMaxM && K % 64 != 0)
        return fail(W4_EUNSUPPORTED, "%s: M = %lld rows take the tiled form, which needs K a multiple of 64 (K = %lld)",
                    fn, static_cast<long long>(M), static_cast<long long>(K));
    if (act != W4_ACT_SILU && act != W4_ACT_GELU_TANH)
        return fail(W4_EINVAL, "%s: act = %d is neither W4_ACT_SILU nor W4_ACT_GELU_TANH", fn, act);
    if (M == 0 || N == 0) return W4_OK;
    W4_REQUIRE_PTR(fn, wq_up);
    W4_REQUIRE_PTR(fn, sz_up);
    return W4_OK;
}
}  // namespace

extern "C" {

int w4_quantize_blockwise(const float* W, int64_t N, int64_t K, int G, int mode, const float* fracs,
                          int n_fracs, uint8_t* packed, uint16_t* scale, uint16_t* zero,
                          uint8_t* clip_idx, hipStream_t stream) {
    return quantize_common("w4_quantize_blockwise", W, N, K, G, mode, fracs, n_fracs, true, packed, scale,
                           zero, clip_idx, nullptr, stream);
}

int w4_mse_clip_search(const float* W, int64_t N, int64_t K, int G, int mode, const float* fracs,
                       int n_fracs, uint8_t* clip_idx, float* sse, hipStream_t stream) {
    return quantize_common("w4_mse_clip_search", W, N, K, G, mode, fracs, n_fracs, false, nullptr, nullptr,
                           nullptr, clip_idx, sse, stream);
}

int w4_prepack(const uint8_t* packed, const uint16_t* scale, const uint16_t* zero, int64_t N, int64_t K,
               int G, int mode, uint32_t* wq, uint32_t* sz, hipStream_t stream) {
    const char* fn = "w4_prepack";
    W4_TRY(check_group(fn, N, K, G));
    W4_TRY(check_mode(fn, mode));
    if (N == 0) return W4_OK;
    W4_REQUIRE_PTR(fn, packed);
    if (!scale) return fail(W4_EINVAL, "%s: scale is NULL", fn);
    if (mode == W4_ASYM && !zero) return fail(W4_EINVAL, "%s: zero is NULL for W4_ASYM", fn);
    W4_REQUIRE_PTR(fn, wq);
    W4_REQUIRE_PTR(fn, sz);
    w4::PrepackParams p{packed, scale, zero, N, K, G, mode == W4_ASYM, wq, sz};
    return hip_status(w4::launch_prepack(p, stream), fn);
}

int w4_quantize_rows_e4m3(const uint16_t* X, int64_t M, int64_t K, uint8_t* xq, float* xscale,
                          hipStream_t stream) {
    const char* fn = "w4_quantize_rows_e4m3";
    if (M < 0) return fail(W4_EINVAL, "%s: M = %lld must be >= 0", fn, static_cast<long long>(M));
    if (K <= 0 || K % 8 != 0)
        return fail(W4_EINVAL, "%s: K = %lld must be a positive multiple of 8", fn, static_cast<long long>(K));
    if (M == 0) return W4_OK;
    W4_REQUIRE_PTR(fn, X);
    W4_REQUIRE_PTR(fn, xq);
    if (!xscale) return fail(W4_EINVAL, "%s: xscale is NULL", fn);
    w4::RowQuantParams p{X, M, K, xq, xscale};
    return hip_status(w4::launch_rowquant(p, stream), fn);
}

size_t w4_gemm_workspace_bytes(int64_t M, int64_t K, int64_t N) {
    if (M <= 0 || K <= 0 || N <= 0) return 0;
    if (M <= w4::kSkinnyMaxM) {
        // optional: the tiled kernel's split from kTiledFromM rows (K a
        // multiple of 64), the streaming kernel's below
        if (M >= w4::kTiledFromM && w4::use_mid(M, K)) return w4::gemm_workspace_bytes(M, K, N);
        return w4::skinny_workspace_bytes(M, K, N);
    }
    return w4::gemm_workspace_bytes(M, K, N);
}

size_t w4a8_gemm_workspace_bytes(int64_t M, int64_t K, int64_t N) {
    if (M <= 0 || K <= 0 || N <= 0) return 0;
    // groups of 128 (or whole rows): the fp8 kernel's own schedule
    const size_t f8 = f8_product(M, K, N, w4::kF8StepK) ? w4::f8_workspace_bytes(M, K, N) : 0;
    // other groups: the bf16 kernels' schedule, with the widened activations
    // where they pay
    const size_t xw = M <= w4::kSkinnyMaxM ? 0 : w4::gemm_xw_bytes(M, K, N);
    const size_t with_xw = xw ? w4::gemm_xw_offset(M, K, N) + xw : 0;
    const size_t base = w4_gemm_workspace_bytes(M, K, N);
    const size_t bf = with_xw > base ? with_xw : base;
    return f8 > bf ? f8 : bf;
}

namespace {
// W4A16 on the tiled kernel: always above the streaming kernel's rows; from
// kTiledFromM rows on when K suits the 64 x 128 tiles and the workspace holds
// their K split (the streaming kernel's workspace stays optional)
bool w4a16_tiled(int64_t M, int64_t K, int64_t N, const void* workspace, size_t workspace_bytes) {
    if (M > w4::kSkinnyMaxM) return true;
    if (M < w4::kTiledFromM || !w4::use_mid(M, K)) return false;
    const size_t need = w4::gemm_workspace_bytes(M, K, N);
    return need == 0 || (workspace && aligned16(workspace) && workspace_bytes >= need);
}

int w4a16_run(const char* fn, const uint16_t* X, int64_t M, int64_t K, const uint32_t* wq, const uint32_t* sz,
              int64_t N, int G, uint16_t* Y, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    W4_TRY(mul_common(fn, X, M, K, wq, sz, N, G, Y, workspace, workspace_bytes, false));
    if (M == 0 || N == 0) return W4_OK;
    w4::MulParams p{X, nullptr, M, K, N, G, wq, sz, Y, false};
    if (!w4a16_tiled(M, K, N, workspace, workspace_bytes))
        return hip_status(w4::launch_skinny(with_skinny_split(p, workspace, workspace_bytes), stream), fn);
    return hip_status(w4::launch_gemm(with_split(p, workspace), stream), fn);
}
}  // namespace

int w4a16_gemm(const uint16_t* X, int64_t M, int64_t K, const uint32_t* wq, const uint32_t* sz, int64_t N,
               int G, uint16_t* Y, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return w4a16_run("w4a16_gemm", X, M, K, wq, sz, N, G, Y, workspace, workspace_bytes, stream);
}

int w4a16_gemm_noalloc(const uint16_t* X, int64_t M, int64_t K, const uint32_t* wq, const uint32_t* sz,
                       int64_t N, int G, uint16_t* Y, hipStream_t stream) {
    const char* fn = "w4a16_gemm_noalloc";
    W4_TRY(check_group(fn, N, K, G));
    if (M < 0) return fail(W4_EINVAL, "%s: M = %lld must be >= 0", fn, static_cast<long long>(M));
    if (M == 0 || N == 0) return W4_OK;
    const size_t need = M <= w4::kSkinnyMaxM ? 0 : w4::gemm_workspace_bytes(M, K, N);
    if (need > W4_NOALLOC_SCRATCH_BYTES)
        return fail(W4_EINVAL, "%s: this shape needs %zu bytes of scratch; the library holds %zu", fn, need,
                    static_cast<size_t>(W4_NOALLOC_SCRATCH_BYTES));
    void* scratch = nullptr;
    W4_TRY(hip_status(w4::noalloc_scratch(&scratch), fn));
    return w4a16_run(fn, X, M, K, wq, sz, N, G, Y, scratch, W4_NOALLOC_SCRATCH_BYTES, stream);
}

int w4a8_gemm(const uint16_t* X, int64_t M, int64_t K, const uint32_t* wq, const uint32_t* sz, int64_t N,
              int G, uint16_t* Y, uint8_t* xq, float* xscale, void* workspace, size_t workspace_bytes,
              hipStream_t stream) {
    const char* fn = "w4a8_gemm";
    W4_TRY(mul_common(fn, X, M, K, wq, sz, N, G, Y, workspace, workspace_bytes, true));
    if (M == 0 || N == 0) return W4_OK;
    W4_REQUIRE_PTR(fn, xq);
    if (!xscale) return fail(W4_EINVAL, "%s: xscale is NULL", fn);
    if (w4::skinny_quantizes_rows(M, K)) {
        // one kernel: row quantization (same arithmetic) and product
        w4::MulParams p{X, nullptr, M, K, N, G, wq, sz, Y, true, xq, xscale};
        return hip_status(w4::launch_skinny(p, stream), fn);
    }
    // above 128 rows, a workspace that also holds the widened activations
    // (w4a8_gemm_workspace_bytes) lets the row quantizer write them and the
    // bf16 tiled kernel run on them
    uint16_t* xw = nullptr;
    const size_t xw_bytes = M > w4::kSkinnyMaxM && !f8_product(M, K, N, G) ? w4::gemm_xw_bytes(M, K, N) : 0;
    if (xw_bytes && workspace && workspace_bytes >= w4::gemm_xw_offset(M, K, N) + xw_bytes)
        xw = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + w4::gemm_xw_offset(M, K, N));
    w4::RowQuantParams rq{X, M, K, xq, xscale, xw};
    W4_TRY(hip_status(w4::launch_rowquant(rq, stream), fn));
    w4::MulParams p{xq, xscale, M, K, N, G, wq, sz, Y, true};
    p.xw = xw;
    if (M <= w4::kSkinnyMaxM && !f8_product(M, K, N, G))
        return hip_status(w4::launch_skinny(with_skinny_split(p, workspace, workspace_bytes), stream), fn);
    return hip_status(w4::launch_gemm(with_split(p, workspace), stream), fn);
}


size_t w4a16_gate_up_workspace_bytes(int64_t M, int64_t K, int64_t N) {
    if (M <= 0 || K <= 0 || N <= 0) return 0;
    return w4::pair_workspace_bytes(M, K, N);
}

int w4a16_gate_up(const uint16_t* X, int64_t M, int64_t K, const uint32_t* wq_gate, const uint32_t* sz_gate,
                  const uint32_t* wq_up, const uint32_t* sz_up, int64_t N, int G, int act, uint16_t* H,
                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
    const char* fn = "w4a16_gate_up";
    W4_TRY(gate_up_common(fn, X, M, K, wq_gate, sz_gate, wq_up, sz_up, N, G, act, H));
    if (M == 0 || N == 0) return W4_OK;
    if (workspace && !aligned16(workspace)) return fail(W4_EINVAL, "%s: workspace is not 16-byte aligned", fn);
    w4::MulParams p{X, nullptr, M, K, N, G, wq_gate, sz_gate, H, false};
    p.wq2 = wq_up;
    p.sz2 = sz_up;
    p.act = act;
    // the optional split of the tiled form's last round
    const size_t need = w4::pair_workspace_bytes(M, K, N);
    if (M > w4::kGateUpMaxM && need > 0 && workspace && workspace_bytes >= need) {
        const w4::GemmSplit g = w4::pair_split(M, K, N);
        p.splits = g.splits;
        p.split_t0 = g.t0;
        p.ws = static_cast<float*>(workspace);
    }
    if (M > w4::kGateUpMaxM) return hip_status(w4::launch_gemm_pair(p, stream), fn);
    return hip_status(w4::launch_skinny(p, stream), fn);
}

size_t w4a8_gate_up_workspace_bytes(int64_t M, int64_t K, int64_t N) {
    if (M <= 0 || K <= 0 || N <= 0) return 0;
    return static_cast<size_t>(M) * static_cast<size_t>(w4::gate_up_amax_tiles(M, N)) * sizeof(float);
}

int w4a8_gate_up(const uint16_t* X, int64_t M, int64_t K, const uint32_t* wq_gate, const uint32_t* sz_gate,
                 const uint32_t* wq_up, const uint32_t* sz_up, int64_t N, int G, int act, uint16_t* H, uint8_t* xq,
                 float* xscale, uint8_t* hq, float* hscale, void* workspace, size_t workspace_bytes,
                 hipStream_t stream) {
    const char* fn = "w4a8_gate_up";
    W4_TRY(gate_up_common(fn, X, M, K, wq_gate, sz_gate, wq_up, sz_up, N, G, act, H));
    if (M == 0 || N == 0) return W4_OK;
    W4_REQUIRE_PTR(fn, xq);
    if (!xscale) return fail(W4_EINVAL, "%s: xscale is NULL", fn);
    const bool emit = hq != nullptr;
    if (emit) {
        if (N % 8 != 0) return fail(W4_EINVAL, "%s: the E4M3 form of H needs N a multiple of 8 (N = %lld)", fn,
                                    static_cast<long long>(N));
        W4_REQUIRE_PTR(fn, hq);
        if (!hscale) return fail(W4_EINVAL, "%s: hq given without hscale", fn);
        const size_t need = w4a8_gate_up_workspace_bytes(M, K, N);
        if (!workspace || workspace_bytes < need)
            return fail(W4_EINVAL, "%s: emitting hq needs a workspace of %zu bytes (w4a8_gate_up_workspace_bytes)",
                        fn, need);
        if (!aligned16(workspace)) return fail(W4_EINVAL, "%s: workspace is not 16-byte aligned", fn);
    } else if (hscale) {
        return fail(W4_EINVAL, "%s: hscale given without hq", fn);
    }
    w4::MulParams p{X, nullptr, M, K, N, G, wq_gate, sz_gate, H, true, xq, xscale};
    p.wq2 = wq_up;
    p.sz2 = sz_up;
    p.act = act;
    if (emit) {
        p.amax_part = static_cast<float*>(workspace);
        p.amax_tiles = w4::gate_up_amax_tiles(M, N);
    }
    if (M > w4::kGateUpMaxM || !w4::skinny_quantizes_rows(M, K)) {
        w4::RowQuantParams rq{X, M, K, xq, xscale};
        W4_TRY(hip_status(w4::launch_rowquant(rq, stream), fn));
        p.X = xq;
        p.xscale = xscale;
        p.xq_out = nullptr;
        p.xscale_out = nullptr;
    }
    W4_TRY(hip_status(M > w4::kGateUpMaxM ? w4::launch_gemm_pair(p, stream) : w4::launch_skinny(p, stream), fn));
    if (!emit) return W4_OK;
    // H's rows quantized to E4M3 from the row maxima the pass left behind
    w4::RowQuantParams hq_p{H, M, N, hq, hscale};
    hq_p.amax_part = p.amax_part;
    hq_p.amax_tiles = p.amax_tiles;
    return hip_status(w4::launch_rowquant(hq_p, stream), fn);
}

int w4a8_gemm_e4m3(const uint8_t* xq, const float* xscale, int64_t M, int64_t K, const uint32_t* wq,
                   const uint32_t* sz, int64_t N, int G, uint16_t* Y, void* workspace, size_t workspace_bytes,
                   hipStream_t stream) {
    const char* fn = "w4a8_gemm_e4m3";
    W4_TRY(mul_common(fn, reinterpret_cast<const uint16_t*>(xq), M, K, wq, sz, N, G, Y, workspace, workspace_bytes,
                      true));
    if (M == 0 || N == 0) return W4_OK;
    if (K % 16 != 0) return fail(W4_EINVAL, "%s: K = %lld must be a multiple of 16", fn, static_cast<long long>(K));
    if (!xscale) return fail(W4_EINVAL, "%s: xscale is NULL", fn);
    w4::MulParams p{xq, xscale, M, K, N, G, wq, sz, Y, true};
    if (M <= w4::kSkinnyMaxM && !f8_product(M, K, N, G))
        return hip_status(w4::launch_skinny(with_skinny_split(p, workspace, workspace_bytes), stream), fn);
    return hip_status(w4::launch_gemm(with_split(p, workspace), stream), fn);
}

int w4_nf4_levels(float* levels) {
    if (!levels) return fail(W4_EINVAL, "w4_nf4_levels: levels is NULL");
    nf4_levels(levels);
    return W4_OK;
}

int w4_nf4_quantize(const float* W, int64_t N, int64_t K, uint8_t* packed, uint8_t* absmax_q, float* absmax_c2,
                    hipStream_t stream) {
    const char* fn = "w4_nf4_quantize";
    W4_TRY(check_nf4_shape(fn, N, K));
    if (N == 0) return W4_OK;
    W4_REQUIRE_PTR(fn, W);
    W4_REQUIRE_PTR(fn, packed);
    if (!absmax_q || !absmax_c2) return fail(W4_EINVAL, "%s: absmax_q or absmax_c2 is NULL", fn);
    w4::Nf4QuantParams p{};
    p.W = W;
    p.n_blocks = N * (K / 64);
    nf4_levels(p.levels);
    p.packed = packed;
    p.absmax_q = absmax_q;
    p.c2 = absmax_c2;
    return hip_status(w4::launch_nf4_quantize(p, stream), fn);
}

int w4_nf4_gemv(const uint16_t* x, int64_t K, const uint8_t* packed, const uint8_t* absmax_q, const float* absmax_c2,
                int64_t N, uint16_t* y, hipStream_t stream) {
    const char* fn = "w4_nf4_gemv";
    W4_TRY(check_nf4_shape(fn, N, K));
    if (K > w4::kNf4MaxK)
        return fail(W4_EUNSUPPORTED, "%s: K = %lld above %lld (one 32-k chunk per lane of a 1024-lane workgroup)", fn,
                    static_cast<long long>(K), static_cast<long long>(w4::kNf4MaxK));
    if (N == 0) return W4_OK;
    W4_REQUIRE_PTR(fn, x);
    W4_REQUIRE_PTR(fn, packed);
    W4_REQUIRE_PTR(fn, y);
    if (!absmax_q || !absmax_c2) return fail(W4_EINVAL, "%s: absmax_q or absmax_c2 is NULL", fn);
    w4::Nf4GemvParams p{};
    p.x = x;
    p.K = K;
    p.N = N;
    p.packed = packed;
    p.absmax_q = absmax_q;
    p.c2 = absmax_c2;
    p.y = y;
    nf4_levels(p.levels);
    return hip_status(w4::launch_nf4_gemv(p, stream), fn);
}

const char* w4_status_string(int status) {
    switch (status) {
        case W4_OK: return "ok";
        case W4_EINVAL: return "invalid argument";
        case W4_EUNSUPPORTED: return "unsupported configuration";
        case W4_EHIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* w4_last_error(void) { return g_last_error; }

int w4_abi_version(void) { return 4; }

static_assert(W4_NOALLOC_SCRATCH_BYTES == w4::kNoAllocScratchBytes, "w4.h and the library agree on the scratch size");

}  // extern "C"
