// Portable on-disk form of a quantized weight and its reader.
//
// gowda.ai "LLM fast inference", "MSE clipping" (last paragraph): a dense
// checkpoint can be exported once into a portable representation of packed
// codes, scales and zero terms, which the runtime rearranges into its GPU
// layout without dequantizing and requantizing; "What the WMT26 paper finds":
// portable int4 codes are specialized for the kernel once, at load.  This
// file holds the host side of that flow: the canonical arrays of
// w4_quantize_blockwise are written as they are, and read back into host
// memory, from where the caller uploads them and runs w4_prepack.
//
// Layout (all integers little-endian):
//   0   char[8]  magic "W4QPORT" + NUL
//   8   u32      version (1)
//   12  u32      header bytes (64 + fracs, rounded up to 64)
//   16  i64      N
//   24  i64      K
//   32  i32      G
//   36  i32      mode (W4_SYM / W4_ASYM)
//   40  i32      number of clip fractions
//   44  u32      flags (bit 0: clip indices present)
//   48  u64      payload bytes
//   56  u64      FNV-1a 64-bit hash of the payload
//   64  f32[n]   clip fractions, then zeros up to the header size
//   payload, each section starting on a 64-byte boundary:
//       packed [N, K/2] u8, scale [N, K/G] fp16, zero [N, K/G] fp16 (asym
//       only), clip index [N, K/G] u8 (if flagged)
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>
#include <vector>

#include "../../include/w4.h"
#include "status.hpp"

namespace {

constexpr char kMagic[8] = {'W', '4', 'Q', 'P', 'O', 'R', 'T', '\0'};
constexpr uint32_t kVersion = 1;
constexpr uint64_t kAlign = 64;

uint64_t round_up(uint64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Sections {
    uint64_t packed, scale, zero, clip, total;   // offsets within the payload, and its size
};

Sections sections(int64_t N, int64_t K, int G, int mode, bool has_clip) {
    const uint64_t groups = static_cast<uint64_t>(N) * static_cast<uint64_t>(K / G);
    Sections s{};
    s.packed = 0;
    s.scale = round_up(static_cast<uint64_t>(N) * static_cast<uint64_t>(K / 2));
    s.zero = round_up(s.scale + 2 * groups);
    s.clip = mode == W4_ASYM ? round_up(s.zero + 2 * groups) : s.zero;
    s.total = has_clip ? round_up(s.clip + groups) : s.clip;
    return s;
}

struct Fnv {
    uint64_t h = 1469598103934665603ull;
    void add(const void* p, size_t n) {
        const uint8_t* b = static_cast<const uint8_t*>(p);
        for (size_t i = 0; i < n; ++i) {
            h ^= b[i];
            h *= 1099511628211ull;
        }
    }
};

using w4::fail;   // the same thread-local message as the other entry points

struct File {
    FILE* f = nullptr;
    ~File() {
        if (f) fclose(f);
    }
};

void put_u32(uint8_t* p, uint32_t v) { memcpy(p, &v, 4); }
void put_u64(uint8_t* p, uint64_t v) { memcpy(p, &v, 8); }
uint32_t get_u32(const uint8_t* p) {
    uint32_t v;
    memcpy(&v, p, 4);
    return v;
}
uint64_t get_u64(const uint8_t* p) {
    uint64_t v;
    memcpy(&v, p, 8);
    return v;
}

int check_shape(const char* fn, int64_t N, int64_t K, int G, int mode, int n_fracs) {
    if (N < 0 || K <= 0) return fail(W4_EINVAL, "%s: bad shape N = %lld, K = %lld", fn, (long long)N, (long long)K);
    if (G != 32 && G != 64 && G != 128 && G != K)
        return fail(W4_EUNSUPPORTED, "%s: group size %d is not one of 32, 64, 128, or K (per-channel)", fn, G);
    if (K % G != 0) return fail(W4_EINVAL, "%s: K = %lld is not a multiple of G = %d", fn, (long long)K, G);
    if (mode != W4_SYM && mode != W4_ASYM) return fail(W4_EINVAL, "%s: mode %d is not W4_SYM or W4_ASYM", fn, mode);
    if (n_fracs < 1 || n_fracs > W4_PORTABLE_MAX_FRACS)
        return fail(W4_EINVAL, "%s: %d clip fractions (1 to %d)", fn, n_fracs, W4_PORTABLE_MAX_FRACS);
    return W4_OK;
}

int read_header(const char* fn, FILE* f, w4_portable_info* info, uint64_t* header_bytes, uint64_t* hash) {
    uint8_t h[64];
    if (fread(h, 1, 64, f) != 64) return fail(W4_EINVAL, "%s: file shorter than a header", fn);
    if (memcmp(h, kMagic, 8) != 0) return fail(W4_EINVAL, "%s: not a portable W4 file (magic)", fn);
    if (get_u32(h + 8) != kVersion) return fail(W4_EUNSUPPORTED, "%s: file version %u, this library reads %u", fn,
                                                get_u32(h + 8), kVersion);
    memset(info, 0, sizeof(*info));
    info->N = static_cast<int64_t>(get_u64(h + 16));
    info->K = static_cast<int64_t>(get_u64(h + 24));
    info->G = static_cast<int32_t>(get_u32(h + 32));
    info->mode = static_cast<int32_t>(get_u32(h + 36));
    info->n_fracs = static_cast<int32_t>(get_u32(h + 40));
    info->has_clip = static_cast<int32_t>(get_u32(h + 44) & 1u);
    info->payload_bytes = get_u64(h + 48);
    *hash = get_u64(h + 56);
    W4_TRY(check_shape(fn, info->N, info->K, info->G, info->mode, info->n_fracs));
    *header_bytes = get_u32(h + 12);
    if (*header_bytes != round_up(64 + 4 * static_cast<uint64_t>(info->n_fracs)))
        return fail(W4_EINVAL, "%s: inconsistent header size", fn);
    if (info->payload_bytes != sections(info->N, info->K, info->G, info->mode, info->has_clip).total)
        return fail(W4_EINVAL, "%s: payload size does not match the shape", fn);
    if (fread(info->fracs, 4, info->n_fracs, f) != static_cast<size_t>(info->n_fracs))
        return fail(W4_EINVAL, "%s: truncated header", fn);
    return W4_OK;
}

}  // namespace

extern "C" {

int w4_portable_save(const char* path, int64_t N, int64_t K, int G, int mode, const float* fracs, int n_fracs,
                     const uint8_t* packed, const uint16_t* scale, const uint16_t* zero, const uint8_t* clip_idx) {
    const char* fn = "w4_portable_save";
    if (!path) return fail(W4_EINVAL, "%s: path is NULL", fn);
    W4_TRY(check_shape(fn, N, K, G, mode, n_fracs));
    if (!fracs) return fail(W4_EINVAL, "%s: fracs is NULL", fn);
    if (N > 0 && (!packed || !scale)) return fail(W4_EINVAL, "%s: packed or scale is NULL", fn);
    if (N > 0 && mode == W4_ASYM && !zero) return fail(W4_EINVAL, "%s: zero is NULL for W4_ASYM", fn);
    const bool has_clip = clip_idx != nullptr;
    const Sections s = sections(N, K, G, mode, has_clip);
    const uint64_t groups = static_cast<uint64_t>(N) * static_cast<uint64_t>(K / G);

    // payload in memory (the weights of one matrix), then its hash
    std::vector<uint8_t> payload(s.total, 0);
    if (N > 0) {
        memcpy(payload.data() + s.packed, packed, static_cast<size_t>(N) * static_cast<size_t>(K / 2));
        memcpy(payload.data() + s.scale, scale, 2 * groups);
        if (mode == W4_ASYM) memcpy(payload.data() + s.zero, zero, 2 * groups);
        if (has_clip) memcpy(payload.data() + s.clip, clip_idx, groups);
    }
    Fnv hash;
    hash.add(payload.data(), payload.size());

    const uint64_t hb = round_up(64 + 4 * static_cast<uint64_t>(n_fracs));
    std::vector<uint8_t> header(hb, 0);
    memcpy(header.data(), kMagic, 8);
    put_u32(header.data() + 8, kVersion);
    put_u32(header.data() + 12, static_cast<uint32_t>(hb));
    put_u64(header.data() + 16, static_cast<uint64_t>(N));
    put_u64(header.data() + 24, static_cast<uint64_t>(K));
    put_u32(header.data() + 32, static_cast<uint32_t>(G));
    put_u32(header.data() + 36, static_cast<uint32_t>(mode));
    put_u32(header.data() + 40, static_cast<uint32_t>(n_fracs));
    put_u32(header.data() + 44, has_clip ? 1u : 0u);
    put_u64(header.data() + 48, s.total);
    put_u64(header.data() + 56, hash.h);
    memcpy(header.data() + 64, fracs, 4 * static_cast<size_t>(n_fracs));

    // written to a temporary name and renamed, so a reader never sees half a file
    const std::string tmp = std::string(path) + ".tmp";
    {
        File out;
        out.f = fopen(tmp.c_str(), "wb");
        if (!out.f) return fail(W4_EINVAL, "%s: cannot open %s for writing", fn, tmp.c_str());
        if (fwrite(header.data(), 1, header.size(), out.f) != header.size() ||
            fwrite(payload.data(), 1, payload.size(), out.f) != payload.size() || fflush(out.f) != 0) {
            remove(tmp.c_str());
            return fail(W4_EINVAL, "%s: write to %s failed", fn, tmp.c_str());
        }
    }
    if (rename(tmp.c_str(), path) != 0) {
        remove(tmp.c_str());
        return fail(W4_EINVAL, "%s: cannot rename %s to %s", fn, tmp.c_str(), path);
    }
    return W4_OK;
}

int w4_portable_info_read(const char* path, w4_portable_info* info) {
    const char* fn = "w4_portable_info_read";
    if (!path || !info) return fail(W4_EINVAL, "%s: path or info is NULL", fn);
    File in;
    in.f = fopen(path, "rb");
    if (!in.f) return fail(W4_EINVAL, "%s: cannot open %s", fn, path);
    uint64_t hb = 0, hash = 0;
    return read_header(fn, in.f, info, &hb, &hash);
}

int w4_portable_load(const char* path, uint8_t* packed, uint16_t* scale, uint16_t* zero, uint8_t* clip_idx) {
    const char* fn = "w4_portable_load";
    if (!path) return fail(W4_EINVAL, "%s: path is NULL", fn);
    File in;
    in.f = fopen(path, "rb");
    if (!in.f) return fail(W4_EINVAL, "%s: cannot open %s", fn, path);
    w4_portable_info info;
    uint64_t hb = 0, want = 0;
    W4_TRY(read_header(fn, in.f, &info, &hb, &want));
    if (info.N > 0 && (!packed || !scale)) return fail(W4_EINVAL, "%s: packed or scale is NULL", fn);
    if (info.N > 0 && info.mode == W4_ASYM && !zero) return fail(W4_EINVAL, "%s: zero is NULL for W4_ASYM", fn);
    if (fseek(in.f, static_cast<long>(hb), SEEK_SET) != 0) return fail(W4_EINVAL, "%s: seek failed", fn);
    std::vector<uint8_t> payload(info.payload_bytes);
    if (fread(payload.data(), 1, payload.size(), in.f) != payload.size())
        return fail(W4_EINVAL, "%s: truncated payload", fn);
    uint8_t extra;
    if (fread(&extra, 1, 1, in.f) != 0) return fail(W4_EINVAL, "%s: trailing bytes after the payload", fn);
    Fnv hash;
    hash.add(payload.data(), payload.size());
    if (hash.h != want) return fail(W4_EINVAL, "%s: payload hash mismatch (corrupted file)", fn);
    const Sections s = sections(info.N, info.K, info.G, info.mode, info.has_clip);
    const uint64_t groups = static_cast<uint64_t>(info.N) * static_cast<uint64_t>(info.K / info.G);
    if (info.N > 0) {
        memcpy(packed, payload.data() + s.packed, static_cast<size_t>(info.N) * static_cast<size_t>(info.K / 2));
        memcpy(scale, payload.data() + s.scale, 2 * groups);
        if (info.mode == W4_ASYM) memcpy(zero, payload.data() + s.zero, 2 * groups);
        if (clip_idx) {
            if (info.has_clip) memcpy(clip_idx, payload.data() + s.clip, groups);
            else memset(clip_idx, 0, groups);
        }
    }
    return W4_OK;
}

}  // extern "C"
