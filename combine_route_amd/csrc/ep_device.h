// Device helpers shared by the gfx950 kernels: row moves through per-row
// buffer resources, wave-level bit counting, and the ordered FP32 fold with
// its round-to-nearest-even cast.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ep_kernels.h"

namespace ep {
namespace dev {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Cache policy of the row moves, as gfx950 buffer-instruction bits (1 = sc0,
// 2 = nt, 16 = sc1). Streaming calls (footprint well past the 256 MB MALL)
// touch every payload row once, so loads stream past the caches (nt); the
// combine's stores stream too; the copies' stores do not. Measured on MI355X
// at 8 ranks x 4096 tokens x 7168 bf16: nt stores in the dispatch copy cost it
// ~40 us a call, plain stores in the combine leave dirty lines that the next
// dispatch pays ~40 us to write back, and cached combine loads cost ~70 us.
// The copies that cast to E4M3 on the way (8-byte stores a lane) stream
// their stores: 340 -> 335 us (ep_dispatch) and 487 -> 479 us
// (ep_dispatch_standard_moe) at that shape.
// Calls that fit in the MALL use plain (cache-allocating) moves: rows an
// expert has just written are still there, and 8 ranks x 128 fp8 tokens runs
// ~10% faster that way.
template <bool kStream>
struct Policy {
    static constexpr int copy_load = kStream ? 2 : 0;
    static constexpr int copy_store = 0;
    static constexpr int cast_store = kStream ? 2 : 0;
    static constexpr int combine_load = kStream ? 2 : 0;
    static constexpr int combine_store = kStream ? 2 : 0;
};

// A combine loads up to kCombineGroup contribution rows, kCombineColumns
// 16-byte columns each, before folding (8 x 2 measured best: smaller groups
// split a top-8 token's rows into two dependent rounds, larger column counts
// cost occupancy).
constexpr int kCombineGroup = 8;
constexpr int kCombineColumns = 2;

// Number of lanes below this one whose bit is set in b.
__device__ __forceinline__ int lanes_below(uint64_t b)
{
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
}

// A value every lane of the wave holds identically, moved to a scalar register.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// A buffer resource covering one row: every access through it is range-checked
// by the hardware against the row's bytes (an out-of-range load reads zero, an
// out-of-range store is dropped), so a row move cannot spill into its
// neighbour. Word 3 is the raw (untyped) buffer format.
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}

template <int AUX>
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, AUX);
}

template <int AUX>
__device__ __forceinline__ void bstore16(u32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t off)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, AUX);
}

template <int DT>
__device__ __forceinline__ void widen(const u32x4& w, float (&f)[8])
{
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if constexpr (DT == 0) {  // bf16: the upper half of a binary32
            f[2 * q] = __builtin_bit_cast(float, w[q] << 16);
            f[2 * q + 1] = __builtin_bit_cast(float, w[q] & 0xFFFF0000u);
        } else {                  // fp16: exact hardware widening
            f[2 * q] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[q] & 0xFFFFu));
            f[2 * q + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[q] >> 16));
        }
    }
}

template <int DT>
__device__ __forceinline__ u32x4 narrow(const float (&f)[8])
{
    u32x4 w;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if constexpr (DT == 0) {  // v_cvt_pk_bf16_f32: round to nearest even
            const f32x2 p = {f[2 * q], f[2 * q + 1]};
            w[q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2));
        } else {                  // v_cvt_f16_f32: round to nearest even
            const uint32_t lo = __builtin_bit_cast(uint16_t, (_Float16)f[2 * q]);
            const uint32_t hi = __builtin_bit_cast(uint16_t, (_Float16)f[2 * q + 1]);
            w[q] = lo | (hi << 16);
        }
    }
    return w;
}

// x rounded to the combine type (nearest even) and read back as FP32, in one
// conversion an element for bf16: v_cvt_pk_bf16_f32 of the pair (0, x) puts
// bf16(x) in the high half over a zero low half, which is bf16(x)'s value as
// a binary32 exactly. fp16 converts there and back.
template <int DT>
__device__ __forceinline__ float round_to(float x)
{
    if constexpr (DT == 0) {
        const f32x2 p = {0.0f, x};
        return __builtin_bit_cast(float, __builtin_convertvector(p, bf16x2));
    } else {
        return (float)(_Float16)x;
    }
}

constexpr float kE4M3Max = 448.0f;

// OCP E4M3 codes (the OFP8 specification: bias 7, no infinities, largest
// finite 448) of 4 FP32 values, one a byte in order: round to nearest even,
// saturating past 448, NaN -> 0x7F. v_cvt_pk_fp8_f32 rounds to nearest even
// but turns overflow into NaN, so values are clamped to +-448 first (NaN kept
// apart, since min/max would drop it); it writes NaN as 0xFF, which no finite
// value can produce, and those bytes become 0x7F. Checked against the
// definition on every bf16 and fp16 value.
__device__ __forceinline__ uint32_t e4m3x4(float f0, float f1, float f2, float f3)
{
    auto clamp = [](float v) {
        return v != v ? v : __builtin_fminf(__builtin_fmaxf(v, -kE4M3Max), kE4M3Max);
    };
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp(f0), clamp(f1), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp(f2), clamp(f3), w, true);
    const uint32_t x = (uint32_t)w;
    // bytes equal to 0xFF: their complement is zero; clear bit 7 of each
    const uint32_t t = ~x;
    const uint32_t ff = ~(((t & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | t) & 0x80808080u;
    return x ^ ff;
}

// 8 bf16 (cast 1) or fp16 (cast 2) elements -> 8 E4M3 codes.
__device__ __forceinline__ u32x2 cast_e4m3(const u32x4& w, int cast)
{
    float f[8];
    if (cast == 2)
        widen<1>(w, f);
    else
        widen<0>(w, f);
    return {e4m3x4(f[0], f[1], f[2], f[3]), e4m3x4(f[4], f[5], f[6], f[7])};
}

// One wave folds the n contribution rows whose row numbers (in units of
// row_bytes from src) are held by lanes 0..n-1 of gl, over the 16-byte
// columns [vbeg, vend) of the output row rdst: for each column every
// contribution is loaded before any is added (G rows x U columns a lane in
// flight), then they are summed in lane order in FP32 starting from the
// first, and the sum is rounded to nearest even once. n = 0 stores +0.
// kWeighted: contribution i is scaled by lane i's gw, the first as a product
// and the rest with one fused multiply-add each.
template <int G, int U, int DT, bool kStream, bool kWeighted = false>
__device__ __forceinline__ void fold_rows(const uint8_t* src, uint32_t row_bytes, int32_t gl,
                                          int n, __amdgpu_buffer_rsrc_t rdst, int vbeg, int vend,
                                          int lane, float gw = 0.0f)
{
    for (int v0 = vbeg; v0 < vend; v0 += kWave * U) {
        float acc[U][8];
        for (int i0 = 0; i0 < n; i0 += G) {
            u32x4 rows[U][G];
#pragma unroll
            for (int q = 0; q < G; ++q) {
                if (i0 + q < n) {
                    const int64_t gq = __builtin_amdgcn_readlane(gl, i0 + q);
                    const __amdgpu_buffer_rsrc_t ry = row_rsrc(src + gq * row_bytes, row_bytes);
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int v = v0 + u * kWave + lane;
                        if (v < vend)
                            rows[u][q] = bload16<Policy<kStream>::combine_load>(
                                ry, (uint32_t)v * 16u);
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < G; ++q) {
                if (i0 + q < n) {
                    float c = 1.0f;
                    if constexpr (kWeighted)
                        c = __builtin_bit_cast(
                            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gw), i0 + q));
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        float f[8];
                        widen<DT>(rows[u][q], f);
                        if (i0 + q == 0) {
#pragma unroll
                            for (int e = 0; e < 8; ++e)
                                acc[u][e] = kWeighted ? c * f[e] : f[e];
                        } else {
#pragma unroll
                            for (int e = 0; e < 8; ++e)
                                acc[u][e] = kWeighted ? __builtin_fmaf(c, f[e], acc[u][e])
                                                      : acc[u][e] + f[e];
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = v0 + u * kWave + lane;
            if (v < vend) {
                if (n == 0) {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        acc[u][e] = 0.0f;
                }
                bstore16<Policy<kStream>::combine_store>(narrow<DT>(acc[u]), rdst,
                                                         (uint32_t)v * 16u);
            }
        }
    }
}

// The same fold, row by row: the wave's piece [vbeg, vend) holds at most
// kWave * R columns, all R of a lane's columns of a row are loaded together,
// and D rows are in flight (the loads of rows i+1 .. i+D-1 are issued before
// row i is added). Same additions in the same order, so the same bits as
// fold_rows. Fewer registers than fold_rows (more waves a SIMD), and a
// token's pieces, run by neighbouring waves, read each contribution row
// whole at about the same time. Two rows in flight: at 8 x 4096 tokens,
// H = 7168, top-8, the combine takes the same time with 2 or 3 (4: +1%) and
// the expert-major inverse, 8 rows a token, 1126 us with 2, 1180 with 3,
// 1260 with 4 and 1503 with 6.
constexpr int kStreamDepth = 2;

template <int R, int DT, bool kStream, bool kWeighted = false>
__device__ __forceinline__ void fold_rows_streamed(const uint8_t* src, uint32_t row_bytes,
                                                   int32_t gl, int n,
                                                   __amdgpu_buffer_rsrc_t rdst, int vbeg,
                                                   int vend, int lane, float gw = 0.0f)
{
    constexpr int D = kStreamDepth;
    float acc[R][8];
    u32x4 buf[D][R];
    // Every load is issued, so that the compiler can wait for one row at a
    // time (with a load skipped on some paths it waits for all of them, and
    // only one row is in flight): a row past the last (i >= n) has an empty
    // resource and a column past the piece an offset at the row's end, and
    // both read zeros without touching memory.
    auto load = [&](int i, u32x4 (&b)[R]) {
        const bool in = i < n;  // uniform
        const int64_t gi = in ? __builtin_amdgcn_readlane(gl, i & (kWave - 1)) : 0;
        const __amdgpu_buffer_rsrc_t ry = row_rsrc(src + gi * row_bytes, in ? row_bytes : 0u);
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const int v = vbeg + u * kWave + lane;
            const uint32_t off = v < vend ? (uint32_t)v * 16u : row_bytes;
            b[u] = bload16<Policy<kStream>::combine_load>(ry, off);
        }
    };
    // row i lives in buf[i % D]; the loop runs D rows a pass so that every
    // buffer index is a constant
#pragma unroll
    for (int j = 0; j < D - 1; ++j)
        load(j, buf[j]);
    for (int i0 = 0; i0 < n; i0 += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            const int i = i0 + j;
            load(i + D - 1, buf[(j + D - 1) % D]);
            if (i < n) {
                float c = 1.0f;
                if constexpr (kWeighted)
                    c = __builtin_bit_cast(
                        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gw), i));
#pragma unroll
                for (int u = 0; u < R; ++u) {
                    float f[8];
                    widen<DT>(buf[j][u], f);
                    if (i == 0) {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            acc[u][e] = kWeighted ? c * f[e] : f[e];
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            acc[u][e] = kWeighted ? __builtin_fmaf(c, f[e], acc[u][e])
                                                  : acc[u][e] + f[e];
                    }
                }
            }
        }
    }
#pragma unroll
    for (int u = 0; u < R; ++u) {
        const int v = vbeg + u * kWave + lane;
        if (v < vend) {
            if (n == 0) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    acc[u][e] = 0.0f;
            }
            bstore16<Policy<kStream>::combine_store>(narrow<DT>(acc[u]), rdst, (uint32_t)v * 16u);
        }
    }
}

// A lane decodes groups of 8 elements, inside one scale block: 8 bytes of
// FP8 codes (two dwords) or 4 bytes of MXFP4 codes (one dword). Its 8 results
// are one 16-byte store, so a wave's store covers 1 KiB contiguously.
constexpr int kGroupElems = 8;

// Decode one group into FP32 with the hardware conversions, which are exact:
// an E4M3 code to FP32 (v_cvt_pk_f32_fp8), then one FP32 multiply by the
// block scale; an E2M1 code times the power-of-two scale (v_cvt_scalef32_pk_
// f32_fp4). Code order follows the row: byte i of dword d holds FP8 element
// 4d + i; the low nibble of byte b holds MXFP4 element 2b.
template <int WIRE>
__device__ __forceinline__ void decode_group(const u32x2& c, uint32_t sbits,
                                             float (&f)[kGroupElems])
{
    if constexpr (WIRE == kWireFp8Block128) {
        const float s = __builtin_bit_cast(float, sbits);
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(c[d], false);
            const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(c[d], true);
            f[4 * d + 0] = lo.x * s;
            f[4 * d + 1] = lo.y * s;
            f[4 * d + 2] = hi.x * s;
            f[4 * d + 3] = hi.y * s;
        }
    } else {
        // 2^(code - 127) as 2^-127 (a subnormal) scaled by 2^code: one
        // exact ldexp, no bias subtraction
        const float s = __builtin_ldexpf(0x1p-127f, (int)(sbits & 0xFFu));
        const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[0], s, 0);
        const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[0], s, 1);
        const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[0], s, 2);
        const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[0], s, 3);
        f[0] = v0.x;
        f[1] = v0.y;
        f[2] = v1.x;
        f[3] = v1.y;
        f[4] = v2.x;
        f[5] = v2.y;
        f[6] = v3.x;
        f[7] = v3.y;
    }
}

// Source rank of flat token `flat` (tokens of all ranks in rank order): a
// binary search over the ranks' first flat tokens.
__device__ __forceinline__ int rank_of_token(const TokenMap& tk, int flat)
{
    int lo = 0, hi = tk.W - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tk.tok_start[mid] <= flat)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// Ids of a row are read KC at a time (KC = min(KB, 16), so registers stay
// bounded at any top-k): chunk c holds slots [c * KC, c * KC + KC), loaded at
// addresses clamped into the row so every load issues before any is used;
// slots past k are loaded but ignored.
template <int KB>
constexpr int id_chunk() { return KB < 16 ? KB : 16; }

// In-tile positions of a tile's (row, expert) pairs, one wave, lane = row.
// The lane's n distinct experts are list[0..n) (indices in [0, count)); its
// positions go to pos[0..n). For a window of 64 * kWords experts at a time,
// each lane ORs its bit into the 64-bit LDS mask of each of its experts (OR
// does not depend on the order the lanes arrive in, so the positions are
// deterministic) and a pair's position is its expert's tile base plus the
// mask's bits below the lane. first[w] holds the tile base of expert
// 64w + lane of the first window (loaded early by the caller), base_at(e)
// loads expert e's; s_bal and s_base hold 64 * kWords entries.
template <int kWords, typename BaseAt>
__device__ __forceinline__ void tile_positions(const int32_t* list, int32_t* pos, int n, int count,
                                               const int (&first)[kWords], BaseAt base_at,
                                               uint64_t* s_bal, int32_t* s_base)
{
    constexpr int kWin = kWords * kWave;
    const int lane = threadIdx.x & (kWave - 1);
    for (int e0 = 0; e0 < count; e0 += kWin) {
#pragma unroll
        for (int w = 0; w < kWords; ++w) {
            const int j = 64 * w + lane;
            s_bal[j] = 0;
            s_base[j] = e0 == 0 ? first[w] : e0 + j < count ? base_at(e0 + j) : 0;
        }
        __builtin_amdgcn_wave_barrier();
        for (int u = 0; u < n; ++u) {
            const int j = list[u] - e0;
            if (j >= 0 && j < kWin)
                __hip_atomic_fetch_or(&s_bal[j], 1ull << lane, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        __builtin_amdgcn_wave_barrier();
        for (int u = 0; u < n; ++u) {
            const int j = list[u] - e0;
            if (j >= 0 && j < kWin)
                pos[u] = s_base[j] + lanes_below(s_bal[j]);
        }
        __builtin_amdgcn_wave_barrier();
    }
}

template <int KC>
__device__ __forceinline__ void load_ids(const int32_t* row, int k, int c, int32_t (&ids)[KC])
{
#pragma unroll
    for (int i = 0; i < KC; ++i)
        ids[i] = row[min(c * KC + i, k - 1)];
}

// Word w of a row's set of local experts: bit b for local expert 64w + b.
// An id is local when it lies in [lo, lo + Er).
template <int KC>
__device__ __forceinline__ uint64_t local_word(const int32_t* row, int k, bool valid, int64_t lo,
                                               int Er, int w)
{
    uint64_t m = 0;
    for (int c = 0; c * KC < k; ++c) {
        int32_t ids[KC];
        load_ids<KC>(row, k, c, ids);
#pragma unroll
        for (int i = 0; i < KC; ++i) {
            const int64_t j = (int64_t)ids[i] - lo;
            const int64_t b = j - 64 * w;
            if (valid && c * KC + i < k && j >= 0 && j < Er && b >= 0 && b < 64)
                m |= 1ull << b;
        }
    }
    return m;
}

}  // namespace dev
}  // namespace ep
