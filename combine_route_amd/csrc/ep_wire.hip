// gfx950 (MI355X, CDNA4) kernels of the quantized combine wire: rows in
// FP8 E4M3 with one FP32 scale per 128 elements, or MXFP4 (E2M1 codes, one
// E8M0 scale per 32 elements). The pages name these wires (fp8_blockwise;
// fp4 with e8m0 scales: "gfx1250 EPv2: ..." PR 726, "MORI-EP User Guide"
// section 10) but not their arithmetic; the conversions follow the OCP OFP8
// and MX v1.0 specifications.
//   quantize  a wave per (row, 512-element chunk): a lane holds 8 elements;
//             a block's absolute maximum is reduced over its 16 (FP8) or 4
//             (MXFP4) lanes with cross-lane xors, then every element is
//             rounded to the format in registers.
//   combine   the combine's gather-fold, with each contribution taken off the
//             wire (code times scale, in FP32) before it is added.
// All conversions are integer and power-of-two arithmetic plus rint (round
// to nearest even), so they are exact functions of their inputs; the two
// block-scale divisions are correctly rounded.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ep_device.h"
#include "ep_kernels.h"

namespace ep {
namespace {

using namespace dev;

__device__ __forceinline__ float from_e4m3(uint32_t c)
{
    const uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
    float v = e == 0 ? (float)m * 0x1p-9f : __builtin_ldexpf((float)(8u + m), (int)e - 10);
    if (e == 15 && m == 7)
        v = __builtin_nanf("");
    return (c & 0x80u) ? -v : v;
}

// OCP E2M1 code (4 bits) of a finite value: nearest of 0, 0.5, 1, 1.5, 2, 3,
// 4, 6, ties to the even code, saturating at 6.
__device__ __forceinline__ uint32_t to_e2m1(float v)
{
    const uint32_t sign = (__builtin_bit_cast(uint32_t, v) >> 28) & 0x8u;
    const float a = __builtin_fabsf(v);
    uint32_t c;
    if (a >= 6.0f)
        c = 7;
    else if (a < 2.0f)
        c = (uint32_t)__builtin_rintf(a * 2.0f);         // 0, 0.5, 1, 1.5, 2
    else if (a < 4.0f)
        c = (uint32_t)__builtin_rintf(a) + 2;            // 2, 3, 4
    else
        c = (uint32_t)__builtin_rintf(a * 0.5f) + 4;     // 4, 6
    return sign | c;
}

__device__ __forceinline__ float from_e2m1(uint32_t c)
{
    const uint32_t e = (c >> 1) & 3u, m = c & 1u;
    const float v = e == 0 ? 0.5f * (float)m : __builtin_ldexpf(1.0f + 0.5f * (float)m, (int)e - 1);
    return (c & 8u) ? -v : v;
}

// Maximum over groups of G consecutive lanes (G a power of two <= 16).
template <int G>
__device__ __forceinline__ float group_max(float v)
{
#pragma unroll
    for (int off = 1; off < G; off <<= 1)
        v = __builtin_fmaxf(v, __shfl_xor(v, off));
    return v;
}

template <int WIRE, int DT>
__global__ __launch_bounds__(256) void ep_quantize_kernel(QuantizeArgs a)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t item = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    const int chunks = (a.H + 511) / 512;
    const int64_t row = item / chunks;
    if (row >= a.rows)
        return;  // whole waves
    const int h0 = (int)(item - row * chunks) * 512 + lane * 8;  // this lane's 8 elements
    const bool valid = h0 < a.H;  // blocks lie wholly inside or outside the row
    float f[8] = {};
    if (valid) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(a.in + (row * a.H + h0) * 2);
        widen<DT>(w, f);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        amax = __builtin_fmaxf(amax, __builtin_fabsf(f[i]));
    if constexpr (WIRE == kWireFp8Block128) {
        amax = group_max<16>(amax);
        const float s = amax > 0.0f ? __fdiv_rn(amax, kE4M3Max) : 1.0f;
        const float r = amax > 0.0f ? __fdiv_rn(kE4M3Max, amax) : 1.0f;
        if (!valid)
            return;
        u32x2 out = {0u, 0u};
#pragma unroll
        for (int i = 0; i < 8; ++i)
            out[i / 4] |= to_e4m3(f[i] * r) << (8 * (i % 4));
        *reinterpret_cast<u32x2*>(a.out + row * a.H + h0) = out;
        if ((lane & 15) == 0)
            reinterpret_cast<float*>(a.scales)[row * (a.H / 128) + h0 / 128] = s;
    } else {
        amax = group_max<4>(amax);
        // the largest E2M1 exponent is 2: the block's largest magnitude lands
        // in [4, 8) after scaling by 2^-E
        int E = -127;
        if (amax > 0.0f)
            E = max(__builtin_amdgcn_frexp_expf(amax) - 3, -127);
        if (!valid)
            return;
        uint32_t out = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            out |= to_e2m1(__builtin_ldexpf(f[i], -E)) << (4 * i);
        *reinterpret_cast<uint32_t*>(a.out + row * (a.H / 2) + h0 / 2) = out;
        if ((lane & 3) == 0)
            a.scales[row * (a.H / 32) + h0 / 32] = (uint8_t)(E + 127);
    }
}

// The 8 elements of one 16-byte output column of a wire row, in FP32.
template <int WIRE, bool kStream>
__device__ __forceinline__ void wire_column(__amdgpu_buffer_rsrc_t ry, __amdgpu_buffer_rsrc_t rs,
                                            int col, float (&f)[8])
{
    constexpr int aux = Policy<kStream>::combine_load;
    if constexpr (WIRE == kWireFp8Block128) {
        const u32x2 c = __builtin_amdgcn_raw_buffer_load_b64(ry, col * 8, 0, aux);
        const float s = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(rs, (col / 16) * 4, 0, aux));
#pragma unroll
        for (int i = 0; i < 8; ++i)
            f[i] = from_e4m3((c[i / 4] >> (8 * (i % 4))) & 0xFFu) * s;
    } else {
        const uint32_t c = __builtin_amdgcn_raw_buffer_load_b32(ry, col * 4, 0, aux);
        const int E = (int)__builtin_amdgcn_raw_buffer_load_b8(rs, col / 4, 0, aux) - 127;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            f[i] = __builtin_ldexpf(from_e2m1((c >> (4 * i)) & 0xFu), E);
    }
}

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

// A wave per (token, row piece), as the combine: the token's contribution
// rows come off the wire column by column (G rows loaded before any is
// added), are summed in the token's rank order in FP32 from the first, and
// rounded to nearest even once.
template <int G, int WIRE, int DT, bool kStream>
__global__ __launch_bounds__(1024) void ep_combine_wire_kernel(WireCombineArgs a, TokenMap tk)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int flat = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (flat >= tk.total)
        return;  // whole waves only
    const int piece = blockIdx.y;
    const int r = rank_of_token(tk, flat);
    const int64_t tok = (int64_t)r * a.M + (flat - tk.tok_start[r]);
    const int32_t gl = lane < a.P ? a.fwd[tok * a.P + lane] : -1;
    const int n = __popcll(__ballot(gl >= 0));  // entries >= 0 form a prefix

    const uint32_t out_bytes = (uint32_t)a.cols * 16u;
    const __amdgpu_buffer_rsrc_t rdst = row_rsrc(a.out + tok * out_bytes, out_bytes);
    const int cbeg = piece * a.piece_cols;
    const int cend = min(a.cols, cbeg + a.piece_cols);
    for (int col = cbeg + lane; col - lane < cend; col += kWave) {
        const bool live = col < cend;
        float acc[8];
        for (int i0 = 0; i0 < n; i0 += G) {
            float v[G][8];
#pragma unroll
            for (int q = 0; q < G; ++q) {
                if (i0 + q < n && live) {
                    const int64_t gq = __builtin_amdgcn_readlane(gl, i0 + q);
                    wire_column<WIRE, kStream>(
                        row_rsrc(a.y + gq * a.row_bytes, a.row_bytes),
                        row_rsrc(a.ys + gq * a.scale_bytes, a.scale_bytes), col, v[q]);
                }
            }
#pragma unroll
            for (int q = 0; q < G; ++q) {
                if (i0 + q < n) {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        acc[e] = (i0 + q == 0) ? v[q][e] : acc[e] + v[q][e];
                }
            }
        }
        if (live) {
            if (n == 0) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    acc[e] = 0.0f;
            }
            bstore16<Policy<kStream>::combine_store>(narrow<DT>(acc), rdst, (uint32_t)col * 16u);
        }
    }

    if (piece == 0 && a.yw != nullptr && lane < a.k) {
        float acc = 0.0f;
        for (int i = 0; i < n; ++i) {
            const int64_t gi = __builtin_amdgcn_readlane(gl, i);
            const float v = a.yw[gi * a.k + lane];
            acc = (i == 0) ? v : acc + v;
        }
        a.out_w[tok * a.k + lane] = acc;
    }
}

template <int G, int WIRE>
hipError_t combine_wire_with(const WireCombineArgs& a, const TokenMap& tk, int dtype, dim3 grid,
                             dim3 block, bool stream, hipStream_t s)
{
    if (dtype == 0) {
        if (stream)
            hipLaunchKernelGGL((ep_combine_wire_kernel<G, WIRE, 0, true>), grid, block, 0, s, a, tk);
        else
            hipLaunchKernelGGL((ep_combine_wire_kernel<G, WIRE, 0, false>), grid, block, 0, s, a,
                               tk);
    } else {
        if (stream)
            hipLaunchKernelGGL((ep_combine_wire_kernel<G, WIRE, 1, true>), grid, block, 0, s, a, tk);
        else
            hipLaunchKernelGGL((ep_combine_wire_kernel<G, WIRE, 1, false>), grid, block, 0, s, a,
                               tk);
    }
    return hipGetLastError();
}

template <int WIRE>
hipError_t combine_wire_fmt(const WireCombineArgs& a, const TokenMap& tk, int dtype, dim3 grid,
                            dim3 block, bool stream, hipStream_t s)
{
    if (a.P <= 1)
        return combine_wire_with<1, WIRE>(a, tk, dtype, grid, block, stream, s);
    if (a.P <= 2)
        return combine_wire_with<2, WIRE>(a, tk, dtype, grid, block, stream, s);
    if (a.P <= 4)
        return combine_wire_with<4, WIRE>(a, tk, dtype, grid, block, stream, s);
    return combine_wire_with<kCombineGroup, WIRE>(a, tk, dtype, grid, block, stream, s);
}

}  // namespace

hipError_t launch_quantize(const QuantizeArgs& a, int wire, int dtype, hipStream_t s)
{
    if (a.rows == 0)
        return hipSuccess;
    const int64_t items = a.rows * ((a.H + 511) / 512);
    const dim3 grid((unsigned)((items + 3) / 4));
    const dim3 block(4 * kWave);
    if (wire == kWireFp8Block128) {
        if (dtype == 0)
            hipLaunchKernelGGL((ep_quantize_kernel<kWireFp8Block128, 0>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((ep_quantize_kernel<kWireFp8Block128, 1>), grid, block, 0, s, a);
    } else {
        if (dtype == 0)
            hipLaunchKernelGGL((ep_quantize_kernel<kWireMxfp4, 0>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((ep_quantize_kernel<kWireMxfp4, 1>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_combine_wire(const WireCombineArgs& a, const TokenMap& tk, int wire, int dtype,
                               int waves, int row_split, bool stream, hipStream_t s)
{
    if (tk.total == 0)
        return hipSuccess;
    const dim3 grid((tk.total + waves - 1) / waves, row_split);
    const dim3 block(waves * kWave);
    if (wire == kWireFp8Block128)
        return combine_wire_fmt<kWireFp8Block128>(a, tk, dtype, grid, block, stream, s);
    return combine_wire_fmt<kWireMxfp4>(a, tk, dtype, grid, block, stream, s);
}

}  // namespace ep
