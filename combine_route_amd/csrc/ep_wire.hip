// gfx950 (MI355X, CDNA4) kernels of the quantized combine wire: rows in
// FP8 E4M3 with one FP32 scale per 128 elements, or MXFP4 (E2M1 codes, one
// E8M0 scale per 32 elements). The pages name these wires (fp8_blockwise;
// fp4 with e8m0 scales: "gfx1250 EPv2: ..." PR 726, "MORI-EP User Guide"
// section 10) but not their arithmetic; the conversions follow the OCP OFP8
// and MX v1.0 specifications.
//   quantize  a wave per (row, piece of up to 8 chunks of 512 elements): a
//             lane holds 8 elements of each chunk; a block's absolute maximum
//             is reduced over its 16 (FP8) or 4 (MXFP4) lanes with
//             cross-lane xors, then every element is rounded to the format in
//             registers.
//   combine   the combine's gather-fold, with each contribution taken off the
//             wire (code times scale, in FP32) before it is added; a lane
//             decodes groups of 8 elements with the hardware conversions and
//             writes each group's 16 output bytes with one store.
// Encoding is power-of-two and integer arithmetic plus the hardware
// conversions (round to nearest even), and decoding is exact, so every result
// is an exact function of its inputs; the two block-scale divisions are
// correctly rounded.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ep_device.h"
#include "ep_kernels.h"

namespace ep {
namespace {

using namespace dev;

// OCP E2M1 codes of 8 finite values times 2^e, element i in nibble i: the
// nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6 with ties to the even code,
// saturating at 6. v_cvt_scalef32_pk_fp4_f32 rounds this way (checked on
// gfx950 against every bf16 value and 2M random binary32 values, ties
// included); the power-of-two scaling is done first with ldexp, which is exact
// here, so the conversion's own scale stays 1.
__device__ __forceinline__ uint32_t e2m1x8(const float (&f)[8], int e)
{
    uint32_t q = 0;
    q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, __builtin_ldexpf(f[0], e),
                                                 __builtin_ldexpf(f[1], e), 1.0f, 0);
    q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, __builtin_ldexpf(f[2], e),
                                                 __builtin_ldexpf(f[3], e), 1.0f, 1);
    q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, __builtin_ldexpf(f[4], e),
                                                 __builtin_ldexpf(f[5], e), 1.0f, 2);
    q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, __builtin_ldexpf(f[6], e),
                                                 __builtin_ldexpf(f[7], e), 1.0f, 3);
    return q;
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

// A wave per (row, piece of up to kQuantChunks chunks of 512 elements): every
// chunk of the piece is loaded (16 bytes a lane) before the first is
// converted. Rows are addressed through per-row buffer resources: a chunk past
// the row end loads zeros and its stores are dropped, and since blocks never
// straddle the end (H is a multiple of the block) no lane needs a guard.
template <int WIRE, int DT, bool kStream>
__global__ __launch_bounds__(256) void ep_quantize_kernel(QuantizeArgs a)
{
    constexpr int ld = Policy<kStream>::combine_load;
    constexpr int st = Policy<kStream>::combine_store;
    // A chunk's scales are 16 bytes of a row's scale line, written by several
    // waves: they stay cache-allocating so the L2 merges them into whole
    // lines (streamed, they cost 10-13% of the kernel's time at 8 x 4096
    // tokens, H = 7168; streaming the codes too, or loading through the
    // caches, was slower).
    constexpr int kScaleStore = 0;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t item = (int64_t)blockIdx.x * (blockDim.x / kWave) + uniform(threadIdx.x / kWave);
    const int64_t row = item / a.pieces;
    if (row >= a.rows)
        return;  // whole waves
    if (a.counts != nullptr) {
        const int64_t g = row / a.group_rows;
        if (row - g * a.group_rows >= (int64_t)a.counts[g])
            return;  // a row past its group's count: whole waves
    }
    const int e0 = (int)(item - row * a.pieces) * a.piece_chunks * kQuantChunk + lane * 8;
    const uint32_t in_bytes = (uint32_t)a.H * 2;
    const __amdgpu_buffer_rsrc_t rin = row_rsrc(a.in + row * in_bytes, in_bytes);
    // chunks past the piece load from past the row: zeros, with no memory access
    u32x4 raw[kQuantChunks];
#pragma unroll
    for (int c = 0; c < kQuantChunks; ++c)
        raw[c] = bload16<ld>(rin, c < a.piece_chunks ? (uint32_t)(e0 + c * kQuantChunk) * 2u
                                                     : in_bytes);
    if constexpr (WIRE == kWireFp8Block128) {
        const __amdgpu_buffer_rsrc_t rout = row_rsrc(a.out + row * a.H, (uint32_t)a.H);
        const uint32_t sbytes = (uint32_t)(a.H / 128) * 4u;
        const __amdgpu_buffer_rsrc_t rsc = row_rsrc(a.scales + row * sbytes, sbytes);
#pragma unroll
        for (int c = 0; c < kQuantChunks; ++c) {
            if (c == 0 || c < a.piece_chunks) {  // the host ensures piece_chunks >= 1
                const int e = e0 + c * kQuantChunk;
                float f[8];
                widen<DT>(raw[c], f);
                float amax = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    amax = __builtin_fmaxf(amax, __builtin_fabsf(f[i]));
                amax = group_max<16>(amax);
                const float s = amax > 0.0f ? __fdiv_rn(amax, kE4M3Max) : 1.0f;
                const float r = amax > 0.0f ? __fdiv_rn(kE4M3Max, amax) : 1.0f;
                const u32x2 q = {e4m3x4(f[0] * r, f[1] * r, f[2] * r, f[3] * r),
                                 e4m3x4(f[4] * r, f[5] * r, f[6] * r, f[7] * r)};
                __builtin_amdgcn_raw_buffer_store_b64(q, rout, (uint32_t)e, 0, st);
                if ((lane & 15) == 0)
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, s), rsc,
                                                          (uint32_t)(e / 128) * 4u, 0, kScaleStore);
            }
        }
    } else {
        const __amdgpu_buffer_rsrc_t rout = row_rsrc(a.out + row * (a.H / 2), (uint32_t)a.H / 2u);
        const __amdgpu_buffer_rsrc_t rsc = row_rsrc(a.scales + row * (a.H / 32), (uint32_t)a.H / 32u);
#pragma unroll
        for (int c = 0; c < kQuantChunks; ++c) {
            if (c == 0 || c < a.piece_chunks) {  // the host ensures piece_chunks >= 1
                const int e = e0 + c * kQuantChunk;
                float f[8];
                widen<DT>(raw[c], f);
                float amax = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    amax = __builtin_fmaxf(amax, __builtin_fabsf(f[i]));
                amax = group_max<4>(amax);
                // the largest E2M1 exponent is 2: the block's largest magnitude
                // lands in [4, 8) after scaling by 2^-E
                int E = -127;
                if (amax > 0.0f)
                    E = max(__builtin_amdgcn_frexp_expf(amax) - 3, -127);
                uint32_t q = e2m1x8(f, -E);
                __builtin_amdgcn_raw_buffer_store_b32(q, rout, (uint32_t)e / 2u, 0, st);
                if ((lane & 3) == 0)
                    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(E + 127), rsc, (uint32_t)e / 32u,
                                                         0, kScaleStore);
            }
        }
    }
}

// 8-element groups a lane decodes at once per contribution row: C columns a
// wave apart (group h and h + 64), so every load and store instruction of
// the wave covers one contiguous span; a lane reads 8 * C bytes of FP8 codes
// or 4 * C bytes of MXFP4 codes a row. Measured on MI355X at 8 x 4096
// tokens, H = 7168, top-8 (FP8 / MXFP4): 330 / 214 us. Four columns: 219 us
// for MXFP4; FP8 spills. A lane owning 16 contiguous elements instead wrote
// its 32 output bytes with two stores that each cover half of every 32-byte
// sector, and the streamed halves reached HBM separately (30% more bytes
// written): 365 / 239 us.
constexpr int kWireColumnsFp8 = 2;
constexpr int kWireColumnsMxfp4 = 2;

// A wave per (token, row piece), as the combine: for each lane's groups the
// token's contribution rows are all loaded (G at a time) before any is
// decoded and added, summed in the token's rank order in FP32 from the
// first, and rounded to nearest even once.
template <int G, int C, int WIRE, int DT, bool kStream>
__global__ __launch_bounds__(1024) void ep_combine_wire_kernel(WireCombineArgs a, TokenMap tk)
{
    constexpr int GE = kGroupElems;
    constexpr int aux = Policy<kStream>::combine_load;
    const int lane = threadIdx.x & (kWave - 1);
    // wave-uniform, so the token's rank search and its output row stay scalar
    // wave items: (token, piece); piece_inner: piece fastest
    const uint32_t item = blockIdx.x * (blockDim.x / kWave) + uniform(threadIdx.x / kWave);
    const uint32_t flat_u = a.piece_inner ? item / (uint32_t)a.pieces : item;
    if (flat_u >= (uint32_t)tk.total)
        return;  // whole waves only
    const int flat = (int)flat_u;
    const int piece = a.piece_inner ? (int)(item - flat_u * (uint32_t)a.pieces) : (int)blockIdx.y;
    const int r = rank_of_token(tk, flat);
    const int64_t tok = (int64_t)r * a.M + (flat - tk.tok_start[r]);
    const int32_t gl = lane < a.P ? a.fwd[tok * a.P + lane] : -1;
    const int n = __popcll(__ballot(gl >= 0));  // entries >= 0 form a prefix

    const uint32_t out_bytes = (uint32_t)a.units * 32u;  // 16 elements of 2 bytes a unit
    const __amdgpu_buffer_rsrc_t rdst = row_rsrc(a.out + tok * out_bytes, out_bytes);
    // the piece's 8-element groups; a scale dword covers 16 of them (128
    // elements), and pieces start on a dword
    const int hbeg = piece * a.piece_units * 2;
    const int hend = min(a.units, (piece + 1) * a.piece_units) * 2;
    // Scale rows are read once: lane l holds dword hbeg / 16 + l of each
    // contribution row of the current group of G, and a code group takes its
    // row's scale from lane (h - hbeg) / 16. A token of at most G rows loads
    // them once; larger ones reload them for every group of rows. Reading the
    // scale on every pass over the row fetched each scale line 7 times at
    // H = 7168.
    uint32_t spre[G];
    auto load_scales = [&](int i0) {
#pragma unroll
        for (int q = 0; q < G; ++q) {
            if (i0 + q < n) {
                const int64_t gq = __builtin_amdgcn_readlane(gl, i0 + q);
                const __amdgpu_buffer_rsrc_t rs = row_rsrc(a.ys + gq * a.scale_bytes, a.scale_bytes);
                const uint32_t off = (uint32_t)(hbeg / 16 + lane) * 4u;
                if (WIRE == kWireFp8Block128 || a.scale_bytes % 4 == 0) {
                    spre[q] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, aux);
                } else {  // MXFP4 scale rows that are not whole dwords: by bytes
                    uint32_t d = 0;
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        d |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rs, off + b, 0, aux)
                             << (8 * b);
                    spre[q] = d;
                }
            }
        }
    };
    const bool regroup = n > G;  // uniform
    if (!regroup)
        load_scales(0);
    for (int h0 = hbeg + lane; h0 - lane < hend; h0 += kWave * C) {
        float acc[C][GE];
        for (int i0 = 0; i0 < n; i0 += G) {
            if (regroup)
                load_scales(i0);
            // MXFP4: every load is issued, in the order the fold takes them,
            // so a row's fold waits for that row only (a row past the token's
            // last has an empty resource and a group past the piece an offset
            // at the row's end: both read zeros without touching memory).
            // FP8 issues only the token's loads and waits for all of them: its
            // 8-byte loads of empty rows cost more than the waits save (at 8 x
            // 4096 tokens, H = 7168, top-8: MXFP4 204 -> 200 us, FP8 288 ->
            // 304 us with every load issued).
            u32x2 raw[G][C];
            if constexpr (WIRE == kWireMxfp4) {
#pragma unroll
                for (int q = 0; q < G; ++q) {
                    const bool in = i0 + q < n;  // uniform
                    const int64_t gq = in ? __builtin_amdgcn_readlane(gl, i0 + q) : 0;
                    const __amdgpu_buffer_rsrc_t ry =
                        row_rsrc(a.y + gq * a.row_bytes, in ? a.row_bytes : 0u);
#pragma unroll
                    for (int c = 0; c < C; ++c) {
                        const int h = h0 + c * kWave;
                        const uint32_t off = h < hend ? (uint32_t)h * 4u : a.row_bytes;
                        raw[q][c] = {__builtin_amdgcn_raw_buffer_load_b32(ry, off, 0, aux), 0u};
                    }
                }
            } else {
#pragma unroll
                for (int q = 0; q < G; ++q) {
#pragma unroll
                    for (int c = 0; c < C; ++c) {
                        const int h = h0 + c * kWave;
                        if (i0 + q < n && h < hend) {
                            const int64_t gq = __builtin_amdgcn_readlane(gl, i0 + q);
                            const __amdgpu_buffer_rsrc_t ry =
                                row_rsrc(a.y + gq * a.row_bytes, a.row_bytes);
                            raw[q][c] = __builtin_amdgcn_raw_buffer_load_b64(ry, h * 8, 0, aux);
                        }
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < G; ++q) {
                if (i0 + q < n) {  // uniform: every lane takes part in the cross-lane reads
#pragma unroll
                    for (int c = 0; c < C; ++c) {
                        const int h = h0 + c * kWave;
                        const uint32_t d = (uint32_t)__shfl((int)spre[q], (h - hbeg) >> 4);
                        // MXFP4: byte (h / 4) mod 4 of the dword
                        const uint32_t sb = WIRE == kWireFp8Block128 ? d : d >> (8 * ((h >> 2) & 3));
                        float f[GE];
                        decode_group<WIRE>(raw[q][c], sb, f);
#pragma unroll
                        for (int e = 0; e < GE; ++e)
                            acc[c][e] = (i0 + q == 0) ? f[e] : acc[c][e] + f[e];
                    }
                }
            }
        }
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int h = h0 + c * kWave;
            if (h < hend) {
                if (n == 0) {
#pragma unroll
                    for (int e = 0; e < GE; ++e)
                        acc[c][e] = 0.0f;
                }
                bstore16<Policy<kStream>::combine_store>(narrow<DT>(acc[c]), rdst,
                                                         (uint32_t)h * 16u);
            }
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
    constexpr int U = WIRE == kWireFp8Block128 ? kWireColumnsFp8 : kWireColumnsMxfp4;
    if (dtype == 0) {
        if (stream)
            hipLaunchKernelGGL((ep_combine_wire_kernel<G, U, WIRE, 0, true>), grid, block, 0, s, a,
                               tk);
        else
            hipLaunchKernelGGL((ep_combine_wire_kernel<G, U, WIRE, 0, false>), grid, block, 0, s,
                               a, tk);
    } else {
        if (stream)
            hipLaunchKernelGGL((ep_combine_wire_kernel<G, U, WIRE, 1, true>), grid, block, 0, s, a,
                               tk);
        else
            hipLaunchKernelGGL((ep_combine_wire_kernel<G, U, WIRE, 1, false>), grid, block, 0, s,
                               a, tk);
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

template <int WIRE, int DT>
void quantize_with(const QuantizeArgs& a, dim3 grid, dim3 block, bool stream, hipStream_t s)
{
    if (stream)
        hipLaunchKernelGGL((ep_quantize_kernel<WIRE, DT, true>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((ep_quantize_kernel<WIRE, DT, false>), grid, block, 0, s, a);
}

}  // namespace

hipError_t launch_quantize(const QuantizeArgs& a, int wire, int dtype, bool stream, hipStream_t s)
{
    if (a.rows == 0)
        return hipSuccess;
    if (a.piece_chunks < 1 || a.piece_chunks > kQuantChunks ||
        (int64_t)a.pieces * a.piece_chunks * kQuantChunk < a.H)
        return hipErrorInvalidValue;
    const int64_t items = a.rows * a.pieces;
    const dim3 grid((unsigned)((items + 3) / 4));
    const dim3 block(4 * kWave);
    if (wire == kWireFp8Block128) {
        if (dtype == 0)
            quantize_with<kWireFp8Block128, 0>(a, grid, block, stream, s);
        else
            quantize_with<kWireFp8Block128, 1>(a, grid, block, stream, s);
    } else {
        if (dtype == 0)
            quantize_with<kWireMxfp4, 0>(a, grid, block, stream, s);
        else
            quantize_with<kWireMxfp4, 1>(a, grid, block, stream, s);
    }
    return hipGetLastError();
}

hipError_t launch_combine_wire(const WireCombineArgs& a, const TokenMap& tk, int wire, int dtype,
                               int waves, bool stream, hipStream_t s)
{
    if (tk.total == 0)
        return hipSuccess;
    const dim3 grid = a.piece_inner
                          ? dim3((unsigned)(((int64_t)tk.total * a.pieces + waves - 1) / waves))
                          : dim3((unsigned)((tk.total + waves - 1) / waves), (unsigned)a.pieces);
    const dim3 block(waves * kWave);
    if (wire == kWireFp8Block128)
        return combine_wire_fmt<kWireFp8Block128>(a, tk, dtype, grid, block, stream, s);
    return combine_wire_fmt<kWireMxfp4>(a, tk, dtype, grid, block, stream, s);
}

}  // namespace ep
