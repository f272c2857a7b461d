// gfx950 (MI355X, CDNA4) kernels of the fused expert-major path ("MORI-EP
// User Guide", section 4 "Standard MoE Compatibility (DeepEP)":
// dispatch_standard_moe, dispatch and layout conversion in one call;
// combine_standard_moe, the combine from the expert-major layout).
//
// The fused dispatch gives every (token, distinct expert) pair the packed row
// that convert_dispatch_output gives it after a dispatch: an expert's list
// keeps the receive order, which is source rank, then source token. Here the
// lists are counting-sorted straight over the source tokens, with the same
// deterministic scheme: per expert, the count of a tile of 64 tokens of one
// source rank, an exclusive scan over (source rank, tile), and the prefix
// inside a tile (the tile's tokens naming the expert below the token). A
// source rank starts a new tile, so a layout range is read off the tile bases.
//   count    a wave per (source rank, tile, 64 experts): one ballot per
//            expert gives how many of the tile's tokens name it.
//   scan     a wave per expert: tile bases, the expert's row count, and its
//            layout range for every source rank. Calls of at most 16 tiles
//            (top-16 or fewer) count and scan in one launch, a block per
//            expert.
//   copy     a block per (source rank, tile, row piece, share of the tile's
//            tokens): wave 0 works out the kept packed row of every (token,
//            expert) pair of the tile into LDS; then every wave loads a token
//            of the block's share once per row piece (16 B a lane) and stores
//            it to each kept packed row; piece-0 blocks also write the per-slot
//            map the combine reads, the scale rows and the source info of
//            their share. Small calls share a tile between blocks so the grid
//            still covers the compute units.
//   combine  a wave per (token, row piece): the result of
//            convert_combine_input followed by the combine, without the
//            intermediate rows. For each of the token's ranks in its rank
//            order: the FP32 fold of the rank's kept expert outputs (in
//            first-occurrence order, weighted or not), rounded to the combine
//            type as the intermediate row would be; those are summed in FP32
//            from the first and rounded once. A rank whose pairs were all
//            dropped adds +0, as its intermediate row would.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ep_device.h"
#include "ep_kernels.h"

namespace ep {
namespace {

using namespace dev;

constexpr int kSxWaves = 4;  // count and scan: waves a block, one tile or list each
// Mask words of a token's expert set the copy keeps in registers (E <= 256),
// and the experts whose tile masks it holds in LDS at a time.
constexpr int kSeenWords = 4;
constexpr int kWinExperts = kSeenWords * kWave;
// The one-launch count and scan: a wave per tile.
constexpr int kCountScanWaves = kCountScanTiles;

// Tokens of source rank r in this call.
__device__ __forceinline__ int tokens_of(const StandardArgs& a, int r)
{
    return max(0, min(a.ntok[r], a.M));
}

// A wave per (source rank, tile, mask word of 64 experts).
template <int KB>
__global__ __launch_bounds__(kSxWaves * kWave) void sx_count_kernel(StandardArgs a)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int tile = blockIdx.x * kSxWaves + uniform(threadIdx.x / kWave);
    const int r = blockIdx.y;
    const int w = blockIdx.z;
    if (tile >= a.Tr)
        return;  // whole waves
    const int T = tokens_of(a, r);
    const int q = tile * kWave + lane;
    const bool valid = q < T;
    const int64_t TT = (int64_t)a.W * a.Tr;
    const int nj = min(kWave, a.E - 64 * w);
    // expert 64w + j at [j * TT]
    int32_t* counts = a.tile_counts + (int64_t)(64 * w) * TT + (int64_t)r * a.Tr + tile;
    if (tile * kWave >= T) {  // no token here
        if (lane < nj)
            counts[(int64_t)lane * TT] = 0;
        return;
    }
    constexpr int KC = id_chunk<KB>();
    const int32_t* ids = a.idx + ((int64_t)r * a.M + (valid ? q : 0)) * a.k;
    const uint64_t m = local_word<KC>(ids, a.k, valid, 0, a.E, w);
    int c = 0;
    for (int jj = 0; jj < nj; ++jj) {
        const uint64_t b = __ballot((m >> jj) & 1);
        if (lane == jj)
            c = __popcll(b);
    }
    if (lane < nj)
        counts[(int64_t)lane * TT] = c;
}

// Expert g's exclusive scan over its (source rank, tile) counts, one wave:
// tile bases, the expert's row count, and its layout range for every source
// rank (a source rank's first tile's base is where its rows start). cnt(t)
// gives tile t's count.
template <typename Count>
__device__ __forceinline__ void scan_expert(const StandardArgs& a, int64_t g, Count cnt)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int TT = a.W * a.Tr;
    int32_t* base = a.tile_base + g * TT;
    // lane s < W: source rank s's first tile; its base is where s's rows start
    const int start_tile = lane < a.W ? lane * a.Tr : TT;
    int start = 0, carry = 0;
    for (int c0 = 0; c0 < TT; c0 += kWave) {
        const int t = c0 + lane;
        const int v = t < TT ? cnt(t) : 0;
        int inc = v;  // inclusive prefix over the wave
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const int u = __shfl_up(inc, o);
            if (lane >= o)
                inc += u;
        }
        const int excl = carry + inc - v;
        if (t < TT)
            base[t] = excl;
        const int at = __shfl(excl, (start_tile - c0) & (kWave - 1));
        if (start_tile >= c0 && start_tile < c0 + kWave)
            start = at;
        carry += __shfl(inc, kWave - 1);
    }
    if (lane == 0)
        a.count[g] = carry;
    int next = __shfl_down(start, 1);
    if (lane == a.W - 1)
        next = carry;
    if (lane < a.W) {
        const int64_t lo = min(start, a.cap);
        const int64_t hi = min(next, a.cap);
        a.layout_range[g * a.W + lane] = (lo << 32) | (hi - lo);
    }
}

__global__ __launch_bounds__(kSxWaves * kWave) void sx_scan_kernel(StandardArgs a)
{
    const int64_t g = (int64_t)blockIdx.x * kSxWaves + uniform(threadIdx.x / kWave);
    if (g >= a.E)
        return;  // whole waves
    const int32_t* cnt = a.tile_counts + g * ((int64_t)a.W * a.Tr);
    scan_expert(a, g, [&](int t) { return cnt[t]; });
}

// Calls of at most kCountScanTiles tiles: the count and the scan in one
// launch, a block per expert. Its waves count the expert's tokens in the
// tiles (a tile a wave, a lane per token, one ballot) into LDS; then wave 0
// scans them as sx_scan_kernel does. Every block reads all the call's ids,
// which is cheap only for small calls.
template <int KB>
__global__ __launch_bounds__(kCountScanWaves * kWave) void sx_count_scan_kernel(StandardArgs a)
{
    __shared__ int32_t s_cnt[kCountScanTiles];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    const int g = blockIdx.x;
    const int TT = a.W * a.Tr;
    if (TT > kCountScanTiles)
        return;  // not launched for such calls
    constexpr int KC = id_chunk<KB>();
    for (int t = wave; t < TT; t += kCountScanWaves) {
        const int r = t / a.Tr;
        const int tile = t - r * a.Tr;
        const int T = tokens_of(a, r);
        const int q = tile * kWave + lane;
        const bool valid = q < T;
        int c = 0;
        if (tile * kWave < T) {  // uniform
            const int32_t* ids = a.idx + ((int64_t)r * a.M + (valid ? q : 0)) * a.k;
            bool names = false;
            for (int c0 = 0; c0 * KC < a.k; ++c0) {
                int32_t id[KC];
                load_ids<KC>(ids, a.k, c0, id);
#pragma unroll
                for (int i = 0; i < KC; ++i)
                    names = names || (c0 * KC + i < a.k && id[i] == g);
            }
            c = __popcll(__ballot(valid && names));
        }
        if (lane == 0)
            s_cnt[t] = c;
    }
    __syncthreads();
    if (wave == 0)
        scan_expert(a, g, [&](int t) { return s_cnt[t]; });
}

// kCast: the source rows are bf16 / fp16 (a.cast) and the packed rows E4M3
// (round to nearest even, saturating at 448): each loaded 16-byte vector of 8
// elements is converted once and 8 bytes are stored to each packed row.
template <int VPL, int KB, bool kStream, bool kCast>
__global__ __launch_bounds__(1024) void sx_copy_kernel(StandardArgs a)
{
    __shared__ int32_t s_e[kWave][KB];  // a token's distinct experts, first-occurrence order
    __shared__ int32_t s_p[kWave][KB];  // their positions, then the kept packed rows
    __shared__ int8_t s_u[kWave][KB];   // each slot's index into s_e; -1: invalid or a repeat
    __shared__ int32_t s_n[kWave];      // kept packed rows of the token
    __shared__ uint64_t s_bal[kWinExperts];  // expert e0 + j: the tile's lanes naming it
    __shared__ int32_t s_base[kWinExperts];  // and its tile base

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    const int nwaves = blockDim.x / kWave;
    const int tile = blockIdx.x / a.token_split;
    const int sub = blockIdx.x - tile * a.token_split;
    const int piece = blockIdx.y;
    const int r = blockIdx.z;
    const int q0 = tile * kWave;
    const int cnt = min(kWave, tokens_of(a, r) - q0);
    // Blocks sharing the tile copy tokens [t_lo, t_hi) of it each; every one
    // works out the whole tile's positions (the in-tile prefix needs them all).
    const int span = (kWave + a.token_split - 1) / a.token_split;
    const int t_lo = sub * span;
    const int t_hi = min(cnt, t_lo + span);
    if (t_lo >= t_hi)
        return;  // the whole block: no token of its own
    const int64_t row0 = (int64_t)r * a.M + q0;
    const int64_t TT = (int64_t)a.W * a.Tr;

    // This wave's items: tokens t_lo + wave, t_lo + wave + nwaves, ... below
    // t_hi, each cut into nch chunks of its row piece [vbeg, vend).
    const uint32_t row_bytes = (uint32_t)a.row_vecs * 16u;
    const int vbeg = piece * a.piece_vecs;
    const int vend = min(a.row_vecs, vbeg + a.piece_vecs);
    const int nch = (vend - vbeg + kWave * VPL - 1) / (kWave * VPL);
    const int nt = t_hi - t_lo;
    const int items = (wave < nt ? (nt - wave + nwaves - 1) / nwaves : 0) * nch;
    auto load_item = [&](int it, u32x4 (&v)[VPL]) {
        const int t = t_lo + wave + (it / nch) * nwaves;
        const int v0 = vbeg + (it % nch) * kWave * VPL;
        const __amdgpu_buffer_rsrc_t rs = row_rsrc(a.x + (row0 + t) * row_bytes, row_bytes);
        // Large pieces: every load issued (a vector past the piece reads zeros
        // from the row's end without touching memory), so that the conversions
        // and stores can wait for one vector at a time; small pieces keep their
        // guarded loads, as the dispatch copy does.
#pragma unroll
        for (int u = 0; u < VPL; ++u) {
            const int vv = v0 + u * kWave + lane;
            if constexpr (VPL >= 8)
                v[u] = bload16<Policy<kStream>::copy_load>(rs, vv < vend ? (uint32_t)vv * 16u
                                                                         : row_bytes);
            else if (vv < vend)
                v[u] = bload16<Policy<kStream>::copy_load>(rs, (uint32_t)vv * 16u);
        }
    };
    auto store_item = [&](int it, const u32x4 (&v)[VPL]) {
        const int t = t_lo + wave + (it / nch) * nwaves;
        const int v0 = vbeg + (it % nch) * kWave * VPL;
        const int n = uniform(s_n[t]);
        // lane i < n: the packed row of the token's i-th kept expert, read
        // from LDS for all of them at once
        const int32_t prow = lane < n ? s_p[t][lane] : 0;
        u32x2 c[kCast ? VPL : 1];
        if constexpr (kCast) {
#pragma unroll
            for (int u = 0; u < VPL; ++u)
                c[u] = cast_e4m3(v[u], a.cast);
        }
        auto store_to = [&](int i) {
            const int64_t gi = __builtin_amdgcn_readlane(prow, i);
            const __amdgpu_buffer_rsrc_t rd =
                row_rsrc(a.px + gi * a.out_row_bytes, a.out_row_bytes);
#pragma unroll
            for (int u = 0; u < VPL; ++u) {
                const int vv = v0 + u * kWave + lane;
                if (vv < vend) {
                    if constexpr (kCast)
                        __builtin_amdgcn_raw_buffer_store_b64(c[u], rd, (int)((uint32_t)vv * 8u), 0,
                                                              Policy<kStream>::cast_store);
                    else
                        bstore16<Policy<kStream>::copy_store>(v[u], rd, (uint32_t)vv * 16u);
                }
            }
        };
        // large pieces: the first packed row outside the loop, so that each of
        // its stores waits for its own vector only
        int i0 = 0;
        if constexpr (VPL >= 8) {
            if (n > 0)
                store_to(0);
            i0 = 1;
        }
        for (int i = i0; i < n; ++i)
            store_to(i);
    };
    // Small pieces (small rows or small calls, where time is latency): each
    // wave's first item loads while wave 0 routes the tile.
    u32x4 A[VPL], B[VPL];
    if (VPL < 8 && items > 0)
        load_item(0, A);

    if (wave == 0) {
        const bool valid = lane < cnt;
        constexpr int KC = id_chunk<KB>();
        const int64_t rowq = row0 + (valid ? lane : 0);
        const int32_t* ids = a.idx + rowq * a.k;
        // The token's distinct experts in first-occurrence order. With at
        // most kSeenWords mask words (E <= 256) its expert set is kept in
        // registers and repeats are found there; else in LDS.
        const int nw = (a.E + kWave - 1) / kWave;
        const bool regs = nw <= kSeenWords;  // uniform
        // the tile bases of experts 64w + lane (the first window), loaded
        // before the ids are read so their latency overlaps the routing
        int bw[kSeenWords];
#pragma unroll
        for (int w = 0; w < kSeenWords; ++w)
            bw[w] = 64 * w + lane < a.E
                        ? a.tile_base[(int64_t)(64 * w + lane) * TT + (int64_t)r * a.Tr + tile]
                        : 0;
        int n = 0;
        uint64_t seen[kSeenWords] = {};
        for (int c = 0; c * KC < a.k; ++c) {
            int32_t id[KC];
            load_ids<KC>(ids, a.k, c, id);
#pragma unroll
            for (int i = 0; i < KC; ++i) {
                const int slot = c * KC + i;
                if (slot >= a.k)
                    continue;
                int u = -1;
                const int e = id[i];
                if (valid && e >= 0 && e < a.E) {
                    bool dup = false;
                    if (regs) {
                        const uint64_t bit = 1ull << (e & (kWave - 1));
#pragma unroll
                        for (int x = 0; x < kSeenWords; ++x) {
                            if (x == (e >> 6)) {
                                dup = (seen[x] & bit) != 0;
                                seen[x] |= bit;
                            }
                        }
                    } else {
                        for (int v = 0; v < n; ++v)
                            dup = dup || s_e[lane][v] == e;
                    }
                    if (!dup) {
                        u = n;
                        s_e[lane][n++] = e;
                    }
                }
                s_u[lane][slot] = (int8_t)u;
            }
        }
        // positions inside the tile, from LDS expert masks
        tile_positions<kSeenWords>(
            s_e[lane], s_p[lane], n, a.E, bw,
            [&](int e) { return a.tile_base[(int64_t)e * TT + (int64_t)r * a.Tr + tile]; }, s_bal,
            s_base);
        // the combine's map: the packed row of each slot that is its expert's
        // first occurrence and was kept, else -1 (each block its own tokens)
        if (piece == 0 && valid && lane >= t_lo && lane < t_hi) {
            for (int slot = 0; slot < a.k; ++slot) {
                const int u = s_u[lane][slot];
                const int p = u >= 0 ? s_p[lane][u] : a.cap;
                a.fslot[rowq * a.k + slot] = p < a.cap ? s_e[lane][u] * a.cap + p : -1;
            }
        }
        int kept = 0;  // positions past the capacity are dropped
        for (int u = 0; u < n; ++u) {
            const int p = s_p[lane][u];
            if (p < a.cap)
                s_p[lane][kept++] = s_e[lane][u] * a.cap + p;
        }
        s_n[lane] = kept;
    }
    __syncthreads();

    const int sd = a.scale_dwords;
    if (piece == 0) {
        for (int t = t_lo + wave; t < t_hi; t += nwaves) {
            const int n = uniform(s_n[t]);
            if (lane < n)
                a.src_info[s_p[t][lane]] = q0 + t;
            for (int c0 = 0; n > 0 && c0 < sd; c0 += kWave) {
                const int c = c0 + lane;
                const uint32_t v = c < sd ? a.sc[(row0 + t) * sd + c] : 0u;
                for (int i = 0; i < n; ++i) {
                    const int64_t gi = uniform(s_p[t][i]);
                    if (c < sd)
                        a.psc[gi * sd + c] = v;
                }
            }
        }
    }

    if constexpr (VPL < 8) {
        // two items in flight: item i + 1 loads while item i stores
        for (int it = 0; it < items; it += 2) {
            if (it + 1 < items)
                load_item(it + 1, B);
            store_item(it, A);
            if (it + 1 < items) {
                if (it + 2 < items)
                    load_item(it + 2, A);
                store_item(it + 1, B);
            }
        }
    } else {
        // large pieces (throughput): one chunk a wave in flight
        for (int it = 0; it < items; ++it) {
            if (uniform(s_n[t_lo + wave + (it / nch) * nwaves]) == 0)
                continue;  // a token without a kept expert is not read
            load_item(it, A);
            store_item(it, A);
        }
    }
}

// Fold-position flags of a kept pair: the last and the first kept pair of
// its rank, and whether ranks without a kept pair come just before its rank.
constexpr int kFoldLast = 1;
constexpr int kFoldGap = 2;
constexpr int kFoldFirstBit = 2;
constexpr int kFoldFirst = 1 << kFoldFirstBit;

// One kept pair into its rank's sum, 8 elements in place: p = c * f for the
// rank's first pair (the product, which is fma(c, f, -0) exactly, signed
// zeros included), else p = fma(c, f, p). The choice is a uniform branch
// inside one asm statement, so both forms write the same registers: written
// as two C++ branches, the compiler joined them with a register copy per
// element, and resetting the sum to -0 after each rank costs an instruction
// per element and rank.
__device__ __forceinline__ void fold_pair8(float (&p)[8], const float (&f)[8], float c, int flags)
{
    asm("s_bitcmp1_b32 %[fl], %[bit]\n\t"
        "s_cbranch_scc1 1f\n\t"
        "v_fmac_f32 %[p0], %[c], %[f0]\n\t"
        "v_fmac_f32 %[p1], %[c], %[f1]\n\t"
        "v_fmac_f32 %[p2], %[c], %[f2]\n\t"
        "v_fmac_f32 %[p3], %[c], %[f3]\n\t"
        "v_fmac_f32 %[p4], %[c], %[f4]\n\t"
        "v_fmac_f32 %[p5], %[c], %[f5]\n\t"
        "v_fmac_f32 %[p6], %[c], %[f6]\n\t"
        "v_fmac_f32 %[p7], %[c], %[f7]\n\t"
        "s_branch 2f\n"
        "1:\n\t"
        "v_mul_f32 %[p0], %[c], %[f0]\n\t"
        "v_mul_f32 %[p1], %[c], %[f1]\n\t"
        "v_mul_f32 %[p2], %[c], %[f2]\n\t"
        "v_mul_f32 %[p3], %[c], %[f3]\n\t"
        "v_mul_f32 %[p4], %[c], %[f4]\n\t"
        "v_mul_f32 %[p5], %[c], %[f5]\n\t"
        "v_mul_f32 %[p6], %[c], %[f6]\n\t"
        "v_mul_f32 %[p7], %[c], %[f7]\n"
        "2:"
        : [p0] "+v"(p[0]), [p1] "+v"(p[1]), [p2] "+v"(p[2]), [p3] "+v"(p[3]),
          [p4] "+v"(p[4]), [p5] "+v"(p[5]), [p6] "+v"(p[6]), [p7] "+v"(p[7])
        : [c] "s"(c), [f0] "v"(f[0]), [f1] "v"(f[1]), [f2] "v"(f[2]), [f3] "v"(f[3]),
          [f4] "v"(f[4]), [f5] "v"(f[5]), [f6] "v"(f[6]), [f7] "v"(f[7]), [fl] "s"(flags),
          [bit] "n"(kFoldFirstBit)
        : "scc");
}

// WIRE: 0 for bf16 / fp16 expert outputs, else the wire of the packed rows
// (kWireFp8Block128, kWireMxfp4), each element decoded exactly before the fold.
template <int G, int U, int DT, bool kStream, bool kWeighted, int WIRE>
__global__ __launch_bounds__(1024) void sx_combine_kernel(StandardCombineArgs a, TokenMap tk)
{
    const int lane = threadIdx.x & (kWave - 1);
    // wave items: (token, piece); piece_inner: piece fastest
    const uint32_t item = blockIdx.x * (blockDim.x / kWave) + uniform(threadIdx.x / kWave);
    const uint32_t flat_u = a.piece_inner ? item / (uint32_t)a.pieces : item;
    if (flat_u >= (uint32_t)tk.total)
        return;  // whole waves only
    const int flat = (int)flat_u;
    const int piece = a.piece_inner ? (int)(item - flat_u * (uint32_t)a.pieces) : (int)blockIdx.y;
    const int r = rank_of_token(tk, flat);
    const int64_t tok = (int64_t)r * a.M + (flat - tk.tok_start[r]);

    // Lane j < k holds slot j of the token.
    const bool has = lane < a.k;
    const int32_t id = has ? a.idx[tok * a.k + lane] : -1;
    const bool valid = has && id >= 0 && id < a.E;
    const int32_t fs = has ? a.fslot[tok * a.k + lane] : -1;
    const bool kept = fs >= 0;
    const int rk = valid ? id / a.Er : -1;
    float c = 0.0f;
    if constexpr (kWeighted)
        c = has ? a.w[tok * a.k + lane] : 0.0f;
    // Each slot's rank: whether it is the rank's first slot (the token's rank
    // order is the order of those), and which lane is. Weighted, a kept slot
    // (its expert's first) sums the weights of every slot naming its expert,
    // in slot order.
    bool rfirst = valid;
    int rsrc = lane;
    const float cw_own = c;
    for (int j = 0; j < a.k; ++j) {
        const int rj = __builtin_amdgcn_readlane(rk, j);
        if (rfirst && j < lane && rj == rk) {
            rfirst = false;
            rsrc = j;
        }
        if constexpr (kWeighted) {
            const int ij = __builtin_amdgcn_readlane(id, j);
            const float wj = __builtin_bit_cast(
                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, cw_own), j));
            if (j > lane && ij == id)
                c = c + wj;
        }
    }
    const uint64_t dmask = __ballot(rfirst);
    const int nD = __popcll(dmask);
    const int dix = __shfl(lanes_below(dmask), rsrc);  // the slot's rank's place in the order
    // Kept pairs in fold order (by rank place, then slot); lane s < nk then
    // holds the s-th: its packed row, weight and rank place.
    const uint64_t kmask = __ballot(kept);
    const int nk = __popcll(kmask);
    int pos = 0, src = 0;
    for (int j = 0; j < a.k; ++j) {
        const int dj = __builtin_amdgcn_readlane(dix, j);
        if (((kmask >> j) & 1) && (dj < dix || (dj == dix && j < lane)))
            ++pos;
    }
    for (int j = 0; j < a.k; ++j) {
        const int pj = __builtin_amdgcn_readlane(pos, j);
        if (((kmask >> j) & 1) && pj == lane)
            src = j;
    }
    // every lane takes part in the cross-lane reads: one from an inactive
    // lane returns 0, and a sequence position can read a slot lane >= nk
    const int32_t gsrc = __shfl(fs, src);
    const int32_t gl = lane < nk ? gsrc : -1;
    const float gw = __shfl(c, src);
    const int dx = __shfl(dix, src);
    const int dprev = __shfl_up(dx, 1);
    const int dnext = __shfl_down(dx, 1);
    int flags = 0;
    if (lane < nk) {
        const int pv = lane == 0 ? -1 : dprev;
        const bool last = lane == nk - 1 || dnext != dx;
        flags = (last ? kFoldLast : 0) | (dx - pv > 1 ? kFoldGap : 0) |
                (dx != pv ? kFoldFirst : 0);
    }
    const int dlast = nk > 0 ? __builtin_amdgcn_readlane(dx, nk - 1) : -1;
    const bool trailing = nD - 1 > dlast;  // ranks without a kept pair after the last

    const uint32_t row_bytes = (uint32_t)a.row_vecs * 16u;  // an output row
    const __amdgpu_buffer_rsrc_t rdst = row_rsrc(a.out + tok * row_bytes, row_bytes);
    const int vbeg = piece * a.piece_vecs;
    const int vend = min(a.row_vecs, vbeg + a.piece_vecs);
    // Wire rows: lane l holds dword vbeg / 16 + l of the scale row of each
    // kept pair of the current group of G (a dword covers 16 groups of 8
    // elements), loaded once when the token has at most G pairs.
    uint32_t spre[WIRE ? G : 1];
    auto load_scales = [&](int i0) {
#pragma unroll
        for (int q = 0; q < G; ++q) {
            if (i0 + q < nk) {
                const int64_t gq = __builtin_amdgcn_readlane(gl, i0 + q);
                const __amdgpu_buffer_rsrc_t rs =
                    row_rsrc(a.pys + gq * a.py_scale_bytes, a.py_scale_bytes);
                const uint32_t off = (uint32_t)(vbeg / 16 + lane) * 4u;
                if (WIRE == kWireFp8Block128 || a.py_scale_bytes % 4 == 0) {
                    spre[q] = __builtin_amdgcn_raw_buffer_load_b32(
                        rs, off, 0, Policy<kStream>::combine_load);
                } else {  // MXFP4 scale rows that are not whole dwords: by bytes
                    uint32_t d = 0;
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        d |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(
                                 rs, off + b, 0, Policy<kStream>::combine_load)
                             << (8 * b);
                    spre[q] = d;
                }
            }
        }
    };
    const bool regroup = nk > G;  // uniform
    if constexpr (WIRE != 0) {
        if (!regroup)
            load_scales(0);
    }
    // A rank's sum starts at its first kept pair (fold_pair8), so it needs
    // no reset between ranks; the total starts at -0, the identity of IEEE
    // addition (-0 + x = x for every x, signed zeros included), so the first
    // rank needs no case of its own.
    float part[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            part[u][e] = -0.0f;
    for (int v0 = vbeg; v0 < vend; v0 += kWave * U) {
        float tot[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                tot[u][e] = -0.0f;
        bool have = false;  // uniform: tot holds a rank's contribution
        for (int i0 = 0; i0 < nk; i0 += G) {
            if constexpr (WIRE != 0) {
                if (regroup)
                    load_scales(i0);
            }
            u32x4 rows[WIRE ? 1 : U][WIRE ? 1 : G];   // bf16 / fp16 rows: 16 B a group
            u32x2 codes[WIRE ? U : 1][WIRE ? G : 1];  // wire rows: 8 B (FP8) or 4 B (MXFP4)
            // Every load is issued, in the order the fold takes them, so a
            // pair's fold waits for its own rows only. A pair past the token's
            // last has an empty resource and a column past the piece an offset
            // at the row's end: both read zeros without touching memory.
            const uint32_t pb = WIRE ? a.py_row_bytes : row_bytes;
            constexpr uint32_t vb = WIRE == 0 ? 16u : WIRE == kWireFp8Block128 ? 8u : 4u;
#pragma unroll
            for (int q = 0; q < G; ++q) {
                const bool in = i0 + q < nk;  // uniform
                const int64_t gq = in ? __builtin_amdgcn_readlane(gl, i0 + q) : 0;
                const __amdgpu_buffer_rsrc_t ry = row_rsrc(a.py + gq * pb, in ? pb : 0u);
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int v = v0 + u * kWave + lane;
                    const uint32_t off = v < vend ? (uint32_t)v * vb : pb;
                    constexpr int ld = Policy<kStream>::combine_load;
                    if constexpr (WIRE == 0)
                        rows[u][q] = bload16<ld>(ry, off);
                    else if constexpr (WIRE == kWireFp8Block128)
                        codes[u][q] = __builtin_amdgcn_raw_buffer_load_b64(ry, off, 0, ld);
                    else
                        codes[u][q] = {__builtin_amdgcn_raw_buffer_load_b32(ry, off, 0, ld), 0u};
                }
            }
#pragma unroll
            for (int q = 0; q < G; ++q) {
                if (i0 + q < nk) {  // uniform: every lane takes part in the cross-lane reads
                    const int fl = __builtin_amdgcn_readlane(flags, i0 + q);
                    const float cq =
                        kWeighted ? __builtin_bit_cast(
                                        float, __builtin_amdgcn_readlane(
                                                   __builtin_bit_cast(int, gw), i0 + q))
                                  : 1.0f;
                    const bool gap = fl & kFoldGap;
                    const bool last = fl & kFoldLast;
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        float f[8];
                        if constexpr (WIRE == 0) {
                            widen<DT>(rows[u][q], f);
                        } else {
                            const int v = v0 + u * kWave + lane;
                            const uint32_t d = (uint32_t)__shfl((int)spre[q], (v - vbeg) >> 4);
                            // MXFP4: byte (v / 4) mod 4 of the dword
                            const uint32_t sb =
                                WIRE == kWireFp8Block128 ? d : d >> (8 * ((v >> 2) & 3));
                            decode_group<WIRE>(codes[u][q], sb, f);
                        }
                        if (gap) {  // ranks whose intermediate rows are +0
#pragma unroll
                            for (int e = 0; e < 8; ++e)
                                tot[u][e] = tot[u][e] + 0.0f;
                        }
                        // unweighted, c = 1: fma(1, f, p) = p + f and 1 * f = f exactly
                        fold_pair8(part[u], f, cq, fl);
                        if (last) {
                            // the rank's intermediate row: rounded to the combine type
#pragma unroll
                            for (int e = 0; e < 8; ++e)
                                tot[u][e] = tot[u][e] + round_to<DT>(part[u][e]);
                        }
                    }
                    have = have || gap || last;
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = v0 + u * kWave + lane;
            if (v < vend) {
                if (!have || trailing) {  // no rank with a kept pair, or +0 ranks after the last
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        tot[u][e] = tot[u][e] + 0.0f;
                }
                bstore16<Policy<kStream>::combine_store>(narrow<DT>(tot[u]), rdst,
                                                         (uint32_t)v * 16u);
            }
        }
    }
}

// Top-k bucket: the smallest of 8, 16, 32, 64 >= k.
int sx_bucket(int k) { return k <= 8 ? 8 : k <= 16 ? 16 : k <= 32 ? 32 : 64; }

template <int VPL, int KB>
hipError_t sx_copy_with(const StandardArgs& a, dim3 grid, dim3 block, bool stream, hipStream_t s)
{
    if (a.cast) {
        if (stream)
            hipLaunchKernelGGL((sx_copy_kernel<VPL, KB, true, true>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((sx_copy_kernel<VPL, KB, false, true>), grid, block, 0, s, a);
    } else {
        if (stream)
            hipLaunchKernelGGL((sx_copy_kernel<VPL, KB, true, false>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((sx_copy_kernel<VPL, KB, false, false>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

template <int VPL>
hipError_t sx_copy_with_vpl(const StandardArgs& a, dim3 grid, dim3 block, bool stream,
                            hipStream_t s)
{
    switch (sx_bucket(a.k)) {
    case 8: return sx_copy_with<VPL, 8>(a, grid, block, stream, s);
    case 16: return sx_copy_with<VPL, 16>(a, grid, block, stream, s);
    case 32: return sx_copy_with<VPL, 32>(a, grid, block, stream, s);
    default: return sx_copy_with<VPL, 64>(a, grid, block, stream, s);
    }
}

template <int G, int U, int DT, bool kStream, int WIRE>
void sx_combine_launch(const StandardCombineArgs& a, const TokenMap& tk, dim3 grid, dim3 block,
                       hipStream_t s)
{
    if (a.w)
        hipLaunchKernelGGL((sx_combine_kernel<G, U, DT, kStream, true, WIRE>), grid, block, 0, s,
                           a, tk);
    else
        hipLaunchKernelGGL((sx_combine_kernel<G, U, DT, kStream, false, WIRE>), grid, block, 0, s,
                           a, tk);
}

template <int G, int U, int DT, bool kStream>
void sx_combine_wire(const StandardCombineArgs& a, const TokenMap& tk, dim3 grid, dim3 block,
                     hipStream_t s)
{
    if (a.wire == kWireFp8Block128)
        sx_combine_launch<G, U, DT, kStream, kWireFp8Block128>(a, tk, grid, block, s);
    else if (a.wire == kWireMxfp4)
        sx_combine_launch<G, U, DT, kStream, kWireMxfp4>(a, tk, grid, block, s);
    else
        sx_combine_launch<G, U, DT, kStream, 0>(a, tk, grid, block, s);
}

template <int G, int U>
hipError_t sx_combine_with(const StandardCombineArgs& a, const TokenMap& tk, int dtype, dim3 grid,
                           dim3 block, bool stream, hipStream_t s)
{
    if (dtype == 0) {
        if (stream)
            sx_combine_wire<G, U, 0, true>(a, tk, grid, block, s);
        else
            sx_combine_wire<G, U, 0, false>(a, tk, grid, block, s);
    } else {
        if (stream)
            sx_combine_wire<G, U, 1, true>(a, tk, grid, block, s);
        else
            sx_combine_wire<G, U, 1, false>(a, tk, grid, block, s);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_standard_count(const StandardArgs& a, hipStream_t s)
{
    const dim3 grid((a.Tr + kSxWaves - 1) / kSxWaves, a.W, (a.E + kWave - 1) / kWave);
    const dim3 block(kSxWaves * kWave);
    switch (sx_bucket(a.k)) {
    case 8: hipLaunchKernelGGL((sx_count_kernel<8>), grid, block, 0, s, a); break;
    case 16: hipLaunchKernelGGL((sx_count_kernel<16>), grid, block, 0, s, a); break;
    case 32: hipLaunchKernelGGL((sx_count_kernel<32>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((sx_count_kernel<64>), grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_standard_count_scan(const StandardArgs& a, hipStream_t s)
{
    const dim3 grid((unsigned)a.E);
    const dim3 block(kCountScanWaves * kWave);
    switch (sx_bucket(a.k)) {
    case 8: hipLaunchKernelGGL((sx_count_scan_kernel<8>), grid, block, 0, s, a); break;
    case 16: hipLaunchKernelGGL((sx_count_scan_kernel<16>), grid, block, 0, s, a); break;
    case 32: hipLaunchKernelGGL((sx_count_scan_kernel<32>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((sx_count_scan_kernel<64>), grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_standard_scan(const StandardArgs& a, hipStream_t s)
{
    hipLaunchKernelGGL(sx_scan_kernel, dim3((unsigned)((a.E + kSxWaves - 1) / kSxWaves)),
                       dim3(kSxWaves * kWave), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_standard_copy(const StandardArgs& a, int waves, int row_split, bool stream,
                                hipStream_t s)
{
    const dim3 grid(a.Tr * a.token_split, row_split, a.W);
    const dim3 block(waves * kWave);
    const int per_lane = (a.piece_vecs + kWave - 1) / kWave;
    if (per_lane <= 1)
        return sx_copy_with_vpl<1>(a, grid, block, stream, s);
    if (per_lane <= 2)
        return sx_copy_with_vpl<2>(a, grid, block, stream, s);
    if (per_lane <= 4)
        return sx_copy_with_vpl<4>(a, grid, block, stream, s);
    return sx_copy_with_vpl<8>(a, grid, block, stream, s);
}

hipError_t launch_standard_combine(const StandardCombineArgs& a, const TokenMap& tk, int dtype,
                                   int waves, bool stream, hipStream_t s)
{
    if (tk.total == 0)
        return hipSuccess;
    const dim3 grid = a.piece_inner
                          ? dim3((unsigned)(((int64_t)tk.total * a.pieces + waves - 1) / waves))
                          : dim3((unsigned)((tk.total + waves - 1) / waves), (unsigned)a.pieces);
    const dim3 block(waves * kWave);
    const int pe = a.k < a.E ? a.k : a.E;  // most kept pairs a token can have
    if (pe <= 1)
        return sx_combine_with<1, 4>(a, tk, dtype, grid, block, stream, s);
    if (pe <= 2)
        return sx_combine_with<2, 4>(a, tk, dtype, grid, block, stream, s);
    if (pe <= 4)
        return sx_combine_with<4, kCombineColumns>(a, tk, dtype, grid, block, stream, s);
    return sx_combine_with<kCombineGroup, kCombineColumns>(a, tk, dtype, grid, block, stream, s);
}

}  // namespace ep
