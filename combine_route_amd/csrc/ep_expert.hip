// gfx950 (MI355X, CDNA4) kernels of the expert-major layout of received rows
// and its inverse ("MORI-EP User Guide", section 4 "Standard MoE
// Compatibility (DeepEP)": convert_dispatch_output, convert_combine_input).
//
// Each rank's received rows are counting-sorted by local expert with the same
// deterministic scheme as the dispatch: one 64-lane ballot per local expert
// over a tile of 64 rows, an exclusive scan over tiles per (rank, expert)
// list, and the ballot prefix (mbcnt) inside a tile. No atomic decides a
// position, and an expert's rows keep the receive order.
//   count    a wave per tile: how many of its rows name each local expert;
//            where each source rank's rows start, with the in-tile prefixes
//            there, for the layout ranges.
//   scan     a wave per list: exclusive scan of its tile counts -> tile bases,
//            the expert's row count and its layout ranges.
//   copy     a block per (tile, row piece, share of the tile's rows): wave 0
//            works out the kept packed row of every (row, local expert) pair
//            of the tile into LDS; then every wave loads a row of the block's
//            share once per row piece (16 B a lane) and stores it to each of
//            the row's packed rows; piece-0 blocks also write the scale rows,
//            the source info and the map the inverse gathers through, for
//            their share. Small calls share a tile between blocks.
//   combine  a wave per (received row, row piece): the row's kept expert
//            outputs, folded in FP32 in first-occurrence order and rounded to
//            nearest even once (the combine's fold).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ep_device.h"
#include "ep_kernels.h"

namespace ep {
namespace {

using namespace dev;

constexpr int kExWaves = 4;  // count and scan: waves a block, one tile or list each
// Local experts whose tile masks the copy holds in LDS at a time.
constexpr int kExWindow = 256;

// Received rows of rank d that the call covers. The dispatch never fills more
// than `rows` (every token goes at most once to a rank); the clamp keeps a
// wrong count from reaching past the tiles.
__device__ __forceinline__ int received(int recv, int rows) { return max(0, min(recv, rows)); }

__device__ __forceinline__ int source_rank(const ExpertArgs& a, int64_t row)
{
    return min(max(a.src_pos[row] / a.WM, 0), a.W - 1);
}

template <int KB>
__global__ __launch_bounds__(kExWaves * kWave) void ex_count_kernel(ExpertArgs a)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int tile = blockIdx.x * kExWaves + uniform(threadIdx.x / kWave);
    const int d = blockIdx.y;
    if (tile >= a.T)
        return;  // whole waves
    const int R = received(a.recv[d], a.rows);
    const int q = tile * kWave + lane;
    const bool valid = q < R;
    const int64_t row0 = (int64_t)d * a.WM;
    const int64_t lo = (int64_t)d * a.Er;
    int32_t* counts = a.tile_counts + lo * a.T + tile;  // list lo + j at [j * T]
    int32_t* start = a.src_start + d * a.W;
    if (tile * kWave >= R) {  // no received row here
        for (int j = lane; j < a.Er; j += kWave)
            counts[(int64_t)j * a.T] = 0;
        if (R == 0 && tile == 0 && lane < a.W)
            start[lane] = 0;
        return;
    }
    constexpr int KC = id_chunk<KB>();
    const int32_t* ids = a.idx + (row0 + (valid ? q : 0)) * a.k;

    // Rows are in source-rank order, so source s starts at the first row
    // whose source is >= s. The row that starts sources (s_prev, s_cur]
    // records itself and, below, its in-tile prefix on every expert; the last
    // row gives every later source the end, R.
    const int s_cur = valid ? source_rank(a, row0 + q) : a.W;
    int s_prev = __shfl_up(s_cur, 1);
    if (lane == 0)
        s_prev = q > 0 ? source_rank(a, row0 + q - 1) : -1;
    const bool starts = valid && s_prev < s_cur;
    if (starts)
        for (int s = s_prev + 1; s <= s_cur; ++s)
            start[s] = q;
    if (valid && q == R - 1)
        for (int s = s_cur + 1; s < a.W; ++s)
            start[s] = R;

    for (int w = 0; 64 * w < a.Er; ++w) {
        const uint64_t m = local_word<KC>(ids, a.k, valid, lo, a.Er, w);
        const int nj = min(kWave, a.Er - 64 * w);
        int c = 0;
        for (int jj = 0; jj < nj; ++jj) {
            const uint64_t b = __ballot((m >> jj) & 1);
            if (lane == jj)
                c = __popcll(b);
            if (starts) {
                const int pre = lanes_below(b);
                int32_t* sp = a.src_prefix + (lo + 64 * w + jj) * a.W;
                for (int s = s_prev + 1; s <= s_cur; ++s)
                    sp[s] = pre;
            }
        }
        if (lane < nj)
            counts[(int64_t)(64 * w + lane) * a.T] = c;
    }
}

// List g's exclusive scan over its tile counts, one wave: tile bases, the
// expert's row count, and its layout range for every source rank. cnt(t)
// gives tile t's count; source(s) the row where source s starts (>= R: none)
// and the list's rows before it in that row's tile.
template <typename Count, typename Source>
__device__ __forceinline__ void scan_list(const ExpertArgs& a, int64_t g, int R, Count cnt,
                                          Source source)
{
    const int lane = threadIdx.x & (kWave - 1);
    int32_t* base = a.tile_base + g * a.T;
    // lane s < W: the row where source s starts and the expert's rows before
    // it in that row's tile
    int start_row = R, pre = 0;
    if (lane < a.W)
        source(lane, start_row, pre);
    const int start_tile = start_row / kWave;
    int start = 0, carry = 0;
    for (int c0 = 0; c0 < a.T; c0 += kWave) {
        const int t = c0 + lane;
        const int v = t < a.T ? cnt(t) : 0;
        int inc = v;  // inclusive prefix over the wave
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const int u = __shfl_up(inc, o);
            if (lane >= o)
                inc += u;
        }
        const int excl = carry + inc - v;
        if (t < a.T)
            base[t] = excl;
        const int at = __shfl(excl, (start_tile - c0) & (kWave - 1));
        if (start_row < R && start_tile >= c0 && start_tile < c0 + kWave)
            start = at + pre;
        carry += __shfl(inc, kWave - 1);
    }
    if (start_row >= R)
        start = carry;
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

__global__ __launch_bounds__(kExWaves * kWave) void ex_scan_kernel(ExpertArgs a)
{
    const int64_t g = (int64_t)blockIdx.x * kExWaves + uniform(threadIdx.x / kWave);
    if (g >= (int64_t)a.W * a.Er)
        return;  // whole waves
    const int d = (int)(g / a.Er);
    const int R = received(a.recv[d], a.rows);
    const int32_t* cnt = a.tile_counts + g * a.T;
    scan_list(a, g, R, [&](int t) { return cnt[t]; }, [&](int s, int& row, int& pre) {
        row = min(a.src_start[d * a.W + s], R);
        if (row < R)
            pre = a.src_prefix[g * a.W + s];
    });
}

// Calls of at most kCountScanTiles tiles a rank and top-k at most
// kCountScanTopK: the count and the scan in one launch, a block per (rank,
// local expert) list. Its waves count the list's rows in one tile each (a
// lane per row, one ballot) into LDS, and the row that starts each source
// rank records itself and the list's rows before it in its tile; then wave
// 0 scans as ex_scan_kernel does. Every block reads its rank's ids.
template <int KB>
__global__ __launch_bounds__(kCountScanTiles * kWave) void ex_count_scan_kernel(ExpertArgs a)
{
    __shared__ int32_t s_cnt[kCountScanTiles];
    __shared__ int32_t s_start[kMaxRanks];  // row where source s starts; R: none
    __shared__ int32_t s_pre[kMaxRanks];    // the list's rows before it in its tile
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    const int64_t g = blockIdx.x;
    const int d = (int)(g / a.Er);
    const int64_t e = g;  // the global id of the list's expert: d * Er + j
    const int R = received(a.recv[d], a.rows);
    if (a.T > kCountScanTiles)
        return;  // not launched for such calls
    if (wave == 0 && lane < a.W) {
        s_start[lane] = R;
        s_pre[lane] = 0;
    }
    __syncthreads();
    const int64_t row0 = (int64_t)d * a.WM;
    constexpr int KC = id_chunk<KB>();
    for (int t = wave; t < a.T; t += kCountScanTiles) {
        const int q = t * kWave + lane;
        const bool valid = q < R;
        int c = 0;
        if (t * kWave < R) {  // uniform
            const int32_t* ids = a.idx + (row0 + (valid ? q : 0)) * a.k;
            bool names = false;
            for (int c0 = 0; c0 * KC < a.k; ++c0) {
                int32_t id[KC];
                load_ids<KC>(ids, a.k, c0, id);
#pragma unroll
                for (int i = 0; i < KC; ++i)
                    names = names || (c0 * KC + i < a.k && id[i] == e);
            }
            const uint64_t b = __ballot(valid && names);
            c = __popcll(b);
            // rows are in source-rank order: the row that starts sources
            // (s_prev, s_cur] records itself and its in-tile prefix
            const int s_cur = valid ? source_rank(a, row0 + q) : a.W;
            int s_prev = __shfl_up(s_cur, 1);
            if (lane == 0)
                s_prev = q > 0 ? source_rank(a, row0 + q - 1) : -1;
            if (valid && s_prev < s_cur) {
                const int pre = lanes_below(b);
                for (int s = s_prev + 1; s <= s_cur; ++s) {
                    s_start[s] = q;
                    s_pre[s] = pre;
                }
            }
        }
        if (lane == 0)
            s_cnt[t] = c;
    }
    __syncthreads();
    if (wave == 0)
        scan_list(a, g, R, [&](int t) { return s_cnt[t]; }, [&](int s, int& row, int& pre) {
            row = s_start[s];
            pre = s_pre[s];
        });
}

template <int VPL, int KB, bool kStream>
__global__ __launch_bounds__(1024) void ex_copy_kernel(ExpertArgs a)
{
    __shared__ int32_t s_j[kWave][KB];  // a row's local experts, first-occurrence order
    __shared__ int32_t s_p[kWave][KB];  // their positions, then the kept packed rows
    __shared__ float s_c[kWave][KB];    // their weights for the row (when a.w is set)
    __shared__ int32_t s_n[kWave];      // kept packed rows of the row
    __shared__ uint64_t s_bal[kExWindow];  // local expert j0 + j: the tile's lanes naming it
    __shared__ int32_t s_base[kExWindow];  // and its tile base

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    const int nwaves = blockDim.x / kWave;
    const int tile = blockIdx.x / a.token_split;
    const int sub = blockIdx.x - tile * a.token_split;
    const int piece = blockIdx.y;
    const int d = blockIdx.z;
    const int R = received(a.recv[d], a.rows);
    const int q0 = tile * kWave;
    const int cnt = min(kWave, R - q0);
    // Blocks sharing the tile copy rows [r_lo, r_hi) of it each; every one
    // works out the whole tile's positions (the in-tile prefix needs them all).
    const int span = (kWave + a.token_split - 1) / a.token_split;
    const int r_lo = sub * span;
    const int r_hi = min(cnt, r_lo + span);
    if (r_lo >= r_hi)
        return;  // the whole block: no row of its own
    const int64_t row0 = (int64_t)d * a.WM + q0;
    const int64_t lo = (int64_t)d * a.Er;

    // This wave's items: rows r_lo + wave, r_lo + wave + nwaves, ... below
    // r_hi, each cut into nch chunks of its row piece [vbeg, vend).
    const uint32_t row_bytes = (uint32_t)a.row_vecs * 16u;
    const int vbeg = piece * a.piece_vecs;
    const int vend = min(a.row_vecs, vbeg + a.piece_vecs);
    const int nch = (vend - vbeg + kWave * VPL - 1) / (kWave * VPL);
    const int nr = r_hi - r_lo;
    const int items = (wave < nr ? (nr - wave + nwaves - 1) / nwaves : 0) * nch;
    auto load_item = [&](int it, u32x4 (&v)[VPL]) {
        const int r = r_lo + wave + (it / nch) * nwaves;
        const int v0 = vbeg + (it % nch) * kWave * VPL;
        const __amdgpu_buffer_rsrc_t rs = row_rsrc(a.x + (row0 + r) * row_bytes, row_bytes);
        // Large pieces: every load issued (a vector past the piece reads zeros
        // from the row's end without touching memory), so that the stores can
        // wait for one vector at a time; small pieces keep their guarded loads.
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
        const int r = r_lo + wave + (it / nch) * nwaves;
        const int v0 = vbeg + (it % nch) * kWave * VPL;
        const int n = uniform(s_n[r]);
        // lane i < n: the packed row of the row's i-th kept expert, read
        // from LDS for all of them at once
        const int32_t prow = lane < n ? s_p[r][lane] : 0;
        auto store_to = [&](int i) {
            const int64_t gi = __builtin_amdgcn_readlane(prow, i);
            const __amdgpu_buffer_rsrc_t rd = row_rsrc(a.px + gi * row_bytes, row_bytes);
#pragma unroll
            for (int u = 0; u < VPL; ++u) {
                const int vv = v0 + u * kWave + lane;
                if (vv < vend)
                    bstore16<Policy<kStream>::copy_store>(v[u], rd, (uint32_t)vv * 16u);
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
        const bool weighted = a.w != nullptr;
        // the first window's tile bases, loaded before the ids are read so
        // their latency overlaps the routing
        int bw[kExWindow / kWave];
#pragma unroll
        for (int w = 0; w < kExWindow / kWave; ++w)
            bw[w] = 64 * w + lane < a.Er ? a.tile_base[(lo + 64 * w + lane) * a.T + tile] : 0;
        // the row's distinct local experts in first-occurrence order; with one
        // mask word (Er <= 64) repeats are found in a register, else in LDS.
        // Weighted: an expert's weight is the sum, in slot order, of the
        // row's weights on the slots naming it.
        int n = 0;
        uint64_t seen = 0;
        for (int c = 0; c * KC < a.k; ++c) {
            int32_t id[KC];
            load_ids<KC>(ids, a.k, c, id);
            float wt[KC];
            if (weighted) {
#pragma unroll
                for (int i = 0; i < KC; ++i)
                    wt[i] = a.w[rowq * a.k + min(c * KC + i, a.k - 1)];
            }
#pragma unroll
            for (int i = 0; i < KC; ++i) {
                const int64_t j = (int64_t)id[i] - lo;
                if (!valid || c * KC + i >= a.k || j < 0 || j >= a.Er)
                    continue;
                bool dup;
                if (a.Er <= kWave) {
                    dup = (seen >> j) & 1;
                    seen |= 1ull << j;
                } else {
                    dup = false;
                    for (int u = 0; u < n; ++u)
                        dup = dup || s_j[lane][u] == (int)j;
                }
                if (!dup) {
                    if (weighted)
                        s_c[lane][n] = wt[i];
                    s_j[lane][n++] = (int)j;
                } else if (weighted) {
                    for (int u = 0; u < n; ++u)
                        if (s_j[lane][u] == (int)j)
                            s_c[lane][u] = s_c[lane][u] + wt[i];
                }
            }
        }
        // positions inside the tile, from LDS expert masks
        tile_positions<kExWindow / kWave>(
            s_j[lane], s_p[lane], n, a.Er, bw,
            [&](int j) { return a.tile_base[(lo + j) * a.T + tile]; }, s_bal, s_base);
        int kept = 0;  // positions past the capacity are dropped
        for (int u = 0; u < n; ++u) {
            const int p = s_p[lane][u];
            if (p < a.cap) {
                if (weighted)
                    s_c[lane][kept] = s_c[lane][u];
                s_p[lane][kept++] = (int32_t)((lo + s_j[lane][u]) * a.cap + p);
            }
        }
        s_n[lane] = kept;
    }
    __syncthreads();

    const int sd = a.scale_dwords;
    if (piece == 0) {
        for (int r = r_lo + wave; r < r_hi; r += nwaves) {
            const int64_t row = row0 + r;
            const int n = uniform(s_n[r]);
            if (lane < a.Pe) {
                a.efwd[row * a.Pe + lane] = lane < n ? s_p[r][lane] : -1;
                if (a.w)
                    a.ew[row * a.Pe + lane] = lane < n ? s_c[r][lane] : 0.0f;
            }
            if (lane < n)
                a.src_info[s_p[r][lane]] = a.src_pos[row] % a.WM;
            for (int c0 = 0; n > 0 && c0 < sd; c0 += kWave) {
                const int c = c0 + lane;
                const uint32_t v = c < sd ? a.sc[row * sd + c] : 0u;
                for (int i = 0; i < n; ++i) {
                    const int64_t gi = uniform(s_p[r][i]);
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
        // large pieces (throughput): one chunk a wave in flight, which keeps
        // the register count, and so the waves resident per SIMD, lowest
        for (int it = 0; it < items; ++it) {
            if (uniform(s_n[r_lo + wave + (it / nch) * nwaves]) == 0)
                continue;  // a row without a kept expert is not read
            load_item(it, A);
            store_item(it, A);
        }
    }
}

template <int G, int U, int DT, bool kStream, bool kWeighted>
__global__ __launch_bounds__(1024) void ex_combine_kernel(ExpertCombineArgs a)
{
    const int lane = threadIdx.x & (kWave - 1);
    // wave items: (row, piece); piece_inner: piece fastest, so a row's
    // pieces run in neighbouring waves
    const uint32_t item = blockIdx.x * (blockDim.x / kWave) + uniform(threadIdx.x / kWave);
    const uint32_t qu = a.piece_inner ? item / (uint32_t)a.pieces : item;
    const int d = blockIdx.z;
    if (qu >= (uint32_t)received(a.recv[d], a.rows))
        return;  // whole waves
    const int q = (int)qu;
    const int piece = a.piece_inner ? (int)(item - qu * (uint32_t)a.pieces) : (int)blockIdx.y;
    const int64_t row = (int64_t)d * a.WM + q;
    const int32_t gl = lane < a.Pe ? a.efwd[row * a.Pe + lane] : -1;
    const int n = __popcll(__ballot(gl >= 0));  // entries >= 0 form a prefix
    float gw = 0.0f;
    if constexpr (kWeighted)
        gw = lane < a.Pe ? a.ew[row * a.Pe + lane] : 0.0f;
    const uint32_t row_bytes = (uint32_t)a.row_vecs * 16u;
    const __amdgpu_buffer_rsrc_t rdst = row_rsrc(a.y + row * row_bytes, row_bytes);
    const int vbeg = piece * a.piece_vecs;
    const int vend = min(a.row_vecs, vbeg + a.piece_vecs);
    if constexpr (G == 0)
        fold_rows_streamed<U, DT, kStream, kWeighted>(a.py, row_bytes, gl, n, rdst, vbeg, vend,
                                                      lane, gw);
    else
        fold_rows<G, U, DT, kStream, kWeighted>(a.py, row_bytes, gl, n, rdst, vbeg, vend, lane,
                                                gw);
}

// Top-k bucket of the expert kernels: the smallest of 8, 16, 32, 64 >= k.
int ex_bucket(int k) { return k <= 8 ? 8 : k <= 16 ? 16 : k <= 32 ? 32 : 64; }

template <int VPL, int KB>
hipError_t ex_copy_with(const ExpertArgs& a, dim3 grid, dim3 block, bool stream, hipStream_t s)
{
    if (stream)
        hipLaunchKernelGGL((ex_copy_kernel<VPL, KB, true>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((ex_copy_kernel<VPL, KB, false>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <int VPL>
hipError_t ex_copy_with_vpl(const ExpertArgs& a, dim3 grid, dim3 block, bool stream,
                            hipStream_t s)
{
    switch (ex_bucket(a.k)) {
    case 8: return ex_copy_with<VPL, 8>(a, grid, block, stream, s);
    case 16: return ex_copy_with<VPL, 16>(a, grid, block, stream, s);
    case 32: return ex_copy_with<VPL, 32>(a, grid, block, stream, s);
    default: return ex_copy_with<VPL, 64>(a, grid, block, stream, s);
    }
}

template <int G, int U, int DT, bool kStream>
void ex_combine_launch(const ExpertCombineArgs& a, dim3 grid, dim3 block, hipStream_t s)
{
    if (a.ew)
        hipLaunchKernelGGL((ex_combine_kernel<G, U, DT, kStream, true>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((ex_combine_kernel<G, U, DT, kStream, false>), grid, block, 0, s, a);
}

template <int G, int U>
hipError_t ex_combine_with(const ExpertCombineArgs& a, int dtype, dim3 grid, dim3 block,
                           bool stream, hipStream_t s)
{
    if (dtype == 0) {
        if (stream)
            ex_combine_launch<G, U, 0, true>(a, grid, block, s);
        else
            ex_combine_launch<G, U, 0, false>(a, grid, block, s);
    } else {
        if (stream)
            ex_combine_launch<G, U, 1, true>(a, grid, block, s);
        else
            ex_combine_launch<G, U, 1, false>(a, grid, block, s);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_expert_count(const ExpertArgs& a, hipStream_t s)
{
    const dim3 grid((a.T + kExWaves - 1) / kExWaves, a.W);
    const dim3 block(kExWaves * kWave);
    switch (ex_bucket(a.k)) {
    case 8: hipLaunchKernelGGL((ex_count_kernel<8>), grid, block, 0, s, a); break;
    case 16: hipLaunchKernelGGL((ex_count_kernel<16>), grid, block, 0, s, a); break;
    case 32: hipLaunchKernelGGL((ex_count_kernel<32>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((ex_count_kernel<64>), grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_expert_count_scan(const ExpertArgs& a, hipStream_t s)
{
    const dim3 grid((unsigned)((int64_t)a.W * a.Er));
    const dim3 block(kCountScanTiles * kWave);
    switch (ex_bucket(a.k)) {
    case 8: hipLaunchKernelGGL((ex_count_scan_kernel<8>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((ex_count_scan_kernel<16>), grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_expert_scan(const ExpertArgs& a, hipStream_t s)
{
    const int64_t lists = (int64_t)a.W * a.Er;
    hipLaunchKernelGGL(ex_scan_kernel, dim3((unsigned)((lists + kExWaves - 1) / kExWaves)),
                       dim3(kExWaves * kWave), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_expert_copy(const ExpertArgs& a, int waves, int row_split, bool stream,
                              hipStream_t s)
{
    if (a.rows == 0)
        return hipSuccess;
    const dim3 grid(a.T * a.token_split, row_split, a.W);
    const dim3 block(waves * kWave);
    const int per_lane = (a.piece_vecs + kWave - 1) / kWave;
    if (per_lane <= 1)
        return ex_copy_with_vpl<1>(a, grid, block, stream, s);
    if (per_lane <= 2)
        return ex_copy_with_vpl<2>(a, grid, block, stream, s);
    if (per_lane <= 4)
        return ex_copy_with_vpl<4>(a, grid, block, stream, s);
    return ex_copy_with_vpl<8>(a, grid, block, stream, s);
}

hipError_t launch_expert_combine(const ExpertCombineArgs& a, int W, int dtype, int waves,
                                 bool stream, hipStream_t s)
{
    if (a.rows == 0)
        return hipSuccess;
    const dim3 grid = a.piece_inner
                          ? dim3((unsigned)(((int64_t)a.rows * a.pieces + waves - 1) / waves), 1, W)
                          : dim3((unsigned)((a.rows + waves - 1) / waves), (unsigned)a.pieces, W);
    const dim3 block(waves * kWave);
    // pieces of up to 2 KB: folded row by row (fold_rows_streamed)
    if (a.piece_vecs <= kWave)
        return ex_combine_with<0, 1>(a, dtype, grid, block, stream, s);
    if (a.piece_vecs <= 2 * kWave)
        return ex_combine_with<0, 2>(a, dtype, grid, block, stream, s);
    if (a.Pe <= 1)
        return ex_combine_with<1, 4>(a, dtype, grid, block, stream, s);
    if (a.Pe <= 2)
        return ex_combine_with<2, 4>(a, dtype, grid, block, stream, s);
    if (a.Pe <= 4)
        return ex_combine_with<4, kCombineColumns>(a, dtype, grid, block, stream, s);
    return ex_combine_with<kCombineGroup, kCombineColumns>(a, dtype, grid, block, stream, s);
}

}  // namespace ep
