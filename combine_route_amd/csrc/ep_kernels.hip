// gfx950 (MI355X, CDNA4) kernels of MoE expert-parallel dispatch and combine.
//
// The method ("feat(ep): add opt-in gfx1201 EP2/EP4 support", How the gfx1201
// kernels work): dispatch maps each token's top-k experts to destination
// ranks, keeps one row per (token, distinct rank), copies the payload and the
// routing metadata to it and records the way back; combine gathers each
// token's rows back, sums them in FP32 and casts to BF16/FP16.
//
// Kernels, all enqueued on the caller's stream, none waiting on another block
// or on a flag:
//   route    per routing tile (16..64 consecutive tokens of one rank) and
//            destination rank, the number of the tile's tokens that go there:
//            one 64-lane ballot per destination over the tokens' masks. For
//            k <= 16 one lane holds one token; for k > 16 the waves of a block
//            share the tile's tokens, one lane per top-k slot.
//   scan     one block per destination rank: exclusive prefix sum of the tile
//            counts in (source rank, tile) order -> first receive slot of every
//            tile on every rank, and the rank's received-row count. With the
//            in-tile ballot prefix this is a counting sort: rows on a rank are
//            ordered by (source rank, source token), and no atomic decides any
//            position. Calls of few tiles fold the scan into the copy kernel,
//            and tiny calls the counting too (LayoutMode).
//   copy     one block per (tile, row piece): routes its tile again (masks,
//            ordered rank lists and ballot prefixes into LDS), then every wave
//            loads a token's piece of the payload row into registers once (16 B
//            a lane) and stores it to each destination row; piece-0 blocks
//            also write the id, weight and scale rows, src_pos and the forward
//            map.
//   combine  one wave per (token, row piece): the token's forward-map entries
//            (at most min(W, k), one a lane) become scalar row numbers; for
//            each 16-byte column every contribution row is loaded before any
//            is added, then folded in the token's rank order in FP32, rounded
//            to nearest even by the hardware conversion, and stored.
//
// Rows move through per-row buffer resources (raw buffer loads and stores,
// 16 bytes a lane, 1 KiB a wave instruction): the cache policy is explicit,
// and the hardware range-checks each access against its own row.
//
// Pure data movement: no MFMA. Work is spread over source tokens (and row
// pieces for small calls), never over destinations, so routing skew does
// not serialise any block.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ep_device.h"
#include "ep_kernels.h"

namespace ep {
namespace {

using namespace dev;

constexpr int kMaxTile = 64;

// Rank r owning tile g: the largest r with tile_start[r] <= g (ranks without
// tiles share their start with the next rank and are skipped).
__device__ __forceinline__ int rank_of_tile(const TileMap& tm, int g)
{
    int lo = 0, hi = tm.W - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tm.tile_start[mid] <= g)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// Destination ranks of one token (one lane). Expert e is on rank e / Er; an id
// outside [0, E) selects none. With kList, the distinct ranks are written to
// list[] in the order their first expert appears in the top-k row. KB >= k is
// the top-k bucket: all KB ids are loaded at once, at addresses clamped into
// the row, so every load issues before any is waited on; ids past k are
// loaded but ignored.
template <bool kList, int KB>
__device__ __forceinline__ uint64_t route_token(const int32_t* row, bool valid, int k, int Er,
                                                int E, uint8_t* list, int& n)
{
    uint64_t m = 0;
    n = 0;
    if (!valid)
        return 0;
    auto take = [&](int32_t e) {
        if ((uint32_t)e < (uint32_t)E) {
            const uint32_t d = (uint32_t)e / (uint32_t)Er;
            const uint64_t bit = 1ull << d;
            if (!(m & bit)) {
                m |= bit;
                if constexpr (kList)
                    list[n] = (uint8_t)d;
                ++n;
            }
        }
    };
    if ((k & 3) == 0) {
        constexpr int NV = KB / 4;
        int4 v[NV];
#pragma unroll
        for (int q = 0; q < NV; ++q)
            v[q] = *reinterpret_cast<const int4*>(row + min(4 * q, k - 4));
#pragma unroll
        for (int q = 0; q < NV; ++q) {
            if (4 * q < k) {
                take(v[q].x);
                take(v[q].y);
                take(v[q].z);
                take(v[q].w);
            }
        }
    } else {
        int32_t v[KB];
#pragma unroll
        for (int q = 0; q < KB; ++q)
            v[q] = row[min(q, k - 1)];
#pragma unroll
        for (int q = 0; q < KB; ++q)
            if (q < k)
                take(v[q]);
    }
    return m;
}

// Routing of a tile's tokens for k > 16, spread over the waves of a block:
// wave w takes tokens w, w + nwaves, ... one at a time, with one lane per
// top-k slot (lane j holds id j). A token's distinct ranks come from a leader
// loop: the lowest lane not yet covered names the next rank, one ballot marks
// every slot on that rank, so each iteration finds one rank, in the order of
// first appearance. Writes the token's destination mask, rank count and (with
// kList) ordered ranks to LDS.
template <bool kList>
__device__ __forceinline__ void route_tile_by_slot(const int32_t* rows, int cnt, int k, int Er,
                                                   int E, uint8_t (*list)[kMaxRanks],
                                                   uint64_t* s_mask, int32_t* s_n)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    const int nwaves = blockDim.x / kWave;
    const int j = min(lane, k - 1);
    for (int tt = wave; tt < cnt; tt += nwaves) {
        const int32_t e = rows[(int64_t)tt * k + j];
        const bool valid = lane < k && (uint32_t)e < (uint32_t)E;
        const int d = valid ? (int)((uint32_t)e / (uint32_t)Er) : -1;
        uint64_t rem = __ballot(valid);
        uint64_t mask = 0;
        int n = 0;
        while (rem) {
            const int leader = __builtin_ctzll(rem);
            const int dl = __builtin_amdgcn_readlane(d, leader);
            rem &= ~__ballot(d == dl);
            if constexpr (kList) {
                if (lane == 0)
                    list[tt][n] = (uint8_t)dl;
            }
            mask |= 1ull << dl;
            ++n;
        }
        if (lane == 0) {
            s_mask[tt] = mask;
            s_n[tt] = n;
        }
    }
}

// ---------------------------------------------------------------------------
// route: per-tile row counts for every destination rank.
// ---------------------------------------------------------------------------
// k <= 16: one wave per tile, one lane per token. k > 16: one block per tile,
// its waves routing the tile's tokens one lane per top-k slot.
template <int KB>
__global__ __launch_bounds__(1024) void ep_route_kernel(RouteArgs a, TileMap tm)
{
    __shared__ uint64_t s_mask[kMaxTile];
    __shared__ int32_t s_n[kMaxTile];
    const int lane = threadIdx.x & (kWave - 1);
    const int g = KB >= 32 ? (int)blockIdx.x
                           : (int)(blockIdx.x * (blockDim.x / kWave) + uniform(threadIdx.x / kWave));
    if (g >= tm.total_tiles)
        return;  // whole waves only (one tile a block when k > 16)
    const int r = rank_of_tile(tm, g);
    const int t0 = (g - tm.tile_start[r]) * tm.tile_tokens;
    const int cnt = min(tm.tile_tokens, tm.ntok[r] - t0);
    uint64_t m;
    if constexpr (KB >= 32) {
        route_tile_by_slot<false>(a.idx + ((int64_t)r * a.M + t0) * a.k, cnt, a.k, a.Er, a.E,
                                  nullptr, s_mask, s_n);
        __syncthreads();
        if (threadIdx.x >= kWave)
            return;
        m = lane < cnt ? s_mask[lane] : 0;
    } else {
        int n;
        m = route_token<false, KB>(a.idx + ((int64_t)r * a.M + t0 + lane) * a.k, lane < cnt,
                                   a.k, a.Er, a.E, nullptr, n);
    }
    int mine = 0;
    for (int d = 0; d < tm.W; ++d) {
        const uint64_t b = __ballot((m >> d) & 1);
        if (lane == d)
            mine = __popcll(b);
    }
    if (lane < tm.W)
        a.tile_counts[(int64_t)lane * a.tile_stride + g] = mine;
}

// ---------------------------------------------------------------------------
// scan: exclusive prefix of one destination rank's tile counts.
// ---------------------------------------------------------------------------
constexpr int kScanThreads = 256;
constexpr int kScanPerThread = 4;

__global__ __launch_bounds__(kScanThreads) void ep_scan_kernel(ScanArgs a)
{
    __shared__ int32_t s_wave[kScanThreads / kWave];
    const int d = blockIdx.x;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    const int32_t* col = a.tile_counts + (int64_t)d * a.tile_stride;
    int32_t* out = a.tile_base + (int64_t)d * a.tile_stride;
    const int n = a.total_tiles;
    int32_t carry = 0;
    for (int base = 0; base < n; base += kScanThreads * kScanPerThread) {
        const int i0 = base + threadIdx.x * kScanPerThread;
        int32_t v[kScanPerThread];
        int32_t sum = 0;
#pragma unroll
        for (int q = 0; q < kScanPerThread; ++q) {
            v[q] = (i0 + q < n) ? col[i0 + q] : 0;
            sum += v[q];
        }
        // inclusive scan of the per-thread sums across the wave
        int32_t x = sum;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int32_t y = __shfl_up(x, off);
            if (lane >= off)
                x += y;
        }
        if (lane == kWave - 1)
            s_wave[wave] = x;
        __syncthreads();
        int32_t before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < kScanThreads / kWave; ++w) {
            before += (w < wave) ? s_wave[w] : 0;
            total += s_wave[w];
        }
        int32_t run = carry + before + x - sum;
#pragma unroll
        for (int q = 0; q < kScanPerThread; ++q) {
            if (i0 + q < n)
                out[i0 + q] = run;
            run += v[q];
        }
        carry += total;
        __syncthreads();
    }
    if (threadIdx.x == 0)
        a.recv[d] = carry;
}

// ---------------------------------------------------------------------------
// copy: payload rows, metadata rows, src_pos and the forward map.
// ---------------------------------------------------------------------------
// One work item of a wave: one chunk (up to 64 x VPL 16-byte vectors) of one
// token's row piece, and, for the first chunk of a piece-0 block, the lane's
// share of the token's id, weight and scale rows.
template <int VPL>
struct CopyItem {
    u32x4 v[VPL];
    int32_t e;
    float wv;
    uint32_t sc;
};

// kInCopy: the block counts every tile of the call itself (kLayoutInCopy, k <=
// 16 only); a separate instantiation, so the other calls do not carry its
// registers. kCast: the payload arrives as bf16 / fp16 (a.cast) and each
// element is received as its OCP E4M3 code (round to nearest even,
// saturating at 448): a vector is 8 elements, 16 bytes loaded (contiguous
// across the wave, as in the plain copy), converted once, and 8 bytes stored
// to each destination.
template <int VPL, int KB, bool kStream, bool kInCopy, bool kCast = false>
__global__ __launch_bounds__(1024) void ep_copy_kernel(CopyArgs a, TileMap tm)
{
    __shared__ uint8_t s_list[kMaxTile][kMaxRanks];  // [token][i]: i-th distinct rank
    __shared__ uint8_t s_loc[kMaxTile][kMaxRanks];   // [token][d]: rows to d before it in the tile
    __shared__ int32_t s_n[kMaxTile];                // distinct ranks of the token
    __shared__ int32_t s_base[kMaxRanks];            // first slot of this tile on rank d
    __shared__ uint64_t s_mask[KB >= 32 ? kMaxTile : 1];  // destination masks (k > 16)

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    const int nwaves = blockDim.x / kWave;
    const int piece = a.piece_inner ? (int)(blockIdx.x % a.pieces) : (int)blockIdx.y;
    const int tshare = a.piece_inner ? (int)(blockIdx.x / a.pieces) : (int)blockIdx.x;
    const int share = tshare % a.token_split;
    const int g = tshare / a.token_split;
    const int r = rank_of_tile(tm, g);
    const int t0 = (g - tm.tile_start[r]) * tm.tile_tokens;
    const int cnt = min(tm.tile_tokens, tm.ntok[r] - t0);
    // this block's tokens of the tile: [tb, te)
    const int per_share = (tm.tile_tokens + a.token_split - 1) / a.token_split;
    const int tb = min(cnt, share * per_share);
    const int te = min(cnt, tb + per_share);

    // This wave's items: tokens tb + wave, tb + wave + nwaves, ... of the
    // tile, each cut into nch chunks of its row piece [vbeg, vend).
    const int vbeg = piece * a.piece_vecs;
    const int vend = min(a.row_vecs, vbeg + a.piece_vecs);
    const int nch = (vend - vbeg + kWave * VPL - 1) / (kWave * VPL);
    const int ntw = wave < te - tb ? (te - tb - wave + nwaves - 1) / nwaves : 0;
    const int items = ntw * nch;
    const bool meta = piece == 0;
    const uint32_t in_bytes = (uint32_t)a.row_vecs * 16u;                  // input row
    const uint32_t row_bytes = kCast ? (uint32_t)a.row_vecs * 8u : in_bytes;  // received row
    const int k = a.k;
    const int per = kWave / k;  // destination id/weight rows per store instruction
    const int j = lane % k;
    const int sub = lane / k;
    const int sd = a.scale_dwords;

    // id, weight and scale rows, src_pos and forward map of one token, from
    // the lane's share (e, wv, sc) of its source rows
    auto store_meta = [&](int tok, int32_t e, float wv, uint32_t sc) {
        const int t = t0 + tok;
        const int64_t src = (int64_t)r * a.M + t;
        const int n = uniform(s_n[tok]);
        if (lane < a.P) {
            int32_t f = -1;
            if (lane < n) {
                const int d = s_list[tok][lane];
                f = d * a.WM + s_base[d] + s_loc[tok][d];
                a.src_pos[f] = r * a.WM + t;
            }
            a.fwd[src * a.P + lane] = f;
        }
        for (int i0 = 0; i0 < n; i0 += per) {
            const int i = i0 + sub;
            if (sub < per && i < n) {
                const int d = s_list[tok][i];
                const int64_t row = (int64_t)d * a.WM + s_base[d] + s_loc[tok][d];
                a.out_idx[row * k + j] = e;
                if (a.w)
                    a.out_w[row * k + j] = wv;
            }
        }
        for (int i = 0; i < n && sd > 0; ++i) {
            const int d = uniform(s_list[tok][i]);
            const int64_t row = (int64_t)d * a.WM + uniform(s_base[d] + s_loc[tok][d]);
            if (lane < sd)
                a.out_sc[row * sd + lane] = sc;
            for (int qd = kWave + lane; qd < sd; qd += kWave)  // scale rows past 64 words
                a.out_sc[row * sd + qd] = a.sc[src * sd + qd];
        }
    };
    auto load_meta = [&](int64_t src, int32_t& e, float& wv, uint32_t& sc) {
        if (sub < per) {
            e = a.idx[src * k + j];
            wv = a.w ? a.w[src * k + j] : 0.0f;
        }
        if (lane < sd)
            sc = a.sc[src * sd + lane];
    };
    // one chunk of a token's row piece to every destination row of the token
    auto store_payload = [&](int tok, int v0, const u32x4 (&raw)[VPL]) {
        const int n = uniform(s_n[tok]);
        u32x2 c[kCast ? VPL : 1];  // a cast's codes, converted once per chunk
        if constexpr (kCast) {
#pragma unroll
            for (int u = 0; u < VPL; ++u)
                c[u] = cast_e4m3(raw[u], a.cast);
        }
        auto store_to = [&](int i) {
            const int d = uniform(s_list[tok][i]);
            const int s = uniform(s_base[d] + s_loc[tok][d]);
            const __amdgpu_buffer_rsrc_t rd =
                row_rsrc(a.out_x + ((int64_t)d * a.WM + s) * row_bytes, row_bytes);
#pragma unroll
            for (int u = 0; u < VPL; ++u) {
                const int vv = v0 + u * kWave + lane;
                if (vv < vend) {
                    if constexpr (kCast)
                        __builtin_amdgcn_raw_buffer_store_b64(c[u], rd, (int)((uint32_t)vv * 8u),
                                                              0, Policy<kStream>::cast_store);
                    else
                        bstore16<Policy<kStream>::copy_store>(raw[u], rd, (uint32_t)vv * 16u);
                }
            }
        };
        // large pieces: the first destination outside the loop, so that each
        // of its stores waits for its own vector only
        int i0 = 0;
        if constexpr (VPL >= 8) {
            if (n > 0)
                store_to(0);
            i0 = 1;
        }
        for (int i = i0; i < n; ++i)
            store_to(i);
    };
    auto load_payload = [&](int64_t src, int v0, u32x4 (&v)[VPL]) {
        const __amdgpu_buffer_rsrc_t rs = row_rsrc(a.x + src * in_bytes, in_bytes);
        // Large pieces: every load issued (a vector past the piece reads zeros
        // from the row's end without touching memory), so that the stores can
        // wait for one vector at a time. Small pieces keep their guarded loads
        // (issuing all of them cost small calls about 2 us a copy).
#pragma unroll
        for (int u = 0; u < VPL; ++u) {
            const int vv = v0 + u * kWave + lane;
            if constexpr (VPL >= 8)
                v[u] = bload16<Policy<kStream>::copy_load>(rs, vv < vend ? (uint32_t)vv * 16u
                                                                         : in_bytes);
            else if (vv < vend)
                v[u] = bload16<Policy<kStream>::copy_load>(rs, (uint32_t)vv * 16u);
        }
    };
    auto load_item = [&](int it, CopyItem<VPL>& I) {
        const int q = it / nch;
        const int c = it - q * nch;
        const int64_t src = (int64_t)r * a.M + t0 + tb + wave + q * nwaves;
        load_payload(src, vbeg + c * kWave * VPL, I.v);
        if (meta && c == 0)
            load_meta(src, I.e, I.wv, I.sc);
    };
    auto store_item = [&](int it, const CopyItem<VPL>& I) {
        const int q = it / nch;
        const int c = it - q * nch;
        const int tok = tb + wave + q * nwaves;
        store_payload(tok, vbeg + c * kWave * VPL, I.v);
        if (meta && c == 0)
            store_meta(tok, I.e, I.wv, I.sc);
    };
    // First slot of this tile on every destination. Large calls read it from
    // the scan kernel. Calls of few tiles sum the per-tile counts before this
    // tile here; calls of few tokens (k <= 16) first count every tile of the
    // call here too, from the ids, into LDS (integer adds: the counts do not
    // depend on the order they arrive in). These sums are the same in every
    // block; block (0, 0) also writes the received-row counts. The sums are
    // spread over the waves, one destination each.
    auto tile_bases = [&]() {
        if (a.layout == kLayoutFromScan) {
            if (wave == 0 && lane < tm.W)
                s_base[lane] = a.tile_base[(int64_t)lane * a.tile_stride + g];
            return;
        }
        extern __shared__ int32_t s_cnt[];  // [total_tiles][W], kInCopy only
        if constexpr (kInCopy) {
            // a wave takes 64 / TT whole tiles a pass, a lane per token; a
            // tile's count on d is the popcount of its lanes' ballot bits
            const int TT = tm.tile_tokens;
            const int per_wave = kWave / TT;
            const int seg = lane / TT;
            const uint64_t seg_bits = TT == 64 ? ~0ull : ((1ull << TT) - 1);
            for (int g0 = wave * per_wave; g0 < tm.total_tiles; g0 += nwaves * per_wave) {
                const int tile = g0 + seg;
                int n;
                uint64_t m = 0;
                if (tile < tm.total_tiles) {
                    const int rr = rank_of_tile(tm, tile);
                    const int t = (tile - tm.tile_start[rr]) * TT + lane % TT;
                    m = route_token<false, KB>(a.idx + ((int64_t)rr * a.M + t) * k,
                                               t < tm.ntok[rr], k, a.Er, a.E, nullptr, n);
                }
                for (int d = 0; d < tm.W; ++d) {
                    const uint64_t b = __ballot((m >> d) & 1);
                    if (lane % TT == 0 && tile < tm.total_tiles)
                        s_cnt[tile * tm.W + d] = __popcll((b >> (seg * TT)) & seg_bits);
                }
            }
            __syncthreads();
        }
        const bool first = g == 0 && share == 0 && piece == 0;
        for (int d = wave; d < tm.W; d += nwaves) {
            const int32_t* col = a.tile_counts + (int64_t)d * a.tile_stride;
            int32_t before = 0, all = 0;
            for (int gg = lane; gg < (first ? tm.total_tiles : g); gg += kWave) {
                const int32_t c = kInCopy ? s_cnt[gg * tm.W + d] : col[gg];
                before += gg < g ? c : 0;
                all += c;
            }
#pragma unroll
            for (int off = kWave / 2; off > 0; off >>= 1) {
                before += __shfl_xor(before, off);
                all += __shfl_xor(all, off);
            }
            if (lane == 0) {
                s_base[d] = before;
                if (first)
                    a.recv[d] = all;
            }
        }
    };
    auto route_tile = [&]() {
        uint64_t m;
        if constexpr (KB >= 32) {
            // every wave routes some of the tile's tokens, then wave 0 ranks them
            route_tile_by_slot<true>(a.idx + ((int64_t)r * a.M + t0) * a.k, cnt, a.k, a.Er, a.E,
                                     s_list, s_mask, s_n);
            __syncthreads();
            if (wave != 0)
                return;
            m = lane < cnt ? s_mask[lane] : 0;
        } else {
            if (wave != 0)
                return;
            int n;
            m = route_token<true, KB>(a.idx + ((int64_t)r * a.M + t0 + lane) * a.k, lane < cnt,
                                      a.k, a.Er, a.E, s_list[lane], n);
            s_n[lane] = n;
        }
        for (int d = 0; d < tm.W; ++d) {
            const bool has = (m >> d) & 1;
            const uint64_t b = __ballot(has);
            if (has)
                s_loc[lane][d] = (uint8_t)lanes_below(b);
        }
    };

    if constexpr (VPL < 8) {
        // Small pieces (small calls, where time is latency): each wave's first
        // item loads while wave 0 routes the tile, then two items in flight,
        // item i+1 loading while item i stores.
        CopyItem<VPL> A, B;
        if (items > 0)
            load_item(0, A);
        tile_bases();
        route_tile();
        __syncthreads();
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
        // Large pieces (throughput): metadata first, then one chunk a wave in
        // flight, which keeps the register count, and so the waves resident
        // per SIMD, at its lowest.
        tile_bases();
        route_tile();
        __syncthreads();
        if (meta) {
            for (int tok = tb + wave; tok < te; tok += nwaves) {
                int32_t e = 0;
                float wv = 0.0f;
                uint32_t sc = 0;
                load_meta((int64_t)r * a.M + t0 + tok, e, wv, sc);
                store_meta(tok, e, wv, sc);
            }
        }
        for (int tok = tb + wave; tok < te; tok += nwaves) {
            const int64_t src = (int64_t)r * a.M + t0 + tok;
            for (int v0 = vbeg; v0 < vend; v0 += kWave * VPL) {
                u32x4 v[VPL];
                load_payload(src, v0, v);
                store_payload(tok, v0, v);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// combine: ordered FP32 gather-sum and RNE cast.
// ---------------------------------------------------------------------------
// G: contribution rows loaded before folding; U: 16-byte columns per lane in
// flight.
template <int G, int U, int DT, bool kStream>
__global__ __launch_bounds__(1024) void ep_combine_kernel(CombineArgs a, TokenMap tk)
{
    const int lane = threadIdx.x & (kWave - 1);
    // wave items: (token, piece); piece_inner: piece fastest, so a token's
    // pieces run in neighbouring waves
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

    const uint32_t row_bytes = (uint32_t)a.row_vecs * 16u;
    const __amdgpu_buffer_rsrc_t rdst = row_rsrc(a.out + tok * row_bytes, row_bytes);
    const int vbeg = piece * a.piece_vecs;
    const int vend = min(a.row_vecs, vbeg + a.piece_vecs);
    if constexpr (G == 0)
        fold_rows_streamed<U, DT, kStream>(a.y, row_bytes, gl, n, rdst, vbeg, vend, lane);
    else
        fold_rows<G, U, DT, kStream>(a.y, row_bytes, gl, n, rdst, vbeg, vend, lane);

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

// Top-k bucket of k: the smallest of 4, 8, 16, 32, 64 that holds it.
int topk_bucket(int k) { return k <= 4 ? 4 : k <= 8 ? 8 : k <= 16 ? 16 : k <= 32 ? 32 : 64; }

template <int VPL, int KB>
hipError_t copy_with(const CopyArgs& a, const TileMap& tm, dim3 grid, dim3 block, bool stream,
                     hipStream_t s)
{
    if (a.cast) {
        if (a.layout == kLayoutInCopy)
            return hipErrorInvalidValue;  // the host never selects it with a cast
        if (stream)
            hipLaunchKernelGGL((ep_copy_kernel<VPL, KB, true, false, true>), grid, block, 0, s,
                               a, tm);
        else
            hipLaunchKernelGGL((ep_copy_kernel<VPL, KB, false, false, true>), grid, block, 0, s,
                               a, tm);
        return hipGetLastError();
    }
    if constexpr (KB <= 16) {
        if (a.layout == kLayoutInCopy) {
            const size_t lds = sizeof(int32_t) * tm.total_tiles * tm.W;
            if (stream)
                hipLaunchKernelGGL((ep_copy_kernel<VPL, KB, true, true>), grid, block, lds, s, a,
                                   tm);
            else
                hipLaunchKernelGGL((ep_copy_kernel<VPL, KB, false, true>), grid, block, lds, s,
                                   a, tm);
            return hipGetLastError();
        }
    }
    if (a.layout == kLayoutInCopy)
        return hipErrorInvalidValue;  // k > 16: the host never selects it
    if (stream)
        hipLaunchKernelGGL((ep_copy_kernel<VPL, KB, true, false>), grid, block, 0, s, a, tm);
    else
        hipLaunchKernelGGL((ep_copy_kernel<VPL, KB, false, false>), grid, block, 0, s, a, tm);
    return hipGetLastError();
}

template <int VPL>
hipError_t copy_with_vpl(const CopyArgs& a, const TileMap& tm, dim3 grid, dim3 block,
                         bool stream, hipStream_t s)
{
    switch (topk_bucket(a.k)) {
    case 4: return copy_with<VPL, 4>(a, tm, grid, block, stream, s);
    case 8: return copy_with<VPL, 8>(a, tm, grid, block, stream, s);
    case 16: return copy_with<VPL, 16>(a, tm, grid, block, stream, s);
    case 32: return copy_with<VPL, 32>(a, tm, grid, block, stream, s);
    default: return copy_with<VPL, 64>(a, tm, grid, block, stream, s);
    }
}

template <int G, int U>
hipError_t combine_with(const CombineArgs& a, const TokenMap& tk, int dtype, dim3 grid,
                        dim3 block, bool stream, hipStream_t s)
{
    if (dtype == 0) {
        if (stream)
            hipLaunchKernelGGL((ep_combine_kernel<G, U, 0, true>), grid, block, 0, s, a, tk);
        else
            hipLaunchKernelGGL((ep_combine_kernel<G, U, 0, false>), grid, block, 0, s, a, tk);
    } else {
        if (stream)
            hipLaunchKernelGGL((ep_combine_kernel<G, U, 1, true>), grid, block, 0, s, a, tk);
        else
            hipLaunchKernelGGL((ep_combine_kernel<G, U, 1, false>), grid, block, 0, s, a, tk);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, const TileMap& tm, hipStream_t s)
{
    if (tm.total_tiles == 0)
        return hipSuccess;
    constexpr int kWaves = 4;  // k <= 16: tiles a block, one a wave
    const dim3 grid((tm.total_tiles + kWaves - 1) / kWaves);
    const dim3 block(kWaves * kWave);
    // k > 16: one tile a block, one wave per token of the tile (up to 16)
    const dim3 grid_tile(tm.total_tiles);
    const dim3 block_tile(min(tm.tile_tokens, 16) * kWave);
    switch (topk_bucket(a.k)) {
    case 4: hipLaunchKernelGGL((ep_route_kernel<4>), grid, block, 0, s, a, tm); break;
    case 8: hipLaunchKernelGGL((ep_route_kernel<8>), grid, block, 0, s, a, tm); break;
    case 16: hipLaunchKernelGGL((ep_route_kernel<16>), grid, block, 0, s, a, tm); break;
    case 32: hipLaunchKernelGGL((ep_route_kernel<32>), grid_tile, block_tile, 0, s, a, tm); break;
    default: hipLaunchKernelGGL((ep_route_kernel<64>), grid_tile, block_tile, 0, s, a, tm); break;
    }
    return hipGetLastError();
}

hipError_t launch_scan(const ScanArgs& a, int W, hipStream_t s)
{
    hipLaunchKernelGGL(ep_scan_kernel, dim3(W), dim3(kScanThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_copy(const CopyArgs& a, const TileMap& tm, int waves, bool stream,
                       hipStream_t s)
{
    if (tm.total_tiles == 0)
        return hipSuccess;
    const int64_t tshares = (int64_t)tm.total_tiles * a.token_split;
    const dim3 grid = a.piece_inner ? dim3((unsigned)(tshares * a.pieces))
                                    : dim3((unsigned)tshares, (unsigned)a.pieces);
    const dim3 block(waves * kWave);
    const int per_lane = (a.piece_vecs + kWave - 1) / kWave;
    if (per_lane <= 1)
        return copy_with_vpl<1>(a, tm, grid, block, stream, s);
    if (per_lane <= 2)
        return copy_with_vpl<2>(a, tm, grid, block, stream, s);
    if (per_lane <= 4)
        return copy_with_vpl<4>(a, tm, grid, block, stream, s);
    return copy_with_vpl<8>(a, tm, grid, block, stream, s);
}

hipError_t launch_combine(const CombineArgs& a, const TokenMap& tk, int dtype, int waves,
                          bool stream, hipStream_t s)
{
    if (tk.total == 0)
        return hipSuccess;
    const dim3 grid = a.piece_inner
                          ? dim3((unsigned)(((int64_t)tk.total * a.pieces + waves - 1) / waves))
                          : dim3((unsigned)((tk.total + waves - 1) / waves), (unsigned)a.pieces);
    const dim3 block(waves * kWave);
    // pieces of up to 2 KB: folded row by row (fold_rows_streamed)
    if (a.piece_vecs <= kWave)
        return combine_with<0, 1>(a, tk, dtype, grid, block, stream, s);
    if (a.piece_vecs <= 2 * kWave)
        return combine_with<0, 2>(a, tk, dtype, grid, block, stream, s);
    if (a.P <= 1)
        return combine_with<1, 4>(a, tk, dtype, grid, block, stream, s);
    if (a.P <= 2)
        return combine_with<2, 4>(a, tk, dtype, grid, block, stream, s);
    if (a.P <= 4)
        return combine_with<4, kCombineColumns>(a, tk, dtype, grid, block, stream, s);
    return combine_with<kCombineGroup, kCombineColumns>(a, tk, dtype, grid, block, stream, s);
}

}  // namespace ep
