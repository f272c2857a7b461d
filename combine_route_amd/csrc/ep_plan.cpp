// Host side of the C ABI in include/ep.h: configuration checks, workspace
// layouts, launch geometry, argument checks and kernel launches, for plans and
// the expert plans made from them.
//
// Every precondition is checked before anything is enqueued, and a failed
// check names the argument, as the gfx125x staging refactor does for an
// unbound or misaligned buffer ("refactor(EPv2): replace per-module __device__
// staging with shared buffer", Caller contract). Plans never allocate device
// memory: the caller's workspace holds all device state.
#include "ep.h"
#include "ep_probe.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "ep_kernels.h"
#include "ep_static.h"

namespace {

thread_local std::string g_error;

int fail(int code, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = buf;
    return code;
}

int ok()
{
    g_error.clear();
    return EP_OK;
}

constexpr size_t kWorkspaceAlign = 256;
// Upper bound of a call's payload rows (every token sent to min(W, k) ranks)
// at which its moves still use the caches: the 256 MB MALL of an MI355X.
constexpr int64_t kKeepBytes = 256ll << 20;
// Most routing tiles a call may have for the copy blocks to sum the tile
// counts themselves instead of a separate scan launch.
constexpr int kScanInCopyTiles = 256;
// Most tokens a call may have for every copy block to count all its tiles
// itself: each block reads every id of the call, which beats a routing
// launch only for tiny calls (measured on MI355X: 2 x 16 tokens 17.5 -> 15.3
// us a call; 8 x 128 tokens 33.9 -> 38.0 us).
constexpr int64_t kLayoutInCopyTokens = 256;
constexpr size_t kPtrAlign = 16;
constexpr int kTimerPool = 1024;
constexpr int kTimedKernels = 12;  // EP_KERNEL_ROUTE .. EP_KERNEL_STANDARD_COMBINE

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int elem_bytes(int dtype) { return dtype == EP_FP8_E4M3 ? 1 : 2; }

// Derived sizes of a configuration; valid only if check_config() passed.
struct Shape {
    int W, M, k, Er, P, H;
    int64_t E, WM;
    int64_t row_bytes;    // dispatch payload row as received
    int64_t x_bytes;      // dispatch payload row as sent (2H with a cast)
    int row_vecs;         // 16-byte vectors of an input row: the copy's work unit
    int64_t crow_bytes;   // combine row
    int64_t scale_bytes;  // scale row
    int tile_stride;      // tiles a rank-major tile array can need (tile 16)
    // workspace offsets
    size_t off_counts, off_base, off_src_pos, off_fwd, total;
};

int check_config(const ep_config_t* c, Shape* s)
{
    if (!c)
        return fail(EP_ERR_NULL, "cfg is NULL");
    if (c->world_size < 1 || c->world_size > ep::kMaxRanks)
        return fail(EP_ERR_ARG, "cfg.world_size = %d: must be in [1, %d]", c->world_size,
                    ep::kMaxRanks);
    if (c->max_num_inp_token_per_rank < 1)
        return fail(EP_ERR_ARG, "cfg.max_num_inp_token_per_rank = %d: must be >= 1",
                    c->max_num_inp_token_per_rank);
    if (c->num_experts_per_token < 1 || c->num_experts_per_token > ep::kMaxTopk)
        return fail(EP_ERR_ARG, "cfg.num_experts_per_token = %d: must be in [1, %d]",
                    c->num_experts_per_token, ep::kMaxTopk);
    if (c->num_experts_per_rank < 1)
        return fail(EP_ERR_ARG, "cfg.num_experts_per_rank = %d: must be >= 1",
                    c->num_experts_per_rank);
    if (c->dispatch_dtype != EP_BF16 && c->dispatch_dtype != EP_FP16 &&
        c->dispatch_dtype != EP_FP8_E4M3)
        return fail(EP_ERR_ARG, "cfg.dispatch_dtype = %d: must be EP_BF16, EP_FP16 or EP_FP8_E4M3",
                    c->dispatch_dtype);
    if (c->combine_dtype != EP_BF16 && c->combine_dtype != EP_FP16)
        return fail(EP_ERR_ARG, "cfg.combine_dtype = %d: must be EP_BF16 or EP_FP16",
                    c->combine_dtype);
    if (c->hidden_dim < 1)
        return fail(EP_ERR_ARG, "cfg.hidden_dim = %d: must be >= 1", c->hidden_dim);
    if (c->combine_wire < EP_WIRE_NONE || c->combine_wire > EP_WIRE_MXFP4)
        return fail(EP_ERR_ARG, "cfg.combine_wire = %d: must be an EP_WIRE_* value",
                    c->combine_wire);
    if (c->combine_wire == EP_WIRE_FP8_BLOCK128 && c->hidden_dim % 128 != 0)
        return fail(EP_ERR_ARG, "cfg.hidden_dim = %d: EP_WIRE_FP8_BLOCK128 needs a multiple of 128",
                    c->hidden_dim);
    if (c->combine_wire == EP_WIRE_MXFP4 && c->hidden_dim % 32 != 0)
        return fail(EP_ERR_ARG, "cfg.hidden_dim = %d: EP_WIRE_MXFP4 needs a multiple of 32",
                    c->hidden_dim);
    if (c->dispatch_cast < EP_CAST_NONE || c->dispatch_cast > EP_CAST_FP8_FROM_FP16)
        return fail(EP_ERR_ARG, "cfg.dispatch_cast = %d: must be an EP_CAST_* value",
                    c->dispatch_cast);
    if (c->dispatch_cast != EP_CAST_NONE && c->dispatch_dtype != EP_FP8_E4M3)
        return fail(EP_ERR_ARG, "cfg.dispatch_cast = %d needs dispatch_dtype = EP_FP8_E4M3",
                    c->dispatch_cast);
    const int64_t W = c->world_size, M = c->max_num_inp_token_per_rank;
    const int64_t row = (int64_t)c->hidden_dim * elem_bytes(c->dispatch_dtype);
    const int64_t crow = (int64_t)c->hidden_dim * 2;
    if (row % 16 != 0 || crow % 16 != 0)
        return fail(EP_ERR_ARG,
                    "cfg.hidden_dim = %d: payload (%lld B) and combine (%lld B) rows must be "
                    "multiples of 16 bytes",
                    c->hidden_dim, (long long)row, (long long)crow);
    if (row >= (int64_t)1 << 31 || crow >= (int64_t)1 << 31)
        return fail(EP_ERR_SIZE, "cfg.hidden_dim = %d: a row must stay below 2^31 bytes",
                    c->hidden_dim);
    if (c->scale_dim < 0)
        return fail(EP_ERR_ARG, "cfg.scale_dim = %d: must be >= 0", c->scale_dim);
    int64_t sbytes = 0;
    if (c->scale_dim > 0) {
        const int sts = c->scale_type_size;
        if (sts != 1 && sts != 2 && sts != 4 && sts != 8)
            return fail(EP_ERR_ARG, "cfg.scale_type_size = %d: must be 1, 2, 4 or 8", sts);
        sbytes = (int64_t)c->scale_dim * sts;
        if (sbytes % 4 != 0)
            return fail(EP_ERR_ARG,
                        "cfg.scale_dim * cfg.scale_type_size = %lld: must be a multiple of 4",
                        (long long)sbytes);
    }
    if (W * W * M > INT32_MAX)
        return fail(EP_ERR_SIZE,
                    "world_size^2 * max_num_inp_token_per_rank = %lld exceeds 2^31 - 1 "
                    "(int32 row numbers)",
                    (long long)(W * W * M));
    if (W * (int64_t)c->num_experts_per_rank > INT32_MAX)
        return fail(EP_ERR_SIZE, "world_size * num_experts_per_rank exceeds 2^31 - 1");

    s->W = (int)W;
    s->M = (int)M;
    s->k = c->num_experts_per_token;
    s->Er = c->num_experts_per_rank;
    s->P = std::min(s->W, s->k);
    s->H = c->hidden_dim;
    s->E = W * c->num_experts_per_rank;
    s->WM = W * M;
    s->row_bytes = row;
    s->x_bytes = c->dispatch_cast != EP_CAST_NONE ? crow : row;
    s->row_vecs = (int)(s->x_bytes / 16);  // 16-byte vectors of an input row
    s->crow_bytes = crow;
    s->scale_bytes = sbytes;
    const int64_t tiles_per_rank = (M + ep::kMinTile - 1) / ep::kMinTile;
    s->tile_stride = (int)(W * tiles_per_rank);
    size_t off = 0;
    s->off_counts = off;
    off = align_up(off + sizeof(int32_t) * (size_t)W * s->tile_stride, kWorkspaceAlign);
    s->off_base = off;
    off = align_up(off + sizeof(int32_t) * (size_t)W * s->tile_stride, kWorkspaceAlign);
    s->off_src_pos = off;
    off = align_up(off + sizeof(int32_t) * (size_t)W * s->WM, kWorkspaceAlign);
    s->off_fwd = off;
    off = align_up(off + sizeof(int32_t) * (size_t)W * M * s->P, kWorkspaceAlign);
    s->total = off;
    return EP_OK;
}

struct Timer {
    std::vector<hipEvent_t> start, stop;
    int next = 0;
    int32_t count = 0;
    double total_ms = 0.0;
};

}  // namespace

struct ep_plan {
    ep_config_t cfg;
    Shape s;
    uint8_t* ws;
    bool dispatched = false;
    int32_t last_ntok[ep::kMaxRanks] = {};
    hipStream_t last_stream = nullptr;
    bool launched = false;
    ep_launch_t launch = {};
    bool timing = false;
    Timer timers[kTimedKernels];
    uint64_t dispatch_gen = 0;  // successful dispatches so far
    int experts = 0;            // live expert plans made from this plan
    bool is_static = false;     // one of the per-device plans of ep_plan_static
};

// Workspace of an expert plan of capacity cap: per-tile expert counts and
// bases ([W * Er][T]), the first received row of each source rank ([W][W]),
// the in-tile prefixes there ([W * Er][W]), the inverse's map and its weights
// ([W][WM][Pe] each, Pe = min(k, Er)). The fused path uses the counts and
// bases as [W * Er][W * Tr] and the map's space as its per-slot map
// [W][M][k]; each region is sized for the larger use.
struct ExShape {
    int32_t cap;
    int Pe;
    int64_t T;   // tiles a rank can need: max(1, ceil(WM / 64))
    int64_t Tr;  // fused path: tiles a source rank can need, max(1, ceil(M / 64))
    size_t off_counts, off_base, off_start, off_prefix, off_efwd, off_ew, total;
};

struct ep_expert_plan {
    ep_plan* plan;
    ExShape e;
    uint8_t* ws;
    bool fused = false;                // the map holds the last fused dispatch's
    int32_t fused_ntok[ep::kMaxRanks] = {};
    bool converted = false;
    bool weighted = false;             // the conversion recorded expert weights
    uint64_t gen = 0;                  // the plan's dispatch that was converted
    const int32_t* recv = nullptr;     // its received-row counts
    int32_t rows = 0;                  // most rows a rank could hold in it
    hipStream_t last_stream = nullptr;
    bool launched = false;
};

namespace {

int expert_shape(const Shape& s, int32_t cap, ExShape* e)
{
    if (cap < 1 || cap > s.WM)
        return fail(EP_ERR_ARG, "cap = %d: must be in [1, W * M = %lld]", cap, (long long)s.WM);
    if ((int64_t)s.W * s.Er * cap > INT32_MAX)
        return fail(EP_ERR_SIZE, "W * num_experts_per_rank * cap exceeds 2^31 - 1 (packed rows "
                    "are int32 in the inverse's map)");
    e->cap = cap;
    e->Pe = std::min(s.k, s.Er);
    e->T = std::max<int64_t>(1, (s.WM + ep::kWave - 1) / ep::kWave);
    e->Tr = std::max<int64_t>(1, (s.M + ep::kWave - 1) / ep::kWave);
    const size_t lists = (size_t)s.W * (size_t)s.Er;
    const size_t tiles = std::max((size_t)e->T, (size_t)s.W * (size_t)e->Tr);
    size_t off = 0;
    e->off_counts = off;
    off = align_up(off + sizeof(int32_t) * lists * tiles, kWorkspaceAlign);
    e->off_base = off;
    off = align_up(off + sizeof(int32_t) * lists * tiles, kWorkspaceAlign);
    e->off_start = off;
    off = align_up(off + sizeof(int32_t) * (size_t)s.W * (size_t)s.W, kWorkspaceAlign);
    e->off_prefix = off;
    off = align_up(off + sizeof(int32_t) * lists * (size_t)s.W, kWorkspaceAlign);
    e->off_efwd = off;
    off = align_up(off + sizeof(int32_t) * std::max((size_t)s.W * (size_t)s.WM * (size_t)e->Pe,
                                                    (size_t)s.W * (size_t)s.M * (size_t)s.k),
                   kWorkspaceAlign);
    e->off_ew = off;
    off = align_up(off + sizeof(float) * (size_t)s.W * (size_t)s.WM * (size_t)e->Pe,
                   kWorkspaceAlign);
    e->total = off;
    return EP_OK;
}

int32_t* ws_counts(ep_plan* p) { return reinterpret_cast<int32_t*>(p->ws + p->s.off_counts); }
int32_t* ws_base(ep_plan* p) { return reinterpret_cast<int32_t*>(p->ws + p->s.off_base); }
int32_t* ws_src_pos(const ep_plan* p)
{
    return reinterpret_cast<int32_t*>(p->ws + p->s.off_src_pos);
}
int32_t* ws_fwd(ep_plan* p) { return reinterpret_cast<int32_t*>(p->ws + p->s.off_fwd); }

// Whether the copy blocks can count every tile of a call themselves: a lane
// per token reads whole id rows (k <= 16), and the counters fit in LDS.
bool layout_in_copy_fits(const ep_plan* p, int ntiles)
{
    const Shape& s = p->s;
    return s.k <= 16 && (int64_t)ntiles * s.W <= ep::kLayoutInCopyCells &&
           p->cfg.dispatch_cast == EP_CAST_NONE;
}

// Most rows any rank can receive from a dispatch of these token counts: a
// token goes at most once to a rank.
int64_t expert_rows(const Shape& s, const int32_t* ntok)
{
    int64_t N = 0;
    for (int r = 0; r < s.W; ++r)
        N += ntok[r];
    return std::min<int64_t>(s.WM, N);
}

// 64-row tiles per rank of the expert-major layout (at least one, so the
// counts and ranges are written even when nothing was received).
int expert_tiles(int64_t rows) { return (int)std::max<int64_t>(1, (rows + ep::kWave - 1) / ep::kWave); }

// Where each rank's tokens start in the flat list of all tokens.
void token_map(const Shape& s, const int32_t* ntok, ep::TokenMap* tk)
{
    *tk = {};
    tk->W = s.W;
    int total = 0;
    for (int r = 0; r < s.W; ++r) {
        tk->tok_start[r] = total;
        total += ntok[r];
    }
    tk->tok_start[s.W] = total;
    tk->total = total;
}

int tiles_for(const int32_t* ntok, int W, int tt)
{
    int n = 0;
    for (int r = 0; r < W; ++r)
        n += (ntok[r] + tt - 1) / tt;
    return n;
}

// Calls of at least 512 tiles of 32 tokens (the automatic geometry's large
// calls) have more blocks than the GPU holds at once: their copy and combine
// grids number the row pieces fastest, so the blocks that run together move
// neighbouring rows. In smaller calls every block is resident from the start
// and that order measured slower (MI355X, 8 x 128 fp8 tokens: combine 18.3 ->
// 20.6 us; 4 x ~1024 top-64 tokens: copy 18.8 -> 20.0 us), so they keep the
// piece in grid y.
bool large_call(const Shape& s, const int32_t* ntok) { return tiles_for(ntok, s.W, 32) >= 512; }

// The grid of an expert-major copy (ep_convert_dispatch_output's over tiles
// of 64 received rows, ep_dispatch_standard_moe's over tiles of 64 source
// tokens): each row cut into pieces and each tile's rows shared by blocks
// until the grid has about a target number of blocks, 1024 up to top-16 and
// 512 above (every block routes its whole tile, which costs more the more
// ids a row has). Calls whose row pieces alone reach the target cut rows to
// reach it and, up to top-16, share each tile among blocks of one row a wave:
// the blocks the GPU starts together then hold neighbouring rows rather than
// rows a tile apart (measured on MI355X, 8 x 4096 tokens, 14 KB rows, top-8:
// expert-major copy 1299 -> 1232 us, fused copy 881 -> 870 us). Smaller calls
// share tiles first (at most one row a wave), then cut rows. A value the
// launch overrides give (row_split, token_split > 0) is kept.
struct ShareGrid {
    int row_split, token_split;
};

ShareGrid share_grid(int64_t tiles, int64_t row_vecs, int k, int waves, int row_split,
                     int token_split)
{
    tiles = std::max<int64_t>(1, tiles);
    const int64_t target = k <= 16 ? 1024 : 512;
    const int max_split = (int)std::min<int64_t>(65535, std::max<int64_t>(1, row_vecs / ep::kWave));
    const int max_share = std::max(1, ep::kWave / std::max(1, waves));
    auto want = [&](int64_t blocks) { return std::max<int64_t>(1, (target + blocks - 1) / blocks); };
    ShareGrid g{row_split, token_split};
    if (g.row_split <= 0 && g.token_split <= 0 && tiles * max_split >= target) {
        g.row_split = (int)std::min<int64_t>(max_split, want(tiles));
        g.token_split = k <= 16 ? max_share : 1;
    }
    if (g.token_split <= 0)
        g.token_split = (int)std::min<int64_t>(max_share, want(tiles * std::max(1, g.row_split)));
    if (g.row_split <= 0)
        g.row_split = (int)std::min<int64_t>(max_split, want(tiles * g.token_split));
    return g;
}

// Tiles of 64 source tokens of a fused dispatch.
int64_t fused_tiles(const Shape& s, const int32_t* ntok)
{
    int64_t tiles = 0;
    for (int r = 0; r < s.W; ++r)
        tiles += (ntok[r] + ep::kWave - 1) / ep::kWave;
    return tiles;
}

// Automatic geometry. Small calls get smaller routing tiles and rows split
// into pieces so that the grid still covers the 256 compute units several
// times over, as the gfx1201 kernels do below 256 tokens ("feat(ep): add
// opt-in gfx1201 EP2/EP4 support", How the gfx1201 kernels work: hidden tiles
// of 512 or 1024 elements).
// Smallest row piece the automatic dispatch geometry cuts for large calls.
constexpr int64_t kMinPieceBytes = 7168;
// Wire codes a combine wave folds in large calls: ep_combine's wire combine,
// and ep_combine_standard_moe's from wire rows.
constexpr int64_t kWirePieceBytes = 1792;
constexpr int64_t kStandardWirePieceBytes = 3584;

// Bytes of one wire row's codes (not its scales); 0 without a wire.
int64_t wire_row_bytes(const ep_plan* p)
{
    const int64_t H = p->s.H;
    return p->cfg.combine_wire == EP_WIRE_FP8_BLOCK128 ? H
           : p->cfg.combine_wire == EP_WIRE_MXFP4      ? H / 2
                                                        : 0;
}

ep_launch_t auto_launch(const ep_plan* p, const int32_t* ntok)
{
    const Shape& s = p->s;
    int64_t N = 0;
    for (int r = 0; r < s.W; ++r)
        N += ntok[r];
    ep_launch_t l;
    constexpr int kTargetBlocks = 1024;
    l.tile_tokens = 16;
    for (int tt : {64, 32}) {
        if (tiles_for(ntok, s.W, tt) >= 512) {
            l.tile_tokens = tt;
            break;
        }
    }
    const int tiles = std::max(1, tiles_for(ntok, s.W, l.tile_tokens));
    const int64_t row_vecs = s.row_vecs;
    const int64_t max_split = std::max<int64_t>(1, row_vecs / ep::kWave);
    if (l.tile_tokens == 16) {
        // small calls: time is load latency; a wave per token keeps every
        // token's loads in flight at once, and rows are cut until the grid
        // covers the compute units several times over
        l.dispatch_waves = 16;
        l.dispatch_token_split = 1;
        l.dispatch_row_split = (int)std::min<int64_t>(
            std::min<int64_t>(max_split, 65535), std::max(1, (kTargetBlocks + tiles - 1) / tiles));
    } else {
        // large calls: rows cut into pieces of at least 7 KB (smaller pieces
        // lose more to the extra blocks than they gain), and up to top-16
        // each tile shared among blocks of one token a wave, so the blocks
        // the GPU starts together hold neighbouring tokens rather than tokens
        // a tile apart (every block routes its whole tile, too costly for
        // more ids a token). Measured on MI355X, 8 x 4096 tokens, top-8, copy
        // kernel us, old rule -> this one: 14 KB bf16 rows 619 -> 592, 7 KB
        // fp8 rows 346 -> 308, 8 KB rows 384 -> 353, bf16 -> E4M3 cast 376 ->
        // 337 (16 waves); 4 x 4096 tokens, top-64, 4 KB rows: 84 -> 66. The
        // cast takes 4 waves as well now that its large pieces keep their
        // loads in flight together (it had waited for each load before
        // issuing the next): 330-334 us with 4 or 16 waves.
        const bool share = s.k <= 16;
        l.dispatch_waves = !share ? (l.tile_tokens >= 64 ? 8 : 16) : 4;
        l.dispatch_token_split = share ? l.tile_tokens / l.dispatch_waves : 1;
        l.dispatch_row_split = (int)std::min<int64_t>(
            max_split, std::max<int64_t>(1, row_vecs * 16 / kMinPieceBytes));
    }
    l.combine_waves = 4;
    const int64_t cblocks = std::max<int64_t>(1, (N + l.combine_waves - 1) / l.combine_waves);
    const int64_t crow_vecs = s.crow_bytes / 16;
    const int64_t cmax_split = std::max<int64_t>(1, crow_vecs / ep::kWave);
    l.combine_row_split = (int)std::min<int64_t>(
        std::min<int64_t>(cmax_split, 65535),
        std::max<int64_t>(1, (kTargetBlocks + cblocks - 1) / cblocks));
    if (l.tile_tokens == 16 && p->cfg.combine_wire == EP_WIRE_NONE) {
        // small calls: pieces of at most 2 KB, folded row by row (8 x 128
        // fp8 tokens, bf16 combine: 33.2 -> 32.6 us a call)
        l.combine_row_split = (int)std::min<int64_t>(
            cmax_split, std::max<int64_t>(l.combine_row_split, (s.crow_bytes + 2047) / 2048));
    }
    if (l.tile_tokens > 16 && p->cfg.combine_wire == EP_WIRE_NONE) {
        // large calls: 1 KB pieces (a wave's columns, folded row by row) and
        // 16 waves a block; a token's pieces run in neighbouring waves, so
        // each contribution row is read whole at about the same time.
        // Measured on MI355X, combine kernel us, old rule (4 waves, whole
        // rows) -> this one: 8 x 4096 tokens, top-8, 14 KB rows 558 -> 471,
        // 8 KB rows 308 -> 273; 8 x 2048 tokens, 14 KB rows 280 -> 235;
        // 4 x 4096 tokens, top-64, 4 KB rows 58 -> 56.
        l.combine_waves = 16;
        l.combine_row_split = (int)cmax_split;
    } else if (l.tile_tokens > 16) {
        // large calls from wire rows: pieces of about 1.75 KB of codes, 4
        // waves a block (8 x 4096 tokens, top-8, H = 7168: FP8 block-128
        // 327 -> 288 us, MXFP4 214 -> 203 us)
        l.combine_waves = 4;
        l.combine_row_split = (int)std::max<int64_t>(1, wire_row_bytes(p) / kWirePieceBytes);
    }
    // rows one call moves at most (every token sent to min(W, k) ranks)
    const int64_t rows_bytes = N * (s.row_bytes + s.crow_bytes) * (1 + s.P);
    l.cache_policy = rows_bytes <= kKeepBytes ? EP_CACHE_KEEP : EP_CACHE_STREAM;
    // few tiles: the copy blocks work out the receive slots themselves
    const int ntiles = tiles_for(ntok, s.W, l.tile_tokens);
    if (ntiles >= 1 && N <= kLayoutInCopyTokens && layout_in_copy_fits(p, ntiles))
        l.layout = EP_LAYOUT_IN_COPY;
    else if (ntiles >= 1 && ntiles <= kScanInCopyTiles)
        l.layout = EP_LAYOUT_SCAN_IN_COPY;
    else
        l.layout = EP_LAYOUT_KERNELS;
    // expert-major layout: 64 received rows a copy tile (share_grid), a row
    // a wave in the inverse, pieces until the grid has about kTargetBlocks
    // blocks
    const int64_t rows = expert_rows(s, ntok);
    l.expert_waves = 8;
    const ShareGrid eg = share_grid((int64_t)s.W * expert_tiles(rows), s.row_bytes / 16, s.k,
                                    l.expert_waves, 0, 0);
    l.expert_row_split = eg.row_split;
    l.expert_token_split = eg.token_split;
    l.expert_combine_waves = 4;
    const int64_t iblocks = std::max<int64_t>(1, s.W * ((rows + 3) / 4));
    l.expert_combine_row_split = (int)std::min<int64_t>(
        std::min<int64_t>(cmax_split, 65535), std::max<int64_t>(1, (kTargetBlocks + iblocks - 1) / iblocks));
    if (l.tile_tokens > 16) {
        // large calls: as the combine, 1 KB pieces and 16 waves a block
        l.expert_combine_waves = 16;
        l.expert_combine_row_split = (int)cmax_split;
    }
    // rows these calls move at most: N * min(W, k) received rows read and
    // N * k (row, expert) pairs written, and the same counts of expert
    // output rows on the way back. The rows they read were just written (by
    // the dispatch, by the experts), so cached moves pay off up to twice the
    // MALL (measured on MI355X: 8 x 128 fp8 tokens, bound 352 MB, 65 us
    // cached vs 85 us streaming; 4 x ~600 top-64 tokens, bound 1.3 GB, 375 us
    // cached vs 317 us streaming).
    const int64_t ex_bytes = N * (s.row_bytes + s.crow_bytes) * (s.P + s.k);
    l.expert_cache_policy = ex_bytes <= 2 * kKeepBytes ? EP_CACHE_KEEP : EP_CACHE_STREAM;
    return l;
}

ep_launch_t effective_launch(const ep_plan* p, const int32_t* ntok)
{
    ep_launch_t l = auto_launch(p, ntok);
    if (p->launch.tile_tokens > 0)
        l.tile_tokens = p->launch.tile_tokens;
    if (p->launch.dispatch_waves > 0)
        l.dispatch_waves = p->launch.dispatch_waves;
    if (p->launch.dispatch_row_split > 0)
        l.dispatch_row_split = p->launch.dispatch_row_split;
    if (p->launch.combine_waves > 0)
        l.combine_waves = p->launch.combine_waves;
    if (p->launch.combine_row_split > 0)
        l.combine_row_split = p->launch.combine_row_split;
    if (p->launch.cache_policy > 0)
        l.cache_policy = p->launch.cache_policy;
    if (p->launch.layout > 0)
        l.layout = p->launch.layout;
    if (p->launch.expert_waves > 0)
        l.expert_waves = p->launch.expert_waves;
    if (p->launch.expert_row_split > 0)
        l.expert_row_split = p->launch.expert_row_split;
    if (p->launch.expert_combine_waves > 0)
        l.expert_combine_waves = p->launch.expert_combine_waves;
    if (p->launch.expert_combine_row_split > 0)
        l.expert_combine_row_split = p->launch.expert_combine_row_split;
    if (p->launch.expert_cache_policy > 0)
        l.expert_cache_policy = p->launch.expert_cache_policy;
    if (p->launch.expert_token_split > 0)
        l.expert_token_split = p->launch.expert_token_split;
    if (p->launch.dispatch_token_split > 0)
        l.dispatch_token_split = p->launch.dispatch_token_split;
    else if (l.dispatch_token_split > 1)
        // a shared tile stays one token a wave under overridden tiles or waves
        l.dispatch_token_split = std::max(1, l.tile_tokens / l.dispatch_waves);
    return l;
}

void timer_drain(Timer& t)
{
    for (int i = 0; i < t.next; ++i) {
        float ms = 0.f;
        if (hipEventSynchronize(t.stop[i]) == hipSuccess &&
            hipEventElapsedTime(&ms, t.start[i], t.stop[i]) == hipSuccess) {
            t.total_ms += ms;
            t.count += 1;
        }
    }
    t.next = 0;
}

void timers_destroy(ep_plan* p)
{
    for (Timer& t : p->timers) {
        for (hipEvent_t e : t.start)
            (void)hipEventDestroy(e);
        for (hipEvent_t e : t.stop)
            (void)hipEventDestroy(e);
        t = Timer();
    }
}

// Launch one kernel, bracketed by timing events when enabled.
template <typename F>
hipError_t timed(ep_plan* p, int kernel, hipStream_t stream, F&& launch)
{
    if (!p->timing)
        return launch();
    Timer& t = p->timers[kernel];
    if (t.next == (int)t.start.size())
        timer_drain(t);
    hipError_t e = hipEventRecord(t.start[t.next], stream);
    if (e != hipSuccess)
        return e;
    e = launch();
    if (e != hipSuccess)
        return e;
    e = hipEventRecord(t.stop[t.next], stream);
    if (e == hipSuccess)
        t.next += 1;
    return e;
}

int check_launch(const ep_plan* p, const ep_launch_t* l)
{
    const Shape& s = p->s;
    if (l->tile_tokens > 0 && l->tile_tokens != 16 && l->tile_tokens != 32 && l->tile_tokens != 64)
        return fail(EP_ERR_ARG, "launch.tile_tokens = %d: must be 16, 32 or 64", l->tile_tokens);
    if (l->dispatch_waves > 16)
        return fail(EP_ERR_ARG, "launch.dispatch_waves = %d: must be <= 16", l->dispatch_waves);
    if (l->combine_waves > 16)
        return fail(EP_ERR_ARG, "launch.combine_waves = %d: must be <= 16", l->combine_waves);
    if (l->layout < 0 || l->layout > EP_LAYOUT_IN_COPY)
        return fail(EP_ERR_ARG, "launch.layout = %d: must be an EP_LAYOUT_* value", l->layout);
    if (l->layout == EP_LAYOUT_IN_COPY && s.k > 16)
        return fail(EP_ERR_ARG, "launch.layout = EP_LAYOUT_IN_COPY needs num_experts_per_token "
                    "<= 16 (it is %d)", s.k);
    if (l->layout == EP_LAYOUT_IN_COPY && p->cfg.dispatch_cast != EP_CAST_NONE)
        return fail(EP_ERR_ARG, "launch.layout = EP_LAYOUT_IN_COPY is not available with a "
                    "dispatch_cast");
    if (l->cache_policy < 0 || l->cache_policy > EP_CACHE_KEEP)
        return fail(EP_ERR_ARG, "launch.cache_policy = %d: must be EP_CACHE_AUTO, "
                    "EP_CACHE_STREAM or EP_CACHE_KEEP", l->cache_policy);
    if (l->expert_cache_policy < 0 || l->expert_cache_policy > EP_CACHE_KEEP)
        return fail(EP_ERR_ARG, "launch.expert_cache_policy = %d: must be EP_CACHE_AUTO, "
                    "EP_CACHE_STREAM or EP_CACHE_KEEP", l->expert_cache_policy);
    if (l->dispatch_row_split > 65535 || l->combine_row_split > 65535)
        return fail(EP_ERR_ARG, "launch row splits must be <= 65535 (grid y limit)");
    if (l->dispatch_row_split > s.row_vecs)
        return fail(EP_ERR_ARG, "launch.dispatch_row_split = %d: must be <= %d",
                    l->dispatch_row_split, s.row_vecs);
    if (l->combine_row_split > s.crow_bytes / 16)
        return fail(EP_ERR_ARG, "launch.combine_row_split = %d: must be <= %lld",
                    l->combine_row_split, (long long)(s.crow_bytes / 16));
    if (l->expert_waves > 16)
        return fail(EP_ERR_ARG, "launch.expert_waves = %d: must be <= 16", l->expert_waves);
    if (l->expert_combine_waves > 16)
        return fail(EP_ERR_ARG, "launch.expert_combine_waves = %d: must be <= 16",
                    l->expert_combine_waves);
    if (l->expert_row_split > 65535 || l->expert_combine_row_split > 65535)
        return fail(EP_ERR_ARG, "launch expert row splits must be <= 65535 (grid y limit)");
    if (l->expert_row_split > s.row_bytes / 16)
        return fail(EP_ERR_ARG, "launch.expert_row_split = %d: must be <= %lld",
                    l->expert_row_split, (long long)(s.row_bytes / 16));
    if (l->expert_combine_row_split > s.crow_bytes / 16)
        return fail(EP_ERR_ARG, "launch.expert_combine_row_split = %d: must be <= %lld",
                    l->expert_combine_row_split, (long long)(s.crow_bytes / 16));
    if (l->expert_token_split > ep::kWave)
        return fail(EP_ERR_ARG, "launch.expert_token_split = %d: must be <= %d",
                    l->expert_token_split, ep::kWave);
    if (l->dispatch_token_split > ep::kWave)
        return fail(EP_ERR_ARG, "launch.dispatch_token_split = %d: must be <= %d",
                    l->dispatch_token_split, ep::kWave);
    return EP_OK;
}

}  // namespace

extern "C" {

size_t ep_workspace_bytes(const ep_config_t* cfg)
{
    Shape s;
    if (check_config(cfg, &s) != EP_OK)
        return 0;
    ok();
    return s.total;
}

int ep_plan_create(const ep_config_t* cfg, void* workspace, size_t workspace_bytes,
                   ep_plan_t** out)
{
    Shape s;
    int rc = check_config(cfg, &s);
    if (rc != EP_OK)
        return rc;
    if (!workspace)
        return fail(EP_ERR_NULL, "workspace is NULL");
    if (!out)
        return fail(EP_ERR_NULL, "out is NULL");
    if (!aligned(workspace, kWorkspaceAlign))
        return fail(EP_ERR_ALIGN, "workspace %p is not %zu-byte aligned", workspace,
                    kWorkspaceAlign);
    if (workspace_bytes < s.total)
        return fail(EP_ERR_SIZE, "workspace_bytes = %zu: ep_workspace_bytes() requires %zu",
                    workspace_bytes, s.total);
    ep_plan* p = new (std::nothrow) ep_plan();
    if (!p)
        return fail(EP_ERR_SIZE, "out of host memory for the plan");
    p->cfg = *cfg;
    p->s = s;
    p->ws = static_cast<uint8_t*>(workspace);
    *out = p;
    return ok();
}

int ep_plan_destroy(ep_plan_t* p)
{
    if (!p)
        return ok();
    if (p->experts > 0)
        return fail(EP_ERR_STATE, "%d expert plan(s) made from this plan still exist: destroy "
                    "them first", p->experts);
    int rc = EP_OK;
    if (p->launched) {
        const hipError_t e = hipStreamSynchronize(p->last_stream);
        if (e != hipSuccess)
            rc = fail(EP_ERR_HIP, "hipStreamSynchronize before destroy: %s", hipGetErrorString(e));
    }
    timers_destroy(p);
    if (p->is_static) {          // the library's own object: emptied, not freed
        p->dispatched = p->launched = false;
        p->last_stream = nullptr;
    } else {
        delete p;
    }
    return rc == EP_OK ? ok() : rc;
}



int ep_dispatch(ep_plan_t* p, const ep_dispatch_args_t* a, void* stream_ptr)
{
    if (!p)
        return fail(EP_ERR_NULL, "plan is NULL");
    if (!a)
        return fail(EP_ERR_NULL, "args is NULL");
    const Shape& s = p->s;
    if (!a->num_tokens)
        return fail(EP_ERR_NULL, "args.num_tokens is NULL");
    for (int r = 0; r < s.W; ++r)
        if (a->num_tokens[r] < 0 || a->num_tokens[r] > s.M)
            return fail(EP_ERR_ARG, "args.num_tokens[%d] = %d: must be in [0, %d]", r,
                        a->num_tokens[r], s.M);
    struct {
        const void* ptr;
        const char* name;
    } req[] = {{a->x, "args.x"},
               {a->indices, "args.indices"},
               {a->out_x, "args.out_x"},
               {a->out_indices, "args.out_indices"},
               {a->recv_num_token, "args.recv_num_token"}};
    for (auto& q : req) {
        if (!q.ptr)
            return fail(EP_ERR_NULL, "%s is NULL", q.name);
        if (!aligned(q.ptr, kPtrAlign))
            return fail(EP_ERR_ALIGN, "%s = %p is not 16-byte aligned", q.name, q.ptr);
    }
    if ((a->weights == nullptr) != (a->out_weights == nullptr))
        return fail(EP_ERR_ARG, "args.weights and args.out_weights must both be set or both NULL");
    if (a->weights && (!aligned(a->weights, kPtrAlign) || !aligned(a->out_weights, kPtrAlign)))
        return fail(EP_ERR_ALIGN, "args.weights / args.out_weights are not 16-byte aligned");
    if (s.scale_bytes > 0) {
        if (!a->scales || !a->out_scales)
            return fail(EP_ERR_NULL,
                        "args.scales and args.out_scales are required (scale_dim = %d)",
                        p->cfg.scale_dim);
        if (!aligned(a->scales, kPtrAlign) || !aligned(a->out_scales, kPtrAlign))
            return fail(EP_ERR_ALIGN, "args.scales / args.out_scales are not 16-byte aligned");
    } else if (a->scales || a->out_scales) {
        return fail(EP_ERR_ARG, "args.scales and args.out_scales must be NULL when scale_dim = 0");
    }
    const ep_launch_t l = effective_launch(p, a->num_tokens);
    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);

    ep::TileMap tm = {};
    tm.W = s.W;
    tm.tile_tokens = l.tile_tokens;
    int tiles = 0;
    for (int r = 0; r < s.W; ++r) {
        tm.tile_start[r] = tiles;
        tm.ntok[r] = a->num_tokens[r];
        tiles += (a->num_tokens[r] + l.tile_tokens - 1) / l.tile_tokens;
    }
    tm.tile_start[s.W] = tiles;
    tm.total_tiles = tiles;
    if (l.layout == EP_LAYOUT_IN_COPY && tiles > 0 && !layout_in_copy_fits(p, tiles))
        return fail(EP_ERR_ARG, "launch.layout = EP_LAYOUT_IN_COPY: %d tiles x %d ranks exceed "
                    "the %d counters of one block", tiles, s.W, ep::kLayoutInCopyCells);

    ep::RouteArgs ra;
    ra.idx = a->indices;
    ra.tile_counts = ws_counts(p);
    ra.M = s.M;
    ra.k = s.k;
    ra.Er = s.Er;
    ra.E = (int32_t)s.E;
    ra.tile_stride = s.tile_stride;

    ep::ScanArgs sa;
    sa.tile_counts = ws_counts(p);
    sa.tile_base = ws_base(p);
    sa.recv = a->recv_num_token;
    sa.total_tiles = tiles;
    sa.tile_stride = s.tile_stride;

    ep::CopyArgs ca;
    ca.x = static_cast<const uint8_t*>(a->x);
    ca.idx = a->indices;
    ca.w = a->weights;
    ca.sc = static_cast<const uint32_t*>(a->scales);
    ca.out_x = static_cast<uint8_t*>(a->out_x);
    ca.out_idx = a->out_indices;
    ca.out_w = a->out_weights;
    ca.out_sc = static_cast<uint32_t*>(a->out_scales);
    ca.tile_base = ws_base(p);
    ca.tile_counts = ws_counts(p);
    ca.recv = a->recv_num_token;
    // a call without tiles launches no copy block: the scan kernel writes the
    // (zero) receive counts then
    ca.layout = tiles == 0                             ? ep::kLayoutFromScan
                : l.layout == EP_LAYOUT_IN_COPY       ? ep::kLayoutInCopy
                : l.layout == EP_LAYOUT_SCAN_IN_COPY  ? ep::kLayoutScanInCopy
                                                       : ep::kLayoutFromScan;
    ca.src_pos = ws_src_pos(p);
    ca.fwd = ws_fwd(p);
    ca.row_vecs = s.row_vecs;
    ca.piece_vecs = (ca.row_vecs + l.dispatch_row_split - 1) / l.dispatch_row_split;
    ca.cast = p->cfg.dispatch_cast;
    ca.scale_dwords = (int32_t)(s.scale_bytes / 4);
    ca.M = s.M;
    ca.k = s.k;
    ca.Er = s.Er;
    ca.E = (int32_t)s.E;
    ca.P = s.P;
    ca.WM = (int32_t)s.WM;
    ca.tile_stride = s.tile_stride;
    ca.pieces = (int32_t)((ca.row_vecs + ca.piece_vecs - 1) / ca.piece_vecs);
    ca.token_split = std::min(l.dispatch_token_split, l.tile_tokens);
    ca.piece_inner = large_call(s, a->num_tokens) ? 1 : 0;
    // a launch's work-items must fit in 32 bits
    const int64_t copy_items = (int64_t)tm.total_tiles * ca.token_split * ca.pieces *
                               l.dispatch_waves * ep::kWave;
    if (copy_items > (int64_t)UINT32_MAX)
        return fail(EP_ERR_ARG, "dispatch copy grid of %lld work-items (tiles x "
                    "dispatch_token_split x row pieces x block) exceeds 2^32 - 1; lower "
                    "dispatch_row_split or dispatch_token_split", (long long)copy_items);

    hipError_t e = hipSuccess;
    if (ca.layout != ep::kLayoutInCopy)
        e = timed(p, EP_KERNEL_ROUTE, stream, [&] { return ep::launch_route(ra, tm, stream); });
    if (e == hipSuccess && ca.layout == ep::kLayoutFromScan)
        e = timed(p, EP_KERNEL_SCAN, stream, [&] { return ep::launch_scan(sa, s.W, stream); });
    if (e == hipSuccess)
        e = timed(p, EP_KERNEL_COPY, stream, [&] {
            return ep::launch_copy(ca, tm, l.dispatch_waves, l.cache_policy == EP_CACHE_STREAM,
                                   stream);
        });
    p->launched = true;
    p->last_stream = stream;
    if (e != hipSuccess) {
        p->dispatched = false;
        return fail(EP_ERR_HIP, "dispatch launch failed: %s", hipGetErrorString(e));
    }
    p->dispatched = true;
    p->dispatch_gen += 1;
    std::memcpy(p->last_ntok, a->num_tokens, sizeof(int32_t) * s.W);
    return ok();
}

int ep_combine(ep_plan_t* p, const ep_combine_args_t* a, void* stream_ptr)
{
    if (!p)
        return fail(EP_ERR_NULL, "plan is NULL");
    if (!a)
        return fail(EP_ERR_NULL, "args is NULL");
    if (!a->y)
        return fail(EP_ERR_NULL, "args.y is NULL");
    if (!a->out)
        return fail(EP_ERR_NULL, "args.out is NULL");
    if (!aligned(a->y, kPtrAlign) || !aligned(a->out, kPtrAlign))
        return fail(EP_ERR_ALIGN, "args.y / args.out are not 16-byte aligned");
    if ((a->y_weights == nullptr) != (a->out_weights == nullptr))
        return fail(EP_ERR_ARG,
                    "args.y_weights and args.out_weights must both be set or both NULL");
    if (a->y_weights && (!aligned(a->y_weights, 4) || !aligned(a->out_weights, 4)))
        return fail(EP_ERR_ALIGN, "args.y_weights / args.out_weights are not 4-byte aligned");
    const int wire = p->cfg.combine_wire;
    if (wire != EP_WIRE_NONE) {
        if (!a->y_scales)
            return fail(EP_ERR_NULL, "args.y_scales is NULL (cfg.combine_wire = %d)", wire);
        if (!aligned(a->y_scales, 4))
            return fail(EP_ERR_ALIGN, "args.y_scales is not 4-byte aligned");
    } else if (a->y_scales) {
        return fail(EP_ERR_ARG, "args.y_scales must be NULL when cfg.combine_wire = EP_WIRE_NONE");
    }
    if (!p->dispatched)
        return fail(EP_ERR_STATE, "combine before any dispatch on this plan");
    const Shape& s = p->s;
    const ep_launch_t l = effective_launch(p, p->last_ntok);
    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);

    ep::TokenMap tk;
    token_map(s, p->last_ntok, &tk);
    const int dtype = p->cfg.combine_dtype == EP_BF16 ? 0 : 1;
    const bool streaming = l.cache_policy == EP_CACHE_STREAM;

    hipError_t e;
    if (wire == EP_WIRE_NONE) {
        ep::CombineArgs ca;
        ca.y = static_cast<const uint8_t*>(a->y);
        ca.yw = a->y_weights;
        ca.out = static_cast<uint8_t*>(a->out);
        ca.out_w = a->out_weights;
        ca.fwd = ws_fwd(p);
        ca.row_vecs = (int32_t)(s.crow_bytes / 16);
        ca.piece_vecs = (ca.row_vecs + l.combine_row_split - 1) / l.combine_row_split;
        ca.pieces = (ca.row_vecs + ca.piece_vecs - 1) / ca.piece_vecs;
        ca.piece_inner = large_call(s, p->last_ntok) ? 1 : 0;
        ca.M = s.M;
        ca.k = s.k;
        ca.P = s.P;
        // a wave per (token, piece); the launch's work-items must fit in 32 bits
        const int64_t items = (int64_t)tk.total * ca.pieces;
        if ((items + l.combine_waves - 1) / l.combine_waves * l.combine_waves * ep::kWave >
            (int64_t)UINT32_MAX)
            return fail(EP_ERR_ARG, "combine grid of %lld waves (tokens x row pieces) exceeds "
                        "2^32 - 1 work-items; lower combine_row_split", (long long)items);
        e = timed(p, EP_KERNEL_COMBINE, stream, [&] {
            return ep::launch_combine(ca, tk, dtype, l.combine_waves, streaming, stream);
        });
    } else {
        ep::WireCombineArgs wa;
        wa.y = static_cast<const uint8_t*>(a->y);
        wa.ys = static_cast<const uint8_t*>(a->y_scales);
        wa.yw = a->y_weights;
        wa.out = static_cast<uint8_t*>(a->out);
        wa.out_w = a->out_weights;
        wa.fwd = ws_fwd(p);
        wa.units = s.H / 16;
        // pieces start on a scale dword (8 units) and a lane holds one dword
        // of each contribution's scale row
        wa.piece_units = (wa.units + l.combine_row_split - 1) / l.combine_row_split;
        wa.piece_units = std::min((wa.piece_units + 7) / 8 * 8, ep::kWirePieceUnits);
        if (wire == EP_WIRE_FP8_BLOCK128) {
            wa.row_bytes = (uint32_t)s.H;
            wa.scale_bytes = (uint32_t)(s.H / 128 * 4);
        } else {
            wa.row_bytes = (uint32_t)(s.H / 2);
            wa.scale_bytes = (uint32_t)(s.H / 32);
        }
        wa.M = s.M;
        wa.k = s.k;
        wa.P = s.P;
        wa.pieces = (wa.units + wa.piece_units - 1) / wa.piece_units;
        wa.piece_inner = large_call(s, p->last_ntok) ? 1 : 0;
        const int64_t witems = (int64_t)tk.total * wa.pieces;
        if ((witems + l.combine_waves - 1) / l.combine_waves * l.combine_waves * ep::kWave >
            (int64_t)UINT32_MAX)
            return fail(EP_ERR_ARG, "combine grid of %lld waves (tokens x row pieces) exceeds "
                        "2^32 - 1 work-items; lower combine_row_split", (long long)witems);
        const int kwire = wire == EP_WIRE_FP8_BLOCK128 ? ep::kWireFp8Block128 : ep::kWireMxfp4;
        e = timed(p, EP_KERNEL_COMBINE, stream, [&] {
            return ep::launch_combine_wire(wa, tk, kwire, dtype, l.combine_waves, streaming,
                                           stream);
        });
    }
    p->launched = true;
    p->last_stream = stream;
    if (e != hipSuccess)
        return fail(EP_ERR_HIP, "combine launch failed: %s", hipGetErrorString(e));
    return ok();
}

int ep_quantize_rows(const void* in, int64_t rows, int32_t hidden, int32_t in_dtype,
                     int32_t wire, void* out, void* scales, const int32_t* row_counts,
                     int64_t group_rows, void* stream_ptr)
{
    if (!in || !out || !scales)
        return fail(EP_ERR_NULL, "in, out and scales are required");
    if (!aligned(in, kPtrAlign) || !aligned(out, kPtrAlign) || !aligned(scales, 4))
        return fail(EP_ERR_ALIGN, "in / out must be 16-byte and scales 4-byte aligned");
    if (in_dtype != EP_BF16 && in_dtype != EP_FP16)
        return fail(EP_ERR_ARG, "in_dtype = %d: must be EP_BF16 or EP_FP16", in_dtype);
    if (wire != EP_WIRE_FP8_BLOCK128 && wire != EP_WIRE_MXFP4)
        return fail(EP_ERR_ARG, "wire = %d: must be EP_WIRE_FP8_BLOCK128 or EP_WIRE_MXFP4", wire);
    if (rows < 0)
        return fail(EP_ERR_ARG, "rows = %lld: must be >= 0", (long long)rows);
    const int block = wire == EP_WIRE_FP8_BLOCK128 ? 128 : 32;
    if (hidden < 1 || hidden % block != 0)
        return fail(EP_ERR_ARG, "hidden = %d: must be a positive multiple of %d", hidden, block);
    if (rows * (int64_t)hidden >= ((int64_t)1 << 40))
        return fail(EP_ERR_SIZE, "rows * hidden is too large");
    if (hidden > (1 << 30))
        return fail(EP_ERR_SIZE, "hidden = %d is too large", hidden);
    if (row_counts) {
        if (!aligned(row_counts, 4))
            return fail(EP_ERR_ALIGN, "row_counts must be 4-byte aligned");
        if (group_rows < 1 || rows % group_rows != 0)
            return fail(EP_ERR_ARG, "group_rows = %lld: must be >= 1 and divide rows = %lld",
                        (long long)group_rows, (long long)rows);
    }
    ep::QuantizeArgs qa;
    qa.in = static_cast<const uint8_t*>(in);
    qa.out = static_cast<uint8_t*>(out);
    qa.scales = static_cast<uint8_t*>(scales);
    qa.counts = row_counts;
    qa.rows = rows;
    qa.group_rows = row_counts ? group_rows : rows;
    qa.H = hidden;
    // a wave per row piece of at most kQuantChunks chunks, pieces as even as
    // the chunk count allows
    const int chunks = (hidden + ep::kQuantChunk - 1) / ep::kQuantChunk;
    qa.pieces = (chunks + ep::kQuantChunks - 1) / ep::kQuantChunks;
    qa.piece_chunks = (chunks + qa.pieces - 1) / qa.pieces;
    // the bytes a call may move against the MALL: past it, loads and stores stream
    const int64_t out_row = wire == EP_WIRE_FP8_BLOCK128 ? hidden + hidden / 32 : hidden / 2 + hidden / 32;
    const bool stream = rows * (2 * (int64_t)hidden + out_row) > kKeepBytes;
    const hipError_t e =
        ep::launch_quantize(qa, wire == EP_WIRE_FP8_BLOCK128 ? ep::kWireFp8Block128 : ep::kWireMxfp4,
                            in_dtype == EP_BF16 ? 0 : 1, stream,
                            static_cast<hipStream_t>(stream_ptr));
    if (e != hipSuccess)
        return fail(EP_ERR_HIP, "quantize launch failed: %s", hipGetErrorString(e));
    return ok();
}

int ep_get_src_token_pos(const ep_plan_t* p, int32_t rank, const int32_t** dev_ptr)
{
    if (!p)
        return fail(EP_ERR_NULL, "plan is NULL");
    if (!dev_ptr)
        return fail(EP_ERR_NULL, "dev_ptr is NULL");
    if (rank < 0 || rank >= p->s.W)
        return fail(EP_ERR_ARG, "rank = %d: must be in [0, %d)", rank, p->s.W);
    *dev_ptr = ws_src_pos(p) + (int64_t)rank * p->s.WM;
    return ok();
}

const char* ep_last_error(void) { return g_error.c_str(); }

int ep_probe_forward_map(const ep_plan_t* p, const int32_t** map, int32_t* stride)
{
    if (!p)
        return fail(EP_ERR_NULL, "plan is NULL");
    if (!map || !stride)
        return fail(EP_ERR_NULL, "map / stride is NULL");
    *map = reinterpret_cast<const int32_t*>(p->ws + p->s.off_fwd);
    *stride = p->s.P;
    return ok();
}

int ep_probe_pattern(const ep_probe_args_t* a, void* stream_ptr)
{
    if (!a)
        return fail(EP_ERR_NULL, "args is NULL");
    if (a->kind < EP_PROBE_READ || a->kind > EP_PROBE_GATHER)
        return fail(EP_ERR_ARG, "args.kind = %d: not an EP_PROBE_* value", a->kind);
    if (a->row_bytes <= 0 || a->row_bytes % 16)
        return fail(EP_ERR_ARG, "args.row_bytes = %d: must be a positive multiple of 16",
                    a->row_bytes);
    if (a->rows < 0)
        return fail(EP_ERR_ARG, "args.rows = %lld: must be >= 0", (long long)a->rows);
    if (a->pieces < 1 || a->pieces > 64)
        return fail(EP_ERR_ARG, "args.pieces = %d: must be in [1, 64]", a->pieces);
    if (a->waves < 1 || a->waves > 16)
        return fail(EP_ERR_ARG, "args.waves = %d: must be in [1, 16]", a->waves);
    if (a->rows * a->pieces > INT32_MAX)
        return fail(EP_ERR_ARG, "args.rows * args.pieces is too large for one launch");
    const bool mapped = a->kind == EP_PROBE_FANOUT || a->kind == EP_PROBE_GATHER;
    if (a->kind != EP_PROBE_WRITE && !a->src)
        return fail(EP_ERR_NULL, "args.src is NULL");
    if (!a->dst)
        return fail(EP_ERR_NULL, "args.dst is NULL");
    if (mapped) {
        if (!a->map)
            return fail(EP_ERR_NULL, "args.map is NULL");
        if (a->stride < 1 || a->stride > 64)
            return fail(EP_ERR_ARG, "args.stride = %d: must be in [1, 64]", a->stride);
        if (a->map_rows < 0)
            return fail(EP_ERR_ARG, "args.map_rows = %lld: must be >= 0",
                        (long long)a->map_rows);
        if (!aligned(a->map, 4))
            return fail(EP_ERR_ALIGN, "args.map is not 4-byte aligned");
    }
    if ((a->src && !aligned(a->src, kPtrAlign)) || !aligned(a->dst, kPtrAlign))
        return fail(EP_ERR_ALIGN, "args.src / args.dst are not 16-byte aligned");
    ep::ProbeArgs pa;
    pa.kind = a->kind;
    pa.row_bytes = (uint32_t)a->row_bytes;
    pa.rows = a->rows;
    pa.src = static_cast<const uint8_t*>(a->src);
    pa.dst = static_cast<uint8_t*>(a->dst);
    pa.map = a->map;
    pa.map_rows = mapped ? a->map_rows : 0;
    pa.stride = mapped ? a->stride : 0;
    pa.pieces = a->pieces;
    const hipError_t e = ep::launch_probe(pa, a->waves, static_cast<hipStream_t>(stream_ptr));
    if (e != hipSuccess)
        return fail(EP_ERR_HIP, "probe launch failed: %s", hipGetErrorString(e));
    return ok();
}

int ep_plan_set_launch(ep_plan_t* p, const ep_launch_t* l)
{
    if (!p)
        return fail(EP_ERR_NULL, "plan is NULL");
    if (!l) {
        p->launch = ep_launch_t{};
        return ok();
    }
    const int rc = check_launch(p, l);
    if (rc != EP_OK)
        return rc;
    p->launch = *l;
    return ok();
}

int ep_plan_get_launch(const ep_plan_t* p, const int32_t* num_tokens, ep_launch_t* out)
{
    if (!p)
        return fail(EP_ERR_NULL, "plan is NULL");
    if (!num_tokens)
        return fail(EP_ERR_NULL, "num_tokens is NULL");
    if (!out)
        return fail(EP_ERR_NULL, "out is NULL");
    for (int r = 0; r < p->s.W; ++r)
        if (num_tokens[r] < 0 || num_tokens[r] > p->s.M)
            return fail(EP_ERR_ARG, "num_tokens[%d] = %d: must be in [0, %d]", r, num_tokens[r],
                        p->s.M);
    *out = effective_launch(p, num_tokens);
    return ok();
}

int ep_plan_set_timing(ep_plan_t* p, int enable)
{
    if (!p)
        return fail(EP_ERR_NULL, "plan is NULL");
    if (!enable) {
        timers_destroy(p);
        p->timing = false;
        return ok();
    }
    timers_destroy(p);
    for (Timer& t : p->timers) {
        for (int i = 0; i < kTimerPool; ++i) {
            hipEvent_t e0 = nullptr, e1 = nullptr;
            if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
                if (e0)
                    (void)hipEventDestroy(e0);
                timers_destroy(p);
                return fail(EP_ERR_HIP, "hipEventCreate failed");
            }
            t.start.push_back(e0);
            t.stop.push_back(e1);
        }
    }
    p->timing = true;
    return ok();
}

size_t ep_expert_workspace_bytes(const ep_plan_t* p, int32_t cap)
{
    if (!p) {
        fail(EP_ERR_NULL, "plan is NULL");
        return 0;
    }
    ExShape e;
    if (expert_shape(p->s, cap, &e) != EP_OK)
        return 0;
    ok();
    return e.total;
}

int ep_expert_plan_create(ep_plan_t* p, int32_t cap, void* workspace, size_t workspace_bytes,
                          ep_expert_plan_t** out)
{
    if (!p)
        return fail(EP_ERR_NULL, "plan is NULL");
    ExShape e;
    const int rc = expert_shape(p->s, cap, &e);
    if (rc != EP_OK)
        return rc;
    if (!workspace)
        return fail(EP_ERR_NULL, "workspace is NULL");
    if (!out)
        return fail(EP_ERR_NULL, "out is NULL");
    if (!aligned(workspace, kWorkspaceAlign))
        return fail(EP_ERR_ALIGN, "workspace %p is not %zu-byte aligned", workspace,
                    kWorkspaceAlign);
    if (workspace_bytes < e.total)
        return fail(EP_ERR_SIZE,
                    "workspace_bytes = %zu: ep_expert_workspace_bytes() requires %zu",
                    workspace_bytes, e.total);
    ep_expert_plan* x = new (std::nothrow) ep_expert_plan();
    if (!x)
        return fail(EP_ERR_SIZE, "out of host memory for the expert plan");
    x->plan = p;
    x->e = e;
    x->ws = static_cast<uint8_t*>(workspace);
    p->experts += 1;
    *out = x;
    return ok();
}

int ep_expert_plan_destroy(ep_expert_plan_t* x)
{
    if (!x)
        return ok();
    int rc = EP_OK;
    if (x->launched) {
        const hipError_t e = hipStreamSynchronize(x->last_stream);
        if (e != hipSuccess)
            rc = fail(EP_ERR_HIP, "hipStreamSynchronize before destroy: %s", hipGetErrorString(e));
    }
    x->plan->experts -= 1;
    delete x;
    return rc == EP_OK ? ok() : rc;
}

int ep_convert_dispatch_output(ep_expert_plan_t* x, const ep_convert_dispatch_args_t* a,
                               void* stream_ptr)
{
    if (!x)
        return fail(EP_ERR_NULL, "plan is NULL");
    if (!a)
        return fail(EP_ERR_NULL, "args is NULL");
    ep_plan* p = x->plan;
    const Shape& s = p->s;
    struct {
        const void* ptr;
        const char* name;
        size_t align;
    } req[] = {{a->x, "args.x", kPtrAlign},
               {a->indices, "args.indices", 4},
               {a->recv_num_token, "args.recv_num_token", 4},
               {a->packed_x, "args.packed_x", kPtrAlign},
               {a->packed_count, "args.packed_count", 4},
               {a->packed_src_info, "args.packed_src_info", 4},
               {a->packed_layout_range, "args.packed_layout_range", 8}};
    for (auto& q : req) {
        if (!q.ptr)
            return fail(EP_ERR_NULL, "%s is NULL", q.name);
        if (!aligned(q.ptr, q.align))
            return fail(EP_ERR_ALIGN, "%s = %p is not %zu-byte aligned", q.name, q.ptr, q.align);
    }
    if (s.scale_bytes > 0) {
        if (!a->scales || !a->packed_scales)
            return fail(EP_ERR_NULL,
                        "args.scales and args.packed_scales are required (scale_dim = %d)",
                        p->cfg.scale_dim);
        if (!aligned(a->scales, 4) || !aligned(a->packed_scales, 4))
            return fail(EP_ERR_ALIGN, "args.scales / args.packed_scales are not 4-byte aligned");
    } else if (a->scales || a->packed_scales) {
        return fail(EP_ERR_ARG,
                    "args.scales and args.packed_scales must be NULL when scale_dim = 0");
    }
    if (a->weights && !aligned(a->weights, 4))
        return fail(EP_ERR_ALIGN, "args.weights = %p is not 4-byte aligned", (const void*)a->weights);
    if (!p->dispatched)
        return fail(EP_ERR_STATE, "convert before any dispatch on the plan");
    const ep_launch_t l = effective_launch(p, p->last_ntok);
    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
    const int64_t rows = expert_rows(s, p->last_ntok);

    ep::ExpertArgs ea;
    ea.x = static_cast<const uint8_t*>(a->x);
    ea.idx = a->indices;
    ea.w = a->weights;
    ea.sc = static_cast<const uint32_t*>(a->scales);
    ea.recv = a->recv_num_token;
    ea.src_pos = ws_src_pos(p);
    ea.px = static_cast<uint8_t*>(a->packed_x);
    ea.psc = static_cast<uint32_t*>(a->packed_scales);
    ea.count = a->packed_count;
    ea.src_info = a->packed_src_info;
    ea.layout_range = a->packed_layout_range;
    ea.tile_counts = reinterpret_cast<int32_t*>(x->ws + x->e.off_counts);
    ea.tile_base = reinterpret_cast<int32_t*>(x->ws + x->e.off_base);
    ea.src_start = reinterpret_cast<int32_t*>(x->ws + x->e.off_start);
    ea.src_prefix = reinterpret_cast<int32_t*>(x->ws + x->e.off_prefix);
    ea.efwd = reinterpret_cast<int32_t*>(x->ws + x->e.off_efwd);
    ea.ew = reinterpret_cast<float*>(x->ws + x->e.off_ew);
    ea.row_vecs = (int32_t)(s.row_bytes / 16);
    const ShareGrid eg = share_grid((int64_t)s.W * expert_tiles(rows), ea.row_vecs, s.k,
                                    l.expert_waves, std::max(0, p->launch.expert_row_split),
                                    std::max(0, p->launch.expert_token_split));
    ea.piece_vecs = (ea.row_vecs + eg.row_split - 1) / eg.row_split;
    ea.token_split = eg.token_split;
    ea.scale_dwords = (int32_t)(s.scale_bytes / 4);
    ea.W = s.W;
    ea.WM = (int32_t)s.WM;
    ea.k = s.k;
    ea.Er = s.Er;
    ea.Pe = x->e.Pe;
    ea.cap = x->e.cap;
    ea.rows = (int32_t)rows;
    ea.T = expert_tiles(rows);
    const int row_split = (ea.row_vecs + ea.piece_vecs - 1) / ea.piece_vecs;

    // small calls count and scan in one launch (timed as the scan)
    const bool one = ea.T <= ep::kCountScanTiles && s.k <= ep::kCountScanTopK &&
                     p->launch.layout != EP_LAYOUT_KERNELS;
    hipError_t e = hipSuccess;
    if (one) {
        e = timed(p, EP_KERNEL_EXPERT_SCAN, stream,
                  [&] { return ep::launch_expert_count_scan(ea, stream); });
    } else {
        e = timed(p, EP_KERNEL_EXPERT_COUNT, stream,
                  [&] { return ep::launch_expert_count(ea, stream); });
        if (e == hipSuccess)
            e = timed(p, EP_KERNEL_EXPERT_SCAN, stream,
                      [&] { return ep::launch_expert_scan(ea, stream); });
    }
    if (e == hipSuccess)
        e = timed(p, EP_KERNEL_EXPERT_COPY, stream, [&] {
            return ep::launch_expert_copy(ea, l.expert_waves, row_split,
                                          l.expert_cache_policy == EP_CACHE_STREAM, stream);
        });
    x->launched = true;
    x->last_stream = stream;
    if (e != hipSuccess) {
        x->converted = false;
        x->fused = false;
        return fail(EP_ERR_HIP, "convert_dispatch_output launch failed: %s", hipGetErrorString(e));
    }
    x->converted = true;
    x->fused = false;
    x->weighted = a->weights != nullptr;
    x->gen = p->dispatch_gen;
    x->recv = a->recv_num_token;
    x->rows = (int32_t)rows;
    return ok();
}

int ep_convert_combine_input(ep_expert_plan_t* x, const ep_convert_combine_args_t* a,
                             void* stream_ptr)
{
    if (!x)
        return fail(EP_ERR_NULL, "plan is NULL");
    if (!a)
        return fail(EP_ERR_NULL, "args is NULL");
    if (!a->packed_y)
        return fail(EP_ERR_NULL, "args.packed_y is NULL");
    if (!a->y)
        return fail(EP_ERR_NULL, "args.y is NULL");
    if (!aligned(a->packed_y, kPtrAlign) || !aligned(a->y, kPtrAlign))
        return fail(EP_ERR_ALIGN, "args.packed_y / args.y are not 16-byte aligned");
    if (a->apply_weights != 0 && a->apply_weights != 1)
        return fail(EP_ERR_ARG, "args.apply_weights = %d: must be 0 or 1", a->apply_weights);
    ep_plan* p = x->plan;
    if (!x->converted)
        return fail(EP_ERR_STATE, "convert_combine_input before any convert_dispatch_output");
    if (!p->dispatched || x->gen != p->dispatch_gen)
        return fail(EP_ERR_STATE, "the plan dispatched again since the last "
                    "convert_dispatch_output on this expert plan");
    if (a->apply_weights && !x->weighted)
        return fail(EP_ERR_STATE, "args.apply_weights = 1, but the last "
                    "convert_dispatch_output was given no weights");
    const Shape& s = p->s;
    const ep_launch_t l = effective_launch(p, p->last_ntok);
    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);

    ep::ExpertCombineArgs ca;
    ca.py = static_cast<const uint8_t*>(a->packed_y);
    ca.recv = x->recv;
    ca.efwd = reinterpret_cast<const int32_t*>(x->ws + x->e.off_efwd);
    ca.ew = a->apply_weights ? reinterpret_cast<const float*>(x->ws + x->e.off_ew) : nullptr;
    ca.y = static_cast<uint8_t*>(a->y);
    ca.row_vecs = (int32_t)(s.crow_bytes / 16);
    ca.piece_vecs = (ca.row_vecs + l.expert_combine_row_split - 1) / l.expert_combine_row_split;
    ca.WM = (int32_t)s.WM;
    ca.Pe = x->e.Pe;
    ca.rows = x->rows;
    ca.pieces = (ca.row_vecs + ca.piece_vecs - 1) / ca.piece_vecs;
    ca.piece_inner = large_call(s, p->last_ntok) ? 1 : 0;
    const int dtype = p->cfg.combine_dtype == EP_BF16 ? 0 : 1;
    // a wave per (row, piece) of each rank; a launch's x work-items must fit
    // in 32 bits
    const int64_t items = (int64_t)ca.rows * ca.pieces;
    if ((items + l.expert_combine_waves - 1) / l.expert_combine_waves * l.expert_combine_waves *
            ep::kWave > (int64_t)UINT32_MAX)
        return fail(EP_ERR_ARG, "inverse grid of %lld waves a rank (rows x row pieces) exceeds "
                    "2^32 - 1 work-items; lower expert_combine_row_split", (long long)items);

    const hipError_t e = timed(p, EP_KERNEL_EXPERT_COMBINE, stream, [&] {
        return ep::launch_expert_combine(ca, s.W, dtype, l.expert_combine_waves,
                                         l.expert_cache_policy == EP_CACHE_STREAM, stream);
    });
    x->launched = true;
    x->last_stream = stream;
    if (e != hipSuccess)
        return fail(EP_ERR_HIP, "convert_combine_input launch failed: %s", hipGetErrorString(e));
    return ok();
}

int ep_dispatch_standard_moe(ep_expert_plan_t* x, const ep_dispatch_standard_args_t* a,
                             void* stream_ptr)
{
    if (!x)
        return fail(EP_ERR_NULL, "plan is NULL");
    if (!a)
        return fail(EP_ERR_NULL, "args is NULL");
    ep_plan* p = x->plan;
    const Shape& s = p->s;
    if (!a->num_tokens)
        return fail(EP_ERR_NULL, "args.num_tokens is NULL");
    struct {
        const void* ptr;
        const char* name;
        size_t align;
    } req[] = {{a->x, "args.x", kPtrAlign},
               {a->indices, "args.indices", 4},
               {a->packed_x, "args.packed_x", kPtrAlign},
               {a->packed_count, "args.packed_count", 4},
               {a->packed_src_info, "args.packed_src_info", 4},
               {a->packed_layout_range, "args.packed_layout_range", 8}};
    for (auto& q : req) {
        if (!q.ptr)
            return fail(EP_ERR_NULL, "%s is NULL", q.name);
        if (!aligned(q.ptr, q.align))
            return fail(EP_ERR_ALIGN, "%s = %p is not %zu-byte aligned", q.name, q.ptr, q.align);
    }
    if (s.scale_bytes > 0) {
        if (!a->scales || !a->packed_scales)
            return fail(EP_ERR_NULL,
                        "args.scales and args.packed_scales are required (scale_dim = %d)",
                        p->cfg.scale_dim);
        if (!aligned(a->scales, 4) || !aligned(a->packed_scales, 4))
            return fail(EP_ERR_ALIGN, "args.scales / args.packed_scales are not 4-byte aligned");
    } else if (a->scales || a->packed_scales) {
        return fail(EP_ERR_ARG,
                    "args.scales and args.packed_scales must be NULL when scale_dim = 0");
    }
    for (int r = 0; r < s.W; ++r)
        if (a->num_tokens[r] < 0 || a->num_tokens[r] > s.M)
            return fail(EP_ERR_ARG, "args.num_tokens[%d] = %d: must be in [0, %d]", r,
                        a->num_tokens[r], s.M);
    const ep_launch_t l = effective_launch(p, a->num_tokens);
    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);

    ep::StandardArgs sa;
    sa.x = static_cast<const uint8_t*>(a->x);
    sa.idx = a->indices;
    sa.sc = static_cast<const uint32_t*>(a->scales);
    sa.px = static_cast<uint8_t*>(a->packed_x);
    sa.psc = static_cast<uint32_t*>(a->packed_scales);
    sa.count = a->packed_count;
    sa.src_info = a->packed_src_info;
    sa.layout_range = a->packed_layout_range;
    sa.tile_counts = reinterpret_cast<int32_t*>(x->ws + x->e.off_counts);
    sa.tile_base = reinterpret_cast<int32_t*>(x->ws + x->e.off_base);
    sa.fslot = reinterpret_cast<int32_t*>(x->ws + x->e.off_efwd);
    sa.row_vecs = s.row_vecs;  // of a source row (bf16 / fp16 with a cast)
    sa.out_row_bytes = (uint32_t)s.row_bytes;
    sa.cast = p->cfg.dispatch_cast;  // 1 bf16, 2 fp16 source rows
    sa.scale_dwords = (int32_t)(s.scale_bytes / 4);
    sa.W = s.W;
    sa.M = s.M;
    sa.k = s.k;
    sa.Er = s.Er;
    sa.E = (int32_t)s.E;
    sa.cap = x->e.cap;
    sa.Tr = (int32_t)x->e.Tr;
    for (int r = 0; r < ep::kMaxRanks; ++r)
        sa.ntok[r] = r < s.W ? a->num_tokens[r] : 0;
    // row pieces and blocks sharing a tile (share_grid), unless overridden
    const ShareGrid fg = share_grid(fused_tiles(s, a->num_tokens), sa.row_vecs, s.k,
                                    l.expert_waves, std::max(0, p->launch.expert_row_split),
                                    std::max(0, p->launch.expert_token_split));
    sa.piece_vecs = (sa.row_vecs + fg.row_split - 1) / fg.row_split;
    const int row_split = (sa.row_vecs + sa.piece_vecs - 1) / sa.piece_vecs;
    sa.token_split = fg.token_split;

    // small calls count and scan in one launch (timed as the scan)
    const bool one = (int64_t)s.W * sa.Tr <= ep::kCountScanTiles &&
                     s.k <= ep::kCountScanTopK && p->launch.layout != EP_LAYOUT_KERNELS;
    hipError_t e = hipSuccess;
    if (one) {
        e = timed(p, EP_KERNEL_STANDARD_SCAN, stream,
                  [&] { return ep::launch_standard_count_scan(sa, stream); });
    } else {
        e = timed(p, EP_KERNEL_STANDARD_COUNT, stream,
                  [&] { return ep::launch_standard_count(sa, stream); });
        if (e == hipSuccess)
            e = timed(p, EP_KERNEL_STANDARD_SCAN, stream,
                      [&] { return ep::launch_standard_scan(sa, stream); });
    }
    if (e == hipSuccess)
        e = timed(p, EP_KERNEL_STANDARD_COPY, stream, [&] {
            return ep::launch_standard_copy(sa, l.expert_waves, row_split,
                                            l.expert_cache_policy == EP_CACHE_STREAM, stream);
        });
    x->launched = true;
    x->last_stream = stream;
    // the map's space now holds the fused map: no conversion is current
    x->converted = false;
    if (e != hipSuccess) {
        x->fused = false;
        return fail(EP_ERR_HIP, "dispatch_standard_moe launch failed: %s", hipGetErrorString(e));
    }
    x->fused = true;
    for (int r = 0; r < ep::kMaxRanks; ++r)
        x->fused_ntok[r] = r < s.W ? a->num_tokens[r] : 0;
    return ok();
}

int ep_combine_standard_moe(ep_expert_plan_t* x, const ep_combine_standard_args_t* a,
                            void* stream_ptr)
{
    if (!x)
        return fail(EP_ERR_NULL, "plan is NULL");
    if (!a)
        return fail(EP_ERR_NULL, "args is NULL");
    ep_plan* p = x->plan;
    const Shape& s = p->s;
    const int wire = p->cfg.combine_wire;
    if (wire != EP_WIRE_NONE) {
        if (!a->packed_y_scales)
            return fail(EP_ERR_NULL, "args.packed_y_scales is required with a combine_wire");
        if (!aligned(a->packed_y_scales, 4))
            return fail(EP_ERR_ALIGN, "args.packed_y_scales must be 4-byte aligned");
    } else if (a->packed_y_scales) {
        return fail(EP_ERR_ARG,
                    "args.packed_y_scales must be NULL when cfg.combine_wire = EP_WIRE_NONE");
    }
    if (!a->packed_y)
        return fail(EP_ERR_NULL, "args.packed_y is NULL");
    if (!a->indices)
        return fail(EP_ERR_NULL, "args.indices is NULL");
    if (!a->out)
        return fail(EP_ERR_NULL, "args.out is NULL");
    if (!aligned(a->packed_y, kPtrAlign) || !aligned(a->out, kPtrAlign))
        return fail(EP_ERR_ALIGN, "args.packed_y / args.out are not 16-byte aligned");
    if (!aligned(a->indices, 4) || (a->weights && !aligned(a->weights, 4)))
        return fail(EP_ERR_ALIGN, "args.indices / args.weights are not 4-byte aligned");
    if (!x->fused)
        return fail(EP_ERR_STATE, "combine_standard_moe before any dispatch_standard_moe on "
                    "this expert plan (or a convert_dispatch_output came since)");
    const ep_launch_t l = effective_launch(p, x->fused_ntok);
    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);

    ep::StandardCombineArgs ca;
    ca.py = static_cast<const uint8_t*>(a->packed_y);
    ca.pys = static_cast<const uint8_t*>(a->packed_y_scales);
    ca.wire = wire == EP_WIRE_FP8_BLOCK128 ? ep::kWireFp8Block128
              : wire == EP_WIRE_MXFP4      ? ep::kWireMxfp4
                                           : 0;
    ca.py_row_bytes = wire == EP_WIRE_FP8_BLOCK128 ? (uint32_t)s.H : (uint32_t)s.H / 2u;
    ca.py_scale_bytes =
        wire == EP_WIRE_FP8_BLOCK128 ? (uint32_t)(s.H / 128 * 4) : (uint32_t)(s.H / 32);
    ca.idx = a->indices;
    ca.w = a->weights;
    ca.fslot = reinterpret_cast<const int32_t*>(x->ws + x->e.off_efwd);
    ca.out = static_cast<uint8_t*>(a->out);
    ca.row_vecs = (int32_t)(s.crow_bytes / 16);
    ca.M = s.M;
    ca.k = s.k;
    ca.Er = s.Er;
    ca.E = (int32_t)s.E;
    ep::TokenMap tk;
    token_map(s, x->fused_ntok, &tk);
    // Automatic geometry of this fold (expert_combine_waves and
    // expert_combine_row_split <= 0): small calls cut rows until about 1024
    // blocks of 4 waves; large calls (numbered piece-fastest) fold pieces of
    // 2 KB with 8 waves a block, or from wire rows pieces of about 3.5 KB of
    // codes with 4 waves (8 x 4096 tokens, top-8, H = 7168, us: bf16 817 ->
    // 737, FP8 block-128 470 -> 455, MXFP4 318 -> 318).
    const bool large = large_call(s, x->fused_ntok);
    int waves = p->launch.expert_combine_waves > 0 ? p->launch.expert_combine_waves
                : large ? (wire != EP_WIRE_NONE ? 4 : 8)
                        : 4;
    int split = l.expert_combine_row_split;
    if (p->launch.expert_combine_row_split <= 0) {
        const int max_split = std::max(1, ca.row_vecs / ep::kWave);
        if (large) {
            const int64_t piece = wire != EP_WIRE_NONE ? kStandardWirePieceBytes : 2048;
            const int64_t bytes = wire != EP_WIRE_NONE ? wire_row_bytes(p) : s.crow_bytes;
            split = (int)std::min<int64_t>(max_split, std::max<int64_t>(1, bytes / piece));
        } else {
            const int64_t blocks = std::max<int64_t>(1, ((int64_t)tk.total + 3) / 4);
            split = (int)std::min<int64_t>(max_split,
                                           std::max<int64_t>(1, (1024 + blocks - 1) / blocks));
        }
    }
    ca.piece_vecs = (ca.row_vecs + split - 1) / split;
    if (ca.wire) {
        // pieces start on a scale dword (16 groups of 8 elements) and a lane
        // holds one dword of each pair's scale row
        ca.piece_vecs = std::min((ca.piece_vecs + 15) / 16 * 16, 16 * ep::kWave);
    }
    ca.pieces = (ca.row_vecs + ca.piece_vecs - 1) / ca.piece_vecs;
    ca.piece_inner = large ? 1 : 0;
    const int64_t items = (int64_t)tk.total * ca.pieces;
    if ((items + waves - 1) / waves * waves * ep::kWave > (int64_t)UINT32_MAX)
        return fail(EP_ERR_ARG, "combine_standard_moe grid of %lld waves (tokens x row pieces) "
                    "exceeds 2^32 - 1 work-items; lower expert_combine_row_split",
                    (long long)items);
    const int dtype = p->cfg.combine_dtype == EP_BF16 ? 0 : 1;

    const hipError_t e = timed(p, EP_KERNEL_STANDARD_COMBINE, stream, [&] {
        return ep::launch_standard_combine(ca, tk, dtype, waves,
                                           l.expert_cache_policy == EP_CACHE_STREAM, stream);
    });
    x->launched = true;
    x->last_stream = stream;
    if (e != hipSuccess)
        return fail(EP_ERR_HIP, "combine_standard_moe launch failed: %s", hipGetErrorString(e));
    return ok();
}

int ep_plan_kernel_time(ep_plan_t* p, int kernel, int32_t* count, double* total_ms)
{
    if (!p)
        return fail(EP_ERR_NULL, "plan is NULL");
    if (kernel < 0 || kernel >= kTimedKernels)
        return fail(EP_ERR_ARG, "kernel = %d: must be an EP_KERNEL_* value", kernel);
    if (!count || !total_ms)
        return fail(EP_ERR_NULL, "count / total_ms is NULL");
    Timer& t = p->timers[kernel];
    timer_drain(t);
    *count = t.count;
    *total_ms = t.total_ms;
    return ok();
}

}  // extern "C"

namespace ep {

int set_error(int code, const char* msg) { return fail(code, "%s", msg); }

// The per-device plans of ep_plan_static, over the library's static scratch.
ep_plan g_static_plans[kMaxDevices];

int static_plan_check(const ep_config_t* cfg, size_t scratch_bytes)
{
    Shape s;
    const int rc = check_config(cfg, &s);
    if (rc != EP_OK)
        return rc;
    if (s.total > scratch_bytes)
        return fail(EP_ERR_SIZE, "this configuration needs a %zu-byte workspace; the static "
                    "scratch of ep_plan_static holds %zu bytes (use ep_plan_create with a "
                    "workspace of ep_workspace_bytes())", s.total, scratch_bytes);
    return EP_OK;
}

int static_plan_reset(const ep_config_t* cfg, void* scratch, size_t scratch_bytes, int device,
                      ep_plan_t** out)
{
    const int rc = static_plan_check(cfg, scratch_bytes);
    if (rc != EP_OK)
        return rc;
    if (device < 0 || device >= kMaxDevices)
        return fail(EP_ERR_ARG, "device %d: ep_plan_static serves devices 0..%d", device,
                    kMaxDevices - 1);
    ep_plan* p = &g_static_plans[device];
    if (p->experts > 0)
        return fail(EP_ERR_STATE, "%d expert plan(s) made from this device's static plan still "
                    "exist: destroy them first", p->experts);
    Shape s;
    check_config(cfg, &s);
    timers_destroy(p);
    p->cfg = *cfg;
    p->s = s;
    p->ws = static_cast<uint8_t*>(scratch);
    p->dispatched = false;
    std::memset(p->last_ntok, 0, sizeof p->last_ntok);
    p->last_stream = nullptr;
    p->launched = false;
    p->launch = ep_launch_t{};
    p->timing = false;
    p->dispatch_gen = 0;
    p->is_static = true;
    *out = p;
    return ok();
}

}  // namespace ep
