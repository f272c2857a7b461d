// Internal interface between the host side of the library (ep_plan.cpp) and
// its gfx950 kernels (ep_kernels.hip). Not installed; the public ABI is
// include/ep.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ep {

constexpr int kWave = 64;       // CDNA wavefront width
constexpr int kMaxRanks = 64;   // a token's destination set is one 64-bit mask
constexpr int kMaxTopk = 64;    // one lane per top-k slot of a token
constexpr int kMinTile = 16;    // smallest routing tile (tokens)

// Where each rank's tokens sit in the flat list of routing tiles, for one
// call. Passed by value (kernel arguments), so it is part of a captured graph.
struct TileMap {
    int32_t W;
    int32_t tile_tokens;                 // TT: 16, 32 or 64
    int32_t total_tiles;
    int32_t tile_start[kMaxRanks + 1];   // first tile of rank r; [W] = total
    int32_t ntok[kMaxRanks];             // T_r
};

// Where the dispatch copy gets each tile's first receive slot on every rank.
enum LayoutMode : int32_t {
    kLayoutFromScan = 0,   // tile_base, written by the scan kernel
    kLayoutScanInCopy = 1, // summed by the copy block from tile_counts
    kLayoutInCopy = 2,     // counted by the copy block from the ids of the whole call
};

// Most (tiles x ranks) counters the copy kernel keeps in LDS in kLayoutInCopy.
constexpr int kLayoutInCopyCells = 4096;

// Token counts as a prefix, for the combine's flat token index.
struct TokenMap {
    int32_t W;
    int32_t total;                       // N = sum of T_r
    int32_t tok_start[kMaxRanks + 1];    // first flat token of rank r
};

struct RouteArgs {
    const int32_t* idx;      // [W][M][k]
    int32_t* tile_counts;    // [W][tile_stride]: rows tile g sends to rank d
    int32_t M, k, Er, E;
    int32_t tile_stride;
};

struct ScanArgs {
    const int32_t* tile_counts;  // [W][tile_stride]
    int32_t* tile_base;          // [W][tile_stride]: first slot of tile g on d
    int32_t* recv;               // [W]
    int32_t total_tiles;
    int32_t tile_stride;
};

struct CopyArgs {
    const uint8_t* x;            // [W][M][row_bytes]
    const int32_t* idx;          // [W][M][k]
    const float* w;              // [W][M][k] or null
    const uint32_t* sc;          // [W][M][scale_dwords] or null
    uint8_t* out_x;              // [W][WM][row_bytes]
    int32_t* out_idx;            // [W][WM][k]
    float* out_w;                // [W][WM][k] or null
    uint32_t* out_sc;            // [W][WM][scale_dwords] or null
    const int32_t* tile_base;    // [W][tile_stride] (kLayoutFromScan)
    const int32_t* tile_counts;  // [W][tile_stride] (kLayoutScanInCopy)
    int32_t* recv;               // [W] (written here unless kLayoutFromScan)
    int32_t layout;              // LayoutMode
    int32_t* src_pos;            // [W][WM]
    int32_t* fwd;                // [W][M][P]
    int32_t row_vecs;            // 16-byte vectors per payload row
    int32_t piece_vecs;          // 16-byte vectors per row piece (one block)
    int32_t scale_dwords;        // 4-byte words per scale row (0: none)
    int32_t M, k, Er, E, P, WM;
    int32_t tile_stride;
};

struct CombineArgs {
    const uint8_t* y;            // [W][WM][H] combine dtype
    const float* yw;             // [W][WM][k] or null
    uint8_t* out;                // [W][M][H]
    float* out_w;                // [W][M][k] or null
    const int32_t* fwd;          // [W][M][P]
    int32_t row_vecs;            // 8-element (16-byte) vectors per row
    int32_t piece_vecs;          // vectors per row piece
    int32_t M, k, P;
};

hipError_t launch_route(const RouteArgs& a, const TileMap& tm, hipStream_t s);
hipError_t launch_scan(const ScanArgs& a, int W, hipStream_t s);
// stream: true = streaming cache policy (rows bypass the caches), false =
// cache-allocating moves.
hipError_t launch_copy(const CopyArgs& a, const TileMap& tm, int waves, int row_split,
                       bool stream, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, const TokenMap& tk, int dtype, int waves,
                          int row_split, bool stream, hipStream_t s);

}  // namespace ep
