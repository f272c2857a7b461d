// Internal interface between the host side of the library (ep_plan.cpp) and
// its gfx950 kernels (ep_kernels.hip: dispatch and combine; ep_expert.hip:
// the expert-major layout of received rows and its inverse; ep_wire.hip: the
// quantized combine wire). Not installed; the public ABI is include/ep.h.
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
    int32_t row_vecs;            // 16-byte vectors per payload row (of x)
    int32_t piece_vecs;          // 16-byte vectors per row piece (one block)
    int32_t scale_dwords;        // 4-byte words per scale row (0: none)
    int32_t M, k, Er, E, P, WM;
    int32_t tile_stride;
    int32_t cast;                // 0: rows copied; 1 / 2: bf16 / fp16 x cast to E4M3
    // Blocks: one per (tile, token share, row piece). piece_inner: a 1-D
    // grid numbered tile, share, piece, the piece fastest, so blocks started
    // together touch neighbouring rows (calls larger than the GPU holds at
    // once); otherwise a 2-D grid, x = (tile, share), y = piece. A share is
    // ceil(tile_tokens / token_split) consecutive tokens.
    int32_t pieces;              // row pieces: ceil(row_vecs / piece_vecs)
    int32_t token_split;         // token shares a tile
    int32_t piece_inner;
};

struct CombineArgs {
    const uint8_t* y;            // [W][WM][H] combine dtype
    const float* yw;             // [W][WM][k] or null
    uint8_t* out;                // [W][M][H]
    float* out_w;                // [W][M][k] or null
    const int32_t* fwd;          // [W][M][P]
    int32_t row_vecs;            // 8-element (16-byte) vectors per row
    int32_t piece_vecs;          // vectors per row piece
    int32_t pieces;              // ceil(row_vecs / piece_vecs): a wave each
    int32_t piece_inner;         // 1: waves numbered (token, piece), piece fastest,
                                 // in a 1-D grid; 0: grid y = piece
    int32_t M, k, P;
};

// Expert-major layout of the received rows of every rank. A tile is 64
// consecutive received rows of one rank (one lane each); T tiles a rank cover
// the most rows any rank can hold in this call. A list is one (rank, local
// expert) pair, g = d * Er + j.
struct ExpertArgs {
    const uint8_t* x;            // [W][WM][row_bytes] received rows
    const int32_t* idx;          // [W][WM][k] their expert ids
    const float* w;              // [W][WM][k] their routing weights, or null
    const uint32_t* sc;          // [W][WM][scale_dwords] or null
    const int32_t* recv;         // [W] received rows of each rank
    const int32_t* src_pos;      // [W][WM] src_rank * WM + src_token
    uint8_t* px;                 // [W][Er][cap][row_bytes]
    uint32_t* psc;               // [W][Er][cap][scale_dwords] or null
    int32_t* count;              // [W][Er] rows naming each local expert
    int32_t* src_info;           // [W][Er][cap] source token index
    int64_t* layout_range;       // [W][Er][W] (lo << 32) | n, clipped to cap
    int32_t* tile_counts;        // [W * Er][T] rows of tile t naming the list's expert
    int32_t* tile_base;          // [W * Er][T] position of tile t's first such row
    int32_t* src_start;          // [W][W] first received row from each source rank
    int32_t* src_prefix;         // [W * Er][W] rows naming the expert in that row's tile before it
    int32_t* efwd;               // [W][WM][Pe] kept packed rows of each received row
    float* ew;                   // [W][WM][Pe] their experts' weights (when w is set)
    int32_t row_vecs;            // 16-byte vectors per payload row
    int32_t piece_vecs;          // vectors per row piece (one block)
    int32_t scale_dwords;        // 4-byte words per scale row (0: none)
    int32_t W, WM, k, Er, Pe, cap;
    int32_t rows;                // most received rows any rank can hold in this call
    int32_t T;                   // tiles a rank: max(1, ceil(rows / 64))
    int32_t token_split;         // copy blocks sharing a tile, each with its share of rows
};

struct ExpertCombineArgs {
    const uint8_t* py;           // [W][Er][cap][H] expert outputs, combine dtype
    const int32_t* recv;         // [W]
    const int32_t* efwd;         // [W][WM][Pe]
    const float* ew;             // [W][WM][Pe] weights to apply, or null (plain sum)
    uint8_t* y;                  // [W][WM][H]
    int32_t row_vecs;            // 16-byte vectors per row
    int32_t piece_vecs;
    int32_t pieces;              // ceil(row_vecs / piece_vecs): a wave each
    int32_t piece_inner;         // as CombineArgs::piece_inner, rows for tokens
    int32_t WM, Pe;
    int32_t rows;                // most received rows any rank can hold in this call
};

// Fused expert-major dispatch and combine (ep_standard.hip): the source
// tokens go straight to the packed rows, and the combine folds the packed
// expert outputs straight into the token's output row.
struct StandardArgs {
    const uint8_t* x;            // [W][M][row_bytes] source tokens
    const int32_t* idx;          // [W][M][k] their expert ids
    const uint32_t* sc;          // [W][M][scale_dwords] or null
    uint8_t* px;                 // [W * Er][cap][row_bytes]
    uint32_t* psc;               // [W * Er][cap][scale_dwords] or null
    int32_t* count;              // [W * Er] tokens naming each expert
    int32_t* src_info;           // [W * Er][cap] source token index within its rank
    int64_t* layout_range;       // [W * Er][W] (lo << 32) | n, clipped to cap
    int32_t* tile_counts;        // [W * Er][W * Tr] tokens of (rank, tile) naming the expert
    int32_t* tile_base;          // [W * Er][W * Tr] position of that tile's first one
    int32_t* fslot;              // [W][M][k] packed row of a kept first-occurrence slot, else -1
    int32_t row_vecs;            // 16-byte vectors per source row
    int32_t piece_vecs;          // vectors per row piece (one block)
    uint32_t out_row_bytes;      // bytes per packed row (half a source row with a cast)
    int32_t cast;                // 0, or the source type (1 bf16, 2 fp16) cast to E4M3
    int32_t scale_dwords;
    int32_t W, M, k, Er, E, cap;
    int32_t Tr;                  // tiles a source rank: max(1, ceil(M / 64))
    int32_t token_split;         // copy blocks sharing a tile, each with its share of tokens
    int32_t ntok[kMaxRanks];     // T_r
};

struct StandardCombineArgs {
    const uint8_t* py;           // [W * Er][cap] expert outputs: combine dtype or wire rows
    const uint8_t* pys;          // [W * Er][cap] wire scale rows, or null
    const int32_t* idx;          // [W][M][k]
    const float* w;              // [W][M][k] routing weights to apply, or null
    const int32_t* fslot;        // [W][M][k]
    uint8_t* out;                // [W][M][H]
    int32_t row_vecs;            // 16-byte vectors (8 elements) per output row
    int32_t piece_vecs;          // with a wire: a multiple of 16, at most 1024
    uint32_t py_row_bytes;       // bytes per wire row (unused without a wire)
    uint32_t py_scale_bytes;     // bytes per wire scale row
    int32_t wire;                // 0, kWireFp8Block128 or kWireMxfp4
    int32_t pieces;              // ceil(row_vecs / piece_vecs): a wave each
    int32_t piece_inner;         // as CombineArgs::piece_inner
    int32_t M, k, Er, E;
};

// Quantized combine wire (ep_wire.hip).
constexpr int kWireFp8Block128 = 1;  // E4M3 codes, one FP32 scale per 128 elements
constexpr int kWireMxfp4 = 2;        // packed E2M1 codes, one E8M0 scale per 32

// A quantize wave converts up to kQuantChunks chunks of kQuantChunk elements.
constexpr int kQuantChunk = 512;
constexpr int kQuantChunks = 8;

struct QuantizeArgs {
    const uint8_t* in;           // [rows][H] bf16 / fp16
    uint8_t* out;                // [rows][H] E4M3 or [rows][H / 2] packed E2M1
    uint8_t* scales;             // [rows][H / 128] float or [rows][H / 32] E8M0
    const int32_t* counts;       // [rows / group_rows] rows kept per group, or null
    int64_t rows;
    int64_t group_rows;
    int32_t H;
    int32_t pieces;              // row pieces (a wave each)
    int32_t piece_chunks;        // chunks of a piece, <= kQuantChunks
};

struct WireCombineArgs {
    const uint8_t* y;            // [W][WM] wire rows of row_bytes
    const uint8_t* ys;           // [W][WM] scale rows of scale_bytes
    const float* yw;             // [W][WM][k] or null
    uint8_t* out;                // [W][M][H] combine dtype
    float* out_w;                // [W][M][k] or null
    const int32_t* fwd;          // [W][M][P]
    int32_t units;               // 16-element units per row (H / 16)
    int32_t piece_units;         // units per row piece: a multiple of 8, <= kWirePieceUnits
    int32_t pieces;              // ceil(units / piece_units): a wave each
    int32_t piece_inner;         // as CombineArgs::piece_inner
    uint32_t row_bytes, scale_bytes;
    int32_t M, k, P;
};

// Most 16-element units in a wire combine's row piece: 64 lanes each hold
// one scale dword (128 elements) of a contribution row.
constexpr int kWirePieceUnits = 512;

hipError_t launch_route(const RouteArgs& a, const TileMap& tm, hipStream_t s);
hipError_t launch_scan(const ScanArgs& a, int W, hipStream_t s);
// stream: true = streaming cache policy (rows bypass the caches), false =
// cache-allocating moves.
hipError_t launch_copy(const CopyArgs& a, const TileMap& tm, int waves, bool stream,
                       hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, const TokenMap& tk, int dtype, int waves,
                          bool stream, hipStream_t s);

hipError_t launch_expert_count(const ExpertArgs& a, hipStream_t s);
// Small calls count and scan in one launch, a tile a wave, and the count
// launch is not made: at most kCountScanTiles tiles (a rank's for the
// expert-major layout, (source rank, tile) pairs for the fused dispatch) and
// top-k at most kCountScanTopK. Every block of it reads the call's ids, which
// measured slower than two launches at 64 tiles of top-64 tokens.
constexpr int kCountScanTiles = 16;
constexpr int kCountScanTopK = 16;
hipError_t launch_expert_count_scan(const ExpertArgs& a, hipStream_t s);
hipError_t launch_expert_scan(const ExpertArgs& a, hipStream_t s);
hipError_t launch_expert_copy(const ExpertArgs& a, int waves, int row_split, bool stream,
                              hipStream_t s);
hipError_t launch_expert_combine(const ExpertCombineArgs& a, int W, int dtype, int waves,
                                 bool stream, hipStream_t s);

hipError_t launch_standard_count(const StandardArgs& a, hipStream_t s);
hipError_t launch_standard_count_scan(const StandardArgs& a, hipStream_t s);
hipError_t launch_standard_scan(const StandardArgs& a, hipStream_t s);
hipError_t launch_standard_copy(const StandardArgs& a, int waves, int row_split, bool stream,
                                hipStream_t s);
hipError_t launch_standard_combine(const StandardCombineArgs& a, const TokenMap& tk, int dtype,
                                   int waves, bool stream, hipStream_t s);
hipError_t launch_quantize(const QuantizeArgs& a, int wire, int dtype, bool stream, hipStream_t s);
hipError_t launch_combine_wire(const WireCombineArgs& a, const TokenMap& tk, int wire, int dtype,
                               int waves, bool stream, hipStream_t s);

// Access-pattern probes (include/ep_probe.h); kind is an EP_PROBE_* value.
struct ProbeArgs {
    int32_t kind;
    uint32_t row_bytes;
    int64_t rows;
    const uint8_t* src;
    uint8_t* dst;
    const int32_t* map;
    int64_t map_rows;
    int32_t stride;
    int32_t pieces;
};
hipError_t launch_probe(const ProbeArgs& a, int waves, hipStream_t s);

}  // namespace ep
