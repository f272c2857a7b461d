/*
 * Access-pattern probes: a measurement aid beside the dispatch/combine ABI
 * of ep.h, not part of the method.
 *
 * The dispatch copy and the combine are bound by HBM bandwidth, and how much
 * of its peak this memory delivers depends on the access pattern: streams
 * read or written at once, and how reads and writes interleave. Each probe
 * moves the bytes of one pattern with the routing, metadata and layout work
 * taken out, so a kernel's rate can be set against the rate the same memory
 * reaches on its own pattern, in the same process, on the same buffers:
 *
 *   EP_PROBE_READ    read  rows x row_bytes of src (streaming loads)
 *   EP_PROBE_WRITE   write rows x row_bytes of dst
 *   EP_PROBE_COPY    dst row i = src row i, i < rows
 *   EP_PROBE_FANOUT  each src row t (t < rows) to every dst row
 *                    map[t * stride + i] >= 0: the dispatch copy's payload
 *                    moves at the dispatch's own destinations when map is
 *                    the plan's forward map ("feat(ep): add opt-in gfx1201
 *                    EP2/EP4 support", Dispatch: one row per (token, rank))
 *   EP_PROBE_GATHER  dst row t = bf16(FP32 sum of the bf16 src rows
 *                    map[t * stride + i] >= 0, in list order): the combine's
 *                    payload moves and fold (same page, Combine)
 *
 * Loads stream past the caches, as the kernels' loads do on calls past the
 * 256 MB MALL; READ writes one word per wave to dst so its loads are used;
 * GATHER's stores stream, the others' do not, as in the kernels.
 */
#ifndef EP_PROBE_H
#define EP_PROBE_H

#include <stdint.h>

#include "ep.h"

#ifdef __cplusplus
extern "C" {
#endif

enum {
    EP_PROBE_READ = 0,
    EP_PROBE_WRITE = 1,
    EP_PROBE_COPY = 2,
    EP_PROBE_FANOUT = 3,
    EP_PROBE_GATHER = 4
};

/* Arguments (device pointers 16-byte aligned, caller-owned):
 *   kind       EP_PROBE_*.
 *   row_bytes  bytes of a row: > 0, a multiple of 16 (of 2 for GATHER rows,
 *              which are bf16).
 *   rows       rows of the pattern (>= 0): src rows of READ, COPY and
 *              FANOUT, dst rows of WRITE and GATHER.
 *   src        READ, COPY: [rows][row_bytes]; FANOUT: [rows][row_bytes];
 *              GATHER: [map_rows][row_bytes]. NULL for WRITE.
 *   dst        WRITE, COPY: [rows][row_bytes]; FANOUT: [map_rows][row_bytes];
 *              GATHER: [rows][row_bytes]; READ: [rows * pieces] uint32.
 *   map        FANOUT / GATHER: int32 [rows][stride] row numbers of dst /
 *              src, a list ended by the first entry < 0 (or by stride).
 *              Entries >= map_rows are skipped. NULL for the others.
 *   map_rows   rows of dst (FANOUT) or src (GATHER).
 *   stride     entries a map row holds (1..64).
 *   pieces     waves a row is split over (1..64): each moves one piece.
 *   waves      waves a block (1..16).
 * Asynchronous on stream (a hipStream_t, NULL for the default stream); no
 * allocation. Errors (nothing enqueued): EP_ERR_NULL, EP_ERR_ALIGN,
 * EP_ERR_ARG (a field out of range); EP_ERR_HIP for a failed launch. */
typedef struct ep_probe_args {
    int32_t kind;
    int32_t row_bytes;
    int64_t rows;
    const void *src;
    void *dst;
    const int32_t *map;
    int64_t map_rows;
    int32_t stride;
    int32_t pieces;
    int32_t waves;
} ep_probe_args_t;

int ep_probe_pattern(const ep_probe_args_t *args, void *stream);

/* The plan's forward map in its workspace: int32 [W][M][stride], stride =
 * min(W, k); entry (r, t, i) is the flat receive row d * W * M + s of the
 * token's i-th distinct rank, -1 past its ranks. Valid once the last
 * ep_dispatch on the plan has completed on its stream, until the next one.
 * Host-only. Errors: EP_ERR_NULL. */
int ep_probe_forward_map(const ep_plan_t *plan, const int32_t **map, int32_t *stride);

#ifdef __cplusplus
}
#endif

#endif /* EP_PROBE_H */
