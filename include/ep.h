/*
 * combine_route_amd: MoE expert-parallel dispatch and combine on one MI355X.
 *
 * C ABI of the GPU library (libcombine_route_amd.so). All W expert-parallel
 * ranks are "virtual": their send and receive buffers live in the one GPU's
 * HBM, side by side, and one call processes every rank at once.
 *
 * Sources (web pages, cited by title and section):
 *  [PR712]  "feat(ep): add opt-in gfx1201 EP2/EP4 support" (ROCm/mori PR 712),
 *           "How the gfx1201 kernels work": the Dispatch and Combine bullets
 *           define the two operations.
 *  [GUIDE]  "MORI-EP User Guide": section 2 (EpDispatchCombineConfig fields),
 *           section 3 (dispatch(), combine(), get_dispatch_src_token_pos()).
 *  [L2]     "MORI (ROCm/mori) — L2 Distillation", section 9: results are views
 *           of preallocated buffers that the next dispatch overwrites.
 *  [PR703]  "refactor(EPv2): replace per-module __device__ staging with shared
 *           buffer" (ROCm/mori PR 703): a caller-allocated buffer sized by one
 *           exported function, and a host-side error naming the argument for a
 *           missing or misaligned buffer (sections "Motivation", "Caller
 *           contract"); receive capacity W * M rows per rank.
 *  [PR726]  "gfx1250 EPv2: EP4 topk-9 geometry; selfFirst follows
 *           MORI_EP_TOKOFF_EXT" (ROCm/mori PR 726): a token has at most
 *           min(W, k) destination rows.
 *  [GUIDE4] "MORI-EP User Guide", section 4 "Standard MoE Compatibility
 *           (DeepEP)": convert_dispatch_output() and convert_combine_input(),
 *           the expert-major (3-D) layout of received rows and its inverse.
 *
 * Notation: W = world_size, M = max_num_inp_token_per_rank, k =
 * num_experts_per_token, Er = num_experts_per_rank, E = W * Er, H =
 * hidden_dim, S = scale_dim, WM = W * M, P = min(W, k). T_r = tokens present
 * on rank r (num_tokens[r] <= M).
 *
 * Semantics (readings of the pages where they are silent are marked R):
 *  - Expert e lives on rank e / Er (R: contiguous blocks, [GUIDE] section 2's
 *    "256 experts / 8 GPUs"). An id outside [0, E) selects no rank (R).
 *  - A token's destination ranks D are its experts' ranks without repeats, in
 *    the order each first appears in its top-k row ([PR712] Dispatch).
 *  - Rank d receives one row per (token, d in D). Its rows are ordered by
 *    (source rank, source token) (R: a deterministic counting-sort layout
 *    replaces the pages' atomic slot reservation). At most WM rows ([PR703]).
 *  - Each received row carries the token's payload row, its whole top-k id
 *    and weight rows verbatim, its scale row, and its source
 *    src_rank * WM + src_token ([GUIDE] get_dispatch_src_token_pos()).
 *  - Combine returns token (r,t) as the FP32 sum of its rows' expert outputs,
 *    in D order, starting from the first, rounded to nearest even into
 *    bf16/fp16 ([PR712] Combine). No routing weight is applied; optional
 *    FP32 weights are summed the same way without a cast. A token with no
 *    rank combines to +0 (R).
 *  All outputs are bit-for-bit deterministic: no atomic operation decides a
 *  position or an order.
 *
 * Errors: every call returns EP_OK (0) or a negative EP_ERR_* code, and
 * ep_last_error() then names the argument at fault. Every precondition is
 * checked on the host before anything is enqueued: on error nothing is
 * enqueued and no output is touched.
 *
 * Devices, streams, threads: a plan's workspace, every buffer passed to it
 * and the streams it is used on belong to one device. A plan holds one
 * routing handle, so a plan must not be used by two threads at once, and its
 * calls on different streams must be ordered by the caller (events); plans
 * are independent of each other. Only sizes and pointers are checked on the
 * host: whether a pointer is device memory of the right size is the
 * caller's responsibility (the Python binding checks both).
 */
#ifndef COMBINE_ROUTE_AMD_EP_H
#define COMBINE_ROUTE_AMD_EP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. Dispatch payload: any of the three (the library copies
 * bytes; EP_FP8_E4M3 is one byte an element). Combine: EP_BF16 or EP_FP16. */
enum { EP_BF16 = 0, EP_FP16 = 1, EP_FP8_E4M3 = 2 };

/* Combine wire formats (the rows the combine reads; R: the pages name
 * fp8_blockwise and fp4 with e8m0 scales, [PR726], [GUIDE] section 10, and
 * the arithmetic follows the OCP OFP8 and MX v1.0 specifications):
 *   EP_WIRE_NONE          rows in combine_dtype.
 *   EP_WIRE_FP8_BLOCK128  OCP E4M3 codes, H bytes a row, with one FP32 scale
 *                         per 128 elements (H / 128 floats a row): value =
 *                         code value * scale.
 *   EP_WIRE_MXFP4         OCP E2M1 codes, two a byte (even element in the low
 *                         nibble), H / 2 bytes a row, with one E8M0 scale per
 *                         32 elements (H / 32 bytes a row): value = code
 *                         value * 2^(scale - 127).
 * ep_quantize_rows writes either from bf16 / fp16 rows. */
enum { EP_WIRE_NONE = 0, EP_WIRE_FP8_BLOCK128 = 1, EP_WIRE_MXFP4 = 2 };

/* Dispatch cast (R: fp8_direct_cast, named by [GUIDE] section 10 and [PR726]):
 *   EP_CAST_NONE           x has dispatch_dtype and its rows are copied.
 *   EP_CAST_FP8_FROM_BF16  x is bf16; dispatch_dtype must be EP_FP8_E4M3;
 *   EP_CAST_FP8_FROM_FP16  x is fp16; every element is received as its OCP
 *                          E4M3 code (round to nearest even, saturating at
 *                          +-448, NaN -> 0x7F), on the fly, with no scale. */
enum { EP_CAST_NONE = 0, EP_CAST_FP8_FROM_BF16 = 1, EP_CAST_FP8_FROM_FP16 = 2 };

enum {
    EP_OK = 0,
    EP_ERR_NULL = -1,  /* a required pointer is NULL                          */
    EP_ERR_ARG = -2,   /* a value out of range or inconsistent                */
    EP_ERR_ALIGN = -3, /* a pointer is not aligned as required                */
    EP_ERR_SIZE = -4,  /* a buffer is too small, or a size overflows          */
    EP_ERR_STATE = -5, /* call order: combine before any dispatch on the plan */
    EP_ERR_HIP = -6    /* the HIP runtime reported an error for a launch      */
};

/* Static configuration, after [GUIDE] section 2's EpDispatchCombineConfig
 * (rank, launch, kernel-type and RDMA fields dropped: one call covers all
 * ranks of one GPU). Valid when:
 *   1 <= world_size <= 64; 1 <= max_num_inp_token_per_rank;
 *   W * W * M <= 2^31 - 1 (src_pos and forward-map entries are int32);
 *   1 <= num_experts_per_token <= 64; 1 <= num_experts_per_rank and
 *   W * num_experts_per_rank <= 2^31 - 1;
 *   hidden_dim >= 1, hidden_dim * elem(dispatch_dtype) % 16 == 0 and
 *   hidden_dim * 2 % 16 == 0 (rows move in 16-byte pieces);
 *   scale_dim >= 0; if scale_dim > 0: scale_type_size in {1, 2, 4, 8} and
 *   scale_dim * scale_type_size % 4 == 0;
 *   dispatch_dtype in {EP_BF16, EP_FP16, EP_FP8_E4M3};
 *   combine_dtype in {EP_BF16, EP_FP16};
 *   combine_wire in EP_WIRE_*: with EP_WIRE_FP8_BLOCK128 hidden_dim % 128 ==
 *   0, with EP_WIRE_MXFP4 hidden_dim % 32 == 0;
 *   dispatch_cast in EP_CAST_*: with a cast, dispatch_dtype == EP_FP8_E4M3. */
typedef struct ep_config {
    int32_t world_size;
    int32_t hidden_dim;
    int32_t scale_dim;
    int32_t scale_type_size;
    int32_t max_num_inp_token_per_rank;
    int32_t num_experts_per_rank;
    int32_t num_experts_per_token;
    int32_t dispatch_dtype;
    int32_t combine_dtype;
    int32_t combine_wire;
    int32_t dispatch_cast;
} ep_config_t;

typedef struct ep_plan ep_plan_t;

/* Bytes of device workspace a plan needs for cfg: routing counts and bases,
 * src_pos [W][WM] int32, the forward map [W][M][P] int32 (the routing handle
 * combine replays). Returns 0 if cfg is NULL or invalid (ep_last_error() says
 * why). [PR703]: one exported function sizes the caller's buffer. */
size_t ep_workspace_bytes(const ep_config_t *cfg);

/* Create a plan. Host-only: validates, records pointers, launches nothing and
 * makes no HIP call. workspace: caller-owned device memory of at least
 * ep_workspace_bytes(cfg) bytes, 256-byte aligned; the plan borrows it and
 * the caller keeps it alive and unused by others until ep_plan_destroy. Its
 * contents need no initialisation.
 * Errors: EP_ERR_NULL (cfg, workspace or out is NULL), EP_ERR_ARG (cfg
 * invalid), EP_ERR_ALIGN (workspace not 256-byte aligned), EP_ERR_SIZE
 * (workspace_bytes too small). On error *out is left unchanged. */
int ep_plan_create(const ep_config_t *cfg, void *workspace, size_t workspace_bytes,
                   ep_plan_t **out);

/* Destroy a plan: waits for the last stream the plan launched on, then frees
 * the plan's host state. The caller frees the workspace afterwards. NULL is a
 * no-op returning EP_OK. EP_ERR_STATE (nothing freed) while expert plans made
 * from it exist. EP_ERR_HIP if that wait fails (the plan is freed anyway).
 * A plan of ep_plan_static is waited for and emptied, not freed. */
int ep_plan_destroy(ep_plan_t *plan);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Like
 * ep_plan_create, but the plan's workspace is the library's own static
 * device array of EP_STATIC_SCRATCH_BYTES (4 MiB; each GPU the library runs
 * on holds one until the process ends), and the plan object is the library's
 * too: one per device, the current device's, reset to cfg by each call. No
 * device or host memory is allocated. The plan serves the current device
 * only; use it with ep_dispatch, ep_combine and the other calls as any plan.
 * Every call on a device returns that device's one plan and shares its one
 * scratch array, whose contents the last call left (nothing in it needs to
 * start at zero): calls of two threads, or work of two streams, that overlap
 * on one device race, so the caller orders them (one stream, or its own
 * events), and a new ep_plan_static call ends the previous plan's state.
 * Errors: EP_ERR_NULL (cfg or out NULL), EP_ERR_ARG (cfg invalid, or a device
 * number past 63), EP_ERR_SIZE (cfg needs a workspace larger than the static
 * array: ep_workspace_bytes(cfg) > EP_STATIC_SCRATCH_BYTES), EP_ERR_STATE
 * (expert plans made from this device's static plan still exist), EP_ERR_HIP
 * (the device or the array's address could not be had). Checks of cfg come
 * first and make no HIP call. */
#define EP_STATIC_SCRATCH_BYTES ((size_t)4 << 20)
int ep_plan_static(const ep_config_t *cfg, ep_plan_t **out);

/* Dispatch arguments. Device pointers are caller-owned, 16-byte aligned, and
 * laid out rank-major with the rank stride fixed by M (not by T_r):
 *   num_tokens     HOST int32 [W]: T_r, 0 <= T_r <= M.
 *   x              [W][M][H] dispatch_dtype (bf16 / fp16 with a dispatch_cast):
 *                  rows t < T_r are read.
 *   indices        [W][M][k] int32 expert ids.
 *   weights        [W][M][k] float, or NULL (then out_weights must be NULL).
 *   scales         [W][M][S] elements of scale_type_size bytes; NULL iff S == 0.
 *   out_x          [W][WM][H] dispatch_dtype.
 *   out_indices    [W][WM][k] int32.
 *   out_weights    [W][WM][k] float, NULL iff weights is NULL.
 *   out_scales     [W][WM][S], NULL iff S == 0.
 *   recv_num_token DEVICE int32 [W]: rows each rank received.
 * Rows s >= recv_num_token[d] of the outputs, and input rows t >= T_r, are
 * neither written nor read. ([GUIDE] section 3, dispatch(): the five outputs
 * and their shapes.) */
typedef struct ep_dispatch_args {
    const int32_t *num_tokens;
    const void *x;
    const int32_t *indices;
    const float *weights;
    const void *scales;
    void *out_x;
    int32_t *out_indices;
    float *out_weights;
    void *out_scales;
    int32_t *recv_num_token;
} ep_dispatch_args_t;

/* Dispatch every rank's tokens ([PR712] Dispatch). Asynchronous on stream (a
 * hipStream_t; NULL = the default stream); no host synchronisation; no
 * allocation; capturable in a HIP graph. Overwrites the plan's routing handle
 * (src_pos and forward map in the workspace): the results of the previous
 * dispatch on this plan are invalid once this call is enqueued ([L2] section
 * 9). The outputs must not overlap the inputs or the workspace.
 * Errors: EP_ERR_NULL, EP_ERR_ARG (T_r out of range, NULL/non-NULL pairing),
 * EP_ERR_ALIGN, EP_ERR_HIP (a launch failed; outputs undefined). */
int ep_dispatch(ep_plan_t *plan, const ep_dispatch_args_t *args, void *stream);

/* Combine arguments (device pointers, 16-byte aligned):
 *   y            [W][WM][H] combine_dtype: expert output for each received
 *                row (rows s < recv_num_token[d] are read). May be the
 *                dispatch's out_x when the types match. With a combine_wire,
 *                [W][WM] rows of that wire format instead.
 *   y_scales     the wire rows' scales, [W][WM][H / 128] float or
 *                [W][WM][H / 32] E8M0 bytes (4-byte aligned); NULL iff
 *                combine_wire is EP_WIRE_NONE.
 *   y_weights    [W][WM][k] float, or NULL (then out_weights must be NULL).
 *   out          [W][M][H] combine_dtype: rows t < T_r of the last dispatch
 *                are written, others untouched. Must not overlap y.
 *   out_weights  [W][M][k] float, NULL iff y_weights is NULL.
 * ([GUIDE] section 3, combine(): combine_output and combine_weights.) */
typedef struct ep_combine_args {
    const void *y;
    const float *y_weights;
    void *out;
    float *out_weights;
    const void *y_scales;
} ep_combine_args_t;

/* Combine ([PR712] Combine) using the routing handle of the last ep_dispatch
 * enqueued on this plan. Asynchronous on stream; no allocation; capturable.
 * May be called any number of times per dispatch (each call recomputes the
 * same sums); no reset between iterations is needed. Two routings in flight
 * need two plans.
 * Errors: EP_ERR_NULL, EP_ERR_ARG (NULL/non-NULL pairing), EP_ERR_ALIGN,
 * EP_ERR_STATE (no dispatch yet on this plan), EP_ERR_HIP. */
int ep_combine(ep_plan_t *plan, const ep_combine_args_t *args, void *stream);

/* Quantize rows[rows][hidden] of in_dtype (EP_BF16 or EP_FP16) into the wire
 * format `wire` (EP_WIRE_FP8_BLOCK128 or EP_WIRE_MXFP4; see EP_WIRE_*), the
 * send side of a quantized combine: out gets the codes, scales the block
 * scales. FP8: s = amax / 448 and codes E4M3(v * (448 / amax)), round to
 * nearest even, saturating (s = 1 for an all-zero block). MXFP4 (the OCP MX
 * conversion): scale 2^(floor(log2 amax) - 2), codes E2M1(v / scale), round
 * to nearest even, saturating at 6 (scale code 0 for an all-zero block).
 * Both wires need finite inputs: a block holding a NaN or an infinity gets
 * unspecified codes and scale (nothing outside the block is affected).
 * Device pointers: in and out 16-byte aligned, scales 4-byte
 * aligned; no plan, no allocation, asynchronous on stream, capturable.
 * row_counts: NULL converts every row. Otherwise the rows form groups of
 * group_rows consecutive rows (rows a multiple of group_rows), row_counts is a
 * device int32 [rows / group_rows] array, and in group g only the first
 * row_counts[g] rows are read and written (the rest of the group's in, out
 * and scales rows are untouched; a count above group_rows means all of them).
 * With recv_num_token and group_rows = world_size * max tokens this converts
 * exactly the rows a combine reads.
 * Errors: EP_ERR_NULL, EP_ERR_ALIGN, EP_ERR_ARG (types, wire, rows < 0,
 * hidden not a positive multiple of the block, group_rows < 1 or not dividing
 * rows when row_counts is given), EP_ERR_SIZE, EP_ERR_HIP. */
int ep_quantize_rows(const void *in, int64_t rows, int32_t hidden, int32_t in_dtype,
                     int32_t wire, void *out, void *scales, const int32_t *row_counts,
                     int64_t group_rows, void *stream);

/* Reverse map of rank `rank` ([GUIDE] section 3, get_dispatch_src_token_pos():
 * src_rank * (world_size * max_num_inp_token_per_rank) + src_token_id).
 * Sets *dev_ptr to a device pointer into the workspace, int32 [WM], of which
 * [0, recv_num_token[rank]) are valid once the last dispatch has completed on
 * its stream; valid until the next ep_dispatch on the plan is enqueued.
 * Makes no HIP call. Errors: EP_ERR_NULL, EP_ERR_ARG (rank not in [0, W)). */
int ep_get_src_token_pos(const ep_plan_t *plan, int32_t rank, const int32_t **dev_ptr);

/* Message for the last error on the calling thread ("" if none). The string
 * stays valid until the next library call on this thread. */
const char *ep_last_error(void);

/* Launch geometry, after the block_num / warp_per_block overrides of
 * [GUIDE] section 3's dispatch() and combine(). A field <= 0 means "choose
 * automatically" (the default). Limits:
 *   tile_tokens          tokens per routing tile: 16, 32 or 64.
 *   dispatch_waves       wavefronts per dispatch-copy block: 1..16.
 *   dispatch_row_split   blocks sharing one tile's rows, each a contiguous
 *                        piece of the row: 1..row_bytes/16.
 *   combine_waves        wavefronts per combine block (a token piece
 *                        each): 1..16.
 *   combine_row_split    pieces a combined row is split into, a wave each:
 *                        1..H/8. A piece of at most 2 KB is folded row by row
 *                        (every contribution row's piece loaded one row at a
 *                        time, two rows in flight); a larger one a column
 *                        chunk at a time. Automatic: calls with 16-token tiles
 *                        cut rows until about 1024 blocks of 4 waves, and
 *                        into pieces of at most 2 KB (rows in the combine
 *                        dtype); larger calls fold 1 KB pieces with 16
 *                        waves, or from wire rows pieces of about 1.75 KB of
 *                        codes with 4 waves.
 *                        In calls of at least 512 tiles of 32 tokens, waves
 *                        are numbered token by token with the pieces fastest
 *                        (neighbouring rows in flight together), as are the
 *                        dispatch copy's blocks (tile, share, piece) and the
 *                        expert-major and fused combines' waves; smaller
 *                        calls, whose blocks are all resident at once, put
 *                        the piece in the grid's y dimension.
 *   cache_policy         EP_CACHE_STREAM: payload rows bypass the caches;
 *                        EP_CACHE_KEEP: rows are cached (best when the call's
 *                        rows fit in the 256 MB last-level cache, e.g. expert
 *                        outputs just written). Automatic: keep when the
 *                        call's rows (every token sent to min(W, k) ranks)
 *                        fit in 256 MB, stream above.
 *   layout               where the receive slots are worked out:
 *                        EP_LAYOUT_KERNELS: a routing kernel counts rows per
 *                        tile and destination, a scan kernel turns the counts
 *                        into first slots (large calls);
 *                        EP_LAYOUT_SCAN_IN_COPY: routing kernel, then each
 *                        dispatch-copy block sums the counts before its tile
 *                        (at most 256 tiles);
 *                        EP_LAYOUT_IN_COPY: no extra kernel; each copy block
 *                        counts every tile of the call itself (k <= 16 and
 *                        tiles x world_size <= 4096, no dispatch_cast;
 *                        otherwise ep_dispatch fails with EP_ERR_ARG).
 *                        Automatic: EP_LAYOUT_IN_COPY up to 256 tokens when
 *                        it fits, else EP_LAYOUT_SCAN_IN_COPY up to 256 tiles,
 *                        else EP_LAYOUT_KERNELS.
 *                        ep_convert_dispatch_output and
 *                        ep_dispatch_standard_moe: EP_LAYOUT_KERNELS makes
 *                        their count and scan two kernels; otherwise a call
 *                        of at most 16 tiles of 64 rows (a rank's received
 *                        rows, resp. (source rank, tile) pairs) with top-k
 *                        <= 16 counts and scans in one kernel, any other in
 *                        two.
 * Geometry, cache policy and layout placement never change results. */
enum {
    EP_LAYOUT_AUTO = 0,
    EP_LAYOUT_KERNELS = 1,
    EP_LAYOUT_SCAN_IN_COPY = 2,
    EP_LAYOUT_IN_COPY = 3
};
enum { EP_CACHE_AUTO = 0, EP_CACHE_STREAM = 1, EP_CACHE_KEEP = 2 };
typedef struct ep_launch {
    int32_t tile_tokens;
    int32_t dispatch_waves;
    int32_t dispatch_row_split;
    int32_t combine_waves;
    int32_t combine_row_split;
    int32_t cache_policy;
    int32_t layout;
    /* Expert-major layout (ep_convert_dispatch_output and its inverse):
     *   expert_waves              wavefronts per copy block (64 received
     *                             rows a block): 1..16.
     *   expert_row_split          pieces a copied row is cut into, a block
     *                             each: 1..row_bytes/16.
     *   expert_combine_waves      wavefronts per inverse block: 1..16.
     *   expert_combine_row_split  pieces an inverse row is split into: 1..H/8
     *                             (folded as combine_row_split says).
     *                             Automatic: as combine_waves and
     *                             combine_row_split for rows in the combine
     *                             dtype. ep_combine_standard_moe takes both
     *                             fields too; its automatic geometry: small
     *                             calls as the combine; large calls fold 2 KB
     *                             pieces with 8 waves, or from wire rows
     *                             pieces of about 3.5 KB of codes with 4.
     *   expert_cache_policy       as cache_policy, for these calls; automatic:
     *                             keep when their rows (each token's
     *                             min(W, k) received rows and k expert rows,
     *                             out and back) stay within 512 MB (rows read
     *                             were just written, so they partly hit the
     *                             256 MB cache), stream above.
     *   expert_token_split        blocks sharing a tile of 64 rows (received
     *                             rows in ep_convert_dispatch_output, source
     *                             tokens in ep_dispatch_standard_moe), each
     *                             copying its share of them: 1..64.
     *   Automatic expert_row_split and expert_token_split: a call whose row
     *   pieces alone give about 1024 copy blocks (512 above top-16) cuts rows
     *   to reach that and, up to top-16, shares each tile among 64 /
     *   expert_waves blocks of one row a wave (above top-16 it shares no
     *   tile); a smaller call shares tiles first (at most 64 / expert_waves
     *   blocks a tile), then cuts rows. ep_plan_get_launch reports the values
     *   of ep_convert_dispatch_output. */
    int32_t expert_waves;
    int32_t expert_row_split;
    int32_t expert_combine_waves;
    int32_t expert_combine_row_split;
    int32_t expert_cache_policy;
    int32_t expert_token_split;
    /* dispatch_token_split: blocks sharing one routing tile of ep_dispatch,
     * each copying ceil(tile_tokens / dispatch_token_split) consecutive
     * tokens of it: 1..64 (values above tile_tokens act as tile_tokens).
     * Blocks are numbered as combine_row_split describes. Every block
     * of a tile routes the whole tile again (its ids only). A launch whose
     * blocks x dispatch_waves x 64 exceed 2^32 - 1 fails with EP_ERR_ARG.
     * Automatic dispatch geometry: calls with 16-token tiles (fewer than
     * 512 tiles of 32 tokens) use 16 waves, no shared tile and rows cut
     * until the grid has about 1024 blocks; larger calls
     * cut rows into pieces of at least 7 KB and, up to top-16, share each
     * tile among blocks of one token a wave (4 waves;
     * dispatch_token_split = tile_tokens / dispatch_waves,
     * recomputed when tile_tokens or dispatch_waves is overridden);
     * above top-16 they share no tile. */
    int32_t dispatch_token_split;
} ep_launch_t;

/* Override (launch != NULL) or reset to automatic (launch == NULL) the plan's
 * geometry. Host-only. EP_ERR_ARG if a field is out of its limits. */
int ep_plan_set_launch(ep_plan_t *plan, const ep_launch_t *launch);

/* The geometry a call with these token counts would use (host [W] int32).
 * Host-only. */
int ep_plan_get_launch(const ep_plan_t *plan, const int32_t *num_tokens, ep_launch_t *out);

/* Per-kernel timing with HIP events, for measurement. While enabled, every
 * kernel the plan launches is bracketed by two events recorded on its
 * stream; ep_plan_kernel_time waits for the recorded events and returns, for
 * one kernel, how many launches were timed and their total milliseconds since
 * enabling. Kernels: EP_KERNEL_ROUTE (per-tile rank counts), EP_KERNEL_SCAN
 * (receive layout), EP_KERNEL_COPY (dispatch row and metadata copy),
 * EP_KERNEL_COMBINE (gather-reduce), and those of the plan's expert plans:
 * EP_KERNEL_EXPERT_COUNT (per-tile expert counts), EP_KERNEL_EXPERT_SCAN
 * (expert lists and layout ranges), EP_KERNEL_EXPERT_COPY (rows into the
 * expert-major layout), EP_KERNEL_EXPERT_COMBINE (the inverse), and the
 * fused path's EP_KERNEL_STANDARD_COUNT, _SCAN, _COPY (ep_dispatch_standard_moe)
 * and EP_KERNEL_STANDARD_COMBINE (ep_combine_standard_moe). A kernel a call
 * does not launch counts nothing: the route and scan kernels of small calls
 * (launch.layout), and the expert and fused count kernels of calls that count
 * and scan in one launch (timed as the scan). Enabling creates the events (no
 * device memory); disabling destroys them. Not for use under graph capture. */
enum {
    EP_KERNEL_ROUTE = 0,
    EP_KERNEL_SCAN = 1,
    EP_KERNEL_COPY = 2,
    EP_KERNEL_COMBINE = 3,
    EP_KERNEL_EXPERT_COUNT = 4,
    EP_KERNEL_EXPERT_SCAN = 5,
    EP_KERNEL_EXPERT_COPY = 6,
    EP_KERNEL_EXPERT_COMBINE = 7,
    EP_KERNEL_STANDARD_COUNT = 8,
    EP_KERNEL_STANDARD_SCAN = 9,
    EP_KERNEL_STANDARD_COPY = 10,
    EP_KERNEL_STANDARD_COMBINE = 11
};
int ep_plan_set_timing(ep_plan_t *plan, int enable);
int ep_plan_kernel_time(ep_plan_t *plan, int kernel, int32_t *count, double *total_ms);

/* ------------------------------------------------------------------------
 * Expert-major layout ([GUIDE4]). After a dispatch, each rank's received
 * rows are regrouped by the local expert that processes them, the layout a
 * grouped GEMM reads ([W][Er][cap][H]); the inverse turns the experts'
 * outputs back into one combine input row per received row.
 *
 * Semantics (readings of [GUIDE4], which names the calls and outputs only):
 *  - On rank d, a received row goes once to each distinct local expert j
 *    (global id d * Er + j) among its ids (R). An expert's rows keep the
 *    receive order, so they are grouped by source rank (R).
 *  - cap (1 <= cap <= WM, chosen by the caller) rows are kept per expert;
 *    rows at positions >= cap are dropped, and the count still includes them,
 *    so count > cap shows an overflow (R). cap = WM never drops.
 *  - src_info is the row's source token index within its source rank (R);
 *    layout_range[d][j][s] = (lo << 32) | (hi - lo), lo and hi the list
 *    positions where source rank s's rows start and end, each clipped to
 *    cap (R).
 *  - The inverse writes, for every received row, the FP32 sum of its kept
 *    experts' outputs in the order its local experts first appear in its ids,
 *    from the first, rounded to nearest even once (R, like combine); a row
 *    with none is +0. On request each output is first scaled by its expert's
 *    routing weight for the row, with a fused multiply-add (R).
 * Deterministic bit for bit, like the rest of the library.
 * ------------------------------------------------------------------------ */
typedef struct ep_expert_plan ep_expert_plan_t;

/* Bytes of device workspace an expert plan of capacity cap needs on top of
 * its plan's: per-tile expert counts and bases, source starts, the map
 * [W][WM][min(k, Er)] int32 the inverse gathers through and its weights
 * [W][WM][min(k, Er)] float. Returns 0 if plan is
 * NULL or cap is out of range (1 <= cap <= WM and W * Er * cap <= 2^31 - 1);
 * ep_last_error() says why. */
size_t ep_expert_workspace_bytes(const ep_plan_t *plan, int32_t cap);

/* Create an expert plan on top of a plan, whose config it shares and whose
 * last dispatch it converts. Host-only, no HIP call. workspace: caller-owned
 * device memory of at least ep_expert_workspace_bytes(plan, cap) bytes,
 * 256-byte aligned, kept alive until ep_expert_plan_destroy; no
 * initialisation needed. The plan must outlive it.
 * Errors: EP_ERR_NULL, EP_ERR_ARG (cap), EP_ERR_ALIGN, EP_ERR_SIZE. */
int ep_expert_plan_create(ep_plan_t *plan, int32_t cap, void *workspace,
                          size_t workspace_bytes, ep_expert_plan_t **out);

/* Waits for the last stream the expert plan launched on, then frees it. NULL
 * is a no-op. EP_ERR_HIP if the wait fails (freed anyway). */
int ep_expert_plan_destroy(ep_expert_plan_t *plan);

/* Arguments of ep_convert_dispatch_output. Inputs are the outputs of the
 * plan's last ep_dispatch (the call reads that dispatch's src_pos from the
 * plan's workspace):
 *   x                    [W][WM][H] dispatch_dtype (the dispatch's out_x),
 *                        16-byte aligned.
 *   indices              [W][WM][k] int32 (out_indices).
 *   weights              [W][WM][k] float (out_weights), or NULL. Given, each
 *                        kept (row, expert) pair records its expert's weight
 *                        for the row, the FP32 sum in slot order of the row's
 *                        weights on the slots naming that expert (R), for a
 *                        weighted inverse.
 *   scales               [W][WM][S] (out_scales); NULL iff S == 0.
 *   recv_num_token       DEVICE int32 [W] (recv_num_token). The expert plan
 *                        keeps this pointer: ep_convert_combine_input reads
 *                        the counts through it again, so the buffer must stay
 *                        allocated and hold the same counts until the last
 *                        inverse of this conversion has run on its stream.
 * Outputs (device, caller-owned, must not overlap the inputs or workspaces):
 *   packed_x             [W][Er][cap][H] dispatch_dtype, 16-byte aligned:
 *                        slots p < min(count, cap) are written.
 *   packed_scales        [W][Er][cap][S]; NULL iff S == 0.
 *   packed_count         [W][Er] int32.
 *   packed_src_info      [W][Er][cap] int32: slots p < min(count, cap).
 *   packed_layout_range  [W][Er][W] int64, 8-byte aligned.
 * Slots past min(count, cap) are left untouched. ([GUIDE4]: the four
 * outputs of convert_dispatch_output, and the scales beside packed_x.) */
typedef struct ep_convert_dispatch_args {
    const void *x;
    const int32_t *indices;
    const float *weights;
    const void *scales;
    const int32_t *recv_num_token;
    void *packed_x;
    void *packed_scales;
    int32_t *packed_count;
    int32_t *packed_src_info;
    int64_t *packed_layout_range;
} ep_convert_dispatch_args_t;

/* Regroup the received rows of every rank by local expert ([GUIDE4]
 * convert_dispatch_output). Asynchronous on stream; no allocation;
 * capturable. Overwrites the expert plan's map: the inverse then works on
 * this conversion.
 * Errors: EP_ERR_NULL, EP_ERR_ALIGN, EP_ERR_ARG (scales pairing),
 * EP_ERR_STATE (no dispatch yet on the plan), EP_ERR_HIP. */
int ep_convert_dispatch_output(ep_expert_plan_t *plan, const ep_convert_dispatch_args_t *args,
                               void *stream);

/* Arguments of ep_convert_combine_input (device pointers 16-byte aligned):
 *   packed_y       [W][Er][cap][H] combine_dtype: the experts' outputs, slot
 *                  for slot with packed_x (slots past min(count, cap) are not
 *                  read).
 *   y              [W][WM][H] combine_dtype: rows q < recv_num_token[d] are
 *                  written (the combine input, ep_combine_args_t.y); others
 *                  untouched. Must not overlap packed_y.
 *   apply_weights  0: the plain sum. 1: each output is scaled by its
 *                  expert's weight for the row (recorded by the conversion,
 *                  which must have been given weights): acc = c * v for the
 *                  first kept output, then acc = fma(c, v, acc) ([GUIDE]
 *                  section 3: combine weights are for a weighted
 *                  combination). The plain combine after it then gives the
 *                  mixture sum over a token's slots of w_i * expert_i(x). */
typedef struct ep_convert_combine_args {
    const void *packed_y;
    void *y;
    int32_t apply_weights;
} ep_convert_combine_args_t;

/* The inverse ([GUIDE4] convert_combine_input), through the map of the last
 * ep_convert_dispatch_output on this expert plan, which must have converted
 * the plan's current dispatch. Asynchronous; no allocation; capturable; may be
 * called any number of times per conversion. It reads the row counts from the
 * recv_num_token buffer that conversion was given (the caller keeps that
 * buffer alive and unchanged meanwhile; a freed or rewritten buffer gives
 * wrong rows, bounded by the capacity W * M).
 * Errors: EP_ERR_NULL, EP_ERR_ALIGN, EP_ERR_ARG (apply_weights not 0 or 1),
 * EP_ERR_STATE (no conversion yet, the plan dispatched again since, or
 * weights asked for and the conversion had none), EP_ERR_HIP. */
int ep_convert_combine_input(ep_expert_plan_t *plan, const ep_convert_combine_args_t *args,
                             void *stream);

/* Arguments of ep_dispatch_standard_moe (device pointers 16-byte aligned, id,
 * count and info arrays 4-byte, layout ranges 8-byte; shapes as in
 * ep_dispatch_args_t and ep_convert_dispatch_args_t):
 *   num_tokens           host [W]: tokens T_r of each source rank, <= M.
 *   x                    [W][M][H] dispatch_dtype (with a dispatch_cast, bf16 or
 *                        fp16, each element written to packed_x as its E4M3
 *                        code); rows t < T_r are read.
 *   indices              [W][M][k] int32 expert ids.
 *   scales               [W][M][scale_dim] or NULL iff scale_dim == 0.
 *   packed_x             [W][Er][cap][H] dispatch_dtype.
 *   packed_scales        [W][Er][cap][scale_dim] or NULL iff scale_dim == 0.
 *   packed_count         [W][Er] int32: tokens naming each expert (dropped
 *                        ones included).
 *   packed_src_info      [W][Er][cap] int32: the source token index within its
 *                        source rank.
 *   packed_layout_range  [W][Er][W] int64: (lo << 32) | (hi - lo), the list
 *                        positions of each source rank's rows, clipped to cap.
 * The routing weights are not part of the layout: ep_combine_standard_moe
 * takes them. */
typedef struct ep_dispatch_standard_args {
    const int32_t *num_tokens;
    const void *x;
    const int32_t *indices;
    const void *scales;
    void *packed_x;
    void *packed_scales;
    int32_t *packed_count;
    int32_t *packed_src_info;
    int64_t *packed_layout_range;
} ep_dispatch_standard_args_t;

/* Dispatch straight into the expert-major layout ([GUIDE4]
 * dispatch_standard_moe: dispatch and format conversion in one call). The
 * outputs are exactly those of ep_dispatch followed by
 * ep_convert_dispatch_output with the same capacity, without the
 * intermediate receive buffer: expert e = d * Er + j keeps the tokens naming
 * it in source-rank, then token order, a token once per distinct expert,
 * positions >= cap dropped. Uses only the expert plan's configuration and
 * workspace (not the plan's routing handle, which it leaves alone); it
 * records the map ep_combine_standard_moe reads and ends any conversion on
 * this expert plan (ep_convert_combine_input then fails until the next
 * ep_convert_dispatch_output). With a dispatch_cast the packed rows hold the
 * E4M3 codes the cast dispatch would have received.
 * Asynchronous on stream; no allocation; capturable.
 * Errors: EP_ERR_NULL, EP_ERR_ALIGN, EP_ERR_ARG (token counts, scales
 * pairing), EP_ERR_HIP. */
int ep_dispatch_standard_moe(ep_expert_plan_t *plan, const ep_dispatch_standard_args_t *args,
                             void *stream);

/* Arguments of ep_combine_standard_moe (device pointers; packed_y and out
 * 16-byte aligned, indices and weights 4-byte):
 *   packed_y  [W][Er][cap][H] combine_dtype: the experts' outputs, slot for
 *             slot with packed_x (slots past min(count, cap) are not read).
 *   indices   [W][M][k] int32: the ids given to the last
 *             ep_dispatch_standard_moe on this expert plan.
 *   weights   [W][M][k] float routing weights to apply, or NULL (the plain
 *             sum).
 *   out       [W][M][H] combine_dtype: rows t < T_r of the last fused
 *             dispatch are written, others untouched. Must not overlap
 *             packed_y.
 *   packed_y_scales  with a combine_wire config, packed_y holds the outputs
 *             as wire rows ([W][Er][cap] rows of that format, as
 *             ep_quantize_rows writes them) and this their scale rows
 *             ([W][Er][cap][H / 128] float or [W][Er][cap][H / 32] E8M0,
 *             4-byte aligned); each element is decoded to its exact value
 *             before the fold. NULL iff combine_wire is EP_WIRE_NONE. */
typedef struct ep_combine_standard_args {
    const void *packed_y;
    const int32_t *indices;
    const float *weights;
    void *out;
    const void *packed_y_scales;
} ep_combine_standard_args_t;

/* Combine straight from the expert-major layout ([GUIDE4]
 * combine_standard_moe). The result is exactly that of
 * ep_convert_combine_input (apply_weights = weights != NULL) followed by
 * ep_combine, without the intermediate rows: for each of the token's ranks in
 * its rank order, the FP32 fold of the rank's kept expert outputs in
 * first-occurrence order (weighted: c * v, then fma), rounded to
 * combine_dtype; those summed in FP32 from the first and rounded once to
 * nearest even. A rank whose pairs were all dropped adds +0. Uses the map of
 * the last ep_dispatch_standard_moe on this expert plan. Asynchronous; no
 * allocation; capturable; may be called any number of times per dispatch.
 * Errors: EP_ERR_NULL, EP_ERR_ALIGN, EP_ERR_ARG (packed_y_scales pairing),
 * EP_ERR_STATE (no fused dispatch yet on this expert plan), EP_ERR_HIP. */
int ep_combine_standard_moe(ep_expert_plan_t *plan, const ep_combine_standard_args_t *args,
                            void *stream);

#ifdef __cplusplus
}
#endif

#endif /* COMBINE_ROUTE_AMD_EP_H */
