/*
 * CPU oracle for MoE expert-parallel dispatch and combine.
 *
 * TEST INFRASTRUCTURE ONLY. This is a plain, slow, single-threaded definition
 * of what dispatch and combine compute. It exists to check the GPU library
 * against; nothing on the product path may include, link or call it. It
 * shares no code, header, table or helper with the GPU library.
 *
 * Sources (web pages, cited by title and section):
 *  [PR712]  "feat(ep): add opt-in gfx1201 EP2/EP4 support" (ROCm/mori PR 712),
 *           section "How the gfx1201 kernels work": the Dispatch and Combine
 *           bullets define the method.
 *  [GUIDE]  "MORI-EP User Guide", section 3 "Operator API": dispatch() and
 *           combine() outputs and shapes; get_dispatch_src_token_pos() gives
 *           the reverse-map encoding.
 *  [PR726]  "gfx1250 EPv2: EP4 topk-9 geometry; selfFirst follows
 *           MORI_EP_TOKOFF_EXT" (ROCm/mori PR 726): a token's combine rows
 *           come from at most min(world size, top-k) distinct ranks.
 *  [PR703]  "refactor(EPv2): replace per-module __device__ staging with shared
 *           buffer" (ROCm/mori PR 703), section "Motivation": the receive
 *           capacity of a rank is world size x max tokens per rank.
 *  [GUIDE4] "MORI-EP User Guide", section 4 "Standard MoE Compatibility
 *           (DeepEP)": convert_dispatch_output() turns a rank's received rows
 *           into the expert-major layout (packed rows, counts, source info,
 *           layout ranges) and convert_combine_input() turns expert-major
 *           outputs back into one combine row per received row.
 *
 * Readings taken where the pages are silent (each also listed in the design
 * notes): expert e lives on rank e / experts_per_rank; received rows on a
 * rank are ordered by (source rank, source token); the combine sum runs in
 * first-occurrence top-k order of the token's distinct ranks, seeded with the
 * first contribution; the FP32 result is rounded to nearest even; an expert
 * id outside [0, E) selects no rank; a token with no rank combines to +0.
 * Expert-major layout (section 4 names the calls and outputs only): a
 * received row goes once to each distinct local expert among its ids; an
 * expert's rows keep the receive order; rows past the capacity are dropped
 * but counted; source info is the source token index; a layout range packs
 * (start << 32) | count of one source rank's rows in an expert's list; the
 * inverse sums a row's kept expert outputs in first-occurrence order like the
 * combine and rounds once; weighted, each output is scaled by the sum of the
 * row's weights on the slots naming its expert, with a fused multiply-add.
 *
 * Parity status: every function here is pinned by tests that do not call it
 * through itself (brute force, a second formulation, closed forms, library
 * conversions); none is "parity unpinned".
 */
#ifndef EP_ORACLE_H
#define EP_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Dispatch, by definition.
 *   W ranks, M = max tokens per rank, k = top-k, Er = experts per rank.
 *   row_bytes   = bytes of one payload row (hidden x element size).
 *   scale_bytes = bytes of one scale row (0: no scales, sc/out_sc unused).
 *   ntok[W]                 tokens present on each rank (<= M).
 *   x[W][M][row_bytes]      payload rows (only t < ntok[r] are read).
 *   idx[W][M][k]            expert ids.
 *   w[W][M][k]              routing weights (may be NULL: out_w unused).
 *   sc[W][M][scale_bytes]   scale rows.
 * Outputs, with WM = W * M:
 *   out_x[W][WM][row_bytes], out_idx[W][WM][k], out_w[W][WM][k],
 *   out_sc[W][WM][scale_bytes]: rows s < recv[d] are written, others untouched.
 *   recv[W]                 rows received by each rank.
 *   src_pos[W][WM]          src_rank * WM + src_token for each received row.
 *   fwd[W][M][P], P = min(W, k): for token (r,t), entry i is d * WM + s for
 *                           the i-th distinct rank d of the token, -1 after.
 * Returns 0, or -1 on a size overflow. */
int oracle_dispatch(int W, int M, int k, int Er, size_t row_bytes, size_t scale_bytes,
                    const int32_t *ntok, const uint8_t *x, const int32_t *idx,
                    const float *w, const uint8_t *sc,
                    uint8_t *out_x, int32_t *out_idx, float *out_w, uint8_t *out_sc,
                    int32_t *recv, int32_t *src_pos, int32_t *fwd);

/* Second formulation of the receive layout: every (d, r, t) triple with d a
 * rank of token (r,t) is sorted by the C library's qsort on (d, r, t), and a
 * row's slot is its position among the triples of its d. Writes recv[W] and
 * src_pos[W][WM]. Returns 0, or -1 if memory runs out. */
int oracle_layout_by_sort(int W, int M, int k, int Er, const int32_t *ntok,
                          const int32_t *idx, int32_t *recv, int32_t *src_pos);

/* Combine, by definition (gather form).
 *   H = hidden size, dtype 0 = bf16, 1 = fp16 for y and out.
 *   fwd[W][M][P] as written by oracle_dispatch.
 *   y[W][WM][H]   expert outputs, one per received row.
 *   y_w[W][WM][k] optional FP32 weights to sum (NULL: out_w unused).
 * out[W][M][H] and out_w[W][M][k]: rows t < ntok[r] are written. */
int oracle_combine(int W, int M, int k, int H, int dtype, const int32_t *ntok,
                   const int32_t *fwd, const uint16_t *y, const float *y_w,
                   uint16_t *out, float *out_w);

/* Combine, second formulation (scatter-add, the push-back of [PR712]
 * Combine): every received row is added into its source token's FP32
 * accumulator, found through src_pos. Rows are pushed in passes by the place
 * their rank takes in the token's distinct-rank order (that place computed
 * from the id row on its own, not from a rank list), the first place seeding
 * the accumulator. Shares no accumulation code with oracle_combine, so the
 * two are independent formulations of one result. Needs idx for the places.
 * Returns 0, -1 if memory runs out, -2 if a token's rows are not exactly one
 * per distinct rank. W <= 64. */
int oracle_combine_push(int W, int M, int k, int Er, int H, int dtype,
                        const int32_t *ntok, const int32_t *idx,
                        const int32_t *recv, const int32_t *src_pos,
                        const uint16_t *y, const float *y_w,
                        uint16_t *out, float *out_w);

/* Expert-major layout of the received rows, by definition ([GUIDE4],
 * convert_dispatch_output).
 *   Inputs are dispatch outputs: recv[W], src_pos[W][WM], x[W][WM][row_bytes],
 *   idx[W][WM][k] (global expert ids), sc[W][WM][scale_bytes] (scale_bytes 0:
 *   sc/psc unused). Er experts per rank; cap = rows kept per local expert.
 * Outputs, for each rank d and local expert j (global id d * Er + j):
 *   count[W][Er]            received rows that name expert j (all of them,
 *                           also those past cap).
 *   px[W][Er][cap][row_bytes], psc[W][Er][cap][scale_bytes],
 *   src_info[W][Er][cap]    the p-th row of j's list (p < min(count, cap)):
 *                           its payload, its scales, its source token index.
 *                           Slots past that are untouched.
 *   layout_range[W][Er][W]  for source rank s: (lo << 32) | (hi - lo), with lo
 *                           and hi the list positions where s's rows start and
 *                           end, each clipped to cap.
 * Returns 0, or -1 if memory runs out. */
int oracle_expert_layout(int W, int M, int k, int Er, int cap, size_t row_bytes,
                         size_t scale_bytes, const int32_t *recv, const int32_t *src_pos,
                         const uint8_t *x, const int32_t *idx, const uint8_t *sc,
                         uint8_t *px, uint8_t *psc, int32_t *count, int32_t *src_info,
                         int64_t *layout_range);

/* The inverse ([GUIDE4], convert_combine_input): for every received row q <
 * recv[d] of rank d, the sum of its kept expert outputs py[d][j][p] (bf16 or
 * fp16, H wide), in the order its local experts first appear in its id row,
 * folded in FP32 from the first and rounded once; a row with none is +0.
 * With routing weights w[W][WM][k] (the dispatched weight rows; NULL for the
 * unweighted sum), each output is scaled by its expert's weight for the row,
 * the FP32 sum of the row's weights on the slots naming that expert (slot
 * order, from the first): acc = c * v for the first kept output, then
 * acc = fma(c, v, acc) ("MORI-EP User Guide", section 3: combine weights are
 * for a weighted combination).
 * Writes y[W][WM][H] rows q < recv[d]; others untouched. Returns 0. */
int oracle_expert_combine(int W, int M, int k, int Er, int cap, int H, int dtype,
                          const int32_t *recv, const int32_t *idx, const float *w,
                          const uint16_t *py, uint16_t *y);

/* ------------------------------------------------------------------------
 * Quantized wires ([PR726] and [GUIDE] section 10 name fp8_direct_cast,
 * fp8_blockwise and fp4 with e8m0 scales without defining them; the
 * definitions below follow the formats' published specifications, OCP
 * "8-bit Floating Point Specification (OFP8)" for E4M3 and OCP
 * "Microscaling Formats (MX) v1.0" for E2M1, E8M0 and the MX conversion).
 * Readings: round to nearest even; finite values past the largest magnitude
 * saturate to it; an E4M3 NaN input becomes 0x7F; blockwise FP8 uses blocks
 * of 128 elements with an FP32 scale s = amax / 448 and elements multiplied
 * by r = 448 / amax (s = 1, r = 1 for an all-zero block); MXFP4 uses blocks
 * of 32 with scale 2^(floor(log2 amax) - 2) (E8M0 code 0 for an all-zero
 * block), two E2M1 codes a byte, the even element in the low nibble. MX
 * inputs are finite.
 * ------------------------------------------------------------------------ */
enum { ORACLE_WIRE_FP8_BLOCK128 = 1, ORACLE_WIRE_MXFP4 = 2 };

/* OCP E4M3 (bias 7, no infinities, largest 448, NaN S.1111.111). */
uint8_t oracle_f32_to_e4m3(float v);
float oracle_e4m3_to_f32(uint8_t c);
/* OCP E2M1 (bias 1, magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6): a 4-bit code. */
uint8_t oracle_f32_to_e2m1(float v);
float oracle_e2m1_to_f32(uint8_t c);

/* Bulk direct cast: bf16 (dtype 0) or fp16 (1) words -> E4M3 codes. */
void oracle_cast_to_e4m3_n(const uint16_t *in, int dtype, uint8_t *out, size_t n);

/* Quantize rows[n][H] of bf16 (dtype 0) / fp16 (1) into a wire format:
 *   ORACLE_WIRE_FP8_BLOCK128: out[n][H] E4M3 codes, scales[n][H/128] float.
 *   ORACLE_WIRE_MXFP4:        out[n][H/2] packed E2M1, scales[n][H/32] E8M0.
 * Returns 0, or -1 if H does not divide into blocks. */
int oracle_quantize_rows(int64_t n, int H, int dtype, int wire, const uint16_t *in,
                         uint8_t *out, void *scales);

/* One element of a wire row, back in FP32: E4M3 value times the block's
 * scale (one FP32 multiply), or E2M1 value times 2^(code - 127) (exact). */
float oracle_wire_value(int wire, const uint8_t *row, const void *scale_row, int h);

/* Combine from a wire (gather form): like oracle_combine, with each
 * contribution element taken through oracle_wire_value before the FP32 fold.
 *   y[W][WM][...] wire rows, y_scales[W][WM][...] their scales. */
int oracle_combine_wire(int W, int M, int k, int H, int dtype, int wire, const int32_t *ntok,
                        const int32_t *fwd, const uint8_t *y, const void *y_scales,
                        uint16_t *out);

/* The expert-major inverse (oracle_expert_combine) with the packed expert
 * outputs on a wire: each element is taken through oracle_wire_value (its
 * exact FP32 value) instead of being widened from bf16 / fp16, then folded
 * the same way.
 *   py[W][Er][cap][...] wire rows, py_scales[W][Er][cap][...] their scales. */
int oracle_expert_combine_wire(int W, int M, int k, int Er, int cap, int H, int dtype, int wire,
                               const int32_t *recv, const int32_t *idx, const float *w,
                               const uint8_t *py, const void *py_scales, uint16_t *y);

/* IEEE 754 conversions used by the combine cast, written from the formats'
 * definitions: binary32 -> bfloat16 / binary16 with round-to-nearest-even,
 * overflow to infinity, NaN to a quiet NaN; and the exact widenings back. */
uint16_t oracle_f32_to_bf16(float f);
uint16_t oracle_f32_to_f16(float f);
float oracle_bf16_to_f32(uint16_t h);
float oracle_f16_to_f32(uint16_t h);

/* Bulk forms of the four conversions, for tests. */
void oracle_f32_to_bf16_n(const float *in, uint16_t *out, size_t n);
void oracle_f32_to_f16_n(const float *in, uint16_t *out, size_t n);
void oracle_bf16_to_f32_n(const uint16_t *in, float *out, size_t n);
void oracle_f16_to_f32_n(const uint16_t *in, float *out, size_t n);

#ifdef __cplusplus
}
#endif

#endif /* EP_ORACLE_H */
