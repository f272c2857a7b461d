/*
 * CPU oracle for MoE expert-parallel dispatch and combine.
 *
 * TEST INFRASTRUCTURE ONLY: a plain, slow, obviously correct definition that
 * the GPU library is checked against. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it. It shares no code with the GPU
 * library. Page citations and the readings taken are listed in ep_oracle.h.
 *
 * Built with a host C compiler in ISO C11 mode: binary32 arithmetic in SSE
 * registers, round-to-nearest-even, no contraction, no reassociation.
 */
#include "ep_oracle.h"

#include <stdlib.h>
#include <string.h>
#include <math.h>

/* ------------------------------------------------------------------------ */
/* IEEE 754 conversions, from the formats' definitions.                      */
/* ------------------------------------------------------------------------ */

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* bfloat16 keeps binary32's sign and 8-bit exponent and the top 7 fraction
 * bits. Binary32 encodings of one sign are ordered like their magnitudes, so
 * rounding to nearest on the encoding is rounding to nearest on the value: drop
 * the low 16 bits, round up when they exceed half, or equal half and the kept
 * part is odd. A carry out of the fraction moves to the next binade, and out of
 * the largest finite value to infinity, as the format requires. */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u = f32_bits(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)
        return 0x7FC0; /* NaN -> quiet NaN */
    uint32_t kept = u >> 16;
    uint32_t dropped = u & 0xFFFFu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))
        kept += 1;
    return (uint16_t)kept;
}

float oracle_bf16_to_f32(uint16_t h) { return bits_f32((uint32_t)h << 16); }

/* binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits; normal values
 * (1 + f/1024) * 2^(e-15) for e in 1..30; subnormals f * 2^-24; e = 31 is
 * infinity / NaN. The largest finite value is 65504; the rounding boundary to
 * infinity is 65520 (a tie that rounds to the even neighbour, which is 2^16,
 * i.e. infinity). */
uint16_t oracle_f32_to_f16(float f)
{
    uint32_t u = f32_bits(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t e32 = (u >> 23) & 0xFFu;
    uint32_t frac = u & 0x007FFFFFu;
    if (e32 == 0xFFu)
        return frac ? (uint16_t)0x7E00 : (uint16_t)(sign | 0x7C00u);
    if (fabsf(f) >= 65520.0f)
        return (uint16_t)(sign | 0x7C00u);
    if (e32 == 0)           /* binary32 zero or subnormal: |f| < 2^-126, far */
        return sign;        /* below half of the smallest binary16 subnormal  */
    /* |f| = sig * 2^(e - 23), sig in [2^23, 2^24), e = unbiased exponent. */
    int e = (int)e32 - 127;
    uint64_t sig = (uint64_t)(frac | 0x00800000u);
    /* binary16 quantum at this magnitude: 2^(max(e, -14) - 10). */
    int qe = (e < -14 ? -14 : e) - 10;
    int shift = qe - (e - 23); /* low bits of sig below the quantum (>= 13) */
    uint64_t n;
    if (shift >= 40) {
        n = 0;              /* far below half a quantum */
    } else {
        n = sig >> shift;
        uint64_t rem = sig & ((1ull << shift) - 1);
        uint64_t half = 1ull << (shift - 1);
        if (rem > half || (rem == half && (n & 1u)))
            n += 1;
    }
    /* magnitude = n * 2^qe. Normal range (e >= -14): n in [1024, 2048],
     * exponent field e + 15 and fraction n - 1024, where n = 2048 carries into
     * the exponent. Subnormal range: the encoding is n itself, and n = 1024
     * is exactly the smallest normal's encoding. Both are one formula. */
    int ebase = (e < -14 ? -14 : e) + 14;
    uint32_t mag = ((uint32_t)ebase << 10) + (uint32_t)n;
    return (uint16_t)(sign | mag);
}

float oracle_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    float v;
    if (e == 0)
        v = ldexpf((float)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexpf((float)(1024 + f), e - 25);
    return sign ? -v : v;
}

void oracle_f32_to_bf16_n(const float *in, uint16_t *out, size_t n)
{ for (size_t i = 0; i < n; ++i) out[i] = oracle_f32_to_bf16(in[i]); }
void oracle_f32_to_f16_n(const float *in, uint16_t *out, size_t n)
{ for (size_t i = 0; i < n; ++i) out[i] = oracle_f32_to_f16(in[i]); }
void oracle_bf16_to_f32_n(const uint16_t *in, float *out, size_t n)
{ for (size_t i = 0; i < n; ++i) out[i] = oracle_bf16_to_f32(in[i]); }
void oracle_f16_to_f32_n(const uint16_t *in, float *out, size_t n)
{ for (size_t i = 0; i < n; ++i) out[i] = oracle_f16_to_f32(in[i]); }

/* ------------------------------------------------------------------------ */
/* Routing: the ordered distinct destination ranks of one token.             */
/* ------------------------------------------------------------------------ */

/* [PR712] "How the gfx1201 kernels work", Dispatch: a token's selected
 * experts map to destination ranks, and experts on the same rank share one
 * payload. Expert e lives on rank e / Er (ranks hold contiguous blocks of
 * experts_per_rank experts; [GUIDE] section 2 shows 256 experts over 8 ranks
 * as 32 a rank). Ranks are listed in the order their first expert appears in
 * the top-k row. An id outside [0, W*Er) selects no rank. */
static int token_ranks(const int32_t *idx_row, int k, int Er, int W, int32_t *ranks)
{
    int n = 0;
    for (int j = 0; j < k; ++j) {
        int32_t e = idx_row[j];
        if (e < 0 || e >= W * Er)
            continue;
        int32_t d = e / Er;
        int seen = 0;
        for (int q = 0; q < n; ++q)
            if (ranks[q] == d)
                seen = 1;
        if (!seen)
            ranks[n++] = d;
    }
    return n;
}

/* ------------------------------------------------------------------------ */
/* Dispatch.                                                                 */
/* ------------------------------------------------------------------------ */

int oracle_dispatch(int W, int M, int k, int Er, size_t row_bytes, size_t scale_bytes,
                    const int32_t *ntok, const uint8_t *x, const int32_t *idx,
                    const float *w, const uint8_t *sc,
                    uint8_t *out_x, int32_t *out_idx, float *out_w, uint8_t *out_sc,
                    int32_t *recv, int32_t *src_pos, int32_t *fwd)
{
    const int64_t WM = (int64_t)W * M;
    if (WM * W > 2147483647LL)
        return -1;
    const int P = W < k ? W : k;

    /* Step 1: each token's ordered distinct ranks. */
    int32_t *ranks = malloc(sizeof(int32_t) * (size_t)WM * (size_t)P);
    int32_t *nr = malloc(sizeof(int32_t) * (size_t)WM);
    int64_t *cnt = calloc((size_t)W * W, sizeof(int64_t));
    int64_t *base = calloc((size_t)W * W, sizeof(int64_t));
    int64_t *run = calloc((size_t)W * W, sizeof(int64_t));
    if (!ranks || !nr || !cnt || !base || !run) {
        free(ranks); free(nr); free(cnt); free(base); free(run);
        return -1;
    }
    for (int r = 0; r < W; ++r)
        for (int t = 0; t < ntok[r]; ++t) {
            int64_t tok = (int64_t)r * M + t;
            nr[tok] = token_ranks(idx + tok * k, k, Er, W, ranks + tok * P);
        }

    /* Step 2: cnt[r][d] tokens of rank r that go to d; the rows rank d
     * receives are grouped by source rank in ascending order, so source r's
     * group on d starts at the sum of the groups of ranks r' < r. */
    for (int r = 0; r < W; ++r)
        for (int t = 0; t < ntok[r]; ++t) {
            int64_t tok = (int64_t)r * M + t;
            for (int i = 0; i < nr[tok]; ++i)
                cnt[(int64_t)r * W + ranks[tok * P + i]] += 1;
        }
    for (int d = 0; d < W; ++d) {
        int64_t acc = 0;
        for (int r = 0; r < W; ++r) {
            base[(int64_t)r * W + d] = acc;
            acc += cnt[(int64_t)r * W + d];
        }
        recv[d] = (int32_t)acc;
    }

    /* Step 3: walk tokens in (rank, token) order; each (token, rank) pair
     * takes the next row of its group. [PR712] Dispatch: one receive row per
     * token per destination rank, the payload and routing metadata copied to
     * it, and the way back to the source recorded. [GUIDE] dispatch() returns
     * the received tokens with their weights, scales and expert indices;
     * get_dispatch_src_token_pos() encodes a row's source as
     * src_rank * (world_size * max_num_inp_token_per_rank) + src_token_id. */
    for (int r = 0; r < W; ++r)
        for (int t = 0; t < ntok[r]; ++t) {
            int64_t tok = (int64_t)r * M + t;
            for (int i = 0; i < P; ++i)
                fwd[tok * P + i] = -1;
            for (int i = 0; i < nr[tok]; ++i) {
                int d = ranks[tok * P + i];
                int64_t s = base[(int64_t)r * W + d] + run[(int64_t)r * W + d];
                run[(int64_t)r * W + d] += 1;
                int64_t row = (int64_t)d * WM + s;
                memcpy(out_x + (size_t)row * row_bytes, x + (size_t)tok * row_bytes, row_bytes);
                memcpy(out_idx + (size_t)row * k, idx + (size_t)tok * k, sizeof(int32_t) * (size_t)k);
                if (w)
                    memcpy(out_w + (size_t)row * k, w + (size_t)tok * k, sizeof(float) * (size_t)k);
                if (scale_bytes)
                    memcpy(out_sc + (size_t)row * scale_bytes, sc + (size_t)tok * scale_bytes, scale_bytes);
                src_pos[row] = (int32_t)((int64_t)r * WM + t);
                fwd[tok * P + i] = (int32_t)row;
            }
        }

    free(ranks); free(nr); free(cnt); free(base); free(run);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Layout, second formulation: sort the (d, r, t) triples.                   */
/* ------------------------------------------------------------------------ */

typedef struct { int32_t d, r, t; } triple_t;

static int triple_cmp(const void *a, const void *b)
{
    const triple_t *x = a, *y = b;
    if (x->d != y->d) return x->d < y->d ? -1 : 1;
    if (x->r != y->r) return x->r < y->r ? -1 : 1;
    if (x->t != y->t) return x->t < y->t ? -1 : 1;
    return 0;
}

int oracle_layout_by_sort(int W, int M, int k, int Er, const int32_t *ntok,
                          const int32_t *idx, int32_t *recv, int32_t *src_pos)
{
    const int64_t WM = (int64_t)W * M;
    const int P = W < k ? W : k;
    triple_t *tri = malloc(sizeof(triple_t) * (size_t)(WM * P + 1));
    int32_t *ranks = malloc(sizeof(int32_t) * (size_t)P);
    if (!tri || !ranks) { free(tri); free(ranks); return -1; }
    int64_t n = 0;
    for (int r = 0; r < W; ++r)
        for (int t = 0; t < ntok[r]; ++t) {
            int nd = token_ranks(idx + ((int64_t)r * M + t) * k, k, Er, W, ranks);
            for (int i = 0; i < nd; ++i) {
                tri[n].d = ranks[i]; tri[n].r = r; tri[n].t = t;
                ++n;
            }
        }
    qsort(tri, (size_t)n, sizeof(triple_t), triple_cmp);
    for (int d = 0; d < W; ++d)
        recv[d] = 0;
    for (int64_t q = 0; q < n; ++q) {
        int d = tri[q].d;
        int64_t s = recv[d]++;
        src_pos[(int64_t)d * WM + s] = (int32_t)((int64_t)tri[q].r * WM + tri[q].t);
    }
    free(tri); free(ranks);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Combine.                                                                  */
/* ------------------------------------------------------------------------ */

static float widen(uint16_t v, int dtype)
{ return dtype == 0 ? oracle_bf16_to_f32(v) : oracle_f16_to_f32(v); }
static uint16_t narrow(float v, int dtype)
{ return dtype == 0 ? oracle_f32_to_bf16(v) : oracle_f32_to_f16(v); }

/* Fold one token's n contribution rows (flat row numbers rows[0..n)) in the
 * given order. [PR712] "How the gfx1201 kernels work", Combine: the source
 * sums its contributions in FP32, then converts the output to BF16/FP16;
 * optional FP32 weights are summed separately and no routing weight is
 * applied. The sum starts from the first contribution and adds the rest one
 * at a time in the token's distinct-rank order; an empty sum is +0. */
static void fold_token(int n, const int64_t *rows, int H, int k, int dtype,
                       const uint16_t *y, const float *y_w, uint16_t *out_row, float *out_w_row)
{
    for (int h = 0; h < H; ++h) {
        if (n == 0) {
            out_row[h] = 0;
            continue;
        }
        float acc = widen(y[(size_t)rows[0] * H + h], dtype);
        for (int i = 1; i < n; ++i)
            acc = acc + widen(y[(size_t)rows[i] * H + h], dtype);
        out_row[h] = narrow(acc, dtype);
    }
    if (y_w && out_w_row) {
        for (int j = 0; j < k; ++j) {
            if (n == 0) {
                out_w_row[j] = 0.0f;
                continue;
            }
            float acc = y_w[(size_t)rows[0] * k + j];
            for (int i = 1; i < n; ++i)
                acc = acc + y_w[(size_t)rows[i] * k + j];
            out_w_row[j] = acc;
        }
    }
}

int oracle_combine(int W, int M, int k, int H, int dtype, const int32_t *ntok,
                   const int32_t *fwd, const uint16_t *y, const float *y_w,
                   uint16_t *out, float *out_w)
{
    const int P = W < k ? W : k;
    int64_t rows[64];
    for (int r = 0; r < W; ++r)
        for (int t = 0; t < ntok[r]; ++t) {
            int64_t tok = (int64_t)r * M + t;
            int n = 0;
            for (int i = 0; i < P; ++i)
                if (fwd[tok * P + i] >= 0)
                    rows[n++] = fwd[tok * P + i];
            fold_token(n, rows, H, k, dtype, y, y_w, out + (size_t)tok * H,
                       out_w ? out_w + (size_t)tok * k : NULL);
        }
    return 0;
}

/* Place of rank d in a token's distinct-rank order, found without building
 * the list: the id row's first expert on d sits at some slot; every rank whose
 * first expert comes before that slot takes an earlier place. -1 if none of
 * the token's ids is on d. */
static int rank_place(const int32_t *idx_row, int k, int Er, int W, int d)
{
    const int64_t E = (int64_t)W * Er;
    int first = -1;
    for (int j = 0; j < k && first < 0; ++j)
        if (idx_row[j] >= 0 && idx_row[j] < E && idx_row[j] / Er == d)
            first = j;
    if (first < 0)
        return -1;
    int place = 0;
    for (int j = 0; j < first; ++j) {
        if (idx_row[j] < 0 || idx_row[j] >= E)
            continue;
        int dj = idx_row[j] / Er, seen_before = 0;
        for (int q = 0; q < j; ++q)
            if (idx_row[q] >= 0 && idx_row[q] < E && idx_row[q] / Er == dj)
                seen_before = 1;
        place += !seen_before;     /* slot j holds the first expert of rank dj */
    }
    return place;
}

int oracle_combine_push(int W, int M, int k, int Er, int H, int dtype,
                        const int32_t *ntok, const int32_t *idx,
                        const int32_t *recv, const int32_t *src_pos,
                        const uint16_t *y, const float *y_w,
                        uint16_t *out, float *out_w)
{
    const int64_t WM = (int64_t)W * M;
    const int P = W < k ? W : k;
    float *acc = malloc(sizeof(float) * (size_t)(WM * H + 1));
    float *accw = malloc(sizeof(float) * (size_t)(WM * k + 1));
    int32_t *added = calloc((size_t)(WM + 1), sizeof(int32_t));
    int rc = 0;
    if (!acc || !accw || !added) {
        rc = -1;
        goto done;
    }
    /* Scatter-add: each received row is pushed back into its source token's
     * FP32 accumulator. The rows of place 0 (the token's first rank) go first
     * and start the accumulator with their value; the rows of place 1 are
     * added next, and so on, so every token adds its contributions in its
     * distinct-rank order ([PR712] Combine: sum in FP32, then convert). */
    for (int place = 0; place < P; ++place)
        for (int d = 0; d < W; ++d)
            for (int32_t s = 0; s < recv[d]; ++s) {
                int64_t row = (int64_t)d * WM + s;
                int64_t p = src_pos[row];
                int64_t tok = (p / WM) * M + p % WM;
                if (rank_place(idx + tok * k, k, Er, W, d) != place)
                    continue;
                if (added[tok] != place) {  /* a place skipped or sent twice */
                    rc = -2;
                    goto done;
                }
                float *a = acc + tok * H;
                const uint16_t *v = y + row * H;
                for (int h = 0; h < H; ++h) {
                    float f = dtype == 0 ? oracle_bf16_to_f32(v[h]) : oracle_f16_to_f32(v[h]);
                    a[h] = place == 0 ? f : a[h] + f;
                }
                if (y_w) {
                    float *aw = accw + tok * k;
                    for (int j = 0; j < k; ++j)
                        aw[j] = place == 0 ? y_w[row * k + j] : aw[j] + y_w[row * k + j];
                }
                added[tok] += 1;
            }
    /* Every token must have received one row from each of its ranks; a token
     * with none sums to +0. The FP32 sum is rounded once to the output type. */
    for (int r = 0; r < W; ++r)
        for (int t = 0; t < ntok[r]; ++t) {
            int64_t tok = (int64_t)r * M + t;
            uint64_t ranks = 0;
            for (int j = 0; j < k; ++j) {
                int32_t e = idx[tok * k + j];
                if (e >= 0 && e < (int64_t)W * Er)
                    ranks |= 1ull << (e / Er);
            }
            int nd = 0;
            for (int d = 0; d < W; ++d)
                nd += (int)((ranks >> d) & 1u);
            if (added[tok] != nd) {
                rc = -2;
                goto done;
            }
            for (int h = 0; h < H; ++h)
                out[tok * H + h] = nd == 0 ? 0
                    : (dtype == 0 ? oracle_f32_to_bf16(acc[tok * H + h])
                                  : oracle_f32_to_f16(acc[tok * H + h]));
            if (y_w && out_w)
                for (int j = 0; j < k; ++j)
                    out_w[tok * k + j] = nd == 0 ? 0.0f : accw[tok * k + j];
        }
done:
    free(acc);
    free(accw);
    free(added);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Expert-major layout and its inverse.                                      */
/* ------------------------------------------------------------------------ */

/* Local experts of one received row on rank d, in the order they first
 * appear in its id row: [GUIDE4] groups a rank's received rows by the local
 * expert that processes them, and an expert processes a row once, so a
 * repeated id adds nothing. Ids of other ranks' experts and ids outside
 * [0, W*Er) are not local. Returns the count; js[] gets j = e - d * Er. */
static int row_local_experts(const int32_t *idx_row, int k, int Er, int d, int32_t *js)
{
    int n = 0;
    for (int i = 0; i < k; ++i) {
        int32_t e = idx_row[i];
        if (e < (int64_t)d * Er || e >= (int64_t)(d + 1) * Er)
            continue;
        int32_t j = e - d * Er;
        int seen = 0;
        for (int q = 0; q < n; ++q)
            if (js[q] == j)
                seen = 1;
        if (!seen)
            js[n++] = j;
    }
    return n;
}

int oracle_expert_layout(int W, int M, int k, int Er, int cap, size_t row_bytes,
                         size_t scale_bytes, const int32_t *recv, const int32_t *src_pos,
                         const uint8_t *x, const int32_t *idx, const uint8_t *sc,
                         uint8_t *px, uint8_t *psc, int32_t *count, int32_t *src_info,
                         int64_t *layout_range)
{
    const int64_t WM = (int64_t)W * M;
    int32_t *js = malloc(sizeof(int32_t) * (size_t)(k > 0 ? k : 1));
    /* srcs[d][j][p]: source rank of the p-th row of expert j's full list */
    int32_t *srcs = malloc(sizeof(int32_t) * (size_t)(WM + 1));
    if (!js || !srcs) { free(js); free(srcs); return -1; }

    for (int d = 0; d < W; ++d) {
        int32_t *cnt = count + (int64_t)d * Er;
        for (int j = 0; j < Er; ++j)
            cnt[j] = 0;
        /* Step 1: walk the rank's received rows in receive order; each (row,
         * local expert) pair takes the next position of that expert's list.
         * Positions below cap are stored: the row's payload, scales and the
         * source token index of its src_pos entry. */
        for (int64_t q = 0; q < recv[d]; ++q) {
            int64_t row = (int64_t)d * WM + q;
            int n = row_local_experts(idx + row * k, k, Er, d, js);
            for (int i = 0; i < n; ++i) {
                int j = js[i];
                int64_t p = cnt[j]++;
                if (p >= cap)
                    continue;
                int64_t slot = ((int64_t)d * Er + j) * cap + p;
                memcpy(px + (size_t)slot * row_bytes, x + (size_t)row * row_bytes, row_bytes);
                if (scale_bytes)
                    memcpy(psc + (size_t)slot * scale_bytes, sc + (size_t)row * scale_bytes,
                           scale_bytes);
                src_info[slot] = (int32_t)(src_pos[row] % WM);
            }
        }
        /* Step 2: layout ranges. For expert j and source rank s, lo counts the
         * list entries whose row came from a rank below s and hi those from a
         * rank up to s; both are clipped to cap, since only kept rows are in
         * packed_x. The lists are walked again entry by entry. */
        for (int j = 0; j < Er; ++j) {
            int64_t n = 0;
            for (int64_t q = 0; q < recv[d]; ++q) {
                int64_t row = (int64_t)d * WM + q;
                int nl = row_local_experts(idx + row * k, k, Er, d, js);
                for (int i = 0; i < nl; ++i)
                    if (js[i] == j)
                        srcs[n++] = (int32_t)(src_pos[row] / WM);
            }
            for (int s = 0; s < W; ++s) {
                int64_t lo = 0, hi = 0;
                for (int64_t p = 0; p < n; ++p) {
                    lo += srcs[p] < s;
                    hi += srcs[p] <= s;
                }
                if (lo > cap) lo = cap;
                if (hi > cap) hi = cap;
                layout_range[((int64_t)d * Er + j) * W + s] = (lo << 32) | (hi - lo);
            }
        }
    }
    free(js);
    free(srcs);
    return 0;
}

/* The value of element h of packed row `row`, as the inverse folds it. */
typedef float (*packed_value_fn)(const void *src, int64_t row, int H, int h);

struct packed_words {
    const uint16_t *py;  /* [rows][H] bf16 / fp16 words */
    int dtype;
};

static float packed_word_value(const void *src, int64_t row, int H, int h)
{
    const struct packed_words *s = src;
    return widen(s->py[(size_t)row * H + h], s->dtype);
}

/* Inverse of the expert-major layout, reading packed values through `value`
 * (the two public forms below differ only in where a value comes from). */
static int expert_combine(int W, int M, int k, int Er, int cap, int H, int dtype,
                          const int32_t *recv, const int32_t *idx, const float *w,
                          packed_value_fn value, const void *src, uint16_t *y)
{
    const int64_t WM = (int64_t)W * M;
    int32_t *js = malloc(sizeof(int32_t) * (size_t)(k > 0 ? k : 1));
    int64_t *rows = malloc(sizeof(int64_t) * (size_t)(k > 0 ? k : 1));
    float *cw = malloc(sizeof(float) * (size_t)(k > 0 ? k : 1));
    int64_t *next = malloc(sizeof(int64_t) * (size_t)Er);
    if (!js || !rows || !cw || !next) { free(js); free(rows); free(cw); free(next); return -1; }
    for (int d = 0; d < W; ++d) {
        for (int j = 0; j < Er; ++j)
            next[j] = 0;
        /* Each received row finds its expert outputs at the positions step 1
         * of the layout gave it, and sums the kept ones in the order its local
         * experts first appear, like the combine sums a token's ranks. */
        for (int64_t q = 0; q < recv[d]; ++q) {
            int64_t row = (int64_t)d * WM + q;
            int n = row_local_experts(idx + row * k, k, Er, d, js);
            int kept = 0;
            for (int i = 0; i < n; ++i) {
                int64_t p = next[js[i]]++;
                if (p >= cap)
                    continue;
                rows[kept] = ((int64_t)d * Er + js[i]) * cap + p;
                if (w) {
                    /* the expert's weight: the row's weights on every slot
                     * that names it, summed in slot order from the first */
                    int first = 1;
                    float c = 0.0f;
                    for (int s = 0; s < k; ++s)
                        if (idx[row * k + s] == d * Er + js[i]) {
                            c = first ? w[row * k + s] : c + w[row * k + s];
                            first = 0;
                        }
                    cw[kept] = c;
                }
                ++kept;
            }
            uint16_t *out = y + (size_t)row * H;
            for (int h = 0; h < H; ++h) {
                if (kept == 0) {
                    out[h] = 0;
                    continue;
                }
                /* unweighted: the first output, then plain FP32 adds (as the
                 * combine folds); weighted: c * v, then one fused
                 * multiply-add per later output */
                float acc = value(src, rows[0], H, h);
                if (w)
                    acc = cw[0] * acc;
                for (int i = 1; i < kept; ++i) {
                    float v = value(src, rows[i], H, h);
                    acc = w ? fmaf(cw[i], v, acc) : acc + v;
                }
                out[h] = narrow(acc, dtype);
            }
        }
    }
    free(js);
    free(rows);
    free(cw);
    free(next);
    return 0;
}

int oracle_expert_combine(int W, int M, int k, int Er, int cap, int H, int dtype,
                          const int32_t *recv, const int32_t *idx, const float *w,
                          const uint16_t *py, uint16_t *y)
{
    struct packed_words src = {py, dtype};
    return expert_combine(W, M, k, Er, cap, H, dtype, recv, idx, w, packed_word_value, &src, y);
}

/* ------------------------------------------------------------------------ */
/* Quantized wires.                                                          */
/* ------------------------------------------------------------------------ */

/* E4M3: a code S.EEEE.MMM is (-1)^S * 2^(E-7) * (1 + M/8) for E >= 1 and
 * (-1)^S * 2^-6 * M/8 for E = 0; S.1111.111 is NaN, so the largest finite
 * magnitude is S.1111.110 = 448. */
float oracle_e4m3_to_f32(uint8_t c)
{
    int sign = c >> 7, e = (c >> 3) & 0xF, m = c & 7;
    if (e == 15 && m == 7)
        return NAN;
    float v = e == 0 ? ldexpf((float)m, -9) : ldexpf((float)(8 + m), e - 10);
    return sign ? -v : v;
}

/* Nearest finite E4M3 value: codes 0..0x7E of one sign are ordered like
 * their magnitudes, so a binary search finds the two neighbours of |v|; the
 * nearer wins and a tie goes to the code whose mantissa is even; beyond 448
 * saturate. */
uint8_t oracle_f32_to_e4m3(float v)
{
    if (isnan(v))
        return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0;
    double a = fabs((double)v);
    if (a >= 448.0)
        return sign | 0x7E;
    int lo = 0, hi = 0x7E;             /* value(lo) <= a < value(hi) */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if ((double)oracle_e4m3_to_f32((uint8_t)mid) <= a)
            lo = mid;
        else
            hi = mid;
    }
    double dlo = a - (double)oracle_e4m3_to_f32((uint8_t)lo);
    double dhi = (double)oracle_e4m3_to_f32((uint8_t)hi) - a;
    int best = dlo < dhi ? lo : dhi < dlo ? hi : ((lo & 1) == 0 ? lo : hi);
    return sign | (uint8_t)best;
}

/* E2M1: S.EE.M is (-1)^S * 2^(E-1) * (1 + M/2) for E >= 1 and (-1)^S * M/2
 * for E = 0: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
float oracle_e2m1_to_f32(uint8_t c)
{
    int sign = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
    float v = e == 0 ? 0.5f * (float)m : ldexpf(1.0f + 0.5f * (float)m, e - 1);
    return sign ? -v : v;
}

uint8_t oracle_f32_to_e2m1(float v)
{
    uint8_t sign = signbit(v) ? 8 : 0;
    double a = fabs((double)v);
    if (a >= 6.0)
        return sign | 7;
    int best = 0;
    double bd = a;
    for (int c = 1; c <= 7; ++c) {
        double d = fabs((double)oracle_e2m1_to_f32((uint8_t)c) - a);
        if (d < bd || (d == bd && (c & 1) == 0 && (best & 1) == 1)) {
            bd = d;
            best = c;
        }
    }
    return sign | (uint8_t)best;
}

void oracle_cast_to_e4m3_n(const uint16_t *in, int dtype, uint8_t *out, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = oracle_f32_to_e4m3(widen(in[i], dtype));
}

int oracle_quantize_rows(int64_t n, int H, int dtype, int wire, const uint16_t *in,
                         uint8_t *out, void *scales)
{
    if (wire == ORACLE_WIRE_FP8_BLOCK128) {
        if (H % 128)
            return -1;
        float *sc = scales;
        for (int64_t r = 0; r < n; ++r)
            for (int b = 0; b < H / 128; ++b) {
                const uint16_t *v = in + r * H + b * 128;
                float amax = 0.0f;
                for (int i = 0; i < 128; ++i)
                    amax = fmaxf(amax, fabsf(widen(v[i], dtype)));
                float s = amax > 0.0f ? amax / 448.0f : 1.0f;
                float rcp = amax > 0.0f ? 448.0f / amax : 1.0f;
                sc[r * (H / 128) + b] = s;
                for (int i = 0; i < 128; ++i)
                    out[r * H + b * 128 + i] = oracle_f32_to_e4m3(widen(v[i], dtype) * rcp);
            }
        return 0;
    }
    if (wire == ORACLE_WIRE_MXFP4) {
        if (H % 32)
            return -1;
        uint8_t *sc = scales;
        for (int64_t r = 0; r < n; ++r)
            for (int b = 0; b < H / 32; ++b) {
                const uint16_t *v = in + r * H + b * 32;
                float amax = 0.0f;
                for (int i = 0; i < 32; ++i)
                    amax = fmaxf(amax, fabsf(widen(v[i], dtype)));
                /* the largest E2M1 exponent is 2 (6 = 1.5 * 2^2): the block's
                 * largest magnitude lands in [4, 8) before saturation */
                int E = -127;
                if (amax > 0.0f) {
                    int e2;
                    frexpf(amax, &e2);          /* amax = f * 2^e2, f in [0.5, 1) */
                    E = e2 - 1 - 2;
                    if (E < -127)
                        E = -127;
                }
                sc[r * (H / 32) + b] = (uint8_t)(E + 127);
                for (int i = 0; i < 32; i += 2) {
                    uint8_t lo = oracle_f32_to_e2m1(ldexpf(widen(v[i], dtype), -E));
                    uint8_t hi = oracle_f32_to_e2m1(ldexpf(widen(v[i + 1], dtype), -E));
                    out[r * (H / 2) + (b * 32 + i) / 2] = (uint8_t)(lo | (hi << 4));
                }
            }
        return 0;
    }
    return -1;
}

float oracle_wire_value(int wire, const uint8_t *row, const void *scale_row, int h)
{
    if (wire == ORACLE_WIRE_FP8_BLOCK128)
        return oracle_e4m3_to_f32(row[h]) * ((const float *)scale_row)[h / 128];
    uint8_t byte = row[h / 2];
    uint8_t code = (h & 1) ? (byte >> 4) : (byte & 0xF);
    return ldexpf(oracle_e2m1_to_f32(code), (int)((const uint8_t *)scale_row)[h / 32] - 127);
}

int oracle_combine_wire(int W, int M, int k, int H, int dtype, int wire, const int32_t *ntok,
                        const int32_t *fwd, const uint8_t *y, const void *y_scales,
                        uint16_t *out)
{
    const int P = W < k ? W : k;
    size_t row_bytes, scale_bytes;
    if (wire == ORACLE_WIRE_FP8_BLOCK128) {
        row_bytes = (size_t)H;
        scale_bytes = sizeof(float) * (size_t)(H / 128);
    } else if (wire == ORACLE_WIRE_MXFP4) {
        row_bytes = (size_t)H / 2;
        scale_bytes = (size_t)(H / 32);
    } else {
        return -1;
    }
    for (int r = 0; r < W; ++r)
        for (int t = 0; t < ntok[r]; ++t) {
            int64_t tok = (int64_t)r * M + t;
            int64_t rows[64];
            int n = 0;
            for (int i = 0; i < P; ++i)
                if (fwd[tok * P + i] >= 0)
                    rows[n++] = fwd[tok * P + i];
            /* [PR712] Combine: FP32 sum in the token's rank order from the
             * first contribution, one rounding; each contribution comes off
             * the wire through its scale first */
            for (int h = 0; h < H; ++h) {
                float acc = 0.0f;
                for (int i = 0; i < n; ++i) {
                    float v = oracle_wire_value(wire, y + (size_t)rows[i] * row_bytes,
                                                (const uint8_t *)y_scales
                                                    + (size_t)rows[i] * scale_bytes, h);
                    acc = i == 0 ? v : acc + v;
                }
                out[(size_t)tok * H + h] = n ? narrow(acc, dtype) : 0;
            }
        }
    return 0;
}

struct packed_wire {
    const uint8_t *codes;   /* [rows][row_bytes] wire rows */
    const uint8_t *scales;  /* [rows][scale_bytes] their scales */
    size_t row_bytes, scale_bytes;
    int wire;
};

static float packed_wire_value(const void *src, int64_t row, int H, int h)
{
    const struct packed_wire *s = src;
    (void)H;
    return oracle_wire_value(s->wire, s->codes + (size_t)row * s->row_bytes,
                             s->scales + (size_t)row * s->scale_bytes, h);
}

int oracle_expert_combine_wire(int W, int M, int k, int Er, int cap, int H, int dtype, int wire,
                               const int32_t *recv, const int32_t *idx, const float *w,
                               const uint8_t *py, const void *py_scales, uint16_t *y)
{
    struct packed_wire src = {py, (const uint8_t *)py_scales, 0, 0, wire};
    if (wire == ORACLE_WIRE_FP8_BLOCK128) {
        src.row_bytes = (size_t)H;
        src.scale_bytes = sizeof(float) * (size_t)(H / 128);
    } else if (wire == ORACLE_WIRE_MXFP4) {
        src.row_bytes = (size_t)H / 2;
        src.scale_bytes = (size_t)(H / 32);
    } else {
        return -1;
    }
    return expert_combine(W, M, k, Er, cap, H, dtype, recv, idx, w, packed_wire_value, &src, y);
}
