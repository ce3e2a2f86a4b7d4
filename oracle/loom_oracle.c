/*
 * loom_oracle.c -- plain, slow CPU oracle for the streaming-reduction hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this library.  The product
 * path (the HIP library and its Python binding) never uses it, and the two
 * share no code, headers, tables or helpers.
 *
 * Every function follows the pages' statement of the computation in source
 * order, one record at a time, with no blocking, fusion or reordering.  It is
 * built with -O2 -fno-fast-math -ffp-contract=off so each float operation is a
 * single IEEE binary32 (or binary64 for the shadow sums) round-to-nearest step.
 *
 * Pages cited ("Loom" documentation):
 *   [TUNE]   "Tune loop unrolling and pipelining"
 *   [CTRL]   "Functions and structured control flow"
 *   [LAUNCH] "Kernels and launch configuration"
 *
 * Readings the pages leave open (each also listed in the design notes):
 *   - order inside a subgroup or vector reduction is unspecified; the oracle
 *     adds lanes / columns in ascending order;
 *   - the int8 dot uses an exact integer accumulate followed by the float
 *     scale, (f32(acc) * w_scale[r]) * x_scale[b], each product rounded once.
 *
 * Every function here is pinned by CPU tests against closed forms, values
 * printed on the pages, exact integer arithmetic or proven error bounds.
 */
#include <stdint.h>
#include <stddef.h>
#include <math.h>
#include <string.h>

/* [TUNE] §Derive full tiles from a ragged loop: the repeated scf.while walks
 * full tiles while at least `tile` records remain and returns the first row
 * after the last full tile together with the remaining (tail) count. */
void oracle_tile_split(int64_t count, int64_t tile, int64_t *final_row, int64_t *tail_count)
{
    int64_t row = 0;
    int64_t remaining = count;
    while (remaining >= tile) {
        row = row + tile;
        remaining = remaining - tile;
    }
    *final_row = row;
    *tail_count = remaining;
}

/* [LAUNCH] §A kernel owns two signatures / §Workload is not workgroup count:
 * the @fill launch configuration rounds the element count up to whole
 * workgroups of 256 work-items. */
int64_t oracle_fill_workgroups(int64_t element_count, int64_t workgroup_size)
{
    int64_t rounded = element_count + (workgroup_size - 1);
    return rounded / workgroup_size;
}

/* [LAUNCH] §Over-dispatch safely: every in-bounds element index copies one
 * value; indices at or beyond the element count touch nothing. */
void oracle_copy_f32(const float *in, float *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = in[i];
}

/* [TUNE] §Derive full tiles from a ragged loop (@guide.sum_full_tiles):
 * values is a [rows_alloc][32] row-major f32 tile, count the logical row
 * count.  Each lane's carried sum starts at initial[lane]; for every row of
 * every full 8-row tile, in row order, the subgroup reduction of that row
 * (the sum of its 32 lane values, here in ascending lane order) is added to
 * the carried sum.  Rows at or after final_row (the tail) are not read. */
void oracle_row_sum_tiles(const float *values, int64_t count, const float *initial,
                          float *sums, int64_t *final_row, int64_t *tail_count)
{
    const int64_t lanes = 32, tile = 8;
    for (int64_t lane = 0; lane < lanes; ++lane) {
        float sum = initial ? initial[lane] : 0.0f;
        int64_t row = 0, remaining = count;
        while (remaining >= tile) {
            for (int64_t tile_row = 0; tile_row < tile; ++tile_row) {
                int64_t source_row = row + tile_row;
                float row_sum = 0.0f;
                for (int64_t l = 0; l < lanes; ++l)
                    row_sum = row_sum + values[source_row * lanes + l];
                sum = sum + row_sum;
            }
            row = row + tile;
            remaining = remaining - tile;
        }
        sums[lane] = sum;
        *final_row = row;
        *tail_count = remaining;
    }
}

/* Row sums of a strided f32 matrix: rows are visited in full 8-row tiles and
 * then the ragged tail ([TUNE] §Derive full tiles; the tail is summed here, as
 * the separate cleanup the same section describes), and each row is reduced
 * over its columns in ascending order in f32 ([TUNE] §Give each motif its own
 * schedule: a row's values are loaded and reduced into one float).
 * Optional shadows: out_f64 = the same sum in binary64, out_abs = sum |x|. */
static void row_sum_one(const float *row, int64_t cols, float *out, double *out_f64, double *out_abs)
{
    float s = 0.0f;
    double d = 0.0, a = 0.0;
    for (int64_t c = 0; c < cols; ++c) {
        s = s + row[c];
        if (out_f64) d = d + (double)row[c];
        if (out_abs) a = a + fabs((double)row[c]);
    }
    *out = s;
    if (out_f64) *out_f64 = d;
    if (out_abs) *out_abs = a;
}

void oracle_row_sums(const float *x, int64_t rows, int64_t cols, int64_t row_stride,
                     float *out, double *out_f64, double *out_abs)
{
    int64_t final_row, tail_count;
    oracle_tile_split(rows, 8, &final_row, &tail_count);
    for (int64_t r = 0; r < final_row; ++r)          /* full tiles, in order */
        row_sum_one(x + r * row_stride, cols, &out[r],
                    out_f64 ? &out_f64[r] : NULL, out_abs ? &out_abs[r] : NULL);
    for (int64_t t = 0; t < tail_count; ++t) {        /* ragged tail */
        int64_t r = final_row + t;
        row_sum_one(x + r * row_stride, cols, &out[r],
                    out_f64 ? &out_f64[r] : NULL, out_abs ? &out_abs[r] : NULL);
    }
}

/* Per-segment column sums: segment s owns rows [offsets[s], offsets[s+1]) of
 * a [*][cols] row-major f32 matrix.  As in the per-lane column sum of
 * [TUNE] §Keep one checked source for experiments (@sum_rows: each lane adds
 * one column over the rows, in row order, one load and one add per row),
 * every column accumulates its rows in source order (the full 8-row tiles
 * and then the tail rows are consecutive, so this is one in-order walk over
 * the segment).  An empty segment yields the initial value +0.0
 * ([CTRL] §Counted loops carry state explicitly).  tail_counts[s] is the
 * segment's tail length from the tile split. */
void oracle_segment_sums(const float *x, const int64_t *offsets, int64_t segments, int64_t cols,
                         float *out, int32_t *tail_counts, double *out_f64, double *out_abs)
{
    for (int64_t s = 0; s < segments; ++s) {
        int64_t begin = offsets[s];
        int64_t length = offsets[s + 1] - offsets[s];
        int64_t final_row, tail_count;
        oracle_tile_split(length, 8, &final_row, &tail_count);
        if (tail_counts) tail_counts[s] = (int32_t)tail_count;
        for (int64_t c = 0; c < cols; ++c) {
            float acc = 0.0f;
            double d = 0.0, a = 0.0;
            for (int64_t r = 0; r < final_row + tail_count; ++r) {  /* = length rows */
                float v = x[(begin + r) * cols + c];
                acc = acc + v;
                d = d + (double)v;
                a = a + fabs((double)v);
            }
            out[s * cols + c] = acc;
            if (out_f64) out_f64[s * cols + c] = d;
            if (out_abs) out_abs[s * cols + c] = a;
        }
    }
}

/* Packed signed-byte dequantization with dot accumulation ([TUNE] §Apply the
 * same controls to a packed dot product: four signed bytes per 32-bit word,
 * unpacked by sign extension, accumulated in record order).  Here the
 * weights are w[rows][k] and the activations x[batch][k], both int8, and the
 * scales are factored out of the sum so it is exact:
 *     acc[r][b] = sum_k w[r][k] * x[b][k]            (exact, 64-bit, then
 *                                                      checked to fit int32)
 *     out[r][b] = (f32(acc[r][b]) * w_scale[r]) * x_scale[b]
 * (the second product is skipped when x_scale is NULL).  The int8 matrices are
 * the byte views of the packed int32 words: byte j of word i is element 4i+j.
 * Returns 0, or -1 if some accumulator does not fit in int32. */
int oracle_i8_dequant_dot(const int8_t *w, const float *w_scale, const int8_t *x, const float *x_scale,
                          int64_t rows, int64_t k, int64_t batch, float *out, int32_t *acc)
{
    int status = 0;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < batch; ++b) {
            int64_t total = 0;
            for (int64_t i = 0; i < k; ++i)
                total = total + (int64_t)w[r * k + i] * (int64_t)x[b * k + i];
            if (total > INT32_MAX || total < INT32_MIN) status = -1;
            int32_t a32 = (int32_t)total;
            if (acc) acc[r * batch + b] = a32;
            float y = (float)a32;
            y = y * w_scale[r];
            if (x_scale) y = y * x_scale[b];
            out[r * batch + b] = y;
        }
    }
    return status;
}

/* IEEE 754 binary16 -> binary32 (exact): sign, 5-bit exponent with bias 15,
 * 10-bit fraction; exponent 0 encodes zero and subnormals (fraction * 2^-24),
 * exponent 31 encodes infinities and NaNs (fraction kept in the top bits). */
float oracle_f16_to_f32(uint16_t h)
{
    uint32_t sign = (uint32_t)(h >> 15) << 31;
    uint32_t exponent = (h >> 10) & 0x1F;
    uint32_t fraction = h & 0x3FF;
    uint32_t bits;
    if (exponent == 0x1F) {
        bits = sign | 0x7F800000u | (fraction << 13);
    } else if (exponent != 0) {
        bits = sign | ((exponent - 15 + 127) << 23) | (fraction << 13);
    } else {
        float magnitude = (float)fraction * 0x1p-24f;   /* exact: fraction < 2^10 */
        float value = sign ? -magnitude : magnitude;
        return value;
    }
    float out;
    memcpy(&out, &bits, sizeof out);
    return out;
}

/* [TUNE] §Apply the same controls to a packed dot product
 * (@streaming_packed_s8_dot_read_ahead).  For every output o, starting from
 * initial[o] (0 if NULL), each record r < count in order contributes
 *     v_j = f32(sign-extended byte j of fields[r][o]) * f32(scales[r][o]),  j = 0..3
 *     sum = sum + v_j * rhs[r][o mod streams][j]   for j = 0, 1, 2, 3 in order
 * (the dot accumulates into the carried sum one product at a time; every
 * product and sum is a separate f32 rounding).  fields and scales are
 * record-major: [records][outputs]; scales are binary16 bit patterns; rhs is
 * [records][streams][4] f32, the activation streams shared by the outputs. */
void oracle_packed_dot(const int32_t *fields, const uint16_t *scales, const float *rhs, int64_t streams,
                       const float *initial, int64_t count, int64_t outputs, float *out,
                       double *out_f64, double *out_abs)
{
    for (int64_t o = 0; o < outputs; ++o) {
        float sum = initial ? initial[o] : 0.0f;
        double d = sum, a = fabs((double)sum);
        int64_t stream = o % streams;
        for (int64_t r = 0; r < count; ++r) {
            uint32_t word = (uint32_t)fields[r * outputs + o];
            float scale = oracle_f16_to_f32(scales[r * outputs + o]);
            const float *act = rhs + (r * streams + stream) * 4;
            for (int j = 0; j < 4; ++j) {
                int8_t byte = (int8_t)(uint8_t)(word >> (8 * j));
                float v = (float)byte * scale;
                float p = v * act[j];
                sum = sum + p;
                d = d + (double)byte * (double)scale * (double)act[j];
                a = a + fabs((double)byte * (double)scale * (double)act[j]);
            }
        }
        out[o] = sum;
        if (out_f64) out_f64[o] = d;
        if (out_abs) out_abs[o] = a;
    }
}

/* [TUNE] §Keep guards and inner loops in the source (@guide.sum_guarded_rows).
 * values is a [rows_alloc][32][4] f32 tile.  The row range is rounded up to a
 * multiple of 4; for every row of that padded range, in order, a lane's
 * partial is 0 for rows at or beyond count (those rows, including the padded
 * one, are never read); otherwise it is the inner sum, from 0, over the first
 * `columns` components of values[row][lane][*] in order, each component 0
 * for lanes at or beyond active_lanes (whose values are never read).  The
 * partial is added to the lane's carried sum, which starts at 0. */
void oracle_sum_guarded_rows(const float *values, int64_t count, int64_t columns, int64_t active_lanes,
                             float *sums)
{
    const int64_t lanes = 32, tile_width = 4;
    int64_t padded = count + (tile_width - 1);
    int64_t end = (padded / tile_width) * tile_width;
    for (int64_t lane = 0; lane < lanes; ++lane) {
        float sum = 0.0f;
        int active = lane < active_lanes;
        for (int64_t row = 0; row < end; ++row) {
            float partial = 0.0f;
            if (row < count) {
                float component_sum = 0.0f;
                for (int64_t column = 0; column < columns; ++column) {
                    float value = 0.0f;
                    if (active) value = values[(row * lanes + lane) * 4 + column];
                    component_sum = component_sum + value;
                }
                partial = component_sum;
            }
            sum = sum + partial;
        }
        sums[lane] = sum;
    }
}

/* [TUNE] §Separate route and payload lookahead (the routed MoE combine): for
 * token t, each route i < routes in order carries a row id and a weight.  A
 * route whose id lies outside [0, num_rows) -- compared as unsigned, so
 * negative ids are outside -- is missing: neither its weight nor its payload
 * row is read and the sum is unchanged.  Otherwise, for every column c,
 *     acc[c] = acc[c] + weights[t][i] * payload[id][c]
 * (the product rounded, then the sum), starting from 0; out[t][c] = acc[c]. */
void oracle_routed_combine(const int32_t *ids, const float *weights, const float *payload, int64_t num_rows,
                           int64_t tokens, int64_t routes, int64_t hidden, float *out, double *out_f64,
                           double *out_abs)
{
    for (int64_t t = 0; t < tokens; ++t) {
        for (int64_t c = 0; c < hidden; ++c) {
            float acc = 0.0f;
            double d = 0.0, a = 0.0;
            for (int64_t i = 0; i < routes; ++i) {
                uint32_t id = (uint32_t)ids[t * routes + i];
                if ((uint64_t)id >= (uint64_t)num_rows) continue;
                float w = weights[t * routes + i];
                float p = payload[(int64_t)id * hidden + c];
                float product = w * p;
                acc = acc + product;
                d = d + (double)w * (double)p;
                a = a + fabs((double)w * (double)p);
            }
            out[t * hidden + c] = acc;
            if (out_f64) out_f64[t * hidden + c] = d;
            if (out_abs) out_abs[t * hidden + c] = a;
        }
    }
}
