/*
 * loom.h -- C ABI of the MI355X (gfx950, CDNA4) streaming-reduction library.
 *
 * The library computes the data-parallel hot path described by the Loom pages
 * "Tune loop unrolling and pipelining" (TUNE), "Functions and structured
 * control flow" (CTRL) and "Kernels and launch configuration" (LAUNCH): a
 * streaming reduction over records in memory -- row-tiled f32 sums with a
 * subgroup (wave64) reduction per row, full 8-row tiles with a separate ragged
 * tail, read-ahead of the next records -- and its extension to packed
 * signed-byte (int8) dequantization with dot accumulation.
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - Return LOOM_OK (0) or a negative loom_status.  All argument checks run on
 *    the host before anything is enqueued; on error nothing is launched and no
 *    output is touched.  Sizes and counts are checked first (LOOM_ERR_RANGE,
 *    LOOM_ERR_SHAPE), including the launch grid's limit of fewer than 2^32
 *    work-items (see each call); a call with nothing to do (no rows,
 *    elements, segments, outputs or tokens) then returns LOOM_OK without
 *    looking at its pointers;
 *    otherwise required pointers (LOOM_ERR_NULL) and then alignment
 *    (LOOM_ERR_ALIGN) are checked.
 *  - Data pointers are device pointers (HIP allocations of the current device,
 *    e.g. a torch tensor's data_ptr()).  The caller owns all memory.  The
 *    library keeps no pointer after returning and allocates no device memory,
 *    except loom_segment_sums in its split and longest-first launches, whose
 *    workspace comes from HIP's stream-ordered allocator (see there;
 *    loom_segment_sums_noalloc never allocates).
 *  - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *    asynchronously on it; outputs are ready once the stream has reached the
 *    enqueued work.  A device-side fault is reported by later HIP calls, not
 *    by the return code; LOOM_ERR_DEVICE means the launch itself was refused
 *    (the thread's last HIP error is cleared before each launch, so an error
 *    left by an earlier, unrelated HIP call is never reported as this one).
 *  - Calls are thread-safe: the shared state is an immutable table and, for
 *    loom_segment_sums_noalloc, a lock-guarded per-device address cache and
 *    the static device array (calls of it that overlap on one GPU race; see
 *    there).
 *  - Matrices are row-major.  Packed int8: an int32 word j of a row holds the
 *    elements 4j..4j+3, element 4j+b in byte b (little-endian), two's
 *    complement -- exactly the bytes of an int8 array viewed as int32.
 */
#ifndef LOOM_H
#define LOOM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum loom_status {
    LOOM_OK = 0,
    LOOM_ERR_NULL = -1,           /* a required pointer is NULL                          */
    LOOM_ERR_RANGE = -2,          /* a size or count outside its documented range        */
    LOOM_ERR_ALIGN = -3,          /* a pointer or stride not aligned as documented       */
    LOOM_ERR_SHAPE = -4,          /* inconsistent shape (e.g. k not a multiple of 4)     */
    LOOM_ERR_UNKNOWN_EXPORT = -5, /* no kernel exports this name                         */
    LOOM_ERR_TOKEN = -6,          /* invalid launch-config token or workload arity       */
    LOOM_ERR_DEVICE = -7          /* the HIP runtime refused the launch                  */
} loom_status;

/* Static, human-readable text for a status code (never NULL). */
const char *loom_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int loom_version(void);

/* ------------------------------------------------------------------------ *
 * Launch configuration (LAUNCH §A kernel owns two signatures, §Workload is  *
 * not workgroup count, §Evaluate the compiled launch contract).             *
 *                                                                           *
 * Each kernel owns the mapping from its logical workload (element, row or   *
 * segment counts) to a physical grid.  An embedding resolves an export name  *
 * to a token once, then evaluates the geometry for any workload without     *
 * compiling anything.  The entry points below use the same evaluation, so   *
 * the host never duplicates the grid arithmetic.                            *
 * ------------------------------------------------------------------------ */
typedef struct loom_launch_config {
    uint32_t workgroups[3];          /* grid, in workgroups                       */
    uint32_t workgroup_size[3];      /* work-items per workgroup                  */
    uint32_t cluster_size[3];        /* always {1,1,1}: gfx950 has no clusters    */
    uint32_t subgroup_size;          /* 64: gfx950 waves are 64 wide              */
    uint32_t workgroup_storage_bytes;/* LDS the kernel needs per workgroup        */
} loom_launch_config;

/* Export names and their workload signatures (each an int64 passed as its
 * uint64 bit pattern):
 *   "copy_f32"        (n)
 *   "row_sum_tiles"   (count)
 *   "row_sums"        (rows, cols)
 *   "segment_sums"    (segments, cols, total_rows)
 *   "i8_dequant_dot"  (rows, k, batch)
 *   "packed_dot"      (outputs, count, streams)
 *   "sum_guarded_rows" (count)
 *   "routed_combine"  (tokens, routes, hidden)
 * lookup: LOOM_ERR_NULL if a pointer is NULL, LOOM_ERR_UNKNOWN_EXPORT if no
 * kernel has that name.  The token stays valid for the life of the process. */
int loom_launch_config_lookup(const char *export_name, uint32_t *token);

/* Evaluates the launch configuration of `token` for the given workload.
 * Pure host arithmetic; no device call.  LOOM_ERR_TOKEN for an unknown token
 * or a workload_count that differs from the export's arity, LOOM_ERR_RANGE
 * for a negative workload value or a grid beyond the hardware limits.
 * A workload with nothing to do yields workgroups {0,1,1}. */
int loom_launch_config_invoke(uint32_t token, const uint64_t *workload_bits,
                              size_t workload_count, loom_launch_config *out);

/* ------------------------------------------------------------------------ *
 * Guarded over-dispatched copy (LAUNCH §Over-dispatch safely and preserve   *
 * the proof).  out[i] = in[i] for 0 <= i < n, on ceil(n/256) workgroups of   *
 * 256 work-items; work-items at or beyond n touch nothing, so out[n..] is   *
 * left as it was (1009 elements run on 4 workgroups).                       *
 *   in, out : f32[n], device, 4-byte aligned; may be NULL only when n == 0  *
 *   n       : 0 <= n <= 2^32 - 256, so the grid stays below 2^32           *
 *             work-items (LOOM_ERR_RANGE otherwise)                         *
 * ------------------------------------------------------------------------ */
int loom_copy_f32(const float *in, float *out, int64_t n, void *stream);

/* ------------------------------------------------------------------------ *
 * Tiled row sum of one 32-lane tile (TUNE §Derive full tiles from a ragged  *
 * loop, @guide.sum_full_tiles).  For lane l < 32:                           *
 *     sums[l] = initial[l] + sum over rows r < final_row of rowsum(r)       *
 * where rowsum(r) is the subgroup reduction of values[r][0..31], rows are   *
 * taken in full tiles of 8 in row order, final_row = 8*floor(count/8) and   *
 * tail_count = count mod 8.  The tail rows [final_row, count) are NOT       *
 * summed and NOT read: they are returned for a separate cleanup.            *
 *   values     : f32[rows_alloc][32], device, 4-byte aligned                *
 *   rows_alloc : rows allocated, 0 <= rows_alloc <= 2^26                    *
 *   count      : logical row count, 0 <= count <= rows_alloc (the page's    *
 *                inclusive range assumption, checked: LOOM_ERR_RANGE)       *
 *   initial    : f32[32] per-lane start value, or NULL for 0.0              *
 *   sums       : f32[32] output                                             *
 *   final_row, tail_count : int32[1] outputs, device                        *
 * ------------------------------------------------------------------------ */
int loom_row_sum_tiles(const float *values, int64_t rows_alloc, int64_t count,
                       const float *initial, float *sums, int32_t *final_row,
                       int32_t *tail_count, void *stream);

/* ------------------------------------------------------------------------ *
 * Streaming row sums (TUNE §Derive full tiles, §Give each motif its own     *
 * schedule, §Read-ahead; CTRL §Pipeline reads ahead of ordered computation) *
 *     out[r] = sum_{c < cols} x[r*row_stride + c],   0 <= r < rows          *
 * Every row is streamed with coalesced loads read ahead of the              *
 * accumulation and finished by cross-lane reductions; how rows map to the   *
 * GPU depends on their width: 1-128 floats are packed several to a 64-lane  *
 * record; 129-768 floats run in full 8-row tiles plus one guarded tail      *
 * tile; a row of 769 floats or more gets a workgroup of its own whose wave  *
 * totals are added in wave order.  f32 accumulation; the summation          *
 * order inside a row is a fixed tree, the same on every call (error         *
 * <= 1e-5 * sum|x| for the documented sizes).                               *
 *   x          : f32, device, 4-byte aligned (16-byte alignment of x and    *
 *                row_stride % 4 == 0 select 128-bit loads)                  *
 *   rows, cols : 0 <= rows < 2^31, 0 <= cols < 2^31; LOOM_ERR_RANGE also    *
 *                when the grid would reach 2^32 work-items, as              *
 *                loom_launch_config_invoke reports for (rows, cols): only   *
 *                past 2^30 - 16 rows of at most 768 floats                  *
 *   row_stride : elements between row starts, row_stride >= cols            *
 *                (LOOM_ERR_SHAPE); 4 * rows * row_stride must fit in an     *
 *                int64 (LOOM_ERR_RANGE)                                     *
 *   out        : f32[rows], device                                          *
 * ------------------------------------------------------------------------ */
int loom_row_sums(const float *x, int64_t rows, int64_t cols, int64_t row_stride,
                  float *out, void *stream);

/* ------------------------------------------------------------------------ *
 * Per-segment column sums (TUNE §Keep one checked source for experiments:   *
 * each lane sums its column over the rows, in row order; §Derive full       *
 * tiles: full 8-row tiles then the tail).                                   *
 *     out[s][c] = sum_{offsets[s] <= r < offsets[s+1]} x[r][c]              *
 *     tail_counts[s] = (offsets[s+1] - offsets[s]) mod 8                    *
 * Each column accumulates its rows in row order in f32, so every output is  *
 * the in-order recurrence bit for bit (an empty segment gives +0.0) --      *
 * except for a few long segments: when segments x ceil(cols / 256) < 192    *
 * and the segments average at least 1024 rows (total_rows / segments), each *
 * segment is split into P contiguous parts of at least 512 rows on average  *
 * (P * segments * ceil(cols / 256) <= 4096), each part summed in row order, *
 * and the part sums added in a fixed order.  With cols <= 512 and P >= 16,  *
 * P is a multiple of 8 and the sums of each run of 8 consecutive parts are  *
 * added in part order, leaving n = P / 8 partials per segment; otherwise    *
 * the n = P part sums are the partials.  The n partials are added as        *
 * contiguous groups of ceil(n / 16) in order, then the group sums in group  *
 * order: the same bits on every call, within 1e-5 * sum|x| of the in-order  *
 * sum.  The partials (4 * segments * n * cols bytes, at most 4 MiB) are     *
 * taken from HIP's stream-ordered allocator on `stream` (hipMallocAsync /   *
 * hipFreeAsync).  A launch that is not split, of 2 to 2^15 segments         *
 * averaging at least 512 rows and of at least 2^26 floats, first sorts the  *
 * segments by length (a one-workgroup pass) so its waves take them longest  *
 * first; the order index (4 * segments bytes) is taken the same way.  These *
 * are the only cases where a call allocates device memory; neither changes  *
 * a bit of output.                                                          *
 *   x           : f32[total_rows][cols], device, row-major, 4-byte aligned  *
 *   total_rows  : rows in x, 0 <= total_rows <= 2^40                        *
 *   offsets     : int64[segments+1], device, CSR row offsets.  A segment    *
 *                 with offsets[s] > offsets[s+1], offsets[s] < 0 or         *
 *                 offsets[s+1] > total_rows reads nothing; its outputs are  *
 *                 set to NaN and its tail count to -1.                      *
 *   segments    : 0 <= segments < 2^31 - 1                                  *
 *   cols        : 0 <= cols <= 2^20                                         *
 *   out         : f32[segments][cols], device                               *
 *   tail_counts : int32[segments], device, or NULL                          *
 * LOOM_ERR_DEVICE also when the stream-ordered allocation fails.            *
 * ------------------------------------------------------------------------ */
int loom_segment_sums(const float *x, int64_t total_rows, const int64_t *offsets,
                      int64_t segments, int64_t cols, float *out,
                      int32_t *tail_counts, void *stream);

/* ------------------------------------------------------------------------ *
 * For callers that cannot allocate device memory -- code under HIP graph    *
 * capture, tight serving loops, harnesses that forbid hipMalloc: the same   *
 * operation, arguments, checks and results (the same bits) as              *
 * loom_segment_sums, but a split launch's partials and a longest-first     *
 * launch's order index live in the library's own static device array of    *
 * 4 MiB (one per GPU the library runs on, kept until the process ends)      *
 * instead of stream-ordered memory, so no call allocates.  Every call on a  *
 * GPU shares that GPU's array and it keeps the last call's contents (each   *
 * launch writes every word of it that it reads):                            *
 * calls that may overlap on one GPU -- on different streams or threads --   *
 * race and must be ordered by the caller.  LOOM_ERR_RANGE if a split would  *
 * need more than the array holds (the split rule keeps every launch within  *
 * it).                                                                      *
 * ------------------------------------------------------------------------ */
int loom_segment_sums_noalloc(const float *x, int64_t total_rows, const int64_t *offsets,
                              int64_t segments, int64_t cols, float *out,
                              int32_t *tail_counts, void *stream);

/* ------------------------------------------------------------------------ *
 * Packed signed-byte dequantization with dot accumulation (TUNE §Apply the  *
 * same controls to a packed dot product; scales factored out of the sum).   *
 *     acc[r][b] = sum_{i < k} w[r][i] * x[b][i]          (exact, int32)     *
 *     out[r][b] = (f32(acc[r][b]) * w_scale[r]) * x_scale[b]                *
 * with each product rounded once to f32; when x_scale is NULL the second    *
 * product is skipped.  One vector runs a v_dot4 (int8x4) GEMV: rows of up  *
 * to 512 bytes packed several to a 1 KiB record, most rows of 3 to 12 KiB   *
 * a workgroup per row, other rows a wave per block of rows.  Several        *
 * vectors run an int8 MFMA kernel.  The results are the same bits either    *
 * way.                                                                      *
 *   w       : int32[rows][k/4] packed int8 weights, device, 4-byte aligned  *
 *   w_scale : f32[rows], device                                             *
 *   x       : int32[batch][k/4] packed int8 activations, device             *
 *   x_scale : f32[batch], device, or NULL (= 1)                             *
 *   rows    : 0 <= rows < 2^31; LOOM_ERR_RANGE also when the grid would     *
 *             reach 2^32 work-items, as loom_launch_config_invoke reports   *
 *             for (rows, k, batch): only at 2^26 rows or more               *
 *   k       : elements per row, k % 4 == 0 (LOOM_ERR_SHAPE), 0 <= k <=      *
 *             131068 so |acc| <= 2^31 - 1 (LOOM_ERR_RANGE)                  *
 *   batch   : 1 <= batch <= 64 (LOOM_ERR_RANGE)                             *
 *   out     : f32[rows][batch], device                                      *
 *   acc     : int32[rows][batch], device, or NULL (not written)             *
 * ------------------------------------------------------------------------ */
int loom_i8_dequant_dot(const int32_t *w, const float *w_scale, const int32_t *x,
                        const float *x_scale, int64_t rows, int64_t k, int64_t batch,
                        float *out, int32_t *acc, void *stream);

/* ------------------------------------------------------------------------ *
 * The pages' literal packed signed-byte dot recurrence (TUNE §Apply the     *
 * same controls to a packed dot product).  For every output o, starting     *
 * from initial[o] (0 if NULL), every record r < count, in record order:     *
 *     v_j = f32(signed byte j of fields[r][o]) * f32(scales[r][o])          *
 *     sum = sum + v_j * rhs[r][o mod streams][j]     for j = 0, 1, 2, 3     *
 * each product and sum a separate f32 rounding (no fused multiply-add), so  *
 * the result is the serial recurrence bit for bit.                          *
 *   fields  : int32[records][outputs], record-major (consecutive outputs    *
 *             contiguous), 4-byte aligned                                   *
 *   scales  : binary16 bit patterns [records][outputs], 2-byte aligned      *
 *   rhs     : f32[records][streams][4] activations, 16-byte aligned; the    *
 *             streams are shared by all outputs (output o reads o mod       *
 *             streams)                                                      *
 *   streams : 1 <= streams < 2^31                                           *
 *   initial : f32[outputs] or NULL                                          *
 *   records : records allocated; 0 <= count <= records, count < 2^31, and   *
 *             4 * records * outputs fits in an int64 (LOOM_ERR_RANGE)     *
 *   outputs : 0 <= outputs <= 255 * (2^31 - 1); LOOM_ERR_RANGE also when    *
 *             the grid would reach 2^32 work-items, as                      *
 *             loom_launch_config_invoke reports for (outputs, count,        *
 *             streams): past 2^32 - 256 outputs, or 2^34 - 1024 when        *
 *             streams divides 64                                            *
 *   out     : f32[outputs]                                                  *
 * ------------------------------------------------------------------------ */
int loom_packed_dot(const int32_t *fields, const uint16_t *scales, const float *rhs, int64_t streams,
                    const float *initial, int64_t records, int64_t count, int64_t outputs, float *out,
                    void *stream);

/* ------------------------------------------------------------------------ *
 * The pages' guarded ragged row sum (TUNE §Keep guards and inner loops in   *
 * the source, @guide.sum_guarded_rows).  For each lane l < 32, rows are      *
 * walked in order up to count rounded up to a multiple of 4; a row at or    *
 * beyond count contributes 0 and is not read; otherwise its partial is the  *
 * in-order f32 sum, from 0, of values[row][l][c] for c < columns, each      *
 * taken as 0 (and not read) when l >= active_lanes.  sums[l] is the in-order *
 * f32 sum of the partials, from 0 -- the serial recurrence bit for bit.     *
 *   values       : f32[rows_alloc][32][4], 16-byte aligned                  *
 *   rows_alloc   : 0 <= rows_alloc <= 2^26                                  *
 *   count        : 0 <= count <= rows_alloc (the padded row need not exist) *
 *   columns      : 0 <= columns <= 4                                        *
 *   active_lanes : 0 <= active_lanes <= 32                                  *
 *   sums         : f32[32]                                                  *
 * ------------------------------------------------------------------------ */
int loom_sum_guarded_rows(const float *values, int64_t rows_alloc, int64_t count, int64_t columns,
                          int64_t active_lanes, float *sums, void *stream);

/* ------------------------------------------------------------------------ *
 * Routed row combine (TUNE §Separate route and payload lookahead: a routed  *
 * MoE combine).  For token t and column c, routes i < routes in order:      *
 *     id = ids[t][i]; if (uint32)id < num_rows:                             *
 *         acc[c] = acc[c] + weights[t][i] * payload[id][c]                  *
 * (product rounded, then added; acc starts at 0); out[t][c] = acc[c].  A   *
 * route whose id is outside [0, num_rows) is missing: neither its weight    *
 * nor its payload row is read.                                              *
 *   ids     : int32[tokens][routes]                                         *
 *   weights : f32[tokens][routes]                                           *
 *   payload : f32[num_rows][hidden] expert-output rows, 16-byte aligned     *
 *   num_rows: 0 <= num_rows < 2^31                                          *
 *   tokens  : 0 <= tokens < 2^31; routes, hidden: 0 .. 2^20                 *
 *   hidden  : a multiple of 4 (LOOM_ERR_SHAPE otherwise)                    *
 *   out     : f32[tokens][hidden], 16-byte aligned                          *
 * ------------------------------------------------------------------------ */
int loom_routed_combine(const int32_t *ids, const float *weights, const float *payload, int64_t num_rows,
                        int64_t tokens, int64_t routes, int64_t hidden, float *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LOOM_H */
