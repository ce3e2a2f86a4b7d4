// i8_dot.hip -- packed signed-byte dequantization with dot accumulation on gfx950.
//
// TUNE = "Tune loop unrolling and pipelining" (Loom pages),
// §Apply the same controls to a packed dot product: each record carries
// packed signed bytes that are unpacked by sign extension and accumulated in
// order.  Here the scales are factored out of the sum, so the accumulation is
// exact int32 and order-free, and the dequantization is one epilogue per
// output: out = (f32(acc) * w_scale[r]) * x_scale[b].
//
// Packed layout: int32 word j of a row holds elements 4j..4j+3 in bytes 0..3.
// Both kernels consume whole 16-byte groups (4 words = 16 int8) per lane and
// never unpack explicitly: v_dot4_i32_i8 and the int8 MFMA sign-extend the
// bytes themselves.
#include "device_common.hpp"
#include "internal.hpp"

namespace loom {

// Schedules (records in flight, record size, load policy).  Each kernel
// instantiation owns its schedule; the macros let a tuning build override it.
#ifndef LOOM_GEMV_DEPTH
#define LOOM_GEMV_DEPTH 6        // five 1 KiB weight blocks in flight per wave
#endif
#ifndef LOOM_MFMA_DEPTH
#define LOOM_MFMA_DEPTH 3        // two 4 KiB records in flight per wave
#endif
#ifndef LOOM_MFMA_SEG_DEPTH
// one 4 KiB record in flight per wave: 8 vectors at k = 8192 measured the same
// as depths 3 and 4 (35.5 / 35.5 / 35.3 us), at k = 16384 39.2 against 42.1 / 42.2
#define LOOM_MFMA_SEG_DEPTH 2
#endif
#ifndef LOOM_MFMA_STREAM
// Non-temporal weight loads.  With LDS staging every load instruction reads
// whole 128 B lines; without it (fragments straight from memory, half a line
// per row) the default policy measured faster.
#define LOOM_MFMA_STREAM 1
#endif
#ifndef LOOM_MFMA_STEPS
#define LOOM_MFMA_STEPS 4        // k steps (KiB of weights per wave) per record
#endif
#ifndef LOOM_I8_COLS_DEPTH
#define LOOM_I8_COLS_DEPTH 3     // records in flight per wave, 17-64 vectors
#endif
#ifndef LOOM_I8_COLS_STAGGER
// First record of workgroup b: (b * STAGGER) mod records.  With every
// workgroup at the same column offset the 17-64 vector shapes ran 2-12 %
// slower; a stagger of 1 was up to 20 % slower at k = 8192, 5 the best of
// 1, 5 and 11 overall.
#define LOOM_I8_COLS_STAGGER 5
#endif
#ifndef LOOM_GEMV_NARROW_DEPTH
#define LOOM_GEMV_NARROW_DEPTH 6
#endif
constexpr int kGemvDepth = LOOM_GEMV_DEPTH;
constexpr int kGemvNarrowDepth = LOOM_GEMV_NARROW_DEPTH;
constexpr int kMfmaDepth = LOOM_MFMA_DEPTH;
constexpr int kMfmaSegDepth = LOOM_MFMA_SEG_DEPTH;
constexpr int kMfmaSteps = LOOM_MFMA_STEPS;
constexpr int kI8ColsDepth = LOOM_I8_COLS_DEPTH;

// 16-byte group of words [c, c+4) of a row with kw words; words at or beyond
// kw read as zero (they contribute nothing to any dot product).  VEC16: the
// host proved every row start 16-byte aligned (so kw % 4 == 0 and a group is
// wholly inside or wholly past the row), and one 128-bit load serves;
// otherwise the group is read as four dwords.  STREAM: the row is read once
// (weights), so the load is non-temporal; activations are reused and cached.
// SELECT: the guards are selects, not branches -- a word past the row is
// loaded from the row's first word (kw > 0 whenever a group is read) and
// replaced by zero -- so every lane issues the same loads and the read-ahead
// keeps its partial waits where many records are partly filled (the packed
// GEMV forms); elsewhere the branches, which need fewer registers, serve.
template <bool FULL, bool VEC16, bool STREAM, bool SELECT = false>
__device__ __forceinline__ int4v load_words(const int32_t *__restrict__ row, int c, int kw) {
    if constexpr (SELECT && VEC16) {
        const bool ok = FULL || c + 4 <= kw;
        const int4v *p = reinterpret_cast<const int4v *>(row + (ok ? c : 0));
        const int4v v = STREAM ? load_stream(p) : *p;
        return ok ? v : int4v{0, 0, 0, 0};
    } else if constexpr (SELECT) {
        int4v v;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bool ok = FULL || c + j < kw;
            const int t = STREAM ? load_stream(row + (ok ? c + j : 0)) : row[ok ? c + j : 0];
            v[j] = ok ? t : 0;
        }
        return v;
    } else {
        if (VEC16 && (FULL || c + 4 <= kw)) {
            const int4v *p = reinterpret_cast<const int4v *>(row + c);
            return STREAM ? load_stream(p) : *p;
        }
        int4v v = {0, 0, 0, 0};
        if (FULL || c + 0 < kw) v.x = row[c + 0];
        if (FULL || c + 1 < kw) v.y = row[c + 1];
        if (FULL || c + 2 < kw) v.z = row[c + 2];
        if (FULL || c + 3 < kw) v.w = row[c + 3];
        return v;
    }
}

// Row row0 + off, clamped to the last row.  row0 is the first row of a tile
// that exists (row0 < rows), so neither this nor a store guard of the form
// off < rows - row0 can overflow, even for rows close to 2^31.
__device__ __forceinline__ int row_clamped(int row0, int off, int rows) { return row0 + min(off, rows - 1 - row0); }

__device__ __forceinline__ int dot16(int4v a, int4v b, int acc) {
    acc = __builtin_amdgcn_sdot4(a.x, b.x, acc, false);
    acc = __builtin_amdgcn_sdot4(a.y, b.y, acc, false);
    acc = __builtin_amdgcn_sdot4(a.z, b.z, acc, false);
    acc = __builtin_amdgcn_sdot4(a.w, b.w, acc, false);
    return acc;
}

// ----------------------------------------------------------------------------
// One vector, rows of whole 1 KiB records and long rows (gemv_form).  One wave owns a block
// of consecutive rows -- gemv_rows_per_wave(k), about 8 KiB of weights --
// which is one contiguous stretch of the weight matrix, and walks it row after
// row.  A record is one 1 KiB column block of one row plus
// the activation group each lane needs at the same columns (16 bytes, reused
// by every wave and kept in the caches), so the read-ahead runs across row
// boundaries and the wave's weights stream in address order.  At the end of
// each row its int32 partials are summed across the wave (exact) into the
// lane that owns the row; one coalesced epilogue then scales and stores every
// row of the wave.  Small blocks make many short waves, so the waves that
// finish last at the end of the launch have little left to read.
// ----------------------------------------------------------------------------
struct GemvRecord {
    int4v xv, wv;
};

// ONE_ROW: rows_per_wave == 1, known at compile time.  FULL: rows of whole
// 1 KiB records; otherwise each row's last record is guarded (this form takes
// such rows only from 12 KiB, one row per wave).
template <bool FULL, bool VEC16, int DEPTH, bool ONE_ROW>
__global__ __launch_bounds__(kWave) void i8_gemv_kernel(const int32_t *__restrict__ w, const float *__restrict__ w_scale,
                                                        const int32_t *__restrict__ x,
                                                        const float *__restrict__ x_scale, int rows, int kw,
                                                        int rows_per_wave, float *__restrict__ out,
                                                        int32_t *__restrict__ acc_out) {
    constexpr int kBlockWords = kWave * 4;
    if constexpr (ONE_ROW) rows_per_wave = 1;
    const int lane = lane_id();
    const int row0 = blockIdx.x * rows_per_wave;
    const int nrows = min(rows_per_wave, rows - row0);
    const int records_per_row = (kw + kBlockWords - 1) / kBlockWords;

    // producer cursor (wave-uniform): the current row and the next column block
    const int32_t *wrow = w + (int64_t)row0 * kw;
    int lcol = 0;
    // consumer state
    int acc = 0, crec = 0, crow = 0, mine = 0;
    // the epilogue's scales, read before the stream (after it, their latency
    // would land on the wave's critical path)
    const float ws = w_scale[row0 + min(lane, nrows - 1)];
    const float xs = x_scale ? x_scale[0] : 1.0f;

    // a row of 8192 bytes is 8 records, most of them in the drain: the straight
    // drain measured about 3 % faster here
    pipelined<DEPTH, GemvRecord, true>(
        nrows * records_per_row,
        [&]() {
            GemvRecord q;
            const int c = lcol + lane * 4;
            q.xv = load_words<FULL, VEC16, false>(x, c, kw);
            q.wv = load_words<FULL, VEC16, true>(wrow, c, kw);
            if (lcol >= kw - kBlockWords) {
                lcol = 0;
                wrow += kw;
            } else {
                lcol += kBlockWords;
            }
            return q;
        },
        [&](const GemvRecord &q) {
            acc = dot16(q.wv, q.xv, acc);
            if (++crec == records_per_row) {
                const int total = wave_sum(acc);
                if (lane == crow) mine = total;
                acc = 0;
                crec = 0;
                ++crow;
            }
        });

    if (lane < nrows) {
        const int row = row0 + lane;
        float y = (float)mine;
        y = y * ws;
        if (x_scale) y = y * xs;
        out[row] = y;
        if (acc_out) acc_out[row] = mine;
    }
}

// ----------------------------------------------------------------------------
// One vector, rows of 6 to 8 whole 1 KiB records, or of 3 to 12 KiB that are
// not whole records (gemv_form): one workgroup per row of WAVES =
// gemv_wide_waves(k) waves.  Wave w reads records 2w and 2w+1 of the row (the
// last wave only 2w when a whole-record count is odd; FULL false: the row's
// last record partly empty, its lanes past the row reading the row's first
// word and adding zero), all of its loads issued at once, weights first;
// folds them with v_dot4 into per-lane int32 partials, reduces them across
// the wave, and the wave totals are added in wave order (exact).  Every wave of the launch reads one contiguous 2 KiB
// stretch of a row, which is what the HBM stream favours, and the code before
// the first load is kept short: a wave lives about one memory round trip, so
// its start-up latency is a visible share of it.  EVEN: the record count is
// even, so no wave tests for a missing second record.  STRIDE: the grid
// stopped at the work-item limit and each workgroup takes every grid.x-th row;
// otherwise workgroup b takes row b and reads no bound first.
// ----------------------------------------------------------------------------
template <bool FULL, bool VEC16, int WAVES, bool EVEN, bool STRIDE>
__global__ __launch_bounds__(kWave * WAVES) void i8_gemv_wide_kernel(
    const int32_t *__restrict__ w, const float *__restrict__ w_scale, const int32_t *__restrict__ x,
    const float *__restrict__ x_scale, int rows, int kw, float *__restrict__ out, int32_t *__restrict__ acc_out) {
    constexpr int kBlockWords = kWave * 4;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    // EVEN: every wave has two records; else the last has one (wave-uniform).
    // Rows that are not whole records read both with guards.
    const bool two = !FULL || EVEN || (2 * wave + 2) * kBlockWords <= kw;
    const int c = 2 * wave * kBlockWords + lane * 4;
    __shared__ int part[WAVES];
    auto one_row = [&](int64_t row) {
        const int32_t *wrow = w + row * kw;
        const int4v w0 = load_words<FULL, VEC16, true, true>(wrow, c, kw);
        int4v w1 = {0, 0, 0, 0}, x1 = {0, 0, 0, 0};
        if (two) w1 = load_words<FULL, VEC16, true, true>(wrow, c + kBlockWords, kw);
        const int4v x0 = load_words<FULL, VEC16, false, true>(x, c, kw);
        if (two) x1 = load_words<FULL, VEC16, false, true>(x, c + kBlockWords, kw);
        // the epilogue's scales, read while the stretch streams in
        const float ws = w_scale[row];
        const float xs = x_scale ? x_scale[0] : 1.0f;
        const int total = wave_sum(dot16(w1, x1, dot16(w0, x0, 0)));
        if (lane == 0) part[wave] = total;
        __syncthreads();
        if (threadIdx.x == 0) {
            int sum = part[0];
#pragma unroll
            for (int v = 1; v < WAVES; ++v) sum += part[v];
            float y = (float)sum;
            y = y * ws;
            if (x_scale) y = y * xs;
            out[row] = y;
            if (acc_out) acc_out[row] = sum;
        }
    };
    if constexpr (!STRIDE) {
        one_row(blockIdx.x);  // the grid has one workgroup per row
    } else {
        for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
            one_row(row);
            __syncthreads();  // part[] is rewritten for the next row
        }
    }
}

// ----------------------------------------------------------------------------
// One vector, rows longer than 512 bytes that are not whole 1 KiB records
// but whole 256-byte (LOG2L = 4) or 512-byte (LOG2L = 5) pieces -- the
// grouped form (gemv_group_log2_lanes): a record puts R = 64 / L rows side by
// side, L = 2^LOG2L lanes and 16 L bytes per row (lane l: row l / L of the
// group, 16-byte group l mod L of the piece), so no record is partly empty
// where a 1 KiB record per row would be; a load instruction reads R rows x
// 16 L contiguous bytes.  The wave owns rows_per_wave consecutive rows (a
// multiple of R, at most 64) and walks them group by group, each group's
// pieces in k order, with the read-ahead running across groups.  At the end
// of a group the first LOG2L steps of the wave reduction sum each row's L
// lanes (exact int32) and a lane permute hands row i of the wave its total in
// lane i.  Rows past the matrix load the wave's first row and drop the value.
// ----------------------------------------------------------------------------
template <bool VEC16, int LOG2L, int DEPTH>
__global__ __launch_bounds__(kWave) void i8_gemv_grouped_kernel(const int32_t *__restrict__ w,
                                                                const float *__restrict__ w_scale,
                                                                const int32_t *__restrict__ x,
                                                                const float *__restrict__ x_scale, int rows, int kw,
                                                                int rows_per_wave, float *__restrict__ out,
                                                                int32_t *__restrict__ acc_out) {
    static_assert(LOG2L >= 1 && LOG2L <= 5, "2 to 32 lanes per row");
    constexpr int L = 1 << LOG2L;
    constexpr int R = kWave / L;
    constexpr int kPieceWords = 4 * L;
    const int lane = lane_id();
    const int sub = lane >> LOG2L;          // row within the group
    const int q4 = (lane & (L - 1)) * 4;    // the lane's first word within the piece
    const int row0 = blockIdx.x * rows_per_wave;
    const int left = min(rows_per_wave, rows - row0);  // rows of this wave (> 0)
    const int pieces = kw / kPieceWords + (kw % kPieceWords != 0);
    const int groups = (left + R - 1) / R;
    const int32_t *first = w + (int64_t)row0 * kw;
    // producer: group lg, piece lp; consumer: group cg, piece cp
    int lg = 0, lp = 0, cg = 0, cp = 0, acc = 0, mine = 0;
    const int32_t *lrow = first + (int64_t)(sub < left ? sub : 0) * kw;
    // the epilogue's scales, read before the stream
    const float ws = w_scale[row0 + min(lane, left - 1)];
    const float xs = x_scale ? x_scale[0] : 1.0f;
    pipelined<DEPTH, GemvRecord>(
        groups * pieces,
        [&]() {
            GemvRecord q;
            const int c = lp * kPieceWords + q4;
            q.wv = load_words<false, VEC16, true, true>(lrow, c, kw);
            q.xv = load_words<false, VEC16, false, true>(x, c, kw);
            if (++lp == pieces) {
                lp = 0;
                ++lg;
                const int r = lg * R + sub;
                lrow = first + (int64_t)(r < left ? r : 0) * kw;
            }
            return q;
        },
        [&](const GemvRecord &q) {
            acc = dot16(q.wv, q.xv, acc);
            if (++cp == pieces) {
                const int total = group_sum<LOG2L>(acc);
                // lane cg * R + i takes the total of row i of the group (held by lane i * L)
                const int i = lane - cg * R;
                const int got = __builtin_amdgcn_ds_bpermute(((i >= 0 && i < R) ? i * L : 0) * 4, total);
                if (i >= 0 && i < R) mine = got;
                acc = 0;
                cp = 0;
                ++cg;
            }
        });
    if (lane < left) {
        const int row = row0 + lane;
        float y = (float)mine;
        y = y * ws;
        if (x_scale) y = y * xs;
        out[row] = y;
        if (acc_out) acc_out[row] = mine;
    }
}

// ----------------------------------------------------------------------------
// One vector, short rows (gemv_form: k <= 512): several rows per 1 KiB
// record, as the narrow row sums pack them.  A record holds R = 64 / L rows
// side by side, L = 2^LOG2L the smallest power of two with 16 L >= k bytes:
// lane l serves row l / L of the record and its 16-byte group l mod L, whose
// activation group is the same for every row, so it is loaded once.  Each
// lane folds its group with v_dot4, the first LOG2L steps of the wave
// reduction sum each aligned group of L lanes (exact int32), and a lane
// permute hands row i of the wave its total in lane i.  A wave owns
// rows_per_wave consecutive rows (whole records of about 8 KiB together, at
// most 64 rows); lanes past the last row load the wave's first row and drop
// the value, so every record issues the same loads.
// ----------------------------------------------------------------------------
template <bool VEC16, int LOG2L, int DEPTH>
__global__ __launch_bounds__(kWave) void i8_gemv_narrow_kernel(const int32_t *__restrict__ w,
                                                               const float *__restrict__ w_scale,
                                                               const int32_t *__restrict__ x,
                                                               const float *__restrict__ x_scale, int rows, int kw,
                                                               int rows_per_wave, float *__restrict__ out,
                                                               int32_t *__restrict__ acc_out) {
    constexpr int L = 1 << LOG2L;
    constexpr int R = kWave / L;
    const int lane = lane_id();
    const int sub = lane >> LOG2L;  // row within the record
    const int c = (lane & (L - 1)) * 4;  // first word of the lane's group
    const int row0 = blockIdx.x * rows_per_wave;
    const int left = min(rows_per_wave, rows - row0);  // rows of this wave that exist (> 0)
    const int nrec = kw > 0 ? (left + R - 1) / R : 0;
    const int4v xv = nrec > 0 ? load_words<false, VEC16, false, true>(x, c, kw) : int4v{0, 0, 0, 0};
    const int32_t *first = w + (int64_t)row0 * kw;
    int lrec = 0, crec = 0, mine = 0;
    // the epilogue's scales, read before the stream
    const float ws = w_scale[row0 + min(lane, left - 1)];
    const float xs = x_scale ? x_scale[0] : 1.0f;
    pipelined<DEPTH, int4v>(
        nrec,
        [&]() {
            const int lr = lrec * R + sub;
            const int4v v = load_words<false, VEC16, true, true>(first + (int64_t)(lr < left ? lr : 0) * kw, c, kw);
            ++lrec;
            return v;
        },
        [&](const int4v &v) {
            const int total = group_sum<LOG2L>(dot16(v, xv, 0));
            // lane crec * R + i takes the total of row i of the record (held by lane i * L)
            const int i = lane - crec * R;
            const int got = __builtin_amdgcn_ds_bpermute(((i >= 0 && i < R) ? i * L : 0) * 4, total);
            if (i >= 0 && i < R) mine = got;
            ++crec;
        });
    if (lane < left) {
        const int row = row0 + lane;
        float y = (float)mine;
        y = y * ws;
        if (x_scale) y = y * xs;
        out[row] = y;
        if (acc_out) acc_out[row] = mine;
    }
}

// ----------------------------------------------------------------------------
// Several vectors (batch >= 2): the shared activations make this a dense
// int8 contraction, so it runs on the matrix cores.  This LDS-staged tile
// kernel takes the batches no other kernel below takes (2 to 6 vectors unless
// 8 waves split k, and 9 to 16 where the row kernel does not apply; mfma_seg,
// i8_rows_chunks).  One workgroup owns a
// 16-row tile; its KS waves (1, 2, 4 or 8: about 2 KiB of every row per wave,
// mfma_ksplit) each take a contiguous share of k (of the records), and their
// int32 partial tiles are added in wave order at the end (exact).  Each k step is one v_mfma_i32_16x16x64_i8:
//   A (16 x 64, weights):  lane l holds 16 bytes of row (l & 15) at byte
//                          offset 16*(l >> 4) of the 64-byte step;
//   B (64 x 16, vectors):  lane l holds the same 16 byte positions of vector
//                          (l & 15) (zero for vectors >= batch);
//   D (16 x 16, int32):    lane l holds rows 4*(l >> 4) + i, i < 4, of
//                          column (l & 15).
// A and B use the same byte-to-k assignment in every lane, so the product
// sums exactly the matching k positions whatever order the hardware uses
// inside a step.  A record is S steps (S KiB of weights per wave); NT tiles
// of 16 vectors cover batch <= 16 * NT.  The accumulators are exact int32.
// ----------------------------------------------------------------------------
// Vector columns at or beyond the batch hold a clamped (valid) row; they are
// zeroed where consumed, so the producer never waits on its own loads.
__device__ __forceinline__ int4v live_b(int4v b, bool live) { return live ? b : int4v{0, 0, 0, 0}; }

template <int S, int NT>
struct MfmaRecord {
    int4v a[S];
    int4v b[NT][S];
};

template <bool FULL, bool VEC16, bool STAGE, int DEPTH, int S, int NT, int KS>
__global__ __launch_bounds__(kWave * KS) void i8_mfma_kernel(const int32_t *__restrict__ w, const float *__restrict__ w_scale,
                                                        const int32_t *__restrict__ x,
                                                        const float *__restrict__ x_scale, int rows, int kw, int batch,
                                                        float *__restrict__ out, int32_t *__restrict__ acc_out) {
    static_assert(!STAGE || S == 4, "LDS staging moves 16 rows x 256 B (4 k steps) per record");
    constexpr int kStepWords = 16;  // 64 int8 per step
    const int lane = lane_id();
    const int m = lane & 15;
    const int g = lane >> 4;
    const int row0 = blockIdx.x * kMfmaTileRows;
    const int32_t *wrow = w + (int64_t)row_clamped(row0, m, rows) * kw;
    // Staged loads: instruction i of a record reads rows 4i..4i+3 of the tile,
    // 256 contiguous bytes each (lane: row 4i + (lane >> 4), chunk lane & 15).
    const int srow = lane >> 4, schunk = lane & 15;
    const int32_t *wstage[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) wstage[i] = w + (int64_t)row_clamped(row0, 4 * i + srow, rows) * kw;
    // Per-wave staging tile: 16 rows x 16 chunks of 16 B; chunk c of row r at
    // slot 16 r + (c ^ r), so both the row-wise writes and the fragment reads
    // (16 rows, one chunk each) fall on distinct banks.
    __shared__ int4v stage[STAGE ? KS : 1][STAGE ? 16 * 16 : 1];
    const int32_t *xrow[NT];
    bool xlive[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int n = t * 16 + m;
        xlive[t] = n < batch;
        xrow[t] = x + (int64_t)min(n, batch - 1) * kw;
    }
    const int steps = (kw + kStepWords - 1) / kStepWords;
    // the same in every lane: keeps the wave's k share and loop count scalar
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    // this wave's contiguous share of the k records
    const int all_records = (steps + S - 1) / S;
    const int per_wave = (all_records + KS - 1) / KS;
    const int first = min(all_records, wave * per_wave);
    const int records = min(all_records, first + per_wave) - first;

    int4v acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = int4v{0, 0, 0, 0};
    // The epilogue's scales (wave 0 writes the tile), read before the stream:
    // read after it, their latency lands on every workgroup's critical path.
    float ws_pre[4] = {}, xs_pre[NT] = {};
    if (wave == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) ws_pre[i] = w_scale[row_clamped(row0, 4 * g + i, rows)];
#pragma unroll
        for (int t = 0; t < NT; ++t) xs_pre[t] = x_scale ? x_scale[min(t * 16 + m, batch - 1)] : 1.0f;
    }

    int lrec = first;
    pipelined<DEPTH, MfmaRecord<S, NT>>(
        records,
        [&]() {
            MfmaRecord<S, NT> q;
            if constexpr (STAGE) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    q.a[i] = load_words<FULL, VEC16, LOOM_MFMA_STREAM != 0>(wstage[i], (lrec * 16 + schunk) * 4, kw);
            }
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const int c = (lrec * S + s) * kStepWords + g * 4;
                if constexpr (!STAGE) q.a[s] = load_words<FULL, VEC16, LOOM_MFMA_STREAM != 0>(wrow, c, kw);
#pragma unroll
                for (int t = 0; t < NT; ++t) q.b[t][s] = load_words<FULL, VEC16, false>(xrow[t], c, kw);
            }
            ++lrec;
            return q;
        },
        [&](const MfmaRecord<S, NT> &q) {
            if constexpr (STAGE) {
                int4v *tile = stage[wave];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 4 * i + srow;
                    tile[16 * r + (schunk ^ r)] = q.a[i];
                }
#pragma unroll
                for (int s = 0; s < S; ++s) {
                    const int4v a = tile[16 * m + ((4 * s + g) ^ m)];
#pragma unroll
                    for (int t = 0; t < NT; ++t)
                        acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, live_b(q.b[t][s], xlive[t]), acc[t], 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int s = 0; s < S; ++s)
#pragma unroll
                    for (int t = 0; t < NT; ++t)
                        acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(q.a[s], live_b(q.b[t][s], xlive[t]), acc[t],
                                                                        0, 0, 0);
            }
        });

    if constexpr (KS > 1) {
        // waves 1.. publish their partial tiles; wave 0 adds them in wave order
        __shared__ int partial[KS > 1 ? KS - 1 : 1][NT][4][kWave];
        if (wave > 0) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) partial[wave - 1][t][i][lane] = acc[t][i];
        }
        __syncthreads();
        if (wave != 0) return;
        for (int v = 0; v < KS - 1; ++v)
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[t][i] += partial[v][t][i][lane];
    }

#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int n = t * 16 + m;
        if (n >= batch) continue;
        const float xs = xs_pre[t];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (4 * g + i < rows - row0) {
                const int row = row0 + 4 * g + i;
                const int a = acc[t][i];
                float y = (float)a;
                y = y * ws_pre[i];
                if (x_scale) y = y * xs;
                out[(int64_t)row * batch + n] = y;
                if (acc_out) acc_out[(int64_t)row * batch + n] = a;
            }
        }
    }
}


// ----------------------------------------------------------------------------
// Seven or eight vectors (two to eight when 8 waves split k; mfma_seg): the
// segment-paired matrix-core kernel, with no LDS staging.  One workgroup owns
// a 16-row tile; its KS waves (mfma_ksplit) each take a contiguous share of k
// in records of 16 rows x 256 bytes, and their int32 partials are added in
// wave order at the end (exact).  A k step's A
// operand is 16 rows x 64 bytes; here its 16 rows are 4 weight rows x 4
// segments of 64 bytes (A row m: weight row 4i + (m >> 2), bytes 64 (m & 3) ..
// of the record's 256), and the B operand's 16 columns are 4 vectors x the
// same 4 segments (column n: vector 4 vg + (n >> 2), segment n & 3).  Lane l
// (m = l & 15, g = l >> 4) holds bytes 64 (m & 3) + 16 g .. + 15 of both, so
// one load instruction reads 4 weight rows x 256 contiguous bytes straight
// into the A layout.  D[m][n] adds segment (m & 3) of a row times segment
// (n & 3) of a vector; only equal segments are wanted.  Lane l holds
// D[4 (l >> 4) + e][l & 15], whose wanted entry is e = l & 3 (row 4i + (l >> 4),
// vector 4 vg + ((l & 15) >> 2)), and the 4 lanes of a quad hold the 4
// segments of one (row, vector) pair, added by two DPP steps after the
// stream.  The matrix cores do 4 times the useful products, a few percent of
// their peak here; in exchange no record passes through LDS.  VG: vector
// groups of 4 (1 up to 4 vectors, 2 up to 8).
// ----------------------------------------------------------------------------
template <int VG>
struct SegRecord {
    int4v a[4];
    int4v b[VG];
};

template <bool FULL, bool VEC16, int DEPTH, int VG, int KS>
__global__ __launch_bounds__(kWave * KS) void i8_mfma_seg_kernel(const int32_t *__restrict__ w,
                                                                 const float *__restrict__ w_scale,
                                                                 const int32_t *__restrict__ x,
                                                                 const float *__restrict__ x_scale, int rows, int kw,
                                                                 int batch, float *__restrict__ out,
                                                                 int32_t *__restrict__ acc_out) {
    constexpr int kRecordWords = 64;       // 256 bytes of a row per record
    constexpr int kOuts = 16 * 4 * VG;     // the tile's outputs: 16 rows x 4 VG vector slots
    constexpr int kPer = (kOuts + kWave * KS - 1) / (kWave * KS);  // outputs per thread
    const int lane = lane_id();
    const int m = lane & 15, g = lane >> 4;
    const int row0 = blockIdx.x * kMfmaTileRows;
    const int loff = (m & 3) * 16 + g * 4;  // words: segment m & 3, 16-byte group g
    const int32_t *wrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) wrow[i] = w + (int64_t)row_clamped(row0, 4 * i + (m >> 2), rows) * kw;
    const int32_t *xrow[VG];
    bool xlive[VG];
#pragma unroll
    for (int vg = 0; vg < VG; ++vg) {
        const int v = 4 * vg + (m >> 2);
        xlive[vg] = v < batch;
        xrow[vg] = x + (int64_t)min(v, batch - 1) * kw;
    }
    // the same in every lane: keeps the wave's k share and loop count scalar
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const int all_records = kw / kRecordWords + (kw % kRecordWords != 0);
    const int per_wave = (all_records + KS - 1) / KS;
    const int first = min(all_records, wave * per_wave);
    const int records = min(all_records, first + per_wave) - first;

    // The epilogue's scales, read before the stream: read after it, their
    // latency lands on every workgroup's critical path.
    float ws_pre[kPer], xs_pre[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int o = (int)threadIdx.x + j * kWave * KS;
        const int r = min(o / (4 * VG), 15), v = o % (4 * VG);
        ws_pre[j] = w_scale[row_clamped(row0, r, rows)];
        xs_pre[j] = x_scale ? x_scale[min(v, batch - 1)] : 1.0f;
    }

    int4v acc[4][VG];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int vg = 0; vg < VG; ++vg) acc[i][vg] = int4v{0, 0, 0, 0};
    int lrec = first;
    pipelined<DEPTH, SegRecord<VG>>(
        records,
        [&]() {
            SegRecord<VG> q;
            const int c = lrec * kRecordWords + loff;
#pragma unroll
            for (int i = 0; i < 4; ++i) q.a[i] = load_words<FULL, VEC16, LOOM_MFMA_STREAM != 0>(wrow[i], c, kw);
#pragma unroll
            for (int vg = 0; vg < VG; ++vg) q.b[vg] = load_words<FULL, VEC16, false>(xrow[vg], c, kw);
            ++lrec;
            return q;
        },
        [&](const SegRecord<VG> &q) {
#pragma unroll
            for (int vg = 0; vg < VG; ++vg) {
                const int4v b = live_b(q.b[vg], xlive[vg]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[i][vg] = __builtin_amdgcn_mfma_i32_16x16x64_i8(q.a[i], b, acc[i][vg], 0, 0, 0);
            }
        });

    // each quad adds its pair's 4 segments; its first lane publishes the sum
    __shared__ int part[KS][kOuts];
    const int e = lane & 3;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int vg = 0; vg < VG; ++vg) {
            const int4v d = acc[i][vg];
            int t = e == 0 ? d[0] : e == 1 ? d[1] : e == 2 ? d[2] : d[3];
            t = t + dpp<kDppQuadSwap1>(t);
            t = t + dpp<kDppQuadSwap2>(t);
            if (e == 0) part[wave][(4 * i + g) * (4 * VG) + 4 * vg + (m >> 2)] = t;
        }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int o = (int)threadIdx.x + j * kWave * KS;
        if (o >= kOuts) break;
        const int r = o / (4 * VG), v = o % (4 * VG);
        if (v >= batch || r >= rows - row0) continue;
        int sum = part[0][o];
#pragma unroll
        for (int q = 1; q < KS; ++q) sum += part[q][o];
        float y = (float)sum;
        y = y * ws_pre[j];
        if (x_scale) y = y * xs_pre[j];
        out[(int64_t)(row0 + r) * batch + v] = y;
        if (acc_out) acc_out[(int64_t)(row0 + r) * batch + v] = sum;
    }
}

// ----------------------------------------------------------------------------
// Nine to sixteen vectors, rows of 4 to 8 KiB streamed whole (the choice of
// kernel is i8_rows_chunks).  One workgroup of 16 waves
// per CU walks 16-row tiles (tile t, t + gridDim.x, ...).  Wave w holds row w
// of the next tile in registers -- its k bytes, one contiguous 1 KiB per load
// instruction -- while the current tile is consumed, then stores it into an
// LDS tile with 16-byte chunk c of row r at slot c ^ r of that row, so both the
// row-wise stores and the 16-row fragment reads fall on distinct banks.
// After a barrier, wave w multiplies the 16 rows by the vectors over its
// 1/16 of k (CHUNKS steps of 64 bytes, in the A/B/D layouts of the kernel
// above; its vector fragments are loaded once and stay in registers for every
// tile), writes its int32 partial tile to LDS, and after a second barrier the
// first 256 threads each add one output's 16 partials (exact) and apply the
// epilogue.  The barriers wait for LDS only: the next tile's row loads stay in
// flight across them.  Every wave of a workgroup runs the same tiles, so all
// reach every barrier.
// ----------------------------------------------------------------------------
template <int CHUNKS, bool VEC16>
__global__ __launch_bounds__(kWave * kI8RowsWaves) void i8_mfma_rows_kernel(
    const int32_t *__restrict__ w, const float *__restrict__ w_scale, const int32_t *__restrict__ x,
    const float *__restrict__ x_scale, int rows, int kw, int batch, float *__restrict__ out,
    int32_t *__restrict__ acc_out) {
    static_assert(CHUNKS >= 1 && CHUNKS <= kI8RowsMaxChunks, "k is 1 to 8 KiB per row");
    constexpr int kUnits = CHUNKS * kWave;  // 16-byte chunks per row (kw = 256 * CHUNKS words)
    __shared__ int4v tile[kMfmaTileRows * kUnits];
    __shared__ int partial[kI8RowsWaves][4][kWave];
    const int lane = lane_id();
    // the same in every lane: keeps the wave's k share and row scalar
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const int ntiles = (int)(((int64_t)rows + kMfmaTileRows - 1) / kMfmaTileRows);
    const int m = lane & 15, g = lane >> 4;

    // this wave's vector fragments, k steps wave * CHUNKS .. + CHUNKS; every
    // lane loads a valid (clamped) vector and columns past the batch are zeroed
    int4v bfrag[CHUNKS];
    const int32_t *xrow = x + (int64_t)min(m, batch - 1) * kw;
#pragma unroll
    for (int s = 0; s < CHUNKS; ++s) {
        const int4v v = load_words<true, VEC16, false>(xrow, (wave * CHUNKS + s) * 16 + g * 4, kw);
        bfrag[s] = m < batch ? v : int4v{0, 0, 0, 0};
    }

    // The epilogue's scales: thread (r, n) < 256 scales output (r, n) of every
    // tile.  x_scale is read once; w_scale[row r of tile t] is read with the
    // tile's rows, before them, so it has arrived when the rows have (read in
    // the epilogue, it would wait for the next tile's loads as well).
    const int er = (threadIdx.x >> 4) & 15, en = threadIdx.x & 15;
    const float xs = x_scale ? x_scale[min(en, batch - 1)] : 1.0f;
    float ws_next = 0.0f, ws = 0.0f;
    int4v rowbuf[CHUNKS];
    auto load_row = [&](int t) {
        ws_next = w_scale[row_clamped(t * kMfmaTileRows, er, rows)];
        // rows past the end load the last row; their outputs are never stored
        const int32_t *src = w + (int64_t)row_clamped(t * kMfmaTileRows, wave, rows) * kw;
#pragma unroll
        for (int j = 0; j < CHUNKS; ++j) rowbuf[j] = load_words<true, VEC16, true>(src, (j * kWave + lane) * 4, kw);
    };

    int t = blockIdx.x;
    if (t < ntiles) load_row(t);
    for (; t < ntiles; t += gridDim.x) {
#pragma unroll
        for (int j = 0; j < CHUNKS; ++j) {
            const int c = j * kWave + lane;
            tile[wave * kUnits + (c ^ wave)] = rowbuf[j];
        }
        ws = ws_next;
        if (t + (int)gridDim.x < ntiles) load_row(t + gridDim.x);
        __syncthreads();
        int4v acc = int4v{0, 0, 0, 0};
#pragma unroll
        for (int s = 0; s < CHUNKS; ++s) {
            const int c = (wave * CHUNKS + s) * 4 + g;
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(tile[m * kUnits + (c ^ m)], bfrag[s], acc, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) partial[wave][i][lane] = acc[i];
        __syncthreads();
        if (threadIdx.x < kMfmaTileRows * 16) {
            // output (r, n) of the tile sits in lane 16 (r / 4) + n, slot r % 4, of every partial
            const int r = er, n = en;
            int sum = 0;
            for (int v = 0; v < kI8RowsWaves; ++v) sum += partial[v][r & 3][(r >> 2) * 16 + n];
            if (n < batch && r < rows - t * kMfmaTileRows) {
                const int row = t * kMfmaTileRows + r;
                float y = (float)sum;
                y = y * ws;
                if (x_scale) y = y * xs;
                out[(int64_t)row * batch + n] = y;
                if (acc_out) acc_out[(int64_t)row * batch + n] = sum;
            }
        }
    }
}

// ----------------------------------------------------------------------------
// More than 16 vectors: one workgroup of 4 waves, one per 16-vector column
// tile (columns past the batch are zeroed), owns RT 16-row tiles, the tiles
// shared evenly between q workgroups per CU (one or two up to 65536 rows).
// The waves split each 256-byte weight record of the workgroup's rows (each
// loads SHARE instructions of 4 rows x 256 B, whole 256-byte pieces) and
// store it into one of two LDS slots, swizzled as in the kernels above; after
// a barrier each wave multiplies all RT tiles of the record by its own vector
// fragments (4 k steps), which it loads once per record for all RT tiles, so
// the vectors are read from the caches once per RT tiles instead of once per
// tile.  Every wave covers the full k for its outputs and stores them
// directly.  A barrier per record is enough with two slots: a wave can only
// overwrite a slot after every wave has passed the next record's barrier,
// that is, after all of them have finished reading it.  (The template also
// takes 2 column tiles and RG row groups of RT tiles each; the library
// launches 4 column tiles and one row group.)
// ----------------------------------------------------------------------------
template <int SHARE> struct ColsRecord {
    int4v a[SHARE];    // this wave's share of the record: SHARE loads of 4 rows x 256 B
    int4v b[4];        // its vector fragments for the record's 4 k steps
};

// At least two waves per SIMD (at most 256 registers): two workgroups of
// four waves share a CU when the rows need two per CU.
template <bool FULL, bool VEC16, int NT, int RT, int RG, int DEPTH>
__global__ __launch_bounds__(kWave * NT * RG, 2) void i8_mfma_cols_kernel(
    const int32_t *__restrict__ w, const float *__restrict__ w_scale, const int32_t *__restrict__ x,
    const float *__restrict__ x_scale, int rows, int kw, int batch, float *__restrict__ out,
    int32_t *__restrict__ acc_out) {
    static_assert(NT == 2 || NT == 4, "two or four column tiles");
    constexpr int kWaves = NT * RG;
    constexpr int kRows = kMfmaTileRows * RT * RG;  // rows per workgroup
    constexpr int kShare = kRows / (4 * kWaves);     // 4-row loads per wave and record
    static_assert(kShare >= 1 && kShare * 4 * kWaves == kRows, "the waves split the record evenly");
    constexpr int kRecordWords = 64;  // 256 bytes of each row
    __shared__ int4v stage[2][kRows * 16];
    const int lane = lane_id();
    // the same in every lane: the wave's column tile, row group and row share stay scalar
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const int ct = wave % NT, group = wave / NT;
    const int m = lane & 15, g = lane >> 4;
    const int row0 = blockIdx.x * kRows;
    // staged loads: instruction i reads rows 4 (wave * kShare + i) .. + 3, 256 contiguous bytes each
    const int srow = lane >> 4, schunk = lane & 15;
    const int32_t *wsrc[kShare];
#pragma unroll
    for (int i = 0; i < kShare; ++i)
        wsrc[i] = w + (int64_t)row_clamped(row0, (wave * kShare + i) * 4 + srow, rows) * kw;
    const int n = ct * 16 + m;  // this lane's vector
    const bool live = n < batch;
    const int32_t *xrow = x + (int64_t)min(n, batch - 1) * kw;
    const int records = (kw + kRecordWords - 1) / kRecordWords;

    // Workgroup b walks the records from (b * STAGGER) mod records, wrapping
    // around: the sums are exact int32, so the order of the records does not
    // change them, and the workgroups' concurrent loads then fall on different
    // column offsets of their rows.
    int lrec = records > 0 ? (int)(((int64_t)blockIdx.x * LOOM_I8_COLS_STAGGER) % records) : 0;
    int crec = 0;
    int4v acc[RT];
#pragma unroll
    for (int j = 0; j < RT; ++j) acc[j] = int4v{0, 0, 0, 0};
    pipelined<DEPTH, ColsRecord<kShare>>(
        records,
        [&]() {
            ColsRecord<kShare> q;
#pragma unroll
            for (int i = 0; i < kShare; ++i)
                q.a[i] = load_words<FULL, VEC16, true>(wsrc[i], lrec * kRecordWords + schunk * 4, kw);
#pragma unroll
            for (int s = 0; s < 4; ++s)
                q.b[s] = load_words<FULL, VEC16, false>(xrow, lrec * kRecordWords + s * 16 + g * 4, kw);
            lrec = lrec + 1 == records ? 0 : lrec + 1;
            return q;
        },
        [&](const ColsRecord<kShare> &q) {
            int4v *slot = stage[crec & 1];
#pragma unroll
            for (int i = 0; i < kShare; ++i) {
                const int r = (wave * kShare + i) * 4 + srow;
                slot[16 * r + (schunk ^ (r & 15))] = q.a[i];
            }
            __syncthreads();
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int4v b = live_b(q.b[s], live);
#pragma unroll
                for (int j = 0; j < RT; ++j) {
                    const int r = (group * RT + j) * kMfmaTileRows + m;
                    acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(slot[16 * r + ((4 * s + g) ^ m)], b, acc[j], 0, 0,
                                                                   0);
                }
            }
            ++crec;
        });

    if (live) {
        const float xs = x_scale ? x_scale[n] : 1.0f;
#pragma unroll
        for (int j = 0; j < RT; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int off = (group * RT + j) * kMfmaTileRows + 4 * g + i;
                if (off < rows - row0) {
                    const int row = row0 + off;
                    float y = (float)acc[j][i];
                    y = y * w_scale[row];
                    if (x_scale) y = y * xs;
                    out[(int64_t)row * batch + n] = y;
                    if (acc_out) acc_out[(int64_t)row * batch + n] = acc[j][i];
                }
            }
    }
}

template <bool FULL, bool VEC16, int RT>
static void launch_mfma_cols4(dim3 grid, dim3 block, hipStream_t stream, const int32_t *w, const float *w_scale,
                              const int32_t *x, const float *x_scale, int rows, int kw, int batch, float *out,
                              int32_t *acc) {
    i8_mfma_cols_kernel<FULL, VEC16, 4, RT, 1, kI8ColsDepth>
        <<<grid, block, 0, stream>>>(w, w_scale, x, x_scale, rows, kw, batch, out, acc);
}

// Returns false, launching nothing, for a row-tile count outside 1..8 (the
// geometry never produces one).
template <bool FULL, bool VEC16>
static bool launch_mfma_cols(dim3 grid, dim3 block, hipStream_t stream, const int32_t *w, const float *w_scale,
                             const int32_t *x, const float *x_scale, int rows, int kw, int batch, float *out,
                             int32_t *acc) {
    // the shapes below are the ones the launch geometry (i8_cols_*) describes
    static_assert(kI8ColsMaxRowTiles == 8, "one instantiation per row-tile count");
    switch (i8_cols_row_tiles(rows)) {
#define LOOM_COLS4_CASE(RT) \
    case RT: launch_mfma_cols4<FULL, VEC16, RT>(grid, block, stream, w, w_scale, x, x_scale, rows, kw, batch, out, acc); return true;
        LOOM_COLS4_CASE(1) LOOM_COLS4_CASE(2) LOOM_COLS4_CASE(3) LOOM_COLS4_CASE(4)
        LOOM_COLS4_CASE(5) LOOM_COLS4_CASE(6) LOOM_COLS4_CASE(7) LOOM_COLS4_CASE(8)
#undef LOOM_COLS4_CASE
        default: return false;
    }
}

template <int CHUNKS>
static void launch_mfma_rows(dim3 grid, bool vec16, hipStream_t stream, const int32_t *w, const float *w_scale,
                             const int32_t *x, const float *x_scale, int rows, int kw, int batch, float *out,
                             int32_t *acc) {
    // only the row lengths i8_rows_chunks admits are instantiated
    if constexpr (CHUNKS >= LOOM_I8_ROWS_MIN_CHUNKS) {
        const dim3 block(kWave * kI8RowsWaves);
        if (vec16)
            i8_mfma_rows_kernel<CHUNKS, true><<<grid, block, 0, stream>>>(w, w_scale, x, x_scale, rows, kw, batch, out,
                                                                          acc);
        else
            i8_mfma_rows_kernel<CHUNKS, false><<<grid, block, 0, stream>>>(w, w_scale, x, x_scale, rows, kw, batch,
                                                                           out, acc);
    }
}

template <bool FULL, bool VEC16>
static bool launch_mfma(dim3 grid, dim3 block, hipStream_t stream, const int32_t *w, const float *w_scale,
                        const int32_t *x, const float *x_scale, int rows, int kw, int batch, float *out,
                        int32_t *acc) {
    constexpr bool kStage = kMfmaStage;
    if (batch > 16)
        return launch_mfma_cols<FULL, VEC16>(grid, block, stream, w, w_scale, x, x_scale, rows, kw, batch, out, acc);
    // the split is the one the launch geometry (mfma_ksplit) describes
    if (mfma_seg(4 * (int64_t)kw, rows, batch)) {
        switch (mfma_ksplit(4 * (int64_t)kw, rows) * 2 + (batch > 4 ? 1 : 0)) {
#define LOOM_SEG_CASE(KS, VG)                                                                                 \
    case KS * 2 + (VG - 1):                                                                                   \
        i8_mfma_seg_kernel<FULL, VEC16, kMfmaSegDepth, VG, KS>                                                \
            <<<grid, block, 0, stream>>>(w, w_scale, x, x_scale, rows, kw, batch, out, acc);                  \
        return true;
            LOOM_SEG_CASE(1, 1) LOOM_SEG_CASE(1, 2) LOOM_SEG_CASE(2, 1) LOOM_SEG_CASE(2, 2)
            LOOM_SEG_CASE(4, 1) LOOM_SEG_CASE(4, 2) LOOM_SEG_CASE(8, 1) LOOM_SEG_CASE(8, 2)
#undef LOOM_SEG_CASE
            default: return false;
        }
    }
    switch (mfma_ksplit(4 * (int64_t)kw, rows)) {
#define LOOM_MFMA_CASE(KS)                                                                                    \
    case KS:                                                                                                  \
        i8_mfma_kernel<FULL, VEC16, kStage, kMfmaDepth, kMfmaSteps, 1, KS>                                    \
            <<<grid, block, 0, stream>>>(w, w_scale, x, x_scale, rows, kw, batch, out, acc);                  \
        return true;
        LOOM_MFMA_CASE(1) LOOM_MFMA_CASE(2) LOOM_MFMA_CASE(4) LOOM_MFMA_CASE(8)
#undef LOOM_MFMA_CASE
        default: return false;
    }
}

template <bool VEC16>
static void launch_gemv_narrow(dim3 grid, dim3 block, hipStream_t stream, const int32_t *w, const float *w_scale,
                               const int32_t *x, const float *x_scale, int rows, int kw, float *out, int32_t *acc) {
    const int rpw = gemv_narrow_rows_per_wave(4 * (int64_t)kw);
    switch (gemv_narrow_log2_lanes(kw)) {
#define LOOM_NARROW_CASE(L2)                                                                                     \
    case L2:                                                                                                     \
        i8_gemv_narrow_kernel<VEC16, L2, kGemvNarrowDepth>                                                       \
            <<<grid, block, 0, stream>>>(w, w_scale, x, x_scale, rows, kw, rpw, out, acc);                      \
        break;
        LOOM_NARROW_CASE(0) LOOM_NARROW_CASE(1) LOOM_NARROW_CASE(2) LOOM_NARROW_CASE(3) LOOM_NARROW_CASE(4)
        default:
        LOOM_NARROW_CASE(5)
#undef LOOM_NARROW_CASE
    }
}

template <int WAVES>
static void launch_gemv_wide_waves(dim3 grid, dim3 block, hipStream_t stream, bool vec16, bool stride,
                                   const int32_t *w, const float *w_scale, const int32_t *x, const float *x_scale,
                                   int rows, int kw, float *out, int32_t *acc) {
#define LOOM_WIDE(F, V, E, S) \
    i8_gemv_wide_kernel<F, V, WAVES, E, S><<<grid, block, 0, stream>>>(w, w_scale, x, x_scale, rows, kw, out, acc)
    const bool full = kw % (kWave * 4) == 0;
    const bool even = kw % (2 * kWave * 4) == 0;
    if (!full) {
        if (vec16 && !stride) LOOM_WIDE(false, true, false, false);
        else if (!stride) LOOM_WIDE(false, false, false, false);
        else if (vec16) LOOM_WIDE(false, true, false, true);
        else LOOM_WIDE(false, false, false, true);
    } else if (vec16 && even && !stride) LOOM_WIDE(true, true, true, false);
    else if (vec16 && !stride) LOOM_WIDE(true, true, false, false);
    else if (!stride) LOOM_WIDE(true, false, false, false);
    else if (vec16) LOOM_WIDE(true, true, false, true);
    else LOOM_WIDE(true, false, false, true);
#undef LOOM_WIDE
}

// The wave count is the one the launch geometry (gemv_wide_waves) gives the
// workgroup; the row lengths gemv_form admits need 2 to 6.
static bool launch_gemv_wide(dim3 grid, dim3 block, hipStream_t stream, bool vec16, bool stride, const int32_t *w,
                             const float *w_scale, const int32_t *x, const float *x_scale, int rows, int kw,
                             float *out, int32_t *acc) {
    switch (block.x / kWave) {
        case 2: launch_gemv_wide_waves<2>(grid, block, stream, vec16, stride, w, w_scale, x, x_scale, rows, kw, out, acc); return true;
        case 3: launch_gemv_wide_waves<3>(grid, block, stream, vec16, stride, w, w_scale, x, x_scale, rows, kw, out, acc); return true;
        case 4: launch_gemv_wide_waves<4>(grid, block, stream, vec16, stride, w, w_scale, x, x_scale, rows, kw, out, acc); return true;
        case 5: launch_gemv_wide_waves<5>(grid, block, stream, vec16, stride, w, w_scale, x, x_scale, rows, kw, out, acc); return true;
        case 6: launch_gemv_wide_waves<6>(grid, block, stream, vec16, stride, w, w_scale, x, x_scale, rows, kw, out, acc); return true;
        default: return false;
    }
}

hipError_t launch_i8_dequant_dot(const loom_launch_config &cfg, const int32_t *w, const float *w_scale,
                                 const int32_t *x, const float *x_scale, int rows, int k_words, int batch,
                                 float *out, int32_t *acc, hipStream_t stream) {
    const dim3 grid(cfg.workgroups[0]), block(cfg.workgroup_size[0]);
    const bool vec16 = (k_words % 4 == 0) && (reinterpret_cast<uintptr_t>(w) % 16 == 0) &&
                       (reinterpret_cast<uintptr_t>(x) % 16 == 0);
    switch (i8_rows_chunks(rows, 4 * (int64_t)k_words, batch)) {
        case 1: launch_mfma_rows<1>(grid, vec16, stream, w, w_scale, x, x_scale, rows, k_words, batch, out, acc); return hipGetLastError();
        case 2: launch_mfma_rows<2>(grid, vec16, stream, w, w_scale, x, x_scale, rows, k_words, batch, out, acc); return hipGetLastError();
        case 3: launch_mfma_rows<3>(grid, vec16, stream, w, w_scale, x, x_scale, rows, k_words, batch, out, acc); return hipGetLastError();
        case 4: launch_mfma_rows<4>(grid, vec16, stream, w, w_scale, x, x_scale, rows, k_words, batch, out, acc); return hipGetLastError();
        case 5: launch_mfma_rows<5>(grid, vec16, stream, w, w_scale, x, x_scale, rows, k_words, batch, out, acc); return hipGetLastError();
        case 6: launch_mfma_rows<6>(grid, vec16, stream, w, w_scale, x, x_scale, rows, k_words, batch, out, acc); return hipGetLastError();
        case 7: launch_mfma_rows<7>(grid, vec16, stream, w, w_scale, x, x_scale, rows, k_words, batch, out, acc); return hipGetLastError();
        case 8: launch_mfma_rows<8>(grid, vec16, stream, w, w_scale, x, x_scale, rows, k_words, batch, out, acc); return hipGetLastError();
        default: break;
    }
    if (i8_use_gemv(4 * (int64_t)k_words, batch)) {
        switch (gemv_form(4 * (int64_t)k_words)) {
            case kGemvNarrow:
                if (vec16)
                    launch_gemv_narrow<true>(grid, block, stream, w, w_scale, x, x_scale, rows, k_words, out, acc);
                else
                    launch_gemv_narrow<false>(grid, block, stream, w, w_scale, x, x_scale, rows, k_words, out, acc);
                break;
            case kGemvGrouped: {
                const int rpw = gemv_group_rows_per_wave(4 * (int64_t)k_words);
                if (gemv_group_log2_lanes(4 * (int64_t)k_words) == 5) {
                    if (vec16)
                        i8_gemv_grouped_kernel<true, 5, kGemvDepth><<<grid, block, 0, stream>>>(
                            w, w_scale, x, x_scale, rows, k_words, rpw, out, acc);
                    else
                        i8_gemv_grouped_kernel<false, 5, kGemvDepth><<<grid, block, 0, stream>>>(
                            w, w_scale, x, x_scale, rows, k_words, rpw, out, acc);
                } else {
                    if (vec16)
                        i8_gemv_grouped_kernel<true, 4, kGemvDepth><<<grid, block, 0, stream>>>(
                            w, w_scale, x, x_scale, rows, k_words, rpw, out, acc);
                    else
                        i8_gemv_grouped_kernel<false, 4, kGemvDepth><<<grid, block, 0, stream>>>(
                            w, w_scale, x, x_scale, rows, k_words, rpw, out, acc);
                }
                break;
            }
            case kGemvWide:
                if (!launch_gemv_wide(grid, block, stream, vec16, (int64_t)grid.x < rows, w, w_scale, x, x_scale,
                                      rows, k_words, out, acc))
                    return hipErrorInvalidConfiguration;
                break;
            default: {
                const int rpw = gemv_rows_per_wave(k_words);
                const bool full = k_words % (kWave * 4) == 0;
                if (full && vec16 && rpw == 1)
                    i8_gemv_kernel<true, true, kGemvDepth, true><<<grid, block, 0, stream>>>(
                        w, w_scale, x, x_scale, rows, k_words, rpw, out, acc);
                else if (full && vec16)
                    i8_gemv_kernel<true, true, kGemvDepth, false><<<grid, block, 0, stream>>>(
                        w, w_scale, x, x_scale, rows, k_words, rpw, out, acc);
                else if (full)
                    i8_gemv_kernel<true, false, kGemvDepth, false><<<grid, block, 0, stream>>>(
                        w, w_scale, x, x_scale, rows, k_words, rpw, out, acc);
                else if (vec16)
                    i8_gemv_kernel<false, true, kGemvDepth, false><<<grid, block, 0, stream>>>(
                        w, w_scale, x, x_scale, rows, k_words, rpw, out, acc);
                else
                    i8_gemv_kernel<false, false, kGemvDepth, false><<<grid, block, 0, stream>>>(
                        w, w_scale, x, x_scale, rows, k_words, rpw, out, acc);
                break;
            }
        }
    } else {
        const bool full = k_words % (16 * kMfmaSteps) == 0;
        bool launched;
        if (full && vec16)
            launched = launch_mfma<true, true>(grid, block, stream, w, w_scale, x, x_scale, rows, k_words, batch, out, acc);
        else if (vec16)
            launched = launch_mfma<false, true>(grid, block, stream, w, w_scale, x, x_scale, rows, k_words, batch, out,
                                                acc);
        else
            launched = launch_mfma<false, false>(grid, block, stream, w, w_scale, x, x_scale, rows, k_words, batch, out,
                                                 acc);
        if (!launched) return hipErrorInvalidConfiguration;
    }
    return hipGetLastError();
}

}  // namespace loom
