// internal.hpp -- declarations shared by the C ABI, the launch-configuration
// table and the kernel launchers.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "loom.h"

namespace loom {

enum ExportId : uint32_t {
    kCopyF32 = 0,
    kRowSumTiles,
    kRowSums,
    kSegmentSums,
    kI8DequantDot,
    kPackedDot,
    kSumGuardedRows,
    kRoutedCombine,
    kExportCount
};

// Launch geometry owned by each kernel (LAUNCH §A kernel owns two signatures).
// `workload` holds the export's workload arguments; returns a loom_status.
int evaluate_launch(ExportId id, const int64_t *workload, loom_launch_config *out);

// HIP launches a grid only while grid.x * block.x stays below 2^32 work-items.
constexpr int64_t kMaxGridWorkItems = (int64_t(1) << 32) - 1;
// Workgroups of a grid-stride launch over `units` (workgroup b takes units
// b, b + grid.x, ...): one per unit up to the work-item limit.
constexpr int64_t grid_stride_groups(int64_t units, int64_t workgroup_size) {
    return units < kMaxGridWorkItems / workgroup_size ? units : kMaxGridWorkItems / workgroup_size;
}

// Rows per full tile ("Tune loop unrolling and pipelining", §Derive full
// tiles from a ragged loop).
constexpr int kTileRows = 8;
// Consecutive tiles one row-sum wave streams (its read-ahead crosses them).
#ifndef LOOM_ROW_SUMS_TILES_PER_WAVE
#define LOOM_ROW_SUMS_TILES_PER_WAVE 2  // 16 short rows per wave
#endif
constexpr int kRowSumsTilesPerWave = LOOM_ROW_SUMS_TILES_PER_WAVE;
static_assert(kTileRows * kRowSumsTilesPerWave <= 64, "one lane per row of a wave's block");
// Rows of 1 to kRowSumsNarrowMaxCols floats are packed several to a record:
// returns log2 of the lanes per row (the smallest power of two L with
// 4 L >= cols), or -1 for wider (or empty) rows.  A narrow wave streams
// kRowSumsNarrowRecords records of 64 / L rows each.
#ifndef LOOM_ROW_SUMS_NARROW_MAX_COLS
#define LOOM_ROW_SUMS_NARROW_MAX_COLS 128
#endif
#ifndef LOOM_ROW_SUMS_NARROW_RECORDS
#define LOOM_ROW_SUMS_NARROW_RECORDS 8
#endif
constexpr int kRowSumsNarrowRecords = LOOM_ROW_SUMS_NARROW_RECORDS;
constexpr int row_sums_narrow_log2_lanes(int64_t cols) {
    if (cols < 1 || cols > LOOM_ROW_SUMS_NARROW_MAX_COLS) return -1;
    int k = 0;
    while ((int64_t(4) << k) < cols) ++k;
    return k;
}
constexpr int64_t row_sums_narrow_rows_per_wave(int64_t cols) {
    return int64_t(64 >> row_sums_narrow_log2_lanes(cols)) * kRowSumsNarrowRecords;
}

// Rows of at least LOOM_ROW_SUMS_WIDE_RECORDS 256-float records (1 KiB each)
// get a workgroup of their own: one wave per LOOM_ROW_SUMS_WIDE_RECORDS
// records, at most kRowSumsWideMaxWaves (4 waves of 4 KiB for 4096 columns).
// Shorter rows keep the wave-per-8-tiles kernel.  Returns the waves per row,
// or 0 for the tiled kernel.
#ifndef LOOM_ROW_SUMS_WIDE_RECORDS
#define LOOM_ROW_SUMS_WIDE_RECORDS 4
#endif
constexpr int kRowSumsWideMaxWaves = 16;
constexpr int row_sums_waves_per_row(int64_t cols) {
    const int64_t records = (cols + 255) / 256;
    if (records < LOOM_ROW_SUMS_WIDE_RECORDS) return 0;
    const int64_t w = records / LOOM_ROW_SUMS_WIDE_RECORDS;
    return w > kRowSumsWideMaxWaves ? kRowSumsWideMaxWaves : (int)w;
}

// Columns of one segment-sum wave: a segment of a wider matrix is spread over
// ceil(cols / kSegmentBlockCols) waves (a 1 KiB record per row each).
constexpr int kSegmentBlockCols = 256;
// Few long segments.  A launch of fewer than kSegmentSplitMinWaves waves
// (segments x column blocks) whose segments average at least
// 2 * kSegmentSplitMinRows rows splits every segment into P contiguous parts
// of at least kSegmentSplitMinRows rows on average, P * waves at most
// kSegmentSplitWaves: each part is summed in row order into a partial, and a
// second pass adds each segment's partials in a fixed order (contiguous
// groups of partials in order, then the groups in group order; one
// kSegmentCombineWaves-wave workgroup per segment and column block).  The
// partials need at most segments * P * cols floats, at most
// kSegmentSplitWaves * 256 (4 MiB).  Returns P, or 1 for the single pass
// (every column's sum in row order).  Over 4 GiB of 256-column rows (one
// MI355X), the single pass took 75.4 ms for one segment, 19.0 ms for 4,
// 1366 us for 64, 704 us for 160 and 606 us for 200 segments; split, 681,
// 650, 652, 657 and 637 us.
#ifndef LOOM_SEGMENT_SPLIT_MIN_WAVES
#define LOOM_SEGMENT_SPLIT_MIN_WAVES 192
#endif
constexpr int64_t kSegmentSplitMinWaves = LOOM_SEGMENT_SPLIT_MIN_WAVES;
constexpr int kSegmentCombineWaves = 16;
constexpr int64_t kSegmentSplitWaves = 4096;
constexpr int64_t kSegmentSplitMinRows = 512;
constexpr int64_t kSegmentSplitMaxBytes = kSegmentSplitWaves * kSegmentBlockCols * 4;
// Runs.  Rows of at most kSegmentRunMaxCols columns split into at least
// 2 * kSegmentRunWaves parts take P a multiple of kSegmentRunWaves and group
// the parts in runs of kSegmentRunWaves consecutive parts, one workgroup per
// run whose waves add their part sums in part order through LDS: the
// partials (and the second pass's reads) shrink to one run sum per run, a
// single segment of 4 M rows leaving 512 KiB for one CU to add instead of
// 4 MiB.  Over 4 GiB (one MI355X), runs of 8 took 643 us for one 256-column
// segment (689 us without), 641 us for 4 (659), 640 us for 128 (648) and
// 642 us for one 512-column segment (669); on 1024-column rows they lost
// (676 vs 640 us for one segment, 696 vs 654 for 16), as did runs of 16
// there, so wider rows keep one partial per part.
#ifndef LOOM_SEGMENT_RUN_WAVES
#define LOOM_SEGMENT_RUN_WAVES 8
#endif
constexpr int kSegmentRunWaves = LOOM_SEGMENT_RUN_WAVES;
constexpr int64_t kSegmentRunMaxCols = 2 * kSegmentBlockCols;
constexpr bool segment_runs_fit(int64_t p, int64_t cols) {
    return kSegmentRunWaves > 1 && cols <= kSegmentRunMaxCols && p >= 2 * kSegmentRunWaves;
}
constexpr int segment_sums_parts(int64_t segments, int64_t cols, int64_t total_rows) {
    const int64_t blocks = cols > 0 ? (cols + kSegmentBlockCols - 1) / kSegmentBlockCols : 1;
    if (segments <= 0 || cols <= 0 || segments * blocks >= kSegmentSplitMinWaves) return 1;
    const int64_t by_waves = kSegmentSplitWaves / (segments * blocks);
    const int64_t by_rows = total_rows / segments / kSegmentSplitMinRows;
    int64_t p = by_waves < by_rows ? by_waves : by_rows;
    if (segment_runs_fit(p, cols)) p -= p % kSegmentRunWaves;  // whole runs
    return p >= 2 ? (int)p : 1;
}
// Runs per segment of a split launch (0: no runs, one partial per part).
constexpr int segment_sums_runs(int64_t segments, int64_t cols, int64_t total_rows) {
    const int p = segment_sums_parts(segments, cols, total_rows);
    return segment_runs_fit(p, cols) ? p / kSegmentRunWaves : 0;
}
// Partial sums per segment that the second pass adds: one per run, else one
// per part.
constexpr int segment_sums_partials(int64_t segments, int64_t cols, int64_t total_rows) {
    const int r = segment_sums_runs(segments, cols, total_rows);
    return r > 0 ? r : segment_sums_parts(segments, cols, total_rows);
}
// Many long segments of uneven length: a single pass over at least
// kSegmentOrderMinFloats floats of 2 to kSegmentOrderMaxSegments segments
// averaging at least kSegmentOrderMinRows rows first sorts the segments by
// length into coarse buckets (one workgroup, a counting sort, 5-11 us) and
// its waves take them longest first, so the launch ends on short segments
// instead of a few long ones running nearly alone.  Every column's sum is
// still the in-order recurrence: only which wave takes which segment
// changes.  Back to back, index order -> longest first, segments of
// U{0..max} rows: 16384 x max 4096 x 256 columns 5085 -> 5008 us, 4096 x 4096
// x 256 1390 -> 1311 us, 2048 x 4096 x 256 752 -> 674 us, 1000 x 20000 x 64
// 820 -> 637 us, 4096 x 2048 x 16 182 -> 171 us; with short segments the
// order pass costs more than it saves (16384 x 512 x 256 693 -> 707 us,
// 3000 x 200 x 256 56 -> 64 us).  Past kSegmentOrderMaxSegments every wave
// takes many segments and index order balances well enough.
constexpr int64_t kSegmentOrderMaxSegments = int64_t(1) << 15;
constexpr int64_t kSegmentOrderMinRows = 512;
#ifndef LOOM_SEGMENT_ORDER_MIN_FLOATS
#define LOOM_SEGMENT_ORDER_MIN_FLOATS (int64_t(1) << 26)
#endif
constexpr int64_t kSegmentOrderMinFloats = LOOM_SEGMENT_ORDER_MIN_FLOATS;
constexpr bool segment_sums_ordered(int64_t segments, int64_t cols, int64_t total_rows) {
    return segment_sums_parts(segments, cols, total_rows) == 1 && segments >= 2 &&
           segments <= kSegmentOrderMaxSegments && cols > 0 && total_rows / segments >= kSegmentOrderMinRows &&
           total_rows * cols >= kSegmentOrderMinFloats;
}
// Device memory a launch needs beyond its inputs and outputs: the partials of
// a split launch, or the order index of a longest-first one (at most
// kSegmentSplitMaxBytes either way).
constexpr int64_t segment_sums_workspace_bytes(int64_t segments, int64_t cols, int64_t total_rows) {
    const int p = segment_sums_parts(segments, cols, total_rows);
    return p > 1 ? segments * segment_sums_partials(segments, cols, total_rows) * cols * 4
                 : segment_sums_ordered(segments, cols, total_rows) ? segments * 4 : 0;
}

// Blocking of the int8 kernels.  One vector always runs a v_dot4 GEMV, in
// one of four forms by row length k (bytes):
//   narrow   k <= LOOM_GEMV_NARROW_MAX_K: several rows packed into each 1 KiB
//            record, a wave per gemv_narrow_rows_per_wave(k) rows;
//   grouped  other k below LOOM_GEMV_GROUPED_MAX_K that is not a multiple of
//            1024: records of 2 rows x 512 B (k a multiple of 512) or 4 rows x
//            256 B, so that the pieces of a row fill its records, a wave per
//            gemv_group_rows_per_wave(k) rows;
//   rows     any other k: a wave per gemv_rows_per_wave(k) consecutive rows
//            (about 8 KiB), read row by row in 1 KiB records (the last one of
//            a row partly filled when k is not a multiple of 1024: a small
//            share of such long rows);
//   wide     k a multiple of 1024 from LOOM_GEMV_WIDE_MIN_K to
//            LOOM_GEMV_WIDE_MAX_K, and k a multiple of 16 (not of 1024)
//            above LOOM_GEMV_WIDE_PARTIAL_MIN_K and below
//            LOOM_GEMV_GROUPED_MAX_K: a workgroup per row of
//            gemv_wide_waves(k) waves, each reading 2 KiB of the row (the
//            row's last record partly empty).
// Over 128 MiB of weights (one MI355X, back-to-back launches) each form was
// kept where it measured fastest: rows of 768 to 8704 bytes that are not whole
// 1 KiB records took 21.0-23.0 us grouped against 23.1-24.5 us in 1 KiB
// records per row or on the matrix cores; from 12288 bytes the partly filled
// record costs less than pairs of 512-byte pieces (k = 12800: 23.5 against
// 23.9 us); a workgroup per row won only at 6-8 KiB rows (k = 6144:
// 20.5 against 20.9 us; k = 4096: 22.2 against 20.7; k = 10240: 22.0 against
// 21.1).  For rows that are not whole records, a workgroup per row with the
// last record partly empty beat the grouped form from 3.25 to 11.5 KiB
// (k = 3328 / 4608 / 7680 / 11008 / 11776: 22.2 / 21.6 / 21.1 / 22.0 /
// 22.4 against 22.9 / 22.7 / 23.4 / 30.9 / 22.8 us; the grouped form gave a
// 11008-byte row only 3048 waves of 4 rows each) and tied at 12800.
// Several vectors run an int8 MFMA kernel: one 16-row matrix-core tile per
// workgroup, whose KSPLIT waves split the k range and combine their int32
// partials through LDS in wave order (exact).  Tuning builds may override the
// macros.
#ifndef LOOM_GEMV_WAVE_BYTES
#define LOOM_GEMV_WAVE_BYTES 8192  // rows and grouped forms: about 8 KiB of weights per wave
#endif
#ifndef LOOM_GEMV_NARROW_MAX_K
#define LOOM_GEMV_NARROW_MAX_K 512
#endif
#ifndef LOOM_GEMV_GROUPED_MAX_K
#define LOOM_GEMV_GROUPED_MAX_K 12288
#endif
#ifndef LOOM_GEMV_WIDE_MIN_K
#define LOOM_GEMV_WIDE_MIN_K 6144
#endif
#ifndef LOOM_GEMV_WIDE_MAX_K
#define LOOM_GEMV_WIDE_MAX_K 8192
#endif
#ifndef LOOM_GEMV_WIDE_PARTIAL_MIN_K
#define LOOM_GEMV_WIDE_PARTIAL_MIN_K 3072
#endif
// the wide form: two 1 KiB records per wave, instantiated for 2 to 6 waves
constexpr int kGemvWideRecords = 2;
constexpr int kGemvWideMaxWaves = 6;
static_assert(LOOM_GEMV_WIDE_MIN_K > 2048 && LOOM_GEMV_WIDE_MAX_K <= 12288 && LOOM_GEMV_WIDE_PARTIAL_MIN_K >= 2048 &&
                  LOOM_GEMV_GROUPED_MAX_K <= 12288,
              "wide GEMV rows of 3 to 12 records: 2 to 6 waves");
enum GemvForm : int { kGemvNarrow = 0, kGemvRows = 1, kGemvWide = 2, kGemvGrouped = 3 };
constexpr GemvForm gemv_form(int64_t k) {
#ifdef LOOM_GEMV_FORCE_FORM
    if (LOOM_GEMV_FORCE_FORM >= 0 && k > LOOM_GEMV_NARROW_MAX_K &&
        (LOOM_GEMV_FORCE_FORM == kGemvGrouped || k % 1024 == 0))
        return (GemvForm)LOOM_GEMV_FORCE_FORM;
#endif
    return k <= LOOM_GEMV_NARROW_MAX_K ? kGemvNarrow
           : k % 1024 != 0 && k % 16 == 0 && k > LOOM_GEMV_WIDE_PARTIAL_MIN_K && k < LOOM_GEMV_GROUPED_MAX_K
               ? kGemvWide
           : k % 1024 != 0 && k < LOOM_GEMV_GROUPED_MAX_K                               ? kGemvGrouped
           : k % 1024 == 0 && k >= LOOM_GEMV_WIDE_MIN_K && k <= LOOM_GEMV_WIDE_MAX_K ? kGemvWide
                                                                                        : kGemvRows;
}
constexpr int gemv_wide_waves(int64_t k) {
    const int64_t records = (k + 1023) / 1024;
    const int64_t wv = (records + kGemvWideRecords - 1) / kGemvWideRecords;
    return wv < 1 ? 1 : wv > kGemvWideMaxWaves ? kGemvWideMaxWaves : (int)wv;
}
constexpr bool i8_use_gemv(int64_t k, int64_t batch) { return batch == 1 && k >= 0; }
// grouped form: log2 of the lanes per row (32 when k is a multiple of 512,
// else 16) and the rows of a wave, whole groups of 64 / L rows of about
// LOOM_GEMV_WAVE_BYTES together, at most 64
constexpr int gemv_group_log2_lanes(int64_t k) { return k % 512 == 0 ? 5 : 4; }
constexpr int gemv_group_rows_per_wave(int64_t k) {
    const int64_t r = int64_t(64) >> gemv_group_log2_lanes(k);
    int64_t g = k > 0 ? LOOM_GEMV_WAVE_BYTES / (r * k) : 1;
    g = g < 1 ? 1 : g > 64 / r ? 64 / r : g;
    return (int)(g * r);
}
constexpr int gemv_rows_per_wave(int64_t k_words) {
    const int64_t r = k_words > 0 ? LOOM_GEMV_WAVE_BYTES / (4 * k_words) : 64;
    return r < 1 ? 1 : r > 64 ? 64 : (int)r;
}
// narrow form: log2 of the lanes per row, the smallest L with 4 L >= k_words
// (at most 32 lanes, so at least two rows per record), and the rows of a
// wave: whole records (64 / L rows each) of about LOOM_GEMV_WAVE_BYTES, at
// most 64 rows
constexpr int gemv_narrow_log2_lanes(int64_t k_words) {
    int l = 0;
    while ((int64_t(4) << l) < k_words) ++l;
    return l;
}
constexpr int gemv_narrow_rows_per_wave(int64_t k) {
    const int64_t r = int64_t(64) >> gemv_narrow_log2_lanes(k / 4);
    const int64_t rec = k > 0 ? LOOM_GEMV_WAVE_BYTES / (r * k) : 64;
    const int64_t rows = r * (rec < 1 ? 1 : rec);
    return rows > 64 ? 64 : (int)rows;
}
// Waves per 16-row tile of the tile kernel, each taking a contiguous 1/KS of
// k: about 2 KiB of every row per wave.  Over ~224 MiB of weights with 2 and
// 8 vectors, the best split was 1 wave up to k = 2048 (k = 512: 41-47 us
// against 69-72 with 4 waves), 2 at k = 4096, 4 at k = 8192 and 8 at
// k = 16384 (41-44 against 44-47 us); with fewer than 512 tiles, 8-wave
// workgroups leave CUs unevenly loaded (k = 32768, 7168 rows: 57 against 42 us
// with 4).
constexpr int mfma_ksplit(int64_t k, int64_t rows) {
    const int64_t tiles = (rows + 15) / 16;
    if (k >= 16384 && tiles >= 512) return 8;
    return k >= 8192 ? 4 : k >= 4096 ? 2 : 1;
}
#ifndef LOOM_MFMA_STAGE
#define LOOM_MFMA_STAGE 1     // weights reach the MFMA through a per-wave LDS tile
#endif
constexpr int kMfmaTileRows = 16;
// The segment-paired kernel (no LDS staging; LDS holds only its waves'
// partial sums: KS x 16 rows x 4 or 8 vector slots) takes 7 or 8 vectors, and
// 2 to 8 when 8 waves split k.  Measured against the LDS-staged tile kernel
// over 224 MiB of weights (one MI355X, the same bits): 8 vectors at k = 8192
// 35.5 against 36.0 us, at k = 16384 39.2 against 41.8; 2 to 5 vectors at
// k = 16384 37.1-38.0 against 38.8-39.7; 7 vectors at k = 4096 and 8192
// 36.5 / 35.4 against 36.7 / 35.6; but 2 to 6 vectors at k = 2048 to 8192
// 34.4-36.2 on the tile kernel against 34.9-37.7.
#ifndef LOOM_MFMA_SEG_MIN_BATCH
#define LOOM_MFMA_SEG_MIN_BATCH 7
#endif
#ifndef LOOM_MFMA_SEG_MAX_BATCH
#define LOOM_MFMA_SEG_MAX_BATCH 8
#endif
constexpr int kMfmaSegMaxBatch = LOOM_MFMA_SEG_MAX_BATCH;
static_assert(kMfmaSegMaxBatch <= 8, "the segment-paired kernel has two vector groups of 4");
constexpr bool mfma_seg(int64_t k, int64_t rows, int64_t batch) {
    return batch <= kMfmaSegMaxBatch && (batch >= LOOM_MFMA_SEG_MIN_BATCH || mfma_ksplit(k, rows) == 8);
}
constexpr uint32_t mfma_seg_lds_bytes(int ks, int64_t batch) { return (uint32_t)ks * 16u * (batch > 4 ? 8u : 4u) * 4u; }
constexpr bool kMfmaStage = LOOM_MFMA_STAGE != 0;
constexpr uint32_t kMfmaStageBytes = 16 * 256;  // per wave: 16 rows x 256 B
// Outputs per lane of the packed-dot recurrence: kPackedDotWide, spaced one
// wave apart, once there are enough outputs to fill the GPU and the stream
// count divides the wave width (every output of a lane then reads the same
// stream); otherwise 1 (the pages' one lane per output, best for the
// latency-bound small shapes).
#ifndef LOOM_PACKED_DOT_WIDE_MIN
#define LOOM_PACKED_DOT_WIDE_MIN 65536
#endif
#ifndef LOOM_PACKED_DOT_WIDE
#define LOOM_PACKED_DOT_WIDE 4
#endif
constexpr int kPackedDotWide = LOOM_PACKED_DOT_WIDE;
constexpr int packed_dot_outputs_per_lane(int64_t outputs, int64_t streams) {
    return (outputs >= LOOM_PACKED_DOT_WIDE_MIN && 64 % streams == 0) ? kPackedDotWide : 1;
}

// Columns of the routed combine per wave (a multiple of 256: 1 KiB slices of
// each selected row).
#ifndef LOOM_ROUTED_COLUMNS
#define LOOM_ROUTED_COLUMNS 1024  // a whole 4 KiB row of the workloads per route: 25% faster than 1 KiB slices
#endif
constexpr int kRoutedColumnsPerWave = LOOM_ROUTED_COLUMNS;

// 16-vector column tiles the MFMA kernels use for a batch: one up to 16
// vectors, else four (17-32 vectors leave some zeroed: at 28672 x 8192 x 32
// the four-tile kernel took 40.3 us against 44.1 us with two tiles of 64-row
// workgroups).
constexpr int mfma_col_tiles(int64_t batch) { return batch <= 16 ? 1 : 4; }

// The column-tile kernel (more than 16 vectors): a workgroup of 4 waves, one
// per 16-vector column tile, owns row_tiles 16-row tiles; each wave multiplies
// all of them by its column tile, so every vector fragment it loads serves
// row_tiles tiles.  The row tiles are shared evenly between q workgroups per
// CU, q = ceil(tiles / (256 * 8)), so that no CU gets a workgroup more than
// another (8 row tiles per wave at most).  At 64 vectors and k = 8192, 28672
// rows (7 tiles per wave, 256 workgroups) took 48.1 us against 56.0 us with 4
// tiles per wave (448 workgroups), 40960 rows (5 tiles, 512 workgroups) 64.3
// against 81.1 us, 57344 rows (7 tiles, 512 workgroups) 85.3 against 108.4 us.
constexpr int kI8ColsMaxRowTiles = 8;
constexpr int64_t kI8ColsCUs = 256;  // an MI355X has 256 CUs
constexpr int i8_cols_row_tiles(int64_t rows) {
    const int64_t tiles = (rows + 15) / 16;
    if (tiles <= 0) return 1;
    const int64_t per_cu = (tiles + kI8ColsCUs * kI8ColsMaxRowTiles - 1) / (kI8ColsCUs * kI8ColsMaxRowTiles);
    return (int)((tiles + kI8ColsCUs * per_cu - 1) / (kI8ColsCUs * per_cu));
}
constexpr int i8_cols_tile_rows(int64_t rows) { return 16 * i8_cols_row_tiles(rows); }
// LDS: two record slots of tile_rows rows x 256 bytes.
constexpr uint32_t i8_cols_lds_bytes(int64_t rows) { return 2u * 256u * (uint32_t)i8_cols_tile_rows(rows); }

// The row-streaming MFMA kernel: one workgroup of 16 waves per CU (an MI355X
// has 256) walks 16-row tiles, each wave streaming one whole row per tile
// into LDS.  It serves batches of 9 to 16 vectors when k is a multiple of
// 1024 from 4096 to 8192 (4 to 8 chunks of 1 KiB per row).  There the
// tile-per-workgroup kernel above slows down as the batch grows (at k = 8192:
// 42.8 against 37.4 us for 16 vectors), while below 9 vectors the two are
// within a few percent and below k = 4096 the short rows leave the row kernel
// waiting on its two barriers per tile (k = 1024: 65 against 48-57 us).
// LDS: the 16-row tile and the 16 waves' int32 partial tiles.
#ifndef LOOM_I8_ROWS_MIN_BATCH
#define LOOM_I8_ROWS_MIN_BATCH 9
#endif
constexpr int kI8RowsWaves = 16;
constexpr int kI8RowsGroups = 256;
#ifndef LOOM_I8_ROWS_MIN_CHUNKS
#define LOOM_I8_ROWS_MIN_CHUNKS 4
#endif
constexpr int kI8RowsMaxChunks = 8;
constexpr int i8_rows_chunks(int64_t rows, int64_t k, int64_t batch) {
    return (batch >= LOOM_I8_ROWS_MIN_BATCH && batch <= 16 && rows >= 16 && k % 1024 == 0 &&
            k >= 1024 * LOOM_I8_ROWS_MIN_CHUNKS && k <= 1024 * kI8RowsMaxChunks)
               ? (int)(k / 1024)
               : 0;
}
constexpr uint32_t i8_rows_lds_bytes(int chunks) {
    return 16u * 1024u * (uint32_t)chunks + (uint32_t)kI8RowsWaves * 4u * 64u * 4u;
}
constexpr int kMaxBatch = 64;
constexpr int64_t kMaxK = 131068;

// Kernel launchers.  Arguments are already validated; geometry comes from
// evaluate_launch.  Each returns the HIP launch status.
hipError_t launch_copy_f32(const loom_launch_config &cfg, const float *in, float *out, int64_t n,
                           hipStream_t stream);
hipError_t launch_row_sum_tiles(const loom_launch_config &cfg, const float *values, int count,
                                const float *initial, float *sums, int32_t *final_row,
                                int32_t *tail_count, hipStream_t stream);
hipError_t launch_row_sums(const loom_launch_config &cfg, const float *x, int rows, int cols,
                           int64_t row_stride, float *out, hipStream_t stream);
// The current device's address of the library's static workspace array
// (kSegmentSplitMaxBytes), looked up on the first call on each device.
hipError_t segment_scratch(void **ptr);
// workspace: segment_sums_workspace_bytes of device memory (NULL when that is
// 0); cfg must be the geometry evaluate_launch gives for the same workload.
hipError_t launch_segment_sums(const loom_launch_config &cfg, const float *x, int64_t total_rows,
                               const int64_t *offsets, int64_t segments, int cols, float *out,
                               int32_t *tail_counts, void *workspace, hipStream_t stream);
hipError_t launch_i8_dequant_dot(const loom_launch_config &cfg, const int32_t *w, const float *w_scale,
                                 const int32_t *x, const float *x_scale, int rows, int k_words,
                                 int batch, float *out, int32_t *acc, hipStream_t stream);

hipError_t launch_packed_dot(const loom_launch_config &cfg, const int32_t *fields, const uint16_t *scales,
                             const float *rhs, int streams, const float *initial, int count, int64_t outputs,
                             float *out, hipStream_t stream);

hipError_t launch_sum_guarded_rows(const loom_launch_config &cfg, const float *values, int count, int columns,
                                   int active_lanes, float *sums, hipStream_t stream);

hipError_t launch_routed_combine(const loom_launch_config &cfg, const int32_t *ids, const float *weights,
                                 const float *payload, int64_t num_rows, int64_t tokens, int routes, int hidden,
                                 float *out, hipStream_t stream);

}  // namespace loom
