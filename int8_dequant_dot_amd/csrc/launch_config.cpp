// launch_config.cpp -- the launch-configuration "program" of every exported
// kernel ("Kernels and launch configuration": §A kernel owns two signatures,
// §Workload is not workgroup count, §Evaluate the compiled launch contract).
//
// Each kernel owns the map from its logical workload to a physical grid.  The
// table is evaluated by loom_launch_config_invoke for embeddings and by every
// entry point before it launches, so the host never repeats the arithmetic.
// Pure host code: nothing here touches the device.
#include <string.h>

#include "internal.hpp"

namespace loom {

namespace {

constexpr uint32_t kSubgroupSize = 64;             // gfx950 wave64

int set(loom_launch_config *c, int64_t workgroups, uint32_t workgroup_size, uint32_t storage) {
    // HIP launches a grid only while grid.x * block.x < 2^32 work-items
    if (workgroups < 0 || workgroups * (int64_t)workgroup_size > kMaxGridWorkItems) return LOOM_ERR_RANGE;
    c->workgroups[0] = (uint32_t)workgroups;
    c->workgroups[1] = 1;
    c->workgroups[2] = 1;
    c->workgroup_size[0] = workgroup_size;
    c->workgroup_size[1] = 1;
    c->workgroup_size[2] = 1;
    c->cluster_size[0] = c->cluster_size[1] = c->cluster_size[2] = 1;
    c->subgroup_size = kSubgroupSize;
    c->workgroup_storage_bytes = storage;
    return LOOM_OK;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int set2(loom_launch_config *c, int64_t gx, int64_t gy, uint32_t workgroup_size, uint32_t storage) {
    if (gy < 0 || gy > 0xFFFF) return LOOM_ERR_RANGE;
    const int st = set(c, gx, workgroup_size, storage);
    if (st == LOOM_OK) c->workgroups[1] = (uint32_t)gy;
    return st;
}

// copy_f32(n): one element per work-item, 256 per workgroup; 1009 -> 4.
int geo_copy(const int64_t *w, loom_launch_config *c) {
    if (w[0] < 0) return LOOM_ERR_RANGE;
    return set(c, ceil_div(w[0], 256), 256, 0);
}

// row_sum_tiles(count): one wave64 walks the whole tile.
int geo_row_sum_tiles(const int64_t *w, loom_launch_config *c) {
    if (w[0] < 0) return LOOM_ERR_RANGE;
    return set(c, 1, kSubgroupSize, 0);
}

// row_sums(rows, cols): narrow rows (1-128 columns) several to a record, one
// wave per kRowSumsNarrowRecords records; long rows (row_sums_waves_per_row > 0) one workgroup
// per row (each taking every grid.x-th row once the grid reaches 2^32
// work-items); the others one wave per block of kRowSumsTilesPerWave tiles of 8
// rows (the last tile the tail).
int geo_row_sums(const int64_t *w, loom_launch_config *c) {
    if (w[0] < 0 || w[1] < 0) return LOOM_ERR_RANGE;
    if (row_sums_narrow_log2_lanes(w[1]) >= 0)
        return set(c, ceil_div(w[0], row_sums_narrow_rows_per_wave(w[1])), kSubgroupSize, 0);
    if (const int waves = row_sums_waves_per_row(w[1]))  // LDS: the wave totals
        return set(c, grid_stride_groups(w[0], kSubgroupSize * waves), kSubgroupSize * waves,
                   4 * kRowSumsWideMaxWaves);
    return set(c, ceil_div(w[0], int64_t(kTileRows) * kRowSumsTilesPerWave), kSubgroupSize, 0);
}

// segment_sums(segments, cols, total_rows): one wave per segment -- or, for a
// few long segments, per part of a segment (segment_sums_parts), the parts
// grouped in workgroups of kSegmentRunWaves waves per run when there are
// runs (segment_sums_runs) -- and block of kSegmentBlockCols columns (at
// least one block, which also writes the segment's tail count when there are
// no columns); past the grid's work-item limit each workgroup takes every
// grid.x-th unit.  A split launch is followed by a pass of one workgroup per
// segment and block that adds the partials.
int geo_segment_sums(const int64_t *w, loom_launch_config *c) {
    if (w[0] < 0 || w[1] < 0 || w[2] < 0) return LOOM_ERR_RANGE;
    const int64_t blocks = w[1] > 0 ? ceil_div(w[1], kSegmentBlockCols) : 1;
    if (const int runs = segment_sums_runs(w[0], w[1], w[2])) {  // LDS: the run's part sums of one column block
        const int64_t size = kSubgroupSize * kSegmentRunWaves;
        return set2(c, grid_stride_groups(w[0] * runs, size), blocks, (uint32_t)size,
                    (uint32_t)(kSegmentRunWaves * kSegmentBlockCols * 4));
    }
    const int64_t units = w[0] * segment_sums_parts(w[0], w[1], w[2]);
    return set2(c, grid_stride_groups(units, kSubgroupSize), blocks, kSubgroupSize, 0);
}

// i8_dequant_dot(rows, k, batch): for one vector, by gemv_form(k), one wave
// per gemv_narrow_rows_per_wave(k), gemv_group_rows_per_wave(k) or
// gemv_rows_per_wave(k) rows, or one workgroup of gemv_wide_waves(k) waves per
// long row; for 9 to 16 vectors and k a multiple of 1024
// from 4096 to 8192, one 16-wave workgroup per CU (at most one per 16-row
// tile) that walks the tiles; for more than 16 vectors, one workgroup per
// i8_cols_tile_rows rows with one wave per 16-vector column tile (LDS: two
// record slots of 256 bytes per row); otherwise one workgroup per
// 16-row matrix-core tile whose mfma_ksplit(k, rows) waves split k (the LDS
// holds their partial sums: for the segment-paired kernel (mfma_seg), its
// 16 x 4 or 16 x 8 per wave; otherwise the partial accumulator tiles and the
// weight staging tiles).
int geo_i8(const int64_t *w, loom_launch_config *c) {
    if (w[0] < 0 || w[1] < 0 || w[2] < 1) return LOOM_ERR_RANGE;
    if (i8_use_gemv(w[1], w[2])) {
        switch (gemv_form(w[1])) {
            case kGemvNarrow: return set(c, ceil_div(w[0], gemv_narrow_rows_per_wave(w[1])), kSubgroupSize, 0);
            case kGemvRows: return set(c, ceil_div(w[0], gemv_rows_per_wave(w[1] / 4)), kSubgroupSize, 0);
            case kGemvGrouped: return set(c, ceil_div(w[0], gemv_group_rows_per_wave(w[1])), kSubgroupSize, 0);
            default: {  // LDS: the wave totals
                const int waves = gemv_wide_waves(w[1]);
                const int64_t size = kSubgroupSize * waves;
                return set(c, grid_stride_groups(w[0], size), (uint32_t)size, 4u * (uint32_t)waves);
            }
        }
    }
    if (const int chunks = i8_rows_chunks(w[0], w[1], w[2])) {
        const int64_t tiles = ceil_div(w[0], kMfmaTileRows);
        return set(c, tiles < kI8RowsGroups ? tiles : kI8RowsGroups, kSubgroupSize * kI8RowsWaves,
                   i8_rows_lds_bytes(chunks));
    }
    if (w[2] > 16)
        return set(c, ceil_div(w[0], i8_cols_tile_rows(w[0])), kSubgroupSize * mfma_col_tiles(w[2]),
                   i8_cols_lds_bytes(w[0]));
    const int ks = mfma_ksplit(w[1], w[0]);
    if (mfma_seg(w[1], w[0], w[2]))
        return set(c, ceil_div(w[0], kMfmaTileRows), kSubgroupSize * ks, mfma_seg_lds_bytes(ks, w[2]));
    return set(c, ceil_div(w[0], kMfmaTileRows), kSubgroupSize * ks,
               (ks - 1) * 4 * kSubgroupSize * 4 + (kMfmaStage ? ks * kMfmaStageBytes : 0));
}

// packed_dot(outputs, count, streams): 256 lanes per workgroup, one output
// per lane, or several for large output counts (see
// packed_dot_outputs_per_lane).
int geo_packed_dot(const int64_t *w, loom_launch_config *c) {
    if (w[0] < 0 || w[1] < 0 || w[2] < 1) return LOOM_ERR_RANGE;
    return set(c, ceil_div(w[0], 256 * packed_dot_outputs_per_lane(w[0], w[2])), 256, 0);
}

// sum_guarded_rows(count): one workgroup of 32 work-items, one per tile lane.
int geo_sum_guarded_rows(const int64_t *w, loom_launch_config *c) {
    if (w[0] < 0) return LOOM_ERR_RANGE;
    return set(c, 1, 32, 0);
}

// routed_combine(tokens, routes, hidden): one wave per token and column block
// (past 2^26 - 1 tokens, each wave takes every grid.x-th token).
int geo_routed_combine(const int64_t *w, loom_launch_config *c) {
    if (w[0] < 0 || w[1] < 0 || w[2] < 0) return LOOM_ERR_RANGE;
    return set2(c, grid_stride_groups(w[0], kSubgroupSize), ceil_div(w[2], kRoutedColumnsPerWave), kSubgroupSize,
                0);
}

struct Export {
    const char *name;
    size_t arity;
    int (*geometry)(const int64_t *, loom_launch_config *);
};

const Export kExports[kExportCount] = {
    {"copy_f32", 1, geo_copy},
    {"row_sum_tiles", 1, geo_row_sum_tiles},
    {"row_sums", 2, geo_row_sums},
    {"segment_sums", 3, geo_segment_sums},
    {"i8_dequant_dot", 3, geo_i8},
    {"packed_dot", 3, geo_packed_dot},
    {"sum_guarded_rows", 1, geo_sum_guarded_rows},
    {"routed_combine", 3, geo_routed_combine},
};

}  // namespace

int evaluate_launch(ExportId id, const int64_t *workload, loom_launch_config *out) {
    return kExports[id].geometry(workload, out);
}

}  // namespace loom

extern "C" int loom_launch_config_lookup(const char *export_name, uint32_t *token) {
    if (!export_name || !token) return LOOM_ERR_NULL;
    for (uint32_t i = 0; i < loom::kExportCount; ++i)
        if (strcmp(export_name, loom::kExports[i].name) == 0) {
            *token = i + 1;  // 0 is never a valid token
            return LOOM_OK;
        }
    return LOOM_ERR_UNKNOWN_EXPORT;
}

extern "C" int loom_launch_config_invoke(uint32_t token, const uint64_t *workload_bits, size_t workload_count,
                                         loom_launch_config *out) {
    if (!out || (!workload_bits && workload_count)) return LOOM_ERR_NULL;
    if (token == 0 || token > loom::kExportCount) return LOOM_ERR_TOKEN;
    const loom::Export &e = loom::kExports[token - 1];
    if (workload_count != e.arity) return LOOM_ERR_TOKEN;
    int64_t w[4];
    for (size_t i = 0; i < workload_count; ++i) memcpy(&w[i], &workload_bits[i], sizeof(int64_t));
    loom_launch_config tmp;
    const int st = e.geometry(w, &tmp);
    if (st == LOOM_OK) *out = tmp;
    return st;
}
