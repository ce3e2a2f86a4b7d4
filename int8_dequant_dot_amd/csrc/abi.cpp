// abi.cpp -- the extern "C" entry points declared in include/loom.h.
//
// Every entry point validates its arguments on the host (sizes, then
// pointers, then alignment), evaluates its kernel's launch configuration
// through the same table embeddings use, and enqueues the kernel on the
// caller's stream.  Nothing is launched when there is nothing to compute or
// when a check fails.
#include <stdint.h>

#include "internal.hpp"

namespace {

bool misaligned(const void *p, uintptr_t a) { return p && (reinterpret_cast<uintptr_t>(p) % a) != 0; }

// Runs a kernel launcher and maps its result.  The thread's last HIP error
// is cleared first, so LOOM_ERR_DEVICE reports this launch only, not an
// error some earlier, unrelated HIP call left behind.
template <typename Launch>
int launch(Launch &&f) {
    (void)hipGetLastError();
    return f() == hipSuccess ? LOOM_OK : LOOM_ERR_DEVICE;
}

constexpr int64_t kMaxRows = 0x7FFFFFFF;        // row / segment counts index a 1-D grid
constexpr int64_t kMaxTileRows = int64_t(1) << 26;
constexpr int64_t kMaxTotalRows = int64_t(1) << 40;
constexpr int64_t kMaxSegmentCols = int64_t(1) << 20;
constexpr int64_t kMaxCopy = (int64_t(1) << 32) - 256;  // one work-item per element, below 2^32 work-items
constexpr int64_t kMaxOutputs = int64_t(0x7FFFFFFF) * 255;

}  // namespace

extern "C" const char *loom_status_string(int status) {
    switch (status) {
        case LOOM_OK: return "ok";
        case LOOM_ERR_NULL: return "a required pointer is NULL";
        case LOOM_ERR_RANGE: return "a size or count is outside its documented range";
        case LOOM_ERR_ALIGN: return "a pointer or stride is not aligned as documented";
        case LOOM_ERR_SHAPE: return "inconsistent shape";
        case LOOM_ERR_UNKNOWN_EXPORT: return "no kernel exports this name";
        case LOOM_ERR_TOKEN: return "invalid launch-config token or workload arity";
        case LOOM_ERR_DEVICE: return "the HIP runtime refused the launch";
        default: return "unknown status";
    }
}

extern "C" int loom_version(void) { return 100; }

extern "C" int loom_copy_f32(const float *in, float *out, int64_t n, void *stream) {
    if (n < 0 || n > kMaxCopy) return LOOM_ERR_RANGE;
    loom_launch_config cfg;
    const int64_t w[1] = {n};
    if (int st = loom::evaluate_launch(loom::kCopyF32, w, &cfg)) return st;
    if (n == 0) return LOOM_OK;
    if (!in || !out) return LOOM_ERR_NULL;
    if (misaligned(in, 4) || misaligned(out, 4)) return LOOM_ERR_ALIGN;
    return launch([&] { return loom::launch_copy_f32(cfg, in, out, n, (hipStream_t)stream); });
}

extern "C" int loom_row_sum_tiles(const float *values, int64_t rows_alloc, int64_t count, const float *initial,
                                  float *sums, int32_t *final_row, int32_t *tail_count, void *stream) {
    if (rows_alloc < 0 || rows_alloc > kMaxTileRows || count < 0 || count > rows_alloc) return LOOM_ERR_RANGE;
    loom_launch_config cfg;
    const int64_t w[1] = {count};
    if (int st = loom::evaluate_launch(loom::kRowSumTiles, w, &cfg)) return st;
    if (!sums || !final_row || !tail_count || (!values && rows_alloc > 0)) return LOOM_ERR_NULL;
    if (misaligned(values, 4) || misaligned(initial, 4) || misaligned(sums, 4) || misaligned(final_row, 4) ||
        misaligned(tail_count, 4))
        return LOOM_ERR_ALIGN;
    return launch([&] {
        return loom::launch_row_sum_tiles(cfg, values, (int)count, initial, sums, final_row, tail_count,
                                          (hipStream_t)stream);
    });
}

extern "C" int loom_row_sums(const float *x, int64_t rows, int64_t cols, int64_t row_stride, float *out,
                             void *stream) {
    if (rows < 0 || rows > kMaxRows || cols < 0 || cols > kMaxRows) return LOOM_ERR_RANGE;
    if (row_stride < cols) return LOOM_ERR_SHAPE;
    if (rows > 0 && row_stride > (INT64_MAX / 4) / rows) return LOOM_ERR_RANGE;
    loom_launch_config cfg;
    const int64_t w[2] = {rows, cols};
    if (int st = loom::evaluate_launch(loom::kRowSums, w, &cfg)) return st;
    if (rows == 0) return LOOM_OK;
    if (!out || (!x && cols > 0)) return LOOM_ERR_NULL;
    if (misaligned(x, 4) || misaligned(out, 4)) return LOOM_ERR_ALIGN;
    return launch(
        [&] { return loom::launch_row_sums(cfg, x, (int)rows, (int)cols, row_stride, out, (hipStream_t)stream); });
}

namespace {

// The checks of both segment-sum entry points, in the documented order; on
// LOOM_OK with *nothing false, cfg holds the launch geometry.
int segment_sums_checks(const float *x, int64_t total_rows, const int64_t *offsets, int64_t segments, int64_t cols,
                        const float *out, const int32_t *tail_counts, loom_launch_config *cfg, bool *nothing) {
    *nothing = true;
    if (segments < 0 || segments > kMaxRows - 1 || cols < 0 || cols > kMaxSegmentCols || total_rows < 0 ||
        total_rows > kMaxTotalRows)
        return LOOM_ERR_RANGE;
    const int64_t w[3] = {segments, cols, total_rows};
    if (int st = loom::evaluate_launch(loom::kSegmentSums, w, cfg)) return st;
    if (segments == 0) return LOOM_OK;
    if (!offsets || (!out && cols > 0) || (!x && total_rows > 0 && cols > 0)) return LOOM_ERR_NULL;
    if (misaligned(offsets, 8) || misaligned(x, 4) || misaligned(out, 4) || misaligned(tail_counts, 4))
        return LOOM_ERR_ALIGN;
    *nothing = false;
    return LOOM_OK;
}

}  // namespace

extern "C" int loom_segment_sums(const float *x, int64_t total_rows, const int64_t *offsets, int64_t segments,
                                 int64_t cols, float *out, int32_t *tail_counts, void *stream) {
    loom_launch_config cfg;
    bool nothing;
    if (int st = segment_sums_checks(x, total_rows, offsets, segments, cols, out, tail_counts, &cfg, &nothing))
        return st;
    if (nothing) return LOOM_OK;
    const int64_t workspace_bytes = loom::segment_sums_workspace_bytes(segments, cols, total_rows);
    if (workspace_bytes == 0)
        return launch([&] {
            return loom::launch_segment_sums(cfg, x, total_rows, offsets, segments, (int)cols, out, tail_counts,
                                             nullptr, (hipStream_t)stream);
        });
    // a split launch's partials or a longest-first launch's order index live
    // in stream-ordered memory, taken and given back on the caller's stream
    return launch([&] {
        void *workspace = nullptr;
        hipError_t e = hipMallocAsync(&workspace, (size_t)workspace_bytes, (hipStream_t)stream);
        if (e != hipSuccess) return e;
        e = loom::launch_segment_sums(cfg, x, total_rows, offsets, segments, (int)cols, out, tail_counts, workspace,
                                      (hipStream_t)stream);
        const hipError_t f = hipFreeAsync(workspace, (hipStream_t)stream);
        return e != hipSuccess ? e : f;
    });
}

extern "C" int loom_segment_sums_noalloc(const float *x, int64_t total_rows, const int64_t *offsets,
                                         int64_t segments, int64_t cols, float *out, int32_t *tail_counts,
                                         void *stream) {
    loom_launch_config cfg;
    bool nothing;
    if (int st = segment_sums_checks(x, total_rows, offsets, segments, cols, out, tail_counts, &cfg, &nothing))
        return st;
    if (nothing) return LOOM_OK;
    const int64_t workspace_bytes = loom::segment_sums_workspace_bytes(segments, cols, total_rows);
    if (workspace_bytes > loom::kSegmentSplitMaxBytes) return LOOM_ERR_RANGE;  // beyond the static array
    return launch([&] {
        void *workspace = nullptr;
        if (workspace_bytes > 0) {
            const hipError_t e = loom::segment_scratch(&workspace);
            if (e != hipSuccess) return e;
        }
        return loom::launch_segment_sums(cfg, x, total_rows, offsets, segments, (int)cols, out, tail_counts,
                                         workspace, (hipStream_t)stream);
    });
}

extern "C" int loom_i8_dequant_dot(const int32_t *w, const float *w_scale, const int32_t *x, const float *x_scale,
                                   int64_t rows, int64_t k, int64_t batch, float *out, int32_t *acc, void *stream) {
    if (k < 0 || k > loom::kMaxK || batch < 1 || batch > loom::kMaxBatch || rows < 0 || rows > kMaxRows)
        return LOOM_ERR_RANGE;
    if (k % 4 != 0) return LOOM_ERR_SHAPE;
    loom_launch_config cfg;
    const int64_t wl[3] = {rows, k, batch};
    if (int st = loom::evaluate_launch(loom::kI8DequantDot, wl, &cfg)) return st;
    if (rows == 0) return LOOM_OK;
    if (!w_scale || !out || (k > 0 && (!w || !x))) return LOOM_ERR_NULL;
    if (misaligned(w, 4) || misaligned(x, 4) || misaligned(w_scale, 4) || misaligned(x_scale, 4) ||
        misaligned(out, 4) || misaligned(acc, 4))
        return LOOM_ERR_ALIGN;
    return launch([&] {
        return loom::launch_i8_dequant_dot(cfg, w, w_scale, x, x_scale, (int)rows, (int)(k / 4), (int)batch, out,
                                           acc, (hipStream_t)stream);
    });
}

extern "C" int loom_packed_dot(const int32_t *fields, const uint16_t *scales, const float *rhs, int64_t streams,
                               const float *initial, int64_t records, int64_t count, int64_t outputs, float *out,
                               void *stream) {
    if (records < 0 || count < 0 || count > records || count > kMaxRows || outputs < 0 || outputs > kMaxOutputs ||
        streams < 1 || streams > kMaxRows)
        return LOOM_ERR_RANGE;
    if (records > 0 && outputs > INT64_MAX / 4 / records) return LOOM_ERR_RANGE;
    loom_launch_config cfg;
    const int64_t w[3] = {outputs, count, streams};
    if (int st = loom::evaluate_launch(loom::kPackedDot, w, &cfg)) return st;
    if (outputs == 0) return LOOM_OK;
    if (!out || (count > 0 && (!fields || !scales || !rhs))) return LOOM_ERR_NULL;
    if (misaligned(fields, 4) || misaligned(scales, 2) || misaligned(rhs, 16) || misaligned(initial, 4) ||
        misaligned(out, 4))
        return LOOM_ERR_ALIGN;
    return launch([&] {
        return loom::launch_packed_dot(cfg, fields, scales, rhs, (int)streams, initial, (int)count, outputs, out,
                                       (hipStream_t)stream);
    });
}

extern "C" int loom_sum_guarded_rows(const float *values, int64_t rows_alloc, int64_t count, int64_t columns,
                                     int64_t active_lanes, float *sums, void *stream) {
    if (rows_alloc < 0 || rows_alloc > kMaxTileRows || count < 0 || count > rows_alloc || columns < 0 ||
        columns > 4 || active_lanes < 0 || active_lanes > 32)
        return LOOM_ERR_RANGE;
    loom_launch_config cfg;
    const int64_t w[1] = {count};
    if (int st = loom::evaluate_launch(loom::kSumGuardedRows, w, &cfg)) return st;
    if (!sums || (!values && rows_alloc > 0)) return LOOM_ERR_NULL;
    if (misaligned(values, 16) || misaligned(sums, 4)) return LOOM_ERR_ALIGN;
    return launch([&] {
        return loom::launch_sum_guarded_rows(cfg, values, (int)count, (int)columns, (int)active_lanes, sums,
                                             (hipStream_t)stream);
    });
}

extern "C" int loom_routed_combine(const int32_t *ids, const float *weights, const float *payload, int64_t num_rows,
                                   int64_t tokens, int64_t routes, int64_t hidden, float *out, void *stream) {
    if (tokens < 0 || tokens > kMaxRows || routes < 0 || routes > (int64_t(1) << 20) || hidden < 0 ||
        hidden > (int64_t(1) << 20) || num_rows < 0 || num_rows > kMaxRows)
        return LOOM_ERR_RANGE;
    if (hidden % 4 != 0) return LOOM_ERR_SHAPE;
    loom_launch_config cfg;
    const int64_t w[3] = {tokens, routes, hidden};
    if (int st = loom::evaluate_launch(loom::kRoutedCombine, w, &cfg)) return st;
    if (tokens == 0 || hidden == 0) return LOOM_OK;
    if (!out || (routes > 0 && (!ids || !weights)) || (num_rows > 0 && !payload)) return LOOM_ERR_NULL;
    if (misaligned(ids, 4) || misaligned(weights, 4) || misaligned(payload, 16) || misaligned(out, 16))
        return LOOM_ERR_ALIGN;
    return launch([&] {
        return loom::launch_routed_combine(cfg, ids, weights, payload, num_rows, tokens, (int)routes, (int)hidden,
                                           out, (hipStream_t)stream);
    });
}
