// guarded_rows.hip -- the pages' guarded ragged row sum on gfx950.
//
// TUNE = "Tune loop unrolling and pipelining" (Loom pages), §Keep guards and
// inner loops in the source (@guide.sum_guarded_rows): a [63][32][4] f32
// tile, a runtime row count, a runtime inner extent (components per row) and
// a runtime number of active lanes; rows are rounded up to groups of four and
// the padded row lies outside the allocation.
#include "device_common.hpp"
#include "internal.hpp"

namespace loom {

#ifndef LOOM_GUARDED_ROWS_DEPTH
#define LOOM_GUARDED_ROWS_DEPTH 3  // the pages' outer read-ahead depth
#endif
constexpr int kGuardedRowsDepth = LOOM_GUARDED_ROWS_DEPTH;

// One work-item per tile lane (a 32-item workgroup, as the page launches it).
// A row's guarded read -- the whole inner loop, with its lane and extent
// guards -- is the producer, so it runs ahead as one unit; the consumer adds
// the components in order from 0 and then adds that partial to the carried
// sum.  Rows from `count` to the padded end contribute the identity: the
// carried sum starts at +0 and an IEEE round-to-nearest sum with +0 never
// yields -0, so adding +0 leaves it unchanged and those rows are skipped
// without changing a bit (and without touching memory).
template <int DEPTH>
__global__ __launch_bounds__(32) void sum_guarded_rows_kernel(const float *__restrict__ values, int count,
                                                              int columns, int active_lanes,
                                                              float *__restrict__ sums) {
    const int lane = threadIdx.x;
    const bool active = lane < active_lanes;
    const float *p = values + lane * 4;
    float sum = 0.0f;
    pipelined<DEPTH, float4v>(
        count,
        [&]() {
            float4v v = {0.0f, 0.0f, 0.0f, 0.0f};
            if (active) {
                if (columns == 4) {
                    v = *reinterpret_cast<const float4v *>(p);
                } else {
                    if (columns > 0) v.x = p[0];
                    if (columns > 1) v.y = p[1];
                    if (columns > 2) v.z = p[2];
                }
            }
            p += 32 * 4;
            return v;
        },
        [&](float4v v) {
            float partial = 0.0f;
            if (columns > 0) partial = partial + v.x;
            if (columns > 1) partial = partial + v.y;
            if (columns > 2) partial = partial + v.z;
            if (columns > 3) partial = partial + v.w;
            sum = sum + partial;
        });
    sums[lane] = sum;
}

hipError_t launch_sum_guarded_rows(const loom_launch_config &cfg, const float *values, int count, int columns,
                                   int active_lanes, float *sums, hipStream_t stream) {
    sum_guarded_rows_kernel<kGuardedRowsDepth><<<dim3(cfg.workgroups[0]), dim3(cfg.workgroup_size[0]), 0, stream>>>(
        values, count, columns, active_lanes, sums);
    return hipGetLastError();
}

}  // namespace loom
