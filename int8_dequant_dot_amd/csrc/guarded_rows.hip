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
#define LOOM_GUARDED_ROWS_DEPTH 8   // rows in flight: the pages' shape is latency-bound
#endif
constexpr int kGuardedRowsDepth = LOOM_GUARDED_ROWS_DEPTH;

// Buffer descriptor word 3 for raw (untyped, 32-bit) buffer access on GFX9.
constexpr int kGuardRawBufferWord3 = 0x00020000;
constexpr int kGuardRowBytes = 32 * 4 * 4;  // one row of the tile: 32 lanes x 4 components

// The first COLS components of one lane's slot of a row, read through a
// buffer descriptor that covers exactly that row: one 128-bit load for all
// four, else one 32-bit load per component (COLS loads, the same on every
// path).  A lane whose offset lies past the row gets zeros from the hardware
// and touches no memory.
template <int COLS>
__device__ __forceinline__ float4v guarded_read(__amdgpu_buffer_rsrc_t row, int offset) {
    if constexpr (COLS == 4)
        return __builtin_bit_cast(float4v, __builtin_amdgcn_raw_buffer_load_b128(row, offset, 0, 0));
    float4v v = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < COLS; ++c)
        v[c] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(row, offset + 4 * c, 0, 0));
    return v;
}

// One work-item per tile lane (a 32-item workgroup, as the page launches it).
// A row's guarded read -- the whole inner loop over COLS components, with its
// lane guard -- is the producer, so it runs ahead as one unit; the consumer
// adds the components in order from 0 and then adds that partial to the
// carried sum.  The inner extent is a template argument and the lane guard is
// the buffer range (an inactive lane's offset lies past the row), so every
// row issues exactly one load instruction on every path and the ring keeps
// DEPTH-1 rows in flight.  Rows from `count` to the padded end contribute the
// identity: the carried sum starts at +0 and an IEEE round-to-nearest sum
// with +0 never yields -0, so adding +0 leaves it unchanged and those rows
// are skipped without changing a bit (and without touching memory).
template <int DEPTH, int COLS>
__global__ __launch_bounds__(32) void sum_guarded_rows_kernel(const float *__restrict__ values, int count,
                                                              int active_lanes, float *__restrict__ sums) {
    const int lane = threadIdx.x;
    const int offset = lane < active_lanes ? lane * 16 : kGuardRowBytes;
    const float *row = values;
    float sum = 0.0f;
    pipelined<DEPTH, float4v>(
        count,
        [&]() {
            const __amdgpu_buffer_rsrc_t rsrc =
                __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(row), 0, kGuardRowBytes, kGuardRawBufferWord3);
            row += 32 * 4;
            return guarded_read<COLS>(rsrc, offset);
        },
        [&](float4v v) {
            float partial = 0.0f;
            if constexpr (COLS > 0) partial = partial + v.x;
            if constexpr (COLS > 1) partial = partial + v.y;
            if constexpr (COLS > 2) partial = partial + v.z;
            if constexpr (COLS > 3) partial = partial + v.w;
            sum = sum + partial;
        });
    sums[lane] = sum;
}

hipError_t launch_sum_guarded_rows(const loom_launch_config &cfg, const float *values, int count, int columns,
                                   int active_lanes, float *sums, hipStream_t stream) {
    const dim3 grid(cfg.workgroups[0]), block(cfg.workgroup_size[0]);
    switch (columns) {
        case 0:
            sum_guarded_rows_kernel<kGuardedRowsDepth, 0><<<grid, block, 0, stream>>>(values, count, active_lanes, sums);
            break;
        case 1:
            sum_guarded_rows_kernel<kGuardedRowsDepth, 1><<<grid, block, 0, stream>>>(values, count, active_lanes, sums);
            break;
        case 2:
            sum_guarded_rows_kernel<kGuardedRowsDepth, 2><<<grid, block, 0, stream>>>(values, count, active_lanes, sums);
            break;
        case 3:
            sum_guarded_rows_kernel<kGuardedRowsDepth, 3><<<grid, block, 0, stream>>>(values, count, active_lanes, sums);
            break;
        default:
            sum_guarded_rows_kernel<kGuardedRowsDepth, 4><<<grid, block, 0, stream>>>(values, count, active_lanes, sums);
            break;
    }
    return hipGetLastError();
}

}  // namespace loom
