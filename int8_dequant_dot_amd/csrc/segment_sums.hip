// segment_sums.hip -- per-segment column sums on gfx950.
//
// TUNE = "Tune loop unrolling and pipelining" (Loom pages).
#include "device_common.hpp"
#include "internal.hpp"

namespace loom {

template <int VEC> struct seg_vec;
template <> struct seg_vec<1> { typedef float type; };
template <> struct seg_vec<4> { typedef float4v type; };

// ----------------------------------------------------------------------------
// TUNE §Keep one checked source for experiments (@sum_rows): each lane sums
// its own column over the rows, one load and one add per row, in row order.
// Here one wave owns one segment and one block of kSegmentBlockCols columns
// (blockIdx.y picks the block, so a wide matrix spreads a segment over several
// waves without changing any column's order).  A lane owns VEC adjacent
// columns of each 64*VEC-column part of the block (one 1 KiB coalesced record
// per row for VEC = 4) and walks the segment's rows in order -- the full
// 8-row tiles and then the tail, which are consecutive -- with the next rows
// read ahead.  No cross-lane reduction is needed, and every column's sum is
// the same in-order f32 recurrence a serial loop computes.  Lanes past the
// last column load from the start of the row instead (always inside the
// matrix) and never store, so every lane issues the same loads and the
// read-ahead keeps its partial waits.  Segments with bad offsets are reported
// in-band and read nothing.
// ----------------------------------------------------------------------------
template <int VEC, bool FULL, int DEPTH>
__global__ __launch_bounds__(kWave) void segment_sums_kernel(const float *__restrict__ x, int64_t total_rows,
                                                             const int64_t *__restrict__ offsets, int64_t segments,
                                                             int cols, float *__restrict__ out,
                                                             int32_t *__restrict__ tail_counts) {
    typedef typename seg_vec<VEC>::type V;
    constexpr int kBlock = kWave * VEC;
    const int lane = lane_id();
    const int block_first = blockIdx.y * kSegmentBlockCols;
    const int block_end = min(cols, block_first + kSegmentBlockCols);
    // one segment per wave; past the grid's work-item limit, every grid.x-th segment
    for (int64_t s = blockIdx.x; s < segments; s += gridDim.x) {
        const int64_t begin = offsets[s];
        const int64_t end = offsets[s + 1];
        float *o = out + s * cols;

        if (!(begin >= 0 && begin <= end && end <= total_rows)) {
            for (int c = block_first + lane; c < block_end; c += kWave) o[c] = __builtin_nanf("");
            if (lane == 0 && blockIdx.y == 0 && tail_counts) tail_counts[s] = -1;
            continue;
        }
        const int64_t length = end - begin;
        if (lane == 0 && blockIdx.y == 0 && tail_counts) tail_counts[s] = (int32_t)(length & (kTileRows - 1));

        for (int cb = block_first; cb < block_end; cb += kBlock) {
            const int c = cb + lane * VEC;
            const bool active = FULL || c < cols;
            // Row base of the next load (wave-uniform) plus the lane's column.
            const float *rp = x + begin * cols + cb;
            const int lane_col = active ? lane * VEC : -cb;  // inactive lanes read the row's first columns
            V acc = V(0.0f);
            pipelined<DEPTH, V>(
                length,
                [&]() {
                    const V v = load_stream(reinterpret_cast<const V *>(rp + lane_col));
                    rp += cols;
                    return v;
                },
                [&](V v) { acc += v; });
            if (active) *reinterpret_cast<V *>(o + c) = acc;
        }
    }
}

// Rows in flight per wave.  A launch of many waves (segments x 256-column
// blocks) over 256 columns keeps HBM busy with 8 rows each (7 KiB per wave);
// few waves, or narrow rows (fewer bytes per row), need a deeper ring.  Over
// ~1-4 GB at depth 8 / 16 / 32: 16384 segments of 256 columns 676.5 / 693.1 /
// 684.4 us; 2048 waves 734.9 / 735.3 / 721.0; 512 waves 276.3 / 195.0 /
// 198.6; 128 waves 912.4 / 525.4 / 336.6; 128 columns (8192 segments) 427.5
// / 353.6 / 344.7; 64 columns (16384 segments) 677.5 / 458.4 / 444.8; 16
// columns 1142.9 / 737.4 / 691.6 us.  The order of every column's sum is the
// same at any depth.
#ifndef LOOM_SEGMENT_SUMS_DEPTH
#define LOOM_SEGMENT_SUMS_DEPTH 8
#endif
constexpr int kSegmentDepth = LOOM_SEGMENT_SUMS_DEPTH;
constexpr int segment_sums_depth(int64_t waves, int cols) {
    const int by_waves = waves <= 256 ? 4 * kSegmentDepth : waves <= 1024 ? 2 * kSegmentDepth : kSegmentDepth;
    const int by_width = cols <= 64 ? 4 * kSegmentDepth : cols <= 128 ? 2 * kSegmentDepth : kSegmentDepth;
    return by_waves > by_width ? by_waves : by_width;
}

template <int DEPTH>
static void launch_segment_sums_depth(dim3 grid, dim3 block, bool vec4, const float *x, int64_t total_rows,
                                      const int64_t *offsets, int64_t segments, int cols, float *out,
                                      int32_t *tail_counts, hipStream_t stream) {
    if (vec4) {
        if (cols % (kWave * 4) == 0)
            segment_sums_kernel<4, true, DEPTH><<<grid, block, 0, stream>>>(x, total_rows, offsets, segments, cols, out,
                                                                            tail_counts);
        else
            segment_sums_kernel<4, false, DEPTH><<<grid, block, 0, stream>>>(x, total_rows, offsets, segments, cols, out,
                                                                             tail_counts);
    } else {
        if (cols % kWave == 0)
            segment_sums_kernel<1, true, DEPTH><<<grid, block, 0, stream>>>(x, total_rows, offsets, segments, cols, out,
                                                                            tail_counts);
        else
            segment_sums_kernel<1, false, DEPTH><<<grid, block, 0, stream>>>(x, total_rows, offsets, segments, cols, out,
                                                                             tail_counts);
    }
}

hipError_t launch_segment_sums(const loom_launch_config &cfg, const float *x, int64_t total_rows,
                               const int64_t *offsets, int64_t segments, int cols, float *out,
                               int32_t *tail_counts, hipStream_t stream) {
    const dim3 grid(cfg.workgroups[0], cfg.workgroups[1]), block(cfg.workgroup_size[0]);
    const bool vec4 = (reinterpret_cast<uintptr_t>(x) % 16 == 0) && (reinterpret_cast<uintptr_t>(out) % 16 == 0) &&
                      (cols % 4 == 0);
    switch (segment_sums_depth((int64_t)cfg.workgroups[0] * cfg.workgroups[1], cols)) {
        case 4 * kSegmentDepth:
            launch_segment_sums_depth<4 * kSegmentDepth>(grid, block, vec4, x, total_rows, offsets, segments, cols,
                                                         out, tail_counts, stream);
            break;
        case 2 * kSegmentDepth:
            launch_segment_sums_depth<2 * kSegmentDepth>(grid, block, vec4, x, total_rows, offsets, segments, cols,
                                                         out, tail_counts, stream);
            break;
        default:
            launch_segment_sums_depth<kSegmentDepth>(grid, block, vec4, x, total_rows, offsets, segments, cols,
                                                     out, tail_counts, stream);
            break;
    }
    return hipGetLastError();
}

}  // namespace loom
