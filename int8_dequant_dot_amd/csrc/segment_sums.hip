// segment_sums.hip -- per-segment column sums on gfx950.
//
// TUNE = "Tune loop unrolling and pipelining" (Loom pages).
#include <mutex>

#include "device_common.hpp"
#include "internal.hpp"

// The workspace (a split launch's partials, a longest-first launch's order
// index) for callers that cannot allocate (loom_segment_sums_noalloc): a
// file-scope device array, one per GPU the library runs on, kept until the
// process ends.  Host code never passes its
// name to a kernel -- in host code the name is only a stand-in, not a device
// address -- but the address hipGetSymbolAddress gives for the current device
// (segment_scratch).
static __device__ __align__(256) float scratch[loom::kSegmentSplitMaxBytes / sizeof(float)];

namespace loom {

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_lock;
void *scratch_address[kMaxDevices];  // per device, looked up on the first call there
}  // namespace

hipError_t segment_scratch(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> guard(scratch_lock);
    if (!scratch_address[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        scratch_address[dev] = p;
    }
    *ptr = scratch_address[dev];
    return hipSuccess;
}

template <int VEC> struct seg_vec;
template <> struct seg_vec<1> { typedef float type; };
template <> struct seg_vec<4> { typedef float4v type; };

// ----------------------------------------------------------------------------
// TUNE §Keep one checked source for experiments (@sum_rows): each lane sums
// its own column over the rows, one load and one add per row, in row order.
// Here one wave owns one unit -- a segment, or with PARTS a part of one -- and
// one block of kSegmentBlockCols columns (blockIdx.y picks the block, so a
// wide matrix spreads a segment over several waves without changing any
// column's order).  A lane owns VEC adjacent columns of each 64*VEC-column
// part of the block (one 1 KiB coalesced record per row for VEC = 4) and
// walks the unit's rows in order -- the full 8-row tiles and then the tail,
// which are consecutive -- with the next rows read ahead.  No cross-lane
// reduction is needed, and every column's sum is the same in-order f32
// recurrence a serial loop computes.  Lanes past the last column load from
// the start of the row instead (always inside the matrix) and never store, so
// every lane issues the same loads and the read-ahead keeps its partial waits.
// Segments with bad offsets are reported in-band and read nothing.
//
// PARTS (few long segments, segment_sums_parts): unit u is part u mod P of
// segment u / P, the rows [len * p / P, len * (p + 1) / P) of the segment,
// and the wave writes its partial column sums to dst = partial[u][cols];
// segment_sums_combine_kernel then adds the P partials of each segment.
// With RUN > 1 waves per workgroup (segment_sums_runs), unit u is run u mod
// R of segment u / R, wave w sums part RUN * (u mod R) + w, and the waves'
// part sums are added in part order through LDS into dst = partial[u][cols]
// (the segment's R partials then go to the second pass).  Otherwise unit u is
// segment order[u] (longest first, segment_sums_ordered) or segment u, and
// dst = out[s][cols].
// ----------------------------------------------------------------------------
template <int VEC, bool FULL, int DEPTH, bool PARTS, int RUN = 1>
__global__ __launch_bounds__(kWave * RUN) void segment_sums_kernel(const float *__restrict__ x, int64_t total_rows,
                                                                   const int64_t *__restrict__ offsets,
                                                                   int64_t units, int parts, int cols,
                                                                   float *__restrict__ dst,
                                                                   int32_t *__restrict__ tail_counts,
                                                                   const int32_t *__restrict__ order) {
    static_assert(RUN == 1 || PARTS, "runs group the parts of a split launch");
    typedef typename seg_vec<VEC>::type V;
    constexpr int kBlock = kWave * VEC;
    __shared__ V run_sums[RUN][RUN > 1 ? kBlock : 1];  // a column group's part sums, one row per wave
    const int lane = lane_id();
    const int wave = RUN > 1 ? __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave)) : 0;
    const int runs = parts / RUN;  // units per segment with RUN > 1
    const int block_first = blockIdx.y * kSegmentBlockCols;
    const int block_end = min(cols, block_first + kSegmentBlockCols);
    // one unit per workgroup; past the grid's work-item limit, every grid.x-th unit
    for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
        const int64_t s = RUN > 1 ? u / runs : PARTS ? u / parts : order ? (int64_t)order[u] : u;
        const int p = RUN > 1 ? (int)(u - s * runs) * RUN + wave : PARTS ? (int)(u - s * parts) : 0;
        const int64_t begin = offsets[s];
        const int64_t end = offsets[s + 1];
        float *o = dst + (PARTS ? u : s) * cols;
        const bool writes_tail = p == 0 && blockIdx.y == 0 && tail_counts;

        if (!(begin >= 0 && begin <= end && end <= total_rows)) {  // the same in every wave of a run
            if (wave == 0)
                for (int c = block_first + lane; c < block_end; c += kWave) o[c] = __builtin_nanf("");
            if (lane == 0 && writes_tail) tail_counts[s] = -1;
            continue;
        }
        const int64_t length = end - begin;
        if (lane == 0 && writes_tail) tail_counts[s] = (int32_t)(length & (kTileRows - 1));
        // this unit's rows (the whole segment without PARTS)
        const int64_t first = PARTS ? begin + length * p / parts : begin;
        const int64_t count = PARTS ? begin + length * (p + 1) / parts - first : length;

        for (int cb = block_first; cb < block_end; cb += kBlock) {
            const int c = cb + lane * VEC;
            const bool active = FULL || c < cols;
            // Row base of the next load (wave-uniform) plus the lane's column.
            const float *rp = x + first * cols + cb;
            const int lane_col = active ? lane * VEC : -cb;  // inactive lanes read the row's first columns
            V acc = V(0.0f);
            // the straight drain for runs: no copies of the ring at the register
            // budget of a run's workgroup
            pipelined<DEPTH, V, (RUN > 1)>(
                count,
                [&]() {
                    const V v = load_stream(reinterpret_cast<const V *>(rp + lane_col));
                    rp += cols;
                    return v;
                },
                [&](V v) { acc += v; });
            if constexpr (RUN > 1) {
                run_sums[wave][lane] = acc;
                __syncthreads();
                if (wave == 0) {
                    V sum = V(0.0f);
                    for (int w = 0; w < RUN; ++w) sum += run_sums[w][lane];
                    if (active) *reinterpret_cast<V *>(o + c) = sum;
                }
                __syncthreads();  // run_sums is rewritten next
            } else {
                if (active) *reinterpret_cast<V *>(o + c) = acc;
            }
        }
    }
}

// The order pass of a longest-first launch (one workgroup): a counting sort
// of the segments by length bucket -- 0 for an empty segment or bad offsets,
// else 1 + 4 floor(log2 len) + the two bits below the leading one -- into
// order[], longest bucket first; within a bucket the order is whatever the
// atomics give, which changes no output.  Each thread reads the offsets of
// kOrderBatch segments before it uses any, and keeps their buckets in LDS for
// the scatter.
constexpr int kOrderBuckets = 1 + 4 * 42;  // lengths of 2^42 rows and more share the top one
constexpr int kOrderThreads = 1024;
constexpr int kOrderBatch = 8;
constexpr int kOrderPerLane = (kOrderBuckets + kWave - 1) / kWave;
static_assert(kSegmentOrderMaxSegments % (kOrderThreads * kOrderBatch) == 0, "whole batches in the LDS array");

__device__ __forceinline__ int length_bucket(int64_t begin, int64_t end, int64_t total_rows) {
    if (!(begin >= 0 && begin < end && end <= total_rows)) return 0;
    const uint64_t len = (uint64_t)(end - begin);
    const int e = min(63 - __builtin_clzll(len), 41);  // floor(log2 len), capped
    const int m = e >= 2 ? (int)((len >> (e - 2)) & 3) : (int)((len << (2 - e)) & 3);
    return 1 + 4 * e + m;
}

__global__ __launch_bounds__(kOrderThreads) void segment_order_kernel(const int64_t *__restrict__ offsets,
                                                                      int64_t segments, int64_t total_rows,
                                                                      int32_t *__restrict__ order) {
    // next[kOrderBuckets + lane] are spare counters for the slots past the
    // last segment (one per lane, so they never contend), so the batches
    // below run without branches
    __shared__ unsigned next[kOrderBuckets + kWave];
    __shared__ uint8_t bucket[kSegmentOrderMaxSegments];
    const int n = (int)min(segments, kSegmentOrderMaxSegments);
    const int spare = kOrderBuckets + (int)(threadIdx.x & (kWave - 1));
    for (int b = threadIdx.x; b < kOrderBuckets + kWave; b += kOrderThreads) next[b] = 0;
    __syncthreads();
    for (int base = 0; base < n; base += kOrderThreads * kOrderBatch) {
        int64_t begin[kOrderBatch], end[kOrderBatch];
#pragma unroll
        for (int j = 0; j < kOrderBatch; ++j) {
            const int s = min(base + j * kOrderThreads + (int)threadIdx.x, n - 1);
            begin[j] = offsets[s];
            end[j] = offsets[s + 1];
        }
#pragma unroll
        for (int j = 0; j < kOrderBatch; ++j) {
            const int s = base + j * kOrderThreads + (int)threadIdx.x;
            const int k = s < n ? length_bucket(begin[j], end[j], total_rows) : spare;
            if (s < n) bucket[s] = (uint8_t)k;
            atomicAdd(&next[k], 1u);
        }
    }
    __syncthreads();
    if (threadIdx.x < kWave) {
        // first position of each bucket, longest bucket first: lane l holds
        // the kOrderPerLane buckets kOrderBuckets - 1 - (kOrderPerLane l + j),
        // and a wave-wide exclusive scan of the lanes' totals places them
        const int lane = (int)threadIdx.x;
        unsigned c[kOrderPerLane], own = 0;
#pragma unroll
        for (int j = 0; j < kOrderPerLane; ++j) {
            const int b = kOrderBuckets - 1 - (kOrderPerLane * lane + j);
            c[j] = b >= 0 ? next[b] : 0u;
            own += c[j];
        }
        unsigned incl = own;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const unsigned y = __shfl_up(incl, d);
            if (lane >= d) incl += y;
        }
        unsigned run = incl - own;
#pragma unroll
        for (int j = 0; j < kOrderPerLane; ++j) {
            const int b = kOrderBuckets - 1 - (kOrderPerLane * lane + j);
            if (b >= 0) next[b] = run;
            run += c[j];
        }
    }
    __syncthreads();
    for (int base = 0; base < n; base += kOrderThreads * kOrderBatch) {
        int k[kOrderBatch];
        unsigned pos[kOrderBatch];
#pragma unroll
        for (int j = 0; j < kOrderBatch; ++j) {
            const int s = base + j * kOrderThreads + (int)threadIdx.x;
            k[j] = s < n ? bucket[min(s, n - 1)] : spare;
        }
#pragma unroll
        for (int j = 0; j < kOrderBatch; ++j) pos[j] = atomicAdd(&next[k[j]], 1u);
#pragma unroll
        for (int j = 0; j < kOrderBatch; ++j) {
            const int s = base + j * kOrderThreads + (int)threadIdx.x;
            if (s < n) order[pos[j]] = s;
        }
    }
}

// The second pass of a split launch: one workgroup of kSegmentCombineWaves
// waves per segment and 256-column block, a lane per VEC adjacent columns
// (VEC = 4: one 1 KiB load per part row of the block).  Wave w adds, in part
// order, the partials of its contiguous run of parts -- parts w * R .. w * R
// + R - 1, R = ceil(P / kSegmentCombineWaves) -- with the partials read ahead,
// and out[s][c] is the sum of the run sums in run order, all in f32 from
// +0.0: a fixed association of the P part sums, so a call gives the same bits
// every time.  A segment with bad offsets has NaN partials, so its outputs
// stay NaN.
template <int VEC, int DEPTH>
__global__ __launch_bounds__(kWave * kSegmentCombineWaves) void segment_sums_combine_kernel(
    const float *__restrict__ partial, int64_t segments, int parts, int cols, float *__restrict__ out) {
    typedef typename seg_vec<VEC>::type V;
    __shared__ V run[kSegmentCombineWaves][kWave];
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const int per = (parts + kSegmentCombineWaves - 1) / kSegmentCombineWaves;
    const int first = min(parts, wave * per);
    const int n = min(parts, first + per) - first;
    const int block_first = blockIdx.y * kSegmentBlockCols;
    const int block_end = min(cols, block_first + kSegmentBlockCols);
    for (int64_t s = blockIdx.x; s < segments; s += gridDim.x) {
        for (int c0 = block_first; c0 < block_end; c0 += kWave * VEC) {
            const int c = c0 + lane * VEC;
            const bool active = c < block_end;  // VEC = 4: cols % 4 == 0, so a group is wholly in or out
            const V *pp = reinterpret_cast<const V *>(partial + (s * parts + first) * cols + (active ? c : block_first));
            const int stride = cols / VEC;
            V acc = V{};
            pipelined<DEPTH, V, true>(  // the straight drain: no copies of the ring at this register budget
                n,
                [&]() {
                    const V v = *pp;
                    pp += stride;
                    return v;
                },
                [&](V v) { acc = acc + v; });
            run[wave][lane] = acc;
            __syncthreads();
            if (wave == 0) {
                V sum = V{};
                for (int v = 0; v < kSegmentCombineWaves; ++v) sum = sum + run[v][lane];
                if (active) *reinterpret_cast<V *>(out + s * cols + c) = sum;
            }
            __syncthreads();  // run[] is rewritten next
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
#ifndef LOOM_SEGMENT_COMBINE_DEPTH
#define LOOM_SEGMENT_COMBINE_DEPTH 8
#endif
constexpr int kSegmentCombineDepth = LOOM_SEGMENT_COMBINE_DEPTH;  // part rows in flight per wave of the combine
constexpr int segment_sums_depth(int64_t waves, int cols) {
    const int by_waves = waves <= 256 ? 4 * kSegmentDepth : waves <= 1024 ? 2 * kSegmentDepth : kSegmentDepth;
    const int by_width = cols <= 64 ? 4 * kSegmentDepth : cols <= 128 ? 2 * kSegmentDepth : kSegmentDepth;
    return by_waves > by_width ? by_waves : by_width;
}

template <int DEPTH, bool PARTS, int RUN>
static void launch_segment_sums_depth(dim3 grid, dim3 block, bool vec4, const float *x, int64_t total_rows,
                                      const int64_t *offsets, int64_t units, int parts, int cols, float *dst,
                                      int32_t *tail_counts, const int32_t *order, hipStream_t stream) {
#define LOOM_SEGMENT_LAUNCH(VEC, FULL)                                                                      \
    segment_sums_kernel<VEC, FULL, DEPTH, PARTS, RUN><<<grid, block, 0, stream>>>(x, total_rows, offsets, units, \
                                                                                 parts, cols, dst, tail_counts, \
                                                                                 order)
    if (vec4) {
        if (cols % (kWave * 4) == 0)
            LOOM_SEGMENT_LAUNCH(4, true);
        else
            LOOM_SEGMENT_LAUNCH(4, false);
    } else {
        if (cols % kWave == 0)
            LOOM_SEGMENT_LAUNCH(1, true);
        else
            LOOM_SEGMENT_LAUNCH(1, false);
    }
#undef LOOM_SEGMENT_LAUNCH
}

// The read-ahead depth follows the launch's wave count and the row width; a
// run's waves keep the base depth (a split launch big enough for the depth to
// matter has thousands of waves, where the base depth is the one chosen
// anyway).
template <bool PARTS, int RUN = 1>
static void launch_segment_units(dim3 grid, dim3 block, bool vec4, const float *x, int64_t total_rows,
                                 const int64_t *offsets, int64_t units, int parts, int cols, float *dst,
                                 int32_t *tail_counts, const int32_t *order, hipStream_t stream) {
    if constexpr (RUN > 1) {
        launch_segment_sums_depth<kSegmentDepth, PARTS, RUN>(grid, block, vec4, x, total_rows, offsets, units, parts,
                                                             cols, dst, tail_counts, order, stream);
    } else {
        switch (segment_sums_depth((int64_t)grid.x * grid.y, cols)) {
            case 4 * kSegmentDepth:
                launch_segment_sums_depth<4 * kSegmentDepth, PARTS, RUN>(grid, block, vec4, x, total_rows, offsets,
                                                                          units, parts, cols, dst, tail_counts, order,
                                                                          stream);
                break;
            case 2 * kSegmentDepth:
                launch_segment_sums_depth<2 * kSegmentDepth, PARTS, RUN>(grid, block, vec4, x, total_rows, offsets,
                                                                          units, parts, cols, dst, tail_counts, order,
                                                                          stream);
                break;
            default:
                launch_segment_sums_depth<kSegmentDepth, PARTS, RUN>(grid, block, vec4, x, total_rows, offsets, units,
                                                                      parts, cols, dst, tail_counts, order, stream);
                break;
        }
    }
}

hipError_t launch_segment_sums(const loom_launch_config &cfg, const float *x, int64_t total_rows,
                               const int64_t *offsets, int64_t segments, int cols, float *out,
                               int32_t *tail_counts, void *workspace, hipStream_t stream) {
    const dim3 grid(cfg.workgroups[0], cfg.workgroups[1]), block(cfg.workgroup_size[0]);
    const int parts = segment_sums_parts(segments, cols, total_rows);
    if (parts <= 1) {
        const bool vec4 = (reinterpret_cast<uintptr_t>(x) % 16 == 0) &&
                          (reinterpret_cast<uintptr_t>(out) % 16 == 0) && (cols % 4 == 0);
        int32_t *order = nullptr;
        if (segment_sums_ordered(segments, cols, total_rows)) {
            order = static_cast<int32_t *>(workspace);
            segment_order_kernel<<<dim3(1), dim3(kOrderThreads), 0, stream>>>(offsets, segments, total_rows, order);
            if (hipError_t e = hipGetLastError()) return e;
        }
        launch_segment_units<false>(grid, block, vec4, x, total_rows, offsets, segments, 1, cols, out, tail_counts,
                                    order, stream);
        return hipGetLastError();
    }
    float *partial = static_cast<float *>(workspace);
    const bool vec4 = (reinterpret_cast<uintptr_t>(x) % 16 == 0) &&
                      (reinterpret_cast<uintptr_t>(partial) % 16 == 0) && (cols % 4 == 0);
    const int runs = segment_sums_runs(segments, cols, total_rows);
    if (runs > 0)
        launch_segment_units<true, kSegmentRunWaves>(grid, block, vec4, x, total_rows, offsets, segments * runs,
                                                     parts, cols, partial, tail_counts, nullptr, stream);
    else
        launch_segment_units<true>(grid, block, vec4, x, total_rows, offsets, segments * parts, parts, cols,
                                   partial, tail_counts, nullptr, stream);
    if (hipError_t e = hipGetLastError()) return e;
    const int partials = runs > 0 ? runs : parts;
    const dim3 cgrid((unsigned)grid_stride_groups(segments, kWave * kSegmentCombineWaves), cfg.workgroups[1]);
    const dim3 cblock(kWave * kSegmentCombineWaves);
    if (vec4 && reinterpret_cast<uintptr_t>(out) % 16 == 0)
        segment_sums_combine_kernel<4, kSegmentCombineDepth><<<cgrid, cblock, 0, stream>>>(partial, segments,
                                                                                          partials, cols, out);
    else
        segment_sums_combine_kernel<1, kSegmentCombineDepth><<<cgrid, cblock, 0, stream>>>(partial, segments,
                                                                                          partials, cols, out);
    return hipGetLastError();
}

}  // namespace loom
