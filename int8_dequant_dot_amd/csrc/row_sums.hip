// row_sums.hip -- the tiled 32-lane row sum and the streaming row sums on gfx950.
//
// TUNE = "Tune loop unrolling and pipelining" (Loom pages).  The streaming
// row sums pick one of three mappings by row width (row_sums_narrow_log2_lanes
// and row_sums_waves_per_row choose; the launch table uses the same rules):
//   1-128 floats      several rows packed into each 64-lane record
//   129-768 floats    one wave per 2 full 8-row tiles, the last tile the tail
//   769+ floats       one workgroup per row, its columns split over 1-16 waves
#include "device_common.hpp"
#include "internal.hpp"

namespace loom {

// ----------------------------------------------------------------------------
// TUNE §Derive full tiles from a ragged loop (@guide.sum_full_tiles).
//
// One wave64 owns the whole [rows][32] tile.  The pages' subgroup is 32 lanes
// wide (one lane per column); a gfx950 wave holds two such rows at once, so a
// record is a pair of rows: lanes 0-31 load row 2p, lanes 32-63 row 2p+1
// (128 B each, one coalesced 256 B access).  Each half reduces its own row,
// and the two row totals are added to the carried sum in row order.  Full
// tiles have an even row count, so pairs never straddle the tail; rows at or
// beyond final_row are never read.
// ----------------------------------------------------------------------------
template <int DEPTH>
__global__ __launch_bounds__(kWave) void row_sum_tiles_kernel(const float *__restrict__ values, int count,
                                                              const float *__restrict__ initial,
                                                              float *__restrict__ sums,
                                                              int32_t *__restrict__ final_row,
                                                              int32_t *__restrict__ tail_count) {
    const int lane = lane_id();
    const int col = lane & 31;
    // The tile walk advances by 8 while at least 8 rows remain: it stops at
    // the largest multiple of 8 not above count, leaving count mod 8 rows.
    const int full_rows = count & ~(kTileRows - 1);
    const int tail = count & (kTileRows - 1);

    float sum = initial ? initial[col] : 0.0f;
    const float *p = values + lane;  // row (lane >> 5), column (lane & 31)
    pipelined<DEPTH, float>(
        full_rows / 2,
        [&]() {
            float v = *p;
            p += 2 * 32;
            return v;
        },
        [&](float v) {
            v = half_wave_sum(v);           // each 32-lane half: its row's total
            sum = sum + readlane(v, 0);     // row 2p
            sum = sum + readlane(v, 32);    // row 2p+1
        });
    if (lane < 32) sums[lane] = sum;
    if (lane == 0) {
        *final_row = full_rows;
        *tail_count = tail;
    }
}

// ----------------------------------------------------------------------------
// Streaming row sums of rows of 129-768 floats.  One wave owns
// kRowSumsTilesPerWave consecutive tiles of 8 rows (the last tile of the
// matrix holds the rows mod 8 tail, so it is the separate guarded tile of
// TUNE §Derive full tiles).  The wave's rows are walked as one stream of
// records -- a record is
// 64 lanes x VEC contiguous floats of one row (1 KiB for VEC = 4) -- so the
// read-ahead crosses row boundaries without draining.  Each lane folds its
// floats into a private partial; at the end of a row the wave64 reduction
// gives the row total (TUNE §Give each motif its own schedule: vector loads
// pre-reduced in registers, then one ordered update per row).
// ----------------------------------------------------------------------------
template <int VEC> struct vec_of;
template <> struct vec_of<1> { typedef float type; };
template <> struct vec_of<4> { typedef float4v type; };

template <int VEC>
__device__ __forceinline__ float fold(typename vec_of<VEC>::type v) {
    if constexpr (VEC == 1) return v;
    else return (v.x + v.y) + (v.z + v.w);
}

template <int VEC, bool FULL, int DEPTH>
__global__ __launch_bounds__(kWave) void row_sums_kernel(const float *__restrict__ x, int rows, int cols,
                                                         int64_t row_stride, float *__restrict__ out) {
    typedef typename vec_of<VEC>::type V;
    constexpr int kBlock = kWave * VEC;  // columns per record
    const int lane = lane_id();
    const int row0 = blockIdx.x * (kTileRows * kRowSumsTilesPerWave);
    const int nrows = min(kTileRows * kRowSumsTilesPerWave, rows - row0);
    const int records_per_row = (cols + kBlock - 1) / kBlock;

    // Producer cursor (wave-uniform, kept in SGPRs): the current row and the
    // first column of the next record.  A lane's load address is that base
    // plus its own 32-bit column offset.
    const float *rp = x + (int64_t)row0 * row_stride;
    int lcol = 0;
    const int lane_col = lane * VEC;
    // consumer state
    V acc = V(0.0f);
    int crec = 0, crow = 0;
    float mine = 0.0f;

    pipelined<DEPTH, V>(
        nrows * records_per_row,
        [&]() {
            const float *bp = rp + lcol;
            V v = V(0.0f);
            // (compared as differences, which cannot overflow for any cols < 2^31)
            if (FULL || lane_col < cols - lcol) v = load_stream(reinterpret_cast<const V *>(bp + lane_col));
            if (lcol >= cols - kBlock) {
                lcol = 0;
                rp += row_stride;
            } else {
                lcol += kBlock;
            }
            return v;
        },
        [&](V v) {
            acc += v;
            if (++crec == records_per_row) {
                const float total = wave_sum(fold<VEC>(acc));
                if (lane == crow) mine = total;
                acc = V(0.0f);
                crec = 0;
                ++crow;
            }
        });
    if (lane < nrows) out[row0 + lane] = mine;
}

// ----------------------------------------------------------------------------
// Row sums of long rows (769 columns and more: at least four 256-float
// records, the last one possibly partial).  One workgroup of
// W = blockDim.x / 64 waves owns one row; wave w streams a contiguous share of
// the row's records (the same 64 x VEC float records as above, about four per
// wave) into a private partial, reduces it across the wave, and the W wave
// totals are added in wave order (a fixed tree: the result does not depend on
// timing).  A row needs no guard and there is no tail tile: every workgroup
// has a whole row.  The many short waves (262,144 of 4 KiB for 65536 rows of
// 4096 floats) keep the end of the launch short, and a matrix with few rows
// still spreads over the GPU.
// ----------------------------------------------------------------------------
template <int VEC, bool FULL, int DEPTH>
__global__ __launch_bounds__(kWave * kRowSumsWideMaxWaves) void row_sums_wide_kernel(const float *__restrict__ x,
                                                                                   int rows, int cols,
                                                                                   int64_t row_stride,
                                                                                   float *__restrict__ out) {
    typedef typename vec_of<VEC>::type V;
    constexpr int kBlock = kWave * VEC;
    const int lane = lane_id();
    const int waves = blockDim.x / kWave;
    // the same in every lane: keeps the wave's share and cursor in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    // (no cols + kBlock - 1: that overflows for rows close to 2^31 floats)
    const int records = cols / kBlock + (cols % kBlock != 0);
    const int per = (records + waves - 1) / waves;
    const int first = min(records, wave * per);
    const int n = min(records, first + per) - first;
    const int lane_col = lane * VEC;
    __shared__ float part[kRowSumsWideMaxWaves];
    // one row per workgroup; past the grid's work-item limit, every grid.x-th row
    for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
        const float *rp = x + row * row_stride;
        int64_t lcol = (int64_t)first * kBlock;
        V acc = V(0.0f);
        pipelined<DEPTH, V>(
            n,
            [&]() {
                V v = V(0.0f);
                if (FULL || lane_col < cols - lcol) v = load_stream(reinterpret_cast<const V *>(rp + lcol + lane_col));
                lcol += kBlock;
                return v;
            },
            [&](V v) { acc += v; });
        const float total = wave_sum(fold<VEC>(acc));
        if (lane == 0) part[wave] = total;
        __syncthreads();
        if (threadIdx.x == 0) {
            float sum = 0.0f;
            for (int w = 0; w < waves; ++w) sum = sum + part[w];
            out[row] = sum;
        }
        if (row + gridDim.x < rows) __syncthreads();  // part[] is rewritten for the next row
    }
}

// ----------------------------------------------------------------------------
// Row sums of narrow rows (1 to 128 columns).  A record packs R = 64 / L rows
// side by side: lane l serves row l / L of the record and its columns
// 4 (l mod L) .. 4 (l mod L) + 3, where L is the smallest power of two with
// 4 L >= cols.  Each lane folds its (up to) four floats, and the first
// log2(L) steps of the wave reduction -- which sum aligned groups of 2, 4,
// ... lanes -- give every lane its row's total; the group's first lane
// stores it.  A wave streams kRowSumsNarrowRecords records.  Lanes past the
// last row or column still issue their load, from the wave's first element,
// and the consumer drops the value, so every record is the same load
// instructions on every path, the producer never waits on its own loads,
// and the read-ahead keeps its partial waits.
// ----------------------------------------------------------------------------
template <bool VEC4, int LOG2L, int DEPTH>
__global__ __launch_bounds__(kWave) void row_sums_narrow_kernel(const float *__restrict__ x, int rows, int cols,
                                                                int64_t row_stride, float *__restrict__ out) {
    constexpr int L = 1 << LOG2L;
    constexpr int R = kWave / L;
    const int lane = lane_id();
    const int sub = lane >> LOG2L;     // row within the record
    const int q = lane & (L - 1);      // float4 column group within the row
    const int row0 = blockIdx.x * (R * kRowSumsNarrowRecords);
    const int left = rows - row0;      // rows of this wave's block that exist
    const int nrec = min(kRowSumsNarrowRecords, (left + R - 1) / R);
    const float *first = x + (int64_t)row0 * row_stride;
    int lrec = 0, crec = 0;
    pipelined<DEPTH, float4v>(
        nrec,
        [&]() {
            const int lr = lrec * R + sub;  // row within the wave's block
            const float *p = first + (int64_t)lr * row_stride + 4 * q;
            float4v v;
            if constexpr (VEC4) {
                v = load_stream(reinterpret_cast<const float4v *>(lr < left && 4 * q < cols ? p : first));
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) v[c] = load_stream(lr < left && 4 * q + c < cols ? p + c : first);
            }
            ++lrec;
            return v;
        },
        [&](float4v v) {
            const int lr = crec * R + sub;
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (!(lr < left && 4 * q + c < cols)) v[c] = 0.0f;
            const float total = group_sum<LOG2L>((v.x + v.y) + (v.z + v.w));
            if (q == 0 && lr < left) out[row0 + lr] = total;
            ++crec;
        });
}

// Read-ahead depths (records in the ring).  Each kernel instantiation owns its
// schedule; the macros let a tuning build override the defaults.
#ifndef LOOM_ROW_SUM_TILES_DEPTH
#define LOOM_ROW_SUM_TILES_DEPTH 4   // the ring holds one full tile (4 row pairs)
#endif
#ifndef LOOM_ROW_SUMS_DEPTH
#define LOOM_ROW_SUMS_DEPTH 6        // 5 KiB per wave in flight
#endif
#ifndef LOOM_ROW_SUMS_WIDE_DEPTH
#define LOOM_ROW_SUMS_WIDE_DEPTH 4   // 3 of a wave's 4 records issued at once; <= 128 VGPRs (16-wave groups)
#endif
constexpr int kRowSumTilesDepth = LOOM_ROW_SUM_TILES_DEPTH;
constexpr int kRowSumsWideDepth = LOOM_ROW_SUMS_WIDE_DEPTH;
constexpr int kRowSumsDepth = LOOM_ROW_SUMS_DEPTH;
#ifndef LOOM_ROW_SUMS_NARROW_DEPTH
#define LOOM_ROW_SUMS_NARROW_DEPTH 6
#endif
constexpr int kRowSumsNarrowDepth = LOOM_ROW_SUMS_NARROW_DEPTH;

template <bool VEC4>
static void launch_row_sums_narrow(dim3 grid, dim3 block, hipStream_t stream, const float *x, int rows, int cols,
                                   int64_t row_stride, float *out) {
    switch (row_sums_narrow_log2_lanes(cols)) {
        case 0: row_sums_narrow_kernel<VEC4, 0, kRowSumsNarrowDepth><<<grid, block, 0, stream>>>(x, rows, cols, row_stride, out); break;
        case 1: row_sums_narrow_kernel<VEC4, 1, kRowSumsNarrowDepth><<<grid, block, 0, stream>>>(x, rows, cols, row_stride, out); break;
        case 2: row_sums_narrow_kernel<VEC4, 2, kRowSumsNarrowDepth><<<grid, block, 0, stream>>>(x, rows, cols, row_stride, out); break;
        case 3: row_sums_narrow_kernel<VEC4, 3, kRowSumsNarrowDepth><<<grid, block, 0, stream>>>(x, rows, cols, row_stride, out); break;
        case 4: row_sums_narrow_kernel<VEC4, 4, kRowSumsNarrowDepth><<<grid, block, 0, stream>>>(x, rows, cols, row_stride, out); break;
        default: row_sums_narrow_kernel<VEC4, 5, kRowSumsNarrowDepth><<<grid, block, 0, stream>>>(x, rows, cols, row_stride, out); break;
    }
}

hipError_t launch_row_sum_tiles(const loom_launch_config &cfg, const float *values, int count,
                                const float *initial, float *sums, int32_t *final_row,
                                int32_t *tail_count, hipStream_t stream) {
    row_sum_tiles_kernel<kRowSumTilesDepth>
        <<<dim3(cfg.workgroups[0]), dim3(cfg.workgroup_size[0]), 0, stream>>>(values, count, initial, sums,
                                                                              final_row, tail_count);
    return hipGetLastError();
}

hipError_t launch_row_sums(const loom_launch_config &cfg, const float *x, int rows, int cols,
                           int64_t row_stride, float *out, hipStream_t stream) {
    const dim3 grid(cfg.workgroups[0]), block(cfg.workgroup_size[0]);
    const bool vec4 = (reinterpret_cast<uintptr_t>(x) % 16 == 0) && (row_stride % 4 == 0) && (cols % 4 == 0);
    if (row_sums_narrow_log2_lanes(cols) >= 0) {
        if (vec4)
            launch_row_sums_narrow<true>(grid, block, stream, x, rows, cols, row_stride, out);
        else
            launch_row_sums_narrow<false>(grid, block, stream, x, rows, cols, row_stride, out);
        return hipGetLastError();
    }
    if (row_sums_waves_per_row(cols) > 0) {
        if (vec4 && cols % (kWave * 4) == 0)
            row_sums_wide_kernel<4, true, kRowSumsWideDepth><<<grid, block, 0, stream>>>(x, rows, cols, row_stride, out);
        else if (vec4)
            row_sums_wide_kernel<4, false, kRowSumsWideDepth><<<grid, block, 0, stream>>>(x, rows, cols, row_stride, out);
        else if (cols % kWave == 0)
            row_sums_wide_kernel<1, true, kRowSumsWideDepth><<<grid, block, 0, stream>>>(x, rows, cols, row_stride, out);
        else
            row_sums_wide_kernel<1, false, kRowSumsWideDepth><<<grid, block, 0, stream>>>(x, rows, cols, row_stride, out);
        return hipGetLastError();
    }
    if (vec4) {
        if (cols % (kWave * 4) == 0)
            row_sums_kernel<4, true, kRowSumsDepth><<<grid, block, 0, stream>>>(x, rows, cols, row_stride, out);
        else
            row_sums_kernel<4, false, kRowSumsDepth><<<grid, block, 0, stream>>>(x, rows, cols, row_stride, out);
    } else {
        if (cols % kWave == 0)
            row_sums_kernel<1, true, kRowSumsDepth><<<grid, block, 0, stream>>>(x, rows, cols, row_stride, out);
        else
            row_sums_kernel<1, false, kRowSumsDepth><<<grid, block, 0, stream>>>(x, rows, cols, row_stride, out);
    }
    return hipGetLastError();
}

}  // namespace loom
