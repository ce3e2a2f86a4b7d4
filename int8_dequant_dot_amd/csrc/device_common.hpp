// device_common.hpp -- gfx950 (CDNA4, wave64) building blocks shared by the
// streaming-reduction kernels: wave reductions and the read-ahead pipeline.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.hpp"
#include "pipeline.hpp"

namespace loom {

constexpr int kWave = 64;          // gfx950 wavefront width

typedef int   int4v   __attribute__((ext_vector_type(4)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned uint2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// Load of data that is streamed exactly once (rows, segment rows, weights):
// a non-temporal load, so the lines are not kept in the caches at the expense
// of data that is reused (the int8 activations).  On MI355X this raises the
// sustained read rate of per-wave contiguous streams by ~12%.
template <typename V>
__device__ __forceinline__ V load_stream(const V *p) {
    return __builtin_nontemporal_load(p);
}

// ---------------------------------------------------------------- cross-lane moves
// DPP controls (GFX9 encoding): quad_perm[1,0,3,2], quad_perm[2,3,0,1],
// row_half_mirror (lane i <- 7-i within 8), row_mirror (lane i <- 15-i within 16).
constexpr int kDppQuadSwap1 = 0xB1;
constexpr int kDppQuadSwap2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
// ds_swizzle bit mode: and_mask 0x1F, or_mask 0, xor_mask 0x10 -> lane ^ 16
// inside each group of 32 lanes.
constexpr int kSwizzleXor16 = (0x10 << 10) | 0x1F;

template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, dpp<CTRL>(__builtin_bit_cast(int, v)));
}
__device__ __forceinline__ int swz16(int v) { return __builtin_amdgcn_ds_swizzle(v, kSwizzleXor16); }
__device__ __forceinline__ float swz16(float v) {
    return __builtin_bit_cast(float, swz16(__builtin_bit_cast(int, v)));
}

// Sum over each group of 32 lanes; every lane of a group receives the same
// bits (each step adds two equal-shaped partial sums, and a + b == b + a).
// All 64 lanes must be active.
template <typename T>
__device__ __forceinline__ T half_wave_sum(T v) {
    v = v + dpp<kDppQuadSwap1>(v);
    v = v + dpp<kDppQuadSwap2>(v);
    v = v + dpp<kDppHalfMirror>(v);
    v = v + dpp<kDppMirror>(v);
    v = v + swz16(v);
    return v;
}

// Sum over each aligned group of 2^LOG2L lanes (LOG2L <= 5): the first
// LOG2L steps of half_wave_sum.  Every lane of a group receives its sum.
template <int LOG2L, typename T>
__device__ __forceinline__ T group_sum(T v) {
    if constexpr (LOG2L >= 1) v = v + dpp<kDppQuadSwap1>(v);
    if constexpr (LOG2L >= 2) v = v + dpp<kDppQuadSwap2>(v);
    if constexpr (LOG2L >= 3) v = v + dpp<kDppHalfMirror>(v);
    if constexpr (LOG2L >= 4) v = v + dpp<kDppMirror>(v);
    if constexpr (LOG2L >= 5) v = v + swz16(v);
    return v;
}

__device__ __forceinline__ float readlane(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ int readlane(int v, int l) { return __builtin_amdgcn_readlane(v, l); }

// Full wave64 sum, returned as a wave-uniform value (the subgroup reduction
// of TUNE §Derive full tiles; the result reaches every lane).  All lanes must
// be active.  For int the result is exact; for float the order is a fixed
// tree: pairs, quads, eights, sixteens, the two 16-lane halves of each 32,
// then the two 32-lane halves.
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
    v = half_wave_sum(v);
    return readlane(v, 0) + readlane(v, 32);
}

}  // namespace loom
