// device_common.hpp -- gfx950 (CDNA4, wave64) building blocks shared by the
// streaming-reduction kernels: wave reductions and the read-ahead pipeline.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.hpp"

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

// ---------------------------------------------------------------- read-ahead
// Software pipeline over n records in source order (TUNE §Choose the control:
// pipeline(depth); CTRL §Pipeline reads ahead of ordered computation).
//
//   load()      issues the next record's loads and returns the (pending) value;
//               called exactly n times, in order.
//   consume(v)  folds the oldest record into the ordered recurrence; called
//               exactly n times, in order.
//
// DEPTH-1 records stay in flight ahead of the consumer.  Loops of at least
// DEPTH-1 records take the pipelined path: an unconditional startup issues
// DEPTH-1 loads, the steady body (unrolled by DEPTH) issues one load and
// consumes the oldest record per step while at least 2*DEPTH-1 records
// remain, and the drain consumes the last DEPTH-1 .. 2*DEPTH-2 records,
// issuing the loads still missing.  The
// ring rotates by renaming, never by copying -- a slot receives its next load
// right after its old value was consumed -- and every path into the steady
// loop has issued the same loads in the same order, so the compiler keeps
// partial vmcnt waits (DEPTH-1 loads stay pending across each consume and
// across the backedge).  A scheduling fence (CTRL §Control instruction
// order: it orders instructions without waiting for loads) after each step's
// load keeps the compiler from sinking future loads below older consumer work
// such as LDS staging.  Loops shorter than DEPTH-1 run serially; an empty
// loop issues no load.
//
// Two forms of the drain.  The compact one is one unrolled loop whose loads
// depend on the remaining count.  The straight one (STRAIGHT_DRAIN) selects,
// by the number of loads still missing (0 .. DEPTH-1, wave-uniform), one of
// DEPTH branch-free sequences, each with the same fence after its loads as
// the steady body.  The compact form is smaller code; the straight form keeps
// every path free of ring copies and of a full wait on entry, which pays
// where the drain is much of the work (short per-wave loops) and costs
// registers elsewhere, so each kernel picks the form that measured faster.
template <int DEPTH, int EXTRA, typename T, typename Load, typename Consume>
__device__ __forceinline__ void pipelined_drain(T (&ring)[DEPTH], Load &load, Consume &consume) {
    // DEPTH-1 records are in the ring and EXTRA more remain to be loaded
#pragma unroll
    for (int j = 0; j < DEPTH - 1 + EXTRA; ++j) {
        if (j < EXTRA) {
            ring[(j + DEPTH - 1) % DEPTH] = load();
            __builtin_amdgcn_sched_barrier(0);
        }
        consume(ring[j % DEPTH]);
    }
}

template <int DEPTH, int E, typename T, typename Load, typename Consume>
__device__ __forceinline__ void pipelined_drain_select(int extra, T (&ring)[DEPTH], Load &load, Consume &consume) {
    if constexpr (E < DEPTH) {
        if (extra == E) {
            pipelined_drain<DEPTH, E>(ring, load, consume);
            return;
        }
        pipelined_drain_select<DEPTH, E + 1>(extra, ring, load, consume);
    }
}

template <int DEPTH, typename T, bool STRAIGHT_DRAIN = false, typename N, typename Load, typename Consume>
__device__ __forceinline__ void pipelined(N n, Load&& load, Consume&& consume) {
    if (DEPTH <= 1 || n < DEPTH - 1) {
        for (N i = 0; i < n; ++i) {
            T v = load();
            consume(v);
        }
        return;
    }
    if constexpr (DEPTH > 1) {
        T ring[DEPTH];
#pragma unroll
        for (int j = 0; j < DEPTH - 1; ++j) ring[j] = load();
        N i = 0;
        for (; i + 2 * DEPTH - 1 <= n; i += DEPTH) {
#pragma unroll
            for (int j = 0; j < DEPTH; ++j) {
                ring[(j + DEPTH - 1) % DEPTH] = load();
                __builtin_amdgcn_sched_barrier(0);
                consume(ring[j]);
            }
        }
        // DEPTH-1 <= n - i <= 2*DEPTH-2 records remain, DEPTH-1 of them loaded
        // (also when the steady loop ran zero times: then n - i = n).
        const int rest = (int)(n - i);
        if constexpr (STRAIGHT_DRAIN) {
            pipelined_drain_select<DEPTH, 0>(rest - (DEPTH - 1), ring, load, consume);
        } else {
#pragma unroll
            for (int j = 0; j < 2 * DEPTH - 1; ++j) {
                if (j < DEPTH - 1 || j < rest) {
                    if (j + DEPTH - 1 < rest) ring[(j + DEPTH - 1) % DEPTH] = load();
                    consume(ring[j % DEPTH]);
                }
            }
        }
    }
}

}  // namespace loom
