// pipeline.hpp -- the read-ahead loop every streaming kernel is built on.
//
// Plain C++ apart from two hooks, so that the same code can be compiled for
// the host and checked there: LOOM_PIPELINE_INLINE (the function qualifiers;
// a device build uses __device__ __forceinline__) and LOOM_SCHED_FENCE() (a
// scheduling fence on gfx950; nothing on the host).
#pragma once

#ifndef LOOM_PIPELINE_INLINE
#define LOOM_PIPELINE_INLINE __device__ __forceinline__
#endif
#ifndef LOOM_SCHED_FENCE
#define LOOM_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)
#endif

namespace loom {

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
LOOM_PIPELINE_INLINE void pipelined_drain(T (&ring)[DEPTH], Load &load, Consume &consume) {
    // DEPTH-1 records are in the ring and EXTRA more remain to be loaded
#pragma unroll
    for (int j = 0; j < DEPTH - 1 + EXTRA; ++j) {
        if (j < EXTRA) {
            ring[(j + DEPTH - 1) % DEPTH] = load();
            LOOM_SCHED_FENCE();
        }
        consume(ring[j % DEPTH]);
    }
}

template <int DEPTH, int E, typename T, typename Load, typename Consume>
LOOM_PIPELINE_INLINE void pipelined_drain_select(int extra, T (&ring)[DEPTH], Load &load, Consume &consume) {
    if constexpr (E < DEPTH) {
        if (extra == E) {
            pipelined_drain<DEPTH, E>(ring, load, consume);
            return;
        }
        pipelined_drain_select<DEPTH, E + 1>(extra, ring, load, consume);
    }
}

template <int DEPTH, typename T, bool STRAIGHT_DRAIN = false, typename N, typename Load, typename Consume>
LOOM_PIPELINE_INLINE void pipelined(N n, Load&& load, Consume&& consume) {
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
                LOOM_SCHED_FENCE();
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
