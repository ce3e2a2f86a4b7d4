// routed_combine.hip -- the routed row combine on gfx950.
//
// TUNE = "Tune loop unrolling and pipelining" (Loom pages), §Separate route
// and payload lookahead: a routed MoE combine reads a row id, then the
// selected expert-output row and the route's weight, and accumulates the
// weighted rows in route order; missing ids suppress both reads.
#include "device_common.hpp"
#include "internal.hpp"

namespace loom {

#ifndef LOOM_ROUTED_DEPTH
#define LOOM_ROUTED_DEPTH 8   // ring depth: up to 7 payload rows in flight per wave
#endif
constexpr int kRoutedDepth = LOOM_ROUTED_DEPTH;
constexpr int kRoutedVecs = kRoutedColumnsPerWave / (kWave * 4);  // float4s per lane per route

// Buffer descriptor word 3 for raw (untyped, 32-bit) buffer access on GFX9.
constexpr int kRawBufferWord3 = 0x00020000;
// Cache-policy bits of a buffer load: non-temporal (the payload is read once).
constexpr int kBufferNonTemporal = 2;

template <int VECS>
struct RoutedRecord {
    float4v p[VECS];  // this lane's columns of the route's payload row (0 if missing)
    float w;      // the route's weight (wave-uniform)
    int valid;    // the route's id is in range (wave-uniform)
};

// One wave per token and block of kRoutedColumnsPerWave columns (VECS 1 KiB
// slices of the selected row per route).  The pages stage the id two
// routes ahead of the payload; here the ids and weights of 64 routes arrive
// in one coalesced load (lane j holds route j) before that chunk's payload
// stream starts, and v_readlane hands each route's id to the producer as a
// wave-uniform value, so the dependent id -> row step costs one load
// latency per 64 routes, not one per route.  Each payload load goes through
// a buffer descriptor covering exactly the selected row -- or nothing, for
// a missing route: the hardware then returns zeros without touching memory.
// The load is issued either way, so every path issues the same loads and
// the ring keeps its partial waits.  The accumulation is in route order, the
// product rounded and then added, as a serial loop computes it.
template <int DEPTH, int VECS>
__global__ __launch_bounds__(kWave) void routed_combine_kernel(const int32_t *__restrict__ ids,
                                                               const float *__restrict__ weights,
                                                               const float *__restrict__ payload, uint32_t num_rows,
                                                               int64_t tokens, int routes, int hidden,
                                                               float *__restrict__ out) {
    const int lane = lane_id();
    const int cb = blockIdx.y * (kWave * 4 * VECS);
    const int c = cb + lane * 4;  // first column of slice 0; slice v adds 256 v
    const uint32_t row_bytes = (uint32_t)hidden * 4u;
    const int lane_offset = c * 4;
    // one token per wave; past the grid's work-item limit, every grid.x-th token
    for (int64_t t = blockIdx.x; t < tokens; t += gridDim.x) {
        const int32_t *tid = ids + t * routes;
        const float *tw = weights + t * routes;

        float4v acc[VECS];
#pragma unroll
        for (int v = 0; v < VECS; ++v) acc[v] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
        // Routes come in chunks of 64: one coalesced metadata load per chunk,
        // then the payload stream of that chunk.  The empty asm makes the
        // metadata opaque, so the compiler keeps it in registers instead of
        // re-loading it (with a full wait) at every use.
        for (int chunk = 0; chunk < routes; chunk += kWave) {
            const int j = chunk + lane;
            int idv = j < routes ? tid[j] : -1;
            float wv = (j < routes && (uint32_t)idv < num_rows) ? tw[j] : 0.0f;
            asm volatile("" : "+v"(idv), "+v"(wv));
            int li = 0;
            pipelined<DEPTH, RoutedRecord<VECS>>(
                min(kWave, routes - chunk),
                [&]() {
                    RoutedRecord<VECS> q;
                    const uint32_t id = (uint32_t)readlane(idv, li);
                    q.valid = id < num_rows;
                    q.w = readlane(wv, li);
                    const float *row = payload + (int64_t)(q.valid ? id : 0) * hidden;
                    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
                        const_cast<float *>(row), 0, q.valid ? row_bytes : 0u, kRawBufferWord3);
#pragma unroll
                    for (int v = 0; v < VECS; ++v)
                        q.p[v] = __builtin_bit_cast(
                            float4v, __builtin_amdgcn_raw_buffer_load_b128(rsrc, lane_offset + v * kWave * 16, 0,
                                                                           kBufferNonTemporal));
                    ++li;
                    return q;
                },
                [&](const RoutedRecord<VECS> &q) {
                    if (q.valid) {
#pragma unroll
                        for (int v = 0; v < VECS; ++v) {
                            acc[v].x = acc[v].x + q.w * q.p[v].x;
                            acc[v].y = acc[v].y + q.w * q.p[v].y;
                            acc[v].z = acc[v].z + q.w * q.p[v].z;
                            acc[v].w = acc[v].w + q.w * q.p[v].w;
                        }
                    }
                });
        }
#pragma unroll
        for (int v = 0; v < VECS; ++v)
            if (c + v * kWave * 4 < hidden)
                *reinterpret_cast<float4v *>(out + t * hidden + c + v * kWave * 4) = acc[v];
    }
}

hipError_t launch_routed_combine(const loom_launch_config &cfg, const int32_t *ids, const float *weights,
                                 const float *payload, int64_t num_rows, int64_t tokens, int routes, int hidden,
                                 float *out, hipStream_t stream) {
    routed_combine_kernel<kRoutedDepth, kRoutedVecs>
        <<<dim3(cfg.workgroups[0], cfg.workgroups[1]), dim3(cfg.workgroup_size[0]), 0, stream>>>(
            ids, weights, payload, (uint32_t)num_rows, tokens, routes, hidden, out);
    return hipGetLastError();
}

}  // namespace loom
