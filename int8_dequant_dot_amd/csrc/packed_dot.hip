// packed_dot.hip -- the pages' literal packed signed-byte dot recurrence on gfx950.
//
// TUNE = "Tune loop unrolling and pipelining" (Loom pages),
// §Apply the same controls to a packed dot product: 2,048 independent
// outputs over up to 128 records; each record brings one word of four packed
// signed bytes and one f16 scale per output and four f32 activations from one
// of 64 streams shared by all outputs; the consumer unpacks and scales the
// bytes and advances an ordered f32 dot accumulation.
#include "device_common.hpp"
#include "internal.hpp"

namespace loom {

#ifndef LOOM_PACKED_DOT_DEPTH
#define LOOM_PACKED_DOT_DEPTH 8  // records in flight per lane: the pages' shape is latency-bound
#endif
#ifndef LOOM_PACKED_DOT_DEPTH_WIDE
#define LOOM_PACKED_DOT_DEPTH_WIDE 6  // several outputs per lane
#endif
constexpr int kPackedDotDepth = LOOM_PACKED_DOT_DEPTH;
constexpr int kPackedDotDepthWide = LOOM_PACKED_DOT_DEPTH_WIDE;

struct PackedRecord {
    int32_t word;       // four signed bytes, element j in byte j
    uint16_t scale;     // binary16 bits
    float4v act;        // the output's activation stream for this record
};

// One record of one output: each of the four products is added to the
// carried sum in turn, one f32 rounding each -- the serial recurrence.
__device__ __forceinline__ float packed_step(float sum, int32_t word, uint16_t scale_bits, float4v act) {
    const float scale = (float)__builtin_bit_cast(_Float16, scale_bits);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float v = (float)(int8_t)(word >> (8 * j)) * scale;
        sum = sum + v * act[j];
    }
    return sum;
}

// One output per lane (the page's mapping: the output index is the lane of
// its [record][output] views).  Records are walked in order through the
// read-ahead ring; fields and scales are read once (non-temporal), the
// activation streams are shared by every output and stay cached.
template <int DEPTH>
__global__ __launch_bounds__(256) void packed_dot_kernel(const int32_t *__restrict__ fields,
                                                         const uint16_t *__restrict__ scales,
                                                         const float *__restrict__ rhs, int streams,
                                                         const float *__restrict__ initial, int count,
                                                         int64_t outputs, float *__restrict__ out) {
    const int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (o >= outputs) return;
    float sum = initial ? initial[o] : 0.0f;
    const int32_t *fp = fields + o;
    const uint16_t *sp = scales + o;
    const float4v *ap = reinterpret_cast<const float4v *>(rhs) + o % streams;
    pipelined<DEPTH, PackedRecord>(
        count,
        [&]() {
            PackedRecord q;
            q.word = load_stream(fp);
            q.scale = load_stream(sp);
            q.act = *ap;
            fp += outputs;
            sp += outputs;
            ap += streams;
            return q;
        },
        [&](const PackedRecord &q) { sum = packed_step(sum, q.word, q.scale, q.act); });
    out[o] = sum;
}

// Wide form with OPL outputs per lane spaced one wave apart: lane l of a wave
// whose block starts at output `base` (a multiple of 64 * OPL) owns outputs
// base + l + 64 j, j < OPL.  When the stream count divides 64, every one of
// them reads stream l mod streams, so a record needs a single 16-byte
// activation load per lane (one contiguous 1 KiB per wave), while each
// output's field word and scale still come from fully coalesced rows.
// Outputs past the end are clamped to the last one for loading and never
// stored.
template <int OPL> struct SpacedRecord {
    int32_t word[OPL];
    uint16_t scale[OPL];
    float4v act;
};

// The work of one wave.  FULL: all 64 * OPL outputs exist, so every load
// address is a wave-uniform row pointer (scalar registers) plus the lane's
// fixed 32-bit offset plus an immediate 256 j / 128 j: no per-record vector
// address arithmetic.  Otherwise outputs past the end are clamped to the
// last one for loading and never stored.
template <int DEPTH, int OPL, bool FULL>
__device__ __forceinline__ void packed_dot_spaced_wave(const int32_t *__restrict__ fields,
                                                       const uint16_t *__restrict__ scales,
                                                       const float *__restrict__ rhs, int streams,
                                                       const float *__restrict__ initial, int count,
                                                       int64_t outputs, float *__restrict__ out, int64_t base) {
    const int lane = lane_id();
    int lo[OPL];  // the lane's outputs, relative to base
    float sum[OPL];
#pragma unroll
    for (int j = 0; j < OPL; ++j) {
        lo[j] = FULL ? lane + kWave * j : (int)(min(base + lane + kWave * j, outputs - 1) - base);
        sum[j] = initial ? initial[base + lo[j]] : 0.0f;
    }
    const int32_t *fp = fields + base;
    const uint16_t *sp = scales + base;
    const float4v *ap = reinterpret_cast<const float4v *>(rhs);
    const int act = lane % streams;
    // the straight drain measured about 2 % faster here (128 records)
    pipelined<DEPTH, SpacedRecord<OPL>, true>(
        count,
        [&]() {
            SpacedRecord<OPL> q;
#pragma unroll
            for (int j = 0; j < OPL; ++j) {
                q.word[j] = load_stream(fp + lo[j]);
                q.scale[j] = load_stream(sp + lo[j]);
            }
            q.act = ap[act];
            fp += outputs;
            sp += outputs;
            ap += streams;
            return q;
        },
        [&](const SpacedRecord<OPL> &q) {
#pragma unroll
            for (int j = 0; j < OPL; ++j) sum[j] = packed_step(sum[j], q.word[j], q.scale[j], q.act);
        });
#pragma unroll
    for (int j = 0; j < OPL; ++j)
        if (FULL || base + lane + kWave * j < outputs) out[base + lane + kWave * j] = sum[j];
}

template <int DEPTH, int OPL>
__global__ __launch_bounds__(256) void packed_dot_spaced_kernel(const int32_t *__restrict__ fields,
                                                                const uint16_t *__restrict__ scales,
                                                                const float *__restrict__ rhs, int streams,
                                                                const float *__restrict__ initial, int count,
                                                                int64_t outputs, float *__restrict__ out) {
    // the wave index within the workgroup is the same in every lane
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const int64_t base = ((int64_t)blockIdx.x * (blockDim.x / kWave) + wave) * (kWave * OPL);
    if (base >= outputs) return;
    if (base + kWave * OPL <= outputs)
        packed_dot_spaced_wave<DEPTH, OPL, true>(fields, scales, rhs, streams, initial, count, outputs, out, base);
    else
        packed_dot_spaced_wave<DEPTH, OPL, false>(fields, scales, rhs, streams, initial, count, outputs, out, base);
}

hipError_t launch_packed_dot(const loom_launch_config &cfg, const int32_t *fields, const uint16_t *scales,
                             const float *rhs, int streams, const float *initial, int count, int64_t outputs,
                             float *out, hipStream_t stream) {
    const dim3 grid(cfg.workgroups[0]), block(cfg.workgroup_size[0]);
    if (packed_dot_outputs_per_lane(outputs, streams) > 1)
        packed_dot_spaced_kernel<kPackedDotDepthWide, kPackedDotWide><<<grid, block, 0, stream>>>(
            fields, scales, rhs, streams, initial, count, outputs, out);
    else
        packed_dot_kernel<kPackedDotDepth><<<grid, block, 0, stream>>>(fields, scales, rhs, streams, initial, count,
                                                                       outputs, out);
    return hipGetLastError();
}

}  // namespace loom
