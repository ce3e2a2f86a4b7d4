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
#define LOOM_PACKED_DOT_DEPTH_WIDE 4  // 4 outputs per lane: 88 B per record
#endif
constexpr int kPackedDotDepth = LOOM_PACKED_DOT_DEPTH;
constexpr int kPackedDotDepthWide = LOOM_PACKED_DOT_DEPTH_WIDE;

template <int OPL> struct PackedRecord;
template <> struct PackedRecord<1> {
    int32_t word;       // four signed bytes, element j in byte j
    uint16_t scale;     // binary16 bits
    float4v act;        // the output's activation stream for this record
};
template <> struct PackedRecord<4> {
    int4v word;         // 4 consecutive outputs
    uint2v scale;       // their 4 binary16 scales
    float4v act[4];     // their 4 consecutive activation streams
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

// Each lane owns OPL consecutive outputs (the page: one, the output index is
// the lane of its [record][output] views).  Records are walked in order
// through the read-ahead ring; fields and scales are read once
// (non-temporal), the activation streams are shared by every output and stay
// cached.  OPL = 4 needs outputs and streams divisible by 4 (consecutive
// outputs then read consecutive streams) and 16-byte aligned rows.
template <int DEPTH, int OPL>
__global__ __launch_bounds__(256) void packed_dot_kernel(const int32_t *__restrict__ fields,
                                                         const uint16_t *__restrict__ scales,
                                                         const float *__restrict__ rhs, int streams,
                                                         const float *__restrict__ initial, int count,
                                                         int64_t outputs, float *__restrict__ out) {
    const int64_t o = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * OPL;
    if (o >= outputs) return;
    float sum[OPL];
#pragma unroll
    for (int i = 0; i < OPL; ++i) sum[i] = initial ? initial[o + i] : 0.0f;
    const int32_t *fp = fields + o;
    const uint16_t *sp = scales + o;
    const float4v *ap = reinterpret_cast<const float4v *>(rhs) + o % streams;
    pipelined<DEPTH, PackedRecord<OPL>>(
        count,
        [&]() {
            PackedRecord<OPL> q;
            if constexpr (OPL == 1) {
                q.word = load_stream(fp);
                q.scale = load_stream(sp);
                q.act = *ap;
            } else {
                q.word = load_stream(reinterpret_cast<const int4v *>(fp));
                q.scale = load_stream(reinterpret_cast<const uint2v *>(sp));
#pragma unroll
                for (int i = 0; i < 4; ++i) q.act[i] = ap[i];
            }
            fp += outputs;
            sp += outputs;
            ap += streams;
            return q;
        },
        [&](const PackedRecord<OPL> &q) {
            if constexpr (OPL == 1) {
                sum[0] = packed_step(sum[0], q.word, q.scale, q.act);
            } else {
                sum[0] = packed_step(sum[0], q.word.x, (uint16_t)(q.scale.x & 0xFFFF), q.act[0]);
                sum[1] = packed_step(sum[1], q.word.y, (uint16_t)(q.scale.x >> 16), q.act[1]);
                sum[2] = packed_step(sum[2], q.word.z, (uint16_t)(q.scale.y & 0xFFFF), q.act[2]);
                sum[3] = packed_step(sum[3], q.word.w, (uint16_t)(q.scale.y >> 16), q.act[3]);
            }
        });
#pragma unroll
    for (int i = 0; i < OPL; ++i) out[o + i] = sum[i];
}

hipError_t launch_packed_dot(const loom_launch_config &cfg, const int32_t *fields, const uint16_t *scales,
                             const float *rhs, int streams, const float *initial, int count, int64_t outputs,
                             float *out, hipStream_t stream) {
    const dim3 grid(cfg.workgroups[0]), block(cfg.workgroup_size[0]);
    if (packed_dot_outputs_per_lane(outputs, streams) == 4) {
        const bool aligned = reinterpret_cast<uintptr_t>(fields) % 16 == 0 && reinterpret_cast<uintptr_t>(scales) % 8 == 0;
        if (!aligned) return hipErrorInvalidValue;  // the entry point checks this first
        packed_dot_kernel<kPackedDotDepthWide, 4><<<grid, block, 0, stream>>>(fields, scales, rhs, streams, initial,
                                                                               count, outputs, out);
    } else {
        packed_dot_kernel<kPackedDotDepth, 1><<<grid, block, 0, stream>>>(fields, scales, rhs, streams, initial,
                                                                           count, outputs, out);
    }
    return hipGetLastError();
}

}  // namespace loom
