// copy.hip -- the over-dispatched guarded copy of "Kernels and launch
// configuration" (§Over-dispatch safely and preserve the proof).
#include "device_common.hpp"
#include "internal.hpp"

namespace loom {

// One element per work-item on ceil(n / 256) workgroups; the final workgroup
// guards its tail with the logical element count.
__global__ __launch_bounds__(256) void copy_f32_kernel(const float *__restrict__ in, float *__restrict__ out,
                                                       int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] = in[i];
}

hipError_t launch_copy_f32(const loom_launch_config &cfg, const float *in, float *out, int64_t n,
                           hipStream_t stream) {
    copy_f32_kernel<<<dim3(cfg.workgroups[0]), dim3(cfg.workgroup_size[0]), 0, stream>>>(in, out, n);
    return hipGetLastError();
}

}  // namespace loom
