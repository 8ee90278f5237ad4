// probe.hip -- ep_probe_e4m3fn (include/ep_probe.h): the pack's clamp + FP8
// conversion applied to an array, for exhaustive checks of the conversion.
#include <stdint.h>

#include "ep_device.h"
#include "ep_internal.h"
#include "ep_probe.h"

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void probe_e4m3fn_kernel(const float4 *__restrict__ in,
                                                                uint32_t *__restrict__ out_hw,
                                                                uint32_t *__restrict__ out_sw,
                                                                int64_t n4)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += stride) {
        const float4 v = in[i];
        const float a = ep::clamp448(v.x), b = ep::clamp448(v.y), c = ep::clamp448(v.z),
                    d = ep::clamp448(v.w);
        if (out_hw)
            out_hw[i] = ep::e4m3fn_x4_hw(a, b, c, d);
        if (out_sw)
            out_sw[i] = ep::e4m3fn_x4_sw(a, b, c, d);
    }
}

} // namespace

extern "C" int ep_probe_e4m3fn(const float *in, uint8_t *out_hw, uint8_t *out_sw, int64_t n,
                               void *stream)
{
    if (n < 0 || n % 4 != 0)
        return EP_ERR_SHAPE;
    if (n == 0)
        return EP_OK;
    if (!in || (!out_hw && !out_sw))
        return EP_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(in) % 16 || reinterpret_cast<uintptr_t>(out_hw) % 16 ||
        reinterpret_cast<uintptr_t>(out_sw) % 16)
        return EP_ERR_ALIGN;
    const int64_t n4 = n / 4;
    const int64_t blocks = (n4 + kThreads - 1) / kThreads;
    const unsigned grid = (unsigned)(blocks < 65536 ? blocks : 65536);
    hipLaunchKernelGGL(probe_e4m3fn_kernel, dim3(grid), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), reinterpret_cast<const float4 *>(in),
                       reinterpret_cast<uint32_t *>(out_hw), reinterpret_cast<uint32_t *>(out_sw),
                       n4);
    return hipGetLastError() == hipSuccess ? EP_OK : EP_ERR_HIP;
}
