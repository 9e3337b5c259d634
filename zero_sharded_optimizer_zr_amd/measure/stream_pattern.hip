// Measurement kernel for the bench, outside the method: the memory-access
// pattern of the fused AdamW kernel (zr_adamw_step) with its arithmetic taken
// out.  Same launch shape as that kernel -- 256 lanes per workgroup, 4
// consecutive elements per lane, one group per lane over a grid that covers the
// array, the tiles in the same order (kAdamwOrder), non-temporal loads and
// stores, 32 KB of dynamic LDS reserved and never touched so that at most 5
// workgroups share a CU -- and the same eight streams:
// a dwordx2 load of the bf16 gradient, dwordx4 loads and stores of the fp32
// master, m and v, a dwordx2 store of the bf16 copy.  Each state value is
// multiplied by `one` (1.0 at run time, so the values stay as they were and
// the stores cannot be folded away) and the gradient bits are stored as the
// copy: 28 bytes per element, about 3 operations instead of about 20.  Timed on
// the same buffers as the AdamW kernel, it gives the bandwidth that access
// pattern reaches on this placement: the ceiling the AdamW rate is compared
// with.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "zr_device.hpp"

namespace {

using namespace zr;

__global__ __launch_bounds__(kBlock) void adamw_pattern_kernel(const u32x2 *grad, f32x4 *master, f32x4 *m, f32x4 *v,
                                                                u32x2 *param, int64_t groups, float one)
{
    for (int64_t i = first_tile<kAdamwOrder>() * kBlock + threadIdx.x; i < groups; i += grid_stride()) {
        u32x2 g = load_stream(grad + i);
        f32x4 a = load_stream(master + i);
        f32x4 mm = load_stream(m + i);
        f32x4 vv = load_stream(v + i);
        store_stream(master + i, a * one);
        store_stream(m + i, mm * one);
        store_stream(v + i, vv * one);
        store_stream(param + i, g);
    }
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace

// Returns 0, or -1 when the buffers or the count do not fit the vector body
// (master, m, v 16-byte aligned; grad and param 8-byte aligned; numel a
// multiple of 4) or the launch fails.
extern "C" __attribute__((visibility("default"))) int zr_measure_adamw_pattern(const void *grad, float *master,
                                                                                float *m, float *v, void *param,
                                                                                int64_t numel, void *stream)
{
    if (numel <= 0 || numel % 4 || !aligned(master, 16) || !aligned(m, 16) || !aligned(v, 16) ||
        !aligned(grad, 8) || !aligned(param, 8))
        return -1;
    const int64_t groups = numel / 4;
    int64_t blocks = (groups + kBlock - 1) / kBlock;
    if (kAdamwOrder == kOneRun)
        blocks = (blocks + kXcds - 1) / kXcds * kXcds;
    if (blocks > 0x7ffffff8)
        blocks = 0x7ffffff8;
    hipLaunchKernelGGL(adamw_pattern_kernel, dim3((unsigned)blocks), dim3(kBlock), 32 * 1024,
                       static_cast<hipStream_t>(stream), static_cast<const u32x2 *>(grad),
                       reinterpret_cast<f32x4 *>(master), reinterpret_cast<f32x4 *>(m),
                       reinterpret_cast<f32x4 *>(v), static_cast<u32x2 *>(param), groups, 1.0f);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}
