// Fused mixed-precision AdamW step on one rank's shard (gfx950).
//
// Per element: read bf16 gradient and fp32 master / m / v, write fp32 master /
// m / v and the bf16 working copy: 28 bytes of HBM traffic.  The update is
// computed in double (about 15 fp64 operations with three divisions and a
// square root, the order of the published update, see adamw_update), which
// leaves the kernel bound by HBM bandwidth as fp32 would: on the same buffers
// it ran at 5,971 GB/s against 5,970 for an fp32 evaluation, and every state
// is the correctly rounded value of the double computation.  Each lane moves 4
// consecutive elements: one dwordx4 of master, m and v in and out, a dwordx2 of
// gradient in and of bf16 copy out, so every wave instruction touches 1 KB (or
// 512 B) of contiguous memory.  One group per lane over a grid that covers the
// shard, non-temporal loads and stores, and at most 5 workgroups per CU (set
// by reserving LDS the kernel never touches): on MI355X, seven concurrent
// streams lose DRAM row locality when every CU is full of waves, and capping
// the residency lifts the sustained rate from about 5.8 to 6.3 TB/s.  No MFMA.
//
// Sources (web pages on DeepSpeed ZeRO-3):
//  - "From DDP to ZeRO: memory sharding" blog (111qqz.com): ledger section
//    (bf16 params and grads, fp32 master, m, v) and "ZeRO-1: why optimizer
//    states can be sharded" (an element's update needs only its own gradient
//    and state, so each rank updates its slice alone);
//  - ZeRO-1/2/3 concept page (compassingai.com), Stage 1 mechanism: the fp32
//    state and master are updated from the reduced gradient and the 16-bit copy
//    is made from the updated fp32 master;
//  - ZeRO tutorial (cnhsyj.com) 3.1: AdamW with lr, betas, eps, weight_decay.
// The update is decoupled-weight-decay Adam (Loshchilov & Hutter, ICLR 2019).
#include "zr_math.hpp"

namespace zr {

// Dynamic LDS reserved per workgroup: 32 KB -> 5 workgroups of 256 per CU.
#ifndef ZR_ADAMW_LDS_CAP
#define ZR_ADAMW_LDS_CAP (32 * 1024)
#endif

__device__ __forceinline__ void adamw_one(const uint16_t *grad, float *master, float *m, float *v,
                                          uint16_t *param, int64_t j, const AdamWScalars &s)
{
    float th = master[j], mm = m[j], vv = v[j];
    adamw_element(bf16_to_f32(grad[j]), th, mm, vv, s);
    master[j] = th;
    m[j] = mm;
    v[j] = vv;
    if (param)
        param[j] = (uint16_t)f32_to_bf16(th);
}

// Vector body over `groups` groups of 4 elements starting at element `head`
// (where master, m and v are 16-byte and gradient and copy 8-byte aligned),
// plus the unaligned head [0, head) and the tail after the last group, done
// element-wise by block 0.
template <bool kParam>
__global__ __launch_bounds__(kBlock) void adamw_vec_kernel(const uint16_t *grad, float *master, float *m, float *v,
                                                           uint16_t *param, int64_t numel, int64_t head,
                                                           int64_t groups, AdamWScalars s)
{
    const u32x2 *g2 = reinterpret_cast<const u32x2 *>(grad + head);
    f32x4 *th4 = reinterpret_cast<f32x4 *>(master + head);
    f32x4 *m4 = reinterpret_cast<f32x4 *>(m + head);
    f32x4 *v4 = reinterpret_cast<f32x4 *>(v + head);
    u32x2 *p2 = kParam ? reinterpret_cast<u32x2 *>(param + head) : nullptr;

    for (int64_t i = first_tile<kAdamwOrder>() * kBlock + threadIdx.x; i < groups; i += grid_stride()) {
        u32x2 g = load_stream(g2 + i);
        f32x4 a = load_stream(th4 + i);
        f32x4 mm = load_stream(m4 + i);
        f32x4 vv = load_stream(v4 + i);

        float gr[4] = {bf16_lo(g.x), bf16_hi(g.x), bf16_lo(g.y), bf16_hi(g.y)};
        float th[4] = {a.x, a.y, a.z, a.w};
        float mo[4] = {mm.x, mm.y, mm.z, mm.w};
        float vo[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
            adamw_element(gr[e], th[e], mo[e], vo[e], s);

        store_stream(th4 + i, f32x4{th[0], th[1], th[2], th[3]});
        store_stream(m4 + i, f32x4{mo[0], mo[1], mo[2], mo[3]});
        store_stream(v4 + i, f32x4{vo[0], vo[1], vo[2], vo[3]});
        if (kParam)
            store_stream(p2 + i, u32x2{pack_bf16x2(th[0], th[1]), pack_bf16x2(th[2], th[3])});
    }

    if (blockIdx.x == 0) {
        int64_t tail_start = head + 4 * groups;
        int64_t edge = head + (numel - tail_start);  // at most 63 + 3
        if ((int64_t)threadIdx.x < edge) {
            int64_t j = (int64_t)threadIdx.x < head ? (int64_t)threadIdx.x : tail_start + (threadIdx.x - head);
            adamw_one(grad, master, m, v, kParam ? param : nullptr, j, s);
        }
    }
}

// Fallback when the buffers' 16-byte phases disagree: element-wise, same bits.
__global__ __launch_bounds__(kBlock) void adamw_scalar_kernel(const uint16_t *grad, float *master, float *m, float *v,
                                                              uint16_t *param, int64_t numel, AdamWScalars s)
{
    for (int64_t j = global_tid(); j < numel; j += grid_stride())
        adamw_one(grad, master, m, v, param, j, s);
}

int adamw_scalar_slots(ScalarSlot *out)
{
    out[0] = slot_of(adamw_vec_kernel<true>);
    out[1] = slot_of(adamw_vec_kernel<false>);
    out[2] = slot_of(adamw_scalar_kernel);
    return 3;
}

zr_status adamw_run(const uint16_t *g, float *master, float *exp_avg, float *exp_avg_sq, uint16_t *p, int64_t numel,
                    const AdamWScalars &s, hipStream_t st)
{
    // elements before master starts a 128-byte line (the gradient's line too
    // when one index starts both); the other buffers must then be aligned
    // (16 B for fp32, 8 B for bf16) for the vector body
    const int64_t head = line_head32(master, g, numel);
    bool vec = aligned_to(exp_avg + head, 16) && aligned_to(exp_avg_sq + head, 16) && aligned_to(g + head, 8) &&
               (!p || aligned_to(p + head, 8));
    if (vec) {
        int64_t groups = (numel - head) / 4;
        dim3 grid = order_grid<kAdamwOrder>((groups + kBlock - 1) / kBlock);
        if (p)
            return launch(adamw_vec_kernel<true>, grid, dim3(kBlock), ZR_ADAMW_LDS_CAP, st, g, master, exp_avg,
                          exp_avg_sq, p, numel, head, groups, s);
        return launch(adamw_vec_kernel<false>, grid, dim3(kBlock), ZR_ADAMW_LDS_CAP, st, g, master, exp_avg,
                      exp_avg_sq, p, numel, head, groups, s);
    }
    dim3 grid = grid_of((numel + kBlock - 1) / kBlock);
    return launch(adamw_scalar_kernel, grid, dim3(kBlock), 0, st, g, master, exp_avg, exp_avg_sq, p, numel, s);
}

}  // namespace zr

using namespace zr;

extern "C" zr_status zr_adamw_step(const void *grad, float *master, float *exp_avg, float *exp_avg_sq, void *param_out,
                                   int64_t numel, const zr_adamw_hparams *hp, void *stream)
{
    clear_error();
    zr_status st0 = check_adamw_hparams("zr_adamw_step", hp);
    if (st0 != ZR_OK)
        return st0;
    if (numel < 0)
        return fail(ZR_EINVAL, "zr_adamw_step: numel < 0");
    if (numel > 0 && (!grad || !master || !exp_avg || !exp_avg_sq))
        return fail(ZR_EINVAL, "zr_adamw_step: NULL buffer");
    if (!aligned_to(grad, 2) || !aligned_to(param_out, 2) || !aligned_to(master, 4) || !aligned_to(exp_avg, 4) ||
        !aligned_to(exp_avg_sq, 4))
        return fail(ZR_EALIGN, "zr_adamw_step: buffers must be naturally aligned (bf16: 2 B, fp32: 4 B)");
    {
        const void *p[5] = {grad, master, exp_avg, exp_avg_sq, param_out};
        int64_t b[5] = {2 * numel, 4 * numel, 4 * numel, 4 * numel, param_out ? 2 * numel : 0};
        int x, y;
        if (any_overlap(p, b, 5, &x, &y))
            return fail(ZR_EINVAL, "zr_adamw_step: buffers %d and %d overlap", x, y);
    }
    if (numel == 0)
        return ZR_OK;
    return adamw_run(static_cast<const uint16_t *>(grad), master, exp_avg, exp_avg_sq,
                     static_cast<uint16_t *>(param_out), numel, adamw_scalars(*hp), static_cast<hipStream_t>(stream));
}
