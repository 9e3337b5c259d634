// Fused gradient mean + AdamW on one rank's shard (gfx950): the ReduceScatter
// arithmetic and the optimizer step in one pass, without the bf16 gradient
// round trip through HBM.
//
// Per element it reads n bf16 contributions and fp32 master / m / v, writes
// fp32 master / m / v and the bf16 copy (and, on request, the bf16 mean):
// 2n + 26 bytes instead of (2n + 2) + 28 for the two kernels in sequence.  The
// mean is rounded to bf16 before the update exactly as the reduce kernel stores
// it, and both steps use the same per-element functions, so the result is bit
// for bit that of zr_reduce_slice followed by zr_adamw_step.
//
// Each lane takes 4 consecutive elements: dwordx2 loads of the contributions
// (all of them in flight for up to 8, else four at a time), dwordx4 loads and
// stores of master, m and v, a dwordx2 store of the copy; non-temporal, one
// group per lane over a grid that covers the shard, residency capped per
// contribution count with reserved LDS the kernel never touches, tiles in runs
// of 256 per XCD (kFusedOrder).  Eight elements per lane and eight or sixteen
// contribution loads in flight at n = 64 measured slower on MI355X (same
// buffers: n = 64 5.80 against 5.49-5.54 TB/s for wider batches, 5.25-5.66 for
// eight elements per lane).
//
// Above 24 contributions the entry point runs the reduce kernel and then the
// AdamW kernel instead (see kFusedMaxN), with the mean in grad_out or, when only
// the copy is asked for, in param_out; the bits are the same either way.  With
// neither output the one-pass kernel runs at any n.
//
// Sources (web pages on DeepSpeed ZeRO-3): "From DDP to ZeRO: memory sharding"
// blog (111qqz.com), "ZeRO-2: why gradients can be sharded too" (after the
// ReduceScatter each rank updates its parameter shard with its gradient shard)
// and "ZeRO-1: why optimizer states can be sharded" (elementwise update);
// ZeRO-1/2/3 concept page (compassingai.com), Stage 1/2 mechanism (reduce the
// gradient slice, then update the fp32 state and master and make the 16-bit
// copy).
#include "zr_math.hpp"

namespace zr {

// Contribution loads in flight per lane: all of them for up to 8 contributions
// (at n = 8, 1.1-2.5% faster than two batches of 4 on the 1T and GPT shards),
// batches of 4 above.
template <int MaxN>
constexpr int fused_batch() { return MaxN == 8 ? 8 : 4; }

// Largest contribution count the one-pass kernel takes when a two-pass schedule
// is possible.  Its saving is the bf16 mean's write and read (2 or 4 of 2n + 26
// bytes per element), a share that shrinks as n grows, while its n + 4
// concurrent streams, read with 8-byte loads, lose DRAM efficiency against the
// reduce kernel's 16-byte loads at 2 workgroups per CU.  Measured on MI355X
// (1.05e8 elements, same buffers, one pass against reduce then AdamW): one pass
// faster by 8% at n = 4, 7% at n = 8, 1% at n = 24; two passes faster by 0.5%
// at n = 32 and 5.5% at n = 64.
constexpr int32_t kFusedMaxN = 24;

// Dynamic LDS reserved per workgroup (160 KB per CU): residency cap by the
// number of concurrent streams, n contributions + 4 state/copy streams.
// Measured on MI355X: n = 4 best at 5 workgroups per CU, n = 8 and n = 64 at 4
// (n = 64 at 2 per CU loses a fifth: its 8-byte contribution loads keep fewer
// bytes in flight per lane than the reduce kernel's 16-byte loads).
inline size_t fused_cap_lds(int32_t n)
{
    return n > 4 ? 40 * 1024 : 32 * 1024;
}

template <int MaxN>
__device__ __forceinline__ void fused_one(const ContribTable<MaxN> &c, int32_t n, float *master, float *m, float *v,
                                          uint16_t *param, uint16_t *gout, int64_t j, const MeanDivisor &d,
                                          const AdamWScalars &s)
{
    uint16_t gb = reduce_one(c, n, j, d);
    if (gout)
        gout[j] = gb;
    float th = master[j], mm = m[j], vv = v[j];
    adamw_element(bf16_to_f32(gb), th, mm, vv, s);
    master[j] = th;
    m[j] = mm;
    v[j] = vv;
    if (param)
        param[j] = (uint16_t)f32_to_bf16(th);
}

// Vector body over `groups` groups of 4 elements from element `head` (master,
// m, v 16-byte aligned there; contributions, copy and mean 8-byte aligned);
// block 0 also does the head [0, head) and the tail element-wise.
// Tile order (first_tile): runs of 256 tiles per XCD, 1-8% faster than launch
// order on the same buffers (most on shards of about 1e8 elements).
constexpr int kFusedOrder = 256;

template <int MaxN, bool kParam, bool kGrad>
__global__ __launch_bounds__(kBlock) void fused_vec_kernel(ContribTable<MaxN> c, int32_t n, float *master, float *m,
                                                           float *v, uint16_t *param, uint16_t *gout, int64_t numel,
                                                           int64_t head, int64_t groups, MeanDivisor d,
                                                           AdamWScalars s)
{
    f32x4 *th4 = reinterpret_cast<f32x4 *>(master + head);
    f32x4 *m4 = reinterpret_cast<f32x4 *>(m + head);
    f32x4 *v4 = reinterpret_cast<f32x4 *>(v + head);
    u32x2 *p2 = kParam ? reinterpret_cast<u32x2 *>(param + head) : nullptr;
    u32x2 *o2 = kGrad ? reinterpret_cast<u32x2 *>(gout + head) : nullptr;

    for (int64_t i = first_tile<kFusedOrder>() * kBlock + threadIdx.x; i < groups; i += grid_stride()) {
        f32x4 a = load_stream(th4 + i);
        f32x4 mm = load_stream(m4 + i);
        f32x4 vv = load_stream(v4 + i);
        float acc[4];
        constexpr int kB = fused_batch<MaxN>();
        for (int32_t k = 0; k < n; k += kB) {
            u32x2 x[kB];
#pragma unroll
            for (int u = 0; u < kB; ++u)
                if (k + u < n)
                    x[u] = load_stream(reinterpret_cast<const u32x2 *>(c.p[k + u] + head) + i);
#pragma unroll
            for (int u = 0; u < kB; ++u) {
                if (k + u == 0) {
                    acc[0] = bf16_lo(x[u].x);
                    acc[1] = bf16_hi(x[u].x);
                    acc[2] = bf16_lo(x[u].y);
                    acc[3] = bf16_hi(x[u].y);
                } else if (k + u < n) {
                    acc[0] += bf16_lo(x[u].x);
                    acc[1] += bf16_hi(x[u].x);
                    acc[2] += bf16_lo(x[u].y);
                    acc[3] += bf16_hi(x[u].y);
                }
            }
        }
        // the mean as the reduce kernel stores it: rounded to bf16
        uint32_t gb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            gb[e] = f32_to_bf16(finish_mean(acc[e], d));
        float th[4] = {a.x, a.y, a.z, a.w};
        float mo[4] = {mm.x, mm.y, mm.z, mm.w};
        float vo[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
            adamw_element(__uint_as_float(gb[e] << 16), th[e], mo[e], vo[e], s);

        store_stream(th4 + i, f32x4{th[0], th[1], th[2], th[3]});
        store_stream(m4 + i, f32x4{mo[0], mo[1], mo[2], mo[3]});
        store_stream(v4 + i, f32x4{vo[0], vo[1], vo[2], vo[3]});
        if (kParam)
            store_stream(p2 + i, u32x2{pack_bf16x2(th[0], th[1]), pack_bf16x2(th[2], th[3])});
        if (kGrad)
            store_stream(o2 + i, u32x2{gb[0] | (gb[1] << 16), gb[2] | (gb[3] << 16)});
    }

    if (blockIdx.x == 0) {
        int64_t tail_start = head + 4 * groups;
        int64_t edge = head + (numel - tail_start);  // at most 63 + 3
        if ((int64_t)threadIdx.x < edge) {
            int64_t j = (int64_t)threadIdx.x < head ? (int64_t)threadIdx.x : tail_start + (threadIdx.x - head);
            fused_one(c, n, master, m, v, kParam ? param : nullptr, kGrad ? gout : nullptr, j, d, s);
        }
    }
}

// Fallback when the buffers' 16-byte phases disagree: element-wise, same bits.
template <int MaxN>
__global__ __launch_bounds__(kBlock) void fused_scalar_kernel(ContribTable<MaxN> c, int32_t n, float *master, float *m,
                                                              float *v, uint16_t *param, uint16_t *gout,
                                                              int64_t numel, MeanDivisor d, AdamWScalars s)
{
    for (int64_t j = global_tid(); j < numel; j += grid_stride())
        fused_one(c, n, master, m, v, param, gout, j, d, s);
}

template <int MaxN, bool kParam, bool kGrad>
static zr_status fused_vec_launch(const ContribTable<MaxN> &c, int32_t n, float *master, float *m, float *v,
                                  uint16_t *param, uint16_t *gout, int64_t numel, int64_t head, int64_t groups,
                                  const MeanDivisor &d, const AdamWScalars &s, hipStream_t st)
{
    return launch(fused_vec_kernel<MaxN, kParam, kGrad>, order_grid<kFusedOrder>((groups + kBlock - 1) / kBlock),
                  dim3(kBlock), fused_cap_lds(n), st, c, n, master, m, v, param, gout, numel, head, groups, d, s);
}

template <int MaxN>
static zr_status fused_launch(const void *const *contribs, int32_t n, float *master, float *m, float *v,
                              uint16_t *param, uint16_t *gout, int64_t numel, const MeanDivisor &d,
                              const AdamWScalars &s, hipStream_t st)
{
    ContribTable<MaxN> c = {};
    for (int32_t k = 0; k < n; ++k)
        c.p[k] = static_cast<const uint16_t *>(contribs[k]);
    const int64_t head = line_head32(master, c.p[0], numel);
    bool vec = aligned_to(m + head, 16) && aligned_to(v + head, 16) && (!param || aligned_to(param + head, 8)) &&
               (!gout || aligned_to(gout + head, 8));
    for (int32_t k = 0; k < n && vec; ++k)
        vec = aligned_to(c.p[k] + head, 8);
    if (!vec)
        return launch(fused_scalar_kernel<MaxN>, grid_of((numel + kBlock - 1) / kBlock), dim3(kBlock), 0, st, c, n,
                      master, m, v, param, gout, numel, d, s);
    const int64_t groups = (numel - head) / 4;
    if (param && gout)
        return fused_vec_launch<MaxN, true, true>(c, n, master, m, v, param, gout, numel, head, groups, d, s, st);
    if (param)
        return fused_vec_launch<MaxN, true, false>(c, n, master, m, v, param, gout, numel, head, groups, d, s, st);
    if (gout)
        return fused_vec_launch<MaxN, false, true>(c, n, master, m, v, param, gout, numel, head, groups, d, s, st);
    return fused_vec_launch<MaxN, false, false>(c, n, master, m, v, param, gout, numel, head, groups, d, s, st);
}

template <int MaxN>
static int fused_slots_for(ScalarSlot *out)
{
    out[0] = slot_of(fused_vec_kernel<MaxN, true, true>);
    out[1] = slot_of(fused_vec_kernel<MaxN, true, false>);
    out[2] = slot_of(fused_vec_kernel<MaxN, false, true>);
    out[3] = slot_of(fused_vec_kernel<MaxN, false, false>);
    out[4] = slot_of(fused_scalar_kernel<MaxN>);
    return 5;
}

int fused_scalar_slots(ScalarSlot *out)
{
    int k = fused_slots_for<8>(out);
    k += fused_slots_for<64>(out + k);
    k += fused_slots_for<kMaxContribs>(out + k);
    return k;
}

}  // namespace zr

using namespace zr;

extern "C" zr_status zr_reduce_adamw_step(const void *const *contribs, int32_t n, float *master, float *exp_avg,
                                          float *exp_avg_sq, void *param_out, void *grad_out, int64_t numel,
                                          const zr_adamw_hparams *hp, void *stream)
{
    clear_error();
    zr_status st0 = check_adamw_hparams("zr_reduce_adamw_step", hp);
    if (st0 != ZR_OK)
        return st0;
    if (!contribs)
        return fail(ZR_EINVAL, "zr_reduce_adamw_step: contribs is NULL");
    if (n < 1 || n > kMaxContribs)
        return fail(ZR_EINVAL, "zr_reduce_adamw_step: n = %d outside [1, %d]", n, kMaxContribs);
    if (numel < 0)
        return fail(ZR_EINVAL, "zr_reduce_adamw_step: numel < 0");
    if (numel > 0 && (!master || !exp_avg || !exp_avg_sq))
        return fail(ZR_EINVAL, "zr_reduce_adamw_step: NULL buffer");
    if (!aligned_to(param_out, 2) || !aligned_to(grad_out, 2) || !aligned_to(master, 4) || !aligned_to(exp_avg, 4) ||
        !aligned_to(exp_avg_sq, 4))
        return fail(ZR_EALIGN, "zr_reduce_adamw_step: buffers must be naturally aligned (bf16: 2 B, fp32: 4 B)");
    {
        const void *p[5] = {master, exp_avg, exp_avg_sq, param_out, grad_out};
        int64_t b[5] = {4 * numel, 4 * numel, 4 * numel, param_out ? 2 * numel : 0, grad_out ? 2 * numel : 0};
        int x, y;
        if (any_overlap(p, b, 5, &x, &y))
            return fail(ZR_EINVAL, "zr_reduce_adamw_step: output buffers %d and %d overlap", x, y);
    }
    for (int32_t k = 0; k < n; ++k) {
        if (numel > 0 && !contribs[k])
            return fail(ZR_EINVAL, "zr_reduce_adamw_step: contribs[%d] is NULL", k);
        if (!aligned_to(contribs[k], 2))
            return fail(ZR_EALIGN, "zr_reduce_adamw_step: contribs[%d] must be 2-byte aligned", k);
        const void *outs[4] = {master, exp_avg, exp_avg_sq, param_out};
        const int64_t ob[4] = {4 * numel, 4 * numel, 4 * numel, 2 * numel};
        for (int o = 0; o < 4; ++o)
            if (outs[o] && overlaps(contribs[k], 2 * numel, outs[o], ob[o]))
                return fail(ZR_EINVAL, "zr_reduce_adamw_step: contribs[%d] overlaps an output", k);
        if (grad_out && !(k == 0 && contribs[k] == grad_out) && overlaps(contribs[k], 2 * numel, grad_out, 2 * numel))
            return fail(ZR_EINVAL,
                        "zr_reduce_adamw_step: grad_out overlaps contribs[%d] (only grad_out == contribs[0] is allowed)",
                        k);
    }
    if (numel == 0)
        return ZR_OK;

    const MeanDivisor d = mean_divisor(n);
    const AdamWScalars s = adamw_scalars(*hp);
    auto p = static_cast<uint16_t *>(param_out);
    auto go = static_cast<uint16_t *>(grad_out);
    hipStream_t st = static_cast<hipStream_t>(stream);
    // Beyond kFusedMaxN contributions the mean and the update run as two passes
    // when there is a bf16 buffer to hold the mean: grad_out, else param_out,
    // which the AdamW pass then overwrites element by element in place.
    uint16_t *mean_buf = go ? go : p;
    if (n > kFusedMaxN && mean_buf) {
        zr_status r = reduce_run(contribs, n, numel, mean_buf, st);
        if (r != ZR_OK)
            return r;
        return adamw_run(mean_buf, master, exp_avg, exp_avg_sq, p, numel, s, st);
    }
    if (n <= 8)
        return fused_launch<8>(contribs, n, master, exp_avg, exp_avg_sq, p, go, numel, d, s, st);
    if (n <= 64)
        return fused_launch<64>(contribs, n, master, exp_avg, exp_avg_sq, p, go, numel, d, s, st);
    return fused_launch<kMaxContribs>(contribs, n, master, exp_avg, exp_avg_sq, p, go, numel, d, s, st);
}
