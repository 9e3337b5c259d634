// fp16 variant of one rank's step with dynamic loss scaling (gfx950).
//
// The backward pass produced fp16 gradients multiplied by the loss scale S.
// The rank averages its n fp16 contributions (fp32 accumulation, fp16 result)
// and flags an inf or NaN anywhere in the mean; the AdamW kernel divides S back
// out and updates fp32 master / m / v, writing an fp16 copy -- or, when the flag
// is set, leaves everything untouched; a one-thread kernel then applies the
// scale rule (halve on overflow; double after `window` clean steps).  The
// scale and the flag live in a small device-resident zr_loss_scale record, so
// no step needs the host to look at the gradient.
//
// Sources (web pages on DeepSpeed ZeRO-3): ZeRO tutorial (cnhsyj.com) 3.1, fp16
// with a dynamic loss scale (window 1000, initial scale 2^16), and 4.2, dynamic
// scaling against fp16 gradients that are very small or very large; ZeRO-1/2/3
// concept page (compassingai.com), 16 B/param table (fp16 parameters and
// gradients) and Stage 1 mechanism (16-bit copy of the updated fp32 master).
// The skip-and-rescale rule is the standard dynamic loss scaling of mixed
// precision training (Micikevicius et al., ICLR 2018).
//
// Kernels: the same streaming design as the bf16 ones (one vector per lane over
// a full grid, non-temporal 16-byte accesses, residency capped with reserved
// LDS), with fp16 <-> fp32 done by the hardware conversions (exact widening;
// round to nearest even for the narrowing, NaN canonicalised to sign | 0x7e00).
#include "zr_math.hpp"

namespace zr {

// ----------------------------------------------------------- fp16 helpers ----

__device__ __forceinline__ float f16_to_f32(uint32_t h16)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h16);
}
__device__ __forceinline__ float f16_lo(uint32_t w) { return f16_to_f32(w & 0xffffu); }
__device__ __forceinline__ float f16_hi(uint32_t w) { return f16_to_f32(w >> 16); }

// fp32 -> fp16 bits, round to nearest even (hardware), NaN -> sign | 0x7e00.
__device__ __forceinline__ uint32_t f32_to_f16(float f)
{
    uint32_t h = __builtin_bit_cast(uint16_t, (_Float16)f);
    return (f != f) ? (((__float_as_uint(f) >> 16) & 0x8000u) | 0x7e00u) : h;
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) { return f32_to_f16(lo) | (f32_to_f16(hi) << 16); }

__device__ __forceinline__ bool f16_nonfinite(uint32_t h16) { return (h16 & 0x7c00u) == 0x7c00u; }

// Sets ls->found_inf when a lane saw a non-finite value: a plain vector store
// of 1, so concurrent writers all write the same value.
__device__ __forceinline__ void flag_if_any(bool bad, zr_loss_scale *ls)
{
    if (bad)
        ls->found_inf = 1;
}

// ------------------------------------------------------------ loss scale ----

__global__ void loss_scale_init_kernel(zr_loss_scale *ls, float initial)
{
    ls->scale = initial;
    ls->good_steps = 0;
    ls->found_inf = 0;
    ls->skipped = 0;
}

__global__ void loss_scale_update_kernel(zr_loss_scale *ls, int32_t window, float factor, float min_scale)
{
    zr_loss_scale s = *ls;
    if (s.found_inf) {
        s.scale = fmaxf(s.scale / factor, min_scale);
        s.good_steps = 0;
        s.skipped += 1;
    } else {
        s.good_steps += 1;
        if (s.good_steps == window) {
            s.scale = s.scale * factor;
            s.good_steps = 0;
        }
    }
    s.found_inf = 0;
    *ls = s;
}

// ------------------------------------------------------- gradient mean ------

// Tile orders (first_tile) of the mean, as the bf16 reduce: runs of 256 tiles
// per XCD, rotated from group to group, up to 8 contributions, launch order
// above; the finite check in runs of 256, not rotated (6-8% over launch order
// on the same buffers; the rotation lost 1%).
constexpr int kReduceOrder = 256;
constexpr int kReduce4Order = 256;
constexpr int kReduceWideOrder = 1;
constexpr bool kReduceRotate = true;
constexpr int kCheckFiniteOrder = 256;

template <int MaxN>
__device__ __forceinline__ uint32_t reduce_one_f16(const ContribTable<MaxN> &c, int32_t n, int64_t j,
                                                   const MeanDivisor &d)
{
    float sum = f16_to_f32(c.p[0][j]);
    for (int32_t k = 1; k < n; ++k)
        sum += f16_to_f32(c.p[k][j]);
    return f32_to_f16(finish_mean(sum, d));
}

// Tiles of kBlock groups in the bf16 reduce's order.
template <int MaxN>
__global__ __launch_bounds__(kBlock) void reduce_f16_vec_kernel(ContribTable<MaxN> c, int32_t n, uint16_t *out,
                                                                int64_t numel, int64_t head, int64_t groups,
                                                                MeanDivisor d, zr_loss_scale *ls)
{
    u32x4 *o4 = reinterpret_cast<u32x4 *>(out + head);
    constexpr int kOrder = MaxN <= 8 ? kReduceOrder : kReduceWideOrder;
    for (int64_t i = first_tile<kOrder, kReduceRotate>() * kBlock + threadIdx.x; i < groups; i += grid_stride()) {
        float acc[8];
        for (int32_t k = 0; k < n; k += 4) {
            u32x4 x[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (k + u < n)
                    x[u] = load_stream(reinterpret_cast<const u32x4 *>(c.p[k + u] + head) + i);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (k + u >= n)
                    continue;
                const uint32_t w[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (k + u == 0) {
                        acc[2 * q] = f16_lo(w[q]);
                        acc[2 * q + 1] = f16_hi(w[q]);
                    } else {
                        acc[2 * q] += f16_lo(w[q]);
                        acc[2 * q + 1] += f16_hi(w[q]);
                    }
                }
            }
        }
        u32x4 r;
        r.x = pack_f16x2(finish_mean(acc[0], d), finish_mean(acc[1], d));
        r.y = pack_f16x2(finish_mean(acc[2], d), finish_mean(acc[3], d));
        r.z = pack_f16x2(finish_mean(acc[4], d), finish_mean(acc[5], d));
        r.w = pack_f16x2(finish_mean(acc[6], d), finish_mean(acc[7], d));
        store_stream(o4 + i, r);
        if (ls) {
            bool bad = false;
            const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
            for (int q = 0; q < 4; ++q)
                bad = bad || f16_nonfinite(w[q] & 0xffffu) || f16_nonfinite(w[q] >> 16);
            flag_if_any(bad, ls);
        }
    }
    if (blockIdx.x == 0) {
        int64_t tail_start = head + 8 * groups;
        int64_t edge = head + (numel - tail_start);
        if ((int64_t)threadIdx.x < edge) {
            int64_t j = (int64_t)threadIdx.x < head ? (int64_t)threadIdx.x : tail_start + (threadIdx.x - head);
            uint32_t h = reduce_one_f16(c, n, j, d);
            out[j] = (uint16_t)h;
            if (ls && f16_nonfinite(h))
                ls->found_inf = 1;
        }
    }
}

// 7 or 8 contributions: 4 elements per lane with every 8-byte load in flight at
// once, tiles in rotated runs of 256, as the bf16 reduce does for the same
// counts.
__global__ __launch_bounds__(kBlock) void reduce4_f16_vec_kernel(ContribTable<8> c, int32_t n, uint16_t *out,
                                                                 int64_t numel, int64_t head, int64_t groups,
                                                                 MeanDivisor d, zr_loss_scale *ls)
{
    u32x2 *o2 = reinterpret_cast<u32x2 *>(out + head);
    for (int64_t i = first_tile<kReduce4Order, kReduceRotate>() * kBlock + threadIdx.x; i < groups;
         i += grid_stride()) {
        u32x2 x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (u < n)
                x[u] = load_stream(reinterpret_cast<const u32x2 *>(c.p[u] + head) + i);
        float acc[4] = {f16_lo(x[0].x), f16_hi(x[0].x), f16_lo(x[0].y), f16_hi(x[0].y)};
#pragma unroll
        for (int u = 1; u < 8; ++u)
            if (u < n) {
                acc[0] += f16_lo(x[u].x);
                acc[1] += f16_hi(x[u].x);
                acc[2] += f16_lo(x[u].y);
                acc[3] += f16_hi(x[u].y);
            }
        const u32x2 r{pack_f16x2(finish_mean(acc[0], d), finish_mean(acc[1], d)),
                      pack_f16x2(finish_mean(acc[2], d), finish_mean(acc[3], d))};
        store_stream(o2 + i, r);
        if (ls)
            flag_if_any(f16_nonfinite(r.x & 0xffffu) || f16_nonfinite(r.x >> 16) || f16_nonfinite(r.y & 0xffffu) ||
                            f16_nonfinite(r.y >> 16),
                        ls);
    }
    if (blockIdx.x == 0) {
        int64_t tail_start = head + 4 * groups;
        int64_t edge = head + (numel - tail_start);  // at most 63 + 3
        if ((int64_t)threadIdx.x < edge) {
            int64_t j = (int64_t)threadIdx.x < head ? (int64_t)threadIdx.x : tail_start + (threadIdx.x - head);
            uint32_t h = reduce_one_f16(c, n, j, d);
            out[j] = (uint16_t)h;
            if (ls && f16_nonfinite(h))
                ls->found_inf = 1;
        }
    }
}

template <int MaxN>
__global__ __launch_bounds__(kBlock) void reduce_f16_scalar_kernel(ContribTable<MaxN> c, int32_t n, uint16_t *out,
                                                                   int64_t numel, MeanDivisor d, zr_loss_scale *ls)
{
    for (int64_t j = global_tid(); j < numel; j += grid_stride()) {
        uint32_t h = reduce_one_f16(c, n, j, d);
        out[j] = (uint16_t)h;
        if (ls && f16_nonfinite(h))
            ls->found_inf = 1;
    }
}

// ------------------------------------------------------------ finite check ----

__global__ __launch_bounds__(kBlock) void check_finite_kernel(const uint16_t *grad, int64_t numel, int64_t head,
                                                              int64_t groups, zr_loss_scale *ls)
{
    const u32x4 *g4 = reinterpret_cast<const u32x4 *>(grad + head);
    for (int64_t i = first_tile<kCheckFiniteOrder>() * kBlock + threadIdx.x; i < groups; i += grid_stride()) {
        u32x4 x = load_stream(g4 + i);
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
        bool bad = false;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            bad = bad || f16_nonfinite(w[q] & 0xffffu) || f16_nonfinite(w[q] >> 16);
        flag_if_any(bad, ls);
    }
    if (blockIdx.x == 0) {
        int64_t tail_start = head + 8 * groups;
        int64_t edge = head + (numel - tail_start);
        if ((int64_t)threadIdx.x < edge) {
            int64_t j = (int64_t)threadIdx.x < head ? (int64_t)threadIdx.x : tail_start + (threadIdx.x - head);
            if (f16_nonfinite(grad[j]))
                ls->found_inf = 1;
        }
    }
}

// ------------------------------------------------------------------ AdamW ----

__device__ __forceinline__ void adamw_one_f16(const uint16_t *grad, float *master, float *m, float *v, uint16_t *param,
                                              int64_t j, double unscale, const AdamWScalars &s)
{
    float th = master[j], mm = m[j], vv = v[j];
    adamw_update((double)f16_to_f32(grad[j]) * unscale * s.grad_scale, th, mm, vv, s);
    master[j] = th;
    m[j] = mm;
    v[j] = vv;
    if (param)
        param[j] = (uint16_t)f32_to_f16(th);
}

template <bool kParam>
__global__ __launch_bounds__(kBlock) void adamw_f16_vec_kernel(const uint16_t *grad, float *master, float *m, float *v,
                                                               uint16_t *param, int64_t numel, int64_t head,
                                                               int64_t groups, AdamWScalars s,
                                                               const zr_loss_scale *ls)
{
    const u32x2 *g2 = reinterpret_cast<const u32x2 *>(grad + head);
    f32x4 *th4 = reinterpret_cast<f32x4 *>(master + head);
    f32x4 *m4 = reinterpret_cast<f32x4 *>(m + head);
    f32x4 *v4 = reinterpret_cast<f32x4 *>(v + head);
    u32x2 *p2 = kParam ? reinterpret_cast<u32x2 *>(param + head) : nullptr;
    // The record is read once, and first used after the data loads are issued,
    // so its latency hides behind theirs instead of delaying them; the empty
    // asm takes the loaded data and the record together, which keeps the loads
    // ahead of the (uniform) early return.
    int32_t skip = ls->found_inf;
    float scale = ls->scale;

    for (int64_t i = first_tile<kAdamwOrder>() * kBlock + threadIdx.x; i < groups; i += grid_stride()) {
        u32x2 g = load_stream(g2 + i);
        f32x4 a = load_stream(th4 + i);
        f32x4 mm = load_stream(m4 + i);
        f32x4 vv = load_stream(v4 + i);
        int32_t sk = skip;
        float sc = scale;
        asm volatile("" : "+v"(g), "+v"(a), "+v"(mm), "+v"(vv), "+s"(sk), "+s"(sc));
        if (sk)  // the whole step is skipped: nothing is written
            return;
        const double unscale = 1.0 / (double)sc;
        float gr[4] = {f16_lo(g.x), f16_hi(g.x), f16_lo(g.y), f16_hi(g.y)};
        float th[4] = {a.x, a.y, a.z, a.w};
        float mo[4] = {mm.x, mm.y, mm.z, mm.w};
        float vo[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
            adamw_update((double)gr[e] * unscale * s.grad_scale, th[e], mo[e], vo[e], s);
        store_stream(th4 + i, f32x4{th[0], th[1], th[2], th[3]});
        store_stream(m4 + i, f32x4{mo[0], mo[1], mo[2], mo[3]});
        store_stream(v4 + i, f32x4{vo[0], vo[1], vo[2], vo[3]});
        if (kParam)
            store_stream(p2 + i, u32x2{pack_f16x2(th[0], th[1]), pack_f16x2(th[2], th[3])});
    }
    if (blockIdx.x == 0 && !skip) {
        int64_t tail_start = head + 4 * groups;
        int64_t edge = head + (numel - tail_start);
        if ((int64_t)threadIdx.x < edge) {
            int64_t j = (int64_t)threadIdx.x < head ? (int64_t)threadIdx.x : tail_start + (threadIdx.x - head);
            adamw_one_f16(grad, master, m, v, kParam ? param : nullptr, j, 1.0 / (double)scale, s);
        }
    }
}

__global__ __launch_bounds__(kBlock) void adamw_f16_scalar_kernel(const uint16_t *grad, float *master, float *m,
                                                                  float *v, uint16_t *param, int64_t numel,
                                                                  AdamWScalars s, const zr_loss_scale *ls)
{
    if (ls->found_inf)
        return;
    const double unscale = 1.0 / (double)ls->scale;
    for (int64_t j = global_tid(); j < numel; j += grid_stride())
        adamw_one_f16(grad, master, m, v, param, j, unscale, s);
}

constexpr size_t kAdamwF16Lds = 32 * 1024;  // 5 workgroups per CU, as for the bf16 step

template <int MaxN>
static zr_status reduce_f16_launch(const void *const *contribs, int32_t n, int64_t numel, uint16_t *out,
                                   zr_loss_scale *ls, hipStream_t st)
{
    ContribTable<MaxN> c = {};
    for (int32_t k = 0; k < n; ++k)
        c.p[k] = static_cast<const uint16_t *>(contribs[k]);
    const MeanDivisor d = mean_divisor(n);
    const int64_t head = line_head16(out, numel);
    if constexpr (MaxN == 8) {
        bool vec4 = n >= 7;  // as the bf16 reduce (kFourPerLaneMinN)
        for (int32_t k = 0; k < n && vec4; ++k)
            vec4 = aligned_to(c.p[k] + head, 8);
        if (vec4) {
            const int64_t groups = (numel - head) / 4, tiles = (groups + kBlock - 1) / kBlock;
            return launch(reduce4_f16_vec_kernel, order_grid<kReduce4Order>(tiles), dim3(kBlock), 32 * 1024, st, c,
                          n, out, numel, head, groups, d, ls);
        }
    }
    bool vec = true;
    for (int32_t k = 0; k < n && vec; ++k)
        vec = aligned_to(c.p[k] + head, 16);
    if (!vec)
        return launch(reduce_f16_scalar_kernel<MaxN>, grid_of((numel + kBlock - 1) / kBlock), dim3(kBlock), 0, st,
                      c, n, out, numel, d, ls);
    // residency cap and tile order as the bf16 reduce
    const int64_t groups = (numel - head) / 8, tiles = (groups + kBlock - 1) / kBlock;
    const size_t lds = n > 8 ? 80 * 1024 : (n > 4 ? 40 * 1024 : 32 * 1024);
    return launch(reduce_f16_vec_kernel<MaxN>, order_grid<MaxN <= 8 ? kReduceOrder : kReduceWideOrder>(tiles),
                  dim3(kBlock), lds, st, c, n, out, numel, head, groups, d, ls);
}

inline zr_status check_ls(const char *who, const void *ls)
{
    if (!ls)
        return fail(ZR_EINVAL, "%s: loss-scale record is NULL", who);
    if (!aligned_to(ls, 4))
        return fail(ZR_EALIGN, "%s: loss-scale record must be 4-byte aligned", who);
    return ZR_OK;
}

int fp16_scalar_slots(ScalarSlot *out)
{
    out[0] = slot_of(adamw_f16_vec_kernel<true>);
    out[1] = slot_of(adamw_f16_vec_kernel<false>);
    out[2] = slot_of(adamw_f16_scalar_kernel);
    return 3;
}

}  // namespace zr

using namespace zr;

extern "C" zr_status zr_loss_scale_init(zr_loss_scale *ls, float initial_scale, void *stream)
{
    clear_error();
    zr_status s = check_ls("zr_loss_scale_init", ls);
    if (s != ZR_OK)
        return s;
    if (!(initial_scale > 0.0f) || !std::isfinite(initial_scale))
        return fail(ZR_EINVAL, "zr_loss_scale_init: initial scale must be finite and > 0");
    return launch(loss_scale_init_kernel, dim3(1), dim3(1), 0, static_cast<hipStream_t>(stream), ls, initial_scale);
}

extern "C" zr_status zr_loss_scale_update(zr_loss_scale *ls, int32_t window, float factor, float min_scale,
                                          void *stream)
{
    clear_error();
    zr_status s = check_ls("zr_loss_scale_update", ls);
    if (s != ZR_OK)
        return s;
    if (window < 1)
        return fail(ZR_EINVAL, "zr_loss_scale_update: window = %d < 1", window);
    if (!(factor > 1.0f) || !std::isfinite(factor))
        return fail(ZR_EINVAL, "zr_loss_scale_update: factor must be finite and > 1");
    if (!(min_scale > 0.0f) || !std::isfinite(min_scale))
        return fail(ZR_EINVAL, "zr_loss_scale_update: min_scale must be finite and > 0");
    return launch(loss_scale_update_kernel, dim3(1), dim3(1), 0, static_cast<hipStream_t>(stream), ls, window,
                  factor, min_scale);
}

extern "C" zr_status zr_reduce_slice_f16(const void *const *contribs, int32_t n, int64_t numel, void *out,
                                         zr_loss_scale *ls, void *stream)
{
    clear_error();
    if (!contribs)
        return fail(ZR_EINVAL, "zr_reduce_slice_f16: contribs is NULL");
    if (n < 1 || n > kMaxContribs)
        return fail(ZR_EINVAL, "zr_reduce_slice_f16: n = %d outside [1, %d]", n, kMaxContribs);
    if (numel < 0)
        return fail(ZR_EINVAL, "zr_reduce_slice_f16: numel < 0");
    if (numel > 0 && !out)
        return fail(ZR_EINVAL, "zr_reduce_slice_f16: out is NULL");
    if (!aligned_to(out, 2))
        return fail(ZR_EALIGN, "zr_reduce_slice_f16: out must be 2-byte aligned");
    if (ls && !aligned_to(ls, 4))
        return fail(ZR_EALIGN, "zr_reduce_slice_f16: loss-scale record must be 4-byte aligned");
    for (int32_t k = 0; k < n; ++k) {
        if (numel > 0 && !contribs[k])
            return fail(ZR_EINVAL, "zr_reduce_slice_f16: contribs[%d] is NULL", k);
        if (!aligned_to(contribs[k], 2))
            return fail(ZR_EALIGN, "zr_reduce_slice_f16: contribs[%d] must be 2-byte aligned", k);
        if (!(k == 0 && contribs[k] == out) && overlaps(contribs[k], 2 * numel, out, 2 * numel))
            return fail(ZR_EINVAL, "zr_reduce_slice_f16: out overlaps contribs[%d] (only out == contribs[0])", k);
        if (ls && overlaps(contribs[k], 2 * numel, ls, sizeof(zr_loss_scale)))
            return fail(ZR_EINVAL, "zr_reduce_slice_f16: the loss-scale record overlaps contribs[%d]", k);
    }
    if (ls && overlaps(out, 2 * numel, ls, sizeof(zr_loss_scale)))
        return fail(ZR_EINVAL, "zr_reduce_slice_f16: the loss-scale record overlaps out");
    if (numel == 0)
        return ZR_OK;
    auto o = static_cast<uint16_t *>(out);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (n <= 8)
        return reduce_f16_launch<8>(contribs, n, numel, o, ls, st);
    if (n <= 64)
        return reduce_f16_launch<64>(contribs, n, numel, o, ls, st);
    return reduce_f16_launch<kMaxContribs>(contribs, n, numel, o, ls, st);
}

extern "C" zr_status zr_check_finite_f16(const void *grad, int64_t numel, zr_loss_scale *ls, void *stream)
{
    clear_error();
    zr_status s = check_ls("zr_check_finite_f16", ls);
    if (s != ZR_OK)
        return s;
    if (numel < 0)
        return fail(ZR_EINVAL, "zr_check_finite_f16: numel < 0");
    if (numel > 0 && !grad)
        return fail(ZR_EINVAL, "zr_check_finite_f16: grad is NULL");
    if (!aligned_to(grad, 2))
        return fail(ZR_EALIGN, "zr_check_finite_f16: grad must be 2-byte aligned");
    if (overlaps(grad, 2 * numel, ls, sizeof(zr_loss_scale)))
        return fail(ZR_EINVAL, "zr_check_finite_f16: the loss-scale record overlaps grad");
    if (numel == 0)
        return ZR_OK;
    auto g = static_cast<const uint16_t *>(grad);
    const int64_t head = line_head16(g, numel);
    const int64_t groups = (numel - head) / 8;
    return launch(check_finite_kernel, order_grid<kCheckFiniteOrder>((groups + kBlock - 1) / kBlock), dim3(kBlock), 0,
                  static_cast<hipStream_t>(stream), g, numel, head, groups, ls);
}

extern "C" zr_status zr_adamw_step_f16(const void *grad, float *master, float *exp_avg, float *exp_avg_sq,
                                       void *param_out, int64_t numel, const zr_adamw_hparams *hp,
                                       const zr_loss_scale *ls, void *stream)
{
    clear_error();
    zr_status st0 = check_adamw_hparams("zr_adamw_step_f16", hp);
    if (st0 != ZR_OK)
        return st0;
    st0 = check_ls("zr_adamw_step_f16", ls);
    if (st0 != ZR_OK)
        return st0;
    if (numel < 0)
        return fail(ZR_EINVAL, "zr_adamw_step_f16: numel < 0");
    if (numel > 0 && (!grad || !master || !exp_avg || !exp_avg_sq))
        return fail(ZR_EINVAL, "zr_adamw_step_f16: NULL buffer");
    if (!aligned_to(grad, 2) || !aligned_to(param_out, 2) || !aligned_to(master, 4) || !aligned_to(exp_avg, 4) ||
        !aligned_to(exp_avg_sq, 4))
        return fail(ZR_EALIGN, "zr_adamw_step_f16: buffers must be naturally aligned (fp16: 2 B, fp32: 4 B)");
    {
        const void *p[6] = {grad, master, exp_avg, exp_avg_sq, param_out, ls};
        int64_t b[6] = {2 * numel, 4 * numel, 4 * numel, 4 * numel, param_out ? 2 * numel : 0,
                        (int64_t)sizeof(zr_loss_scale)};
        int x, y;
        if (any_overlap(p, b, 6, &x, &y))
            return fail(ZR_EINVAL, "zr_adamw_step_f16: buffers %d and %d overlap", x, y);
    }
    if (numel == 0)
        return ZR_OK;
    const AdamWScalars s = adamw_scalars(*hp);
    auto g = static_cast<const uint16_t *>(grad);
    auto p = static_cast<uint16_t *>(param_out);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t head = line_head32(master, g, numel);
    bool vec = aligned_to(exp_avg + head, 16) && aligned_to(exp_avg_sq + head, 16) && aligned_to(g + head, 8) &&
               (!p || aligned_to(p + head, 8));
    if (!vec)
        return launch(adamw_f16_scalar_kernel, grid_of((numel + kBlock - 1) / kBlock), dim3(kBlock), 0, st, g,
                      master, exp_avg, exp_avg_sq, p, numel, s, ls);
    const int64_t groups = (numel - head) / 4;
    dim3 grid = order_grid<kAdamwOrder>((groups + kBlock - 1) / kBlock);
    if (p)
        return launch(adamw_f16_vec_kernel<true>, grid, dim3(kBlock), kAdamwF16Lds, st, g, master, exp_avg,
                      exp_avg_sq, p, numel, head, groups, s, ls);
    return launch(adamw_f16_vec_kernel<false>, grid, dim3(kBlock), kAdamwF16Lds, st, g, master, exp_avg, exp_avg_sq,
                  p, numel, head, groups, s, ls);
}
