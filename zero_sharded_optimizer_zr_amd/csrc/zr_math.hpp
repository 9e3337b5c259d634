// Per-element arithmetic shared by the reduce, AdamW and fused reduce+AdamW
// kernels, and the host-side preparation of its scalars.  Every code path of
// every kernel goes through these functions, so the fused kernel gives the
// same bits as the reduce followed by the AdamW step.
#pragma once

#include <cmath>
#include <type_traits>

#include "zr_device.hpp"
#include "zr_internal.hpp"

namespace zr {

// ------------------------------------------------------------ gradient mean --

struct MeanDivisor {
    float n;       // (float)n
    float inv;     // 1/n, exact when n is a power of two
    int32_t pow2;  // multiply by inv (same bits as dividing by n) instead of dividing
};

inline MeanDivisor mean_divisor(int32_t n)
{
    MeanDivisor d;
    d.n = (float)n;
    d.inv = 1.0f / (float)n;
    d.pow2 = (n & (n - 1)) == 0;
    return d;
}

// fp32 sum of the n contributions (ascending order) -> their mean, rounded once.
__device__ __forceinline__ float finish_mean(float sum, const MeanDivisor &d)
{
    return d.pow2 ? sum * d.inv : __fdiv_rn(sum, d.n);
}

constexpr int kMaxContribs = 256;

// n device pointers of bf16 contributions, passed by value in the kernel
// arguments (tables of 8, 64 or 256 keep the argument block small).
template <int MaxN>
struct ContribTable {
    const uint16_t *p[MaxN];
};

// bf16 mean of the contributions at element j: the element-wise path.
template <int MaxN>
__device__ __forceinline__ uint16_t reduce_one(const ContribTable<MaxN> &c, int32_t n, int64_t j,
                                               const MeanDivisor &d)
{
    float sum = bf16_to_f32(c.p[0][j]);
    for (int32_t k = 1; k < n; ++k)
        sum += bf16_to_f32(c.p[k][j]);
    return (uint16_t)f32_to_bf16(finish_mean(sum, d));
}

// -------------------------------------------------------------------- AdamW --

// The step's hyper-parameters and bias corrections, in double, as the update
// uses them.
struct AdamWScalars {
    double lr;
    double beta1, one_minus_beta1;
    double beta2, one_minus_beta2;
    double eps;
    double decay;  // 1 - lr * weight_decay
    double bias1;  // 1 - beta1^t
    double bias2;  // 1 - beta2^t
    double grad_scale;
};

// Decoupled-weight-decay Adam on one element from the gradient g (already
// scaled, in double).  The fp32 state is widened exactly; every operation is
// one IEEE double operation -- correctly rounded division and square root, no
// FMA contraction -- in the order of the published update (decay, moments,
// bias-corrected moments, step); each new state is rounded once to fp32.  fp64
// arithmetic costs nothing measurable here (the kernels are bound by HBM: the
// AdamW kernel measured 5,971 GB/s in double against 5,970 in fp32 on the same
// buffers) and keeps the cancellation in th - lr * m_hat / (...) exact to
// double precision, so the fp32 results are the correctly rounded values of
// the double computation, not within a few fp32 ulps of them.
__device__ __forceinline__ void adamw_update(double g, float &th, float &m, float &v, const AdamWScalars &s)
{
    double t = (double)th * s.decay;
    const double mm = s.beta1 * (double)m + s.one_minus_beta1 * g;
    const double vv = s.beta2 * (double)v + s.one_minus_beta2 * g * g;
    const double m_hat = mm / s.bias1;
    const double v_hat = vv / s.bias2;
    t = t - s.lr * m_hat / (__builtin_sqrt(v_hat) + s.eps);
    th = (float)t;
    m = (float)mm;
    v = (float)vv;
}

// The update from a bf16 gradient value (exact in fp32) times grad_scale.
__device__ __forceinline__ void adamw_element(float graw, float &th, float &m, float &v, const AdamWScalars &s)
{
    adamw_update((double)graw * s.grad_scale, th, m, v, s);
}

// Validates the hyper-parameters (ZR_EINVAL with a message naming `who`).
inline zr_status check_adamw_hparams(const char *who, const zr_adamw_hparams *hp)
{
    if (!hp)
        return fail(ZR_EINVAL, "%s: hp is NULL", who);
    if (hp->step < 1)
        return fail(ZR_EINVAL, "%s: step = %lld < 1", who, (long long)hp->step);
    if (!(hp->beta1 >= 0.0 && hp->beta1 < 1.0) || !(hp->beta2 >= 0.0 && hp->beta2 < 1.0))
        return fail(ZR_EINVAL, "%s: betas outside [0, 1)", who);
    if (!(hp->eps > 0.0) || !std::isfinite(hp->eps))
        return fail(ZR_EINVAL, "%s: eps must be finite and > 0", who);
    if (!(hp->lr >= 0.0) || !std::isfinite(hp->lr) || !(hp->weight_decay >= 0.0) || !std::isfinite(hp->weight_decay))
        return fail(ZR_EINVAL, "%s: lr and weight_decay must be finite and >= 0", who);
    if (!std::isfinite(hp->grad_scale))
        return fail(ZR_EINVAL, "%s: grad_scale must be finite", who);
    return ZR_OK;
}

// Per-step scalars, in double (t enters only through the bias corrections).
inline AdamWScalars adamw_scalars(const zr_adamw_hparams &hp)
{
    const double t = (double)hp.step;
    AdamWScalars s;
    s.lr = hp.lr;
    s.beta1 = hp.beta1;
    s.one_minus_beta1 = 1.0 - hp.beta1;
    s.beta2 = hp.beta2;
    s.one_minus_beta2 = 1.0 - hp.beta2;
    s.eps = hp.eps;
    s.decay = 1.0 - hp.lr * hp.weight_decay;
    s.bias1 = 1.0 - std::pow(hp.beta1, t);
    s.bias2 = 1.0 - std::pow(hp.beta2, t);
    s.grad_scale = hp.grad_scale;
    return s;
}

// ------------------------------------------- launches after validation --

// The mean of n contributions into out (zr_reduce_slice without its checks:
// out may be contribs[0], nothing else may overlap).
zr_status reduce_run(const void *const *contribs, int32_t n, int64_t numel, uint16_t *out, hipStream_t st);

// AdamW on master / m / v from the bf16 gradient g, the copy into p (may be
// NULL).  p may be g itself: every element is read before it is written, by the
// same lane.
zr_status adamw_run(const uint16_t *g, float *master, float *exp_avg, float *exp_avg_sq, uint16_t *p, int64_t numel,
                    const AdamWScalars &s, hipStream_t st);

// ------------------------------------------------- graph parameter slots --

// A kernel that takes the per-step AdamW scalars by value, as captured graphs
// see it: its host-side address, its argument count and the position of the
// AdamWScalars argument (deduced from the signature at compile time).
struct ScalarSlot {
    const void *func;
    int nargs;
    int index;
};

template <typename T, typename... A>
constexpr int arg_index()
{
    constexpr bool match[] = {std::is_same<T, A>::value..., false};
    for (int i = 0; i < (int)sizeof...(A); ++i)
        if (match[i])
            return i;
    return -1;
}

template <typename... A>
ScalarSlot slot_of(void (*kernel)(A...))
{
    static_assert(arg_index<AdamWScalars, A...>() >= 0, "kernel takes no AdamWScalars");
    return ScalarSlot{reinterpret_cast<const void *>(kernel), (int)sizeof...(A), arg_index<AdamWScalars, A...>()};
}

// The AdamW-family kernels of each translation unit (adamw.hip, fused.hip,
// fp16.hip); each writes its slots to `out` and returns how many.
int adamw_scalar_slots(ScalarSlot *out);
int fused_scalar_slots(ScalarSlot *out);
int fp16_scalar_slots(ScalarSlot *out);
constexpr int kMaxScalarSlots = 64;

// No two of `count` buffers (pointer, byte length) may overlap; NULL entries
// are skipped.  Returns the index pair of the first overlap through a, b.
inline bool any_overlap(const void *const *p, const int64_t *bytes, int count, int *a, int *b)
{
    for (int i = 0; i < count; ++i)
        for (int j = i + 1; j < count; ++j)
            if (p[i] && p[j] && overlaps(p[i], bytes[i], p[j], bytes[j])) {
                *a = i;
                *b = j;
                return true;
            }
    return false;
}

}  // namespace zr
