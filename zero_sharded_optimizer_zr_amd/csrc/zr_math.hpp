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

struct AdamWScalars {
    float beta1, one_minus_beta1;
    float beta2, one_minus_beta2;
    float decay;           // 1 - lr * weight_decay
    float step_size;       // lr / (1 - beta1^t)
    float inv_sqrt_bias2;  // 1 / sqrt(1 - beta2^t)
    float eps;
    float grad_scale;
};

// Decoupled-weight-decay Adam on one element: IEEE fp32 operations (correctly
// rounded square root and division), no FMA contraction.
__device__ __forceinline__ void adamw_element(float graw, float &th, float &m, float &v, const AdamWScalars &s)
{
    float g = graw * s.grad_scale;
    th = th * s.decay;
    m = s.beta1 * m + s.one_minus_beta1 * g;
    v = s.beta2 * v + (s.one_minus_beta2 * g) * g;
    float denom = sqrt_rn(v) * s.inv_sqrt_bias2 + s.eps;
    th = th - s.step_size * __fdiv_rn(m, denom);
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

// Per-step scalars computed in double, each rounded once to fp32.
inline AdamWScalars adamw_scalars(const zr_adamw_hparams &hp)
{
    const double t = (double)hp.step;
    const double bias1 = 1.0 - std::pow(hp.beta1, t);
    const double bias2 = 1.0 - std::pow(hp.beta2, t);
    AdamWScalars s;
    s.beta1 = (float)hp.beta1;
    s.one_minus_beta1 = (float)(1.0 - hp.beta1);
    s.beta2 = (float)hp.beta2;
    s.one_minus_beta2 = (float)(1.0 - hp.beta2);
    s.decay = (float)(1.0 - hp.lr * hp.weight_decay);
    s.step_size = (float)(hp.lr / bias1);
    s.inv_sqrt_bias2 = (float)(1.0 / std::sqrt(bias2));
    s.eps = (float)hp.eps;
    s.grad_scale = (float)hp.grad_scale;
    return s;
}

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
