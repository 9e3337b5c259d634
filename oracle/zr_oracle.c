/*
 * zr_oracle.c -- plain, slow, scalar CPU oracle for the floating-point steps of
 * one rank's share of a ZeRO-3 step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links or calls this
 * file; only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * load it.  It shares no source, header or helper with the GPU path.
 *
 * Build (see oracle/build.py):  gcc -O2 -std=c11 -fPIC -shared -ffp-contract=off
 * No -ffast-math: every float/double operation below is one IEEE-754 operation
 * in round-to-nearest-even, evaluated in the order written.
 *
 * Sources (web pages on DeepSpeed ZeRO-3):
 *  - "From DDP to ZeRO: memory sharding" blog (111qqz.com), section on aligning
 *    the ledger: bf16 parameters and gradients, fp32 master weights and fp32
 *    AdamW first/second moments.
 *  - same blog, section "ZeRO-2: why gradients can be sharded": the worked
 *    ReduceScatter example, where each rank receives its slice of the averaged
 *    gradient.
 *  - ZeRO-1/2/3 concept page (compassingai.com), "Three-stage mechanism", Stage 1:
 *    each rank updates its fp32 optimizer state and fp32 master slice with the
 *    reduced gradient, then converts the fp32 master to the 16-bit working copy.
 *  - ZeRO tutorial (cnhsyj.com), section 3.1: the optimizer is AdamW with
 *    lr / betas / eps / weight_decay hyper-parameters.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ---------------------------------------------------------------- bf16 ---- */

/* bf16 -> fp32 is exact: the bf16 bits are the upper half of the fp32 bits. */
static float bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* fp32 -> bf16, round to nearest, ties to even, on the upper 16 bits.
 * NaN stays NaN (sign and upper payload kept, quiet bit forced).  Values that
 * round past the largest finite bf16 become infinity, as IEEE rounding says. */
static uint16_t f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lower = u & 0xffffu;
    uint32_t upper = u >> 16;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1u;
    return (uint16_t)upper;
}

void zr_oracle_bf16_from_f32(const float *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = f32_to_bf16(x[i]);
}

void zr_oracle_f32_from_bf16(const uint16_t *x, int64_t n, float *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = bf16_to_f32(x[i]);
}

/* -------------------------------------------------------------- reduce ---- */

/*
 * Local arithmetic of the gradient ReduceScatter on the owned slice: the mean
 * of n bf16 gradient contributions, element by element.
 *
 * Follows the ddp-to-zero blog, "ZeRO-2: why gradients can be sharded": rank r
 * receives slice r of the averaged gradient (two ranks with [2,6] and [4,10]
 * give [3] and [8]); the AllReduce-is-ReduceScatter-plus-AllGather identity in
 * "why ZeRO-2's traffic is close to DDP's" makes that slice equal to the same
 * slice of the AllReduce mean.  Gradients are bf16 (ledger section).
 *
 * Precision reading: the contributions are accumulated in fp32 in ascending
 * contribution order, starting from contribution 0, divided once by n, and the
 * mean is rounded to bf16.  contribs[k] is read at element i before out[i] is
 * written, so out may be the same array as contribs[0].
 */
void zr_oracle_reduce(const uint16_t *const *contribs, int32_t n, int64_t numel, uint16_t *out)
{
    for (int64_t i = 0; i < numel; ++i) {
        float sum = bf16_to_f32(contribs[0][i]);
        for (int32_t k = 1; k < n; ++k)
            sum = sum + bf16_to_f32(contribs[k][i]);
        float mean = sum / (float)n;
        out[i] = f32_to_bf16(mean);
    }
}

/* --------------------------------------------------------------- AdamW ---- */

/*
 * One decoupled-weight-decay Adam (AdamW) step over a shard, in double
 * precision, on fp32 master/m/v and a bf16 gradient; the new fp32 states are
 * stored, then the bf16 working copy is made from the stored fp32 master.
 *
 * Follows: the ddp-to-zero blog's ledger section (state dtypes and roles);
 * "ZeRO-1: why optimizer states can be sharded" (each element's update needs
 * only its own gradient and m, v); the concept page's Stage 1 mechanism (fp32
 * state update from the reduced gradient, then the 16-bit copy from the fp32
 * master); tutorial section 3.1 (AdamW with lr, betas, eps, weight_decay).
 * The pages print no AdamW formula; the update below is the published one
 * (Loshchilov & Hutter, "Decoupled Weight Decay Regularization", ICLR 2019),
 * arranged as PyTorch documents torch.optim.AdamW without amsgrad:
 *
 *   g  <- grad * grad_scale
 *   th <- th * (1 - lr*wd)
 *   m  <- beta1*m + (1-beta1)*g
 *   v  <- beta2*v + (1-beta2)*g*g
 *   th <- th - lr * (m / (1-beta1^t)) / (sqrt(v / (1-beta2^t)) + eps)
 *   p  <- bf16(th)
 *
 * param_out may be NULL (no 16-bit copy).  step >= 1.
 */
void zr_oracle_adamw(const uint16_t *grad, float *master, float *exp_avg, float *exp_avg_sq,
                     uint16_t *param_out, int64_t numel,
                     double lr, double beta1, double beta2, double eps,
                     double weight_decay, double grad_scale, int64_t step)
{
    double bias1 = 1.0 - pow(beta1, (double)step);
    double bias2 = 1.0 - pow(beta2, (double)step);
    double decay = 1.0 - lr * weight_decay;
    for (int64_t i = 0; i < numel; ++i) {
        double g = (double)bf16_to_f32(grad[i]) * grad_scale;
        double th = (double)master[i];
        double m = (double)exp_avg[i];
        double v = (double)exp_avg_sq[i];

        th = th * decay;
        m = beta1 * m + (1.0 - beta1) * g;
        v = beta2 * v + (1.0 - beta2) * g * g;
        double m_hat = m / bias1;
        double v_hat = v / bias2;
        th = th - lr * m_hat / (sqrt(v_hat) + eps);

        master[i] = (float)th;
        exp_avg[i] = (float)m;
        exp_avg_sq[i] = (float)v;
        if (param_out)
            param_out[i] = f32_to_bf16(master[i]);
    }
}
