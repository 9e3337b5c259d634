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

/* ---------------------------------------------------------------- fp16 ---- */

/*
 * fp16 variant of the step (fp16 parameters and gradients with dynamic loss
 * scaling): the ZeRO tutorial (cnhsyj.com) 3.1 configures fp16 with a dynamic
 * loss scale (window 1000, initial scale 2^16) and 4.2 recommends dynamic
 * scaling for fp16 gradients that are very small or very large; the ZeRO-1/2/3
 * concept page (compassingai.com), 16 B/param table and Stage 1 mechanism, uses
 * fp16 parameters and gradients and a 16-bit copy of the fp32 master.
 */

/* fp16 -> fp32, exact. */
static float f16_to_f32(uint16_t h)
{
    uint32_t sign = (uint32_t)(h >> 15) << 31;
    uint32_t exp = (h >> 10) & 0x1fu;
    uint32_t man = h & 0x3ffu;
    float f;
    if (exp == 0x1fu) {                     /* inf or NaN */
        uint32_t u = sign | 0x7f800000u | (man << 13);
        memcpy(&f, &u, sizeof f);
        return f;
    }
    if (exp == 0) {                         /* zero or subnormal: man * 2^-24 */
        f = (float)man * 5.9604644775390625e-08f;
        return sign ? -f : f;
    }
    uint32_t u = sign | ((exp + 112u) << 23) | (man << 13);
    memcpy(&f, &u, sizeof f);
    return f;
}

/* fp32 -> fp16, round to nearest, ties to even; overflow -> inf; NaN -> the
 * quiet NaN 0x7e00 with the input's sign. */
static uint16_t f32_to_f16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    float a = fabsf(f);
    if (a != a)
        return (uint16_t)(sign | 0x7e00u);
    if (a >= 65520.0f)                      /* 65504 + half an ulp rounds up to inf */
        return (uint16_t)(sign | 0x7c00u);
    if (a < 6.103515625e-05f) {             /* below 2^-14: subnormal result, unit 2^-24 */
        double q = (double)a * 16777216.0;  /* exact: a is a float, 2^24 scaling */
        double r = floor(q);
        double rem = q - r;
        uint32_t m = (uint32_t)r;
        if (rem > 0.5 || (rem == 0.5 && (m & 1u)))
            m += 1u;                        /* may carry into the smallest normal, 0x0400 */
        return (uint16_t)(sign | m);
    }
    /* normal: keep 10 fraction bits of the fp32 significand, RNE on the 13 dropped */
    uint32_t au = u & 0x7fffffffu;
    uint32_t exp = (au >> 23) - 112u;       /* rebias 127 -> 15 */
    uint32_t man = (au >> 13) & 0x3ffu;
    uint32_t dropped = au & 0x1fffu;
    uint32_t h = (exp << 10) | man;
    if (dropped > 0x1000u || (dropped == 0x1000u && (man & 1u)))
        h += 1u;                            /* carries into the exponent correctly */
    return (uint16_t)(sign | h);
}

void zr_oracle_f16_from_f32(const float *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = f32_to_f16(x[i]);
}

void zr_oracle_f32_from_f16(const uint16_t *x, int64_t n, float *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = f16_to_f32(x[i]);
}

/* Mean of n fp16 contributions: fp32 sum in ascending k, one division, fp16. */
void zr_oracle_reduce_f16(const uint16_t *const *contribs, int32_t n, int64_t numel, uint16_t *out)
{
    for (int64_t i = 0; i < numel; ++i) {
        float sum = f16_to_f32(contribs[0][i]);
        for (int32_t k = 1; k < n; ++k)
            sum = sum + f16_to_f32(contribs[k][i]);
        out[i] = f32_to_f16(sum / (float)n);
    }
}

/* 1 if any fp16 value is inf or NaN. */
int32_t zr_oracle_found_inf_f16(const uint16_t *x, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        if ((x[i] & 0x7c00u) == 0x7c00u)
            return 1;
    return 0;
}

/*
 * AdamW step on an fp16 gradient scaled by the loss scale: the gradient is
 * divided by the scale (multiplied by 1/scale) before the update, and the
 * 16-bit copy is fp16.  Otherwise the same update as zr_oracle_adamw, in
 * double, stored in fp32.  The caller skips the call for a step whose
 * gradient overflowed.
 */
void zr_oracle_adamw_f16(const uint16_t *grad, float *master, float *exp_avg, float *exp_avg_sq,
                         uint16_t *param_out, int64_t numel,
                         double lr, double beta1, double beta2, double eps,
                         double weight_decay, double grad_scale, int64_t step, double loss_scale)
{
    double bias1 = 1.0 - pow(beta1, (double)step);
    double bias2 = 1.0 - pow(beta2, (double)step);
    double decay = 1.0 - lr * weight_decay;
    double unscale = 1.0 / loss_scale;
    for (int64_t i = 0; i < numel; ++i) {
        double g = (double)f16_to_f32(grad[i]) * unscale * grad_scale;
        double th = (double)master[i];
        double m = (double)exp_avg[i];
        double v = (double)exp_avg_sq[i];

        th = th * decay;
        m = beta1 * m + (1.0 - beta1) * g;
        v = beta2 * v + (1.0 - beta2) * g * g;
        th = th - lr * (m / bias1) / (sqrt(v / bias2) + eps);

        master[i] = (float)th;
        exp_avg[i] = (float)m;
        exp_avg_sq[i] = (float)v;
        if (param_out)
            param_out[i] = f32_to_f16(master[i]);
    }
}

/* ------------------------------------------------- int8 block quantizing ---- */

/*
 * Quantized weights for the parameter AllGather (ZeRO++ qwZ): the ZeRO-1/2/3
 * concept page (compassingai.com), ZeRO++ section, quantizes the weights sent
 * in the AllGather to int8 (or int4) to cut its volume, and leaves the details
 * to DeepSpeed.  Reading taken: symmetric block-wise int8.  For each block of
 * `block` consecutive elements (the last block may be shorter):
 *   amax  = max |x|                       (fp32, exact)
 *   s     = amax / 127                    (one fp32 division)
 *   q     = 0 if s == 0, else rint(x / s) (fp32 division, ties to even),
 *           clamped to [-127, 127]
 * and the receiver rebuilds x' = bf16(q * s) (one fp32 product, then bf16
 * round to nearest even).  Inputs are finite.
 */
void zr_oracle_quantize_int8(const uint16_t *src, int64_t numel, int32_t block, int8_t *q, float *scales)
{
    int64_t nblocks = (numel + block - 1) / block;
    for (int64_t b = 0; b < nblocks; ++b) {
        int64_t lo = b * block;
        int64_t hi = lo + block < numel ? lo + block : numel;
        float amax = 0.0f;
        for (int64_t i = lo; i < hi; ++i) {
            float a = fabsf(bf16_to_f32(src[i]));
            if (a > amax)
                amax = a;
        }
        float s = amax / 127.0f;
        scales[b] = s;
        for (int64_t i = lo; i < hi; ++i) {
            if (s == 0.0f) {
                q[i] = 0;
                continue;
            }
            float r = rintf(bf16_to_f32(src[i]) / s);
            if (r > 127.0f)
                r = 127.0f;
            if (r < -127.0f)
                r = -127.0f;
            q[i] = (int8_t)r;
        }
    }
}

void zr_oracle_dequantize_int8(const int8_t *q, const float *scales, int64_t numel, int32_t block, uint16_t *dst)
{
    for (int64_t i = 0; i < numel; ++i) {
        float x = (float)q[i] * scales[i / block];
        dst[i] = f32_to_bf16(x);
    }
}

/* ------------------------------------------------- int4 block quantizing ---- */

/*
 * The same ZeRO++ sentence of the concept page names int4 beside int8 and gives
 * no details.  Reading taken: the int8 rule above with 7 in place of 127,
 *   s = amax / 7,  q = 0 if s == 0, else rint(x / s) clamped to [-7, 7]
 * (symmetric codes: -8 never occurs), two codes per byte -- element 2j in the
 * low four bits of byte j, element 2j + 1 in the high four bits, each a 4-bit
 * two's-complement number -- and, for an odd count, 0 in the high four bits of
 * the last byte.  The receiver rebuilds x' = bf16(q * s) as for int8.
 */
void zr_oracle_quantize_int4(const uint16_t *src, int64_t numel, int32_t block, uint8_t *q4, float *scales)
{
    memset(q4, 0, (size_t)((numel + 1) / 2));
    int64_t nblocks = (numel + block - 1) / block;
    for (int64_t b = 0; b < nblocks; ++b) {
        int64_t lo = b * block;
        int64_t hi = lo + block < numel ? lo + block : numel;
        float amax = 0.0f;
        for (int64_t i = lo; i < hi; ++i) {
            float a = fabsf(bf16_to_f32(src[i]));
            if (a > amax)
                amax = a;
        }
        float s = amax / 7.0f;
        scales[b] = s;
        for (int64_t i = lo; i < hi; ++i) {
            int code = 0;
            if (s != 0.0f) {
                float r = rintf(bf16_to_f32(src[i]) / s);
                if (r > 7.0f)
                    r = 7.0f;
                if (r < -7.0f)
                    r = -7.0f;
                code = (int)r;
            }
            uint8_t nibble = (uint8_t)(code & 0xF);
            q4[i / 2] |= (i % 2) ? (uint8_t)(nibble << 4) : nibble;
        }
    }
}

void zr_oracle_dequantize_int4(const uint8_t *q4, const float *scales, int64_t numel, int32_t block, uint16_t *dst)
{
    for (int64_t i = 0; i < numel; ++i) {
        int nibble = (q4[i / 2] >> (4 * (i % 2))) & 0xF;
        int code = nibble >= 8 ? nibble - 16 : nibble;
        dst[i] = f32_to_bf16((float)code * scales[i / block]);
    }
}
