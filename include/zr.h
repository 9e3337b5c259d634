/*
 * zr.h -- C ABI of libzr: one data-parallel rank's share of a ZeRO-3 training
 * step on one AMD Instinct MI355X (gfx950).
 *
 * The share has four parts, each an entry point below:
 *   1. a flat, padded partition layout with rank slices and small-tensor
 *      persistence                                  (zr_layout_*)
 *   2. the local arithmetic of the gradient ReduceScatter: the mean of n bf16
 *      gradient contributions over the owned slice  (zr_reduce_slice)
 *   3. a fused mixed-precision AdamW step on the slice (zr_adamw_step)
 *   4. bit copies between per-tensor bf16 views and the flat buffer
 *                                                    (zr_pack / zr_unpack)
 * and 2 + 3 in one pass (zr_reduce_adamw_step), an fp16 variant of 2 + 3
 * with dynamic loss scaling (zr_*_f16, zr_loss_scale_*), int8 and int4 block
 * quantization of the bf16 shard for a quantized parameter AllGather
 * (zr_quantize_int8 / zr_dequantize_int8 / zr_unpack_int8 and the _int4
 * forms), the ZeRO-Offload step with the optimizer on the host
 * (zr_offload_adamw_step, zr_host_adamw_step), and captured steps replayed as
 * HIP graphs (zr_graph_*).
 *
 * Sources are web pages on DeepSpeed ZeRO-3, cited by title and section:
 *   [ENC]  "DeepSpeed ZeRO-3", encyclopedia entry (baike.kuaisou.com)
 *   [BLOG] "From DDP to ZeRO: memory sharding", blog (111qqz.com)
 *   [TUT]  ZeRO-1/2/3 tutorial (cnhsyj.com), numbered sections
 *   [ART]  "DeepSpeed Zero-3 parameter partitioning and on-demand access",
 *          article (hotelren.com)
 *   [CON]  "ZeRO-1/2/3 (Zero Redundancy Optimizer, three stages)",
 *          concept page (compassingai.com)
 *
 * Conventions for every call:
 *   - Validation first.  Every argument is checked on the host before any HIP
 *     call; a rejected call launches nothing and writes nothing, returns a
 *     non-zero zr_status and sets the calling thread's zr_last_error().
 *   - Asynchronous.  Device work is enqueued on `stream` (a hipStream_t; NULL is
 *     the null stream) and the call returns without synchronising.  A failed
 *     launch returns ZR_EHIP with the HIP error string in zr_last_error().
 *   - The library never allocates device memory.  Every device buffer belongs to
 *     the caller and must stay alive until the enqueued work has finished.
 *   - Element counts and offsets are int64.  bf16 buffers need 2-byte and fp32
 *     buffers 4-byte alignment (else ZR_EALIGN); 16-byte alignment is not
 *     required and gives the same bits as aligned buffers.
 *   - bf16 data is passed as raw 16-bit patterns (void*).
 *   - Two environment variables exist for testing and change no result:
 *     ZR_MAX_GRID (an integer >= 8) caps the workgroups of every launch -- each
 *     kernel loops over the work its grid does not cover; ZR_HOST_SIMD
 *     ("avx2" or "scalar") caps the instruction set of the host AdamW.
 */
#ifndef ZR_H
#define ZR_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Exported from libzr.so (the library is built with hidden visibility). */
#define ZR_API __attribute__((visibility("default")))

#define ZR_ABI_VERSION 1

typedef int32_t zr_status;
#define ZR_OK      0
#define ZR_EINVAL  1   /* malformed argument: NULL pointer, negative count, bad hyper-parameter, overlap */
#define ZR_ERANGE  2   /* index, rank or range outside what the layout or buffer allows; capacity too small */
#define ZR_EALIGN  3   /* buffer not naturally aligned for its element type */
#define ZR_ENOMEM  4   /* host allocation failed */
#define ZR_EHIP    5   /* HIP launch error */

/* Opaque, immutable after creation; safe to read from many threads at once. */
typedef struct zr_layout zr_layout;

typedef struct zr_layout_info {
    int64_t psi;            /* elements in all tensors */
    int64_t psi_part;       /* elements in partitioned tensors */
    int64_t psi_persist;    /* elements in persistent (replicated) tensors */
    int64_t psi_pad;        /* flat buffer length: psi_part rounded up to a multiple of n_d */
    int64_t shard;          /* elements per rank: psi_pad / n_d */
    int64_t threshold;      /* persistence threshold the layout was built with */
    int32_t n_d;            /* data-parallel ranks */
    int32_t n_tensors;
    int32_t n_partitioned;
    int32_t n_persistent;
} zr_layout_info;

/* A piece of one partitioned tensor inside a flat range. */
typedef struct zr_fragment {
    int32_t tensor;         /* index in the list given to zr_layout_create */
    int32_t reserved;       /* 0 */
    int64_t tensor_offset;  /* first element of the piece inside the tensor */
    int64_t flat_offset;    /* first element of the piece inside the flat buffer */
    int64_t numel;          /* elements in the piece (> 0) */
} zr_fragment;

/* A device bf16 window holding elements [first, first + count) of one tensor. */
typedef struct zr_view {
    void   *ptr;
    int64_t first;
    int64_t count;
} zr_view;

/* AdamW hyper-parameters.  The library derives the per-step scalars in double
 * and rounds each once to fp32 for the device. */
typedef struct zr_adamw_hparams {
    double  lr;
    double  beta1;
    double  beta2;
    double  eps;
    double  weight_decay;
    double  grad_scale;     /* the bf16 gradient is multiplied by this first (1.0 for a mean) */
    int64_t step;           /* t >= 1, the step's bias-correction exponent */
} zr_adamw_hparams;

/* ------------------------------------------------------------- layout ---- */

/*
 * Build the partition of a tensor list over n_d ranks.
 *
 * [ART] minimal ZeRO-3 config and its small-parameter residency paragraph:
 * tensors with fewer than `persist_threshold` elements (default 100000) are not
 * partitioned; they stay whole on every rank, in a separate replicated region
 * laid out in list order.  [TUT] 3.2 (contiguous gradient buffer) and 2.1 (rank
 * 0 owns the first 1/N_d, rank 1 the next): the other tensors are concatenated
 * in list order, with no gaps, into one flat buffer that is cut into n_d equal
 * contiguous slices; [BLOG] "ZeRO-3: why parameters can be sharded too" (8
 * parameters on 4 GPUs).  The pages assume n_d divides the count; here the flat
 * buffer is padded at its end to psi_pad = ceil(psi_part / n_d) * n_d, and the
 * padding is zero.
 *
 * numels: host array of n_tensors element counts (>= 0; 0 is allowed).
 * n_tensors >= 0; n_d >= 1; persist_threshold >= 0 (0: nothing is persistent).
 * On success *out owns host memory released by zr_layout_destroy.
 * Errors: ZR_EINVAL (NULL pointer, negative count, n_d < 1, negative threshold,
 * int64 overflow of a sum), ZR_ENOMEM.
 */
ZR_API zr_status zr_layout_create(const int64_t *numels, int32_t n_tensors, int32_t n_d,
                           int64_t persist_threshold, zr_layout **out);

/* Free a layout and the host memory it owns; NULL is ignored.  The layout is
 * the host-side record of the partition that zr_layout_create describes
 * ([TUT] 2.1); no device memory is involved. */
ZR_API void zr_layout_destroy(zr_layout *layout);

/* Sizes and counts of a layout: psi and its split into partitioned and
 * persistent elements ([ART] small-parameter residency paragraph: tensors
 * under the threshold stay whole on every rank), the padded flat length and
 * the per-rank slice ([TUT] 2.1: each rank owns 1/N_d of the flat buffer;
 * [ENC] Principle: each rank keeps 1/N_d of parameters, gradients and
 * optimizer state).  Errors: ZR_EINVAL (NULL). */
ZR_API zr_status zr_layout_query(const zr_layout *layout, zr_layout_info *out);

/* Tensor t: *persistent = 1 if replicated, and *offset = its offset in the
 * persistent region; else *persistent = 0 and *offset = its flat offset.
 * [ART] small-parameter residency paragraph (tensors under
 * stage3_param_persistence_threshold are kept whole on every rank rather than
 * partitioned) and minimal ZeRO-3 config (threshold 100000); [TUT] 3.2
 * (partitioned tensors live in one contiguous buffer, in list order).
 * Either output pointer may be NULL.  Errors: ZR_EINVAL, ZR_ERANGE (t). */
ZR_API zr_status zr_layout_tensor(const zr_layout *layout, int32_t t, int32_t *persistent, int64_t *offset);

/* Flat range [begin, end) = [rank * shard, (rank + 1) * shard) owned by rank
 * ([TUT] 2.1).  Errors: ZR_EINVAL, ZR_ERANGE (rank outside [0, n_d)). */
ZR_API zr_status zr_layout_rank_range(const zr_layout *layout, int32_t rank, int64_t *begin, int64_t *end);

/*
 * The pieces of partitioned tensors inside flat [begin, end), 0 <= begin <=
 * end <= psi_pad, in flat order ([BLOG] "ZeRO-3: why parameters can be sharded
 * too": one tensor may be split across ranks).  Empty tensors yield no piece.
 * Two-call idiom: writes min(count, cap) entries to out (out may be NULL when
 * cap is 0) and sets *n to the full count; returns ZR_ERANGE if cap < count.
 * Errors: ZR_EINVAL, ZR_ERANGE (range, capacity).
 */
ZR_API zr_status zr_layout_fragments(const zr_layout *layout, int64_t begin, int64_t end,
                              zr_fragment *out, int32_t cap, int32_t *n);

/*
 * Exact per-rank model-state bytes of this layout at ZeRO stage 0..3, 16 bytes
 * per element as 2 (bf16 param) + 2 (bf16 grad) + 12 (fp32 master, m, v):
 * [BLOG] ledger section; [CON] per-stage memory formulas (16 psi;
 * 4 psi + 12 psi/N_d; 2 psi + 14 psi/N_d; 16 psi/N_d); [ENC] principle section.
 * Owned state is one shard (padding included) plus every persistent tensor:
 *   stage 0: 16 psi
 *   stage 1: 4 psi + 12 (shard + psi_persist)
 *   stage 2: 2 psi + 14 (shard + psi_persist)
 *   stage 3: 16 (shard + psi_persist)
 * Errors: ZR_EINVAL, ZR_ERANGE (stage), ZR_EINVAL on int64 overflow.
 */
ZR_API zr_status zr_layout_ledger_bytes(const zr_layout *layout, int32_t stage, int64_t *bytes);

/* -------------------------------------------------------- pack/unpack ---- */

/*
 * Gather flat elements [begin, end) of the bf16 flat buffer from per-tensor
 * views: flat[j - begin] = element (j - offset_t) of the tensor t covering j,
 * and 0 where j lies in the padding.  Every element of the range is written.
 * This is the local half of the parameter AllGather and of the contiguous
 * gradient buffer ([BLOG] "ZeRO-1: why optimizer states can be sharded", the
 * [9] + [18] -> [9, 18] example; [TUT] 3.2 contiguous_gradients).
 *
 * views: host array of n_views == n_tensors entries, indexed by tensor.  The
 * entry of a partitioned tensor with elements in the range must cover those
 * elements (first <= piece start, piece end <= first + count) else ZR_ERANGE;
 * other entries (persistent tensors, tensors outside the range) are not read
 * and may be zeroed.  flat: device pointer to flat element `begin`, holding
 * end - begin bf16.  The views must not overlap flat.  Bit copy: any 16-bit
 * pattern (NaN payloads, -0, subnormals) is moved unchanged.
 * Errors: ZR_EINVAL, ZR_ERANGE, ZR_EALIGN, ZR_EHIP.
 */
ZR_API zr_status zr_pack(const zr_layout *layout, const zr_view *views, int32_t n_views,
                  void *flat, int64_t begin, int64_t end, void *stream);

/*
 * Inverse of zr_pack: scatter flat elements [begin, end) into the views.  Only
 * tensor elements inside the range are written; the padding goes nowhere.
 * Same argument rules as zr_pack.  This is the step after the AllGather that
 * turns the gathered flat bf16 buffer back into per-tensor parameters
 * ([BLOG] "ZeRO-1: why optimizer states can be sharded"; [CON] Stage 3
 * mechanism, gather before compute).
 */
ZR_API zr_status zr_unpack(const zr_layout *layout, const void *flat, int64_t begin, int64_t end,
                    const zr_view *views, int32_t n_views, void *stream);

/* ------------------------------------------------------------- reduce ---- */

/*
 * out[i] = bf16( (g_0[i] + g_1[i] + ... + g_{n-1}[i]) / n ) for 0 <= i < numel:
 * the mean of n bf16 gradient contributions, summed in fp32 in ascending k,
 * divided once by n, rounded to nearest even.  On a rank this is its slice of
 * the ReduceScatter ([BLOG] "ZeRO-2: why gradients can be sharded too", the
 * [2,6] + [4,10] -> rank 0 [3], rank 1 [8] example; [CON] Stage 2 and 3
 * mechanism).  Run over the persistent region it is the AllReduce mean.
 *
 * contribs: host array of n device pointers to bf16 [numel], 1 <= n <= 256.
 * out: device bf16 [numel]; it may be exactly contribs[0] (in place) and must
 * not otherwise overlap a contribution.  numel >= 0 (0 enqueues nothing).
 * Errors: ZR_EINVAL, ZR_EALIGN, ZR_EHIP.
 */
ZR_API zr_status zr_reduce_slice(const void *const *contribs, int32_t n, int64_t numel, void *out, void *stream);

/* -------------------------------------------------------------- AdamW ---- */

/*
 * One AdamW step on a shard, in place, fused with the bf16 working copy:
 *   g  = grad[i] * grad_scale
 *   th = th * (1 - lr * weight_decay)
 *   m  = beta1 * m + (1 - beta1) * g
 *   v  = beta2 * v + (1 - beta2) * g * g
 *   th = th - lr * (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)
 *   param_out[i] = bf16(th)   (round to nearest even)
 * computed in double, one IEEE operation at a time in this order (correctly
 * rounded division and square root, no fused multiply-add), on the fp32 state
 * and the bf16 gradient widened exactly and on the hyper-parameters as given;
 * each new state is rounded once to fp32 and the copy to bf16 from that fp32
 * master.  Each element uses only its own gradient and state ([BLOG]
 * "ZeRO-1: why optimizer states can be sharded"), so N_d shard updates
 * concatenate to the unsharded update; states are fp32 and the copy is bf16
 * ([BLOG] ledger section); the copy is made from the updated fp32 master
 * ([CON] Stage 1 mechanism); AdamW and its hyper-parameters: [TUT] 3.1.  The
 * formula is decoupled-weight-decay Adam (Loshchilov & Hutter, ICLR 2019).
 *
 * grad: device bf16 [numel].  master, exp_avg, exp_avg_sq: device fp32 [numel],
 * updated in place.  param_out: device bf16 [numel] or NULL (no copy).  No two
 * of the five buffers may overlap.  numel >= 0.  hp: host pointer; lr >= 0,
 * 0 <= beta1 < 1, 0 <= beta2 < 1, eps > 0, weight_decay >= 0, finite
 * grad_scale, step >= 1.
 * Errors: ZR_EINVAL, ZR_EALIGN, ZR_EHIP.
 */
ZR_API zr_status zr_adamw_step(const void *grad, float *master, float *exp_avg, float *exp_avg_sq,
                        void *param_out, int64_t numel, const zr_adamw_hparams *hp, void *stream);

/* ------------------------------------------------- fused reduce + AdamW ---- */

/*
 * zr_reduce_slice followed by zr_adamw_step in one pass over the shard: the
 * mean of the n bf16 gradient contributions is formed in fp32 (ascending k,
 * one division by n), rounded to bf16, and used at once as the gradient of the
 * AdamW update, without the bf16 gradient's round trip through memory.  Every
 * output is bit for bit what the two calls in sequence produce.  Above 24
 * contributions, where the one-pass kernel's concurrent streams cost more DRAM
 * efficiency than the mean's round trip saves, the call runs the two kernels
 * one after the other with the mean in grad_out or, without grad_out, in
 * param_out (which then receives the copy); with neither output the one-pass
 * kernel runs at any n.  After the
 * ReduceScatter each rank updates its parameter shard with its gradient shard
 * ([BLOG] "ZeRO-2: why gradients can be sharded too" and "ZeRO-1: why optimizer
 * states can be sharded"; [CON] Stage 1 and Stage 2 mechanism).
 *
 * contribs: host array of n device pointers to bf16 [numel], 1 <= n <= 256.
 * master, exp_avg, exp_avg_sq: device fp32 [numel], updated in place.
 * param_out: device bf16 [numel] or NULL.  grad_out: device bf16 [numel] or
 * NULL; when given it receives the bf16 mean (what zr_reduce_slice writes) and
 * may be exactly contribs[0].  No other overlap between a contribution and an
 * output, or between two outputs, is allowed.  hp as for zr_adamw_step.
 * Errors: ZR_EINVAL, ZR_EALIGN, ZR_EHIP.
 */
ZR_API zr_status zr_reduce_adamw_step(const void *const *contribs, int32_t n, float *master, float *exp_avg,
                                      float *exp_avg_sq, void *param_out, void *grad_out, int64_t numel,
                                      const zr_adamw_hparams *hp, void *stream);

/* ------------------------------------------------- fp16 + loss scaling ---- */

/*
 * fp16 variant of the step with dynamic loss scaling.  The backward pass gives
 * fp16 gradients multiplied by the loss scale S.  Per step:
 *   zr_reduce_slice_f16   mean of the n fp16 contributions (fp32 sum, one
 *                         division, fp16 round to nearest even); sets
 *                         ls->found_inf if any mean is inf or NaN;
 *   zr_adamw_step_f16     when ls->found_inf is clear: AdamW on g / S with an
 *                         fp16 copy; when it is set: nothing is written (the
 *                         step is skipped);
 *   zr_loss_scale_update  on overflow S <- max(S / factor, min_scale) and the
 *                         clean-step count restarts; otherwise after `window`
 *                         consecutive clean steps S <- S * factor; then
 *                         ls->found_inf is cleared.
 * [TUT] 3.1 (fp16 with a dynamic loss scale, window 1000, initial scale 2^16)
 * and 4.2 (dynamic scaling for fp16 gradients that are very small or very
 * large); [CON] 16 B/param table (fp16 parameters and gradients) and Stage 1
 * mechanism (16-bit copy of the updated fp32 master).  The skip-and-rescale
 * rule is standard dynamic loss scaling (Micikevicius et al., ICLR 2018).
 * fp16 NaN results are the quiet NaN sign | 0x7e00.
 *
 * The record lives in device memory (caller-allocated, 4-byte aligned) and is
 * only read and written by the kernels, in stream order; the host never has to
 * synchronise to run a step.
 */
typedef struct zr_loss_scale {
    float   scale;       /* current loss scale S */
    int32_t good_steps;  /* consecutive clean steps since the last change */
    int32_t found_inf;   /* set by the overflow checks, cleared by zr_loss_scale_update */
    int32_t skipped;     /* steps skipped so far */
} zr_loss_scale;

/* Device record <- {initial_scale, 0, 0, 0}.  initial_scale finite and > 0.
 * Errors: ZR_EINVAL, ZR_EALIGN, ZR_EHIP. */
ZR_API zr_status zr_loss_scale_init(zr_loss_scale *ls, float initial_scale, void *stream);

/* Mean of n fp16 contributions into out (fp16 [numel]); ls may be NULL (no
 * overflow flag).  Same buffer rules as zr_reduce_slice; ls must not overlap
 * a buffer.  Errors: ZR_EINVAL, ZR_EALIGN, ZR_EHIP. */
ZR_API zr_status zr_reduce_slice_f16(const void *const *contribs, int32_t n, int64_t numel, void *out,
                                     zr_loss_scale *ls, void *stream);

/* Sets ls->found_inf if any of grad (fp16 [numel]) is inf or NaN (for
 * gradients reduced by other means).  Errors: ZR_EINVAL, ZR_EALIGN, ZR_EHIP. */
ZR_API zr_status zr_check_finite_f16(const void *grad, int64_t numel, zr_loss_scale *ls, void *stream);

/* AdamW on the fp16 gradient divided by ls->scale (then times hp->grad_scale),
 * fp16 copy into param_out (or NULL); skipped entirely while ls->found_inf is
 * set: nothing is written (the data is read before the flag is consulted).
 * The bias corrections use hp->step exactly as passed: the library never
 * advances or rewinds it, and a skipped call does not change it by itself.  A
 * caller that follows the usual rule of dynamic loss scaling (the optimizer
 * step does not advance on a skipped step) passes the count of applied steps,
 * calls made minus ls->skipped; passing the count of calls advances t over
 * skips.  Same buffer rules as zr_adamw_step.
 * Errors: ZR_EINVAL, ZR_EALIGN, ZR_EHIP. */
ZR_API zr_status zr_adamw_step_f16(const void *grad, float *master, float *exp_avg, float *exp_avg_sq,
                                   void *param_out, int64_t numel, const zr_adamw_hparams *hp,
                                   const zr_loss_scale *ls, void *stream);

/* The scale rule above (one device thread).  window >= 1, factor finite and
 * > 1, min_scale finite and > 0.  Errors: ZR_EINVAL, ZR_EALIGN, ZR_EHIP. */
ZR_API zr_status zr_loss_scale_update(zr_loss_scale *ls, int32_t window, float factor, float min_scale,
                                      void *stream);

/* ------------------------------------------------- int8 weight gather ---- */

/*
 * Quantized parameter AllGather: before the gather the rank turns its bf16
 * parameter shard into int8 codes plus one fp32 scale per block (about 1 byte
 * per element instead of 2), and after it every rank turns the gathered codes
 * back into bf16.  [CON] ZeRO++ section (qwZ: the weights carried by the
 * AllGather are quantized to int8 or int4 to cut its volume; the scheme is left
 * to DeepSpeed); [ENC] history section (ZeRO++ as the follow-up that reduces
 * communication volume).  Reading taken: symmetric, block-wise, per block of
 * `block` consecutive elements (the last block may be shorter):
 *   amax = max |x|, s = amax / 127 (fp32), q = rint(x / s) clamped to
 *   [-127, 127] (ties to even; q = 0 when s = 0);  x' = bf16(q * s)
 * with every division and product one fp32 operation, so the codes, scales and
 * rebuilt values are exact functions of the input bits.  The input must be
 * finite.
 *
 * block is 256, 512, 1024 or 2048.  scales has ceil(numel / block) fp32
 * entries.  bf16 buffers need 2-byte and scales 4-byte alignment (else
 * ZR_EALIGN); q has no alignment rule, and buffers that are 16-byte (bf16)
 * and 8-byte (int8) aligned take the vector path (same bits).  No two buffers
 * may overlap.  numel == 0 is a no-op.  Errors: ZR_EINVAL, ZR_EALIGN, ZR_EHIP.
 */
ZR_API zr_status zr_quantize_int8(const void *src, int64_t numel, int32_t block, int8_t *q, float *scales,
                                  void *stream);

/* Rebuilds bf16 dst[numel] from the codes and scales of zr_quantize_int8. */
ZR_API zr_status zr_dequantize_int8(const int8_t *q, const float *scales, int64_t numel, int32_t block, void *dst,
                                    void *stream);

/*
 * Dequantize-on-unpack for the quantized AllGather over the partition: every
 * rank r quantizes its shard, flat elements [r S, (r+1) S), with
 * zr_quantize_int8 -- so blocks restart at every shard, and a shard's last
 * block is short when `block` does not divide S -- and the gather concatenates
 * codes and scales in rank order (ceil(S / block) scales per rank).  This call
 * rebuilds flat elements [begin, end) as bf16(code * scale of their block) and
 * writes them into the tensor views like zr_unpack, without a bf16 flat buffer
 * in between.  [CON] ZeRO++ section (qwZ) and Stage 3 mechanism (parameters
 * gathered before compute); [BLOG] "ZeRO-3: why parameters can be sharded
 * too".
 *
 * q[k] is the code of flat element begin + k (end - begin bytes); scales[0] is
 * the scale of the block that holds element begin and the following entries
 * are the next blocks in gathered order; scales must be 4-byte aligned.  Views
 * and their rules are those of zr_unpack (views may not overlap the codes or
 * the scales).  Persistent tensors and the padding are not written.
 * begin == end is a no-op.  Errors: ZR_EINVAL, ZR_ERANGE, ZR_EALIGN, ZR_EHIP.
 */
ZR_API zr_status zr_unpack_int8(const zr_layout *layout, const int8_t *q, const float *scales, int32_t block,
                                int64_t begin, int64_t end, const zr_view *views, int32_t n_views, void *stream);

/*
 * int4 codes for the same AllGather.  [CON] ZeRO++ section names int4 beside
 * int8 for qwZ and gives no details; the rule taken is the int8 one with 7 in
 * place of 127: per block s = amax / 7, q = rint(x / s) clamped to [-7, 7]
 * (q = 0 when s = 0), rebuilt as bf16(q * s).  Codes are 4-bit two's
 * complement, two per byte: element 2j in the low four bits of byte j, element
 * 2j + 1 in the high four bits; an odd count leaves 0 in the last byte's high
 * four bits.
 *
 * zr_quantize_int4: q4 holds ceil(numel / 2) bytes, scales ceil(numel / block)
 * fp32; buffer rules and errors as zr_quantize_int8 (q4 has no alignment rule;
 * 16-byte bf16 and 4-byte code buffers take the vector path, same bits).
 * zr_dequantize_int4: the inverse for numel elements.
 */
ZR_API zr_status zr_quantize_int4(const void *src, int64_t numel, int32_t block, uint8_t *q4, float *scales,
                                  void *stream);
ZR_API zr_status zr_dequantize_int4(const uint8_t *q4, const float *scales, int64_t numel, int32_t block, void *dst,
                                    void *stream);

/*
 * Dequantize-on-unpack of an int4 AllGather: every rank quantizes its shard
 * with zr_quantize_int4, so blocks and the packing restart at every shard --
 * ceil(S / 2) bytes and ceil(S / block) scales per rank -- and the gather
 * concatenates them in rank order.  q4[0] is the byte that holds the code of
 * flat element begin (in its high four bits when begin - r S is odd, r the
 * rank of begin); scales[0] is the scale of the block that holds element
 * begin.  Otherwise as zr_unpack_int8.
 */
ZR_API zr_status zr_unpack_int4(const zr_layout *layout, const uint8_t *q4, const float *scales, int32_t block,
                                int64_t begin, int64_t end, const zr_view *views, int32_t n_views, void *stream);

/* ------------------------------------------------ ZeRO-Offload step ----- */

/*
 * ZeRO-Offload: the shard's fp32 master / exp_avg / exp_avg_sq live in host
 * memory and the AdamW update runs on the host CPU; the bf16 gradient shard
 * crosses PCIe to the host and the bf16 parameter copy crosses back.  [TUT]
 * 3.2 (cpu_offload moves optimizer states, gradients and even parameters to CPU
 * memory; PCIe becomes the bottleneck); [CON] history (ZeRO-Offload: fp32
 * optimizer states and part of the compute on the CPU); [ENC] history (ZeRO-2
 * Offload, ZeRO-3 Offload); [ART] tuning notes (offload_optimizer to cpu).
 *
 * The host update performs the IEEE fp32 operations of zr_adamw_step, in the
 * same order and on the same fp32 scalars, so it gives the same bits as the GPU
 * kernel (AVX-512 or AVX2 chosen at run time; scalar tails).
 */

/* Smallest staging buffer zr_offload_adamw_step accepts (bytes). */
#define ZR_OFFLOAD_MIN_STAGING 65536

/*
 * zr_adamw_step on host buffers: grad (bf16 [numel]), master / exp_avg /
 * exp_avg_sq (fp32 [numel], in place), param_out (bf16 [numel] or NULL), all
 * in host memory.  threads: host threads to use, 0 = every CPU the process may
 * run on.  Synchronous.  Buffer rules as zr_adamw_step (2- and 4-byte
 * alignment, no overlaps).  Errors: ZR_EINVAL, ZR_EALIGN.
 */
ZR_API zr_status zr_host_adamw_step(const void *grad, float *master, float *exp_avg, float *exp_avg_sq,
                                    void *param_out, int64_t numel, const zr_adamw_hparams *hp, int32_t threads);

/* Instruction set the host update uses: "avx512", "avx2" or "scalar". */
ZR_API const char *zr_host_simd(void);

/*
 * The offloaded step: grad (device, bf16 [numel]) -> host AdamW on master /
 * exp_avg / exp_avg_sq (host, fp32 [numel], in place) -> param_out (device,
 * bf16 [numel], or NULL for no copy).  staging is caller-owned pinned host
 * memory (hipHostMalloc), 64-byte aligned, of staging_bytes >=
 * ZR_OFFLOAD_MIN_STAGING; the shard goes through it in chunks of
 * staging_bytes / 12 elements (rounded down to a multiple of 64; three chunks
 * in flight), so that the copies of neighbouring chunks overlap the host update
 * of one.  Gradient copies are enqueued on `stream`, after the work already
 * there (e.g. the reduce that produced grad); parameter copies go on a stream
 * the library keeps per device.  The call is synchronous: it returns when the states are updated and
 * every parameter has reached the device (or, on an error, when the copies it
 * enqueued have finished); being synchronous, it cannot be recorded into a
 * captured step (ZR_EINVAL while `stream` is being captured).  Errors:
 * ZR_EINVAL, ZR_EALIGN, ZR_EHIP.
 */
ZR_API zr_status zr_offload_adamw_step(const void *grad, float *master, float *exp_avg, float *exp_avg_sq,
                                       void *param_out, int64_t numel, const zr_adamw_hparams *hp, void *staging,
                                       int64_t staging_bytes, int32_t threads, void *stream);

/* ------------------------------------------------------ captured steps ---- */

/*
 * A sequence of the calls above, recorded once on a stream as a HIP graph and
 * replayed as one launch (an execution facility: the operations are those of
 * the recorded calls).  A training loop repeats the same calls on the same
 * buffers every step; on small shards the launches dominate the step.
 *
 *   zr_graph_capture_begin(s);  ...calls on stream s...;  zr_graph_capture_end(s, &g);
 *   for each step: zr_graph_set_adamw(g, &hp_t); zr_graph_launch(g, s);
 *
 * Buffers, sizes, layouts and the fp16 loss-scale record are fixed at
 * capture; the AdamW hyper-parameters (step t, lr, ...) of every recorded
 * AdamW-family call (zr_adamw_step, zr_reduce_adamw_step, zr_adamw_step_f16)
 * are replaced by zr_graph_set_adamw, which affects the following launches
 * (until then the captured values apply).  A replay gives the same bits as
 * the eager calls.  The calls are validated at capture time, as usual, and
 * enqueue nothing then.  zr_offload_adamw_step synchronises with the host and
 * cannot be recorded.  Launching the same graph on two streams at once races.
 */
typedef struct zr_graph zr_graph;

/* Starts recording on `stream` (not the null stream; thread-local capture
 * mode).  Errors: ZR_EINVAL, ZR_EHIP. */
ZR_API zr_status zr_graph_capture_begin(void *stream);

/* Ends the recording and instantiates it; *out owns it (zr_graph_destroy).
 * Errors: ZR_EINVAL (NULL argument, nothing recorded), ZR_ENOMEM, ZR_EHIP. */
ZR_API zr_status zr_graph_capture_end(void *stream, zr_graph **out);

/* Kernel nodes recorded, and how many of them take AdamW hyper-parameters.
 * Either output may be NULL.  Errors: ZR_EINVAL. */
ZR_API zr_status zr_graph_info(const zr_graph *g, int32_t *kernels, int32_t *adamw_nodes);

/* Hyper-parameters for every AdamW-family node of the following launches
 * (validated like zr_adamw_step).  Errors: ZR_EINVAL, ZR_EHIP. */
ZR_API zr_status zr_graph_set_adamw(zr_graph *g, const zr_adamw_hparams *hp);

/* Replays the graph on `stream`.  Errors: ZR_EINVAL, ZR_EHIP. */
ZR_API zr_status zr_graph_launch(zr_graph *g, void *stream);

/* Releases the graph; NULL is ignored.  Wait for its launches to finish
 * first. */
ZR_API void zr_graph_destroy(zr_graph *g);

/* ------------------------------------------------------------- misc ------ */

/* Message for the last failing call on this thread ("" if none). */
ZR_API const char *zr_last_error(void);

/* ZR_ABI_VERSION of the loaded library. */
ZR_API int32_t zr_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ZR_H */
