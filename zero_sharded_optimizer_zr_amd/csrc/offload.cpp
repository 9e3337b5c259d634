// ZeRO-Offload shard step: the fp32 master, exp_avg and exp_avg_sq of the
// rank's shard live in host memory and the AdamW update runs on the host CPU;
// the bf16 gradient shard comes down over PCIe and the bf16 parameter copy goes
// back up.
//
// Host AdamW: the same IEEE double operations, in the same order and without
// FMA contraction, as the GPU kernel (zr_adamw_step), on the same double
// scalars, each state rounded once to fp32, so both give the same bits.
// AVX-512 (8 double lanes) or AVX2 (4 double lanes) chosen at run time,
// scalar tails; the bf16 copy is rounded to nearest even with integer
// arithmetic, NaN kept quiet.  Work is split over a persistent pool of host
// threads in contiguous ranges.
//
// Offload pipeline: the shard is processed in chunks that fit a third of the
// caller's pinned staging buffer (a bf16 gradient slot and a bf16 parameter
// slot per third).  Gradient copies go on the caller's stream, so the first one
// follows whatever produced the gradient; parameter copies go on a stream of
// their own, so both directions of PCIe are busy at once.  While the host
// updates chunk i, the gradients of chunks i+1 and i+2 come down and the
// parameters of chunks i-1 and i-2 go up.  The call returns when every
// parameter has reached the device.
//
// Sources (web pages on DeepSpeed ZeRO-3): ZeRO tutorial (cnhsyj.com) 3.2
// (cpu_offload moves optimizer states, gradients and even parameters to CPU
// memory; PCIe bandwidth becomes the bottleneck); ZeRO-1/2/3 concept page
// (compassingai.com), history (ZeRO-Offload: fp32 optimizer states and part
// of the compute on the CPU, bounded by PCIe); encyclopedia entry
// (baike.kuaisou.com), history (ZeRO-2 Offload moves optimizer states and
// gradients to CPU memory, ZeRO-3 Offload adds parameters); Zero-3 article
// (hotelren.com), tuning notes (offload_optimizer / offload_param to cpu).
#include <immintrin.h>
#include <sched.h>
#include <unistd.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <condition_variable>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

#include "zr_math.hpp"

namespace zr {
namespace {

// ------------------------------------------------------------- host AdamW --

inline float host_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

inline uint16_t host_f32_to_bf16(float f)
{
    uint32_t u;
    std::memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x40u);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

void adamw_scalar(const uint16_t *g, float *th, float *m, float *v, uint16_t *p, int64_t n, const AdamWScalars &s)
{
    for (int64_t i = 0; i < n; ++i) {
        const double gr = (double)host_bf16_to_f32(g[i]) * s.grad_scale;
        double t = (double)th[i] * s.decay;
        const double mm = s.beta1 * (double)m[i] + s.one_minus_beta1 * gr;
        const double vv = s.beta2 * (double)v[i] + s.one_minus_beta2 * gr * gr;
        const double m_hat = mm / s.bias1;
        const double v_hat = vv / s.bias2;
        t = t - s.lr * m_hat / (std::sqrt(v_hat) + s.eps);
        th[i] = (float)t;
        m[i] = (float)mm;
        v[i] = (float)vv;
        if (p)
            p[i] = host_f32_to_bf16(th[i]);
    }
}

// bf16 bits (round to nearest even, NaN kept quiet) of 8 fp32 lanes, as uint16
__attribute__((target("avx2"))) inline __m128i bf16x8_avx2(__m256 x)
{
    const __m256i one = _mm256_set1_epi32(1), half = _mm256_set1_epi32(0x7fff);
    const __m256i absm = _mm256_set1_epi32(0x7fffffff), inf = _mm256_set1_epi32(0x7f800000);
    const __m256i u = _mm256_castps_si256(x);
    const __m256i hi = _mm256_srli_epi32(u, 16);
    __m256i r = _mm256_srli_epi32(_mm256_add_epi32(_mm256_add_epi32(u, half), _mm256_and_si256(hi, one)), 16);
    // |u| and inf are non-negative as int32, so the signed compare orders them
    const __m256i nan = _mm256_cmpgt_epi32(_mm256_and_si256(u, absm), inf);
    r = _mm256_blendv_epi8(r, _mm256_or_si256(hi, _mm256_set1_epi32(0x40)), nan);
    // 8 x int32 (all <= 0xffff) -> 8 x uint16
    return _mm256_castsi256_si128(_mm256_permute4x64_epi64(_mm256_packus_epi32(r, r), 0x08));
}

// 8 elements per iteration, 8 double lanes.
__attribute__((target("avx512f,avx512bw,avx512vl,avx2"))) void adamw_avx512(const uint16_t *g, float *th, float *m,
                                                                           float *v, uint16_t *p, int64_t n,
                                                                           const AdamWScalars &s)
{
    const __m512d gs = _mm512_set1_pd(s.grad_scale), dec = _mm512_set1_pd(s.decay);
    const __m512d b1 = _mm512_set1_pd(s.beta1), c1 = _mm512_set1_pd(s.one_minus_beta1);
    const __m512d b2 = _mm512_set1_pd(s.beta2), c2 = _mm512_set1_pd(s.one_minus_beta2);
    const __m512d bc1 = _mm512_set1_pd(s.bias1), bc2 = _mm512_set1_pd(s.bias2);
    const __m512d lr = _mm512_set1_pd(s.lr), eps = _mm512_set1_pd(s.eps);
    int64_t i = 0;
    for (; i + 8 <= n; i += 8) {
        const __m128i gh = _mm_loadu_si128(reinterpret_cast<const __m128i *>(g + i));
        const __m256 gf = _mm256_castsi256_ps(_mm256_slli_epi32(_mm256_cvtepu16_epi32(gh), 16));
        const __m512d gr = _mm512_mul_pd(_mm512_cvtps_pd(gf), gs);
        __m512d t = _mm512_mul_pd(_mm512_cvtps_pd(_mm256_loadu_ps(th + i)), dec);
        const __m512d mm = _mm512_add_pd(_mm512_mul_pd(b1, _mm512_cvtps_pd(_mm256_loadu_ps(m + i))),
                                         _mm512_mul_pd(c1, gr));
        const __m512d vv = _mm512_add_pd(_mm512_mul_pd(b2, _mm512_cvtps_pd(_mm256_loadu_ps(v + i))),
                                         _mm512_mul_pd(_mm512_mul_pd(c2, gr), gr));
        const __m512d m_hat = _mm512_div_pd(mm, bc1);
        const __m512d v_hat = _mm512_div_pd(vv, bc2);
        t = _mm512_sub_pd(t, _mm512_div_pd(_mm512_mul_pd(lr, m_hat), _mm512_add_pd(_mm512_sqrt_pd(v_hat), eps)));
        const __m256 tf = _mm512_cvtpd_ps(t);
        _mm256_storeu_ps(th + i, tf);
        _mm256_storeu_ps(m + i, _mm512_cvtpd_ps(mm));
        _mm256_storeu_ps(v + i, _mm512_cvtpd_ps(vv));
        if (p)
            _mm_storeu_si128(reinterpret_cast<__m128i *>(p + i), bf16x8_avx2(tf));
    }
    adamw_scalar(g + i, th + i, m + i, v + i, p ? p + i : nullptr, n - i, s);
}

// 8 elements per iteration as two halves of 4 double lanes.
__attribute__((target("avx2"))) void adamw_avx2(const uint16_t *g, float *th, float *m, float *v, uint16_t *p,
                                                int64_t n, const AdamWScalars &s)
{
    const __m256d gs = _mm256_set1_pd(s.grad_scale), dec = _mm256_set1_pd(s.decay);
    const __m256d b1 = _mm256_set1_pd(s.beta1), c1 = _mm256_set1_pd(s.one_minus_beta1);
    const __m256d b2 = _mm256_set1_pd(s.beta2), c2 = _mm256_set1_pd(s.one_minus_beta2);
    const __m256d bc1 = _mm256_set1_pd(s.bias1), bc2 = _mm256_set1_pd(s.bias2);
    const __m256d lr = _mm256_set1_pd(s.lr), eps = _mm256_set1_pd(s.eps);
    int64_t i = 0;
    for (; i + 8 <= n; i += 8) {
        const __m128i gh = _mm_loadu_si128(reinterpret_cast<const __m128i *>(g + i));
        const __m256 gf = _mm256_castsi256_ps(_mm256_slli_epi32(_mm256_cvtepu16_epi32(gh), 16));
        const __m256 thf = _mm256_loadu_ps(th + i), mf = _mm256_loadu_ps(m + i), vf = _mm256_loadu_ps(v + i);
        __m128 to[2], mo[2], vo[2];
        for (int h = 0; h < 2; ++h) {
            const __m128 gq = h ? _mm256_extractf128_ps(gf, 1) : _mm256_castps256_ps128(gf);
            const __m128 tq = h ? _mm256_extractf128_ps(thf, 1) : _mm256_castps256_ps128(thf);
            const __m128 mq = h ? _mm256_extractf128_ps(mf, 1) : _mm256_castps256_ps128(mf);
            const __m128 vq = h ? _mm256_extractf128_ps(vf, 1) : _mm256_castps256_ps128(vf);
            const __m256d gr = _mm256_mul_pd(_mm256_cvtps_pd(gq), gs);
            __m256d t = _mm256_mul_pd(_mm256_cvtps_pd(tq), dec);
            const __m256d mm = _mm256_add_pd(_mm256_mul_pd(b1, _mm256_cvtps_pd(mq)), _mm256_mul_pd(c1, gr));
            const __m256d vv = _mm256_add_pd(_mm256_mul_pd(b2, _mm256_cvtps_pd(vq)), _mm256_mul_pd(_mm256_mul_pd(c2, gr), gr));
            const __m256d m_hat = _mm256_div_pd(mm, bc1);
            const __m256d v_hat = _mm256_div_pd(vv, bc2);
            t = _mm256_sub_pd(t, _mm256_div_pd(_mm256_mul_pd(lr, m_hat), _mm256_add_pd(_mm256_sqrt_pd(v_hat), eps)));
            to[h] = _mm256_cvtpd_ps(t);
            mo[h] = _mm256_cvtpd_ps(mm);
            vo[h] = _mm256_cvtpd_ps(vv);
        }
        const __m256 tf = _mm256_set_m128(to[1], to[0]);
        _mm256_storeu_ps(th + i, tf);
        _mm256_storeu_ps(m + i, _mm256_set_m128(mo[1], mo[0]));
        _mm256_storeu_ps(v + i, _mm256_set_m128(vo[1], vo[0]));
        if (p)
            _mm_storeu_si128(reinterpret_cast<__m128i *>(p + i), bf16x8_avx2(tf));
    }
    adamw_scalar(g + i, th + i, m + i, v + i, p ? p + i : nullptr, n - i, s);
}

using AdamWFn = void (*)(const uint16_t *, float *, float *, float *, uint16_t *, int64_t, const AdamWScalars &);

// ZR_HOST_SIMD=scalar|avx2|avx512 caps the instruction set (for tests); by
// default the widest one the CPU supports.
AdamWFn pick_adamw(const char **name)
{
    const char *cap = std::getenv("ZR_HOST_SIMD");
    const int limit = !cap ? 2 : !std::strcmp(cap, "scalar") ? 0 : !std::strcmp(cap, "avx2") ? 1 : 2;
    __builtin_cpu_init();
    if (limit >= 2 && __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
        __builtin_cpu_supports("avx512vl")) {
        *name = "avx512";
        return adamw_avx512;
    }
    if (limit >= 1 && __builtin_cpu_supports("avx2")) {
        *name = "avx2";
        return adamw_avx2;
    }
    *name = "scalar";
    return adamw_scalar;
}

// ------------------------------------------------------------ thread pool --

int affinity_cpus()
{
    cpu_set_t set;
    if (sched_getaffinity(0, sizeof set, &set) == 0)
        return std::max(1, CPU_COUNT(&set));
    return std::max(1u, std::thread::hardware_concurrency());
}

// Persistent workers; run(k, fn) calls fn(0 .. k-1) across the workers and the
// calling thread and returns when all calls have finished.
class Pool {
public:
    explicit Pool(int n) : pid_(getpid())
    {
        for (int i = 0; i + 1 < n; ++i)
            workers_.emplace_back([this] { loop(); });
    }
    ~Pool()
    {
        {
            std::lock_guard<std::mutex> lk(mu_);
            stop_ = true;
        }
        cv_.notify_all();
        for (auto &t : workers_)
            t.join();
    }
    int size() const { return (int)workers_.size() + 1; }
    pid_t pid() const { return pid_; }

    void run(int tasks, const std::function<void(int)> &fn)
    {
        std::lock_guard<std::mutex> one_at_a_time(run_mu_);  // callers on several threads take turns
        std::unique_lock<std::mutex> lk(mu_);
        job_ = &fn;
        tasks_ = tasks;
        next_.store(0);
        busy_ = (int)workers_.size();
        ++gen_;
        lk.unlock();
        cv_.notify_all();
        work();
        lk.lock();
        done_.wait(lk, [this] { return busy_ == 0; });
        job_ = nullptr;
    }

private:
    void work()
    {
        for (int k = next_.fetch_add(1); k < tasks_; k = next_.fetch_add(1))
            (*job_)(k);
    }
    void loop()
    {
        uint64_t seen = 0;
        std::unique_lock<std::mutex> lk(mu_);
        for (;;) {
            cv_.wait(lk, [&] { return stop_ || gen_ != seen; });
            if (stop_)
                return;
            seen = gen_;
            lk.unlock();
            work();
            lk.lock();
            if (--busy_ == 0)
                done_.notify_one();
        }
    }

    std::vector<std::thread> workers_;
    std::mutex run_mu_, mu_;
    std::condition_variable cv_, done_;
    const std::function<void(int)> *job_ = nullptr;
    int tasks_ = 0;
    std::atomic<int> next_{0};
    int busy_ = 0;
    uint64_t gen_ = 0;
    bool stop_ = false;
    pid_t pid_;
};

std::mutex g_pool_mu;

// The process-wide pool, sized to the CPUs this process may run on.  After a
// fork the child has none of the parent's threads, so it gets a pool of its
// own (the parent's object is abandoned, not destroyed, in the child).
Pool &pool()
{
    static Pool *p = nullptr;
    std::lock_guard<std::mutex> lk(g_pool_mu);
    if (!p || p->pid() != getpid())
        p = new Pool(affinity_cpus());
    return *p;
}

struct HostAdamW {
    AdamWFn fn;
    const char *isa;
};

const HostAdamW &host_adamw()
{
    static const HostAdamW h = [] {
        HostAdamW x;
        x.fn = pick_adamw(&x.isa);
        return x;
    }();
    return h;
}

// AdamW over n elements on `threads` host threads (0: all of the pool's).
void host_step(const uint16_t *g, float *th, float *m, float *v, uint16_t *p, int64_t n, const AdamWScalars &s,
               int threads)
{
    Pool &P = pool();
    const int T = threads > 0 ? std::min(threads, P.size()) : P.size();
    const int64_t min_per_task = 1 << 14;
    const int tasks = (int)std::max<int64_t>(1, std::min<int64_t>(T, n / min_per_task));
    const AdamWFn fn = host_adamw().fn;
    if (tasks == 1) {
        fn(g, th, m, v, p, n, s);
        return;
    }
    // contiguous ranges, multiples of 16 elements except the last
    const int64_t per = ((n + tasks - 1) / tasks + 15) / 16 * 16;
    P.run(tasks, [&](int k) {
        const int64_t lo = std::min(n, (int64_t)k * per), hi = std::min(n, lo + per);
        if (lo < hi)
            fn(g + lo, th + lo, m + lo, v + lo, p ? p + lo : nullptr, hi - lo, s);
    });
}

zr_status check_host_buffers(const char *who, const void *grad, const float *master, const float *m, const float *v,
                             const void *param, int64_t numel, bool param_on_host)
{
    if (numel < 0)
        return fail(ZR_EINVAL, "%s: numel < 0", who);
    if (numel == 0)
        return ZR_OK;
    if (!grad || !master || !m || !v)
        return fail(ZR_EINVAL, "%s: NULL buffer", who);
    if (!aligned_to(grad, 2) || (param && !aligned_to(param, 2)))
        return fail(ZR_EALIGN, "%s: bf16 buffers must be 2-byte aligned", who);
    if (!aligned_to(master, 4) || !aligned_to(m, 4) || !aligned_to(v, 4))
        return fail(ZR_EALIGN, "%s: fp32 buffers must be 4-byte aligned", who);
    const void *p[5] = {master, m, v, param_on_host ? grad : nullptr, param_on_host ? param : nullptr};
    int64_t b[5] = {4 * numel, 4 * numel, 4 * numel, 2 * numel, 2 * numel};
    int x, y;
    if (any_overlap(p, b, 5, &x, &y))
        return fail(ZR_EINVAL, "%s: buffers %d and %d overlap", who, x, y);
    return ZR_OK;
}

// Waits for a HIP event by polling (a copy of one chunk takes a fraction of a
// millisecond, and a blocking wait's wake-up latency is a sizeable part of
// that); returns ZR_EHIP with the message on failure, or when the event has
// not completed after kWaitLimit (a chunk's copy, queued behind the caller's
// earlier work, should take far less).
constexpr std::chrono::seconds kWaitLimit(300);

zr_status wait_event(hipEvent_t e, const char *who)
{
    const auto start = std::chrono::steady_clock::now();
    for (uint32_t spin = 0;; ++spin) {
        const hipError_t err = hipEventQuery(e);
        if (err == hipSuccess)
            return ZR_OK;
        if (err != hipErrorNotReady)
            return fail(ZR_EHIP, "%s: %s", who, hipGetErrorString(err));
        for (int k = 0; k < 64; ++k)
            _mm_pause();
        if ((spin & 1023) == 1023 && std::chrono::steady_clock::now() - start > kWaitLimit)
            return fail(ZR_EHIP, "%s: a copy did not complete within %lld s", who, (long long)kWaitLimit.count());
    }
}

// Staging slots in flight: chunk i uses slot i % kSlots, so while the host
// updates chunk i, the gradients of chunks i+1 and i+2 can be coming down and
// the parameters of chunks i-1 and i-2 going up.
constexpr int kSlots = 3;

struct Events {
    hipEvent_t e[2 * kSlots] = {};  // gradient copy done [0, kSlots), parameter copy done [kSlots, 2 kSlots)
    ~Events()
    {
        for (auto x : e)
            if (x)
                (void)hipEventDestroy(x);
    }
};

// The stream of the parameter copies, one per device, made on first use (the
// gradient copies go on the caller's stream, after the work that produced the
// gradient; on a stream of their own the two directions of PCIe run at once).
zr_status upload_stream(hipStream_t *out, const char *who)
{
    static std::mutex mu;
    static std::vector<hipStream_t> streams;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return fail(ZR_EHIP, "%s: hipGetDevice failed", who);
    std::lock_guard<std::mutex> lk(mu);
    if ((int)streams.size() <= dev)
        streams.resize(dev + 1, nullptr);
    if (!streams[dev] && hipStreamCreateWithFlags(&streams[dev], hipStreamNonBlocking) != hipSuccess) {
        streams[dev] = nullptr;
        return fail(ZR_EHIP, "%s: hipStreamCreateWithFlags failed", who);
    }
    *out = streams[dev];
    return ZR_OK;
}

}  // namespace
}  // namespace zr

using namespace zr;

extern "C" zr_status zr_host_adamw_step(const void *grad, float *master, float *exp_avg, float *exp_avg_sq,
                                        void *param_out, int64_t numel, const zr_adamw_hparams *hp, int32_t threads)
{
    clear_error();
    const char *who = "zr_host_adamw_step";
    zr_status st = check_adamw_hparams(who, hp);
    if (st != ZR_OK)
        return st;
    if (threads < 0)
        return fail(ZR_EINVAL, "%s: threads < 0", who);
    st = check_host_buffers(who, grad, master, exp_avg, exp_avg_sq, param_out, numel, true);
    if (st != ZR_OK || numel == 0)
        return st;
    host_step(static_cast<const uint16_t *>(grad), master, exp_avg, exp_avg_sq, static_cast<uint16_t *>(param_out),
              numel, adamw_scalars(*hp), threads);
    return ZR_OK;
}

extern "C" const char *zr_host_simd(void) { return host_adamw().isa; }

extern "C" zr_status zr_offload_adamw_step(const void *grad, float *master, float *exp_avg, float *exp_avg_sq,
                                           void *param_out, int64_t numel, const zr_adamw_hparams *hp, void *staging,
                                           int64_t staging_bytes, int32_t threads, void *stream)
{
    clear_error();
    const char *who = "zr_offload_adamw_step";
    zr_status st = check_adamw_hparams(who, hp);
    if (st != ZR_OK)
        return st;
    if (threads < 0)
        return fail(ZR_EINVAL, "%s: threads < 0", who);
    st = check_host_buffers(who, grad, master, exp_avg, exp_avg_sq, param_out, numel, false);
    if (st != ZR_OK)
        return st;
    if (numel > 0 && param_out && overlaps(grad, 2 * numel, param_out, 2 * numel))
        return fail(ZR_EINVAL, "%s: grad and param_out overlap", who);
    if (!staging || staging_bytes < ZR_OFFLOAD_MIN_STAGING)
        return fail(ZR_EINVAL, "%s: staging must be at least %d bytes of pinned host memory", who,
                    (int)ZR_OFFLOAD_MIN_STAGING);
    if (!aligned_to(staging, 64))
        return fail(ZR_EALIGN, "%s: staging must be 64-byte aligned", who);
    {
        const void *p[4] = {master, exp_avg, exp_avg_sq, staging};
        int64_t b[4] = {4 * numel, 4 * numel, 4 * numel, staging_bytes};
        int x, y;
        if (any_overlap(p, b, 4, &x, &y))
            return fail(ZR_EINVAL, "%s: buffers %d and %d overlap (staging is 3)", who, x, y);
    }
    if (numel == 0)
        return ZR_OK;
    // The call waits for its own copies, so it cannot be recorded into a graph.
    hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(static_cast<hipStream_t>(stream), &capture) != hipSuccess)
        return fail(ZR_EHIP, "%s: hipStreamIsCapturing failed", who);
    if (capture != hipStreamCaptureStatusNone)
        return fail(ZR_EINVAL, "%s: the stream is being captured; this call is synchronous and cannot be recorded",
                    who);

    const AdamWScalars s = adamw_scalars(*hp);
    hipStream_t str = static_cast<hipStream_t>(stream), up = nullptr;
    if (param_out && (st = upload_stream(&up, who)) != ZR_OK)
        return st;
    // chunk: elements per slot pair (a gradient and a parameter slot)
    const int64_t chunk = std::min<int64_t>(numel, staging_bytes / (4 * kSlots) / 64 * 64);
    const int64_t nchunks = (numel + chunk - 1) / chunk;
    uint16_t *gslot[kSlots], *pslot[kSlots];
    for (int k = 0; k < kSlots; ++k) {
        gslot[k] = static_cast<uint16_t *>(staging) + (2 * k) * chunk;
        pslot[k] = static_cast<uint16_t *>(staging) + (2 * k + 1) * chunk;
    }
    const uint16_t *g = static_cast<const uint16_t *>(grad);
    uint16_t *pd = static_cast<uint16_t *>(param_out);

    Events ev;
    for (auto &e : ev.e)
        if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess)
            return fail(ZR_EHIP, "%s: hipEventCreateWithFlags failed", who);
    hipEvent_t *fetched = ev.e, *sent = ev.e + kSlots;

    auto len_of = [&](int64_t i) { return std::min(chunk, numel - i * chunk); };
    auto fetch = [&](int64_t i) -> zr_status {  // gradient chunk i -> slot i % kSlots
        const int k = (int)(i % kSlots);
        if (hipMemcpyAsync(gslot[k], g + i * chunk, 2 * len_of(i), hipMemcpyDeviceToHost, str) != hipSuccess ||
            hipEventRecord(fetched[k], str) != hipSuccess)
            return fail(ZR_EHIP, "%s: gradient copy of chunk %lld failed", who, (long long)i);
        return ZR_OK;
    };
    // On a failure after copies were enqueued, wait for them before returning,
    // so that the caller may free or reuse the staging buffer at once.
    auto bail = [&](zr_status e) {
        (void)hipStreamSynchronize(str);
        if (up)
            (void)hipStreamSynchronize(up);
        return e;
    };

    for (int64_t i = 0; i < kSlots && i < nchunks; ++i)
        if ((st = fetch(i)) != ZR_OK)
            return bail(st);
    for (int64_t i = 0; i < nchunks; ++i) {
        const int k = (int)(i % kSlots);
        const int64_t off = i * chunk, len = len_of(i);
        if ((st = wait_event(fetched[k], who)) != ZR_OK)
            return bail(st);
        if (pd && i >= kSlots && (st = wait_event(sent[k], who)) != ZR_OK)  // parameter slot k is free again
            return bail(st);
        host_step(gslot[k], master + off, exp_avg + off, exp_avg_sq + off, pd ? pslot[k] : nullptr, len, s, threads);
        if (pd && (hipMemcpyAsync(pd + off, pslot[k], 2 * len, hipMemcpyHostToDevice, up) != hipSuccess ||
                   hipEventRecord(sent[k], up) != hipSuccess))
            return bail(fail(ZR_EHIP, "%s: parameter copy of chunk %lld failed", who, (long long)i));
        if (i + kSlots < nchunks && (st = fetch(i + kSlots)) != ZR_OK)
            return bail(st);
    }
    if (pd && (st = wait_event(sent[(nchunks - 1) % kSlots], who)) != ZR_OK)  // the last parameter copy
        return bail(st);
    return ZR_OK;
}
