// Local arithmetic of the gradient ReduceScatter on one rank's slice (gfx950):
// out = bf16(mean of n bf16 contributions), summed in fp32 in ascending
// contribution order, divided once by n, rounded to nearest even.
//
// Per element: n two-byte reads and one two-byte write, a few fp32 adds: bound
// by HBM bandwidth at (2n + 2) bytes per element.  Each lane takes 8
// consecutive elements (one 16-byte non-temporal load per contribution, one
// 16-byte store), one group per lane over a grid that covers the slice;
// contribution loads are issued four at a time so several 16-byte reads are in
// flight per lane.  With n + 1 concurrent streams the DRAM rows thrash when
// every CU is full of waves, so the kernel caps its residency with LDS it
// reserves and never touches, and for up to 8 contributions it deals its tiles
// to the XCDs in runs (kReduceOrder).  Measured on MI355X against uncapped,
// launch order, on the same buffers: n = 4 at 5 workgroups per CU with one
// contiguous run per XCD 6.06 -> 6.43 TB/s; n = 8 at 4 per CU 5.66 -> 5.99
// TB/s (the cap alone gained nothing at n <= 8 in this arrangement), and runs
// of 256 tiles, rotated, gained another 2-3%; n = 64 at 2 per CU in launch
// order 5.8 -> 6.1-6.3 TB/s, where the contiguous runs lost a tenth.  Two
// 8-element chunks per lane (twice the loads in flight) lost 3-4% at n = 4
// and n = 8 at every cap from 3 to 5 workgroups per CU.  For 7 and 8
// contributions a second kernel takes 4 elements per lane with all n 8-byte
// loads in flight at once (see kFourPerLaneMinN).  The n device pointers travel
// by value in the kernel arguments.
//
// Sources (web pages on DeepSpeed ZeRO-3): "From DDP to ZeRO: memory sharding"
// blog (111qqz.com), "ZeRO-2: why gradients can be sharded too" (ReduceScatter
// leaves rank r with slice r of the averaged gradient: [2,6] and [4,10] give
// [3] and [8]) and its ledger section (bf16 gradients); ZeRO-1/2/3 concept page
// (compassingai.com), Stage 2 and Stage 3 mechanism.
#include "zr_math.hpp"

namespace zr {

constexpr int kLoadBatch = 4;  // contribution loads in flight per lane

// From this many contributions (up to 8) the 4-elements-per-lane kernel runs:
// 8 one-pass 8-byte loads per lane beat two batches of 4 16-byte loads.
// Measured on MI355X (same buffers, 1.95e9 elements unless noted): n = 8
// 0.775 of peak against 0.751 (the GPT shard's 1.2e8: 0.777 against 0.737),
// n = 7 0.768 against 0.758, n = 6 0.731 against 0.769, n = 5 0.686 against
// 0.776, n = 4 0.649 against 0.802.
constexpr int32_t kFourPerLaneMinN = 7;

// Dynamic LDS reserved per workgroup (160 KB per CU): residency cap by n.
inline size_t residency_cap_lds(int32_t n)
{
    if (n > 8)
        return 80 * 1024;  // 2 workgroups per CU
    if (n > 4)
        return 40 * 1024;  // 4 workgroups per CU
    return 32 * 1024;      // 5 workgroups per CU
}


__device__ __forceinline__ void add8(float (&acc)[8], u32x4 x)
{
    acc[0] += bf16_lo(x.x);
    acc[1] += bf16_hi(x.x);
    acc[2] += bf16_lo(x.y);
    acc[3] += bf16_hi(x.y);
    acc[4] += bf16_lo(x.z);
    acc[5] += bf16_hi(x.z);
    acc[6] += bf16_lo(x.w);
    acc[7] += bf16_hi(x.w);
}

__device__ __forceinline__ void set8(float (&acc)[8], u32x4 x)
{
    acc[0] = bf16_lo(x.x);
    acc[1] = bf16_hi(x.x);
    acc[2] = bf16_lo(x.y);
    acc[3] = bf16_hi(x.y);
    acc[4] = bf16_lo(x.z);
    acc[5] = bf16_hi(x.z);
    acc[6] = bf16_lo(x.w);
    acc[7] = bf16_hi(x.w);
}

// Tile orders (first_tile): runs of 256 tiles per XCD for up to 8
// contributions (1 MB of each contribution per run; +0.5-3.5% over the single
// run per XCD or launch order, on the same buffers), rotated from group to
// group (another 2%); launch order above 8 (runs lost up to 4% at n = 64).
constexpr int kReduceOrder = 256;  // 8 elements per lane, up to 6 contributions
constexpr int kReduce4Order = 256;  // 4 per lane, 7 or 8
constexpr int kReduceWideOrder = 1;  // more than 8
constexpr bool kReduceRotate = true;

// Tile order of the 8-element reduce: up to 8 contributions, or more.
template <int MaxN>
constexpr int reduce_order()
{
    return MaxN <= 8 ? kReduceOrder : kReduceWideOrder;
}

// Vector body over `groups` groups of 8 elements from element `head` (where
// every contribution and the output are 16-byte aligned), in tiles of kBlock
// groups in the order reduce_order<MaxN>(); block 0 also does the unaligned
// head [0, head) and the tail element-wise.  out may be c.p[0]: each lane
// reads all its inputs before it writes.
template <int MaxN>
__global__ __launch_bounds__(kBlock) void reduce_vec_kernel(ContribTable<MaxN> c, int32_t n, uint16_t *out,
                                                            int64_t numel, int64_t head, int64_t groups,
                                                            MeanDivisor d)
{
    u32x4 *o4 = reinterpret_cast<u32x4 *>(out + head);
    for (int64_t i = first_tile<reduce_order<MaxN>(), kReduceRotate>() * kBlock + threadIdx.x; i < groups;
         i += grid_stride()) {
        float acc[8];
        for (int32_t k = 0; k < n; k += kLoadBatch) {
            u32x4 x[kLoadBatch];
#pragma unroll
            for (int u = 0; u < kLoadBatch; ++u)
                if (k + u < n)
                    x[u] = load_stream(reinterpret_cast<const u32x4 *>(c.p[k + u] + head) + i);
#pragma unroll
            for (int u = 0; u < kLoadBatch; ++u) {
                if (k + u == 0)
                    set8(acc, x[u]);
                else if (k + u < n)
                    add8(acc, x[u]);
            }
        }
        u32x4 r;
        r.x = pack_bf16x2(finish_mean(acc[0], d), finish_mean(acc[1], d));
        r.y = pack_bf16x2(finish_mean(acc[2], d), finish_mean(acc[3], d));
        r.z = pack_bf16x2(finish_mean(acc[4], d), finish_mean(acc[5], d));
        r.w = pack_bf16x2(finish_mean(acc[6], d), finish_mean(acc[7], d));
        store_stream(o4 + i, r);
    }
    if (blockIdx.x == 0) {
        int64_t tail_start = head + 8 * groups;
        int64_t edge = head + (numel - tail_start);
        if ((int64_t)threadIdx.x < edge) {
            int64_t j = (int64_t)threadIdx.x < head ? (int64_t)threadIdx.x : tail_start + (threadIdx.x - head);
            out[j] = reduce_one(c, n, j, d);
        }
    }
}

// 7 or 8 contributions, 4 elements per lane: one 8-byte load per contribution,
// all of them in flight before the sum (ascending k, the same bits as above),
// one 8-byte store, at most 5 workgroups per CU; tiles in the order
// kReduce4Order.
__global__ __launch_bounds__(kBlock) void reduce4_vec_kernel(ContribTable<8> c, int32_t n, uint16_t *out, int64_t numel,
                                                             int64_t head, int64_t groups, MeanDivisor d)
{
    u32x2 *o2 = reinterpret_cast<u32x2 *>(out + head);
    for (int64_t i = first_tile<kReduce4Order, kReduceRotate>() * kBlock + threadIdx.x; i < groups;
         i += grid_stride()) {
        u32x2 x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (u < n)
                x[u] = load_stream(reinterpret_cast<const u32x2 *>(c.p[u] + head) + i);
        float acc[4] = {bf16_lo(x[0].x), bf16_hi(x[0].x), bf16_lo(x[0].y), bf16_hi(x[0].y)};
#pragma unroll
        for (int u = 1; u < 8; ++u)
            if (u < n) {
                acc[0] += bf16_lo(x[u].x);
                acc[1] += bf16_hi(x[u].x);
                acc[2] += bf16_lo(x[u].y);
                acc[3] += bf16_hi(x[u].y);
            }
        store_stream(o2 + i, u32x2{pack_bf16x2(finish_mean(acc[0], d), finish_mean(acc[1], d)),
                                   pack_bf16x2(finish_mean(acc[2], d), finish_mean(acc[3], d))});
    }
    if (blockIdx.x == 0) {
        int64_t tail_start = head + 4 * groups;
        int64_t edge = head + (numel - tail_start);  // at most 63 + 3
        if ((int64_t)threadIdx.x < edge) {
            int64_t j = (int64_t)threadIdx.x < head ? (int64_t)threadIdx.x : tail_start + (threadIdx.x - head);
            out[j] = reduce_one(c, n, j, d);
        }
    }
}

// Fallback when the buffers' 16-byte phases disagree: element-wise, same bits.
template <int MaxN>
__global__ __launch_bounds__(kBlock) void reduce_scalar_kernel(ContribTable<MaxN> c, int32_t n, uint16_t *out,
                                                               int64_t numel, MeanDivisor d)
{
    for (int64_t j = global_tid(); j < numel; j += grid_stride())
        out[j] = reduce_one(c, n, j, d);
}

template <int MaxN>
static zr_status reduce_launch(const void *const *contribs, int32_t n, int64_t numel, uint16_t *out,
                               hipStream_t st, const MeanDivisor &d)
{
    ContribTable<MaxN> c = {};
    for (int32_t k = 0; k < n; ++k)
        c.p[k] = static_cast<const uint16_t *>(contribs[k]);
    const int64_t head = line_head16(out, numel);
    if constexpr (MaxN == 8) {
        // 7 or 8 contributions: 4 elements per lane, every load in flight at once
        bool vec4 = n >= kFourPerLaneMinN;
        for (int32_t k = 0; k < n && vec4; ++k)
            vec4 = aligned_to(c.p[k] + head, 8);
        if (vec4) {
            const int64_t groups = (numel - head) / 4, tiles = (groups + kBlock - 1) / kBlock;
            return launch(reduce4_vec_kernel, order_grid<kReduce4Order>(tiles), dim3(kBlock), 32 * 1024, st, c, n,
                          out, numel, head, groups, d);
        }
    }
    bool vec = true;
    for (int32_t k = 0; k < n && vec; ++k)
        vec = aligned_to(c.p[k] + head, 16);
    if (vec) {
        const int64_t groups = (numel - head) / 8, tiles = (groups + kBlock - 1) / kBlock;
        return launch(reduce_vec_kernel<MaxN>, order_grid<reduce_order<MaxN>()>(tiles), dim3(kBlock),
                      residency_cap_lds(n), st, c, n, out, numel, head, groups, d);
    }
    return launch(reduce_scalar_kernel<MaxN>, grid_of((numel + kBlock - 1) / kBlock), dim3(kBlock), 0, st, c, n,
                  out, numel, d);
}

zr_status reduce_run(const void *const *contribs, int32_t n, int64_t numel, uint16_t *out, hipStream_t st)
{
    const MeanDivisor d = mean_divisor(n);
    if (n <= 8)
        return reduce_launch<8>(contribs, n, numel, out, st, d);
    if (n <= 64)
        return reduce_launch<64>(contribs, n, numel, out, st, d);
    return reduce_launch<kMaxContribs>(contribs, n, numel, out, st, d);
}

}  // namespace zr

using namespace zr;

extern "C" zr_status zr_reduce_slice(const void *const *contribs, int32_t n, int64_t numel, void *out, void *stream)
{
    clear_error();
    if (!contribs)
        return fail(ZR_EINVAL, "zr_reduce_slice: contribs is NULL");
    if (n < 1 || n > kMaxContribs)
        return fail(ZR_EINVAL, "zr_reduce_slice: n = %d outside [1, %d]", n, kMaxContribs);
    if (numel < 0)
        return fail(ZR_EINVAL, "zr_reduce_slice: numel < 0");
    if (numel > 0 && !out)
        return fail(ZR_EINVAL, "zr_reduce_slice: out is NULL");
    if (!aligned_to(out, 2))
        return fail(ZR_EALIGN, "zr_reduce_slice: out must be 2-byte aligned");
    for (int32_t k = 0; k < n; ++k) {
        if (numel > 0 && !contribs[k])
            return fail(ZR_EINVAL, "zr_reduce_slice: contribs[%d] is NULL", k);
        if (!aligned_to(contribs[k], 2))
            return fail(ZR_EALIGN, "zr_reduce_slice: contribs[%d] must be 2-byte aligned", k);
        bool same = contribs[k] == out;
        if (!(k == 0 && same) && overlaps(contribs[k], 2 * numel, out, 2 * numel))
            return fail(ZR_EINVAL, "zr_reduce_slice: out overlaps contribs[%d] (only out == contribs[0] is allowed)", k);
    }
    if (numel == 0)
        return ZR_OK;

    return reduce_run(contribs, n, numel, static_cast<uint16_t *>(out), static_cast<hipStream_t>(stream));
}
