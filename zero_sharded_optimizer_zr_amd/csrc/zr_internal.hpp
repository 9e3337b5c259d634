// Host-side internals shared by the translation units of libzr.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <functional>
#include <tuple>
#include <utility>
#include <vector>

#include "zr.h"

struct zr_layout {
    std::vector<int64_t> numel;       // per tensor
    std::vector<int64_t> offset;      // flat offset, or offset in the persistent region
    std::vector<uint8_t> persistent;  // per tensor
    // non-empty partitioned tensors in flat order, for range queries
    std::vector<int32_t> part_tensor;
    std::vector<int64_t> part_begin;
    int64_t psi = 0, psi_part = 0, psi_persist = 0, psi_pad = 0, shard = 0, threshold = 0;
    int32_t n_d = 1, n_tensors = 0, n_partitioned = 0, n_persistent = 0;
};

namespace zr {

// Records a message for zr_last_error() on this thread and returns `status`.
zr_status fail(zr_status status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Enumerates the fragments of [begin, end) (range already validated).
void for_each_fragment(const zr_layout &L, int64_t begin, int64_t end,
                       const std::function<void(const zr_fragment &)> &fn);

// Most workgroups one launch gets: what one grid dimension allows, or fewer
// when the environment sets ZR_MAX_GRID (>= 8; a testing knob).  Every kernel
// loops over the work its grid does not cover, so results never depend on it.
inline int64_t max_grid()
{
    const char *s = std::getenv("ZR_MAX_GRID");
    const long long v = s ? std::atoll(s) : 0;
    return v >= 8 && v < 0x7fffffff ? (int64_t)v : (int64_t)0x7fffffff;
}

// Grid of `blocks` workgroups, clamped to max_grid() (kernels loop over any
// remainder).
inline dim3 grid_of(int64_t blocks)
{
    if (blocks < 1)
        blocks = 1;
    const int64_t cap = max_grid();
    if (blocks > cap)
        blocks = cap;
    return dim3((unsigned)blocks);
}

// Grid for `tiles` tiles dealt to the XCDs in contiguous runs: a multiple of
// 8, clamped to max_grid() rounded down to 8 (kernels loop over the rest).
inline dim3 xcd_grid_of(int64_t tiles)
{
    if (tiles < 1)
        tiles = 1;
    tiles = (tiles + 7) / 8 * 8;
    const int64_t cap = max_grid() / 8 * 8;
    if (tiles > cap)
        tiles = cap;
    return dim3((unsigned)tiles);
}

// Grid for `tiles` tiles taken in the order first_tile<R>() gives (R = 0, one
// run per XCD, needs a multiple of 8).
template <int R>
inline dim3 order_grid(int64_t tiles)
{
    return R == 0 ? xcd_grid_of(tiles) : grid_of(tiles);
}

inline bool aligned_to(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// First element of a streaming kernel's vector body, at most 63 and never past
// n: where the 2-byte array b16 starts a 128-byte line, so that its wave-wide
// accesses cover whole lines.  Elements before it (and the tail after the last
// vector group) are done element-wise.  A body starting 32 or 48 bytes into a
// line ran the AdamW kernel at 0.67 of peak against 0.76 on whole lines.
inline int64_t line_head16(const void *b16, int64_t n)
{
    const int64_t h = (int64_t)(((128 - (reinterpret_cast<uintptr_t>(b16) & 127)) & 127) / 2);
    return h < n ? h : n;
}

// The same for a kernel led by the fp32 array f32: where f32 starts a 128-byte
// line and, when one element index does both (the usual case of arrays sliced
// at the same element offset from line-aligned buffers), where the 2-byte array
// b16 does too.  Either way f32's 16-byte phase at the head is the one the
// vector body needs.
inline int64_t line_head32(const float *f32, const void *b16, int64_t n)
{
    const uintptr_t a = reinterpret_cast<uintptr_t>(f32);
    int64_t h = (int64_t)(((128 - (a & 127)) & 127) / 4);
    const int64_t h2 = line_head16(b16, 64);
    if (((a + 4 * (uintptr_t)h2) & 127) == 0)
        h = h2;
    return h < n ? h : n;
}

inline bool overlaps(const void *a, int64_t abytes, const void *b, int64_t bbytes)
{
    auto x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return abytes > 0 && bbytes > 0 && x < y + static_cast<uintptr_t>(bbytes) &&
           y < x + static_cast<uintptr_t>(abytes);
}

// Launches `kernel` through hipLaunchKernel so the status of this launch is
// returned directly (no sticky-error ambiguity).  `lds_bytes` of dynamic LDS is
// reserved per workgroup; the streaming kernels never touch it and use it only
// to cap how many workgroups a compute unit holds at once (160 KB of LDS per CU
// on gfx950), which bounds the bytes in flight per HBM channel.
template <typename... Params, typename... Args>
zr_status launch(void (*kernel)(Params...), dim3 grid, dim3 block, size_t lds_bytes, hipStream_t stream,
                 Args &&...args)
{
    std::tuple<Params...> values(std::forward<Args>(args)...);
    void *ptrs[sizeof...(Params) > 0 ? sizeof...(Params) : 1];
    std::apply([&](auto &...v) {
        int i = 0;
        ((ptrs[i++] = static_cast<void *>(&v)), ...);
    }, values);
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, ptrs, lds_bytes, stream);
    if (e != hipSuccess)
        return fail(ZR_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ZR_OK;
}

}  // namespace zr
