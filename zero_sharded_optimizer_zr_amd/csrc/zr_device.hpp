// Device helpers shared by the gfx950 kernels of libzr.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace zr {

// Native clang vectors: one 16-byte (dwordx4) or 8-byte (dwordx2) global
// access per lane.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 256;  // 4 wave64 per workgroup

// Every buffer the kernels touch is in global memory.  Pointers that arrive
// through a descriptor table (not as kernel arguments) are generic to the
// compiler, which then emits flat instructions (counted against both the
// vector-memory and the scalar/LDS counters); casting to the global address
// space gives global_load / global_store with scalar-base addressing.
template <typename T>
using global_ptr = __attribute__((address_space(1))) T *;

// Streaming accesses: every byte is touched once, so loads and stores carry the
// non-temporal hint (the caches do not keep the line for reuse).
template <typename T>
__device__ __forceinline__ T load_stream(const T *p)
{
    return __builtin_nontemporal_load((global_ptr<const T>)p);
}

template <typename T>
__device__ __forceinline__ void store_stream(T *p, T v)
{
    __builtin_nontemporal_store(v, (global_ptr<T>)p);
}

// Ordinary (cached) global load, for data that neighbouring lanes share.
template <typename T>
__device__ __forceinline__ T load_global(const T *p)
{
    return *(global_ptr<const T>)p;
}

// bf16 -> fp32 is exact: the 16 bits are the upper half of the fp32 pattern.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16 bits, round to nearest even on the upper half; NaN stays NaN
// (sign and upper payload kept, quiet bit set).
__device__ __forceinline__ uint32_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    return ((u & 0x7fffffffu) > 0x7f800000u) ? ((u >> 16) | 0x40u) : r;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// Global thread index and stride over a 1-D grid, 64-bit.  Every kernel is
// launched with kBlock threads, so the block size is a compile-time constant:
// reading blockDim.x would cost a vector load from the dispatch packet (and a
// full memory wait) before each wave's first real load.
__device__ __forceinline__ int64_t global_tid() { return (int64_t)blockIdx.x * kBlock + threadIdx.x; }
__device__ __forceinline__ int64_t grid_stride() { return (int64_t)gridDim.x * kBlock; }

// Tile orders.  MI355X deals workgroups round-robin to its 8 XCDs (workgroup b
// runs on XCD b mod 8), each with its own L2.  A launch of G workgroups takes
// its tiles in rounds of G (a workgroup that loops takes the tile gridDim.x
// further on), and first_tile<R>() orders the tiles of a round:
//  - R = 1: launch order, workgroup b takes tile b;
//  - R > 1: runs of R consecutive tiles per XCD: in group g of 8R tiles, XCD x
//    takes the R tiles of slot x (tiles xR ... xR + R - 1 of the group), or with
//    kRotate those of slot (x + g) mod 8, so that its runs move through the
//    slots from group to group; the round's last, partial group stays in
//    launch order;
//  - R = kOneRun: one run per XCD, grid / 8 tiles long (grid a multiple of 8).
// Each is a permutation of the round's tiles, so any grid covers the data.
constexpr int kXcds = 8;
constexpr int kOneRun = 0;
template <int R, bool kRotate = false>
__device__ __forceinline__ int64_t first_tile()
{
    const int64_t b = blockIdx.x;
    if constexpr (R == kOneRun) {
        return (b % kXcds) * (gridDim.x / kXcds) + b / kXcds;
    } else if constexpr (R == 1) {
        return b;
    } else {
        constexpr int64_t group = (int64_t)kXcds * R;
        if (b >= (int64_t)gridDim.x / group * group)
            return b;
        const int64_t j = b / kXcds, g = j / R;
        const int64_t slot = kRotate ? (b % kXcds + g) % kXcds : b % kXcds;
        return g * group + slot * R + j % R;
    }
}

// Tile order of the AdamW kernels (bf16 and fp16 gradients) and of their
// access-pattern kernel: runs of 256 tiles (1 MB of each fp32 array) per XCD,
// 2.6-2.9% faster than launch order on the same buffers (rotating the runs
// moved it by -0.4 to +0.6%, so they are not rotated).  The other kernel
// families set theirs beside their kernels.
constexpr int kAdamwOrder = 256;

}  // namespace zr
