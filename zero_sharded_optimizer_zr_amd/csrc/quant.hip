// Symmetric block-wise int8 and int4 quantization of a bf16 shard, and its
// inverse, for a quantized parameter AllGather (gfx950).
//
// The rank quantizes its updated bf16 parameter shard before the AllGather
// (1 byte -- int8 -- or half a byte -- int4 -- per element plus one fp32 scale
// per block, instead of 2 bytes) and every rank dequantizes the gathered
// buffer before unpacking it.  Per block of B elements, with Q = 127 (int8) or
// 7 (int4): amax = max |x|, s = amax / Q, q = rint(x / s) clamped to [-Q, Q]
// (q = 0 when s = 0); x' = bf16(q * s), every result correctly rounded (ties
// to even), so codes, scales and rebuilt values are exact functions of the
// input bits.  int4 codes are 4-bit two's complement, two per byte: element 2j
// in the low four bits of byte j, element 2j + 1 in the high four bits (0 for
// an odd count's last byte).
//
// Tiles: one wave owns kTile = 2048 consecutive elements, as 4 chunks of 512;
// in chunk c lane l holds elements c * 512 + 8 l .. + 7, so every load and
// store instruction of the wave covers one contiguous 512-element span (16 B of
// bf16, 8 B of int8 or 4 B of int4 codes per lane).  A tile holds 2048 / B
// whole blocks.  The
// block maxima of a tile are reduced within rows of 16 lanes by DPP and across
// rows on the scalar unit; one exact division pair for all the tile's blocks
// runs in lanes 0 .. 2048 / B - 1, which also store the tile's scales in one
// instruction.  Bound by HBM: 3 (int8) or 2.5 (int4) bytes per element plus 4
// per block.  The
// quantizer's workgroups take their tiles in runs per XCD, at most 5 per CU
// (LDS reserved and never touched): on MI355X, same buffers, 1.75e9 elements,
// B = 2048, one contiguous run per XCD with the cap 6.17 -> 6.53 TB/s against
// launch order uncapped (the run alone 6.31, the cap alone 6.31; 3 per CU
// 5.64), and runs of 64 workgroups another 1.6-5.8%.  The dequantizers take
// runs of 64 too, uncapped (see kDequantizeOrder).
//
// Source (web pages on DeepSpeed ZeRO-3): ZeRO-1/2/3 concept page
// (compassingai.com), ZeRO++ section -- qwZ quantizes the weights carried by
// the AllGather to int8 or int4 to reduce its volume (details left to
// DeepSpeed); the encyclopedia entry (baike.kuaisou.com), history section,
// names ZeRO++ as the follow-up aimed at communication volume.
#include "zr_math.hpp"

namespace zr {

constexpr int kLaneVec = 8;
constexpr int kChunk = 64 * kLaneVec;
constexpr int kTileChunks = 4;
constexpr int kTile = kChunk * kTileChunks;
constexpr int kRow = 16 * kLaneVec;  // elements of one DPP row of 16 lanes

// Tiles whose block scales are all 0 or at least 2^-100 take quantize_fast;
// a tile with a tinier scale (where its FMA remainder can underflow) divides
// exactly.  As the bit pattern of a non-negative float.
constexpr uint32_t kFastMinScaleBits = 0x0d800000u;  // 2^-100

// Wave identity as a scalar: threadIdx.x >> 6 is the same in every lane.
__device__ __forceinline__ int64_t wave_id()
{
    return (int64_t)blockIdx.x * (kBlock / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

__device__ __forceinline__ float wave_max(float a)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        a = fmaxf(a, __shfl_xor(a, off, 64));
    return a;
}

// Non-negative floats order as their bit patterns, so maxima of |x| are taken
// on the unsigned patterns (no NaN can occur: inputs are finite).
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_umax(uint32_t a)
{
    const uint32_t b = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, kCtrl, 0xf, 0xf, false);
    return a > b ? a : b;
}

// Every lane of each row of 16 lanes gets the row's maximum: swap neighbours,
// swap pairs, mirror halves of 8, mirror the row.
__device__ __forceinline__ uint32_t row_umax(uint32_t a)
{
    a = dpp_umax<0xb1>(a);   // quad_perm [1, 0, 3, 2]
    a = dpp_umax<0x4e>(a);   // quad_perm [2, 3, 0, 1]
    a = dpp_umax<0x141>(a);  // row_half_mirror
    a = dpp_umax<0x140>(a);  // row_mirror
    return a;
}

__device__ __forceinline__ uint32_t read_lane(uint32_t v, int lane) { return (uint32_t)__builtin_amdgcn_readlane((int)v, lane); }

// Exact code of one element: rint(x / s) clamped to [-kQ, kQ], 0 for s == 0
// (then the quotient is NaN and a select replaces it).
template <int kQ>
__device__ __forceinline__ int32_t quantize_one(float x, float s)
{
    float r = rintf(__fdiv_rn(x, s));
    r = fminf(fmaxf(r, -(float)kQ), (float)kQ);
    return s == 0.0f ? 0 : (int32_t)r;
}

// Code of one element from s and r = RN(1 / s) (0 when s is 0), for s == 0 or
// s >= 2^-100.  The quotient RN(x / s) comes from one Markstein correction step
// instead of a division: q0 = RN(x * r), rem = x - q0 * s (one FMA, exact),
// q1 = RN(q0 + rem * r) (one FMA) -- P. Markstein, "Computation of elementary
// functions on the IBM RISC System/6000 processor" (IBM J. Res. Dev., 1990);
// Muller et al., "Handbook of Floating-Point Arithmetic", division with FMA.
// For bf16 x, s = RN(amax / kQ) >= 2^-100 and |x| <= amax, rint(q1) equals
// rint(RN(x / s)) for every pair, for kQ = 127 and for kQ = 7 (q1 is RN(x / s)
// itself whenever |x / s| >= 1/4), as exhaustive enumeration of all bf16
// (x, amax) pairs on the CPU shows.  A plain RN(x * r) would not do: bf16
// inputs put about 0.3% of quotients within 2^-14 of a half step, and 3e-4 of
// them round the other way.  s == 0 (an all-zero block) gives q1 = 0 through
// r = 0.
template <int kQ>
__device__ __forceinline__ int32_t quantize_fast(float x, float s, float r)
{
    const float q0 = x * r;
    const float rem = __fmaf_rn(-q0, s, x);
    const float q1 = __fmaf_rn(rem, r, q0);
    return (int32_t)fminf(fmaxf(rintf(q1), -(float)kQ), (float)kQ);
}

__device__ __forceinline__ uint32_t pack4(const int32_t *v)
{
    return (v[0] & 0xffu) | (v[1] & 0xffu) << 8 | (v[2] & 0xffu) << 16 | (uint32_t)(v[3] & 0xff) << 24;
}

// Eight int4 codes, element e in bits 4e .. 4e + 3.
__device__ __forceinline__ uint32_t pack8_nibbles(const int32_t *v)
{
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        w |= (uint32_t)(v[e] & 0xf) << (4 * e);
    return w;
}

// The signed int4 code in bits 4e .. 4e + 3 of w.
__device__ __forceinline__ int32_t nibble_code(uint32_t w, int e) { return (int32_t)(w << (28 - 4 * e)) >> 28; }

// Bytes of codes for n elements.
template <int kQ>
constexpr int64_t code_bytes(int64_t n)
{
    return kQ == 7 ? (n + 1) / 2 : n;
}

// One wave quantizes one tile.  kFull: the tile lies wholly inside the buffer
// (every tile but a short last one), so no element needs a guard.  q is the
// code buffer as bytes (int8 codes, or int4 codes two per byte).
template <int B, bool kFull, int kQ>
__device__ __forceinline__ void quantize_tile(const uint16_t *src, int64_t numel, uint8_t *q, float *scales,
                                              int64_t base, int lane)
{
    static_assert(kTile % B == 0 && B % kRow == 0, "block must be whole rows and divide the tile");
    constexpr int kBlocks = kTile / B;                      // blocks per tile
    constexpr int kRowsPerBlock = B / kRow;
    constexpr int kChunksPerBlock = B >= kChunk ? B / kChunk : 1;
    constexpr int kChains = kTileChunks / kChunksPerBlock;  // row reductions per tile

    float x[kTileChunks][kLaneVec];
    uint32_t a[kTileChunks];
#pragma unroll
    for (int c = 0; c < kTileChunks; ++c) {
        const int64_t i = base + c * kChunk + lane * kLaneVec;
        if (kFull) {
            u32x4 w = load_stream(reinterpret_cast<const u32x4 *>(src + i));
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                x[c][2 * h] = bf16_lo(w[h]);
                x[c][2 * h + 1] = bf16_hi(w[h]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < kLaneVec; ++e)
                x[c][e] = i + e < numel ? bf16_to_f32(src[i + e]) : 0.0f;
        }
        float m = 0.0f;
#pragma unroll
        for (int e = 0; e < kLaneVec; ++e)
            m = fmaxf(m, fabsf(x[c][e]));
        a[c] = __float_as_uint(m);
    }
    // Row maxima (rows of chunks of one block are merged lane by lane first),
    // then block maxima on the scalar unit, in tile order.
    uint32_t bmax[kBlocks];
#pragma unroll
    for (int k = 0; k < kChains; ++k) {
        uint32_t v = a[k * kChunksPerBlock];
#pragma unroll
        for (int j = 1; j < kChunksPerBlock; ++j)
            v = v > a[k * kChunksPerBlock + j] ? v : a[k * kChunksPerBlock + j];
        v = row_umax(v);
        uint32_t rows[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            rows[j] = read_lane(v, 16 * j);
        if (kRowsPerBlock == 2) {           // two blocks per chunk
            bmax[2 * k] = rows[0] > rows[1] ? rows[0] : rows[1];
            bmax[2 * k + 1] = rows[2] > rows[3] ? rows[2] : rows[3];
        } else {                            // one block per chain
            const uint32_t lo = rows[0] > rows[1] ? rows[0] : rows[1];
            const uint32_t hi = rows[2] > rows[3] ? rows[2] : rows[3];
            bmax[k] = lo > hi ? lo : hi;
        }
    }
    // Lane b < kBlocks holds block b's amax; s and r for every block at once.
    uint32_t am = 0;
#pragma unroll
    for (int b = 0; b < kBlocks; ++b)
        am = lane == b ? bmax[b] : am;
    const float sv = __fdiv_rn(__uint_as_float(am), (float)kQ);
    const float rv = sv == 0.0f ? 0.0f : __fdiv_rn(1.0f, sv);
    if (lane < kBlocks && (kFull || base + (int64_t)lane * B < numel))
        scales[base / B + lane] = sv;
    uint32_t sb[kBlocks], rb[kBlocks];
    bool fast = true;
#pragma unroll
    for (int b = 0; b < kBlocks; ++b) {
        sb[b] = read_lane(__float_as_uint(sv), b);
        rb[b] = read_lane(__float_as_uint(rv), b);
        fast = fast && (sb[b] == 0 || sb[b] >= kFastMinScaleBits);
    }
#pragma unroll
    for (int c = 0; c < kTileChunks; ++c) {
        // this lane's block in chunk c
        const int b0 = kRowsPerBlock == 2 ? 2 * c : c / kChunksPerBlock;
        float s = __uint_as_float(sb[b0]), r = __uint_as_float(rb[b0]);
        if (kRowsPerBlock == 2 && lane >= 32) {
            s = __uint_as_float(sb[b0 + 1]);
            r = __uint_as_float(rb[b0 + 1]);
        }
        int32_t v[kLaneVec];
        if (fast) {
#pragma unroll
            for (int e = 0; e < kLaneVec; ++e)
                v[e] = quantize_fast<kQ>(x[c][e], s, r);
        } else {
#pragma unroll
            for (int e = 0; e < kLaneVec; ++e)
                v[e] = quantize_one<kQ>(x[c][e], s);
        }
        const int64_t i = base + c * kChunk + lane * kLaneVec;
        if constexpr (kQ == 127) {
            if (kFull) {
                store_stream(reinterpret_cast<u32x2 *>(q + i), u32x2{pack4(v), pack4(v + 4)});
            } else {
#pragma unroll
                for (int e = 0; e < kLaneVec; ++e)
                    if (i + e < numel)
                        q[i + e] = (uint8_t)v[e];
            }
        } else {  // i is a multiple of 8: the lane owns bytes i / 2 .. i / 2 + 3
            if (kFull) {
                store_stream(reinterpret_cast<uint32_t *>(q + i / 2), pack8_nibbles(v));
            } else {
#pragma unroll
                for (int e = 0; e < kLaneVec; e += 2)
                    if (i + e < numel)
                        q[(i + e) / 2] = (uint8_t)((v[e] & 0xf) | (i + e + 1 < numel ? (v[e + 1] & 0xf) << 4 : 0));
            }
        }
    }
}

// Tile orders (first_tile), in workgroups of kBlock / 64 tiles (8192
// elements): runs of 64 per XCD for the quantizers (1.6-5.8% over one run per
// XCD) and the dequantizers (int8 about 5% over launch order, int4 4%).
constexpr int kQuantizeOrder = 64;
constexpr int kDequantizeOrder = 64;

// Vector path: src 16-byte aligned, codes 8-byte (int8) or 4-byte (int4) aligned.
template <int B, int kQ>
__global__ __launch_bounds__(kBlock) void quantize_vec_kernel(const uint16_t *src, int64_t numel, uint8_t *q,
                                                              float *scales, int64_t ntiles)
{
    // workgroups in the order kQuantizeOrder, kBlock / 64 tiles each, then the
    // same again gridDim.x workgroups further on
    const int lane = threadIdx.x & 63;
    const int64_t stride = (int64_t)gridDim.x * (kBlock / 64);
    const int64_t first =
        first_tile<kQuantizeOrder>() * (kBlock / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    for (int64_t tile = first; tile < ntiles; tile += stride) {
        const int64_t base = tile * kTile;
        if (base + kTile <= numel)
            quantize_tile<B, true, kQ>(src, numel, q, scales, base, lane);
        else
            quantize_tile<B, false, kQ>(src, numel, q, scales, base, lane);
    }
}

// Element-wise path for any natural alignment: one wave per block (int4: one
// lane per pair of elements, so that no two lanes share a byte; blocks start
// at even elements).
template <int kQ>
__global__ __launch_bounds__(kBlock) void quantize_scalar_kernel(const uint16_t *src, int64_t numel, int32_t B,
                                                                 uint8_t *q, float *scales, int64_t nblocks)
{
    const int lane = threadIdx.x & 63;
    for (int64_t blk = wave_id(); blk < nblocks; blk += (int64_t)gridDim.x * (kBlock / 64)) {
        const int64_t lo = blk * B;
        const int64_t hi = lo + B < numel ? lo + B : numel;
        float amax = 0.0f;
        for (int64_t i = lo + lane; i < hi; i += 64)
            amax = fmaxf(amax, fabsf(bf16_to_f32(src[i])));
        amax = wave_max(amax);
        const float s = __fdiv_rn(amax, (float)kQ);
        if (lane == 0)
            scales[blk] = s;
        if constexpr (kQ == 127) {
            for (int64_t i = lo + lane; i < hi; i += 64)
                q[i] = (uint8_t)quantize_one<kQ>(bf16_to_f32(src[i]), s);
        } else {
            for (int64_t i = lo + 2 * lane; i < hi; i += 128) {
                const int32_t c0 = quantize_one<kQ>(bf16_to_f32(src[i]), s);
                const int32_t c1 = i + 1 < hi ? quantize_one<kQ>(bf16_to_f32(src[i + 1]), s) : 0;
                q[i / 2] = (uint8_t)((c0 & 0xf) | (c1 & 0xf) << 4);
            }
        }
    }
}

// A whole tile.  int4: every code and scale load of the lane's chunks is
// issued before the first store.  The codes and the output may alias as far as
// the compiler knows, so a load placed after a store waits for it; chunk by
// chunk, each wave waited out one memory latency per chunk, and issuing the
// loads first made the kernel 7.5% faster (12% with runs of 64 workgroups per
// XCD; same buffers, same bits).  int8 stays chunk by chunk: its loads first
// measured 2.3% slower.
template <int B, int kQ>
__device__ __forceinline__ void dequantize_full_tile(const uint8_t *q, const float *scales, uint16_t *dst,
                                                     int64_t base, int lane)
{
    if constexpr (kQ == 127) {
#pragma unroll
        for (int c = 0; c < kTileChunks; ++c) {
            const int64_t i = base + c * kChunk + lane * kLaneVec;
            // B >= 512: one block per chunk, the same for every lane
            const float s = B >= kChunk ? scales[(base + c * kChunk) / B] : scales[i / B];
            const u32x2 w = load_stream(reinterpret_cast<const u32x2 *>(q + i));
            u32x4 o;
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const uint32_t word = w[h / 2] >> (16 * (h % 2));
                o[h] = pack_bf16x2((float)(int8_t)word * s, (float)(int8_t)(word >> 8) * s);
            }
            store_stream(reinterpret_cast<u32x4 *>(dst + i), o);
        }
    } else {
        uint32_t w[kTileChunks];
        float s[kTileChunks];
#pragma unroll
        for (int c = 0; c < kTileChunks; ++c) {
            const int64_t i = base + c * kChunk + lane * kLaneVec;
            w[c] = load_stream(reinterpret_cast<const uint32_t *>(q + i / 2));
            s[c] = B >= kChunk ? scales[(base + c * kChunk) / B] : scales[i / B];
        }
#pragma unroll
        for (int c = 0; c < kTileChunks; ++c) {
            const int64_t i = base + c * kChunk + lane * kLaneVec;
            u32x4 o;
#pragma unroll
            for (int h = 0; h < 4; ++h)
                o[h] = pack_bf16x2((float)nibble_code(w[c], 2 * h) * s[c], (float)nibble_code(w[c], 2 * h + 1) * s[c]);
            store_stream(reinterpret_cast<u32x4 *>(dst + i), o);
        }
    }
}

// The last tile, which may end inside a chunk: element by element.
template <int B, int kQ>
__device__ __forceinline__ void dequantize_last_tile(const uint8_t *q, const float *scales, int64_t numel,
                                                     uint16_t *dst, int64_t base, int lane)
{
    for (int c = 0; c < kTileChunks; ++c) {
        if (base + c * kChunk >= numel)
            break;
        const int64_t i = base + c * kChunk + lane * kLaneVec;
#pragma unroll
        for (int e = 0; e < kLaneVec; ++e) {
            if (i + e >= numel)
                break;
            const int32_t code =
                kQ == 127 ? (int32_t)(int8_t)q[i + e] : nibble_code(q[(i + e) / 2], (int)((i + e) & 1));
            dst[i + e] = (uint16_t)f32_to_bf16((float)code * scales[(i + e) / B]);
        }
    }
}

// Vector path: dst 16-byte aligned, codes 8-byte (int8) or 4-byte (int4) aligned.
template <int B, int kQ>
__global__ __launch_bounds__(kBlock) void dequantize_vec_kernel(const uint8_t *q, const float *scales, int64_t numel,
                                                                uint16_t *dst, int64_t ntiles)
{
    const int lane = threadIdx.x & 63;
    const int64_t first =
        first_tile<kDequantizeOrder>() * (kBlock / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    for (int64_t tile = first; tile < ntiles; tile += (int64_t)gridDim.x * (kBlock / 64)) {
        const int64_t base = tile * kTile;
        if (base + kTile <= numel)
            dequantize_full_tile<B, kQ>(q, scales, dst, base, lane);
        else
            dequantize_last_tile<B, kQ>(q, scales, numel, dst, base, lane);
    }
}

template <int kQ>
__global__ __launch_bounds__(kBlock) void dequantize_scalar_kernel(const uint8_t *q, const float *scales,
                                                                   int64_t numel, int32_t B, uint16_t *dst)
{
    for (int64_t i = global_tid(); i < numel; i += grid_stride()) {
        const int32_t code = kQ == 127 ? (int32_t)(int8_t)q[i] : nibble_code(q[i / 2], (int)(i & 1));
        dst[i] = (uint16_t)f32_to_bf16((float)code * scales[i / B]);
    }
}

inline bool valid_block(int32_t b) { return b == 256 || b == 512 || b == 1024 || b == 2048; }

// The quantizer and its inverse for either code format (kQ = 127: int8,
// kQ = 7: int4); `who` names the entry point in messages.
template <int kQ>
zr_status quantize_launch(const char *who, const void *src, int64_t numel, int32_t block, uint8_t *q,
                          float *scales, void *stream)
{
    if (!valid_block(block))
        return fail(ZR_EINVAL, "%s: block = %d, must be 256, 512, 1024 or 2048", who, block);
    if (numel < 0)
        return fail(ZR_EINVAL, "%s: numel < 0", who);
    if (numel > 0 && (!src || !q || !scales))
        return fail(ZR_EINVAL, "%s: NULL buffer", who);
    if (!aligned_to(src, 2) || !aligned_to(scales, 4))
        return fail(ZR_EALIGN, "%s: src must be 2-byte and scales 4-byte aligned", who);
    const int64_t nblocks = (numel + block - 1) / block;
    {
        const void *p[3] = {src, q, scales};
        int64_t b[3] = {2 * numel, code_bytes<kQ>(numel), 4 * nblocks};
        int x, y;
        if (any_overlap(p, b, 3, &x, &y))
            return fail(ZR_EINVAL, "%s: buffers %d and %d overlap", who, x, y);
    }
    if (numel == 0)
        return ZR_OK;
    auto s = static_cast<const uint16_t *>(src);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (!(aligned_to(s, 16) && aligned_to(q, kQ == 127 ? 8 : 4)))
        return launch(quantize_scalar_kernel<kQ>, grid_of((nblocks + 3) / 4), dim3(kBlock), 0, st, s, numel, block,
                      q, scales, nblocks);
    const int64_t ntiles = (numel + kTile - 1) / kTile;
    const dim3 grid = order_grid<kQuantizeOrder>((ntiles + 3) / 4);
    constexpr size_t lds = 32 * 1024;  // 5 workgroups per CU
    switch (block) {
    case 256: return launch(quantize_vec_kernel<256, kQ>, grid, dim3(kBlock), lds, st, s, numel, q, scales, ntiles);
    case 512: return launch(quantize_vec_kernel<512, kQ>, grid, dim3(kBlock), lds, st, s, numel, q, scales, ntiles);
    case 1024:
        return launch(quantize_vec_kernel<1024, kQ>, grid, dim3(kBlock), lds, st, s, numel, q, scales, ntiles);
    default:
        return launch(quantize_vec_kernel<2048, kQ>, grid, dim3(kBlock), lds, st, s, numel, q, scales, ntiles);
    }
}

template <int kQ>
zr_status dequantize_launch(const char *who, const uint8_t *q, const float *scales, int64_t numel, int32_t block,
                            void *dst, void *stream)
{
    if (!valid_block(block))
        return fail(ZR_EINVAL, "%s: block = %d, must be 256, 512, 1024 or 2048", who, block);
    if (numel < 0)
        return fail(ZR_EINVAL, "%s: numel < 0", who);
    if (numel > 0 && (!dst || !q || !scales))
        return fail(ZR_EINVAL, "%s: NULL buffer", who);
    if (!aligned_to(dst, 2) || !aligned_to(scales, 4))
        return fail(ZR_EALIGN, "%s: dst must be 2-byte and scales 4-byte aligned", who);
    const int64_t nblocks = (numel + block - 1) / block;
    {
        const void *p[3] = {dst, q, scales};
        int64_t b[3] = {2 * numel, code_bytes<kQ>(numel), 4 * nblocks};
        int x, y;
        if (any_overlap(p, b, 3, &x, &y))
            return fail(ZR_EINVAL, "%s: buffers %d and %d overlap", who, x, y);
    }
    if (numel == 0)
        return ZR_OK;
    auto d = static_cast<uint16_t *>(dst);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (!(aligned_to(d, 16) && aligned_to(q, kQ == 127 ? 8 : 4)))
        return launch(dequantize_scalar_kernel<kQ>, grid_of((numel + kBlock - 1) / kBlock), dim3(kBlock), 0, st, q,
                      scales, numel, block, d);
    const int64_t ntiles = (numel + kTile - 1) / kTile;
    const dim3 grid = order_grid<kDequantizeOrder>((ntiles + 3) / 4);
    switch (block) {
    case 256: return launch(dequantize_vec_kernel<256, kQ>, grid, dim3(kBlock), 0, st, q, scales, numel, d, ntiles);
    case 512: return launch(dequantize_vec_kernel<512, kQ>, grid, dim3(kBlock), 0, st, q, scales, numel, d, ntiles);
    case 1024:
        return launch(dequantize_vec_kernel<1024, kQ>, grid, dim3(kBlock), 0, st, q, scales, numel, d, ntiles);
    default:
        return launch(dequantize_vec_kernel<2048, kQ>, grid, dim3(kBlock), 0, st, q, scales, numel, d, ntiles);
    }
}

}  // namespace zr

using namespace zr;

extern "C" zr_status zr_quantize_int8(const void *src, int64_t numel, int32_t block, int8_t *q, float *scales,
                                      void *stream)
{
    clear_error();
    return quantize_launch<127>("zr_quantize_int8", src, numel, block, reinterpret_cast<uint8_t *>(q), scales,
                                stream);
}

extern "C" zr_status zr_dequantize_int8(const int8_t *q, const float *scales, int64_t numel, int32_t block, void *dst,
                                        void *stream)
{
    clear_error();
    return dequantize_launch<127>("zr_dequantize_int8", reinterpret_cast<const uint8_t *>(q), scales, numel, block,
                                  dst, stream);
}

extern "C" zr_status zr_quantize_int4(const void *src, int64_t numel, int32_t block, uint8_t *q4, float *scales,
                                      void *stream)
{
    clear_error();
    return quantize_launch<7>("zr_quantize_int4", src, numel, block, q4, scales, stream);
}

extern "C" zr_status zr_dequantize_int4(const uint8_t *q4, const float *scales, int64_t numel, int32_t block,
                                        void *dst, void *stream)
{
    clear_error();
    return dequantize_launch<7>("zr_dequantize_int4", q4, scales, numel, block, dst, stream);
}
