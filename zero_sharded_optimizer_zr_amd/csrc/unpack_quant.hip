// Dequantize-on-unpack: the receiver side of a quantized parameter AllGather
// (gfx950), for int8 and int4 codes.  The gathered buffer holds, for flat
// elements [begin, end) of the partition, one int8 code per element and one
// fp32 scale per block; blocks are those of the ranks that quantized their own
// shards (zr_quantize_int8 on elements [r S, (r+1) S)), so the block grid
// restarts at every shard and a shard's last block is short when the block
// size does not divide S.  Every
// element is rebuilt as bf16(code * scale) and written straight into its
// tensor view: 1 byte read and 2 bytes written per element, where dequantizing
// into a flat bf16 buffer and unpacking that would move 7.
//
// Like the bf16 unpack: the host turns the layout's fragments of [begin, end),
// split at shard boundaries, into descriptors {codes, destination, scale of the
// first block, phase in that block, count}, passed by value in batches; every
// workgroup rebuilds one tile of 4096 elements of one descriptor (two chunks of
// 8 per lane, 2048 elements apart, each one aligned 16-byte store), found by a
// binary search over the batch's compact array of first tiles; tiles go to the
// 8 XCDs in contiguous runs (a grid smaller than the tile count loops, every
// gridDim.x-th tile).  Codes come in as
// two aligned 8-byte words per lane, funnel-shifted (v_alignbyte) when the
// source's byte phase differs from the destination's; a lane's 8 elements
// span at most two blocks (blocks are >= 256 elements and a descriptor lies in
// one shard).  The head before the destination's first 128-byte line and the
// tail are rebuilt element-wise.
//
// int4 codes (zr_unpack_int4) take the same path with the codes packed two
// per byte and per shard: a descriptor starts at the byte that holds its first
// element's code, in the high four bits when that element's position in the
// shard is odd, and a lane's 8 codes are 32 bits at a bit offset (8 per byte
// phase, 4 for the odd nibble) uniform per descriptor, taken from two aligned
// 4-byte words by a 64-bit shift when the offset is not 0.  Chunks per lane
// and tile order are chosen per launch (launch_batches): two in XCD runs for a
// batch of a few whole shards, four in launch order for a batch of a model's
// tensors.  The int4 code loads are ordinary cached loads: with the non-temporal
// hint these 4-byte-per-lane loads fetched 4.3% more than the code bytes from
// HBM (FETCH_SIZE), and ran 1% slower; cached, the fetch equals the code and
// scale bytes.  (The int8 code loads, 8 bytes per lane, fetch exactly their
// bytes either way and keep the hint.)
//
// Eight elements are rebuilt for every 16 bytes written, so the vector
// instructions per element decide as much as HBM does.  Two things keep them
// few.  When every chunk of a descriptor starts on a multiple of 8 in the
// block grid (uniform per descriptor, and the case of whole shards and of
// views aligned like them), a chunk's 8 elements share one block: one scale
// load and no per-element scale select.  And the bf16 rounding is the packed
// hardware conversion, one instruction per pair, whose bits equal the integer
// round-to-nearest-even on every fp32 pattern.  On the 7e9 gather (same
// buffers, MI355X, four sessions) they took int4 from 0.707-0.712 of the HBM
// peak to 0.786-0.790 and int8 from 0.774-0.778 to 0.802-0.806.
//
// Measured equal or slower, same buffers: the wave's scales fetched once with
// scalar loads (int8 +1%, int4 -10%), one chunk per lane (int8 -11%), a
// residency cap for int4 (-6%), and widening codes with v_cvt_f32_ubyte and a
// fused multiply-add by the scale minus a bias (slower, and wrong in the sign
// of zero products).
//
// Reads past a descriptor's last code stay inside the aligned 8-byte (int8) or
// 4-byte (int4) word that holds that code.
//
// Sources (web pages on DeepSpeed ZeRO-3): ZeRO-1/2/3 concept page
// (compassingai.com), ZeRO++ section (qwZ: quantized weights in the AllGather)
// and Stage 3 mechanism (full parameters gathered before compute); "From DDP to
// ZeRO: memory sharding" blog (111qqz.com), "ZeRO-3: why parameters can be
// sharded too" (a tensor split across ranks).
#include <algorithm>
#include <vector>

#include "zr_device.hpp"
#include "zr_internal.hpp"

namespace zr {

namespace {

constexpr int kPerLane = 2;                          // 8-element chunks per lane (int8 codes)
constexpr int64_t kTileLanes = kBlock * kPerLane;  // 8-element chunks per tile
// int4 codes: chunks per lane, per launch (see launch_batches)
constexpr int kPerLane4Few = 2;   // a batch of a few large descriptors
constexpr int kPerLane4Many = 4;  // a batch of many
constexpr int kFewDesc = 8;
constexpr int kMaxDesc = 64;            // 64 * (8 + 40) B of descriptors per launch

struct QDesc {
    const int8_t *src;   // code of the first element
    uint16_t *dst;       // its place in the tensor view
    const float *scale;  // scale of the block holding the first element
    int64_t n;           // elements
    int32_t phase;       // position of the first element inside its block
    int32_t reserved;
};

struct QBatch {
    int32_t count;
    int32_t lg_block;
    int64_t first_tile[kMaxDesc];  // prefix sums of the descriptors' tiles
    QDesc d[kMaxDesc];
};

// Elements before dst reaches a 128-byte line (at most 63): the vector body then
// writes whole lines.  With 16-byte alignment only, a destination 16 or 48 bytes
// into a line (shard sizes that are not multiples of 64 elements) made every
// wave's stores straddle a partial line at both ends: the 1T shard's gather ran
// at 0.73 (int8) and 0.75 (int4) of peak against 0.78 with whole lines.
__host__ __device__ __forceinline__ int64_t head_of(const uint16_t *dst, int64_t n)
{
    int64_t h = (int64_t)(((128 - (reinterpret_cast<uintptr_t>(dst) & 127)) & 127) / 2);
    return h < n ? h : n;
}

// Bytes [r, r + 8) of the 16-byte little-endian concatenation a|b, r in 1..7.
__device__ __forceinline__ u32x2 funnel8(u32x2 a, u32x2 b, uint32_t r)
{
    const uint32_t rr = r & 3;
    if (r < 4)
        return u32x2{__builtin_amdgcn_alignbyte(a.y, a.x, rr), __builtin_amdgcn_alignbyte(b.x, a.y, rr)};
    return u32x2{__builtin_amdgcn_alignbyte(b.x, a.y, rr), __builtin_amdgcn_alignbyte(b.y, b.x, rr)};
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 values as packed bf16 in one instruction (v_cvt_pk_bf16_f32: round to
// nearest even, NaN kept quiet with its upper payload).  Its bits equal
// pack_bf16x2's on every one of the 2^32 fp32 bit patterns (checked on MI355X
// for both halves), where the integer rounding takes about fifteen vector
// instructions per pair: with 8 elements rebuilt per 16 bytes written, that
// made these kernels as bound by vector issue as by HBM.
__device__ __forceinline__ uint32_t pack_bf16x2_hw(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ uint32_t rebuild2(uint32_t codes, int k, float s0, float s1)
{
    const float lo = (float)(int8_t)(codes >> (8 * k)) * s0;
    const float hi = (float)(int8_t)(codes >> (8 * k + 8)) * s1;
    return pack_bf16x2_hw(lo, hi);
}

// A chunk's 8 int8 codes (x.x holds elements 0-3, x.y 4-7) times one scale.
__device__ __forceinline__ u32x4 rebuild8_one(u32x2 x, float s)
{
    float e[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        e[j] = (float)(int8_t)(x.x >> (8 * j)) * s;
        e[4 + j] = (float)(int8_t)(x.y >> (8 * j)) * s;
    }
    return u32x4{pack_bf16x2_hw(e[0], e[1]), pack_bf16x2_hw(e[2], e[3]), pack_bf16x2_hw(e[4], e[5]),
                 pack_bf16x2_hw(e[6], e[7])};
}

// The lane's chunks of tile t: every load first, then the arithmetic and the
// stores.  kShift: the codes' byte phase differs from the destination's (two
// words per chunk, funnel-shifted); kFull: every chunk of the tile is inside
// the descriptor's aligned body, so no lane needs a guard; kOne: every chunk
// starts on a multiple of 8 in the block grid, so its 8 elements share one
// block and one scale (blocks are multiples of 8).  All three are uniform per
// workgroup.
template <bool kShift, bool kFull, bool kOne>
__device__ __forceinline__ void rebuild_chunks(const u32x2 *s2, uint32_t shift, uint16_t *out, const float *scale,
                                               int64_t e_base, int lg, int64_t c0, int64_t body)
{
    u32x2 w[kPerLane], w2[kPerLane];
    float sa[kPerLane], sb[kPerLane];
    int32_t split[kPerLane];  // elements of the chunk in its first block
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) {
        const int64_t c = c0 + k * kBlock;
        if (kFull || c < body) {
            w[k] = load_stream(s2 + c);
            if (kShift)
                w2[k] = load_stream(s2 + c + 1);
            const int64_t e0 = e_base + 8 * c;  // position of the chunk's first element in the block grid
            const int64_t j0 = e0 >> lg;
            sa[k] = load_global(scale + j0);
            if (!kOne) {
                sb[k] = load_global(scale + ((e0 + 7) >> lg));
                split[k] = (int32_t)(((j0 + 1) << lg) - e0);
            }
        }
    }
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) {
        const int64_t c = c0 + k * kBlock;
        if (!kFull && c >= body)
            break;
        const u32x2 x = kShift ? funnel8(w[k], w2[k], shift) : w[k];
        if (kOne) {
            store_stream(reinterpret_cast<u32x4 *>(out) + c, rebuild8_one(x, sa[k]));
            continue;
        }
        float s[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            s[e] = e < split[k] ? sa[k] : sb[k];
        const u32x4 o{rebuild2(x.x, 0, s[0], s[1]), rebuild2(x.x, 2, s[2], s[3]), rebuild2(x.y, 0, s[4], s[5]),
                      rebuild2(x.y, 2, s[6], s[7])};
        store_stream(reinterpret_cast<u32x4 *>(out) + c, o);
    }
}

__device__ __forceinline__ uint32_t rebuild2_nibbles(uint32_t codes, int k, float s0, float s1)
{
    const float lo = (float)((int32_t)(codes << (28 - 4 * k)) >> 28) * s0;
    const float hi = (float)((int32_t)(codes << (24 - 4 * k)) >> 28) * s1;
    return pack_bf16x2_hw(lo, hi);
}

// A chunk's 8 int4 codes (nibble e of x is element e) times one scale.
__device__ __forceinline__ u32x4 rebuild4_one(uint32_t x, float s)
{
    float e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        e[j] = (float)((int32_t)(x << (28 - 4 * j)) >> 28) * s;
    return u32x4{pack_bf16x2_hw(e[0], e[1]), pack_bf16x2_hw(e[2], e[3]), pack_bf16x2_hw(e[4], e[5]),
                 pack_bf16x2_hw(e[6], e[7])};
}

// int4 codes: a chunk's 8 codes are the 32 bits that start `shift` bits into
// the aligned word pair s1[c], s1[c + 1] (shift = 8 * byte phase + 4 * nibble
// phase, uniform per descriptor; kShift: shift != 0, so the second word holds
// some of them).  Otherwise as rebuild_chunks.
template <int PL, bool kShift, bool kFull, bool kOne>
__device__ __forceinline__ void rebuild_chunks4(const uint32_t *s1, uint32_t shift, uint16_t *out, const float *scale,
                                                int64_t e_base, int lg, int64_t c0, int64_t body)
{
    uint32_t w[PL], w2[PL];
    float sa[PL], sb[PL];
    int32_t split[PL];
#pragma unroll
    for (int k = 0; k < PL; ++k) {
        const int64_t c = c0 + k * kBlock;
        if (kFull || c < body) {
            w[k] = load_global(s1 + c);  // cached: see the header
            if (kShift)
                w2[k] = load_global(s1 + c + 1);
            const int64_t e0 = e_base + 8 * c;
            const int64_t j0 = e0 >> lg;
            sa[k] = load_global(scale + j0);
            if (!kOne) {
                sb[k] = load_global(scale + ((e0 + 7) >> lg));
                split[k] = (int32_t)(((j0 + 1) << lg) - e0);
            }
        }
    }
#pragma unroll
    for (int k = 0; k < PL; ++k) {
        const int64_t c = c0 + k * kBlock;
        if (!kFull && c >= body)
            break;
        const uint32_t x = kShift ? (uint32_t)((((uint64_t)w2[k] << 32) | w[k]) >> shift) : w[k];
        if (kOne) {
            store_stream(reinterpret_cast<u32x4 *>(out) + c, rebuild4_one(x, sa[k]));
            continue;
        }
        float s[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            s[e] = e < split[k] ? sa[k] : sb[k];
        const u32x4 o{rebuild2_nibbles(x, 0, s[0], s[1]), rebuild2_nibbles(x, 2, s[2], s[3]),
                      rebuild2_nibbles(x, 4, s[4], s[5]), rebuild2_nibbles(x, 6, s[6], s[7])};
        store_stream(reinterpret_cast<u32x4 *>(out) + c, o);
    }
}

// The instantiation of the chunk rebuild for the workgroup's (shift != 0, full)
// pair; kOne as the caller found it.
template <bool kOne>
__device__ __forceinline__ void chunks8(const u32x2 *s2, uint32_t shift, bool full, uint16_t *out, const float *scale,
                                        int64_t e_base, int lg, int64_t c0, int64_t body)
{
    if (shift == 0) {
        if (full)
            rebuild_chunks<false, true, kOne>(s2, shift, out, scale, e_base, lg, c0, body);
        else
            rebuild_chunks<false, false, kOne>(s2, shift, out, scale, e_base, lg, c0, body);
    } else {
        if (full)
            rebuild_chunks<true, true, kOne>(s2, shift, out, scale, e_base, lg, c0, body);
        else
            rebuild_chunks<true, false, kOne>(s2, shift, out, scale, e_base, lg, c0, body);
    }
}

template <int PL, bool kOne>
__device__ __forceinline__ void chunks4(const uint32_t *s1, uint32_t shift, bool full, uint16_t *out,
                                        const float *scale, int64_t e_base, int lg, int64_t c0, int64_t body)
{
    if (shift == 0) {
        if (full)
            rebuild_chunks4<PL, false, true, kOne>(s1, shift, out, scale, e_base, lg, c0, body);
        else
            rebuild_chunks4<PL, false, false, kOne>(s1, shift, out, scale, e_base, lg, c0, body);
    } else {
        if (full)
            rebuild_chunks4<PL, true, true, kOne>(s1, shift, out, scale, e_base, lg, c0, body);
        else
            rebuild_chunks4<PL, true, false, kOne>(s1, shift, out, scale, e_base, lg, c0, body);
    }
}

// Index of the descriptor holding `tile`: a binary search over the batch's
// compact array of first tiles (uniform per workgroup, scalar loads).
__device__ __forceinline__ int find_desc(const QBatch &batch, int64_t tile)
{
    int lo = 0, hi = batch.count - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (batch.first_tile[mid] <= tile)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// int4: D.src is the byte holding the code of the descriptor's first element,
// in its high four bits when the element's position in the shard is odd (its
// position in the block, D.phase, has the same parity: blocks are even).
template <int PL>
__device__ __forceinline__ void unpack_int4_tile(const QBatch &batch, int64_t tile)
{
    const int k = find_desc(batch, tile);
    const QDesc &D = batch.d[k];
    constexpr int64_t kTileLanes4 = kBlock * PL;
    const uint8_t *src = reinterpret_cast<const uint8_t *>(D.src);
    uint16_t *dst = D.dst;
    const float *scale = D.scale;
    const int64_t n = D.n;
    const int64_t phase = D.phase;
    const int lg = batch.lg_block;
    const int64_t t = tile - batch.first_tile[k];

    const int64_t head = head_of(dst, n);
    const int64_t body = (n - head) / 8;
    const int64_t tail_start = head + 8 * body;

    const int64_t nib0 = (phase & 1) + head;  // nibble of element `head`, from src's low nibble
    const uintptr_t a = reinterpret_cast<uintptr_t>(src) + (uintptr_t)(nib0 >> 1);
    const uint32_t shift = (uint32_t)(8 * (a & 3) + 4 * (nib0 & 1));  // uniform per descriptor
    const uint32_t *s1 = reinterpret_cast<const uint32_t *>(a & ~(uintptr_t)3);
    uint16_t *out = dst + head;
    const int64_t c0 = t * kTileLanes4 + threadIdx.x;
    const int64_t e_base = phase + head;
    const bool full = (t + 1) * kTileLanes4 <= body;
    if ((e_base & 7) == 0)
        chunks4<PL, true>(s1, shift, full, out, scale, e_base, lg, c0, body);
    else
        chunks4<PL, false>(s1, shift, full, out, scale, e_base, lg, c0, body);

    if (t == 0) {
        const int64_t edge = head + (n - tail_start);  // at most 63 + 7
        if ((int64_t)threadIdx.x < edge) {
            const int64_t j = (int64_t)threadIdx.x < head ? (int64_t)threadIdx.x : tail_start + (threadIdx.x - head);
            const int64_t nj = (phase & 1) + j;
            const int32_t code = (int32_t)((uint32_t)src[nj >> 1] << (28 - 4 * (nj & 1))) >> 28;
            dst[j] = (uint16_t)f32_to_bf16((float)code * scale[(phase + j) >> lg]);
        }
    }
}

__device__ __forceinline__ void unpack_int8_tile(const QBatch &batch, int64_t tile)
{
    const int k = find_desc(batch, tile);
    const QDesc &D = batch.d[k];
    const int8_t *src = D.src;
    uint16_t *dst = D.dst;
    const float *scale = D.scale;
    const int64_t n = D.n;
    const int64_t phase = D.phase;
    const int lg = batch.lg_block;
    const int64_t t = tile - batch.first_tile[k];

    const int64_t head = head_of(dst, n);
    const int64_t body = (n - head) / 8;  // aligned 16-byte destination chunks
    const int64_t tail_start = head + 8 * body;

    const uintptr_t s_addr = reinterpret_cast<uintptr_t>(src + head);
    const uint32_t shift = (uint32_t)(s_addr & 7);  // uniform per descriptor
    const u32x2 *s2 = reinterpret_cast<const u32x2 *>(s_addr - shift);
    uint16_t *out = dst + head;                      // 16-byte aligned
    const int64_t c0 = t * kTileLanes + threadIdx.x;
    const int64_t e_base = phase + head;
    const bool full = (t + 1) * kTileLanes <= body;
    if ((e_base & 7) == 0)
        chunks8<true>(s2, shift, full, out, scale, e_base, lg, c0, body);
    else
        chunks8<false>(s2, shift, full, out, scale, e_base, lg, c0, body);

    if (t == 0) {
        const int64_t edge = head + (n - tail_start);  // at most 63 + 7
        if ((int64_t)threadIdx.x < edge) {
            const int64_t j = (int64_t)threadIdx.x < head ? (int64_t)threadIdx.x : tail_start + (threadIdx.x - head);
            dst[j] = (uint16_t)f32_to_bf16((float)src[j] * scale[(phase + j) >> lg]);
        }
    }
}

// Tile orders (first_tile): one contiguous run per XCD for the int8 kernel and
// for int4 batches of a few descriptors, launch order for int4 batches of many
// (runs lost 2-9% there).
constexpr int kUnpack8Order = kOneRun;
constexpr int kUnpack4FewOrder = kOneRun;
constexpr int kUnpack4ManyOrder = 1;

// int8: a workgroup takes tile first_tile(), then every gridDim.x-th after it.
__global__ __launch_bounds__(kBlock) void unpack_int8_kernel(QBatch batch, int64_t total_tiles)
{
    for (int64_t tile = first_tile<kUnpack8Order>(); tile < total_tiles; tile += gridDim.x)
        unpack_int8_tile(batch, tile);
}

// int4: PL chunks per lane, tiles in the order kOrder.
template <int PL, int kOrder>
__global__ __launch_bounds__(kBlock) void unpack_int4_kernel(QBatch batch, int64_t total_tiles)
{
    for (int64_t tile = first_tile<kOrder>(); tile < total_tiles; tile += gridDim.x)
        unpack_int4_tile<PL>(batch, tile);
}

// int4 batches of at most kFewDesc descriptors (whole shards: a flat model's
// gather) run two chunks per lane with the tiles in XCD runs; larger batches
// (a model's tensors) run four chunks per lane in launch order.  Measured on the
// gathers of flat models (4 shards of 1.75e9 or 1.95e9 elements, 64 of 1.1e8)
// and of the Llama- and GPT-style layouts (MI355X, same buffers), the rule
// picks the faster of the two on each: 0.784 and 0.779 against 0.769 and 0.734
// for the four-shard gathers, 0.734 against 0.673 for 64 shards, 0.796-0.802
// against 0.673-0.682 for the model layouts.
zr_status launch_batches(const std::vector<QDesc> &pieces, int lg_block, bool int4, hipStream_t st)
{
    size_t i = 0;
    while (i < pieces.size()) {
        QBatch batch{};
        batch.lg_block = lg_block;
        const int count = (int)std::min<size_t>(pieces.size() - i, (size_t)kMaxDesc);
        const bool few = count <= kFewDesc;
        const int64_t lanes = kBlock * (int4 ? (few ? kPerLane4Few : kPerLane4Many) : kPerLane);
        int64_t tiles = 0;
        for (int k = 0; k < count; ++k) {
            const QDesc &p = pieces[i + k];
            const int64_t body = (p.n - head_of(p.dst, p.n)) / 8;
            batch.d[k] = p;
            batch.first_tile[k] = tiles;
            tiles += std::max<int64_t>(1, (body + lanes - 1) / lanes);
        }
        batch.count = count;
        i += count;
        zr_status s;
        if (!int4)
            s = launch(unpack_int8_kernel, order_grid<kUnpack8Order>(tiles), dim3(kBlock), 0, st, batch, tiles);
        else if (few)
            s = launch(unpack_int4_kernel<kPerLane4Few, kUnpack4FewOrder>, order_grid<kUnpack4FewOrder>(tiles),
                       dim3(kBlock), 0, st, batch, tiles);
        else
            s = launch(unpack_int4_kernel<kPerLane4Many, kUnpack4ManyOrder>, order_grid<kUnpack4ManyOrder>(tiles),
                       dim3(kBlock), 0, st, batch, tiles);
        if (s != ZR_OK)
            return s;
    }
    return ZR_OK;
}

int log2_block(int32_t b)
{
    switch (b) {
    case 256: return 8;
    case 512: return 9;
    case 1024: return 10;
    case 2048: return 11;
    default: return -1;
    }
}

// The receiver of a quantized AllGather for either code format (int4: codes
// two per byte, packed per shard).
zr_status unpack_quant(const char *who, bool int4, const zr_layout *L, const uint8_t *q, const float *scales,
                       int32_t block, int64_t begin, int64_t end, const zr_view *views, int32_t n_views, void *stream)
{
    if (!L)
        return fail(ZR_EINVAL, "%s: layout is NULL", who);
    const int lg = log2_block(block);
    if (lg < 0)
        return fail(ZR_EINVAL, "%s: block = %d, must be 256, 512, 1024 or 2048", who, block);
    if (begin < 0 || begin > end || end > L->psi_pad)
        return fail(ZR_ERANGE, "%s: range [%lld, %lld) outside [0, %lld]", who, (long long)begin, (long long)end,
                    (long long)L->psi_pad);
    if (n_views != L->n_tensors)
        return fail(ZR_EINVAL, "%s: n_views = %d but the layout has %d tensors", who, n_views, L->n_tensors);
    if (n_views > 0 && !views)
        return fail(ZR_EINVAL, "%s: views is NULL", who);
    if (begin == end)
        return ZR_OK;
    if (!q || !scales)
        return fail(ZR_EINVAL, "%s: NULL codes or scales", who);
    if (!aligned_to(scales, 4))
        return fail(ZR_EALIGN, "%s: scales must be 4-byte aligned", who);

    const int64_t S = L->shard;
    const int64_t per_rank = (S + block - 1) / block;
    const int64_t bytes_per_rank = (S + 1) / 2;
    auto gathered_block = [&](int64_t i) { return (i / S) * per_rank + (i % S) / block; };
    // byte of the gathered codes that holds element i's code
    auto code_byte = [&](int64_t i) { return int4 ? (i / S) * bytes_per_rank + (i % S) / 2 : i; };
    const int64_t g0 = gathered_block(begin);
    const int64_t n_scales = gathered_block(end - 1) - g0 + 1;
    const int64_t code_bytes = code_byte(end - 1) - code_byte(begin) + 1;
    if (overlaps(q, code_bytes, scales, 4 * n_scales))
        return fail(ZR_EINVAL, "%s: codes and scales overlap", who);

    std::vector<QDesc> pieces;
    zr_status bad = ZR_OK;
    for_each_fragment(*L, begin, end, [&](const zr_fragment &f) {
        if (bad != ZR_OK)
            return;
        const zr_view &v = views[f.tensor];
        if (!v.ptr) {
            bad = fail(ZR_EINVAL, "%s: view of tensor %d is NULL but the range needs it", who, f.tensor);
            return;
        }
        if (!aligned_to(v.ptr, 2)) {
            bad = fail(ZR_EALIGN, "%s: view of tensor %d must be 2-byte aligned", who, f.tensor);
            return;
        }
        if (v.first < 0 || v.count < 0 || f.tensor_offset < v.first ||
            f.tensor_offset + f.numel > v.first + v.count) {
            bad = fail(ZR_ERANGE, "%s: view of tensor %d holds [%lld, %lld), the range needs [%lld, %lld)", who,
                       f.tensor, (long long)v.first, (long long)(v.first + v.count), (long long)f.tensor_offset,
                       (long long)(f.tensor_offset + f.numel));
            return;
        }
        if (overlaps(v.ptr, 2 * v.count, q, code_bytes) || overlaps(v.ptr, 2 * v.count, scales, 4 * n_scales)) {
            bad = fail(ZR_EINVAL, "%s: view of tensor %d overlaps the codes or the scales", who, f.tensor);
            return;
        }
        uint16_t *out = static_cast<uint16_t *>(v.ptr) + (f.tensor_offset - v.first);
        // split at shard boundaries: a descriptor's blocks (and int4 bytes) belong to one rank
        int64_t flat = f.flat_offset, done = 0;
        while (done < f.numel) {
            const int64_t r = flat / S;
            const int64_t piece = std::min(f.numel - done, (r + 1) * S - flat);
            QDesc d{};
            d.src = reinterpret_cast<const int8_t *>(q + (code_byte(flat) - code_byte(begin)));
            d.dst = out + done;
            d.scale = scales + (gathered_block(flat) - g0);
            d.n = piece;
            d.phase = (int32_t)((flat - r * S) % block);
            pieces.push_back(d);
            flat += piece;
            done += piece;
        }
    });
    if (bad != ZR_OK)
        return bad;
    return launch_batches(pieces, lg, int4, static_cast<hipStream_t>(stream));
}

}  // namespace
}  // namespace zr

using namespace zr;

extern "C" zr_status zr_unpack_int8(const zr_layout *L, const int8_t *q, const float *scales, int32_t block,
                                    int64_t begin, int64_t end, const zr_view *views, int32_t n_views, void *stream)
{
    clear_error();
    return unpack_quant("zr_unpack_int8", false, L, reinterpret_cast<const uint8_t *>(q), scales, block, begin, end,
                        views, n_views, stream);
}

extern "C" zr_status zr_unpack_int4(const zr_layout *L, const uint8_t *q4, const float *scales, int32_t block,
                                    int64_t begin, int64_t end, const zr_view *views, int32_t n_views, void *stream)
{
    clear_error();
    return unpack_quant("zr_unpack_int4", true, L, q4, scales, block, begin, end, views, n_views, stream);
}
