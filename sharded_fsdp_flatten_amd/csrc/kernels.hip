// kernels.hip -- HIP kernels of the per-rank FSDP data path for CDNA4 (gfx950).
//
// All four operations are HBM-streaming: none is a dense contraction, so no
// MFMA is used.  What matters on MI355X (measured, see the tile constants) is:
//   - fully coalesced 128-bit loads (64 lanes x 16 B = 1 KiB per instruction),
//     marked non-temporal: each byte is read once, and the nt hint lifts
//     read streaming from ~6.5 to ~7.2 TB/s;
//   - ONE SMALL TILE PER WORKGROUP (1-2 KiB per wave), never a persistent
//     grid-stride loop: the dispatcher then keeps the workgroups in flight on a
//     compact address window, which HBM serves with far fewer row switches
//     (a grid-stride version of the same copy runs ~20% slower).  The one
//     exception is the many-rank reduction's sweep (below): there the window
//     that matters is over ranks, and a longer run per wave keeps it compact;
//   - outputs stored non-temporally (streamed, never re-read by the kernel); the
//     copies' whole tiles with device-scope nt buffer stores, which stream out
//     faster than the default-scope ones (as do the local accumulation's and the
//     reductions' whole tiles; AdamW and the unscale keep default-scope nt stores).
// The kernels:
//   - segcopy: one engine for flatten (FSDP1 and FSDP2), copy-out, the cast and
//     the bf16 copies.  The host planner turns the layout into a short table of
//     (src, dst, length[, block stride]) segments passed in the kernel argument
//     block; each workgroup takes one tile of one segment (the tile -> segment
//     lookup is wave-uniform, on scalar registers: the segment with the most tiles
//     and every segment's first tile are loaded with the table's header, and the
//     others are found by counting), so no lane ever searches and every tile is a
//     straight streaming copy.  Launches of
//     2^15 tiles or more hand each XCD runs of 256 consecutive tiles.  When source
//     and destination are not 16-byte co-aligned, a scalar head aligns the
//     destination and the source is read in place with dword-aligned 16-byte
//     loads; only a bf16 source at an odd element offset is staged through LDS.
//   - grad_reduce: each lane owns 8 consecutive outputs and loads their 8 bf16
//     from 8 ranks at a time (one 16-byte load each, or a shifted pair when a
//     contribution is only 2-byte aligned) before adding them in rank order;
//     whole tiles swap halves across lanes so each store writes 1 KiB; the tile
//     the output's end cuts runs first, its last len % 8 outputs one per lane.
//     From 32 ranks and 12,288 whole tiles on, a row-major sweep instead: each
//     wave holds 16 tiles' sums with one rank in flight (flat sums), or 8 tiles'
//     group sums and totals with two ranks in flight where the runs are long
//     (hybrid sums, and flat ones as a single group) and one where they are
//     short, and walks the ranks in order, the grid sized to be resident at once
//     (each XCD one contiguous run of waves), so HBM serves a few contribution
//     rows at a time.  More ranks than one launch holds (128) take several launches that
//     carry their exact running sums through the output or a caller's workspace.
//   - adamw: elementwise over 8 elements per lane, 128-bit loads and stores.
//     Its state is read and written back in place: plain loads measure faster
//     than nt ones (6.5 vs 5.6 TB/s), and nt stores put its writes in HBM within
//     its own launch (plain stores leave them dirty in the 256 MB Infinity Cache,
//     which costs the next kernels, or AdamW itself once they outgrow it).
//   - accumulate: 16-byte bf16 loads (8 per lane), exchanged across lanes so that
//     each fp32 load and store instruction covers 1 KiB (a long accumulation hands
//     each XCD runs of 128 blocks); unscale: in place, four 16-byte vectors per lane.
//   - sqnorm: per-parameter sums of squares in binary64, one tile per workgroup
//     into a workspace, then one workgroup per parameter, in fixed orders.
// Every binary32 step is one IEEE operation, in the order the CPU oracle fixes;
// contraction into FMA is disabled for this file.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstddef>
#include <cstdint>
#include <cmath>
#include <vector>

#include "kernels.h"

#pragma clang fp contract(off)

namespace fsdp {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));

// Launch shapes and access policies, each measured on MI355X (the figures are TB/s on the
// GPT-175B block unit unless stated; alternating processes on one box).
constexpr int kThreads = 256;        // copy engine workgroup (also accumulate, unscale)
constexpr int kF32Vpl = 1;           // 4-element vectors per lane per tile, fp32 output
constexpr int kBF16Vpl = 2;          // 4-element vectors per lane per tile, fp32 -> bf16
constexpr int kB16Vpl = 1;           // 8-element vectors per lane per tile, bf16 -> bf16
// Whole-tile stores of the copies: buffer stores with this cache-policy operand, 18 =
// sc1 (device scope) + nt.  Against global nt stores: copy-out 6.48-6.50 vs 6.44-6.45,
// rank flatten 5.26-5.39 vs 4.87-4.94 (HIP events), bf16 copies 6.65-6.69 vs 6.24-6.30;
// nt alone (2) matched the global ones, and sc1 alone slowed the next kernel (AdamW) by a
// third.
constexpr int kTileStoreCpol = 18;
// From this many tiles (workgroups) on, a copy hands each of the eight XCDs runs of
// kXcdChunk consecutive tiles instead of every eighth tile.  Copy-out (885k tiles):
// dispatch order 6.46-6.49, one contiguous run per XCD 6.61-6.65, runs of 64 / 128 / 256 /
// 512 tiles 6.65-6.67 / 6.76 / 6.76-6.78 / 6.62-6.63.  One run per XCD made 64-256 MB
// copies 3-7% slower.  From 2^15 tiles on (rocprofv3, alternating processes, against 2^18):
// the T5 block's copy-out (98k tiles) 177.8-181.6 against 186.3-189.4 us, its local
// accumulation 306-325 against 328-332 us, the FSDP2 rows copy-out (41k tiles) 75.6-78.2
// against 79.4-80.1 us, fp32 copies of 268 MB - 1 GB 1-2% faster; 2^14 (which also takes
// the T5 rank flatten, 25k tiles) measured the same as 2^15.
constexpr uint32_t kXcdMinTiles = 1u << 15;
constexpr uint32_t kXcdChunk = 256u;
constexpr int kReduceThreads = 64;   // reduction tile kernel: one wave per 512-output tile
constexpr int kReduceAhead = 8;      // ranks loaded before their adds in the tile kernel
// The tile kernel needs few registers (47 VGPRs), so up to 8 of its waves per SIMD would be
// resident, and more contribution rows in flight at once read more slowly.  Each workgroup
// reserves this much LDS it does not use, which caps residency at 29 workgroups per CU (7.25
// waves per SIMD).  rocprofv3, alternating processes on one box: the T5 block's 8-way reduction
// 80.3-80.4 against 84.7-85.2 us uncapped (6, 5, 4 waves per SIMD: 81.1-81.8, 85.3-85.5,
// 90.1 us), the GPT-175B hybrid accumulating reduction on this kernel 570.7-572.1 against
// 594.5-595.9 us; the GPT-2-L block's 10.5-10.6 us either way.
constexpr unsigned kReduceLdsCap = 5632;
constexpr int kSweepMinRanks = 32;   // by default a launch sweeps ranks row-major from this many
constexpr int kSweepMinTiles = 12288;  // ... and from this many whole 512-output tiles on
// Shapes of the sweep.  The wide one (flat sums) holds 16 tiles' sums per wave and one rank
// in flight (8/12/16 tiles: 6.23/6.36/6.53 TB/s).  The grouped ones hold 8 tiles' group sums
// and totals, with two ranks in flight (232 VGPRs, 2 waves per SIMD) where every run of that
// shape holds at least kGroupSweepMinRunTiles tiles, its waves then filling the device (the
// flat sum takes it too, as one group), else one (168 VGPRs, 3 waves per SIMD; the hybrid sum
// only).  Measurements in launch_reduce_sweep.
constexpr int kSweepV = 16;
constexpr int kGroupSweepV = 8;
constexpr int kGroupSweepLongAhead = 2;
constexpr int64_t kGroupSweepMinRunTiles = 12288;
// 4-element vectors per lane in the gradient unscale: four from kUnscaleLongLen elements on, two
// below, where four leave too few workgroups for the device (rocprofv3 medians, three rounds of
// alternating processes, each launch after a 1 GiB read): GPT-175B shard (14.2 M) 19.36-19.46 us
// with four against 19.82-19.86 with two and 19.38-20.06 with one; T5 shard (25.2 M) 30.50-30.64
// against 30.40-30.46 and 31.82-32.14; GPT-2-L shard (2.5 M) 7.82-7.90 against 6.10-6.14 and
// 6.12-6.24 us.
constexpr int kUnscaleVpl = 4;
constexpr int kUnscaleShortVpl = 2;
constexpr int64_t kUnscaleLongLen = int64_t{1} << 23;
// The in-place local accumulation over all L of the GPT-175B unit (885k blocks of 2048) takes
// runs of 128 blocks per XCD: 6.38-6.40 TB/s, against 5.87-5.88 in dispatch order and runs of
// 16 / 32 / 64 / 256 blocks 5.98-5.99 / 6.12-6.21 / 6.32-6.34 / 6.37-6.38 (HIP events, two
// rounds in one process).
constexpr uint32_t kAccXcdChunk = 128u;
constexpr int kAdamThreads = 256;
// AdamW reads p, g, m, v with plain loads (nt loads: 5.57 against 6.46) and stores whole
// blocks with buffer stores of this cache policy, 2 = nt: 6.62-6.65 against 6.48-6.55 for
// global nt stores; device-scope nt stores (18) 5.46-5.59.
constexpr int kAdamStoreCpol = 2;

constexpr int kMaxSegs = 48;           // segments per launch (kernel-argument budget)
constexpr int kMaxContrib = 128;       // contribution pointers per reduce launch
static_assert(kReduceThreads % 64 == 0, "reduce workgroups are whole wave64s (lane exchange)");

// ---------------------------------------------------------------------------
// memory helpers: vector global accesses with the non-temporal hint (streamed
// once), plain variants for in-place state.
// ---------------------------------------------------------------------------
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f4 ld4(const float* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const f4*>(p));
}
__device__ __forceinline__ u4 ldu4(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u4*>(p));
}
// 16-byte loads from addresses that are only 4-byte aligned (global loads of
// several dwords need dword alignment only); they read exactly those 16 bytes.
typedef float f4w __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u4w __attribute__((ext_vector_type(4), aligned(4)));
__device__ __forceinline__ f4 ld4w(const float* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const f4w*>(p));
}
__device__ __forceinline__ u4 ldu4w(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u4w*>(p));
}
__device__ __forceinline__ void st4(float* p, f4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<f4*>(p));
}
__device__ __forceinline__ void stu4(void* p, u4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u4*>(p));
}
__device__ __forceinline__ void stu2(void* p, u2 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u2*>(p));
}

// fp32 pair -> packed bf16 pair (element 0 in the low half), round to nearest
// even: gfx950's v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    f2 x = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf2));
}
__device__ __forceinline__ uint16_t to_bf16(float a) {
    return static_cast<uint16_t>(pack_bf16x2(a, 0.0f) & 0xFFFFu);
}

// Buffer stores of whole blocks.  The resource spans `bytes` from `base`, an address that is
// the same in every lane (taken from the first active lane, so the resource sits in scalar
// registers); word 3 holds the 32-bit data format CDNA's buffer instructions need.  Callers
// store only at offsets inside the block, so the range check never drops a store.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(void* base, int bytes) {
    const uint64_t b = reinterpret_cast<uintptr_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32));
    return __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo), 0, bytes, 0x00020000);
}
template <int kCpol>
__device__ __forceinline__ void bst4(__amdgpu_buffer_rsrc_t r, int off, f4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), r, off, 0, kCpol);
}
template <int kCpol>
__device__ __forceinline__ void bst2(__amdgpu_buffer_rsrc_t r, int off, u2 v) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kCpol);
}

// Element pipes of the copy engine.  A vector is one 16-byte source load (4 fp32
// or 8 bf16) and one store of the same element count (16 bytes, or 8 bytes for
// fp32 -> bf16); `gather` re-reads a bf16 vector from LDS at an element shift.  kVpl vectors per lane make a tile of kThreads * E * kVpl
// elements, lane l owning vectors l, l + kThreads, ... so every load and store
// instruction is contiguous across the wave.  `put_tile` stores a whole tile from
// its first element, which every lane of the workgroup shares.
template <typename SrcT, typename DstT> struct Cp;
template <> struct Cp<float, float> {
    static constexpr int E = 4, kVpl = kF32Vpl;
    static constexpr unsigned kDstAlign = 16;  // bytes a vector store needs
    using V = f4;
    __device__ static V load(const float* p) { return ld4(p); }
    __device__ static V loadw(const float* p) { return ld4w(p); }
    __device__ static void put(float* d, V x) { st4(d, x); }
    __device__ static void put_tile(float* d, const V* x) {
        const auto r = block_rsrc(d, kThreads * E * kVpl * 4);
#pragma unroll
        for (int u = 0; u < kVpl; ++u)
            bst4<kTileStoreCpol>(r, 16 * (threadIdx.x + u * kThreads), x[u]);
    }
    __device__ static void put1(float* d, float x) { *d = x; }
    __device__ static void zero(float* d) { st4(d, f4{0.0f, 0.0f, 0.0f, 0.0f}); }
    __device__ static void zero1(float* d) { *d = 0.0f; }
};
template <> struct Cp<float, uint16_t> {
    static constexpr int E = 4, kVpl = kBF16Vpl;
    static constexpr unsigned kDstAlign = 8;
    using V = f4;
    __device__ static V load(const float* p) { return ld4(p); }
    __device__ static V loadw(const float* p) { return ld4w(p); }
    __device__ static void put(uint16_t* d, V x) {
        stu2(d, u2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])});
    }
    __device__ static void put_tile(uint16_t* d, const V* x) {
        const auto r = block_rsrc(d, kThreads * E * kVpl * 2);
#pragma unroll
        for (int u = 0; u < kVpl; ++u)
            bst2<kTileStoreCpol>(r, 8 * (threadIdx.x + u * kThreads),
                                 u2{pack_bf16x2(x[u][0], x[u][1]), pack_bf16x2(x[u][2], x[u][3])});
    }
    __device__ static void put1(uint16_t* d, float x) { *d = to_bf16(x); }
    __device__ static void zero(uint16_t* d) { stu2(d, u2{0u, 0u}); }
    __device__ static void zero1(uint16_t* d) { *d = 0; }
};
template <> struct Cp<uint16_t, uint16_t> {
    static constexpr int E = 8, kVpl = kB16Vpl;
    static constexpr unsigned kDstAlign = 16;
    using V = u4;
    __device__ static V load(const uint16_t* p) { return ldu4(p); }
    __device__ static V loadw(const uint16_t* p) { return ldu4w(p); }
    __device__ static V gather(const uint16_t* p) {
        return u4{p[0] | (uint32_t{p[1]} << 16), p[2] | (uint32_t{p[3]} << 16),
                  p[4] | (uint32_t{p[5]} << 16), p[6] | (uint32_t{p[7]} << 16)};
    }
    __device__ static void put(uint16_t* d, V x) { stu4(d, x); }
    __device__ static void put_tile(uint16_t* d, const V* x) {
        const auto r = block_rsrc(d, kThreads * E * kVpl * 2);
#pragma unroll
        for (int u = 0; u < kVpl; ++u)
            bst4<kTileStoreCpol>(r, 16 * (threadIdx.x + u * kThreads), __builtin_bit_cast(f4, x[u]));
    }
    __device__ static void put1(uint16_t* d, uint16_t x) { *d = x; }
    __device__ static void zero(uint16_t* d) { stu4(d, u4{0u, 0u, 0u, 0u}); }
    __device__ static void zero1(uint16_t* d) { *d = 0; }
};
template <typename SrcT, typename DstT>
constexpr int tile_elems() { return kThreads * Cp<SrcT, DstT>::E * Cp<SrcT, DstT>::kVpl; }

// ---------------------------------------------------------------------------
// segcopy
// ---------------------------------------------------------------------------
// One segment of a launch; the fields a one-block segment reads come first (the strides are
// read only by segments of several blocks).
struct DevSeg {
    const void* src;  // nullptr: zero fill
    void* dst;
    int64_t blk_n, last_n;
    uint32_t nblk, tiles_per_blk, tile0, unused;
    int64_t src_stride, dst_stride;
};
// A launch's segments, passed by value in the kernel-argument block: a table of kCap entries,
// the smallest of 1, 4, 8, 16 and kMaxSegs that holds the launch's segments, with the segments'
// first tiles in one array next to the header and a copy of the segment with the most tiles.
// The kernel also takes the header and that segment's one-block fields as scalar arguments
// ahead of the table: the dispatch preloads those into scalar registers (kernel-argument
// preloading, 16 dwords), so that segment's tiles start without a scalar load.
template <int kCap>
struct SegTable {
    uint32_t ntiles;
    uint32_t nseg;
    uint32_t xcd_runs;      // tiles in XCD-chunked order (xcd_chunked)
    uint32_t hot_tiles;     // tiles of `hot`
    uint32_t start[kCap];   // seg[i].tile0; 0xFFFFFFFF past nseg
    DevSeg hot;             // the segment with the most tiles (the only one in one-segment tables)
    DevSeg seg[kCap];
};
static_assert(sizeof(SegTable<kMaxSegs>) <= 4096 - 64, "segment table and scalar arguments must fit one kernel argument block");

// The dispatcher deals a launch's workgroups to MI355X's eight XCDs in turn (workgroup b to
// XCD b % 8).  This maps b to the tile it runs so that each XCD takes one contiguous run of
// the G tiles (the first G % 8 XCDs one tile more).  It is a bijection of [0, G) whatever the
// placement, so results never depend on it; only speed does.
__device__ __forceinline__ uint32_t xcd_contiguous(uint32_t b, uint32_t G) {
    const uint32_t x = b & 7u, loc = b >> 3, per = G >> 3, rem = G & 7u;
    return x * per + (x < rem ? x : rem) + loc;
}

// The same in groups of 8 C tiles: inside each group XCD x takes the C tiles from x C on, so
// the eight XCDs work through one compact window of the launch; a last, partial group is
// split by xcd_contiguous.  Also a bijection of [0, G).
template <uint32_t C>
__device__ __forceinline__ uint32_t xcd_chunked(uint32_t b, uint32_t G) {
    constexpr uint32_t span = 8u * C;
    const uint32_t full = G / span * span;
    if (b >= full) return full + xcd_contiguous(b - full, G - full);
    const uint32_t r = b % span;
    return b - r + (r & 7u) * C + (r >> 3);
}

// n <= tile elements; s 16-byte aligned (kWord: 4-byte aligned), d aligned for its
// vector store.
template <typename SrcT, typename DstT, bool kWord = false>
__device__ __forceinline__ void tile_aligned(const SrcT* __restrict__ s, DstT* __restrict__ d,
                                             int n) {
    using P = Cp<SrcT, DstT>;
    constexpr int E = P::E, kVpl = P::kVpl;
    const auto load = [](const SrcT* p) { return kWord ? P::loadw(p) : P::load(p); };
    const int nv = n / E;
    if (nv == kThreads * kVpl) {  // full tile: all loads issued before any store
        typename P::V x[kVpl];
#pragma unroll
        for (int u = 0; u < kVpl; ++u) x[u] = load(s + E * (threadIdx.x + u * kThreads));
        P::put_tile(d, x);
        return;
    }
    for (int v = threadIdx.x; v < nv; v += kThreads) P::put(d + E * v, load(s + E * v));
    for (int e = E * nv + threadIdx.x; e < n; e += kThreads) P::put1(d + e, s[e]);
}

// Elements of DstT from d up to the next boundary its vector store needs.
template <typename SrcT, typename DstT>
__device__ __forceinline__ int head_to_align(const DstT* d) {
    constexpr unsigned a = Cp<SrcT, DstT>::kDstAlign;
    return static_cast<int>(((a - (reinterpret_cast<uintptr_t>(d) & (a - 1))) & (a - 1)) /
                            sizeof(DstT));
}

template <typename SrcT, typename DstT>
__device__ __forceinline__ void tile_zero(DstT* d, int n) {
    using P = Cp<SrcT, DstT>;
    constexpr int E = P::E;
    const int h = min(head_to_align<SrcT, DstT>(d), n);
    if (static_cast<int>(threadIdx.x) < h) P::zero1(d + threadIdx.x);
    d += h;
    n -= h;
    const int nv = n / E;
    for (int v = threadIdx.x; v < nv; v += kThreads) P::zero(d + E * v);
    for (int e = E * nv + threadIdx.x; e < n; e += kThreads) P::zero1(d + e);
}

// Any element-aligned source and destination.  A short head of scalar stores
// aligns the destination.  A source then 4-byte aligned (always, for fp32) is read
// with 16-byte loads at its own address.  A bf16 source at an odd element offset is
// loaded as aligned 16-byte vectors (covering exactly the 16-byte blocks that hold
// the tile, so no access leaves them) into LDS and re-read at the shift; that path
// has tile-uniform control flow (barriers).
template <typename SrcT, typename DstT>
__device__ __forceinline__ void tile_general(const SrcT* s, DstT* d, int n, SrcT* lds) {
    using P = Cp<SrcT, DstT>;
    constexpr int E = P::E;
    const int h = min(head_to_align<SrcT, DstT>(d), n);
    if (static_cast<int>(threadIdx.x) < h) P::put1(d + threadIdx.x, s[threadIdx.x]);
    s += h;
    d += h;
    n -= h;
    const int shift = static_cast<int>((reinterpret_cast<uintptr_t>(s) & 15u) / sizeof(SrcT));
    if (shift == 0) {
        tile_aligned<SrcT, DstT>(s, d, n);
        return;
    }
    if constexpr (sizeof(SrcT) >= 4) {
        tile_aligned<SrcT, DstT, true>(s, d, n);
    } else {
        if ((shift & 1) == 0) {  // tile-uniform
            tile_aligned<SrcT, DstT, true>(s, d, n);
            return;
        }
        const SrcT* base = s - shift;
        const int nload = (shift + n + E - 1) / E;  // <= tile/E + 1 vectors
        for (int v = threadIdx.x; v < nload; v += kThreads)
            *reinterpret_cast<typename P::V*>(lds + E * v) = P::load(base + E * v);
        __syncthreads();
        const int nv = n / E;
        for (int v = threadIdx.x; v < nv; v += kThreads) P::put(d + E * v, P::gather(lds + shift + E * v));
        for (int e = E * nv + threadIdx.x; e < n; e += kThreads) P::put1(d + e, lds[shift + e]);
        __syncthreads();
    }
}

// Tile `local` of segment sg (tiles count from the segment's first).
template <typename SrcT, typename DstT, bool kGeneral>
__device__ __forceinline__ void copy_tile(const DevSeg& sg, uint32_t local, SrcT* lds) {
    constexpr int kTile = tile_elems<SrcT, DstT>();
    const uint32_t b = sg.nblk == 1 ? 0u : local / sg.tiles_per_blk;
    const uint32_t tb = local - b * sg.tiles_per_blk;
    const int64_t e0 = static_cast<int64_t>(tb) * kTile;
    const int64_t bn = (b + 1 == sg.nblk) ? sg.last_n : sg.blk_n;
    if (e0 >= bn) return;
    const int n = static_cast<int>(min(static_cast<int64_t>(kTile), bn - e0));
    // block offsets only for segments of several blocks: a one-block segment never reads its
    // strides (they lie outside the preloaded part of the table)
    int64_t doff = e0, soff = e0;
    if (sg.nblk != 1) {
        doff += static_cast<int64_t>(b) * sg.dst_stride;
        soff += static_cast<int64_t>(b) * sg.src_stride;
    }
    DstT* d = static_cast<DstT*>(sg.dst) + doff;
    if (sg.src == nullptr) {
        tile_zero<SrcT, DstT>(d, n);
        return;
    }
    const SrcT* s = static_cast<const SrcT*>(sg.src) + soff;
    if constexpr (kGeneral)
        tile_general<SrcT, DstT>(s, d, n, lds);
    else
        tile_aligned<SrcT, DstT>(s, d, n);
}

// One tile per workgroup (grid = number of tiles).  A workgroup's first vector load waits for
// whatever locates its tile, so the segment with the most tiles (the only one, in one-segment
// launches) comes as scalar arguments ahead of the table, which the dispatch preloads into
// scalar registers (kernel-argument preloading, 16 dwords): that segment's tiles issue their
// loads without a scalar load.  Against the same fields read from the table with every load
// pinned at the start (rocprofv3 medians, three rounds of alternating processes, each launch
// after a 1 GiB read): GPT-175B rank flatten 18.40-18.76 against 18.70-19.24 us, its rank
// cast 14.42-14.52 against 14.68-14.88, GPT-2-L rank flatten 5.28-5.64 against 5.64-5.98 and
// copy-out 20.26-20.42 against 20.70-20.88 us; only the GPT-2-L rank cast measured the same or
// slower (4.96-5.38 against 4.86-5.02 us).  Tiles outside the big segment look up theirs:
// the segments' first tiles are loaded together (pinned by empty asm statements; the compiler
// would otherwise issue each load just before its compare, after the previous one's wait),
// counted on scalar registers, and the segment is loaded.  Counting instead of a binary search
// of the table (a dependent load per step): GPT-2-L block copy-out 20.34-20.52 against
// 21.08-21.30 us, FSDP2 rows unit flatten 14.88-15.06 against 15.16-15.48 us.  The first tiles
// are pinned only in tables of up to 8 entries: with 16 the compiler splits their loads into two
// rounds.  Five to eight segments take the 8-entry table: the GPT-2-L block's rank 2 (two large
// segments among five) 5.62-5.76 us against 6.06-6.30 in the 16-entry table.
template <typename SrcT, typename DstT, bool kGeneral, int kCap>
__global__ __launch_bounds__(kThreads) void segcopy_kernel(
    uint32_t ntiles, uint32_t xcdr, uint32_t hot_tiles, uint32_t hot_tile0, const void* hot_src,
    void* hot_dst, int64_t hot_blk_n, int64_t hot_last_n, uint32_t hot_nblk, uint32_t hot_tpb,
    SegTable<kCap> t) {
    constexpr int kTile = tile_elems<SrcT, DstT>();
    __shared__ __attribute__((aligned(16))) SrcT lds[kGeneral && sizeof(SrcT) == 2 ? kTile + 16 : 8];
    // the hot segment from the preloaded arguments; its strides (read by segments of several
    // blocks only) from the table
    DevSeg z;
    z.src = hot_src;
    z.dst = hot_dst;
    z.blk_n = hot_blk_n;
    z.last_n = hot_last_n;
    z.nblk = hot_nblk;
    z.tiles_per_blk = hot_tpb;
    z.tile0 = hot_tile0;
    z.unused = 0;
    z.src_stride = t.hot.src_stride;
    z.dst_stride = t.hot.dst_stride;
    const uint32_t tile = xcdr ? xcd_chunked<kXcdChunk>(blockIdx.x, ntiles) : blockIdx.x;
    const uint32_t local = tile - hot_tile0;
    if (kCap == 1 || local < hot_tiles) {
        if constexpr (!kGeneral) {
            // the common case first, in as few scalar instructions as possible: a whole tile
            // of a one-block segment
            const int64_t e0 = static_cast<int64_t>(local) * kTile;
            if (hot_nblk == 1 && hot_src != nullptr && e0 + kTile <= hot_last_n) {
                tile_aligned<SrcT, DstT>(static_cast<const SrcT*>(hot_src) + e0,
                                         static_cast<DstT*>(hot_dst) + e0, kTile);
                return;
            }
        }
        copy_tile<SrcT, DstT, kGeneral>(z, local, lds);
        return;
    }
    // the segment holding this tile (wave-uniform): the number of later segments that start
    // at or before it, the starts loaded together (one round trip; without the pins the
    // compiler loads each just before its compare, after the previous one's wait)
    if constexpr (kCap <= 8) {
#pragma unroll
        for (int i = 1; i < kCap; ++i) asm volatile("" ::"s"(t.start[i]));
    }
    uint32_t k = 0;
#pragma unroll
    for (int i = 1; i < kCap; ++i) k += t.start[i] <= tile ? 1u : 0u;
    const DevSeg& sg = t.seg[k];
    copy_tile<SrcT, DstT, kGeneral>(sg, tile - sg.tile0, lds);
}

// ---------------------------------------------------------------------------
// gradient reduction
// ---------------------------------------------------------------------------
enum PreMode { kPreNone = 0, kPreRecip = 1, kPreDiv = 2 };

// A reduction over more ranks than one launch's pointer table holds takes several
// launches in rank order (plan_reduce); between them the running sums sit in HBM, stored
// exactly: the total (the flat sum, or the sum of the completed groups) in `carry_t`, and,
// when a group is longer than one launch, that group's partial sum in `carry_s`.  The
// flags say what a launch loads and stores; per output the operations and their order
// are those of one launch over all ranks.
constexpr uint32_t kTIn = kReduceTIn, kSIn = kReduceSIn, kTOut = kReduceTOut,
                   kSOut = kReduceSOut, kLast = kReduceLast;

struct ReduceArgs {
    const uint16_t* c[kMaxContrib];
    float* out;
    float* carry_t;
    float* carry_s;
    int64_t len;
    int32_t nc;      // contributions in this launch
    int32_t group;   // hybrid: ranks per group
    int32_t pos0;    // hybrid: position of this launch's first rank in its group
    uint32_t flags;
    float pre, rpre, post;
};

// One term: a bf16 (already in the upper half of `bits`) widened exactly, then
// divided by pre.  For a power-of-two pre whose reciprocal is a normal float,
// x*(1/pre) is the same correctly rounded value as x/pre.
template <int kPre>
__device__ __forceinline__ float term(uint32_t bits, const ReduceArgs& a) {
    const float f = __builtin_bit_cast(float, bits);
    if constexpr (kPre == kPreNone) return f;
    else if constexpr (kPre == kPreRecip) return f * a.rpre;
    else return f / a.pre;
}

template <int kPre>
__device__ __forceinline__ void set8(float* acc, u4 x, const ReduceArgs& a) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        acc[2 * q] = term<kPre>(x[q] << 16, a);
        acc[2 * q + 1] = term<kPre>(x[q] & 0xFFFF0000u, a);
    }
}

template <int kPre>
__device__ __forceinline__ void add8(float* acc, u4 x, const ReduceArgs& a) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        acc[2 * q] = acc[2 * q] + term<kPre>(x[q] << 16, a);
        acc[2 * q + 1] = acc[2 * q + 1] + term<kPre>(x[q] & 0xFFFF0000u, a);
    }
}

// How the vector path reads a rank's 8 bf16 (the output is 16-byte aligned unless
// kLdScalar): kLdWord, every contribution at least 4-byte aligned: one four-dword
// load (global loads of several dwords need dword alignment only).  kLdHalf, some
// contribution only 2-byte aligned: such a rank's 8 elements are read as the four
// dwords that start one element early plus the dword after them, then shifted by
// one element.
enum : int { kLdScalar = 0, kLdWord = 1, kLdHalf = 2 };

// Rank r's elements j0 .. j0+7 (j0 a multiple of 8, all inside the rank's buffer),
// read in two steps so that a batch of ranks issues all its loads before any shift.
// kLdHalf: o = 1 when the buffer is only 2-byte aligned, else 0; the lane reads four
// dwords from element j0 - o on and one at element j0 + 6 + o (j0 + 7 and j0 + 8 when
// o = 1; when o = 0 two of the lane's own, unused).  Each dword read holds at least
// one of the lane's 8 elements, so no read reaches a page the buffer does not.
struct Raw {
    u4 v;
    uint32_t w4;
};

__device__ __forceinline__ int half_off(const uint16_t* c) {
    return static_cast<int>(reinterpret_cast<uintptr_t>(c) >> 1) & 1;
}

template <int kLd>
__device__ __forceinline__ Raw load_raw(const ReduceArgs& a, int r, int64_t j0) {
    Raw x;
    if constexpr (kLd == kLdWord) {
        x.v = ldu4w(a.c[r] + j0);
    } else {
        const int o = half_off(a.c[r]);
        const uint16_t* p = a.c[r] + j0 - o;  // dword aligned
        x.v = ldu4w(p);
        x.w4 = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p + 6 + 2 * o));
    }
    return x;
}

template <int kLd>
__device__ __forceinline__ u4 finish(const Raw& x, const ReduceArgs& a, int r) {
    if constexpr (kLd == kLdWord) {
        return x.v;
    } else {
        const uint32_t b = 2u * static_cast<uint32_t>(half_off(a.c[r]));  // bytes
        const uint32_t w[5] = {x.v[0], x.v[1], x.v[2], x.v[3], x.w4};
        u4 y;
#pragma unroll
        for (int q = 0; q < 4; ++q) y[q] = __builtin_amdgcn_alignbyte(w[q + 1], w[q], b);
        return y;
    }
}

__device__ __forceinline__ void load_out8(float* v, const float* out) {
    const f4 lo = ld4(out), hi = ld4(out + 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        v[q] = lo[q];
        v[4 + q] = hi[q];
    }
}

// Adds ranks [r, end) to acc in rank order, loading kAhead ranks before their adds.
template <int kPre, int kLd>
__device__ __forceinline__ void add_ranks(float* acc, int r, int end, int64_t j0,
                                          const ReduceArgs& a) {
    for (; r + kReduceAhead <= end; r += kReduceAhead) {
        Raw x[kReduceAhead];
#pragma unroll
        for (int u = 0; u < kReduceAhead; ++u) x[u] = load_raw<kLd>(a, r + u, j0);
#pragma unroll
        for (int u = 0; u < kReduceAhead; ++u) add8<kPre>(acc, finish<kLd>(x[u], a, r + u), a);
    }
    for (; r < end; ++r) add8<kPre>(acc, finish<kLd>(load_raw<kLd>(a, r, j0), a, r), a);
}

// One output, for buffers that are not 16-byte aligned and for the ragged last tile.
// Up to 8 ranks are loaded before their adds, which run in the vector path's order.
template <int kPre, bool kHybrid, bool kAccum>
__device__ __forceinline__ void reduce_one(const ReduceArgs& a, int64_t j) {
    constexpr int kBatch = 8;
    bool have = (a.flags & kTIn) != 0;
    float acc = have ? a.carry_t[j] : 0.0f;
    float s = (kHybrid && (a.flags & kSIn)) ? a.carry_s[j] : 0.0f;
    int pos = a.pos0;
    for (int r = 0; r < a.nc; r += kBatch) {
        const int cnt = min(kBatch, a.nc - r);
        float t[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            if (u < cnt) t[u] = term<kPre>(static_cast<uint32_t>(a.c[r + u][j]) << 16, a);
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            if (u >= cnt) break;
            if constexpr (!kHybrid) {
                // one running sum in rank order
                acc = have ? acc + t[u] : t[u];
                have = true;
            } else {
                // group sums, each folded into the total after the group's last rank
                s = pos == 0 ? t[u] : s + t[u];
                if (++pos == a.group) {
                    acc = have ? acc + s : s;
                    have = true;
                    pos = 0;
                }
            }
        }
    }
    if (a.flags & kLast) {
        acc = acc / a.post;
        if constexpr (kAccum) acc = a.out[j] + acc;
        a.out[j] = acc;
        return;
    }
    if (a.flags & kTOut) a.carry_t[j] = acc;
    if (kHybrid && (a.flags & kSOut)) a.carry_s[j] = s;
}

// Stores a wave's 512 outputs of one whole tile, lane l holding outputs 8l .. 8l+7
// in acc: the halves are swapped across lanes (ds_bpermute, no LDS allocation) so
// that each store instruction writes 1 KiB of whole cache lines.  lane l stores
// outputs 4l .. 4l+3 of each 256-output half, which lane 32h + l/2 holds.  The
// stores are the copies' device-scope nt buffer stores (the 2 KiB block is 16-byte
// aligned: the whole-tile path runs only on 16-byte-aligned outputs and workspace
// slots).  Against global nt stores, HIP-event medians, alternating processes on one
// box: the 8-way tile reduction of 25.2 M outputs 79.9-81.1 against 81.1-82.6 us and of
// 10.5 M 38.2-38.6 against 38.8-39.6 us; the 128-way sweeps (flat, and hybrid
// accumulating) unchanged (533.0-536.2 against 533.0-536.7 us, 542.0-542.6 against
// 541.8-543.7 us); default-scope nt buffer stores like AdamW's measured as the global ones.
__device__ __forceinline__ void store_whole8(float* wave_out, const float* acc) {
    const int lane = threadIdx.x & 63;
    const auto rs = block_rsrc(wave_out, 2048);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int src = 32 * h + (lane >> 1);
        float w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float lo = __shfl(acc[i], src, 64);
            const float hi = __shfl(acc[4 + i], src, 64);
            w[i] = (lane & 1) ? hi : lo;
        }
        bst4<kTileStoreCpol>(rs, 4 * (256 * h + 4 * lane), f4{w[0], w[1], w[2], w[3]});
    }
}

// A lane's 8 outputs j0 .. j0+7 into `base` (an array indexed like the output).
// kWhole: the wave's whole tile at once (every lane of the wave takes part).
template <bool kWhole>
__device__ __forceinline__ void store8(float* base, int64_t j0, const float* v) {
    if constexpr (kWhole) {
        store_whole8(base + (j0 - 8 * static_cast<int64_t>(threadIdx.x & 63)), v);
    } else {
        st4(base + j0, f4{v[0], v[1], v[2], v[3]});
        st4(base + j0 + 4, f4{v[4], v[5], v[6], v[7]});
    }
}

// End of a launch for a lane's 8 outputs: the last launch divides the total by post,
// adds it to what `out` holds when accumulating, and stores it; an earlier launch
// stores what the next one carries on with.
template <bool kAccum, bool kWhole, bool kHybrid>
__device__ __forceinline__ void finish8(const ReduceArgs& a, int64_t j0, float* acc, const float* s) {
    if (a.flags & kLast) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = acc[e] / a.post;
        if constexpr (kAccum) {
            float prev[8];
            load_out8(prev, a.out + j0);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = prev[e] + acc[e];
        }
        store8<kWhole>(a.out, j0, acc);
        return;
    }
    if (a.flags & kTOut) store8<kWhole>(a.carry_t, j0, acc);
    if (kHybrid && (a.flags & kSOut)) store8<kWhole>(a.carry_s, j0, s);
}

// The 8 outputs j0 .. j0+7 of one lane over this launch's ranks.  kWhole: the tile
// is whole and is stored with store_whole8; otherwise each lane stores its own 8.
template <int kPre, int kLd, bool kHybrid, bool kAccum, bool kWhole>
__device__ __forceinline__ void reduce_lane(const ReduceArgs& a, int64_t j0) {
    float acc[8];
    if constexpr (!kHybrid) {
        int r = 0;
        if (a.flags & kTIn) {
            load_out8(acc, a.carry_t + j0);
        } else {
            set8<kPre>(acc, finish<kLd>(load_raw<kLd>(a, 0, j0), a, 0), a);
            r = 1;
        }
        add_ranks<kPre, kLd>(acc, r, a.nc, j0, a);
        finish8<kAccum, kWhole, false>(a, j0, acc, acc);
    } else {
        // Loads run kReduceAhead ranks ahead regardless of group boundaries; a
        // wave-uniform position-in-group counter starts each group's sum at its first
        // rank and folds it into the total after its last.
        bool have = (a.flags & kTIn) != 0;
        if (have) {
            load_out8(acc, a.carry_t + j0);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = 0.0f;  // not read before the first fold
        }
        float s[8];
        int pos = a.pos0;
        if (a.flags & kSIn) {
            load_out8(s, a.carry_s + j0);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) s[e] = 0.0f;  // pos0 == 0: set by the first rank
        }
        for (int r = 0; r < a.nc; r += kReduceAhead) {
            const int n = min(kReduceAhead, a.nc - r);
            Raw x[kReduceAhead];
#pragma unroll
            for (int u = 0; u < kReduceAhead; ++u)
                if (u < n) x[u] = load_raw<kLd>(a, r + u, j0);
#pragma unroll
            for (int u = 0; u < kReduceAhead; ++u) {
                if (u >= n) break;
                const u4 v = finish<kLd>(x[u], a, r + u);
                if (pos == 0) set8<kPre>(s, v, a); else add8<kPre>(s, v, a);
                if (++pos == a.group) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[e] = have ? acc[e] + s[e] : s[e];
                    have = true;
                    pos = 0;
                }
            }
        }
        finish8<kAccum, kWhole, true>(a, j0, acc, s);
    }
}

// One tile of kReduceThreads * 8 outputs per workgroup.  Each lane owns 8
// consecutive outputs; for every rank it loads their 8 bf16 as one 16-byte
// vector (a wave reads 1 KiB contiguous per rank), kReduceAhead ranks at a time,
// then adds them strictly in rank order.  Hybrid: the same within each group of
// ranks, then the group sums in group order.  kLd: how contributions are read
// (the output is 16-byte aligned unless kLd is kLdScalar).
// The tile that the output's end cuts runs first (workgroup 0), so that its longer
// work overlaps the others': its lanes with 8 outputs take the vector path, then
// the last len % 8 outputs take one lane each.
template <int kPre, int kLd, bool kHybrid, bool kAccum>
__global__ __launch_bounds__(kReduceThreads) void reduce_kernel(ReduceArgs a) {
    constexpr int kEpt = 8;
    constexpr int64_t kPerBlk = static_cast<int64_t>(kReduceThreads) * kEpt;
    const int64_t ntiles = (a.len + kPerBlk - 1) / kPerBlk;
    int64_t blk = blockIdx.x;
    if (a.len % kPerBlk != 0) blk = blk == 0 ? ntiles - 1 : blk - 1;
    if constexpr (kLd != kLdScalar) {
        const int64_t j0 = blk * kPerBlk + static_cast<int64_t>(threadIdx.x) * kEpt;
        if (blk * kPerBlk + kPerBlk <= a.len) {
            reduce_lane<kPre, kLd, kHybrid, kAccum, true>(a, j0);
            return;
        }
        if (j0 + kEpt <= a.len) reduce_lane<kPre, kLd, kHybrid, kAccum, false>(a, j0);
        const int64_t j = (a.len & ~static_cast<int64_t>(kEpt - 1)) + threadIdx.x;
        if (j < a.len) reduce_one<kPre, kHybrid, kAccum>(a, j);
    } else {
#pragma unroll
        for (int e = 0; e < kEpt; ++e) {
            const int64_t j = blk * kPerBlk + static_cast<int64_t>(e) * kReduceThreads + threadIdx.x;
            if (j < a.len) reduce_one<kPre, kHybrid, kAccum>(a, j);
        }
    }
}

// Many ranks: a row-major sweep.  A tile kernel wave reads 1 KiB from every rank for
// its 512 outputs, so the waves in flight read from all ranks' rows at once (128
// contribution rows on a 128-rank shard), and HBM serves that many scattered streams
// more slowly than a few (read-only: 6.5 against 7.0 TB/s).  Here each wave owns kV
// consecutive whole tiles (8 kV sums per lane) and walks the ranks in order, with the
// next kA ranks' kV vectors in flight; the host sizes the grid so that every wave is
// resident at once, so the waves move through the ranks together and HBM serves a few
// rows at a time.  Per output the operations and their order are those of the tile path
// (whole-dword contributions), so the results are identical.  The grouped shape
// (kHybrid) keeps a second set of kV x 8 sums per lane (the group's), folded into the
// total after each group's last rank.  Block layout of a launch: the tile the output's
// end cuts (if any), then n_single whole tiles that take the tile path, then the sweep
// waves.
struct SweepArgs {
    ReduceArgs r;
    int64_t t_first;   // first whole tile (512 outputs) of this launch
    int32_t cut;       // 1: block 0 reduces the tile the output's end cuts
    int32_t n_single;  // then this many blocks reduce one whole tile each
};

template <int kPre, bool kAccum, bool kHybrid, int kV, int kA>
__device__ __forceinline__ void sweep_wave(const ReduceArgs& a, int64_t t0) {
    constexpr int kTile = 512;
    const int lane = threadIdx.x & 63;
    // element offset of the lane's first vector from the run's start (vector v: + 512 v)
    const int64_t base = t0 * kTile;
    const int off = 8 * lane;
    // The sums start from -0.0f: -0 + t == t for every t (a NaN comes out quiet, as the
    // divide by post makes it anyway), so the first add gives the tile path's first
    // assignment, for the flat sum, a group's sum and the total alike.
    float acc[kV][8];                // the flat sum; hybrid: the total of completed groups
    float s[kHybrid ? kV : 1][8];    // hybrid: the current group's sum
    if (a.flags & kTIn) {
#pragma unroll
        for (int v = 0; v < kV; ++v) load_out8(acc[v], a.carry_t + base + off + kTile * v);
    } else {
#pragma unroll
        for (int v = 0; v < kV; ++v)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[v][e] = -0.0f;
    }
    if constexpr (kHybrid) {
        if (a.flags & kSIn) {
#pragma unroll
            for (int v = 0; v < kV; ++v) load_out8(s[v], a.carry_s + base + off + kTile * v);
        } else {
#pragma unroll
            for (int v = 0; v < kV; ++v)
#pragma unroll
                for (int e = 0; e < 8; ++e) s[v][e] = -0.0f;
        }
    }
    int pos = a.pos0;
    // kA ranks' vectors in flight: slot q holds rank r + q while rank r is added.  With
    // kA = 2 the reload is conditional (the last ranks have none), and the compiler loads
    // into fresh registers, then waits for those loads before the adds of the rank in hand:
    // each wave streams a burst, then computes.  That measured faster than the forms that
    // overlap the two (the grouped 128-way reduction of the GPT-175B shard, rocprofv3:
    // 535-541 us against 557-577 us for explicit overlapped, copy-and-wait and
    // unconditional-reload versions).
    u4 x[kA][kV];
#pragma unroll
    for (int q = 0; q < kA; ++q) {
        if (q >= a.nc) break;
        const uint16_t* cq = a.c[q] + base;
#pragma unroll
        for (int v = 0; v < kV; ++v) x[q][v] = ldu4w(cq + off + kTile * v);
    }
    int r = 0;
    for (; r + kA < a.nc; r += kA) {
#pragma unroll
        for (int q = 0; q < kA; ++q) {
            // rank r + q is added, and its slot reloaded with rank r + q + kA (if any)
            const bool more = kA == 1 || r + q + kA < a.nc;  // kA == 1: the loop bound
            const uint16_t* cn = a.c[more ? r + q + kA : 0] + base;
#pragma unroll
            for (int v = 0; v < kV; ++v) {
                // one vector at a time, its adds before its reload: no second copy of any
                // vector is live
                if constexpr (kHybrid) add8<kPre>(s[v], x[q][v], a);
                else add8<kPre>(acc[v], x[q][v], a);
                if (more) x[q][v] = ldu4w(cn + off + kTile * v);
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (kHybrid) {
                // a group that ends with this rank is folded into the total (wave-uniform)
                if (++pos == a.group) {
#pragma unroll
                    for (int v = 0; v < kV; ++v)
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            acc[v][e] = acc[v][e] + s[v][e];
                            s[v][e] = -0.0f;
                        }
                    pos = 0;
                }
            }
        }
    }
    // the last ranks r .. nc - 1, already loaded into slots 0 .. nc - 1 - r
#pragma unroll
    for (int q = 0; q < kA; ++q) {
        if (r + q >= a.nc) break;
#pragma unroll
        for (int v = 0; v < kV; ++v) {
            if constexpr (kHybrid) add8<kPre>(s[v], x[q][v], a);
            else add8<kPre>(acc[v], x[q][v], a);
        }
        if constexpr (kHybrid) {
            if (++pos == a.group) {
#pragma unroll
                for (int v = 0; v < kV; ++v)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        acc[v][e] = acc[v][e] + s[v][e];
                        s[v][e] = -0.0f;
                    }
                pos = 0;
            }
        }
    }
#pragma unroll
    for (int v = 0; v < kV; ++v) {
        if constexpr (kHybrid) finish8<kAccum, true, true>(a, base + off + kTile * v, acc[v], s[v]);
        else finish8<kAccum, true, false>(a, base + off + kTile * v, acc[v], acc[v]);
    }
}

template <int kPre, bool kAccum, bool kHybrid, int kV, int kA>
__global__ __launch_bounds__(64) void reduce_sweep_kernel(SweepArgs s) {
    const ReduceArgs& a = s.r;
    constexpr int64_t kTile = 512;
    // the whole grid is resident: each XCD takes one contiguous run of the blocks, so it reads
    // one contiguous eighth of every contribution row (6.57-6.59 against 6.52-6.54 TB/s for
    // every eighth block, alternating processes on one box)
    int64_t b = xcd_contiguous(blockIdx.x, gridDim.x);
    if (s.cut) {
        if (b == 0) {
            // the cut tile: lanes with 8 outputs take the vector path, then the last
            // len % 8 outputs one lane each
            const int64_t t = a.len / kTile;
            const int64_t j0 = t * kTile + 8 * static_cast<int64_t>(threadIdx.x);
            if (j0 + 8 <= a.len) reduce_lane<kPre, kLdWord, kHybrid, kAccum, false>(a, j0);
            const int64_t j = (a.len & ~int64_t{7}) + threadIdx.x;
            if (j < a.len) reduce_one<kPre, kHybrid, kAccum>(a, j);
            return;
        }
        --b;
    }
    if (b < s.n_single) {
        reduce_lane<kPre, kLdWord, kHybrid, kAccum, true>(
            a, (s.t_first + b) * kTile + 8 * static_cast<int64_t>(threadIdx.x));
        return;
    }
    sweep_wave<kPre, kAccum, kHybrid, kV, kA>(a, s.t_first + s.n_single + (b - s.n_single) * kV);
}

// ---------------------------------------------------------------------------
// local gradient accumulation (no communication): acc = (init ? 0 : acc) + fp32(g)
// ---------------------------------------------------------------------------
// One block of 8 * kThreads elements per workgroup, 512 per wave.  Each lane reads 8
// consecutive bf16 with one 16-byte load (1 KiB per wave instruction), and the wave's fp32
// accumulator with two 16-byte loads and two stores that each cover 1 KiB contiguous: in half
// h, lane l takes elements 256h + 4l .. 256h + 4l + 3, whose bf16 lane 32h + l/2 holds
// (exchanged across lanes with ds_bpermute, no LDS allocation).  Against 8-byte bf16 loads
// with 4 elements per lane (4 per lane and vector, 4 vectors: 6.02-6.07 TB/s over the
// GPT-175B unit's 1.8 G elements) this measured 6.32-6.34 TB/s; with 16-byte fp32 accesses
// at a 32-byte stride instead of the exchange 5.32-5.52.  Grids of 2^15 blocks or more hand
// each XCD runs of kAccXcdChunk blocks.
template <bool kInit, bool kVec>
__global__ __launch_bounds__(kThreads) void accumulate_kernel(const uint16_t* __restrict__ g,
                                                              float* __restrict__ acc,
                                                              int64_t len) {
    constexpr int64_t kPerBlk = static_cast<int64_t>(kThreads) * 8;
    const uint32_t blk = gridDim.x >= kXcdMinTiles
                             ? xcd_chunked<kAccXcdChunk>(blockIdx.x, gridDim.x)
                             : blockIdx.x;
    const int64_t base = static_cast<int64_t>(blk) * kPerBlk;
    if (kVec && base + kPerBlk <= len) {
        const int lane = threadIdx.x & 63;
        const int64_t wb = base + 512 * static_cast<int64_t>(threadIdx.x >> 6);
        const u4 x = ldu4w(g + wb + 8 * lane);
        f4 y[2];
        if constexpr (!kInit) {
            y[0] = ld4(acc + wb + 4 * lane);
            y[1] = ld4(acc + wb + 256 + 4 * lane);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int src = 32 * h + (lane >> 1);
            const uint32_t a0 = __shfl(x[0], src, 64), a1 = __shfl(x[1], src, 64);
            const uint32_t b0 = __shfl(x[2], src, 64), b1 = __shfl(x[3], src, 64);
            const uint32_t w0 = (lane & 1) ? b0 : a0, w1 = (lane & 1) ? b1 : a1;
            const f4 w = {__builtin_bit_cast(float, w0 << 16), __builtin_bit_cast(float, w0 & 0xFFFF0000u),
                          __builtin_bit_cast(float, w1 << 16), __builtin_bit_cast(float, w1 & 0xFFFF0000u)};
            f4 r;
            if constexpr (kInit) {
                r = w;
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) r[q] = y[h][q] + w[q];
            }
            // device-scope nt buffer stores: 2,809-2,817 us against 2,820-2,836 with nt
            // global stores over the GPT-175B unit's L (four processes on two boxes)
            bst4<kTileStoreCpol>(block_rsrc(acc + wb, 2048), 4 * (256 * h + 4 * lane), r);
        }
        return;
    }
    for (int e = 0; e < 8; ++e) {
        const int64_t j = base + static_cast<int64_t>(e) * kThreads + threadIdx.x;
        if (j < len) {
            const float w = __builtin_bit_cast(float, static_cast<uint32_t>(g[j]) << 16);
            acc[j] = kInit ? w : acc[j] + w;
        }
    }
}

// ---------------------------------------------------------------------------
// AdamW
// ---------------------------------------------------------------------------
struct AdamArgs {
    float* p;
    const float* g;
    float* m;
    float* v;
    uint16_t* pb;
    int64_t len;
    AdamScalars s;
};

__device__ __forceinline__ void adam1(float& p, float g, float& m, float& v, const AdamScalars& s) {
    p = p * s.decay;
    m = s.b1 * m + s.omb1 * g;
    const float gg = g * g;
    v = s.b2 * v + s.omb2 * gg;
    const float den = sqrtf(v) / s.bc2s + s.eps;
    p = p - s.step_size * (m / den);
}

__device__ __forceinline__ void adam_one(const AdamArgs& a, int64_t j) {
    float p = a.p[j], m = a.m[j], v = a.v[j];
    adam1(p, a.g[j], m, v, a.s);
    a.p[j] = p;
    a.m[j] = m;
    a.v[j] = v;
    if (a.pb) a.pb[j] = to_bf16(p);
}

// One tile of kAdamThreads * 8 elements per workgroup; lane l owns vectors l and
// l + kAdamThreads (4 elements each) of every array.
template <bool kVec, bool kBf16>
// The arrays and the length are scalar arguments, so they arrive preloaded in scalar registers;
// the per-step scalars follow as a struct (read after the loads are issued).
__global__ __launch_bounds__(kAdamThreads) void adamw_kernel(float* p_, const float* g_, float* m_,
                                                             float* v_, uint16_t* pb_, int64_t len,
                                                             AdamScalars sc) {
    const AdamArgs a{p_, g_, m_, v_, pb_, len, sc};
    constexpr int64_t kPerBlk = static_cast<int64_t>(kAdamThreads) * 8;
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kPerBlk;
    if constexpr (kVec) {
        if (base + kPerBlk <= a.len) {
            f4 p[2], g[2], m[2], v[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int64_t o = base + 4 * (threadIdx.x + h * kAdamThreads);
                p[h] = *reinterpret_cast<const f4*>(a.p + o);
                g[h] = *reinterpret_cast<const f4*>(a.g + o);
                m[h] = *reinterpret_cast<const f4*>(a.m + o);
                v[h] = *reinterpret_cast<const f4*>(a.v + o);
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float pp = p[h][q], mm = m[h][q], vv = v[h][q];
                    adam1(pp, g[h][q], mm, vv, a.s);
                    p[h][q] = pp;
                    m[h][q] = mm;
                    v[h][q] = vv;
                }
            }
            const auto rp = block_rsrc(a.p + base, kPerBlk * 4), rm = block_rsrc(a.m + base, kPerBlk * 4),
                       rv = block_rsrc(a.v + base, kPerBlk * 4);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int o = 16 * (threadIdx.x + h * kAdamThreads);
                bst4<kAdamStoreCpol>(rp, o, p[h]);
                bst4<kAdamStoreCpol>(rm, o, m[h]);
                bst4<kAdamStoreCpol>(rv, o, v[h]);
                if constexpr (kBf16)
                    bst2<kAdamStoreCpol>(block_rsrc(a.pb + base, kPerBlk * 2), o / 2,
                                         u2{pack_bf16x2(p[h][0], p[h][1]), pack_bf16x2(p[h][2], p[h][3])});
            }
            return;
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int64_t j = base + static_cast<int64_t>(e) * kAdamThreads + threadIdx.x;
        if (j < a.len) adam_one(a, j);
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
bool aligned_to(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Grid of `tiles` workgroups, one tile each (checked < 2^31 by the callers).
dim3 grid_of(int64_t tiles) { return dim3(static_cast<unsigned>(std::max<int64_t>(1, tiles))); }

// Launch with the smallest table that holds the launch's segments.
template <typename SrcT, typename DstT, int kCap>
void launch_table(const SegTable<kMaxSegs>& full, bool general, uint64_t tiles, hipStream_t stream) {
    SegTable<kCap> t{};
    t.ntiles = full.ntiles;
    t.nseg = full.nseg;
    t.xcd_runs = full.xcd_runs;
    uint32_t hot = 0;
    for (int i = 0; i < kCap; ++i) t.start[i] = 0xFFFFFFFFu;
    for (uint32_t i = 0; i < full.nseg; ++i) {
        t.seg[i] = full.seg[i];
        t.start[i] = full.seg[i].tile0;
        const uint32_t end = i + 1 < full.nseg ? full.seg[i + 1].tile0 : full.ntiles;
        if (end - full.seg[i].tile0 > t.hot_tiles) {
            t.hot_tiles = end - full.seg[i].tile0;
            hot = i;
        }
    }
    t.hot = full.seg[hot];
    const DevSeg& h = t.hot;
    if (general)
        hipLaunchKernelGGL((segcopy_kernel<SrcT, DstT, true, kCap>), grid_of(tiles), dim3(kThreads), 0,
                           stream, t.ntiles, t.xcd_runs, t.hot_tiles, h.tile0, h.src, h.dst, h.blk_n,
                           h.last_n, h.nblk, h.tiles_per_blk, t);
    else
        hipLaunchKernelGGL((segcopy_kernel<SrcT, DstT, false, kCap>), grid_of(tiles), dim3(kThreads), 0,
                           stream, t.ntiles, t.xcd_runs, t.hot_tiles, h.tile0, h.src, h.dst, h.blk_n,
                           h.last_n, h.nblk, h.tiles_per_blk, t);
}

template <typename SrcT, typename DstT>
hipError_t launch_segcopy_t(const std::vector<CopySeg>& segs, hipStream_t stream) {
    constexpr int64_t kTile = tile_elems<SrcT, DstT>();
    constexpr uintptr_t kDstAlign = Cp<SrcT, DstT>::kDstAlign;
    size_t i = 0;
    while (i < segs.size()) {
        SegTable<kMaxSegs> t{};
        uint64_t tiles = 0;
        bool general = false;
        for (; i < segs.size() && t.nseg < static_cast<uint32_t>(kMaxSegs); ++i) {
            const CopySeg& c = segs[i];
            if (c.nblk <= 0 || c.blk_n <= 0) continue;
            DevSeg& d = t.seg[t.nseg++];
            d.src = c.src;
            d.dst = c.dst;
            d.blk_n = c.blk_n;
            d.last_n = c.last_n;
            d.src_stride = c.src_stride;
            d.dst_stride = c.dst_stride;
            const uint64_t tpb = static_cast<uint64_t>((c.blk_n + kTile - 1) / kTile);
            const uint64_t seg_tiles = tpb * static_cast<uint64_t>(c.nblk);
            if (c.nblk > 0xFFFFFFFFll || tpb > 0xFFFFFFFFull || tiles + seg_tiles > 0x7FFFFFFFull)
                return hipErrorInvalidValue;
            d.nblk = static_cast<uint32_t>(c.nblk);
            d.tiles_per_blk = static_cast<uint32_t>(tpb);
            d.tile0 = static_cast<uint32_t>(tiles);
            tiles += seg_tiles;
            // the vector path needs every block start aligned (tiles are multiples of 16 B)
            bool ok = aligned_to(c.dst, kDstAlign) &&
                      (c.nblk == 1 || (c.dst_stride * sizeof(DstT)) % kDstAlign == 0);
            if (c.src)
                ok = ok && aligned_to(c.src, 16) &&
                     (c.nblk == 1 || (c.src_stride * sizeof(SrcT)) % 16 == 0);
            general = general || !ok;
        }
        if (t.nseg == 0) continue;
        t.ntiles = static_cast<uint32_t>(tiles);
        t.xcd_runs = tiles >= kXcdMinTiles ? 1u : 0u;
        if (t.nseg <= 1) launch_table<SrcT, DstT, 1>(t, general, tiles, stream);
        else if (t.nseg <= 4) launch_table<SrcT, DstT, 4>(t, general, tiles, stream);
        else if (t.nseg <= 8) launch_table<SrcT, DstT, 8>(t, general, tiles, stream);
        else if (t.nseg <= 16) launch_table<SrcT, DstT, 16>(t, general, tiles, stream);
        else launch_table<SrcT, DstT, kMaxSegs>(t, general, tiles, stream);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int kPre, int kLd>
void launch_reduce_mode(const ReduceArgs& a, bool hybrid, bool accum, dim3 grid,
                        hipStream_t stream) {
    const dim3 block(kReduceThreads);
    const unsigned lds = kReduceLdsCap;  // residency cap (unused LDS)
    if (hybrid) {
        if (accum) hipLaunchKernelGGL((reduce_kernel<kPre, kLd, true, true>), grid, block, lds, stream, a);
        else hipLaunchKernelGGL((reduce_kernel<kPre, kLd, true, false>), grid, block, lds, stream, a);
    } else {
        if (accum) hipLaunchKernelGGL((reduce_kernel<kPre, kLd, false, true>), grid, block, lds, stream, a);
        else hipLaunchKernelGGL((reduce_kernel<kPre, kLd, false, false>), grid, block, lds, stream, a);
    }
}

// ---------------------------------------------------------------------------
// sharded gradient scaler: g *= inv_scale, flag non-finite inputs
// ---------------------------------------------------------------------------
// In place: plain loads and nt stores (as AdamW).  A wave that saw a non-finite
// input has one lane store 1.0f into the flag (vector store; every writer stores
// the same value, so concurrent stores agree).  found == nullptr: scaling only.
template <bool kVec, int kV>
__global__ __launch_bounds__(kThreads) void unscale_kernel(float* __restrict__ g, int64_t len,
                                                           float inv, float* __restrict__ found) {
    constexpr int64_t kPerBlk = static_cast<int64_t>(kThreads) * 4 * kV;
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kPerBlk;
    bool bad = false;
    if (kVec && base + kPerBlk <= len) {
        f4 x[kV];
#pragma unroll
        for (int h = 0; h < kV; ++h) x[h] = *reinterpret_cast<const f4*>(g + base + 4 * (threadIdx.x + h * kThreads));
#pragma unroll
        for (int h = 0; h < kV; ++h) {
            f4 y;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                bad = bad || !__builtin_isfinite(x[h][q]);
                y[q] = x[h][q] * inv;
            }
            st4(g + base + 4 * (threadIdx.x + h * kThreads), y);
        }
    } else {
        for (int e = 0; e < 4 * kV; ++e) {
            const int64_t j = base + static_cast<int64_t>(e) * kThreads + threadIdx.x;
            if (j < len) {
                const float x = g[j];
                bad = bad || !__builtin_isfinite(x);
                g[j] = x * inv;
            }
        }
    }
    if (found == nullptr) return;  // scaling only (uniform)
    const uint64_t mask = __ballot(bad);
    if (mask != 0 && (threadIdx.x & 63) == static_cast<unsigned>(__builtin_ctzll(mask))) *found = 1.0f;
}

// ---------------------------------------------------------------------------
// per-parameter sums of squares of a gradient shard, in binary64
// ---------------------------------------------------------------------------
constexpr int kSqThreads = 256;
constexpr int kSqPerThread = 16;  // four 4-float vectors
constexpr int64_t kSqTile = static_cast<int64_t>(kSqThreads) * kSqPerThread;

struct SqRun {
    int64_t offset;   // first element of the run in the shard
    int64_t n;        // elements
    uint32_t tile0;   // first workspace slot
    uint32_t ntiles;
    int32_t out;      // parameter index
    int32_t unused;
};
// A launch's runs, passed by value in the kernel-argument block: a table of kCap entries (1, 4,
// 8, 16 or kMaxSegs), with the runs' first tiles in one array next to the header and a copy of the
// run with the most tiles, for the lookup of the copy engine's segment table.
template <int kCap>
struct SqTable {
    const float* g;
    double* partial;
    double* out;
    uint32_t nrun;
    uint32_t unused;
    uint32_t start[kCap];  // run[i].tile0; 0xFFFFFFFF past nrun
    SqRun hot;             // the run with the most tiles (stage 1 takes it as scalar arguments)
    SqRun run[kCap];
};
static_assert(sizeof(SqTable<kMaxSegs>) <= 4096 - 64, "run table and scalar arguments must fit one kernel argument block");

// Block sum of one double per thread, in a fixed order: a shuffle tree inside each
// wave, then the waves' sums in wave order.  Returns the sum in thread 0.
__device__ __forceinline__ double block_sum(double v, double* lds) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = v + __shfl_down(v, o, 64);
    if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = v;
    __syncthreads();
    double s = 0.0;
    if (threadIdx.x == 0)
        for (int w = 0; w < kSqThreads / 64; ++w) s = s + lds[w];
    return s;
}

// Stage 1: one tile of one run per workgroup -> one partial sum.  Each lane adds
// the squares of its 16 elements in order (a binary32 square is exact in binary64).
// Loads need dword alignment only (runs start at any element).
__device__ __forceinline__ void sq_tile(const float* g0, double* partial, const SqRun& r,
                                        uint32_t tile, double* lds) {
    const int64_t e0 = static_cast<int64_t>(tile - r.tile0) * kSqTile;
    const int64_t n = min(kSqTile, r.n - e0);
    const float* g = g0 + r.offset + e0;
    double acc = 0.0;
    if (n == kSqTile) {
        f4 x[kSqPerThread / 4];
#pragma unroll
        for (int h = 0; h < kSqPerThread / 4; ++h) x[h] = ld4w(g + 4 * (threadIdx.x + h * kSqThreads));
#pragma unroll
        for (int h = 0; h < kSqPerThread / 4; ++h)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const double d = static_cast<double>(x[h][q]);
                acc = acc + d * d;
            }
    } else {
        for (int64_t e = threadIdx.x; e < n; e += kSqThreads) {
            const double d = static_cast<double>(g[e]);
            acc = acc + d * d;
        }
    }
    const double s = block_sum(acc, lds);
    if (threadIdx.x == 0) partial[tile] = s;
}

// The tile's run is found as the copy engine finds a tile's segment: the run with the most
// tiles comes as scalar arguments ahead of the table (preloaded in scalar registers), and only
// tiles outside that run load the runs' first tiles (together, pinned by the empty asm
// statements) and count those that start at or before them.
template <int kCap>
__global__ __launch_bounds__(kSqThreads) void sqnorm_partial_kernel(
    const float* g, double* partial, int64_t hot_offset, int64_t hot_n, uint32_t hot_tile0,
    uint32_t hot_ntiles, SqTable<kCap> t) {
    __shared__ double lds[kSqThreads / 64];
    const uint32_t tile = blockIdx.x;
    if (kCap == 1 || tile - hot_tile0 < hot_ntiles) {
        SqRun z;
        z.offset = hot_offset;
        z.n = hot_n;
        z.tile0 = hot_tile0;
        z.ntiles = hot_ntiles;
        z.out = 0;
        z.unused = 0;
        sq_tile(g, partial, z, tile, lds);
        return;
    }
    if constexpr (kCap <= 8) {
#pragma unroll
        for (int i = 1; i < kCap; ++i) asm volatile("" ::"s"(t.start[i]));
    }
    uint32_t k = 0;
#pragma unroll
    for (int i = 1; i < kCap; ++i) k += t.start[i] <= tile ? 1u : 0u;
    sq_tile(g, partial, t.run[k], tile, lds);
}

// Stage 2: one workgroup per run sums its partials in a fixed order (lane order
// within strided passes, then the block tree) and writes the parameter's result.
// Each lane loads up to kSqFinalAhead of its partials before adding them (in the same
// order), so their round trips overlap instead of following one another.
constexpr int kSqFinalAhead = 8;
__global__ __launch_bounds__(kSqThreads) void sqnorm_final_kernel(SqTable<kMaxSegs> t) {
    __shared__ double lds[kSqThreads / 64];
    const SqRun& r = t.run[blockIdx.x];
    const double* p = t.partial + r.tile0;
    double acc = 0.0;
    uint32_t i = threadIdx.x;
    for (; i + (kSqFinalAhead - 1) * kSqThreads < r.ntiles; i += kSqFinalAhead * kSqThreads) {
        double v[kSqFinalAhead];
#pragma unroll
        for (int u = 0; u < kSqFinalAhead; ++u) v[u] = p[i + u * kSqThreads];
#pragma unroll
        for (int u = 0; u < kSqFinalAhead; ++u) acc = acc + v[u];
    }
    for (; i < r.ntiles; i += kSqThreads) acc = acc + p[i];
    const double s = block_sum(acc, lds);
    if (threadIdx.x == 0) t.out[r.out] = s;
}

}  // namespace

hipError_t launch_segcopy(const std::vector<CopySeg>& segs, Pipe pipe, hipStream_t stream) {
    switch (pipe) {
        case Pipe::kF32toF32: return launch_segcopy_t<float, float>(segs, stream);
        case Pipe::kF32toBF16: return launch_segcopy_t<float, uint16_t>(segs, stream);
        case Pipe::kBF16toBF16: return launch_segcopy_t<uint16_t, uint16_t>(segs, stream);
    }
    return hipErrorInvalidValue;
}

// Workgroups of a reduce_sweep_kernel instantiation resident at once on the current device
// (occupancy per CU times CUs), queried once per device; 0 if unknown.
constexpr int kMaxDevices = 64;
template <int kPre, bool kAccum, bool kHybrid, int kV, int kA>
int64_t sweep_capacity() {
    static std::atomic<int64_t> cap[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    int64_t c = cap[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &per_cu, reinterpret_cast<const void*>(&reduce_sweep_kernel<kPre, kAccum, kHybrid, kV, kA>),
                64, 0) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        c = int64_t{per_cu} * cus;
        cap[dev].store(c > 0 ? c : -1, std::memory_order_relaxed);
    }
    return c > 0 ? c : 0;
}

// The sweep over one launch's ranks, one kernel launch per run of plan_sweep_runs (runs whose
// grids are resident at once), in output order; *err gets the first launch error.  Returns
// false, having launched nothing, when the output holds fewer whole tiles than a sweep wave
// or the occupancy is unknown.
template <int kPre, bool kAccum, bool kHybrid, int kV, int kA>
bool try_sweep(const ReduceArgs& a, hipStream_t stream, hipError_t* err) {
    constexpr int64_t kTile = 512;
    std::vector<SweepRun> runs;
    if (!plan_sweep_runs(a.len / kTile, a.len % kTile != 0, kV,
                         sweep_capacity<kPre, kAccum, kHybrid, kV, kA>(), &runs))
        return false;
    for (const SweepRun& r : runs) {
        SweepArgs s{};
        s.r = a;
        s.t_first = r.t_first;
        s.cut = r.cut;
        s.n_single = r.n_single;
        hipLaunchKernelGGL((reduce_sweep_kernel<kPre, kAccum, kHybrid, kV, kA>),
                           dim3(static_cast<unsigned>(r.blocks)), dim3(64), 0, stream, s);
        *err = hipGetLastError();
        if (*err != hipSuccess) break;
    }
    return true;
}

// Which shape: the grouped one with two ranks in flight where its runs are long (the flat
// sum as one group that spans every rank: the group's sum is the running sum, carried in and
// out where the flat path carries its total, and the last launch ends the group, whose sum
// then becomes the total as it is, no total having come before it; per output the operations
// and their order are the flat ones).  Otherwise the wide shape for a flat sum and the grouped
// one with one rank in flight for a hybrid one.  rocprofv3, cold cache, in TB/s, flat sums:
// the grouped against the wide shape, 128 ranks over 14.2 M outputs (two runs of 13,825
// tiles) 6.66 against 6.46, over 26.2 M (four runs) 6.54 against 6.28; 64 ranks 6.53 / 6.35
// and 6.35 / 6.19; 32 ranks 6.15 / 6.17 and 5.99 / 5.97; but over 8.4 M outputs, two runs of
// 8,192 tiles, 5.36 against 6.55 at 128 ranks.  Hybrid groups of 8, accumulating, two ranks in
// flight against one, 128 ranks: 3.5 M outputs (one run of 6,912 tiles) 4.85 against 6.52,
// 7.1 M (13,824) 6.63-6.67 against 6.47, 8.4 M (two runs of 8,192) 5.37 against 6.31, 14.2 M
// 6.63-6.65 against 6.50; 256 ranks alike.
template <int kPre, bool kAccum>
bool launch_reduce_sweep_t(const ReduceArgs& a, bool hybrid, hipStream_t stream, hipError_t* err) {
    constexpr int kLong = kGroupSweepLongAhead;
    std::vector<SweepRun> runs;
    if (plan_sweep_runs(a.len / 512, a.len % 512 != 0, kGroupSweepV,
                        sweep_capacity<kPre, kAccum, true, kGroupSweepV, kLong>(), &runs) &&
        runs.back().n_tiles >= kGroupSweepMinRunTiles) {  // the last run is the shortest
        if (hybrid) return try_sweep<kPre, kAccum, true, kGroupSweepV, kLong>(a, stream, err);
        ReduceArgs g = a;
        g.flags = (a.flags & kLast) | ((a.flags & kTIn) ? kSIn : 0u) | ((a.flags & kTOut) ? kSOut : 0u);
        g.carry_s = a.carry_t;
        g.carry_t = nullptr;
        g.pos0 = (a.flags & kTIn) ? 1 : 0;  // a carried-in sum is continued, not restarted
        g.group = g.pos0 + a.nc + ((a.flags & kLast) ? 0 : 1);
        return try_sweep<kPre, kAccum, true, kGroupSweepV, kLong>(g, stream, err);
    }
    if (hybrid) return try_sweep<kPre, kAccum, true, kGroupSweepV, 1>(a, stream, err);
    return try_sweep<kPre, kAccum, false, kSweepV, 1>(a, stream, err);
}

template <int kPre>
bool launch_reduce_sweep(const ReduceArgs& a, bool hybrid, bool accum, hipStream_t stream,
                         hipError_t* err) {
    return accum ? launch_reduce_sweep_t<kPre, true>(a, hybrid, stream, err)
                 : launch_reduce_sweep_t<kPre, false>(a, hybrid, stream, err);
}

template <int kPre>
void launch_reduce_tiles(const ReduceArgs& a, int ld, bool hybrid, bool accum, dim3 grid,
                         hipStream_t stream) {
    if (ld == kLdWord) launch_reduce_mode<kPre, kLdWord>(a, hybrid, accum, grid, stream);
    else if (ld == kLdHalf) launch_reduce_mode<kPre, kLdHalf>(a, hybrid, accum, grid, stream);
    else launch_reduce_mode<kPre, kLdScalar>(a, hybrid, accum, grid, stream);
}

int64_t reduce_workspace_floats(int64_t n_contrib, int64_t len, int64_t group, bool accumulate) {
    if (len <= 0 || n_contrib <= 0) return 0;
    ReducePlan plan;
    plan_reduce(n_contrib, group, accumulate, kMaxContrib, &plan);
    return plan.ws_slots * reduce_ws_pitch(len);
}

hipError_t launch_grad_reduce(const uint16_t* const* contribs, int64_t n_contrib, int64_t len,
                              float pre, float post, int64_t group, bool accumulate, float* out,
                              float* workspace, ReduceKernel kernel, hipStream_t stream) {
    if (len <= 0 || n_contrib <= 0) return hipSuccess;
    // one group of all ranks, or groups of one, are the flat sequential sum
    const bool hybrid = group > 1 && group < n_contrib;
    if (hybrid && n_contrib % group != 0) return hipErrorInvalidValue;
    ReducePlan plan;
    plan_reduce(n_contrib, group, accumulate, kMaxContrib, &plan);
    if (plan.ws_slots > 0 && workspace == nullptr) return hipErrorInvalidValue;
    const int64_t pitch = reduce_ws_pitch(len);
    float* carry_t = plan.t_slot < 0 ? out : workspace + plan.t_slot * pitch;
    float* carry_s = plan.s_slot < 0 ? nullptr : workspace + plan.s_slot * pitch;
    int mode = kPreDiv;
    float rpre = 1.0f;
    if (pre == 1.0f) {
        mode = kPreNone;
    } else {
        int e = 0;
        const float mant = std::frexp(std::fabs(pre), &e);
        rpre = 1.0f / pre;
        if (mant == 0.5f && std::isnormal(rpre) && rpre * pre == 1.0f) mode = kPreRecip;
    }
    // vector path when the output (and the workspace) is 16-byte aligned; contributions
    // only 2-byte aligned are read one element early and shifted
    bool all4 = true;
    for (int64_t r = 0; r < n_contrib; ++r) all4 = all4 && aligned_to(contribs[r], 4);
    const bool vec_out = aligned_to(out, 16) && (workspace == nullptr || aligned_to(workspace, 16));
    const int ld = !vec_out ? kLdScalar : all4 ? kLdWord : kLdHalf;
    const int64_t per_blk = static_cast<int64_t>(kReduceThreads) * 8;
    const int64_t blocks = (len + per_blk - 1) / per_blk;
    if (blocks > 0x7FFFFFFFll) return hipErrorInvalidValue;
    const int64_t whole_tiles = len / per_blk;
    for (const ReduceLaunch& l : plan.launches) {
        ReduceArgs a{};
        a.nc = static_cast<int32_t>(l.nc);
        for (int32_t r = 0; r < a.nc; ++r) a.c[r] = contribs[l.r0 + r];
        a.out = out;
        a.carry_t = carry_t;
        a.carry_s = carry_s;
        a.len = len;
        a.group = static_cast<int32_t>(hybrid ? group : n_contrib);
        a.pos0 = static_cast<int32_t>(l.pos0);
        a.flags = l.flags;
        a.pre = pre;
        a.rpre = rpre;
        a.post = post;
        // the row-major sweep where its loads apply (whole dwords); by default only where it
        // measured faster: many ranks in the launch and a long output
        const bool sweep = ld == kLdWord && kernel != ReduceKernel::kTiles &&
                           (kernel == ReduceKernel::kSweep ||
                            (a.nc >= kSweepMinRanks && whole_tiles >= kSweepMinTiles));
        if (sweep) {
            hipError_t swept = hipSuccess;
            bool ran = false;
            if (mode == kPreNone) ran = launch_reduce_sweep<kPreNone>(a, hybrid, accumulate, stream, &swept);
            else if (mode == kPreRecip) ran = launch_reduce_sweep<kPreRecip>(a, hybrid, accumulate, stream, &swept);
            else ran = launch_reduce_sweep<kPreDiv>(a, hybrid, accumulate, stream, &swept);
            if (swept != hipSuccess) return swept;
            if (ran) continue;
        }
        const dim3 grid = grid_of(blocks);
        if (mode == kPreNone) launch_reduce_tiles<kPreNone>(a, ld, hybrid, accumulate, grid, stream);
        else if (mode == kPreRecip) launch_reduce_tiles<kPreRecip>(a, ld, hybrid, accumulate, grid, stream);
        else launch_reduce_tiles<kPreDiv>(a, ld, hybrid, accumulate, grid, stream);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_grad_accumulate(const uint16_t* grad, float* acc, int64_t len, bool init,
                                  hipStream_t stream) {
    if (len <= 0) return hipSuccess;
    const int64_t per_blk = static_cast<int64_t>(kThreads) * 8;
    const int64_t blocks = (len + per_blk - 1) / per_blk;
    if (blocks > 0x7FFFFFFFll) return hipErrorInvalidValue;
    // 16-byte bf16 loads need dword alignment only
    const bool vec = aligned_to(grad, 4) && aligned_to(acc, 16);
    const dim3 grid = grid_of(blocks), block(kThreads);
    if (init) {
        if (vec) hipLaunchKernelGGL((accumulate_kernel<true, true>), grid, block, 0, stream, grad, acc, len);
        else hipLaunchKernelGGL((accumulate_kernel<true, false>), grid, block, 0, stream, grad, acc, len);
    } else {
        if (vec) hipLaunchKernelGGL((accumulate_kernel<false, true>), grid, block, 0, stream, grad, acc, len);
        else hipLaunchKernelGGL((accumulate_kernel<false, false>), grid, block, 0, stream, grad, acc, len);
    }
    return hipGetLastError();
}

hipError_t launch_adamw(float* p, const float* g, float* m, float* v, uint16_t* pb, int64_t len,
                        const AdamScalars& s, hipStream_t stream) {
    if (len <= 0) return hipSuccess;
    const bool vec = aligned_to(p, 16) && aligned_to(g, 16) && aligned_to(m, 16) &&
                     aligned_to(v, 16) && (pb == nullptr || aligned_to(pb, 8));
    const int64_t per_blk = static_cast<int64_t>(kAdamThreads) * 8;
    const int64_t blocks = (len + per_blk - 1) / per_blk;
    if (blocks > 0x7FFFFFFFll) return hipErrorInvalidValue;
    if (vec) {
        if (pb)
            hipLaunchKernelGGL((adamw_kernel<true, true>), grid_of(blocks), dim3(kAdamThreads), 0,
                               stream, p, g, m, v, pb, len, s);
        else
            hipLaunchKernelGGL((adamw_kernel<true, false>), grid_of(blocks), dim3(kAdamThreads),
                               0, stream, p, g, m, v, pb, len, s);
    } else {
        hipLaunchKernelGGL((adamw_kernel<false, false>), grid_of(blocks), dim3(kAdamThreads), 0,
                           stream, p, g, m, v, pb, len, s);
    }
    return hipGetLastError();
}

hipError_t launch_grad_unscale(float* g, int64_t len, float inv_scale, float* found_inf,
                               hipStream_t stream) {
    if (len <= 0) return hipSuccess;
    const bool longer = len >= kUnscaleLongLen;
    const int64_t per_blk = static_cast<int64_t>(kThreads) * 4 * (longer ? kUnscaleVpl : kUnscaleShortVpl);
    const int64_t blocks = (len + per_blk - 1) / per_blk;
    if (blocks > 0x7FFFFFFFll) return hipErrorInvalidValue;
    const dim3 grid = grid_of(blocks), block(kThreads);
    const bool vec = aligned_to(g, 16);
    if (longer) {
        if (vec)
            hipLaunchKernelGGL((unscale_kernel<true, kUnscaleVpl>), grid, block, 0, stream, g, len, inv_scale, found_inf);
        else
            hipLaunchKernelGGL((unscale_kernel<false, kUnscaleVpl>), grid, block, 0, stream, g, len, inv_scale, found_inf);
    } else {
        if (vec)
            hipLaunchKernelGGL((unscale_kernel<true, kUnscaleShortVpl>), grid, block, 0, stream, g, len, inv_scale, found_inf);
        else
            hipLaunchKernelGGL((unscale_kernel<false, kUnscaleShortVpl>), grid, block, 0, stream, g, len, inv_scale, found_inf);
    }
    return hipGetLastError();
}

// Scratch for callers that cannot allocate device memory: the binary64 partial sums of the
// sums of squares, one fixed array per GPU (a global of this code object, so every device the
// library runs on holds its own copy until the process ends).  Only its device address is
// used on the host; the name here is a host-side stand-in.
constexpr int64_t kScratchDoubles = int64_t{1} << 18;  // 2 MiB
static __device__ __align__(256) double scratch[kScratchDoubles];

int64_t sqnorm_scratch_doubles() { return kScratchDoubles; }

hipError_t sqnorm_scratch(double** out) {
    // the address of the current device's copy, looked up on the first call on that device
    static std::atomic<double*> addr[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    double* p = addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        void* q = nullptr;
        e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (q == nullptr) return hipErrorInvalidSymbol;
        p = static_cast<double*>(q);
        addr[dev].store(p, std::memory_order_release);  // racing first calls store the same address
    }
    *out = p;
    return hipSuccess;
}

namespace {

// Stage 1 over the non-empty runs of `busy` (first tile 0), with the smallest table that holds
// them.
template <int kCap>
void launch_sq_partial(const SqTable<kMaxSegs>& busy, uint32_t tiles, hipStream_t stream) {
    SqTable<kCap> t{};
    t.g = busy.g;
    t.partial = busy.partial;
    t.out = busy.out;
    t.nrun = busy.nrun;
    uint32_t hot = 0;
    for (int i = 0; i < kCap; ++i) t.start[i] = 0xFFFFFFFFu;
    for (uint32_t i = 0; i < busy.nrun; ++i) {
        t.run[i] = busy.run[i];
        t.start[i] = busy.run[i].tile0;
        if (busy.run[i].ntiles > busy.run[hot].ntiles) hot = i;
    }
    t.hot = busy.run[hot];
    const SqRun& h = t.hot;
    hipLaunchKernelGGL((sqnorm_partial_kernel<kCap>), grid_of(tiles), dim3(kSqThreads), 0, stream,
                       t.g, t.partial, h.offset, h.n, h.tile0, h.ntiles, t);
}

}  // namespace

int64_t sqnorm_tiles(const std::vector<ParamRun>& runs) {
    int64_t n = 0;
    for (const ParamRun& r : runs) n += (r.n + kSqTile - 1) / kSqTile;
    return n;
}

hipError_t launch_grad_sqnorm(const float* g, const std::vector<ParamRun>& runs, double* partial,
                              double* out, hipStream_t stream) {
    // Runs go kMaxSegs to a launch pair; workspace slots are numbered across all runs.
    int64_t slot = 0;
    for (size_t i0 = 0; i0 < runs.size(); i0 += kMaxSegs) {
        const size_t i1 = std::min(runs.size(), i0 + static_cast<size_t>(kMaxSegs));
        SqTable<kMaxSegs> all{}, busy{};  // every run of the batch / only the non-empty ones
        all.g = busy.g = g;
        all.partial = busy.partial = partial;
        all.out = busy.out = out;
        uint32_t tiles = 0;
        for (size_t i = i0; i < i1; ++i) {
            const int64_t nt = (runs[i].n + kSqTile - 1) / kSqTile;
            if (slot + nt > 0xFFFFFFFFll) return hipErrorInvalidValue;
            SqRun r{runs[i].offset, runs[i].n, static_cast<uint32_t>(slot),
                    static_cast<uint32_t>(nt), static_cast<int32_t>(i), 0};
            all.run[all.nrun++] = r;
            if (nt > 0) busy.run[busy.nrun++] = r;
            slot += nt;
            tiles += static_cast<uint32_t>(nt);
        }
        // tiles of this batch are workspace slots [first, first + tiles): stage 1 uses
        // the tile index relative to the batch's first slot
        if (busy.nrun > 0) {
            const uint32_t first = busy.run[0].tile0;
            for (uint32_t j = 0; j < busy.nrun; ++j) busy.run[j].tile0 -= first;
            busy.partial = partial + first;
            if (busy.nrun == 1) launch_sq_partial<1>(busy, tiles, stream);
            else if (busy.nrun <= 4) launch_sq_partial<4>(busy, tiles, stream);
            else if (busy.nrun <= 8) launch_sq_partial<8>(busy, tiles, stream);
            else if (busy.nrun <= 16) launch_sq_partial<16>(busy, tiles, stream);
            else launch_sq_partial<kMaxSegs>(busy, tiles, stream);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL(sqnorm_final_kernel, dim3(all.nrun), dim3(kSqThreads), 0, stream, all);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace fsdp

