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
//     faster than the default-scope ones (the in-place kernels keep the latter).
// The kernels:
//   - segcopy: one engine for flatten (FSDP1 and FSDP2), copy-out, the cast and
//     the bf16 copies.  The host planner turns the layout into a short table of
//     (src, dst, length[, block stride]) segments passed in the kernel argument
//     block; each workgroup takes one tile of one segment (the tile -> segment
//     lookup is a wave-uniform binary search on scalar registers), so no lane
//     ever searches and every tile is a straight streaming copy.  Launches of
//     2^18 tiles or more hand each XCD runs of 256 consecutive tiles.  When source
//     and destination are not 16-byte co-aligned, a scalar head aligns the
//     destination and the source is read in place with dword-aligned 16-byte
//     loads; only a bf16 source at an odd element offset is staged through LDS.
//   - grad_reduce: each lane owns 8 consecutive outputs and loads their 8 bf16
//     from 8 ranks at a time (one 16-byte load each, or a shifted pair when a
//     contribution is only 2-byte aligned) before adding them in rank order;
//     whole tiles swap halves across lanes so each store writes 1 KiB; the tile
//     the output's end cuts runs first, its last len % 8 outputs one per lane.
//     From 32 ranks and 12,288 whole tiles on, a row-major sweep instead: each
//     wave holds 16 tiles' sums and walks the ranks in order, the grid sized to be
//     resident at once (each XCD one contiguous run of waves), so HBM serves a few
//     contribution rows at a time.
//   - adamw: elementwise over 8 elements per lane, 128-bit loads and stores.
//     Its state is read and written back in place: plain loads measure faster
//     than nt ones (6.5 vs 5.6 TB/s), and nt stores put its writes in HBM within
//     its own launch (plain stores leave them dirty in the 256 MB Infinity Cache,
//     which costs the next kernels, or AdamW itself once they outgrow it).
//   - accumulate, unscale: elementwise in place, four 16-byte vectors per lane
//     (a long accumulation hands each XCD runs of 64 blocks).
//   - sqnorm: per-parameter sums of squares in binary64, one tile per workgroup
//     into a workspace, then one workgroup per parameter, in fixed orders.
// Every binary32 step is one IEEE operation, in the order the CPU oracle fixes;
// contraction into FMA is disabled for this file.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
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

// Launch shapes (tuned on MI355X; each can be overridden with -D for tuning builds).
#ifndef FSDP_COPY_THREADS
#define FSDP_COPY_THREADS 256
#endif
#ifndef FSDP_F32_VPL
#define FSDP_F32_VPL 1      // 4-element vectors per lane per tile, fp32 output
#endif
#ifndef FSDP_BF16_VPL
#define FSDP_BF16_VPL 2     // 4-element vectors per lane per tile, bf16 output
#endif
#ifndef FSDP_B16_VPL
#define FSDP_B16_VPL 1      // 8-element vectors per lane per tile, bf16 -> bf16
#endif
#ifndef FSDP_REDUCE_THREADS
#define FSDP_REDUCE_THREADS 64
#endif
#ifndef FSDP_REDUCE_AHEAD
#define FSDP_REDUCE_AHEAD 8
#endif
#ifndef FSDP_SWEEP_MIN_RANKS
#define FSDP_SWEEP_MIN_RANKS 32  // the reduction sweeps ranks row-major from this many on
#endif
#ifndef FSDP_SWEEP_V
#define FSDP_SWEEP_V 16          // whole tiles a sweep wave holds (8, 12, 16: 6.23, 6.36, 6.53 TB/s)
#endif
#ifndef FSDP_SWEEP_MIN_TILES
#define FSDP_SWEEP_MIN_TILES 12288  // and from this many whole 512-output tiles on
#endif
#ifndef FSDP_TILE_STORE_CPOL
// Whole-tile stores of the copies: 0 = global nt stores, else the cache-policy operand of
// buffer stores (2 nt, 16 sc1 = device scope, 18 both).  Device-scope nt stores (18) against
// global nt stores on the GPT-175B unit (HIP events, alternating processes on one box):
// copy-out 6.48-6.50 vs 6.44-6.45 TB/s, rank flatten 5.26-5.39 vs 4.87-4.94, bf16 copies
// 6.65-6.69 vs 6.24-6.30; buffer nt stores (2) matched the global ones, and sc1 alone slowed
// the next kernel (AdamW) by a third.
#define FSDP_TILE_STORE_CPOL 18
#endif
#ifndef FSDP_XCD_MIN_TILES
// From this many tiles (workgroups) on, a copy hands each of the eight XCDs runs of
// FSDP_XCD_CHUNK consecutive tiles instead of every eighth tile.  GPT-175B copy-out (885k
// tiles), one box, alternating processes: dispatch order 6.46-6.49 TB/s, one contiguous run
// per XCD 6.61-6.65, runs of 64 / 128 / 256 / 512 tiles 6.65-6.67 / 6.76 / 6.76-6.78 /
// 6.62-6.63.  One run per XCD made 64-256 MB copies 3-7% slower; runs of 256 left every
// size from 8 MB to 1 GB as fast as the dispatch order.
#define FSDP_XCD_MIN_TILES (1u << 18)
#endif
#ifndef FSDP_XCD_CHUNK
#define FSDP_XCD_CHUNK 256u
#endif
#ifndef FSDP_ACC_XCD_CHUNK
// The in-place local accumulation over all L (442k blocks) takes runs of 64 blocks per XCD:
// 6.09-6.12 vs 6.01-6.08 TB/s in dispatch order; runs of 16 / 32 / 256 blocks 5.88-5.95 /
// 5.96-6.01 / 5.99-6.00, one run per XCD 5.94-5.95 (one box, alternating processes).
#define FSDP_ACC_XCD_CHUNK 64u
#endif
#ifndef FSDP_ACC_VPL
#define FSDP_ACC_VPL 4          // 4-element vectors per lane in the local accumulation (1/2/4: 5.70/5.96/6.07 TB/s)
#endif
#ifndef FSDP_UNSCALE_VPL
#define FSDP_UNSCALE_VPL 4      // 4-element vectors per lane in the gradient unscale
#endif
#ifndef FSDP_ACC_NT
#define FSDP_ACC_NT 1       // local accumulation: nt measured faster (5.9 vs 5.6 TB/s)
#endif
#ifndef FSDP_ADAM_THREADS
#define FSDP_ADAM_THREADS 256
#endif
#ifndef FSDP_ADAM_NT_LOAD
#define FSDP_ADAM_NT_LOAD 0   // AdamW reads p, g, m, v with plain loads
#endif
#ifndef FSDP_ADAM_NT_STORE
#define FSDP_ADAM_NT_STORE 1  // and streams p, m, v back with nt stores
#endif
#ifndef FSDP_ADAM_STORE_CPOL
// AdamW's whole-block stores: 0 = global stores (nt as FSDP_ADAM_NT_STORE says), else buffer
// stores with this cache-policy operand.  Buffer nt stores (2) measured 6.62-6.65 TB/s against
// 6.48-6.55 for global nt stores; device-scope nt stores (18) 5.46-5.59.  Those also slowed
// the in-place accumulation and unscale, which keep global stores.
#define FSDP_ADAM_STORE_CPOL 2
#endif

constexpr int kThreads = FSDP_COPY_THREADS;
constexpr int kMaxSegs = 48;           // segments per launch (kernel-argument budget)
constexpr int kMaxContrib = 128;       // contribution pointers per reduce launch
constexpr int kReduceThreads = FSDP_REDUCE_THREADS;
static_assert(kReduceThreads % 64 == 0, "reduce workgroups are whole wave64s (lane exchange)");
constexpr int kAdamThreads = FSDP_ADAM_THREADS;

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
template <bool kNT>
__device__ __forceinline__ f4 ld4s(const float* p) {
    if constexpr (kNT) return ld4(p);
    else return *reinterpret_cast<const f4*>(p);
}
template <bool kNT>
__device__ __forceinline__ void st4s(float* p, f4 v) {
    if constexpr (kNT) st4(p, v);
    else *reinterpret_cast<f4*>(p) = v;
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
    static constexpr int E = 4, kVpl = FSDP_F32_VPL;
    static constexpr unsigned kDstAlign = 16;  // bytes a vector store needs
    using V = f4;
    __device__ static V load(const float* p) { return ld4(p); }
    __device__ static V loadw(const float* p) { return ld4w(p); }
    __device__ static void put(float* d, V x) { st4(d, x); }
    __device__ static void put_tile(float* d, const V* x) {
#if FSDP_TILE_STORE_CPOL
        const auto r = block_rsrc(d, kThreads * E * kVpl * 4);
#pragma unroll
        for (int u = 0; u < kVpl; ++u)
            bst4<FSDP_TILE_STORE_CPOL>(r, 16 * (threadIdx.x + u * kThreads), x[u]);
#else
#pragma unroll
        for (int u = 0; u < kVpl; ++u) put(d + E * (threadIdx.x + u * kThreads), x[u]);
#endif
    }
    __device__ static void put1(float* d, float x) { *d = x; }
    __device__ static void zero(float* d) { st4(d, f4{0.0f, 0.0f, 0.0f, 0.0f}); }
    __device__ static void zero1(float* d) { *d = 0.0f; }
};
template <> struct Cp<float, uint16_t> {
    static constexpr int E = 4, kVpl = FSDP_BF16_VPL;
    static constexpr unsigned kDstAlign = 8;
    using V = f4;
    __device__ static V load(const float* p) { return ld4(p); }
    __device__ static V loadw(const float* p) { return ld4w(p); }
    __device__ static void put(uint16_t* d, V x) {
        stu2(d, u2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])});
    }
    __device__ static void put_tile(uint16_t* d, const V* x) {
#if FSDP_TILE_STORE_CPOL
        const auto r = block_rsrc(d, kThreads * E * kVpl * 2);
#pragma unroll
        for (int u = 0; u < kVpl; ++u)
            bst2<FSDP_TILE_STORE_CPOL>(r, 8 * (threadIdx.x + u * kThreads),
                                       u2{pack_bf16x2(x[u][0], x[u][1]), pack_bf16x2(x[u][2], x[u][3])});
#else
#pragma unroll
        for (int u = 0; u < kVpl; ++u) put(d + E * (threadIdx.x + u * kThreads), x[u]);
#endif
    }
    __device__ static void put1(uint16_t* d, float x) { *d = to_bf16(x); }
    __device__ static void zero(uint16_t* d) { stu2(d, u2{0u, 0u}); }
    __device__ static void zero1(uint16_t* d) { *d = 0; }
};
template <> struct Cp<uint16_t, uint16_t> {
    static constexpr int E = 8, kVpl = FSDP_B16_VPL;
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
#if FSDP_TILE_STORE_CPOL
        const auto r = block_rsrc(d, kThreads * E * kVpl * 2);
#pragma unroll
        for (int u = 0; u < kVpl; ++u)
            bst4<FSDP_TILE_STORE_CPOL>(r, 16 * (threadIdx.x + u * kThreads),
                                       __builtin_bit_cast(f4, x[u]));
#else
#pragma unroll
        for (int u = 0; u < kVpl; ++u) put(d + E * (threadIdx.x + u * kThreads), x[u]);
#endif
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
struct DevSeg {
    const void* src;  // nullptr: zero fill
    void* dst;
    int64_t blk_n, last_n, src_stride, dst_stride;
    uint32_t nblk, tiles_per_blk, tile0, unused;
};
struct SegTable {
    uint32_t ntiles;
    uint32_t nseg;
    uint32_t xcd_runs;  // tiles in XCD-chunked order (xcd_chunked)
    uint32_t unused;
    DevSeg seg[kMaxSegs];
};
static_assert(sizeof(SegTable) <= 4096, "segment table must fit one kernel argument block");

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

// One tile per workgroup (grid = number of tiles).
template <typename SrcT, typename DstT, bool kGeneral>
__global__ __launch_bounds__(kThreads) void segcopy_kernel(SegTable t) {
    constexpr int kTile = tile_elems<SrcT, DstT>();
    __shared__ __attribute__((aligned(16))) SrcT lds[kGeneral && sizeof(SrcT) == 2 ? kTile + 16 : 8];
    const uint32_t tile =
        t.xcd_runs ? xcd_chunked<FSDP_XCD_CHUNK>(blockIdx.x, t.ntiles) : blockIdx.x;
    // wave-uniform lookup of the segment holding this tile
    uint32_t lo = 0, hi = t.nseg - 1;
    while (lo < hi) {
        const uint32_t mid = (lo + hi + 1) >> 1;
        if (t.seg[mid].tile0 <= tile) lo = mid; else hi = mid - 1;
    }
    const DevSeg& sg = t.seg[lo];
    const uint32_t local = tile - sg.tile0;
    const uint32_t b = sg.nblk == 1 ? 0u : local / sg.tiles_per_blk;
    const uint32_t tb = local - b * sg.tiles_per_blk;
    const int64_t e0 = static_cast<int64_t>(tb) * kTile;
    const int64_t bn = (b + 1 == sg.nblk) ? sg.last_n : sg.blk_n;
    if (e0 >= bn) return;
    const int n = static_cast<int>(min(static_cast<int64_t>(kTile), bn - e0));
    DstT* d = static_cast<DstT*>(sg.dst) + static_cast<int64_t>(b) * sg.dst_stride + e0;
    if (sg.src == nullptr) {
        tile_zero<SrcT, DstT>(d, n);
        return;
    }
    const SrcT* s = static_cast<const SrcT*>(sg.src) + static_cast<int64_t>(b) * sg.src_stride + e0;
    if constexpr (kGeneral)
        tile_general<SrcT, DstT>(s, d, n, lds);
    else
        tile_aligned<SrcT, DstT>(s, d, n);
}

// ---------------------------------------------------------------------------
// gradient reduction
// ---------------------------------------------------------------------------
enum PreMode { kPreNone = 0, kPreRecip = 1, kPreDiv = 2 };

struct ReduceArgs {
    const uint16_t* c[kMaxContrib];
    float* out;
    int64_t len;
    int32_t nc;          // contributions in this launch
    int32_t group;       // hybrid: ranks per group (the launch holds whole groups)
    int32_t first;       // the sum starts in this launch (else out holds the partial)
    int32_t last;        // this launch divides by post (and accumulates)
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
    constexpr int kAhead = FSDP_REDUCE_AHEAD;
    for (; r + kAhead <= end; r += kAhead) {
        Raw x[kAhead];
#pragma unroll
        for (int u = 0; u < kAhead; ++u) x[u] = load_raw<kLd>(a, r + u, j0);
#pragma unroll
        for (int u = 0; u < kAhead; ++u) add8<kPre>(acc, finish<kLd>(x[u], a, r + u), a);
    }
    for (; r < end; ++r) add8<kPre>(acc, finish<kLd>(load_raw<kLd>(a, r, j0), a, r), a);
}

// One output, for buffers that are not 16-byte aligned and for the ragged last tile.
// Up to 8 ranks are loaded before their adds, which run in the vector path's order.
template <int kPre, bool kHybrid, bool kAccum>
__device__ __forceinline__ void reduce_one(const ReduceArgs& a, int64_t j) {
    constexpr int kBatch = 8;
    bool have = !a.first;
    float acc = have ? a.out[j] : 0.0f;
    float s = 0.0f;
    int pos = 0;
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
                // one running sum in rank order, continuing the previous launch's
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
    if (a.last) {
        acc = acc / a.post;
        if constexpr (kAccum) acc = a.out[j] + acc;
    }
    a.out[j] = acc;
}

// Stores a wave's 512 outputs of one whole tile, lane l holding outputs 8l .. 8l+7
// in acc: the halves are swapped across lanes (ds_bpermute, no LDS allocation) so
// that each store instruction writes 1 KiB of whole cache lines.  lane l stores
// outputs 4l .. 4l+3 of each 256-output half, which lane 32h + l/2 holds.
__device__ __forceinline__ void store_whole8(float* wave_out, const float* acc) {
    const int lane = threadIdx.x & 63;
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
        st4(wave_out + 256 * h + 4 * lane, f4{w[0], w[1], w[2], w[3]});
    }
}

// The 8 outputs j0 .. j0+7 of one lane over this launch's ranks.  kWhole: the tile
// is whole and is stored with store_whole8; otherwise each lane stores its own 8.
template <int kPre, int kLd, bool kHybrid, bool kAccum, bool kWhole>
__device__ __forceinline__ void reduce_lane(const ReduceArgs& a, int64_t j0) {
    constexpr int kEpt = 8;
    constexpr int kAhead = FSDP_REDUCE_AHEAD;
    float acc[kEpt];
    if constexpr (!kHybrid) {
        int r = 0;
        if (a.first) {
            set8<kPre>(acc, finish<kLd>(load_raw<kLd>(a, 0, j0), a, 0), a);
            r = 1;
        } else {
            load_out8(acc, a.out + j0);
        }
        add_ranks<kPre, kLd>(acc, r, a.nc, j0, a);
    } else {
        // Loads run kAhead ranks ahead regardless of group boundaries; a wave-uniform
        // position-in-group counter starts each group's sum at its first rank and
        // folds it into the total after its last.
        bool have = !a.first;
        if (have) load_out8(acc, a.out + j0);
        float s[kEpt];
        int pos = 0;
        for (int r = 0; r < a.nc; r += kAhead) {
            const int n = min(kAhead, a.nc - r);
            Raw x[kAhead];
#pragma unroll
            for (int u = 0; u < kAhead; ++u)
                if (u < n) x[u] = load_raw<kLd>(a, r + u, j0);
#pragma unroll
            for (int u = 0; u < kAhead; ++u) {
                if (u >= n) break;
                const u4 v = finish<kLd>(x[u], a, r + u);
                if (pos == 0) set8<kPre>(s, v, a); else add8<kPre>(s, v, a);
                if (++pos == a.group) {
#pragma unroll
                    for (int e = 0; e < kEpt; ++e) acc[e] = have ? acc[e] + s[e] : s[e];
                    have = true;
                    pos = 0;
                }
            }
        }
    }
    if (a.last) {
#pragma unroll
        for (int e = 0; e < kEpt; ++e) acc[e] = acc[e] / a.post;
        if constexpr (kAccum) {
            float prev[kEpt];
            load_out8(prev, a.out + j0);
#pragma unroll
            for (int e = 0; e < kEpt; ++e) acc[e] = prev[e] + acc[e];
        }
    }
    if constexpr (kWhole) {
        store_whole8(a.out + (j0 - 8 * static_cast<int64_t>(threadIdx.x & 63)), acc);
    } else {
        st4(a.out + j0, f4{acc[0], acc[1], acc[2], acc[3]});
        st4(a.out + j0 + 4, f4{acc[4], acc[5], acc[6], acc[7]});
    }
}

// One tile of kReduceThreads * 8 outputs per workgroup.  Each lane owns 8
// consecutive outputs; for every rank it loads their 8 bf16 as one 16-byte
// vector (a wave reads 1 KiB contiguous per rank), kAhead ranks at a time, then
// adds them strictly in rank order.  Hybrid: the same within each group of
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
// consecutive whole tiles (8 kV accumulators per lane) and walks the ranks in order,
// loading rank r + 1's kV vectors while it adds rank r's; the host sizes the grid so
// that every wave is resident at once, so the waves move through the ranks together
// and HBM serves a few rows at a time.  Per output the operations and their order are
// those of the tile path (flat sum, whole-dword contributions), so the results are
// identical.  Block layout of a launch: the tile the output's end cuts (if any), then
// n_single whole tiles that take the tile path, then the sweep waves.
struct SweepArgs {
    ReduceArgs r;
    int64_t t_first;   // first whole tile (512 outputs) of this launch
    int32_t cut;       // 1: block 0 reduces the tile the output's end cuts
    int32_t n_single;  // then this many blocks reduce one whole tile each
};

template <int kPre, bool kAccum, int kV>
__device__ __forceinline__ void sweep_wave(const ReduceArgs& a, int64_t t0) {
    constexpr int kTile = 512;
    const int lane = threadIdx.x & 63;
    // element offset of the lane's first vector from the run's start (vector v: + 512 v)
    const int64_t base = t0 * kTile;
    const int off = 8 * lane;
    float acc[kV][8];
    if (a.first) {
        // -0 + t == t for every t (a NaN comes out quiet, as the divide by post makes
        // it anyway), so adding rank 0 to -0 gives the tile path's first term
#pragma unroll
        for (int v = 0; v < kV; ++v)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[v][e] = -0.0f;
    } else {
#pragma unroll
        for (int v = 0; v < kV; ++v) load_out8(acc[v], a.out + base + off + kTile * v);
    }
    u4 x[kV];  // rank r's vectors
    const uint16_t* c0 = a.c[0] + base;
#pragma unroll
    for (int v = 0; v < kV; ++v) x[v] = ldu4w(c0 + off + kTile * v);
    for (int r = 0; r + 1 < a.nc; ++r) {
        const uint16_t* cn = a.c[r + 1] + base;
#pragma unroll
        for (int v = 0; v < kV; ++v) {
            // one vector at a time, its adds before its reload: no second copy of any
            // vector is live, so the wave holds 12 kV registers of data
            add8<kPre>(acc[v], x[v], a);
            x[v] = ldu4w(cn + off + kTile * v);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int v = 0; v < kV; ++v) add8<kPre>(acc[v], x[v], a);
#pragma unroll
    for (int v = 0; v < kV; ++v) {
        float* o = a.out + base + kTile * v;
        if (a.last) {
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[v][e] = acc[v][e] / a.post;
            if constexpr (kAccum) {
                float prev[8];
                load_out8(prev, o + off);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[v][e] = prev[e] + acc[v][e];
            }
        }
        store_whole8(o, acc[v]);
    }
}

template <int kPre, bool kAccum, int kV>
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
            if (j0 + 8 <= a.len) reduce_lane<kPre, kLdWord, false, kAccum, false>(a, j0);
            const int64_t j = (a.len & ~int64_t{7}) + threadIdx.x;
            if (j < a.len) reduce_one<kPre, false, kAccum>(a, j);
            return;
        }
        --b;
    }
    if (b < s.n_single) {
        reduce_lane<kPre, kLdWord, false, kAccum, true>(
            a, (s.t_first + b) * kTile + 8 * static_cast<int64_t>(threadIdx.x));
        return;
    }
    sweep_wave<kPre, kAccum, kV>(a, s.t_first + s.n_single + (b - s.n_single) * kV);
}

// ---------------------------------------------------------------------------
// local gradient accumulation (no communication): acc = (init ? 0 : acc) + fp32(g)
// ---------------------------------------------------------------------------
template <bool kInit, bool kVec>
__global__ __launch_bounds__(kThreads) void accumulate_kernel(const uint16_t* __restrict__ g,
                                                              float* __restrict__ acc,
                                                              int64_t len) {
    constexpr int kV = FSDP_ACC_VPL;
    constexpr int64_t kPerBlk = static_cast<int64_t>(kThreads) * 4 * kV;
    const uint32_t blk = gridDim.x >= FSDP_XCD_MIN_TILES
                             ? xcd_chunked<FSDP_ACC_XCD_CHUNK>(blockIdx.x, gridDim.x)
                             : blockIdx.x;
    const int64_t base = static_cast<int64_t>(blk) * kPerBlk;
    if (kVec && base + kPerBlk <= len) {
        // lane l owns elements [4l, 4l+4) of each of the tile's kV slices of 4 * kThreads
        u2 x[kV];
        f4 y[kV];
#pragma unroll
        for (int h = 0; h < kV; ++h) {
            const int64_t o = base + 4 * (threadIdx.x + h * kThreads);
            x[h] = __builtin_nontemporal_load(reinterpret_cast<const u2*>(g + o));
            if constexpr (!kInit) y[h] = ld4s<FSDP_ACC_NT != 0>(acc + o);
        }
#pragma unroll
        for (int h = 0; h < kV; ++h) {
            const f4 w = {__builtin_bit_cast(float, x[h][0] << 16),
                          __builtin_bit_cast(float, x[h][0] & 0xFFFF0000u),
                          __builtin_bit_cast(float, x[h][1] << 16),
                          __builtin_bit_cast(float, x[h][1] & 0xFFFF0000u)};
            f4 r;
            if constexpr (kInit) {
                r = w;
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) r[q] = y[h][q] + w[q];
            }
            st4s<FSDP_ACC_NT != 0>(acc + base + 4 * (threadIdx.x + h * kThreads), r);
        }
        return;
    }
    for (int e = 0; e < 4 * kV; ++e) {
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
__global__ __launch_bounds__(kAdamThreads) void adamw_kernel(AdamArgs a) {
    constexpr bool kNTL = FSDP_ADAM_NT_LOAD != 0;
    constexpr bool kNTS = FSDP_ADAM_NT_STORE != 0;
    constexpr int64_t kPerBlk = static_cast<int64_t>(kAdamThreads) * 8;
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kPerBlk;
    if constexpr (kVec) {
        if (base + kPerBlk <= a.len) {
            f4 p[2], g[2], m[2], v[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int64_t o = base + 4 * (threadIdx.x + h * kAdamThreads);
                p[h] = ld4s<kNTL>(a.p + o);
                g[h] = ld4s<kNTL>(a.g + o);
                m[h] = ld4s<kNTL>(a.m + o);
                v[h] = ld4s<kNTL>(a.v + o);
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
#if FSDP_ADAM_STORE_CPOL
            const auto rp = block_rsrc(a.p + base, kPerBlk * 4), rm = block_rsrc(a.m + base, kPerBlk * 4),
                       rv = block_rsrc(a.v + base, kPerBlk * 4);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int o = 16 * (threadIdx.x + h * kAdamThreads);
                bst4<FSDP_ADAM_STORE_CPOL>(rp, o, p[h]);
                bst4<FSDP_ADAM_STORE_CPOL>(rm, o, m[h]);
                bst4<FSDP_ADAM_STORE_CPOL>(rv, o, v[h]);
                if constexpr (kBf16)
                    bst2<FSDP_ADAM_STORE_CPOL>(block_rsrc(a.pb + base, kPerBlk * 2), o / 2,
                                                 u2{pack_bf16x2(p[h][0], p[h][1]),
                                                    pack_bf16x2(p[h][2], p[h][3])});
            }
#else
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int64_t o = base + 4 * (threadIdx.x + h * kAdamThreads);
                st4s<kNTS>(a.p + o, p[h]);
                st4s<kNTS>(a.m + o, m[h]);
                st4s<kNTS>(a.v + o, v[h]);
                if constexpr (kBf16)
                    stu2(a.pb + o, u2{pack_bf16x2(p[h][0], p[h][1]), pack_bf16x2(p[h][2], p[h][3])});
            }
#endif
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

template <typename SrcT, typename DstT>
hipError_t launch_segcopy_t(const std::vector<CopySeg>& segs, hipStream_t stream) {
    constexpr int64_t kTile = tile_elems<SrcT, DstT>();
    constexpr uintptr_t kDstAlign = Cp<SrcT, DstT>::kDstAlign;
    size_t i = 0;
    while (i < segs.size()) {
        SegTable t{};
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
        t.xcd_runs = tiles >= FSDP_XCD_MIN_TILES ? 1u : 0u;
        if (general)
            hipLaunchKernelGGL((segcopy_kernel<SrcT, DstT, true>), grid_of(tiles), dim3(kThreads),
                               0, stream, t);
        else
            hipLaunchKernelGGL((segcopy_kernel<SrcT, DstT, false>), grid_of(tiles), dim3(kThreads),
                               0, stream, t);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int kPre, int kLd>
void launch_reduce_mode(const ReduceArgs& a, bool hybrid, bool accum, dim3 grid,
                        hipStream_t stream) {
    const dim3 block(kReduceThreads);
    if (hybrid) {
        if (accum) hipLaunchKernelGGL((reduce_kernel<kPre, kLd, true, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((reduce_kernel<kPre, kLd, true, false>), grid, block, 0, stream, a);
    } else {
        if (accum) hipLaunchKernelGGL((reduce_kernel<kPre, kLd, false, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((reduce_kernel<kPre, kLd, false, false>), grid, block, 0, stream, a);
    }
}

// ---------------------------------------------------------------------------
// sharded gradient scaler: g *= inv_scale, flag non-finite inputs
// ---------------------------------------------------------------------------
// In place: plain loads and nt stores (as AdamW).  A wave that saw a non-finite
// input has one lane store 1.0f into the flag (vector store; every writer stores
// the same value, so concurrent stores agree).  found == nullptr: scaling only.
template <bool kVec>
__global__ __launch_bounds__(kThreads) void unscale_kernel(float* __restrict__ g, int64_t len,
                                                           float inv, float* __restrict__ found) {
    constexpr int kV = FSDP_UNSCALE_VPL;
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
struct SqTable {
    const float* g;
    double* partial;
    double* out;
    uint32_t nrun;
    uint32_t unused;
    SqRun run[kMaxSegs];
};
static_assert(sizeof(SqTable) <= 4096, "run table must fit one kernel argument block");

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
__global__ __launch_bounds__(kSqThreads) void sqnorm_partial_kernel(SqTable t) {
    __shared__ double lds[kSqThreads / 64];
    const uint32_t tile = blockIdx.x;
    uint32_t lo = 0, hi = t.nrun - 1;  // wave-uniform: last non-empty run with tile0 <= tile
    while (lo < hi) {
        const uint32_t mid = (lo + hi + 1) >> 1;
        if (t.run[mid].tile0 <= tile) lo = mid; else hi = mid - 1;
    }
    const SqRun& r = t.run[lo];
    const int64_t e0 = static_cast<int64_t>(tile - r.tile0) * kSqTile;
    const int64_t n = min(kSqTile, r.n - e0);
    const float* g = t.g + r.offset + e0;
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
    if (threadIdx.x == 0) t.partial[tile] = s;
}

// Stage 2: one workgroup per run sums its partials in a fixed order (lane order
// within strided passes, then the block tree) and writes the parameter's result.
__global__ __launch_bounds__(kSqThreads) void sqnorm_final_kernel(SqTable t) {
    __shared__ double lds[kSqThreads / 64];
    const SqRun& r = t.run[blockIdx.x];
    double acc = 0.0;
    for (uint32_t i = threadIdx.x; i < r.ntiles; i += kSqThreads) acc = acc + t.partial[r.tile0 + i];
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

// Workgroups of reduce_sweep_kernel<kPre, kAccum, kSweepV> resident at once on the
// current device (occupancy per CU times CUs), queried once per device; 0 if unknown.
constexpr int kSweepV = FSDP_SWEEP_V;
constexpr int kMaxDevices = 64;
template <int kPre, bool kAccum>
int64_t sweep_capacity() {
    static std::atomic<int64_t> cap[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    int64_t c = cap[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &per_cu, reinterpret_cast<const void*>(&reduce_sweep_kernel<kPre, kAccum, kSweepV>),
                64, 0) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        c = int64_t{per_cu} * cus;
        cap[dev].store(c > 0 ? c : -1, std::memory_order_relaxed);
    }
    return c > 0 ? c : 0;
}

// The sweep over this launch's ranks, one launch per run of plan_sweep_runs (runs whose
// grids are resident at once), in output order; *err gets the first launch error.  Returns
// false, having launched nothing, when the output is too short or the occupancy unknown.
template <int kPre, bool kAccum>
bool try_sweep(const ReduceArgs& a, hipStream_t stream, hipError_t* err) {
    constexpr int64_t kTile = 512;
    const int64_t tiles = a.len / kTile;
    if (tiles < FSDP_SWEEP_MIN_TILES) return false;
    std::vector<SweepRun> runs;
    if (!plan_sweep_runs(tiles, a.len % kTile != 0, kSweepV, sweep_capacity<kPre, kAccum>(), &runs))
        return false;
    for (const SweepRun& r : runs) {
        SweepArgs s{};
        s.r = a;
        s.t_first = r.t_first;
        s.cut = r.cut;
        s.n_single = r.n_single;
        hipLaunchKernelGGL((reduce_sweep_kernel<kPre, kAccum, kSweepV>),
                           dim3(static_cast<unsigned>(r.blocks)), dim3(64), 0, stream, s);
        *err = hipGetLastError();
        if (*err != hipSuccess) break;
    }
    return true;
}

// The sweep, for a flat sum over at least FSDP_SWEEP_MIN_RANKS contributions that are all
// at least 4-byte aligned into a 16-byte-aligned output; false if it does not apply.
bool launch_reduce_sweep(const ReduceArgs& a, int mode, bool accum, hipStream_t stream,
                         hipError_t* err) {
    if (a.nc < FSDP_SWEEP_MIN_RANKS) return false;
    if (mode == kPreNone)
        return accum ? try_sweep<kPreNone, true>(a, stream, err) : try_sweep<kPreNone, false>(a, stream, err);
    if (mode == kPreRecip)
        return accum ? try_sweep<kPreRecip, true>(a, stream, err) : try_sweep<kPreRecip, false>(a, stream, err);
    return accum ? try_sweep<kPreDiv, true>(a, stream, err) : try_sweep<kPreDiv, false>(a, stream, err);
}

hipError_t launch_grad_reduce(const uint16_t* const* contribs, int64_t n_contrib, int64_t len,
                              float pre, float post, int64_t group, bool accumulate, float* out,
                              hipStream_t stream) {
    if (len <= 0 || n_contrib <= 0) return hipSuccess;
    // one group of all ranks, or groups of one, are the flat sequential sum
    const bool hybrid = group > 1 && group < n_contrib;
    if (hybrid && (n_contrib % group != 0 || group > kMaxContrib)) return hipErrorInvalidValue;
    if (accumulate && n_contrib > kMaxContrib) return hipErrorInvalidValue;
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
    // vector path when the output is 16-byte aligned; contributions only 2-byte
    // aligned are read one element early and shifted
    bool all4 = true;
    for (int64_t r = 0; r < n_contrib; ++r) all4 = all4 && aligned_to(contribs[r], 4);
    const int ld = !aligned_to(out, 16) ? kLdScalar : all4 ? kLdWord : kLdHalf;
    const int64_t per_blk = static_cast<int64_t>(kReduceThreads) * 8;
    const int64_t blocks = (len + per_blk - 1) / per_blk;
    if (blocks > 0x7FFFFFFFll) return hipErrorInvalidValue;
    // a launch holds up to kMaxContrib ranks; hybrid launches hold whole groups, so
    // the running value carried in `out` between launches is always a complete sum
    const int64_t chunk = hybrid ? (kMaxContrib / group) * group : kMaxContrib;
    for (int64_t r0 = 0; r0 < n_contrib; r0 += chunk) {
        ReduceArgs a{};
        a.nc = static_cast<int32_t>(std::min<int64_t>(chunk, n_contrib - r0));
        for (int32_t r = 0; r < a.nc; ++r) a.c[r] = contribs[r0 + r];
        a.out = out;
        a.len = len;
        a.group = static_cast<int32_t>(hybrid ? group : a.nc);
        a.first = r0 == 0;
        a.last = r0 + a.nc == n_contrib;
        a.pre = pre;
        a.rpre = rpre;
        a.post = post;
        const dim3 grid = grid_of(blocks);
        hipError_t swept = hipSuccess;
        if (!hybrid && ld == kLdWord && launch_reduce_sweep(a, mode, accumulate, stream, &swept)) {
            if (swept != hipSuccess) return swept;
            continue;
        }
        if (mode == kPreNone) {
            if (ld == kLdWord) launch_reduce_mode<kPreNone, kLdWord>(a, hybrid, accumulate, grid, stream);
            else if (ld == kLdHalf) launch_reduce_mode<kPreNone, kLdHalf>(a, hybrid, accumulate, grid, stream);
            else launch_reduce_mode<kPreNone, kLdScalar>(a, hybrid, accumulate, grid, stream);
        } else if (mode == kPreRecip) {
            if (ld == kLdWord) launch_reduce_mode<kPreRecip, kLdWord>(a, hybrid, accumulate, grid, stream);
            else if (ld == kLdHalf) launch_reduce_mode<kPreRecip, kLdHalf>(a, hybrid, accumulate, grid, stream);
            else launch_reduce_mode<kPreRecip, kLdScalar>(a, hybrid, accumulate, grid, stream);
        } else {
            if (ld == kLdWord) launch_reduce_mode<kPreDiv, kLdWord>(a, hybrid, accumulate, grid, stream);
            else if (ld == kLdHalf) launch_reduce_mode<kPreDiv, kLdHalf>(a, hybrid, accumulate, grid, stream);
            else launch_reduce_mode<kPreDiv, kLdScalar>(a, hybrid, accumulate, grid, stream);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_grad_accumulate(const uint16_t* grad, float* acc, int64_t len, bool init,
                                  hipStream_t stream) {
    if (len <= 0) return hipSuccess;
    const int64_t per_blk = static_cast<int64_t>(kThreads) * 4 * FSDP_ACC_VPL;
    const int64_t blocks = (len + per_blk - 1) / per_blk;
    if (blocks > 0x7FFFFFFFll) return hipErrorInvalidValue;
    const bool vec = aligned_to(grad, 8) && aligned_to(acc, 16);
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
    AdamArgs a{p, g, m, v, pb, len, s};
    const bool vec = aligned_to(p, 16) && aligned_to(g, 16) && aligned_to(m, 16) &&
                     aligned_to(v, 16) && (pb == nullptr || aligned_to(pb, 8));
    const int64_t per_blk = static_cast<int64_t>(kAdamThreads) * 8;
    const int64_t blocks = (len + per_blk - 1) / per_blk;
    if (blocks > 0x7FFFFFFFll) return hipErrorInvalidValue;
    if (vec) {
        if (pb)
            hipLaunchKernelGGL((adamw_kernel<true, true>), grid_of(blocks), dim3(kAdamThreads), 0,
                               stream, a);
        else
            hipLaunchKernelGGL((adamw_kernel<true, false>), grid_of(blocks), dim3(kAdamThreads),
                               0, stream, a);
    } else {
        hipLaunchKernelGGL((adamw_kernel<false, false>), grid_of(blocks), dim3(kAdamThreads), 0,
                           stream, a);
    }
    return hipGetLastError();
}

hipError_t launch_grad_unscale(float* g, int64_t len, float inv_scale, float* found_inf,
                               hipStream_t stream) {
    if (len <= 0) return hipSuccess;
    const int64_t per_blk = static_cast<int64_t>(kThreads) * 4 * FSDP_UNSCALE_VPL;
    const int64_t blocks = (len + per_blk - 1) / per_blk;
    if (blocks > 0x7FFFFFFFll) return hipErrorInvalidValue;
    const dim3 grid = grid_of(blocks), block(kThreads);
    if (aligned_to(g, 16))
        hipLaunchKernelGGL((unscale_kernel<true>), grid, block, 0, stream, g, len, inv_scale, found_inf);
    else
        hipLaunchKernelGGL((unscale_kernel<false>), grid, block, 0, stream, g, len, inv_scale, found_inf);
    return hipGetLastError();
}

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
        SqTable all{}, busy{};  // every run of the batch / only the non-empty ones
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
            hipLaunchKernelGGL(sqnorm_partial_kernel, grid_of(tiles), dim3(kSqThreads), 0, stream, busy);
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

