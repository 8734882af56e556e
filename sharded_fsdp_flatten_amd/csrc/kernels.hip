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
//     (a grid-stride version of the same copy runs ~20% slower);
//   - outputs stored non-temporally (streamed, never re-read by the kernel).
// The kernels:
//   - segcopy: one engine for flatten (FSDP1 and FSDP2) and copy-out.  The host
//     planner turns the layout into a short table of (src, dst, length[, block
//     stride]) segments passed in the kernel argument block; each workgroup
//     takes one tile of one segment (the tile -> segment lookup is a
//     wave-uniform binary search on scalar registers), so no lane ever searches
//     and every tile is a straight streaming copy.  When a segment's source and
//     destination are not 16-byte co-aligned, the tile is staged through LDS
//     and re-read at the element shift, so HBM still sees only aligned vector
//     loads and stores.
//   - grad_reduce: each lane owns 8 consecutive outputs, loads 8 bf16 of 8
//     ranks at a time (128-bit each) before adding them in rank order.
//   - adamw: elementwise over 8 elements per lane, 128-bit loads and stores.
//     Its state is read and written back in place, and here the plain cache
//     policy measures faster than the non-temporal one (6.5 vs 5.6 TB/s).
// Every floating-point step is one IEEE binary32 operation, in the order the
// CPU oracle fixes; contraction into FMA is disabled for this file.
#include <hip/hip_runtime.h>

#include <algorithm>
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
#ifndef FSDP_REDUCE_THREADS
#define FSDP_REDUCE_THREADS 64
#endif
#ifndef FSDP_REDUCE_AHEAD
#define FSDP_REDUCE_AHEAD 8
#endif
#ifndef FSDP_ADAM_THREADS
#define FSDP_ADAM_THREADS 256
#endif
#ifndef FSDP_ADAM_NT
#define FSDP_ADAM_NT 0      // p, m, v are read and written back in place: plain accesses
#endif

constexpr int kThreads = FSDP_COPY_THREADS;
constexpr int kMaxSegs = 48;           // segments per launch (kernel-argument budget)
constexpr int kMaxContrib = 128;       // contribution pointers per reduce launch
constexpr int kReduceThreads = FSDP_REDUCE_THREADS;
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

// Output element traits.  A vector is 4 elements: one 16-byte fp32 load feeds
// one 16-byte fp32 store or one 8-byte bf16 store.  kVpl vectors per lane make a
// tile of kThreads * 4 * kVpl elements, lane l owning vectors l, l + kThreads, ...
// so every load and store instruction is contiguous across the wave.
template <typename OutT> struct Out;
template <> struct Out<float> {
    static constexpr int kVpl = FSDP_F32_VPL;
    static constexpr int kAlign = 16;  // bytes a vector store needs
    __device__ static void put(float* d, f4 x) { st4(d, x); }
    __device__ static void put1(float* d, float x) { *d = x; }
    __device__ static void zero(float* d) { st4(d, f4{0.0f, 0.0f, 0.0f, 0.0f}); }
    __device__ static void zero1(float* d) { *d = 0.0f; }
};
template <> struct Out<uint16_t> {
    static constexpr int kVpl = FSDP_BF16_VPL;
    static constexpr int kAlign = 8;
    __device__ static void put(uint16_t* d, f4 x) {
        stu2(d, u2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])});
    }
    __device__ static void put1(uint16_t* d, float x) { *d = to_bf16(x); }
    __device__ static void zero(uint16_t* d) { stu2(d, u2{0u, 0u}); }
    __device__ static void zero1(uint16_t* d) { *d = 0; }
};
template <typename OutT>
constexpr int tile_elems() { return kThreads * 4 * Out<OutT>::kVpl; }

// ---------------------------------------------------------------------------
// segcopy
// ---------------------------------------------------------------------------
struct DevSeg {
    const float* src;  // nullptr: zero fill
    void* dst;
    int64_t blk_n, last_n, src_stride, dst_stride;
    uint32_t nblk, tiles_per_blk, tile0, unused;
};
struct SegTable {
    uint32_t ntiles;
    uint32_t nseg;
    DevSeg seg[kMaxSegs];
};
static_assert(sizeof(SegTable) <= 4096, "segment table must fit one kernel argument block");

// n <= tile elements; s 16-byte aligned, d aligned for its vector store.
template <typename OutT>
__device__ __forceinline__ void tile_aligned(const float* __restrict__ s, OutT* __restrict__ d,
                                             int n) {
    constexpr int kVpl = Out<OutT>::kVpl;
    const int nv = n >> 2;
    if (nv == kThreads * kVpl) {  // full tile: all loads issued before any store
        f4 x[kVpl];
#pragma unroll
        for (int u = 0; u < kVpl; ++u) x[u] = ld4(s + 4 * (threadIdx.x + u * kThreads));
#pragma unroll
        for (int u = 0; u < kVpl; ++u) Out<OutT>::put(d + 4 * (threadIdx.x + u * kThreads), x[u]);
        return;
    }
    for (int v = threadIdx.x; v < nv; v += kThreads) Out<OutT>::put(d + 4 * v, ld4(s + 4 * v));
    for (int e = 4 * nv + threadIdx.x; e < n; e += kThreads) Out<OutT>::put1(d + e, s[e]);
}

// Elements of OutT from d up to the next boundary its vector store needs.
template <typename OutT>
__device__ __forceinline__ int head_to_align(const OutT* d) {
    constexpr unsigned a = Out<OutT>::kAlign;
    return static_cast<int>(((a - (reinterpret_cast<uintptr_t>(d) & (a - 1))) & (a - 1)) /
                            sizeof(OutT));
}

template <typename OutT>
__device__ __forceinline__ void tile_zero(OutT* d, int n) {
    const int h = min(head_to_align(d), n);
    if (static_cast<int>(threadIdx.x) < h) Out<OutT>::zero1(d + threadIdx.x);
    d += h;
    n -= h;
    const int nv = n >> 2;
    for (int v = threadIdx.x; v < nv; v += kThreads) Out<OutT>::zero(d + 4 * v);
    for (int e = 4 * nv + threadIdx.x; e < n; e += kThreads) Out<OutT>::zero1(d + e);
}

// Any 4-byte-aligned source and element-aligned destination.  A short head of
// scalar stores aligns the destination; if the source is then off a 16-byte
// boundary by `shift` floats, the tile is loaded as aligned 128-bit vectors
// (covering exactly the 16-byte blocks that hold the tile, so no access leaves
// them) into LDS and re-read at the shift.  Tile-uniform control flow (barriers).
template <typename OutT>
__device__ __forceinline__ void tile_general(const float* s, OutT* d, int n, float* lds) {
    const int h = min(head_to_align(d), n);
    if (static_cast<int>(threadIdx.x) < h) Out<OutT>::put1(d + threadIdx.x, s[threadIdx.x]);
    s += h;
    d += h;
    n -= h;
    const int shift = static_cast<int>((reinterpret_cast<uintptr_t>(s) & 15u) >> 2);
    if (shift == 0) {
        tile_aligned<OutT>(s, d, n);
        return;
    }
    const float* base = s - shift;
    const int nload = (shift + n + 3) >> 2;  // <= tile/4 + 2 vectors
    for (int v = threadIdx.x; v < nload; v += kThreads)
        *reinterpret_cast<f4*>(lds + 4 * v) = ld4(base + 4 * v);
    __syncthreads();
    const int nv = n >> 2;
    for (int v = threadIdx.x; v < nv; v += kThreads) {
        const float* x = lds + shift + 4 * v;
        Out<OutT>::put(d + 4 * v, f4{x[0], x[1], x[2], x[3]});
    }
    for (int e = 4 * nv + threadIdx.x; e < n; e += kThreads)
        Out<OutT>::put1(d + e, lds[shift + e]);
    __syncthreads();
}

// One tile per workgroup (grid = number of tiles).
template <typename OutT, bool kGeneral>
__global__ __launch_bounds__(kThreads) void segcopy_kernel(SegTable t) {
    constexpr int kTile = tile_elems<OutT>();
    __shared__ __attribute__((aligned(16))) float lds[kGeneral ? kTile + 16 : 4];
    const uint32_t tile = blockIdx.x;
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
    OutT* d = static_cast<OutT*>(sg.dst) + static_cast<int64_t>(b) * sg.dst_stride + e0;
    if (sg.src == nullptr) {
        tile_zero<OutT>(d, n);
        return;
    }
    const float* s = sg.src + static_cast<int64_t>(b) * sg.src_stride + e0;
    if constexpr (kGeneral)
        tile_general<OutT>(s, d, n, lds);
    else
        tile_aligned<OutT>(s, d, n);
}

// ---------------------------------------------------------------------------
// gradient reduction
// ---------------------------------------------------------------------------
enum PreMode { kPreNone = 0, kPreRecip = 1, kPreDiv = 2 };

struct ReduceArgs {
    const uint16_t* c[kMaxContrib];
    float* out;
    int64_t len;
    int32_t nc;     // contributions in this launch
    int32_t first;  // this launch holds rank 0's term: start from it
    int32_t last;   // this launch applies the post divide
    int32_t unused;
    float pre, rpre, post, unused2;
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
__device__ __forceinline__ void add8(float* acc, u4 x, const ReduceArgs& a) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        acc[2 * q] = acc[2 * q] + term<kPre>(x[q] << 16, a);
        acc[2 * q + 1] = acc[2 * q + 1] + term<kPre>(x[q] & 0xFFFF0000u, a);
    }
}

template <int kPre>
__device__ __forceinline__ void reduce_one(const ReduceArgs& a, int64_t j) {
    float acc;
    int r = 0;
    if (a.first) {
        acc = term<kPre>(static_cast<uint32_t>(a.c[0][j]) << 16, a);
        r = 1;
    } else {
        acc = a.out[j];
    }
    for (; r < a.nc; ++r) acc = acc + term<kPre>(static_cast<uint32_t>(a.c[r][j]) << 16, a);
    if (a.last) acc = acc / a.post;
    a.out[j] = acc;
}

// One tile of kReduceThreads * 8 outputs per workgroup.  Each lane owns 8
// consecutive outputs; for every rank it loads their 8 bf16 as one 16-byte
// vector, kAhead ranks at a time, then adds them strictly in rank order.
template <int kPre, bool kVec>
__global__ __launch_bounds__(kReduceThreads) void reduce_kernel(ReduceArgs a) {
    constexpr int kEpt = 8;
    constexpr int kAhead = FSDP_REDUCE_AHEAD;
    constexpr int64_t kPerBlk = static_cast<int64_t>(kReduceThreads) * kEpt;
    const int64_t blk = blockIdx.x;
    if constexpr (kVec) {
        const int64_t j0 = blk * kPerBlk + static_cast<int64_t>(threadIdx.x) * kEpt;
        if (j0 + kEpt <= a.len) {
            float acc[kEpt];
            int r = 0;
            if (a.first) {
                const u4 x = ldu4(a.c[0] + j0);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[2 * q] = term<kPre>(x[q] << 16, a);
                    acc[2 * q + 1] = term<kPre>(x[q] & 0xFFFF0000u, a);
                }
                r = 1;
            } else {
                const f4 lo = ld4(a.out + j0), hi = ld4(a.out + j0 + 4);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[q] = lo[q];
                    acc[4 + q] = hi[q];
                }
            }
            for (; r + kAhead <= a.nc; r += kAhead) {
                u4 x[kAhead];
#pragma unroll
                for (int u = 0; u < kAhead; ++u) x[u] = ldu4(a.c[r + u] + j0);
#pragma unroll
                for (int u = 0; u < kAhead; ++u) add8<kPre>(acc, x[u], a);
            }
            for (; r < a.nc; ++r) add8<kPre>(acc, ldu4(a.c[r] + j0), a);
            if (a.last) {
#pragma unroll
                for (int e = 0; e < kEpt; ++e) acc[e] = acc[e] / a.post;
            }
            st4(a.out + j0, f4{acc[0], acc[1], acc[2], acc[3]});
            st4(a.out + j0 + 4, f4{acc[4], acc[5], acc[6], acc[7]});
        } else {
            for (int64_t j = j0; j < a.len && j < j0 + kEpt; ++j) reduce_one<kPre>(a, j);
        }
    } else {
#pragma unroll
        for (int e = 0; e < kEpt; ++e) {
            const int64_t j = blk * kPerBlk + static_cast<int64_t>(e) * kReduceThreads + threadIdx.x;
            if (j < a.len) reduce_one<kPre>(a, j);
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
    constexpr bool kNT = FSDP_ADAM_NT != 0;
    constexpr int64_t kPerBlk = static_cast<int64_t>(kAdamThreads) * 8;
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kPerBlk;
    if constexpr (kVec) {
        if (base + kPerBlk <= a.len) {
            f4 p[2], g[2], m[2], v[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int64_t o = base + 4 * (threadIdx.x + h * kAdamThreads);
                p[h] = ld4s<kNT>(a.p + o);
                g[h] = ld4s<kNT>(a.g + o);
                m[h] = ld4s<kNT>(a.m + o);
                v[h] = ld4s<kNT>(a.v + o);
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
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int64_t o = base + 4 * (threadIdx.x + h * kAdamThreads);
                st4s<kNT>(a.p + o, p[h]);
                st4s<kNT>(a.m + o, m[h]);
                st4s<kNT>(a.v + o, v[h]);
                if constexpr (kBf16)
                    stu2(a.pb + o, u2{pack_bf16x2(p[h][0], p[h][1]), pack_bf16x2(p[h][2], p[h][3])});
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

template <typename OutT>
hipError_t launch_segcopy_t(const std::vector<CopySeg>& segs, hipStream_t stream) {
    constexpr int64_t kTile = tile_elems<OutT>();
    constexpr uintptr_t kDstAlign = Out<OutT>::kAlign;
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
                      (c.nblk == 1 || (c.dst_stride * sizeof(OutT)) % kDstAlign == 0);
            if (c.src)
                ok = ok && aligned_to(c.src, 16) && (c.nblk == 1 || (c.src_stride * 4) % 16 == 0);
            general = general || !ok;
        }
        if (t.nseg == 0) continue;
        t.ntiles = static_cast<uint32_t>(tiles);
        if (general)
            hipLaunchKernelGGL((segcopy_kernel<OutT, true>), grid_of(tiles), dim3(kThreads), 0,
                               stream, t);
        else
            hipLaunchKernelGGL((segcopy_kernel<OutT, false>), grid_of(tiles), dim3(kThreads), 0,
                               stream, t);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_segcopy(const std::vector<CopySeg>& segs, OutType out, hipStream_t stream) {
    return out == OutType::kF32 ? launch_segcopy_t<float>(segs, stream)
                                : launch_segcopy_t<uint16_t>(segs, stream);
}

hipError_t launch_grad_reduce(const uint16_t* const* contribs, int64_t n_contrib, int64_t len,
                              float pre, float post, float* out, hipStream_t stream) {
    if (len <= 0 || n_contrib <= 0) return hipSuccess;
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
    bool vec = aligned_to(out, 16);
    for (int64_t r = 0; r < n_contrib; ++r) vec = vec && aligned_to(contribs[r], 16);
    const int64_t per_blk = static_cast<int64_t>(kReduceThreads) * 8;
    const int64_t blocks = (len + per_blk - 1) / per_blk;
    if (blocks > 0x7FFFFFFFll) return hipErrorInvalidValue;
    for (int64_t r0 = 0; r0 < n_contrib; r0 += kMaxContrib) {
        ReduceArgs a{};
        a.nc = static_cast<int32_t>(std::min<int64_t>(kMaxContrib, n_contrib - r0));
        for (int32_t r = 0; r < a.nc; ++r) a.c[r] = contribs[r0 + r];
        a.out = out;
        a.len = len;
        a.first = r0 == 0;
        a.last = r0 + a.nc == n_contrib;
        a.pre = pre;
        a.rpre = rpre;
        a.post = post;
#define FSDP_LAUNCH_REDUCE(MODE)                                                              \
    do {                                                                                      \
        if (vec)                                                                              \
            hipLaunchKernelGGL((reduce_kernel<MODE, true>), grid_of(blocks),                  \
                               dim3(kReduceThreads), 0, stream, a);                           \
        else                                                                                  \
            hipLaunchKernelGGL((reduce_kernel<MODE, false>), grid_of(blocks),                 \
                               dim3(kReduceThreads), 0, stream, a);                           \
    } while (0)
        if (mode == kPreNone) FSDP_LAUNCH_REDUCE(kPreNone);
        else if (mode == kPreRecip) FSDP_LAUNCH_REDUCE(kPreRecip);
        else FSDP_LAUNCH_REDUCE(kPreDiv);
#undef FSDP_LAUNCH_REDUCE
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
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

}  // namespace fsdp
