// kernels.hip -- HIP kernels of the per-rank FSDP data path for CDNA4 (gfx950).
//
// All four operations are HBM-streaming: none is a dense contraction, so no
// MFMA is used.  What matters on MI355X is keeping enough 128-bit, fully
// coalesced HBM requests in flight on all 256 CUs:
//   - segcopy: one engine for flatten (FSDP1 and FSDP2) and copy-out.  The host
//     planner turns the layout into a short table of (src, dst, length[, block
//     stride]) segments passed in the kernel argument block; each workgroup
//     takes a 4096-element tile of one segment (the tile -> segment lookup is a
//     wave-uniform binary search on scalar registers), so no lane ever searches
//     and every tile is a straight streaming copy.  When a segment's source and
//     destination are not 16-byte co-aligned, the tile is staged through LDS
//     and re-read at the element shift, so HBM still sees only aligned 128-bit
//     loads and stores.
//   - grad_reduce: each lane owns 8 consecutive outputs, loads 8 bf16 of 8
//     ranks at a time (128-bit each) before adding them in rank order.
//   - adamw: elementwise over 8 elements per lane, 128-bit loads and stores.
// Every floating-point step is one IEEE binary32 operation, in the order the
// CPU oracle fixes; contraction into FMA is disabled for this file.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cmath>
#include <mutex>
#include <vector>

#include "kernels.h"

#pragma clang fp contract(off)

namespace fsdp {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;          // 4 wave64s per workgroup
constexpr int kTile = 4096;            // elements per segcopy tile
constexpr int kMaxSegs = 48;           // segments per launch (kernel-argument budget)
constexpr int kLdsFloats = kTile + 16; // realignment staging: tile + shift + slack
constexpr int kMaxContrib = 128;       // contribution pointers per reduce launch

// ---------------------------------------------------------------------------
// memory helpers: 128-bit global accesses; outputs are streamed (never re-read
// by the same kernel), so stores are non-temporal.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f4 ld4(const float* p) { return *reinterpret_cast<const f4*>(p); }
__device__ __forceinline__ u4 ldu4(const void* p) { return *reinterpret_cast<const u4*>(p); }
__device__ __forceinline__ void st4(float* p, f4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<f4*>(p));
}
__device__ __forceinline__ void stu4(void* p, u4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u4*>(p));
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

// Output element traits: V outputs form one 16-byte store.
template <typename OutT> struct Out;
template <> struct Out<float> {
    static constexpr int V = 4;
    __device__ static void put(float* d, const float* x) { st4(d, f4{x[0], x[1], x[2], x[3]}); }
    __device__ static void put1(float* d, float x) { *d = x; }
    __device__ static void zero(float* d) { st4(d, f4{0.0f, 0.0f, 0.0f, 0.0f}); }
    __device__ static void zero1(float* d) { *d = 0.0f; }
};
template <> struct Out<uint16_t> {
    static constexpr int V = 8;
    __device__ static void put(uint16_t* d, const float* x) {
        stu4(d, u4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                   pack_bf16x2(x[6], x[7])});
    }
    __device__ static void put1(uint16_t* d, float x) { *d = to_bf16(x); }
    __device__ static void zero(uint16_t* d) { stu4(d, u4{0u, 0u, 0u, 0u}); }
    __device__ static void zero1(uint16_t* d) { *d = 0; }
};

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

// n <= kTile elements; s and d 16-byte aligned.
template <typename OutT>
__device__ __forceinline__ void tile_aligned(const float* __restrict__ s, OutT* __restrict__ d,
                                             int n) {
    constexpr int V = Out<OutT>::V;
    constexpr int kPer = kTile / V / kThreads;  // vectors per lane in a full tile
    const int nv = n / V;
    if (nv == kTile / V) {
        float x[kPer][V];
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const float* src = s + (threadIdx.x + u * kThreads) * V;
#pragma unroll
            for (int q = 0; q < V / 4; ++q) {
                const f4 t = ld4(src + 4 * q);
                x[u][4 * q + 0] = t[0];
                x[u][4 * q + 1] = t[1];
                x[u][4 * q + 2] = t[2];
                x[u][4 * q + 3] = t[3];
            }
        }
#pragma unroll
        for (int u = 0; u < kPer; ++u) Out<OutT>::put(d + (threadIdx.x + u * kThreads) * V, x[u]);
        return;
    }
    for (int v = threadIdx.x; v < nv; v += kThreads) {
        float x[V];
#pragma unroll
        for (int q = 0; q < V / 4; ++q) {
            const f4 t = ld4(s + v * V + 4 * q);
            x[4 * q + 0] = t[0];
            x[4 * q + 1] = t[1];
            x[4 * q + 2] = t[2];
            x[4 * q + 3] = t[3];
        }
        Out<OutT>::put(d + v * V, x);
    }
    for (int e = nv * V + threadIdx.x; e < n; e += kThreads) Out<OutT>::put1(d + e, s[e]);
}

// Elements of OutT from d up to the next 16-byte boundary.
template <typename OutT>
__device__ __forceinline__ int head_to_align(const OutT* d) {
    return static_cast<int>(((16u - (reinterpret_cast<uintptr_t>(d) & 15u)) & 15u) / sizeof(OutT));
}

template <typename OutT>
__device__ __forceinline__ void tile_zero(OutT* d, int n) {
    constexpr int V = Out<OutT>::V;
    const int h = min(head_to_align(d), n);
    if (static_cast<int>(threadIdx.x) < h) Out<OutT>::zero1(d + threadIdx.x);
    d += h;
    n -= h;
    const int nv = n / V;
    for (int v = threadIdx.x; v < nv; v += kThreads) Out<OutT>::zero(d + v * V);
    for (int e = nv * V + threadIdx.x; e < n; e += kThreads) Out<OutT>::zero1(d + e);
}

// Any 4-byte-aligned source and element-aligned destination.  A short head of
// scalar stores aligns the destination; if the source is then off a 16-byte
// boundary by `shift` floats, the tile is loaded as aligned 128-bit vectors
// (covering the 16-byte blocks that hold the tile, so no access leaves them)
// into LDS and re-read at the shift.  Tile-uniform control flow (barriers).
template <typename OutT>
__device__ __forceinline__ void tile_general(const float* s, OutT* d, int n, float* lds) {
    constexpr int V = Out<OutT>::V;
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
    const int nload = (shift + n + 3) >> 2;  // <= (kTile + 6) / 4 vectors
    for (int v = threadIdx.x; v < nload; v += kThreads)
        *reinterpret_cast<f4*>(lds + 4 * v) = ld4(base + 4 * v);
    __syncthreads();
    const int nv = n / V;
    for (int v = threadIdx.x; v < nv; v += kThreads) {
        float x[V];
#pragma unroll
        for (int q = 0; q < V; ++q) x[q] = lds[shift + v * V + q];
        Out<OutT>::put(d + v * V, x);
    }
    for (int e = nv * V + threadIdx.x; e < n; e += kThreads)
        Out<OutT>::put1(d + e, lds[shift + e]);
    __syncthreads();
}

template <typename OutT, bool kGeneral>
__global__ __launch_bounds__(kThreads) void segcopy_kernel(SegTable t) {
    __shared__ __attribute__((aligned(16))) float lds[kGeneral ? kLdsFloats : 4];
    for (uint32_t tile = blockIdx.x; tile < t.ntiles; tile += gridDim.x) {
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
        if (e0 >= bn) continue;
        const int n = static_cast<int>(min(static_cast<int64_t>(kTile), bn - e0));
        OutT* d = static_cast<OutT*>(sg.dst) + static_cast<int64_t>(b) * sg.dst_stride + e0;
        if (sg.src == nullptr) {
            tile_zero<OutT>(d, n);
            continue;
        }
        const float* s = sg.src + static_cast<int64_t>(b) * sg.src_stride + e0;
        if constexpr (kGeneral)
            tile_general<OutT>(s, d, n, lds);
        else
            tile_aligned<OutT>(s, d, n);
    }
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

template <int kPre, bool kVec>
__global__ __launch_bounds__(kThreads) void reduce_kernel(ReduceArgs a) {
    constexpr int kEpt = 8;  // outputs per lane
    constexpr int kU = 8;    // ranks loaded ahead of their adds
    constexpr int64_t kPerBlk = static_cast<int64_t>(kThreads) * kEpt;
    const int64_t nblk = (a.len + kPerBlk - 1) / kPerBlk;
    for (int64_t blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
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
                for (; r + kU <= a.nc; r += kU) {
                    u4 x[kU];
#pragma unroll
                    for (int u = 0; u < kU; ++u) x[u] = ldu4(a.c[r + u] + j0);
#pragma unroll
                    for (int u = 0; u < kU; ++u) add8<kPre>(acc, x[u], a);
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
                const int64_t j = blk * kPerBlk + static_cast<int64_t>(e) * kThreads + threadIdx.x;
                if (j < a.len) reduce_one<kPre>(a, j);
            }
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

template <bool kVec, bool kBf16>
__global__ __launch_bounds__(kThreads) void adamw_kernel(AdamArgs a) {
    constexpr int kEpt = 8;
    constexpr int64_t kPerBlk = static_cast<int64_t>(kThreads) * kEpt;
    const int64_t nblk = (a.len + kPerBlk - 1) / kPerBlk;
    for (int64_t blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
        if constexpr (kVec) {
            const int64_t j0 = blk * kPerBlk + static_cast<int64_t>(threadIdx.x) * kEpt;
            if (j0 + kEpt <= a.len) {
                f4 p[2], g[2], m[2], v[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    p[h] = ld4(a.p + j0 + 4 * h);
                    g[h] = ld4(a.g + j0 + 4 * h);
                    m[h] = ld4(a.m + j0 + 4 * h);
                    v[h] = ld4(a.v + j0 + 4 * h);
                }
                float pe[kEpt];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float pp = p[h][q], mm = m[h][q], vv = v[h][q];
                        adam1(pp, g[h][q], mm, vv, a.s);
                        p[h][q] = pp;
                        m[h][q] = mm;
                        v[h][q] = vv;
                        pe[4 * h + q] = pp;
                    }
                }
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    st4(a.p + j0 + 4 * h, p[h]);
                    st4(a.m + j0 + 4 * h, m[h]);
                    st4(a.v + j0 + 4 * h, v[h]);
                }
                if constexpr (kBf16)
                    stu4(a.pb + j0, u4{pack_bf16x2(pe[0], pe[1]), pack_bf16x2(pe[2], pe[3]),
                                       pack_bf16x2(pe[4], pe[5]), pack_bf16x2(pe[6], pe[7])});
            } else {
                for (int64_t j = j0; j < a.len && j < j0 + kEpt; ++j) adam_one(a, j);
            }
        } else {
#pragma unroll
            for (int e = 0; e < kEpt; ++e) {
                const int64_t j = blk * kPerBlk + static_cast<int64_t>(e) * kThreads + threadIdx.x;
                if (j < a.len) adam_one(a, j);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Upper bound on workgroups per launch (each workgroup then walks its tiles
// with a grid stride); large enough that every launch here is one tile per
// workgroup and the dispatcher balances the tail.
constexpr int64_t kMaxGrid = int64_t{1} << 30;

unsigned grid_for(int64_t work_items) {
    return static_cast<unsigned>(std::max<int64_t>(1, std::min(work_items, kMaxGrid)));
}

}  // namespace

hipError_t launch_segcopy(const std::vector<CopySeg>& segs, OutType out, hipStream_t stream) {
    const size_t out_size = out == OutType::kF32 ? 4 : 2;
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
            bool ok = aligned16(c.dst) && (c.nblk == 1 || (c.dst_stride * out_size) % 16 == 0);
            if (c.src)
                ok = ok && aligned16(c.src) && (c.nblk == 1 || (c.src_stride * 4) % 16 == 0);
            general = general || !ok;
        }
        if (t.nseg == 0) continue;
        t.ntiles = static_cast<uint32_t>(tiles);
        const dim3 grid(grid_for(static_cast<int64_t>(tiles))), block(kThreads);
        if (out == OutType::kF32) {
            if (general)
                hipLaunchKernelGGL((segcopy_kernel<float, true>), grid, block, 0, stream, t);
            else
                hipLaunchKernelGGL((segcopy_kernel<float, false>), grid, block, 0, stream, t);
        } else {
            if (general)
                hipLaunchKernelGGL((segcopy_kernel<uint16_t, true>), grid, block, 0, stream, t);
            else
                hipLaunchKernelGGL((segcopy_kernel<uint16_t, false>), grid, block, 0, stream, t);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
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
    bool vec = aligned16(out);
    for (int64_t r = 0; r < n_contrib; ++r) vec = vec && aligned16(contribs[r]);
    const int64_t per_blk = static_cast<int64_t>(kThreads) * 8;
    const dim3 grid(grid_for((len + per_blk - 1) / per_blk)), block(kThreads);
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
            hipLaunchKernelGGL((reduce_kernel<MODE, true>), grid, block, 0, stream, a);       \
        else                                                                                  \
            hipLaunchKernelGGL((reduce_kernel<MODE, false>), grid, block, 0, stream, a);      \
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
    const bool vec = aligned16(p) && aligned16(g) && aligned16(m) && aligned16(v) &&
                     (pb == nullptr || aligned16(pb));
    const int64_t per_blk = static_cast<int64_t>(kThreads) * 8;
    const dim3 grid(grid_for((len + per_blk - 1) / per_blk)), block(kThreads);
    if (vec) {
        if (pb) hipLaunchKernelGGL((adamw_kernel<true, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((adamw_kernel<true, false>), grid, block, 0, stream, a);
    } else {
        hipLaunchKernelGGL((adamw_kernel<false, false>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace fsdp
