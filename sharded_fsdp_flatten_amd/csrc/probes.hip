// probes.hip -- hardware floor probes for the benchmark (libfsdpprobe.so).
//
// Not part of the data path: these kernels let the benchmark split the duration of a
// short cold-cache copy (the flatten of one rank's shard) into what any kernel of that
// shape pays and what the copy itself costs.  Each has the flatten's launch shape: one
// tile of 1024 fp32 per 256-thread workgroup, 16-byte vector accesses, loads marked
// non-temporal and whole tiles stored with device-scope non-temporal buffer stores (the
// data path's copy engine stores the same way).
//   empty : the grid alone (dispatch, wave start and end, no memory access);
//   read  : the loads alone (a data-dependent store that never fires keeps them live);
//   write : the stores alone;
//   copy  : loads then stores with no segment table and no lookup.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int64_t kTile = 4 * kThreads;  // fp32 elements per workgroup
constexpr int kStoreCpol = 18;           // sc1 (device scope) + nt

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(float* base) {
    const uint64_t b = reinterpret_cast<uintptr_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32));
    return __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo), 0,
        static_cast<int>(kTile * 4), 0x00020000);
}

__global__ __launch_bounds__(kThreads) void probe_empty_kernel() {}

// n is a multiple of 4; the last tile may be partial.
__global__ __launch_bounds__(kThreads) void probe_read_kernel(const float* __restrict__ s, int64_t n,
                                                              float* __restrict__ sink) {
    const int64_t e = static_cast<int64_t>(blockIdx.x) * kTile + 4 * threadIdx.x;
    if (e >= n) return;
    const f4 x = __builtin_nontemporal_load(reinterpret_cast<const f4*>(s + e));
    // a test of the loaded values that the compiler cannot decide (a test of their bit
    // patterns was folded away, loads included)
    const float t = x[0] + x[1] + x[2] + x[3];
    if (t == 1234.5f) *sink = t;
}

__global__ __launch_bounds__(kThreads) void probe_write_kernel(float* __restrict__ d, int64_t n) {
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kTile;
    const f4 z = {1.0f, 2.0f, 3.0f, 4.0f};
    if (t0 + kTile <= n) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, z), tile_rsrc(d + t0),
                                               16 * threadIdx.x, 0, kStoreCpol);
        return;
    }
    const int64_t e = t0 + 4 * threadIdx.x;
    if (e < n) __builtin_nontemporal_store(z, reinterpret_cast<f4*>(d + e));
}

__global__ __launch_bounds__(kThreads) void probe_copy_kernel(const float* __restrict__ s,
                                                              float* __restrict__ d, int64_t n) {
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kTile;
    const int64_t e = t0 + 4 * threadIdx.x;
    if (e >= n) return;
    const f4 x = __builtin_nontemporal_load(reinterpret_cast<const f4*>(s + e));
    if (t0 + kTile <= n) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, x), tile_rsrc(d + t0),
                                               16 * threadIdx.x, 0, kStoreCpol);
        return;
    }
    __builtin_nontemporal_store(x, reinterpret_cast<f4*>(d + e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Workgroups covering n elements; 0 when n is unusable (see the entry points).
int64_t tiles_of(int64_t n) { return (n + kTile - 1) / kTile; }

int launched() { return hipGetLastError() == hipSuccess ? 0 : 3; }

}  // namespace

// Return codes: 0 launched; 1 bad size (n must be positive, a multiple of 4 and at most
// 2^31 - 1 tiles; threads in [1, 1024]); 2 a pointer NULL or not 16-byte aligned; 3 the
// launch failed.
extern "C" {

__attribute__((visibility("default"))) int fsdp_probe_empty(int64_t blocks, int32_t threads,
                                                            void* stream) {
    if (blocks < 1 || blocks > 0x7FFFFFFF || threads < 1 || threads > kThreads) return 1;
    hipLaunchKernelGGL(probe_empty_kernel, dim3(static_cast<unsigned>(blocks)),
                       dim3(static_cast<unsigned>(threads)), 0, static_cast<hipStream_t>(stream));
    return launched();
}

__attribute__((visibility("default"))) int fsdp_probe_read(const float* src, int64_t n, float* sink,
                                                           void* stream) {
    if (n < 4 || n % 4 != 0 || tiles_of(n) > 0x7FFFFFFF) return 1;
    if (!src || !sink || !aligned16(src)) return 2;
    hipLaunchKernelGGL(probe_read_kernel, dim3(static_cast<unsigned>(tiles_of(n))), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), src, n, sink);
    return launched();
}

__attribute__((visibility("default"))) int fsdp_probe_write(float* dst, int64_t n, void* stream) {
    if (n < 4 || n % 4 != 0 || tiles_of(n) > 0x7FFFFFFF) return 1;
    if (!dst || !aligned16(dst)) return 2;
    hipLaunchKernelGGL(probe_write_kernel, dim3(static_cast<unsigned>(tiles_of(n))), dim3(kThreads),
                       0, static_cast<hipStream_t>(stream), dst, n);
    return launched();
}

__attribute__((visibility("default"))) int fsdp_probe_copy(const float* src, float* dst, int64_t n,
                                                           void* stream) {
    if (n < 4 || n % 4 != 0 || tiles_of(n) > 0x7FFFFFFF) return 1;
    if (!src || !dst || !aligned16(src) || !aligned16(dst)) return 2;
    hipLaunchKernelGGL(probe_copy_kernel, dim3(static_cast<unsigned>(tiles_of(n))), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), src, dst, n);
    return launched();
}

}  // extern "C"
