// kernels.h -- launchers of the HIP kernels (host-callable, defined in kernels.hip).
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <vector>

#include "plan.h"

namespace fsdp {

// Element type written by the segment-copy engine.
enum class OutType { kF32, kBF16 };

// Execute planned segments (fp32 sources; fp32 or bf16 destinations; null
// source = zero fill).  Splits into several launches if the table is larger
// than one kernel argument block holds.
hipError_t launch_segcopy(const std::vector<CopySeg>& segs, OutType out, hipStream_t stream);

// fp32 reduction of `n_contrib` bf16 contributions of `len` elements each.
hipError_t launch_grad_reduce(const uint16_t* const* contribs, int64_t n_contrib, int64_t len,
                              float pre, float post, float* out, hipStream_t stream);

// Derived AdamW scalars, each already rounded once to float on the host.
struct AdamScalars {
    float decay, b1, omb1, b2, omb2, step_size, bc2s, eps;
};

hipError_t launch_adamw(float* p, const float* g, float* m, float* v, uint16_t* pb, int64_t len,
                        const AdamScalars& s, hipStream_t stream);

}  // namespace fsdp
