// kernels.h -- launchers of the HIP kernels (host-callable, defined in kernels.hip).
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <vector>

#include "plan.h"

namespace fsdp {

// Element types moved by the segment-copy engine: source -> destination.
enum class Pipe { kF32toF32, kF32toBF16, kBF16toBF16 };

// Execute planned segments (null source = zero fill).  Splits into several
// launches if the table is larger than one kernel argument block holds.
hipError_t launch_segcopy(const std::vector<CopySeg>& segs, Pipe pipe, hipStream_t stream);

// fp32 reduction of `n_contrib` bf16 contributions of `len` elements each:
// in groups of `group` consecutive ranks (group == n_contrib: one flat sum),
// divided by pre (each term) and post (the total); with `accumulate` the
// result is added to what `out` holds.
hipError_t launch_grad_reduce(const uint16_t* const* contribs, int64_t n_contrib, int64_t len,
                              float pre, float post, int64_t group, bool accumulate, float* out,
                              hipStream_t stream);

// acc = (init ? 0 : acc) + fp32(grad), elementwise over len.
hipError_t launch_grad_accumulate(const uint16_t* grad, float* acc, int64_t len, bool init,
                                  hipStream_t stream);

// Derived AdamW scalars, each already rounded once to float on the host.
struct AdamScalars {
    float decay, b1, omb1, b2, omb2, step_size, bc2s, eps;
};

hipError_t launch_adamw(float* p, const float* g, float* m, float* v, uint16_t* pb, int64_t len,
                        const AdamScalars& s, hipStream_t stream);

// g *= inv_scale over len elements, in place; *found_inf = 1 if any input is not
// finite (never cleared).
hipError_t launch_grad_unscale(float* g, int64_t len, float inv_scale, float* found_inf,
                               hipStream_t stream);

// Tiles (= binary64 partial sums held in the workspace) of a sum of squares over runs.
int64_t sqnorm_tiles(const std::vector<ParamRun>& runs);

// out[i] = sum of g[runs[i].offset + j]^2 over j < runs[i].n, in binary64, for every
// run i (0 for an empty run); `partial` holds sqnorm_tiles(runs) doubles.
hipError_t launch_grad_sqnorm(const float* g, const std::vector<ParamRun>& runs, double* partial,
                              double* out, hipStream_t stream);

}  // namespace fsdp
