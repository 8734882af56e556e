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

// Which reduction kernel runs: the default choice (the row-major sweep for many ranks and
// long outputs, else the tile kernel), the tile kernel only, or the sweep wherever its loads
// apply (every contribution 4-byte aligned, the output and workspace 16-byte aligned, at
// least one sweep wave of whole tiles).
enum class ReduceKernel { kAuto = 0, kTiles = 1, kSweep = 2 };

// Floats of workspace launch_grad_reduce needs (0: none): the sums it carries between
// launches when the ranks do not fit one launch and the output cannot carry them.
int64_t reduce_workspace_floats(int64_t n_contrib, int64_t len, int64_t group, bool accumulate);

// fp32 reduction of `n_contrib` bf16 contributions of `len` elements each:
// in groups of `group` consecutive ranks (group <= 1 or >= n_contrib: one flat sum),
// divided by pre (each term) and post (the total); with `accumulate` the
// result is added to what `out` holds.  `workspace` holds reduce_workspace_floats
// floats (16-byte aligned), or is unused when that is 0.
hipError_t launch_grad_reduce(const uint16_t* const* contribs, int64_t n_contrib, int64_t len,
                              float pre, float post, int64_t group, bool accumulate, float* out,
                              float* workspace, ReduceKernel kernel, hipStream_t stream);

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

// The library's own scratch for the partial sums of launch_grad_sqnorm, for callers that
// cannot allocate: sqnorm_scratch_doubles() doubles per GPU; *out receives the current
// device's copy (looked up on the first call on each device).  Calls that use it at the
// same time on one GPU race.
int64_t sqnorm_scratch_doubles();
hipError_t sqnorm_scratch(double** out);

}  // namespace fsdp
