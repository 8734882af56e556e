/*
 * fsdp_flatten.h -- C ABI of the per-rank FSDP data path on MI355X (gfx950).
 *
 * One rank's share of one FSDP unit: shard the unit's parameters, copy a
 * gathered unit out into per-parameter bf16 tensors, reduce the N ranks' bf16
 * gradient contributions for this rank's shard in fp32, and run AdamW on the
 * shard.  Every call runs hand-written HIP kernels on the caller's stream.
 *
 * Sources (sections as named on each page):
 *   [P1] "PyTorch FSDP: Experiences on Scaling Fully Sharded Data Parallel"
 *   [P2] "FSDP Under The Hood: ZeRO-3 The PyTorch Way"
 *   [P3] "FSDP Architecture"
 *   [P4] "FSDP (Fully Sharded Data Parallel)"
 *
 * Conventions for every call
 *   - Sizes and offsets are int64 element counts.  fp32 data is `float`; bf16
 *     data is passed as its 16-bit pattern (`uint16_t`).
 *   - "Device pointer" means memory the GPU can read or write (hipMalloc'd,
 *     e.g. a torch CUDA tensor's data_ptr()).  Tables of device pointers
 *     (`params`, `outs`, `contribs`) are HOST arrays whose entries are device
 *     pointers; the library reads the host array during the call only.
 *   - The caller owns every buffer.  The data calls allocate no device
 *     memory, free nothing and do not synchronise: they enqueue kernels on
 *     `stream` (a hipStream_t; NULL is the default stream) and return.
 *     Buffers must stay alive until that work has finished.
 *   - Errors: every argument is validated on the host, before any HIP call;
 *     a call that returns any status but FSDP_OK or FSDP_E_HIP has launched
 *     nothing and written nothing.  FSDP_E_HIP means a launch failed
 *     (hipGetLastError); a call that launches several kernels may have
 *     enqueued the ones before it.  Faults inside kernels surface at the
 *     caller's next synchronisation, as for any HIP work.  fsdp_last_error()
 *     returns a message for the calling thread's last non-OK status.
 *   - Pointer alignment is not an error: data at least 4-byte aligned is read
 *     with 16-byte loads where it sits (a scalar head first aligns outputs),
 *     and bf16 data at odd element offsets is realigned in the kernels.
 *     Misaligned below the element size is FSDP_E_ALIGN.
 *   - No call allocates device memory, synchronises or records a memset, so
 *     every call can be captured in a HIP graph and replayed.  Calls build
 *     small host tables; if host memory runs out they return FSDP_E_NOMEM.
 *     No C++ exception leaves the library.
 *   - Inputs and outputs must not overlap, except that fsdp_adam_shard updates
 *     param, exp_avg and exp_avg_sq in place.
 *   - A unit with no elements makes every call a no-op that returns FSDP_OK.
 */
#ifndef FSDP_FLATTEN_H
#define FSDP_FLATTEN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Symbols of the ABI are the only ones the library exports. */
#if defined(__GNUC__) || defined(__clang__)
#define FSDP_API __attribute__((visibility("default")))
#else
#define FSDP_API
#endif

#define FSDP_ABI_VERSION 3
#define FSDP_ALL_RANKS (-1)
#define FSDP_MAX_NDIM 8

typedef enum {
    FSDP_OK = 0,
    FSDP_E_ARG = 1,          /* null or inconsistent argument                 */
    FSDP_E_RANGE = 2,        /* value out of its range (N, k, beta, step ...) */
    FSDP_E_ALIGN = 3,        /* pointer not aligned to its element size       */
    FSDP_E_OVERFLOW = 4,     /* a size overflows int64                        */
    FSDP_E_NOMEM = 5,        /* host memory exhausted (plan or launch tables) */
    FSDP_E_HIP = 6,          /* a HIP runtime call or kernel launch failed    */
    FSDP_E_UNSUPPORTED = 7   /* valid request the library does not handle     */
} fsdp_status;

/* How a unit is sharded. */
typedef enum {
    /* FSDP1 FlatParameter ([P1] section 3.4, "FlatParameter: Flattening,
     * Concatenation, and Sharding", Fig. 3): the parameters are flattened
     * row-major, concatenated in list order into T elements, right-padded
     * with +0.0 to L = N*S where S = ceil(T/N), and rank k owns elements
     * [k*S, (k+1)*S) ([P1] section 3.4, "Sharding Strategies").              */
    FSDP_FLAT = 1,
    /* FSDP2 per-parameter dim-0 sharding ([P2] section 2, "Sharding geometry";
     * [P4] "FSDP1 vs FSDP2", torch.chunk(dim=0)): parameter i with m_i rows of
     * r_i elements (a 0-d parameter is 1 row of 1) is cut into chunks of
     * c_i = ceil(m_i/N) rows; rank k holds rows [min(m_i,k*c_i),
     * min(m_i,(k+1)*c_i)).  Rank k's segment has P_r = sum_i c_i*r_i
     * elements: the parameters in order, each zero-padded to c_i rows, so
     * every rank sends an equal AllGather input.  A gathered buffer holds the
     * N segments in rank order (N*P_r elements).                              */
    FSDP_ROWS = 2
} fsdp_layout;

/* Opaque plan of one unit (the analogue of a FlatParamHandle, [P1] section
 * 3.4): parameter shapes, offsets and sizes.  Host memory only. */
typedef struct fsdp_unit fsdp_unit;

typedef struct {
    int32_t layout;        /* FSDP_FLAT or FSDP_ROWS                           */
    int32_t n_params;      /* p                                                */
    int64_t N;             /* shard count                                      */
    int64_t T;             /* elements of the unit (sum of numel)              */
    int64_t S;             /* elements of one rank's shard (FLAT: ceil(T/N);
                              ROWS: P_r)                                       */
    int64_t L;             /* N*S: elements of the gathered buffer             */
    int64_t pad;           /* L - T                                            */
    int64_t valid;         /* elements of rank k's shard that are real data
                              (not padding); 0 when k == FSDP_ALL_RANKS        */
    int64_t bytes_per_rank;/* steady-state bytes rank k keeps for this unit:
                              fp32 param 4S + fp32 grad 4S + Adam m,v 8S
                              ([P3] per-GPU memory breakdown, 16P/N)           */
} fsdp_unit_sizes;

/* AdamW hyper-parameters.  The scalars derived from them are computed in
 * double on the host and rounded once to float (see fsdp_adam_shard). */
typedef struct {
    double lr;             /* finite                                           */
    double beta1;          /* [0, 1)                                           */
    double beta2;          /* [0, 1)                                           */
    double eps;            /* finite, >= 0                                     */
    double weight_decay;   /* finite                                           */
    int64_t step;          /* t >= 1: the step being taken (1 for the first)   */
} fsdp_adamw_cfg;

/* Which kernel fsdp_grad_reduce_shard_ex runs (fsdp_reduce_opts.kernel). */
typedef enum {
    /* The library's choice: the row-major sweep when a launch holds 32 or more ranks and
     * the shard 12,288 or more whole 512-output tiles (about 6.3 M outputs), else the
     * tile kernel.  The sweep sizes its grid to be resident on an otherwise idle device;
     * when kernels on other streams hold compute units, its waves that do not fit start
     * only as others finish, and a shard long enough to take two launches then finishes
     * well after the tile kernel would (beside a batch of GEMMs on MI355X: 1.8-1.9 ms
     * against 1.06-1.10 ms for a 128-rank GPT-175B shard, 0.53 against 0.61 ms alone).
     * A caller that overlaps the reduction with compute and needs its result early
     * chooses FSDP_REDUCE_TILES. */
    FSDP_REDUCE_AUTO = 0,
    /* The tile kernel: one 512-output tile per 64-thread workgroup, many short
     * workgroups, which fill whatever compute units are free. */
    FSDP_REDUCE_TILES = 1,
    /* The row-major sweep wherever its loads apply (every contribution 4-byte aligned,
     * grad_shard and workspace 16-byte aligned, at least one sweep wave of whole tiles);
     * the tile kernel otherwise. */
    FSDP_REDUCE_SWEEP = 2
} fsdp_reduce_kernel;

/* Options of fsdp_grad_reduce_shard_ex. */
typedef struct {
    float pre_divide;      /* finite, non-zero: divides every term before it is added     */
    float post_divide;     /* finite, non-zero: divides the total                         */
    int32_t group;         /* ranks per sharding group (hybrid sharding).  0, 1 or N: one
                              flat sequential sum; otherwise it must divide N             */
    int32_t accumulate;    /* non-zero: add the result to what grad_shard already holds   */
    int32_t kernel;        /* an fsdp_reduce_kernel (0: FSDP_REDUCE_AUTO)                 */
    int32_t reserved;      /* ignored; set it to 0                                        */
    float* workspace;      /* device pointer, 16-byte aligned: fp32 scratch of at least
                              fsdp_grad_reduce_workspace floats, or NULL when that is 0  */
    int64_t workspace_len; /* floats the workspace holds                                  */
} fsdp_reduce_opts;

/* Version of this header the library was built from (FSDP_ABI_VERSION). */
FSDP_API int32_t fsdp_abi_version(void);

/* Message for the calling thread's last non-OK status ("" if none).  The
 * string stays valid until the thread's next call into the library. */
FSDP_API const char* fsdp_last_error(void);

/* Short fixed name of a status code ("FSDP_OK", "FSDP_E_ARG", ...). */
FSDP_API const char* fsdp_status_string(int32_t status);

/*
 * Plan a unit.  n_params >= 0 parameters; parameter i has ndims[i] in
 * [0, FSDP_MAX_NDIM] dimensions, taken in order from `dims` (so `dims` holds
 * sum(ndims) entries, each >= 0).  N >= 1.  On success *out receives a handle
 * that the caller frees with fsdp_unit_destroy.  Allocates host memory only;
 * makes no HIP call.  Errors: FSDP_E_ARG (null out, null ndims with
 * n_params > 0, or null dims when sum(ndims) > 0), FSDP_E_RANGE (layout, N,
 * n_params, a dim or ndim out of range), FSDP_E_OVERFLOW (a size beyond
 * int64), FSDP_E_NOMEM.
 */
FSDP_API fsdp_status fsdp_unit_create(int32_t layout, int32_t n_params, const int32_t* ndims,
                             const int64_t* dims, int32_t N, fsdp_unit** out);

/* Free a unit.  Work already enqueued does not use the unit (every call copies
 * what its kernels need into their arguments), so no synchronisation is
 * needed first.  NULL is accepted.  Always returns FSDP_OK. */
FSDP_API fsdp_status fsdp_unit_destroy(fsdp_unit* unit);

/* Sizes of the unit, and of rank k's shard (k in [0,N) or FSDP_ALL_RANKS).
 * Host only.  Errors: FSDP_E_ARG (NULL unit or out), FSDP_E_RANGE (k). */
FSDP_API fsdp_status fsdp_unit_info(const fsdp_unit* unit, int32_t k, fsdp_unit_sizes* out);

/* Element offset of parameter i inside the FLAT flat buffer, or inside every
 * rank's ROWS segment (the q_i of FSDP_ROWS).  Host only.  Errors: FSDP_E_ARG
 * (NULL unit or offset), FSDP_E_RANGE (i outside [0, n_params)). */
FSDP_API fsdp_status fsdp_unit_param_offset(const fsdp_unit* unit, int32_t i, int64_t* offset);

/* Recommended row pitch, in elements, of a stacked [N][pitch] bf16 buffer that
 * receives the N gradient contributions of fsdp_grad_reduce_shard (row r holds
 * contribution r in its first S elements): S rounded up to a whole 128-byte
 * line (a multiple of 64 elements).  The reduction reads each contribution in
 * runs of 16 KiB (32 or more ranks, long shards) or 1 KiB (otherwise); a row
 * that starts mid-line touches one more line per run (at N = 128 on the
 * GPT-175B block: 0.45% more HBM reads and a 1% slower reduction than
 * line-aligned rows; 6.25% and 6% with 1 KiB runs).  Any layout works; this
 * one is fastest.
 * Host only.  Errors: FSDP_E_ARG (null unit or pitch). */
FSDP_API fsdp_status fsdp_unit_recv_pitch(const fsdp_unit* unit, int64_t* pitch);

/*
 * Shard a unit ([P1] section 3.4, FlatParameter, Fig. 3; [P2] section 2).
 *   params : host array of n_params device pointers, parameter i holding
 *            numel_i contiguous fp32 elements (row-major); entries of
 *            zero-size parameters may be NULL.
 *   k      : rank in [0, N), or FSDP_ALL_RANKS to write every rank's shard
 *            one after another (the gathered layout, L elements).
 *   shard  : device pointer, S fp32 elements (L for FSDP_ALL_RANKS).
 * FLAT writes shard[j] = F[k*S + j] with F the padded flat buffer; ROWS writes
 * rank k's segment (its rows of every parameter, zero rows up to c_i).
 * Results are bit-exact copies.
 * Errors: FSDP_E_ARG (NULL unit; NULL params table or entry of a non-empty
 * parameter; NULL shard with elements to write), FSDP_E_RANGE (k neither in
 * [0, N) nor FSDP_ALL_RANKS), FSDP_E_ALIGN (a pointer not 4-byte aligned),
 * FSDP_E_NOMEM, FSDP_E_HIP.
 */
FSDP_API fsdp_status fsdp_flatten_shard(const fsdp_unit* unit, const float* const* params, int32_t k,
                               float* shard, void* stream);

/*
 * Copy a gathered unit out into per-parameter bf16 tensors with an fp32->bf16
 * cast, round to nearest even, NaN kept NaN ([P1] section 3.4, "Native Mixed
 * Precision and the Sharded Gradient Scaler": one full-to-low cast per
 * FlatParameter; [P1] section 3.4, "Autograd Integration": parameters are
 * split views of the unsharded FlatParameter; [P2] section 4, bf16 compute
 * params).
 *   gathered : device pointer, L fp32 elements (the N shards in rank order).
 *              FLAT padding is never read.
 *   outs     : host array of n_params device pointers, output i holding numel_i
 *              bf16 elements (NULL allowed for zero-size parameters).
 * Errors: FSDP_E_ARG (NULL unit; NULL gathered with T > 0; NULL outs table or
 * entry of a non-empty parameter), FSDP_E_ALIGN (gathered not 4-byte or an
 * output not 2-byte aligned), FSDP_E_NOMEM, FSDP_E_HIP.
 */
FSDP_API fsdp_status fsdp_unflatten_copyout(const fsdp_unit* unit, const float* gathered,
                                   uint16_t* const* outs, void* stream);

/*
 * Reduce the N ranks' bf16 gradient contributions for one shard in fp32
 * ([P1] section 3.4, "Sharding Strategies" and "Communication layout": the
 * ReduceScatter sums and rank k keeps its chunk; [P1] "Native Mixed
 * Precision": low-precision collectives; [P2] section 3 and section 4:
 * reduce_dtype fp32).
 *   contribs    : host array of N device pointers; contribs[r] holds rank r's
 *                 S bf16 gradient elements for this shard.
 *   pre_divide  : finite, non-zero; divides every term before it is added.
 *   post_divide : finite, non-zero; divides the sum.
 *   grad_shard  : device pointer, S fp32 outputs.
 * out[j] = ((c_0[j]/pre + c_1[j]/pre) + ... + c_{N-1}[j]/pre) / post, each
 * operation one rounded binary32 operation, summed in rank order from rank 0.
 * Errors: FSDP_E_ARG (NULL unit; with S > 0, a NULL contribs table or entry, or
 * a NULL grad_shard), FSDP_E_RANGE (pre_divide or post_divide zero or not
 * finite), FSDP_E_ALIGN (a contribution not 2-byte or grad_shard not 4-byte
 * aligned), FSDP_E_NOMEM, FSDP_E_HIP.
 */
FSDP_API fsdp_status fsdp_grad_reduce_shard(const fsdp_unit* unit, const uint16_t* const* contribs,
                                   float pre_divide, float post_divide, float* grad_shard,
                                   void* stream);

/*
 * One AdamW step on rank-local, position-aligned shards ([P3]: parameter,
 * gradient and both Adam moments are kept for the same positions and updated
 * with no communication; [P1] section 3.2; [P2] appendix, torch.optim.AdamW).
 *   param, exp_avg, exp_avg_sq : device pointers, S fp32 each, updated in place.
 *   grad        : device pointer, S fp32.
 *   cfg         : host pointer, read during the call.
 *   param_bf16  : device pointer to S bf16 outputs receiving bf16(new param),
 *                 or NULL.
 * Scalars (double, rounded once to float): decay = 1 - lr*wd,
 * step_size = lr/(1 - beta1^t), bc2s = sqrt(1 - beta2^t).  Per element, each
 * a rounded binary32 operation: p = p*decay; m = beta1*m + (1-beta1)*g;
 * v = beta2*v + (1-beta2)*(g*g); p = p - step_size*(m/(sqrt(v)/bc2s + eps)).
 * Errors: FSDP_E_ARG (NULL unit or cfg; with S > 0, a NULL param, grad,
 * exp_avg or exp_avg_sq), FSDP_E_RANGE (step < 1; beta1 or beta2 outside
 * [0, 1); lr or weight_decay not finite; eps negative or not finite),
 * FSDP_E_ALIGN (an fp32 pointer not 4-byte or param_bf16 not 2-byte aligned),
 * FSDP_E_NOMEM, FSDP_E_HIP.
 */
FSDP_API fsdp_status fsdp_adam_shard(const fsdp_unit* unit, float* param, const float* grad,
                            float* exp_avg, float* exp_avg_sq, const fsdp_adamw_cfg* cfg,
                            uint16_t* param_bf16, void* stream);

/* ------------------------------------------------------------------------
 * Beyond the four calls: casting before the gather, the FSDP2 copy-in,
 * gradient accumulation and hybrid sharding.
 * ------------------------------------------------------------------------ */

/*
 * Cast fp32 to bf16 (round to nearest even, NaN kept NaN) over rank k's shard
 * (S elements) or, with k == FSDP_ALL_RANKS, over the whole gathered / unsharded
 * layout (L elements).  The pages cast the full-precision shard to low
 * precision once per FlatParameter and all-gather the low-precision copy
 * ([P1] section 3.4, "Native Mixed Precision and the Sharded Gradient Scaler";
 * [P2] section 5: FSDP2 gathers the bf16 copy); the same cast turns an
 * fp32-accumulated gradient into the bf16 ReduceScatter input.
 *   src : device pointer, fp32.   dst : device pointer, bf16 (same count).
 * Errors: FSDP_E_ARG (NULL unit; NULL src or dst with elements to cast),
 * FSDP_E_RANGE (k), FSDP_E_ALIGN, FSDP_E_NOMEM, FSDP_E_HIP.
 */
FSDP_API fsdp_status fsdp_cast_to_bf16(const fsdp_unit* unit, int32_t k, const float* src,
                                       uint16_t* dst, void* stream);

/*
 * Copy a gathered bf16 unit (the AllGather of bf16 shards: L elements, FLAT
 * padding never read, or N*P_r for ROWS) out into per-parameter bf16 tensors --
 * the copy-out of fsdp_unflatten_copyout when the cast happened before the
 * gather.  Bit-identical to casting after the gather.
 *   gathered : device pointer, bf16.   outs : host array of n_params device
 *   pointers, bf16, numel_i each (NULL allowed for zero-size parameters).
 * Errors as fsdp_unflatten_copyout (gathered 2-byte aligned).
 */
FSDP_API fsdp_status fsdp_unflatten_copyout_bf16(const fsdp_unit* unit, const uint16_t* gathered,
                                                 uint16_t* const* outs, void* stream);

/*
 * fsdp_flatten_shard for bf16 tensors.  With k == FSDP_ALL_RANKS on the
 * per-parameter bf16 gradients this is the FSDP2 copy-in: it writes the
 * ReduceScatter input, every rank's segment in rank order with each
 * parameter's rows padded to c_i rows by zeros ([P2] section 3: gradients
 * reduce-scatter per parameter; [P1] section 3.4, "Communication layout":
 * the unsharded gradient in the FlatParameter layout for FSDP1).
 *   params : host array of n_params device pointers, bf16.
 *   shard  : device pointer, bf16, S elements (L for FSDP_ALL_RANKS).
 * Errors as fsdp_flatten_shard (pointers 2-byte aligned).
 */
FSDP_API fsdp_status fsdp_flatten_shard_bf16(const fsdp_unit* unit, const uint16_t* const* params,
                                             int32_t k, uint16_t* shard, void* stream);

/*
 * fsdp_grad_reduce_shard with hybrid sharding, accumulation and a choice of kernel.
 * Hybrid sharding ([P1] section 3.4, "Sharding Strategies": a ReduceScatter
 * inside each sharding group, then an AllReduce across the replication
 * groups; the sum over all ranks equals the sum of the group sums): the N
 * contributions form N/group groups of consecutive ranks; each group is summed
 * in rank order, then the group sums in group order; then / post_divide.
 * Accumulation with communication ([P1] section 3.4, "Communication
 * Optimizations: Overlapping, Prefetching, and Accumulation", "Gradient
 * Accumulation Variants"): out = out + result.
 * Any N and group: one kernel launch holds up to 128 ranks, and the sums a
 * longer reduction carries from one launch to the next are stored exactly
 * (results do not depend on the split).  The output carries them, except
 * when it must keep its old value (accumulate) or a group is longer than one
 * launch: then they go to the caller's workspace (see
 * fsdp_grad_reduce_workspace; calls that share a workspace on one stream run
 * in order, on different streams they must not share one).  The workspace
 * must not overlap grad_shard or any contribution (not checked).
 * Errors as fsdp_grad_reduce_shard, plus FSDP_E_ARG (opts NULL; workspace NULL
 * when one is needed), FSDP_E_RANGE (group does not divide N; kernel not an
 * fsdp_reduce_kernel; workspace_len below what is needed) and FSDP_E_ALIGN
 * (workspace not 16-byte aligned when one is needed).
 */
FSDP_API fsdp_status fsdp_grad_reduce_shard_ex(const fsdp_unit* unit, const uint16_t* const* contribs,
                                               const fsdp_reduce_opts* opts, float* grad_shard,
                                               void* stream);

/*
 * Floats of workspace fsdp_grad_reduce_shard_ex needs for these options (its
 * group and accumulate; the other fields are not read): 0 when N <= 128, or
 * when neither accumulating nor hybrid with groups of more than 128 ranks;
 * else one or two slots of S rounded up to 64 floats (two when accumulating
 * with groups of more than 128 ranks).  Host only.
 * Errors: FSDP_E_ARG (NULL unit, opts or n_floats), FSDP_E_RANGE (group).
 */
FSDP_API fsdp_status fsdp_grad_reduce_workspace(const fsdp_unit* unit, const fsdp_reduce_opts* opts,
                                                int64_t* n_floats);

/*
 * Gradient accumulation without communication ([P1] section 3.4, "Gradient
 * Accumulation Variants": each rank accumulates the unsharded gradient
 * locally and reduces once, on the last micro-batch):
 * acc[j] = (init ? 0 : acc[j]) + fp32(grad[j]) over rank k's shard (S elements)
 * or, with k == FSDP_ALL_RANKS, the whole unsharded layout (L elements).
 *   grad : device pointer, bf16.   acc : device pointer, fp32, updated in place.
 * Errors: FSDP_E_ARG (NULL unit; NULL grad or acc with elements to add),
 * FSDP_E_RANGE (k), FSDP_E_ALIGN, FSDP_E_NOMEM, FSDP_E_HIP.
 */
FSDP_API fsdp_status fsdp_grad_accumulate(const fsdp_unit* unit, int32_t k, const uint16_t* grad,
                                          float* acc, int32_t init, void* stream);

/*
 * Sharded gradient scaler, the per-rank half ([P1] section 3.4 "Native Mixed
 * Precision and the Sharded Gradient Scaler": the scale is global, so every
 * rank unscales its own shard by the same factor, and overflow detection must
 * be combined across ranks so that all of them skip or take the step):
 *   grad[j] = grad[j] * inv_scale   (one rounded binary32 multiply)
 * over rank k's shard (S elements) or, with k == FSDP_ALL_RANKS, the whole
 * layout (L elements), and *found_inf = 1.0f if any grad[j] was not finite
 * before the multiply.  The flag is never cleared here: the caller zeroes it,
 * may share it between several shards, and combines it across ranks (a max
 * all-reduce).
 *   grad      : device pointer, fp32, updated in place.
 *   inv_scale : finite.
 *   found_inf : device pointer to one float, or NULL to scale only (the
 *               clip-coefficient multiply of gradient clipping: after the
 *               norms of fsdp_grad_sqnorm are combined across ranks, every rank
 *               scales its shard by the same coefficient).
 * Errors: FSDP_E_ARG (NULL unit or grad; inv_scale not finite), FSDP_E_RANGE
 * (k), FSDP_E_ALIGN, FSDP_E_HIP.  With no elements (an empty unit) nothing is
 * launched and grad may be NULL.
 */
FSDP_API fsdp_status fsdp_grad_unscale(const fsdp_unit* unit, int32_t k, float* grad,
                                       float inv_scale, float* found_inf, void* stream);

/* Doubles of workspace fsdp_grad_sqnorm needs for rank k (k in [0, N)):
 * one binary64 partial per 4096-element tile of each parameter's run. */
FSDP_API fsdp_status fsdp_grad_sqnorm_workspace(const fsdp_unit* unit, int32_t k,
                                                int64_t* n_doubles);

/*
 * Per-parameter sums of squares of rank k's gradient shard.  The pages note
 * that statistics of original parameters (gradient-clipping norms, per-
 * parameter optimizer statistics) are wrong when taken over flat shards, which
 * ignore parameter boundaries ([P1] section 6, the mathematical-equivalence
 * limitation).  The unit plan knows the boundaries, so
 *   out[i] = sum of grad[j]^2 over the shard elements of parameter i
 * (padding belongs to no parameter; FSDP2 zero rows are not counted), each
 * square and sum in binary64.  Summed over the N ranks (one all-reduce of
 * n_params doubles) out[i] is parameter i's squared gradient norm, and the
 * sum over i the global squared norm that clipping needs.
 * Deterministic for a given unit and rank: every tile is summed in a fixed
 * order into the workspace, then each parameter's tiles in a fixed order.
 *   grad      : device pointer, fp32, S elements (k in [0, N)).
 *   workspace : device pointer, at least fsdp_grad_sqnorm_workspace doubles,
 *               overwritten; workspace_len its length in doubles.
 *   out       : device pointer, n_params doubles, written (0 for parameters
 *               the rank holds none of).
 * Calls that share a workspace on one stream run in order; on different
 * streams they must not share one.
 * Errors: FSDP_E_ARG (NULL pointers), FSDP_E_RANGE (k, or workspace_len too
 * small), FSDP_E_ALIGN, FSDP_E_HIP.
 */
FSDP_API fsdp_status fsdp_grad_sqnorm(const fsdp_unit* unit, int32_t k, const float* grad,
                                      double* workspace, int64_t workspace_len, double* out,
                                      void* stream);

/*
 * fsdp_grad_sqnorm for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * per-parameter sums of squares, bit for bit, with the partial sums kept in the
 * library's own scratch instead of a caller's workspace.  The scratch is one fixed
 * array of 262,144 doubles (2 MiB) on each GPU the library runs on, held until the
 * process ends; its address is looked up on the first call on each device.  It keeps
 * the last call's contents and needs no clearing: every partial sum a call reads, the
 * same call has written first.  Calls that run at the same time on one GPU (other
 * streams, other threads) share the array and race: order them, or give each its own
 * workspace through fsdp_grad_sqnorm.  Allocates no device memory (it builds small host
 * tables, as every call does).
 *   grad : device pointer, fp32, S elements (k in [0, N)).
 *   out  : device pointer, n_params doubles, written.
 * Errors: FSDP_E_ARG (NULL pointers), FSDP_E_RANGE (k, or rank k's shard needs more
 * than 262,144 partial sums: more than 2^30 elements, or runs of many parameters whose
 * 4096-element tiles add up past that), FSDP_E_ALIGN, FSDP_E_HIP (the scratch's address
 * cannot be obtained, or a launch failed).
 */
FSDP_API fsdp_status fsdp_grad_sqnorm_noalloc(const fsdp_unit* unit, int32_t k, const float* grad,
                                              double* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FSDP_FLATTEN_H */
