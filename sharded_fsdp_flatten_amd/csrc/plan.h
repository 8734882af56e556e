// plan.h -- host-side unit planner: sizes, offsets and the copy segments that the
// data-movement kernels execute.  Pure integer arithmetic; no HIP.
//
// Layouts follow "PyTorch FSDP: Experiences on Scaling Fully Sharded Data
// Parallel" section 3.4 ("FlatParameter: Flattening, Concatenation, and
// Sharding", Fig. 3) for FSDP1 and "FSDP Under The Hood: ZeRO-3 The PyTorch Way"
// section 2 ("Sharding geometry") with torch.chunk(dim=0) semantics for FSDP2.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace fsdp {

enum Layout : int32_t { kFlat = 1, kRows = 2 };

struct ParamPlan {
    std::vector<int64_t> shape;
    int64_t numel = 0;
    int64_t rows = 0;        // m: length of dim 0 (1 for a 0-d parameter)
    int64_t row_len = 0;     // r: elements per row (product of trailing dims)
    int64_t chunk_rows = 0;  // c = ceil(m/N) (FSDP2)
    int64_t offset = 0;      // FLAT: first flat index; ROWS: offset q_i inside a rank segment
};

struct UnitPlan {
    int32_t layout = kFlat;
    int64_t N = 1;
    int64_t T = 0;    // elements of the unit
    int64_t S = 0;    // elements of one rank's shard (FLAT ceil(T/N), ROWS P_r)
    int64_t L = 0;    // N*S
    int64_t pad = 0;  // L - T
    std::vector<ParamPlan> params;

    // Real (non-padding) elements of rank k's shard.
    int64_t valid(int64_t k) const;
};

// Builds the plan; returns 0 or an fsdp_status code with *err set.
int plan_create(int32_t layout, int32_t n_params, const int32_t* ndims, const int64_t* dims,
                int32_t N, UnitPlan* out, std::string* err);

// One planned movement: `nblk` blocks; block b moves `blk_n` elements (the last
// block `last_n`) from src + b*src_stride to dst + b*dst_stride.  src == nullptr
// means "write zeros".  Strides and counts are in elements of the respective
// buffer (fp32 or bf16 for either side; the element sizes are the caller's).
struct CopySeg {
    const void* src = nullptr;
    void* dst = nullptr;
    int64_t blk_n = 0;
    int64_t last_n = 0;
    int64_t src_stride = 0;
    int64_t dst_stride = 0;
    int64_t nblk = 0;
};

// Segments that write rank k's shard (k = -1: every rank, gathered layout) into
// `out` from the parameters; `esize` is the element size in bytes of both.
void plan_flatten(const UnitPlan& u, const void* const* params, int64_t k, void* out,
                  size_t esize, std::vector<CopySeg>* segs);

// Segments that copy the gathered buffer (elements of `src_esize` bytes) out
// into per-parameter tensors (elements of `dst_esize` bytes).
void plan_copyout(const UnitPlan& u, const void* gathered, size_t src_esize, void* const* outs,
                  size_t dst_esize, std::vector<CopySeg>* segs);

// One segment covering rank k's shard (k = -1: the whole gathered buffer):
// src and dst index the same positions.
void plan_whole(const UnitPlan& u, int64_t k, const void* src, void* dst,
                std::vector<CopySeg>* segs);
// Where each parameter's real elements sit inside rank k's shard (k in [0, N)):
// run i starts `offset` elements into the shard and holds `n` of parameter i's
// elements (n = 0 when the rank holds none).  FLAT: the intersection of the
// parameter's range with [kS, (k+1)S); ROWS: the rows of the rank's chunk, from q_i.
struct ParamRun {
    int64_t offset = 0;
    int64_t n = 0;
};
void plan_param_runs(const UnitPlan& u, int64_t k, std::vector<ParamRun>* runs);

// One launch of the many-rank reduction's sweep: whole tiles [t_first, t_first + n_tiles)
// of the output; its grid is `cut` workgroups for the tile the output's end cuts (only in
// the last run), then n_single workgroups of one whole tile each (n_tiles mod kv), then one
// workgroup per kv whole tiles: `blocks` workgroups in all.
struct SweepRun {
    int64_t t_first = 0;
    int64_t n_tiles = 0;
    int32_t cut = 0;
    int32_t n_single = 0;
    int64_t blocks = 0;
};
// Splits `tiles` whole tiles (plus a cut tile when `cut_tile`) into as few runs of nearly
// equal length as keep every run's grid within `capacity` workgroups (those resident at
// once), kv tiles per sweep workgroup.  Returns false, leaving `runs` empty, when tiles < kv
// or capacity <= kv (no run fits).
bool plan_sweep_runs(int64_t tiles, bool cut_tile, int64_t kv, int64_t capacity,
                     std::vector<SweepRun>* runs);

// A reduction over more ranks than one launch's pointer table holds (`cap`) takes several
// launches in rank order.  Between them the running sums sit in HBM, stored exactly: the
// total (the flat sum, or the sum of the completed groups) and, when a group is longer
// than one launch, that group's partial sum.  Each launch's flags say what it loads and
// stores.
enum ReduceFlag : uint32_t {
    kReduceTIn = 1u,    // the total so far is carried in (else it starts in this launch)
    kReduceSIn = 2u,    // the partial sum of this launch's first group is carried in
    kReduceTOut = 4u,   // not the last launch: the total is carried out
    kReduceSOut = 8u,   // not the last launch: the last group's partial sum is carried out
    kReduceLast = 16u,  // the last launch: total / post (+ the old value) is the result
};
struct ReduceLaunch {
    int64_t r0 = 0;     // first rank
    int64_t nc = 0;     // ranks
    int64_t pos0 = 0;   // position of rank r0 in its group
    uint32_t flags = 0;
};
struct ReducePlan {
    std::vector<ReduceLaunch> launches;
    // Where the carried sums live: -1 the output itself, else that slot of the caller's
    // workspace (slot i starts i * reduce_ws_pitch(S) floats in).  The total is carried in
    // the output unless the result is accumulated into it (the output then keeps the old
    // value until the last launch).
    int t_slot = -1;
    int s_slot = -1;
    int ws_slots = 0;   // workspace slots the plan uses
};
// Groups of `group` consecutive ranks (group <= 1 or >= n: one flat sum), at most `cap`
// ranks per launch.  Groups that fit a launch are never split: a launch holds whole groups
// (as many as fit); a longer group takes ceil(group / cap) launches of its own.
// n >= 1, cap >= 1; group divides n when 1 < group < n.
void plan_reduce(int64_t n, int64_t group, bool accumulate, int64_t cap, ReducePlan* plan);
// Floats between workspace slots for a shard of S elements: S rounded up to 64 (256 bytes),
// so every slot of a 16-byte-aligned workspace is 16-byte aligned.
int64_t reduce_ws_pitch(int64_t S);

}  // namespace fsdp
