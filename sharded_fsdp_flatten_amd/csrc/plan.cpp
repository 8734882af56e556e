// plan.cpp -- unit planner (host integer arithmetic only).
#include "plan.h"

#include <algorithm>
#include <limits>

namespace fsdp {
namespace {

constexpr int64_t kI64Max = std::numeric_limits<int64_t>::max();

// a*b and a+b with overflow detection (operands are non-negative).
bool mul_ok(int64_t a, int64_t b, int64_t* out) {
    if (a != 0 && b > kI64Max / a) return false;
    *out = a * b;
    return true;
}
bool add_ok(int64_t a, int64_t b, int64_t* out) {
    if (b > kI64Max - a) return false;
    *out = a + b;
    return true;
}
int64_t ceil_div(int64_t a, int64_t b) { return a / b + (a % b != 0); }

// Rows [lo, hi) of a dim-0 chunked parameter held by rank k (torch.chunk: chunks
// of c rows; ranks past the last chunk hold none).
void rank_rows(const ParamPlan& p, int64_t k, int64_t* lo, int64_t* hi) {
    const int64_t c = p.chunk_rows;
    // k*c cannot overflow: k < N and c*N <= m + N - 1 fits (checked at create).
    *lo = std::min(p.rows, k * c);
    *hi = std::min(p.rows, (k + 1) * c);
}

}  // namespace

int64_t UnitPlan::valid(int64_t k) const {
    if (k < 0 || k >= N) return 0;
    if (layout == kFlat) {
        const int64_t lo = k * S;
        const int64_t hi = std::min(T, lo + S);
        return hi > lo ? hi - lo : 0;
    }
    int64_t v = 0;
    for (const ParamPlan& p : params) {
        int64_t lo, hi;
        rank_rows(p, k, &lo, &hi);
        v += (hi - lo) * p.row_len;
    }
    return v;
}

int plan_create(int32_t layout, int32_t n_params, const int32_t* ndims, const int64_t* dims,
                int32_t N, UnitPlan* out, std::string* err) {
    // status codes match fsdp_status in include/fsdp_flatten.h
    constexpr int kArg = 1, kRange = 2, kOverflow = 4;
    if (layout != kFlat && layout != kRows) {
        *err = "layout must be FSDP_FLAT (1) or FSDP_ROWS (2)";
        return kRange;
    }
    if (N < 1) {
        *err = "N (shard count) must be >= 1";
        return kRange;
    }
    if (n_params < 0) {
        *err = "n_params must be >= 0";
        return kRange;
    }
    if (n_params > 0 && !ndims) {
        *err = "ndims must not be NULL when n_params > 0";
        return kArg;
    }
    int64_t total_dims = 0;  // dims holds sum(ndims) entries; it may be NULL when that is 0
    for (int32_t i = 0; i < n_params; ++i) total_dims += ndims[i] > 0 ? ndims[i] : 0;
    if (total_dims > 0 && !dims) {
        *err = "dims must not be NULL when some parameter has dimensions";
        return kArg;
    }
    UnitPlan u;
    u.layout = layout;
    u.N = N;
    u.params.resize(static_cast<size_t>(n_params));
    int64_t d = 0;
    for (int32_t i = 0; i < n_params; ++i) {
        if (ndims[i] < 0 || ndims[i] > 8) {
            *err = "parameter " + std::to_string(i) + ": ndim must be in [0, 8]";
            return kRange;
        }
        ParamPlan& p = u.params[static_cast<size_t>(i)];
        int64_t numel = 1;
        for (int32_t a = 0; a < ndims[i]; ++a, ++d) {
            const int64_t x = dims[d];
            if (x < 0) {
                *err = "parameter " + std::to_string(i) + ": negative dimension";
                return kRange;
            }
            p.shape.push_back(x);
            if (!mul_ok(numel, x, &numel)) {
                *err = "parameter " + std::to_string(i) + ": element count overflows int64";
                return kOverflow;
            }
        }
        p.numel = numel;
        if (ndims[i] == 0) {
            p.rows = 1;
            p.row_len = 1;
        } else {
            p.rows = p.shape[0];
            int64_t row_len = 1;
            for (int32_t a = 1; a < ndims[i]; ++a)
                if (!mul_ok(row_len, p.shape[static_cast<size_t>(a)], &row_len)) {
                    *err = "parameter " + std::to_string(i) + ": row length overflows int64";
                    return kOverflow;
                }
            p.row_len = row_len;
        }
        if (!add_ok(u.T, numel, &u.T)) {
            *err = "unit element count overflows int64";
            return kOverflow;
        }
    }
    if (layout == kFlat) {
        int64_t off = 0;
        for (ParamPlan& p : u.params) {
            p.offset = off;
            off += p.numel;
        }
        u.S = ceil_div(u.T, N);
        if (!mul_ok(u.S, N, &u.L)) {
            *err = "padded unit length overflows int64";
            return kOverflow;
        }
    } else {
        int64_t q = 0;
        for (ParamPlan& p : u.params) {
            p.chunk_rows = ceil_div(p.rows, N);
            int64_t seg, tmp;
            if (!mul_ok(p.chunk_rows, p.row_len, &seg) || !mul_ok(p.chunk_rows, N, &tmp)) {
                *err = "rank segment size overflows int64";
                return kOverflow;
            }
            p.offset = q;
            if (!add_ok(q, seg, &q)) {
                *err = "rank segment size overflows int64";
                return kOverflow;
            }
        }
        u.S = q;
        if (!mul_ok(u.S, N, &u.L)) {
            *err = "gathered length overflows int64";
            return kOverflow;
        }
    }
    u.pad = u.L - u.T;
    int64_t bytes;  // the 16*S per-rank ledger must be representable
    if (!mul_ok(u.S, 16, &bytes)) {
        *err = "per-rank byte count overflows int64";
        return kOverflow;
    }
    *out = std::move(u);
    return 0;
}

namespace {
const void* at(const void* p, int64_t e, size_t esize) {
    return static_cast<const char*>(p) + e * static_cast<int64_t>(esize);
}
void* at(void* p, int64_t e, size_t esize) {
    return static_cast<char*>(p) + e * static_cast<int64_t>(esize);
}
}  // namespace

void plan_flatten(const UnitPlan& u, const void* const* params, int64_t k, void* out,
                  size_t esize, std::vector<CopySeg>* segs) {
    segs->clear();
    if (u.layout == kFlat) {
        const int64_t base = k < 0 ? 0 : k * u.S;
        const int64_t len = k < 0 ? u.L : u.S;
        for (size_t i = 0; i < u.params.size(); ++i) {
            const ParamPlan& p = u.params[i];
            const int64_t lo = std::max(p.offset, base);
            const int64_t hi = std::min(p.offset + p.numel, base + len);
            if (lo >= hi) continue;
            CopySeg s;
            s.src = at(params[i], lo - p.offset, esize);
            s.dst = at(out, lo - base, esize);
            s.blk_n = s.last_n = hi - lo;
            s.nblk = 1;
            segs->push_back(s);
        }
        const int64_t zlo = std::max(u.T, base);
        if (zlo < base + len) {
            CopySeg s;
            s.dst = at(out, zlo - base, esize);
            s.blk_n = s.last_n = base + len - zlo;
            s.nblk = 1;
            segs->push_back(s);
        }
        return;
    }
    // ROWS: ranks [k0, k1) write one after another, rank segment of S elements each.
    const int64_t k0 = k < 0 ? 0 : k;
    const int64_t k1 = k < 0 ? u.N : k + 1;
    for (size_t i = 0; i < u.params.size(); ++i) {
        const ParamPlan& p = u.params[i];
        const int64_t c = p.chunk_rows, r = p.row_len;
        const int64_t seg_n = c * r;
        if (seg_n == 0) continue;
        // ranks whose chunk is complete (c rows), the one short rank, then empty ranks
        const int64_t n_full = p.rows / c;
        const int64_t short_rows = p.rows - n_full * c;
        void* base = at(out, p.offset, esize);
        {  // full ranks in [k0, k1)
            const int64_t a = k0, b = std::min(k1, n_full);
            if (a < b) {
                CopySeg s;
                s.src = at(params[i], a * seg_n, esize);
                s.dst = at(base, (a - k0) * u.S, esize);
                s.blk_n = s.last_n = seg_n;
                s.src_stride = seg_n;
                s.dst_stride = u.S;
                s.nblk = b - a;
                segs->push_back(s);
            }
        }
        int64_t first_empty = n_full;
        if (short_rows > 0) {
            first_empty = n_full + 1;
            const int64_t ks = n_full;
            if (ks >= k0 && ks < k1) {
                CopySeg s;
                s.src = at(params[i], ks * seg_n, esize);
                s.dst = at(base, (ks - k0) * u.S, esize);
                s.blk_n = s.last_n = short_rows * r;
                s.nblk = 1;
                segs->push_back(s);
                CopySeg z;
                z.dst = at(base, (ks - k0) * u.S + short_rows * r, esize);
                z.blk_n = z.last_n = (c - short_rows) * r;
                z.nblk = 1;
                segs->push_back(z);
            }
        }
        {  // empty ranks: c zero rows each
            const int64_t a = std::max(k0, first_empty), b = k1;
            if (a < b) {
                CopySeg z;
                z.dst = at(base, (a - k0) * u.S, esize);
                z.blk_n = z.last_n = seg_n;
                z.dst_stride = u.S;
                z.nblk = b - a;
                segs->push_back(z);
            }
        }
    }
}

void plan_copyout(const UnitPlan& u, const void* gathered, size_t src_esize, void* const* outs,
                  size_t dst_esize, std::vector<CopySeg>* segs) {
    segs->clear();
    for (size_t i = 0; i < u.params.size(); ++i) {
        const ParamPlan& p = u.params[i];
        if (p.numel == 0) continue;
        if (u.layout == kFlat) {
            CopySeg s;
            s.src = at(gathered, p.offset, src_esize);
            s.dst = outs[i];
            s.blk_n = s.last_n = p.numel;
            s.nblk = 1;
            segs->push_back(s);
            continue;
        }
        const int64_t c = p.chunk_rows, r = p.row_len;
        const int64_t seg_n = c * r;
        const int64_t n_full = p.rows / c;
        const int64_t short_rows = p.rows - n_full * c;
        if (n_full > 0) {
            CopySeg s;
            s.src = at(gathered, p.offset, src_esize);
            s.dst = outs[i];
            s.blk_n = s.last_n = seg_n;
            s.src_stride = u.S;
            s.dst_stride = seg_n;
            s.nblk = n_full;
            segs->push_back(s);
        }
        if (short_rows > 0) {
            CopySeg s;
            s.src = at(gathered, n_full * u.S + p.offset, src_esize);
            s.dst = at(outs[i], n_full * seg_n, dst_esize);
            s.blk_n = s.last_n = short_rows * r;
            s.nblk = 1;
            segs->push_back(s);
        }
    }
}

void plan_whole(const UnitPlan& u, int64_t k, const void* src, void* dst,
                std::vector<CopySeg>* segs) {
    segs->clear();
    const int64_t n = k < 0 ? u.L : u.S;
    if (n == 0) return;
    CopySeg s;
    s.src = src;
    s.dst = dst;
    s.blk_n = s.last_n = n;
    s.nblk = 1;
    segs->push_back(s);
}

void plan_param_runs(const UnitPlan& u, int64_t k, std::vector<ParamRun>* runs) {
    runs->assign(u.params.size(), ParamRun{});
    for (size_t i = 0; i < u.params.size(); ++i) {
        const ParamPlan& p = u.params[i];
        ParamRun& run = (*runs)[i];
        if (u.layout == kFlat) {
            const int64_t lo = std::max(p.offset, k * u.S);
            const int64_t hi = std::min(p.offset + p.numel, (k + 1) * u.S);
            if (hi > lo) {
                run.offset = lo - k * u.S;
                run.n = hi - lo;
            }
        } else {
            int64_t lo, hi;
            rank_rows(p, k, &lo, &hi);
            run.offset = p.offset;
            run.n = (hi - lo) * p.row_len;
        }
    }
}

bool plan_sweep_runs(int64_t tiles, bool cut_tile, int64_t kv, int64_t capacity,
                     std::vector<SweepRun>* runs) {
    runs->clear();
    if (kv < 1 || tiles < kv || capacity <= kv) return false;
    // a run of n tiles takes cut + (n mod kv) + n/kv <= 1 + (kv - 1) + n/kv workgroups, so
    // n <= kv * (capacity - kv) keeps it within capacity
    const int64_t per_run = kv * (capacity - kv);
    const int64_t n_runs = (tiles + per_run - 1) / per_run;
    const int64_t each = (tiles + n_runs - 1) / n_runs;
    for (int64_t t = 0; t < tiles; t += each) {
        SweepRun r;
        r.t_first = t;
        r.n_tiles = std::min(each, tiles - t);
        r.cut = (t + r.n_tiles == tiles && cut_tile) ? 1 : 0;
        r.n_single = static_cast<int32_t>(r.n_tiles % kv);
        r.blocks = r.cut + r.n_single + r.n_tiles / kv;
        runs->push_back(r);
    }
    return true;
}

void plan_reduce(int64_t n, int64_t group, bool accumulate, int64_t cap, ReducePlan* plan) {
    plan->launches.clear();
    const bool hybrid = group > 1 && group < n;
    const int64_t F = hybrid ? group : n;
    if (!hybrid || F <= cap) {
        // every launch holds whole groups: only the total crosses launches
        const int64_t chunk = hybrid ? (cap / F) * F : cap;
        for (int64_t r0 = 0; r0 < n; r0 += chunk) {
            ReduceLaunch l;
            l.r0 = r0;
            l.nc = std::min(chunk, n - r0);
            const bool last = r0 + l.nc == n;
            l.flags = (r0 > 0 ? kReduceTIn : 0u) | (last ? kReduceLast : kReduceTOut);
            plan->launches.push_back(l);
        }
        const bool multi = plan->launches.size() > 1;
        plan->t_slot = multi && accumulate ? 0 : -1;
        plan->s_slot = -1;
        plan->ws_slots = multi && accumulate ? 1 : 0;
        return;
    }
    // groups longer than a launch: each takes launches of its own; a group's partial sum
    // crosses them, and the total is loaded and stored only by a group's last launch
    const int64_t groups = n / F;
    for (int64_t g = 0; g < groups; ++g)
        for (int64_t p0 = 0; p0 < F; p0 += cap) {
            ReduceLaunch l;
            l.r0 = g * F + p0;
            l.nc = std::min(cap, F - p0);
            l.pos0 = p0;
            const bool completes = p0 + l.nc == F;
            const bool last = completes && g + 1 == groups;
            l.flags = (p0 > 0 ? kReduceSIn : 0u) | (completes && g > 0 ? kReduceTIn : 0u) |
                      (last ? kReduceLast : completes ? kReduceTOut : kReduceSOut);
            plan->launches.push_back(l);
        }
    plan->t_slot = accumulate ? 0 : -1;
    plan->s_slot = accumulate ? 1 : 0;
    plan->ws_slots = accumulate ? 2 : 1;
}

int64_t reduce_ws_pitch(int64_t S) { return (S + 63) / 64 * 64; }

}  // namespace fsdp
