// plan_check.cpp -- host-only check of the unit planner, built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_planner_sanitized.py.
//
// For random units of both layouts it applies the planned copy segments to host buffers
// (64-bit elements that encode parameter and position, so every misplaced, missing or
// duplicated element is visible) and checks them against a brute-force statement of the
// layouts: FSDP1 flat buffer = concatenated parameters + zero padding, rank k owning
// [kS, (k+1)S); FSDP2 segment = per parameter the rows of the rank's torch.chunk chunk,
// then zero rows up to the chunk size.  It also checks the per-parameter runs of a rank's
// shard and that oversized units are rejected as overflows, not wrapped.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <random>
#include <string>
#include <vector>

#include "plan.h"

namespace {

int g_fail = 0;
#define CHECK(c, ...)                                                        \
    do {                                                                     \
        if (!(c)) {                                                          \
            if (g_fail++ < 20) {                                             \
                std::fprintf(stderr, "FAIL %s:%d: %s: ", __FILE__, __LINE__, #c); \
                std::fprintf(stderr, __VA_ARGS__);                           \
                std::fprintf(stderr, "\n");                                  \
            }                                                                \
        }                                                                    \
    } while (0)

uint64_t code(int64_t i, int64_t e) { return (static_cast<uint64_t>(i) << 40) | static_cast<uint64_t>(e + 1); }

struct Unit {
    std::vector<std::vector<int64_t>> shapes;
    int64_t numel(size_t i) const {
        int64_t n = 1;
        for (int64_t d : shapes[i]) n *= d;
        return n;
    }
    int64_t rows(size_t i) const { return shapes[i].empty() ? 1 : shapes[i][0]; }
    int64_t row_len(size_t i) const {
        int64_t r = 1;
        for (size_t a = 1; a < shapes[i].size(); ++a) r *= shapes[i][a];
        return r;
    }
};

// Applies segments to real host buffers; `out_lo/out_hi` bound the destination buffer
// (every write must land inside), `hits` counts writes per destination element.
void apply(const std::vector<fsdp::CopySeg>& segs, const uint64_t* out_lo, int64_t out_n,
           std::vector<int>* hits, const std::vector<const uint64_t*>& src_lo,
           const std::vector<int64_t>& src_n) {
    for (const fsdp::CopySeg& s : segs) {
        CHECK(s.nblk >= 1 && s.blk_n >= 1 && s.last_n >= 1 && s.last_n <= s.blk_n, "segment shape");
        for (int64_t b = 0; b < s.nblk; ++b) {
            const int64_t n = b + 1 == s.nblk ? s.last_n : s.blk_n;
            uint64_t* d = static_cast<uint64_t*>(s.dst) + b * s.dst_stride;
            const uint64_t* src = s.src ? static_cast<const uint64_t*>(s.src) + b * s.src_stride : nullptr;
            if (src) {
                bool inside = false;
                for (size_t q = 0; q < src_lo.size(); ++q)
                    inside = inside || (src >= src_lo[q] && src + n <= src_lo[q] + src_n[q]);
                CHECK(inside, "source block outside every source buffer");
                if (!inside) continue;
            }
            const int64_t j0 = d - out_lo;
            CHECK(j0 >= 0 && j0 + n <= out_n, "destination block outside the buffer");
            if (!(j0 >= 0 && j0 + n <= out_n)) continue;
            for (int64_t e = 0; e < n; ++e) {
                d[e] = src ? src[e] : 0;
                ++(*hits)[static_cast<size_t>(j0 + e)];
            }
        }
    }
}

// Expected gathered buffer (all ranks) by the layout definitions.
std::vector<uint64_t> expected_gathered(const Unit& u, int32_t layout, int64_t N, int64_t* S_out) {
    std::vector<uint64_t> g;
    if (layout == fsdp::kFlat) {
        for (size_t i = 0; i < u.shapes.size(); ++i)
            for (int64_t e = 0; e < u.numel(i); ++e) g.push_back(code(static_cast<int64_t>(i), e));
        const int64_t T = static_cast<int64_t>(g.size());
        const int64_t S = (T + N - 1) / N;
        g.resize(static_cast<size_t>(S * N), 0);
        *S_out = S;
        return g;
    }
    int64_t S = 0;
    for (size_t i = 0; i < u.shapes.size(); ++i) S += (u.rows(i) + N - 1) / N * u.row_len(i);
    *S_out = S;
    for (int64_t k = 0; k < N; ++k)
        for (size_t i = 0; i < u.shapes.size(); ++i) {
            const int64_t m = u.rows(i), r = u.row_len(i), c = (m + N - 1) / N;
            for (int64_t row = k * c; row < (k + 1) * c; ++row)
                for (int64_t col = 0; col < r; ++col)
                    g.push_back(row < m ? code(static_cast<int64_t>(i), row * r + col) : 0);
        }
    return g;
}

void check_unit(const Unit& u, int32_t layout, int32_t N, std::mt19937_64& rng) {
    std::vector<int32_t> ndims;
    std::vector<int64_t> dims;
    for (const auto& s : u.shapes) {
        ndims.push_back(static_cast<int32_t>(s.size()));
        dims.insert(dims.end(), s.begin(), s.end());
    }
    fsdp::UnitPlan p;
    std::string err;
    const int rc = fsdp::plan_create(layout, static_cast<int32_t>(u.shapes.size()), ndims.data(),
                                     dims.data(), N, &p, &err);
    CHECK(rc == 0, "plan_create failed: %s", err.c_str());
    if (rc != 0) return;
    int64_t S = 0;
    const std::vector<uint64_t> want = expected_gathered(u, layout, N, &S);
    CHECK(p.S == S && p.L == S * N, "sizes S %lld vs %lld", (long long)p.S, (long long)S);
    std::vector<std::vector<uint64_t>> params(u.shapes.size());
    std::vector<const uint64_t*> plo;
    std::vector<int64_t> pn;
    std::vector<const void*> pptr;
    for (size_t i = 0; i < u.shapes.size(); ++i) {
        params[i].resize(static_cast<size_t>(u.numel(i)) + 1);  // +1: never a zero-size buffer
        for (int64_t e = 0; e < u.numel(i); ++e) params[i][static_cast<size_t>(e)] = code(static_cast<int64_t>(i), e);
        plo.push_back(params[i].data());
        pn.push_back(u.numel(i));
        pptr.push_back(params[i].data());
    }
    // flatten: every rank (a sample for large N) and all ranks at once
    std::vector<int64_t> ks = {-1};
    for (int64_t k = 0; k < N; ++k)
        if (N <= 16 || k < 2 || k == N - 1 || rng() % 8 == 0) ks.push_back(k);
    for (int64_t k : ks) {
        const int64_t n = k < 0 ? p.L : p.S;
        std::vector<uint64_t> out(static_cast<size_t>(n) + 1, ~0ull);
        std::vector<int> hits(static_cast<size_t>(n) + 1, 0);
        std::vector<fsdp::CopySeg> segs;
        fsdp::plan_flatten(p, pptr.data(), k, out.data(), sizeof(uint64_t), &segs);
        apply(segs, out.data(), n, &hits, plo, pn);
        for (int64_t j = 0; j < n; ++j) {
            const uint64_t w = want[static_cast<size_t>((k < 0 ? 0 : k * p.S) + j)];
            CHECK(hits[static_cast<size_t>(j)] == 1, "flatten k=%lld element %lld written %d times",
                  (long long)k, (long long)j, hits[static_cast<size_t>(j)]);
            CHECK(out[static_cast<size_t>(j)] == w, "flatten k=%lld element %lld", (long long)k, (long long)j);
        }
        if (k >= 0) {
            CHECK(p.valid(k) == [&] {
                int64_t v = 0;
                for (int64_t j = 0; j < n; ++j) v += want[static_cast<size_t>(k * p.S + j)] != 0;
                return v;
            }(), "valid(%lld)", (long long)k);
            // the per-parameter runs: inside the shard, disjoint, exactly the parameter's elements
            std::vector<fsdp::ParamRun> runs;
            fsdp::plan_param_runs(p, k, &runs);
            CHECK(runs.size() == u.shapes.size(), "run count");
            std::vector<int> own(static_cast<size_t>(n) + 1, 0);
            for (size_t i = 0; i < runs.size(); ++i) {
                CHECK(runs[i].n >= 0 && runs[i].offset >= 0 && runs[i].offset + runs[i].n <= n, "run %zu bounds", i);
                for (int64_t e = 0; e < runs[i].n; ++e) {
                    const uint64_t w = want[static_cast<size_t>(k * p.S + runs[i].offset + e)];
                    CHECK(w != 0 && (w >> 40) == i, "run %zu element %lld", i, (long long)e);
                    ++own[static_cast<size_t>(runs[i].offset + e)];
                }
            }
            for (int64_t j = 0; j < n; ++j)
                CHECK(own[static_cast<size_t>(j)] == (want[static_cast<size_t>(k * p.S + j)] != 0 ? 1 : 0),
                      "run coverage k=%lld element %lld", (long long)k, (long long)j);
        }
    }
    // copy-out of the gathered buffer into per-parameter tensors
    std::vector<std::vector<uint64_t>> outs(u.shapes.size());
    std::vector<void*> optr;
    for (size_t i = 0; i < u.shapes.size(); ++i) {
        outs[i].assign(static_cast<size_t>(u.numel(i)) + 1, ~0ull);
        optr.push_back(outs[i].data());
    }
    std::vector<fsdp::CopySeg> segs;
    fsdp::plan_copyout(p, want.data(), sizeof(uint64_t), optr.data(), sizeof(uint64_t), &segs);
    for (size_t i = 0; i < u.shapes.size(); ++i) {
        // apply only the segments that write parameter i's tensor
        std::vector<fsdp::CopySeg> mine;
        for (const auto& s : segs) {
            const uint64_t* d = static_cast<const uint64_t*>(s.dst);
            if (d >= outs[i].data() && d < outs[i].data() + outs[i].size()) mine.push_back(s);
        }
        std::vector<int> hits(outs[i].size(), 0);
        apply(mine, outs[i].data(), u.numel(i), &hits, {want.data()}, {static_cast<int64_t>(want.size())});
        for (int64_t e = 0; e < u.numel(i); ++e) {
            CHECK(hits[static_cast<size_t>(e)] == 1, "copy-out param %zu element %lld written %d times", i,
                  (long long)e, hits[static_cast<size_t>(e)]);
            CHECK(outs[i][static_cast<size_t>(e)] == code(static_cast<int64_t>(i), e), "copy-out param %zu element %lld",
                  i, (long long)e);
        }
    }
}

Unit random_unit(std::mt19937_64& rng) {
    Unit u;
    const int p = static_cast<int>(rng() % 70);
    for (int i = 0; i < p; ++i) {
        std::vector<int64_t> s;
        const int nd = static_cast<int>(rng() % 4);
        for (int a = 0; a < nd; ++a) s.push_back(static_cast<int64_t>(rng() % (a == 0 ? 40 : 9)));
        u.shapes.push_back(s);
    }
    return u;
}

void check_overflow() {
    fsdp::UnitPlan p;
    std::string err;
    const int32_t nd2[] = {2};
    const int64_t huge[] = {int64_t(1) << 62, 8};
    CHECK(fsdp::plan_create(fsdp::kFlat, 1, nd2, huge, 4, &p, &err) == 4, "numel overflow");
    const int32_t nd11[] = {1, 1};
    const int64_t two[] = {int64_t(1) << 62, int64_t(1) << 62};
    CHECK(fsdp::plan_create(fsdp::kFlat, 2, nd11, two, 4, &p, &err) == 4, "T overflow");
    const int64_t big1[] = {(int64_t(1) << 62) + 1};
    CHECK(fsdp::plan_create(fsdp::kFlat, 1, nd11, big1, 4, &p, &err) == 4, "L = N*S overflow");
    const int32_t nd2b[] = {2};
    const int64_t rows[] = {3, int64_t(1) << 61};
    CHECK(fsdp::plan_create(fsdp::kRows, 1, nd2b, rows, 2, &p, &err) == 4, "rows segment overflow");
    const int64_t ledger[] = {int64_t(1) << 60};
    CHECK(fsdp::plan_create(fsdp::kFlat, 1, nd11, ledger, 1, &p, &err) == 4, "16*S overflow");
    const int64_t ok[] = {5};
    CHECK(fsdp::plan_create(fsdp::kFlat, 1, nd11, ok, 2147483647, &p, &err) == 0 && p.S == 1, "huge N");
}

// The reduction sweep's runs: for random tile counts, kv and capacities, the runs cover the
// whole tiles [0, tiles) in order, each exactly once; every run's grid (cut + single tiles +
// kv-tile workgroups) fits the capacity; only the last run has the cut tile; the split uses
// the fewest runs the per-run bound allows.  Unusable inputs are refused.
void check_sweep_runs(std::mt19937_64& rng, int iters) {
    std::vector<fsdp::SweepRun> runs;
    CHECK(!fsdp::plan_sweep_runs(15, true, 16, 2048, &runs) && runs.empty(), "tiles < kv refused");
    CHECK(!fsdp::plan_sweep_runs(1000, false, 16, 16, &runs), "capacity <= kv refused");
    CHECK(!fsdp::plan_sweep_runs(1000, false, 16, 0, &runs), "unknown capacity refused");
    for (int it = 0; it < iters; ++it) {
        const int64_t kv = 1 + static_cast<int64_t>(rng() % 20);
        const int64_t cap = kv + 1 + static_cast<int64_t>(rng() % (it % 3 == 0 ? 40 : 5000));
        const int64_t tiles = kv + static_cast<int64_t>(rng() % (it % 4 == 0 ? 200 : 20000000));
        const bool cut = (rng() & 1) != 0;
        CHECK(fsdp::plan_sweep_runs(tiles, cut, kv, cap, &runs) && !runs.empty(), "sweep planned");
        const int64_t per_run = kv * (cap - kv);
        CHECK(static_cast<int64_t>(runs.size()) == (tiles + per_run - 1) / per_run, "fewest runs");
        int64_t next = 0;
        for (size_t i = 0; i < runs.size(); ++i) {
            const fsdp::SweepRun& r = runs[i];
            CHECK(r.t_first == next && r.n_tiles >= 1, "runs contiguous");
            CHECK(r.n_tiles <= runs[0].n_tiles && (i + 1 == runs.size() || r.n_tiles == runs[0].n_tiles),
                  "runs of equal length, the last no longer");
            CHECK(r.n_single == r.n_tiles % kv, "single tiles");
            CHECK(r.cut == ((i + 1 == runs.size() && cut) ? 1 : 0), "cut tile only in the last run");
            CHECK(r.blocks == r.cut + r.n_single + r.n_tiles / kv && r.blocks <= cap &&
                      r.blocks < (int64_t(1) << 31), "grid fits");
            next += r.n_tiles;
        }
        CHECK(next == tiles, "every whole tile once");
    }
}

}  // namespace

// The reduction's launch plans: for random rank counts, group sizes, launch capacities and
// accumulation, run the plan the way the kernels do -- each launch loads what its flags
// say it carries in, adds its ranks in order (a group's sum starting at its first rank and
// folded into the total after its last), and stores what it carries out, in binary32 --
// with an unwritten workspace (NaN) and the old value in the output, and compare the result
// bit for bit with one sequential pass over all ranks.  Also checks the structure: every
// rank once and in order, at most cap ranks per launch, whole groups per launch when a
// group fits one, the flags of the first and last launches, and the workspace slots.
uint32_t bits(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return u;
}

void check_reduce_plans(std::mt19937_64& rng, int iters) {
    std::normal_distribution<float> nd(0.0f, 1.0f);
    for (int it = 0; it < iters; ++it) {
        const int64_t n = 1 + static_cast<int64_t>(rng() % (it % 3 == 0 ? 700 : 140));
        std::vector<int64_t> divisors = {0};
        for (int64_t d = 1; d <= n; ++d)
            if (n % d == 0) divisors.push_back(d);
        const int64_t group = divisors[rng() % divisors.size()];
        const int64_t cap = it % 4 == 0 ? 128 : 1 + static_cast<int64_t>(rng() % 130);
        const bool accumulate = rng() % 2 == 0;
        fsdp::ReducePlan plan;
        fsdp::plan_reduce(n, group, accumulate, cap, &plan);
        const bool hybrid = group > 1 && group < n;
        const int64_t F = hybrid ? group : n;
        // structure
        CHECK(!plan.launches.empty(), "reduce plan has launches");
        int64_t next = 0;
        for (size_t i = 0; i < plan.launches.size(); ++i) {
            const fsdp::ReduceLaunch& l = plan.launches[i];
            CHECK(l.r0 == next && l.nc >= 1 && l.nc <= cap, "launch ranks in order within cap");
            CHECK(!hybrid || l.pos0 == l.r0 % F, "launch pos0 is the rank's place in its group");
            if (hybrid && F <= cap) CHECK(l.r0 % F == 0 && l.nc % F == 0, "whole groups per launch");
            const bool last = i + 1 == plan.launches.size();
            CHECK(((l.flags & fsdp::kReduceLast) != 0) == last, "only the last launch finishes");
            if (i == 0) CHECK((l.flags & (fsdp::kReduceTIn | fsdp::kReduceSIn)) == 0, "first launch carries nothing in");
            next = l.r0 + l.nc;
        }
        CHECK(next == n, "every rank reduced");
        CHECK(plan.ws_slots >= 0 && plan.ws_slots <= 2 && plan.t_slot < plan.ws_slots &&
                  plan.s_slot < plan.ws_slots, "workspace slots in range");
        if (accumulate && plan.launches.size() > 1) CHECK(plan.t_slot >= 0, "old value kept");
        // values: a few outputs, terms of mixed magnitude so that the order matters
        constexpr int kOut = 3;
        const float post = (rng() % 2) ? 3.0f : 8.0f;
        std::vector<float> t(static_cast<size_t>(n * kOut));
        for (float& x : t) x = nd(rng) * std::ldexp(1.0f, static_cast<int>(rng() % 24) - 12);
        float old[kOut], want[kOut];
        for (int j = 0; j < kOut; ++j) {
            old[j] = nd(rng);
            float total = 0.0f;
            for (int64_t g = 0; g < n / F; ++g) {
                float sg = t[static_cast<size_t>(g * F * kOut + j)];
                for (int64_t r = g * F + 1; r < (g + 1) * F; ++r) sg = sg + t[static_cast<size_t>(r * kOut + j)];
                total = g == 0 ? sg : total + sg;
            }
            const float fresh = total / post;
            want[j] = accumulate ? old[j] + fresh : fresh;
        }
        const float nan = std::numeric_limits<float>::quiet_NaN();
        std::vector<float> out(old, old + kOut), ws(static_cast<size_t>(2 * kOut), nan);
        float* carry_t = plan.t_slot < 0 ? out.data() : ws.data() + plan.t_slot * kOut;
        float* carry_s = plan.s_slot < 0 ? nullptr : ws.data() + plan.s_slot * kOut;
        for (const fsdp::ReduceLaunch& l : plan.launches) {
            for (int j = 0; j < kOut; ++j) {
                bool have = (l.flags & fsdp::kReduceTIn) != 0;
                float acc = have ? carry_t[j] : nan;
                float sg = (l.flags & fsdp::kReduceSIn) ? carry_s[j] : nan;
                int64_t pos = l.pos0;
                for (int64_t r = l.r0; r < l.r0 + l.nc; ++r) {
                    const float x = t[static_cast<size_t>(r * kOut + j)];
                    if (!hybrid) {
                        acc = have ? acc + x : x;
                        have = true;
                    } else {
                        sg = pos == 0 ? x : sg + x;
                        if (++pos == F) {
                            acc = have ? acc + sg : sg;
                            have = true;
                            pos = 0;
                        }
                    }
                }
                if (l.flags & fsdp::kReduceLast) {
                    acc = acc / post;
                    out[static_cast<size_t>(j)] = accumulate ? out[static_cast<size_t>(j)] + acc : acc;
                } else {
                    if (l.flags & fsdp::kReduceTOut) carry_t[j] = acc;
                    if (l.flags & fsdp::kReduceSOut) {
                        CHECK(carry_s != nullptr, "a carried group sum has a slot");
                        if (carry_s) carry_s[j] = sg;
                    }
                }
            }
        }
        for (int j = 0; j < kOut; ++j)
            CHECK(bits(out[static_cast<size_t>(j)]) == bits(want[j]), "planned reduction equals the sequential one");
    }
}

int main(int argc, char** argv) {
    const int iters = argc > 1 ? std::atoi(argv[1]) : 400;
    std::mt19937_64 rng(12345);
    for (int it = 0; it < iters; ++it) {
        const Unit u = random_unit(rng);
        const int32_t N = static_cast<int32_t>(1 + rng() % (it % 5 == 0 ? 300 : 17));
        check_unit(u, fsdp::kFlat, N, rng);
        check_unit(u, fsdp::kRows, N, rng);
    }
    check_overflow();
    check_sweep_runs(rng, 20 * iters);
    check_reduce_plans(rng, 10 * iters);
    if (g_fail) {
        std::fprintf(stderr, "%d failures\n", g_fail);
        return 1;
    }
    std::printf("planner ok: %d units x 2 layouts\n", iters);
    return 0;
}
