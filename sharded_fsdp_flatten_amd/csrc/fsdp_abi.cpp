// fsdp_abi.cpp -- the C ABI declared in include/fsdp_flatten.h.
//
// Every entry point validates all of its arguments on the host first and only
// then makes HIP calls, so a call that fails validation launches and writes
// nothing (and works on a machine without a GPU).  No C++ exception leaves an
// entry point: each body runs under guarded().
#include "fsdp_flatten.h"

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdio>
#include <memory>
#include <new>
#include <string>
#include <vector>

#include "kernels.h"
#include "plan.h"

struct fsdp_unit {
    fsdp::UnitPlan plan;
};

namespace {

thread_local std::string g_last_error;

fsdp_status fail(fsdp_status s, const std::string& msg) {
    g_last_error = msg;
    return s;
}

fsdp_status ok() {
    g_last_error.clear();
    return FSDP_OK;
}

// Runs an entry point's body so that no C++ exception crosses the C ABI: host memory
// exhaustion (a plan's tables are std::vectors) becomes FSDP_E_NOMEM, anything else
// FSDP_E_UNSUPPORTED.  The message store itself may fail under exhaustion; then the
// message is left empty.
template <typename F>
fsdp_status guarded(const char* who, F&& body) noexcept {
    fsdp_status s;
    const char* what;
    try {
        return body();
    } catch (const std::bad_alloc&) {
        s = FSDP_E_NOMEM;
        what = ": out of host memory";
    } catch (...) {
        s = FSDP_E_UNSUPPORTED;
        what = ": unexpected internal error";
    }
    try {
        g_last_error = std::string(who) + what;
    } catch (...) {
        g_last_error.clear();
    }
    return s;
}

bool aligned_to(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

fsdp_status hip_fail(hipError_t e, const char* what) {
    return fail(FSDP_E_HIP, std::string(what) + ": " + hipGetErrorName(e) + " (" +
                                hipGetErrorString(e) + ")");
}

// A table of n device pointers to buffers of counts[i] elements of `elem` bytes:
// non-null where the count is non-zero, aligned to the element size.
fsdp_status check_ptr_table(const void* const* table, size_t n, const int64_t* counts,
                            int64_t uniform_count, size_t elem, const char* name) {
    bool any = false;
    for (size_t i = 0; i < n; ++i) any = any || (counts ? counts[i] : uniform_count) > 0;
    if (!any) return FSDP_OK;
    if (!table) return fail(FSDP_E_ARG, std::string(name) + " table is NULL");
    for (size_t i = 0; i < n; ++i) {
        const int64_t c = counts ? counts[i] : uniform_count;
        if (c == 0) continue;
        if (!table[i])
            return fail(FSDP_E_ARG, std::string(name) + "[" + std::to_string(i) + "] is NULL");
        if (!aligned_to(table[i], elem))
            return fail(FSDP_E_ALIGN, std::string(name) + "[" + std::to_string(i) +
                                          "] is not aligned to its element size");
    }
    return FSDP_OK;
}

fsdp_status check_buf(const void* p, int64_t count, size_t elem, const char* name) {
    if (count == 0) return FSDP_OK;
    if (!p) return fail(FSDP_E_ARG, std::string(name) + " is NULL");
    if (!aligned_to(p, elem))
        return fail(FSDP_E_ALIGN, std::string(name) + " is not aligned to its element size");
    return FSDP_OK;
}

// The group of a reduction's options, checked: 0 and N are one flat sum (returned as N).
fsdp_status reduce_group(const fsdp::UnitPlan& u, const fsdp_reduce_opts* opts, int64_t* group) {
    int64_t g = opts->group;
    if (g < 0 || g > u.N) return fail(FSDP_E_RANGE, "group must be in [0, N]");
    if (g == 0) g = u.N;
    if (u.N % g != 0) return fail(FSDP_E_RANGE, "group must divide N");
    *group = g;
    return FSDP_OK;
}

fsdp_status reduce_impl(const fsdp_unit* unit, const uint16_t* const* contribs,
                        const fsdp_reduce_opts* opts, float* grad_shard, void* stream,
                        const char* who) {
    if (!unit) return fail(FSDP_E_ARG, "unit is NULL");
    if (!opts) return fail(FSDP_E_ARG, "opts is NULL");
    const fsdp::UnitPlan& u = unit->plan;
    const float pre = opts->pre_divide, post = opts->post_divide;
    if (!std::isfinite(pre) || pre == 0.0f)
        return fail(FSDP_E_RANGE, "pre_divide must be finite and non-zero");
    if (!std::isfinite(post) || post == 0.0f)
        return fail(FSDP_E_RANGE, "post_divide must be finite and non-zero");
    int64_t group = 0;
    fsdp_status s;
    if ((s = reduce_group(u, opts, &group)) != FSDP_OK) return s;
    if (opts->kernel != FSDP_REDUCE_AUTO && opts->kernel != FSDP_REDUCE_TILES &&
        opts->kernel != FSDP_REDUCE_SWEEP)
        return fail(FSDP_E_RANGE, "kernel must be FSDP_REDUCE_AUTO, _TILES or _SWEEP");
    if ((s = check_ptr_table(reinterpret_cast<const void* const*>(contribs),
                             static_cast<size_t>(u.N), nullptr, u.S, sizeof(uint16_t),
                             "contribs")) != FSDP_OK)
        return s;
    if ((s = check_buf(grad_shard, u.S, sizeof(float), "grad_shard")) != FSDP_OK) return s;
    const int64_t need = fsdp::reduce_workspace_floats(u.N, u.S, group, opts->accumulate != 0);
    float* ws = need > 0 ? opts->workspace : nullptr;
    if (need > 0) {
        if (!ws) return fail(FSDP_E_ARG, "these options need a workspace of " +
                                             std::to_string(need) + " floats; workspace is NULL");
        if (!aligned_to(ws, 16)) return fail(FSDP_E_ALIGN, "workspace is not 16-byte aligned");
        if (opts->workspace_len < need)
            return fail(FSDP_E_RANGE, "workspace holds " + std::to_string(opts->workspace_len) +
                                          " floats; these options need " + std::to_string(need));
    }
    if (u.S == 0) return ok();
    const hipError_t e = fsdp::launch_grad_reduce(
        contribs, u.N, u.S, pre, post, group, opts->accumulate != 0, grad_shard, ws,
        static_cast<fsdp::ReduceKernel>(opts->kernel), static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, (std::string(who) + " launch").c_str());
    return ok();
}

fsdp_status check_rank(const fsdp::UnitPlan& u, int32_t k) {
    if (k != FSDP_ALL_RANKS && (k < 0 || k >= u.N))
        return fail(FSDP_E_RANGE, "k must be in [0, N) or FSDP_ALL_RANKS");
    return FSDP_OK;
}

std::vector<int64_t> param_numels(const fsdp::UnitPlan& u) {
    std::vector<int64_t> n;
    n.reserve(u.params.size());
    for (const auto& p : u.params) n.push_back(p.numel);
    return n;
}

}  // namespace

extern "C" {

int32_t fsdp_abi_version(void) { return FSDP_ABI_VERSION; }

const char* fsdp_last_error(void) { return g_last_error.c_str(); }

const char* fsdp_status_string(int32_t s) {
    switch (s) {
        case FSDP_OK: return "FSDP_OK";
        case FSDP_E_ARG: return "FSDP_E_ARG";
        case FSDP_E_RANGE: return "FSDP_E_RANGE";
        case FSDP_E_ALIGN: return "FSDP_E_ALIGN";
        case FSDP_E_OVERFLOW: return "FSDP_E_OVERFLOW";
        case FSDP_E_NOMEM: return "FSDP_E_NOMEM";
        case FSDP_E_HIP: return "FSDP_E_HIP";
        case FSDP_E_UNSUPPORTED: return "FSDP_E_UNSUPPORTED";
        default: return "FSDP_E_UNKNOWN";
    }
}

fsdp_status fsdp_unit_create(int32_t layout, int32_t n_params, const int32_t* ndims,
                             const int64_t* dims, int32_t N, fsdp_unit** out) {
    return guarded("fsdp_unit_create", [&]() -> fsdp_status {
        if (!out) return fail(FSDP_E_ARG, "out is NULL");
        *out = nullptr;
        // freed on every early return and on an exception (the guard reports it)
        std::unique_ptr<fsdp_unit> u(new (std::nothrow) fsdp_unit);
        if (!u) return fail(FSDP_E_NOMEM, "cannot allocate the unit plan");
        std::string err;
        const int rc = fsdp::plan_create(layout, n_params, ndims, dims, N, &u->plan, &err);
        if (rc != 0) return fail(static_cast<fsdp_status>(rc), err);
        *out = u.release();
        return ok();
    });
}

fsdp_status fsdp_unit_destroy(fsdp_unit* unit) {
    return guarded("fsdp_unit_destroy", [&]() -> fsdp_status {
        delete unit;
        return ok();
    });
}

fsdp_status fsdp_unit_info(const fsdp_unit* unit, int32_t k, fsdp_unit_sizes* out) {
    return guarded("fsdp_unit_info", [&]() -> fsdp_status {
        if (!unit || !out) return fail(FSDP_E_ARG, "unit and out must not be NULL");
        const fsdp::UnitPlan& u = unit->plan;
        if (k != FSDP_ALL_RANKS && (k < 0 || k >= u.N))
            return fail(FSDP_E_RANGE, "k must be in [0, N) or FSDP_ALL_RANKS");
        out->layout = u.layout;
        out->n_params = static_cast<int32_t>(u.params.size());
        out->N = u.N;
        out->T = u.T;
        out->S = u.S;
        out->L = u.L;
        out->pad = u.pad;
        out->valid = k == FSDP_ALL_RANKS ? 0 : u.valid(k);
        out->bytes_per_rank = 16 * u.S;
        return ok();
    });
}

fsdp_status fsdp_unit_param_offset(const fsdp_unit* unit, int32_t i, int64_t* offset) {
    return guarded("fsdp_unit_param_offset", [&]() -> fsdp_status {
        if (!unit || !offset) return fail(FSDP_E_ARG, "unit and offset must not be NULL");
        if (i < 0 || static_cast<size_t>(i) >= unit->plan.params.size())
            return fail(FSDP_E_RANGE, "parameter index out of range");
        *offset = unit->plan.params[static_cast<size_t>(i)].offset;
        return ok();
    });
}

fsdp_status fsdp_unit_recv_pitch(const fsdp_unit* unit, int64_t* pitch) {
    return guarded("fsdp_unit_recv_pitch", [&]() -> fsdp_status {
        if (!unit || !pitch) return fail(FSDP_E_ARG, "unit and pitch must not be NULL");
        constexpr int64_t kLine = 64;  // bf16 elements per 128-byte line
        const int64_t S = unit->plan.S;
        // S <= L fits int64 with room for the round-up (plan_create bounds L)
        *pitch = (S + kLine - 1) / kLine * kLine;
        return ok();
    });
}

fsdp_status fsdp_flatten_shard(const fsdp_unit* unit, const float* const* params, int32_t k,
                               float* shard, void* stream) {
    return guarded("fsdp_flatten_shard", [&]() -> fsdp_status {
        if (!unit) return fail(FSDP_E_ARG, "unit is NULL");
        const fsdp::UnitPlan& u = unit->plan;
        if (k != FSDP_ALL_RANKS && (k < 0 || k >= u.N))
            return fail(FSDP_E_RANGE, "k must be in [0, N) or FSDP_ALL_RANKS");
        const int64_t out_len = k == FSDP_ALL_RANKS ? u.L : u.S;
        const std::vector<int64_t> numels = param_numels(u);
        fsdp_status s = check_ptr_table(reinterpret_cast<const void* const*>(params), numels.size(),
                                        numels.data(), 0, sizeof(float), "params");
        if (s != FSDP_OK) return s;
        if ((s = check_buf(shard, out_len, sizeof(float), "shard")) != FSDP_OK) return s;
        if (out_len == 0) return ok();
        std::vector<fsdp::CopySeg> segs;
        fsdp::plan_flatten(u, reinterpret_cast<const void* const*>(params), k, shard, sizeof(float),
                           &segs);
        const hipError_t e =
            fsdp::launch_segcopy(segs, fsdp::Pipe::kF32toF32, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return hip_fail(e, "fsdp_flatten_shard launch");
        return ok();
    });
}

fsdp_status fsdp_unflatten_copyout(const fsdp_unit* unit, const float* gathered,
                                   uint16_t* const* outs, void* stream) {
    return guarded("fsdp_unflatten_copyout", [&]() -> fsdp_status {
        if (!unit) return fail(FSDP_E_ARG, "unit is NULL");
        const fsdp::UnitPlan& u = unit->plan;
        const std::vector<int64_t> numels = param_numels(u);
        fsdp_status s;
        if ((s = check_buf(gathered, u.T > 0 ? u.L : 0, sizeof(float), "gathered")) != FSDP_OK)
            return s;
        if ((s = check_ptr_table(reinterpret_cast<const void* const*>(outs), numels.size(),
                                 numels.data(), 0, sizeof(uint16_t), "outs")) != FSDP_OK)
            return s;
        if (u.T == 0) return ok();
        std::vector<fsdp::CopySeg> segs;
        fsdp::plan_copyout(u, gathered, sizeof(float), reinterpret_cast<void* const*>(outs),
                           sizeof(uint16_t), &segs);
        const hipError_t e =
            fsdp::launch_segcopy(segs, fsdp::Pipe::kF32toBF16, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return hip_fail(e, "fsdp_unflatten_copyout launch");
        return ok();
    });
}

fsdp_status fsdp_grad_reduce_shard(const fsdp_unit* unit, const uint16_t* const* contribs,
                                   float pre_divide, float post_divide, float* grad_shard,
                                   void* stream) {
    return guarded("fsdp_grad_reduce_shard", [&]() -> fsdp_status {
        fsdp_reduce_opts opts{};
        opts.pre_divide = pre_divide;
        opts.post_divide = post_divide;
        return reduce_impl(unit, contribs, &opts, grad_shard, stream, "fsdp_grad_reduce_shard");
    });
}

fsdp_status fsdp_grad_reduce_shard_ex(const fsdp_unit* unit, const uint16_t* const* contribs,
                                      const fsdp_reduce_opts* opts, float* grad_shard,
                                      void* stream) {
    return guarded("fsdp_grad_reduce_shard_ex", [&]() -> fsdp_status {
        return reduce_impl(unit, contribs, opts, grad_shard, stream, "fsdp_grad_reduce_shard_ex");
    });
}

fsdp_status fsdp_grad_reduce_workspace(const fsdp_unit* unit, const fsdp_reduce_opts* opts,
                                       int64_t* n_floats) {
    return guarded("fsdp_grad_reduce_workspace", [&]() -> fsdp_status {
        if (!unit || !opts || !n_floats)
            return fail(FSDP_E_ARG, "unit, opts and n_floats must not be NULL");
        const fsdp::UnitPlan& u = unit->plan;
        int64_t group = 0;
        const fsdp_status s = reduce_group(u, opts, &group);
        if (s != FSDP_OK) return s;
        *n_floats = fsdp::reduce_workspace_floats(u.N, u.S, group, opts->accumulate != 0);
        return ok();
    });
}

fsdp_status fsdp_adam_shard(const fsdp_unit* unit, float* param, const float* grad,
                            float* exp_avg, float* exp_avg_sq, const fsdp_adamw_cfg* cfg,
                            uint16_t* param_bf16, void* stream) {
    return guarded("fsdp_adam_shard", [&]() -> fsdp_status {
        if (!unit) return fail(FSDP_E_ARG, "unit is NULL");
        if (!cfg) return fail(FSDP_E_ARG, "cfg is NULL");
        const fsdp::UnitPlan& u = unit->plan;
        if (cfg->step < 1) return fail(FSDP_E_RANGE, "step must be >= 1");
        if (!(cfg->beta1 >= 0.0 && cfg->beta1 < 1.0)) return fail(FSDP_E_RANGE, "beta1 not in [0,1)");
        if (!(cfg->beta2 >= 0.0 && cfg->beta2 < 1.0)) return fail(FSDP_E_RANGE, "beta2 not in [0,1)");
        if (!std::isfinite(cfg->lr)) return fail(FSDP_E_RANGE, "lr must be finite");
        if (!std::isfinite(cfg->eps) || cfg->eps < 0.0)
            return fail(FSDP_E_RANGE, "eps must be finite and >= 0");
        if (!std::isfinite(cfg->weight_decay)) return fail(FSDP_E_RANGE, "weight_decay must be finite");
        fsdp_status s;
        if ((s = check_buf(param, u.S, sizeof(float), "param")) != FSDP_OK) return s;
        if ((s = check_buf(grad, u.S, sizeof(float), "grad")) != FSDP_OK) return s;
        if ((s = check_buf(exp_avg, u.S, sizeof(float), "exp_avg")) != FSDP_OK) return s;
        if ((s = check_buf(exp_avg_sq, u.S, sizeof(float), "exp_avg_sq")) != FSDP_OK) return s;
        if (param_bf16 && !aligned_to(param_bf16, sizeof(uint16_t)))
            return fail(FSDP_E_ALIGN, "param_bf16 is not aligned to its element size");
        // Kingma & Ba's bias corrections and decoupled decay, scalars in double,
        // each rounded once to float.
        const double t = static_cast<double>(cfg->step);
        fsdp::AdamScalars sc;
        sc.decay = static_cast<float>(1.0 - cfg->lr * cfg->weight_decay);
        sc.b1 = static_cast<float>(cfg->beta1);
        sc.omb1 = static_cast<float>(1.0 - cfg->beta1);
        sc.b2 = static_cast<float>(cfg->beta2);
        sc.omb2 = static_cast<float>(1.0 - cfg->beta2);
        sc.step_size = static_cast<float>(cfg->lr / (1.0 - std::pow(cfg->beta1, t)));
        sc.bc2s = static_cast<float>(std::sqrt(1.0 - std::pow(cfg->beta2, t)));
        sc.eps = static_cast<float>(cfg->eps);
        if (u.S == 0) return ok();
        const hipError_t e = fsdp::launch_adamw(param, grad, exp_avg, exp_avg_sq, param_bf16, u.S, sc,
                                                static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return hip_fail(e, "fsdp_adam_shard launch");
        return ok();
    });
}

fsdp_status fsdp_cast_to_bf16(const fsdp_unit* unit, int32_t k, const float* src, uint16_t* dst,
                              void* stream) {
    return guarded("fsdp_cast_to_bf16", [&]() -> fsdp_status {
        if (!unit) return fail(FSDP_E_ARG, "unit is NULL");
        const fsdp::UnitPlan& u = unit->plan;
        fsdp_status s;
        if ((s = check_rank(u, k)) != FSDP_OK) return s;
        const int64_t n = k == FSDP_ALL_RANKS ? u.L : u.S;
        if ((s = check_buf(src, n, sizeof(float), "src")) != FSDP_OK) return s;
        if ((s = check_buf(dst, n, sizeof(uint16_t), "dst")) != FSDP_OK) return s;
        if (n == 0) return ok();
        std::vector<fsdp::CopySeg> segs;
        fsdp::plan_whole(u, k, src, dst, &segs);
        const hipError_t e =
            fsdp::launch_segcopy(segs, fsdp::Pipe::kF32toBF16, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return hip_fail(e, "fsdp_cast_to_bf16 launch");
        return ok();
    });
}

fsdp_status fsdp_unflatten_copyout_bf16(const fsdp_unit* unit, const uint16_t* gathered,
                                        uint16_t* const* outs, void* stream) {
    return guarded("fsdp_unflatten_copyout_bf16", [&]() -> fsdp_status {
        if (!unit) return fail(FSDP_E_ARG, "unit is NULL");
        const fsdp::UnitPlan& u = unit->plan;
        const std::vector<int64_t> numels = param_numels(u);
        fsdp_status s;
        if ((s = check_buf(gathered, u.T > 0 ? u.L : 0, sizeof(uint16_t), "gathered")) != FSDP_OK)
            return s;
        if ((s = check_ptr_table(reinterpret_cast<const void* const*>(outs), numels.size(),
                                 numels.data(), 0, sizeof(uint16_t), "outs")) != FSDP_OK)
            return s;
        if (u.T == 0) return ok();
        std::vector<fsdp::CopySeg> segs;
        fsdp::plan_copyout(u, gathered, sizeof(uint16_t), reinterpret_cast<void* const*>(outs),
                           sizeof(uint16_t), &segs);
        const hipError_t e =
            fsdp::launch_segcopy(segs, fsdp::Pipe::kBF16toBF16, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return hip_fail(e, "fsdp_unflatten_copyout_bf16 launch");
        return ok();
    });
}

fsdp_status fsdp_flatten_shard_bf16(const fsdp_unit* unit, const uint16_t* const* params,
                                    int32_t k, uint16_t* shard, void* stream) {
    return guarded("fsdp_flatten_shard_bf16", [&]() -> fsdp_status {
        if (!unit) return fail(FSDP_E_ARG, "unit is NULL");
        const fsdp::UnitPlan& u = unit->plan;
        fsdp_status s;
        if ((s = check_rank(u, k)) != FSDP_OK) return s;
        const int64_t out_len = k == FSDP_ALL_RANKS ? u.L : u.S;
        const std::vector<int64_t> numels = param_numels(u);
        if ((s = check_ptr_table(reinterpret_cast<const void* const*>(params), numels.size(),
                                 numels.data(), 0, sizeof(uint16_t), "params")) != FSDP_OK)
            return s;
        if ((s = check_buf(shard, out_len, sizeof(uint16_t), "shard")) != FSDP_OK) return s;
        if (out_len == 0) return ok();
        std::vector<fsdp::CopySeg> segs;
        fsdp::plan_flatten(u, reinterpret_cast<const void* const*>(params), k, shard,
                           sizeof(uint16_t), &segs);
        const hipError_t e =
            fsdp::launch_segcopy(segs, fsdp::Pipe::kBF16toBF16, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return hip_fail(e, "fsdp_flatten_shard_bf16 launch");
        return ok();
    });
}

fsdp_status fsdp_grad_accumulate(const fsdp_unit* unit, int32_t k, const uint16_t* grad,
                                 float* acc, int32_t init, void* stream) {
    return guarded("fsdp_grad_accumulate", [&]() -> fsdp_status {
        if (!unit) return fail(FSDP_E_ARG, "unit is NULL");
        const fsdp::UnitPlan& u = unit->plan;
        fsdp_status s;
        if ((s = check_rank(u, k)) != FSDP_OK) return s;
        const int64_t n = k == FSDP_ALL_RANKS ? u.L : u.S;
        if ((s = check_buf(grad, n, sizeof(uint16_t), "grad")) != FSDP_OK) return s;
        if ((s = check_buf(acc, n, sizeof(float), "acc")) != FSDP_OK) return s;
        if (n == 0) return ok();
        const hipError_t e =
            fsdp::launch_grad_accumulate(grad, acc, n, init != 0, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return hip_fail(e, "fsdp_grad_accumulate launch");
        return ok();
    });
}

fsdp_status fsdp_grad_unscale(const fsdp_unit* unit, int32_t k, float* grad, float inv_scale,
                              float* found_inf, void* stream) {
    return guarded("fsdp_grad_unscale", [&]() -> fsdp_status {
        if (!unit) return fail(FSDP_E_ARG, "unit is NULL");
        const fsdp::UnitPlan& u = unit->plan;
        fsdp_status s;
        if ((s = check_rank(u, k)) != FSDP_OK) return s;
        if (!std::isfinite(inv_scale)) return fail(FSDP_E_ARG, "inv_scale must be finite");
        const int64_t n = k == FSDP_ALL_RANKS ? u.L : u.S;
        if ((s = check_buf(grad, n, sizeof(float), "grad")) != FSDP_OK) return s;
        if (n == 0) return ok();
        if (found_inf && !aligned_to(found_inf, sizeof(float)))
            return fail(FSDP_E_ALIGN, "found_inf is not aligned to its element size");
        const hipError_t e = fsdp::launch_grad_unscale(grad, n, inv_scale, found_inf,
                                                       static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return hip_fail(e, "fsdp_grad_unscale launch");
        return ok();
    });
}

fsdp_status fsdp_grad_sqnorm_workspace(const fsdp_unit* unit, int32_t k, int64_t* n_doubles) {
    return guarded("fsdp_grad_sqnorm_workspace", [&]() -> fsdp_status {
        if (!unit || !n_doubles) return fail(FSDP_E_ARG, "unit and n_doubles must not be NULL");
        const fsdp::UnitPlan& u = unit->plan;
        if (k < 0 || k >= u.N) return fail(FSDP_E_RANGE, "k must be in [0, N)");
        std::vector<fsdp::ParamRun> runs;
        fsdp::plan_param_runs(u, k, &runs);
        *n_doubles = fsdp::sqnorm_tiles(runs);
        return ok();
    });
}

fsdp_status fsdp_grad_sqnorm(const fsdp_unit* unit, int32_t k, const float* grad,
                             double* workspace, int64_t workspace_len, double* out, void* stream) {
    return guarded("fsdp_grad_sqnorm", [&]() -> fsdp_status {
        if (!unit) return fail(FSDP_E_ARG, "unit is NULL");
        const fsdp::UnitPlan& u = unit->plan;
        if (k < 0 || k >= u.N) return fail(FSDP_E_RANGE, "k must be in [0, N)");
        std::vector<fsdp::ParamRun> runs;
        fsdp::plan_param_runs(u, k, &runs);
        const int64_t need = fsdp::sqnorm_tiles(runs);
        fsdp_status s;
        if ((s = check_buf(grad, u.S, sizeof(float), "grad")) != FSDP_OK) return s;
        if ((s = check_buf(out, static_cast<int64_t>(runs.size()), sizeof(double), "out")) != FSDP_OK)
            return s;
        if (workspace_len < need)
            return fail(FSDP_E_RANGE, "workspace holds " + std::to_string(workspace_len) +
                                          " doubles; this rank needs " + std::to_string(need));
        if ((s = check_buf(workspace, need, sizeof(double), "workspace")) != FSDP_OK) return s;
        if (runs.empty()) return ok();
        const hipError_t e = fsdp::launch_grad_sqnorm(grad, runs, workspace, out,
                                                      static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return hip_fail(e, "fsdp_grad_sqnorm launch");
        return ok();
    });
}

fsdp_status fsdp_grad_sqnorm_noalloc(const fsdp_unit* unit, int32_t k, const float* grad,
                                     double* out, void* stream) {
    return guarded("fsdp_grad_sqnorm_noalloc", [&]() -> fsdp_status {
        if (!unit) return fail(FSDP_E_ARG, "unit is NULL");
        const fsdp::UnitPlan& u = unit->plan;
        if (k < 0 || k >= u.N) return fail(FSDP_E_RANGE, "k must be in [0, N)");
        std::vector<fsdp::ParamRun> runs;
        fsdp::plan_param_runs(u, k, &runs);
        const int64_t need = fsdp::sqnorm_tiles(runs);
        fsdp_status s;
        if ((s = check_buf(grad, u.S, sizeof(float), "grad")) != FSDP_OK) return s;
        if ((s = check_buf(out, static_cast<int64_t>(runs.size()), sizeof(double), "out")) != FSDP_OK)
            return s;
        if (need > fsdp::sqnorm_scratch_doubles())
            return fail(FSDP_E_RANGE, "rank " + std::to_string(k) + " needs " + std::to_string(need) +
                                          " partial sums; the library's scratch holds " +
                                          std::to_string(fsdp::sqnorm_scratch_doubles()) +
                                          " (use fsdp_grad_sqnorm with a workspace)");
        if (runs.empty()) return ok();
        double* partial = nullptr;
        hipError_t e = fsdp::sqnorm_scratch(&partial);
        if (e != hipSuccess) return hip_fail(e, "fsdp_grad_sqnorm_noalloc scratch lookup");
        e = fsdp::launch_grad_sqnorm(grad, runs, partial, out, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return hip_fail(e, "fsdp_grad_sqnorm_noalloc launch");
        return ok();
    });
}

}  // extern "C"
