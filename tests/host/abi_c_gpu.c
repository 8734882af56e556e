/* The data path driven from C alone (no Python, no torch): device buffers from hipMalloc,
 * every call through include/fsdp_flatten.h, results compared bit for bit with the CPU
 * oracle's C functions (oracle/liboracle.so, declared here).  Inputs come from a local
 * xorshift generator.  Prints "ok" and exits 0 when every check holds; exits 1 on a
 * mismatch, 2 on a setup or HIP error. */
#include "fsdp_flatten.h"

#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* the oracle (oracle/fsdp_oracle.c) */
int orc_flat_shard(int32_t p, const int64_t* numel, const float* const* params, int64_t N,
                   int64_t k, float* out);
void orc_flat_copyout(int32_t p, const int64_t* numel, const float* gathered,
                      uint16_t* const* outs);
void orc_grad_reduce(int64_t N, int64_t len, const uint16_t* const* contribs, float pre,
                     float post, float* out);
void orc_adamw(int64_t len, float* p, const float* g, float* m, float* v, double lr,
               double beta1, double beta2, double eps, double wd, int64_t step, uint16_t* pb);

static int failures = 0;

#define HIP(x)                                                                     \
    do {                                                                           \
        hipError_t e_ = (x);                                                       \
        if (e_ != hipSuccess) {                                                    \
            fprintf(stderr, "%s:%d: %s: %s\n", __FILE__, __LINE__, #x,             \
                    hipGetErrorString(e_));                                        \
            exit(2);                                                               \
        }                                                                          \
    } while (0)
#define OK(x)                                                                      \
    do {                                                                           \
        fsdp_status s_ = (x);                                                      \
        if (s_ != FSDP_OK) {                                                       \
            fprintf(stderr, "%s:%d: %s: %s: %s\n", __FILE__, __LINE__, #x,         \
                    fsdp_status_string(s_), fsdp_last_error());                    \
            exit(2);                                                               \
        }                                                                          \
    } while (0)

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (uint32_t)(rng >> 16);
}
/* a float in about [-0.05, 0.05] */
static float next_f(void) { return ((float)(next_u32() & 0xFFFFFF) / 16777216.0f - 0.5f) * 0.1f; }
/* a finite bf16 bit pattern of magnitude about 1e-3 */
static uint16_t next_bf16(void) { return (uint16_t)(0x3A00u + (next_u32() % 0x0400u)) | (uint16_t)(next_u32() & 0x8000u); }

static void* xmalloc(size_t n) {
    void* p = malloc(n ? n : 1);
    if (!p) { fprintf(stderr, "out of host memory\n"); exit(2); }
    return p;
}
static void* dmalloc(size_t n) {
    void* p = NULL;
    HIP(hipMalloc(&p, n ? n : 16));
    return p;
}
static void same(const void* got, const void* want, size_t bytes, const char* what) {
    if (memcmp(got, want, bytes) != 0) {
        fprintf(stderr, "mismatch: %s\n", what);
        ++failures;
    }
}

static void reduce_case(int32_t N, int64_t S, float pre, float post) {
    const int64_t dims[1] = {(int64_t)N * S};
    const int32_t ndims[1] = {1};
    fsdp_unit* u = NULL;
    uint16_t** h = (uint16_t**)xmalloc(sizeof(uint16_t*) * (size_t)N);
    uint16_t** d = (uint16_t**)xmalloc(sizeof(uint16_t*) * (size_t)N);
    float* want = (float*)xmalloc(sizeof(float) * (size_t)S);
    float* got = (float*)xmalloc(sizeof(float) * (size_t)S);
    float* dout = (float*)dmalloc(sizeof(float) * (size_t)S);
    char what[96];
    int32_t r;
    OK(fsdp_unit_create(FSDP_FLAT, 1, ndims, dims, N, &u));
    for (r = 0; r < N; ++r) {
        int64_t j;
        h[r] = (uint16_t*)xmalloc(sizeof(uint16_t) * (size_t)S);
        for (j = 0; j < S; ++j) h[r][j] = next_bf16();
        d[r] = (uint16_t*)dmalloc(sizeof(uint16_t) * (size_t)S);
        HIP(hipMemcpy(d[r], h[r], sizeof(uint16_t) * (size_t)S, hipMemcpyHostToDevice));
    }
    OK(fsdp_grad_reduce_shard(u, (const uint16_t* const*)d, pre, post, dout, NULL));
    HIP(hipDeviceSynchronize());
    HIP(hipMemcpy(got, dout, sizeof(float) * (size_t)S, hipMemcpyDeviceToHost));
    orc_grad_reduce(N, S, (const uint16_t* const*)h, pre, post, want);
    snprintf(what, sizeof what, "reduce N=%d S=%lld", (int)N, (long long)S);
    same(got, want, sizeof(float) * (size_t)S, what);
    for (r = 0; r < N; ++r) {
        free(h[r]);
        HIP(hipFree(d[r]));
    }
    free(h); free(d); free(want); free(got);
    HIP(hipFree(dout));
    OK(fsdp_unit_destroy(u));
}

int main(void) {
    /* a padded, ragged FLAT unit: [1000,37], [37], [13,7,3], a 0-d parameter; N = 5 */
    enum { P = 4, NR = 5 };
    const int32_t ndims[P] = {2, 1, 3, 0};
    const int64_t dims[6] = {1000, 37, 37, 13, 7, 3};
    const int64_t numel[P] = {37000, 37, 273, 1};
    fsdp_unit* u = NULL;
    fsdp_unit_sizes sz;
    float* hp[P];
    float* dp[P];
    uint16_t* hout[P];
    uint16_t* dout[P];
    uint16_t* want16[P];
    float *wantL, *gotL, *dL, *dS, *wantS;
    int32_t i;
    int64_t j, S, L;

    OK(fsdp_unit_create(FSDP_FLAT, P, ndims, dims, NR, &u));
    OK(fsdp_unit_info(u, FSDP_ALL_RANKS, &sz));
    S = sz.S;
    L = sz.L;
    if (sz.T != 37311 || S != 7463 || L != 37315 || sz.pad != 4) {
        fprintf(stderr, "unexpected sizes\n");
        return 1;
    }
    for (i = 0; i < P; ++i) {
        hp[i] = (float*)xmalloc(sizeof(float) * (size_t)numel[i]);
        for (j = 0; j < numel[i]; ++j) hp[i][j] = next_f();
        dp[i] = (float*)dmalloc(sizeof(float) * (size_t)numel[i]);
        HIP(hipMemcpy(dp[i], hp[i], sizeof(float) * (size_t)numel[i], hipMemcpyHostToDevice));
    }
    /* flatten: all ranks (the gathered layout), then rank 3 */
    wantL = (float*)xmalloc(sizeof(float) * (size_t)L);
    gotL = (float*)xmalloc(sizeof(float) * (size_t)L);
    dL = (float*)dmalloc(sizeof(float) * (size_t)L);
    OK(fsdp_flatten_shard(u, (const float* const*)dp, FSDP_ALL_RANKS, dL, NULL));
    HIP(hipDeviceSynchronize());
    HIP(hipMemcpy(gotL, dL, sizeof(float) * (size_t)L, hipMemcpyDeviceToHost));
    if (orc_flat_shard(P, numel, (const float* const*)hp, NR, -1, wantL) != 0) return 2;
    same(gotL, wantL, sizeof(float) * (size_t)L, "flatten, all ranks");
    wantS = (float*)xmalloc(sizeof(float) * (size_t)S);
    dS = (float*)dmalloc(sizeof(float) * (size_t)S);
    OK(fsdp_flatten_shard(u, (const float* const*)dp, 3, dS, NULL));
    HIP(hipDeviceSynchronize());
    HIP(hipMemcpy(gotL, dS, sizeof(float) * (size_t)S, hipMemcpyDeviceToHost));
    if (orc_flat_shard(P, numel, (const float* const*)hp, NR, 3, wantS) != 0) return 2;
    same(gotL, wantS, sizeof(float) * (size_t)S, "flatten, rank 3");
    /* copy-out of the gathered unit */
    for (i = 0; i < P; ++i) {
        hout[i] = (uint16_t*)xmalloc(sizeof(uint16_t) * (size_t)numel[i]);
        want16[i] = (uint16_t*)xmalloc(sizeof(uint16_t) * (size_t)numel[i]);
        dout[i] = (uint16_t*)dmalloc(sizeof(uint16_t) * (size_t)numel[i]);
    }
    OK(fsdp_unflatten_copyout(u, dL, (uint16_t* const*)dout, NULL));
    HIP(hipDeviceSynchronize());
    orc_flat_copyout(P, numel, wantL, (uint16_t* const*)want16);
    for (i = 0; i < P; ++i) {
        HIP(hipMemcpy(hout[i], dout[i], sizeof(uint16_t) * (size_t)numel[i], hipMemcpyDeviceToHost));
        same(hout[i], want16[i], sizeof(uint16_t) * (size_t)numel[i], "copy-out");
    }
    /* AdamW, two steps on rank 3's shard with a gradient from the generator */
    {
        float* hg = (float*)xmalloc(sizeof(float) * (size_t)S);
        float* hm = (float*)calloc((size_t)S, sizeof(float));
        float* hv = (float*)calloc((size_t)S, sizeof(float));
        float* got = (float*)xmalloc(sizeof(float) * (size_t)S);
        uint16_t* hpb = (uint16_t*)xmalloc(sizeof(uint16_t) * (size_t)S);
        uint16_t* gpb = (uint16_t*)xmalloc(sizeof(uint16_t) * (size_t)S);
        float *dg = (float*)dmalloc(sizeof(float) * (size_t)S), *dm = (float*)dmalloc(sizeof(float) * (size_t)S);
        float* dv = (float*)dmalloc(sizeof(float) * (size_t)S);
        uint16_t* dpb = (uint16_t*)dmalloc(sizeof(uint16_t) * (size_t)S);
        fsdp_adamw_cfg cfg = {1e-3, 0.9, 0.999, 1e-8, 0.01, 1};
        int64_t t;
        if (!hm || !hv) return 2;
        HIP(hipMemset(dm, 0, sizeof(float) * (size_t)S));
        HIP(hipMemset(dv, 0, sizeof(float) * (size_t)S));
        for (t = 1; t <= 2; ++t) {
            for (j = 0; j < S; ++j) hg[j] = next_f() * 0.01f;
            HIP(hipMemcpy(dg, hg, sizeof(float) * (size_t)S, hipMemcpyHostToDevice));
            cfg.step = t;
            OK(fsdp_adam_shard(u, dS, dg, dm, dv, &cfg, dpb, NULL));
            orc_adamw(S, wantS, hg, hm, hv, cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay,
                      t, hpb);
        }
        HIP(hipDeviceSynchronize());
        HIP(hipMemcpy(got, dS, sizeof(float) * (size_t)S, hipMemcpyDeviceToHost));
        same(got, wantS, sizeof(float) * (size_t)S, "adamw param");
        HIP(hipMemcpy(got, dm, sizeof(float) * (size_t)S, hipMemcpyDeviceToHost));
        same(got, hm, sizeof(float) * (size_t)S, "adamw exp_avg");
        HIP(hipMemcpy(got, dv, sizeof(float) * (size_t)S, hipMemcpyDeviceToHost));
        same(got, hv, sizeof(float) * (size_t)S, "adamw exp_avg_sq");
        HIP(hipMemcpy(gpb, dpb, sizeof(uint16_t) * (size_t)S, hipMemcpyDeviceToHost));
        same(gpb, hpb, sizeof(uint16_t) * (size_t)S, "adamw bf16 copy");
        free(hg); free(hm); free(hv); free(got); free(hpb); free(gpb);
        HIP(hipFree(dg)); HIP(hipFree(dm)); HIP(hipFree(dv)); HIP(hipFree(dpb));
    }
    /* reductions: 5 ranks over the unit's shard (tile path, true division), and 32 ranks over
     * 12,288 whole 512-output tiles plus 7 (the many-rank sweep, reciprocal pre-divide) */
    reduce_case(NR, S, 3.0f, 2.5f);
    reduce_case(32, (int64_t)12288 * 512 + 7, 4.0f, 8.0f);

    for (i = 0; i < P; ++i) {
        free(hp[i]); free(hout[i]); free(want16[i]);
        HIP(hipFree(dp[i])); HIP(hipFree(dout[i]));
    }
    free(wantL); free(gotL); free(wantS);
    HIP(hipFree(dL)); HIP(hipFree(dS));
    OK(fsdp_unit_destroy(u));
    if (failures) {
        fprintf(stderr, "%d mismatch(es)\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
