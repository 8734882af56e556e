/* The C ABI used from C: include/fsdp_flatten.h compiled as C99 (-pedantic) and the library
 * linked by a C program.  Host-side calls only (no GPU needed): the unit plan's sizes for
 * units whose sizes the layout definitions fix by hand, and error statuses of calls that
 * fail validation before any HIP call.  Prints "ok" and exits 0 when every check holds. */
#include "fsdp_flatten.h"

#include <stdint.h>
#include <stdio.h>
#include <string.h>

static int failures = 0;

#define CHECK(cond)                                                     \
    do {                                                                \
        if (!(cond)) {                                                  \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__,      \
                    __LINE__, #cond);                                   \
            ++failures;                                                 \
        }                                                               \
    } while (0)

static fsdp_unit_sizes info(const fsdp_unit* u, int32_t k) {
    fsdp_unit_sizes s;
    memset(&s, 0, sizeof s);
    CHECK(fsdp_unit_info(u, k, &s) == FSDP_OK);
    return s;
}

int main(void) {
    CHECK(fsdp_abi_version() == FSDP_ABI_VERSION);
    CHECK(strcmp(fsdp_status_string(FSDP_E_ALIGN), "FSDP_E_ALIGN") == 0);
    CHECK(strcmp(fsdp_status_string(99), "FSDP_E_UNKNOWN") == 0);

    /* Linear(4 -> 3) over 16 ranks: T = 12 + 3 = 15, S = ceil(15/16) = 1, L = 16, one pad
     * element on rank 15; the bias starts at flat offset 12. */
    {
        const int32_t ndims[2] = {2, 1};
        const int64_t dims[3] = {3, 4, 3};
        fsdp_unit* u = NULL;
        int64_t off = -1, pitch = -1;
        fsdp_unit_sizes s;
        CHECK(fsdp_unit_create(FSDP_FLAT, 2, ndims, dims, 16, &u) == FSDP_OK && u != NULL);
        s = info(u, FSDP_ALL_RANKS);
        CHECK(s.layout == FSDP_FLAT && s.n_params == 2 && s.N == 16);
        CHECK(s.T == 15 && s.S == 1 && s.L == 16 && s.pad == 1 && s.bytes_per_rank == 16);
        CHECK(info(u, 14).valid == 1 && info(u, 15).valid == 0);
        CHECK(fsdp_unit_param_offset(u, 1, &off) == FSDP_OK && off == 12);
        CHECK(fsdp_unit_param_offset(u, 2, &off) == FSDP_E_RANGE);
        CHECK(fsdp_unit_recv_pitch(u, &pitch) == FSDP_OK && pitch == 64);
        /* validation failures: no HIP call is made */
        CHECK(fsdp_flatten_shard(u, NULL, 16, NULL, NULL) == FSDP_E_RANGE);
        CHECK(fsdp_grad_reduce_shard(u, NULL, 0.0f, 1.0f, NULL, NULL) == FSDP_E_RANGE);
        CHECK(strlen(fsdp_last_error()) > 0);
        {
            fsdp_adamw_cfg cfg = {1e-3, 0.9, 0.999, 1e-8, 0.01, 0};
            CHECK(fsdp_adam_shard(u, NULL, NULL, NULL, NULL, &cfg, NULL, NULL) == FSDP_E_RANGE);
            cfg.step = 1;
            cfg.beta1 = 1.0;
            CHECK(fsdp_adam_shard(u, NULL, NULL, NULL, NULL, &cfg, NULL, NULL) == FSDP_E_RANGE);
        }
        {
            fsdp_reduce_opts o;
            int64_t n = -1;
            memset(&o, 0, sizeof o);
            o.pre_divide = 1.0f;
            o.post_divide = 1.0f;
            o.group = 3; /* 3 does not divide 16 */
            CHECK(fsdp_grad_reduce_shard_ex(u, NULL, &o, NULL, NULL) == FSDP_E_RANGE);
            CHECK(fsdp_grad_reduce_workspace(u, &o, &n) == FSDP_E_RANGE);
            o.group = 4;
            o.accumulate = 1;
            CHECK(fsdp_grad_reduce_workspace(u, &o, &n) == FSDP_OK && n == 0);
            o.kernel = 3; /* not an fsdp_reduce_kernel */
            CHECK(fsdp_grad_reduce_shard_ex(u, NULL, &o, NULL, NULL) == FSDP_E_RANGE);
        }
        CHECK(fsdp_unit_destroy(u) == FSDP_OK);
    }

    /* 512 ranks (one launch holds 128): a [512, 3] parameter, S = 3.  The workspace holds
     * the sums carried between launches in slots of S rounded up to 64 floats: one when the
     * output keeps its old value (accumulate) or a group spans launches, two for both. */
    {
        const int32_t ndims[1] = {2};
        const int64_t dims[2] = {512, 3};
        fsdp_unit* u = NULL;
        fsdp_reduce_opts o;
        int64_t n = -1;
        uint16_t* fake_contribs[512];
        float* fake_out = (float*)(uintptr_t)0x100000;
        int r;
        memset(&o, 0, sizeof o);
        o.pre_divide = 16.0f;
        o.post_divide = 32.0f;
        CHECK(fsdp_unit_create(FSDP_FLAT, 1, ndims, dims, 512, &u) == FSDP_OK);
        CHECK(info(u, FSDP_ALL_RANKS).S == 3);
        CHECK(fsdp_grad_reduce_workspace(u, &o, &n) == FSDP_OK && n == 0);
        o.accumulate = 1;
        CHECK(fsdp_grad_reduce_workspace(u, &o, &n) == FSDP_OK && n == 64);
        o.group = 8;
        CHECK(fsdp_grad_reduce_workspace(u, &o, &n) == FSDP_OK && n == 64);
        o.group = 256;
        CHECK(fsdp_grad_reduce_workspace(u, &o, &n) == FSDP_OK && n == 128);
        o.accumulate = 0;
        CHECK(fsdp_grad_reduce_workspace(u, &o, &n) == FSDP_OK && n == 64);
        o.group = 8;
        CHECK(fsdp_grad_reduce_workspace(u, &o, &n) == FSDP_OK && n == 0);
        /* workspace errors are found before any HIP call (the pointers are never used) */
        for (r = 0; r < 512; ++r) fake_contribs[r] = (uint16_t*)(uintptr_t)(0x200000 + 64 * r);
        o.group = 256;
        CHECK(fsdp_grad_reduce_shard_ex(u, (const uint16_t* const*)fake_contribs, &o, fake_out,
                                        NULL) == FSDP_E_ARG);
        o.workspace = (float*)(uintptr_t)0x300008;
        o.workspace_len = 64;
        CHECK(fsdp_grad_reduce_shard_ex(u, (const uint16_t* const*)fake_contribs, &o, fake_out,
                                        NULL) == FSDP_E_ALIGN);
        o.workspace = (float*)(uintptr_t)0x300000;
        o.workspace_len = 63;
        CHECK(fsdp_grad_reduce_shard_ex(u, (const uint16_t* const*)fake_contribs, &o, fake_out,
                                        NULL) == FSDP_E_RANGE);
        CHECK(fsdp_unit_destroy(u) == FSDP_OK);
    }

    /* FSDP2 rows: a [5, 3] parameter over 4 ranks is chunked into 2, 2, 1, 0 rows of 3,
     * every rank's segment padded to 2 rows: P_r = 6, L = 24; and a 0-d parameter is one
     * row of one element (rank 0 holds it). */
    {
        const int32_t ndims[1] = {2};
        const int64_t dims[2] = {5, 3};
        fsdp_unit* u = NULL;
        fsdp_unit_sizes s;
        CHECK(fsdp_unit_create(FSDP_ROWS, 1, ndims, dims, 4, &u) == FSDP_OK);
        s = info(u, FSDP_ALL_RANKS);
        CHECK(s.T == 15 && s.S == 6 && s.L == 24 && s.pad == 9);
        CHECK(info(u, 0).valid == 6 && info(u, 1).valid == 6 && info(u, 2).valid == 3 &&
              info(u, 3).valid == 0);
        CHECK(fsdp_unit_destroy(u) == FSDP_OK);
    }
    {
        const int32_t ndims[2] = {0, 2};
        const int64_t dims[2] = {4, 2};
        fsdp_unit* u = NULL;
        int64_t off = -1;
        CHECK(fsdp_unit_create(FSDP_ROWS, 2, ndims, dims, 2, &u) == FSDP_OK);
        CHECK(info(u, FSDP_ALL_RANKS).S == 1 + 2 * 2);
        CHECK(info(u, 0).valid == 5 && info(u, 1).valid == 4);
        CHECK(fsdp_unit_param_offset(u, 1, &off) == FSDP_OK && off == 1);
        CHECK(fsdp_unit_destroy(u) == FSDP_OK);
    }

    /* creation errors */
    {
        const int32_t ndims[1] = {2};
        const int64_t dims[2] = {3, 4};
        const int64_t huge[2] = {(int64_t)1 << 62, 4};
        const int64_t neg[2] = {3, -1};
        fsdp_unit* u = NULL;
        CHECK(fsdp_unit_create(FSDP_FLAT, 1, ndims, dims, 0, &u) == FSDP_E_RANGE && u == NULL);
        CHECK(fsdp_unit_create(3, 1, ndims, dims, 2, &u) == FSDP_E_RANGE);
        CHECK(fsdp_unit_create(FSDP_FLAT, 1, ndims, dims, 2, NULL) == FSDP_E_ARG);
        CHECK(fsdp_unit_create(FSDP_FLAT, 1, ndims, neg, 2, &u) == FSDP_E_RANGE);
        CHECK(fsdp_unit_create(FSDP_FLAT, 1, ndims, huge, 2, &u) == FSDP_E_OVERFLOW);
        CHECK(fsdp_unit_create(FSDP_FLAT, 1, NULL, dims, 2, &u) == FSDP_E_ARG);
        CHECK(strlen(fsdp_last_error()) > 0);
        CHECK(fsdp_unit_destroy(NULL) == FSDP_OK);
    }

    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
