/*
 * fsdp_oracle.c -- CPU oracle for the per-rank FSDP data path.
 *
 * TEST INFRASTRUCTURE ONLY.  This file states, as plainly as possible, what
 * each step of the path computes, so that the HIP library can be checked
 * against it element by element.  It is slow on purpose: it materialises whole
 * buffers the way the definitions describe them and walks them with plain
 * loops.  Only the test suite, the package smoke check and the CPU-baseline leg
 * of the benchmark load it; the library never does, and the two share no code,
 * headers or tables.
 *
 * Build: gcc -O2 -std=c99 -ffp-contract=off -fno-fast-math -fPIC -shared
 * (every float operation below is one IEEE-754 binary32 operation with
 * round-to-nearest-even; no fused multiply-add, no reassociation, no flushing
 * of subnormals).
 *
 * Sources (the pages this follows; sections named as they appear there):
 *   [P1] "PyTorch FSDP: Experiences on Scaling Fully Sharded Data Parallel"
 *        (paper summary, paper-graph-ui.vercel.app)
 *   [P2] "FSDP Under The Hood: ZeRO-3 The PyTorch Way" (dominator-index.github.io)
 *   [P3] "FSDP Architecture" (mbrenndoerfer.com, FSDP series)
 *   [P4] "FSDP (Fully Sharded Data Parallel)" (gunjandhanuka.github.io concept page)
 *
 * Pinned against what the pages and mathematics fix by tests/test_oracle_*.py.
 * Parity unpinned: the bit pattern of NaN results (only NaN-ness is fixed).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Small helpers                                                             */
/* ------------------------------------------------------------------------ */

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
static int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }

/* bf16 -> fp32 is exact: a bfloat16 is the upper half of a binary32. */
float orc_bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/*
 * fp32 -> bf16, round to nearest with ties to even.
 * The pages cast the full-precision parameter to low precision once per
 * FlatParameter ([P1] §3.4 "Native Mixed Precision and the Sharded Gradient
 * Scaler", parameter-level casting); they do not name a rounding mode.  The
 * reading taken is IEEE-754's default, round-to-nearest-even, applied to the
 * 16 bits that bfloat16 drops from a binary32:
 *   - keep the upper 16 bits;
 *   - if the dropped 16 bits are above half, or exactly half and the kept
 *     part is odd, add one to the kept part (a carry into the exponent is the
 *     correct rounding; it turns FLT_MAX into infinity);
 *   - subnormals are rounded like any other value (no flushing);
 *   - NaN stays NaN (sign kept, quiet bit set).
 */
uint16_t orc_bf16(float x) {
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    uint32_t kept = u >> 16;
    uint32_t dropped = u & 0xFFFFu;
    int is_nan = ((u & 0x7F800000u) == 0x7F800000u) && ((u & 0x007FFFFFu) != 0);
    if (is_nan) return (uint16_t)(kept | 0x0040u);
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;
    return (uint16_t)kept;
}

void orc_bf16_array(int64_t n, const float* x, uint16_t* y) {
    for (int64_t i = 0; i < n; ++i) y[i] = orc_bf16(x[i]);
}

/* ------------------------------------------------------------------------ */
/* FSDP1: the FlatParameter                                                  */
/* ------------------------------------------------------------------------ */

/*
 * Sizes of a FlatParameter over N ranks ([P1] §3.4 "FlatParameter:
 * Flattening, Concatenation, and Sharding"): the unit's parameters are
 * flattened and concatenated (T elements), padded on the right so that the
 * length is a multiple of N (pad <= N-1), and cut into N
 * equal chunks of S elements.
 * out[0]=T, out[1]=S, out[2]=L=N*S, out[3]=pad=L-T.
 */
void orc_flat_sizes(int32_t p, const int64_t* numel, int64_t N, int64_t* out) {
    int64_t T = 0;
    for (int32_t i = 0; i < p; ++i) T += numel[i];
    int64_t S = ceil_div(T, N);
    out[0] = T;
    out[1] = S;
    out[2] = N * S;
    out[3] = N * S - T;
}

/*
 * The padded flat buffer F itself: flatten each parameter (row-major), append
 * them in unit order, then append `pad` zeros ([P1] §3.4, FlatParameter,
 * Fig. 3).  The padding value is not given on the pages; +0.0f is taken.
 * Returns a malloc'd buffer of L floats (NULL on allocation failure or L==0).
 */
static float* build_flat(int32_t p, const int64_t* numel, const float* const* params,
                         int64_t N, int64_t* L_out) {
    int64_t sz[4];
    orc_flat_sizes(p, numel, N, sz);
    int64_t L = sz[2];
    *L_out = L;
    float* F = (float*)malloc((size_t)(L > 0 ? L : 1) * sizeof(float));
    if (!F) return NULL;
    int64_t w = 0;
    for (int32_t i = 0; i < p; ++i)
        for (int64_t j = 0; j < numel[i]; ++j) F[w++] = params[i][j];
    while (w < L) F[w++] = 0.0f;
    return F;
}

/*
 * Rank k's shard of the FlatParameter: the k-th of the N equal chunks
 * ([P1] §3.4 "Sharding Strategies": rank i owns the i-th chunk; Fig. 3).
 * k in [0,N) writes S floats.  k == -1 writes all of F (L floats), which is
 * also what an AllGather of the N shards in rank order produces ([P1] §3.4,
 * FlatParameter, "Communication layout").
 * Returns 0, or -1 if memory ran out.
 */
int orc_flat_shard(int32_t p, const int64_t* numel, const float* const* params, int64_t N,
                   int64_t k, float* out) {
    int64_t L;
    float* F = build_flat(p, numel, params, N, &L);
    if (!F) return -1;
    if (k < 0) {
        for (int64_t j = 0; j < L; ++j) out[j] = F[j];
    } else {
        int64_t S = L / N;
        for (int64_t j = 0; j < S; ++j) out[j] = F[k * S + j];
    }
    free(F);
    return 0;
}

/*
 * Copy-out: given the gathered (unsharded) FlatParameter, produce each original
 * parameter as a bf16 tensor.  Parameter i is the slice of F that starts at the
 * sum of the sizes before it, as torch.split with the parameters' sizes would
 * cut it ([P1] §3.4 "Autograd Integration"); each element is cast once to bf16
 * ([P1] §3.4 "Native Mixed Precision", parameter-level casting; bf16 compute
 * params of [P2] §4, MixedPrecisionPolicy).  Padding is never read.
 */
void orc_flat_copyout(int32_t p, const int64_t* numel, const float* gathered,
                      uint16_t* const* outs) {
    int64_t off = 0;
    for (int32_t i = 0; i < p; ++i) {
        for (int64_t j = 0; j < numel[i]; ++j) outs[i][j] = orc_bf16(gathered[off + j]);
        off += numel[i];
    }
}

/* ------------------------------------------------------------------------ */
/* FSDP2: per-parameter dim-0 sharding                                       */
/* ------------------------------------------------------------------------ */

/*
 * FSDP2 shards every parameter on its own along dim 0, with torch.chunk
 * ([P2] §2 "Sharding geometry"; [P4] "FSDP1 vs FSDP2").  A parameter is given
 * as m rows of r elements (r = product of the trailing dims; a 0-d parameter
 * is one row of one element).  torch.chunk(m, N) makes chunks of c = ceil(m/N)
 * rows; rank k's rows are [min(m, k*c), min(m, (k+1)*c)) -- ranks past the
 * last chunk hold no rows.
 *
 * The pages do not say how the per-rank shards sit in the AllGather buffer.
 * Reading taken (AllGather wants equal inputs, [P1] §3.4 FlatParameter,
 * Fig. 2a): every rank sends one segment of P_r = sum_i c_i*r_i elements, the
 * parameters in unit order, each padded with zero rows to c_i rows; the
 * gathered buffer holds the N segments in rank order.
 */
void orc_rows_sizes(int32_t p, const int64_t* m, const int64_t* r, int64_t N, int64_t* P_r) {
    int64_t s = 0;
    for (int32_t i = 0; i < p; ++i) s += ceil_div(m[i], N) * r[i];
    *P_r = s;
}

/* Rank k's segment (P_r floats); k == -1 writes all N segments (N*P_r floats). */
int orc_rows_shard(int32_t p, const int64_t* m, const int64_t* r, const float* const* params,
                   int64_t N, int64_t k, float* out) {
    int64_t P_r;
    orc_rows_sizes(p, m, r, N, &P_r);
    int64_t k_lo = k < 0 ? 0 : k, k_hi = k < 0 ? N : k + 1;
    int64_t w = 0;
    for (int64_t kk = k_lo; kk < k_hi; ++kk) {
        for (int32_t i = 0; i < p; ++i) {
            int64_t c = ceil_div(m[i], N);
            int64_t row_lo = min64(m[i], kk * c);
            int64_t row_hi = min64(m[i], (kk + 1) * c);
            for (int64_t e = row_lo * r[i]; e < row_hi * r[i]; ++e) out[w++] = params[i][e];
            for (int64_t e = (row_hi - row_lo) * r[i]; e < c * r[i]; ++e) out[w++] = 0.0f;
        }
    }
    (void)P_r;
    return 0;
}

/*
 * Copy-out of gathered FSDP2 shards: rebuild each parameter by concatenating,
 * in rank order, the valid rows each rank holds, and cast to bf16.
 */
void orc_rows_copyout(int32_t p, const int64_t* m, const int64_t* r, int64_t N,
                      const float* gathered, uint16_t* const* outs) {
    int64_t P_r;
    orc_rows_sizes(p, m, r, N, &P_r);
    for (int32_t i = 0; i < p; ++i) {
        /* where parameter i starts inside every rank's segment */
        int64_t q = 0;
        for (int32_t j = 0; j < i; ++j) q += ceil_div(m[j], N) * r[j];
        int64_t c = ceil_div(m[i], N);
        int64_t w = 0;
        for (int64_t kk = 0; kk < N; ++kk) {
            int64_t row_lo = min64(m[i], kk * c);
            int64_t row_hi = min64(m[i], (kk + 1) * c);
            const float* seg = gathered + kk * P_r + q;
            for (int64_t e = 0; e < (row_hi - row_lo) * r[i]; ++e) outs[i][w++] = orc_bf16(seg[e]);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Gradient reduction                                                        */
/* ------------------------------------------------------------------------ */

/*
 * ReduceScatter math for rank k: each of the N ranks contributes its gradient
 * slice for shard k; the slices are summed and rank k keeps the result
 * ([P1] §3.4 "Sharding Strategies" and "Communication layout"; [P3] backward
 * pass, step 3).  The contributions travel in bf16 ([P1] §3.4 "Native Mixed
 * Precision", low-precision collectives) and the reduction runs in fp32
 * ([P2] §3 "fp32 reduction"; [P2] §4 reduce_dtype=torch.float32).
 *
 * The pages define a plain sum and give no order.  Readings taken:
 *   - each term is divided by `pre` before it is added and the sum by `post`
 *     after (pre = post = 1 is the pages' plain sum);
 *   - the order is sequential over ranks r = 0..N-1 starting from term 0 (so
 *     that -0 contributions stay -0);
 *   - each step is one rounded binary32 operation; division is true division.
 */
void orc_grad_reduce(int64_t N, int64_t len, const uint16_t* const* contribs, float pre,
                     float post, float* out) {
    for (int64_t j = 0; j < len; ++j) {
        float acc = orc_bf16_to_f32(contribs[0][j]) / pre;
        for (int64_t r = 1; r < N; ++r) {
            float term = orc_bf16_to_f32(contribs[r][j]) / pre;
            acc = acc + term;
        }
        out[j] = acc / post;
    }
}

/* ------------------------------------------------------------------------ */
/* AdamW on the local shard                                                  */
/* ------------------------------------------------------------------------ */

/*
 * The optimizer step is local: rank k holds the parameter, gradient and both
 * Adam moments for the same positions and updates them with no communication
 * ([P3] "three-way alignment"; [P1] §3.2 information flow).  The optimizer is
 * Adam with its two states ([P1] §5 setup), AdamW in the page's training
 * script ([P2] appendix, torch.optim.AdamW).
 *
 * The pages give no formula.  Reading taken: Kingma & Ba (2015), Algorithm 1,
 * with bias correction, and the decoupled weight decay of Loshchilov & Hutter
 * (2019) applied first as p <- p*(1 - lr*wd):
 *   scalars (double, each rounded once to float):
 *     decay = 1 - lr*wd, b1 = beta1, omb1 = 1 - beta1, b2 = beta2,
 *     omb2 = 1 - beta2, step_size = lr / (1 - beta1^t),
 *     bc2s = sqrt(1 - beta2^t), epsf = eps
 *   per element, in this order (binary32):
 *     p = p*decay
 *     m = b1*m + omb1*g
 *     v = b2*v + omb2*(g*g)
 *     den = sqrt(v)/bc2s + epsf
 *     p = p - step_size*(m/den)
 *   optionally pb = bf16(p).
 * step t counts from 1; m and v start at zero.
 */
void orc_adamw(int64_t len, float* p, const float* g, float* m, float* v, double lr,
               double beta1, double beta2, double eps, double wd, int64_t step, uint16_t* pb) {
    float decay = (float)(1.0 - lr * wd);
    float b1 = (float)beta1;
    float omb1 = (float)(1.0 - beta1);
    float b2 = (float)beta2;
    float omb2 = (float)(1.0 - beta2);
    float step_size = (float)(lr / (1.0 - pow(beta1, (double)step)));
    float bc2s = (float)sqrt(1.0 - pow(beta2, (double)step));
    float epsf = (float)eps;
    for (int64_t j = 0; j < len; ++j) {
        float pj = p[j] * decay;
        float gj = g[j];
        float mj = b1 * m[j] + omb1 * gj;
        float gg = gj * gj;
        float vj = b2 * v[j] + omb2 * gg;
        float den = sqrtf(vj) / bc2s + epsf;
        float upd = mj / den;
        pj = pj - step_size * upd;
        p[j] = pj;
        m[j] = mj;
        v[j] = vj;
        if (pb) pb[j] = orc_bf16(pj);
    }
}

/* ------------------------------------------------------------------------ */
/* 16-bit layouts (bf16 parameters and gradients moved without arithmetic)  */
/* ------------------------------------------------------------------------ */

/*
 * The same FlatParameter and FSDP2 layouts as above, for 16-bit elements:
 * casting before the AllGather moves bf16 parameters ([P1] section 3.4,
 * "Native Mixed Precision": collectives in low precision; [P2] section 5:
 * the bf16 copy is what FSDP2 gathers), and the ReduceScatter input is the
 * unsharded bf16 gradient laid out like the FlatParameter ([P1] section 3.4,
 * "Communication layout").  Padding is the bit pattern 0x0000 (+0.0).
 */
int orc_flat_shard_u16(int32_t p, const int64_t* numel, const uint16_t* const* params, int64_t N,
                       int64_t k, uint16_t* out) {
    int64_t sz[4];
    orc_flat_sizes(p, numel, N, sz);
    int64_t L = sz[2], S = sz[1];
    uint16_t* F = (uint16_t*)malloc((size_t)(L > 0 ? L : 1) * sizeof(uint16_t));
    if (!F) return -1;
    int64_t w = 0;
    for (int32_t i = 0; i < p; ++i)
        for (int64_t j = 0; j < numel[i]; ++j) F[w++] = params[i][j];
    while (w < L) F[w++] = 0;
    if (k < 0) {
        for (int64_t j = 0; j < L; ++j) out[j] = F[j];
    } else {
        for (int64_t j = 0; j < S; ++j) out[j] = F[k * S + j];
    }
    free(F);
    return 0;
}

void orc_flat_copyout_u16(int32_t p, const int64_t* numel, const uint16_t* gathered,
                          uint16_t* const* outs) {
    int64_t off = 0;
    for (int32_t i = 0; i < p; ++i) {
        for (int64_t j = 0; j < numel[i]; ++j) outs[i][j] = gathered[off + j];
        off += numel[i];
    }
}

int orc_rows_shard_u16(int32_t p, const int64_t* m, const int64_t* r, const uint16_t* const* params,
                       int64_t N, int64_t k, uint16_t* out) {
    int64_t k_lo = k < 0 ? 0 : k, k_hi = k < 0 ? N : k + 1;
    int64_t w = 0;
    for (int64_t kk = k_lo; kk < k_hi; ++kk) {
        for (int32_t i = 0; i < p; ++i) {
            int64_t c = ceil_div(m[i], N);
            int64_t row_lo = min64(m[i], kk * c);
            int64_t row_hi = min64(m[i], (kk + 1) * c);
            for (int64_t e = row_lo * r[i]; e < row_hi * r[i]; ++e) out[w++] = params[i][e];
            for (int64_t e = (row_hi - row_lo) * r[i]; e < c * r[i]; ++e) out[w++] = 0;
        }
    }
    return 0;
}

void orc_rows_copyout_u16(int32_t p, const int64_t* m, const int64_t* r, int64_t N,
                          const uint16_t* gathered, uint16_t* const* outs) {
    int64_t P_r;
    orc_rows_sizes(p, m, r, N, &P_r);
    for (int32_t i = 0; i < p; ++i) {
        int64_t q = 0;
        for (int32_t j = 0; j < i; ++j) q += ceil_div(m[j], N) * r[j];
        int64_t c = ceil_div(m[i], N);
        int64_t w = 0;
        for (int64_t kk = 0; kk < N; ++kk) {
            int64_t row_lo = min64(m[i], kk * c);
            int64_t row_hi = min64(m[i], (kk + 1) * c);
            const uint16_t* seg = gathered + kk * P_r + q;
            for (int64_t e = 0; e < (row_hi - row_lo) * r[i]; ++e) outs[i][w++] = seg[e];
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Gradient reduction with hybrid groups and accumulation                   */
/* ------------------------------------------------------------------------ */

/*
 * Hybrid sharding ([P1] section 3.4, "Sharding Strategies": summing the W/F
 * sharding groups' in-group totals gives the total over every rank):
 * the N ranks form N/F groups of F consecutive ranks; each group's terms are
 * summed first (the ReduceScatter inside the sharding group), then the group
 * sums (the AllReduce across replicas).  Reading taken for the order: both
 * levels sequential, in rank and group order, each starting from its first
 * term.  group == N is the flat reduction; so is group == 1.
 *
 * Gradient accumulation with communication ([P1] section 3.4 "Communication
 * Optimizations: Overlapping, Prefetching, and Accumulation", "Gradient
 * Accumulation Variants": every micro-batch is still reduced, and each rank
 * accumulates its sharded gradient): when `accumulate` is non-zero the
 * existing shard value is kept and the fresh reduction (already divided by
 * post) is added to it, out = out + fresh.
 */
void orc_grad_reduce_ex(int64_t N, int64_t len, const uint16_t* const* contribs, float pre,
                        float post, int64_t group, int accumulate, float* out) {
    for (int64_t j = 0; j < len; ++j) {
        float total = 0.0f;
        for (int64_t g = 0; g < N / group; ++g) {
            float s = orc_bf16_to_f32(contribs[g * group][j]) / pre;
            for (int64_t r = g * group + 1; r < (g + 1) * group; ++r) {
                float term = orc_bf16_to_f32(contribs[r][j]) / pre;
                s = s + term;
            }
            total = (g == 0) ? s : total + s;
        }
        float fresh = total / post;
        out[j] = accumulate ? out[j] + fresh : fresh;
    }
}

/*
 * Gradient accumulation without communication ([P1] section 3.4,
 * "Gradient Accumulation Variants": each rank accumulates the unsharded
 * gradients locally and the reduction runs only on the last micro-batch): the
 * micro-batch's bf16 gradient is widened exactly and added to an fp32
 * accumulator; init != 0 starts the accumulator from this gradient.  The pages
 * do not give the accumulator's precision; fp32 (the reduction precision) is
 * taken.
 */
void orc_grad_accumulate(int64_t n, const uint16_t* grad, float* acc, int init) {
    for (int64_t j = 0; j < n; ++j) {
        float g = orc_bf16_to_f32(grad[j]);
        acc[j] = init ? g : acc[j] + g;
    }
}

/* ------------------------------------------------------------------------ */
/* Sharded optimizer statistics (per-rank halves)                            */
/* ------------------------------------------------------------------------ */

/*
 * Sharded gradient scaler, the per-rank half ([P1] section 3.4 "Native Mixed
 * Precision and the Sharded Gradient Scaler"): every rank unscales its own
 * gradient shard by the one global factor and records whether the shard holds
 * an overflow; the ranks then combine their flags (a max all-reduce) so that
 * all of them take or skip the step together.  Readings taken (the pages give
 * no implementation): the gradient is multiplied by inv_scale = 1/scale (one
 * rounded binary32 multiply per element); the check looks at the value before
 * it is multiplied; the flag is a float that is set to 1 when a non-finite
 * value is seen and is never cleared here (the caller clears it, so several
 * shards can share one flag).
 */
void orc_grad_unscale(int64_t n, float* g, float inv_scale, float* found_inf) {
    for (int64_t j = 0; j < n; ++j) {
        float x = g[j];
        if (!isfinite(x)) *found_inf = 1.0f;
        g[j] = x * inv_scale;
    }
}

/*
 * Per-parameter sums of squares of rank k's FLAT gradient shard.  The pages
 * warn that statistics of original parameters (norms for gradient clipping,
 * per-parameter optimizer statistics) are no longer correct when computed on
 * flat shards, because a shard ignores parameter boundaries ([P1] section 6
 * "Limitations", the mathematical-equivalence caveat).  The unit's layout
 * knows the boundaries: every shard element [kS, (k+1)S) of the flat buffer is
 * attributed to the parameter it came from (padding to none), and
 *   out[i] = sum of g_j^2 over the shard elements of parameter i,
 * with each square and each addition in binary64 (the square of a binary32 is
 * exact in binary64), in shard order.  Summed over the N ranks (an all-reduce
 * of p numbers) out[i] is parameter i's squared gradient norm; the sum over i
 * is the global one.
 */
void orc_flat_sqnorm(int32_t p, const int64_t* numel, int64_t N, int64_t k, const float* shard,
                     double* out) {
    int64_t T = 0;
    for (int32_t i = 0; i < p; ++i) T += numel[i];
    int64_t S = ceil_div(T, N);
    for (int32_t i = 0; i < p; ++i) out[i] = 0.0;
    int32_t i = 0;
    int64_t off = 0; /* start of parameter i in the flat buffer */
    for (int64_t j = 0; j < S; ++j) {
        int64_t g = k * S + j;
        if (g >= T) break; /* padding */
        while (g >= off + numel[i]) { off += numel[i]; ++i; }
        double x = (double)shard[j];
        out[i] = out[i] + x * x;
    }
}

/*
 * The same for rank k's FSDP2 segment: parameter i occupies, from offset q_i,
 * the rows of the rank's chunk followed by zero rows up to c_i; only the rows
 * the rank holds count.
 */
void orc_rows_sqnorm(int32_t p, const int64_t* m, const int64_t* r, int64_t N, int64_t k,
                     const float* seg, double* out) {
    int64_t q = 0;
    for (int32_t i = 0; i < p; ++i) {
        int64_t c = ceil_div(m[i], N);
        int64_t rows = min64(m[i], (k + 1) * c) - min64(m[i], k * c);
        out[i] = 0.0;
        for (int64_t e = 0; e < rows * r[i]; ++e) {
            double x = (double)seg[q + e];
            out[i] = out[i] + x * x;
        }
        q += c * r[i];
    }
}
