/*
 * oracle.c -- plain fp64 CPU oracle for the inverse-RoPE + VHA postmix path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header or table with the HIP library.
 *
 * Sources (cited by page title and part of the page):
 *   [P1772] PaddleFleet PR #1772, "Fuse HCA inverse RoPE into the VHA postmix,
 *           and the sparse-attention KV index remap": PR body, item 1
 *           ("fuse_inv_rope_into_vha_postmix"); the follow-up commit that
 *           changed the backward route; the Chinese description, part 一;
 *           and, for the KV index remap at the end of this file, PR body
 *           item 2 ("sparse_attn_global_kv_idx_remap_fusion") and part 二.
 *
 * What the pages fix:
 *   - The HCA layer applies an inverse RoPE to the attention output O and
 *     feeds the full-width result to the ungrouped VHA postmix, an [nh,nh]
 *     GEMM that contracts the head axis ([P1772] body item 1).
 *   - RoPE touches only the trailing qk_pos_emb_head_dim (= pe) channels of
 *     each head; the leading nope channels pass through ([P1772] body item 1).
 *   - The postmix is matmul(M, X): row index of M = output head
 *     ([P1772] description 一, split-N property).
 *   - dM[h,h'] = sum over tokens t and channels c of dOut[t,h,c]*O_roped[t,h',c]
 *     ([P1772] description 一).
 *   - The backward of the unfused path is the RoPE backward applied to the
 *     GEMM's input gradient ([P1772] follow-up commit: rope_full_out_of_place
 *     plus matmul_grad).
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   R1 pairing: rotate-half, channel nope+i pairs with nope+pe/2+i.
 *   R2 frequencies: inv_freq[i] = theta^(-2i/pe), exponent over pe.
 *   R3 angle: phi = positions[s]*inv_freq[i], evaluated in fp64.
 *   R4 "inverse" RoPE = rotation by -phi (the transpose of RoPE's rotation).
 *   R5 positions are given per token row.
 *
 * Everything is evaluated in fp64 with plain loops, in the order the
 * definition states: first the rotated operand, then the head contraction.
 * Inputs may be fp64 or raw bf16 bit patterns (decoded exactly to fp64).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ------------------------------------------------------------------ */
/* input decoding                                                      */
/* ------------------------------------------------------------------ */

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
static double bf16_bits_to_double(uint16_t b)
{
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Load n consecutive elements starting at element offset `off` of a tensor
 * that is either fp64 (is_bf16 == 0) or bf16 bits (is_bf16 == 1). */
static void load_elems(const void *base, int is_bf16, int64_t off, int64_t n,
                       double *dst)
{
    if (is_bf16) {
        const uint16_t *p = (const uint16_t *)base + off;
        for (int64_t i = 0; i < n; ++i) dst[i] = bf16_bits_to_double(p[i]);
    } else {
        const double *p = (const double *)base + off;
        for (int64_t i = 0; i < n; ++i) dst[i] = p[i];
    }
}

/* ------------------------------------------------------------------ */
/* RoPE angles (R2, R3)                                                */
/* ------------------------------------------------------------------ */

/* cos/sin of phi[i] = position * theta^(-2i/pe), i < pe/2, in fp64. */
static void angles_for_position(double theta, int32_t pe, int32_t position,
                                double *cs, double *sn)
{
    int32_t h2 = pe / 2;
    for (int32_t i = 0; i < h2; ++i) {
        double inv_freq = pow(theta, -2.0 * (double)i / (double)pe);
        double phi = (double)position * inv_freq;
        cs[i] = cos(phi);
        sn[i] = sin(phi);
    }
}

void oracle_rope_angles(double theta, int32_t pe, const int32_t *positions,
                        int64_t sq, double *cos_out, double *sin_out)
{
    int32_t h2 = pe / 2;
    for (int64_t s = 0; s < sq; ++s)
        angles_for_position(theta, pe, positions[s], cos_out + s * h2,
                            sin_out + s * h2);
}

/* ------------------------------------------------------------------ */
/* rotations on one head row of d = nope + pe channels (R1, R4)        */
/* ------------------------------------------------------------------ */

/* direction = -1: inverse RoPE (rotate each pair by -phi);
 * direction = +1: RoPE (rotate by +phi).
 * Pair i is (x[nope+i], x[nope+h2+i]), read as the complex number
 * x[nope+i] + j*x[nope+h2+i] multiplied by exp(direction*j*phi). */
static void rotate_head(const double *x, double *y, int32_t nope, int32_t pe,
                        const double *cs, const double *sn, int direction)
{
    int32_t h2 = pe / 2;
    for (int32_t c = 0; c < nope; ++c) y[c] = x[c];
    for (int32_t i = 0; i < h2; ++i) {
        double a = x[nope + i];
        double b = x[nope + h2 + i];
        double s = (double)direction * sn[i];
        y[nope + i] = a * cs[i] - b * s;
        y[nope + h2 + i] = b * cs[i] + a * s;
    }
}

/* ------------------------------------------------------------------ */
/* a tiny parallel-for over token rows                                 */
/* ------------------------------------------------------------------ */

typedef void (*range_fn)(void *ctx, int64_t lo, int64_t hi, int tid);

typedef struct {
    range_fn fn;
    void *ctx;
    int64_t lo, hi;
    int tid;
} range_task;

static void *range_thread(void *arg)
{
    range_task *t = (range_task *)arg;
    t->fn(t->ctx, t->lo, t->hi, t->tid);
    return NULL;
}

int32_t oracle_default_threads(void)
{
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n < 1 ? 1 : (int32_t)n;
}

/* Split [0, n) into nthreads contiguous chunks; chunk t goes to thread t. */
static int parallel_rows(int32_t nthreads, int64_t n, range_fn fn, void *ctx)
{
    if (nthreads < 1) nthreads = 1;
    if (n < nthreads) nthreads = n > 0 ? (int32_t)n : 1;
    if (nthreads == 1) {
        fn(ctx, 0, n, 0);
        return 0;
    }
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * nthreads);
    range_task *tasks = (range_task *)malloc(sizeof(range_task) * nthreads);
    if (!th || !tasks) {
        free(th);
        free(tasks);
        return -1;
    }
    for (int32_t t = 0; t < nthreads; ++t) {
        tasks[t].fn = fn;
        tasks[t].ctx = ctx;
        tasks[t].lo = n * t / nthreads;
        tasks[t].hi = n * (t + 1) / nthreads;
        tasks[t].tid = t;
        pthread_create(&th[t], NULL, range_thread, &tasks[t]);
    }
    for (int32_t t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
    free(th);
    free(tasks);
    return 0;
}

/* ------------------------------------------------------------------ */
/* shared problem description                                          */
/* ------------------------------------------------------------------ */

typedef struct {
    const void *x;   /* [sq, nh, d]: O (forward, dW) or dY (dx)        */
    int x_bf16;
    const void *y;   /* second [sq, nh, d] operand (dW: O), else NULL   */
    int y_bf16;
    const void *w;   /* [nh, nh], row index = output head               */
    int w_bf16;
    const int32_t *positions;
    double theta;
    int64_t sq;
    int32_t nh, nope, pe;
    double *out;     /* fwd/dx: [sq, nh, d]; dW: [nthreads, nh, nh]      */
    int abs_terms;   /* dW only: sum |dY * X| instead of dY * X          */
} problem;

static int shape_ok(int64_t sq, int32_t nh, int32_t nope, int32_t pe)
{
    return sq >= 0 && nh >= 1 && nope >= 0 && pe >= 0 && (pe % 2) == 0 &&
           (nope + pe) > 0;
}

/* ------------------------------------------------------------------ */
/* forward: Y[s,g,:] = sum_h W[g,h] * inv_rope(O)[s,h,:]                */
/* ------------------------------------------------------------------ */

static void fwd_rows(void *vctx, int64_t lo, int64_t hi, int tid)
{
    (void)tid;
    problem *p = (problem *)vctx;
    int32_t nh = p->nh, d = p->nope + p->pe, h2 = p->pe / 2;
    double *w = (double *)malloc(sizeof(double) * nh * nh);
    double *o = (double *)malloc(sizeof(double) * nh * d);
    double *x = (double *)malloc(sizeof(double) * nh * d);
    double *cs = (double *)malloc(sizeof(double) * (h2 + 1));
    double *sn = (double *)malloc(sizeof(double) * (h2 + 1));
    load_elems(p->w, p->w_bf16, 0, (int64_t)nh * nh, w);
    for (int64_t s = lo; s < hi; ++s) {
        angles_for_position(p->theta, p->pe, p->positions[s], cs, sn);
        load_elems(p->x, p->x_bf16, s * nh * d, (int64_t)nh * d, o);
        /* 1. materialise the inverse-rotated operand X = inv_rope(O) */
        for (int32_t h = 0; h < nh; ++h)
            rotate_head(o + h * d, x + h * d, p->nope, p->pe, cs, sn, -1);
        /* 2. head mix */
        double *y = p->out + s * nh * d;
        for (int32_t g = 0; g < nh; ++g)
            for (int32_t c = 0; c < d; ++c) {
                double acc = 0.0;
                for (int32_t h = 0; h < nh; ++h) acc += w[g * nh + h] * x[h * d + c];
                y[g * d + c] = acc;
            }
    }
    free(w); free(o); free(x); free(cs); free(sn);
}

static int run_fwd(problem *p, int32_t nthreads)
{
    if (!shape_ok(p->sq, p->nh, p->nope, p->pe)) return -2;
    return parallel_rows(nthreads, p->sq, fwd_rows, p);
}

int oracle_fwd_bf16(const uint16_t *O, const uint16_t *W,
                    const int32_t *positions, double theta, int64_t sq,
                    int32_t nh, int32_t nope, int32_t pe, double *Y,
                    int32_t nthreads)
{
    problem p = {O, 1, NULL, 0, W, 1, positions, theta, sq, nh, nope, pe, Y, 0};
    return run_fwd(&p, nthreads);
}

int oracle_fwd_f64(const double *O, const double *W, const int32_t *positions,
                   double theta, int64_t sq, int32_t nh, int32_t nope,
                   int32_t pe, double *Y, int32_t nthreads)
{
    problem p = {O, 0, NULL, 0, W, 0, positions, theta, sq, nh, nope, pe, Y, 0};
    return run_fwd(&p, nthreads);
}

/* ------------------------------------------------------------------ */
/* backward, input gradient:                                           */
/*   dX[s,h,:] = sum_g W[g,h] * dY[s,g,:]   (GEMM input gradient)      */
/*   dO[s,h,:] = rope(dX[s,h,:])             (RoPE backward = adjoint   */
/*                                            of the inverse rotation)  */
/* ------------------------------------------------------------------ */

static void dx_rows(void *vctx, int64_t lo, int64_t hi, int tid)
{
    (void)tid;
    problem *p = (problem *)vctx;
    int32_t nh = p->nh, d = p->nope + p->pe, h2 = p->pe / 2;
    double *w = (double *)malloc(sizeof(double) * nh * nh);
    double *dy = (double *)malloc(sizeof(double) * nh * d);
    double *dx = (double *)malloc(sizeof(double) * nh * d);
    double *cs = (double *)malloc(sizeof(double) * (h2 + 1));
    double *sn = (double *)malloc(sizeof(double) * (h2 + 1));
    load_elems(p->w, p->w_bf16, 0, (int64_t)nh * nh, w);
    for (int64_t s = lo; s < hi; ++s) {
        angles_for_position(p->theta, p->pe, p->positions[s], cs, sn);
        load_elems(p->x, p->x_bf16, s * nh * d, (int64_t)nh * d, dy);
        /* 1. gradient of the head mix with respect to its input */
        for (int32_t h = 0; h < nh; ++h)
            for (int32_t c = 0; c < d; ++c) {
                double acc = 0.0;
                for (int32_t g = 0; g < nh; ++g) acc += w[g * nh + h] * dy[g * d + c];
                dx[h * d + c] = acc;
            }
        /* 2. backward of the inverse rotation: rotate by +phi */
        double *out = p->out + s * nh * d;
        for (int32_t h = 0; h < nh; ++h)
            rotate_head(dx + h * d, out + h * d, p->nope, p->pe, cs, sn, +1);
    }
    free(w); free(dy); free(dx); free(cs); free(sn);
}

static int run_dx(problem *p, int32_t nthreads)
{
    if (!shape_ok(p->sq, p->nh, p->nope, p->pe)) return -2;
    return parallel_rows(nthreads, p->sq, dx_rows, p);
}

int oracle_bwd_dx_bf16(const uint16_t *dY, const uint16_t *W,
                       const int32_t *positions, double theta, int64_t sq,
                       int32_t nh, int32_t nope, int32_t pe, double *dO,
                       int32_t nthreads)
{
    problem p = {dY, 1, NULL, 0, W, 1, positions, theta, sq, nh, nope, pe, dO, 0};
    return run_dx(&p, nthreads);
}

int oracle_bwd_dx_f64(const double *dY, const double *W,
                      const int32_t *positions, double theta, int64_t sq,
                      int32_t nh, int32_t nope, int32_t pe, double *dO,
                      int32_t nthreads)
{
    problem p = {dY, 0, NULL, 0, W, 0, positions, theta, sq, nh, nope, pe, dO, 0};
    return run_dx(&p, nthreads);
}

/* ------------------------------------------------------------------ */
/* backward, weight gradient:                                          */
/*   dW[g,h] = sum_s sum_c dY[s,g,c] * inv_rope(O)[s,h,c]               */
/* Each thread sums its contiguous token range into its own fp64 slab; */
/* the slabs are then added in thread order.                           */
/* ------------------------------------------------------------------ */

static void dw_rows(void *vctx, int64_t lo, int64_t hi, int tid)
{
    problem *p = (problem *)vctx;
    int32_t nh = p->nh, d = p->nope + p->pe, h2 = p->pe / 2;
    double *acc = p->out + (int64_t)tid * nh * nh;
    double *dy = (double *)malloc(sizeof(double) * nh * d);
    double *o = (double *)malloc(sizeof(double) * nh * d);
    double *x = (double *)malloc(sizeof(double) * nh * d);
    double *cs = (double *)malloc(sizeof(double) * (h2 + 1));
    double *sn = (double *)malloc(sizeof(double) * (h2 + 1));
    for (int64_t i = 0; i < (int64_t)nh * nh; ++i) acc[i] = 0.0;
    for (int64_t s = lo; s < hi; ++s) {
        angles_for_position(p->theta, p->pe, p->positions[s], cs, sn);
        load_elems(p->x, p->x_bf16, s * nh * d, (int64_t)nh * d, dy);
        load_elems(p->y, p->y_bf16, s * nh * d, (int64_t)nh * d, o);
        for (int32_t h = 0; h < nh; ++h)
            rotate_head(o + h * d, x + h * d, p->nope, p->pe, cs, sn, -1);
        for (int32_t g = 0; g < nh; ++g)
            for (int32_t h = 0; h < nh; ++h) {
                double t = 0.0;
                if (p->abs_terms)
                    for (int32_t c = 0; c < d; ++c) t += fabs(dy[g * d + c] * x[h * d + c]);
                else
                    for (int32_t c = 0; c < d; ++c) t += dy[g * d + c] * x[h * d + c];
                acc[g * nh + h] += t;
            }
    }
    free(dy); free(o); free(x); free(cs); free(sn);
}

static int run_dw(problem *p, double *dW, int32_t nthreads)
{
    if (!shape_ok(p->sq, p->nh, p->nope, p->pe)) return -2;
    int32_t nh = p->nh;
    if (nthreads < 1) nthreads = 1;
    if (p->sq < nthreads) nthreads = p->sq > 0 ? (int32_t)p->sq : 1;
    double *slabs = (double *)calloc((size_t)nthreads * nh * nh, sizeof(double));
    if (!slabs) return -1;
    p->out = slabs;
    int rc = parallel_rows(nthreads, p->sq, dw_rows, p);
    for (int64_t i = 0; i < (int64_t)nh * nh; ++i) {
        double t = 0.0;
        for (int32_t k = 0; k < nthreads; ++k) t += slabs[(int64_t)k * nh * nh + i];
        dW[i] = t;
    }
    free(slabs);
    return rc;
}

int oracle_bwd_dw_bf16(const uint16_t *dY, const uint16_t *O,
                       const int32_t *positions, double theta, int64_t sq,
                       int32_t nh, int32_t nope, int32_t pe, double *dW,
                       int32_t nthreads)
{
    problem p = {dY, 1, O, 1, NULL, 0, positions, theta, sq, nh, nope, pe, NULL, 0};
    return run_dw(&p, dW, nthreads);
}

int oracle_bwd_dw_f64(const double *dY, const double *O,
                      const int32_t *positions, double theta, int64_t sq,
                      int32_t nh, int32_t nope, int32_t pe, double *dW,
                      int32_t nthreads)
{
    problem p = {dY, 0, O, 0, NULL, 0, positions, theta, sq, nh, nope, pe, NULL, 0};
    return run_dw(&p, dW, nthreads);
}

/* The magnitude of the terms of each weight-gradient entry,
 *   A[g,h] = sum_s sum_c |dY[s,g,c] * inv_rope(O)[s,h,c]|,
 * the same loops with each product's absolute value.  A[g,h] / |dW[g,h]| is
 * the condition number of the sum: an entry that cancels to far below A[g,h]
 * cannot be computed in fp32 to a small relative error in any order, and
 * u * A[g,h] (u = 2^-24) is the size of one rounding at the largest magnitude
 * a partial sum of its terms can reach.  The parity tests use it to bound
 * such entries. */
int oracle_bwd_dw_abs_bf16(const uint16_t *dY, const uint16_t *O,
                           const int32_t *positions, double theta, int64_t sq,
                           int32_t nh, int32_t nope, int32_t pe, double *A,
                           int32_t nthreads)
{
    problem p = {dY, 1, O, 1, NULL, 0, positions, theta, sq, nh, nope, pe, NULL, 1};
    return run_dw(&p, A, nthreads);
}

/* ------------------------------------------------------------------ */
/* element-wise rotations on whole tensors (building blocks for pins)  */
/* ------------------------------------------------------------------ */

int oracle_rotate_f64(const double *X, double *out, const int32_t *positions,
                      double theta, int64_t sq, int32_t nh, int32_t nope,
                      int32_t pe, int32_t direction)
{
    if (!shape_ok(sq, nh, nope, pe) || (direction != 1 && direction != -1)) return -2;
    int32_t d = nope + pe, h2 = pe / 2;
    double *cs = (double *)malloc(sizeof(double) * (h2 + 1));
    double *sn = (double *)malloc(sizeof(double) * (h2 + 1));
    for (int64_t s = 0; s < sq; ++s) {
        angles_for_position(theta, pe, positions[s], cs, sn);
        for (int32_t h = 0; h < nh; ++h)
            rotate_head(X + (s * nh + h) * d, out + (s * nh + h) * d, nope, pe,
                        cs, sn, direction);
    }
    free(cs); free(sn);
    return 0;
}

/* ------------------------------------------------------------------ */
/* single outputs, computed one by one (checks at full size)           */
/* ------------------------------------------------------------------ */

/* inverse-rotated channel c of head h at token s, from bf16 O */
static double inv_rope_elem_bf16(const uint16_t *O, int64_t s, int32_t h,
                                 int32_t c, int32_t nh, int32_t nope,
                                 int32_t pe, const double *cs, const double *sn)
{
    int32_t d = nope + pe, h2 = pe / 2;
    const uint16_t *row = O + (s * nh + h) * d;
    if (c < nope) return bf16_bits_to_double(row[c]);
    int32_t i = (c - nope) % h2;
    double a = bf16_bits_to_double(row[nope + i]);
    double b = bf16_bits_to_double(row[nope + h2 + i]);
    if (c < nope + h2) return a * cs[i] + b * sn[i];
    return b * cs[i] - a * sn[i];
}

/* Y at flat indices idx[k] = (s*nh + g)*d + c */
int oracle_fwd_at_bf16(const uint16_t *O, const uint16_t *W,
                       const int32_t *positions, double theta, int64_t sq,
                       int32_t nh, int32_t nope, int32_t pe, const int64_t *idx,
                       int64_t n, double *out)
{
    if (!shape_ok(sq, nh, nope, pe)) return -2;
    int32_t d = nope + pe, h2 = pe / 2;
    double *cs = (double *)malloc(sizeof(double) * (h2 + 1));
    double *sn = (double *)malloc(sizeof(double) * (h2 + 1));
    for (int64_t k = 0; k < n; ++k) {
        int64_t s = idx[k] / ((int64_t)nh * d);
        int32_t g = (int32_t)((idx[k] / d) % nh);
        int32_t c = (int32_t)(idx[k] % d);
        angles_for_position(theta, pe, positions[s], cs, sn);
        double acc = 0.0;
        for (int32_t h = 0; h < nh; ++h)
            acc += bf16_bits_to_double(W[g * nh + h]) *
                   inv_rope_elem_bf16(O, s, h, c, nh, nope, pe, cs, sn);
        out[k] = acc;
    }
    free(cs); free(sn);
    return 0;
}

/* dO at flat indices idx[k] = (s*nh + h)*d + c */
int oracle_bwd_dx_at_bf16(const uint16_t *dY, const uint16_t *W,
                          const int32_t *positions, double theta, int64_t sq,
                          int32_t nh, int32_t nope, int32_t pe,
                          const int64_t *idx, int64_t n, double *out)
{
    if (!shape_ok(sq, nh, nope, pe)) return -2;
    int32_t d = nope + pe, h2 = pe / 2;
    double *cs = (double *)malloc(sizeof(double) * (h2 + 1));
    double *sn = (double *)malloc(sizeof(double) * (h2 + 1));
    for (int64_t k = 0; k < n; ++k) {
        int64_t s = idx[k] / ((int64_t)nh * d);
        int32_t h = (int32_t)((idx[k] / d) % nh);
        int32_t c = (int32_t)(idx[k] % d);
        angles_for_position(theta, pe, positions[s], cs, sn);
        /* the GEMM input gradient at channel c and, for pe channels, at the
         * partner channel; then the +phi rotation of that pair */
        int32_t ca = c, cb = c;
        if (c >= nope) {
            int32_t i = (c - nope) % h2;
            ca = nope + i;
            cb = nope + h2 + i;
        }
        double ga = 0.0, gb = 0.0;
        for (int32_t g = 0; g < nh; ++g) {
            double wg = bf16_bits_to_double(W[g * nh + h]);
            ga += wg * bf16_bits_to_double(dY[(s * nh + g) * d + ca]);
            gb += wg * bf16_bits_to_double(dY[(s * nh + g) * d + cb]);
        }
        if (c < nope) {
            out[k] = ga;
        } else {
            int32_t i = (c - nope) % h2;
            if (c < nope + h2) out[k] = ga * cs[i] - gb * sn[i];
            else out[k] = gb * cs[i] + ga * sn[i];
        }
    }
    free(cs); free(sn);
    return 0;
}

/* dW at flat indices idx[k] = g*nh + h, each a full sum over (s, c) */
typedef struct {
    const uint16_t *dY, *O;
    const int32_t *positions;
    double theta;
    int64_t sq;
    int32_t nh, nope, pe;
    const int64_t *idx;
    int64_t n;
    double *slabs; /* [nthreads, n] */
} dw_at_ctx;

static void dw_at_rows(void *vctx, int64_t lo, int64_t hi, int tid)
{
    dw_at_ctx *p = (dw_at_ctx *)vctx;
    int32_t nh = p->nh, d = p->nope + p->pe, h2 = p->pe / 2;
    double *cs = (double *)malloc(sizeof(double) * (h2 + 1));
    double *sn = (double *)malloc(sizeof(double) * (h2 + 1));
    double *acc = p->slabs + (int64_t)tid * p->n;
    for (int64_t k = 0; k < p->n; ++k) acc[k] = 0.0;
    for (int64_t s = lo; s < hi; ++s) {
        angles_for_position(p->theta, p->pe, p->positions[s], cs, sn);
        for (int64_t k = 0; k < p->n; ++k) {
            int32_t g = (int32_t)(p->idx[k] / nh), h = (int32_t)(p->idx[k] % nh);
            double t = 0.0;
            for (int32_t c = 0; c < d; ++c)
                t += bf16_bits_to_double(p->dY[(s * nh + g) * d + c]) *
                     inv_rope_elem_bf16(p->O, s, h, c, nh, p->nope, p->pe, cs, sn);
            acc[k] += t;
        }
    }
    free(cs); free(sn);
}

int oracle_bwd_dw_at_bf16(const uint16_t *dY, const uint16_t *O,
                          const int32_t *positions, double theta, int64_t sq,
                          int32_t nh, int32_t nope, int32_t pe,
                          const int64_t *idx, int64_t n, double *out,
                          int32_t nthreads)
{
    if (!shape_ok(sq, nh, nope, pe)) return -2;
    if (nthreads < 1) nthreads = 1;
    if (sq < nthreads) nthreads = sq > 0 ? (int32_t)sq : 1;
    double *slabs = (double *)calloc((size_t)nthreads * (n > 0 ? n : 1), sizeof(double));
    if (!slabs) return -1;
    dw_at_ctx ctx = {dY, O, positions, theta, sq, nh, nope, pe, idx, n, slabs};
    int rc = parallel_rows(nthreads, sq, dw_at_rows, &ctx);
    for (int64_t k = 0; k < n; ++k) {
        double t = 0.0;
        for (int32_t j = 0; j < nthreads; ++j) t += slabs[(int64_t)j * n + k];
        out[k] = t;
    }
    free(slabs);
    return rc;
}

/* ------------------------------------------------------------------ */
/* KV column index remap ([P1772] PR body item 2 and description part */
/* 二): a per-batch-local index table [b*sq, topk] becomes flat-global */
/* by adding b * seqlen_kv to every valid (non-negative) entry of the  */
/* rows of batch b.  Reading: negative entries are padding and become  */
/* pad_value.  Plain per-element definition.                           */
/* ------------------------------------------------------------------ */

int oracle_kv_remap(const int32_t *idx, int64_t rows, int64_t sq, int64_t topk,
                    int64_t seqlen_kv, int32_t pad_value, int32_t *out)
{
    if (rows < 0 || sq < 1 || topk < 0 || seqlen_kv < 0 || rows % sq != 0) return -2;
    for (int64_t r = 0; r < rows; ++r) {
        int64_t b = r / sq;
        for (int64_t k = 0; k < topk; ++k) {
            int32_t v = idx[r * topk + k];
            out[r * topk + k] = v >= 0 ? (int32_t)(v + b * seqlen_kv) : pad_value;
        }
    }
    return 0;
}
