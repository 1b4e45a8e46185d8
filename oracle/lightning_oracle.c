/*
 * Lightning Attention oracle: plain fp64 CPU reference.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load this library. The GPU product path
 * never calls it, links it, or shares a line of code with it.
 *
 * What it computes: the per-token ("cumsum") recurrence that the block form of
 * Lightning Attention re-associates exactly.
 *   - MiniMax Signal Lab · M1 (ailearn.mscapital.top), §03 Lightning Attention:
 *     the block formulas (D_ij = e^{-s_h(i-j)}·[i>=j], O_intra, O_inter, and the
 *     state update S_t = e^{-s_h B} S_{t-1} + (K_t ⊙ d_k)^T V_t) applied with a
 *     block of a single token reduce to
 *         S <- e^{-s_h} S + k^T v            (state is d_key x d_value)
 *         o  = q S                           (q is a row vector; the token sees
 *                                             its own key, D_ii = 1)
 *   - fishai news commentary on M1: the block split exists to avoid this
 *     token-by-token cumulative sum, so the cumsum is the plain definition the
 *     block form must reproduce.
 * A decode step is one iteration of the same loop body.
 *
 * Precision: every value is read as float (bf16 and fp32 inputs are exactly
 * representable) and all arithmetic is fp64. The slope is the fp32 slope value
 * widened to fp64; the per-token decay is exp(-s) in fp64.
 *
 * Parity status: pinned (brute-force quadratic form, block-size invariance,
 * one-hot closed forms, special cases and invariants in the CPU test suite).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One independent (sequence, head) unit. Token i of the unit has its q, k and v
 * rows at q + i*in_stride, k + i*in_stride, v + i*in_stride (float elements).
 * s0: d*d initial state (row = key index, column = value index) or NULL (zero).
 * o:  output row i at o + i*o_stride, or NULL (state-only).
 * s_final: d*d final state, or NULL. s_final may equal s0. */
typedef struct {
    const float *q, *k, *v;
    long long in_stride;
    long long len;
    double slope;
    const double *s0;
    double *o;
    long long o_stride;
    double *s_final;
} lto_unit;

static void run_unit(const lto_unit *u, int d, double *S)
{
    const double lam = exp(-u->slope);
    if (u->s0)
        memcpy(S, u->s0, sizeof(double) * (size_t)d * (size_t)d);
    else
        memset(S, 0, sizeof(double) * (size_t)d * (size_t)d);

    for (long long i = 0; i < u->len; ++i) {
        const float *qi = u->q + i * u->in_stride;
        const float *ki = u->k + i * u->in_stride;
        const float *vi = u->v + i * u->in_stride;
        /* S <- lam*S + k_i^T v_i */
        for (int r = 0; r < d; ++r) {
            const double kr = (double)ki[r];
            double *Sr = S + (size_t)r * d;
            for (int c = 0; c < d; ++c)
                Sr[c] = lam * Sr[c] + kr * (double)vi[c];
        }
        /* o_i = q_i S (the state that already includes token i) */
        if (u->o) {
            double *oi = u->o + i * u->o_stride;
            for (int c = 0; c < d; ++c)
                oi[c] = 0.0;
            for (int r = 0; r < d; ++r) {
                const double qr = (double)qi[r];
                const double *Sr = S + (size_t)r * d;
                for (int c = 0; c < d; ++c)
                    oi[c] += qr * Sr[c];
            }
        }
    }
    if (u->s_final)
        memcpy(u->s_final, S, sizeof(double) * (size_t)d * (size_t)d);
}

/* Runs n_units independent units, OpenMP-parallel over units.
 * n_threads <= 0 uses the OpenMP default. Returns 0, or -1 on bad arguments or
 * allocation failure. */
int lto_recurrence(const lto_unit *units, int n_units, int d, int n_threads)
{
    if (!units || n_units < 0 || d <= 0)
        return -1;
    int failed = 0;
#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
#pragma omp parallel
    {
        double *S = (double *)malloc(sizeof(double) * (size_t)d * (size_t)d);
        if (!S) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int n = 0; n < n_units; ++n)
            if (S)
                run_unit(&units[n], d, S);
        free(S);
    }
    return failed ? -1 : 0;
}

/* Number of threads an OpenMP parallel region would use (for reporting). */
int lto_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
