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

/*
 * Backward of the recurrence above (gradients of a scalar loss
 *   l = sum_i dout_i . o_i + <ds, S_L>
 * with respect to q, k, v and S_0). The pages give no backward; this is the
 * plain reverse-mode derivative of the per-token recurrence:
 *   dq_t = dout_t S_t^T                 (S_t: state after token t)
 *   G_t  = q_t^T dout_t + e^{-s} G_{t+1},  G_L = q_L^T dout_L + ds
 *   dk_t = G_t v_t,  dv_t = G_t^T k_t,  dS_0 = e^{-s} G_1
 * dout rows follow the q/k/v layout; dq/dk/dv rows the o layout of
 * lto_unit; ds and ds0 are d*d (NULL = zero / not written).
 */
typedef struct {
    const float *q, *k, *v, *dout;
    long long in_stride;
    long long len;
    double slope;
    const double *s0;
    const double *ds;
    double *dq, *dk, *dv;
    long long o_stride;
    double *ds0;
} lto_bwd_unit;

static void run_bwd_unit(const lto_bwd_unit *u, int d, double *S)
{
    const double lam = exp(-u->slope);
    const size_t dd = (size_t)d * (size_t)d;
    /* forward sweep: S_t and dq_t */
    if (u->s0)
        memcpy(S, u->s0, sizeof(double) * dd);
    else
        memset(S, 0, sizeof(double) * dd);
    for (long long i = 0; i < u->len; ++i) {
        const float *ki = u->k + i * u->in_stride;
        const float *vi = u->v + i * u->in_stride;
        const float *gi = u->dout + i * u->in_stride;
        for (int r = 0; r < d; ++r)
            for (int c = 0; c < d; ++c)
                S[(size_t)r * d + c] = lam * S[(size_t)r * d + c] + (double)ki[r] * (double)vi[c];
        double *dqi = u->dq + i * u->o_stride;
        for (int r = 0; r < d; ++r) {
            double acc = 0.0;
            for (int c = 0; c < d; ++c)
                acc += S[(size_t)r * d + c] * (double)gi[c];
            dqi[r] = acc;
        }
    }
    /* reverse sweep: S now holds R = e^{-s} G_{t+1} (ds for the last token) */
    if (u->ds)
        memcpy(S, u->ds, sizeof(double) * dd);
    else
        memset(S, 0, sizeof(double) * dd);
    for (long long i = u->len - 1; i >= 0; --i) {
        const float *qi = u->q + i * u->in_stride;
        const float *ki = u->k + i * u->in_stride;
        const float *vi = u->v + i * u->in_stride;
        const float *gi = u->dout + i * u->in_stride;
        /* G_t = q_t^T dout_t + R */
        for (int r = 0; r < d; ++r)
            for (int c = 0; c < d; ++c)
                S[(size_t)r * d + c] += (double)qi[r] * (double)gi[c];
        double *dki = u->dk + i * u->o_stride;
        double *dvi = u->dv + i * u->o_stride;
        for (int c = 0; c < d; ++c)
            dvi[c] = 0.0;
        for (int r = 0; r < d; ++r) {
            double acc = 0.0;
            const double kr = (double)ki[r];
            for (int c = 0; c < d; ++c) {
                acc += S[(size_t)r * d + c] * (double)vi[c];
                dvi[c] += S[(size_t)r * d + c] * kr;
            }
            dki[r] = acc;
        }
        for (size_t e = 0; e < dd; ++e)
            S[e] *= lam;
    }
    if (u->ds0)
        memcpy(u->ds0, S, sizeof(double) * dd);
}

int lto_backward(const lto_bwd_unit *units, int n_units, int d, int n_threads)
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
                run_bwd_unit(&units[n], d, S);
        free(S);
    }
    return failed ? -1 : 0;
}
