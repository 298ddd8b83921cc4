/*
 * bdssm_oracle.c -- plain, slow, fp64 CPU oracle of the block-restricted
 * bidirectional selective scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load this library.  The GPU library
 * shares no code, header, table or helper with it, and neither calls the other.
 *
 * Pages cited (all describe arXiv 2607.02805, "Training Hybrid Block Diffusion
 * Language Models with Partial Bidirectionality"):
 *   [ABS]  the paper's abstract, as printed on the newx.sg page (section
 *          "Abstract") and on the gptget.net page (section "原文摘要").
 *   [SUM]  the newx.sg page, section "AI Summary".
 *   [DE-M] the gist.science German page, "Technische Zusammenfassung",
 *          subsection "Methodik" (the same text is in "Sintesi Tecnica /
 *          Metodologia" on the Italian page and "Resumo Técnico /
 *          Metodologia" on the Portuguese page).
 *   [DE-P] same page, subsection "Problemstellung".
 *
 * What is computed.  The pages name Mamba's linear-time selective state-space
 * mixer [ABS] but print no formula, no shapes and no precision.  The reading
 * taken here is the standard Mamba-1 selective scan with a diagonal real A:
 * for every (batch b, channel d) row and every state n,
 *     forward:  hf_t[n] = exp(dt_t * A[d,n]) * hf_{t-1}[n] + dt_t * B_t[n] * x_t
 * (zero-order hold for A, Euler step for B), starting from hf_{-1} = h0
 * (zero, a supplied initial state, or the prefix cache).
 * The reverse scan is confined to the active block [ABS], [SUM], [DE-M]: for
 * each block of L tokens aligned at multiples of L from token 0, a state that
 * starts at zero after the block's last token runs toward the block's first
 * token with the same per-token coefficients:
 *     reverse:  hr_t[n] = exp(dt_t * A[d,n]) * hr_{t+1}[n] + dt_t * B_t[n] * x_t
 * (so token t is counted in both directions).  The output is
 *     y_t = sum_n C_t[n] * (hf_t[n] + hr_t[n]) + Dskip[d] * x_t.
 * The cache is the forward state after the last committed token: it depends
 * on the clean prefix alone [DE-M]; the reverse state is never cached because
 * it depends on later tokens of the block [ABS], [DE-P].
 * Setting L = T reproduces the full-sequence reverse scan of the earlier
 * bidirectional hybrids the pages contrast with [ABS], [DE-P].
 * The two-stream all-block training form [DE-M] (prefix caches built by
 * scanning the clean prefix; downstream block losses train them) runs every
 * noisy L-block from the clean stream's forward state before that block:
 * oracle_train_blocks below.
 *
 * Everything is fp64; stream inputs (fp32, bf16 or fp64) are widened exactly
 * per element; A, Dskip and states are fp64 (fp32 values convert exactly).
 * Rows are independent, so an OpenMP loop over (b,d) is the only parallelism;
 * every row is a plain sequential loop over tokens with exp() from libm.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_F64 2

/* exact widening of one input element */
static double ld(const void *p, size_t i, int dtype)
{
    if (dtype == ORACLE_F64) return ((const double *)p)[i];
    if (dtype == ORACLE_BF16) {
        uint32_t bits = ((uint32_t)((const uint16_t *)p)[i]) << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return (double)((const float *)p)[i];
}

/*
 * Optional fusions of a Mamba-1 layer around the scan (the pages are silent on
 * them; they follow the Mamba-1 layer): the raw step size plus a per-channel
 * bias, passed through softplus, gives dt; the output is gated by silu(z).
 */
static double step_size(double raw, double bias, int softplus)
{
    const double v = raw + bias;
    if (!softplus) return v;
    /* softplus(v) = log(1 + e^v), written so that neither branch overflows */
    return v > 0.0 ? v + log1p(exp(-v)) : log1p(exp(v));
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/*
 * Optionally the reverse scan has operands of its own (a bidirectional Mamba
 * layer whose reverse direction has its own projections and A): step size
 * dt_r (with its own bias, same softplus setting), B_r, C_r and A_r.  The
 * forward scan, and so the cache, never sees them.  With dt_r == NULL the
 * reverse shares the forward's operands.
 */
typedef struct {
    const void *dt, *Bm, *Cm;
    const double *A, *dt_bias;
} rev_operands;

static int pick_reverse(rev_operands *r, const void *dt, const void *Bm, const void *Cm,
                        const double *A, const double *dt_bias, const void *dt_r,
                        const void *B_r, const void *C_r, const double *A_r,
                        const double *dt_bias_r)
{
    if (dt_r == NULL) {
        r->dt = dt; r->Bm = Bm; r->Cm = Cm; r->A = A; r->dt_bias = dt_bias;
        return 0;
    }
    if (B_r == NULL || C_r == NULL || A_r == NULL) return -1;
    r->dt = dt_r; r->Bm = B_r; r->Cm = C_r; r->A = A_r; r->dt_bias = dt_bias_r;
    return 0;
}

int oracle_version(void) { return 5; }

/* Threads the OpenMP loop over rows will use (1 without OpenMP). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Core routine.  Shapes (row-major, contiguous):
 *   x, dt: [batch, T, D]     Bm, Cm: [batch, T, N]     (dtype: fp32, bf16 or fp64)
 *   A: [D, N] fp64     Dskip: [D] fp64
 *   h0:    [batch, D, N] or NULL (zero)
 * Outputs (any may be NULL):
 *   y, yf, yr: [batch, T, D]  (yf = sum_n C*hf, yr = sum_n C*hr, y = yf+yr+Dskip*x)
 *   hT:        [batch, D, N]  forward state after token T-1
 *   bounds:    [batch, T/L+1, D, N]  forward state before token 0 and after
 *              every L-th token (bounds[:,0] = h0)
 * L must divide T (L >= 1).  Cm may be NULL only when y, yf and yr are NULL.
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int oracle_scan_ex(int64_t batch, int64_t T, int64_t D, int64_t N, int64_t L, int dtype,
                   const void *x, const void *dt, const void *Bm, const void *Cm,
                   const double *A, const double *Dskip, const double *h0,
                   const double *dt_bias, int dt_softplus, const void *z,
                   const void *dt_r, const void *B_r, const void *C_r, const double *A_r,
                   const double *dt_bias_r,
                   double *y, double *yf, double *yr, double *hT, double *bounds)
{
    const int want_y = (y != NULL) || (yf != NULL) || (yr != NULL);
    rev_operands rv;
    if (pick_reverse(&rv, dt, Bm, Cm, A, dt_bias, dt_r, B_r, C_r, A_r, dt_bias_r)) return -1;
    if (batch < 0 || T < 0 || D < 0 || N < 1 || L < 1) return -1;
    if (T % L != 0) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16 && dtype != ORACLE_F64) return -1;
    if (T > 0 && (x == NULL || dt == NULL || Bm == NULL)) return -1;
    if (A == NULL) return -1;
    if (want_y && T > 0 && (Cm == NULL || Dskip == NULL)) return -1;
    const int64_t nb = T / L;
    int fail = 0;

#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < D; ++d) {
            double *h = (double *)malloc((size_t)N * sizeof(double));
            double *r = (double *)malloc((size_t)N * sizeof(double));
            double *fwd = want_y ? (double *)malloc((size_t)(T > 0 ? T : 1) * sizeof(double)) : NULL;
            if (!h || !r || (want_y && !fwd)) {
                free(h); free(r); free(fwd);
#pragma omp atomic write
                fail = 1;
                continue;
            }
            for (int64_t n = 0; n < N; ++n)
                h[n] = h0 ? h0[(b * D + d) * N + n] : 0.0;
            if (bounds)
                for (int64_t n = 0; n < N; ++n)
                    bounds[((b * (nb + 1) + 0) * D + d) * N + n] = h[n];

            /* forward, causal, over the whole row */
            for (int64_t t = 0; t < T; ++t) {
                const size_t ix = (size_t)((b * T + t) * D + d);
                const size_t ib = (size_t)((b * T + t) * N);
                const double dtv = step_size(ld(dt, ix, dtype), dt_bias ? dt_bias[d] : 0.0, dt_softplus);
                const double xv = ld(x, ix, dtype);
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    const double decay = exp(dtv * A[d * N + n]);
                    const double inject = dtv * ld(Bm, ib + n, dtype) * xv;
                    h[n] = decay * h[n] + inject;
                    if (want_y) acc += ld(Cm, ib + n, dtype) * h[n];
                }
                if (want_y) fwd[t] = acc;
                if (bounds && (t + 1) % L == 0)
                    for (int64_t n = 0; n < N; ++n)
                        bounds[((b * (nb + 1) + (t + 1) / L) * D + d) * N + n] = h[n];
            }
            if (hT)
                for (int64_t n = 0; n < N; ++n) hT[(b * D + d) * N + n] = h[n];

            /* reverse, restricted to each L-token block, from zero at its end */
            if (want_y) {
                for (int64_t k = 0; k < nb; ++k) {
                    for (int64_t n = 0; n < N; ++n) r[n] = 0.0;
                    for (int64_t t = k * L + L - 1; t >= k * L; --t) {
                        const size_t ix = (size_t)((b * T + t) * D + d);
                        const size_t ib = (size_t)((b * T + t) * N);
                        const double dtv = step_size(ld(rv.dt, ix, dtype), rv.dt_bias ? rv.dt_bias[d] : 0.0, dt_softplus);
                        const double xv = ld(x, ix, dtype);
                        double acc = 0.0;
                        for (int64_t n = 0; n < N; ++n) {
                            const double decay = exp(dtv * rv.A[d * N + n]);
                            const double inject = dtv * ld(rv.Bm, ib + n, dtype) * xv;
                            r[n] = decay * r[n] + inject;
                            acc += ld(rv.Cm, ib + n, dtype) * r[n];
                        }
                        if (yf) yf[ix] = fwd[t];
                        if (yr) yr[ix] = acc;
                        if (y) y[ix] = (fwd[t] + acc + Dskip[d] * xv) * (z ? silu(ld(z, ix, dtype)) : 1.0);
                    }
                }
            }
            free(h); free(r); free(fwd);
        }
    }
    return fail ? -1 : 0;
}

/* The core routine without the fusions. */
int oracle_scan(int64_t batch, int64_t T, int64_t D, int64_t N, int64_t L, int dtype,
                const void *x, const void *dt, const void *Bm, const void *Cm,
                const double *A, const double *Dskip, const double *h0,
                double *y, double *yf, double *yr, double *hT, double *bounds)
{
    return oracle_scan_ex(batch, T, D, N, L, dtype, x, dt, Bm, Cm, A, Dskip, h0, NULL, 0, NULL,
                          NULL, NULL, NULL, NULL, NULL, y, yf, yr, hT, bounds);
}

/* ---- the five entry points, each a composition of the core routine ---- */

/* Clean-context prefill: forward over t_ctx tokens from h_init (NULL = 0);
 * h_cache <- forward state after the last context token.  When y is given it
 * also receives the clean-stream output (forward + in-block reverse per
 * committed block), i.e. what committing the blocks one by one would emit. */
int oracle_prefill(int64_t batch, int64_t D, int64_t N, int64_t L, int dtype, int64_t t_ctx,
                   const void *x, const void *dt, const void *Bm, const void *Cm,
                   const double *A, const double *Dskip, const double *h_init,
                   double *h_cache, double *y)
{
    return oracle_scan(batch, t_ctx, D, N, L, dtype, x, dt, Bm, Cm, A, Dskip, h_init,
                       y, NULL, NULL, h_cache, NULL);
}

/* One denoising step on the active block of exactly L tokens: forward from the
 * cache (not modified) plus the in-block reverse from zero; y: [batch, L, D]. */
int oracle_block_step(int64_t batch, int64_t D, int64_t N, int64_t L, int dtype,
                      const double *h_cache, const void *x, const void *dt, const void *Bm,
                      const void *Cm, const double *A, const double *Dskip, double *y)
{
    if (h_cache == NULL || y == NULL) return -1;
    return oracle_scan(batch, L, D, N, L, dtype, x, dt, Bm, Cm, A, Dskip, h_cache,
                       y, NULL, NULL, NULL, NULL);
}

/* Commit a finished block (L clean tokens): h_cache <- forward state after it.
 * The update is computed into a temporary so that input and output may be the
 * same buffer.  y (optional) equals block_step on the same inputs. */
int oracle_commit(int64_t batch, int64_t D, int64_t N, int64_t L, int dtype,
                  double *h_cache, const void *x, const void *dt, const void *Bm,
                  const void *Cm, const double *A, const double *Dskip, double *y)
{
    if (h_cache == NULL) return -1;
    const size_t ns = (size_t)(batch * D * N);
    double *tmp = (double *)malloc((ns ? ns : 1) * sizeof(double));
    if (!tmp) return -1;
    int rc = oracle_scan(batch, L, D, N, L, dtype, x, dt, Bm, Cm, A, Dskip, h_cache,
                         y, NULL, NULL, tmp, NULL);
    if (rc == 0) memcpy(h_cache, tmp, ns * sizeof(double));
    free(tmp);
    return rc;
}

/* All-block training form: continuous forward over T tokens from h_init
 * (NULL = 0) plus the reverse segmented into L-token blocks. */
int oracle_train_scan(int64_t batch, int64_t D, int64_t N, int64_t L, int dtype, int64_t T,
                      const void *x, const void *dt, const void *Bm, const void *Cm,
                      const double *A, const double *Dskip, const double *h_init,
                      double *y, double *h_bounds)
{
    return oracle_scan(batch, T, D, N, L, dtype, x, dt, Bm, Cm, A, Dskip, h_init,
                       y, NULL, NULL, NULL, h_bounds);
}

/* Two-stream training form, noisy stream: every L-block k runs its forward
 * scan from h0_blocks[b, k] (layout [batch, T/L + 1, D, N], the layout of the
 * bounds output; entry T/L is not read) and the reverse inside the block.
 * No state crosses a block boundary.  y: [batch, T, D]. */
int oracle_train_blocks_ex(int64_t batch, int64_t T, int64_t D, int64_t N, int64_t L, int dtype,
                           const void *x, const void *dt, const void *Bm, const void *Cm,
                           const double *A, const double *Dskip, const double *h0_blocks,
                           const double *dt_bias, int dt_softplus, const void *z,
                           const void *dt_r, const void *B_r, const void *C_r, const double *A_r,
                           const double *dt_bias_r, double *y)
{
    rev_operands rv;
    if (pick_reverse(&rv, dt, Bm, Cm, A, dt_bias, dt_r, B_r, C_r, A_r, dt_bias_r)) return -1;
    if (batch < 0 || T < 0 || D < 0 || N < 1 || L < 1 || T % L != 0) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16 && dtype != ORACLE_F64) return -1;
    if (T > 0 && (!x || !dt || !Bm || !Cm || !A || !Dskip || !h0_blocks || !y)) return -1;
    const int64_t nb = T / L;
    int fail = 0;
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < D; ++d) {
            double *h = (double *)malloc((size_t)N * sizeof(double));
            double *r = (double *)malloc((size_t)N * sizeof(double));
            double *fwd = (double *)malloc((size_t)L * sizeof(double));
            if (!h || !r || !fwd) {
                free(h); free(r); free(fwd);
#pragma omp atomic write
                fail = 1;
                continue;
            }
            for (int64_t k = 0; k < nb; ++k) {
                for (int64_t n = 0; n < N; ++n)
                    h[n] = h0_blocks[((b * (nb + 1) + k) * D + d) * N + n];
                /* forward through the block from its clean start state */
                for (int64_t t = k * L; t < k * L + L; ++t) {
                    const size_t ix = (size_t)((b * T + t) * D + d);
                    const size_t ib = (size_t)((b * T + t) * N);
                    const double dtv = step_size(ld(dt, ix, dtype), dt_bias ? dt_bias[d] : 0.0, dt_softplus);
                    const double xv = ld(x, ix, dtype);
                    double acc = 0.0;
                    for (int64_t n = 0; n < N; ++n) {
                        const double decay = exp(dtv * A[d * N + n]);
                        h[n] = decay * h[n] + dtv * ld(Bm, ib + n, dtype) * xv;
                        acc += ld(Cm, ib + n, dtype) * h[n];
                    }
                    fwd[t - k * L] = acc;
                }
                /* reverse inside the block from zero */
                for (int64_t n = 0; n < N; ++n) r[n] = 0.0;
                for (int64_t t = k * L + L - 1; t >= k * L; --t) {
                    const size_t ix = (size_t)((b * T + t) * D + d);
                    const size_t ib = (size_t)((b * T + t) * N);
                    const double dtv = step_size(ld(rv.dt, ix, dtype), rv.dt_bias ? rv.dt_bias[d] : 0.0, dt_softplus);
                    const double xv = ld(x, ix, dtype);
                    double acc = 0.0;
                    for (int64_t n = 0; n < N; ++n) {
                        const double decay = exp(dtv * rv.A[d * N + n]);
                        r[n] = decay * r[n] + dtv * ld(rv.Bm, ib + n, dtype) * xv;
                        acc += ld(rv.Cm, ib + n, dtype) * r[n];
                    }
                    y[ix] = (fwd[t - k * L] + acc + Dskip[d] * xv) * (z ? silu(ld(z, ix, dtype)) : 1.0);
                }
            }
            free(h); free(r); free(fwd);
        }
    }
    return fail ? -1 : 0;
}

int oracle_train_blocks(int64_t batch, int64_t T, int64_t D, int64_t N, int64_t L, int dtype,
                        const void *x, const void *dt, const void *Bm, const void *Cm,
                        const double *A, const double *Dskip, const double *h0_blocks, double *y)
{
    return oracle_train_blocks_ex(batch, T, D, N, L, dtype, x, dt, Bm, Cm, A, Dskip, h0_blocks,
                                  NULL, 0, NULL, NULL, NULL, NULL, NULL, NULL, y);
}

/* Full-sequence bidirectional baseline: the reverse runs over the whole
 * sequence (one segment of length T), forward from zero. */
int oracle_full_scan(int64_t batch, int64_t D, int64_t N, int dtype, int64_t T,
                     const void *x, const void *dt, const void *Bm, const void *Cm,
                     const double *A, const double *Dskip, double *y)
{
    if (T == 0) return 0;
    return oracle_scan(batch, T, D, N, T, dtype, x, dt, Bm, Cm, A, Dskip, NULL,
                       y, NULL, NULL, NULL, NULL);
}

/* ------------------------------------------------------------------------
 * Reverse-mode gradients of the scan (the backward pass of the training
 * forms).  The pages say the all-block objective lets downstream block losses
 * train the prefix scan [DE-M]; this is the derivative that does it, written
 * out from the two recurrences above for one (b, d) row and state n, with
 * a_t = exp(dt_t A[d,n]) and u_t = dt_t B_t[n] x_t:
 *   hf_t = a_t hf_{t-1} + u_t          (hf_{-1} = h0, or the block's start
 *                                       state in the two-stream form)
 *   hr_t = a_t hr_{t+1} + u_t          (hr = 0 after each block's last token)
 *   y_t  = sum_n C_t[n] (hf_t + hr_t) + Dskip x_t
 * Adjoints, given dy_t = dJ/dy_t (and dbounds = dJ/dbounds if the bounds feed
 * a later computation, as the clean stream's do in the two-stream form):
 *   gf_t = dy_t C_t[n] + a_{t+1} gf_{t+1} (+ dbounds[(t+1)/L] at block ends)
 *          -- right to left over the whole row (continuous form), or inside
 *             each block only (two-stream form)
 *   gr_t = dy_t C_t[n] + a_{t-1} gr_{t-1}
 *          -- left to right inside each block (the reverse scan's adjoint)
 *   du_t = gf_t + gr_t,   da_t = gf_t hf_{t-1} + gr_t hr_{t+1}
 * and then, by the chain rule through a_t and u_t:
 *   ddt_t    += sum_n du_t B_t[n] x_t + da_t a_t A[d,n]
 *   dx_t     += sum_n du_t dt_t B_t[n]   + dy_t Dskip
 *   dB_t[n]  += du_t dt_t x_t            (summed over channels d)
 *   dC_t[n]  += dy_t (hf_t + hr_t)       (summed over channels d)
 *   dA[d,n]  += da_t a_t dt_t            (summed over batch and tokens)
 *   dDskip   += dy_t x_t
 *   dh0[n]    = a_0 gf_0 (+ dbounds[0])  continuous form
 *   dh0_blocks[k][n] = a_{kL} gf_{kL}    two-stream form (entry T/L: zero)
 *
 * Arguments: the forward inputs (stream dtype as in oracle_scan), exactly one
 * of h0 (continuous form; NULL = zero start) or h0_blocks (two-stream form,
 * [batch, T/L+1, D, N]) as selected by `blocks`, dy [batch, T, D] fp64, dbounds
 * (continuous form only, [batch, T/L+1, D, N] fp64, or NULL).  Outputs (fp64,
 * any may be NULL, all overwritten): dx, ddt [batch, T, D]; dB, dC
 * [batch, T, N]; dA [D, N]; dDskip [D]; dh0 [batch, D, N] (continuous);
 * dh0_blocks [batch, T/L+1, D, N] (two-stream).
 * Rows run in parallel; the cross-row sums (dB, dC over channels, dA and
 * dDskip over batch and tokens) are accumulated per thread and added in
 * thread order afterwards.
 */
/*
 * With the optional fusions of the forward (oracle_scan_ex: dt = dt_stream +
 * dt_bias, through softplus when dt_softplus; output multiplied by silu(z)),
 * the same chain rule runs on the effective step size and on the gradient of
 * the ungated output:
 *   v_t = dt_stream_t + dt_bias, dt_t = softplus(v_t) (or v_t); every term
 *     above uses dt_t;
 *   g_t = dy_t silu(z_t) takes the place of dy_t in every term above;
 *   dz_t = dy_t y_pre_t silu'(z_t), y_pre_t = sum_n C_t (hf_t + hr_t) + Dskip x_t,
 *     silu'(z) = s(z) (1 + z (1 - s(z))), s = the logistic function;
 *   ddt (the gradient of the dt stream) = ddt_t softplus'(v_t) = ddt_t s(v_t)
 *     (or ddt_t); d_dt_bias[d] = the sum over batch and tokens of that.
 * dt_bias, z may be NULL (no bias, no gate); dz [batch, T, D] and d_dt_bias [D]
 * (fp64) may be NULL.  Separate reverse-direction operands are not taken.
 */
static double sigmoid(double v) { return v >= 0.0 ? 1.0 / (1.0 + exp(-v)) : exp(v) / (1.0 + exp(v)); }

int oracle_scan_bwd_ex(int64_t batch, int64_t T, int64_t D, int64_t N, int64_t L, int dtype,
                       const void *x, const void *dt, const void *Bm, const void *Cm,
                       const double *A, const double *Dskip, int blocks, const double *h0,
                       const double *h0_blocks, const double *dy, const double *dbounds,
                       const double *dt_bias, int dt_softplus, const void *z,
                       double *dx, double *ddt, double *dB, double *dC, double *dA,
                       double *dDskip, double *dh0, double *dh0_blocks, double *dz,
                       double *d_dt_bias)
{
    if (batch < 0 || T < 0 || D < 0 || N < 1 || L < 1 || T % L != 0) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16 && dtype != ORACLE_F64) return -1;
    if (!A || !Dskip) return -1;
    if (T > 0 && (!x || !dt || !Bm || !Cm || !dy)) return -1;
    if (blocks && (h0 || dbounds || (T > 0 && !h0_blocks))) return -1;
    if (!blocks && (h0_blocks || dh0_blocks)) return -1;
    const int64_t nb = T / L;
    const size_t n_tok = (size_t)(batch * T * D), n_bc = (size_t)(batch * T * N);
    if (dx) memset(dx, 0, n_tok * sizeof(double));
    if (ddt) memset(ddt, 0, n_tok * sizeof(double));
    if (dB) memset(dB, 0, n_bc * sizeof(double));
    if (dC) memset(dC, 0, n_bc * sizeof(double));
    if (dA) memset(dA, 0, (size_t)(D * N) * sizeof(double));
    if (dDskip) memset(dDskip, 0, (size_t)D * sizeof(double));
    if (dh0) memset(dh0, 0, (size_t)(batch * D * N) * sizeof(double));
    if (dh0_blocks) memset(dh0_blocks, 0, (size_t)(batch * (nb + 1) * D * N) * sizeof(double));
    if (dz) memset(dz, 0, n_tok * sizeof(double));
    if (d_dt_bias) memset(d_dt_bias, 0, (size_t)D * sizeof(double));
    if (batch == 0 || D == 0) return 0;

    int nthr = 1;
#ifdef _OPENMP
    nthr = omp_get_max_threads();
#endif
    /* per-thread partial sums of the cross-row gradients */
    const size_t part = 2 * n_bc + (size_t)(D * N) + 2 * (size_t)D;
    double *parts = (double *)calloc((size_t)nthr * part, sizeof(double));
    if (!parts) return -1;
    int fail = 0;

#pragma omp parallel num_threads(nthr)
    {
        int tid = 0;
#ifdef _OPENMP
        tid = omp_get_thread_num();
#endif
        double *my_dB = parts + (size_t)tid * part;
        double *my_dC = my_dB + n_bc;
        double *my_dA = my_dC + n_bc;
        double *my_dD = my_dA + D * N;
        double *my_dbias = my_dD + D;
        const size_t tn = (size_t)(T > 0 ? T : 1) * (size_t)N;
        double *a = (double *)malloc(tn * sizeof(double));      /* a_t[n]       */
        double *hp = (double *)malloc(tn * sizeof(double));     /* hf_{t-1}[n]  */
        double *rn = (double *)malloc(tn * sizeof(double));     /* hr_{t+1}[n]  */
        double *gr = (double *)malloc(tn * sizeof(double));     /* gr_t[n]      */
        double *h = (double *)malloc((size_t)N * sizeof(double));
        double *q = (double *)malloc((size_t)N * sizeof(double));
        if (!a || !hp || !rn || !gr || !h || !q) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(static) collapse(2)
        for (int64_t b = 0; b < batch; ++b) {
            for (int64_t d = 0; d < D; ++d) {
                if (fail) continue;
                /* forward: decays and the state before every token */
                for (int64_t t = 0; t < T; ++t) {
                    if (t == 0 || (blocks && t % L == 0)) {
                        for (int64_t n = 0; n < N; ++n) {
                            if (blocks) h[n] = h0_blocks[((b * (nb + 1) + t / L) * D + d) * N + n];
                            else h[n] = h0 ? h0[(b * D + d) * N + n] : 0.0;
                        }
                    }
                    const size_t ix = (size_t)((b * T + t) * D + d);
                    const size_t ib = (size_t)((b * T + t) * N);
                    const double dtv = step_size(ld(dt, ix, dtype), dt_bias ? dt_bias[d] : 0.0, dt_softplus);
                    const double xv = ld(x, ix, dtype);
                    for (int64_t n = 0; n < N; ++n) {
                        const double at = exp(dtv * A[d * N + n]);
                        a[t * N + n] = at;
                        hp[t * N + n] = h[n];
                        h[n] = at * h[n] + dtv * ld(Bm, ib + n, dtype) * xv;
                    }
                }
                /* in-block reverse: the state after every token (hr_{t+1}) */
                for (int64_t k = 0; k < nb; ++k) {
                    for (int64_t n = 0; n < N; ++n) h[n] = 0.0;
                    for (int64_t t = k * L + L - 1; t >= k * L; --t) {
                        const size_t ix = (size_t)((b * T + t) * D + d);
                        const size_t ib = (size_t)((b * T + t) * N);
                        const double dtv = step_size(ld(dt, ix, dtype), dt_bias ? dt_bias[d] : 0.0, dt_softplus);
                        const double xv = ld(x, ix, dtype);
                        for (int64_t n = 0; n < N; ++n) {
                            rn[t * N + n] = h[n];
                            h[n] = a[t * N + n] * h[n] + dtv * ld(Bm, ib + n, dtype) * xv;
                        }
                    }
                }
                /* adjoint of the in-block reverse, left to right in each block */
                for (int64_t k = 0; k < nb; ++k) {
                    for (int64_t n = 0; n < N; ++n) q[n] = 0.0;
                    for (int64_t t = k * L; t < k * L + L; ++t) {
                        const size_t ix = (size_t)((b * T + t) * D + d);
                        const size_t ib = (size_t)((b * T + t) * N);
                        const double gy = z ? dy[ix] * silu(ld(z, ix, dtype)) : dy[ix];
                        for (int64_t n = 0; n < N; ++n) {
                            const double g = gy * ld(Cm, ib + n, dtype) + q[n];
                            gr[t * N + n] = g;
                            q[n] = a[t * N + n] * g;
                        }
                    }
                }
                /* adjoint of the forward, right to left, and every gradient */
                for (int64_t n = 0; n < N; ++n) q[n] = 0.0;
                for (int64_t t = T - 1; t >= 0; --t) {
                    const size_t ix = (size_t)((b * T + t) * D + d);
                    const size_t ib = (size_t)((b * T + t) * N);
                    const double vraw = ld(dt, ix, dtype) + (dt_bias ? dt_bias[d] : 0.0);
                    const double dtv = step_size(ld(dt, ix, dtype), dt_bias ? dt_bias[d] : 0.0, dt_softplus);
                    const double xv = ld(x, ix, dtype);
                    const double zv = z ? ld(z, ix, dtype) : 0.0;
                    const double gy = z ? dy[ix] * silu(zv) : dy[ix];
                    const int block_end = (t + 1) % L == 0;
                    if (blocks && block_end)
                        for (int64_t n = 0; n < N; ++n) q[n] = 0.0;
                    double sdt = 0.0, sx = 0.0, ypre = Dskip[d] * xv;
                    for (int64_t n = 0; n < N; ++n) {
                        const double bv = ld(Bm, ib + n, dtype), cv = ld(Cm, ib + n, dtype);
                        double gf = gy * cv + q[n];
                        if (!blocks && block_end && dbounds)
                            gf += dbounds[((b * (nb + 1) + (t + 1) / L) * D + d) * N + n];
                        const double at = a[t * N + n];
                        const double u = dtv * bv * xv;
                        const double du = gf + gr[t * N + n];
                        const double da = gf * hp[t * N + n] + gr[t * N + n] * rn[t * N + n];
                        sdt += du * bv * xv + da * at * A[d * N + n];
                        sx += du * dtv * bv;
                        my_dB[ib + n] += du * dtv * xv;
                        const double hsum = (at * hp[t * N + n] + u) + (at * rn[t * N + n] + u);
                        my_dC[ib + n] += gy * hsum;
                        ypre += cv * hsum;
                        my_dA[d * N + n] += da * at * dtv;
                        q[n] = at * gf;
                    }
                    /* the dt stream's gradient: through softplus when it is used */
                    const double draw = dt_softplus ? sdt * sigmoid(vraw) : sdt;
                    if (ddt) ddt[ix] = draw;
                    my_dbias[d] += draw;
                    if (dx) dx[ix] = sx + gy * Dskip[d];
                    my_dD[d] += gy * xv;
                    if (dz && z) {
                        const double s = sigmoid(zv);
                        dz[ix] = dy[ix] * ypre * s * (1.0 + zv * (1.0 - s));
                    }
                    if (blocks && t % L == 0 && dh0_blocks)
                        for (int64_t n = 0; n < N; ++n)
                            dh0_blocks[((b * (nb + 1) + t / L) * D + d) * N + n] = q[n];
                }
                if (!blocks && dh0)
                    for (int64_t n = 0; n < N; ++n)
                        dh0[(b * D + d) * N + n] =
                            q[n] + (dbounds ? dbounds[((b * (nb + 1)) * D + d) * N + n] : 0.0);
            }
        }
        free(a); free(hp); free(rn); free(gr); free(h); free(q);
    }
    if (!fail) {
        for (int th = 0; th < nthr; ++th) {
            const double *p = parts + (size_t)th * part;
            if (dB) for (size_t i = 0; i < n_bc; ++i) dB[i] += p[i];
            if (dC) for (size_t i = 0; i < n_bc; ++i) dC[i] += p[n_bc + i];
            if (dA) for (int64_t i = 0; i < D * N; ++i) dA[i] += p[2 * n_bc + i];
            if (dDskip) for (int64_t i = 0; i < D; ++i) dDskip[i] += p[2 * n_bc + D * N + i];
            if (d_dt_bias) for (int64_t i = 0; i < D; ++i) d_dt_bias[i] += p[2 * n_bc + D * N + D + i];
        }
    }
    free(parts);
    return fail ? -1 : 0;
}

/* ------------------------------------------------------------------------
 * The same gradients when the reverse scan has operands of its own (see
 * rev_operands: dt_r with its own bias and the same softplus setting, B_r,
 * C_r, A_r).  The two recurrences then share only x:
 *   hf_t = a_t hf_{t-1} + u_t,      a_t = exp(dt_t A),     u_t = dt_t B_t x_t
 *   hr_t = ar_t hr_{t+1} + ur_t,    ar_t = exp(dtr_t A_r), ur_t = dtr_t B_r_t x_t
 *   y_t  = (sum_n C_t hf_t + C_r_t hr_t + Dskip x_t) [silu(z_t)]
 * Adjoints (g = dy, or dy silu(z) with the gate):
 *   gf_t = g_t C_t + a_{t+1} gf_{t+1}       (+ dbounds at block ends, as before)
 *   gr_t = g_t C_r_t + ar_{t-1} gr_{t-1}    (left to right inside each block)
 * and every term splits by direction:
 *   forward operands:  ddt  += sum_n gf B x + gf hf_{t-1} a A;  dB += gf dt x;
 *                      dC += g hf_t;  dA += gf hf_{t-1} a dt
 *   reverse operands:  ddt_r += sum_n gr B_r x + gr hr_{t+1} ar A_r;
 *                      dB_r += gr dtr x;  dC_r += g hr_t;  dA_r += gr hr_{t+1} ar dtr
 *   dx += sum_n gf dt B + gr dtr B_r  (+ g Dskip)
 * The dt streams' gradients go through softplus'(v) = s(v) of their own v, and
 * d_dt_bias / d_dt_bias_r sum them.  With the reverse sharing the forward's
 * operands these are the terms of oracle_scan_bwd_ex, added pairwise.
 * Arguments as in oracle_scan_bwd_ex plus the reverse operands (dt_r, B_r, C_r
 * in the stream dtype, A_r [D, N] and dt_bias_r [D] fp64, dt_bias_r may be
 * NULL) and their gradients (fp64, any may be NULL): ddt_r [batch, T, D],
 * dB_r, dC_r [batch, T, N], dA_r [D, N], d_dt_bias_r [D].
 */
int oracle_scan_bwd_sep(int64_t batch, int64_t T, int64_t D, int64_t N, int64_t L, int dtype,
                        const void *x, const void *dt, const void *Bm, const void *Cm,
                        const double *A, const double *Dskip, int blocks, const double *h0,
                        const double *h0_blocks, const double *dy, const double *dbounds,
                        const double *dt_bias, int dt_softplus, const void *z,
                        const void *dt_r, const void *B_r, const void *C_r, const double *A_r,
                        const double *dt_bias_r,
                        double *dx, double *ddt, double *dB, double *dC, double *dA,
                        double *dDskip, double *dh0, double *dh0_blocks, double *dz,
                        double *d_dt_bias, double *ddt_r, double *dB_r, double *dC_r,
                        double *dA_r, double *d_dt_bias_r)
{
    if (batch < 0 || T < 0 || D < 0 || N < 1 || L < 1 || T % L != 0) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16 && dtype != ORACLE_F64) return -1;
    if (!A || !Dskip || !A_r) return -1;
    if (T > 0 && (!x || !dt || !Bm || !Cm || !dy || !dt_r || !B_r || !C_r)) return -1;
    if (blocks && (h0 || dbounds || (T > 0 && !h0_blocks))) return -1;
    if (!blocks && (h0_blocks || dh0_blocks)) return -1;
    const int64_t nb = T / L;
    const size_t n_tok = (size_t)(batch * T * D), n_bc = (size_t)(batch * T * N);
    double *outs_tok[] = {dx, ddt, dz, ddt_r};
    for (int i = 0; i < 4; ++i) if (outs_tok[i]) memset(outs_tok[i], 0, n_tok * sizeof(double));
    double *outs_bc[] = {dB, dC, dB_r, dC_r};
    for (int i = 0; i < 4; ++i) if (outs_bc[i]) memset(outs_bc[i], 0, n_bc * sizeof(double));
    if (dA) memset(dA, 0, (size_t)(D * N) * sizeof(double));
    if (dA_r) memset(dA_r, 0, (size_t)(D * N) * sizeof(double));
    if (dDskip) memset(dDskip, 0, (size_t)D * sizeof(double));
    if (d_dt_bias) memset(d_dt_bias, 0, (size_t)D * sizeof(double));
    if (d_dt_bias_r) memset(d_dt_bias_r, 0, (size_t)D * sizeof(double));
    if (dh0) memset(dh0, 0, (size_t)(batch * D * N) * sizeof(double));
    if (dh0_blocks) memset(dh0_blocks, 0, (size_t)(batch * (nb + 1) * D * N) * sizeof(double));
    if (batch == 0 || D == 0) return 0;

    int nthr = 1;
#ifdef _OPENMP
    nthr = omp_get_max_threads();
#endif
    /* per-thread partial sums: dB, dC, dB_r, dC_r, dA, dA_r, dDskip, the two bias sums */
    const size_t part = 4 * n_bc + 2 * (size_t)(D * N) + 3 * (size_t)D;
    double *parts = (double *)calloc((size_t)nthr * part, sizeof(double));
    if (!parts) return -1;
    int fail = 0;

#pragma omp parallel num_threads(nthr)
    {
        int tid = 0;
#ifdef _OPENMP
        tid = omp_get_thread_num();
#endif
        double *my_dB = parts + (size_t)tid * part;
        double *my_dC = my_dB + n_bc;
        double *my_dBr = my_dC + n_bc;
        double *my_dCr = my_dBr + n_bc;
        double *my_dA = my_dCr + n_bc;
        double *my_dAr = my_dA + D * N;
        double *my_dD = my_dAr + D * N;
        double *my_dbias = my_dD + D;
        double *my_dbias_r = my_dbias + D;
        const size_t tn = (size_t)(T > 0 ? T : 1) * (size_t)N;
        double *a = (double *)malloc(tn * sizeof(double));      /* a_t[n]        */
        double *ar = (double *)malloc(tn * sizeof(double));     /* ar_t[n]       */
        double *hp = (double *)malloc(tn * sizeof(double));     /* hf_{t-1}[n]   */
        double *rn = (double *)malloc(tn * sizeof(double));     /* hr_{t+1}[n]   */
        double *gr = (double *)malloc(tn * sizeof(double));     /* gr_t[n]       */
        double *h = (double *)malloc((size_t)N * sizeof(double));
        double *q = (double *)malloc((size_t)N * sizeof(double));
        if (!a || !ar || !hp || !rn || !gr || !h || !q) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(static) collapse(2)
        for (int64_t b = 0; b < batch; ++b) {
            for (int64_t d = 0; d < D; ++d) {
                if (fail) continue;
                const double bias = dt_bias ? dt_bias[d] : 0.0, bias_r = dt_bias_r ? dt_bias_r[d] : 0.0;
                /* forward recurrence: its decays and the state before every token */
                for (int64_t t = 0; t < T; ++t) {
                    if (t == 0 || (blocks && t % L == 0)) {
                        for (int64_t n = 0; n < N; ++n) {
                            if (blocks) h[n] = h0_blocks[((b * (nb + 1) + t / L) * D + d) * N + n];
                            else h[n] = h0 ? h0[(b * D + d) * N + n] : 0.0;
                        }
                    }
                    const size_t ix = (size_t)((b * T + t) * D + d);
                    const size_t ib = (size_t)((b * T + t) * N);
                    const double dtv = step_size(ld(dt, ix, dtype), bias, dt_softplus);
                    const double xv = ld(x, ix, dtype);
                    for (int64_t n = 0; n < N; ++n) {
                        const double at = exp(dtv * A[d * N + n]);
                        a[t * N + n] = at;
                        hp[t * N + n] = h[n];
                        h[n] = at * h[n] + dtv * ld(Bm, ib + n, dtype) * xv;
                    }
                }
                /* reverse recurrence in each block, on its own operands: the state after every token */
                for (int64_t k = 0; k < nb; ++k) {
                    for (int64_t n = 0; n < N; ++n) h[n] = 0.0;
                    for (int64_t t = k * L + L - 1; t >= k * L; --t) {
                        const size_t ix = (size_t)((b * T + t) * D + d);
                        const size_t ib = (size_t)((b * T + t) * N);
                        const double dtr = step_size(ld(dt_r, ix, dtype), bias_r, dt_softplus);
                        const double xv = ld(x, ix, dtype);
                        for (int64_t n = 0; n < N; ++n) {
                            const double at = exp(dtr * A_r[d * N + n]);
                            ar[t * N + n] = at;
                            rn[t * N + n] = h[n];
                            h[n] = at * h[n] + dtr * ld(B_r, ib + n, dtype) * xv;
                        }
                    }
                }
                /* adjoint of the reverse recurrence, left to right in each block */
                for (int64_t k = 0; k < nb; ++k) {
                    for (int64_t n = 0; n < N; ++n) q[n] = 0.0;
                    for (int64_t t = k * L; t < k * L + L; ++t) {
                        const size_t ix = (size_t)((b * T + t) * D + d);
                        const size_t ib = (size_t)((b * T + t) * N);
                        const double gy = z ? dy[ix] * silu(ld(z, ix, dtype)) : dy[ix];
                        for (int64_t n = 0; n < N; ++n) {
                            const double g = gy * ld(C_r, ib + n, dtype) + q[n];
                            gr[t * N + n] = g;
                            q[n] = ar[t * N + n] * g;
                        }
                    }
                }
                /* adjoint of the forward recurrence, right to left, and every gradient */
                for (int64_t n = 0; n < N; ++n) q[n] = 0.0;
                for (int64_t t = T - 1; t >= 0; --t) {
                    const size_t ix = (size_t)((b * T + t) * D + d);
                    const size_t ib = (size_t)((b * T + t) * N);
                    const double v = ld(dt, ix, dtype) + bias, vr = ld(dt_r, ix, dtype) + bias_r;
                    const double dtv = step_size(ld(dt, ix, dtype), bias, dt_softplus);
                    const double dtr = step_size(ld(dt_r, ix, dtype), bias_r, dt_softplus);
                    const double xv = ld(x, ix, dtype);
                    const double zv = z ? ld(z, ix, dtype) : 0.0;
                    const double gy = z ? dy[ix] * silu(zv) : dy[ix];
                    const int block_end = (t + 1) % L == 0;
                    if (blocks && block_end)
                        for (int64_t n = 0; n < N; ++n) q[n] = 0.0;
                    double sdt = 0.0, sdt_r = 0.0, sx = 0.0, ypre = Dskip[d] * xv;
                    for (int64_t n = 0; n < N; ++n) {
                        const double bv = ld(Bm, ib + n, dtype), cv = ld(Cm, ib + n, dtype);
                        const double bvr = ld(B_r, ib + n, dtype), cvr = ld(C_r, ib + n, dtype);
                        double gf = gy * cv + q[n];
                        if (!blocks && block_end && dbounds)
                            gf += dbounds[((b * (nb + 1) + (t + 1) / L) * D + d) * N + n];
                        const double at = a[t * N + n], atr = ar[t * N + n];
                        const double g_r = gr[t * N + n];
                        const double hf_t = at * hp[t * N + n] + dtv * bv * xv;
                        const double hr_t = atr * rn[t * N + n] + dtr * bvr * xv;
                        /* forward operands */
                        const double da = gf * hp[t * N + n];
                        sdt += gf * bv * xv + da * at * A[d * N + n];
                        my_dB[ib + n] += gf * dtv * xv;
                        my_dC[ib + n] += gy * hf_t;
                        my_dA[d * N + n] += da * at * dtv;
                        /* reverse operands */
                        const double da_r = g_r * rn[t * N + n];
                        sdt_r += g_r * bvr * xv + da_r * atr * A_r[d * N + n];
                        my_dBr[ib + n] += g_r * dtr * xv;
                        my_dCr[ib + n] += gy * hr_t;
                        my_dAr[d * N + n] += da_r * atr * dtr;
                        sx += gf * dtv * bv + g_r * dtr * bvr;
                        ypre += cv * hf_t + cvr * hr_t;
                        q[n] = at * gf;
                    }
                    const double draw = dt_softplus ? sdt * sigmoid(v) : sdt;
                    const double draw_r = dt_softplus ? sdt_r * sigmoid(vr) : sdt_r;
                    if (ddt) ddt[ix] = draw;
                    if (ddt_r) ddt_r[ix] = draw_r;
                    my_dbias[d] += draw;
                    my_dbias_r[d] += draw_r;
                    if (dx) dx[ix] = sx + gy * Dskip[d];
                    my_dD[d] += gy * xv;
                    if (dz && z) {
                        const double s = sigmoid(zv);
                        dz[ix] = dy[ix] * ypre * s * (1.0 + zv * (1.0 - s));
                    }
                    if (blocks && t % L == 0 && dh0_blocks)
                        for (int64_t n = 0; n < N; ++n)
                            dh0_blocks[((b * (nb + 1) + t / L) * D + d) * N + n] = q[n];
                }
                if (!blocks && dh0)
                    for (int64_t n = 0; n < N; ++n)
                        dh0[(b * D + d) * N + n] =
                            q[n] + (dbounds ? dbounds[((b * (nb + 1)) * D + d) * N + n] : 0.0);
            }
        }
        free(a); free(ar); free(hp); free(rn); free(gr); free(h); free(q);
    }
    if (!fail) {
        for (int th = 0; th < nthr; ++th) {
            const double *p = parts + (size_t)th * part;
            double *dst[] = {dB, dC, dB_r, dC_r};
            for (int i = 0; i < 4; ++i)
                if (dst[i]) for (size_t j = 0; j < n_bc; ++j) dst[i][j] += p[i * n_bc + j];
            const double *pa = p + 4 * n_bc;
            if (dA) for (int64_t i = 0; i < D * N; ++i) dA[i] += pa[i];
            if (dA_r) for (int64_t i = 0; i < D * N; ++i) dA_r[i] += pa[D * N + i];
            const double *pd = pa + 2 * D * N;
            if (dDskip) for (int64_t i = 0; i < D; ++i) dDskip[i] += pd[i];
            if (d_dt_bias) for (int64_t i = 0; i < D; ++i) d_dt_bias[i] += pd[D + i];
            if (d_dt_bias_r) for (int64_t i = 0; i < D; ++i) d_dt_bias_r[i] += pd[2 * D + i];
        }
    }
    free(parts);
    return fail ? -1 : 0;
}

int oracle_scan_bwd(int64_t batch, int64_t T, int64_t D, int64_t N, int64_t L, int dtype,
                    const void *x, const void *dt, const void *Bm, const void *Cm,
                    const double *A, const double *Dskip, int blocks, const double *h0,
                    const double *h0_blocks, const double *dy, const double *dbounds,
                    double *dx, double *ddt, double *dB, double *dC, double *dA,
                    double *dDskip, double *dh0, double *dh0_blocks)
{
    return oracle_scan_bwd_ex(batch, T, D, N, L, dtype, x, dt, Bm, Cm, A, Dskip, blocks, h0,
                              h0_blocks, dy, dbounds, NULL, 0, NULL, dx, ddt, dB, dC, dA, dDskip,
                              dh0, dh0_blocks, NULL, NULL);
}
