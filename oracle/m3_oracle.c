/*
 * m3_oracle.c -- plain, sequential fp64 CPU reference for the Mamba-3 SSM layer core.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that the HIP library is checked against.
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg may build, load or
 * call it.  It shares no code, header, table or helper with the GPU library, and it never
 * receives a value produced by the GPU library.
 *
 * Every quantity is computed in double precision, one (batch, head) at a time, one time step
 * after another, exactly in the order the defining equations state.  The only parallelism is
 * an OpenMP loop over independent (batch, head) pairs, which does not change any arithmetic.
 *
 * Sources (pages on "Mamba-3: Improved Sequence Modeling using State Space Principles"):
 *  - aipaper.cc summary, section 4.1, Proposition 1: the exponential-trapezoidal recurrence
 *    h_t = alpha_t h_{t-1} + beta_t B_{t-1} x_{t-1} + gamma_t B_t x_t with
 *    alpha_t = exp(dt_t A_t), beta_t = (1 - lambda_t) dt_t exp(dt_t A_t), gamma_t = lambda_t dt_t.
 *  - same page, section 4.2, Propositions 2 and 3: a complex diagonal transition is a real SSM
 *    with 2x2 block rotations, and the rotations are absorbed into B and C as the cumulative
 *    product prod_{i<=t} R_i^T ("RoPE trick").
 *  - same page, section 4.3: MIMO update H_t = a_t H_{t-1} + B_t X_t^T.
 *  - metaphor-xennon SSM family comparison, section 2.2: rotation matrix
 *    R_t = [[cos(dt theta), -sin(dt theta)], [sin(dt theta), cos(dt theta)]].
 *  - papernotes.org summary, "key design" item 4: BCNorm (RMSNorm after the B/C projections)
 *    and a learnable head-specific B/C bias.
 *
 * Readings where the pages are silent (each is listed in the design notes of the repository):
 *  - The previous-input (beta) term is carried by the full complex transition, so in the
 *    rotated frame the recurrence is the real trapezoid recurrence on rotated B and C.
 *  - The rotation angle of step t is dt_t * theta_t[k] for pair k = (2k, 2k+1); the cumulative
 *    angle includes the current step.
 *  - BCNorm is an RMS over the N entries of each (batch, step, head, rank) vector with
 *    eps added to the mean square, an optional per-head weight, then the bias, then rotation.
 *  - The returned state is the kernel frame g_t = R(Phi_t)^T h_t, returned with Phi_t.
 *  - MIMO output mixing, when requested, is y[p] = sum_r w_out[h, r, p] * Y[r, p].
 *
 * The two *_backward functions at the end are the exact gradients of the two forward functions
 * (reverse-mode, one step after another in reverse time order): the pages define no backward
 * pass, so the gradient of the forward definition is the definition followed.
 *
 * Layouts (row-major, all double):
 *  B, C, Bbar, Cbar  [b, L, H, R, N]      x  [b, L, H, R, P]      dt, lam  [b, L, H]
 *  theta             [b, L, H, N/2]       A  [H]                  normw  [H, N]     bias  [H, R, N]
 *  phi               [b, H, N/2]          h  [b, H, N, P]         Bbar_prev [b, H, R, N]
 *  x_prev            [b, H, R, P]         w_out [H, R, P]
 *  y                 [b, L, H, P] when w_out is given, else [b, L, H, R, P]
 */
#include <math.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdlib.h>
#include <string.h>

/*
 * BCNorm + bias + cumulative rotation (papernotes item 4; aipaper section 4.2 Proposition 3;
 * metaphor-xennon section 2.2 rotation matrix).
 *
 * For every (batch, head): Phi starts at phi_in (zero when phi_in is NULL); at each step t,
 * Phi[k] += dt_t * theta_t[k]; then for each rank r and each of B and C:
 *   v      = raw vector (N entries)
 *   v_norm = v / sqrt(mean(v^2) + eps) * w        (only when bcnorm != 0; w = 1 when NULL)
 *   v_b    = v_norm + bias[h, r, :]               (bias skipped when NULL)
 *   out    = R(Phi)^T v_b on each pair (2k, 2k+1):
 *            out[2k]   =  cos(Phi[k]) v_b[2k] + sin(Phi[k]) v_b[2k+1]
 *            out[2k+1] = -sin(Phi[k]) v_b[2k] + cos(Phi[k]) v_b[2k+1]
 * phi_out receives the final, unreduced Phi.
 */
void m3o_bcnorm_rope(int64_t nb, int64_t L, int64_t H, int64_t R, int64_t N,
                     int bcnorm, double eps,
                     const double *B, const double *C, const double *dt, const double *theta,
                     const double *normw_B, const double *normw_C,
                     const double *bias_B, const double *bias_C,
                     const double *phi_in,
                     double *Bbar, double *Cbar, double *phi_out)
{
    const int64_t K = N / 2;
    int64_t bh;
#pragma omp parallel for schedule(dynamic, 1)
    for (bh = 0; bh < nb * H; ++bh) {
        const int64_t ib = bh / H, h = bh % H;
        double *phi = (double *)malloc(sizeof(double) * K);
        double *v = (double *)malloc(sizeof(double) * N);
        for (int64_t k = 0; k < K; ++k)
            phi[k] = phi_in ? phi_in[(ib * H + h) * K + k] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
            const int64_t row = (ib * L + t) * H + h;   /* index of (b, t, h) */
            const double d = dt[row];
            for (int64_t k = 0; k < K; ++k)
                phi[k] += d * theta[row * K + k];
            for (int which = 0; which < 2; ++which) {
                const double *src = which == 0 ? B : C;
                double *dst = which == 0 ? Bbar : Cbar;
                const double *w = which == 0 ? normw_B : normw_C;
                const double *bias = which == 0 ? bias_B : bias_C;
                for (int64_t r = 0; r < R; ++r) {
                    const double *in = src + (row * R + r) * N;
                    double *out = dst + (row * R + r) * N;
                    for (int64_t n = 0; n < N; ++n)
                        v[n] = in[n];
                    if (bcnorm) {
                        double ms = 0.0;
                        for (int64_t n = 0; n < N; ++n)
                            ms += v[n] * v[n];
                        ms /= (double)N;
                        const double inv = 1.0 / sqrt(ms + eps);
                        for (int64_t n = 0; n < N; ++n)
                            v[n] = v[n] * inv * (w ? w[h * N + n] : 1.0);
                    }
                    if (bias)
                        for (int64_t n = 0; n < N; ++n)
                            v[n] += bias[(h * R + r) * N + n];
                    for (int64_t k = 0; k < K; ++k) {
                        const double c = cos(phi[k]), s = sin(phi[k]);
                        out[2 * k] = c * v[2 * k] + s * v[2 * k + 1];
                        out[2 * k + 1] = -s * v[2 * k] + c * v[2 * k + 1];
                    }
                }
            }
        }
        for (int64_t k = 0; k < K; ++k)
            phi_out[(ib * H + h) * K + k] = phi[k];
        free(phi);
        free(v);
    }
}

/*
 * The exponential-trapezoidal MIMO recurrence on rotated B and C (aipaper section 4.1
 * Proposition 1, section 4.3 MIMO), written out step by step for every (batch, head):
 *
 *   g_{-1} = h_in (zero when NULL)
 *   u_{-1} = sum_r Bbar_prev[r, :]^T x_prev[r, :]   (zero when either is NULL)
 *   for t = 0 .. L-1:
 *     alpha = exp(dt_t A_h),  beta = (1 - lam_t) dt_t alpha,  gamma = lam_t dt_t
 *     u_t   = sum_r Bbar_t[r, :]^T x_t[r, :]                   (N x P)
 *     g_t   = alpha g_{t-1} + beta u_{t-1} + gamma u_t
 *     Y_t[r, :] = Cbar_t[r, :] g_t                             (R x P)
 *     y_t[p] = sum_r w_out[h, r, p] Y_t[r, p]   if w_out, else y_t = Y_t
 *   h_out = g_{L-1}
 *
 * h_out may alias h_in.
 */
void m3o_scan(int64_t nb, int64_t L, int64_t H, int64_t R, int64_t P, int64_t N,
              const double *x, const double *Bbar, const double *Cbar,
              const double *dt, const double *A, const double *lam, const double *w_out,
              const double *h_in, const double *Bbar_prev, const double *x_prev,
              double *y, double *h_out)
{
    const int64_t NP = N * P;
    int64_t bh;
#pragma omp parallel for schedule(dynamic, 1)
    for (bh = 0; bh < nb * H; ++bh) {
        const int64_t ib = bh / H, h = bh % H;
        double *g = (double *)malloc(sizeof(double) * NP);
        double *u = (double *)malloc(sizeof(double) * NP);
        double *uprev = (double *)malloc(sizeof(double) * NP);
        double *Y = (double *)malloc(sizeof(double) * R * P);

        for (int64_t i = 0; i < NP; ++i)
            g[i] = h_in ? h_in[(ib * H + h) * NP + i] : 0.0;
        memset(uprev, 0, sizeof(double) * NP);
        if (Bbar_prev && x_prev) {
            for (int64_t r = 0; r < R; ++r) {
                const double *bp = Bbar_prev + ((ib * H + h) * R + r) * N;
                const double *xp = x_prev + ((ib * H + h) * R + r) * P;
                for (int64_t n = 0; n < N; ++n)
                    for (int64_t p = 0; p < P; ++p)
                        uprev[n * P + p] += bp[n] * xp[p];
            }
        }

        for (int64_t t = 0; t < L; ++t) {
            const int64_t row = (ib * L + t) * H + h;
            const double d = dt[row], lm = lam[row];
            const double alpha = exp(d * A[h]);
            const double beta = (1.0 - lm) * d * alpha;
            const double gamma = lm * d;

            memset(u, 0, sizeof(double) * NP);
            for (int64_t r = 0; r < R; ++r) {
                const double *bt = Bbar + (row * R + r) * N;
                const double *xt = x + (row * R + r) * P;
                for (int64_t n = 0; n < N; ++n)
                    for (int64_t p = 0; p < P; ++p)
                        u[n * P + p] += bt[n] * xt[p];
            }
            for (int64_t i = 0; i < NP; ++i)
                g[i] = alpha * g[i] + beta * uprev[i] + gamma * u[i];

            for (int64_t r = 0; r < R; ++r) {
                const double *ct = Cbar + (row * R + r) * N;
                for (int64_t p = 0; p < P; ++p) {
                    double acc = 0.0;
                    for (int64_t n = 0; n < N; ++n)
                        acc += ct[n] * g[n * P + p];
                    Y[r * P + p] = acc;
                }
            }
            if (w_out) {
                double *yt = y + row * P;
                for (int64_t p = 0; p < P; ++p) {
                    double acc = 0.0;
                    for (int64_t r = 0; r < R; ++r)
                        acc += w_out[(h * R + r) * P + p] * Y[r * P + p];
                    yt[p] = acc;
                }
            } else {
                double *yt = y + row * R * P;
                for (int64_t i = 0; i < R * P; ++i)
                    yt[i] = Y[i];
            }
            double *tmp = uprev;
            uprev = u;
            u = tmp;
        }
        for (int64_t i = 0; i < NP; ++i)
            h_out[(ib * H + h) * NP + i] = g[i];
        free(g);
        free(u);
        free(uprev);
        free(Y);
    }
}

/* Number of OpenMP threads the oracle runs with (reported next to its timings). */
int m3o_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads of later parallel loops (n >= 1); used to time the oracle on one host core. */
void m3o_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/*
 * Gradients of m3o_scan (the adjoint of each step of the recurrence above, taken in reverse
 * order; nothing here is chunked or reordered).  Given dy (same layout as y) and dh_out (NULL =
 * 0), returns dx, dBbar, dCbar, ddt, dlam (layouts of their inputs), dA [H] and dw_out [H, R, P]
 * (summed over the batch; dw_out only when w_out is given), dh_in [b, H, N, P], dBbar_prev and
 * dx_prev (only when both Bbar_prev and x_prev are given).  The forward states g_{-1..L-1} and
 * inputs u_{-1..L-1} are recomputed and kept for the reverse sweep.
 *
 * Per step, with alpha = exp(dt A), beta = (1 - lam) dt alpha, gamma = lam dt:
 *   dY[r]    = w_out[r] o dy  (or dy[r]);      dw_out[r] += Y[r] o dy
 *   dCbar[r] = dY[r] g_t^T;                    dg_t += sum_r Cbar[r]^T dY[r]
 *   dalpha = <dg_t, g_{t-1}>, dbeta = <dg_t, u_{t-1}>, dgamma = <dg_t, u_t>
 *   du_t = gamma dg_t + beta_{t+1} dg_{t+1};   dBbar[r] = du_t x[r],  dx[r] = du_t^T Bbar[r]
 *   dg_{t-1} = alpha dg_t
 *   ddt  = dalpha A alpha + dbeta (1 - lam) alpha (1 + dt A) + dgamma lam
 *   dlam = -dbeta dt alpha + dgamma dt
 *   dA  += dalpha dt alpha + dbeta (1 - lam) dt dt alpha
 */
void m3o_scan_backward(int64_t nb, int64_t L, int64_t H, int64_t R, int64_t P, int64_t N,
                       const double *x, const double *Bbar, const double *Cbar,
                       const double *dt, const double *A, const double *lam, const double *w_out,
                       const double *h_in, const double *Bbar_prev, const double *x_prev,
                       const double *dy, const double *dh_out,
                       double *dx, double *dBbar, double *dCbar, double *ddt, double *dA, double *dlam,
                       double *dw_out, double *dh_in, double *dBbar_prev, double *dx_prev)
{
    const int64_t NP = N * P;
    double *dA_part = (double *)calloc((size_t)(nb * H), sizeof(double));
    double *dw_part = w_out ? (double *)calloc((size_t)(nb * H * R * P), sizeof(double)) : NULL;
    int64_t bh;
#pragma omp parallel for schedule(dynamic, 1)
    for (bh = 0; bh < nb * H; ++bh) {
        const int64_t ib = bh / H, h = bh % H;
        /* forward: g[t + 1] = g_t and u[t + 1] = u_t for t = -1 .. L-1 */
        double *g = (double *)calloc((size_t)((L + 1) * NP), sizeof(double));
        double *u = (double *)calloc((size_t)((L + 1) * NP), sizeof(double));
        double *dg = (double *)malloc(sizeof(double) * NP);
        double *dU = (double *)malloc(sizeof(double) * NP);
        double *dcarry = (double *)calloc((size_t)NP, sizeof(double));
        double *dY = (double *)malloc(sizeof(double) * R * P);
        for (int64_t i = 0; i < NP; ++i)
            g[i] = h_in ? h_in[(ib * H + h) * NP + i] : 0.0;
        if (Bbar_prev && x_prev) {
            for (int64_t r = 0; r < R; ++r) {
                const double *bp = Bbar_prev + ((ib * H + h) * R + r) * N;
                const double *xp = x_prev + ((ib * H + h) * R + r) * P;
                for (int64_t n = 0; n < N; ++n)
                    for (int64_t p = 0; p < P; ++p)
                        u[n * P + p] += bp[n] * xp[p];
            }
        }
        for (int64_t t = 0; t < L; ++t) {
            const int64_t row = (ib * L + t) * H + h;
            const double d = dt[row], lm = lam[row];
            const double alpha = exp(d * A[h]), beta = (1.0 - lm) * d * alpha, gamma = lm * d;
            double *ut = u + (t + 1) * NP;
            for (int64_t r = 0; r < R; ++r) {
                const double *bt = Bbar + (row * R + r) * N;
                const double *xt = x + (row * R + r) * P;
                for (int64_t n = 0; n < N; ++n)
                    for (int64_t p = 0; p < P; ++p)
                        ut[n * P + p] += bt[n] * xt[p];
            }
            for (int64_t i = 0; i < NP; ++i)
                g[(t + 1) * NP + i] = alpha * g[t * NP + i] + beta * u[t * NP + i] + gamma * ut[i];
        }
        /* reverse sweep */
        for (int64_t i = 0; i < NP; ++i)
            dg[i] = dh_out ? dh_out[(ib * H + h) * NP + i] : 0.0;
        for (int64_t t = L - 1; t >= 0; --t) {
            const int64_t row = (ib * L + t) * H + h;
            const double d = dt[row], lm = lam[row];
            const double alpha = exp(d * A[h]), beta = (1.0 - lm) * d * alpha, gamma = lm * d;
            const double *gt = g + (t + 1) * NP, *gp = g + t * NP;
            const double *ut = u + (t + 1) * NP, *up = u + t * NP;
            /* output y_t */
            for (int64_t r = 0; r < R; ++r) {
                const double *ct = Cbar + (row * R + r) * N;
                for (int64_t p = 0; p < P; ++p) {
                    double acc = 0.0;
                    for (int64_t n = 0; n < N; ++n)
                        acc += ct[n] * gt[n * P + p];
                    if (w_out) {
                        const double dyp = dy[row * P + p];
                        dY[r * P + p] = w_out[(h * R + r) * P + p] * dyp;
                        dw_part[(bh * R + r) * P + p] += acc * dyp;
                    } else {
                        dY[r * P + p] = dy[(row * R + r) * P + p];
                    }
                }
                double *dct = dCbar + (row * R + r) * N;
                for (int64_t n = 0; n < N; ++n) {
                    double acc = 0.0;
                    for (int64_t p = 0; p < P; ++p)
                        acc += dY[r * P + p] * gt[n * P + p];
                    dct[n] = acc;
                }
                for (int64_t n = 0; n < N; ++n)
                    for (int64_t p = 0; p < P; ++p)
                        dg[n * P + p] += ct[n] * dY[r * P + p];
            }
            /* g_t = alpha g_{t-1} + beta u_{t-1} + gamma u_t */
            double dal = 0.0, dbe = 0.0, dga = 0.0;
            for (int64_t i = 0; i < NP; ++i) {
                dal += dg[i] * gp[i];
                dbe += dg[i] * up[i];
                dga += dg[i] * ut[i];
            }
            for (int64_t i = 0; i < NP; ++i) {
                dU[i] = gamma * dg[i] + dcarry[i];   /* du_t = gamma_t dg_t + beta_{t+1} dg_{t+1} */
                dcarry[i] = beta * dg[i];
                dg[i] = alpha * dg[i];
            }
            /* u_t = sum_r Bbar_t[r] x_t[r]^T */
            for (int64_t r = 0; r < R; ++r) {
                const double *bt = Bbar + (row * R + r) * N;
                const double *xt = x + (row * R + r) * P;
                double *dbt = dBbar + (row * R + r) * N;
                double *dxt = dx + (row * R + r) * P;
                for (int64_t n = 0; n < N; ++n) {
                    double acc = 0.0;
                    for (int64_t p = 0; p < P; ++p)
                        acc += dU[n * P + p] * xt[p];
                    dbt[n] = acc;
                }
                for (int64_t p = 0; p < P; ++p) {
                    double acc = 0.0;
                    for (int64_t n = 0; n < N; ++n)
                        acc += dU[n * P + p] * bt[n];
                    dxt[p] = acc;
                }
            }
            ddt[row] = dal * A[h] * alpha + dbe * (1.0 - lm) * alpha * (1.0 + d * A[h]) + dga * lm;
            dlam[row] = -dbe * d * alpha + dga * d;
            dA_part[bh] += dal * d * alpha + dbe * (1.0 - lm) * d * d * alpha;
        }
        for (int64_t i = 0; i < NP; ++i)
            dh_in[(ib * H + h) * NP + i] = dg[i];
        if (Bbar_prev && x_prev && dBbar_prev && dx_prev) {
            for (int64_t r = 0; r < R; ++r) {
                const double *bp = Bbar_prev + ((ib * H + h) * R + r) * N;
                const double *xp = x_prev + ((ib * H + h) * R + r) * P;
                double *dbp = dBbar_prev + ((ib * H + h) * R + r) * N;
                double *dxp = dx_prev + ((ib * H + h) * R + r) * P;
                for (int64_t n = 0; n < N; ++n) {
                    double acc = 0.0;
                    for (int64_t p = 0; p < P; ++p)
                        acc += dcarry[n * P + p] * xp[p];
                    dbp[n] = acc;
                }
                for (int64_t p = 0; p < P; ++p) {
                    double acc = 0.0;
                    for (int64_t n = 0; n < N; ++n)
                        acc += dcarry[n * P + p] * bp[n];
                    dxp[p] = acc;
                }
            }
        }
        free(g);
        free(u);
        free(dg);
        free(dU);
        free(dcarry);
        free(dY);
    }
    /* sums over the batch, in a fixed order */
    for (int64_t h = 0; h < H; ++h) {
        double acc = 0.0;
        for (int64_t ib = 0; ib < nb; ++ib)
            acc += dA_part[ib * H + h];
        dA[h] = acc;
    }
    if (w_out) {
        for (int64_t i = 0; i < H * R * P; ++i) {
            const int64_t h = i / (R * P), rp = i % (R * P);
            double acc = 0.0;
            for (int64_t ib = 0; ib < nb; ++ib)
                acc += dw_part[(ib * H + h) * R * P + rp];
            dw_out[i] = acc;
        }
    }
    free(dA_part);
    free(dw_part);
}

/*
 * Gradients of m3o_bcnorm_rope (the adjoint of each forward step, in reverse order).  Given
 * dBbar, dCbar (layout of Bbar) and dphi_out (NULL = 0), returns dB, dC, ddt (the rotation's
 * share only: dt also enters the scan), dtheta, dphi_in, and, summed over the batch, dnormw_B,
 * dnormw_C [H, N] (when bcnorm) and dbias_B, dbias_C [H, R, N].
 *
 * Per pair k of a rotated vector, out = R(Phi)^T vb:
 *   dvb[2k] = cos dout[2k] - sin dout[2k+1],   dvb[2k+1] = sin dout[2k] + cos dout[2k+1]
 *   dPhi[k] += dout[2k] out[2k+1] - dout[2k+1] out[2k]
 * BCNorm vn = v inv w, inv = (mean(v^2) + eps)^(-1/2):
 *   dw += dvb v inv,   dv = w inv dvb - inv^3 v / N * sum_m dvb[m] w[m] v[m]
 * Angles Phi_t = Phi_{t-1} + dt_t theta_t, reversed: S = dphi_out + sum_{i >= t} dPhi_i,
 *   dtheta_t = S dt_t,  ddt_t = <S, theta_t>,  dphi_in = S after step 0.
 */
void m3o_bcnorm_rope_backward(int64_t nb, int64_t L, int64_t H, int64_t R, int64_t N,
                              int bcnorm, double eps,
                              const double *B, const double *C, const double *dt, const double *theta,
                              const double *normw_B, const double *normw_C,
                              const double *bias_B, const double *bias_C, const double *phi_in,
                              const double *dBbar, const double *dCbar, const double *dphi_out,
                              double *dB, double *dC, double *ddt, double *dtheta, double *dphi_in,
                              double *dnormw_B, double *dnormw_C, double *dbias_B, double *dbias_C)
{
    const int64_t K = N / 2;
    double *dw_part = (double *)calloc((size_t)(nb * H * 2 * N), sizeof(double));
    double *db_part = (double *)calloc((size_t)(nb * H * 2 * R * N), sizeof(double));
    int64_t bh;
#pragma omp parallel for schedule(dynamic, 1)
    for (bh = 0; bh < nb * H; ++bh) {
        const int64_t ib = bh / H, h = bh % H;
        double *phi = (double *)malloc(sizeof(double) * (size_t)((L + 1) * K));   /* Phi_t for t = -1 .. L-1 */
        double *v = (double *)malloc(sizeof(double) * N);
        double *vb = (double *)malloc(sizeof(double) * N);
        double *dvb = (double *)malloc(sizeof(double) * N);
        double *dphi = (double *)malloc(sizeof(double) * K);
        double *S = (double *)malloc(sizeof(double) * K);
        for (int64_t k = 0; k < K; ++k)
            phi[k] = phi_in ? phi_in[(ib * H + h) * K + k] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
            const int64_t row = (ib * L + t) * H + h;
            for (int64_t k = 0; k < K; ++k)
                phi[(t + 1) * K + k] = phi[t * K + k] + dt[row] * theta[row * K + k];
        }
        for (int64_t k = 0; k < K; ++k)
            S[k] = dphi_out ? dphi_out[(ib * H + h) * K + k] : 0.0;
        for (int64_t t = L - 1; t >= 0; --t) {
            const int64_t row = (ib * L + t) * H + h;
            const double *ph = phi + (t + 1) * K;
            memset(dphi, 0, sizeof(double) * K);
            for (int which = 0; which < 2; ++which) {
                const double *src = which == 0 ? B : C;
                const double *dout_all = which == 0 ? dBbar : dCbar;
                double *dsrc_all = which == 0 ? dB : dC;
                const double *w = which == 0 ? normw_B : normw_C;
                const double *bias = which == 0 ? bias_B : bias_C;
                for (int64_t r = 0; r < R; ++r) {
                    const double *in = src + (row * R + r) * N;
                    const double *dout = dout_all + (row * R + r) * N;
                    double *dsrc = dsrc_all + (row * R + r) * N;
                    /* forward of this vector */
                    double inv = 1.0, ms = 0.0;
                    for (int64_t n = 0; n < N; ++n)
                        v[n] = in[n];
                    if (bcnorm) {
                        for (int64_t n = 0; n < N; ++n)
                            ms += v[n] * v[n];
                        ms /= (double)N;
                        inv = 1.0 / sqrt(ms + eps);
                    }
                    for (int64_t n = 0; n < N; ++n) {
                        const double wn = bcnorm ? (w ? w[h * N + n] : 1.0) * inv : 1.0;
                        vb[n] = v[n] * wn + (bias ? bias[(h * R + r) * N + n] : 0.0);
                    }
                    /* rotation */
                    for (int64_t k = 0; k < K; ++k) {
                        const double c = cos(ph[k]), s = sin(ph[k]);
                        const double o0 = c * vb[2 * k] + s * vb[2 * k + 1];
                        const double o1 = -s * vb[2 * k] + c * vb[2 * k + 1];
                        dvb[2 * k] = c * dout[2 * k] - s * dout[2 * k + 1];
                        dvb[2 * k + 1] = s * dout[2 * k] + c * dout[2 * k + 1];
                        dphi[k] += dout[2 * k] * o1 - dout[2 * k + 1] * o0;
                    }
                    /* bias, weight, RMS normalisation */
                    for (int64_t n = 0; n < N; ++n)
                        db_part[((bh * 2 + which) * R + r) * N + n] += dvb[n];
                    if (bcnorm) {
                        double sdot = 0.0;
                        for (int64_t n = 0; n < N; ++n) {
                            const double wn = w ? w[h * N + n] : 1.0;
                            dw_part[(bh * 2 + which) * N + n] += dvb[n] * v[n] * inv;
                            sdot += dvb[n] * wn * v[n];
                        }
                        for (int64_t n = 0; n < N; ++n) {
                            const double wn = w ? w[h * N + n] : 1.0;
                            dsrc[n] = wn * inv * dvb[n] - inv * inv * inv * v[n] / (double)N * sdot;
                        }
                    } else {
                        for (int64_t n = 0; n < N; ++n)
                            dsrc[n] = dvb[n];
                    }
                }
            }
            /* Phi_t = Phi_{t-1} + dt_t theta_t */
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                S[k] += dphi[k];
                dtheta[row * K + k] = S[k] * dt[row];
                acc += S[k] * theta[row * K + k];
            }
            ddt[row] = acc;
        }
        for (int64_t k = 0; k < K; ++k)
            dphi_in[(ib * H + h) * K + k] = S[k];
        free(phi);
        free(v);
        free(vb);
        free(dvb);
        free(dphi);
        free(S);
    }
    for (int64_t h = 0; h < H; ++h) {
        for (int which = 0; which < 2; ++which) {
            double *dw = which == 0 ? dnormw_B : dnormw_C;
            double *db = which == 0 ? dbias_B : dbias_C;
            for (int64_t n = 0; n < N; ++n) {
                double acc = 0.0;
                for (int64_t ib = 0; ib < nb; ++ib)
                    acc += dw_part[((ib * H + h) * 2 + which) * N + n];
                if (dw) dw[h * N + n] = bcnorm ? acc : 0.0;
            }
            for (int64_t rn = 0; rn < R * N; ++rn) {
                double acc = 0.0;
                for (int64_t ib = 0; ib < nb; ++ib)
                    acc += db_part[((ib * H + h) * 2 + which) * R * N + rn];
                if (db) db[h * R * N + rn] = acc;
            }
        }
    }
    free(dw_part);
    free(db_part);
}
