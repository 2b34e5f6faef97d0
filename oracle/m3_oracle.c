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
