/*
 * m3scan.h -- C ABI of libm3scan, the MI355X (gfx950) library for the Mamba-3 SSM layer core.
 *
 * The layer core is the exponential-trapezoidal selective recurrence with a data-dependent
 * rotation of the state and MIMO rank R:
 *
 *   h_t = alpha_t R_t h_{t-1} + beta_t R_t B_{t-1} x_{t-1}^T + gamma_t B_t x_t^T,   y_t = C_t^T h_t
 *   alpha_t = exp(dt_t A),  beta_t = (1 - lambda_t) dt_t exp(dt_t A),  gamma_t = lambda_t dt_t
 *
 * (aipaper.cc summary of "Mamba-3: Improved Sequence Modeling using State Space Principles",
 * section 4.1 Proposition 1 for the recurrence, section 4.2 Propositions 2-3 for the rotation,
 * section 4.3 for MIMO).  The rotation R_t is block-diagonal with 2x2 blocks of angle
 * dt_t * theta_t[k] on the pairs (2k, 2k+1) (metaphor-xennon SSM comparison, section 2.2).  As
 * Proposition 3 states, it is applied as a cumulative rotation of B and C, so the state
 * recurrence itself stays real with a scalar decay:
 *
 *   m3_bcnorm_rope   BCNorm + bias + cumulative rotation:  Bbar_t = R(Phi_t)^T Btilde_t, same for C
 *   m3_prefill       chunked scan over a whole sequence (structured-mask matrix form)
 *   m3_layer_prefill the two above in one pass (rotation applied while staging each chunk)
 *   m3_decode_step   one new token for a batch of resident states
 *   m3_layer_decode_step  the rotation and one decode step in one launch
 *   m3_layer_backward     gradients of m3_layer_prefill (with m3_layer_chunk_states, the
 *                         forward pass that saves what the backward pass reads)
 *
 * Frame of the state.  The state the library keeps, returns and accepts is the rotated frame
 * g_t = R(Phi_t)^T h_t.  Together with the angle Phi_t (returned by m3_bcnorm_rope) it fully
 * determines h_t = R(Phi_t) g_t.  In this frame the previous-input term uses the rotated
 * previous input: g_t = alpha_t g_{t-1} + beta_t Bbar_{t-1}^T x_{t-1} + gamma_t Bbar_t^T x_t.
 *
 * Conventions for every entry point:
 *  - Memory.  All tensor pointers are device pointers, owned by the caller, dense row-major in
 *    the layouts stated below, and must stay valid until the work queued on `stream` has run.
 *    The library never allocates in these calls; a call that needs scratch memory takes a
 *    caller-provided workspace whose size the matching *_workspace_bytes function returns.
 *  - Alignment.  Pointers to x, B, C, Bbar, Cbar, theta, y, h, h_in, h_out must be 16-byte
 *    aligned; every other pointer must be aligned to its element size.
 *  - dtype.  "io" tensors have the element type dims->io (fp32 or bf16, bf16 stored as its
 *    16-bit pattern).  The state h, the angle phi and every per-head constant are fp32.
 *  - Asynchrony.  Every call only validates its arguments and enqueues kernels on `stream`.
 *    M3_OK means "validated and enqueued"; faults during execution surface at the caller's
 *    next synchronisation.  Calls on one stream run in order.
 *  - Errors.  A non-OK status leaves every output untouched and sets a message readable with
 *    m3_last_error() on the calling thread.  Numeric values live in device memory and are not
 *    validated.  The kernels assume that the decay never grows, i.e. dt * A <= 0 at every step
 *    (dt > 0 after softplus and A <= 0, as the method defines them): the chunked kernels clamp
 *    the exponent of each decay factor exp(A * sum of dt) at 0, so with dt * A > 0 their results
 *    are not those of the recurrence (no error is reported).  NaN and Inf propagate.
 *  - Device.  The current HIP device must be a gfx950 GPU, else M3_E_NODEVICE.
 *  - Threads.  Calls from several host threads are safe; calls that write the same buffers
 *    must be ordered by the caller.
 */
#ifndef M3SCAN_H
#define M3SCAN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    M3_OK = 0,
    M3_E_NULL = 1,        /* a required pointer is NULL                                    */
    M3_E_DIMS = 2,        /* a size is negative, odd where it must be even, or inconsistent */
    M3_E_ALIGN = 3,       /* a pointer violates the alignment rule above                    */
    M3_E_DTYPE = 4,       /* dims->io is not M3_F32 or M3_BF16                             */
    M3_E_UNSUPPORTED = 5, /* valid, but outside the shapes the library has kernels for     */
    M3_E_NODEVICE = 6,    /* no current HIP device, or it is not gfx950                     */
    M3_E_LAUNCH = 7,      /* the HIP runtime refused a kernel launch                        */
    M3_E_WORKSPACE = 8,   /* workspace NULL or smaller than *_workspace_bytes returned      */
    M3_E_ALIAS = 9        /* outputs overlap inputs in a way the call does not allow        */
} m3_status;

typedef enum { M3_F32 = 0, M3_BF16 = 1 } m3_dtype;

/* dims->flags */
#define M3_BCNORM 1u /* apply the RMS normalisation in m3_bcnorm_rope (else only bias + rotation) */

typedef struct {
    int64_t batch;   /* b                                                                    */
    int64_t seqlen;  /* L: time steps in this call (1 for m3_decode_step)                    */
    int64_t nheads;  /* H                                                                    */
    int64_t headdim; /* P: width of x and y per rank                                         */
    int64_t dstate;  /* N: state size per head dim (even: N/2 rotation pairs)                */
    int64_t rank;    /* R: MIMO rank, 1 = SISO                                                */
    int64_t chunk;   /* Q: time steps per chunk in m3_prefill; 0 = library default (64/R)    */
    int32_t io;      /* m3_dtype of the io tensors                                            */
    uint32_t flags;  /* M3_BCNORM                                                             */
    float eps;       /* added to the mean square in BCNorm (e.g. 1e-5)                        */
    int64_t ngroups; /* G: raw B and C shared by groups of H / G heads; 0 = one per head (G = H) */
} m3_dims;

/*
 * Head groups (dims->ngroups).  The calls that take the raw projections B and C
 * (m3_bcnorm_rope, m3_layer_prefill, m3_layer_prefill_varlen, m3_layer_decode_step,
 * m3_layer_chunk_states, m3_layer_backward) accept them with G <= H head slots instead of H: head
 * h reads slot h / (H / G), so the H / G consecutive heads of a group share one B and one C row.
 * Each head still applies its own BCNorm weight, bias and rotation, and everything else (x, dt,
 * theta, lambda, the state, the outputs, the rotated Bbar and Cbar) stays per head: the result
 * is that of the same call with each group's rows repeated for every head of the group.  The
 * pages define B and C per head; sharing them across heads is a layout option of this library
 * that cuts the bytes of B and C read by H / G.  G must divide H (else M3_E_DIMS); 0 means H.
 * m3_prefill and m3_decode_step take rotated, per-head Bbar and Cbar and require G = H (or 0).
 * The layouts below write B and C as [.., H, R, N]; with groups read [.., G, R, N].  In
 * m3_layer_backward the gradients dB and dC have the grouped layout: the sums over each group's
 * heads.
 */

/*
 * m3_bcnorm_rope -- BCNorm, head bias and cumulative rotation of B and C.
 *
 * Defined by: papernotes.org summary of Mamba-3, key design 4 (RMSNorm on the B and C
 * projections, "BCNorm", and a learnable head-specific B/C bias); aipaper.cc summary, section
 * 4.2 Proposition 3 (B and C multiplied by the cumulative product of R_i^T, i = 0..t);
 * metaphor-xennon section 2.2 (R_t has angle dt_t * theta_t).
 *
 * For every (b, t, h, r) and each of B and C (vector v of N entries):
 *   vt = v / sqrt(mean(v^2) + eps) * normw[h, :]   if dims->flags & M3_BCNORM, else vt = v
 *   vt = vt + bias[h, r, :]                         if bias is not NULL
 *   Phi_t[k] = Phi_in[k] + sum_{i<=t} dt_i theta_i[k]       (k < N/2; the current step included)
 *   out[2k] = cos(Phi_t[k]) vt[2k] + sin(Phi_t[k]) vt[2k+1]
 *   out[2k+1] = -sin(Phi_t[k]) vt[2k] + cos(Phi_t[k]) vt[2k+1]
 *
 * Arguments (shapes use the dims fields; "io" = dims->io):
 *   B, C        [b, L, H, R, N] io   raw projections                                  required
 *   dt          [b, L, H] io         step size (positive; already passed through softplus) required
 *   theta       [b, L, H, N/2] io    rotation rate per pair                            required
 *   normw_B/C   [H, N] f32           BCNorm weight; NULL = 1                            optional
 *   bias_B/C    [H, R, N] f32        head bias; NULL = 0                                optional
 *   phi_in      [b, H, N/2] f32      angle carried in from earlier steps; NULL = 0      optional
 *   Bbar, Cbar  [b, L, H, R, N] io   rotated outputs                                   required
 *   phi_out     [b, H, N/2] f32      angle after the last step, reduced to [-pi, pi]    required
 *   workspace   device scratch of m3_bcnorm_rope_workspace_bytes(dims) bytes (may be NULL
 *               when that is 0)
 * phi_out may be the same buffer as phi_in (decode carries the angle in place); no other
 * output may overlap an input.  The library has kernels for N in {16, 32, 64, 128, 256} and
 * 1 <= R <= 64; other shapes return M3_E_UNSUPPORTED.
 */
m3_status m3_bcnorm_rope(const m3_dims* dims, const void* B, const void* C, const void* dt,
                         const void* theta, const float* normw_B, const float* normw_C,
                         const float* bias_B, const float* bias_C, const float* phi_in,
                         void* Bbar, void* Cbar, float* phi_out, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace m3_bcnorm_rope needs for these dims (0 for short sequences). */
size_t m3_bcnorm_rope_workspace_bytes(const m3_dims* dims);

/*
 * m3_prefill -- the exponential-trapezoidal recurrence over a whole sequence, in chunks.
 *
 * Defined by: aipaper.cc summary, section 4.1 Proposition 1 (recurrence and alpha, beta,
 * gamma), section 4.3 (MIMO update H_t = a_t H_{t-1} + B_t X_t^T); papernotes.org, key design 1
 * (the structured mask of the recurrence is a 1-semiseparable decay times a 2-band matrix and
 * still allows chunked matrix products).  Computed exactly (up to rounding) as, per (b, h):
 *
 *   g_{-1} = h_in,   u_{-1} = sum_r Bbar_prev[r]^T x_prev[r]
 *   u_t = sum_r Bbar_t[r]^T x_t[r]                                   (N x P)
 *   g_t = alpha_t g_{t-1} + beta_t u_{t-1} + gamma_t u_t,   alpha_t = exp(dt_t A[h])
 *   Y_t[r] = Cbar_t[r] g_t                                           (R x P)
 *   y_t[p] = sum_r w_out[h, r, p] Y_t[r, p] if w_out is given, else y_t = Y_t
 *
 * Arguments:
 *   x           [b, L, H, R, P] io    inputs                                          required
 *   Bbar, Cbar  [b, L, H, R, N] io    rotated B, C (from m3_bcnorm_rope)                required
 *   dt, lam     [b, L, H] io          step size and trapezoid weight lambda             required
 *   A           [H] f32               decay rate per head (<= 0)                        required
 *   w_out       [H, R, P] f32         output mixing over ranks; NULL = no mixing         optional
 *   h_in        [b, H, N, P] f32      state carried in; NULL = 0                         optional
 *   Bbar_prev   [b, H, R, N] io       rotated Bbar of the step before this call; NULL = 0 optional
 *   x_prev      [b, H, R, P] io       x of the step before this call; NULL = 0           optional
 *   y           [b, L, H, P] io if w_out, else [b, L, H, R, P] io                      required
 *   h_out       [b, H, N, P] f32      final state g_{L-1} (may be the same buffer as h_in) required
 *   Bbar_last   [b, H, R, N] io       copy of Bbar at step L-1 (for a following decode)  optional
 *   x_last      [b, H, R, P] io       copy of x at step L-1                              optional
 *   workspace   m3_prefill_workspace_bytes(dims) bytes, 16-byte aligned, or NULL        optional
 * With a workspace, a call with few (b, h) pairs (fewer than two per compute unit) and long
 * sequences splits each sequence into segments of a multiple of 512 steps that run in parallel:
 * pass 1 runs every segment in full, y included, segment 0 from the call's carry and the others
 * from a zero carry; a small kernel chains the segments' end states into true ones and h_out
 * (the recurrence is linear in its carry: the end state of segment s is its own end state plus
 * the incoming state decayed by exp(A sum of dt over the segment)); pass 2 reruns the first steps
 * of segments 1, 2, ... from their true carries, in whole chunks, until the carry's decay from
 * the segment's start, exp(A sum of dt), has stayed below 2^-48 (a segment whose carry never
 * decays that far is rerun whole).  The y left from the zero-carry run past that point lacks only
 * the carry's share, below 2^-48 of the carried state's contribution (2^-24 below float
 * rounding); the other results are those of one pass up to rounding order.
 * m3_prefill_workspace_bytes returns 0 when no split would be used;
 * with NULL the call always runs one pass per sequence.  A non-NULL workspace smaller than the
 * returned size is M3_E_WORKSPACE; one that overlaps any argument is M3_E_ALIAS.
 * Any L >= 0 is accepted (L = 0 copies the carried state to the outputs), as long as one
 * sequence's rows of a tensor span less than 2^31 bytes: (L + 3 chunk) * H * R * max(N, P) * io
 * size < 2^31, else M3_E_DIMS (the kernel addresses a sequence with 32-bit offsets; a longer
 * sequence is split into calls, which the carried state and last step make exact).
 * dims->chunk * R must be 16, 32, 48 or 64.  The library has kernels for (N, P) in {(16,16),
 * (64,64), (128,64)} and R in {1, 2, 4, 8, 16} dividing 16; other shapes return
 * M3_E_UNSUPPORTED.
 */
m3_status m3_prefill(const m3_dims* dims, const void* x, const void* Bbar, const void* Cbar,
                     const void* dt, const float* A, const void* lam, const float* w_out,
                     const float* h_in, const void* Bbar_prev, const void* x_prev, void* y,
                     float* h_out, void* Bbar_last, void* x_last, void* workspace,
                     size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace m3_prefill uses for these dims on the current device (0: it does
 * not split them).  The split depends on the device's compute-unit count. */
size_t m3_prefill_workspace_bytes(const m3_dims* dims);

/*
 * m3_layer_prefill -- m3_bcnorm_rope followed by m3_prefill, in one pass over the sequence.
 *
 * Defined by: the two calls it stands for (see them above).  papernotes.org, key design 4, notes
 * that BCNorm, the bias and the rotation only change the projections the scan consumes; here
 * they are applied while each chunk of raw B and C is staged on chip, so the rotated Bbar and
 * Cbar never travel through device memory.  The results are those of
 *
 *   m3_bcnorm_rope(dims, B, C, dt, theta, normw_B, normw_C, bias_B, bias_C, phi_in,
 *                  Bbar, Cbar, phi_out)
 *   m3_prefill(dims, x, Bbar, Cbar, dt, A, lam, w_out, h_in, Bbar_prev, x_prev,
 *              y, h_out, Bbar_last, x_last)
 *
 * up to rounding order (the rotated values are rounded to the io type at the same point).
 * Arguments are those of the two calls, with the same shapes, optionality and meaning; Bbar_last
 * receives the rotated Bbar of the last step, as m3_prefill would return it.  dims->chunk = 0
 * picks 32 / R steps per chunk.  h_out may be the h_in buffer and phi_out the phi_in buffer;
 * no other output may overlap an input.  The library has kernels for (N, P) in {(16, 16),
 * (64, 64), (128, 64)}, R in {1, 2, 4, 8, 16} and chunk * R in {16, 32, 64};
 * other shapes return M3_E_UNSUPPORTED.  The sequence length limit of m3_prefill applies (with
 * the angle carried as phi_in / phi_out when a sequence is split).  The workspace (optional,
 * m3_layer_prefill_workspace_bytes(dims) bytes, 16-byte aligned) enables the sequence split of
 * m3_prefill, for the same dims and with the same passes.  The later segments' first pass also
 * starts from angle zero (y depends only on the differences of the angles inside a segment when
 * the carried state is zero); the chaining adds up the segments' angle sums into true start
 * angles and turns the end states and last Bbar rows by them (the call's Bbar_last is thereby
 * rounded to the io type twice).  Workspace errors as m3_prefill.
 */
m3_status m3_layer_prefill(const m3_dims* dims, const void* x, const void* B, const void* C,
                           const void* dt, const void* theta, const float* normw_B,
                           const float* normw_C, const float* bias_B, const float* bias_C,
                           const float* A, const void* lam, const float* w_out,
                           const float* phi_in, const float* h_in, const void* Bbar_prev,
                           const void* x_prev, void* y, float* h_out, float* phi_out,
                           void* Bbar_last, void* x_last, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace m3_layer_prefill uses for these dims on the current device (0: it
 * does not split them). */
size_t m3_layer_prefill_workspace_bytes(const m3_dims* dims);

/*
 * m3_decode_step -- one new token for each of b * H resident states, updated in place.
 *
 * Defined by: aipaper.cc summary, section 4.1 Proposition 1 and section 4.3 (the same
 * recurrence as m3_prefill with L = 1); papernotes.org key design 3 (decode is bound by the
 * memory traffic of the state; MIMO adds work per byte).  Per (b, h):
 *
 *   h    <- alpha h + beta Bbar_prev^T x_prev + gamma Bbar^T x      (rank-2R update, fp32)
 *   Y[r] =  Cbar[r] h                                               (after the update)
 *   y[p] =  sum_r w_out[h, r, p] Y[r, p] if w_out, else y = Y
 *
 * Arguments (dims->seqlen must be 1):
 *   h           [b, H, N, P] f32      state, read and overwritten                       required
 *   Bbar_prev   [b, H, R, N] io       rotated B of the previous token                   required
 *   x_prev      [b, H, R, P] io       x of the previous token                           required
 *   x           [b, H, R, P] io       x of this token                                   required
 *   Bbar, Cbar  [b, H, R, N] io       rotated B, C of this token (m3_bcnorm_rope, L = 1) required
 *   dt, lam     [b, H] io                                                               required
 *   A           [H] f32                                                                 required
 *   w_out       [H, R, P] f32 or NULL                                                   optional
 *   y           [b, H, P] io if w_out, else [b, H, R, P] io                            required
 * The caller keeps (Bbar, x) of this token as (Bbar_prev, x_prev) of the next one, e.g. by
 * swapping buffers; nothing is copied.  P must be a power of two with 4 <= P <= 256, N <= 256,
 * R <= 8.
 */
m3_status m3_decode_step(const m3_dims* dims, float* h, const void* Bbar_prev,
                         const void* x_prev, const void* x, const void* Bbar, const void* Cbar,
                         const void* dt, const float* A, const void* lam, const float* w_out,
                         void* y, hipStream_t stream);

/* Message describing the last non-OK status returned on the calling thread ("" if none). */
const char* m3_last_error(void);

/* Library version string. */
const char* m3_version(void);

/*
 * m3_layer_prefill_varlen -- m3_layer_prefill over a packed batch of sequences of different
 * lengths (serving: prompts of mixed lengths without padding).
 *
 * Defined by: m3_layer_prefill, applied to each sequence separately.  Sequence s (s < b =
 * dims->batch) is tokens cu_seqlens[s] .. cu_seqlens[s+1] - 1 of T = dims->seqlen packed tokens:
 *   cu_seqlens  [b + 1] int32 (device), cu_seqlens[0] = 0, non-decreasing, cu_seqlens[b] = T
 *   x [T, H, R, P], B, C [T, H, R, N], dt, lam [T, H], theta [T, H, N/2] io; y [T, H, P] (with
 *   w_out) or [T, H, R, P]
 *   per-sequence tensors as in m3_layer_prefill: h_in, h_out [b, H, N, P], phi_in, phi_out
 *   [b, H, N/2], Bbar_prev, Bbar_last [b, H, R, N], x_prev, x_last [b, H, R, P]
 * An empty sequence passes its carry through (h_out = h_in, phi_out = phi_in reduced, Bbar_last
 * = Bbar_prev, x_last = x_prev).  cu_seqlens is read on the device; offsets outside [0, T] are
 * clamped into it, so no access leaves the packed arrays.  Shapes, aliasing and errors as
 * m3_layer_prefill (cu_seqlens NULL: M3_E_NULL).
 */
m3_status m3_layer_prefill_varlen(const m3_dims* dims, const int32_t* cu_seqlens, const void* x,
                                  const void* B, const void* C, const void* dt, const void* theta,
                                  const float* normw_B, const float* normw_C, const float* bias_B,
                                  const float* bias_C, const float* A, const void* lam,
                                  const float* w_out, const float* phi_in, const float* h_in,
                                  const void* Bbar_prev, const void* x_prev, void* y, float* h_out,
                                  float* phi_out, void* Bbar_last, void* x_last,
                                  hipStream_t stream);

/*
 * m3_layer_decode_step -- m3_bcnorm_rope (L = 1) followed by m3_decode_step, in one launch.
 *
 * Defined by: the two calls it stands for (see them above); papernotes.org, key design 4 (the
 * normalisation, bias and rotation only change what the recurrence consumes).  The token's raw B
 * and C are normalised, biased and rotated by Phi + dt * theta inside the decode kernel; the
 * results are those of
 *
 *   m3_bcnorm_rope(dims, B, C, dt, theta, normw_B, normw_C, bias_B, bias_C, phi,
 *                  Bbar_out, Cbar, phi)
 *   m3_decode_step(dims, h, Bbar_prev, x_prev, x, Bbar_out, Cbar, dt, A, lam, w_out, y)
 *
 * up to rounding order.  Arguments (dims->seqlen must be 1):
 *   h           [b, H, N, P] f32     state, updated in place                            required
 *   phi         [b, H, N/2] f32      carried angle, advanced in place                   required
 *   Bbar_prev, x_prev                as in m3_decode_step (the previous token's rotated B and x)
 *   x           [b, H, R, P] io      the token's input                                  required
 *   B, C        [b, H, R, N] io      the token's raw projections                        required
 *   dt, lam     [b, H] io; theta [b, H, N/2] io; A, normw_*, bias_*, w_out as before
 *   y           [b, H, P] io (with w_out) or [b, H, R, P]                               required
 *   Bbar_out    [b, H, R, N] io      the token's rotated B: the next step's Bbar_prev   required
 * The caller swaps the Bbar_prev / Bbar_out buffers (and passes x as the next x_prev) between
 * steps.  No output may overlap an input or another output.  Shapes as m3_decode_step.
 */
m3_status m3_layer_decode_step(const m3_dims* dims, float* h, float* phi, const void* Bbar_prev,
                               const void* x_prev, const void* x, const void* B, const void* C,
                               const void* dt, const void* theta, const float* normw_B,
                               const float* normw_C, const float* bias_B, const float* bias_C,
                               const float* A, const void* lam, const float* w_out, void* y,
                               void* Bbar_out, hipStream_t stream);

/*
 * m3_layer_backward_chunk -- time steps per chunk of the backward pass for these dims (the
 * chunk of the states m3_layer_chunk_states saves), or 0 when no backward kernel covers them.
 * Chunks are 64 rows (step, rank) for bf16 io and 32 rows for fp32 io at P = 64, 16 rows at
 * P = 16; steps per chunk = rows / R.
 */
int64_t m3_layer_backward_chunk(const m3_dims* dims);

/*
 * m3_layer_chunk_states -- the state and angle at the entry of every backward chunk.
 *
 * Defined by: the recurrence of m3_prefill on the rotated B of m3_bcnorm_rope (aipaper.cc
 * summary, section 4.1 Proposition 1, section 4.2 Proposition 3, section 4.3), with the chunk
 * Q = m3_layer_backward_chunk(dims).  For chunk c (steps cQ .. cQ + Q - 1), per (b, h):
 *
 *   states[b, h, c] = (G_{cQ-1})^T,  G_{t} = g_t + c_{t+1} Bbar_t^T x_t  (the shifted state)
 *   phis[b, h, c]   = Phi_{cQ-1} (reduced to [-pi, pi]),  Phi_{-1} = phi_in
 *
 * where c_{t} = (1 - lambda_t) dt_t, g_t is m3_prefill's state (g_{-1} = h_in) and the shifted
 * state is the one the chunked form carries between chunks (its G_{-1} = h_in + c_0 u_{-1}).
 * Arguments are those of m3_layer_prefill with the same meaning (only the B side is used), plus:
 *   states  [b, H, nchunk, P, N] io   entry states, transposed              required
 *   phis    [b, H, nchunk, N/2] f32   entry angles                         required
 * with nchunk = ceil(L / Q).  Neither output may overlap an input or the other.  Shapes: (N, P)
 * in {(16,16), (64,64), (128,64)}, R in {1, 2, 4}; dense batches only.  m3_layer_backward calls
 * this itself; it is exported for checkpointing and for tests.
 */
m3_status m3_layer_chunk_states(const m3_dims* dims, const void* x, const void* B, const void* dt,
                                const void* theta, const float* normw_B, const float* bias_B,
                                const float* A, const void* lam, const float* phi_in,
                                const float* h_in, const void* Bbar_prev, const void* x_prev,
                                void* states, float* phis, hipStream_t stream);

/* Bytes of device workspace m3_layer_backward needs for these dims (0 when unsupported). */
size_t m3_layer_backward_workspace_bytes(const m3_dims* dims);

/*
 * m3_layer_backward -- gradients of m3_layer_prefill with respect to all of its inputs.
 *
 * Defined by: the derivative of the computation m3_layer_prefill defines (the pages give the
 * forward only: aipaper.cc summary, sections 4.1-4.3; papernotes.org, key design 4; the
 * cumulative angle of section 4.2 Proposition 3).  Given the cotangents dy (of y), dh_out (of
 * h_out) and dphi_out (of phi_out), it returns, up to rounding, the exact gradient of
 *   <dy, y> + <dh_out, h_out> + <dphi_out, phi_out>
 * with respect to every input, computed by the reverse chunked pass (the gradient of each
 * chunk's matrix products, the state cotangent carried from the last chunk to the first, the
 * rotation and BCNorm undone per row, the angle cotangent summed from the end).  Arguments:
 *   x .. x_prev   the forward inputs of m3_layer_prefill, same shapes and optionality
 *   dy            [b, L, H, P] io with w_out, else [b, L, H, R, P] io             required
 *   dh_out        [b, H, N, P] f32; NULL = 0                                      optional
 *   dphi_out      [b, H, N/2] f32; NULL = 0                                       optional
 *   dx            [b, L, H, R, P] io                                              required
 *   dB, dC        [b, L, H, R, N] io   (of the raw B and C)                       required
 *   ddt, dlam     [b, L, H] io   (ddt includes the angle's share)                 required
 *   dtheta        [b, L, H, N/2] io                                               required
 *   dA            [H] f32   summed over the batch                                 required
 *   dnormw_B, dnormw_C [H, N] f32   summed over the batch; 0 without M3_BCNORM   optional
 *   dbias_B, dbias_C   [H, R, N] f32 summed over the batch                        optional
 *   dw_out        [H, R, P] f32 summed over the batch (only with w_out)           optional
 *   dphi_in       [b, H, N/2] f32                                                 required
 *   dh_in         [b, H, N, P] f32                                                required
 *   dBbar_prev    [b, H, R, N] io; 0 when Bbar_prev or x_prev is NULL             optional
 *   dx_prev       [b, H, R, P] io; 0 when Bbar_prev or x_prev is NULL             optional
 *   workspace     m3_layer_backward_workspace_bytes(dims) bytes, 16-byte aligned  required
 * Gradients of per-head parameters are reduced over the batch in a fixed order (results do not
 * depend on scheduling).  Outputs may not overlap inputs, the workspace or each other.  dims->chunk
 * must be 0 or m3_layer_backward_chunk(dims); dense batches only.  Shapes: (N, P) in {(16,16),
 * (64,64), (128,64)}, R in {1, 2, 4}; others return M3_E_UNSUPPORTED.
 */
m3_status m3_layer_backward(const m3_dims* dims, const void* x, const void* B, const void* C,
                            const void* dt, const void* theta, const float* normw_B,
                            const float* normw_C, const float* bias_B, const float* bias_C,
                            const float* A, const void* lam, const float* w_out,
                            const float* phi_in, const float* h_in, const void* Bbar_prev,
                            const void* x_prev, const void* dy, const float* dh_out,
                            const float* dphi_out, void* dx, void* dB, void* dC, void* ddt,
                            void* dtheta, float* dA, void* dlam, float* dnormw_B, float* dnormw_C,
                            float* dbias_B, float* dbias_C, float* dw_out, float* dphi_in,
                            float* dh_in, void* dBbar_prev, void* dx_prev, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/*
 * m3_layer_prefill_noalloc -- m3_layer_prefill for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * For: those callers.  Arguments, results and errors are those of m3_layer_prefill without the
 * workspace: where m3_layer_prefill would split few long sequences into segments (when
 * m3_layer_prefill_workspace_bytes(dims) > 0), this call uses a device array the library holds
 * instead of a caller workspace.  The call allocates nothing (no hipMalloc, hipFree or allocating
 * library routine).
 *   - Limit.  The array holds M3_NOALLOC_SCRATCH_BYTES (32 MiB) per GPU, enough for the split of
 *     b = 1, L = 16384, H = 64, R = 4, N = 128, P = 64 (about 18 MB).  Dims whose split needs more
 *     return M3_E_WORKSPACE (call m3_layer_prefill with a workspace instead).  Dims that do not
 *     split use no scratch.
 *   - Sharing.  Every call on one GPU uses that GPU's one array, whose contents persist from
 *     call to call (each call writes every scratch element before reading it; nothing needs to
 *     start at zero).  Calls that may run at the same time on one GPU (on different streams, or
 *     from several host threads without ordering) race on the array: the caller must order them.
 *   - Memory.  Each GPU the library runs on holds its copy of the array from the library's load
 *     until the process ends.
 */
#define M3_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
m3_status m3_layer_prefill_noalloc(const m3_dims* dims, const void* x, const void* B, const void* C,
                                   const void* dt, const void* theta, const float* normw_B,
                                   const float* normw_C, const float* bias_B, const float* bias_C,
                                   const float* A, const void* lam, const float* w_out,
                                   const float* phi_in, const float* h_in, const void* Bbar_prev,
                                   const void* x_prev, void* y, float* h_out, float* phi_out,
                                   void* Bbar_last, void* x_last, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* M3SCAN_H */
