// prefill.hip -- m3_prefill: the exponential-trapezoidal recurrence over a sequence, in chunks.
//
// Method.  aipaper.cc summary of Mamba-3, section 4.1 Proposition 1:
//   g_t = alpha_t g_{t-1} + beta_t u_{t-1} + gamma_t u_t,  u_t = Bbar_t^T x_t,  Y_t = Cbar_t g_t,
// with the MIMO rank-R product of section 4.3.  papernotes.org, key design 1: the matrix of this
// recurrence is a 1-semiseparable decay times a 2-band (trapezoid) matrix, so it still runs as
// chunked matrix products (the SSD form Y = (L o C B^T) X, metaphor-xennon section 1.3).
//
// Shifted state.  With c_t = (1 - lambda_t) dt_t (so beta_t = c_t alpha_t) define
// G_t = g_t + c_{t+1} u_t.  Then G_t = alpha_t G_{t-1} + mu_t u_t with mu_t = gamma_t + c_{t+1},
// and y_t = Cbar_t G_t - c_{t+1} Cbar_t u_t.  Inside a chunk starting at t0, with
// l_t = sum_{t0<=i<=t} dt_i A (so exp(l_t - l_s) is the decay from s to t):
//   Y_t = sum_{s<t} exp(l_t - l_s) mu_s Cbar_t u_s + gamma_t Cbar_t u_t + exp(l_t) Cbar_t G_{t0-1}
// i.e. the mask entry is exp(l_t - l_s) mu_s below the diagonal and gamma_t on it (the
// "decay x 2-band" matrix), and the carried state is G.  The chunk then passes on
//   G_end = exp(l_end) G_{t0-1} + sum_s exp(l_end - l_s) mu_s u_s.
// At the call's last step c_L is taken as 0, so the returned G is the true state g_{L-1}; at the
// call's first step G_{-1} = h_in + c_0 Bbar_prev^T x_prev.  The trapezoid's link across chunk
// boundaries is therefore one scalar (dt, lambda of the next step), not a B/x halo.
//
// Mapping on gfx950.  One workgroup per (b, h) walks the chunks in order and keeps the N x P fp32
// state in MFMA accumulator registers, so chunk states never travel through HBM.  A chunk holds
// QR = Q * R rows (t, r).  Wave w owns the 16 columns [16w, 16w + 16) of P.
//   1. S^T = Bbar Cbar^T (QR x QR, K = N) on MFMA, only the causal 16x16 tiles, shared out among
//      the waves; the mask is applied in registers and M = L o S goes to LDS.
//   2. Y^T (own 16 columns x QR) = state^T Cbar^T * exp(l) + X^T M^T: the state is the A operand
//      straight from the accumulator registers (an MFMA D tile of S[n][p] is an A tile of S^T).
//   3. state = exp(l_end) state + (Bbar^T)(w o X), w_s = exp(l_end - l_s) mu_s.
// The chunk's Bbar, Cbar and x tiles sit in LDS exactly as they are laid out in memory (rows
// (t, r)), written with 16-byte stores.  Operands that need the other orientation (X^T and
// Bbar^T, contracted over the rows) are read with gfx950's transposing LDS read
// (ds_read_b64_tr_b16): in each group of 16 lanes, lane j points at 4 consecutive elements of
// row k0 + j/4, columns c0 + 4 (j % 4); lane i then receives rows k0..k0+3 of column c0 + i.
// The next chunk's tiles are loaded into registers while the current chunk computes.
//
// Operands: bf16 inputs run v_mfma_f32_16x16x16_bf16 (fp32 accumulate); fp32 inputs run
// v_mfma_f32_16x16x4_f32 four times per 16-wide K block.  In every product the same lane -> K
// slot assignment is used for both operands, which is all the result depends on.
#include "m3_device.h"
#include "m3_launch.h"

namespace m3 {

namespace {

typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
typedef __attribute__((address_space(3))) char lds_char;

template <typename T> struct Mma;

template <> struct Mma<bf16> {
    typedef shortx4 frag;
    static constexpr int PAD = 16;  // elements of padding per LDS row (32 bytes)
    // lane gets p[0..3] (4 consecutive elements along K)
    static __device__ __forceinline__ frag ldk(const bf16* p) { return *(const shortx4*)p; }
    // transposed read: `row` points at tile[k0 + 4g][c0] for this lane's group g; lane (l16, g)
    // receives tile[k0 + 4g + m][c0 + l16], m = 0..3
    static __device__ __forceinline__ frag ldt(const bf16* row, int ld, int l16) {
        const bf16* p = row + (l16 >> 2) * ld + 4 * (l16 & 3);
        return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(lds_char*)p);
    }
    static __device__ __forceinline__ floatx4 mma(frag a, frag b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
    }
    // two 16-wide K blocks.  They could run as one v_mfma_f32_16x16x32_bf16 (its K slots pair up
    // symmetrically for A and B), but with this toolchain a VALU write that follows that
    // instruction can clobber its A/B registers while later passes still read them, so the pair
    // runs as two 16x16x16 instructions.
    static __device__ __forceinline__ floatx4 mma2(frag a0, frag a1, frag b0, frag b1, floatx4 c) {
        return mma(a1, b1, mma(a0, b0, c));
    }
    static __device__ __forceinline__ frag pack(floatx4 v) {
        const uint2 u = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        return __builtin_bit_cast(frag, u);
    }
    static __device__ __forceinline__ floatx4 unpack(frag f) {
        floatx4 v;
        v[0] = __uint_as_float((uint32_t)(uint16_t)f[0] << 16);
        v[1] = __uint_as_float((uint32_t)(uint16_t)f[1] << 16);
        v[2] = __uint_as_float((uint32_t)(uint16_t)f[2] << 16);
        v[3] = __uint_as_float((uint32_t)(uint16_t)f[3] << 16);
        return v;
    }
    static __device__ __forceinline__ void st(bf16* p, frag f) { *(shortx4*)p = f; }
};

template <> struct Mma<float> {
    typedef floatx4 frag;
    static constexpr int PAD = 4;
    static __device__ __forceinline__ frag ldk(const float* p) { return *(const floatx4*)p; }
    static __device__ __forceinline__ frag ldt(const float* row, int ld, int l16) {
        frag f;
        f[0] = row[l16];
        f[1] = row[ld + l16];
        f[2] = row[2 * ld + l16];
        f[3] = row[3 * ld + l16];
        return f;
    }
    static __device__ __forceinline__ floatx4 mma(frag a, frag b, floatx4 c) {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
        return c;
    }
    static __device__ __forceinline__ floatx4 mma2(frag a0, frag a1, frag b0, frag b1, floatx4 c) {
        return mma(a1, b1, mma(a0, b0, c));
    }
    static __device__ __forceinline__ frag pack(floatx4 v) { return v; }
    static __device__ __forceinline__ floatx4 unpack(frag f) { return f; }
    static __device__ __forceinline__ void st(float* p, frag f) { *(floatx4*)p = f; }
};

// acc += sum over K blocks k < NK of A_k B_k, two blocks per instruction where possible.
// fa(k), fb(k) return the fragments of 16-wide K block k.
template <typename MM, int NK, typename FA, typename FB>
__device__ __forceinline__ floatx4 kchain(FA fa, FB fb, floatx4 acc) {
#pragma unroll
    for (int k = 0; k + 1 < NK; k += 2) acc = MM::mma2(fa(k), fa(k + 1), fb(k), fb(k + 1), acc);
    if (NK & 1) acc = MM::mma(fa(NK - 1), fb(NK - 1), acc);
    return acc;
}

// four consecutive output values to global memory
__device__ __forceinline__ void store4(float* p, floatx4 v) { *(floatx4*)p = v; }
__device__ __forceinline__ void store4(bf16* p, floatx4 v) {
    *(uint2*)p = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}

template <typename T, int N, int P, int NIB>
__global__ __launch_bounds__(P / 16 * 64, 2) void prefill_kernel(PrefillArgs a) {
    using MM = Mma<T>;
    using F = typename MM::frag;
    constexpr int NW = P / 16, NT = NW * 64;
    constexpr int LDN = N + MM::PAD, LDP = P + MM::PAD, LDQ = 64 + MM::PAD;
    constexpr int VE = 16 / sizeof(T);           // elements per 16-byte vector
    constexpr int VPN = N / VE, VPP = P / VE;    // vectors per row of Bbar/Cbar and of x
    constexpr int MAXC = (64 * VPN + NT - 1) / NT;
    constexpr int MAXX = (64 * VPP + NT - 1) / NT;
    constexpr int NB = N / 16;

    __shared__ __align__(16) T sC[64 * LDN];     // Cbar rows of the chunk  [i][n]
    __shared__ __align__(16) T sB[64 * LDN];     // Bbar rows               [s][n]
    __shared__ __align__(16) T sX[64 * LDP];     // x rows                  [s][p]
    __shared__ __align__(16) T sM[64 * LDQ];     // masked scores           [i][s]
    // per-row (t, r) copies of the chunk's per-step scalars, rewritten every chunk: log2 decay
    // l_t, gamma_t, mu_t, exp(l_t), w_t = exp(l_end - l_t) mu_t, and the row's step t
    __shared__ __align__(16) float rL2[64], rGam[64], rMu[64], rEl[64], rW[64];
    __shared__ __align__(16) int rT[64];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, l16 = lane & 15;
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / a.H;
    const int h = (int)(bh % a.H);
    constexpr int QR = 16 * NIB;                 // rows (t, r) per chunk
    const int H = a.H, R = a.R, Q = a.Q;
    const int rl2 = __builtin_ctz((unsigned)R), rmask = R - 1;
    const int64_t L = a.L;
    const int64_t nchunk = (L + Q - 1) / Q;
    const float Alog2 = a.A[h] * kLog2e;
    // (b, t = 0, h) bases; step t of this (b, h) is t * H rows further
    const int64_t row_bh = b * L * a.H + h;
    const T* Xg = (const T*)a.x + row_bh * a.R * P;
    const T* Bg = (const T*)a.Bbar + row_bh * a.R * N;
    const T* Cg = (const T*)a.Cbar + row_bh * a.R * N;
    const T* dtg = (const T*)a.dt + row_bh;
    const T* lamg = (const T*)a.lam + row_bh;
    const int pcol = 16 * wave + l16;            // this lane's column of P in MFMA tiles
    const int64_t HRN = (int64_t)H * R * N, HRP = (int64_t)H * R * P;

    // ---- staging: this thread moves 16-byte vectors k = 0, 1, ... of each tile.  Vector k is
    // chunk row i = i0 + k * (NT / VPN) (row (t, r) = (i >> rl2, i & rmask)), 16-byte column cv0.
    static_assert(NT % VPN == 0 && NT % VPP == 0, "vectors per row must divide the block");
    constexpr int RKC = NT / VPN, RKX = NT / VPP;            // chunk rows per k
    const int iC0 = tid / VPN, cC0 = tid % VPN, iX0 = tid / VPP, cX0 = tid % VPP;
    const int HRN32 = H * R * N, HRP32 = H * R * P;
    auto offC = [&](int k) { const int i = iC0 + k * RKC; return (i >> rl2) * HRN32 + (i & rmask) * N + cC0 * VE; };
    auto offX = [&](int k) { const int i = iX0 + k * RKX; return (i >> rl2) * HRP32 + (i & rmask) * P + cX0 * VE; };

    // ---- chunk prefetch into registers --------------------------------------------------
    uint4 rc[MAXC], rb[MAXC], rx[MAXX];
    float rd = 0.f, rl = 0.f, rdn = 0.f, rln = 0.f;
    auto load_chunk = [&](int64_t c) {
        const int64_t t0 = c * Q;
        const T* cb = Cg + t0 * HRN32;
        const T* bb = Bg + t0 * HRN32;
        const T* xb = Xg + t0 * HRP32;
        if (t0 + Q <= L) {   // a full chunk: every row exists
#pragma unroll
            for (int k = 0; k < MAXC; ++k) {
                if (iC0 + k * RKC < QR) {
                    rc[k] = *(const uint4*)(cb + offC(k));
                    rb[k] = *(const uint4*)(bb + offC(k));
                }
            }
#pragma unroll
            for (int k = 0; k < MAXX; ++k)
                if (iX0 + k * RKX < QR) rx[k] = *(const uint4*)(xb + offX(k));
        } else {             // the ragged last chunk: rows past the sequence end are zero
            const int nvalid = (int)(L - t0);
#pragma unroll
            for (int k = 0; k < MAXC; ++k) {
                const int i = iC0 + k * RKC;
                rc[k] = make_uint4(0, 0, 0, 0);
                rb[k] = make_uint4(0, 0, 0, 0);
                if (i < QR && (i >> rl2) < nvalid) {
                    rc[k] = *(const uint4*)(cb + offC(k));
                    rb[k] = *(const uint4*)(bb + offC(k));
                }
            }
#pragma unroll
            for (int k = 0; k < MAXX; ++k) {
                const int i = iX0 + k * RKX;
                rx[k] = make_uint4(0, 0, 0, 0);
                if (i < QR && (i >> rl2) < nvalid) rx[k] = *(const uint4*)(xb + offX(k));
            }
        }
        if (wave == 0) {
            const int64_t t = t0 + lane;
            const bool in = lane < Q && t < L;
            const bool inn = lane < Q && t + 1 < L;
            rd = in ? load_f32(dtg + t * H) : 0.f;
            rl = in ? load_f32(lamg + t * H) : 0.f;
            rdn = inn ? load_f32(dtg + (t + 1) * H) : 0.f;
            rln = inn ? load_f32(lamg + (t + 1) * H) : 0.f;
        }
    };
    auto store_chunk = [&]() {
#pragma unroll
        for (int k = 0; k < MAXC; ++k) {
            const int i = iC0 + k * RKC;
            if (i < QR) {
                *(uint4*)(sC + i * LDN + cC0 * VE) = rc[k];
                *(uint4*)(sB + i * LDN + cC0 * VE) = rb[k];
            }
        }
#pragma unroll
        for (int k = 0; k < MAXX; ++k) {
            const int i = iX0 + k * RKX;
            if (i < QR) *(uint4*)(sX + i * LDP + cX0 * VE) = rx[k];
        }
        if (wave == 0) {
            // l_t in log2 units: inclusive prefix sum of dt * A over the chunk
            float l2 = rd * Alog2;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const float n = shfl_up(l2, o);
                if (lane >= o) l2 += n;
            }
            const float gam = rl * rd;
            const float mu = gam + (1.0f - rln) * rdn;
            const float l2end = shfl(l2, Q - 1);
            const float el = fast_exp2(l2);
            const float w = fast_exp2(fminf(l2end - l2, 0.f)) * mu;
            // lane = chunk row s; its step is s >> rl2 (rows past Q * R are never read)
            const int ts = lane >> rl2;
            rL2[lane] = shfl(l2, ts);
            rGam[lane] = shfl(gam, ts);
            rMu[lane] = shfl(mu, ts);
            rEl[lane] = shfl(el, ts);
            rW[lane] = shfl(w, ts);
            rT[lane] = ts;
        }
    };

    // ---- carried-in state: G_{-1} = h_in + c_0 Bbar_prev^T x_prev ------------------------
    floatx4 st[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int m = 0; m < 4; ++m)
            st[nb][m] = a.h_in ? a.h_in[(bh * N + 16 * nb + 4 * g + m) * P + pcol] : 0.f;
    if (a.Bbar_prev && a.x_prev && L > 0) {
        const float c0 = (1.0f - load_f32(lamg)) * load_f32(dtg);
        const T* Bp = (const T*)a.Bbar_prev + bh * R * N;
        const T* xp = (const T*)a.x_prev + bh * R * P;
        for (int r = 0; r < R; ++r) {
            const float xv = c0 * load_f32(xp + r * P + pcol);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int m = 0; m < 4; ++m) st[nb][m] += load_f32(Bp + r * N + 16 * nb + 4 * g + m) * xv;
        }
    }

    T* ymix = (T*)a.y + row_bh * P;            // [b, L, H, P] when mixing
    T* yraw = (T*)a.y + row_bh * a.R * P;      // [b, L, H, R, P] otherwise

    // output mixing weights for this lane's (r, 4 columns)
    floatx4 wo = {1.f, 1.f, 1.f, 1.f};
    if (a.w_out) {
        const int r = l16 & rmask;
#pragma unroll
        for (int m = 0; m < 4; ++m) wo[m] = a.w_out[(h * R + r) * P + 16 * wave + 4 * g + m];
    }

    // loop-invariant LDS fragment addresses for this lane
    const T* pB_k = sB + l16 * LDN + 4 * g;                 // + 16 sb LDN + 16 kb
    const T* pC_k = sC + l16 * LDN + 4 * g;                 // + 16 ib LDN + 16 kb
    const T* pM_k = sM + l16 * LDQ + 4 * g;                 // + 16 ib LDQ + 16 sb
    const T* pX_t = sX + 4 * g * LDP + 16 * wave;           // + 16 sb LDP
    const T* pB_t = sB + 4 * g * LDN;                       // + 16 sb LDN + 16 nb

    if (nchunk > 0) load_chunk(0);
    for (int64_t c = 0; c < nchunk; ++c) {
        store_chunk();
        __syncthreads();
        if (c + 1 < nchunk) load_chunk(c + 1);
        const int64_t t0 = c * Q;

        // 1. masked scores M[i][s] = L(t_i, t_s) * Cbar_i . Bbar_s on the causal tiles
#pragma unroll
        for (int ib = 0; ib < NIB; ++ib) {
#pragma unroll
            for (int sb = 0; sb <= ib; ++sb) {
                const int tau = ib * (ib + 1) / 2 + sb;
                if (tau % NW != wave) continue;
                const T* pb = pB_k + 16 * sb * LDN;
                const T* pc = pC_k + 16 * ib * LDN;
                floatx4 acc = kchain<MM, NB>([&](int k) { return MM::ldk(pb + 16 * k); },
                                             [&](int k) { return MM::ldk(pc + 16 * k); },
                                             floatx4{0.f, 0.f, 0.f, 0.f});
                const int i = 16 * ib + l16;
                const int ti = rT[i];
                const float l2i = rL2[i], gi = rGam[i];
                const floatx4 l2s = *(const floatx4*)(rL2 + 16 * sb + 4 * g);
                const floatx4 mus = *(const floatx4*)(rMu + 16 * sb + 4 * g);
                const int4 ts = *(const int4*)(rT + 16 * sb + 4 * g);
                const int tsv[4] = {ts.x, ts.y, ts.z, ts.w};
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    // below the diagonal exp(l_t - l_s) mu_s, on it gamma_t, above it 0
                    const float e = fast_exp2(fminf(l2i - l2s[m], 0.f)) * mus[m];
                    const float below = tsv[m] < ti ? 1.f : 0.f;
                    const float diag = tsv[m] == ti ? gi : 0.f;
                    acc[m] *= fmaf(e, below, diag);
                }
                MM::st(sM + i * LDQ + 16 * sb + 4 * g, MM::pack(acc));
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        __syncthreads();

        // X^T fragments of this wave's 16 columns, for every 16 rows of the chunk
        F xf[NIB];
#pragma unroll
        for (int sb = 0; sb < NIB; ++sb) xf[sb] = MM::ldt(pX_t + 16 * sb * LDP, LDP, l16);

        // 2. Y^T for this wave's 16 columns: state part, scaled by exp(l_t), plus X^T M^T
        F sa[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) sa[nb] = MM::pack(st[nb]);
#pragma unroll
        for (int ib = 0; ib < NIB; ++ib) {
            const T* pc = pC_k + 16 * ib * LDN;
            floatx4 y = kchain<MM, NB>([&](int k) { return sa[k]; }, [&](int k) { return MM::ldk(pc + 16 * k); },
                                       floatx4{0.f, 0.f, 0.f, 0.f});
            const int i = 16 * ib + l16;
            const float el = rEl[i];
#pragma unroll
            for (int m = 0; m < 4; ++m) y[m] *= el;
            const T* pm = pM_k + 16 * ib * LDQ;
            // K = s over the causal blocks 0..ib (pairs in one instruction, an odd last block alone)
#pragma unroll
            for (int k = 0; k < NIB; k += 2) {
                if (k + 1 <= ib)
                    y = MM::mma2(xf[k], xf[k + 1], MM::ldk(pm + 16 * k), MM::ldk(pm + 16 * (k + 1)), y);
                else if (k <= ib)
                    y = MM::mma(xf[k], MM::ldk(pm + 16 * k), y);
            }
            // lane holds Y[(t, r) = i][p = 16 wave + 4 g + m]
            const int tl = i >> rl2, r = i & rmask;
            const int64_t t = t0 + tl;
            const bool valid = t < L;
            const int p = 16 * wave + 4 * g;
            if (a.w_out) {
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    float v = y[m] * wo[m];
                    for (int o = 1; o < R; o <<= 1) v += shfl_xor(v, o);
                    y[m] = v;
                }
                if (valid && r == 0) store4(ymix + t * H * P + p, y);
            } else if (valid) {
                store4(yraw + (t * H * R + r) * P + p, y);
            }
            __builtin_amdgcn_sched_barrier(0);
        }

        // 3. state update: G = exp(l_end) G + Bbar^T (w o X)
        const float dec = rEl[QR - 1];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int m = 0; m < 4; ++m) st[nb][m] *= dec;
        F xw[NIB];
#pragma unroll
        for (int sb = 0; sb < NIB; ++sb) {
            floatx4 xs = MM::unpack(xf[sb]);
            const floatx4 ws = *(const floatx4*)(rW + 16 * sb + 4 * g);
#pragma unroll
            for (int m = 0; m < 4; ++m) xs[m] *= ws[m];
            xw[sb] = MM::pack(xs);
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const T* pt = pB_t + 16 * nb;
            st[nb] = kchain<MM, NIB>([&](int k) { return MM::ldt(pt + 16 * k * LDN, LDN, l16); },
                                     [&](int k) { return xw[k]; }, st[nb]);
        }
        __syncthreads();
    }

    // ---- outputs: final state and the last step's (Bbar, x) ------------------------------
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int m = 0; m < 4; ++m) a.h_out[(bh * N + 16 * nb + 4 * g + m) * P + pcol] = st[nb][m];
    if (L > 0) {
        if (a.Bbar_last)
            for (int e = tid; e < R * N; e += NT)
                ((T*)a.Bbar_last)[bh * R * N + e] = Bg[(L - 1) * HRN32 + e];
        if (a.x_last)
            for (int e = tid; e < R * P; e += NT) ((T*)a.x_last)[bh * R * P + e] = Xg[(L - 1) * HRP32 + e];
    }
}

template <typename T, int N, int P>
hipError_t launch_np(const PrefillArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)(a.b * a.H)), block(P / 16 * 64);
    switch (a.Q * a.R) {
        case 16: hipLaunchKernelGGL((prefill_kernel<T, N, P, 1>), grid, block, 0, s, a); break;
        case 32: hipLaunchKernelGGL((prefill_kernel<T, N, P, 2>), grid, block, 0, s, a); break;
        case 48: hipLaunchKernelGGL((prefill_kernel<T, N, P, 3>), grid, block, 0, s, a); break;
        case 64: hipLaunchKernelGGL((prefill_kernel<T, N, P, 4>), grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const PrefillArgs& a, hipStream_t s) {
    if (a.N == 16 && a.P == 16) return launch_np<T, 16, 16>(a, s);
    if (a.N == 64 && a.P == 64) return launch_np<T, 64, 64>(a, s);
    if (a.N == 128 && a.P == 64) return launch_np<T, 128, 64>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace

bool prefill_supported(int N, int P, int R, int QR, bool /*bf16_io*/) {
    const bool np = (N == 16 && P == 16) || (N == 64 && P == 64) || (N == 128 && P == 64);
    const bool r = R == 1 || R == 2 || R == 4 || R == 8 || R == 16;
    const bool q = QR >= 16 && QR <= 64 && QR % 16 == 0 && QR % R == 0;
    return np && r && q;
}

hipError_t launch_prefill(const PrefillArgs& a, bool bf16_io, hipStream_t s) {
    return bf16_io ? launch_t<bf16>(a, s) : launch_t<float>(a, s);
}

}  // namespace m3
