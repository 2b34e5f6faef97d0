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
// At the call's last step c_{L} is taken as 0, so the returned G is the true state g_{L-1};
// at the call's first step G_{-1} = h_in + c_0 Bbar_prev^T x_prev.  The trapezoid's link across
// chunk boundaries is therefore one scalar (dt, lambda of the next step), not a B/x halo.
//
// Mapping on gfx950.  One workgroup per (b, h) walks the chunks in order and keeps the N x P
// fp32 state in MFMA accumulator registers, so chunk states never travel through HBM.  The
// chunk holds QR = Q * R rows (t, r).  Wave w owns the 16 columns [16w, 16w + 16) of P.
//   1. S^T = Bbar Cbar^T (QR x QR, K = N) on MFMA, only the causal 16x16 tiles, shared out
//      among the waves; the mask is applied in registers and M = L o S goes to LDS.
//   2. Y^T (own 16 columns x QR) = state^T Cbar^T * exp(l) + X^T M^T: the state is the A
//      operand straight from the accumulator registers (an MFMA D tile of S[n][p] is an A tile
//      of S^T), M comes back from LDS.
//   3. state = exp(l_end) state + (Bbar^T)(w o X), w_s = exp(l_end - l_s) mu_s.
// Every MFMA operand read from LDS is four consecutive elements along K.  X and Bbar are
// staged transposed so that holds for the products over s.  The next chunk's tiles are loaded
// into registers while the current chunk computes.
//
// Operands: bf16 inputs run v_mfma_f32_16x16x16_bf16 (fp32 accumulate); fp32 inputs run
// v_mfma_f32_16x16x4_f32 four times per 16-wide K block.  The same lane->K slot assignment is
// used for both operands of every product, which is all the result depends on.
#include "m3_device.h"
#include "m3_launch.h"

namespace m3 {

namespace {

template <typename T> struct Mma;

template <> struct Mma<bf16> {
    typedef shortx4 frag;
    static __device__ __forceinline__ frag lds(const bf16* p) { return *(const shortx4*)p; }
    static __device__ __forceinline__ floatx4 mma(frag a, frag b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ frag pack(floatx4 v) {
        frag f;
        f[0] = (short)bf16_bits_rne(v[0]);
        f[1] = (short)bf16_bits_rne(v[1]);
        f[2] = (short)bf16_bits_rne(v[2]);
        f[3] = (short)bf16_bits_rne(v[3]);
        return f;
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
    static __device__ __forceinline__ frag lds(const float* p) { return *(const floatx4*)p; }
    static __device__ __forceinline__ floatx4 mma(frag a, frag b, floatx4 c) {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
        return c;
    }
    static __device__ __forceinline__ frag pack(floatx4 v) { return v; }
    static __device__ __forceinline__ floatx4 unpack(frag f) { return f; }
    static __device__ __forceinline__ void st(float* p, frag f) { *(floatx4*)p = f; }
};

// four consecutive output values to global memory
__device__ __forceinline__ void store4(float* p, floatx4 v) { *(floatx4*)p = v; }
__device__ __forceinline__ void store4(bf16* p, floatx4 v) {
    const uint32_t lo = (uint32_t)bf16_bits_rne(v[0]) | ((uint32_t)bf16_bits_rne(v[1]) << 16);
    const uint32_t hi = (uint32_t)bf16_bits_rne(v[2]) | ((uint32_t)bf16_bits_rne(v[3]) << 16);
    *(uint2*)p = make_uint2(lo, hi);
}

template <typename T, int N, int P>
__global__ __launch_bounds__(P / 16 * 64) void prefill_kernel(PrefillArgs a) {
    using MM = Mma<T>;
    using F = typename MM::frag;
    constexpr int NW = P / 16, NT = NW * 64;
    constexpr int PAD = 16 / sizeof(T);          // one 16-byte vector of padding per row
    constexpr int LDN = N + PAD, LDQ = 64 + PAD;
    constexpr int VE = 16 / sizeof(T);           // elements per 16-byte vector
    constexpr int VPN = N / VE, VPP = P / VE;    // vectors per row of Bbar/Cbar and of x
    constexpr int MAXC = (64 * VPN + NT - 1) / NT;
    constexpr int MAXX = (64 * VPP + NT - 1) / NT;
    constexpr int NB = N / 16;

    __shared__ __align__(16) T sC[64 * LDN];     // Cbar rows of the chunk  [i][n]
    __shared__ __align__(16) T sB[64 * LDN];     // Bbar rows               [s][n]
    __shared__ __align__(16) T sBT[N * LDQ];     // Bbar transposed         [n][s]
    __shared__ __align__(16) T sXT[P * LDQ];     // x transposed            [p][s]
    __shared__ __align__(16) T sM[64 * LDQ];     // masked scores           [i][s]
    __shared__ float sL2[64], sGam[64], sMu[64], sEl[64], sW[64];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, l16 = lane & 15;
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / a.H;
    const int h = (int)(bh % a.H);
    const int H = a.H, R = a.R, Q = a.Q, QR = Q * R, nIB = QR / 16;
    const int64_t L = a.L;
    const int64_t nchunk = (L + Q - 1) / Q;
    const float Alog2 = a.A[h] * kLog2e;
    const T* Xg = (const T*)a.x;
    const T* Bg = (const T*)a.Bbar;
    const T* Cg = (const T*)a.Cbar;
    const T* dtg = (const T*)a.dt;
    const T* lamg = (const T*)a.lam;
    const int pcol = 16 * wave + l16;            // this lane's column of P in MFMA tiles

    // ---- chunk prefetch into registers --------------------------------------------------
    uint4 rc[MAXC], rb[MAXC], rx[MAXX];
    float rd = 0.f, rl = 0.f, rdn = 0.f, rln = 0.f;
    auto load_chunk = [&](int64_t c) {
        const int64_t t0 = c * Q;
#pragma unroll
        for (int k = 0; k < MAXC; ++k) {
            const int v = tid + k * NT;
            rc[k] = make_uint4(0, 0, 0, 0);
            rb[k] = make_uint4(0, 0, 0, 0);
            if (v < QR * VPN) {
                const int i = v / VPN, cv = v % VPN;
                const int64_t t = t0 + i / R;
                if (t < L) {
                    const int64_t off = ((((b * L + t) * H + h) * R) + i % R) * N + cv * VE;
                    rc[k] = *(const uint4*)(Cg + off);
                    rb[k] = *(const uint4*)(Bg + off);
                }
            }
        }
#pragma unroll
        for (int k = 0; k < MAXX; ++k) {
            const int v = tid + k * NT;
            rx[k] = make_uint4(0, 0, 0, 0);
            if (v < QR * VPP) {
                const int i = v / VPP, cv = v % VPP;
                const int64_t t = t0 + i / R;
                if (t < L) {
                    const int64_t off = ((((b * L + t) * H + h) * R) + i % R) * P + cv * VE;
                    rx[k] = *(const uint4*)(Xg + off);
                }
            }
        }
        if (wave == 0) {
            const int64_t t = t0 + lane;
            const bool in = lane < Q && t < L;
            const bool inn = lane < Q && t + 1 < L;
            const int64_t row = (b * L + t) * H + h;
            rd = in ? load_f32(dtg + row) : 0.f;
            rl = in ? load_f32(lamg + row) : 0.f;
            rdn = inn ? load_f32(dtg + row + H) : 0.f;
            rln = inn ? load_f32(lamg + row + H) : 0.f;
        }
    };
    auto store_chunk = [&]() {
#pragma unroll
        for (int k = 0; k < MAXC; ++k) {
            const int v = tid + k * NT;
            if (v < QR * VPN) {
                const int i = v / VPN, cv = v % VPN;
                *(uint4*)(sC + i * LDN + cv * VE) = rc[k];
                *(uint4*)(sB + i * LDN + cv * VE) = rb[k];
                const T* e = (const T*)&rb[k];
#pragma unroll
                for (int q = 0; q < VE; ++q) sBT[(cv * VE + q) * LDQ + i] = e[q];
            }
        }
#pragma unroll
        for (int k = 0; k < MAXX; ++k) {
            const int v = tid + k * NT;
            if (v < QR * VPP) {
                const int i = v / VPP, cv = v % VPP;
                const T* e = (const T*)&rx[k];
#pragma unroll
                for (int q = 0; q < VE; ++q) sXT[(cv * VE + q) * LDQ + i] = e[q];
            }
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
            sL2[lane] = l2;
            sGam[lane] = gam;
            sMu[lane] = mu;
            sEl[lane] = exp2f(l2);
            sW[lane] = exp2f(l2end - l2) * mu;
        }
    };

    // ---- carried-in state: G_{-1} = h_in + c_0 Bbar_prev^T x_prev ------------------------
    floatx4 st[NB];
    {
        float c0 = 0.f;
        if (L > 0) {
            const int64_t row0 = (b * L) * H + h;
            c0 = (1.0f - load_f32(lamg + row0)) * load_f32(dtg + row0);
        }
        const T* Bp = (const T*)a.Bbar_prev;
        const T* xp = (const T*)a.x_prev;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int n = 16 * nb + 4 * g + m;
                float v = a.h_in ? a.h_in[(bh * N + n) * P + pcol] : 0.f;
                if (Bp && xp) {
                    float u = 0.f;
                    for (int r = 0; r < R; ++r)
                        u += load_f32(Bp + (bh * R + r) * N + n) * load_f32(xp + (bh * R + r) * P + pcol);
                    v += c0 * u;
                }
                st[nb][m] = v;
            }
    }

    // output mixing weights for this lane's (r, 4 columns)
    floatx4 wo = {1.f, 1.f, 1.f, 1.f};
    if (a.w_out) {
        const int r = l16 % R;
#pragma unroll
        for (int m = 0; m < 4; ++m) wo[m] = a.w_out[(h * R + r) * P + 16 * wave + 4 * g + m];
    }

    if (nchunk > 0) load_chunk(0);
    for (int64_t c = 0; c < nchunk; ++c) {
        store_chunk();
        __syncthreads();
        if (c + 1 < nchunk) load_chunk(c + 1);
        const int64_t t0 = c * Q;

        // 1. masked scores M[i][s] = L(t_i, t_s) * Cbar_i . Bbar_s on the causal tiles
        int tau = 0;
        for (int ib = 0; ib < nIB; ++ib) {
            for (int sb = 0; sb <= ib; ++sb, ++tau) {
                if (tau % NW != wave) continue;
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < NB; ++kb) {
                    const F fa = MM::lds(sB + (16 * sb + l16) * LDN + 16 * kb + 4 * g);
                    const F fb = MM::lds(sC + (16 * ib + l16) * LDN + 16 * kb + 4 * g);
                    acc = MM::mma(fa, fb, acc);
                }
                const int i = 16 * ib + l16;
                const int ti = i / R;
                const float l2i = sL2[ti], gi = sGam[ti];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int ts = (16 * sb + 4 * g + m) / R;
                    const float f = ts < ti ? exp2f(l2i - sL2[ts]) * sMu[ts] : (ts == ti ? gi : 0.f);
                    acc[m] *= f;
                }
                MM::st(sM + i * LDQ + 16 * sb + 4 * g, MM::pack(acc));
            }
        }
        __syncthreads();

        // 2. Y^T for this wave's 16 columns: state part, scaled by exp(l_t), plus X^T M^T
        F sa[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) sa[nb] = MM::pack(st[nb]);
        for (int ib = 0; ib < nIB; ++ib) {
            floatx4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NB; ++kb)
                y = MM::mma(sa[kb], MM::lds(sC + (16 * ib + l16) * LDN + 16 * kb + 4 * g), y);
            const int i = 16 * ib + l16;
            const float el = sEl[i / R];
#pragma unroll
            for (int m = 0; m < 4; ++m) y[m] *= el;
            for (int sb = 0; sb <= ib; ++sb) {
                const F fa = MM::lds(sXT + pcol * LDQ + 16 * sb + 4 * g);
                const F fb = MM::lds(sM + i * LDQ + 16 * sb + 4 * g);
                y = MM::mma(fa, fb, y);
            }
            // lane holds Y[(t, r) = i][p = 16 wave + 4 g + m]
            const int tl = i / R, r = i % R;
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
                if (valid && r == 0) store4((T*)a.y + ((b * L + t) * H + h) * P + p, y);
            } else if (valid) {
                store4((T*)a.y + (((b * L + t) * H + h) * R + r) * P + p, y);
            }
        }

        // 3. state update: G = exp(l_end) G + Bbar^T (w o X)
        const float dec = sEl[Q - 1];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int m = 0; m < 4; ++m) st[nb][m] *= dec;
        for (int sb = 0; sb < nIB; ++sb) {
            floatx4 xf = MM::unpack(MM::lds(sXT + pcol * LDQ + 16 * sb + 4 * g));
#pragma unroll
            for (int m = 0; m < 4; ++m) xf[m] *= sW[(16 * sb + 4 * g + m) / R];
            const F fx = MM::pack(xf);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                st[nb] = MM::mma(MM::lds(sBT + (16 * nb + l16) * LDQ + 16 * sb + 4 * g), fx, st[nb]);
        }
        __syncthreads();
    }

    // ---- outputs: final state and the last step's (Bbar, x) ------------------------------
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int m = 0; m < 4; ++m) a.h_out[(bh * N + 16 * nb + 4 * g + m) * P + pcol] = st[nb][m];
    if (L > 0) {
        const int64_t rowl = ((b * L + L - 1) * H + h) * R;
        if (a.Bbar_last)
            for (int e = tid; e < R * N; e += NT) ((T*)a.Bbar_last)[bh * R * N + e] = Bg[rowl * N + e];
        if (a.x_last)
            for (int e = tid; e < R * P; e += NT) ((T*)a.x_last)[bh * R * P + e] = Xg[rowl * P + e];
    }
}

template <typename T>
hipError_t launch_t(const PrefillArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)(a.b * a.H));
    if (a.N == 16 && a.P == 16)
        hipLaunchKernelGGL((prefill_kernel<T, 16, 16>), grid, dim3(64), 0, s, a);
    else if (a.N == 64 && a.P == 64)
        hipLaunchKernelGGL((prefill_kernel<T, 64, 64>), grid, dim3(256), 0, s, a);
    else if (a.N == 128 && a.P == 64)
        hipLaunchKernelGGL((prefill_kernel<T, 128, 64>), grid, dim3(256), 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
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
