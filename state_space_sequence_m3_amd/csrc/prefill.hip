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
// QR = Q * R rows (t, r).  Wave w owns the 16 columns [16w, 16w + 16) of P.  Per chunk:
//   stage  the chunk's Bbar, Cbar and x rows (loaded into registers during the previous chunk) go to
//          LDS, the next chunk's loads are issued, wave 0 turns dt and lambda into per-row scalars;
//          barrier.
//   part 1 everything that needs only this chunk's tiles and the carried state, as independent MFMA
//          chains interleaved along K: the state part of Y^T (state^T Cbar^T, the state is the A
//          operand straight from its accumulator registers: an MFMA D tile of S[n][p] is an A tile
//          of S^T), this wave's share of the causal 16x16 tiles of S^T = Bbar Cbar^T, and the state
//          update  state = exp(l_end) state + (Bbar^T)(w o X), w_s = exp(l_end - l_s) mu_s.  The
//          score tiles are masked in registers and M = L o S goes to LDS; barrier.
//   part 2 Y^T += X^T M^T, then output mixing and the stores.
// Two barriers per chunk: nothing reads the staged tiles after the second, so the next chunk's
// staging may overwrite them, and M is rewritten only after the next chunk's first barrier.
// Operands that need the other orientation (X^T and Bbar^T, contracted over the rows) are read
// with gfx950's transposing LDS read (ds_read_b64_tr_b16): in each group of 16 lanes, lane j
// points at 4 consecutive elements of row k0 + j/4, columns c0 + 4 (j % 4); lane i then receives
// rows k0..k0+3 of column c0 + i.  LDS rows are padded so that the 32 lanes one cycle serves land
// on distinct banks (64 banks of 4 bytes): rows read along K get 8 extra elements, rows read with
// the transposing read 16.
// Global traffic goes through raw buffer descriptors that end at the sequence's last row: loads
// past it return zero and stores past it are dropped, so the ragged last chunk needs no branches.
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
    // LDS row padding in elements: tiles read along K (8 bytes a lane), tiles read transposed
    static constexpr int PADK = 8, PADT = 16;
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
    static constexpr int PADK = 8, PADT = 8;
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
    static __device__ __forceinline__ frag pack(floatx4 v) { return v; }
    static __device__ __forceinline__ floatx4 unpack(frag f) { return f; }
    static __device__ __forceinline__ void st(float* p, frag f) { *(floatx4*)p = f; }
};

// four consecutive output values through a buffer descriptor
__device__ __forceinline__ void store4(rsrc_t r, uint32_t off, floatx4 v, float) {
    buffer_store16(r, off, __builtin_bit_cast(uint4, v));
}
__device__ __forceinline__ void store4(rsrc_t r, uint32_t off, floatx4 v, bf16) {
    buffer_store8(r, off, make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])));
}

// causal 16x16 tile number tau = ib (ib + 1) / 2 + sb (sb <= ib < 4) -> row block ib
__device__ __forceinline__ int tile_ib(int tau) { return (tau >= 1) + (tau >= 3) + (tau >= 6); }

// unpack one 16-byte vector of io elements to floats
__device__ __forceinline__ void unpack16(uint4 v, float (&o)[4], float) {
    o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
    o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
}
__device__ __forceinline__ void unpack16(uint4 v, float (&o)[8], bf16) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = __uint_as_float(w[i] << 16);
        o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ uint4 pack16(const float (&v)[4], float) {
    return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3]));
}
__device__ __forceinline__ uint4 pack16(const float (&v)[8], bf16) {
    return make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
}

// FUSED: the chunk's B and C arrive raw and are normalised (BCNorm), biased and rotated by the
// cumulative angle while they are staged (papernotes.org, key design 4; aipaper.cc section 4.2
// Proposition 3), so the rotated Bbar and Cbar never go through HBM.
template <typename T, int N, int P, int NIB, bool FUSED>
__global__ __launch_bounds__(P / 16 * 64, 2) void prefill_kernel(PrefillArgs a) {
    using MM = Mma<T>;
    using F = typename MM::frag;
    constexpr int NW = P / 16, NT = NW * 64;
    constexpr int QR = 16 * NIB;                 // rows (t, r) per chunk
    constexpr int NB = N / 16;
    constexpr int LDC = N + MM::PADK, LDB = N + MM::PADT, LDX = P + MM::PADT, LDM = QR + MM::PADK;
    constexpr int VE = 16 / sizeof(T);           // elements per 16-byte vector
    constexpr int VPN = N / VE, VPP = P / VE;    // vectors per row of Bbar/Cbar and of x
    static_assert(NT % VPN == 0 && NT % VPP == 0, "vectors per row must divide the block");
    constexpr int RKC = NT / VPN, RKX = NT / VPP;                // chunk rows per staging step
    constexpr int MAXC = (QR + RKC - 1) / RKC, MAXX = (QR + RKX - 1) / RKX;
    constexpr bool FULLC = MAXC * RKC == QR, FULLX = MAXX * RKX == QR;
    constexpr int NTILE = NIB * (NIB + 1) / 2, NSLOT = (NTILE + NW - 1) / NW;
    // fused angle scan: K rotation pairs, VT angle increments per 16-byte theta vector, NVT vectors
    // per step; thread tau scans column v = tau / TPV over steps j * SPT .. j * SPT + SPT - 1
    constexpr int K = N / 2, VT = VE, NVT = K / VT;
    constexpr int SPT = NVT * QR > NT ? NVT * QR / NT : 1, TPV = FUSED ? QR / SPT : 16;
    static_assert(!FUSED || (TPV <= 64 && NVT * TPV <= NT && (QR & (QR - 1)) == 0), "angle scan layout");
    constexpr int LDPHI = K + 8;                 // padded angle rows (fp32)
    constexpr int RB = NIB > 2 ? 4 : 16;         // ranks whose bias fits in LDS
    constexpr int FZ = FUSED ? 1 : 0;            // sizes the fused-only LDS arrays

    __shared__ __align__(16) T sC[QR * LDC];     // Cbar rows of the chunk  [i][n]
    __shared__ __align__(16) T sB[QR * LDB];     // Bbar rows               [s][n]
    __shared__ __align__(16) T sX[QR * LDX];     // x rows                  [s][p]
    __shared__ __align__(16) T sM[QR * LDM];     // masked scores           [i][s]
    // per-row (t, r) copies of the chunk's per-step scalars, rewritten every chunk: log2 decay
    // l_t, gamma_t, mu_t, exp(l_t) and w_t = exp(l_end - l_t) mu_t
    __shared__ __align__(16) float rL2[64], rGam[64], rMu[64], rEl[64], rW[64];
    // fused only: the chunk's angles Phi[t][k], BCNorm weights [B, C][n], biases [B, C][r][n]
    __shared__ __align__(16) float sPhi[FZ * QR * LDPHI + 1];
    __shared__ __align__(16) float sWt[FZ * 2 * N + 1];
    __shared__ __align__(16) float sBias[FZ * 2 * RB * N + 1];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, l16 = lane & 15;
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / a.H;
    const int h = (int)(bh % a.H);
    const int H = a.H, R = a.R, Q = a.Q;
    const int rl2 = __builtin_ctz((unsigned)R), rmask = R - 1;
    const int64_t L = a.L;
    const int64_t nchunk = (L + Q - 1) / Q;
    const float Alog2 = a.A[h] * kLog2e;
    // (b, t = 0, h) bases; step t of this (b, h) is t * H rows further
    const int64_t row_bh = b * L * H + h;
    const int64_t HRN = (int64_t)H * R * N, HRP = (int64_t)H * R * P;
    const T* Xg = (const T*)a.x + row_bh * R * P;
    const T* Bg = (const T*)a.Bbar + row_bh * R * N;
    const T* Cg = (const T*)a.Cbar + row_bh * R * N;
    const T* dtg = (const T*)a.dt + row_bh;
    const T* lamg = (const T*)a.lam + row_bh;
    const int pcol = 16 * wave + l16;            // this lane's column of P in MFMA tiles
    // bytes from a chunk's first row to the end of the sequence's last row (t = L - 1)
    auto tail_bytes = [&](int64_t t0, int64_t step, int64_t row) {
        return clamp_bytes(((L - t0 - 1) * step + row) * (int64_t)sizeof(T));
    };

    // ---- staging: this thread moves 16-byte vectors k = 0, 1, ... of each tile.  Vector k is
    // chunk row i = i0 + k * RK (row (t, r) = (i >> rl2, i & rmask)), 16-byte column c0.
    const int iC0 = tid / VPN, cC0 = tid % VPN, iX0 = tid / VPP, cX0 = tid % VPP;
    const int HRN32 = (int)HRN, HRP32 = (int)HRP;
    auto offC = [&](int k) {
        const int i = iC0 + k * RKC;
        return (uint32_t)(((i >> rl2) * HRN32 + (i & rmask) * N + cC0 * VE) * (int)sizeof(T));
    };
    auto offX = [&](int k) {
        const int i = iX0 + k * RKX;
        return (uint32_t)(((i >> rl2) * HRP32 + (i & rmask) * P + cX0 * VE) * (int)sizeof(T));
    };

    // ---- chunk prefetch into registers --------------------------------------------------
    uint4 rc[MAXC], rb[MAXC], rx[MAXX];
    float nd = 0.f, nl = 0.f, ndn = 0.f, nln = 0.f;   // wave 0: dt, lambda at t and t + 1
    auto load_chunk = [&](int64_t c) {
        const int64_t t0 = c * Q;
        const uint32_t nbc = tail_bytes(t0, HRN, (int64_t)R * N), nbx = tail_bytes(t0, HRP, (int64_t)R * P);
        const rsrc_t dC = make_rsrc(Cg + t0 * HRN, nbc), dB = make_rsrc(Bg + t0 * HRN, nbc);
        const rsrc_t dX = make_rsrc(Xg + t0 * HRP, nbx);
#pragma unroll
        for (int k = 0; k < MAXC; ++k) {
            if (FULLC || iC0 + k * RKC < QR) {
                rc[k] = buffer_load16(dC, offC(k));
                rb[k] = buffer_load16(dB, offC(k));
            }
        }
#pragma unroll
        for (int k = 0; k < MAXX; ++k)
            if (FULLX || iX0 + k * RKX < QR) rx[k] = buffer_load16(dX, offX(k));
        if (wave == 0) {
            const int64_t t = t0 + lane;
            const bool in = lane < Q && t < L;
            const bool inn = lane < Q && t + 1 < L;
            nd = in ? load_f32(dtg + t * H) : 0.f;
            nl = in ? load_f32(lamg + t * H) : 0.f;
            ndn = inn ? load_f32(dtg + (t + 1) * H) : 0.f;
            nln = inn ? load_f32(lamg + (t + 1) * H) : 0.f;
        }
    };
    // ---- fused: angle increments of a chunk and their prefix scan ----------------------
    const int tau = tid, tv = tau / TPV, tj = tau % TPV;
    const bool scanner = FUSED && tau < NVT * TPV;
    uint4 rth[SPT];
    float rdt[SPT];
    const T* thg = (const T*)a.theta + row_bh * K;
    const int64_t HK = (int64_t)H * K;
    auto load_theta = [&](int64_t c) {
        if (!scanner) return;
        const int64_t t0 = c * Q;
        const rsrc_t dT = make_rsrc(thg + t0 * HK, tail_bytes(t0, HK, K));
#pragma unroll
        for (int s = 0; s < SPT; ++s) {
            const int t = tj * SPT + s;
            const bool in = t < Q;   // steps past the chunk (R > 1 leaves rows of the tile unused)
            rth[s] = in ? buffer_load16(dT, (uint32_t)((t * (int)HK + tv * VT) * (int)sizeof(T)))
                        : make_uint4(0, 0, 0, 0);
            rdt[s] = in && t0 + t < L ? load_f32(dtg + (t0 + t) * H) : 0.f;
        }
    };
    // Phi[t] = Phi[t0 - 1] + sum_{t0 <= i <= t} dt_i theta_i for the chunk starting at c * Q, into
    // sPhi.  The carried angle is the previous chunk's last row, read by the same wave that
    // rewrites it (reads come before writes in one wave's LDS order); chunk 0 starts from phi_in.
    auto scan = [&](int64_t c) {
        if (!scanner) return;
        float acc[SPT][VT];
#pragma unroll
        for (int s = 0; s < SPT; ++s) {
            float f[VT];
            unpack16(rth[s], f, T{});
#pragma unroll
            for (int e = 0; e < VT; ++e) acc[s][e] = (s ? acc[s - 1][e] : 0.f) + rdt[s] * f[e];
        }
        float base[VT];
#pragma unroll
        for (int e = 0; e < VT; ++e) {
            const int k = tv * VT + e;
            const float carry = c == 0 ? (a.phi_in ? wrap_angle(a.phi_in[bh * K + k]) : 0.f)
                                       : sPhi[(Q - 1) * LDPHI + k];
            const float tot = acc[SPT - 1][e];
            base[e] = carry + seg_scan_add<TPV>(tot, lane) - tot;
        }
#pragma unroll
        for (int s = 0; s < SPT; ++s) {
            float* dst = sPhi + (tj * SPT + s) * LDPHI + tv * VT;
#pragma unroll
            for (int e = 0; e < VT; e += 4)
                *(floatx4*)(dst + e) = floatx4{wrap_angle(base[e] + acc[s][e]), wrap_angle(base[e + 1] + acc[s][e + 1]),
                                               wrap_angle(base[e + 2] + acc[s][e + 2]), wrap_angle(base[e + 3] + acc[s][e + 3])};
        }
    };
    // fused: raw B and C rows of this thread -> BCNorm, weight, bias, rotation -> LDS.  When the
    // staging step RKC is a multiple of every supported R, all rows of a thread have the same
    // rank, and the thread's weights and biases stay in registers (loaded after the prologue).
    const float invN = 1.0f / (float)N;
    constexpr bool WREG = FUSED && RKC % 16 == 0;
    float cwB[WREG ? VE : 1], cwC[WREG ? VE : 1], cbB[WREG ? VE : 1], cbC[WREG ? VE : 1];
    auto stage_bc = [&](int k, int i) {
        const int t = i >> rl2, r = i & rmask;
        float xb[VE], xc[VE];
        unpack16(rb[k], xb, T{});
        unpack16(rc[k], xc, T{});
        float sb = 1.f, sc = 1.f;
        if (a.bcnorm) {   // RMS over the row's N values, spread over VPN consecutive lanes
            float qb = 0.f, qc = 0.f;
#pragma unroll
            for (int e = 0; e < VE; ++e) {
                qb = fmaf(xb[e], xb[e], qb);
                qc = fmaf(xc[e], xc[e], qc);
            }
            qb = group_sum(qb, VPN);
            qc = group_sum(qc, VPN);
            // hardware 1/sqrt; the clamp keeps its argument out of the denormal range (an all-zero
            // row stays zero either way)
            sb = __builtin_amdgcn_rsqf(fmaxf(fmaf(qb, invN, a.eps), 1e-30f));
            sc = __builtin_amdgcn_rsqf(fmaxf(fmaf(qc, invN, a.eps), 1e-30f));
        }
        const int n0 = cC0 * VE;
        const float* ph = sPhi + t * LDPHI + n0 / 2;
        if (WREG) {
#pragma unroll
            for (int e = 0; e < VE; ++e) {
                xb[e] = fmaf(xb[e] * sb, cwB[e % (WREG ? VE : 1)], cbB[e % (WREG ? VE : 1)]);
                xc[e] = fmaf(xc[e] * sc, cwC[e % (WREG ? VE : 1)], cbC[e % (WREG ? VE : 1)]);
            }
        } else {
            const float* wB = sWt + n0;
            const float* wC = sWt + N + n0;
            const float* bB = sBias + r * N + n0;
            const float* bC = sBias + (RB + r) * N + n0;
#pragma unroll
            for (int e = 0; e < VE; ++e) {
                xb[e] = fmaf(xb[e] * sb, wB[e], bB[e]);
                xc[e] = fmaf(xc[e] * sc, wC[e], bC[e]);
            }
        }
#pragma unroll
        for (int q = 0; q < VE / 2; ++q) {
            float sn, cs;
            __sincosf(ph[q], &sn, &cs);   // |angle| <= pi
            const float b0 = xb[2 * q], b1 = xb[2 * q + 1], c0 = xc[2 * q], c1 = xc[2 * q + 1];
            xb[2 * q] = fmaf(cs, b0, sn * b1);
            xb[2 * q + 1] = fmaf(cs, b1, -sn * b0);
            xc[2 * q] = fmaf(cs, c0, sn * c1);
            xc[2 * q + 1] = fmaf(cs, c1, -sn * c0);
        }
        *(uint4*)(sC + i * LDC + n0) = pack16(xc, T{});
        *(uint4*)(sB + i * LDB + n0) = pack16(xb, T{});
    };

    auto store_tiles = [&]() {
#pragma unroll
        for (int k = 0; k < MAXC; ++k) {
            const int i = iC0 + k * RKC;
            if (FULLC || i < QR) {
                if (FUSED) {
                    stage_bc(k, i);
                } else {
                    *(uint4*)(sC + i * LDC + cC0 * VE) = rc[k];
                    *(uint4*)(sB + i * LDB + cC0 * VE) = rb[k];
                }
            }
        }
#pragma unroll
        for (int k = 0; k < MAXX; ++k) {
            const int i = iX0 + k * RKX;
            if (FULLX || i < QR) *(uint4*)(sX + i * LDX + cX0 * VE) = rx[k];
        }
    };
    // wave 0: the chunk's per-step scalars (lane = step) -> per-row copies in LDS.  Lanes past
    // the chunk only add to later lanes of the scan, which are never read.
    auto stage_scalars = [&](float d, float lm, float dn, float lmn) {
        const float l2 = wave_scan_add(d * Alog2);   // l_t in log2 units, inclusive over the chunk
        const float gam = lm * d;
        const float mu = gam + (1.0f - lmn) * dn;
        const float l2end = lane_value(l2, Q - 1);
        const float el = fast_exp2(l2);
        const float w = fast_exp2(fminf(l2end - l2, 0.f)) * mu;
        if (R == 1) {
            rL2[lane] = l2;
            rGam[lane] = gam;
            rMu[lane] = mu;
            rEl[lane] = el;
            rW[lane] = w;
        } else {   // row s holds step s >> rl2 (rows past Q * R are never read)
            const int ts = lane >> rl2;
            rL2[lane] = shfl(l2, ts);
            rGam[lane] = shfl(gam, ts);
            rMu[lane] = shfl(mu, ts);
            rEl[lane] = shfl(el, ts);
            rW[lane] = shfl(w, ts);
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

    // outputs: mixed [b, L, H, P] with w_out, else [b, L, H, R, P]
    const bool mix = a.w_out != nullptr;
    T* yg = (T*)a.y + row_bh * (mix ? P : (int64_t)R * P);
    const int64_t ystep = mix ? (int64_t)H * P : HRP, yrow = mix ? P : (int64_t)R * P;
    floatx4 wo = {1.f, 1.f, 1.f, 1.f};          // mixing weights for this lane's (r, 4 columns)
    if (mix) {
        const int r = l16 & rmask;
#pragma unroll
        for (int m = 0; m < 4; ++m) wo[m] = a.w_out[(h * R + r) * P + 16 * wave + 4 * g + m];
    }

    // loop-invariant LDS fragment addresses for this lane
    const T* pC_k = sC + l16 * LDC + 4 * g;                 // + 16 ib LDC + 16 kb
    const T* pB_k = sB + l16 * LDB + 4 * g;                 // + 16 sb LDB + 16 kb
    const T* pM_k = sM + l16 * LDM + 4 * g;                 // + 16 ib LDM + 16 sb
    const T* pX_t = sX + 4 * g * LDX + 16 * wave;           // + 16 sb LDX
    const T* pB_t = sB + 4 * g * LDB;                       // + 16 sb LDB + 16 nb
    // this wave's score tiles: tau = wave, wave + NW, ...; a wave with fewer tiles than NSLOT
    // recomputes tile NTILE - 1 in its spare slot and drops the copy
    int sIb[NSLOT], sSb[NSLOT];
    bool sOn[NSLOT];
    const T* pSB[NSLOT];
    const T* pSC[NSLOT];
#pragma unroll
    for (int j = 0; j < NSLOT; ++j) {
        const int tau0 = wave + NW * j;
        sOn[j] = tau0 < NTILE;
        const int tau = sOn[j] ? tau0 : NTILE - 1;
        sIb[j] = tile_ib(tau);
        sSb[j] = tau - sIb[j] * (sIb[j] + 1) / 2;
        pSB[j] = pB_k + 16 * sSb[j] * LDB;
        pSC[j] = pC_k + 16 * sIb[j] * LDC;
    }

    if (FUSED) {
        // BCNorm weights (1 without BCNorm or without weights) and biases (0 when absent)
        for (int e = tid; e < 2 * N; e += NT) {
            const float* w = e < N ? a.normw_B : a.normw_C;
            sWt[e] = a.bcnorm && w ? w[h * N + (e % N)] : 1.f;
        }
        for (int e = tid; e < 2 * RB * N; e += NT) {
            const int which = e / (RB * N), r = (e / N) % RB;
            const float* bias = which == 0 ? a.bias_B : a.bias_C;
            sBias[e] = bias && r < R ? bias[(h * R + r) * N + (e % N)] : 0.f;
        }
        if (nchunk > 0) {
            load_theta(0);
            scan(0);
        }
        __syncthreads();
        if (WREG) {
            const int n0 = cC0 * VE, r0 = iC0 & rmask;
#pragma unroll
            for (int e = 0; e < (WREG ? VE : 1); ++e) {
                cwB[e] = sWt[n0 + e];
                cwC[e] = sWt[N + n0 + e];
                cbB[e] = sBias[r0 * N + n0 + e];
                cbC[e] = sBias[(RB + r0) * N + n0 + e];
            }
        }
    }
    if (nchunk > 0) load_chunk(0);
    for (int64_t c = 0; c < nchunk; ++c) {
        const float cd = nd, cl = nl, cdn = ndn, cln = nln;
        store_tiles();
        if (FUSED && c + 1 < nchunk) load_theta(c + 1);   // scanned at the end of this chunk's part 1
        if (c + 1 < nchunk) load_chunk(c + 1);   // the next chunk's loads fly during this one
        if (wave == 0) stage_scalars(cd, cl, cdn, cln);
        __syncthreads();
        const int64_t t0 = c * Q;

        // ---- part 1 -------------------------------------------------------------------------
        // X^T fragments of this wave's 16 columns, and w o X for the state update
        F xf[NIB], xw[NIB];
#pragma unroll
        for (int sb = 0; sb < NIB; ++sb) xf[sb] = MM::ldt(pX_t + 16 * sb * LDX, LDX, l16);
#pragma unroll
        for (int sb = 0; sb < NIB; ++sb) {
            floatx4 xs = MM::unpack(xf[sb]);
            const floatx4 ws = *(const floatx4*)(rW + 16 * sb + 4 * g);
#pragma unroll
            for (int m = 0; m < 4; ++m) xs[m] *= ws[m];
            xw[sb] = MM::pack(xs);
        }
        const float dec = rEl[QR - 1];
        floatx4 y[NIB], acc[NSLOT];
#pragma unroll
        for (int ib = 0; ib < NIB; ++ib) y[ib] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < NSLOT; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
        // Fragments of K block k: Cbar for every row block, the score tiles' Bbar and Cbar, and
        // Bbar^T for state rows 16k..16k+15.  Block k + 1 is read while block k computes; the
        // scheduling barriers keep each read one block ahead of its use and the live registers at
        // two blocks' worth.
        F fc[2][NIB], fsb[2][NSLOT], fsc[2][NSLOT], fbt[2][NIB];
        auto fetch = [&](int k, int s) {
#pragma unroll
            for (int ib = 0; ib < NIB; ++ib) fc[s][ib] = MM::ldk(pC_k + 16 * ib * LDC + 16 * k);
#pragma unroll
            for (int j = 0; j < NSLOT; ++j) {
                fsb[s][j] = MM::ldk(pSB[j] + 16 * k);
                fsc[s][j] = MM::ldk(pSC[j] + 16 * k);
            }
#pragma unroll
            for (int sb = 0; sb < NIB; ++sb) fbt[s][sb] = MM::ldt(pB_t + 16 * sb * LDB + 16 * k, LDB, l16);
        };
        fetch(0, 0);
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const int s = k & 1;
            __builtin_amdgcn_sched_barrier(0);
            if (k + 1 < NB) fetch(k + 1, s ^ 1);
            // state part of Y^T, K block k (state rows 16k.., before the update)
            const F sa = MM::pack(st[k]);
#pragma unroll
            for (int ib = 0; ib < NIB; ++ib) y[ib] = MM::mma(sa, fc[s][ib], y[ib]);
            // this wave's S^T tiles
#pragma unroll
            for (int j = 0; j < NSLOT; ++j) acc[j] = MM::mma(fsb[s][j], fsc[s][j], acc[j]);
            // state rows of N block k
#pragma unroll
            for (int m = 0; m < 4; ++m) st[k][m] *= dec;
#pragma unroll
            for (int sb = 0; sb < NIB; ++sb) st[k] = MM::mma(fbt[s][sb], xw[sb], st[k]);
        }
        __builtin_amdgcn_sched_barrier(0);
        // fused: angles of the next chunk (its staging reads them after the coming barrier)
        if (FUSED && c + 1 < nchunk) scan(c + 1);
        // mask the score tiles: lane holds S^T[s = 16 sb + 4 g + m][i = 16 ib + l16]
#pragma unroll
        for (int j = 0; j < NSLOT; ++j) {
            if (!sOn[j]) continue;
            const int i = 16 * sIb[j] + l16, s0 = 16 * sSb[j] + 4 * g;
            const int ti = i >> rl2;
            const float l2i = rL2[i], gi = rGam[i];
            const floatx4 l2s = *(const floatx4*)(rL2 + s0);
            const floatx4 mus = *(const floatx4*)(rMu + s0);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                // below the diagonal exp(l_t - l_s) mu_s, on it gamma_t, above it 0
                const int ts = (s0 + m) >> rl2;
                const float e = fast_exp2(fminf(l2i - l2s[m], 0.f)) * mus[m];
                const float below = ts < ti ? 1.f : 0.f;
                const float diag = ts == ti ? gi : 0.f;
                acc[j][m] *= fmaf(e, below, diag);
            }
            MM::st(sM + i * LDM + s0, MM::pack(acc[j]));
        }
#pragma unroll
        for (int ib = 0; ib < NIB; ++ib) {
            const float el = rEl[16 * ib + l16];
#pragma unroll
            for (int m = 0; m < 4; ++m) y[ib][m] *= el;
        }
        __syncthreads();

        // ---- part 2: Y^T += X^T M^T, mixing, stores ------------------------------------------
#pragma unroll
        for (int sb = 0; sb < NIB; ++sb)
#pragma unroll
            for (int ib = sb; ib < NIB; ++ib)
                y[ib] = MM::mma(xf[sb], MM::ldk(pM_k + 16 * ib * LDM + 16 * sb), y[ib]);
        const rsrc_t dY = make_rsrc(yg + t0 * ystep, tail_bytes(t0, ystep, yrow));
#pragma unroll
        for (int ib = 0; ib < NIB; ++ib) {
            // lane holds Y[(t, r) = i][p = 16 wave + 4 g + m]
            const int i = 16 * ib + l16;
            const int tl = i >> rl2, r = i & rmask;
            const int p = 16 * wave + 4 * g;
            floatx4 yv = y[ib];
            uint32_t off;
            if (mix) {
#pragma unroll
                for (int m = 0; m < 4; ++m) yv[m] = group_sum(yv[m] * wo[m], R);
                // one lane per step stores the mixed row; the others aim past the descriptor
                off = r == 0 ? (uint32_t)((tl * H * P + p) * (int)sizeof(T)) : 0x80000000u;
            } else {
                off = (uint32_t)(((tl * H * R + r) * P + p) * (int)sizeof(T));
            }
            store4(dY, off, yv, T{});
        }
    }

    // ---- outputs: final state and the last step's (Bbar, x) ------------------------------
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int m = 0; m < 4; ++m) a.h_out[(bh * N + 16 * nb + 4 * g + m) * P + pcol] = st[nb][m];
    if (L > 0) {
        // the last chunk's tiles are still in LDS (nothing is staged after it)
        const int tlast = (int)(L - 1 - (nchunk - 1) * Q);
        if (a.Bbar_last) {
            for (int e = tid; e < R * N; e += NT) {
                T v;
                if (FUSED) v = sB[(tlast * R + e / N) * LDB + e % N];   // rotated here, never in HBM
                else v = Bg[(L - 1) * HRN + e];
                ((T*)a.Bbar_last)[bh * R * N + e] = v;
            }
        }
        if (a.x_last)
            for (int e = tid; e < R * P; e += NT) ((T*)a.x_last)[bh * R * P + e] = Xg[(L - 1) * HRP + e];
        if (FUSED && a.phi_out)
            for (int k = tid; k < K; k += NT) a.phi_out[bh * K + k] = sPhi[(Q - 1) * LDPHI + k];
    }
}

template <typename T, int N, int P, bool FUSED>
hipError_t launch_np(const PrefillArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)(a.b * a.H)), block(P / 16 * 64);
    switch (a.Q * a.R) {
        case 16: hipLaunchKernelGGL((prefill_kernel<T, N, P, 1, FUSED>), grid, block, 0, s, a); break;
        case 32: hipLaunchKernelGGL((prefill_kernel<T, N, P, 2, FUSED>), grid, block, 0, s, a); break;
        case 48:
            if (FUSED) return hipErrorInvalidValue;
            hipLaunchKernelGGL((prefill_kernel<T, N, P, 3, false>), grid, block, 0, s, a);
            break;
        case 64: hipLaunchKernelGGL((prefill_kernel<T, N, P, 4, FUSED>), grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T, bool FUSED>
hipError_t launch_t(const PrefillArgs& a, hipStream_t s) {
    if (a.N == 16 && a.P == 16) return launch_np<T, 16, 16, FUSED>(a, s);
    if (a.N == 64 && a.P == 64) return launch_np<T, 64, 64, FUSED>(a, s);
    if (a.N == 128 && a.P == 64) return launch_np<T, 128, 64, FUSED>(a, s);
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
    return bf16_io ? launch_t<bf16, false>(a, s) : launch_t<float, false>(a, s);
}

bool layer_supported(int N, int P, int R, int QR, bool bf16_io) {
    // chunk rows 16, 32 or 64 (the angle scan wants a power-of-two step count); the 64-row tile
    // keeps the biases of at most 4 ranks in LDS
    return prefill_supported(N, P, R, QR, bf16_io) && QR != 48 && (QR < 48 || R <= 4);
}

hipError_t launch_layer(const PrefillArgs& a, bool bf16_io, hipStream_t s) {
    return bf16_io ? launch_t<bf16, true>(a, s) : launch_t<float, true>(a, s);
}

}  // namespace m3
