// backward.hip -- gradients of the layer core (m3_layer_chunk_states, m3_layer_backward).
//
// Forward being differentiated.  The fused layer core: BCNorm, head bias and cumulative rotation
// of B and C (papernotes.org summary, key design 4; aipaper.cc summary, section 4.2,
// Proposition 3), then the exponential-trapezoidal recurrence (aipaper.cc section 4.1,
// Proposition 1) with the MIMO rank-R update (section 4.3), run in chunks in its shifted-state
// form.  With c_t = (1 - lambda_t) dt_t, gamma_t = lambda_t dt_t, mu_t = gamma_t + c_{t+1} and,
// inside a chunk starting at t0, l_t = A sum_{t0 <= i <= t} dt_i:
//   Y_i   = sum_s L(i, s) (Cbar_i . Bbar_s) x_s + exp(l_i) Cbar_i S_in
//   S_out = exp(l_end) S_in + sum_s w_s Bbar_s^T x_s,           w_s = exp(l_end - l_s) mu_s
// where rows i, s are (step, rank) pairs and L(i, s) is exp(l_i - l_s) mu_s when s's step is
// before i's, gamma_i when the steps are equal, 0 after.  The pages give no backward pass; the
// kernels compute the exact gradient of this computation (the fp64 oracle's backward is the
// step-by-step gradient of the plain recurrence; the two agree because the chunked form is an
// exact reordering).
//
// Adjoint of one chunk, given dY (the output cotangent, w_out o dy when outputs are mixed) and
// dS_out (the state cotangent after the chunk), with S = Cbar Bbar^T and dP = dY X^T (QR x QR):
//   M1 = L o S,  dS = L o dP,  dL = dP o S
//   dX     = M1^T dY + diag(w) Bbar dS_out
//   dBbar  = dS^T Cbar + diag(w) X dS_out^T
//   dCbar  = dS Bbar + diag(exp(l)) dY S_in^T
//   dS_in  = exp(l_end) dS_out + Cbar^T diag(exp(l)) dY
// and for the per-step scalars (summed over ranks):
//   dmu_s   = sum_{i after s} exp(l_i - l_s) dL(i, s) + exp(l_end - l_s) dw_s
//   dgamma_t = sum over the step's diagonal block of dL
//   dl_i   += sum_{s before i} mu_s exp(l_i - l_s) dL(i, s) + exp(l_i) Cbar_i . (S_in dY_i)
//   dl_s   -= mu_s * (the first sum of dmu_s) + w_s dw_s
//   dl_end += sum_s w_s dw_s + exp(l_end) <dS_out, S_in>,   dw_s = Bbar_s . (dS_out x_s)
// then dl -> d(dt) and dA through the within-chunk prefix sum, and dgamma, dmu -> d(lambda),
// d(dt) (mu_t also reaches step t + 1, possibly in the next chunk).  The rotation and BCNorm are
// undone per row: dB~ = R(Phi) dBbar (the rotation's transpose undone), dPhi per pair from the
// rotated output, the RMS norm's Jacobian, and the angle's reverse prefix sum gives dtheta and the
// rotation's share of d(dt).
//
// Mapping on gfx950.  Three kernels per call (plus a small reduction):
//   chunk_states_kernel  one workgroup per (b, h) walks the chunks forward with the state in MFMA
//                        accumulators (as the forward prefill does) and writes each chunk's
//                        entry state S_in (io type, transposed [P][N]) and entry angle (fp32) to a
//                        workspace: the backward needs them in reverse order.
//   backward_kernel      one workgroup per (b, h) walks the chunks backward with dS in MFMA
//                        accumulators.  Wave w owns row block w of the chunk (16 rows) for dX, dBbar,
//                        dCbar and the recomputed Y, and P / (16 NW) column blocks of dS.  Every
//                        product above is one bf16 (or fp32) MFMA chain on LDS tiles; the
//                        elementwise rotation / norm adjoint runs on the gradient tiles after they
//                        are moved to LDS in fp32.  Per-(b, h) sums of the per-head parameters'
//                        gradients go to the workspace and are reduced over the batch in a fixed
//                        order (deterministic).  Each chunk's per-step sums of the scalar
//                        gradients' terms go to the workspace too:
//   step_grads_kernel    turns them into d(dt), d(lambda) and dA, every chunk independently, so
//                        that serial per-step work stays off the backward kernel's chunk chain.
#include <type_traits>

#include "m3_device.h"
#include "m3_launch.h"
#include "m3_mma.h"

namespace m3 {

namespace {

// WPB waves share each 16-row block of a chunk (the backward pass runs WPB = 2: two waves per
// SIMD, each with half of the row block's column blocks and half of the state tiles).
template <typename T, int N_, int P_, int NIB_, int R_, int WPB_ = 1>
struct Shape {
    static constexpr int N = N_, P = P_, NIB = NIB_, R = R_, WPB = WPB_;
    static constexpr int NW = NIB * WPB, NT = 64 * NW, QR = 16 * NIB, Q = QR / R;
    static constexpr int RL2 = R == 1 ? 0 : (R == 2 ? 1 : 2);
    static constexpr int NB = N / 16, PB = P / 16, PPW = PB / NW;
    // a wave's share of a row block's column work: PBH of the P blocks, NBH of the N blocks
    static constexpr int PBH = PB / WPB, NBH = NB / WPB;
    // a wave's tiles of the N x P state (cotangent): SCW column blocks of SRW row blocks each,
    // column group wave % NCG, row group wave / NCG
    static constexpr int SCW = PB >= NW ? PB / NW : 1, NCG = PB / SCW, SRW = NB / (NW / NCG);
    static_assert(PB % WPB == 0 && NB % WPB == 0, "column blocks per wave");
    static_assert(NCG * SCW == PB && (NW / NCG) * SRW == NB && NW % NCG == 0, "state tiles per wave");
    static constexpr int PADT = Mma<T>::PADT, PADK = Mma<T>::PADK;
    static constexpr int LDB = N + PADT, LDX = P + PADT, LDS = N + PADT, LDM = QR + PADT;
    // the backward kernel reads most of its tiles both along K and transposed, and no row padding
    // serves both without bank conflicts: the tiles read mostly along K (Bbar, Cbar, x, dY and the
    // entry state) take the K padding, the state cotangent and the score tiles the transposed one
    static constexpr int LDBK = N + PADK, LDXK = P + PADK, LDSK = N + PADK;
    static constexpr int VE = 16 / (int)sizeof(T), VPN = N / VE, VPP = P / VE;
    static constexpr int RKC = NT / VPN, RKX = NT / VPP;
    static constexpr int MAXC = (QR + RKC - 1) / RKC, MAXX = (QR + RKX - 1) / RKX;
    static constexpr bool FULLC = MAXC * RKC == QR, FULLX = MAXX * RKX == QR;
    static constexpr int MAXS = (P + RKC - 1) / RKC;          // state rows [p][n] staged like B rows
    static constexpr bool FULLS = MAXS * RKC == P;
    static constexpr int K = N / 2, VT = VE, NVT = K / VT;
    static constexpr int TPV0 = NT / NVT, TPV = Q < TPV0 ? Q : TPV0, SPT = Q / TPV;
    static constexpr int LDPHI = K + 4, LDF = N + 4, LDD = K + 4;
    // byte offsets of the backward kernel's tiles in its shared tile region
    static constexpr int SZB = QR * LDBK * (int)sizeof(T), SZX = QR * LDXK * (int)sizeof(T);
    static constexpr int SZSK = P * LDSK * (int)sizeof(T), SZS = P * LDS * (int)sizeof(T);
    static constexpr int SZM = QR * LDM * (int)sizeof(T);
    static constexpr int OFF_B = 0, OFF_C = SZB, OFF_X = 2 * SZB, OFF_Y = OFF_X + SZX, OFF_S = OFF_Y + SZX,
                         OFF_DS = OFF_S + SZSK, OFF_M1 = OFF_DS + SZS, OFF_DSC = OFF_M1 + SZM, TILES = OFF_DSC + SZM;
    // after the products the region holds the fp32 gradient rows and the per-row angle gradients
    static constexpr int OFF_FB = 0, OFF_FC = QR * LDF * 4, OFF_FPHI = 2 * QR * LDF * 4,
                         ALIAS = OFF_FPHI + QR * LDD * 4, FINAL = N * (P + 4) * 4;
    static_assert(NT % VPN == 0 && NT % VPP == 0 && RKC % R == 0 && RKX % R == 0, "staging layout");
    static_assert(NVT >= 1 && NVT * TPV <= NT && TPV <= 64 && (TPV & (TPV - 1)) == 0, "angle scan layout");
    static_assert(ALIAS <= TILES && FINAL <= TILES, "aliased LDS");
    // bf16 tiles of 64- or 128-element rows are stored unpadded with their 8-byte pieces permuted
    // per row (tile_off), which serves both the reads along K and the transposed reads without bank
    // conflicts; the other shapes keep the padded rows above (the tile sizes cover both).
    static constexpr bool SWZ = sizeof(T) == 2 && (N == 64 || N == 128) && P == 64 && QR == 64;
    // the score tiles (L o S, L o dP) lie past the gradient rows: their upper triangle, zeroed once
    // before the chunk loop, stays zero
    static_assert(ALIAS <= OFF_M1, "score tiles outside the aliased region");
    static_assert(R == 1 || R == 2 || R == 4, "rank");
};

// Raw B or C row vector (VE elements of row i, columns n0..) -> BCNorm, weight, bias, rotation
// by the row's angles; `inv` is the row's 1 / RMS (1 without BCNorm).  Also used to recompute the
// unrotated, normalised vector in the adjoint.
template <typename T, int VE>
__device__ __forceinline__ void norm_bias(const float (&v)[VE], float inv, const float* w, const float* bias,
                                          bool has_w, float (&vb)[VE]) {
    if (has_w) {
#pragma unroll
        for (int e = 0; e < VE; ++e) vb[e] = fmaf(v[e] * inv, w[e], bias[e]);
    } else {
#pragma unroll
        for (int e = 0; e < VE; ++e) vb[e] = fmaf(v[e], inv, bias[e]);
    }
}

// sum over aligned groups of W lanes of the squares of a row vector's pieces -> 1 / RMS
template <int VE>
__device__ __forceinline__ float row_inv_rms(const float (&v)[VE], int W, float invN, float eps) {
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < VE; ++e) part[e & 3] = fmaf(v[e], v[e], part[e & 3]);
    const float q = group_sum((part[0] + part[1]) + (part[2] + part[3]), W);
    return __builtin_amdgcn_rsqf(fmaxf(fmaf(q, invN, eps), 1e-30f));
}

template <typename T, int N, int P, int NIB, int R>
__global__ __launch_bounds__(NIB * 64, 1) void chunk_states_kernel(BackwardArgs a) {
    using S = Shape<T, N, P, NIB, R>;
    using MM = Mma<T>;
    using F = typename MM::frag;
    constexpr int NW = S::NW, NT = S::NT, QR = S::QR, Q = S::Q, RL2 = S::RL2, NB = S::NB, PPW = S::PPW;
    static_assert(S::WPB == 1 && S::PB % NW == 0, "state column blocks per wave");
    constexpr int LDB = S::LDB, LDX = S::LDX, VE = S::VE, VPN = S::VPN, VPP = S::VPP;
    constexpr int RKC = S::RKC, RKX = S::RKX, MAXC = S::MAXC, MAXX = S::MAXX;
    constexpr int K = S::K, VT = S::VT, NVT = S::NVT, TPV = S::TPV, SPT = S::SPT, LDPHI = S::LDPHI;

    __shared__ __align__(16) T sB[QR * LDB];
    __shared__ __align__(16) T sX[QR * LDX];
    __shared__ __align__(16) float sPhi[Q * LDPHI];
    __shared__ __align__(16) float rW[64];
    __shared__ float rDec;
    __shared__ __align__(16) float sWt[N], sBias[R * N];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, l16 = lane & 15;
    // heads that share raw B and C run on one XCD (consecutive items), so its L2 serves the group
    const int64_t bh = a.G > 0 && a.G < a.H ? xcd_item(blockIdx.x, gridDim.x) : (int64_t)blockIdx.x;
    const int64_t b = bh / a.H;
    const int h = (int)(bh % a.H);
    const int H = a.H;
    const int64_t L = a.L, nchunk = (L + Q - 1) / Q;
    const float Alog2 = a.A[h] * kLog2e;
    const int64_t row_bh = b * L * H + h;
    // raw B rows: the head's own, or its group slot's (GS slots per step, SBC elements per step)
    const int GS = bc_slots(H, a.G);
    const int64_t row_bc = b * L * GS + bc_slot(h, H, a.G);
    const int64_t SBC = (int64_t)GS * R * N, HRP = (int64_t)H * R * P, HK = (int64_t)H * K;
    const T* Xg = (const T*)a.x + row_bh * R * P;
    const T* Bg = (const T*)a.B + row_bc * R * N;
    const T* dtg = (const T*)a.dt + row_bh;
    const T* lamg = (const T*)a.lam + row_bh;
    const T* thg = (const T*)a.theta + row_bh * K;
    auto tail_bytes = [&](int64_t t0, int64_t step, int64_t row) {
        return clamp_bytes(((L - t0 - 1) * step + row) * (int64_t)sizeof(T));
    };
    typedef typename IoBits<T>::type Bits;

    for (int e = tid; e < N; e += NT) sWt[e] = a.bcnorm && a.normw_B ? a.normw_B[h * N + e] : 1.f;
    for (int e = tid; e < R * N; e += NT) sBias[e] = a.bias_B ? a.bias_B[h * R * N + e] : 0.f;

    // staging layout: thread moves 16-byte vectors of rows i = i0 + k * RK, column c0
    const int iC0 = tid / VPN, cC0 = tid % VPN, iX0 = tid / VPP, cX0 = tid % VPP;
    const int rC = iC0 & (R - 1);
    auto offC = [&](int k) {
        const int i = iC0 + k * RKC;
        return (uint32_t)(((i >> RL2) * (int)SBC + (i & (R - 1)) * N + cC0 * VE) * (int)sizeof(T));
    };
    auto offX = [&](int k) {
        const int i = iX0 + k * RKX;
        return (uint32_t)(((i >> RL2) * (int)HRP + (i & (R - 1)) * P + cX0 * VE) * (int)sizeof(T));
    };
    // angle layout: thread (tv, tj) scans pairs tv * VT .. over steps tj * SPT .. tj * SPT + SPT - 1
    const int tv = tid / TPV, tj = tid % TPV;
    const bool scanner = tid < NVT * TPV;
    float carry[VT];
#pragma unroll
    for (int e = 0; e < VT; ++e) {
        const int k = tv * VT + e;
        carry[e] = scanner && a.phi_in ? wrap_angle(a.phi_in[bh * K + k]) : 0.f;
    }

    // G_{-1} = h_in + c_0 Bbar_prev^T x_prev; wave w owns state columns p in blocks w * PPW ..
    floatx4 st[PPW][NB];
#pragma unroll
    for (int j = 0; j < PPW; ++j)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int p = 16 * (wave * PPW + j) + l16;
                st[j][nb][m] = a.h_in ? a.h_in[(bh * N + 16 * nb + 4 * g + m) * P + p] : 0.f;
            }
    if (a.Bbar_prev && a.x_prev && L > 0) {
        const float c0 = (1.0f - load_f32(lamg)) * load_f32(dtg);
        const T* Bp = (const T*)a.Bbar_prev + bh * R * N;
        const T* xp = (const T*)a.x_prev + bh * R * P;
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int j = 0; j < PPW; ++j) {
                const float xv = c0 * load_f32(xp + r * P + 16 * (wave * PPW + j) + l16);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int m = 0; m < 4; ++m) st[j][nb][m] += load_f32(Bp + r * N + 16 * nb + 4 * g + m) * xv;
            }
    }

    const float invN = 1.0f / (float)N;
    const bool has_w = a.bcnorm && a.normw_B;
    for (int64_t c = 0; c < nchunk; ++c) {
        const int64_t t0 = c * Q;
        // ---- loads
        uint4 rb[MAXC], rx[MAXX];
        {
            const rsrc_t dB = make_rsrc(Bg + t0 * SBC, tail_bytes(t0, SBC, (int64_t)R * N));
            const rsrc_t dX = make_rsrc(Xg + t0 * HRP, tail_bytes(t0, HRP, (int64_t)R * P));
#pragma unroll
            for (int k = 0; k < MAXC; ++k)
                rb[k] = buffer_load16_stream(dB, S::FULLC || iC0 + k * RKC < QR ? offC(k) : 0x80000000u);
#pragma unroll
            for (int k = 0; k < MAXX; ++k)
                rx[k] = buffer_load16_stream(dX, S::FULLX || iX0 + k * RKX < QR ? offX(k) : 0x80000000u);
        }
        uint4 rth[SPT];
        Bits rdt[SPT];
        {
            const rsrc_t dT = make_rsrc(thg + t0 * HK, tail_bytes(t0, HK, K));
            const rsrc_t dD = make_rsrc(dtg + t0 * H, tail_bytes(t0, H, 1));
#pragma unroll
            for (int s = 0; s < SPT; ++s) {
                const int t = tj * SPT + s;
                rth[s] = buffer_load16(dT, (uint32_t)((t * (int)HK + tv * VT) * (int)sizeof(T)));
                rdt[s] = buffer_load_bits(dD, (uint32_t)(t * H * (int)sizeof(T)), T{});
            }
        }
        Bits nd, nl, ndn, nln;
        {
            const rsrc_t dD = make_rsrc(dtg + t0 * H, tail_bytes(t0, H, 1));
            const rsrc_t dL = make_rsrc(lamg + t0 * H, tail_bytes(t0, H, 1));
            const uint32_t o0 = (uint32_t)(lane * H * (int)sizeof(T)), o1 = o0 + (uint32_t)(H * (int)sizeof(T));
            nd = buffer_load_bits(dD, o0, T{});
            nl = buffer_load_bits(dL, o0, T{});
            ndn = buffer_load_bits(dD, o1, T{});
            nln = buffer_load_bits(dL, o1, T{});
        }
        // ---- angles of the chunk; the entry angle is saved for the backward pass
        if (scanner) {
            if (tj == 0) {
                float* dst = a.ws_phi + (bh * nchunk + c) * K + tv * VT;
#pragma unroll
                for (int e = 0; e < VT; ++e) dst[e] = carry[e];
            }
            float acc[SPT][VT];
#pragma unroll
            for (int s = 0; s < SPT; ++s) {
                float f[VT];
                unpack16(rth[s], f, T{});
                const float d = bits_to_f32(rdt[s]);
#pragma unroll
                for (int e = 0; e < VT; ++e) acc[s][e] = (s ? acc[s - 1][e] : 0.f) + d * f[e];
            }
#pragma unroll
            for (int e = 0; e < VT; ++e) {
                const float tot = acc[SPT - 1][e];
                const float incl = seg_scan_add<TPV>(tot, lane);
                const float gtot = shfl(incl, (lane & ~(TPV - 1)) + TPV - 1);
                const float base = carry[e] + incl - tot;
#pragma unroll
                for (int s = 0; s < SPT; ++s) sPhi[(tj * SPT + s) * LDPHI + tv * VT + e] = wrap_angle(base + acc[s][e]);
                carry[e] = wrap_angle(carry[e] + gtot);
            }
        }
#pragma unroll
        for (int k = 0; k < MAXX; ++k) {
            const int i = iX0 + k * RKX;
            if (S::FULLX || i < QR) *(uint4*)(sX + i * LDX + cX0 * VE) = rx[k];
        }
        if (wave == NW - 1) {
            const float d = bits_to_f32(nd), lm = bits_to_f32(nl), dn = bits_to_f32(ndn), lmn = bits_to_f32(nln);
            const float l2 = wave_scan_add(d * Alog2);
            const float mu = lm * d + (1.0f - lmn) * dn;
            const float l2end = lane_value(l2, Q - 1);
            const float w = fast_exp2(fminf(l2end - l2, 0.f)) * mu;
            rW[lane] = shfl(w, lane >> RL2);
            if (lane == 0) rDec = fast_exp2(l2end);
        }
        __syncthreads();
        // ---- BCNorm + bias + rotation of B -> sB
#pragma unroll
        for (int k = 0; k < MAXC; ++k) {
            const int i = iC0 + k * RKC;
            float v[VE];
            unpack16(rb[k], v, T{});
            const float inv = a.bcnorm ? row_inv_rms<VE>(v, VPN, invN, a.eps) : 1.f;
            if (!(S::FULLC || i < QR)) continue;
            float vb[VE];
            norm_bias<T, VE>(v, inv, sWt + cC0 * VE, sBias + rC * N + cC0 * VE, has_w, vb);
            const float* ph = sPhi + (i >> RL2) * LDPHI + cC0 * VE / 2;
#pragma unroll
            for (int q = 0; q < VE / 2; ++q) {
                float sn, cs;
                __sincosf(ph[q], &sn, &cs);
                const float x0 = vb[2 * q], x1 = vb[2 * q + 1];
                vb[2 * q] = fmaf(cs, x0, sn * x1);
                vb[2 * q + 1] = fmaf(cs, x1, -sn * x0);
            }
            *(uint4*)(sB + i * LDB + cC0 * VE) = pack16(vb, T{});
        }
        __syncthreads();
        // ---- save the entry state (transposed, io type), then the update
        {
            T* dst = (T*)a.ws_states + (bh * nchunk + c) * (int64_t)P * N;
#pragma unroll
            for (int j = 0; j < PPW; ++j) {
                const int p = 16 * (wave * PPW + j) + l16;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) MM::st(dst + p * N + 16 * nb + 4 * g, MM::pack(st[j][nb]));
            }
        }
        const float dec = rDec;
        F xw[NIB][PPW];
#pragma unroll
        for (int sb = 0; sb < NIB; ++sb) {
            const floatx4 ws = *(const floatx4*)(rW + 16 * sb + 4 * g);
#pragma unroll
            for (int j = 0; j < PPW; ++j) {
                floatx4 xs = MM::unpack(MM::ldt(sX + (16 * sb + 4 * g) * LDX + 16 * (wave * PPW + j), LDX, l16));
#pragma unroll
                for (int m = 0; m < 4; ++m) xs[m] *= ws[m];
                xw[sb][j] = MM::pack(xs);
            }
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
            for (int j = 0; j < PPW; ++j)
#pragma unroll
                for (int m = 0; m < 4; ++m) st[j][nb][m] *= dec;
#pragma unroll
            for (int sb = 0; sb < NIB; ++sb) {
                const F bt = MM::ldt(sB + (16 * sb + 4 * g) * LDB + 16 * nb, LDB, l16);
#pragma unroll
                for (int j = 0; j < PPW; ++j) st[j][nb] = MM::mma(bt, xw[sb][j], st[j][nb]);
            }
        }
        __syncthreads();
    }
}

// Element offset of (row, col) in a bf16 tile of LD = 64 or 128 elements a row, stored unpadded
// with the row's 8-byte pieces (4 elements, col / 4) permuted by an XOR with
//   s(row) = 4 (row % 8) + 2 (row / 8 % 2)            (128-element rows, 32 pieces: one row per
//                                                      256-byte line of the 64 banks)
//   s(row) = 4 (row / 2 % 4) + 2 (row / 8 % 2)        (64-element rows, 16 pieces: two rows a line)
// The 32 lanes that one cycle serves read, along K, 16 rows x 2 pieces and, transposed, 8 rows x
// 4 pieces (a 16-row block and a 4-piece-aligned column): both land on 32 distinct piece slots.
// s is even, so the two pieces of a 16-byte store stay adjacent.  col is a multiple of 4.
// Transposed 16-bit read of one lane's 4 x 16-bit piece at p (the swizzled tiles give each lane
// its own address: the four rows a lane gathers are not a fixed stride apart).
__device__ __forceinline__ Mma<bf16>::frag ldt_lane_bf16(const bf16* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(lds_char*)p);
}

// Element (row, col) of a 16-bit LDS tile with LD elements per row.  Unswizzled (SWZ false) the
// rows are padded (LD includes the padding).  Swizzled, rows are unpadded and the row's 8-byte
// pieces (4 elements; piece q covers columns 4q .. 4q + 3) are permuted: piece q is stored at
// q ^ s(row).  LDS has 64 four-byte banks, i.e. 32 eight-byte bank pairs; an unpadded 128-element
// row starts on pair 0, a 64-element row on pair 0 or 16.  The products read two patterns: along
// K (16 rows x pieces 2g', 2g' + 1 per half-wave) and transposed (8 rows x 4 consecutive pieces per
// half-wave).  s(row) = 4 (row mod 8) + 2 ((row / 8) mod 2) for 128-element rows and
// 4 ((row / 2) mod 4) + 2 ((row / 8) mod 2) for 64-element rows sends both patterns to 32 distinct
// pairs, so neither conflicts; s is even, so a 16-byte write (pieces 2q', 2q' + 1) stays one
// contiguous 16-byte store.
template <bool SWZ, int LD>
__device__ __forceinline__ int tile_off(int row, int col) {
    if constexpr (!SWZ) {
        return row * LD + col;
    } else {
        static_assert(LD == 64 || LD == 128, "swizzled row length");
        const int s = LD == 128 ? 4 * (row & 7) + 2 * ((row >> 3) & 1) : 4 * ((row >> 1) & 3) + 2 * ((row >> 3) & 1);
        return row * LD + (((col >> 2) ^ s) << 2);
    }
}
// transposed fragment read of rows row0 .. row0 + 3 of each lane group (the caller's row0
// includes 4 g), columns col0 ..
template <bool SWZ, int LD, typename T>
__device__ __forceinline__ typename Mma<T>::frag tile_ldt(const T* tile, int row0, int col0, int l16) {
    if constexpr (SWZ) return ldt_lane_bf16(tile + tile_off<true, LD>(row0 + (l16 >> 2), col0 + 4 * (l16 & 3)));
    else return Mma<T>::ldt(tile + row0 * LD + col0, LD, l16);
}

template <typename T, int N, int P, int NIB, int R, int WPB>
__global__ __launch_bounds__(NIB * WPB * 64, 1) void backward_kernel(BackwardArgs a) {
    using S = Shape<T, N, P, NIB, R, WPB>;
    using MM = Mma<T>;
    using F = typename MM::frag;
    constexpr int NW = S::NW, NT = S::NT, QR = S::QR, Q = S::Q, RL2 = S::RL2, NB = S::NB, PB = S::PB;
    constexpr int PBH = S::PBH, NBH = S::NBH, SCW = S::SCW, SRW = S::SRW, NCG = S::NCG;
    constexpr bool SWZ = S::SWZ;   // see tile_off
    constexpr int LDB = SWZ ? N : S::LDBK, LDX = SWZ ? P : S::LDXK, LDSS = SWZ ? N : S::LDSK, LDS = SWZ ? N : S::LDS,
                  LDM = SWZ ? QR : S::LDM, VE = S::VE, VPN = S::VPN, VPP = S::VPP;
    constexpr int RKC = S::RKC, RKX = S::RKX, MAXC = S::MAXC, MAXX = S::MAXX, MAXS = S::MAXS;
    constexpr int K = S::K, VT = S::VT, NVT = S::NVT, TPV = S::TPV, SPT = S::SPT, LDPHI = S::LDPHI,
                  LDF = S::LDF, LDD = S::LDD;
    constexpr int NTILE = NIB * (NIB + 1) / 2, NSLOT = (NTILE + NW - 1) / NW;

    __shared__ __align__(16) char tiles[S::TILES];
    T* sB = (T*)(tiles + S::OFF_B);      // rotated B rows      [s][n]
    T* sC = (T*)(tiles + S::OFF_C);      // rotated C rows      [i][n]
    T* sX = (T*)(tiles + S::OFF_X);      // x rows              [s][p]
    T* sDY = (T*)(tiles + S::OFF_Y);     // dY rows             [i][p]
    T* sSt = (T*)(tiles + S::OFF_S);     // entry state         [p][n]
    T* sDSt = (T*)(tiles + S::OFF_DS);   // state cotangent     [p][n]
    T* sM1 = (T*)(tiles + S::OFF_M1);    // L o S               [i][s]
    T* sDS = (T*)(tiles + S::OFF_DSC);   // L o dP              [i][s]
    float* fB = (float*)(tiles + S::OFF_FB);      // dBbar rows (fp32)  [s][n]   (after the products)
    float* fC = (float*)(tiles + S::OFF_FC);      // dCbar rows (fp32)  [i][n]
    float* fPhi = (float*)(tiles + S::OFF_FPHI);  // per-row angle gradients [i][k]
    __shared__ __align__(16) float sPhi[Q * LDPHI];
    // per-row (t, r) scalars of the chunk
    __shared__ __align__(16) float rL2[64], rEl[64], rGam[64], rMu[64], rW[64];
    __shared__ float rEnd[2];   // l_end (log2 units), exp(l_end)
    // per-row partial gradients (per wave where several waves add to a row)
    __shared__ __align__(16) float pMu[NW * 64], pLi[NW * 64], pGam[NW * 64], rDw[WPB * 64], rDlo[WPB * 64];
    __shared__ float pSS[NW], red[NW];
    __shared__ __align__(16) float rotdd[NVT * 64];
    __shared__ __align__(16) float sWt[2 * N], sBias[2 * R * N], sWo[R * P];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, l16 = lane & 15;
    constexpr bool kAllBlocks = sizeof(T) == 4;   // see the score-tile zeroing below
    // row block rbw of the chunk (16 rows), half hf of its column work; state tiles: column group
    // cg, row group rg
    const int rbw = wave % NIB, hf = wave / NIB, cg = wave % NCG, rg = wave / NCG;
    // heads that share raw B and C run on one XCD (consecutive items), so its L2 serves the group
    const int64_t bh = a.G > 0 && a.G < a.H ? xcd_item(blockIdx.x, gridDim.x) : (int64_t)blockIdx.x;
    const int64_t b = bh / a.H;
    const int h = (int)(bh % a.H);
    const int H = a.H;
    const int64_t L = a.L, nchunk = (L + Q - 1) / Q;
    const float A = a.A[h], Alog2 = A * kLog2e;
    const int64_t row_bh = b * L * H + h;
    // raw B and C rows: the head's own, or its group slot's (GS slots per step, SBC elements per
    // step); their gradient rows have the same layout
    const int GS = bc_slots(H, a.G);
    const int64_t row_bc = b * L * GS + bc_slot(h, H, a.G);
    const int64_t SBC = (int64_t)GS * R * N, HRP = (int64_t)H * R * P, HK = (int64_t)H * K;
    const bool mix = a.w_out != nullptr;
    const int64_t ystep = mix ? (int64_t)H * P : HRP, yrow = mix ? P : (int64_t)R * P;
    const T* Xg = (const T*)a.x + row_bh * R * P;
    const T* Bg = (const T*)a.B + row_bc * R * N;
    const T* Cg = (const T*)a.C + row_bc * R * N;
    const T* dtg = (const T*)a.dt + row_bh;
    const T* lamg = (const T*)a.lam + row_bh;
    const T* thg = (const T*)a.theta + row_bh * K;
    const T* dyg = (const T*)a.dy + row_bh * yrow;
    T* dXg = (T*)a.dx + row_bh * R * P;
    // dB, dC rows: the call's outputs (one slot per head), or, with head groups, this head's
    // plane of the workspace (plane h mod H/G, each plane in the grouped layout), which
    // group_sum_kernel adds up per group afterwards
    const int64_t plane = a.ws_dB ? (int64_t)(h % (H / GS)) * a.b * L * GS * R * N : 0;
    T* dBg = (a.ws_dB ? (T*)a.ws_dB + plane : (T*)a.dB) + row_bc * R * N;
    T* dCg = (a.ws_dC ? (T*)a.ws_dC + plane : (T*)a.dC) + row_bc * R * N;
    T* dthg = (T*)a.dtheta + row_bh * K;
    auto tail_bytes = [&](int64_t t0, int64_t step, int64_t row) {
        return clamp_bytes(((L - t0 - 1) * step + row) * (int64_t)sizeof(T));
    };
    typedef typename IoBits<T>::type Bits;

    for (int e = tid; e < 2 * N; e += NT) {
        const float* w = e < N ? a.normw_B : a.normw_C;
        sWt[e] = a.bcnorm && w ? w[h * N + (e % N)] : 1.f;
    }
    for (int e = tid; e < 2 * R * N; e += NT) {
        const int which = e / (R * N), rn = e % (R * N);
        const float* bias = which == 0 ? a.bias_B : a.bias_C;
        sBias[e] = bias ? bias[h * R * N + rn] : 0.f;
    }
    for (int e = tid; e < NW * 64; e += NT) pMu[e] = pLi[e] = pGam[e] = 0.f;
    // fp32: the products that take a row block's score tiles run over every block, those above
    // the diagonal included, which S4 never writes and which therefore hold zeros.  Skipping those
    // blocks by a branch on the wave's row block let the compiler copy an accumulator out of its
    // MFMA chain at the join with too few wait states on the skipping path (an 8-pass fp32 MFMA
    // needs about ten), which then read it before the chain's last product had landed.  The bf16
    // instances keep the branches (their compiled code has no such read; a host test scans the
    // compiled kernels for it).
    if constexpr (kAllBlocks)
        for (int e = tid; e < 2 * S::SZM / 4; e += NT) ((uint32_t*)(tiles + S::OFF_M1))[e] = 0u;

    // ---- staging layout (B, C, state rows: vectors of rows iC0 + k RKC; x, dY: iX0 + k RKX); the
    // chunk loop derives it and its row offsets from the thread index itself, the sums after the
    // loop use the B/C rows' part
    const int iC0 = tid / VPN, cC0 = tid % VPN;
    const int rC = iC0 & (R - 1);
    // w_out of this head for the dY staging, read from LDS in the chunk loop (kept in registers,
    // the compiler spilled it)
    for (int e = tid; e < R * P; e += NT) sWo[e] = mix ? a.w_out[h * R * P + e] : 1.f;

    // ---- angle layout and the running angle cotangent (starts at dphi_out)
    const int tv = tid / TPV, tj = tid % TPV;
    const bool scanner = tid < NVT * TPV;
    float dcarry[VT];
#pragma unroll
    for (int e = 0; e < VT; ++e) dcarry[e] = scanner && a.dphi_out ? a.dphi_out[bh * K + tv * VT + e] : 0.f;

    // ---- state cotangent (starts at dh_out): the wave's tiles, column blocks cg SCW + j of row
    // blocks rg SRW + i
    floatx4 st[SCW][SRW];
#pragma unroll
    for (int j = 0; j < SCW; ++j)
#pragma unroll
        for (int i = 0; i < SRW; ++i)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int p = 16 * (cg * SCW + j) + l16, n = 16 * (rg * SRW + i) + 4 * g + m;
                st[j][i][m] = a.dh_out ? a.dh_out[(bh * N + n) * P + p] : 0.f;
            }

    // per-thread sums over the sequence: BCNorm weight and bias gradients of the thread's columns
    // (its rows all have rank rC), the mixing-weight gradient of the lane's (rank, columns)
    float accW[2][VE], accBias[2][VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) accW[0][e] = accW[1][e] = accBias[0][e] = accBias[1][e] = 0.f;
    floatx4 accMix[PBH];
#pragma unroll
    for (int pb = 0; pb < PBH; ++pb) accMix[pb] = floatx4{0.f, 0.f, 0.f, 0.f};

    const float invN = 1.0f / (float)N;
    const bool has_w = a.bcnorm && (a.normw_B || a.normw_C);

    // score tiles of this wave: tau = wave, wave + NW, ... (a spare slot recomputes the last tile)
    int sIb[NSLOT], sSb[NSLOT];
    bool sOn[NSLOT];
#pragma unroll
    for (int j = 0; j < NSLOT; ++j) {
        const int tau0 = wave + NW * j;
        sOn[j] = tau0 < NTILE;
        const int tau = sOn[j] ? tau0 : NTILE - 1;
        sIb[j] = tile_ib(tau);
        sSb[j] = tau - sIb[j] * (sIb[j] + 1) / 2;
    }

    for (int64_t c = nchunk - 1; c >= 0; --c) {
        // The thread-index arithmetic is redone each chunk from an opaque copy of the index (a
        // register move the compiler cannot look through): hoisted out of the loop, the offsets
        // were kept in scratch memory and reloaded every chunk, a memory round trip per use that
        // one wave per SIMD cannot hide; recomputed, each costs a few VALU instructions.
        int tid_o;
        asm volatile("v_mov_b32 %0, %1" : "=v"(tid_o) : "v"(tid));
        const int tid = tid_o, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
        const int iC0 = tid / VPN, cC0 = tid % VPN, iX0 = tid / VPP, cX0 = tid % VPP;
        const int rC = iC0 & (R - 1);
        const int tv = tid / TPV, tj = tid % TPV;
        const bool scanner = tid < NVT * TPV;
        const int wrow = 16 * rbw + l16;   // this lane's chunk row in the wave's row block
        auto offC = [&](int k) {
            const int i = iC0 + k * RKC;
            return (uint32_t)(((i >> RL2) * (int)SBC + (i & (R - 1)) * N + cC0 * VE) * (int)sizeof(T));
        };
        auto offX = [&](int k) {
            const int i = iX0 + k * RKX;
            return (uint32_t)(((i >> RL2) * (int)HRP + (i & (R - 1)) * P + cX0 * VE) * (int)sizeof(T));
        };
        auto offY = [&](int k) {   // dy: mixed rows are per step
            const int i = iX0 + k * RKX;
            return mix ? (uint32_t)(((i >> RL2) * H * P + cX0 * VE) * (int)sizeof(T)) : offX(k);
        };
        const int64_t t0 = c * Q;
        // ================= S1: loads ===================================================
        uint4 rb[MAXC], rc[MAXC], rx[MAXX], ry[MAXX], rs[MAXS];
        {
            const uint32_t nbc = tail_bytes(t0, SBC, (int64_t)R * N);
            const rsrc_t dB = make_rsrc(Bg + t0 * SBC, nbc), dC = make_rsrc(Cg + t0 * SBC, nbc);
            const rsrc_t dX = make_rsrc(Xg + t0 * HRP, tail_bytes(t0, HRP, (int64_t)R * P));
            const rsrc_t dYr = make_rsrc(dyg + t0 * ystep, tail_bytes(t0, ystep, yrow));
            const rsrc_t dS = make_rsrc((const T*)a.ws_states + (bh * nchunk + c) * (int64_t)P * N,
                                        (uint32_t)(P * N * (int)sizeof(T)));
#pragma unroll
            for (int k = 0; k < MAXC; ++k) {
                const bool in = S::FULLC || iC0 + k * RKC < QR;
                rb[k] = buffer_load16(dB, in ? offC(k) : 0x80000000u);
                rc[k] = buffer_load16(dC, in ? offC(k) : 0x80000000u);
            }
#pragma unroll
            for (int k = 0; k < MAXX; ++k) {
                const bool in = S::FULLX || iX0 + k * RKX < QR;
                rx[k] = buffer_load16_stream(dX, in ? offX(k) : 0x80000000u);
                ry[k] = buffer_load16_stream(dYr, in ? offY(k) : 0x80000000u);
            }
#pragma unroll
            for (int k = 0; k < MAXS; ++k) {
                const int p = iC0 + k * RKC;
                rs[k] = buffer_load16(dS, S::FULLS || p < P ? (uint32_t)((p * N + cC0 * VE) * (int)sizeof(T)) : 0x80000000u);
            }
        }
        uint4 rth[SPT];
        Bits rdt[SPT];
        float phin[VT];
        {
            const rsrc_t dT = make_rsrc(thg + t0 * HK, tail_bytes(t0, HK, K));
            const rsrc_t dD = make_rsrc(dtg + t0 * H, tail_bytes(t0, H, 1));
#pragma unroll
            for (int s = 0; s < SPT; ++s) {
                const int t = tj * SPT + s;
                rth[s] = buffer_load16(dT, (uint32_t)((t * (int)HK + tv * VT) * (int)sizeof(T)));
                rdt[s] = buffer_load_bits(dD, (uint32_t)(t * H * (int)sizeof(T)), T{});
            }
            const float* src = a.ws_phi + (bh * nchunk + c) * K + (scanner ? tv * VT : 0);
#pragma unroll
            for (int e = 0; e < VT; ++e) phin[e] = src[e];
        }
        Bits nd, nl, ndn, nln;
        {
            const rsrc_t dD = make_rsrc(dtg + t0 * H, tail_bytes(t0, H, 1));
            const rsrc_t dL = make_rsrc(lamg + t0 * H, tail_bytes(t0, H, 1));
            const uint32_t o0 = (uint32_t)(lane * H * (int)sizeof(T)), o1 = o0 + (uint32_t)(H * (int)sizeof(T));
            nd = buffer_load_bits(dD, o0, T{});
            nl = buffer_load_bits(dL, o0, T{});
            ndn = buffer_load_bits(dD, o1, T{});
            nln = buffer_load_bits(dL, o1, T{});
        }
        // dy of the lane's rows and columns for the mixing-weight gradient
        uint4 dyv[PBH];
        if (mix) {
            const rsrc_t dYr = make_rsrc(dyg + t0 * ystep, tail_bytes(t0, ystep, yrow));
            const int t = wrow >> RL2;
#pragma unroll
            for (int pb = 0; pb < PBH; ++pb) {
                const uint32_t off = (uint32_t)((t * H * P + 16 * (hf * PBH + pb) + 4 * g) * (int)sizeof(T));
                if constexpr (sizeof(T) == 2) {
                    const uint2 u = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(dYr, (int)off, 0, 0));
                    dyv[pb] = make_uint4(u.x, u.y, 0u, 0u);
                } else {
                    dyv[pb] = buffer_load16(dYr, off);
                }
            }
        }

        // ================= S2: angles, tiles, scalars ==================================
        if (scanner) {
            float acc[SPT][VT];
#pragma unroll
            for (int s = 0; s < SPT; ++s) {
                float f[VT];
                unpack16(rth[s], f, T{});
                const float d = bits_to_f32(rdt[s]);
#pragma unroll
                for (int e = 0; e < VT; ++e) acc[s][e] = (s ? acc[s - 1][e] : 0.f) + d * f[e];
            }
#pragma unroll
            for (int e = 0; e < VT; ++e) {
                const float tot = acc[SPT - 1][e];
                const float base = phin[e] + seg_scan_add<TPV>(tot, lane) - tot;
#pragma unroll
                for (int s = 0; s < SPT; ++s) sPhi[(tj * SPT + s) * LDPHI + tv * VT + e] = wrap_angle(base + acc[s][e]);
            }
        }
#pragma unroll
        for (int k = 0; k < MAXX; ++k) {
            const int i = iX0 + k * RKX;
            if (!(S::FULLX || i < QR)) continue;
            *(uint4*)(sX + tile_off<SWZ, LDX>(i, cX0 * VE)) = rx[k];
            if (mix) {
                float f[VE];
                unpack16(ry[k], f, T{});
#pragma unroll
                for (int e = 0; e < VE; ++e) f[e] *= sWo[(i & (R - 1)) * P + cX0 * VE + e];
                *(uint4*)(sDY + tile_off<SWZ, LDX>(i, cX0 * VE)) = pack16(f, T{});
            } else {
                *(uint4*)(sDY + tile_off<SWZ, LDX>(i, cX0 * VE)) = ry[k];
            }
        }
#pragma unroll
        for (int k = 0; k < MAXS; ++k) {
            const int p = iC0 + k * RKC;
            if (S::FULLS || p < P) *(uint4*)(sSt + tile_off<SWZ, LDSS>(p, cC0 * VE)) = rs[k];
        }
#pragma unroll
        for (int j = 0; j < SCW; ++j) {
            const int p = 16 * (cg * SCW + j) + l16;
#pragma unroll
            for (int i = 0; i < SRW; ++i) MM::st(sDSt + tile_off<SWZ, LDS>(p, 16 * (rg * SRW + i) + 4 * g), MM::pack(st[j][i]));
        }
        const float cd = bits_to_f32(nd), cl = bits_to_f32(nl), cdn = bits_to_f32(ndn), cln = bits_to_f32(nln);
        if (wave == NW - 1) {
            const float l2 = wave_scan_add(cd * Alog2);
            const float gam = cl * cd;
            const float mu = gam + (1.0f - cln) * cdn;
            const float l2end = lane_value(l2, Q - 1);
            const float el = fast_exp2(l2);
            const float w = fast_exp2(fminf(l2end - l2, 0.f)) * mu;
            if constexpr (R == 1) {   // row = step
                rL2[lane] = l2;
                rGam[lane] = gam;
                rMu[lane] = mu;
                rEl[lane] = el;
                rW[lane] = w;
            } else {                  // row s holds step s >> RL2
                const int ts = lane >> RL2;
                rL2[lane] = shfl(l2, ts);
                rGam[lane] = shfl(gam, ts);
                rMu[lane] = shfl(mu, ts);
                rEl[lane] = shfl(el, ts);
                rW[lane] = shfl(w, ts);
            }
            if (lane == 0) {
                rEnd[0] = l2end;
                rEnd[1] = fast_exp2(l2end);
            }
        }
        __syncthreads();   // (1)

        // ================= S3: BCNorm + bias + rotation of B and C -> sB, sC ===========
        float inv[MAXC][2];
#pragma unroll
        for (int k = 0; k < MAXC; ++k) {
            const int i = iC0 + k * RKC;
            float v[2][VE];
            unpack16(rb[k], v[0], T{});
            unpack16(rc[k], v[1], T{});
#pragma unroll
            for (int which = 0; which < 2; ++which)
                inv[k][which] = a.bcnorm ? row_inv_rms<VE>(v[which], VPN, invN, a.eps) : 1.f;
            if (!(S::FULLC || i < QR)) continue;
            float cs[VE / 2], sn[VE / 2];
            const float* ph = sPhi + (i >> RL2) * LDPHI + cC0 * VE / 2;
#pragma unroll
            for (int q = 0; q < VE / 2; ++q) __sincosf(ph[q], &sn[q], &cs[q]);
#pragma unroll
            for (int which = 0; which < 2; ++which) {
                float vb[VE];
                norm_bias<T, VE>(v[which], inv[k][which], sWt + which * N + cC0 * VE,
                                 sBias + (which * R + rC) * N + cC0 * VE, has_w, vb);
#pragma unroll
                for (int q = 0; q < VE / 2; ++q) {
                    const float x0 = vb[2 * q], x1 = vb[2 * q + 1];
                    vb[2 * q] = fmaf(cs[q], x0, sn[q] * x1);
                    vb[2 * q + 1] = fmaf(cs[q], x1, -sn[q] * x0);
                }
                *(uint4*)((which == 0 ? sB : sC) + tile_off<SWZ, LDB>(i, cC0 * VE)) = pack16(vb, T{});
            }
        }
        __syncthreads();   // (2)

        // ================= S4: products that need only the staged tiles ================
        // score tiles S^T and dP^T (lane: s = 16 sb + 4 g + m, i = 16 ib + l16), masks
#pragma unroll
        for (int j = 0; j < NSLOT; ++j) {
            if (!sOn[j]) continue;
            const int ib = sIb[j], sb = sSb[j];
            floatx4 sv = {0.f, 0.f, 0.f, 0.f}, dv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NB; ++kb)
                sv = MM::mma(MM::ldk(sB + tile_off<SWZ, LDB>(16 * sb + l16, 16 * kb + 4 * g)),
                             MM::ldk(sC + tile_off<SWZ, LDB>(16 * ib + l16, 16 * kb + 4 * g)), sv);
#pragma unroll
            for (int kb = 0; kb < PB; ++kb)
                dv = MM::mma(MM::ldk(sX + tile_off<SWZ, LDX>(16 * sb + l16, 16 * kb + 4 * g)),
                             MM::ldk(sDY + tile_off<SWZ, LDX>(16 * ib + l16, 16 * kb + 4 * g)), dv);
            const int i = 16 * ib + l16, s0 = 16 * sb + 4 * g;
            const int ti = i >> RL2;
            const float l2i = rL2[i], gi = rGam[i];
            const floatx4 l2s = *(const floatx4*)(rL2 + s0);
            const floatx4 mus = *(const floatx4*)(rMu + s0);
            floatx4 m1, ds;
            float li = 0.f, gsum = 0.f;
            floatx4 emu;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int ts = (s0 + m) >> RL2;
                const float e = fast_exp2(fminf(l2i - l2s[m], 0.f));
                const bool below = ts < ti, diag = ts == ti;
                const float lm = below ? e * mus[m] : (diag ? gi : 0.f);
                m1[m] = lm * sv[m];
                ds[m] = lm * dv[m];
                const float dl = dv[m] * sv[m];
                const float E = below ? e * dl : 0.f;
                emu[m] = E;
                li = fmaf(mus[m], E, li);
                gsum += diag ? dl : 0.f;
            }
            MM::st(sM1 + tile_off<SWZ, LDM>(i, s0), MM::pack(m1));
            MM::st(sDS + tile_off<SWZ, LDM>(i, s0), MM::pack(ds));
            // row i: sums over s (m in the lane, then the four lane groups)
            li += shfl_xor(li, 16);
            li += shfl_xor(li, 32);
            gsum += shfl_xor(gsum, 16);
            gsum += shfl_xor(gsum, 32);
            if (g == 0) {
                pLi[wave * 64 + i] += li;
                pGam[wave * 64 + i] += gsum;
            }
            // column s: sums over i (the 16 lanes of a row group)
#pragma unroll
            for (int m = 0; m < 4; ++m) emu[m] = group_sum(emu[m], 16);
            if (l16 == 0) {
#pragma unroll
                for (int m = 0; m < 4; ++m) pMu[wave * 64 + s0 + m] += emu[m];
            }
        }
        // dX^T (rows p in this wave's column blocks, columns s in its row block): first the state
        // part w_s dS_out^T Bbar^T
        floatx4 dxa[PBH];
#pragma unroll
        for (int pb = 0; pb < PBH; ++pb) {
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NB; ++kb)
                acc = MM::mma(MM::ldk(sDSt + tile_off<SWZ, LDS>(16 * (hf * PBH + pb) + l16, 16 * kb + 4 * g)),
                              MM::ldk(sB + tile_off<SWZ, LDB>(wrow, 16 * kb + 4 * g)), acc);
            const float ws = rW[wrow];
#pragma unroll
            for (int m = 0; m < 4; ++m) acc[m] *= ws;
            dxa[pb] = acc;
        }
        // dBbar^T (rows n in this wave's half, columns s = the row block): Z = dS_out X^T,
        // dw_s = Bbar_s . Z_s (this half's share; the halves are added in the scalar step)
        floatx4 dba[NBH];
        {
            float dw = 0.f;
#pragma unroll
            for (int nb = 0; nb < NBH; ++nb) {
                const int nbg = hf * NBH + nb;
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < PB; ++kb)
                    acc = MM::mma(tile_ldt<SWZ, LDS>(sDSt, 16 * kb + 4 * g, 16 * nbg, l16),
                                  MM::ldk(sX + tile_off<SWZ, LDX>(wrow, 16 * kb + 4 * g)), acc);
                const floatx4 bv = MM::unpack(MM::ldk(sB + tile_off<SWZ, LDB>(wrow, 16 * nbg + 4 * g)));
#pragma unroll
                for (int m = 0; m < 4; ++m) dw = fmaf(bv[m], acc[m], dw);
                dba[nb] = acc;
            }
            dw += shfl_xor(dw, 16);
            dw += shfl_xor(dw, 32);
            if (g == 0) rDw[hf * 64 + wrow] = dw;
            const float ws = rW[wrow];
#pragma unroll
            for (int nb = 0; nb < NBH; ++nb)
#pragma unroll
                for (int m = 0; m < 4; ++m) dba[nb][m] *= ws;
        }
        // dCbar^T (rows n, columns i = this wave's rows): exp(l_i) S_in dY_i, and
        // dl_i += Cbar_i . that
        floatx4 dca[NBH];
        {
            const float el = rEl[wrow];
            float dlo = 0.f;
#pragma unroll
            for (int nb = 0; nb < NBH; ++nb) {
                const int nbg = hf * NBH + nb;
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < PB; ++kb)
                    acc = MM::mma(tile_ldt<SWZ, LDSS>(sSt, 16 * kb + 4 * g, 16 * nbg, l16),
                                  MM::ldk(sDY + tile_off<SWZ, LDX>(wrow, 16 * kb + 4 * g)), acc);
                const floatx4 cv = MM::unpack(MM::ldk(sC + tile_off<SWZ, LDB>(wrow, 16 * nbg + 4 * g)));
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    acc[m] *= el;
                    dlo = fmaf(cv[m], acc[m], dlo);
                }
                dca[nb] = acc;
            }
            dlo += shfl_xor(dlo, 16);
            dlo += shfl_xor(dlo, 32);
            if (g == 0) rDlo[hf * 64 + wrow] = dlo;
        }
        // recomputed Y^T (rows p in this wave's column blocks, columns i = the row block), state
        // part, when mixing
        floatx4 ya[PBH];
        if (mix) {
            const float el = rEl[wrow];
#pragma unroll
            for (int pb = 0; pb < PBH; ++pb) {
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < NB; ++kb)
                    acc = MM::mma(MM::ldk(sSt + tile_off<SWZ, LDSS>(16 * (hf * PBH + pb) + l16, 16 * kb + 4 * g)),
                                  MM::ldk(sC + tile_off<SWZ, LDB>(wrow, 16 * kb + 4 * g)), acc);
#pragma unroll
                for (int m = 0; m < 4; ++m) acc[m] *= el;
                ya[pb] = acc;
            }
        }
        // <dS_out, S_in> over this wave's state tiles
        {
            float ss = 0.f;
#pragma unroll
            for (int j = 0; j < SCW; ++j) {
                const int p = 16 * (cg * SCW + j) + l16;
#pragma unroll
                for (int i = 0; i < SRW; ++i) {
                    const floatx4 sv = MM::unpack(MM::ldk(sSt + tile_off<SWZ, LDSS>(p, 16 * (rg * SRW + i) + 4 * g)));
#pragma unroll
                    for (int m = 0; m < 4; ++m) ss = fmaf(st[j][i][m], sv[m], ss);
                }
            }
            ss = group_sum(ss, 64);
            if (lane == 0) pSS[wave] = ss;
        }
        __syncthreads();   // (3)

        // ================= S5: products with the masked score tiles; state cotangent ===
        // dX^T += dY^T M1 (i blocks at or after this wave's s block)
#pragma unroll
        for (int pb = 0; pb < PBH; ++pb)
#pragma unroll
            for (int ib = 0; ib < NIB; ++ib)
                if (kAllBlocks || ib >= rbw)   // fp32: every block (zero tiles past the triangle)
                    dxa[pb] = MM::mma(tile_ldt<SWZ, LDX>(sDY, 16 * ib + 4 * g, 16 * (hf * PBH + pb), l16),
                                      tile_ldt<SWZ, LDM>(sM1, 16 * ib + 4 * g, 16 * rbw, l16), dxa[pb]);
        // dBbar^T += Cbar^T dS
#pragma unroll
        for (int nb = 0; nb < NBH; ++nb)
#pragma unroll
            for (int ib = 0; ib < NIB; ++ib)
                if (kAllBlocks || ib >= rbw)   // fp32: every block (zero tiles past the triangle)
                    dba[nb] = MM::mma(tile_ldt<SWZ, LDB>(sC, 16 * ib + 4 * g, 16 * (hf * NBH + nb), l16),
                                      tile_ldt<SWZ, LDM>(sDS, 16 * ib + 4 * g, 16 * rbw, l16), dba[nb]);
        // dCbar^T += Bbar^T dS^T (s blocks at or before this wave's i block)
#pragma unroll
        for (int nb = 0; nb < NBH; ++nb)
#pragma unroll
            for (int sb = 0; sb < NIB; ++sb)
                if (kAllBlocks || sb <= rbw)   // fp32: every block (zero tiles past the triangle)
                    dca[nb] = MM::mma(tile_ldt<SWZ, LDB>(sB, 16 * sb + 4 * g, 16 * (hf * NBH + nb), l16),
                                      MM::ldk(sDS + tile_off<SWZ, LDM>(wrow, 16 * sb + 4 * g)), dca[nb]);
        // recomputed Y^T += X^T M1^T; mixing-weight gradient sum_t Y[t, r, p] dy[t, p]
        if (mix) {
#pragma unroll
            for (int pb = 0; pb < PBH; ++pb) {
#pragma unroll
                for (int sb = 0; sb < NIB; ++sb)
                    if (kAllBlocks || sb <= rbw)   // fp32: every block (zero tiles past the triangle)
                        ya[pb] = MM::mma(tile_ldt<SWZ, LDX>(sX, 16 * sb + 4 * g, 16 * (hf * PBH + pb), l16),
                                         MM::ldk(sM1 + tile_off<SWZ, LDM>(wrow, 16 * sb + 4 * g)), ya[pb]);
                float f[VE];
                unpack16(dyv[pb], f, T{});
#pragma unroll
                for (int m = 0; m < 4; ++m) accMix[pb][m] = fmaf(ya[pb][m], f[m], accMix[pb][m]);
            }
        }
        // state cotangent: dS_in = exp(l_end) dS_out + Cbar^T diag(exp(l)) dY
        {
            const float dec = rEnd[1];
#pragma unroll
            for (int j = 0; j < SCW; ++j) {
                const int pb = cg * SCW + j;
                F yb[NIB];
#pragma unroll
                for (int ib = 0; ib < NIB; ++ib) {
                    floatx4 yv = MM::unpack(tile_ldt<SWZ, LDX>(sDY, 16 * ib + 4 * g, 16 * pb, l16));
                    const floatx4 el = *(const floatx4*)(rEl + 16 * ib + 4 * g);
#pragma unroll
                    for (int m = 0; m < 4; ++m) yv[m] *= el[m];
                    yb[ib] = MM::pack(yv);
                }
#pragma unroll
                for (int i = 0; i < SRW; ++i) {
                    const int nb = rg * SRW + i;
#pragma unroll
                    for (int m = 0; m < 4; ++m) st[j][i][m] *= dec;
#pragma unroll
                    for (int ib = 0; ib < NIB; ++ib)
                        st[j][i] = MM::mma(tile_ldt<SWZ, LDB>(sC, 16 * ib + 4 * g, 16 * nb, l16), yb[ib], st[j][i]);
                }
            }
        }
        // dx stores: lane holds dX[s = wrow][p = 16 pb + 4 g + m]
        {
            const rsrc_t dXo = make_rsrc(dXg + t0 * HRP, tail_bytes(t0, HRP, (int64_t)R * P));
            const int tl = wrow >> RL2, r = wrow & (R - 1);
#pragma unroll
            for (int pb = 0; pb < PBH; ++pb)
                store4(dXo, (uint32_t)((tl * (int)HRP + r * P + 16 * (hf * PBH + pb) + 4 * g) * (int)sizeof(T)), dxa[pb],
                       T{});
        }
        __syncthreads();   // (4)

        // ================= S6: gradient rows to LDS (fp32) ==============================
        // The raw B and C rows are read again for the adjoint below (the first read left them in
        // L2): holding them from S1 through the products took registers that then spilled.
        {
            const uint32_t nbc = tail_bytes(t0, SBC, (int64_t)R * N);
            const rsrc_t dB = make_rsrc(Bg + t0 * SBC, nbc), dC = make_rsrc(Cg + t0 * SBC, nbc);
#pragma unroll
            for (int k = 0; k < MAXC; ++k) {
                const bool in = S::FULLC || iC0 + k * RKC < QR;
                rb[k] = buffer_load16_stream(dB, in ? offC(k) : 0x80000000u);
                rc[k] = buffer_load16_stream(dC, in ? offC(k) : 0x80000000u);
            }
        }
#pragma unroll
        for (int nb = 0; nb < NBH; ++nb) {
            *(floatx4*)(fB + wrow * LDF + 16 * (hf * NBH + nb) + 4 * g) = dba[nb];
            *(floatx4*)(fC + wrow * LDF + 16 * (hf * NBH + nb) + 4 * g) = dca[nb];
        }
        __syncthreads();   // (5)

        // ================= S7: rotation and BCNorm adjoint per row =====================
        {
            const uint32_t nbc = tail_bytes(t0, SBC, (int64_t)R * N);
            const rsrc_t dBo = make_rsrc(dBg + t0 * SBC, nbc), dCo = make_rsrc(dCg + t0 * SBC, nbc);
#pragma unroll
            for (int k = 0; k < MAXC; ++k) {
                const int i = iC0 + k * RKC;
                const bool in = S::FULLC || i < QR;
                float v[2][VE], dout[2][VE];
                unpack16(rb[k], v[0], T{});
                unpack16(rc[k], v[1], T{});
                float cs[VE / 2], sn[VE / 2], dph[VE / 2];
                const int ii = in ? i : 0;
                const float* ph = sPhi + (ii >> RL2) * LDPHI + cC0 * VE / 2;
#pragma unroll
                for (int q = 0; q < VE / 2; ++q) {
                    __sincosf(ph[q], &sn[q], &cs[q]);
                    dph[q] = 0.f;
                }
                // With vn = v / RMS (the normalised raw row), vb = vn w + bias and dvb = R(Phi) dout
                // (the rotation undone): the angle cotangent of a pair is dvb0 vb1 - dvb1 vb0
                // (the rotation's derivative is the rotation by a further quarter turn, which
                // commutes with it), and the BCNorm adjoint is dv = (w dvb - vn <w dvb, vn> / N) / RMS.
                float dvb[2][VE], vn[2][VE], sdot[2];
#pragma unroll
                for (int which = 0; which < 2; ++which) {
                    const float* src = (which == 0 ? fB : fC) + ii * LDF + cC0 * VE;
#pragma unroll
                    for (int e = 0; e < VE; e += 4) {
                        const floatx4 d4 = *(const floatx4*)(src + e);
                        dout[which][e] = d4[0];
                        dout[which][e + 1] = d4[1];
                        dout[which][e + 2] = d4[2];
                        dout[which][e + 3] = d4[3];
                    }
                    const float* ww = sWt + which * N + cC0 * VE;   // 1 without weights
                    const float* bb = sBias + (which * R + rC) * N + cC0 * VE;
                    const float iv = inv[k][which];
                    float sd = 0.f;
#pragma unroll
                    for (int q = 0; q < VE / 2; ++q) {
                        const float n0 = v[which][2 * q] * iv, n1 = v[which][2 * q + 1] * iv;
                        vn[which][2 * q] = n0;
                        vn[which][2 * q + 1] = n1;
                        const float x0 = fmaf(n0, ww[2 * q], bb[2 * q]), x1 = fmaf(n1, ww[2 * q + 1], bb[2 * q + 1]);
                        const float d0 = dout[which][2 * q], d1 = dout[which][2 * q + 1];
                        const float e0 = fmaf(cs[q], d0, -sn[q] * d1), e1 = fmaf(sn[q], d0, cs[q] * d1);
                        dvb[which][2 * q] = e0;
                        dvb[which][2 * q + 1] = e1;
                        dph[q] += fmaf(e0, x1, -e1 * x0);
                    }
#pragma unroll
                    for (int e = 0; e < VE; ++e) {
                        if (in) {
                            accBias[which][e] += dvb[which][e];
                            accW[which][e] = fmaf(dvb[which][e], vn[which][e], accW[which][e]);
                        }
                        sd = fmaf(dvb[which][e] * ww[e], vn[which][e], sd);
                    }
                    sdot[which] = sd;
                }
                if (a.bcnorm) {
                    sdot[0] = group_sum(sdot[0], VPN);
                    sdot[1] = group_sum(sdot[1], VPN);
                }
                if (!in) continue;
#pragma unroll
                for (int which = 0; which < 2; ++which) {
                    float dv[VE];
                    if (a.bcnorm) {
                        const float iv = inv[k][which];
                        const float* ww = sWt + which * N + cC0 * VE;
                        const float sN = sdot[which] * invN;
#pragma unroll
                        for (int e = 0; e < VE; ++e) dv[e] = iv * fmaf(-vn[which][e], sN, ww[e] * dvb[which][e]);
                    } else {
#pragma unroll
                        for (int e = 0; e < VE; ++e) dv[e] = dvb[which][e];
                    }
                    buffer_store16(which == 0 ? dBo : dCo, offC(k), pack16(dv, T{}));
                }
                float* dst = fPhi + i * LDD + cC0 * VE / 2;
#pragma unroll
                for (int q = 0; q < VE / 2; ++q) dst[q] = dph[q];
            }
        }
        __syncthreads();   // (6)

        // ================= S8: reverse angle scan -> dtheta, rotation share of d(dt) ===
        if (scanner) {
            float d[SPT][VT];
#pragma unroll
            for (int s = 0; s < SPT; ++s) {
                const int t = tj * SPT + s;
#pragma unroll
                for (int e = 0; e < VT; ++e) {
                    float acc = 0.f;
#pragma unroll
                    for (int r = 0; r < R; ++r) acc += fPhi[(t * R + r) * LDD + tv * VT + e];
                    d[s][e] = acc;
                }
            }
            // suffix sums inside the thread's steps, then over the segments after it
#pragma unroll
            for (int s = SPT - 2; s >= 0; --s)
#pragma unroll
                for (int e = 0; e < VT; ++e) d[s][e] += d[s + 1][e];
            float above[VT];
#pragma unroll
            for (int e = 0; e < VT; ++e) {
                const float tot = d[0][e];
                const float incl = seg_scan_add<TPV>(tot, lane);
                const float gtot = shfl(incl, (lane & ~(TPV - 1)) + TPV - 1);
                above[e] = dcarry[e] + gtot - incl;
                dcarry[e] += gtot;
            }
            const rsrc_t dTo = make_rsrc(dthg + t0 * HK, tail_bytes(t0, HK, K));
#pragma unroll
            for (int s = 0; s < SPT; ++s) {
                const int t = tj * SPT + s;
                const float dd = bits_to_f32(rdt[s]);
                float f[VT], o[VT];
                unpack16(rth[s], f, T{});
                float rot = 0.f;
#pragma unroll
                for (int e = 0; e < VT; ++e) {
                    const float Sv = above[e] + d[s][e];
                    o[e] = dd * Sv;
                    rot = fmaf(f[e], Sv, rot);
                }
                buffer_store16(dTo, (uint32_t)((t * (int)HK + tv * VT) * (int)sizeof(T)), pack16(o, T{}));
                rotdd[tv * 64 + t] = rot;
            }
        }
        __syncthreads();   // (7)

        // ================= S9: per-step sums of the chunk's row partials -> workspace =====
        // record [MU, GM, LI, DW, ROT][step], then ss: the per-step scalar gradients that need
        // them run afterwards in step_grads_kernel, off this kernel's chunk chain.  Each thread
        // zeroes the partials it read for the next chunk.
        {
            float* rec = a.ws_scal + (bh * nchunk + c) * (5 * Q + 3);
            for (int e = tid; e <= 5 * Q; e += NT) {
                const int k = e / Q, s = e - k * Q;
                float acc = 0.f;
                if (k == 5) {
#pragma unroll
                    for (int w = 0; w < NW; ++w) acc += pSS[w];
                } else if (k == 4) {
#pragma unroll
                    for (int v2 = 0; v2 < NVT; ++v2) acc += rotdd[v2 * 64 + s];
                } else {
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const int row = s * R + r;
                        if (k == 3) {
#pragma unroll
                            for (int hh = 0; hh < WPB; ++hh) acc += rDw[hh * 64 + row];
                        } else {
                            float* part = k == 0 ? pMu : k == 1 ? pGam : pLi;
#pragma unroll
                            for (int w = 0; w < NW; ++w) {
                                acc += part[w * 64 + row];
                                part[w * 64 + row] = 0.f;
                            }
                            if (k == 2) {
#pragma unroll
                                for (int hh = 0; hh < WPB; ++hh) acc += rDlo[hh * 64 + row];
                            }
                        }
                    }
                }
                rec[e] = acc;
            }
        }
    }

    // ---- after the first chunk: carried-in inputs, step 0, outputs -------------------------
    // dh_in = dS_{-1}
#pragma unroll
    for (int j = 0; j < SCW; ++j)
#pragma unroll
        for (int i = 0; i < SRW; ++i)
#pragma unroll
            for (int m = 0; m < 4; ++m)
                a.dh_in[(bh * N + 16 * (rg * SRW + i) + 4 * g + m) * P + 16 * (cg * SCW + j) + l16] = st[j][i][m];
    float dc0 = 0.f;
    const bool carry_in = a.Bbar_prev && a.x_prev && L > 0;
    if (carry_in) {
        // dS_{-1} to LDS (fp32 [n][p]); u_{-1} = Bbar_prev^T x_prev enters with weight c_0
        float* fS = (float*)tiles;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < SCW; ++j)
#pragma unroll
            for (int i = 0; i < SRW; ++i)
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    fS[(16 * (rg * SRW + i) + 4 * g + m) * (P + 4) + 16 * (cg * SCW + j) + l16] = st[j][i][m];
        __syncthreads();
        const float c0 = (1.0f - load_f32(lamg)) * load_f32(dtg);
        const T* Bp = (const T*)a.Bbar_prev + bh * R * N;
        const T* xp = (const T*)a.x_prev + bh * R * P;
        float part = 0.f;
        for (int e = tid; e < R * P; e += NT) {   // dx_prev[r][p] = c_0 sum_n dS[n][p] Bp[r][n]
            const int r = e / P, p = e % P;
            float acc = 0.f;
            for (int n = 0; n < N; ++n) acc = fmaf(fS[n * (P + 4) + p], load_f32(Bp + r * N + n), acc);
            part = fmaf(acc, load_f32(xp + e), part);
            if (a.dx_prev) ((T*)a.dx_prev)[bh * R * P + e] = from_f32<T>(c0 * acc);
        }
        for (int e = tid; e < R * N; e += NT) {   // dBbar_prev[r][n] = c_0 sum_p dS[n][p] xp[r][p]
            const int r = e / N, n = e % N;
            float acc = 0.f;
            for (int p = 0; p < P; ++p) acc = fmaf(fS[n * (P + 4) + p], load_f32(xp + r * P + p), acc);
            if (a.dBbar_prev) ((T*)a.dBbar_prev)[bh * R * N + e] = from_f32<T>(c0 * acc);
        }
        part = group_sum(part, 64);
        if (lane == 0) red[wave] = part;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < NW; ++w) dc0 += red[w];
    } else {
        for (int e = tid; e < R * P; e += NT)
            if (a.dx_prev) ((T*)a.dx_prev)[bh * R * P + e] = T{};
        for (int e = tid; e < R * N; e += NT)
            if (a.dBbar_prev) ((T*)a.dBbar_prev)[bh * R * N + e] = T{};
    }
    // the carried-in input's share of mu's gradient before step 0 (c_0 = (1 - lambda_0) dt_0
    // weighs it), for step_grads_kernel: slot 5 Q + 1 of the first chunk's record
    if (tid == 0 && nchunk > 0) a.ws_scal[bh * nchunk * (5 * Q + 3) + 5 * Q + 1] = dc0;
    // angle cotangent before the first step
    if (scanner && tj == 0) {
#pragma unroll
        for (int e = 0; e < VT; ++e) a.dphi_in[bh * K + tv * VT + e] = dcarry[e];
    }
    // BCNorm weight and bias gradients: sum over the threads that share columns (and rank)
    {
        float* part = a.ws_part + bh * a.rec;
        float* pw = part + 1 + R * P;           // [2][N]
        float* pbias = pw + 2 * N;              // [2][R][N]
        __syncthreads();
        float* fw = (float*)tiles;              // [2][N] then [2][R][N]
        float* fbias = fw + 2 * N;
        for (int e = tid; e < 2 * N + 2 * R * N; e += NT) fw[e] = 0.f;
        __syncthreads();
        // threads of one column vector: tid = iC0 * VPN + cC0; rows iC0 have rank iC0 & (R - 1)
        for (int src = 0; src < NT / VPN; ++src) {
            if (iC0 == src) {
#pragma unroll
                for (int which = 0; which < 2; ++which)
#pragma unroll
                    for (int e = 0; e < VE; ++e) {
                        fw[which * N + cC0 * VE + e] += accW[which][e];
                        fbias[(which * R + rC) * N + cC0 * VE + e] += accBias[which][e];
                    }
            }
            __syncthreads();
        }
        for (int e = tid; e < 2 * N; e += NT) pw[e] = a.bcnorm ? fw[e] : 0.f;
        for (int e = tid; e < 2 * R * N; e += NT) pbias[e] = fbias[e];
        // mixing weights: lane (l16, g) holds (r = wrow & (R - 1), p = 16 pb + 4 g + m)
        __syncthreads();
        float* fmix = (float*)tiles;            // [R][P]
        for (int e = tid; e < R * P; e += NT) fmix[e] = 0.f;
        __syncthreads();
        if (mix) {
            // lanes l16 = r, r + R, ... of a row group hold the same (r, p): sum them
#pragma unroll
            for (int pb = 0; pb < PBH; ++pb)
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    float v = accMix[pb][m];
                    v += __shfl_xor(v, 8, 64);
                    if (R <= 4) v += __shfl_xor(v, 4, 64);
                    if (R <= 2) v += __shfl_xor(v, 2, 64);
                    if (R <= 1) v += __shfl_xor(v, 1, 64);
                    accMix[pb][m] = v;
                }
            for (int w = 0; w < NW; ++w) {
                if (wave == w && l16 < R) {
#pragma unroll
                    for (int pb = 0; pb < PBH; ++pb)
#pragma unroll
                        for (int m = 0; m < 4; ++m) fmix[l16 * P + 16 * (hf * PBH + pb) + 4 * g + m] += accMix[pb][m];
                }
                __syncthreads();
            }
        }
        for (int e = tid; e < R * P; e += NT) part[1 + e] = fmix[e];
    }
}

// Per-step scalar gradients d(dt) and d(lambda) and each chunk's share of dA, from the step sums
// the backward kernel leaves per chunk (record [MU, GM, LI, DW, ROT][Q], ss, and in the first
// chunk's record the carried-in input's dmu before step 0).  For each step t of a chunk:
//   dmu_t  = MU_t + exp(l_end - l_t) DW_t
//   dl_t   = LI_t - mu_t MU_t - w_t DW_t  (+ sum_s w_s DW_s + exp(l_end) ss at the last step)
//   d(dt)_t  = A sum_{t' >= t} dl_t' + lambda_t (GM_t + dmu_t) + ROT_t + (1 - lambda_t) dmu_{t-1}
//   dlam_t   = dt_t (GM_t + dmu_t) - dt_t dmu_{t-1}
//   dA_chunk = sum_t dt_t sum_{t' >= t} dl_t'
// with l_t, mu_t and w_t recomputed from dt, lambda and A as the backward kernel forms them.  The
// previous step's dmu comes from the lane below; for a chunk's first step from the previous
// chunk's last step (whose decay to its chunk end is exp(0) = 1), or, at step 0, the carried-in
// input's.  No chunk depends on another's result.  One workgroup per (chunk, block of 64 heads,
// batch): dt and lambda of the chunk's steps (and the step after) for the 64 heads are read as
// whole rows into LDS, each of the 16 waves takes 4 heads (lane = step; their record values
// loaded first) and writes its gradients back over its heads' columns, and the gradient rows are
// stored whole: per-head columns would
// read and write 2-byte pieces of lines that 64 workgroups share.  The dA share goes to slot
// 5 Q + 2 of the chunk's record; reduce_partials_kernel adds the shares.
constexpr int kStepWaves = 16, kStepLd = 65;

template <typename T>
__global__ __launch_bounds__(64 * kStepWaves) void step_grads_kernel(BackwardArgs a, int Q) {
    // dt, lambda: [Q + 1][65] each (rows of 65 floats: a head's column, read with lane = step,
    // then falls in 64 different banks; rows of 64 would put the whole column in one bank)
    extern __shared__ float step_tiles[];
    float* sd = step_tiles;
    float* sl = step_tiles + (Q + 1) * kStepLd;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t c = blockIdx.x, b = blockIdx.z;
    const int hb = (int)blockIdx.y * 64, H = a.H;
    const int64_t L = a.L, nchunk = (L + Q - 1) / Q, t0 = c * Q;
    const int REC = 5 * Q + 3;
    const T* dtg = (const T*)a.dt + b * L * H;
    const T* lamg = (const T*)a.lam + b * L * H;
    const bool live = lane < Q;
    // the wave's heads j = wave + 16 k: their record values are loaded for all four heads first
    constexpr int HPW = 64 / kStepWaves;
    float MU[HPW], GM[HPW], LI[HPW], DW[HPW], ROT[HPW], SS[HPW], PA[HPW], PB[HPW], AH[HPW];
    const int ls = live ? lane : 0;   // every load in bounds; lanes past the chunk are masked at use
#pragma unroll
    for (int k = 0; k < HPW; ++k) {
        const int h = hb + wave + kStepWaves * k;
        const float* rec = a.ws_scal + ((b * H + (h < H ? h : 0)) * nchunk + c) * REC;
        AH[k] = a.A[h < H ? h : 0];
        MU[k] = rec[ls];
        GM[k] = rec[Q + ls];
        LI[k] = rec[2 * Q + ls];
        DW[k] = rec[3 * Q + ls];
        ROT[k] = rec[4 * Q + ls];
        SS[k] = rec[5 * Q];
        PA[k] = c > 0 ? rec[Q - 1 - REC] : rec[5 * Q + 1];
        PB[k] = c > 0 ? rec[4 * Q - 1 - REC] : 0.f;
    }
    // the dt and lambda rows (at most 65 x 64 values: Q <= 64), all loads issued before any use
    constexpr int TL = (65 * 64 + 64 * kStepWaves - 1) / (64 * kStepWaves);
    typedef typename IoBits<T>::type Bits;
    Bits vd[TL], vl[TL];
    bool vin[TL];
#pragma unroll
    for (int i = 0; i < TL; ++i) {   // unconditional loads of in-bounds addresses, masked below
        const int e = tid + i * 64 * kStepWaves, st = e >> 6, j = e & 63;
        const int64_t t = t0 + st;
        vin[i] = e < (Q + 1) * 64 && t < L && hb + j < H;
        const int64_t o = vin[i] ? t * H + hb + j : 0;
        vd[i] = *(const Bits*)(dtg + o);
        vl[i] = *(const Bits*)(lamg + o);
    }
#pragma unroll
    for (int i = 0; i < TL; ++i) {
        const int e = tid + i * 64 * kStepWaves;
        if (e < (Q + 1) * 64) {
            const int o = (e >> 6) * kStepLd + (e & 63);
            sd[o] = vin[i] ? bits_to_f32(vd[i]) : 0.f;
            sl[o] = vin[i] ? bits_to_f32(vl[i]) : 0.f;
        }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < HPW; ++k) {
        const int j = wave + kStepWaves * k, h = hb + j;
        if (h >= H) break;
        const float A = AH[k], Alog2 = A * kLog2e;
        const float cd = live ? sd[lane * kStepLd + j] : 0.f, cl = live ? sl[lane * kStepLd + j] : 0.f;
        const float cdn = live ? sd[(lane + 1) * kStepLd + j] : 0.f, cln = live ? sl[(lane + 1) * kStepLd + j] : 0.f;
        const float l2 = wave_scan_add(cd * Alog2);
        const float gam = cl * cd;
        const float mu = gam + (1.0f - cln) * cdn;
        const float l2end = lane_value(l2, Q - 1);
        const float ed = live ? fast_exp2(fminf(l2end - l2, 0.f)) : 0.f;
        const float wv = ed * mu;
        const float mu_s = live ? MU[k] : 0.f, gm_s = live ? GM[k] : 0.f, li_s = live ? LI[k] : 0.f;
        const float dw_s = live ? DW[k] : 0.f, rot_s = live ? ROT[k] : 0.f;
        const float dmu = mu_s + ed * dw_s;
        float dl = li_s - mu * mu_s - wv * dw_s;
        const float lend = lane_value(wave_scan_add(wv * dw_s), 63) + fast_exp2(l2end) * SS[k];
        if (lane == Q - 1) dl += lend;
        dl = live ? dl : 0.f;
        const float pre = wave_scan_add(dl);
        const float suf = lane_value(pre, 63) - pre + dl;
        const float gsum = gm_s + dmu;
        const float up = shfl_up(dmu, 1);
        const float prev = lane == 0 ? PA[k] + PB[k] : up;
        float ddt = fmaf(A, suf, fmaf(cl, gsum, rot_s));
        float dlam = cd * gsum;
        ddt = fmaf(1.0f - cl, prev, ddt);
        dlam = fmaf(-cd, prev, dlam);
        const float dA = group_sum(cd * suf, 64);
        if (lane == 0) a.ws_scal[((b * H + h) * nchunk + c) * REC + 5 * Q + 2] = dA;
        if (live) {   // this wave's own column: read above, by this lane
            sd[lane * kStepLd + j] = ddt;
            sl[lane * kStepLd + j] = dlam;
        }
    }
    __syncthreads();
    T* ddtg = (T*)a.ddt + b * L * H;
    T* dlamg = (T*)a.dlam + b * L * H;
    for (int e = tid; e < Q * 64; e += 64 * kStepWaves) {
        const int st = e >> 6, j = e & 63;
        const int64_t t = t0 + st;
        if (t < L && hb + j < H) {
            ddtg[t * H + hb + j] = from_f32<T>(sd[st * kStepLd + j]);
            dlamg[t * H + hb + j] = from_f32<T>(sl[st * kStepLd + j]);
        }
    }
}

// Sums of the per-(b, h) partial records over the batch, in batch order; dA from the per-chunk
// shares (thread j adds shares j, j + 256, ... of the (batch, chunk) list, then a fixed tree over
// the threads: the same order on every run).
__global__ __launch_bounds__(256) void reduce_partials_kernel(BackwardArgs a, int Q) {
    const int h = blockIdx.x;
    const int R = a.R, P = a.P, N = a.N;
    {
        __shared__ float red[256];
        const int64_t nchunk = (a.L + Q - 1) / Q, n = a.b * nchunk;
        const int REC = 5 * Q + 3;
        float acc = 0.f;
#pragma unroll 4
        for (int64_t i = threadIdx.x; i < n; i += 256) {
            const int64_t bb = i / nchunk, cc = i - bb * nchunk;
            acc += a.ws_scal[((bb * a.H + h) * nchunk + cc) * REC + 5 * Q + 2];
        }
        red[threadIdx.x] = acc;
        __syncthreads();
        for (int w = 128; w > 0; w >>= 1) {
            if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
            __syncthreads();
        }
        if (threadIdx.x == 0) a.dA[h] = red[0];
    }
    for (int e = threadIdx.x + 1; e < a.rec; e += 256) {
        float acc = 0.f;
#pragma unroll 8
        for (int64_t b = 0; b < a.b; ++b) acc += a.ws_part[(b * a.H + h) * a.rec + e];
        if (e < 1 + R * P) {
            if (a.dw_out) a.dw_out[h * R * P + (e - 1)] = acc;
        } else if (e < 1 + R * P + 2 * N) {
            const int f = e - 1 - R * P;
            float* dst = f < N ? a.dnormw_B : a.dnormw_C;
            if (dst) dst[h * N + f % N] = acc;
        } else {
            const int f = e - 1 - R * P - 2 * N;
            float* dst = f < R * N ? a.dbias_B : a.dbias_C;
            if (dst) dst[h * R * N + f % (R * N)] = acc;
        }
    }
}

// Head groups: dB and dC of each group slot are the sums of the H / G per-head planes, added in
// fp32 in plane order (the same order on every run).  One 16-byte vector per thread and step of
// a grid-stride loop; blockIdx.y picks B (0) or C (1).
template <typename T>
__global__ __launch_bounds__(256) void group_sum_kernel(BackwardArgs a) {
    constexpr int VE = 16 / (int)sizeof(T);
    const int planes = a.H / a.G;
    const int64_t n = a.b * a.L * a.G * a.R * a.N;   // elements per plane (R N is a multiple of 16)
    const T* src = (const T*)(blockIdx.y == 0 ? a.ws_dB : a.ws_dC);
    T* dst = (T*)(blockIdx.y == 0 ? a.dB : a.dC);
    for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < n / VE; v += (int64_t)gridDim.x * 256) {
        float acc[VE];
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[e] = 0.f;
        for (int j = 0; j < planes; ++j) {
            float f[VE];
            unpack16(*(const uint4*)(src + j * n + v * VE), f, T{});
#pragma unroll
            for (int e = 0; e < VE; ++e) acc[e] += f[e];
        }
        *(uint4*)(dst + v * VE) = pack16(acc, T{});
    }
}

// waves per 16-row block of the backward kernel: two where the column blocks split evenly (two
// waves per SIMD), one for the 16 x 16 shape
template <int N, int P> constexpr int backward_wpb() { return (N / 16) % 2 == 0 && (P / 16) % 2 == 0 ? 2 : 1; }

template <typename T, int N, int P, int NIB, int R>
hipError_t launch_nipr(const BackwardArgs& a, bool states_only, hipStream_t s) {
    const dim3 grid((unsigned)(a.b * a.H)), block(NIB * 64);
    if (!states_only && a.b > 65535) return hipErrorInvalidValue;   // step_grads_kernel's grid z
    hipLaunchKernelGGL((chunk_states_kernel<T, N, P, NIB, R>), grid, block, 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || states_only) return e;
    constexpr int WPB = backward_wpb<N, P>();
    hipLaunchKernelGGL((backward_kernel<T, N, P, NIB, R, WPB>), grid, dim3(NIB * WPB * 64), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr int Q = Shape<T, N, P, NIB, R, WPB>::Q;
    const int64_t nchunk = (a.L + Q - 1) / Q;
    if (nchunk > 0) {
        const dim3 sgrid((unsigned)nchunk, (unsigned)((a.H + 63) / 64), (unsigned)a.b);
        hipLaunchKernelGGL(step_grads_kernel<T>, sgrid, dim3(64 * kStepWaves), 2 * (Q + 1) * kStepLd * sizeof(float), s, a, Q);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(reduce_partials_kernel, dim3((unsigned)a.H), dim3(256), 0, s, a, Q);
    e = hipGetLastError();
    const int64_t vecs = a.ws_dB ? a.b * a.L * a.G * R * N / (16 / (int64_t)sizeof(T)) : 0;
    if (e != hipSuccess || vecs == 0) return e;
    const unsigned blocks = (unsigned)((vecs + 255) / 256 < 2048 ? (vecs + 255) / 256 : 2048);
    hipLaunchKernelGGL(group_sum_kernel<T>, dim3(blocks, 2), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <typename T, int N, int P, int NIB>
hipError_t launch_nip(const BackwardArgs& a, bool states_only, hipStream_t s) {
    switch (a.R) {
        case 1: return launch_nipr<T, N, P, NIB, 1>(a, states_only, s);
        case 2: return launch_nipr<T, N, P, NIB, 2>(a, states_only, s);
        case 4: return launch_nipr<T, N, P, NIB, 4>(a, states_only, s);
        default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t launch_bwd_t(const BackwardArgs& a, bool states_only, hipStream_t s) {
    constexpr int NIB64 = sizeof(T) == 2 ? 4 : 2;   // chunk rows 64 (bf16) or 32 (fp32) at P = 64
    if (a.N == 16 && a.P == 16) return launch_nip<T, 16, 16, 1>(a, states_only, s);
    if (a.N == 64 && a.P == 64) return launch_nip<T, 64, 64, NIB64>(a, states_only, s);
    if (a.N == 128 && a.P == 64) return launch_nip<T, 128, 64, NIB64>(a, states_only, s);
    return hipErrorInvalidValue;
}

}  // namespace

bool backward_supported(int N, int P, int R) {
    const bool np = (N == 16 && P == 16) || (N == 64 && P == 64) || (N == 128 && P == 64);
    return np && (R == 1 || R == 2 || R == 4);
}

int backward_chunk_rows(int P, bool bf16_io) { return P == 16 ? 16 : (bf16_io ? 64 : 32); }

hipError_t launch_chunk_states(const BackwardArgs& a, bool bf16_io, hipStream_t s) {
    return bf16_io ? launch_bwd_t<bf16>(a, true, s) : launch_bwd_t<float>(a, true, s);
}

hipError_t launch_backward(const BackwardArgs& a, bool bf16_io, hipStream_t s) {
    return bf16_io ? launch_bwd_t<bf16>(a, false, s) : launch_bwd_t<float>(a, false, s);
}

}  // namespace m3
