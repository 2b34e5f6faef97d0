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
#include <type_traits>

#include "m3_device.h"
#include "m3_launch.h"
#include "m3_mma.h"

namespace m3 {

namespace {

// FUSED: the chunk's B and C arrive raw and are normalised (BCNorm), biased and rotated by the
// cumulative angle while they are staged (papernotes.org, key design 4; aipaper.cc section 4.2
// Proposition 3), so the rotated Bbar and Cbar never go through HBM.
//
// Chunk tiles of 16 or 32 rows are software-pipelined: the LDS tiles, per-row scalars, scores and
// angles are double-buffered by chunk parity, chunk c + 1 is staged (and, fused, normalised and
// rotated) in slices between the MFMA K blocks of chunk c's part 1, and one barrier per chunk
// remains.  The raw loads of chunk c + 2 are issued at the start of chunk c into the register set
// of that parity, so they have a whole chunk to arrive.  Tiles of 48 or 64 rows do not fit twice
// in LDS and run the same steps with two barriers per chunk.
// PAIR (fused, ranks R >= 2): each thread stages two neighbouring rows of one step (see rowC).
// A split sequence's later segments run first from a zero carry (pass 1).  The carried-in
// state's share of y at step t of a segment is that state times 2^{l2}, l2 the log2 decay from the
// segment's start through t; once l2 < -kFixLog2 for the rest of the segment the share is below
// 2^-48 of the state, 2^-24 below float rounding, and pass 2 reruns only the steps before.
constexpr float kFixLog2 = 48.0f;

template <typename T, int N, int P, int NIB, bool FUSED, bool PAIR = false>
__global__ __launch_bounds__(P / 16 * 64, 2) void prefill_kernel(PrefillArgs a) {
    using MM = Mma<T>;
    using F = typename MM::frag;
    constexpr int NW = P / 16, NT = NW * 64;
    constexpr int QR = 16 * NIB;                 // rows (t, r) per chunk
    constexpr int NB = N / 16;
    constexpr bool PIPE = NIB <= 2;
    constexpr int NBUF = PIPE ? 2 : 1;
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
    // padded angle rows (fp32): with K + 12 the column walk of the scan (runs of 2 or 8 steps)
    // and the row writes of its first phase reach distinct banks
    constexpr int LDPHI = K + 12;
    // the scan's column walk: wave w owns angle columns [w KWL, (w + 1) KWL) (the columns its
    // lanes load), lane = column j + KWL * run r, run r covers steps r SRUN .. r SRUN + SRUN - 1
    constexpr int KWL = FUSED ? (VT * 64 / TPV < K ? VT * 64 / TPV : K) : 64;
    constexpr int NW2 = FUSED ? K / KWL : 0, SEGW = 64 / KWL, SRUN = (QR + SEGW - 1) / SEGW;
    static_assert(!FUSED || (NW2 <= NW && KWL >= 8 && KWL * SEGW == 64 && SRUN * SEGW <= QR), "column walk layout");
    constexpr int FZ = FUSED ? 1 : 0;            // sizes the fused-only LDS arrays
    constexpr int TC = QR * LDC, TB = QR * LDB, TX = QR * LDX, TM = QR * LDM, TPH = QR * LDPHI;

    // buffer b of each (b = chunk parity when pipelined)
    __shared__ __align__(16) T sC[NBUF * TC];    // Cbar rows of the chunk  [i][n]
    __shared__ __align__(16) T sB[NBUF * TB];    // Bbar rows               [s][n]
    __shared__ __align__(16) T sX[NBUF * TX];    // x rows                  [s][p]
    __shared__ __align__(16) T sM[NBUF * TM];    // masked scores           [i][s]
    // per-row (t, r) copies of the chunk's per-step scalars: log2 decay l_t, gamma_t, mu_t,
    // exp(l_t) and w_t = exp(l_end - l_t) mu_t
    __shared__ __align__(16) float rL2[NBUF * 64], rGam[NBUF * 64], rMu[NBUF * 64], rEl[NBUF * 64],
        rW[NBUF * 64];
    // fused only: the chunk's angles Phi[t][k]; in the dynamic LDS the BCNorm weights [B, C][n]
    // and the biases [B, C][r][n] ((2 N + 2 R N) floats, sized at launch)
    __shared__ __align__(16) float sPhi[FZ * NBUF * TPH + 1];
    extern __shared__ __align__(16) float dyn_lds[];
    float* sWt = dyn_lds;
    float* sBias = dyn_lds + 2 * N;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, l16 = lane & 15;
    // a split sequence: pass 1 runs every segment of each (b, h), pass 2 segments 1 .. nseg-1
    // (their first ws_fix steps)
    const int segs = a.pass == 2 ? a.nseg - 1 : a.nseg;
    // heads that share raw B and C run on one XCD (consecutive items), so its L2 serves the group
    const int64_t item = a.G > 0 && a.G < a.H ? xcd_item(blockIdx.x, gridDim.x) : (int64_t)blockIdx.x;
    const int64_t bh = a.pass ? item / segs : item;
    const int seg = a.pass ? (int)(item % segs) + (a.pass == 2 ? 1 : 0) : 0;
    const int64_t b = bh / a.H;
    const int h = (int)(bh % a.H);
    const int H = a.H, R = a.R, Q = a.Q;
    const int rl2 = __builtin_ctz((unsigned)R), rmask = R - 1;
    // dense: sequence b is steps [0, L) of [b, L, ...]; packed: tokens [cu[b], cu[b+1]) of T,
    // clamped into [0, T) so that any offsets stay inside the packed arrays; split: the segment's
    // steps (never empty: the host makes the last segment hold the tail)
    int64_t L = a.L, t_first = b * a.L;
    if (a.cu_seqlens) {
        const int64_t s0 = min(max((int64_t)a.cu_seqlens[b], (int64_t)0), a.T);
        const int64_t s1 = min(max((int64_t)a.cu_seqlens[b + 1], s0), a.T);
        t_first = s0;
        L = s1 - s0;
    }
    if (a.pass) {
        t_first += seg * a.seglen;
        L = min(a.seglen, a.L - seg * a.seglen);
        if (a.pass == 2) L = min(L, (int64_t)a.ws_fix[bh * a.nseg + seg]);
    }
    // carried in: the call's carry (no split, or segment 0), none (the later segments in pass 1),
    // or the chained state entering the segment (pass 2)
    const bool own_carry = seg == 0;
    const int64_t nchunk = (L + Q - 1) / Q;
    const float Alog2 = a.A[h] * kLog2e;
    // (b, t = 0, h) bases; step t of this (b, h) is t * H rows further
    const int64_t row_bh = t_first * H + h;
    // B and C rows: per head (Bbar, Cbar), or the raw rows of the head's group slot (fused);
    // SBC = B or C elements per step
    const int GS = bc_slots(H, a.G);
    const int64_t row_bc = t_first * GS + bc_slot(h, H, a.G);
    const int64_t SBC = (int64_t)GS * R * N, HRP = (int64_t)H * R * P;
    const T* Xg = (const T*)a.x + row_bh * R * P;
    const T* Bg = (const T*)a.Bbar + row_bc * R * N;
    const T* Cg = (const T*)a.Cbar + row_bc * R * N;
    const T* dtg = (const T*)a.dt + row_bh;
    const T* lamg = (const T*)a.lam + row_bh;
    const float* hin = nullptr;
    const T* Bprev = nullptr;
    const T* xprev = nullptr;
    // (A split writes h_out only in the chaining kernel, after pass 1's segment 0 has read h_in,
    // so the carry may be updated in place.)
    if (own_carry) {
        hin = a.h_in ? a.h_in + bh * (int64_t)(N * P) : nullptr;
        Bprev = a.Bbar_prev ? (const T*)a.Bbar_prev + bh * (int64_t)(R * N) : nullptr;
        xprev = a.x_prev ? (const T*)a.x_prev + bh * (int64_t)(R * P) : nullptr;
    } else if (a.pass == 2) {
        // the state entering the segment, the previous step's term included (the chaining adds it)
        hin = a.ws_state + (bh * a.nseg + seg - 1) * (int64_t)(N * P);
    }
    const int pcol = 16 * wave + l16;            // this lane's column of P in MFMA tiles
    // One buffer descriptor per stream over this sequence: from step 0 of this (b, h) to the end
    // of its last row (t = L - 1).  A chunk adds its byte offset (32 bits: the whole sequence
    // spans less than 2^31 bytes, which the host checks) to the per-lane offsets; loads past the
    // last row read zero and stores there are dropped, so the ragged last chunk needs no branches.
    auto seq_bytes = [&](int64_t step, int64_t row) {
        return L > 0 ? clamp_bytes(((L - 1) * step + row) * (int64_t)sizeof(T)) : 0u;
    };
    constexpr uint32_t ES = sizeof(T);
    auto step_off = [&](int64_t t0, int64_t step) { return (uint32_t)t0 * (uint32_t)(step * ES); };

    // ---- staging: this thread moves 16-byte vectors k = 0, 1, ... of each tile.  Vector k is
    // chunk row i = i0 + k * RK (row (t, r) = (i >> rl2, i & rmask)), 16-byte column c0.
    const int iC0 = tid / VPN, cC0 = tid % VPN, iX0 = tid / VPP, cX0 = tid % VPP;
    const int SBC32 = (int)SBC, HRP32 = (int)HRP;
    // With ranks (R >= 2) and a chunk of two staging steps, the fused kernel gives each thread two
    // neighbouring rows, 2 iC0 and 2 iC0 + 1: two ranks of one step, which share their rotation
    // angles, so the sine and cosine are taken once for both (the rows of MIMO are 4 per step).
    constexpr bool pair_rows = PAIR && FUSED && MAXC == 2 && FULLC;
    auto rowC = [&](int k) { return pair_rows ? 2 * iC0 + k : iC0 + k * RKC; };
    auto offC = [&](int k) {
        const int i = rowC(k);
        return (uint32_t)(((i >> rl2) * SBC32 + (i & rmask) * N + cC0 * VE) * (int)sizeof(T));
    };
    auto offX = [&](int k) {
        const int i = iX0 + k * RKX;
        return (uint32_t)(((i >> rl2) * HRP32 + (i & rmask) * P + cX0 * VE) * (int)sizeof(T));
    };

    // ---- chunk prefetch into registers (set = chunk parity when pipelined) ----------------
    uint4 rc[NBUF][MAXC], rb[NBUF][MAXC], rx[NBUF][MAXX];
    typedef typename IoBits<T>::type Bits;
    Bits nd[NBUF], nl[NBUF], ndn[NBUF], nln[NBUF];   // dt, lambda at t and t + 1 (io bits; the last wave uses them)
    const rsrc_t dCs = make_rsrc(Cg, seq_bytes(SBC, (int64_t)R * N));
    const rsrc_t dBs = make_rsrc(Bg, seq_bytes(SBC, (int64_t)R * N));
    const rsrc_t dXs = make_rsrc(Xg, seq_bytes(HRP, (int64_t)R * P));
    const rsrc_t dDs = make_rsrc(dtg, seq_bytes(H, 1));
    const rsrc_t dLs = make_rsrc(lamg, seq_bytes(H, 1));
    // part: 0 = Cbar rows, 1 = Bbar rows, 2 = x rows, 3 = step scalars; -1 = all
    auto load_chunk = [&](int64_t c, int set, int part = -1) {
        const int64_t t0 = c * Q;
        if (part < 0 || part == 0) {
            const uint32_t o = step_off(t0, SBC);
#pragma unroll
            for (int k = 0; k < MAXC; ++k)
                if (FULLC || rowC(k) < QR) rc[set][k] = buffer_load16_stream(dCs, offC(k) + o);
        }
        if (part < 0 || part == 1) {
            const uint32_t o = step_off(t0, SBC);
#pragma unroll
            for (int k = 0; k < MAXC; ++k)
                if (FULLC || rowC(k) < QR) rb[set][k] = buffer_load16_stream(dBs, offC(k) + o);
        }
        if (part < 0 || part == 2) {
            const uint32_t o = step_off(t0, HRP);
#pragma unroll
            for (int k = 0; k < MAXX; ++k)
                if (FULLX || iX0 + k * RKX < QR) rx[set][k] = buffer_load16_stream(dXs, offX(k) + o);
        }
        if (part < 0 || part == 3) {
            // steps t0 + lane and t0 + lane + 1; zero past the sequence end.  Only lanes 0..Q are
            // read (lane Q holds the step after the chunk); the other lanes, and the waves other
            // than the last, issue the same loads aimed past the descriptor (no memory access),
            // so that the number of loads in flight is the same on every path and the
            // compiler's wait counts stay exact.  Step t0 + lane + 1 is the next lane's value;
            // lane 63 loads its own only for 64-step chunks.
            const uint32_t o0 = wave == NW - 1 && lane <= Q ? (uint32_t)(lane * H * (int)sizeof(T)) + step_off(t0, H) : 0x80000000u;
            const uint32_t o1 = wave == NW - 1 && lane == 63 && Q == 64 ? o0 + (uint32_t)(H * (int)sizeof(T)) : 0x80000000u;
            nd[set] = buffer_load_bits(dDs, o0, T{});
            nl[set] = buffer_load_bits(dLs, o0, T{});
            if constexpr (QR == 64) {   // only a 64-step chunk reads past lane 63
                ndn[set] = buffer_load_bits(dDs, o1, T{});
                nln[set] = buffer_load_bits(dLs, o1, T{});
            } else {
                ndn[set] = nln[set] = Bits{};
            }
        }
    };
    // ---- fused: angle increments of a chunk and their prefix scan ----------------------
    const int tau = tid, tv = tau / TPV, tj = tau % TPV;
    const bool scanner = FUSED && tau < NVT * TPV;
    uint4 rth[SPT];
    Bits rdt[SPT];
    const T* thg = (const T*)a.theta + row_bh * K;
    const int64_t HK = (int64_t)H * K;
    const rsrc_t dTs = make_rsrc(thg, FUSED ? seq_bytes(HK, K) : 0u);
    auto load_theta = [&](int64_t c) {
        if (!FUSED) return;
        const int64_t t0 = c * Q;
        const uint32_t ot = step_off(t0, HK), od = step_off(t0, H);
#pragma unroll
        for (int s = 0; s < SPT; ++s) {
            // steps past the chunk (R > 1 leaves rows of the tile unused) and threads that do not
            // scan aim past the descriptor; with 32 steps per column the upper half of a wave
            // repeats the lower half's steps and takes their dt by a shuffle in the scan
            const int t = tj * SPT + s;
            const bool in = scanner && t < Q;
            rth[s] = buffer_load16(dTs, in ? (uint32_t)((t * (int)HK + tv * VT) * (int)sizeof(T)) + ot : 0x80000000u);
            const bool dt_lane = in && !(TPV == 32 && lane >= 32);
            rdt[s] = buffer_load_bits(dDs, dt_lane ? (uint32_t)(t * H * (int)sizeof(T)) + od : 0x80000000u, T{});
        }
    };
    // Phi[t] = Phi[t0 - 1] + sum_{t0 <= i <= t} dt_i theta_i for the chunk starting at c * Q, into
    // angle buffer `out`, in turns (revolutions: the unit of the hardware sine and cosine).  Only
    // the carried angle is reduced to [-1/2, 1/2]; inside a chunk the rows stay within a few turns
    // of it, well inside the hardware sine's input range.  Two phases, both inside each wave's
    // own columns (so no barrier): the loading lanes write the increments dt_t theta_t[k] to the
    // rows, then lane (j, r) walks run r of column j, a serial sum of SRUN rows, and the runs'
    // totals are chained across the wave's runs by lane swaps.  Rows past the chunk's steps
    // hold zero increments (their loads aim past the descriptor), so a run that covers them ends
    // on the last step's angle.  The carried angle is the last row of buffer `prev` (the previous
    // chunk), read first: without pipelining prev == out.  Chunk 0 starts from phi_in (radians).
    const int kcol = wave * KWL + (lane & (KWL - 1)), run = lane / KWL;
    // angle carried in (radians): the call's (no split, and segment 0 of pass 1), none (the
    // later segments of pass 1: their angles run from zero), or the segment's true start angle
    // from the chaining (pass 2).  A pass-1 segment from zero has the y of its true angles (y
    // depends on differences of the angles in a segment only, and on the carried state, which is
    // zero there); its end state and last Bbar row come out rotated back by its start angle,
    // which the chaining applies.
    const float* phin = nullptr;
    if (FUSED) {
        if (a.pass == 0 || (a.pass == 1 && seg == 0)) phin = a.phi_in ? a.phi_in + bh * K : nullptr;
        else if (a.pass == 2) phin = a.seg_phi + (bh * a.nseg + seg) * (int64_t)K;
    }
    auto scan = [&](int64_t c, int out, int prev) {
        if (!FUSED) return;
        const bool colwave = wave < NW2;
        float carry = 0.f;
        if (colwave)
            carry = c == 0 ? (phin ? wrap_turns(phin[kcol] * kInvTwoPi) : 0.f)
                           : wrap_turns(sPhi[prev * TPH + (Q - 1) * LDPHI + kcol]);
        float* ph = sPhi + out * TPH;
        if (scanner) {
#pragma unroll
            for (int s = 0; s < SPT; ++s) {
                float f[VT];
                unpack16(rth[s], f, T{});
                float d = bits_to_f32(rdt[s]) * kInvTwoPi;
                if (TPV == 32) d = shfl(d, lane & 31);
                float* dst = ph + (tj * SPT + s) * LDPHI + tv * VT;
#pragma unroll
                for (int e = 0; e < VT; e += 4)
                    *(floatx4*)(dst + e) = floatx4{d * f[e], d * f[e + 1], d * f[e + 2], d * f[e + 3]};
            }
        }
        if (colwave) {
            float* col = ph + run * SRUN * LDPHI + kcol;
            // every read goes out before the first sum waits on one
            float acc[SRUN];
#pragma unroll
            for (int s = 0; s < SRUN; ++s) acc[s] = col[s * LDPHI];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 1; s < SRUN; ++s) acc[s] += acc[s - 1];
            const float base = carry + run_exclusive_sum<KWL>(acc[SRUN - 1], lane);
#pragma unroll
            for (int s = 0; s < SRUN; ++s) col[s * LDPHI] = base + acc[s];
        }
    };
    // fused: raw B and C rows -> BCNorm, weight, bias, rotation -> tile buffer `buf`.  B and C go
    // one after the other to keep few values live; they share the row's angles.
    const float invN = 1.0f / (float)N;
    const bool has_w = a.bcnorm && (a.normw_B || a.normw_C);
    // the angles of row i's step for this thread's pairs (LDS read + hardware sin/cos, in turns)
    auto row_angles = [&](int i, int buf, float (&cs)[VE / 2], float (&sn)[VE / 2]) {
        const float* ph = sPhi + buf * TPH + (i >> rl2) * LDPHI + cC0 * VE / 2;
#pragma unroll
        for (int q = 0; q < VE / 2; ++q) {
            sn[q] = __builtin_amdgcn_sinf(ph[q]);
            cs[q] = __builtin_amdgcn_cosf(ph[q]);
        }
    };
    auto stage_bc = [&](int set, int k, int i, int buf, const float (&cs)[VE / 2], const float (&sn)[VE / 2]) {
        const int r = i & rmask;
        const int n0 = cC0 * VE;
        float sc[2] = {1.f, 1.f};
        if (a.bcnorm) {   // RMS over the row's N values, spread over VPN consecutive lanes
            constexpr int NR = 2;   // rows normalised: B and C
            float q2[2] = {0.f, 0.f};
#pragma unroll
            for (int which = 0; which < NR; ++which) q2[which] = sumsq16(which == 0 ? rb[set][k] : rc[set][k], T{});
            // the two rows' lane sums interleave
#pragma unroll
            for (int which = 0; which < NR; ++which) q2[which] = group_sum(q2[which], VPN);
#pragma unroll
            for (int which = 0; which < NR; ++which)
                // hardware 1/sqrt; the clamp keeps its argument out of the denormal range (an
                // all-zero row stays zero either way)
                sc[which] = __builtin_amdgcn_rsqf(fmaxf(fmaf(q2[which], invN, a.eps), 1e-30f));
        }
#pragma unroll
        for (int which = 0; which < 2; ++which) {
            float x[VE];
            unpack16(which == 0 ? rb[set][k] : rc[set][k], x, T{});
            const float* bw = sBias + (which * R + r) * N + n0;
            if (has_w) {
                const float* ww = sWt + which * N + n0;
#pragma unroll
                for (int e = 0; e < VE; ++e) x[e] = fmaf(x[e] * sc[which], ww[e], bw[e]);
            } else {
#pragma unroll
                for (int e = 0; e < VE; ++e) x[e] = fmaf(x[e], sc[which], bw[e]);
            }
#pragma unroll
            for (int q = 0; q < VE / 2; ++q) {
                const float x0 = x[2 * q], x1 = x[2 * q + 1];
                x[2 * q] = fmaf(cs[q], x0, sn[q] * x1);
                x[2 * q + 1] = fmaf(cs[q], x1, -sn[q] * x0);
            }
            if (which == 0) *(uint4*)(sB + buf * TB + i * LDB + n0) = pack16(x, T{});
            else *(uint4*)(sC + buf * TC + i * LDC + n0) = pack16(x, T{});
        }
    };
    // the last wave (the one with the fewest score tiles): the chunk's per-step scalars (lane =
    // step) -> per-row copies in LDS.  Lanes past the chunk only add to later lanes of the scan,
    // which are never read.
    float l2sum = 0.f;   // pass 1: the segment's log2 decay, sum of the chunks' (last wave)
    // pass 1 (last wave): chunks staged so far, and how many of them have a step whose log2 decay
    // from the segment's start (the carried-in state's factor in y) is above -kFixLog2; a chunk's
    // 64 lanes include the step after it (a conservative superset)
    int staged_chunks = 0, fix_chunks = 0;
    auto stage_scalars = [&](float d, float lm, float dn63, float lmn63, int buf) {
        // dt, lambda of step t + 1: the next lane's, lane 63's own load (the shuffles run in every
        // lane: a lane reading an inactive lane would get zero)
        const float dsh = __shfl_down(d, 1, 64), lsh = __shfl_down(lm, 1, 64);
        const float dn = lane < 63 ? dsh : dn63;
        const float lmn = lane < 63 ? lsh : lmn63;
        const float l2 = wave_scan_add(d * Alog2);   // l_t in log2 units, inclusive over the chunk
        const float gam = lm * d;
        const float mu = gam + (1.0f - lmn) * dn;
        const float l2end = lane_value(l2, Q - 1);
        if (a.pass == 1) {
            ++staged_chunks;
            if (__any(l2sum + l2 >= -kFixLog2)) fix_chunks = staged_chunks;
        }
        if (a.pass == 1) l2sum += l2end;
        const float el = fast_exp2(l2);
        const float w = fast_exp2(fminf(l2end - l2, 0.f)) * mu;
        float* o = rL2 + buf * 64;
        if (R == 1) {
            o[lane] = l2;
            rGam[buf * 64 + lane] = gam;
            rMu[buf * 64 + lane] = mu;
            rEl[buf * 64 + lane] = el;
            rW[buf * 64 + lane] = w;
        } else {   // row s holds step s >> rl2 (rows past Q * R are never read)
            const int ts = lane >> rl2;
            o[lane] = shfl(l2, ts);
            rGam[buf * 64 + lane] = shfl(gam, ts);
            rMu[buf * 64 + lane] = shfl(mu, ts);
            rEl[buf * 64 + lane] = shfl(el, ts);
            rW[buf * 64 + lane] = shfl(w, ts);
        }
    };
    // staging item j of register set `set` into buffer `buf`: the B/C row vectors, then the x
    // vectors, then (wave 0) the scalars
    constexpr int NITEM = MAXC + MAXX + 1;
    auto stage_item = [&](int j, int set, int buf) {
        if (j < MAXC) {
            const int i = rowC(j);
            if (FULLC || i < QR) {
                if (FUSED) {
                    float cs[VE / 2], sn[VE / 2];
                    if constexpr (pair_rows) {   // both rows (one step) in the first item, one set of angles
                        if (j == 0) {
                            row_angles(i, buf, cs, sn);
                            stage_bc(set, 0, i, buf, cs, sn);
                            stage_bc(set, 1, i + 1, buf, cs, sn);
                        }
                    } else {
                        row_angles(i, buf, cs, sn);
                        stage_bc(set, j, i, buf, cs, sn);
                    }
                } else {
                    *(uint4*)(sC + buf * TC + i * LDC + cC0 * VE) = rc[set][j];
                    *(uint4*)(sB + buf * TB + i * LDB + cC0 * VE) = rb[set][j];
                }
            }
        } else if (j < MAXC + MAXX) {
            const int k = j - MAXC, i = iX0 + k * RKX;
            if (FULLX || i < QR) *(uint4*)(sX + buf * TX + i * LDX + cX0 * VE) = rx[set][k];
        } else if (wave == NW - 1) {
            stage_scalars(bits_to_f32(nd[set]), bits_to_f32(nl[set]), bits_to_f32(ndn[set]),
                          bits_to_f32(nln[set]), buf);
        }
    };

    // ---- carried-in state: G_{-1} = h_in + c_0 Bbar_prev^T x_prev ------------------------
    floatx4 st[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int m = 0; m < 4; ++m)
            st[nb][m] = hin ? hin[(16 * nb + 4 * g + m) * P + pcol] : 0.f;
    if (Bprev && xprev && L > 0) {
        const float c0 = (1.0f - load_f32(lamg)) * load_f32(dtg);
        for (int r = 0; r < R; ++r) {
            const float xv = c0 * load_f32(xprev + r * P + pcol);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int m = 0; m < 4; ++m) st[nb][m] += load_f32(Bprev + r * N + 16 * nb + 4 * g + m) * xv;
        }
    }

    // outputs: mixed [b, L, H, P] with w_out, else [b, L, H, R, P]
    const bool mix = a.w_out != nullptr;
    T* yg = (T*)a.y + row_bh * (mix ? P : (int64_t)R * P);
    const int64_t ystep = mix ? (int64_t)H * P : HRP, yrow = mix ? P : (int64_t)R * P;
    const rsrc_t dYs = make_rsrc(yg, seq_bytes(ystep, yrow));
    floatx4 wo = {1.f, 1.f, 1.f, 1.f};          // mixing weights for this lane's (r, 4 columns)
    if (mix) {
        const int r = l16 & rmask;
#pragma unroll
        for (int m = 0; m < 4; ++m) wo[m] = a.w_out[(h * R + r) * P + 16 * wave + 4 * g + m];
    }

    // loop-invariant LDS fragment addresses for this lane (buffer 0; buffer b is b * T? further)
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

    // ---- one chunk on buffer `buf`: part 1 (calling hook(k) in K block k), after_part1(),
    // masks, a barrier, part 2 ------------------------------------------------------------
    auto chunk_compute = [&](int buf, int64_t c, auto hook, auto after_part1) {
        const int64_t t0 = c * Q;
        const T* tC = pC_k + buf * TC;
        const T* tBt = pB_t + buf * TB;
        const float* sL2 = rL2 + buf * 64;
        const float* sGm = rGam + buf * 64;
        const float* sMu = rMu + buf * 64;
        const float* sEl = rEl + buf * 64;
        const float* sW = rW + buf * 64;
        // X^T fragments of this wave's 16 columns, and w o X for the state update
        F xf[NIB], xw[NIB];
#pragma unroll
        for (int sb = 0; sb < NIB; ++sb) xf[sb] = MM::ldt(pX_t + buf * TX + 16 * sb * LDX, LDX, l16);
#pragma unroll
        for (int sb = 0; sb < NIB; ++sb) {
            floatx4 xs = MM::unpack(xf[sb]);
            const floatx4 ws = *(const floatx4*)(sW + 16 * sb + 4 * g);
#pragma unroll
            for (int m = 0; m < 4; ++m) xs[m] *= ws[m];
            xw[sb] = MM::pack(xs);
        }
        const float dec = sEl[QR - 1];
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
            for (int ib = 0; ib < NIB; ++ib) fc[s][ib] = MM::ldk(tC + 16 * ib * LDC + 16 * k);
#pragma unroll
            for (int j = 0; j < NSLOT; ++j) {
                fsb[s][j] = MM::ldk(pSB[j] + buf * TB + 16 * k);
                fsc[s][j] = MM::ldk(pSC[j] + buf * TC + 16 * k);
            }
#pragma unroll
            for (int sb = 0; sb < NIB; ++sb) fbt[s][sb] = MM::ldt(tBt + 16 * sb * LDB + 16 * k, LDB, l16);
        };
        fetch(0, 0);
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const int s = k & 1;
            __builtin_amdgcn_sched_barrier(0);
            if (k + 1 < NB) fetch(k + 1, s ^ 1);
            hook(k);
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
        after_part1();
        // mask the score tiles: lane holds S^T[s = 16 sb + 4 g + m][i = 16 ib + l16]
#pragma unroll
        for (int j = 0; j < NSLOT; ++j) {
            if (!sOn[j]) continue;
            const int i = 16 * sIb[j] + l16, s0 = 16 * sSb[j] + 4 * g;
            const int ti = i >> rl2;
            const float l2i = sL2[i], gi = sGm[i];
            const floatx4 l2s = *(const floatx4*)(sL2 + s0);
            const floatx4 mus = *(const floatx4*)(sMu + s0);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                // below the diagonal exp(l_t - l_s) mu_s, on it gamma_t, above it 0
                const int ts = (s0 + m) >> rl2;
                const float e = fast_exp2(fminf(l2i - l2s[m], 0.f)) * mus[m];
                const float below = ts < ti ? 1.f : 0.f;
                const float diag = ts == ti ? gi : 0.f;
                acc[j][m] *= fmaf(e, below, diag);
            }
            MM::st(sM + buf * TM + i * LDM + s0, MM::pack(acc[j]));
        }
#pragma unroll
        for (int ib = 0; ib < NIB; ++ib) {
            const float el = sEl[16 * ib + l16];
#pragma unroll
            for (int m = 0; m < 4; ++m) y[ib][m] *= el;
        }
        __syncthreads();

        // ---- part 2: Y^T += X^T M^T, mixing, stores --------------------------------------
#pragma unroll
        for (int sb = 0; sb < NIB; ++sb)
#pragma unroll
            for (int ib = sb; ib < NIB; ++ib)
                y[ib] = MM::mma(xf[sb], MM::ldk(pM_k + buf * TM + 16 * ib * LDM + 16 * sb), y[ib]);
        const uint32_t oy = step_off(t0, ystep);
        // lane holds Y[(t, r) = i][p = 16 wave + 4 g + m] of row block ib
        const int p = 16 * wave + 4 * g;
        auto store_mixed = [&](auto RW) {   // RW: the rank as a compile-time width
            constexpr int RR = decltype(RW)::value;
#pragma unroll
            for (int ib = 0; ib < NIB; ++ib) {
                const int i = 16 * ib + l16;
                floatx4 yv = y[ib];
#pragma unroll
                for (int m = 0; m < 4; ++m) yv[m] = group_sum(yv[m] * wo[m], RR);
                // one lane per step stores the mixed row; the others aim past the descriptor
                const uint32_t off = (i & (RR - 1)) == 0 ? (uint32_t)(((i / RR) * H * P + p) * (int)sizeof(T)) + oy
                                                         : 0x80000000u;
                store4(dYs, off, yv, T{});
            }
        };
        if (!mix) {
#pragma unroll
            for (int ib = 0; ib < NIB; ++ib) {
                const int i = 16 * ib + l16;
                const int tl = i >> rl2, r = i & rmask;
                store4(dYs, (uint32_t)(((tl * H * R + r) * P + p) * (int)sizeof(T)) + oy, y[ib], T{});
            }
        } else {
            switch (R) {
                case 1: store_mixed(std::integral_constant<int, 1>{}); break;
                case 2: store_mixed(std::integral_constant<int, 2>{}); break;
                case 4: store_mixed(std::integral_constant<int, 4>{}); break;
                case 8: store_mixed(std::integral_constant<int, 8>{}); break;
                default: store_mixed(std::integral_constant<int, 16>{}); break;
            }
        }
    };

    // ---- prologue ---------------------------------------------------------------------
    // Chunk loads are issued on every path, also for chunks past the end (their descriptors hold
    // zero bytes, so nothing is read), and every thread loads its angle increments; the compiler's
    // wait counts then match the loads actually in flight.
    if (FUSED) {
        // BCNorm weights (1 without BCNorm or without weights) and biases (0 when absent)
        for (int e = tid; e < 2 * N; e += NT) {
            const float* w = e < N ? a.normw_B : a.normw_C;
            sWt[e] = a.bcnorm && w ? w[h * N + (e % N)] : 1.f;
        }
        for (int e = tid; e < 2 * R * N; e += NT) {
            const int which = e / (R * N), rn = e % (R * N);
            const float* bias = which == 0 ? a.bias_B : a.bias_C;
            sBias[e] = bias ? bias[h * R * N + rn] : 0.f;
        }
        if (nchunk > 0) {
            load_theta(0);
            scan(0, 0, 0);
        }
        if (PIPE && nchunk > 1) {
            load_theta(1);
            scan(1, 1, 0);
        }
        if (PIPE) load_theta(2);
        __syncthreads();
    }
    if (nchunk > 0) load_chunk(0, 0);
    auto no_hook = [&](int) {};

    if constexpr (PIPE) {
        if (nchunk > 0) {
#pragma unroll
            for (int j = 0; j < NITEM; ++j) stage_item(j, 0, 0);
        }
        load_chunk(1, 1);
        __builtin_amdgcn_s_waitcnt(0);   // nothing from the prologue stays in flight into the loop
        __syncthreads();
        // chunk c on buffer p = c & 1 (p compile-time in each half of the unrolled pair)
        auto iter = [&](auto PB, int64_t c) {
            constexpr int p = decltype(PB)::value, q = p ^ 1;
            const bool has1 = c + 1 < nchunk, has2 = c + 2 < nchunk;
            // stage chunk c + 1 (register set q) into buffer q, item j after K block
            // (2 j + 1) NB / (2 NITEM); fused: the angles of chunk c + 2 in K block NB / 2.  The
            // loads of chunk c + 2 go out in four parts over the K blocks, so that their issue
            // does not stall the wave in one burst.
            auto hook = [&](int k) {
#pragma unroll
                for (int part = 0; part < 4; ++part)
                    if (part * NB / 4 == k) load_chunk(c + 2, p, part);
                if (has1) {
#pragma unroll
                    for (int j = 0; j < NITEM; ++j)
                        if ((2 * j + 1) * NB / (2 * NITEM) == k) stage_item(j, q, q);
                }
                if (FUSED && k == NB / 2) {
                    if (has2) scan(c + 2, p, q);
                    load_theta(c + 3);
                }
            };
            auto after = [&]() {};
            chunk_compute(p, c, hook, after);
        };
        // whole pairs in the loop and an odd last chunk after it: a pair whose second half could be
        // skipped would give the loop head a path on which the compiler must assume few memory
        // operations since the last half's loads, and it would wait for nearly all of them there
        int64_t c = 0;
        for (; c + 1 < nchunk; c += 2) {
            iter(std::integral_constant<int, 0>{}, c);
            iter(std::integral_constant<int, 1>{}, c + 1);
        }
        if (c < nchunk) iter(std::integral_constant<int, 0>{}, c);
    } else {
        for (int64_t c = 0; c < nchunk; ++c) {
#pragma unroll
            for (int j = 0; j < MAXC + MAXX; ++j) stage_item(j, 0, 0);
            const float cd = bits_to_f32(nd[0]), cl = bits_to_f32(nl[0]);
            const float cdn = bits_to_f32(ndn[0]), cln = bits_to_f32(nln[0]);
            load_theta(c + 1);    // scanned at the end of this chunk's part 1
            load_chunk(c + 1, 0);   // the next chunk's loads fly during this one
            if (wave == NW - 1) stage_scalars(cd, cl, cdn, cln, 0);
            __syncthreads();
            auto after = [&]() {
                if (FUSED && c + 1 < nchunk) scan(c + 1, 0, 0);
            };
            chunk_compute(0, c, no_hook, after);
        }
    }

    // ---- outputs: final state and the last step's (Bbar, x) ------------------------------
    // no split: the call's; pass 1: the segment's end state, last Bbar row and (fused) end angle
    // into the workspace, and the call's x_last from the last segment (segment_combine writes
    // h_out, Bbar_last and phi_out); pass 2: none
    const bool last_seg = a.pass == 0 || seg == a.nseg - 1;
    float* hout = a.pass == 1 ? a.ws_state + (bh * a.nseg + seg) * (int64_t)(N * P)
                              : (a.pass == 0 ? a.h_out + bh * (int64_t)(N * P) : nullptr);
    T* Blast = a.pass == 1 ? (T*)a.ws_bbar + (bh * a.nseg + seg) * (int64_t)(R * N)
               : (a.pass == 0 && a.Bbar_last ? (T*)a.Bbar_last + bh * (int64_t)(R * N) : nullptr);
    T* xlast = a.pass != 2 && last_seg && a.x_last ? (T*)a.x_last + bh * (int64_t)(R * P) : nullptr;
    float* phout = !FUSED ? nullptr
                   : (a.pass == 1 ? a.ws_phiend + (bh * a.nseg + seg) * (int64_t)K
                                  : (a.pass == 0 && a.phi_out ? a.phi_out + bh * K : nullptr));
    if (a.pass == 1 && wave == NW - 1 && lane == 0) {
        a.ws_l2[bh * a.nseg + seg] = l2sum;
        a.ws_fix[bh * a.nseg + seg] = (int)min((int64_t)fix_chunks * Q, L);
    }
    if (hout) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int m = 0; m < 4; ++m) hout[(16 * nb + 4 * g + m) * P + pcol] = st[nb][m];
    }
    if (L > 0) {
        // the last chunk's tiles and angles are still in LDS (nothing is staged after it)
        const int lb = PIPE ? (int)((nchunk - 1) & 1) : 0;
        const int tlast = (int)(L - 1 - (nchunk - 1) * Q);
        if (Blast) {
            for (int e = tid; e < R * N; e += NT) {
                T v;
                if (FUSED) v = sB[lb * TB + (tlast * R + e / N) * LDB + e % N];   // rotated here only
                else v = Bg[(L - 1) * SBC + e];
                Blast[e] = v;
            }
        }
        if (xlast)
            for (int e = tid; e < R * P; e += NT) xlast[e] = Xg[(L - 1) * HRP + e];
        if (phout)
            for (int k = tid; k < K; k += NT) phout[k] = wrap_turns(sPhi[lb * TPH + (Q - 1) * LDPHI + k]) * kTwoPi;
    } else {
        // an empty sequence of a packed batch: the carry passes through unchanged
        if (Blast)
            for (int e = tid; e < R * N; e += NT) Blast[e] = Bprev ? Bprev[e] : T{};
        if (xlast)
            for (int e = tid; e < R * P; e += NT) xlast[e] = xprev ? xprev[e] : T{};
        if (phout)
            for (int k = tid; k < K; k += NT) phout[k] = phin ? wrap_angle(phin[k]) : 0.f;
    }
}

// Between the passes of a split sequence.  Angles (fused calls): segment 1 starts at segment 0's
// end angle from pass 1 (segment 0 ran at its true angles) and segment s + 1 at segment s's start
// plus the angle sum segment s formed from zero in pass 1; a segment that ran from angle 0 has
// its end state and last Bbar row off by a rotation by its start angle, and rotations of a pair
// add, so turning each (2k, 2k + 1) row pair by pair k's start angle gives the true ones.  States:
// the true end state of segment s (1 <= s <= nseg - 1; the last one is the call's h_out) is its
// own end state (from zero, turned) plus the carried state that enters it, decayed over the
// segment:
//   g_end(s) = g_local(s) + 2^{l2(s)} (g_end(s - 1) + c_{t0} Bbar_{t0-1}^T x_{t0-1})
// with l2(s) = log2 e * A * sum_{t in s} dt_t (saved by pass 1), t0 the segment's first step and
// c_{t0} = (1 - lambda_{t0}) dt_{t0}: the recurrence is linear in its carry, and the carry term is
// the one the scan adds for a carried (Bbar_prev, x_prev).  The state entering segment s,
// g_end(s - 1) + c_{t0} Bbar_{t0-1}^T x_{t0-1}, replaces g_end(s - 1) in the workspace: pass 2
// starts segment s from it.  Each thread carries row pairs (2k, 2k + 1) of one state column p,
// kCombinePairs (row pair, column) items per workgroup (two per thread, in registers along the
// chain).  Pair k's true start angles and the call's Bbar_last and phi_out come from the first
// workgroup of each (b, h) at the end.
constexpr int kCombinePairs = 512;
constexpr int kCombineBlk = 8;   // segments whose inputs are read ahead of the chain
// (x0, x1) turned by the angle with cosine cs and sine sn, as the staging rotates a row pair
__device__ __forceinline__ void turn_pair(float cs, float sn, float& x0, float& x1) {
    const float a = x0, b = x1;
    x0 = fmaf(cs, a, sn * b);
    x1 = fmaf(cs, b, -sn * a);
}
template <typename T, int R>
__global__ __launch_bounds__(256) void segment_combine_kernel(PrefillArgs a) {
    const int N = a.N, P = a.P, H = a.H, K = N / 2, nseg = a.nseg;
    const int64_t NP = (int64_t)N * P, KP = (int64_t)K * P;
    const int G = (int)((KP + kCombinePairs - 1) / kCombinePairs);
    const int64_t bh = blockIdx.x / G, b = bh / H;
    const int h = (int)(bh % H), part = (int)(blockIdx.x % G);
    const bool fused = a.ws_phiend != nullptr;
    const T* bb = (const T*)a.ws_bbar + bh * nseg * (int64_t)(R * N);
    const float* phe = fused ? a.ws_phiend + bh * nseg * (int64_t)K : nullptr;
    const float* gst = a.ws_state + bh * nseg * NP;
    bool on[2];
    int kk[2], pp[2];
    float g0[2], g1[2];
    float ph[2], php[2];   // fused: start angles of the block's first segment and of the one before
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int64_t e = (int64_t)part * kCombinePairs + threadIdx.x + 256 * j;
        on[j] = e < KP;
        kk[j] = on[j] ? (int)(e / P) : 0;
        pp[j] = on[j] ? (int)(e % P) : 0;
        g0[j] = on[j] ? gst[(2 * kk[j]) * P + pp[j]] : 0.f;   // segment 0: already true
        g1[j] = on[j] ? gst[(2 * kk[j] + 1) * P + pp[j]] : 0.f;
        ph[j] = fused ? phe[kk[j]] : 0.f;                        // segment 1 starts where 0 ended
        php[j] = 0.f;                                            // (segment 0's Bbar row is true)
    }
    // Segments in blocks of kCombineBlk: every input of a block (decays, c0, angle sums, the
    // carried-in outer products u, the segments' own end states) is read before any result is
    // written back, since a load that follows a store to the workspace waits for it; only the
    // chain through g is sequential.
    for (int s0 = 1; s0 < nseg; s0 += kCombineBlk) {
        float decay[kCombineBlk], c0[kCombineBlk], ua[kCombineBlk][2], ub[kCombineBlk][2];
        float oa[kCombineBlk][2], ob[kCombineBlk][2], ang[kCombineBlk + 1][2];
#pragma unroll
        for (int j = 0; j < 2; ++j) ang[0][j] = ph[j];
#pragma unroll
        for (int i = 0; i < kCombineBlk; ++i) {
            const int s = s0 + i < nseg ? s0 + i : s0;   // past the last one: unused
            decay[i] = exp2f(a.ws_l2[bh * nseg + s]);
            const int64_t row0 = (b * a.L + s * a.seglen) * H + h;   // step t0 of this head
            c0[i] = (1.0f - load_f32((const T*)a.lam + row0)) * load_f32((const T*)a.dt + row0);
            const T* Bp = bb + (s - 1) * (int64_t)(R * N);
            const T* xp = (const T*)a.x + (row0 - H) * R * P;
            const float* gs = gst + s * NP;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                // the next segment's start angle: this one's plus its own sum from zero
                ang[i + 1][j] = fused ? wrap_angle(ang[i][j] + phe[s * K + kk[j]]) : 0.f;
                float u0 = 0.f, u1 = 0.f;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float xv = load_f32(xp + r * P + pp[j]);
                    u0 = fmaf(load_f32(Bp + r * N + 2 * kk[j]), xv, u0);
                    u1 = fmaf(load_f32(Bp + r * N + 2 * kk[j] + 1), xv, u1);
                }
                float v0 = gs[(2 * kk[j]) * P + pp[j]], v1 = gs[(2 * kk[j] + 1) * P + pp[j]];
                if (fused) {
                    float sn, cs;
                    // the previous segment's Bbar row ran from its start angle's zero (the sum over
                    // ranks commutes with the pair's rotation; segment 0's row is already true)
                    if (s > 1) {
                        __sincosf(i == 0 ? php[j] : ang[i - 1][j], &sn, &cs);
                        turn_pair(cs, sn, u0, u1);
                    }
                    __sincosf(ang[i][j], &sn, &cs);
                    turn_pair(cs, sn, v0, v1);
                }
                ua[i][j] = u0;
                ub[i][j] = u1;
                oa[i][j] = v0;
                ob[i][j] = v1;
            }
        }
#pragma unroll
        for (int i = 0; i < kCombineBlk; ++i) {
            const int s = s0 + i;
            if (s >= nseg) break;
            float* gin = a.ws_state + (bh * nseg + s - 1) * NP;   // read in an earlier block
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                if (!on[j]) continue;
                const float c0a = fmaf(c0[i], ua[i][j], g0[j]), c0b = fmaf(c0[i], ub[i][j], g1[j]);
                gin[(2 * kk[j]) * P + pp[j]] = c0a;
                gin[(2 * kk[j] + 1) * P + pp[j]] = c0b;
                g0[j] = fmaf(decay[i], c0a, oa[i][j]);
                g1[j] = fmaf(decay[i], c0b, ob[i][j]);
                if (s + 1 == nseg) {
                    a.h_out[bh * NP + (2 * kk[j]) * P + pp[j]] = g0[j];
                    a.h_out[bh * NP + (2 * kk[j] + 1) * P + pp[j]] = g1[j];
                }
            }
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            php[j] = ang[kCombineBlk - 1][j];
            ph[j] = ang[kCombineBlk][j];
        }
    }
    // The first workgroup of the (b, h), one thread per row pair k: the true start angles of
    // segments 1 .. nseg-1 (pass 2 reads them), the call's phi_out and its Bbar_last (the last
    // segment's row turned by that segment's start angle: its second rounding to the io type).
    if (part != 0) return;
    for (int k = threadIdx.x; k < K; k += blockDim.x) {
        float sn = 0.f, cs = 1.f;
        if (fused) {
            float phs = phe[k];   // start angle of segment 1
            for (int s = 1; s < nseg; ++s) {
                a.seg_phi[(bh * nseg + s) * K + k] = phs;
                if (s + 1 < nseg) phs = wrap_angle(phs + phe[s * K + k]);
            }
            __sincosf(phs, &sn, &cs);
            if (a.phi_out) a.phi_out[bh * K + k] = wrap_angle(phs + phe[(nseg - 1) * K + k]);
        }
        if (a.Bbar_last) {
            const T* src = bb + (nseg - 1) * (int64_t)(R * N);
            T* dst = (T*)a.Bbar_last + bh * (int64_t)(R * N);
            for (int r = 0; r < R; ++r) {
                float v0 = load_f32(src + r * N + 2 * k), v1 = load_f32(src + r * N + 2 * k + 1);
                turn_pair(cs, sn, v0, v1);
                dst[r * N + 2 * k] = from_f32<T>(v0);
                dst[r * N + 2 * k + 1] = from_f32<T>(v1);
            }
        }
    }
}

template <typename T, int N, int P, bool FUSED>
hipError_t launch_np(const PrefillArgs& a, hipStream_t s) {
    const int64_t per_bh = a.pass == 0 ? 1 : (a.pass == 2 ? a.nseg - 1 : a.nseg);
    const dim3 grid((unsigned)(a.b * a.H * per_bh)), block(P / 16 * 64);
    // fused: BCNorm weights and biases in dynamic LDS
    const size_t dyn = FUSED ? (size_t)(2 * N + 2 * a.R * N) * sizeof(float) : 0;
    switch (a.Q * a.R) {
        case 16: hipLaunchKernelGGL((prefill_kernel<T, N, P, 1, FUSED>), grid, block, dyn, s, a); break;
        case 32:
            // fused with ranks: two rows of one step per staging thread (angles taken once)
            if (FUSED && a.R >= 2)
                hipLaunchKernelGGL((prefill_kernel<T, N, P, 2, FUSED, true>), grid, block, dyn, s, a);
            else
                hipLaunchKernelGGL((prefill_kernel<T, N, P, 2, FUSED>), grid, block, dyn, s, a);
            break;
        case 48:
            if (FUSED || a.pass) return hipErrorInvalidValue;   // never split (48 does not divide 512)
            hipLaunchKernelGGL((prefill_kernel<T, N, P, 3, false>), grid, block, 0, s, a);
            break;
        case 64: hipLaunchKernelGGL((prefill_kernel<T, N, P, 4, FUSED>), grid, block, dyn, s, a); break;
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
    // chunk rows 16, 32 or 64 (the angle scan wants a power-of-two step count)
    return prefill_supported(N, P, R, QR, bf16_io) && QR != 48;
}

hipError_t launch_layer(const PrefillArgs& a, bool bf16_io, hipStream_t s) {
    return bf16_io ? launch_t<bf16, true>(a, s) : launch_t<float, true>(a, s);
}

template <typename T>
hipError_t launch_combine_t(const PrefillArgs& a, dim3 grid, hipStream_t s) {
    switch (a.R) {   // the ranks as a constant: the loads of a block of segments go out together
        case 1: hipLaunchKernelGGL((segment_combine_kernel<T, 1>), grid, dim3(256), 0, s, a); break;
        case 2: hipLaunchKernelGGL((segment_combine_kernel<T, 2>), grid, dim3(256), 0, s, a); break;
        case 4: hipLaunchKernelGGL((segment_combine_kernel<T, 4>), grid, dim3(256), 0, s, a); break;
        case 8: hipLaunchKernelGGL((segment_combine_kernel<T, 8>), grid, dim3(256), 0, s, a); break;
        case 16: hipLaunchKernelGGL((segment_combine_kernel<T, 16>), grid, dim3(256), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_segment_combine(const PrefillArgs& a, bool bf16_io, hipStream_t s) {
    const int64_t G = ((int64_t)(a.N / 2) * a.P + kCombinePairs - 1) / kCombinePairs;
    const dim3 grid((unsigned)(a.b * a.H * G));
    return bf16_io ? launch_combine_t<bf16>(a, grid, s) : launch_combine_t<float>(a, grid, s);
}

}  // namespace m3
