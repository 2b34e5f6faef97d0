// decode.hip -- m3_decode_step kernel: one token, b*H resident fp32 states updated in place.
//
// Recurrence: aipaper.cc summary of Mamba-3, section 4.1 Proposition 1 (alpha, beta, gamma) and
// section 4.3 (MIMO: the update is a rank-R product B X^T).  In the rotated frame the step is
//   h <- alpha h + beta Bbar_prev^T x_prev + gamma Bbar^T x,   Y[r] = Cbar[r] h,
// a rank-2R update of an N x P fp32 matrix followed by R dot products over N.  Per (b, h) the
// state (N*P*4 bytes) is read once and written once; everything else is a few hundred bytes, so
// the kernel is bound by HBM bandwidth (papernotes.org, key design 3: decode is memory bound).
//
// Fused step (FUSED): the token's B and C arrive raw and are first normalised (BCNorm), biased and
// rotated by the carried angle advanced by dt * theta (papernotes.org, key design 4; aipaper.cc
// section 4.2 Proposition 3), which is m3_bcnorm_rope with L = 1 done in the staging of this
// kernel: wave w takes ranks w, w + 4, ..., lane k takes rotation pairs k, k + 64, ...
//
// Mapping: one 256-thread workgroup per (b, h).  Thread t owns the float4 columns
// [4t mod P, 4t mod P + 4) of rows n = (4t + 1024 k) / P, so a wave reads 1 KB contiguous per
// load and every thread's p-range is fixed (P divides 1024).  The small per-token vectors are
// staged once in LDS as fp32.  The Y partial sums are reduced across lanes that share a
// p-range with xor shuffles, then across the four waves through LDS.
#include <atomic>

#include "m3_device.h"
#include "m3_launch.h"

namespace m3 {

namespace {

constexpr int kDecThreads = 256;
constexpr int kDecBatch = 8;   // float4 state loads in flight per thread
constexpr int kMaxDevices = 64;

template <typename T, int R, bool FUSED>
__global__ __launch_bounds__(kDecThreads) void decode_step_kernel(DecodeArgs a) {
    // staging pool: Bprev, B, C (R*N each) and xprev, x (R*P each); reused for the Y reduction
    __shared__ float pool[5 * R * 256];
    float* sBp = pool;
    float* sBt = sBp + R * a.N;
    float* sCt = sBt + R * a.N;
    float* sXp = sCt + R * a.N;
    float* sXt = sXp + R * a.P;

    const int N = a.N, P = a.P;
    const int64_t bh = blockIdx.x;
    const int h = (int)(bh % a.H);
    const int tid = threadIdx.x;

    const T* Bp = (const T*)a.Bbar_prev + bh * R * N;
    // the token's B and C: per head, or (fused, head groups) the raw rows of the head's slot
    const int64_t rowBC = FUSED ? (bh / a.H) * bc_slots(a.H, a.G) + bc_slot(h, a.H, a.G) : bh;
    const T* Bt = (const T*)a.Bbar + rowBC * R * N;
    const T* Ct = (const T*)a.Cbar + rowBC * R * N;
    const T* xp = (const T*)a.x_prev + bh * R * P;
    const T* xt = (const T*)a.x + bh * R * P;
    float4* hp = (float4*)(a.h + bh * (int64_t)N * P);
    const int nq = (N * P) >> 2;
    float4 g0[kDecBatch];   // the first batch of the state
    auto load_state0 = [&]() {
#pragma unroll
        for (int k = 0; k < kDecBatch; ++k) {
            const int q = tid + k * kDecThreads;
            if (q < nq) g0[k] = hp[q];
        }
    };
    const float d = load_f32((const T*)a.dt + bh);
    if (FUSED) {
        // The token's rotation: Phi = Phi_carried + dt * theta on pairs k = lane, lane + 64, ...
        // The small loads go out first, then the first batch of the state, so that waiting for
        // the former (the vector memory counter drains in order) does not wait for the latter.
        const int wave = tid >> 6, lane = tid & 63, K = N / 2;
        constexpr int KMAX = 2;                    // pairs per lane (N <= 256)
        constexpr int RPW = (R + 3) / 4;           // ranks per wave
        const T* th = (const T*)a.theta + bh * K;
        float* phi = a.phi + bh * K;
        float ph[KMAX], tv[KMAX];
        float raw[RPW][2][KMAX][2], wt[2][KMAX][2], bs[RPW][2][KMAX][2];
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            const int k = lane + 64 * j;
            ph[j] = k < K ? phi[k] : 0.f;
            tv[j] = k < K ? load_f32(th + k) : 0.f;
#pragma unroll
            for (int wc = 0; wc < 2; ++wc) {
                const float* w = wc == 0 ? a.normw_B : a.normw_C;
#pragma unroll
                for (int e = 0; e < 2; ++e) wt[wc][j][e] = (a.bcnorm && w && k < K) ? w[h * N + 2 * k + e] : 1.f;
            }
#pragma unroll
            for (int i = 0; i < RPW; ++i) {
                const int r = wave + 4 * i;
#pragma unroll
                for (int wc = 0; wc < 2; ++wc) {
                    const T* src = (wc == 0 ? Bt : Ct) + r * N;
                    const float* bias = wc == 0 ? a.bias_B : a.bias_C;
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const bool in = r < R && k < K;
                        raw[i][wc][j][e] = in ? load_f32(src + 2 * k + e) : 0.f;
                        bs[i][wc][j][e] = (in && bias) ? bias[(h * R + r) * N + 2 * k + e] : 0.f;
                    }
                }
            }
        }
        for (int e = tid; e < R * N; e += kDecThreads) sBp[e] = load_f32(Bp + e);
        load_state0();
        float cs[KMAX], sn[KMAX], ang[KMAX];
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            ang[j] = wrap_angle(ph[j] + d * tv[j]);
            __sincosf(ang[j], &sn[j], &cs[j]);
        }
        const float invN = 1.0f / (float)N;
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int r = wave + 4 * i;
            if (r >= R) break;
#pragma unroll
            for (int wc = 0; wc < 2; ++wc) {
                float q = 0.f;
#pragma unroll
                for (int j = 0; j < KMAX; ++j)
                    q = fmaf(raw[i][wc][j][0], raw[i][wc][j][0], fmaf(raw[i][wc][j][1], raw[i][wc][j][1], q));
                const float sc = a.bcnorm ? rsqrtf(group_sum(q, 64) * invN + a.eps) : 1.f;
                float* dst = (wc == 0 ? sBt : sCt) + r * N;
#pragma unroll
                for (int j = 0; j < KMAX; ++j) {
                    const int k = lane + 64 * j;
                    if (k >= K) continue;
                    const float u0 = fmaf(raw[i][wc][j][0] * sc, wt[wc][j][0], bs[i][wc][j][0]);
                    const float u1 = fmaf(raw[i][wc][j][1] * sc, wt[wc][j][1], bs[i][wc][j][1]);
                    const float o0 = cs[j] * u0 + sn[j] * u1;
                    const float o1 = -sn[j] * u0 + cs[j] * u1;
                    dst[2 * k] = o0;
                    dst[2 * k + 1] = o1;
                    if (wc == 0) {   // the rotated B is the next step's Bbar_prev
                        T* bo = (T*)a.Bbar_out + (bh * R + r) * N;
                        bo[2 * k] = from_f32<T>(o0);
                        bo[2 * k + 1] = from_f32<T>(o1);
                    }
                }
            }
        }
        __syncthreads();   // every wave has read the carried angle before wave 0 rewrites it
        if (wave == 0) {
#pragma unroll
            for (int j = 0; j < KMAX; ++j)
                if (lane + 64 * j < K) phi[lane + 64 * j] = ang[j];
        }
    } else {
        for (int e = tid; e < R * N; e += kDecThreads) {
            sBp[e] = load_f32(Bp + e);
            sBt[e] = load_f32(Bt + e);
            sCt[e] = load_f32(Ct + e);
        }
        load_state0();
    }
    for (int e = tid; e < R * P; e += kDecThreads) {
        sXp[e] = load_f32(xp + e);
        sXt[e] = load_f32(xt + e);
    }
    const float lm = load_f32((const T*)a.lam + bh);
    const float alpha = __expf(d * a.A[h]);
    const float beta = (1.0f - lm) * d * alpha;
    const float gamma = lm * d;
    __syncthreads();

    const int p0 = (4 * tid) & (P - 1);
    float yp[R][4];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) yp[r][j] = 0.0f;

    float xpv[R][4], xtv[R][4];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            xpv[r][j] = sXp[r * P + p0 + j];
            xtv[r][j] = sXt[r * P + p0 + j];
        }

    for (int base = tid; base < nq; base += kDecThreads * kDecBatch) {
        float4 g[kDecBatch];
#pragma unroll
        for (int k = 0; k < kDecBatch; ++k) {
            const int q = base + k * kDecThreads;
            if (base == tid) g[k] = g0[k];
            else if (q < nq) g[k] = hp[q];
        }
#pragma unroll
        for (int k = 0; k < kDecBatch; ++k) {
            const int q = base + k * kDecThreads;
            if (q < nq) {
                const int n = (4 * q) / P;
                float up[4] = {0.f, 0.f, 0.f, 0.f}, ut[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float bp = sBp[r * N + n], bt = sBt[r * N + n];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        up[j] += bp * xpv[r][j];
                        ut[j] += bt * xtv[r][j];
                    }
                }
                float4 v = g[k];
                v.x = alpha * v.x + beta * up[0] + gamma * ut[0];
                v.y = alpha * v.y + beta * up[1] + gamma * ut[1];
                v.z = alpha * v.z + beta * up[2] + gamma * ut[2];
                v.w = alpha * v.w + beta * up[3] + gamma * ut[3];
                hp[q] = v;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float c = sCt[r * N + n];
                    yp[r][0] += c * v.x;
                    yp[r][1] += c * v.y;
                    yp[r][2] += c * v.z;
                    yp[r][3] += c * v.w;
                }
            }
        }
    }

    // lanes l and l ^ m (m >= P/4) hold the same p-range: reduce them
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            for (int m = P >> 2; m < 64; m <<= 1) yp[r][j] += shfl_xor(yp[r][j], m);

    __syncthreads();  // staging pool is reused below
    float* sY = pool;                 // [4 waves][R][P]
    float* sYt = pool + 4 * R * P;    // [R][P]
    const int wave = tid >> 6, lane = tid & 63;
    if (lane < (P >> 2)) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j) sY[(wave * R + r) * P + p0 + j] = yp[r][j];
    }
    __syncthreads();
    for (int e = tid; e < R * P; e += kDecThreads)
        sYt[e] = sY[e] + sY[R * P + e] + sY[2 * R * P + e] + sY[3 * R * P + e];
    __syncthreads();
    T* y = (T*)a.y;
    if (a.w_out) {
        for (int p = tid; p < P; p += kDecThreads) {
            float acc = 0.0f;
#pragma unroll
            for (int r = 0; r < R; ++r) acc += a.w_out[(h * R + r) * P + p] * sYt[r * P + p];
            y[bh * P + p] = from_f32<T>(acc);
        }
    } else {
        for (int e = tid; e < R * P; e += kDecThreads) y[bh * R * P + e] = from_f32<T>(sYt[e]);
    }
}

// ---------------------------------------------------------------------------------------------
// Streaming form for the common shapes (N x P in {128 x 64, 64 x 64}, R <= 4): a persistent grid
// of as many workgroups as the GPU holds at once walks the (b, h) pairs q, q + G, q + 2G, ...
// While pair q is updated, the state and the token inputs of pair q + G are already in flight
// (registers), so a workgroup keeps HBM reads outstanding through its whole life instead of
// alternating between a load phase and a compute phase.  G is a multiple of H (or covers every
// pair at once), so a workgroup always serves the same head: the per-head constants (A, BCNorm
// weights, biases, mixing weights) are staged in LDS once.  Per pair there is one barrier: the
// staged vectors and the Y partial sums are double-buffered by pair parity.
//
// LDS: per parity, Bbar_prev, Bbar, Cbar as [n][r] (one LDS read serves every rank of a row) and
// x_prev, x as [r][p]; per parity, the Y partial sums [wave][r][p]; the head constants.
// NTS: the states of the call are far larger than the last-level cache, so every step streams
// them from DRAM: their loads and stores are non-temporal (a read-modify-write stream in place
// moves ~10% more that way; for states the cache can partly hold, the default policy is faster).
template <typename T, int N, int P, int R, bool FUSED, bool NTS>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(FUSED && R == 4 ? 3 : 4))) void decode_stream_kernel(DecodeArgs a) {
    constexpr int NT = kDecThreads, K = N / 2;
    constexpr int NQ = N * P / (4 * NT);                 // float4 of state per thread per pair
    constexpr int ROWS = 4 * NT / P;                     // rows between a thread's float4 slots
    constexpr int JN = (R * N + NT - 1) / NT, JP = (R * P + NT - 1) / NT;
    constexpr int KMAX = (K + 63) / 64, RPW = (R + 3) / 4;
    constexpr int VB = 3 * N * R + 2 * R * P;            // floats per staging buffer
    constexpr int YB = 4 * R * P;                        // floats per Y partial buffer
    constexpr int CB = 2 * N + 2 * R * N + R * P;        // head constants
    static_assert(NQ >= 1 && NQ * 4 * NT == N * P && (P & (P - 1)) == 0 && P <= 4 * NT, "state layout");
    static_assert(R == 1 || R == 2 || R == 4, "rank");
    typedef typename IoBits<T>::type Bits;
    __shared__ __align__(16) float smem[2 * VB + 2 * YB + CB];
    float* sWB = smem + 2 * VB + 2 * YB;   // BCNorm weights [N] (B, then C)
    float* sWC = sWB + N;
    float* sbB = sWC + N;                  // biases [R][N]
    float* sbC = sbB + R * N;
    float* sWo = sbC + R * N;              // mixing weights [R][P]

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int H = a.H;
    const int64_t npairs = a.b * H, G = gridDim.x;
    const int h = (int)(blockIdx.x % H);
    const int p0 = (4 * tid) & (P - 1), n0 = (4 * tid) / P;
    constexpr uint32_t ES = sizeof(T);

    // ---- head constants (every pair of this workgroup has head h)
    for (int e = tid; e < N; e += NT) {
        sWB[e] = (FUSED && a.bcnorm && a.normw_B) ? a.normw_B[h * N + e] : 1.f;
        sWC[e] = (FUSED && a.bcnorm && a.normw_C) ? a.normw_C[h * N + e] : 1.f;
    }
    for (int e = tid; e < R * N; e += NT) {
        sbB[e] = (FUSED && a.bias_B) ? a.bias_B[h * R * N + e] : 0.f;
        sbC[e] = (FUSED && a.bias_C) ? a.bias_C[h * R * N + e] : 0.f;
    }
    for (int e = tid; e < R * P; e += NT) sWo[e] = a.w_out ? a.w_out[h * R * P + e] : 0.f;
    const float Ah = a.A[h];

    // ---- token inputs of the pair in flight (raw bits) and its state
    Bits rBp[JN], rB[JN], rC[JN], rXp[JP], rX[JP], rdt, rlam;
    Bits fB[RPW][KMAX][2], fC[RPW][KMAX][2], fth[KMAX];
    float fph[KMAX];
    uint4 gc[NQ], gn[NQ];
    // every load is issued (zero-sized descriptors past the last pair), so the wait counts the
    // compiler derives are the same on every path; token inputs go out before the state
    auto load_pair = [&](int64_t qq, uint4 (&g)[NQ]) {
        const bool ok = qq < npairs;
        const int64_t bh = ok ? qq : 0;
        const rsrc_t rsBp = make_rsrc((const T*)a.Bbar_prev + bh * R * N, ok ? R * N * ES : 0);
        // the token's B and C: per head, or (fused, head groups) the raw rows of the head's slot
        const int64_t rowBC = FUSED ? (bh / H) * bc_slots(H, a.G) + bc_slot(h, H, a.G) : bh;
        const rsrc_t rsB = make_rsrc((const T*)a.Bbar + rowBC * R * N, ok ? R * N * ES : 0);
        const rsrc_t rsC = make_rsrc((const T*)a.Cbar + rowBC * R * N, ok ? R * N * ES : 0);
        const rsrc_t rsXp = make_rsrc((const T*)a.x_prev + bh * R * P, ok ? R * P * ES : 0);
        const rsrc_t rsX = make_rsrc((const T*)a.x + bh * R * P, ok ? R * P * ES : 0);
        rdt = buffer_load_bits(make_rsrc((const T*)a.dt + bh, ok ? ES : 0), 0, T{});
        rlam = buffer_load_bits(make_rsrc((const T*)a.lam + bh, ok ? ES : 0), 0, T{});
#pragma unroll
        for (int j = 0; j < JN; ++j) rBp[j] = buffer_load_bits(rsBp, (tid + NT * j) * ES, T{});
#pragma unroll
        for (int j = 0; j < JP; ++j) {
            rXp[j] = buffer_load_bits(rsXp, (tid + NT * j) * ES, T{});
            rX[j] = buffer_load_bits(rsX, (tid + NT * j) * ES, T{});
        }
        if (!FUSED) {
#pragma unroll
            for (int j = 0; j < JN; ++j) {
                rB[j] = buffer_load_bits(rsB, (tid + NT * j) * ES, T{});
                rC[j] = buffer_load_bits(rsC, (tid + NT * j) * ES, T{});
            }
        } else {
            // rank wave + 4 i, rotation pair lane + 64 j: elements 2k, 2k + 1 of the row
            const rsrc_t rsTh = make_rsrc((const T*)a.theta + bh * K, ok ? K * ES : 0);
            const rsrc_t rsPh = make_rsrc(a.phi + bh * K, ok ? K * 4 : 0);
#pragma unroll
            for (int j = 0; j < KMAX; ++j) {
                const int k = lane + 64 * j;
                const uint32_t kk = k < K ? (uint32_t)k : (uint32_t)K;   // past the row: reads zero
                fth[j] = buffer_load_bits(rsTh, kk * ES, T{});
                fph[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsPh, (int)(kk * 4), 0, 0));
#pragma unroll
                for (int i = 0; i < RPW; ++i) {
                    const int r = wave + 4 * i;
                    const uint32_t o = r < R && k < K ? (uint32_t)(r * N + 2 * k) * ES : (uint32_t)(R * N) * ES;
                    fB[i][j][0] = buffer_load_bits(rsB, o, T{});
                    fB[i][j][1] = buffer_load_bits(rsB, o + ES, T{});
                    fC[i][j][0] = buffer_load_bits(rsC, o, T{});
                    fC[i][j][1] = buffer_load_bits(rsC, o + ES, T{});
                }
            }
        }
        const rsrc_t rsH = make_rsrc(a.h + bh * (int64_t)(N * P), ok ? N * P * 4 : 0);
#pragma unroll
        for (int k = 0; k < NQ; ++k)
            g[k] = NTS ? buffer_load16_stream(rsH, (uint32_t)(tid + NT * k) * 16)
                       : buffer_load16(rsH, (uint32_t)(tid + NT * k) * 16);
    };

    // ---- stage a pair's token vectors into LDS buffer `par`; returns its step scalars
    float ang[KMAX];
    auto stage = [&](int64_t qq, int par, float& alpha, float& beta, float& gamma) {
        float* sBp = smem + par * VB;
        float* sB = sBp + N * R;
        float* sC = sB + N * R;
        float* sXp = sC + N * R;
        float* sX = sXp + R * P;
        const float d = bits_to_f32(rdt), lm = bits_to_f32(rlam);
        alpha = __expf(d * Ah);
        beta = (1.0f - lm) * d * alpha;
        gamma = lm * d;
#pragma unroll
        for (int j = 0; j < JN; ++j) {
            const int e = tid + NT * j;
            if (e < R * N) {
                const int r = e / N, n = e - r * N;
                sBp[n * R + r] = bits_to_f32(rBp[j]);
                if (!FUSED) {
                    sB[n * R + r] = bits_to_f32(rB[j]);
                    sC[n * R + r] = bits_to_f32(rC[j]);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < JP; ++j) {
            const int e = tid + NT * j;
            if (e < R * P) {
                sXp[e] = bits_to_f32(rXp[j]);
                sX[e] = bits_to_f32(rX[j]);
            }
        }
        if (FUSED) {
            // the token's rotation: Phi = Phi_carried + dt * theta; BCNorm, weight, bias, rotate
            float cs[KMAX], sn[KMAX];
#pragma unroll
            for (int j = 0; j < KMAX; ++j) {
                ang[j] = wrap_angle(fph[j] + d * bits_to_f32(fth[j]));
                __sincosf(ang[j], &sn[j], &cs[j]);
            }
            const float invN = 1.0f / (float)N;
#pragma unroll
            for (int i = 0; i < RPW; ++i) {
                const int r = wave + 4 * i;
                if (r >= R) break;
#pragma unroll
                for (int wc = 0; wc < 2; ++wc) {
                    float v[KMAX][2];
                    float q2 = 0.f;
#pragma unroll
                    for (int j = 0; j < KMAX; ++j)
#pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            v[j][e] = bits_to_f32(wc == 0 ? fB[i][j][e] : fC[i][j][e]);
                            q2 = fmaf(v[j][e], v[j][e], q2);
                        }
                    const float sc = a.bcnorm ? rsqrtf(group_sum(q2, 64) * invN + a.eps) : 1.f;
                    const float* w = wc == 0 ? sWB : sWC;
                    const float* bias = (wc == 0 ? sbB : sbC) + r * N;
                    float* dst = wc == 0 ? sB : sC;
#pragma unroll
                    for (int j = 0; j < KMAX; ++j) {
                        const int k = lane + 64 * j;
                        if (k >= K) continue;
                        const float u0 = fmaf(v[j][0] * sc, w[2 * k], bias[2 * k]);
                        const float u1 = fmaf(v[j][1] * sc, w[2 * k + 1], bias[2 * k + 1]);
                        const float o0 = cs[j] * u0 + sn[j] * u1;
                        const float o1 = -sn[j] * u0 + cs[j] * u1;
                        dst[(2 * k) * R + r] = o0;
                        dst[(2 * k + 1) * R + r] = o1;
                        if (wc == 0) {   // the rotated B is the next step's Bbar_prev
                            T* bo = (T*)a.Bbar_out + (qq * R + r) * N;
                            bo[2 * k] = from_f32<T>(o0);
                            bo[2 * k + 1] = from_f32<T>(o1);
                        }
                    }
                }
            }
        }
    };
    // after the barrier that follows a pair's staging, every wave has consumed the carried angle
    auto write_angle = [&](int64_t qq) {
        if (FUSED && wave == 0) {
#pragma unroll
            for (int j = 0; j < KMAX; ++j)
                if (lane + 64 * j < K) a.phi[qq * K + lane + 64 * j] = ang[j];
        }
    };

    // ---- update pair qq's state (in gc) with the vectors of buffer `par`; Y partials to LDS
    auto compute = [&](int64_t qq, int par, float alpha, float beta, float gamma) {
        const float* sBp = smem + par * VB;
        const float* sB = sBp + N * R;
        const float* sC = sB + N * R;
        const float* sXp = sC + N * R;
        const float* sX = sXp + R * P;
        float xb[R][4], xg[R][4], yp[R][4];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float4 u = *(const float4*)(sXp + r * P + p0);
            const float4 w = *(const float4*)(sX + r * P + p0);
            xb[r][0] = beta * u.x; xb[r][1] = beta * u.y; xb[r][2] = beta * u.z; xb[r][3] = beta * u.w;
            xg[r][0] = gamma * w.x; xg[r][1] = gamma * w.y; xg[r][2] = gamma * w.z; xg[r][3] = gamma * w.w;
#pragma unroll
            for (int j = 0; j < 4; ++j) yp[r][j] = 0.f;
        }
        const rsrc_t rsH = make_rsrc(a.h + qq * (int64_t)(N * P), N * P * 4);
#pragma unroll
        for (int k = 0; k < NQ; ++k) {
            const int n = n0 + ROWS * k;
            float bp[R], bt[R], ct[R];
            if (R == 4) {
                const float4 u = *(const float4*)(sBp + n * 4), v = *(const float4*)(sB + n * 4),
                             w = *(const float4*)(sC + n * 4);
                bp[0] = u.x; bp[R > 1 ? 1 : 0] = u.y; bp[R > 2 ? 2 : 0] = u.z; bp[R > 3 ? 3 : 0] = u.w;
                bt[0] = v.x; bt[R > 1 ? 1 : 0] = v.y; bt[R > 2 ? 2 : 0] = v.z; bt[R > 3 ? 3 : 0] = v.w;
                ct[0] = w.x; ct[R > 1 ? 1 : 0] = w.y; ct[R > 2 ? 2 : 0] = w.z; ct[R > 3 ? 3 : 0] = w.w;
            } else if (R == 2) {
                const float2 u = *(const float2*)(sBp + n * 2), v = *(const float2*)(sB + n * 2),
                             w = *(const float2*)(sC + n * 2);
                bp[0] = u.x; bp[R > 1 ? 1 : 0] = u.y;
                bt[0] = v.x; bt[R > 1 ? 1 : 0] = v.y;
                ct[0] = w.x; ct[R > 1 ? 1 : 0] = w.y;
            } else {
                bp[0] = sBp[n]; bt[0] = sB[n]; ct[0] = sC[n];
            }
            float g[4] = {__uint_as_float(gc[k].x), __uint_as_float(gc[k].y), __uint_as_float(gc[k].z),
                          __uint_as_float(gc[k].w)};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float v = alpha * g[j];
#pragma unroll
                for (int r = 0; r < R; ++r) v = fmaf(bt[r], xg[r][j], fmaf(bp[r], xb[r][j], v));
                g[j] = v;
            }
            (NTS ? buffer_store16_stream : buffer_store16)(rsH, (uint32_t)(tid + NT * k) * 16,
                           make_uint4(__float_as_uint(g[0]), __float_as_uint(g[1]), __float_as_uint(g[2]),
                                      __float_as_uint(g[3])));
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int j = 0; j < 4; ++j) yp[r][j] = fmaf(ct[r], g[j], yp[r][j]);
        }
        // lanes l and l ^ m (m >= P/4) hold the same columns
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int m = P / 4; m < 64; m <<= 1) yp[r][j] += shfl_xor(yp[r][j], m);
        float* sY = smem + 2 * VB + par * YB;
        if (lane < P / 4) {
#pragma unroll
            for (int r = 0; r < R; ++r)
                *(float4*)(sY + (wave * R + r) * P + p0) = make_float4(yp[r][0], yp[r][1], yp[r][2], yp[r][3]);
        }
    };
    // ---- after the barrier: sum the four waves' partials, mix, store y of pair qq
    auto finish = [&](int64_t qq, int par) {
        const float* sY = smem + 2 * VB + par * YB;
        T* y = (T*)a.y;
        if (a.w_out) {
            for (int p = tid; p < P; p += NT) {
                float acc = 0.f;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float s = (sY[r * P + p] + sY[(R + r) * P + p]) + (sY[(2 * R + r) * P + p] + sY[(3 * R + r) * P + p]);
                    acc = fmaf(sWo[r * P + p], s, acc);
                }
                y[qq * P + p] = from_f32<T>(acc);
            }
        } else {
            for (int e = tid; e < R * P; e += NT)
                y[qq * R * P + e] = from_f32<T>((sY[e] + sY[R * P + e]) + (sY[2 * R * P + e] + sY[3 * R * P + e]));
        }
    };

    int64_t q = blockIdx.x;
    float al, be, ga, nal = 0.f, nbe = 0.f, nga = 0.f;
    load_pair(q, gc);
    __syncthreads();   // head constants
    stage(q, 0, al, be, ga);
    __syncthreads();
    write_angle(q);
    int par = 0;
    for (; q < npairs; q += G) {
        const int64_t qn = q + G;
        load_pair(qn, gn);
        compute(q, par, al, be, ga);
        if (qn < npairs) stage(qn, par ^ 1, nal, nbe, nga);
        __syncthreads();
        finish(q, par);
        if (qn < npairs) write_angle(qn);
#pragma unroll
        for (int k = 0; k < NQ; ++k) gc[k] = gn[k];
        al = nal; be = nbe; ga = nga;
        par ^= 1;
    }
}

// resident workgroups of a kernel on the current device (all CUs), cached per device
template <typename K>
int resident_workgroups(K kernel, std::atomic<int> (&cache)[kMaxDevices]) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < kMaxDevices) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int ncu = 0, per = 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, reinterpret_cast<const void*>(kernel), kDecThreads, 0) !=
        hipSuccess)
        return 0;
    const int c = ncu * per;
    if (dev < kMaxDevices && c > 0) cache[dev].store(c, std::memory_order_relaxed);
    return c;
}

// the streaming kernel's grid for this call, or 0 when it does not apply (then the per-pair
// kernel runs): every pair at once, else a multiple of H that the GPU holds at once
inline int64_t stream_grid(int64_t npairs, int H, int resident) {
    if (resident <= 0) return 0;
    if (npairs <= resident) return npairs;
    const int64_t g = (int64_t)(resident / H) * H;
    return g;
}

// states larger than this stream from DRAM on every step (the last-level cache is 256 MB)
constexpr int64_t kStreamStateBytes = (int64_t)512 << 20;

template <typename T, int N, int P, int R, bool FUSED, bool NTS>
hipError_t launch_stream_nts(const DecodeArgs& a, hipStream_t s, bool& done) {
    static std::atomic<int> cache[kMaxDevices];
    auto kern = decode_stream_kernel<T, N, P, R, FUSED, NTS>;
    const int64_t grid = stream_grid(a.b * a.H, a.H, resident_workgroups(kern, cache));
    done = grid > 0;
    if (!done) return hipSuccess;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kDecThreads), 0, s, a);
    return hipGetLastError();
}

template <typename T, int N, int P, int R, bool FUSED>
hipError_t launch_stream(const DecodeArgs& a, hipStream_t s, bool& done) {
    const bool nts = a.b * a.H * (int64_t)N * P * 4 > kStreamStateBytes;
    return nts ? launch_stream_nts<T, N, P, R, FUSED, true>(a, s, done)
               : launch_stream_nts<T, N, P, R, FUSED, false>(a, s, done);
}

template <typename T, int N, int P, bool FUSED>
hipError_t launch_stream_np(const DecodeArgs& a, hipStream_t s, bool& done) {
    switch (a.R) {
        case 1: return launch_stream<T, N, P, 1, FUSED>(a, s, done);
        case 2: return launch_stream<T, N, P, 2, FUSED>(a, s, done);
        case 4: return launch_stream<T, N, P, 4, FUSED>(a, s, done);
        default: done = false; return hipSuccess;
    }
}

template <typename T, bool FUSED>
hipError_t launch_t(const DecodeArgs& a, hipStream_t s) {
    bool done = false;
    hipError_t e = hipSuccess;
    if (a.N == 128 && a.P == 64) e = launch_stream_np<T, 128, 64, FUSED>(a, s, done);
    else if (a.N == 64 && a.P == 64) e = launch_stream_np<T, 64, 64, FUSED>(a, s, done);
    if (e != hipSuccess || done) return e;
    const dim3 grid((unsigned)(a.b * a.H)), block(kDecThreads);
    switch (a.R) {
        case 1: hipLaunchKernelGGL((decode_step_kernel<T, 1, FUSED>), grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL((decode_step_kernel<T, 2, FUSED>), grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL((decode_step_kernel<T, 4, FUSED>), grid, block, 0, s, a); break;
        case 8: hipLaunchKernelGGL((decode_step_kernel<T, 8, FUSED>), grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

bool decode_supported(int N, int P, int R) {
    const bool p_ok = P >= 4 && P <= 256 && (P & (P - 1)) == 0;
    const bool r_ok = R == 1 || R == 2 || R == 4 || R == 8;
    return p_ok && r_ok && N >= 1 && N <= 256;
}

hipError_t launch_decode(const DecodeArgs& a, bool bf16_io, hipStream_t s) {
    return bf16_io ? launch_t<bf16, false>(a, s) : launch_t<float, false>(a, s);
}

hipError_t launch_layer_decode(const DecodeArgs& a, bool bf16_io, hipStream_t s) {
    return bf16_io ? launch_t<bf16, true>(a, s) : launch_t<float, true>(a, s);
}

}  // namespace m3
