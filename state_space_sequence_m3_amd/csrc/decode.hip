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
#include "m3_device.h"
#include "m3_launch.h"

namespace m3 {

namespace {

constexpr int kDecThreads = 256;
constexpr int kDecBatch = 8;   // float4 state loads in flight per thread

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
    const T* Bt = (const T*)a.Bbar + bh * R * N;
    const T* Ct = (const T*)a.Cbar + bh * R * N;
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

template <typename T, bool FUSED>
hipError_t launch_t(const DecodeArgs& a, hipStream_t s) {
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
