// bcnorm_rope.hip -- m3_bcnorm_rope: BCNorm + head bias + cumulative rotation of B and C.
//
// BCNorm (RMS normalisation of each projected B/C vector, with an optional weight) and the
// head-specific bias: papernotes.org summary of Mamba-3, key design 4.  The rotation: aipaper.cc
// summary, section 4.2 Proposition 3 -- B_t and C_t are multiplied by the cumulative product of
// R_i^T over i = 0..t, where R_i is block-diagonal with 2x2 blocks of angle dt_i * theta_i[k]
// (metaphor-xennon SSM comparison, section 2.2).  The blocks commute, so the product is one
// rotation by Phi_t[k] = Phi_in[k] + sum_{i<=t} dt_i theta_i[k] on each pair (2k, 2k+1).
//
// The angle is a prefix sum along the sequence, the only sequential part.  Long sequences are
// cut into segments of kSegLen steps, one workgroup of four waves per (b, h, segment), each wave
// walking a quarter of the segment: angle_partial_kernel sums dt*theta over every quarter in
// parallel, angle_scan_kernel turns those sums into quarter start angles (a scan over a few dozen
// quarters per (b, h)) and the final angle, and bcnorm_rope_kernel does the elementwise work, each
// wave carrying its quarter's angle in registers.  A sequence of one segment has no partial pass:
// its waves sum their quarters' increments first and exchange them through LDS.  Angles are kept
// reduced to [-pi, pi] so the fp32 rounding of the running sum stays at the size of one ulp of pi.
//
// Lane mapping: each (t, r) row of N values is split over N/8 lanes, 8 values (4 rotation
// pairs) per lane, so one wave instruction moves 512/N whole rows.  The RMS over N is a
// shuffle reduction within a row's N/8 lanes.
#include "m3_device.h"
#include "m3_launch.h"

namespace m3 {

namespace {

constexpr int64_t kSegLen = 512;
constexpr int kParts = 4;   // waves (quarters) per segment in the partial pass and the main pass

__device__ __forceinline__ void load4(const float* p, float o[4]) {
    const float4 v = *(const float4*)p;
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
}
__device__ __forceinline__ void load4(const bf16* p, float o[4]) {
    const uint2 v = *(const uint2*)p;
    o[0] = __uint_as_float(v.x << 16);
    o[1] = __uint_as_float(v.x & 0xffff0000u);
    o[2] = __uint_as_float(v.y << 16);
    o[3] = __uint_as_float(v.y & 0xffff0000u);
}
__device__ __forceinline__ void load8(const float* p, float o[8]) {
    load4(p, o);
    load4(p + 4, o + 4);
}
__device__ __forceinline__ void load8(const bf16* p, float o[8]) {
    const uint4 v = *(const uint4*)p;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = __uint_as_float(w[i] << 16);
        o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void store8(float* p, const float v[8]) {
    ((float4*)p)[0] = make_float4(v[0], v[1], v[2], v[3]);
    ((float4*)p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}
__device__ __forceinline__ void store8(bf16* p, const float v[8]) {
    *(uint4*)p = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                            pack_bf16x2(v[6], v[7]));
}

// Raw (still packed) 8- and 4-element loads, so a prefetched block costs few registers.
template <typename T> struct Raw;
template <> struct Raw<bf16> {
    typedef uint4 v8;
    typedef uint2 v4;
    static __device__ __forceinline__ v8 ld8(const bf16* p) { return *(const uint4*)p; }
    // read-once rows (B, C): non-temporal, so that they do not displace the output rows in L2
    static __device__ __forceinline__ v8 ld8s(const bf16* p) {
        return __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4*)p));
    }
    static __device__ __forceinline__ v4 ld4(const bf16* p) { return *(const uint2*)p; }
    static __device__ __forceinline__ v4 ld4s(const bf16* p) {
        typedef unsigned u32x2v __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(uint2, __builtin_nontemporal_load((const u32x2v*)p));
    }
    static __device__ __forceinline__ void un8(v8 v, float o[8]) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = __uint_as_float(w[i] << 16);
            o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ void un4(v4 v, float o[4]) {
        o[0] = __uint_as_float(v.x << 16);
        o[1] = __uint_as_float(v.x & 0xffff0000u);
        o[2] = __uint_as_float(v.y << 16);
        o[3] = __uint_as_float(v.y & 0xffff0000u);
    }
};
template <> struct Raw<float> {
    struct v8 { float4 a, b; };
    typedef float4 v4;
    static __device__ __forceinline__ v8 ld8(const float* p) { return v8{((const float4*)p)[0], ((const float4*)p)[1]}; }
    static __device__ __forceinline__ v8 ld8s(const float* p) {
        return v8{__builtin_bit_cast(float4, __builtin_nontemporal_load((const floatx4*)p)),
                  __builtin_bit_cast(float4, __builtin_nontemporal_load((const floatx4*)p + 1))};
    }
    static __device__ __forceinline__ v4 ld4(const float* p) { return *(const float4*)p; }
    static __device__ __forceinline__ v4 ld4s(const float* p) { return __builtin_bit_cast(float4, __builtin_nontemporal_load((const floatx4*)p)); }
    static __device__ __forceinline__ void un8(v8 v, float o[8]) {
        o[0] = v.a.x; o[1] = v.a.y; o[2] = v.a.z; o[3] = v.a.w;
        o[4] = v.b.x; o[5] = v.b.y; o[6] = v.b.z; o[7] = v.b.w;
    }
    static __device__ __forceinline__ void un4(v4 v, float o[4]) { o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w; }
};

// Sum of dt * theta over each quarter of each segment: seg_phi[b, h, seg, quarter, :].  Wave w
// sums steps [t0 + w sub, t0 + (w + 1) sub) with sub = ceil(segment length / 4), the quarter the
// main pass's wave w walks.
template <typename T, int N>
__global__ __launch_bounds__(64 * kParts) void angle_partial_kernel(BcnormRopeArgs a) {
    constexpr int LPR = N / 8, RPW = 64 / LPR, K = N / 2;
    const int64_t id = blockIdx.x;
    const int seg = (int)(id % a.nseg);
    const int64_t bh = id / a.nseg;
    const int64_t b = bh / a.H;
    const int h = (int)(bh % a.H);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int c = lane % LPR, j = lane / LPR;
    const int64_t t0 = seg * a.seglen;
    const int64_t t1 = t0 + a.seglen < a.L ? t0 + a.seglen : a.L;
    const int64_t sub = (t1 - t0 + kParts - 1) / kParts;
    const int64_t w0 = t0 + wave * sub < t1 ? t0 + wave * sub : t1;
    const int64_t w1 = w0 + sub < t1 ? w0 + sub : t1;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int64_t t = w0 + j; t < w1; t += RPW) {
        const int64_t row = (b * a.L + t) * a.H + h;
        const float d = load_f32((const T*)a.dt + row);
        float th[4];
        load4((const T*)a.theta + row * K + 4 * c, th);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] += d * th[q];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
        for (int m = LPR; m < 64; m <<= 1) acc[q] += shfl_xor(acc[q], m);
    if (j == 0) {
        float* dst = a.seg_phi + ((bh * a.nseg + seg) * kParts + wave) * K + 4 * c;
#pragma unroll
        for (int q = 0; q < 4; ++q) dst[q] = acc[q];
    }
}

// Quarter sums -> quarter start angles (exclusive scan, phi_in added), in place; the inclusive
// total is the final angle phi_out.  A thread reads a block of kScanBlk quarter sums before it
// writes any back: a load that follows a store to the same array waits for it, so one value at a
// time would cost a memory round trip per quarter.
constexpr int kScanBlk = 8;
__global__ void angle_scan_kernel(BcnormRopeArgs a) {
    const int K = a.N / 2;
    const int64_t bh = blockIdx.x;
    const int64_t nq = (int64_t)a.nseg * kParts;
    for (int k = threadIdx.x; k < K; k += blockDim.x) {
        float run = a.phi_in ? wrap_angle(a.phi_in[bh * K + k]) : 0.0f;
        float* col = a.seg_phi + bh * nq * K + k;
        for (int64_t s0 = 0; s0 < nq; s0 += kScanBlk) {
            float v[kScanBlk];
#pragma unroll
            for (int i = 0; i < kScanBlk; ++i) v[i] = s0 + i < nq ? col[(s0 + i) * K] : 0.0f;
#pragma unroll
            for (int i = 0; i < kScanBlk; ++i) {
                if (s0 + i < nq) {
                    col[(s0 + i) * K] = run;
                    run = wrap_angle(run + v[i]);
                }
            }
        }
        a.phi_out[bh * K + k] = run;
    }
}

template <typename T, int N, int NW>
__global__ __launch_bounds__(NW * 64) void bcnorm_rope_kernel(BcnormRopeArgs a) {
    constexpr int LPR = N / 8, RPW = 64 / LPR, K = N / 2;
    __shared__ float wsum[NW][K];
    // heads that share raw B and C run on one XCD (consecutive items), so its L2 serves the group
    const int64_t id = a.G > 0 && a.G < a.H ? xcd_item(blockIdx.x, gridDim.x) : (int64_t)blockIdx.x;
    const int seg = (int)(id % a.nseg);
    const int64_t bh = id / a.nseg;
    const int64_t b = bh / a.H;
    const int h = (int)(bh % a.H);
    const int R = a.R;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int c = lane % LPR, j = lane / LPR;

    const int64_t t0 = seg * a.seglen;
    const int64_t t1 = t0 + a.seglen < a.L ? t0 + a.seglen : a.L;
    const int64_t sub = (t1 - t0 + NW - 1) / NW;
    const int64_t w0 = t0 + wave * sub < t1 ? t0 + wave * sub : t1;
    const int64_t w1 = w0 + sub < t1 ? w0 + sub : t1;

    // angle at the start of this wave's quarter, for this lane's 4 pairs: from the partial pass
    // (several segments), else phi_in shifted by the waves before it
    float start[4];
    if (a.seg_phi) {
        static_assert(NW == 1 || NW == kParts, "quarters");
        const float* src = a.seg_phi + ((bh * a.nseg + seg) * kParts + wave) * K + 4 * c;
#pragma unroll
        for (int q = 0; q < 4; ++q) start[q] = src[q];
    } else {
    float phi[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) phi[q] = a.phi_in ? wrap_angle(a.phi_in[bh * K + 4 * c + q]) : 0.0f;

    // each wave sums the angle increments of its quarter; waves before it shift its start
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int64_t t = w0 + j; t < w1; t += RPW) {
        const int64_t row = (b * a.L + t) * a.H + h;
        const float d = load_f32((const T*)a.dt + row);
        float th[4];
        load4((const T*)a.theta + row * K + 4 * c, th);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] += d * th[q];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
        for (int m = LPR; m < 64; m <<= 1) acc[q] += shfl_xor(acc[q], m);
    if (j == 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) wsum[wave][4 * c + q] = acc[q];
    }
    __syncthreads();
    float total[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        float s = 0.0f, tot = 0.0f;
        for (int w = 0; w < NW; ++w) {
            const float v = wsum[w][4 * c + q];
            if (w < wave) s += v;
            tot += v;
        }
        start[q] = wrap_angle(phi[q] + s);
        total[q] = wrap_angle(phi[q] + tot);
    }
    if (wave == 0 && j == 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) a.phi_out[bh * K + 4 * c + q] = total[q];
    }
    }

    // per-lane constants: BCNorm weights for this lane's 8 columns
    float wB[8], wC[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        wB[e] = a.normw_B ? a.normw_B[h * N + 8 * c + e] : 1.0f;
        wC[e] = a.normw_C ? a.normw_C[h * N + 8 * c + e] : 1.0f;
    }
    const float invN = 1.0f / (float)N;
    // when R divides the rows per wave instruction, row group j always holds rank j % R, so its
    // bias is fixed for the whole walk
    const bool bias_fixed = RPW % R == 0;
    float bB[8], bC[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        bB[e] = (bias_fixed && a.bias_B) ? a.bias_B[(h * R + j % R) * N + 8 * c + e] : 0.0f;
        bC[e] = (bias_fixed && a.bias_C) ? a.bias_C[(h * R + j % R) * N + 8 * c + e] : 0.0f;
    }

    // walk the quarter, RPW rows rho = (t - w0) * R + r at a time; row rho of this wave lives at
    // (rho / R) * H * R * N + (rho % R) * N past the (b, w0, h) row of the outputs, and at
    // (rho / R) * GS * R * N + (rho % R) * N past the (b, w0, slot) row of raw B and C (GS = G
    // head slots, H when every head has its own)
    const int64_t nrows = (w1 - w0) * R;
    const int64_t row_w0 = (b * a.L + w0) * a.H + h;
    const int GS = bc_slots(a.H, a.G);
    const int64_t row_in = (b * a.L + w0) * GS + bc_slot(h, a.H, a.G);
    const int64_t HRN = (int64_t)a.H * R * N, SBC = (int64_t)GS * R * N, HK = (int64_t)a.H * K;
    const T* Bq = (const T*)a.B + row_in * R * N + 8 * c;
    const T* Cq = (const T*)a.C + row_in * R * N + 8 * c;
    T* Bo = (T*)a.Bbar + row_w0 * R * N + 8 * c;
    T* Co = (T*)a.Cbar + row_w0 * R * N + 8 * c;
    const T* thq = (const T*)a.theta + row_w0 * K + 4 * c;
    const T* dtq = (const T*)a.dt + row_w0;

    // blocks of RPW rows, kDepth in flight (still packed) ahead of the one being computed; slot s
    // of the register ring holds blocks s, s + kDepth, ...
    using RW = Raw<T>;
    constexpr int kDepth = 3;
    typename RW::v8 nB[kDepth], nC[kDepth];
    typename RW::v4 nT[kDepth];
    T nD[kDepth];
    // A lane's row rho = rho0 + j is step tl = rho / R, rank r = rho % R of the quarter; both are
    // carried from block to block (RPW rows further: RPW / R steps and RPW % R ranks, with a carry)
    // instead of dividing.  Rows past the end reload the quarter's last row (result unused).
    struct Pos { int tl, r; };
    const int qadv = RPW / R, madv = RPW % R;
    auto advance = [&](Pos p) {
        p.tl += qadv;
        p.r += madv;
        if (p.r >= R) { p.r -= R; p.tl += 1; }
        return p;
    };
    const int nrows32 = (int)nrows;   // at most kSegLen * R
    const Pos plast = {nrows32 > 0 ? (nrows32 - 1) / R : 0, nrows32 > 0 ? (nrows32 - 1) % R : 0};
    auto load_block = [&](int rho0, Pos p, int slot) {
        const Pos u = rho0 + j < nrows32 ? p : plast;
        const int64_t o = (int64_t)u.tl * SBC + u.r * N;
        nB[slot] = RW::ld8s(Bq + o);
        nC[slot] = RW::ld8s(Cq + o);
        nT[slot] = RW::ld4s(thq + (int64_t)u.tl * HK);
        nD[slot] = dtq[(int64_t)u.tl * a.H];
    };
    float phi_acc[4] = {start[0], start[1], start[2], start[3]};
    Pos pcur = {j / R, j % R}, pld = pcur;
#pragma unroll
    for (int s = 0; s < kDepth; ++s) {
        if (s * RPW < nrows32) load_block(s * RPW, pld, s);
        pld = advance(pld);
    }
    for (int rho_base = 0; rho_base < nrows32; rho_base += kDepth * RPW)
#pragma unroll
    for (int slot = 0; slot < kDepth; ++slot) {
        const int rho0 = rho_base + slot * RPW;
        if (rho0 >= nrows32) break;
        float vb[8], vc[8], th[4];
        RW::un8(nB[slot], vb);
        RW::un8(nC[slot], vc);
        RW::un4(nT[slot], th);
        const float d = to_f32(nD[slot]);
        if (rho0 + kDepth * RPW < nrows32) load_block(rho0 + kDepth * RPW, pld, slot);
        pld = advance(pld);

        const Pos pc = pcur;
        pcur = advance(pcur);
        const bool valid = rho0 + j < nrows32;
        const int r = pc.r;
        // angle: each step's increment enters once, on the step's first row (r == 0); an
        // inclusive prefix over the row groups gives every row the angle of its own step
        float my_phi[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float inc = (valid && r == 0) ? d * th[q] : 0.0f;
            for (int o = LPR; o < 64; o <<= 1) {
                const float v = shfl_up(inc, o);
                if (lane >= o) inc += v;
            }
            my_phi[q] = phi_acc[q] + inc;   // within a few radians of the reduced carry
            phi_acc[q] = wrap_angle(phi_acc[q] + shfl(inc, (RPW - 1) * LPR + c));
        }

        if (a.bcnorm) {
            float sb = 0.f, sc = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                sb += vb[e] * vb[e];
                sc += vc[e] * vc[e];
            }
            sb = group_sum(sb, LPR);   // DPP inside the row's lanes
            sc = group_sum(sc, LPR);
            const float ib = rsqrtf(sb * invN + a.eps), ic = rsqrtf(sc * invN + a.eps);
            if (bias_fixed) {   // norm, weight and bias in one multiply-add
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    vb[e] = fmaf(vb[e], ib * wB[e], bB[e]);
                    vc[e] = fmaf(vc[e], ic * wC[e], bC[e]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    vb[e] *= ib * wB[e];
                    vc[e] *= ic * wC[e];
                }
            }
        }
        if (bias_fixed) {
            if (!a.bcnorm) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    vb[e] += bB[e];
                    vc[e] += bC[e];
                }
            }
        } else {
            if (a.bias_B) {
                float bb[8];
                load8(a.bias_B + (h * R + r) * N + 8 * c, bb);
#pragma unroll
                for (int e = 0; e < 8; ++e) vb[e] += bb[e];
            }
            if (a.bias_C) {
                float bc[8];
                load8(a.bias_C + (h * R + r) * N + 8 * c, bc);
#pragma unroll
                for (int e = 0; e < 8; ++e) vc[e] += bc[e];
            }
        }
        float ob[8], oc[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float s, co;
            __sincosf(my_phi[q], &s, &co);
            ob[2 * q] = co * vb[2 * q] + s * vb[2 * q + 1];
            ob[2 * q + 1] = -s * vb[2 * q] + co * vb[2 * q + 1];
            oc[2 * q] = co * vc[2 * q] + s * vc[2 * q + 1];
            oc[2 * q + 1] = -s * vc[2 * q] + co * vc[2 * q + 1];
        }
        if (valid) {
            const int64_t off = (int64_t)pc.tl * HRN + pc.r * N;
            store8(Bo + off, ob);
            store8(Co + off, oc);
        }
    }
}

template <typename T, int N>
hipError_t launch_n(const BcnormRopeArgs& a, hipStream_t s) {
    const unsigned nbh = (unsigned)(a.b * a.H);
    if (a.nseg > 1) {
        hipLaunchKernelGGL((angle_partial_kernel<T, N>), dim3(nbh * a.nseg), dim3(64 * kParts), 0, s, a);
        hipLaunchKernelGGL(angle_scan_kernel, dim3(nbh), dim3(N / 2 < 64 ? 64 : N / 2), 0, s, a);
    }
    // a single-wave workgroup when the segment has too few rows to share among four waves
    const int64_t steps = a.L < a.seglen ? a.L : a.seglen;
    if (steps * a.R >= 4 * (512 / N))
        hipLaunchKernelGGL((bcnorm_rope_kernel<T, N, 4>), dim3(nbh * a.nseg), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((bcnorm_rope_kernel<T, N, 1>), dim3(nbh * a.nseg), dim3(64), 0, s, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const BcnormRopeArgs& a, hipStream_t s) {
    switch (a.N) {
        case 16: return launch_n<T, 16>(a, s);
        case 32: return launch_n<T, 32>(a, s);
        case 64: return launch_n<T, 64>(a, s);
        case 128: return launch_n<T, 128>(a, s);
        case 256: return launch_n<T, 256>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool bcnorm_rope_supported(int N, int R) {
    return (N == 16 || N == 32 || N == 64 || N == 128 || N == 256) && R >= 1 && R <= 64;
}

int64_t bcnorm_rope_seglen() { return kSegLen; }
int bcnorm_rope_parts() { return kParts; }

hipError_t launch_bcnorm_rope(const BcnormRopeArgs& a, bool bf16_io, hipStream_t s) {
    return bf16_io ? launch_t<bf16>(a, s) : launch_t<float>(a, s);
}

}  // namespace m3
