// m3_mma.h -- MFMA fragment access and small vector helpers shared by the chunked kernels
// (prefill and backward).  16x16x16 tiles: lane (l16 = lane % 16, g = lane / 16) holds
//   A operand  A[row = l16][k = 4g .. 4g + 3]
//   B operand  B[k = 4g .. 4g + 3][col = l16]
//   result     D[row = 4g + m][col = l16], m = 0..3
// so a result tile of X is directly the B operand of X and the A operand of X^T.
#pragma once

#include "m3_device.h"

namespace m3 {

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
// sum of the squares of one 16-byte vector of io elements (bf16 pairs: v_dot2_f32_bf16, whose
// products of two bf16 values are exact in fp32), as a tree rather than one chain
__device__ __forceinline__ float sumsq16(uint4 v, float) {
    const float a = __uint_as_float(v.x), b = __uint_as_float(v.y), c = __uint_as_float(v.z), d = __uint_as_float(v.w);
    return fmaf(a, a, b * b) + fmaf(c, c, d * d);
}
__device__ __forceinline__ float sumsq16(uint4 v, bf16) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t p = __builtin_bit_cast(bf16x2_t, v.x), q = __builtin_bit_cast(bf16x2_t, v.y);
    const bf16x2_t r = __builtin_bit_cast(bf16x2_t, v.z), s = __builtin_bit_cast(bf16x2_t, v.w);
    return __builtin_amdgcn_fdot2_f32_bf16(q, q, __builtin_amdgcn_fdot2_f32_bf16(p, p, 0.f, false), false) +
           __builtin_amdgcn_fdot2_f32_bf16(s, s, __builtin_amdgcn_fdot2_f32_bf16(r, r, 0.f, false), false);
}
__device__ __forceinline__ uint4 pack16(const float (&v)[4], float) {
    return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3]));
}
__device__ __forceinline__ uint4 pack16(const float (&v)[8], bf16) {
    return make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
}

}  // namespace m3
