// m3_device.h -- device-side helpers shared by the libm3scan kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "m3_mapping.h"

namespace m3 {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));

// bf16 is carried as its raw 16-bit pattern.
struct bf16 {
    uint16_t bits;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return __uint_as_float((uint32_t)v.bits << 16); }

// float -> bf16 bits, round to nearest even (gfx950 converts in hardware: v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t bf16_bits_rne(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
// two floats -> packed bf16 pair (lo in bits 0..15), one v_cvt_pk_bf16_f32
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef float floatx2_v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2_v){lo, hi}, bf16x2_v));
}
// 2^x with the hardware instruction (no denormal fix-up; tiny results flush to zero)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return bf16{bf16_bits_rne(v)}; }

__device__ __forceinline__ float load_f32(const float* p) { return *p; }
__device__ __forceinline__ float load_f32(const bf16* p) { return to_f32(*p); }

// Wave-wide helpers (wave64).
__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }
__device__ __forceinline__ float shfl_up(float v, int d) { return __shfl_up(v, d, 64); }
__device__ __forceinline__ float shfl(float v, int src) { return __shfl(v, src, 64); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kTwoPi = 6.283185307179586f;
constexpr float kInvTwoPi = 0.15915494309189535f;

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (no LDS crossbar): a
// Hillis-Steele scan inside each row of 16 lanes (row_shr 1, 2, 4, 8; lanes with no source get 0),
// then row 15's total is broadcast into rows 1 and 3 and row 31's into rows 2 and 3.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_move(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, true));
}
__device__ __forceinline__ float wave_scan_add(float v) {
    v += dpp_move<0x111, 0xf>(v);   // row_shr:1
    v += dpp_move<0x112, 0xf>(v);   // row_shr:2
    v += dpp_move<0x114, 0xf>(v);   // row_shr:4
    v += dpp_move<0x118, 0xf>(v);   // row_shr:8
    v += dpp_move<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
    v += dpp_move<0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3
    return v;
}
// Sum over aligned groups of R lanes (R = 1, 2, ..., 64): inside each row of 16 lanes with DPP
// moves (quad_perm swaps inside quads, then half-row and row mirrors, each of which pairs two
// groups that already hold uniform partial sums); across rows with gfx950's swaps, which applied
// to (v, v) return both rows of a pair (v_permlane16_swap: rows (0, 0, 2, 2) and (1, 1, 3, 3);
// v_permlane32_swap: rows (0, 1, 0, 1) and (2, 3, 2, 3)), so their sum is the pair's in every
// lane, in VALU (no LDS crossbar), and the same value an exchange of the partners would give.
__device__ __forceinline__ float group_sum(float v, int R) {
    if (R >= 2) v += dpp_move<0xB1, 0xf>(v);    // quad_perm [1, 0, 3, 2]
    if (R >= 4) v += dpp_move<0x4E, 0xf>(v);    // quad_perm [2, 3, 0, 1]
    if (R >= 8) v += dpp_move<0x141, 0xf>(v);   // row_half_mirror
    if (R >= 16) v += dpp_move<0x140, 0xf>(v);  // row_mirror
    if (R >= 32) {
        const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    }
    if (R >= 64) {
        const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    }
    return v;
}
// Inclusive prefix sum inside aligned groups of W lanes (W a power of two, at most 64).  Inside a
// row of 16 lanes it is the Hillis-Steele steps of wave_scan_add, with the steps that would reach
// across a group of fewer than 16 lanes masked off.
template <int W>
__device__ __forceinline__ float seg_scan_add(float v, int lane) {
    static_assert(W >= 1 && W <= 64 && (W & (W - 1)) == 0, "group width");
    const int j = lane & (W - 1);
    if (W >= 2) { const float u = dpp_move<0x111, 0xf>(v); v += (W >= 16 || j >= 1) ? u : 0.f; }
    if (W >= 4) { const float u = dpp_move<0x112, 0xf>(v); v += (W >= 16 || j >= 2) ? u : 0.f; }
    if (W >= 8) { const float u = dpp_move<0x114, 0xf>(v); v += (W >= 16 || j >= 4) ? u : 0.f; }
    if (W >= 16) v += dpp_move<0x118, 0xf>(v);
    if (W >= 32) v += dpp_move<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
    if (W >= 64) v += dpp_move<0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3
    return v;
}
// Exclusive sum over runs of W lanes (run r = lanes [r W, (r + 1) W), column j = lane % W): the
// sum of v over runs r' < r in lane (r, j).  W = 64, 32, 16 or 8.  Inside a 16-lane row by DPP
// shifts; across rows by gfx950's swaps, all in VALU (no LDS crossbar): v_permlane16_swap applied
// to (v, v) gives rows (0, 0, 2, 2) and (1, 1, 3, 3) of v, v_permlane32_swap rows (0, 1, 0, 1) and
// (2, 3, 2, 3).
__device__ __forceinline__ float rows_exclusive_sum(float v, int lane) {   // runs = rows (W = 16)
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const float below = __uint_as_float(p[0]);                       // row r - 1 in odd rows
    const float pair = below + __uint_as_float(p[1]);                // rows 2q + 2q+1, in both
    const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(pair), __float_as_uint(pair), false, false);
    return ((lane & 16) ? below : 0.f) + (lane >= 32 ? __uint_as_float(h[0]) : 0.f);
}
template <int W>
__device__ __forceinline__ float run_exclusive_sum(float v, int lane) {
    static_assert(W == 8 || W == 16 || W == 32 || W == 64, "run width");
    if constexpr (W == 64) {
        return 0.f;
    } else if constexpr (W == 32) {
        const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        return lane >= 32 ? __uint_as_float(h[0]) : 0.f;
    } else if constexpr (W == 16) {
        return rows_exclusive_sum(v, lane);
    } else {
        // two runs per row: the upper run takes the lower one's value (row_shr:8), and the row's
        // total for each column is v plus its partner (row_shr:8 + row_shl:8, zero outside the row)
        const float lo = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, true));
        const float hi = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x108, 0xf, 0xf, true));
        return lo + rows_exclusive_sum(v + lo + hi, lane);
    }
}
__device__ __forceinline__ float lane_value(float v, int src_lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src_lane));
}

// Raw buffer access (stride 0): loads at or past `bytes` return zero and stores there are
// dropped, so the tail of a sequence needs no branches.  The fourth descriptor word is the gfx9
// default data format.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buffer_load16(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
// The same for data read exactly once (a streamed input): non-temporal, so that it does not
// displace lines that stay in use in L2 (among them the output rows being written back).
__device__ __forceinline__ uint4 buffer_load16_stream(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2));
}
__device__ __forceinline__ void buffer_store8(rsrc_t r, uint32_t off, uint2 v) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, (int)off, 0, 0);
}
__device__ __forceinline__ void buffer_store16(rsrc_t r, uint32_t off, uint4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, 0);
}
// non-temporal store (data not read again soon through this cache level)
__device__ __forceinline__ void buffer_store16_stream(rsrc_t r, uint32_t off, uint4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, 2);
}
// one io element as raw bits (loaded now, converted where it is used, so the load need not be
// waited for at once); past the descriptor's end it reads as zero
template <typename T> struct IoBits;
template <> struct IoBits<float> { typedef uint32_t type; };
template <> struct IoBits<bf16> { typedef uint16_t type; };
__device__ __forceinline__ uint32_t buffer_load_bits(rsrc_t r, uint32_t off, float) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint16_t buffer_load_bits(rsrc_t r, uint32_t off, bf16) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
__device__ __forceinline__ float bits_to_f32(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ float bits_to_f32(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }
// bytes of `n` elements, clamped to what a descriptor can hold
__device__ __forceinline__ uint32_t clamp_bytes(int64_t n) {
    return n <= 0 ? 0u : (n >= 0xffffffffLL ? 0xffffffffu : (uint32_t)n);
}

// Reduce an angle to [-pi, pi] (any representative gives the same rotation).
__device__ __forceinline__ float wrap_angle(float a) { return a - kTwoPi * rintf(a * kInvTwoPi); }
// The same for an angle in turns (revolutions): reduced to [-1/2, 1/2].
__device__ __forceinline__ float wrap_turns(float a) { return a - rintf(a); }

}  // namespace m3
