// m3_device.h -- device-side helpers shared by the libm3scan kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
// two floats -> packed bf16 pair (lo in bits 0..15)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)bf16_bits_rne(lo) | ((uint32_t)bf16_bits_rne(hi) << 16);
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

// Reduce an angle to [-pi, pi] (any representative gives the same rotation).
__device__ __forceinline__ float wrap_angle(float a) { return a - kTwoPi * rintf(a * kInvTwoPi); }

}  // namespace m3
