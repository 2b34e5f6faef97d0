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

// Round-to-nearest-even float -> bf16 (NaN stays NaN).
__device__ __forceinline__ uint16_t bf16_bits_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

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
