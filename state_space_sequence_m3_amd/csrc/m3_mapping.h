// m3_mapping.h -- index maps shared by the kernels and the host (no HIP types, so host code and
// host-side tests can include it).
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define M3_HD __host__ __device__ __forceinline__
#else
#define M3_HD inline
#endif

namespace m3 {

// Raw B and C with G head slots shared by groups of H / G consecutive heads: the slot of head h,
// and the slots per step (G = 0: one slot per head).
M3_HD int bc_slot(int h, int H, int G) { return G > 0 ? h / (H / G) : h; }
M3_HD int bc_slots(int H, int G) { return G > 0 ? G : H; }

// XCD-aware order of a grid's work items.  The dispatcher hands workgroup i to XCD i mod 8, each
// XCD with its own L2; this maps workgroup i to item (i mod 8) * n/8 + i / 8, so that every XCD
// takes one contiguous range of items in order (n a multiple of 8, else the identity).
// Neighbouring items, such as the heads of a group that read the same raw B and C, then meet in
// one L2.  The map is a permutation of [0, n): every item runs exactly once, but in no fixed
// order relative to the others (so no workgroup may wait on, or race with, another one).
constexpr int kXcds = 8;
M3_HD int64_t xcd_item(int64_t i, int64_t n) {
    return n % kXcds == 0 ? (i % kXcds) * (n / kXcds) + i / kXcds : i;
}

}  // namespace m3
