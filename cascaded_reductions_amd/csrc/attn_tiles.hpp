// LDS layout of the bf16 attention K and V tiles, shared by the incremental and the
// whole-row prefill kernels.
#pragma once

#include "common.hpp"

namespace rf {

// LDS chunk swizzles of the bf16 attention K and V tiles (rows of D bf16 values in
// 16-byte chunks). The LDS serves 256 bytes per cycle: a 16-lane group of 16-byte K
// reads (rows l32 = 16i .. 16i + 15 at one logical chunk) and a 32-lane group of 8-byte
// transposed V reads (4 lanes on each of 8 key rows, two adjacent chunks per row; the
// hardware may pair lane groups 0 + 1 or 0 + 2). At D = 64 a row is 128 bytes, so rows
// of one parity share bank halves; at D = 128 a row is a whole bank row. The XOR masks
// below give every row of such a group its own banks (an XOR with row & 7 repeats every
// 8 rows and put rows 8 apart on the same banks).
template <int D>
__device__ __forceinline__ int attn_k_swz(int row) {
    if constexpr (D == 64) return (row >> 1) & 7;
    else return row & 15;
}
template <int D>
__device__ __forceinline__ int attn_v_swz(int key) {
    if constexpr (D == 64) return (((key >> 2) & 1) << 1) | (((key >> 1) & 1) << 2);
    else return (((key >> 2) & 1) << 1) | ((key & 1) << 2) | (((key >> 1) & 1) << 3);
}

}  // namespace rf
