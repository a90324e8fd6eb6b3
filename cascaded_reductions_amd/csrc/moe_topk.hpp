// Sorted top-k lists for the MoE gate (the top-k step of the explainer
// "RedFuser框架：AI加速器中的算子融合技术解析", section 4.2).
//
// Experts are ranked by (score descending, index ascending). Each (score, index) entry is
// packed into one 64-bit key that orders the same way as unsigned integers: the score's
// bits made monotonic in the high word (after turning -0 into +0, which compares equal to
// it) and the complemented index in the low word. The ranking is a strict total order on
// distinct indices, so the K best of a set do not depend on how the set is split over lanes
// or in which order the pieces are merged; and a comparison is one 64-bit compare and a
// select, with no divergent branches. The lists of the sixteen lanes of a DPP row are
// merged through DPP moves instead of LDS permutes.
#pragma once

#include "common.hpp"

namespace rf {
namespace moe {

// Key of (score s, expert i), i >= 0; keys of finite scores are nonzero, and 0 is the key of
// an empty entry, which ranks after every real one.
__device__ __forceinline__ uint64_t make_key(float s, int i) {
    const uint32_t u = __float_as_uint(s + 0.f);              // -0 -> +0 (round to nearest)
    const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return (uint64_t(o) << 32) | uint32_t(~uint32_t(i));
}
__device__ __forceinline__ float key_score(uint64_t key) {
    const uint32_t o = uint32_t(key >> 32);
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
__device__ __forceinline__ int key_index(uint64_t key) { return int(~uint32_t(key)); }

// Compare-exchange: afterwards a holds the better (larger) key.
__device__ __forceinline__ void order(uint64_t& a, uint64_t& b) {
    const bool sw = b > a;
    const uint64_t hi = sw ? b : a, lo = sw ? a : b;
    a = hi;
    b = lo;
}

template <int K>
__device__ __forceinline__ void clear(uint64_t (&l)[K]) {
#pragma unroll
    for (int r = 0; r < K; ++r) l[r] = 0;
}

// Insert a key into the sorted list: each slot keeps the better key and passes the other
// one down; the last one falls off.
template <int K>
__device__ __forceinline__ void insert(uint64_t (&l)[K], uint64_t key) {
#pragma unroll
    for (int r = 0; r < K; ++r) order(l[r], key);
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_key(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_update_dpp(0, int(uint32_t(v)), CTRL, 0xF, 0xF, false);
    const uint32_t hi = __builtin_amdgcn_update_dpp(0, int(uint32_t(v >> 32)), CTRL, 0xF, 0xF, false);
    return (uint64_t(hi) << 32) | lo;
}

// Merge this lane's sorted list with the one of the lane that the DPP control CTRL maps to
// (a disjoint set of experts). Taking, slot by slot, the better of this list and the
// partner's list read backwards keeps the K best of the union as a bitonic sequence;
// log2(K) half-cleaner stages sort it.
template <int CTRL, int K>
__device__ __forceinline__ void merge_dpp(uint64_t (&l)[K]) {
    static_assert((K & (K - 1)) == 0, "the bitonic merge needs a power-of-two list length");
    uint64_t o[K];
#pragma unroll
    for (int r = 0; r < K; ++r) o[r] = dpp_key<CTRL>(l[r]);
#pragma unroll
    for (int r = 0; r < K; ++r) l[r] = o[K - 1 - r] > l[r] ? o[K - 1 - r] : l[r];
#pragma unroll
    for (int s = K / 2; s >= 1; s >>= 1)
#pragma unroll
        for (int r = 0; r < K; ++r)
            if ((r & s) == 0) order(l[r], l[r + s]);
}

// Merge the lists of the sixteen lanes of each DPP row; afterwards every lane of the row
// holds the row's K best. The pairings are lane xor 1 and xor 2 (quad permutes), then
// lane i with 7 - i (half-row mirror) and lane i with 15 - i (row mirror): each stage
// joins two groups that hold disjoint experts.
template <int K>
__device__ __forceinline__ void merge_row16(uint64_t (&l)[K]) {
    merge_dpp<0xB1, K>(l);
    merge_dpp<0x4E, K>(l);
    merge_dpp<0x141, K>(l);
    merge_dpp<0x140, K>(l);
}

// Softmax over the first k (k <= K) entries of a merged list; writes the token's k indices
// and weights.
template <int K>
__device__ __forceinline__ void write_softmax(const uint64_t (&l)[K], int k, int32_t* idx, float* wout) {
    const float top = key_score(l[0]);
    float den = 0.f;
    float ex[K];
#pragma unroll
    for (int r = 0; r < K; ++r) {
        ex[r] = r < k ? __expf(key_score(l[r]) - top) : 0.f;
        den += ex[r];
    }
    const float inv = 1.f / den;
#pragma unroll
    for (int r = 0; r < K; ++r) {
        if (r < k) {
            idx[r] = key_index(l[r]);
            wout[r] = ex[r] * inv;
        }
    }
}

}  // namespace moe
}  // namespace rf
