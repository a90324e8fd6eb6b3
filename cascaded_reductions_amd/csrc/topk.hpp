// Sorted top-k lists, for the MoE gate (the top-k step of the explainer
// "RedFuser框架：AI加速器中的算子融合技术解析", section 4.2) and the top-k row cascade.
//
// Entries are ranked by (score descending, index ascending). Each (score, index) entry is
// packed into one 64-bit key that orders the same way as unsigned integers: the score's
// bits made monotonic in the high word (after turning -0 into +0, which compares equal to
// it) and the complemented index in the low word. The ranking is a strict total order on
// distinct indices, so the K best of a set do not depend on how the set is split over lanes
// or in which order the pieces are merged; and a comparison is one 64-bit compare and a
// select, with no divergent branches. Lists of neighbouring lanes are merged through DPP
// moves instead of LDS permutes. NaN scores never enter a list.
#pragma once

#include "common.hpp"

namespace rf {
namespace topk {

// The key of an empty slot: (-inf, 2^31 - 1), which ranks after every entry with a smaller
// index.
constexpr uint64_t kEmpty = (uint64_t(0x007FFFFFu) << 32) | 0x80000000u;

// The high word of a key: the score's bits made monotonic as an unsigned integer (negative
// values complemented, the sign set on the others), -0 first turned into +0. A NaN becomes 0,
// below every key of a real score and below kEmpty, so it never enters a list.
__device__ __forceinline__ uint32_t score_word(float s) {
    const uint32_t u = __float_as_uint(s + 0.f);              // -0 -> +0 (round to nearest)
    const uint32_t o = u ^ (uint32_t(int32_t(u) >> 31) | 0x80000000u);
    return o > 0xFF800000u ? 0u : o;                          // above +inf: a positive NaN
}

// Key of (score s, index i), 0 <= i < 2^31 - 1.
__device__ __forceinline__ uint64_t make_key(float s, int i) {
    return (uint64_t(score_word(s)) << 32) | uint32_t(~uint32_t(i));
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
    for (int r = 0; r < K; ++r) l[r] = kEmpty;
}

// Insert a key into the sorted list: each slot keeps the better key and passes the other
// one down; the last one falls off.
template <int K>
__device__ __forceinline__ void insert(uint64_t (&l)[K], uint64_t key) {
#pragma unroll
    for (int r = 0; r < K; ++r) order(l[r], key);
}

// Fold four keys in at once: sort them (a five-exchange network), then keep the K best of
// the list and the sorted four. The four, padded with empty slots to K and read backwards,
// meet only the last four slots; the result is bitonic and log2(K) half-cleaner stages sort
// it. The same K keys as four single inserts, with 17 exchanges instead of 4 K.
template <int K>
__device__ __forceinline__ void insert4(uint64_t (&l)[K], uint64_t a, uint64_t b, uint64_t c, uint64_t d) {
    static_assert(K >= 4 && (K & (K - 1)) == 0, "four at a time needs a power-of-two list of at least 4");
    order(a, b);
    order(c, d);
    order(a, c);
    order(b, d);
    order(b, c);
    const uint64_t n[4] = {a, b, c, d};
#pragma unroll
    for (int r = K - 4; r < K; ++r) l[r] = n[K - 1 - r] > l[r] ? n[K - 1 - r] : l[r];
#pragma unroll
    for (int s = K / 2; s >= 1; s >>= 1)
#pragma unroll
        for (int r = 0; r < K; ++r)
            if ((r & s) == 0) order(l[r], l[r + s]);
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_key(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_update_dpp(0, int(uint32_t(v)), CTRL, 0xF, 0xF, false);
    const uint32_t hi = __builtin_amdgcn_update_dpp(0, int(uint32_t(v >> 32)), CTRL, 0xF, 0xF, false);
    return (uint64_t(hi) << 32) | lo;
}

// Merge the sorted list o (a disjoint set of entries) into the sorted list l. Taking, slot
// by slot, the better of l and o read backwards keeps the K best of the union as a bitonic
// sequence; log2(K) half-cleaner stages sort it.
template <int K>
__device__ __forceinline__ void merge(uint64_t (&l)[K], const uint64_t (&o)[K]) {
    static_assert((K & (K - 1)) == 0, "the bitonic merge needs a power-of-two list length");
#pragma unroll
    for (int r = 0; r < K; ++r) l[r] = o[K - 1 - r] > l[r] ? o[K - 1 - r] : l[r];
#pragma unroll
    for (int s = K / 2; s >= 1; s >>= 1)
#pragma unroll
        for (int r = 0; r < K; ++r)
            if ((r & s) == 0) order(l[r], l[r + s]);
}

// Merge this lane's list with the one of the lane that the DPP control CTRL maps to.
template <int CTRL, int K>
__device__ __forceinline__ void merge_dpp(uint64_t (&l)[K]) {
    uint64_t o[K];
#pragma unroll
    for (int r = 0; r < K; ++r) o[r] = dpp_key<CTRL>(l[r]);
    merge<K>(l, o);
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

}  // namespace topk
}  // namespace rf
