// A generic cascaded reduction in incremental form, for one row at a time.
//
// The technical summary "RedFuser: An Automatic Operator Fusion Framework for
// Cascaded Reductions on AI Accelerators" (Methodologie 1-2) and the explainer
// "RedFuser框架：AI加速器中的算子融合技术解析" (sections 2.2-2.3) describe a chain
// of reductions d_i = (+)_j G_i(x_j, d_1 .. d_{i-1}) that can be fused into one
// loop when each G_i factors as H_i(d) (x) G'_i(x): the loop then keeps running
// values of every d_i, and when an earlier d moves, the later running values
// are corrected by H_i(d_new) H_i^-1(d_old) instead of being recomputed.
// Running values of disjoint parts of a row combine with the same rule, so the
// state of a cascade is a commutative monoid.
//
// A cascade is described here by a spec type with
//   struct State                          the running values (trivially copyable),
//   static State identity()               the monoid's identity,
//   static void absorb(State&, float x, int32_t j, const float* payload)
//                                         fold element j in (the incremental update),
//   static State combine(const State&, const State&)
//                                         merge two partial states (order independent
//                                         in exact arithmetic),
//   static constexpr int kPayload         payload values per element (0: none),
// and the row kernel (row_cascade.hip) folds a row with it: every lane absorbs a
// strided part of the row, then the 64 lane states are merged with xor shuffles
// in a fixed order, so results are deterministic.
#pragma once

#include "common.hpp"

namespace rf {
namespace cascade {

// Moves a State between lanes word by word.
template <class S>
__device__ __forceinline__ S shfl_xor_state(const S& s, int mask) {
    static_assert(sizeof(S) % 4 == 0, "states are made of 32-bit words");
    constexpr int W = int(sizeof(S) / 4);
    uint32_t w[W];
    __builtin_memcpy(w, &s, sizeof(S));
#pragma unroll
    for (int i = 0; i < W; ++i) w[i] = uint32_t(__shfl_xor(int(w[i]), mask, 64));
    S out;
    __builtin_memcpy(&out, w, sizeof(S));
    return out;
}

// ---------------------------------------------------------------- logsumexp
// d1 = max x, d2 = sum exp(x - d1): the two-reduction head of safe softmax.
struct LogSumExp {
    struct State {
        float m, s;
    };
    static constexpr int kPayload = 0;
    __device__ static State identity() { return {kNegInf, 0.f}; }
    __device__ static void absorb(State& st, float x, int32_t, const float*) {
        if (x > st.m) {                                   // the running max moves: rescale s
            st.s = st.s * __expf(st.m - x) + 1.f;        // (exp(-inf) = 0 for the first element)
            st.m = x;
        } else if (x != kNegInf) {                        // exp(-inf) adds nothing (and -inf - -inf is NaN)
            st.s += __expf(x - st.m);
        }
    }
    __device__ static State combine(const State& a, const State& b) {
        const float m = fmaxf(a.m, b.m);
        if (m == kNegInf) return identity();
        return {m, a.s * __expf(a.m - m) + b.s * __expf(b.m - m)};
    }
};

// ---------------------------------------------------------------- softmax-weighted sum
// d1 = max x, d2 = sum exp(x - d1), d3 = sum exp(x - d1) v / d2: the attention chain with
// the scores given (P payload values per element).
template <int P>
struct SoftmaxWeighted {
    struct State {
        float m, s, o[P];
    };
    static constexpr int kPayload = P;
    __device__ static State identity() {
        State st;
        st.m = kNegInf;
        st.s = 0.f;
#pragma unroll
        for (int i = 0; i < P; ++i) st.o[i] = 0.f;
        return st;
    }
    __device__ static void absorb(State& st, float x, int32_t, const float* v) {
        if (x == kNegInf) return;                         // a masked element adds nothing
        const float m = fmaxf(st.m, x);
        const float alpha = st.m == kNegInf ? 0.f : __expf(st.m - m);
        const float p = __expf(x - m);
        st.s = st.s * alpha + p;
#pragma unroll
        for (int i = 0; i < P; ++i) st.o[i] = st.o[i] * alpha + p * v[i];
        st.m = m;
    }
    __device__ static State combine(const State& a, const State& b) {
        const float m = fmaxf(a.m, b.m);
        if (m == kNegInf) return identity();
        const float wa = a.m == kNegInf ? 0.f : __expf(a.m - m);
        const float wb = b.m == kNegInf ? 0.f : __expf(b.m - m);
        State st;
        st.m = m;
        st.s = a.s * wa + b.s * wb;
#pragma unroll
        for (int i = 0; i < P; ++i) st.o[i] = a.o[i] * wa + b.o[i] * wb;
        return st;
    }
};

// ---------------------------------------------------------------- top-k, then softmax over the k
// d1 = the K best (score, index) pairs under (score descending, index ascending); the softmax
// over them is applied once at the end. The monoid is "merge two sorted lists, keep K".
template <int K>
struct TopK {
    struct State {
        float s[K];
        int32_t i[K];
    };
    static constexpr int kPayload = 0;
    __device__ static bool better(float s1, int32_t i1, float s2, int32_t i2) {
        return s1 > s2 || (s1 == s2 && i1 < i2);
    }
    __device__ static State identity() {
        State st;
#pragma unroll
        for (int r = 0; r < K; ++r) {
            st.s[r] = kNegInf;
            st.i[r] = 0x7FFFFFFF;
        }
        return st;
    }
    __device__ static void insert(State& st, float s, int32_t i) {
#pragma unroll
        for (int r = 0; r < K; ++r) {
            if (better(s, i, st.s[r], st.i[r])) {
                const float s2 = st.s[r];
                const int32_t i2 = st.i[r];
                st.s[r] = s;
                st.i[r] = i;
                s = s2;
                i = i2;
            }
        }
    }
    __device__ static void absorb(State& st, float x, int32_t j, const float*) { insert(st, x, j); }
    __device__ static State combine(const State& a, const State& b) {
        State st = a;
#pragma unroll
        for (int r = 0; r < K; ++r) insert(st, b.s[r], b.i[r]);
        return st;
    }
};

// ---------------------------------------------------------------- mean and variance
// d1 = mean, d2 = sum (x - d1)^2: when the mean moves by delta, the running sum of squares
// is corrected instead of recomputed (Welford's update; partial states merge with the
// pairwise rule of Chan, Golub and LeVeque).
struct MeanVar {
    struct State {
        uint32_t n;          // an integer count: a float one stops growing at 2^24
        float mean, m2;
    };
    static constexpr int kPayload = 0;
    __device__ static State identity() { return {0u, 0.f, 0.f}; }
    __device__ static void absorb(State& st, float x, int32_t, const float*) {
        st.n += 1u;
        const float d = x - st.mean;
        st.mean += d / float(st.n);
        st.m2 += d * (x - st.mean);
    }
    __device__ static State combine(const State& a, const State& b) {
        const uint32_t n = a.n + b.n;
        if (n == 0u) return identity();
        const float d = b.mean - a.mean;
        const float fb = float(b.n) / float(n);
        return {n, a.mean + d * fb, a.m2 + b.m2 + d * d * float(a.n) * fb};
    }
};

}  // namespace cascade
}  // namespace rf
