// A generic cascaded reduction in incremental form.
//
// The technical summary "RedFuser: An Automatic Operator Fusion Framework for
// Cascaded Reductions on AI Accelerators" (Methodologie 1-2) and the explainer
// "RedFuser框架：AI加速器中的算子融合技术解析" (sections 2.2-2.3) describe a chain
// of reductions d_i = (+)_i over j of F_i(x_j, d_1 .. d_{i-1}) that can be fused
// into one loop when three conditions hold:
//   decomposability   F_i(x, d) = G_i(x) (x)_i H_i(d),
//   distributivity    (+)_i distributes over (x)_i, so
//                     d_i = H_i(d) (x)_i ((+)_j G_i(x_j)),
//   invertibility     H_i has an inverse under (x)_i (or a correction mechanism).
// The loop then keeps a running value of every later reduction relative to the
// current value of the earlier ones, and when an earlier d moves from d_old to
// d_new it corrects the running value by H_i(d_new) (x) H_i^-1(d_old) instead of
// recomputing it. Running values of disjoint parts of a row combine with the same
// correction, so the state of a cascade is a commutative monoid.
//
// Cascade<Spec> below derives the incremental update (absorb) and the merge of two
// partial states (combine) from a Spec that names the pieces of that statement:
//
//   Lead                         the leading reduction d_1 (the one the others depend on)
//   lead_identity()              its identity
//   lead_plus(lead, x, j)        lead (+)_1 G_1(x_j)
//   lead_merge(a, b)             a (+)_1 b
//   lead_is_identity(lead)       no element absorbed yet (nothing to correct)
//   H                            values of the H_i in a form closed under (x)
//   h_of(lead)                   H(d_1)
//   h_inv(h), h_mul(a, b)        the inverse and the product (x)
//   g_of(x)                      G(x) in the same form (the term of element x is
//                                g_of(x) (x) h_of(lead))
//   is_null(x)                   the element's terms are the identity of (+) (a masked
//                                score: exp(-inf) = 0), so only the lead sees it
//   Acc                          the running values of d_2 .. d_n
//   acc_identity()
//   acc_plus(acc, term, x, payload)   acc (+)= the realised term (payload: extra factors
//                                     of G, e.g. the values of a softmax-weighted sum)
//   acc_scale(acc, c, lead_old)  acc (x)= c, where c = H(d_new) (x) H^-1(d_old); lead_old
//                                lets an affine group (a translation of the mean) use the
//                                count it acts on
//   acc_merge(acc, other)        acc (+)= other (both relative to the same lead)
//   kPayload                     payload values per element (0: none)
//
// The row kernels (row_cascade.hip) fold rows with Cascade<Spec>::absorb and
// Cascade<Spec>::combine; the matrix-core kernel (cascade_gemm.hip) takes the lead,
// the correction and the per-element weights from the same engine and leaves the
// (+) of the last level, a contraction with a weight matrix, to the MFMA units.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "topk.hpp"

namespace rf {
namespace cascade {

// ---------------------------------------------------------------- the engine

// Whether a spec folds four elements at once (lead_plus4); only specs without a dependent
// level (no running values, no payload) give it.
template <class S, class = void>
struct has_plus4 : std::false_type {};
template <class S>
struct has_plus4<S, std::void_t<decltype(&S::lead_plus4)>> : std::true_type {
    static_assert(S::kPayload == 0, "lead_plus4 is for cascades without a payload");
};

// Whether a spec advances its lead over a block of elements in one step (lead_plus_block<N>),
// equal in exact arithmetic to N lead_plus.
template <class S, class = void>
struct has_plus_block : std::false_type {};
template <class S>
struct has_plus_block<S, std::void_t<decltype(&S::template lead_plus_block<4>)>> : std::true_type {};

template <class Spec>
struct Cascade {
    using Lead = typename Spec::Lead;
    using Acc = typename Spec::Acc;
    using H = typename Spec::H;
    struct State {
        Lead lead;
        [[no_unique_address]] Acc acc;   // takes no space when a cascade has no dependent level
    };
    static constexpr int kPayload = Spec::kPayload;

    __device__ static State identity() { return {Spec::lead_identity(), Spec::acc_identity()}; }

    // H(d_new) (x) H^-1(d_old): what the running values are multiplied by when the lead moves.
    __device__ static H correction(const Lead& old, const Lead& now) {
        return Spec::h_mul(Spec::h_of(now), Spec::h_inv(Spec::h_of(old)));
    }

    // The running values of a state whose lead is `old`, re-expressed relative to `now`.
    __device__ static void rebase(Acc& acc, const Lead& old, const Lead& now) {
        if (Spec::lead_is_identity(old)) acc = Spec::acc_identity();
        else Spec::acc_scale(acc, correction(old, now), old);
    }

    // The term G(x) (x) H(d) of element x under the lead d.
    __device__ static H term(float x, const Lead& lead) { return Spec::h_mul(Spec::g_of(x), Spec::h_of(lead)); }

    // Fold element j in: advance the lead, correct the running values if it moved, then add
    // the element's terms relative to the new lead.
    __device__ static void absorb(State& st, float x, int32_t j, const float* payload) {
        const Lead now = Spec::lead_plus(st.lead, x, j);
        if (Spec::lead_moved(st.lead, now)) rebase(st.acc, st.lead, now);
        st.lead = now;
        if (!Spec::is_null(x)) Spec::acc_plus(st.acc, term(x, now), x, payload);
    }

    // Fold elements j0 .. j0 + 3 in at once: the incremental form at a coarser step. The lead
    // advances over all four, the running values are corrected once, by
    // H(lead after the four) (x) H^-1(lead before), and the four terms are added relative to
    // the new lead. Equal to four single absorbs in exact arithmetic; a quarter of the
    // corrections. A spec with no dependent level may give lead_plus4, the same lead as four
    // lead_plus in fewer steps.
    __device__ static void absorb4(State& st, const float (&x)[4], int32_t j0, const float* payload) {
        if constexpr (has_plus4<Spec>::value) {
            st.lead = Spec::lead_plus4(st.lead, x, j0);
        } else {
            Lead now = st.lead;
#pragma unroll
            for (int e = 0; e < 4; ++e) now = Spec::lead_plus(now, x[e], j0 + e);
            if (Spec::lead_moved(st.lead, now)) rebase(st.acc, st.lead, now);
            st.lead = now;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (!Spec::is_null(x[e])) Spec::acc_plus(st.acc, term(x[e], now), x[e], payload ? payload + e * kPayload : nullptr);
        }
    }

    // The same over N elements of a row without a payload (indices j[e]): one lead update,
    // one correction, N terms.
    template <int N>
    __device__ static void absorb_n(State& st, const float (&x)[N], const int32_t (&j)[N]) {
        static_assert(kPayload == 0, "absorb_n is for cascades without a payload");
        Lead now = st.lead;
        if constexpr (has_plus_block<Spec>::value) {
            now = Spec::template lead_plus_block<N>(st.lead, x);
        } else {
#pragma unroll
            for (int e = 0; e < N; ++e) now = Spec::lead_plus(now, x[e], j[e]);
        }
        if (Spec::lead_moved(st.lead, now)) rebase(st.acc, st.lead, now);
        st.lead = now;
#pragma unroll
        for (int e = 0; e < N; ++e)
            if (!Spec::is_null(x[e])) Spec::acc_plus(st.acc, term(x[e], now), x[e], nullptr);
    }

    // Merge two partial states: both running values are rebased onto the merged lead.
    __device__ static State combine(const State& a, const State& b) {
        State st;
        st.lead = Spec::lead_merge(a.lead, b.lead);
        st.acc = a.acc;
        Acc other = b.acc;
        rebase(st.acc, a.lead, st.lead);
        rebase(other, b.lead, st.lead);
        Spec::acc_merge(st.acc, other);
        return st;
    }
};

// ---------------------------------------------------------------- groups for H

// Positive scale factors e^t held as their exponent t, so products and inverses never
// overflow: (x) adds exponents, the inverse negates, and a factor is realised only when
// it is applied. Base: e (natural) or 2 (with the inputs pre-scaled by log2 e).
template <bool BASE2>
struct ExpScale {
    float t;
    __device__ static ExpScale mul(const ExpScale& a, const ExpScale& b) { return {a.t + b.t}; }
    __device__ static ExpScale inv(const ExpScale& a) { return {-a.t}; }
    __device__ float value() const { return BASE2 ? exp2_fast(t) : __expf(t); }
};

// Translations of the real line (for centred moments): (x) adds shifts, the inverse negates.
struct Shift {
    float t;
    __device__ static Shift mul(const Shift& a, const Shift& b) { return {a.t + b.t}; }
    __device__ static Shift inv(const Shift& a) { return {-a.t}; }
};

// Non-zero real factors held as their value: (x) multiplies, the inverse is the reciprocal.
struct Ratio {
    float v;
    __device__ static Ratio mul(const Ratio& a, const Ratio& b) { return {a.v * b.v}; }
    __device__ static Ratio inv(const Ratio& a) { return {1.f / a.v}; }
};

// Moves a trivially copyable value between lanes word by word.
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

// The same through a DPP move within each row of 16 lanes (CTRL: a quad permute or a
// mirror), without the LDS permute.
template <int CTRL, class S>
__device__ __forceinline__ S dpp_state(const S& s) {
    static_assert(sizeof(S) % 4 == 0, "states are made of 32-bit words");
    constexpr int W = int(sizeof(S) / 4);
    uint32_t w[W];
    __builtin_memcpy(w, &s, sizeof(S));
#pragma unroll
    for (int i = 0; i < W; ++i) w[i] = uint32_t(__builtin_amdgcn_update_dpp(0, int(w[i]), CTRL, 0xF, 0xF, false));
    S out;
    __builtin_memcpy(&out, w, sizeof(S));
    return out;
}

// Whether a spec's merge is exact and independent of grouping (so any pairing of lanes that
// joins disjoint groups gives the same state): kOrderFree.
template <class S, class = void>
struct order_free : std::false_type {};
template <class S>
struct order_free<S, std::void_t<decltype(S::kOrderFree)>> : std::bool_constant<S::kOrderFree> {};

// ---------------------------------------------------------------- the max-led exponential cascades
// d1 = max x (ascending max, identity -inf), H(d1) = e^(-d1), G(x) = e^x: the safe softmax's
// head. A masked element (-inf) moves no maximum and adds no term.
template <bool BASE2>
struct MaxLed {
    using Lead = float;
    using H = ExpScale<BASE2>;
    __device__ static Lead lead_identity() { return kNegInf; }
    __device__ static Lead lead_plus(Lead m, float x, int32_t) { return fmaxf(m, x); }
    __device__ static Lead lead_merge(Lead a, Lead b) { return fmaxf(a, b); }
    __device__ static bool lead_is_identity(Lead m) { return m == kNegInf; }
    __device__ static bool lead_moved(Lead old, Lead now) { return now != old; }
    __device__ static H h_of(Lead m) { return {-m}; }
    __device__ static H h_inv(const H& h) { return H::inv(h); }
    __device__ static H h_mul(const H& a, const H& b) { return H::mul(a, b); }
    __device__ static H g_of(float x) { return {x}; }
    __device__ static bool is_null(float x) { return x == kNegInf; }
};

// logsumexp: d1 = max x, d2 = sum exp(x - d1); the result is d1 + ln d2.
struct LogSumExp : MaxLed<false> {
    struct Acc {
        float s;
    };
    static constexpr int kPayload = 0;
    __device__ static Acc acc_identity() { return {0.f}; }
    __device__ static void acc_plus(Acc& a, const H& term, float, const float*) { a.s += term.value(); }
    __device__ static void acc_scale(Acc& a, const H& c, Lead) { a.s *= c.value(); }
    __device__ static void acc_merge(Acc& a, const Acc& b) { a.s += b.s; }
};

// softmax-weighted sum: d1 = max x, d2 = sum exp(x - d1), d3 = sum exp(x - d1) v / d2: the
// attention chain with the scores given (P payload values per element). d3's factor 1 / d2
// is applied once at the end (distributivity), so the running values are (d2, the
// unnormalised d3), both scaled by the same correction.
template <int P>
struct SoftmaxWeighted : MaxLed<false> {
    struct Acc {
        float s, o[P];
    };
    static constexpr int kPayload = P;
    __device__ static Acc acc_identity() {
        Acc a;
        a.s = 0.f;
#pragma unroll
        for (int i = 0; i < P; ++i) a.o[i] = 0.f;
        return a;
    }
    __device__ static void acc_plus(Acc& a, const H& term, float, const float* v) {
        const float p = term.value();
        a.s += p;
#pragma unroll
        for (int i = 0; i < P; ++i) a.o[i] = fmaf(p, v[i], a.o[i]);
    }
    __device__ static void acc_scale(Acc& a, const H& c, Lead) {
        const float f = c.value();
        a.s *= f;
#pragma unroll
        for (int i = 0; i < P; ++i) a.o[i] *= f;
    }
    __device__ static void acc_merge(Acc& a, const Acc& b) {
        a.s += b.s;
#pragma unroll
        for (int i = 0; i < P; ++i) a.o[i] += b.o[i];
    }
};

// ---------------------------------------------------------------- top-k, then softmax over the k
// d1 = the K best (score, index) pairs under (score descending, index ascending), held as
// the 64-bit rank keys of topk.hpp (a branch-free insert per element, a bitonic merge of two
// lists); the softmax over them is a final H applied once at the end, so no running value
// depends on d1.
template <int K>
struct TopK {
    struct Lead {
        uint64_t key[K];
        __device__ float score(int r) const { return topk::key_score(key[r]); }
        __device__ int32_t index(int r) const { return topk::key_index(key[r]); }
    };
    struct H {};
    struct Acc {};
    static constexpr int kPayload = 0;
    static constexpr bool kOrderFree = true;      // the K best of a set: exact, any grouping
    __device__ static Lead lead_identity() {
        Lead l;
        topk::clear<K>(l.key);
        return l;
    }
    __device__ static Lead lead_plus(Lead l, float x, int32_t j) {
        topk::insert<K>(l.key, topk::make_key(x, j));
        return l;
    }
    // Four consecutive elements j0 .. j0 + 3 at once (the same list as four lead_plus).
    __device__ static Lead lead_plus4(Lead l, const float (&x)[4], int32_t j0) {
        topk::insert4<K>(l.key, topk::make_key(x[0], j0), topk::make_key(x[1], j0 + 1), topk::make_key(x[2], j0 + 2),
                         topk::make_key(x[3], j0 + 3));
        return l;
    }
    __device__ static Lead lead_merge(const Lead& a, const Lead& b) {
        Lead l = a;
        topk::merge<K>(l.key, b.key);
        return l;
    }
    __device__ static bool lead_is_identity(const Lead&) { return false; }
    __device__ static bool lead_moved(const Lead&, const Lead&) { return false; }
    __device__ static H h_of(const Lead&) { return {}; }
    __device__ static H h_inv(const H&) { return {}; }
    __device__ static H h_mul(const H&, const H&) { return {}; }
    __device__ static H g_of(float) { return {}; }
    __device__ static bool is_null(float) { return true; }
    __device__ static Acc acc_identity() { return {}; }
    __device__ static void acc_plus(Acc&, const H&, float, const float*) {}
    __device__ static void acc_scale(Acc&, const H&, const Lead&) {}
    __device__ static void acc_merge(Acc&, const Acc&) {}
};

// ---------------------------------------------------------------- mean and variance
// d1 = mean, d2 = sum (x - d1)^2. H is the translation by -d1 and G(x) = x, so a term is the
// squared shifted value. Moving the centre of a sum of squares whose first moment about the
// old centre is zero (the old centre is the old mean) by t adds n t^2: the correction
// mechanism of this cascade. Absorbing one element is then Welford's update, and merging two
// states the pairwise rule of Chan, Golub and LeVeque.
struct MeanVar {
    struct Lead {
        uint32_t n;          // an integer count: a float one stops growing at 2^24
        float mean;
    };
    using H = Shift;
    struct Acc {
        float m2;
    };
    static constexpr int kPayload = 0;
    __device__ static Lead lead_identity() { return {0u, 0.f}; }
    __device__ static Lead lead_plus(const Lead& l, float x, int32_t) {
        const uint32_t n = l.n + 1u;
        return {n, l.mean + (x - l.mean) / float(n)};
    }
    // N elements at once: the mean moves by the sum of their deviations from the old mean over
    // the new count (one division instead of N).
    template <int N>
    __device__ static Lead lead_plus_block(const Lead& l, const float (&x)[N]) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < N; ++e) d += x[e] - l.mean;
        const uint32_t n = l.n + uint32_t(N);
        return {n, l.mean + d / float(n)};
    }
    __device__ static Lead lead_merge(const Lead& a, const Lead& b) {
        const uint32_t n = a.n + b.n;
        if (n == 0u) return lead_identity();
        return {n, a.mean + (b.mean - a.mean) * (float(b.n) / float(n))};
    }
    __device__ static bool lead_is_identity(const Lead& l) { return l.n == 0u; }
    __device__ static bool lead_moved(const Lead&, const Lead&) { return true; }
    __device__ static H h_of(const Lead& l) { return {-l.mean}; }
    __device__ static H h_inv(const H& h) { return H::inv(h); }
    __device__ static H h_mul(const H& a, const H& b) { return H::mul(a, b); }
    __device__ static H g_of(float x) { return {x}; }
    __device__ static bool is_null(float) { return false; }
    __device__ static Acc acc_identity() { return {0.f}; }
    __device__ static void acc_plus(Acc& a, const H& term, float, const float*) { a.m2 = fmaf(term.t, term.t, a.m2); }
    __device__ static void acc_scale(Acc& a, const H& c, const Lead& old) { a.m2 = fmaf(float(old.n) * c.t, c.t, a.m2); }
    __device__ static void acc_merge(Acc& a, const Acc& b) { a.m2 += b.m2; }
};

// ---------------------------------------------------------------- row-scaled GEMM cascades
// The leads and groups of the matrix-core instances (cascade_gemm.hip). A row x of [M, K]
// is reduced against the K x N weight W: y = (+)_k G(x_k) (x) H(d1) w_k, where the last
// (+) is the contraction done on the matrix cores, so only the per-element weight
// realise(g_of(x) (x) h_of(d1)) is needed from the spec, plus the correction.

// y = softmax(x) W and lse = ln sum exp(x): d1 = max x (in base-2 units of x log2 e),
// d2 = sum 2^(x' - d1), d3 = sum 2^(x' - d1) w / d2. The kernel takes x' = x log2 e.
// The row sum d2 is the running value kept on the vector ALUs; d3's running value is the
// matrix-core accumulator, scaled by the same factor.
struct SoftmaxGemm : MaxLed<true> {
    struct Acc {
        float s;
    };
    static constexpr int kPayload = 0;
    __device__ static Acc acc_identity() { return {0.f}; }
    __device__ static void acc_plus(Acc& a, const H& term, float, const float*) { a.s += term.value(); }
    __device__ static void acc_scale(Acc& a, const H& c, Lead) { a.s *= c.value(); }
    __device__ static void acc_merge(Acc& a, const Acc& b) { a.s += b.s; }
    __device__ static float weight(const H& term) { return term.value(); }
    __device__ static float factor(const H& c) { return c.value(); }
};

// y = (x / max |x|) W: d1 = max |x| (identity 0), H(d1) = 1 / d1, G(x) = x, (x) = *. The
// correction when the row's absolute maximum grows from a to b is a / b.
struct AbsMaxGemm {
    using Lead = float;
    using H = Ratio;
    __device__ static Lead lead_identity() { return 0.f; }
    __device__ static Lead lead_plus(Lead a, float x, int32_t) { return fmaxf(a, fabsf(x)); }
    __device__ static Lead lead_merge(Lead a, Lead b) { return fmaxf(a, b); }
    __device__ static bool lead_is_identity(Lead a) { return a == 0.f; }
    __device__ static bool lead_moved(Lead old, Lead now) { return now != old; }
    __device__ static H h_of(Lead a) { return {1.f / a}; }
    __device__ static H h_inv(const H& h) { return H::inv(h); }
    __device__ static H h_mul(const H& a, const H& b) { return H::mul(a, b); }
    __device__ static H g_of(float x) { return {x}; }
    __device__ static bool is_null(float x) { return x == 0.f; }
    // The only running value is the matrix-core accumulator.
    struct Acc {};
    static constexpr int kPayload = 0;
    __device__ static Acc acc_identity() { return {}; }
    __device__ static void acc_plus(Acc&, const H&, float, const float*) {}
    __device__ static void acc_scale(Acc&, const H&, Lead) {}
    __device__ static void acc_merge(Acc&, const Acc&) {}
    __device__ static float weight(const H& term) { return term.v; }
    __device__ static float factor(const H& c) { return c.v; }
};

}  // namespace cascade
}  // namespace rf
