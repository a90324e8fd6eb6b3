// Row cascades built from the generic incremental template (cascade.hpp: Cascade<Spec>).
//
// A group of G lanes folds one row of x [R, N] (fp32; G from 4 to 64 so that every lane
// absorbs at least 32 elements): lane i absorbs elements 4i .. 4i+3 of every 4G-element
// stretch (16-byte loads; i, i+G, i+2G, i+3G with a 4-value payload), then the group's
// states are merged by xor shuffles in a fixed order and the group's first lane writes the
// row's result. The instances are the cascades the technical summary "RedFuser: An
// Automatic Operator Fusion Framework for Cascaded Reductions on AI Accelerators"
// (Methodologie 1-2) and the explainer
// "RedFuser框架：AI加速器中的算子融合技术解析" (sections 2.2, 4.1, 4.2) use as examples,
// plus mean/variance as a cascade outside attention:
//   logsumexp                 out[r] = max + ln(sum exp(x - max))
//   softmax-weighted sum      out[r, :] = sum_j softmax(x)_j payload[r, j, :]   (P values)
//   top-k then softmax        out[r, i] = softmax over the k best, out_idx[r, i] their index
//   mean / variance           out[r, 0] = mean, out[r, 1] = population variance
#include "cascade.hpp"
#include "launch.hpp"

namespace rf {
namespace {

using namespace cascade;

// G lanes fold one row (G in {4, 8, 16, 32, 64}; 64 / G rows per wave): lane i of the group
// absorbs elements 4i .. 4i+3 of every 4G-element stretch, or i + G e (e = 0..3) with a
// 4-value payload (eight, or four for a large state, streaming 16-byte loads in flight when
// there is no payload), then the group's states are merged by xor shuffles within the group,
// in a fixed order (for a merge that is exact in any grouping, by DPP moves where the group
// fits a row of 16 lanes).
template <class Spec, int G>
__device__ __forceinline__ typename Cascade<Spec>::State fold_row(const float* __restrict__ xr,
                                                                  const float* __restrict__ pr, int64_t N, int li) {
    using C = Cascade<Spec>;
    constexpr int P = C::kPayload;
    constexpr int STRIDE = 4 * G;
    typename C::State st = C::identity();
    auto absorb4 = [&](const float4& v, int64_t j0) {
        const float xs[4] = {v.x, v.y, v.z, v.w};
        C::absorb4(st, xs, int32_t(j0), P ? pr + j0 * P : nullptr);
    };
    const bool vec = (N & 3) == 0;            // 16-byte loads need aligned rows
    // Eight loads in flight when only x is read (nontemporal: the row is read once), four for
    // a large state (top-k: its registers would cost occupancy); with a payload its loads
    // already overlap.
    constexpr int UN = sizeof(typename C::State) > 32 ? 4 : 8;
    const int64_t full4 = vec && P == 0 ? N / (UN * STRIDE) * (UN * STRIDE) : 0;
    int64_t j0 = 4 * li;
    for (; j0 < full4; j0 += UN * STRIDE) {
        float4 v[UN];
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            typedef float fx4 __attribute__((ext_vector_type(4)));
            const fx4 t = __builtin_nontemporal_load(reinterpret_cast<const fx4*>(xr + j0 + u * STRIDE));
            v[u] = make_float4(t[0], t[1], t[2], t[3]);
        }
        if constexpr (has_plus4<Spec>::value || P != 0) {   // (this loop runs only without a payload)
#pragma unroll
            for (int u = 0; u < UN; ++u) absorb4(v[u], j0 + u * STRIDE);
        } else {
            // The whole batch at once: one correction for 4 UN elements.
            float xs[4 * UN];
            int32_t js[4 * UN];
#pragma unroll
            for (int u = 0; u < UN; ++u) {
                xs[4 * u] = v[u].x; xs[4 * u + 1] = v[u].y; xs[4 * u + 2] = v[u].z; xs[4 * u + 3] = v[u].w;
#pragma unroll
                for (int e = 0; e < 4; ++e) js[4 * u + e] = int32_t(j0 + u * STRIDE + e);
            }
            C::template absorb_n<4 * UN>(st, xs, js);
        }
    }
    // With a payload of P <= 8 values, UPW stretches of x and payload are loaded before any
    // is absorbed. For P = 1 and 2 a lane takes the 4 consecutive elements 4i .. 4i+3 of a
    // stretch (1 + P 16-byte loads). For P = 4 and 8 an element's payload is one or two whole
    // 16-byte pieces, so lane i takes elements i, i + G, i + 2G and i + 3G instead ("spread"):
    // its x loads then read, across the group, one contiguous run of G x 4 bytes and its
    // payload loads runs of 16 bytes at a P x 4-byte stride, where the consecutive mapping's
    // payload loads have a 4 P x 4-byte lane stride (measured at 4096 x 8192: P = 4 98.5
    // against 111.7 us, P = 8 186 against 313 us; P = 16 was slower spread, 551 against 464 us,
    // and keeps the consecutive mapping). The cascade's result does not depend on the order in
    // which a lane absorbs its elements.
    constexpr bool SPREAD = P == 4 || P == 8;
    constexpr int UPW = P == 0 ? 1 : P <= 1 ? 4 : P <= 2 ? 3 : P <= 4 ? 4 : P <= 8 ? 2 : 1;
    if constexpr (UPW > 1 || SPREAD) {
        typedef float fx4 __attribute__((ext_vector_type(4)));
        const int64_t fullp = vec ? N / (UPW * STRIDE) * (UPW * STRIDE) : 0;
        for (; j0 < fullp; j0 += UPW * STRIDE) {
            fx4 xv[UPW];
            float pv[UPW][4 * P];
#pragma unroll
            for (int u = 0; u < UPW; ++u) {
                if constexpr (SPREAD) {
                    const int64_t je0 = j0 - 4 * li + u * STRIDE + li;   // the lane's first element
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int64_t je = je0 + int64_t(G) * e;
                        xv[u][e] = __builtin_nontemporal_load(xr + je);
#pragma unroll
                        for (int c = 0; c < P / 4; ++c) {
                            const fx4 t = __builtin_nontemporal_load(reinterpret_cast<const fx4*>(pr + je * P + 4 * c));
#pragma unroll
                            for (int i = 0; i < 4; ++i) pv[u][P * e + 4 * c + i] = t[i];
                        }
                    }
                } else {
                    const int64_t j = j0 + u * STRIDE;
                    xv[u] = __builtin_nontemporal_load(reinterpret_cast<const fx4*>(xr + j));
#pragma unroll
                    for (int c = 0; c < P; ++c) {
                        // Cached loads: lane i's P 16-byte loads of a stretch share cache lines
                        // with lane i + 1's, so a streaming hint would fetch each line again.
                        const fx4 t = *reinterpret_cast<const fx4*>(pr + j * P + 4 * c);
#pragma unroll
                        for (int e = 0; e < 4; ++e) pv[u][4 * c + e] = t[e];
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < UPW; ++u) {
                const float xs[4] = {xv[u][0], xv[u][1], xv[u][2], xv[u][3]};
                C::absorb4(st, xs, int32_t(j0 + u * STRIDE), pv[u]);
            }
        }
    }
    const int64_t full = vec ? N / STRIDE * STRIDE : 0;
    for (; j0 < full; j0 += STRIDE) absorb4(*reinterpret_cast<const float4*>(xr + j0), j0);
    for (int64_t j = full + li; j < N; j += G) C::absorb(st, xr[j], int32_t(j), P ? pr + j * P : nullptr);
    if constexpr (order_free<Spec>::value) {
        // Any pairing that joins disjoint groups gives the same state: DPP moves within the
        // row (lane xor 1, xor 2, then the half-row and row mirrors), LDS permutes above 16.
        if constexpr (G >= 2) st = C::combine(st, dpp_state<0xB1>(st));
        if constexpr (G >= 4) st = C::combine(st, dpp_state<0x4E>(st));
        if constexpr (G >= 8) st = C::combine(st, dpp_state<0x141>(st));
        if constexpr (G >= 16) st = C::combine(st, dpp_state<0x140>(st));
        if constexpr (G >= 32) st = C::combine(st, shfl_xor_state(st, 16));
        if constexpr (G >= 64) st = C::combine(st, shfl_xor_state(st, 32));
    } else {
#pragma unroll
        for (int mask = G / 2; mask >= 1; mask >>= 1) st = C::combine(st, shfl_xor_state(st, mask));
    }
    return st;
}

// Row r of this thread: 4 waves of 64 / G rows each per workgroup.
template <int G>
__device__ __forceinline__ int64_t row_of(int& li) {
    li = int(threadIdx.x) & (G - 1);
    return int64_t(blockIdx.x) * (256 / G) + (threadIdx.x / G);
}

template <int G>
__global__ __launch_bounds__(256) void lse_kernel(const float* __restrict__ x, int64_t R, int64_t N,
                                                  float* __restrict__ out) {
    int li;
    const int64_t r = row_of<G>(li);
    if (r >= R) return;
    const auto st = fold_row<LogSumExp, G>(x + r * N, nullptr, N, li);
    if (li == 0) out[r] = st.lead + __logf(st.acc.s);
}

template <int G, int P>
__global__ __launch_bounds__(256) void softmax_weighted_kernel(const float* __restrict__ x,
                                                               const float* __restrict__ payload, int64_t R,
                                                               int64_t N, float* __restrict__ out) {
    int li;
    const int64_t r = row_of<G>(li);
    if (r >= R) return;
    const auto st = fold_row<SoftmaxWeighted<P>, G>(x + r * N, payload + r * N * P, N, li);
    for (int i0 = 0; i0 < P; i0 += G) {
        const int i = i0 + li;
        float o = st.acc.o[0];
#pragma unroll
        for (int c = 1; c < P; ++c) o = i == c ? st.acc.o[c] : o;
        if (i < P) out[r * P + i] = o / st.acc.s;
    }
}

template <int G>
__global__ __launch_bounds__(256) void topk_softmax_kernel(const float* __restrict__ x, int64_t R, int64_t N, int k,
                                                           float* __restrict__ out, int32_t* __restrict__ out_idx) {
    constexpr int K = 8;
    int li;
    const int64_t r = row_of<G>(li);
    if (r >= R) return;
    const auto st = fold_row<TopK<K>, G>(x + r * N, nullptr, N, li);
    // Every lane of the row's group holds the merged list; lane li writes entries 2 li and
    // 2 li + 1, so a wave's stores cover its rows' outputs contiguously, as whole lines (k even)
    // with streaming stores that leave no dirty lines for the end-of-kernel write-back.
    {
        float e[K], den = 0.f;
#pragma unroll
        for (int i = 0; i < K; ++i) {
            e[i] = i < k ? __expf(st.lead.score(i) - st.lead.score(0)) : 0.f;
            den += e[i];
        }
        const float inv = 1.f / den;
        typedef float fx2 __attribute__((ext_vector_type(2)));
        typedef int32_t ix2 __attribute__((ext_vector_type(2)));
        const int i0 = 2 * li;
        float w0 = 0.f, w1 = 0.f;
        int32_t x0 = 0, x1 = 0;
#pragma unroll
        for (int i = 0; i < K; ++i) {
            if (i == i0) { w0 = e[i] * inv; x0 = st.lead.index(i); }
            if (i == i0 + 1) { w1 = e[i] * inv; x1 = st.lead.index(i); }
        }
        if (i0 + 1 < k) {
            if ((k & 1) == 0) {
                const fx2 wv = {w0, w1};
                const ix2 iv = {x0, x1};
                __builtin_nontemporal_store(wv, reinterpret_cast<fx2*>(out + r * k + i0));
                __builtin_nontemporal_store(iv, reinterpret_cast<ix2*>(out_idx + r * k + i0));
            } else {
                out[r * k + i0] = w0; out[r * k + i0 + 1] = w1;
                out_idx[r * k + i0] = x0; out_idx[r * k + i0 + 1] = x1;
            }
        } else if (i0 < k) {
            out[r * k + i0] = w0;
            out_idx[r * k + i0] = x0;
        }
    }
}

template <int G>
__global__ __launch_bounds__(256) void mean_var_kernel(const float* __restrict__ x, int64_t R, int64_t N,
                                                       float* __restrict__ out) {
    int li;
    const int64_t r = row_of<G>(li);
    if (r >= R) return;
    const auto st = fold_row<MeanVar, G>(x + r * N, nullptr, N, li);
    if (li == 0) {
        out[r * 2] = st.lead.mean;
        out[r * 2 + 1] = st.acc.m2 / float(st.lead.n);
    }
}

template <int G>
hipError_t launch_g(int kind, const float* x, const float* payload, int64_t R, int64_t N, int P, int k, float* out,
                    int32_t* out_idx, hipStream_t stream) {
    const int64_t blocks = ceil_div(R, int64_t(256 / G));
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    const dim3 grid{unsigned(blocks), 1u, 1u}, block{256u, 1u, 1u};
    switch (kind) {
        case 0: hipLaunchKernelGGL(lse_kernel<G>, grid, block, 0, stream, x, R, N, out); break;
        case 1:
            switch (P) {
                case 1: hipLaunchKernelGGL((softmax_weighted_kernel<G, 1>), grid, block, 0, stream, x, payload, R, N, out); break;
                case 2: hipLaunchKernelGGL((softmax_weighted_kernel<G, 2>), grid, block, 0, stream, x, payload, R, N, out); break;
                case 4: hipLaunchKernelGGL((softmax_weighted_kernel<G, 4>), grid, block, 0, stream, x, payload, R, N, out); break;
                case 8: hipLaunchKernelGGL((softmax_weighted_kernel<G, 8>), grid, block, 0, stream, x, payload, R, N, out); break;
                case 16: hipLaunchKernelGGL((softmax_weighted_kernel<G, 16>), grid, block, 0, stream, x, payload, R, N, out); break;
                default: return hipErrorInvalidValue;
            }
            break;
        case 2: hipLaunchKernelGGL(topk_softmax_kernel<G>, grid, block, 0, stream, x, R, N, k, out, out_idx); break;
        case 3: hipLaunchKernelGGL(mean_var_kernel<G>, grid, block, 0, stream, x, R, N, out); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_row_cascade(int kind, const float* x, const float* payload, int64_t R, int64_t N, int P, int k,
                              float* out, int32_t* out_idx, hipStream_t stream) {
    // Lanes per row: enough that each lane absorbs at least 32 elements (64 for top-k, where
    // every merge level costs as much as folding in about five elements), at most a wave.
    const int64_t per_lane = kind == 2 ? 64 : 32;
    int64_t g = 4;
    while (g < 64 && N >= per_lane * 2 * g) g *= 2;
    switch (g) {
        case 4: return launch_g<4>(kind, x, payload, R, N, P, k, out, out_idx, stream);
        case 8: return launch_g<8>(kind, x, payload, R, N, P, k, out, out_idx, stream);
        case 16: return launch_g<16>(kind, x, payload, R, N, P, k, out, out_idx, stream);
        case 32: return launch_g<32>(kind, x, payload, R, N, P, k, out, out_idx, stream);
        default: return launch_g<64>(kind, x, payload, R, N, P, k, out, out_idx, stream);
    }
}

}  // namespace rf
