// Row cascades built from the generic incremental template (cascade.hpp).
//
// One wave folds one row of x [R, N] (fp32): lane l absorbs elements 4l .. 4l+3 of every
// 256-element stretch (16-byte loads), then the 64 lane states are merged by xor shuffles
// in a fixed order and lane 0 writes the row's result. The instances are the cascades
// the technical summary "RedFuser: An Automatic Operator Fusion Framework for Cascaded
// Reductions on AI Accelerators" (Methodologie 1-2) and the explainer
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

template <class Spec>
__device__ __forceinline__ typename Spec::State fold_row(const float* __restrict__ xr, const float* __restrict__ pr,
                                                         int64_t N, int lane) {
    constexpr int P = Spec::kPayload;
    typename Spec::State st = Spec::identity();
    const int64_t full = (N & 3) == 0 ? (N & ~int64_t(255)) : 0;   // 16-byte loads need aligned rows
    for (int64_t j0 = 4 * lane; j0 < full; j0 += 256) {
        const float4 v = *reinterpret_cast<const float4*>(xr + j0);
        const float xs[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) Spec::absorb(st, xs[e], int32_t(j0 + e), P ? pr + (j0 + e) * P : nullptr);
    }
    for (int64_t j = full + lane; j < N; j += 64) Spec::absorb(st, xr[j], int32_t(j), P ? pr + j * P : nullptr);
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1) st = Spec::combine(st, shfl_xor_state(st, mask));
    return st;
}

__global__ __launch_bounds__(256) void lse_kernel(const float* __restrict__ x, int64_t R, int64_t N,
                                                  float* __restrict__ out) {
    const int64_t r = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (r >= R) return;
    const auto st = fold_row<LogSumExp>(x + r * N, nullptr, N, lane);
    if (lane == 0) out[r] = st.m + __logf(st.s);
}

template <int P>
__global__ __launch_bounds__(256) void softmax_weighted_kernel(const float* __restrict__ x,
                                                               const float* __restrict__ payload, int64_t R,
                                                               int64_t N, float* __restrict__ out) {
    const int64_t r = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (r >= R) return;
    const auto st = fold_row<SoftmaxWeighted<P>>(x + r * N, payload + r * N * P, N, lane);
    if (lane < P) {
        float o = st.o[0];
#pragma unroll
        for (int i = 1; i < P; ++i) o = lane == i ? st.o[i] : o;
        out[r * P + lane] = o / st.s;
    }
}

__global__ __launch_bounds__(256) void topk_softmax_kernel(const float* __restrict__ x, int64_t R, int64_t N, int k,
                                                           float* __restrict__ out, int32_t* __restrict__ out_idx) {
    constexpr int K = 8;
    const int64_t r = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (r >= R) return;
    const auto st = fold_row<TopK<K>>(x + r * N, nullptr, N, lane);
    if (lane == 0) {
        float e[K], den = 0.f;
#pragma unroll
        for (int i = 0; i < K; ++i) {
            e[i] = i < k ? __expf(st.s[i] - st.s[0]) : 0.f;
            den += e[i];
        }
        const float inv = 1.f / den;
#pragma unroll
        for (int i = 0; i < K; ++i)
            if (i < k) {
                out[r * k + i] = e[i] * inv;
                out_idx[r * k + i] = st.i[i];
            }
    }
}

__global__ __launch_bounds__(256) void mean_var_kernel(const float* __restrict__ x, int64_t R, int64_t N,
                                                       float* __restrict__ out) {
    const int64_t r = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (r >= R) return;
    const auto st = fold_row<MeanVar>(x + r * N, nullptr, N, lane);
    if (lane == 0) {
        out[r * 2] = st.mean;
        out[r * 2 + 1] = st.m2 / st.n;
    }
}

}  // namespace

hipError_t launch_row_cascade(int kind, const float* x, const float* payload, int64_t R, int64_t N, int P, int k,
                              float* out, int32_t* out_idx, hipStream_t stream) {
    const int64_t blocks = ceil_div(R, int64_t(4));
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    const dim3 grid{unsigned(blocks), 1u, 1u}, block{256u, 1u, 1u};
    switch (kind) {
        case 0: hipLaunchKernelGGL(lse_kernel, grid, block, 0, stream, x, R, N, out); break;
        case 1:
            switch (P) {
                case 1: hipLaunchKernelGGL(softmax_weighted_kernel<1>, grid, block, 0, stream, x, payload, R, N, out); break;
                case 2: hipLaunchKernelGGL(softmax_weighted_kernel<2>, grid, block, 0, stream, x, payload, R, N, out); break;
                case 4: hipLaunchKernelGGL(softmax_weighted_kernel<4>, grid, block, 0, stream, x, payload, R, N, out); break;
                case 8: hipLaunchKernelGGL(softmax_weighted_kernel<8>, grid, block, 0, stream, x, payload, R, N, out); break;
                case 16: hipLaunchKernelGGL(softmax_weighted_kernel<16>, grid, block, 0, stream, x, payload, R, N, out); break;
                default: return hipErrorInvalidValue;
            }
            break;
        case 2: hipLaunchKernelGGL(topk_softmax_kernel, grid, block, 0, stream, x, R, N, k, out, out_idx); break;
        case 3: hipLaunchKernelGGL(mean_var_kernel, grid, block, 0, stream, x, R, N, out); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace rf
