// Single-segment fused attention, fp32 inputs, on the fp32 matrix cores.
//
// The softmax -> GEMM cascade (explainer "RedFuser框架：AI加速器中的算子融合技术解析",
// sections 2.2 and 4.1) evaluated in its incremental form (section 2.3; technical
// summary, Methodologie 2): per query row a running maximum m, a running sum s of
// exponentials and an unnormalised accumulator o~ are rescaled by exp(m_old - m_new)
// whenever the maximum grows, and o = o~ / s is formed once at the end.
//
// Mapping (wave64, v_mfma_f32_16x16x4_f32):
//  * a workgroup owns 16 query rows and NW waves (8 for D = 64, 4 for D = 128);
//    wave w walks key tiles of 16
//    keys t = w, w + NW, ... (an intra-block split of the key axis), loading tile
//    t + NW's K and V into registers before it works on tile t;
//  * scores are formed transposed, S^T = K Q^T, so that each lane holds one query
//    row (lane % 16) and four keys (4 * (lane / 16) + r): the row statistics are
//    lane-local plus a two-step butterfly over the lane groups;
//  * the output is formed transposed too, O^T = V^T P^T, so the P^T fragment in
//    registers is directly the MFMA B operand and the accumulator rows again
//    belong to the lane's own query (the rescale by alpha is lane-local);
//  * at the end the NW per-wave states (m, s, o~) are merged through LDS with the
//    same (max, sum, partial-O) combination the multi-segment merge uses.
// Scores are kept in base-2 units (x * scale * log2 e) so that exp is v_exp_f32.
#include "common.hpp"
#include "launch.hpp"

namespace rf {
namespace {

template <int D, int kNW>
__global__ __launch_bounds__(kNW * 64) void attn_fwd_f32_kernel(const float* __restrict__ q,
                                                                const float* __restrict__ k,
                                                                const float* __restrict__ v,
                                                                float* __restrict__ o,
                                                                float* __restrict__ lse,
                                                                int64_t Sq, int64_t Sk, int nqb,
                                                                float scale_log2) {
    constexpr int C = D / 4;      // contraction slots per lane group for Q K^T
    constexpr int DB = D / 16;    // 16-wide output column blocks
    __shared__ float sm_m[kNW][16];
    __shared__ float sm_s[kNW][16];
    __shared__ float sm_o[kNW][16][D + 1];

    const int64_t bh = blockIdx.x / nqb;
    const int64_t q0 = int64_t(blockIdx.x % nqb) * 16;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, g = lane >> 4;

    const float* qh = q + bh * Sq * D;
    const float* kh = k + bh * Sk * D;
    const float* vh = v + bh * Sk * D;

    // Q^T operand: lane (query r16, group g) holds Q[q0 + r16][g*C + c], c = 0..C-1.
    float qf[C];
    {
        const int64_t qi = q0 + r16 < Sq ? q0 + r16 : Sq - 1;
        const float4* src = reinterpret_cast<const float4*>(qh + qi * D + g * C);
#pragma unroll
        for (int c = 0; c < C / 4; ++c) {
            float4 t = src[c];
            qf[4 * c] = t.x; qf[4 * c + 1] = t.y; qf[4 * c + 2] = t.z; qf[4 * c + 3] = t.w;
        }
    }

    float m = kNegInf, s = 0.f;
    f32x4 acc[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};

    // K operand of a key tile: lane (key r16, group g) holds K[kb + r16][g*C + c]; V operand:
    // lane holds V[kb + 4g + r][16b + r16] for key slot r and column block b. Keys past the
    // axis re-read the last key (their scores are masked).
    auto load_kv = [&](int64_t kb, float4 (&kf)[C / 4], float (&vf)[4][DB]) {
        const int64_t kj = kb + r16 < Sk ? kb + r16 : Sk - 1;
        const float4* src = reinterpret_cast<const float4*>(kh + kj * D + g * C);
#pragma unroll
        for (int c = 0; c < C / 4; ++c) kf[c] = src[c];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t vj = kb + 4 * g + r < Sk ? kb + 4 * g + r : Sk - 1;
            const float* vrow = vh + vj * D + r16;
#pragma unroll
            for (int b = 0; b < DB; ++b) vf[r][b] = vrow[16 * b];
        }
    };

    // The next tile's K and V are loaded before the current tile is processed, so one
    // memory round trip overlaps the MFMA and softmax work of the tile before.
    const int64_t kstep = int64_t(kNW) * 16;
    float4 kf[C / 4];
    float vf[4][DB];
    int64_t kb = int64_t(wave) * 16;
    if (kb < Sk) load_kv(kb, kf, vf);
    for (; kb < Sk; kb += kstep) {
        const bool more = kb + kstep < Sk;
        float4 kn[C / 4];
        float vn[4][DB];
        if (more) load_kv(kb + kstep, kn, vn);
        f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < C / 4; ++c) {
            const float4 t = kf[c];
            st = __builtin_amdgcn_mfma_f32_16x16x4f32(t.x, qf[4 * c + 0], st, 0, 0, 0);
            st = __builtin_amdgcn_mfma_f32_16x16x4f32(t.y, qf[4 * c + 1], st, 0, 0, 0);
            st = __builtin_amdgcn_mfma_f32_16x16x4f32(t.z, qf[4 * c + 2], st, 0, 0, 0);
            st = __builtin_amdgcn_mfma_f32_16x16x4f32(t.w, qf[4 * c + 3], st, 0, 0, 0);
        }
        // st[r] = S[query q0 + r16][key kb + 4g + r] (unscaled).
        float x[4];
        float tmax = kNegInf;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            x[r] = (kb + 4 * g + r < Sk) ? st[r] * scale_log2 : kNegInf;
            tmax = fmaxf(tmax, x[r]);
        }
        tmax = xor_max(tmax, 16);
        tmax = xor_max(tmax, 32);
        const float m_new = fmaxf(m, tmax);
        const float m_use = m_new == kNegInf ? 0.f : m_new;     // no key seen yet: keep p = 0
        const float alpha = exp2_fast(m - m_use);               // m = -inf -> 0
        float p[4], psum = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            p[r] = exp2_fast(x[r] - m_use);
            psum += p[r];
        }
        psum = xor_sum(psum, 16);
        psum = xor_sum(psum, 32);
        s = alpha * s + psum;
        m = m_new;
#pragma unroll
        for (int b = 0; b < DB; ++b) acc[b] *= alpha;
        // O^T += V^T P^T, one MFMA per key slot r: lane group g contributes key kb + 4g + r.
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int b = 0; b < DB; ++b)
                acc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf[r][b], p[r], acc[b], 0, 0, 0);
        if (more) {
#pragma unroll
            for (int c = 0; c < C / 4; ++c) kf[c] = kn[c];
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int b = 0; b < DB; ++b) vf[r][b] = vn[r][b];
        }
    }

    // acc[b][i] = o~[query q0 + r16][16b + 4g + i]. Merge the NW wave states.
    if (g == 0) {
        sm_m[wave][r16] = m;
        sm_s[wave][r16] = s;
    }
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) sm_o[wave][r16][16 * b + 4 * g + i] = acc[b][i];
    __syncthreads();

    for (int e = threadIdx.x; e < 16 * D; e += kNW * 64) {
        const int row = e / D, d = e % D;
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < kNW; ++w) M = fmaxf(M, sm_m[w][row]);
        float S = 0.f, O = 0.f;
#pragma unroll
        for (int w = 0; w < kNW; ++w) {
            const float mw = sm_m[w][row];
            const float wt = mw == kNegInf ? 0.f : exp2_fast(mw - M);
            S += wt * sm_s[w][row];
            O += wt * sm_o[w][row][d];
        }
        const int64_t qi = q0 + row;
        if (qi < Sq) {
            o[(bh * Sq + qi) * D + d] = O / S;
            if (lse && d == 0) lse[bh * Sq + qi] = (M + __log2f(S)) * kLn2;
        }
    }
}

}  // namespace

hipError_t launch_attn_fwd_f32(const float* q, const float* k, const float* v, float* o,
                               float* lse, int64_t BH, int64_t Sq, int64_t Sk, int D,
                               float scale, hipStream_t stream) {
    const int64_t nqb = ceil_div(Sq, 16);
    const int64_t blocks = BH * nqb;
    if (blocks > INT32_MAX || nqb > INT32_MAX) return hipErrorInvalidValue;
    const float sl2 = scale * kLog2e;
    if (D == 64)
        hipLaunchKernelGGL((attn_fwd_f32_kernel<64, 8>), dim3(unsigned(blocks)), dim3(8 * 64), 0, stream, q, k,
                           v, o, lse, Sq, Sk, int(nqb), sl2);
    else
        hipLaunchKernelGGL((attn_fwd_f32_kernel<128, 4>), dim3(unsigned(blocks)), dim3(4 * 64), 0, stream, q, k,
                           v, o, lse, Sq, Sk, int(nqb), sl2);
    return hipGetLastError();
}

}  // namespace rf
