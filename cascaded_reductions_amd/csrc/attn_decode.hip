// Multi-segment decode attention: the split kernel and the merge kernel.
//
// Decode has one query token per (batch, head) row, so the key axis is the only
// source of parallelism. The Multi-Segment strategy (technical summary
// "RedFuser: An Automatic Operator Fusion Framework for Cascaded Reductions on AI
// Accelerators", Methodologie 3; explainer "RedFuser框架：AI加速器中的算子融合技术解析",
// section 3.3, inter-block merge) splits it into segments reduced independently
// in the incremental form, then merges the per-segment (max, sum, partial-O)
// triples with the monoid combination of the fusion conditions (Methodologie 1).
//
// Split kernel, one wave per (row, segment). The work is HBM-bound (one FLOP per
// byte), so it runs on the vector ALUs with 16-byte coalesced loads: a key row of
// D bf16 values is read by D/8 lanes (8 values each), so one wave load covers
// 64*8/D consecutive keys ("key slots"). Each key slot keeps its own running
// (m, s, o~) over the keys it sees; the slots are merged with cross-lane
// exchanges at the end. Scores are in base-2 units (q pre-scaled by
// scale * log2 e); the stored maxima are converted back to natural units.
#include "common.hpp"
#include "launch.hpp"

namespace rf {
namespace {

// DIRECT: a single segment per row (the Single-Segment strategy for decode): the wave
// normalises its own state and writes o (bf16 or fp32) and lse; no partials, no merge.
template <int D, int U, bool DIRECT = false>
__global__ __launch_bounds__(64) void decode_split_kernel(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v,
                                                          int64_t L, int64_t nseg, int64_t seglen,
                                                          float scale_log2, float* __restrict__ part_m,
                                                          float* __restrict__ part_s,
                                                          float* __restrict__ part_o,
                                                          void* __restrict__ out = nullptr, int out_bf16 = 0,
                                                          float* __restrict__ lse = nullptr) {
    constexpr int LPK = D / 8;      // lanes per key row
    constexpr int KPW = 64 / LPK;   // key slots per wave load
    const int64_t wid = blockIdx.x; // row * nseg + segment
    const int64_t r = wid / nseg, t = wid - r * nseg;
    const int lane = threadIdx.x;
    const int slot = lane / LPK, c = lane % LPK;

    const int64_t a = t * seglen;
    const int64_t b = a + seglen < L ? a + seglen : L;

    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;
    float m = kNegInf, s = 0.f;

    if (a < b) {
        float qf[8];
        {
            const uint4 qr = *reinterpret_cast<const uint4*>(q + r * D + c * 8);
            const uint32_t w[4] = {qr.x, qr.y, qr.z, qr.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                qf[2 * i] = bf16_lo(w[i]) * scale_log2;
                qf[2 * i + 1] = bf16_hi(w[i]) * scale_log2;
            }
        }
        const uint16_t* kr = k + r * L * D + c * 8;
        const uint16_t* vr = v + r * L * D + c * 8;
        for (int64_t j0 = a; j0 < b; j0 += KPW * U) {
            u32x4 kk[U], vv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                int64_t j = j0 + u * KPW + slot;
                j = j < b ? j : b - 1;  // masked below; the clamped row is valid
                kk[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kr + j * D));
                vv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vr + j * D));
            }
            float x[U];
            float mx = kNegInf;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t w[4] = {kk[u][0], kk[u][1], kk[u][2], kk[u][3]};
                float dot = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    dot = fmaf(qf[2 * i], bf16_lo(w[i]), dot);
                    dot = fmaf(qf[2 * i + 1], bf16_hi(w[i]), dot);
                }
                dot = LPK == 16 ? row16_sum(dot) : row8_sum(dot);
                x[u] = (j0 + u * KPW + slot < b) ? dot : kNegInf;
                mx = fmaxf(mx, x[u]);
            }
            const float m_new = fmaxf(m, mx);
            const float m_use = m_new == kNegInf ? 0.f : m_new;
            const float alpha = exp2_fast(m - m_use);
            s *= alpha;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] *= alpha;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float p = exp2_fast(x[u] - m_use);
                s += p;
                const uint32_t w[4] = {vv[u][0], vv[u][1], vv[u][2], vv[u][3]};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    o[2 * i] = fmaf(p, bf16_lo(w[i]), o[2 * i]);
                    o[2 * i + 1] = fmaf(p, bf16_hi(w[i]), o[2 * i + 1]);
                }
            }
            m = m_new;
        }
        // Merge the key slots: lanes with the same c and different slot.
#pragma unroll
        for (int mask = LPK; mask < 64; mask <<= 1) {
            const float m2 = __shfl_xor(m, mask, 64);
            const float s2 = __shfl_xor(s, mask, 64);
            const float M = fmaxf(m, m2);
            const float w1 = m == kNegInf ? 0.f : exp2_fast(m - M);
            const float w2 = m2 == kNegInf ? 0.f : exp2_fast(m2 - M);
            s = w1 * s + w2 * s2;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = w1 * o[e] + w2 * __shfl_xor(o[e], mask, 64);
            m = M;
        }
    }
    if constexpr (DIRECT) {
        if (slot == 0) {                      // L >= 1, so the single segment is never empty
            const float inv = 1.f / s;
            if (out_bf16) {
                uint4 w;
                w.x = pack_bf16x2(o[0] * inv, o[1] * inv);
                w.y = pack_bf16x2(o[2] * inv, o[3] * inv);
                w.z = pack_bf16x2(o[4] * inv, o[5] * inv);
                w.w = pack_bf16x2(o[6] * inv, o[7] * inv);
                *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + r * D + c * 8) = w;
            } else {
                float4* dst = reinterpret_cast<float4*>(static_cast<float*>(out) + r * D + c * 8);
                dst[0] = make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
                dst[1] = make_float4(o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv);
            }
            if (lse && c == 0) lse[r] = m * kLn2 + __logf(s);
        }
    } else if (slot == 0) {
        float4* dst = reinterpret_cast<float4*>(part_o + wid * D + c * 8);
        dst[0] = make_float4(o[0], o[1], o[2], o[3]);
        dst[1] = make_float4(o[4], o[5], o[6], o[7]);
        if (c == 0) {
            part_m[wid] = m == kNegInf ? kNegInf : m * kLn2;
            part_s[wid] = s;
        }
    }
}

// One wave per row. D = 512: lane l owns the column groups [4l + 256v, +4), v = 0, 1, so
// every 16-byte load instruction of the wave reads 1 KiB of contiguous partials. Smaller D:
// lane owns D/64 adjacent columns. For D = 512 and 128 the loads of four segments are
// issued before their products are added; each column adds the segments in segment order.
template <int D>
__global__ __launch_bounds__(256) void segment_merge_kernel(const float* __restrict__ part_m,
                                                            const float* __restrict__ part_s,
                                                            const float* __restrict__ part_o,
                                                            int64_t rows, int nseg, int out_bf16,
                                                            void* __restrict__ out, float* __restrict__ lse) {
    constexpr int PER = D / 64;
    constexpr bool GROUPED = PER % 4 == 0;    // column groups of 4 at a stride of 256
    constexpr int NV = GROUPED ? PER / 4 : 1;
    const int lane = threadIdx.x & 63;
    const int64_t r = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (r >= rows) return;
    const float* pm = part_m + r * nseg;
    const float* ps = part_s + r * nseg;
    const float* po = part_o + r * nseg * D + (GROUPED ? 4 * lane : lane * PER);

    float M = kNegInf;
    for (int t = lane; t < nseg; t += 64) M = fmaxf(M, pm[t]);
    M = wave_max(M);
    const float M2 = M * kLog2e;

    float S = 0.f, O[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) O[i] = 0.f;
    // O[4v + e] is column 4 * lane + 256 v + e when GROUPED, else column lane * PER + i.
    auto add_grouped = [&](float wt, const float4 (&x)[NV]) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            O[4 * v + 0] = fmaf(wt, x[v].x, O[4 * v + 0]);
            O[4 * v + 1] = fmaf(wt, x[v].y, O[4 * v + 1]);
            O[4 * v + 2] = fmaf(wt, x[v].z, O[4 * v + 2]);
            O[4 * v + 3] = fmaf(wt, x[v].w, O[4 * v + 3]);
        }
    };
    for (int t0 = 0; t0 < nseg; t0 += 64) {
        const int t = t0 + lane;
        float w = 0.f;
        if (t < nseg) {
            const float mt = pm[t];
            w = mt == kNegInf ? 0.f : exp2_fast(mt * kLog2e - M2);
            S += w * ps[t];
        }
        const int n = nseg - t0 < 64 ? nseg - t0 : 64;
        int tt = 0;
        constexpr int UB = 4;                     // segments whose loads are in flight together
        if constexpr (GROUPED) {
            for (; tt + UB <= n; tt += UB) {
                float4 x[UB][NV];
#pragma unroll
                for (int u = 0; u < UB; ++u)
#pragma unroll
                    for (int v = 0; v < NV; ++v)
                        x[u][v] = *reinterpret_cast<const float4*>(po + int64_t(t0 + tt + u) * D + 256 * v);
#pragma unroll
                for (int u = 0; u < UB; ++u) add_grouped(__shfl(w, tt + u, 64), x[u]);
            }
        } else if constexpr (PER == 2) {
            for (; tt + UB <= n; tt += UB) {
                float2 x[UB];
#pragma unroll
                for (int u = 0; u < UB; ++u) x[u] = *reinterpret_cast<const float2*>(po + int64_t(t0 + tt + u) * D);
#pragma unroll
                for (int u = 0; u < UB; ++u) {
                    const float wt = __shfl(w, tt + u, 64);
                    O[0] = fmaf(wt, x[u].x, O[0]);
                    O[1] = fmaf(wt, x[u].y, O[1]);
                }
            }
        }
        for (; tt < n; ++tt) {
            const float wt = __shfl(w, tt, 64);
            const float* src = po + int64_t(t0 + tt) * D;
            if constexpr (GROUPED) {
                float4 x[NV];
#pragma unroll
                for (int v = 0; v < NV; ++v) x[v] = *reinterpret_cast<const float4*>(src + 256 * v);
                add_grouped(wt, x);
            } else if constexpr (PER == 2) {
                const float2 x = *reinterpret_cast<const float2*>(src);
                O[0] = fmaf(wt, x.x, O[0]);
                O[1] = fmaf(wt, x.y, O[1]);
            } else {
                O[0] = fmaf(wt, src[0], O[0]);
            }
        }
    }
    S = wave_sum(S);
    const bool empty = !(S > 0.f);
    const float inv = empty ? 0.f : 1.f / S;
    if constexpr (GROUPED) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            float val[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) val[e] = empty ? 0.f : O[4 * v + e] * inv;
            const int64_t idx = r * D + 4 * lane + 256 * v;
            if (out_bf16)
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + idx) =
                    make_uint2(pack_bf16x2(val[0], val[1]), pack_bf16x2(val[2], val[3]));
            else
                *reinterpret_cast<float4*>(static_cast<float*>(out) + idx) = make_float4(val[0], val[1], val[2], val[3]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const float val = empty ? 0.f : O[i] * inv;
            const int64_t idx = r * D + lane * PER + i;
            if (out_bf16)
                static_cast<uint16_t*>(out)[idx] = uint16_t(f32_to_bf16_rne(val));
            else
                static_cast<float*>(out)[idx] = val;
        }
    }
    if (lse && lane == 0) lse[r] = empty ? kNegInf : M + __logf(S);
}

}  // namespace

hipError_t launch_decode_split(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t R,
                               int64_t L, int D, int64_t nseg, float scale, float* part_m,
                               float* part_s, float* part_o, hipStream_t stream) {
    const int64_t blocks = R * nseg;
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    const int64_t seglen = ceil_div(L, nseg);
    const float sl2 = scale * kLog2e;
    if (D == 128)
        hipLaunchKernelGGL((decode_split_kernel<128, 4>), dim3(unsigned(blocks)), dim3(64), 0, stream, q, k, v, L,
                           nseg, seglen, sl2, part_m, part_s, part_o);
    else
        hipLaunchKernelGGL((decode_split_kernel<64, 4>), dim3(unsigned(blocks)), dim3(64), 0, stream, q, k, v, L,
                           nseg, seglen, sl2, part_m, part_s, part_o);
    return hipGetLastError();
}

hipError_t launch_decode_direct(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t R, int64_t L, int D,
                                float scale, bool out_bf16, void* o, float* lse, hipStream_t stream) {
    if (R > INT32_MAX) return hipErrorInvalidValue;
    const float sl2 = scale * kLog2e;
    if (D == 128)
        hipLaunchKernelGGL((decode_split_kernel<128, 4, true>), dim3(unsigned(R)), dim3(64), 0, stream, q, k, v, L,
                           int64_t(1), L, sl2, nullptr, nullptr, nullptr, o, int(out_bf16), lse);
    else
        hipLaunchKernelGGL((decode_split_kernel<64, 4, true>), dim3(unsigned(R)), dim3(64), 0, stream, q, k, v, L,
                           int64_t(1), L, sl2, nullptr, nullptr, nullptr, o, int(out_bf16), lse);
    return hipGetLastError();
}

hipError_t launch_segment_merge(const float* part_m, const float* part_s, const float* part_o,
                                int64_t rows, int64_t nseg, int D, bool out_bf16, void* o, float* lse,
                                hipStream_t stream) {
    const int64_t blocks = ceil_div(rows, 4);
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    if (D == 512)
        hipLaunchKernelGGL(segment_merge_kernel<512>, dim3(unsigned(blocks)), dim3(256), 0, stream, part_m, part_s,
                           part_o, rows, int(nseg), int(out_bf16), o, lse);
    else if (D == 128)
        hipLaunchKernelGGL(segment_merge_kernel<128>, dim3(unsigned(blocks)), dim3(256), 0, stream, part_m, part_s,
                           part_o, rows, int(nseg), int(out_bf16), o, lse);
    else
        hipLaunchKernelGGL(segment_merge_kernel<64>, dim3(unsigned(blocks)), dim3(256), 0, stream, part_m, part_s,
                           part_o, rows, int(nseg), int(out_bf16), o, lse);
    return hipGetLastError();
}

}  // namespace rf
