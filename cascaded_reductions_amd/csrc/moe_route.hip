// Fused MoE gate: scores = X W_gate -> top-k -> softmax over the k selected.
//
// The cascade of the explainer "RedFuser框架：AI加速器中的算子融合技术解析",
// section 4.2, in one launch; the score matrix is never written (except as an
// optional debug output).
//
// The gate GEMM reads X once (16.8 MB at 2048 x 4096) but every token needs the
// whole W_gate, so a kernel that gives each workgroup a few tokens and all of
// the hidden axis would stream W through every CU. Instead the hidden axis is
// split into ranges (the Multi-Segment idea of the technical summary
// "RedFuser: An Automatic Operator Fusion Framework for Cascaded Reductions on
// AI Accelerators", Methodologie 3, applied to the GEMM's sum):
//  * workgroup (token block b, range r) stages W[range r] once in LDS, streams
//    its 64 tokens' X[range r] straight into bf16 MFMA operands
//    (v_mfma_f32_16x16x32_bf16; W enters through the transposing LDS read, so
//    the [Hd, E] layout needs no transpose in memory), and writes a 64 x E
//    partial score block to the workspace;
//  * the last workgroup to finish a token block (a per-block counter) adds the
//    partial blocks in range order -- a fixed order, so results are
//    deterministic -- and runs the top-k and the softmax in registers: four
//    lanes per token each keep a sorted top-k list over a quarter of the
//    experts, merged with two cross-lane steps. It then resets the counter.
// Experts are ranked by (score descending, index ascending).
#include "common.hpp"
#include "launch.hpp"

namespace rf {
namespace {

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int TBM = 64;               // tokens per token block
constexpr int kLdsElems = 32768;      // W slice capacity (bf16 elements, 64 KiB)

struct MoeGeom {
    int64_t ntb, nranges;
    int hr;
    size_t cnt_bytes, part_bytes;
};

MoeGeom moe_geom(int64_t T, int64_t Hd, int64_t E) {
    MoeGeom g;
    g.ntb = ceil_div(T, TBM);
    int hr = int(kLdsElems / E) / 32 * 32;
    if (hr > 512) hr = 512;
    while (hr > 128 && g.ntb * ceil_div(Hd, hr) < 256) hr = hr / 2 / 32 * 32;
    g.hr = hr;
    g.nranges = ceil_div(Hd, hr);
    g.cnt_bytes = size_t(ceil_div(g.ntb * 4, 256) * 256);
    g.part_bytes = size_t(g.ntb * g.nranges * TBM * E * 4);
    return g;
}

__device__ __forceinline__ bf16x4_t lds_read_tr16(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)(p));
}

// (s1, i1) ranks before (s2, i2).
__device__ __forceinline__ bool better(float s1, int i1, float s2, int i2) {
    return s1 > s2 || (s1 == s2 && i1 < i2);
}

// Insert (s, i) into the sorted list (ts, ti) of length K (descending rank).
template <int K>
__device__ __forceinline__ void topk_insert(float (&ts)[K], int (&ti)[K], float s, int i) {
#pragma unroll
    for (int r = 0; r < K; ++r) {
        if (better(s, i, ts[r], ti[r])) {
            const float s2 = ts[r];
            const int i2 = ti[r];
            ts[r] = s;
            ti[r] = i;
            s = s2;
            i = i2;
        }
    }
}

template <int NEB, int K>
__global__ __launch_bounds__(256) void moe_route_kernel(const uint16_t* __restrict__ x,
                                                        const uint16_t* __restrict__ wg, int64_t T,
                                                        int64_t Hd, int hr, int64_t nranges, int swz, int k,
                                                        int32_t* __restrict__ idx, float* __restrict__ wout,
                                                        float* __restrict__ scores, unsigned* __restrict__ cnt,
                                                        float* __restrict__ part) {
    constexpr int E = NEB * 16;
    constexpr int CH = E / 8;         // 16-byte chunks per W row
    __shared__ __attribute__((aligned(16))) uint16_t wsm[kLdsElems];
    __shared__ int sm_last;

    const int64_t tb = blockIdx.x / nranges;
    const int64_t rg = blockIdx.x - tb * nranges;
    const int64_t h0 = rg * hr;
    const int hlen = int(Hd - h0 < hr ? Hd - h0 : hr);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g = lane >> 4;

    // Stage W[h0 .. h0 + hlen) (row-major [hd][E]) in LDS; 16-byte chunks swizzled per row.
    for (int i = tid; i < hlen * CH; i += 256) {
        const int row = i / CH, ch = i - row * CH;
        const u32x4 val = *reinterpret_cast<const u32x4*>(wg + (h0 + row) * E + ch * 8);
        const int pc = ch ^ (((row & 3) << 1) & swz);
        *reinterpret_cast<u32x4*>(&wsm[row * E + pc * 8]) = val;
    }

    // A operand: lane (token l16 of this wave's 16, group g) holds X[token][h0 + 32c + 8g .. +7].
    int64_t tok = tb * TBM + 16 * wave + l16;
    tok = tok < T ? tok : T - 1;
    const uint16_t* xr = x + tok * Hd + h0 + 8 * g;
    f32x4 acc[NEB];
#pragma unroll
    for (int b = 0; b < NEB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    __syncthreads();

    const int nc = hlen / 32;
    const int j = l16;
    for (int c0 = 0; c0 < nc; c0 += 8) {
        u32x4 xa[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (c0 + u < nc) xa[u] = *reinterpret_cast<const u32x4*>(xr + 32 * (c0 + u));
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (c0 + u >= nc) break;
            const int c = c0 + u;
            // B operand: lane (expert l16 of block b, group g) holds W[32c + 8g + e][16b + l16];
            // group lane j reads rows 32c + 8g + j/4 (+4), columns 16b + 4(j%4) .. +3.
            const int r0 = 32 * c + 8 * g + (j >> 2);
            const int r1 = r0 + 4;
#pragma unroll
            for (int b = 0; b < NEB; ++b) {
                const int col = 16 * b + 4 * (j & 3);
                const int p0 = r0 * E + ((((col >> 3) ^ (((r0 & 3) << 1) & swz))) << 3) + (col & 7);
                const int p1 = r1 * E + ((((col >> 3) ^ (((r1 & 3) << 1) & swz))) << 3) + (col & 7);
                const bf16x4_t lo = lds_read_tr16(wsm + p0);
                const bf16x4_t hi = lds_read_tr16(wsm + p1);
                const bf16x8_t wb = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[u]),
                                                                  __builtin_bit_cast(bf16x8, wb), acc[b], 0, 0, 0);
            }
        }
    }

    // acc[b][r] = partial score of token (16*wave + 4g + r) for expert 16b + l16.
    float* pblk = part + ((tb * nranges + rg) * TBM) * E;
#pragma unroll
    for (int b = 0; b < NEB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) pblk[(16 * wave + 4 * g + r) * E + 16 * b + l16] = acc[b][r];

    // Publish the partial block; the last workgroup of this token block reduces.
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const unsigned old = atomicAdd(&cnt[tb], 1u);
        sm_last = old == unsigned(nranges - 1);
    }
    __syncthreads();
    if (!sm_last) return;
    __threadfence();

    // Reduction: wave w handles tokens 16w .. 16w + 15; four lanes per token, each
    // owning a contiguous quarter of the experts.
    constexpr int EQ = E / 4;
    const int tt = lane >> 2, qq = lane & 3;
    const int tl = 16 * wave + tt;
    const int64_t t_out = tb * TBM + tl;
    const bool valid = t_out < T;
    float ts[K];
    int ti[K];
#pragma unroll
    for (int r = 0; r < K; ++r) {
        ts[r] = kNegInf;
        ti[r] = 0x7FFFFFFF;
    }
    if (valid) {
        const float* base = part + (tb * nranges * TBM + tl) * E + qq * EQ;
#pragma unroll
        for (int e4 = 0; e4 < EQ; e4 += 4) {
            float4 s4 = *reinterpret_cast<const float4*>(base + e4);
            for (int64_t r = 1; r < nranges; ++r) {
                const float4 p4 = *reinterpret_cast<const float4*>(base + r * TBM * E + e4);
                s4.x += p4.x;
                s4.y += p4.y;
                s4.z += p4.z;
                s4.w += p4.w;
            }
            if (scores) *reinterpret_cast<float4*>(scores + t_out * E + qq * EQ + e4) = s4;
            const int e0 = qq * EQ + e4;
            topk_insert<K>(ts, ti, s4.x, e0);
            topk_insert<K>(ts, ti, s4.y, e0 + 1);
            topk_insert<K>(ts, ti, s4.z, e0 + 2);
            topk_insert<K>(ts, ti, s4.w, e0 + 3);
        }
    }
    // Merge the four lanes' lists (lanes differing in bits 0 and 1).
#pragma unroll
    for (int mask = 1; mask <= 2; mask <<= 1) {
        float os[K];
        int oi[K];
#pragma unroll
        for (int r = 0; r < K; ++r) {
            os[r] = __shfl_xor(ts[r], mask, 64);
            oi[r] = __shfl_xor(ti[r], mask, 64);
        }
#pragma unroll
        for (int r = 0; r < K; ++r) topk_insert<K>(ts, ti, os[r], oi[r]);
    }
    // The list holds the K best; the first k (k <= K) are the output, and the
    // softmax runs over exactly those k scores.
    if (valid && qq == 0) {
        float den = 0.f;
        float ex[K];
#pragma unroll
        for (int r = 0; r < K; ++r) {
            ex[r] = r < k ? __expf(ts[r] - ts[0]) : 0.f;
            den += ex[r];
        }
        const float inv = 1.f / den;
#pragma unroll
        for (int r = 0; r < K; ++r) {
            if (r < k) {
                idx[t_out * k + r] = ti[r];
                wout[t_out * k + r] = ex[r] * inv;
            }
        }
    }
    if (tid == 0) cnt[tb] = 0u;   // every other workgroup of this block has already counted
}

template <int NEB>
hipError_t launch_e(int k, dim3 grid, hipStream_t stream, const uint16_t* x, const uint16_t* w, int64_t T, int64_t Hd,
                    int hr, int64_t nranges, int swz, int32_t* idx, float* wout, float* scores, unsigned* cnt,
                    float* part) {
    // A top-2 fast path; any other k up to 8 keeps an 8-entry list.
    if (k == 2)
        hipLaunchKernelGGL((moe_route_kernel<NEB, 2>), grid, dim3(256), 0, stream, x, w, T, Hd, hr, nranges, swz, k,
                           idx, wout, scores, cnt, part);
    else
        hipLaunchKernelGGL((moe_route_kernel<NEB, 8>), grid, dim3(256), 0, stream, x, w, T, Hd, hr, nranges, swz, k,
                           idx, wout, scores, cnt, part);
    return hipGetLastError();
}

}  // namespace

size_t moe_workspace_bytes(int64_t T, int64_t Hd, int64_t E) {
    const MoeGeom g = moe_geom(T, Hd, E);
    return g.cnt_bytes + g.part_bytes;
}

hipError_t launch_moe_route(const uint16_t* x, const uint16_t* w_gate, int64_t T, int64_t Hd, int E, int k,
                            int32_t* idx, float* w, float* scores, void* workspace, hipStream_t stream) {
    const MoeGeom g = moe_geom(T, Hd, E);
    const int64_t blocks = g.ntb * g.nranges;
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    const int CH = E / 8;
    const int swz = (CH >= 8 && (CH & (CH - 1)) == 0) ? 6 : 0;
    unsigned* cnt = static_cast<unsigned*>(workspace);
    float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + g.cnt_bytes);
    const dim3 grid{unsigned(blocks), 1u, 1u};
#define RF_MOE_E(NB) \
    case NB: return launch_e<NB>(k, grid, stream, x, w_gate, T, Hd, g.hr, g.nranges, swz, idx, w, scores, cnt, part);
    switch (E / 16) {
        RF_MOE_E(1) RF_MOE_E(2) RF_MOE_E(3) RF_MOE_E(4) RF_MOE_E(5) RF_MOE_E(6) RF_MOE_E(7) RF_MOE_E(8)
        RF_MOE_E(9) RF_MOE_E(10) RF_MOE_E(11) RF_MOE_E(12) RF_MOE_E(13) RF_MOE_E(14) RF_MOE_E(15) RF_MOE_E(16)
        default: return hipErrorInvalidValue;
    }
#undef RF_MOE_E
}

}  // namespace rf
