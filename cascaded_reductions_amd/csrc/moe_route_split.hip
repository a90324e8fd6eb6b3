// MoE gate in two launches over a split hidden axis, kept beside the one-launch form
// (moe_route.hip) for comparison: scores = X W_gate -> top-k -> softmax over the k.
//
// The cascade of the explainer "RedFuser框架：AI加速器中的算子融合技术解析", section 4.2,
// with the hidden axis split into ranges (the Multi-Segment idea of the technical summary
// "RedFuser: An Automatic Operator Fusion Framework for Cascaded Reductions on AI
// Accelerators", Methodologie 3, applied to the GEMM's sum):
//  * workgroup (token block b, range r) stages W[range r] once in LDS, streams its 64
//    tokens' X[range r] straight into bf16 MFMA operands (v_mfma_f32_16x16x32_bf16; W
//    enters through the transposing LDS read, so the [Hd, E] layout needs no transpose in
//    memory), and writes a 64 x E partial score block to the workspace;
//  * a second launch adds each token's range partials in range order -- a fixed order, so
//    results are deterministic -- and runs the top-k and the softmax in registers: sixteen
//    lanes per token each keep a sorted top-k list over a sixteenth of the experts, merged
//    with four DPP steps (topk.hpp).
// Each CU reads only its range of W (64 KiB at 4096 x 64) instead of all of it, at the cost
// of the partial scores' round trip (4 MiB at 2048 tokens) and a second launch; the kernel
// boundary orders the two phases (the explainer's multi-kernel level, section 3.3).
// Experts are ranked by (score descending, index ascending).
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "topk.hpp"

namespace rf {
namespace {

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int TBM = 64;               // tokens per token block
constexpr int kLdsElems = 32768;      // W slice capacity (bf16 elements, 64 KiB)

struct MoeGeom {
    int64_t ntb, nranges;
    int hr;
    size_t part_bytes;
};

// Width of the hidden range one workgroup reduces: as wide as the 64 KiB LDS slice
// allows, at most 512 (16 MFMA K-chunks of 32).
constexpr int range_width(int E) { return (kLdsElems / E) / 32 * 32 < 512 ? (kLdsElems / E) / 32 * 32 : 512; }

MoeGeom moe_geom(int64_t T, int64_t Hd, int64_t E) {
    MoeGeom g;
    g.ntb = ceil_div(T, TBM);
    g.hr = range_width(int(E));
    g.nranges = ceil_div(Hd, g.hr);
    g.part_bytes = size_t(g.ntb * g.nranges * TBM * E * 4);
    return g;
}

__device__ __forceinline__ bf16x4_t lds_read_tr16(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)(p));
}

// Phase 1: partial scores of 64 tokens over one hidden range.
template <int NEB>
__global__ __launch_bounds__(256) void moe_partial_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ wg, int64_t T,
                                                          int64_t Hd, int hr, int64_t nranges, int swz,
                                                          float* __restrict__ part) {
    constexpr int E = NEB * 16;
    constexpr int CH = E / 8;         // 16-byte chunks per W row
    constexpr int NCH = range_width(E) / 32;   // K-chunks of a full range (the last range may be shorter)
    __shared__ __attribute__((aligned(16))) uint16_t wsm[kLdsElems];

    const int64_t tb = blockIdx.x / nranges;
    const int64_t rg = blockIdx.x - tb * nranges;
    const int64_t h0 = rg * hr;
    const int hlen = int(Hd - h0 < hr ? Hd - h0 : hr);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g = lane >> 4;

    // Issue every load of the workgroup before waiting on any: the W slice goes to LDS,
    // the X operands to registers.
    //
    // W[h0 .. h0 + hlen) is row-major [hd][E] in LDS with its 16-byte chunks swizzled
    // per row. When a row has a power-of-two number of chunks, direct global-to-LDS
    // loads fill it (one wave instruction = 1 KiB = 64 / CH rows; lane i lands in row
    // i / CH, physical chunk i % CH, so it fetches the logical chunk that maps there).
    if constexpr ((CH & (CH - 1)) == 0) {
        constexpr int RPW = 64 / CH;
        const int nwl = hlen / RPW;
        for (int wl = wave; wl < nwl; wl += 4) {
            const int r0 = wl * RPW;
            const int row = r0 + lane / CH;
            const int ch = (lane % CH) ^ (((row & 3) << 1) & swz);
            lds_dma16(wg + (h0 + row) * E + ch * 8, &wsm[r0 * E]);
        }
    } else {
        for (int i0 = 0; i0 < hlen * CH; i0 += 8 * 256) {
            u32x4 val[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = i0 + u * 256 + tid;
                if (i < hlen * CH) {
                    const int row = i / CH, ch = i - row * CH;
                    val[u] = *reinterpret_cast<const u32x4*>(wg + (h0 + row) * E + ch * 8);
                }
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = i0 + u * 256 + tid;
                if (i < hlen * CH) {
                    const int row = i / CH, ch = i - row * CH;
                    *reinterpret_cast<u32x4*>(&wsm[row * E + ch * 8]) = val[u];   // no swizzle (swz = 0)
                }
            }
        }
    }

    // A operand: lane (token l16 of this wave's 16, group g) holds X[token][h0 + 32c + 8g .. +7].
    int64_t tok = tb * TBM + 16 * wave + l16;
    tok = tok < T ? tok : T - 1;
    const uint16_t* xr = x + tok * Hd + h0 + 8 * g;
    const int nc = hlen / 32;                 // <= NCH
    u32x4 xa[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int cc = c < nc ? c : nc - 1;   // the tail range re-reads its last chunk (unused)
        xa[c] = *reinterpret_cast<const u32x4*>(xr + 32 * cc);
    }

    f32x4 acc[NEB];
#pragma unroll
    for (int b = 0; b < NEB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Only the W slice must be complete before the barrier: the X loads were issued after
    // it, so waiting until NCH loads remain leaves exactly the X chunks in flight. Chunk c
    // of X is then waited for just before its MFMAs (the compiler counts those loads), so
    // the matrix work on the first chunks overlaps the arrival of the later ones. (The W
    // loads are issued through inline assembly, which keeps the compiler from waiting for
    // every load before the first LDS read.)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NCH) : "memory");
    __syncthreads();

    const int j = l16;
    // Full ranges take a loop without a chunk test (so no load is sunk below the
    // barrier); only the last, shorter range skips the chunks past its end.
    auto mfma_chunks = [&](auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            if (!FULL && c >= nc) continue;
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
                acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[c]),
                                                                  __builtin_bit_cast(bf16x8, wb), acc[b], 0, 0, 0);
            }
        }
    };
    if (nc == NCH) mfma_chunks(std::true_type{});
    else mfma_chunks(std::false_type{});

    // acc[b][r] = partial score of token (16*wave + 4g + r) for expert 16b + l16.
    float* pblk = part + ((tb * nranges + rg) * TBM) * E;
#pragma unroll
    for (int b = 0; b < NEB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) pblk[(16 * wave + 4 * g + r) * E + 16 * b + l16] = acc[b][r];

}

// Phase 2: sixteen lanes per token (4 tokens per wave, one wave per workgroup, so 2048
// tokens spread over 512 workgroups); lane q of a token owns experts [q * NEB, q * NEB + NEB).
constexpr int RED_T = 64;             // threads per reduce workgroup

template <int NEB, int K>
__global__ __launch_bounds__(RED_T) void moe_reduce_kernel(const float* __restrict__ part, int64_t T, int64_t nranges,
                                                         int k, int32_t* __restrict__ idx, float* __restrict__ wout,
                                                         float* __restrict__ scores) {
    constexpr int E = NEB * 16;
    const int tid = threadIdx.x;
    const int q = tid & 15;
    const int64_t t_out = int64_t(blockIdx.x) * (RED_T / 16) + (tid >> 4);
    const bool valid = t_out < T;
    uint64_t list[K];
    topk::clear<K>(list);
    if (valid) {
        // Sum the range partials in range order (deterministic), loading RB ranges' worth
        // of this lane's experts before adding, so the loads overlap.
        const int64_t tb = t_out / TBM;
        const int64_t tl = t_out - tb * TBM;
        const float* base = part + (tb * nranges * TBM + tl) * E + q * NEB;
        constexpr int RB = NEB >= 8 ? 4 : 8;
        float sum[NEB];
#pragma unroll
        for (int e = 0; e < NEB; ++e) sum[e] = 0.f;
        for (int64_t r0 = 0; r0 < nranges; r0 += RB) {
            float buf[RB][NEB];
#pragma unroll
            for (int rr = 0; rr < RB; ++rr)
                if (r0 + rr < nranges)
#pragma unroll
                    for (int e = 0; e < NEB; ++e) buf[rr][e] = base[(r0 + rr) * TBM * E + e];
#pragma unroll
            for (int rr = 0; rr < RB; ++rr)
                if (r0 + rr < nranges)
#pragma unroll
                    for (int e = 0; e < NEB; ++e) sum[e] += buf[rr][e];
        }
#pragma unroll
        for (int e = 0; e < NEB; ++e) {
            if (scores) scores[t_out * E + q * NEB + e] = sum[e];
            topk::insert<K>(list, topk::make_key(sum[e], q * NEB + e));
        }
    }
    // Merge the sixteen lanes' lists of a token (one DPP row; a row is wholly valid or not).
    topk::merge_row16<K>(list);
    // Every lane of the row now holds the K best; the first k (k <= K) are the output, and
    // the softmax runs over exactly those k scores.
    if (valid && q == 0) topk::write_softmax<K>(list, k, idx + t_out * k, wout + t_out * k);
}

template <int NEB>
hipError_t launch_e(int k, const MoeGeom& g, int swz, hipStream_t stream, const uint16_t* x, const uint16_t* w,
                    int64_t T, int64_t Hd, int32_t* idx, float* wout, float* scores, float* part) {
    const dim3 grid1{unsigned(g.ntb * g.nranges), 1u, 1u};
    hipLaunchKernelGGL((moe_partial_kernel<NEB>), grid1, dim3(256), 0, stream, x, w, T, Hd, g.hr, g.nranges, swz,
                       part);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 grid2{unsigned(ceil_div(T, int64_t(RED_T / 16))), 1u, 1u};
    // A top-2 fast path; any other k up to 8 keeps an 8-entry list.
    if (k == 2)
        hipLaunchKernelGGL((moe_reduce_kernel<NEB, 2>), grid2, dim3(RED_T), 0, stream, part, T, g.nranges, k, idx, wout,
                           scores);
    else
        hipLaunchKernelGGL((moe_reduce_kernel<NEB, 8>), grid2, dim3(RED_T), 0, stream, part, T, g.nranges, k, idx, wout,
                           scores);
    return hipGetLastError();
}

}  // namespace

size_t moe_split_workspace_bytes(int64_t T, int64_t Hd, int64_t E) {
    return moe_geom(T, Hd, E).part_bytes;
}

hipError_t launch_moe_route_split(const uint16_t* x, const uint16_t* w_gate, int64_t T, int64_t Hd, int E, int k,
                                  int32_t* idx, float* w, float* scores, void* workspace, hipStream_t stream) {
    const MoeGeom g = moe_geom(T, Hd, E);
    if (g.ntb * g.nranges > INT32_MAX || ceil_div(T, int64_t(RED_T / 16)) > INT32_MAX) return hipErrorInvalidValue;
    const int CH = E / 8;
    const int swz = (CH >= 8 && (CH & (CH - 1)) == 0) ? 6 : 0;
    float* part = static_cast<float*>(workspace);
#define RF_MOE_E(NB) \
    case NB: return launch_e<NB>(k, g, swz, stream, x, w_gate, T, Hd, idx, w, scores, part);
    switch (E / 16) {
        RF_MOE_E(1) RF_MOE_E(2) RF_MOE_E(3) RF_MOE_E(4) RF_MOE_E(5) RF_MOE_E(6) RF_MOE_E(7) RF_MOE_E(8)
        RF_MOE_E(9) RF_MOE_E(10) RF_MOE_E(11) RF_MOE_E(12) RF_MOE_E(13) RF_MOE_E(14) RF_MOE_E(15) RF_MOE_E(16)
        default: return hipErrorInvalidValue;
    }
#undef RF_MOE_E
}

}  // namespace rf
