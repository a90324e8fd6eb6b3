// Fused MoE gate in one kernel: scores = X W_gate -> top-k -> softmax over the k selected.
//
// The cascade of the explainer "RedFuser框架：AI加速器中的算子融合技术解析", section 4.2,
// as a single kernel that never stores the score matrix (only the optional debug copy
// is written). Experts are ranked by (score descending, index ascending).
//
// Each workgroup owns TB = 8 tokens and all E experts, so no workgroup depends on
// another (no partial scores leave the chip and no second launch is needed):
//  * its NW waves (8 up to E = 64, 4 above) split the hidden axis into contiguous shares
//    and stream their share of W_gate ([32 hidden x E] bf16 chunks) and of the 8 tokens'
//    X through wave-private LDS rings filled by direct global-to-LDS loads a few chunks
//    ahead (none past the end of the share), so every wave runs without barriers until
//    the end; two waves per SIMD keep one wave's loads in flight while the other computes;
//  * the gate GEMM runs on v_mfma_f32_16x16x32_bf16 with the tokens as the M dimension
//    (8 of 16 rows used) and W entering through the transposing LDS read, so the [Hd, E]
//    layout needs no transpose in memory;
//  * the waves' partial scores are added through LDS in a fixed order (deterministic),
//    then sixteen lanes per token keep sorted top-k lists over a sixteenth of the experts,
//    merged by four DPP steps (topk.hpp), and the first lane applies the softmax.
// Every workgroup reads the whole W_gate (E * Hd * 2 bytes, 0.5 MiB at 4096 x 64) from its
// XCD's L2 and X once; the per-CU rate of those L2 reads bounds the kernel (the two-launch
// form in moe_route_split.hip reads a range of W per CU instead, and exchanges partials).
#include "common.hpp"
#include "launch.hpp"
#include "topk.hpp"

namespace rf {
namespace {

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int TB = 8;                 // tokens per workgroup

// Waves per workgroup: two per SIMD while a wave's ring (20 KiB of LDS) still holds a
// chunk pair in flight beside the one being used, one per SIMD (36 KiB rings) above.
constexpr int waves_for(int E) { return E <= 64 ? 8 : 4; }

__device__ __forceinline__ bf16x4_t lds_read_tr16(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)(p));
}

// Ring geometry for E experts: a W chunk is 32 hidden rows x E bf16 (E / 16 KiB), an X
// chunk pair is the 8 tokens x 64 hidden values (1 KiB). DEPTH chunk slots per wave, of
// which DEPTH / 2 - 1 pairs are in flight ahead of the pair in use.
template <int NEB>
struct Ring {
    static constexpr int E = NEB * 16;
    static constexpr int NW = waves_for(E);
    static constexpr int WAVE_LDS = NW == 8 ? 20 * 1024 : 36 * 1024;
    static constexpr int WCH = 64 * E;                       // bytes of one W chunk
    static constexpr int WLOADS = WCH / 1024;                // wave loads per W chunk
    static constexpr int DEPTH0 = (WAVE_LDS - 4096) / WCH;   // W slots that fit beside the X slots
    static constexpr int DEPTH = DEPTH0 >= 8 ? 8 : DEPTH0 >= 4 ? 4 : 2;   // power of two
    static constexpr int XPAIRS = DEPTH / 2;                 // X slots (one per chunk pair)
    static constexpr int AHEAD = DEPTH / 2 - 1;
    static_assert(DEPTH * WCH + XPAIRS * 1024 <= WAVE_LDS, "the wave's ring must fit its LDS share");
    static_assert(NW * WAVE_LDS <= 160 * 1024, "the rings must fit the CU's LDS");
    static constexpr int PSTRIDE = E + 16;                   // floats per partial-score row
    static_assert(NW * TB * PSTRIDE * 4 <= NW * WAVE_LDS, "the partial scores reuse the rings");
};

// Wait until the loads of the pair in use have landed, with `left` more pairs of this wave
// issued after it (left >= N: N pairs; the wait count must be an immediate).
template <int N, int LPS>
__device__ __forceinline__ void wait_pairs(int left) {
    if constexpr (N == 0) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
        if (left >= N) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N * LPS) : "memory");
        else wait_pairs<N - 1, LPS>(left);
    }
}

template <int NEB, int K>
__global__ __launch_bounds__(Ring<NEB>::NW * 64) void moe_gate_kernel(const uint16_t* __restrict__ x,
                                                              const uint16_t* __restrict__ wg, int64_t T,
                                                              int64_t Hd, int k, int swz, int32_t* __restrict__ idx,
                                                              float* __restrict__ wout, float* __restrict__ scores) {
    using R = Ring<NEB>;
    constexpr int E = R::E;
    constexpr int NW = R::NW;
    constexpr int DEPTH = R::DEPTH;
    constexpr int LPS = 2 * R::WLOADS + 1;    // direct loads per chunk pair (two W chunks + one X pair)
    __shared__ __attribute__((aligned(16))) unsigned char smem[NW * R::WAVE_LDS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g = lane >> 4;
    const int64_t t0 = int64_t(blockIdx.x) * TB;

    unsigned char* const ring = smem + wave * R::WAVE_LDS;
    unsigned char* const wslots = ring;                       // DEPTH x WCH
    unsigned char* const xslots = ring + DEPTH * R::WCH;      // XPAIRS x 1 KiB

    // This wave's contiguous share of the hidden axis, in 32-wide chunks, taken in pairs.
    const int64_t nch = Hd / 32;
    const int64_t per = (nch + NW - 1) / NW;
    const int64_t c_begin = wave * per < nch ? wave * per : nch;
    const int64_t c_end = c_begin + per < nch ? c_begin + per : nch;
    const int my = int(c_end - c_begin);      // chunks of this wave (wave-uniform)
    const int npairs = (my + 1) / 2;

    // X pair loads: lane i fetches token i / 8 (clamped to T - 1), 16 bytes of its 128-byte row of
    // the pair's 64 hidden values; it lands at physical piece (i % 8) of token row i / 8, so it
    // fetches the logical piece (i % 8) ^ (token & 7). The wave-uniform base is token t0's row.
    const int xt = lane >> 3;
    int64_t xtok = t0 + xt;
    xtok = xtok < T ? xtok : T - 1;
    const int64_t tb0 = t0 < T ? t0 : T - 1;
    const int x_lp = ((lane & 7) ^ xt) & 7;   // the logical piece this lane fetches
    const uint32_t x_row = uint32_t((xtok - tb0) * Hd * 2);   // < 2^32: the host bounds Hd below 2^26
    const uint16_t* xw = x + tb0 * Hd;        // wave-uniform
    // W chunk loads: lane i of wave load l lands in chunk row (l * 1024 + 16 i) / (2E), physical
    // 16-byte chunk ((l * 1024 + 16 i) % (2E)) / 16, and fetches the logical chunk mapped there.
    uint32_t w_lane[R::WLOADS];
#pragma unroll
    for (int l = 0; l < R::WLOADS; ++l) {
        const int byte = l * 1024 + 16 * lane;
        const int row = byte / (2 * E);
        const int pc = (byte % (2 * E)) / 16;
        const int lc = pc ^ (((row & 3) << 1) & swz);
        w_lane[l] = uint32_t(row * E * 2 + lc * 16);
    }
    auto issue_pair = [&](int p) {            // chunks 2p and 2p + 1 of this wave (p < npairs)
        const int64_t c0 = c_begin + 2 * p;
        const uint32_t xs = lds_addr(xslots) + uint32_t((p % R::XPAIRS) * 1024);
        // A pair whose second chunk is past the hidden axis (an odd chunk count) fetches the
        // first chunk's pieces in its place (unused), so no load runs past the end of X.
        const int lp = (c0 + 1 >= nch && x_lp >= 4) ? x_lp - 4 : x_lp;
        lds_dma16_sb(xw, x_row + uint32_t(c0 * 64 + lp * 16), xs);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            int64_t c = c0 + h;
            c = c < c_end ? c : c_end - 1;    // the odd tail re-reads the last chunk (unused)
            const uint16_t* wsrc = wg + c * 32 * E;
            const uint32_t ws = lds_addr(wslots) + uint32_t(((2 * p + h) % DEPTH) * R::WCH);
#pragma unroll
            for (int l = 0; l < R::WLOADS; ++l) lds_dma16_sb(wsrc, w_lane[l], ws + uint32_t(l * 1024));
        }
    };

    f32x4 acc[NEB];
#pragma unroll
    for (int b = 0; b < NEB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};

    // B operand offsets: lane (expert l16 of block b, group g) holds W[8g + e][16b + l16], read
    // as rows 8g + j/4 and 8g + 4 + j/4, columns 16b + 4(j%4) .. +3 of a 16-lane group (j = l16).
    int b_off[NEB][2];
#pragma unroll
    for (int b = 0; b < NEB; ++b) {
        const int r0 = 8 * g + (l16 >> 2), r1 = r0 + 4;
        const int col = 16 * b + 4 * (l16 & 3);
        b_off[b][0] = r0 * E + ((((col >> 3) ^ (((r0 & 3) << 1) & swz))) << 3) + (col & 7);
        b_off[b][1] = r1 * E + ((((col >> 3) ^ (((r1 & 3) << 1) & swz))) << 3) + (col & 7);
    }
    // A operand: lane (token l16 & 7, group g) reads the 8 hidden values 32h + 8g .. +7 of its token
    // (h = the chunk within the pair): logical piece 4h + g of the token's row. Rows 8..15 of the
    // 16-row MFMA repeat tokens 0..7; their results are not used.
    const int at = l16 & 7;
    const int a_off[2] = {at * 128 + ((((0 + g) ^ at) & 7) * 16), at * 128 + ((((4 + g) ^ at) & 7) * 16)};

    // Prologue: up to AHEAD pairs in flight. No load is issued past the wave's last pair, so
    // the last AHEAD waits count fewer pairs. (A wave with no chunks, when the hidden axis has
    // fewer chunks than waves, loads nothing and contributes zeros.)
#pragma unroll
    for (int p = 0; p < R::AHEAD; ++p)
        if (p < npairs) issue_pair(p);
    for (int p = 0; p < npairs; ++p) {
        if (p + R::AHEAD < npairs) issue_pair(p + R::AHEAD);   // into the slots pair p - 1 used
        wait_pairs<R::AHEAD, LPS>(npairs - 1 - p);             // pair p is in
        const unsigned char* xs = xslots + (p % R::XPAIRS) * 1024;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if (2 * p + h < my) {
                const uint16_t* ws = reinterpret_cast<const uint16_t*>(wslots + ((2 * p + h) % DEPTH) * R::WCH);
                const bf16x8 xa = *reinterpret_cast<const bf16x8*>(xs + a_off[h]);
#pragma unroll
                for (int b = 0; b < NEB; ++b) {
                    const bf16x4_t lo = lds_read_tr16(ws + b_off[b][0]);
                    const bf16x4_t hi = lds_read_tr16(ws + b_off[b][1]);
                    const bf16x8_t wb = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, __builtin_bit_cast(bf16x8, wb), acc[b], 0, 0,
                                                                      0);
                }
            }
        }
    }

    // acc[b][r] = partial score of token 4g + r (g < 2: tokens 0..7) for expert 16b + l16. The
    // waves' partials meet in LDS ([wave][token][expert] fp32, rows padded to E + 16 floats so
    // the four tokens a wave reads below sit in different banks; the rings are free after the
    // barrier) and are added in wave order.
    constexpr int PS = R::PSTRIDE;
    __syncthreads();
    float* part = reinterpret_cast<float*>(smem);
    if (g < 2) {
#pragma unroll
        for (int b = 0; b < NEB; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) part[(wave * TB + 4 * g + r) * PS + 16 * b + l16] = acc[b][r];
    }
    __syncthreads();

    // Sixteen lanes per token, one DPP row each (waves 0 and 1: 128 threads for 8 tokens); lane
    // q of a token owns experts q, q + 16, ..., q + 16 (NEB - 1).
    if (tid >= TB * 16) return;               // whole waves only: no barrier follows
    const int tok = tid >> 4, q = tid & 15;
    const int64_t t_out = t0 + tok;
    uint64_t list[K];
    topk::clear<K>(list);
#pragma unroll
    for (int e = 0; e < NEB; ++e) {
        const int ex = 16 * e + q;
        float s = part[tok * PS + ex];
#pragma unroll
        for (int w = 1; w < NW; ++w) s += part[(w * TB + tok) * PS + ex];
        if (scores && t_out < T) scores[t_out * E + ex] = s;
        topk::insert<K>(list, topk::make_key(s, ex));
    }
    topk::merge_row16<K>(list);
    // Every lane of the row now holds the K best; the first k (k <= K) are the output, and the
    // softmax runs over exactly those k scores.
    if (t_out < T && q == 0) topk::write_softmax<K>(list, k, idx + t_out * k, wout + t_out * k);
}

template <int NEB>
hipError_t launch_e(int k, int swz, hipStream_t stream, const uint16_t* x, const uint16_t* w, int64_t T, int64_t Hd,
                    int32_t* idx, float* wout, float* scores) {
    const dim3 grid{unsigned(ceil_div(T, TB)), 1u, 1u};
    // A top-2 fast path; any other k up to 8 keeps an 8-entry list.
    if (k == 2)
        hipLaunchKernelGGL((moe_gate_kernel<NEB, 2>), grid, dim3(Ring<NEB>::NW * 64), 0, stream, x, w, T, Hd, k, swz, idx, wout,
                           scores);
    else
        hipLaunchKernelGGL((moe_gate_kernel<NEB, 8>), grid, dim3(Ring<NEB>::NW * 64), 0, stream, x, w, T, Hd, k, swz, idx, wout,
                           scores);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_moe_route(const uint16_t* x, const uint16_t* w_gate, int64_t T, int64_t Hd, int E, int k,
                            int32_t* idx, float* w, float* scores, hipStream_t stream) {
    if (ceil_div(T, TB) > INT32_MAX) return hipErrorInvalidValue;
    const int CH = E / 8;
    // Swizzle the W chunks only when a row has a power-of-two count (>= 8) of 16-byte chunks.
    const int swz = (CH >= 8 && (CH & (CH - 1)) == 0) ? 6 : 0;
#define RF_MOE_E(NB) \
    case NB: return launch_e<NB>(k, swz, stream, x, w_gate, T, Hd, idx, w, scores);
    switch (E / 16) {
        RF_MOE_E(1) RF_MOE_E(2) RF_MOE_E(3) RF_MOE_E(4) RF_MOE_E(5) RF_MOE_E(6) RF_MOE_E(7) RF_MOE_E(8)
        RF_MOE_E(9) RF_MOE_E(10) RF_MOE_E(11) RF_MOE_E(12) RF_MOE_E(13) RF_MOE_E(14) RF_MOE_E(15) RF_MOE_E(16)
        default: return hipErrorInvalidValue;
    }
#undef RF_MOE_E
}

}  // namespace rf
