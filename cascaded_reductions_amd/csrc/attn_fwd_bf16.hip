// Single-segment fused attention, bf16 inputs, on the bf16 matrix cores.
//
// The softmax -> GEMM cascade (explainer "RedFuser框架：AI加速器中的算子融合技术解析",
// sections 2.2 and 4.1) in its incremental form (section 2.3; technical summary
// "RedFuser: An Automatic Operator Fusion Framework for Cascaded Reductions on AI
// Accelerators", Methodologie 2): one workgroup owns a block of query rows and
// walks the whole key axis (Single-Segment strategy, Methodologie 3), keeping
// per row a reference maximum, a running sum of exponentials and an
// unnormalised output accumulator; O = o~ / s is formed once at the end.
//
// gfx950 mapping (wave64, v_mfma_f32_32x32x16_bf16, 32 query rows per wave):
//  * S^T = K Q^T: the Q^T operand stays in registers for the whole loop; the
//    K operand is read from LDS (16 bytes per lane). In the 32x32 accumulator
//    layout each lane owns one query row (lane % 32) and 16 of every 32 keys,
//    so the row maximum needs a single cross-lane step (lanes l and l ^ 32).
//  * O^T += V^T P^T: the probabilities, converted to bf16 in registers, are
//    already laid out as the B operand; the V^T operand comes from LDS through
//    the transposing 64-bit read (ds_read_b64_tr_b16), so V is never transposed
//    in memory.
//  * K/V tiles of 64 keys are double-buffered in LDS; 16-byte chunks are
//    XOR-swizzled per key row so that both the K reads and the transposed V
//    reads are free of bank conflicts.
//  * The reference maximum is only moved (and the state rescaled) when a tile's
//    maximum exceeds it by more than 2^8; otherwise exponentials up to 2^8 are
//    accumulated against the stale reference. This is exact in exact arithmetic
//    (the reference cancels in o~ / s and in lse = ref + log s) and skips most
//    rescales.
//  * Workgroups of one head are placed on one XCD (workgroups are dispatched
//    round-robin over the 8 XCDs), so the head's K and V are fetched into that
//    XCD's L2 once.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace rf {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int KB = 64;          // keys per tile
constexpr float kRescaleSlack = 8.f;

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    bf16x2_t t = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, t);
}

__device__ __forceinline__ bf16x4_t lds_read_tr16(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) bf16x4_t*)(p));
}

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void attn_fwd_bf16_kernel(const uint16_t* __restrict__ q,
                                                                const uint16_t* __restrict__ k,
                                                                const uint16_t* __restrict__ v,
                                                                uint16_t* __restrict__ o,
                                                                float* __restrict__ lse,
                                                                int64_t Sq, int64_t Sk, int nqb,
                                                                float sl2, uint32_t qsign) {
    constexpr int BM = 32 * NW;      // query rows per workgroup
    constexpr int NT = NW * 64;      // threads
    constexpr int CH = D / 8;        // 16-byte chunks per row
    constexpr int TCH = KB * CH;     // chunks per K (or V) tile
    constexpr int LPT = 2 * TCH / NT;  // chunks loaded per thread per tile (K then V)
    constexpr int NC = D / 16;       // K=16 slices of the head dimension
    constexpr int DB = D / 32;       // 32-wide output column blocks
    static_assert(2 * TCH % NT == 0, "tile chunks must divide among threads");

    __shared__ __attribute__((aligned(16))) uint16_t smem[2][2][KB * D];   // [stage][K, V][row * D]

    // Workgroup -> (head, query block); heads stay on one XCD when the grid divides by 8.
    int64_t bid = blockIdx.x;
    const int64_t total = int64_t(gridDim.x);
    if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
    const int64_t bh = bid / nqb;
    const int64_t q0 = (bid - bh * nqb) * BM;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, h = lane >> 5;

    const uint16_t* kh = k + bh * Sk * D;
    const uint16_t* vh = v + bh * Sk * D;

    // Q^T operand: lane (query l32, half h) holds Q[row][16c + 8h .. +7]; the sign of
    // Q is flipped for a negative scale so that sl2 = |scale| log2(e) >= 0.
    const int64_t qrow = q0 + 32 * wave + l32;
    bf16x8 qf[NC];
    {
        const int64_t qr = qrow < Sq ? qrow : Sq - 1;
        const uint16_t* src = q + (bh * Sq + qr) * D + 8 * h;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            u32x4 t = *reinterpret_cast<const u32x4*>(src + 16 * c);
            t ^= qsign;
            qf[c] = __builtin_bit_cast(bf16x8, t);
        }
    }

    const int64_t ntiles = ceil_div(Sk, KB);
    u32x4 stage_regs[LPT];

    auto load_tile = [&](int64_t t) {
#pragma unroll
        for (int j = 0; j < LPT; ++j) {
            const int i = tid + j * NT;
            const int which = i / TCH;           // 0: K, 1: V
            const int rem = i - which * TCH;
            const int key = rem / CH, ch = rem % CH;
            int64_t gk = t * KB + key;
            gk = gk < Sk ? gk : Sk - 1;          // rows past the end hold a valid (masked) key
            const uint16_t* src = (which ? vh : kh) + gk * D + ch * 8;
            stage_regs[j] = *reinterpret_cast<const u32x4*>(src);
        }
    };
    auto store_tile = [&](int st) {
#pragma unroll
        for (int j = 0; j < LPT; ++j) {
            const int i = tid + j * NT;
            const int which = i / TCH;
            const int rem = i - which * TCH;
            const int key = rem / CH, ch = rem % CH;
            const int sw = which ? (ch ^ ((key & 3) << 1)) : (ch ^ (key & 7));
            *reinterpret_cast<u32x4*>(&smem[st][which][key * D + sw * 8]) = stage_regs[j];
        }
    };

    f32x16 acc_o[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) acc_o[b] = f32x16{};
    float m_ref = kNegInf, s_part = 0.f;

    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int64_t t = 0; t < ntiles; ++t) {
        const int st = int(t & 1);
        if (t + 1 < ntiles) load_tile(t + 1);

        const uint16_t* ks = smem[st][0];
        const uint16_t* vs = smem[st][1];

        // S^T for two 32-key blocks.
        f32x16 acc_s[2];
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
            acc_s[kb2] = f32x16{};
            const int key = kb2 * 32 + l32;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const int ch = (2 * c + h) ^ (key & 7);
                const u32x4 kf = *reinterpret_cast<const u32x4*>(ks + key * D + ch * 8);
                acc_s[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf), qf[c],
                                                                      acc_s[kb2], 0, 0, 0);
            }
        }

        // Mask keys past the end, row maximum (lanes l and l ^ 32 share a query).
        const int64_t kvalid = Sk - t * KB;
        float mx = kNegInf;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kb2 * 32 + (r >> 2) * 8 + 4 * h + (r & 3);
                if (kvalid < KB && key >= kvalid) acc_s[kb2][r] = kNegInf;
                mx = fmaxf(mx, acc_s[kb2][r]);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mx2 = mx * sl2;

        const bool need = mx2 > m_ref + kRescaleSlack;
        if (__any(need)) {
            const float ref = need ? mx2 : m_ref;
            const float alpha = exp2_fast(m_ref - ref);   // -inf -> 0 on the first tile
            s_part *= alpha;
#pragma unroll
            for (int b = 0; b < DB; ++b) acc_o[b] *= alpha;
            m_ref = ref;
        }

        // p = 2^(x - ref) in fp32, summed per lane, packed to bf16 as the P^T operand.
        // Masked keys (last tile only) get p = 0 by selection: with a zero scale a
        // masked -inf score would otherwise turn into NaN.
        uint32_t pk[2][8];
        auto probs = [&](auto tail) {
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    float p0 = exp2_fast(fmaf(acc_s[kb2][r], sl2, -m_ref));
                    float p1 = exp2_fast(fmaf(acc_s[kb2][r + 1], sl2, -m_ref));
                    if constexpr (decltype(tail)::value) {
                        const int key = kb2 * 32 + (r >> 2) * 8 + 4 * h + (r & 3);
                        p0 = key < kvalid ? p0 : 0.f;
                        p1 = key + 1 < kvalid ? p1 : 0.f;
                    }
                    s_part += p0 + p1;
                    pk[kb2][r >> 1] = pack_bf16(p0, p1);
                }
        };
        if (kvalid < KB)
            probs(std::true_type{});
        else
            probs(std::false_type{});

        // O^T += V^T P^T over four 16-key chunks.
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            const u32x4 pb = {pk[kc >> 1][(kc & 1) * 4 + 0], pk[kc >> 1][(kc & 1) * 4 + 1],
                              pk[kc >> 1][(kc & 1) * 4 + 2], pk[kc >> 1][(kc & 1) * 4 + 3]};
            const int j = lane & 15;
#pragma unroll
            for (int b = 0; b < DB; ++b) {
                // 16-lane group: rows kc*16 + 4h + j/4 (+8), columns 32b + 16*(l32/16) + 4*(j%4).
                const int d = 32 * b + 16 * (l32 >> 4) + 4 * (j & 3);
                const int key0 = kc * 16 + 4 * h + (j >> 2);
                const int key1 = key0 + 8;
                const int p0 = key0 * D + (((d >> 3) ^ ((key0 & 3) << 1)) << 3) + (d & 7);
                const int p1 = key1 * D + (((d >> 3) ^ ((key1 & 3) << 1)) << 3) + (d & 7);
                const bf16x4_t lo = lds_read_tr16(vs + p0);
                const bf16x4_t hi = lds_read_tr16(vs + p1);
                const bf16x8_t va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                acc_o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va),
                                                                    __builtin_bit_cast(bf16x8, pb), acc_o[b], 0, 0,
                                                                    0);
            }
        }

        if (t + 1 < ntiles) store_tile(st ^ 1);
        __syncthreads();
    }

    // Epilogue: s = both halves' partial sums; O = o~ / s; lse = ln 2 (ref + log2 s).
    const float s = s_part + __shfl_xor(s_part, 32, 64);
    if (qrow < Sq) {
        const float inv = 1.f / s;
        uint16_t* dst = o + (bh * Sq + qrow) * D;
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d = 32 * b + g4 * 8 + 4 * h;
                u32x2 w = {pack_bf16(acc_o[b][4 * g4] * inv, acc_o[b][4 * g4 + 1] * inv),
                           pack_bf16(acc_o[b][4 * g4 + 2] * inv, acc_o[b][4 * g4 + 3] * inv)};
                *reinterpret_cast<u32x2*>(dst + d) = w;
            }
        if (lse && h == 0) lse[bh * Sq + qrow] = (m_ref + __log2f(s)) * kLn2;
    }
}

template <int D, int NW>
hipError_t launch_t(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse, int64_t BH,
                    int64_t Sq, int64_t Sk, float scale, hipStream_t stream) {
    const int64_t nqb = ceil_div(Sq, 32 * NW);
    const int64_t blocks = BH * nqb;
    if (blocks > INT32_MAX || nqb > INT32_MAX) return hipErrorInvalidValue;
    const float sl2 = (scale < 0.f ? -scale : scale) * kLog2e;
    const uint32_t qsign = scale < 0.f ? 0x80008000u : 0u;
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, NW>), dim3(unsigned(blocks)), dim3(NW * 64), 0, stream, q, k, v, o,
                       lse, Sq, Sk, int(nqb), sl2, qsign);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
                                int64_t BH, int64_t Sq, int64_t Sk, int D, float scale, hipStream_t stream) {
    if (D == 64) return launch_t<64, 2>(q, k, v, o, lse, BH, Sq, Sk, scale, stream);
    return launch_t<128, 2>(q, k, v, o, lse, BH, Sq, Sk, scale, stream);
}

}  // namespace rf
