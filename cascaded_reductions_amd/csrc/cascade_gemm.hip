// Row-scaled GEMM cascades on the matrix cores, from the generic template (cascade.hpp).
//
// For each row x of X [M, K] (fp32) and a weight W [K, N] (bf16), the cascades
//   softmax-scaled    y = sum_k softmax(x)_k W[k, :],  stat = ln sum_k exp(x_k)
//   absmax-scaled     y = sum_k (x_k / max|x|) W[k, :], stat = max_k |x_k|
// are two instances of one kernel template (technical summary "RedFuser: An Automatic
// Operator Fusion Framework for Cascaded Reductions on AI Accelerators", Methodologie
// 1-2; explainer "RedFuser框架：AI加速器中的算子融合技术解析", sections 2.2-2.3 and 4.1):
// the lead d1 (row maximum or absolute maximum), the correction H(d_new) (x) H^-1(d_old)
// applied to the running output when the lead moves, and the per-element weights
// G(x) (x) H(d1) all come from Cascade<Spec>; the last reduction, a contraction with W,
// runs on v_mfma_f32_32x32x16_bf16 with each weight split into two bf16 parts.
//
// gfx950 mapping: a workgroup of 4 waves owns 128 rows (32 per wave) and walks K in chunks
// of 32, starting at a chunk that differs between workgroups (the cascade's result does not
// depend on the order in which a row's entries are absorbed). Each chunk's W slice [32 x N]
// bf16 and each wave's X slice [32 x 32] fp32 go to LDS by direct global-to-LDS loads issued
// two chunks ahead (3-slot rings), so no registers hold data in flight. The output is formed
// as Y^T = W^T P^T (as the attention kernels form O^T = V^T P^T): W^T comes from LDS through
// the transposing read (ds_read_b64_tr_b16) and P^T is the packed weights as each lane
// computes them, so every lane owns one row and the lead's correction is a per-lane scale.
// The output rows leave through an LDS staging tile as whole lines with streaming stores.
#include <type_traits>

#include "attn_tiles.hpp"
#include "cascade.hpp"
#include "launch.hpp"

namespace rf {
namespace {

using cascade::AbsMaxGemm;
using cascade::Cascade;
using cascade::SoftmaxGemm;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float fx4 __attribute__((ext_vector_type(4)));

constexpr int KC = 32;         // K per chunk
constexpr int NW = 4;           // waves per workgroup
constexpr int ROWS = 32 * NW;   // rows per workgroup (32 per wave)
constexpr int STAGES = 3;
constexpr int XSLOT = ROWS * KC * 4;   // bytes of X per stage (16 KiB)

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    bf16x2_t t = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, t);
}

__device__ __forceinline__ bf16x4_t lds_read_tr16(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)(p));
}

// X slice of a wave in LDS: [32 rows][8 pieces of 16 bytes], piece index XOR-swizzled by
// (row >> 1) & 7: a 16-lane read group takes 16 consecutive rows at one logical piece; rows
// r and r + 1 sit in different halves of a 256-byte bank row, and the swizzle gives the 8
// even (and the 8 odd) rows 8 distinct pieces, so the group is conflict-free.
__device__ __forceinline__ int x_swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int x_piece(int row, int piece) { return row * 8 + (piece ^ x_swz(row)); }

template <class Spec, int N>
__global__ __launch_bounds__(NW * 64, 2) void cascade_gemm_kernel(const float* __restrict__ x,
                                                              const uint16_t* __restrict__ w, int64_t M, int64_t K,
                                                              float xscale, float* __restrict__ y,
                                                              float* __restrict__ stat) {
    using C = Cascade<Spec>;
    using Lead = typename Spec::Lead;
    constexpr bool SOFTMAX = std::is_same<Spec, SoftmaxGemm>::value;
    constexpr int CH = N / 8;                 // 16-byte chunks per W row
    constexpr int RPW = 64 / CH;              // W rows per wave load
    constexpr int WSLOT = KC * N * 2;         // bytes of W per stage
    constexpr int WL = WSLOT / 1024;          // wave loads per W slice
    constexpr int WPW = WL / NW;              // ... per wave
    constexpr int DB = N / 32;                // 32-wide output blocks
    constexpr int LPC = 4 + WPW;              // direct loads per wave per chunk
    static_assert(WPW >= 1 && WL % NW == 0, "every wave loads a share of the W slice");
    static_assert(NW * 32 * (N + 4) * 4 <= STAGES * (XSLOT + WSLOT), "the output staging tile reuses the rings");

    __shared__ __attribute__((aligned(16))) unsigned char smem[STAGES * (XSLOT + WSLOT)];
    unsigned char* const xring = smem;                       // [stage][wave][32 rows x 128 B]
    uint16_t* const wring = reinterpret_cast<uint16_t*>(smem + STAGES * XSLOT);   // [stage][32 x N]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, h = lane >> 5;
    const int64_t row0 = int64_t(blockIdx.x) * ROWS + 32 * wave;   // first row of this wave
    const int64_t row = row0 + l32;
    const int K32 = int(K);                   // the host bounds K below 2^24
    const int nchunks = (K32 + KC - 1) / KC;

    // ---- direct loads. X: wave load l of a chunk covers the wave's rows 8l .. 8l + 7 (lane i:
    // row 8l + i/8, physical piece i%8, fetching the logical piece that maps there). Rows past M
    // re-read row M - 1 and pieces past K re-read the row's first piece (masked in compute).
    const uint32_t xl_base = lds_addr(xring) + uint32_t(wave * 32 * 128);
    const int64_t rb = row0 < M ? row0 : M - 1;   // a wave wholly past M re-reads row M - 1
    uint32_t x_src[4];                        // byte offset of the lane's row from row rb
    int x_piece_k[4];                         // the first column of its logical piece within a chunk
#pragma unroll
    for (int l = 0; l < 4; ++l) {
        const int r = 8 * l + (lane >> 3);
        const int pc = lane & 7;
        const int lc = pc ^ x_swz(r);
        int64_t gr = row0 + r;
        gr = gr < M ? gr : M - 1;
        x_src[l] = uint32_t((gr - rb) * K * 4);   // < 2^32: the host bounds K below 2^24
        x_piece_k[l] = lc * 4;
    }
    const float* xw = x + rb * K;             // wave-uniform base
    // W: wave w fills wave loads w*WPW .. w*WPW + WPW - 1 of the slice; lane i lands in slice row
    // l*RPW + i/CH, physical chunk i%CH, and fetches the logical chunk the read swizzle maps there.
    uint32_t w_off[WPW];
#pragma unroll
    for (int l = 0; l < WPW; ++l) {
        const int wl = wave * WPW + l;
        const int r = wl * RPW + lane / CH;
        const int pc = lane % CH;
        const int lc = pc ^ attn_v_swz<N>(r);
        w_off[l] = uint32_t(r * N + lc * 8);  // element offset within the slice
    }
    // Workgroups start their walk over K at different chunks and wrap around. Rows are K * 4
    // bytes apart, so when every workgroup reads the same columns at once the chip's reads
    // pile onto a few memory channels; the start is spread over the chunks per XCD
    // (workgroup b runs on XCD b % 8, so b >> 3 numbers an XCD's workgroups).
    const int first = int((blockIdx.x >> 3) % unsigned(nchunks));
    auto chunk_of = [&](int t) {               // the chunk walked at step t (t >= nchunks: the last)
        const int c = first + (t < nchunks ? t : nchunks - 1);
        return c < nchunks ? c : c - nchunks;
    };
    auto issue = [&](int t) {
        const int st = t % STAGES;
        const int k0 = chunk_of(t) * KC;
        const uint32_t xl = xl_base + uint32_t(st * XSLOT);
        const unsigned char* wl = reinterpret_cast<const unsigned char*>(wring) + st * WSLOT + wave * WPW * 1024;
        if (k0 + KC <= K32) {                 // the whole chunk lies inside K (wave-uniform)
#pragma unroll
            for (int l = 0; l < 4; ++l) lds_dma16_sb(xw, x_src[l] + uint32_t((k0 + x_piece_k[l]) * 4), xl + l * 1024);
#pragma unroll
            for (int l = 0; l < WPW; ++l) lds_dma16(w + int64_t(k0) * N + w_off[l], wl + l * 1024);
        } else {
#pragma unroll
            for (int l = 0; l < 4; ++l) {
                const int k = k0 + x_piece_k[l];
                lds_dma16_sb(xw, x_src[l] + uint32_t((k < K32 ? k : 0) * 4), xl + l * 1024);
            }
#pragma unroll
            for (int l = 0; l < WPW; ++l) {
                const int r = (wave * WPW + l) * RPW + lane / CH;
                const int kr = k0 + r < K32 ? k0 + r : K32 - 1;   // rows past K re-read row K - 1
                lds_dma16(w + int64_t(kr) * N + (w_off[l] - r * N), wl + l * 1024);
            }
        }
    };

    // Transposed W^T fragment offsets (the attention kernels' V-read layout, with the K index
    // in the key's place): lane (n-row l32, half h) reads slice rows kc*16 + 4h + j/4 (+8).
    int v_off[2][DB][2];
    {
        const int j16 = lane & 15;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int b = 0; b < DB; ++b) {
                const int d = 32 * b + 16 * (l32 >> 4) + 4 * (j16 & 3);
                const int key0 = kc * 16 + 4 * h + (j16 >> 2);
                const int key1 = key0 + 8;
                v_off[kc][b][0] = key0 * N + (((d >> 3) ^ attn_v_swz<N>(key0)) << 3) + (d & 7);
                v_off[kc][b][1] = key1 * N + (((d >> 3) ^ attn_v_swz<N>(key1)) << 3) + (d & 7);
            }
    }

    f32x16 acc[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) acc[b] = f32x16{};
    Lead lead = Spec::lead_identity();
    float s_part = 0.f;                       // the row sum's share of this lane (softmax only)
    const bf16x2_t ones = {(__bf16)1.f, (__bf16)1.f};

    // Prologue: chunks 0 .. STAGES - 2 in flight.
#pragma unroll
    for (int t = 0; t < STAGES - 1; ++t) issue(t);

    for (int t = 0; t < nchunks; ++t) {
        const int st = t % STAGES;
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((STAGES - 2) * LPC) : "memory");   // chunk t is in
        __syncthreads();
        issue(t + STAGES - 1);               // into the slot chunk t - 1 used
        // The lane's 16 values: pieces h, 2 + h, 4 + h, 6 + h of its row (columns 4h + 8c .. +3).
        const unsigned char* xs = xring + st * XSLOT + wave * 32 * 128;
        float xv[16];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const fx4 v = *reinterpret_cast<const fx4*>(xs + x_piece(l32, 2 * c + h) * 16);
#pragma unroll
            for (int e = 0; e < 4; ++e) xv[4 * c + e] = v[e] * xscale;
        }
        const int kc0 = chunk_of(t) * KC;
        if (kc0 + KC > K32) {                 // the last chunk runs past K (wave-uniform): null entries
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (kc0 + 8 * c + 4 * h + e >= K32) xv[4 * c + e] = SOFTMAX ? kNegInf : 0.f;
        }
        // The lead over this chunk: the lane's 16 values, then its partner lane (l ^ 32).
        Lead tl = lead;
#pragma unroll
        for (int e = 0; e < 16; ++e) tl = Spec::lead_plus(tl, xv[e], 0);
        {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tl), __float_as_uint(tl), false, false);
            tl = Spec::lead_merge(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
        const bool moved = Spec::lead_moved(lead, tl);
        if (__any(moved)) {
            // H(d_new) (x) H^-1(d_old) for the running output (and the row sum) of the rows whose
            // lead moved; an identity lead has absorbed nothing, so its running values stay 0.
            const float f = !moved ? 1.f : Spec::lead_is_identity(lead) ? 0.f : Spec::factor(C::correction(lead, tl));
#pragma unroll
            for (int b = 0; b < DB; ++b) acc[b] *= f;
            s_part *= f;
            lead = tl;
        }
        // Weights G(x) (x) H(d1) in the P^T operand order, each split into a bf16 head and a
        // bf16 tail (p = head + tail to about 2^-17 relative), so the contraction on the bf16
        // matrix cores loses no more than fp32 accumulation does; the row sum reads the same
        // two parts, so numerator and denominator see identical weights.
        // A null entry's term is exactly 0 against any lead but the identity (which only a row
        // with nothing but null entries so far still holds), so the entries are tested only
        // when some lane of the wave still has the identity lead.
        uint32_t ph[8], pt[8];
        auto weights = [&](auto test_null) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float a = xv[2 * i], b = xv[2 * i + 1];
                float pa = Spec::weight(C::term(a, lead));
                float pb = Spec::weight(C::term(b, lead));
                if constexpr (decltype(test_null)::value) {
                    pa = Spec::is_null(a) ? 0.f : pa;
                    pb = Spec::is_null(b) ? 0.f : pb;
                }
                ph[i] = pack_bf16(pa, pb);
                pt[i] = pack_bf16(pa - bf16_lo(ph[i]), pb - bf16_hi(ph[i]));
                if constexpr (SOFTMAX) {
                    s_part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, ph[i]), ones, s_part, false);
                    s_part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pt[i]), ones, s_part, false);
                }
            }
        };
        if (__any(Spec::lead_is_identity(lead))) weights(std::true_type{});
        else weights(std::false_type{});
        // Y^T += W^T (P_head + P_tail)^T over the chunk's two 16-wide K slices.
        const uint16_t* ws = wring + st * (WSLOT / 2);
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            const u32x4 bh = {ph[kc * 4 + 0], ph[kc * 4 + 1], ph[kc * 4 + 2], ph[kc * 4 + 3]};
            const u32x4 bt = {pt[kc * 4 + 0], pt[kc * 4 + 1], pt[kc * 4 + 2], pt[kc * 4 + 3]};
#pragma unroll
            for (int b = 0; b < DB; ++b) {
                const bf16x4_t lo = lds_read_tr16(ws + v_off[kc][b][0]);
                const bf16x4_t hi = lds_read_tr16(ws + v_off[kc][b][1]);
                const bf16x8_t wa = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, wa),
                                                                  __builtin_bit_cast(bf16x8, bh), acc[b], 0, 0, 0);
                acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, wa),
                                                                  __builtin_bit_cast(bf16x8, bt), acc[b], 0, 0, 0);
            }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // retire the trailing (unused) loads

    // Epilogue: the final H applied once (distributivity): 1 / sum for the softmax.
    float scale_out = 1.f;
    if constexpr (SOFTMAX) {
        const float s = s_part + __shfl_xor(s_part, 32, 64);
        scale_out = 1.f / s;
        if (row < M && h == 0 && stat) stat[row] = (lead + __log2f(s)) * kLn2;
    } else {
        if (row < M && h == 0 && stat) stat[row] = lead;
    }
    // The wave's 32 output rows go to an LDS staging tile (the rings are free once every wave
    // is past its last chunk; rows padded by 16 bytes), then out as whole lines, 16 bytes per
    // lane, with streaming stores: written through while the kernel runs, they leave no dirty
    // lines for the end-of-kernel write-back (2.4-6 us of an 80 us kernel at 65536 x 128).
    __syncthreads();
    {
        constexpr int SRF = N + 4;
        float* stg = reinterpret_cast<float*>(smem) + wave * 32 * SRF;
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const fx4 v = {acc[b][4 * q4] * scale_out, acc[b][4 * q4 + 1] * scale_out,
                               acc[b][4 * q4 + 2] * scale_out, acc[b][4 * q4 + 3] * scale_out};
                *reinterpret_cast<fx4*>(stg + l32 * SRF + 32 * b + 8 * q4 + 4 * h) = v;
            }
        asm volatile("" ::: "memory");   // the wave reads back its own staging writes
        constexpr int PPR = N / 4;
#pragma unroll
        for (int it = 0; it < 32 * PPR / 64; ++it) {
            const int idx = it * 64 + lane;
            const int r = idx / PPR, piece = idx % PPR;
            const fx4 v = *reinterpret_cast<const fx4*>(stg + r * SRF + piece * 4);
            if (row0 + r < M) __builtin_nontemporal_store(v, reinterpret_cast<fx4*>(y + (row0 + r) * N + piece * 4));
        }
    }
}

template <class Spec, int N>
hipError_t launch_n(const float* x, const uint16_t* w, int64_t M, int64_t K, float xscale, float* y, float* stat,
                    hipStream_t stream) {
    const int64_t blocks = ceil_div(M, int64_t(ROWS));
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((cascade_gemm_kernel<Spec, N>), dim3(unsigned(blocks)), dim3(NW * 64), 0, stream, x, w, M, K,
                       xscale, y, stat);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_cascade_gemm(int kind, const float* x, const uint16_t* w, int64_t M, int64_t K, int N, float* y,
                               float* stat, hipStream_t stream) {
    if (kind == 0) {                          // softmax-scaled: the kernel works in base 2
        if (N == 64) return launch_n<SoftmaxGemm, 64>(x, w, M, K, kLog2e, y, stat, stream);
        if (N == 128) return launch_n<SoftmaxGemm, 128>(x, w, M, K, kLog2e, y, stat, stream);
    } else if (kind == 1) {
        if (N == 64) return launch_n<AbsMaxGemm, 64>(x, w, M, K, 1.f, y, stat, stream);
        if (N == 128) return launch_n<AbsMaxGemm, 128>(x, w, M, K, 1.f, y, stat, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace rf
