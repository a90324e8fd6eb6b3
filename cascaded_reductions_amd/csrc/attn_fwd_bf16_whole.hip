// Whole-row (non-incremental) fused attention for short key axes, bf16 inputs.
//
// The explainer "RedFuser框架：AI加速器中的算子融合技术解析" (section 5.2) recommends the
// non-incremental form for rows shorter than 256 keys and the incremental form
// from 256 on. Here the non-incremental form is the plain three-pass cascade of
// its section 2.1 kept on chip: a workgroup loads the head's whole K and V
// (at most 8 tiles of 32 keys) into LDS at once, each wave forms every score of
// its 32 query rows in registers, takes the exact row maximum, and then the
// exponentials, their sum and P V -- no running maximum and no rescaling.
//
// gfx950 mapping: 4 waves of 32 query rows (128 queries per workgroup), scores as
// S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (lane = query row l % 32, 16 keys of
// every 32-key tile), O^T += V^T P^T with V^T read through ds_read_b64_tr_b16.
// The LDS layout and its XOR swizzles are those of the incremental kernel.
// NT (the number of key tiles) is a template parameter so that the score array
// stays in registers.
#include "attn_tiles.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace rf {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int KT = 32;   // keys per tile

__device__ __forceinline__ uint32_t pack2(float a, float b) {
    bf16x2_t t = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, t);
}

__device__ __forceinline__ bf16x4_t read_tr16(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)(p));
}

template <int D, int NT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
void attn_whole_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                            const uint16_t* __restrict__ v, uint16_t* __restrict__ o, float* __restrict__ lse,
                            int64_t Sq, int Sk, int nqb, float sl2, uint32_t qsign) {
    constexpr int TILE = KT * D;             // elements of one tile
    constexpr int CH = D / 8;                // 16-byte chunks per key row
    constexpr int RPW = 64 / CH;             // key rows per 1 KiB wave load
    constexpr int WL = TILE * 2 / 1024;      // wave loads per tile
    constexpr int NC = D / 16;               // K=16 slices of the head dimension
    constexpr int DB = D / 32;               // 32-wide output column blocks
    // K tiles, then V tiles; the output staging tiles reuse the region at the end.
    constexpr int SRW = D + 8;                // staging row stride (bf16): 16 bytes of padding
    constexpr int LDS_ELEMS = 2 * NT * TILE > 4 * 32 * SRW ? 2 * NT * TILE : 4 * 32 * SRW;
    __shared__ __attribute__((aligned(16))) uint16_t smem[LDS_ELEMS];
    uint16_t* const ks = smem;
    uint16_t* const vs = smem + NT * TILE;

    int64_t bid = blockIdx.x;
    const int64_t total = int64_t(gridDim.x);
    if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);   // heads stay on one XCD
    const int64_t bh = bid / nqb;
    const int64_t q0 = (bid - bh * nqb) * 128;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, h = lane >> 5;

    // Every wave loads a quarter of the 2 * NT * WL wave loads; rows past the key axis
    // re-read the last key (their scores are masked, their probabilities are zero).
    {
        const uint16_t* kh_ptr = k + bh * int64_t(Sk) * D;
        const uint16_t* vh_ptr = v + bh * int64_t(Sk) * D;
        for (int i = wave; i < 2 * NT * WL; i += 4) {
            const int kind = i / (NT * WL);          // 0: K, 1: V
            const int li = i - kind * NT * WL;       // wave load within the K or V array
            const int row = li * RPW + lane / CH;    // key row of this lane
            const int pc = lane % CH;
            const int lc = kind ? (pc ^ attn_v_swz<D>(row)) : (pc ^ attn_k_swz<D>(row));
            const int grow = row < Sk ? row : Sk - 1;
            const uint16_t* src = (kind ? vh_ptr : kh_ptr) + int64_t(grow) * D + lc * 8;
            lds_dma16(src, smem + kind * NT * TILE + li * RPW * D);
        }
    }

    // Q^T operand (as in the incremental kernel): lane (query l32, half h) holds
    // Q[row][16c + 8h .. +7], with the sign flipped for a negative scale.
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
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // Pass 1: every score of the row block, and the exact row maximum.
    f32x16 s[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const uint16_t* kt = ks + t * TILE;
        f32x16 acc = f32x16{};
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const u32x4 kf = *reinterpret_cast<const u32x4*>(kt + l32 * D + (((2 * c + h) ^ attn_k_swz<D>(l32)) << 3));
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf), qf[c], acc, 0, 0, 0);
        }
        s[t] = acc;
    }
    // Keys of the last tile at or past Sk (accumulator entry r of lane (l32, h) is key
    // 8 (r / 4) + 4 h + r % 4 of its tile).
    const int kvalid = Sk - (NT - 1) * KT;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int key = (r >> 2) * 8 + 4 * h + (r & 3);
        if (key >= kvalid) s[NT - 1][r] = kNegInf;
    }
    float mx = kNegInf;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
    {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    const float m2 = mx * sl2;                 // the maximum in base-2 units (sl2 >= 0)

    // Passes 2 and 3: exponentials against the exact maximum, their sum, and P V.
    f32x16 acc_o[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) acc_o[b] = f32x16{};
    float ssum = 0.f;
    const bf16x2_t ones = {(__bf16)1.f, (__bf16)1.f};
    const int j16 = lane & 15;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        uint32_t pk[8];
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            float p0 = exp2_fast(fmaf(s[t][r], sl2, -m2));
            float p1 = exp2_fast(fmaf(s[t][r + 1], sl2, -m2));
            if (t == NT - 1) {                 // masked keys: probability 0 (also for scale 0)
                const int key = (r >> 2) * 8 + 4 * h + (r & 3);
                p0 = key < kvalid ? p0 : 0.f;
                p1 = key + 1 < kvalid ? p1 : 0.f;
            }
            const uint32_t w = pack2(p0, p1);
            pk[r >> 1] = w;
            ssum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), ones, ssum, false);
        }
        const uint16_t* vt = vs + t * TILE;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            const u32x4 pb = {pk[kc * 4 + 0], pk[kc * 4 + 1], pk[kc * 4 + 2], pk[kc * 4 + 3]};
#pragma unroll
            for (int b = 0; b < DB; ++b) {
                // 16-lane group: rows kc*16 + 4h + j/4 (+8), columns 32b + 16*(l32/16) + 4*(j%4).
                const int d = 32 * b + 16 * (l32 >> 4) + 4 * (j16 & 3);
                const int key0 = kc * 16 + 4 * h + (j16 >> 2);
                const int key1 = key0 + 8;
                const bf16x4_t lo = read_tr16(vt + key0 * D + (((d >> 3) ^ attn_v_swz<D>(key0)) << 3) + (d & 7));
                const bf16x4_t hi = read_tr16(vt + key1 * D + (((d >> 3) ^ attn_v_swz<D>(key1)) << 3) + (d & 7));
                const bf16x8_t va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                acc_o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va),
                                                                    __builtin_bit_cast(bf16x8, pb), acc_o[b], 0, 0, 0);
            }
        }
    }

    // Epilogue: o = o~ / s (the two lane halves hold the two halves of each tile's keys). The
    // wave's 32 rows go to an LDS staging tile (in the K/V region, free once every wave is
    // past its PV), then out as whole lines, 16 bytes per lane, with
    // streaming stores that leave no dirty lines for the end-of-kernel write-back.
    const float srow = ssum + __shfl_xor(ssum, 32, 64);
    __syncthreads();
    uint16_t* stg = smem + wave * 32 * SRW;
    {
        const float inv = 1.f / srow;
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d = 32 * b + g4 * 8 + 4 * h;
                const u32x2 w = {pack2(acc_o[b][4 * g4] * inv, acc_o[b][4 * g4 + 1] * inv),
                                 pack2(acc_o[b][4 * g4 + 2] * inv, acc_o[b][4 * g4 + 3] * inv)};
                *reinterpret_cast<u32x2*>(stg + l32 * SRW + d) = w;
            }
        if (lse && h == 0 && qrow < Sq) lse[bh * Sq + qrow] = (m2 + __log2f(srow)) * kLn2;
    }
    asm volatile("" ::: "memory");            // the wave reads back its own staging writes
    constexpr int PPR = D / 8;                // 16-byte pieces per row
#pragma unroll
    for (int it = 0; it < 32 * PPR / 64; ++it) {
        const int idx = it * 64 + lane;
        const int row = idx / PPR, piece = idx % PPR;
        const u32x4 val = *reinterpret_cast<const u32x4*>(stg + row * SRW + piece * 8);
        const int64_t grow = q0 + 32 * wave + row;
        if (grow < Sq) __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(o + (bh * Sq + grow) * D + piece * 8));
    }
}

template <int D, int NT>
hipError_t launch_nt(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse, int64_t BH,
                     int64_t Sq, int64_t Sk, float scale, hipStream_t stream) {
    const int64_t nqb = ceil_div(Sq, 128);
    const int64_t blocks = BH * nqb;
    if (blocks > INT32_MAX || nqb > INT32_MAX) return hipErrorInvalidValue;
    const float sl2 = (scale < 0.f ? -scale : scale) * kLog2e;
    const uint32_t qsign = scale < 0.f ? 0x80008000u : 0u;
    hipLaunchKernelGGL((attn_whole_bf16_kernel<D, NT>), dim3(unsigned(blocks)), dim3(256), 0, stream, q, k, v, o,
                       lse, Sq, int(Sk), int(nqb), sl2, qsign);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse, int64_t BH,
                    int64_t Sq, int64_t Sk, float scale, hipStream_t stream) {
    switch (ceil_div(Sk, int64_t(KT))) {
        case 1: return launch_nt<D, 1>(q, k, v, o, lse, BH, Sq, Sk, scale, stream);
        case 2: return launch_nt<D, 2>(q, k, v, o, lse, BH, Sq, Sk, scale, stream);
        case 3: return launch_nt<D, 3>(q, k, v, o, lse, BH, Sq, Sk, scale, stream);
        case 4: return launch_nt<D, 4>(q, k, v, o, lse, BH, Sq, Sk, scale, stream);
        case 5: return launch_nt<D, 5>(q, k, v, o, lse, BH, Sq, Sk, scale, stream);
        case 6: return launch_nt<D, 6>(q, k, v, o, lse, BH, Sq, Sk, scale, stream);
        case 7: return launch_nt<D, 7>(q, k, v, o, lse, BH, Sq, Sk, scale, stream);
        case 8: return launch_nt<D, 8>(q, k, v, o, lse, BH, Sq, Sk, scale, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_attn_whole_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
                                  int64_t BH, int64_t Sq, int64_t Sk, int D, float scale, hipStream_t stream) {
    if (Sk < 1 || Sk > kWholeRowMaxKeys) return hipErrorInvalidValue;
    if (D == 64) return launch_d<64>(q, k, v, o, lse, BH, Sq, Sk, scale, stream);
    return launch_d<128>(q, k, v, o, lse, BH, Sq, Sk, scale, stream);
}

}  // namespace rf
