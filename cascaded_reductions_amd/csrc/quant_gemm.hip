// Dynamic FP8 quantisation fused with an FP8 GEMM.
//
// The cascade of the explainer "RedFuser框架：AI加速器中的算子融合技术解析",
// section 4.3: scale = max|X| / 448 per row, codes = round(X / scale) to OCP
// E4M3FN, then Y = codes . W dequantised by the row and column scales. The
// scale needs the whole row's maximum before any code can be formed, and
// rounding has no incremental form (its inverse does not exist). The cascade is
// built in two forms with identical results: two launches on one stream (the
// explainer's multi-kernel level, section 3.3; the faster form, parts 1 and 2
// below), and one launch (section 4.3's full fusion; part 3) in which every
// output tile reduces its own rows' maxima and quantises X in LDS. The two-launch
// form:
//  1. quant_rows: one wave per row keeps the row in registers, reduces the
//     absolute maximum (an integer max over the bf16 magnitude bits), forms
//     sigma = a / 448 and each code from the IEEE fp32 quotient x / sigma
//     (reciprocal + one FMA correction, correctly rounded) with the hardware
//     round-to-nearest-even E4M3FN conversion (v_cvt_pk_fp8_f32, which keeps the
//     sign of zero and saturates at 448);
//  2. fp8_gemm: 256 x 256 output tiles, 8 waves, K steps of 128 code bytes
//     double buffered in LDS (filled by direct global-to-LDS loads, so no
//     registers are spent on staging). Both operands are K-contiguous, so no
//     transposes are needed. The product is formed as C^T = W X^T so that every
//     lane ends with four consecutive output columns of one row; the epilogue
//     applies (acc * sigma_i) * w_scale_j and rounds to bf16.
//
// Accumulation precision. The product must be accumulated in fp32. gfx950's
// FP8 matrix instructions (v_mfma_scale_f32_*_f8f6f4 and v_mfma_f32_*_fp8_fp8)
// align the products of one instruction to the largest of them and keep only
// 13 bits below it (measured: 2^16 + 2^3 is kept, 2^16 + 2^2 is lost), which on
// rows with x20 outliers leaves near-cancelling outputs visibly wrong. The
// codes are therefore converted exactly to bf16 in registers after the LDS read
// and multiplied on v_mfma_f32_32x32x16_bf16, whose accumulation keeps fp32
// precision (2^16 + 2^-6 is kept). Operands stay 8-bit in HBM and LDS.
#include "common.hpp"
#include "launch.hpp"

namespace rf {
namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ 1. per-row quantisation

constexpr int QT = 256;   // threads per workgroup
constexpr float kMinRecipSigma = 0x1p-60f;   // smallest row scale quantised through the reciprocal

__device__ __forceinline__ uint32_t codes4(float a, float b, float c, float d) {
    int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
    return uint32_t(v);
}

// The IEEE fp32 quotient x / sigma from the correctly rounded reciprocal r = 1 / sigma:
// q0 = x r is within one ulp of x / sigma, the residual x - q0 sigma is exact in one
// FMA, and q0 + residual * r rounded once is the correctly rounded quotient
// (Markstein, IBM J. Res. Dev. 34(1), 1990). Overflow cannot occur (|q| <= 448). The
// residual is exact whenever x >= 2^-103; with sigma >= 2^-60 every x whose code can be
// non-zero (x >= sigma 2^-10) is far above that, and a smaller x gives a quotient far
// below the smallest E4M3FN subnormal, whose code (+-0) does not depend on the last
// bits. (Rows with sigma < 2^-60, where 1 / sigma may even overflow, divide instead.)
// The correction turns x = -0 into +0, so the sign is restored from x (sigma > 0: the
// quotient always has the sign of x).
__device__ __forceinline__ float div_rn(float x, float sigma, float r) {
    const float q0 = x * r;
    const float e = fmaf(-q0, sigma, x);
    return __builtin_copysignf(fmaf(e, r, q0), x);
}

// Eight bf16 values of a row -> eight E4M3FN codes (two dwords, in order), all +0 for a
// zero row. Shared by both forms of the cascade, so their codes agree bit for bit.
__device__ __forceinline__ uint2 codes8(const u32x4& t, float sigma, float r) {
    uint32_t out0 = 0u, out1 = 0u;
    if (sigma >= kMinRecipSigma) {
        float q[8];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            q[2 * w] = div_rn(bf16_lo(t[w]), sigma, r);
            q[2 * w + 1] = div_rn(bf16_hi(t[w]), sigma, r);
        }
        out0 = codes4(q[0], q[1], q[2], q[3]);
        out1 = codes4(q[4], q[5], q[6], q[7]);
    } else if (sigma > 0.f) {                  // rows of tiny magnitude: IEEE division
        float q[8];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            q[2 * w] = bf16_lo(t[w]) / sigma;
            q[2 * w + 1] = bf16_hi(t[w]) / sigma;
        }
        out0 = codes4(q[0], q[1], q[2], q[3]);
        out1 = codes4(q[4], q[5], q[6], q[7]);
    }
    return make_uint2(out0, out1);
}

// One wave per row, four rows per workgroup. NCT > 0: lane l holds chunks l, l + 64, ...
// (at most NCT chunks of 8 values), all loaded before the first use so every 16-byte
// load of the row is in flight at once, and the row stays in registers between the
// absmax and the quantisation; NCT == 0: the row is streamed twice. The absmax is
// reduced across the wave by xor shuffles: no LDS and no barrier.
constexpr int QROWS = QT / 64;

__device__ __forceinline__ uint32_t absmax8(const u32x4& t, uint32_t m) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        m = max(m, t[w] & 0x7FFFu);             // bf16 magnitude bits order like the magnitudes
        m = max(m, (t[w] >> 16) & 0x7FFFu);
    }
    return m;
}

template <int NCT>
__global__ __launch_bounds__(QT) void quant_rows_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                        uint8_t* __restrict__ codes, float* __restrict__ xs) {
    const int lane = threadIdx.x & 63;
    const int64_t row = int64_t(blockIdx.x) * QROWS + (threadIdx.x >> 6);
    if (row >= M) return;                      // whole waves only: no barrier follows
    const u32x4* xr = reinterpret_cast<const u32x4*>(x + row * K);
    uint2* cr = reinterpret_cast<uint2*>(codes + row * K);
    const int nch = int(K / 8);

    uint32_t amax = 0;
    u32x4 v[NCT > 0 ? NCT : 1];
    if constexpr (NCT > 0) {
#pragma unroll
        for (int i = 0; i < NCT; ++i) {
            const int ch = lane + i * 64;
            v[i] = ch < nch ? __builtin_nontemporal_load(xr + ch) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < NCT; ++i) amax = absmax8(v[i], amax);
    } else {
        for (int ch = lane; ch < nch; ch += 64) amax = absmax8(xr[ch], amax);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) amax = max(amax, uint32_t(__shfl_xor(int(amax), m, 64)));

    const float a = bf16_to_f32(amax);
    const float sigma = a / 448.0f;            // IEEE fp32 division
    const float r = 1.0f / sigma;              // IEEE fp32 division (inf for a zero row; unused then)
    if (lane == 0) xs[row] = sigma;

    // Streaming stores (each wave instruction writes 512 contiguous bytes): no dirty lines are
    // left for the end-of-kernel write-back.
    auto quant8 = [&](const u32x4& t, int ch) {
        const uint2 c = codes8(t, sigma, r);
        __builtin_nontemporal_store(u32x2{c.x, c.y}, reinterpret_cast<u32x2*>(cr + ch));
    };
    if constexpr (NCT > 0) {
#pragma unroll
        for (int i = 0; i < NCT; ++i) {
            const int ch = lane + i * 64;
            if (ch < nch) quant8(v[i], ch);
        }
    } else {
        for (int ch = lane; ch < nch; ch += 64) quant8(xr[ch], ch);
    }
}

// ------------------------------------------------------------------ 2. FP8 GEMM

constexpr int BT = 256;        // tile rows (N) and columns (M)
constexpr int BK = 128;        // bytes of K per step
constexpr int GW = 8;          // waves
constexpr int GT = GW * 64;    // threads
constexpr int TILE_BYTES = BT * BK;                     // 32 KiB per operand per stage
constexpr int GM = 8;          // tile columns per group in the tile order (see tile_of)

// Eight E4M3FN codes (two dwords) -> eight bf16 values. Every E4M3FN value is exactly
// representable in bf16, so the conversion (v_cvt_scalef32_pk_bf16_fp8, scale 1) is exact.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
    const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
    const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
    const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
    const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
    const u32x4 u = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, c),
                     __builtin_bit_cast(uint32_t, d)};
    return __builtin_bit_cast(bf16x8, u);
}

// LDS row of 128 bytes = 8 chunks of 16 bytes, chunk index XOR-swizzled by row.
// The LDS serves a wave's 16-byte reads 16 lanes (256 bytes, all 64 banks) per cycle, and
// the 16 lanes of a read group take 16 consecutive rows at one logical chunk: rows r and
// r + 1 differ in their 128-byte half of a bank row, and (row >> 1) & 7 gives the eight
// even (or odd) rows eight distinct chunks, so the group is conflict-free. (An XOR with
// row & 7 repeats every 8 rows and put rows r and r + 8 on the same banks.)
__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ ((row >> 1) & 7)) << 4); }

// Tile order. Workgroups are dispatched round-robin over the 8 XCDs, so workgroup b runs
// on XCD b % 8; renumbering makes each XCD own a contiguous range of logical tiles. The
// logical order walks groups of GM tile columns (M) with the tile rows (N) inside, so an
// XCD's range of 32 tiles at 16 x 16 tiles is a 4 (N) x 8 (M) block: it reads 4 W panels
// and 8 X panels into its L2 instead of 2 and 16.
__device__ __forceinline__ void tile_of(int64_t bid, int64_t total, int64_t tiles_m, int64_t tiles_n, int64_t& tn,
                                        int64_t& tm) {
    if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
    const int64_t group = bid / (GM * tiles_n);
    const int64_t first = group * GM;
    const int64_t width = tiles_m - first < GM ? tiles_m - first : GM;
    const int64_t in = bid - group * GM * tiles_n;
    tn = in / width;
    tm = first + (in - tn * width);
}

// Operands of one K slice (32 code bytes of every row) in a wave's registers. Lane (row l32,
// half g) holds the 16 bytes [32p + 16g, +16) of its rows; after the exact bf16 conversion,
// bytes 0-7 feed the first K=16 MFMA of a pair and bytes 8-15 the second (the same
// slot-to-k map for both operands). A wave owns a 128 (N) x 64 (M) block of the tile:
// four 32-row W blocks (a) by two 32-row X blocks (b).
struct SliceRegs {
    u32x4 a[4], b[2];
};
struct Operands {
    bf16x8 alo[4], ahi[4], blo[2], bhi[2];
};
__device__ __forceinline__ void convert(const SliceRegs& r, Operands& o) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        o.alo[a] = fp8x8_to_bf16(r.a[a][0], r.a[a][1]);
        o.ahi[a] = fp8x8_to_bf16(r.a[a][2], r.a[a][3]);
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        o.blo[b] = fp8x8_to_bf16(r.b[b][0], r.b[b][1]);
        o.bhi[b] = fp8x8_to_bf16(r.b[b][2], r.b[b][3]);
    }
}
__device__ __forceinline__ void mfmas(const Operands& o, f32x16 (&acc)[4][2]) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.alo[a], o.blo[b], acc[a][b], 0, 0, 0);
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.ahi[a], o.bhi[b], acc[a][b], 0, 0, 0);
        }
}

// acc[a][b][r] = C^T[n][m]: n = n0 + wn*128 + a*32 + (r/4)*8 + 4g + r%4, m = m0 + wm*64 + b*32 + l32.
// Epilogue: scale by sigma_m (row_scale(local row)) and w_scale_n, round to bf16 and stage the
// wave's 64 (m) x 128 (n) block in LDS (stg: 16 KiB per wave, free after the last barrier),
// then write whole rows with 16-byte stores so every output line is written once and completely.
template <class RowScale>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[4][2], uint8_t* stage_lds, RowScale row_scale,
                                           const float* __restrict__ ws, int64_t M, int64_t N, int64_t m0,
                                           int64_t n0, uint16_t* __restrict__ y) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, g = lane >> 5;
    const int wn = wave >> 2, wm = wave & 3;
    uint16_t* stg = reinterpret_cast<uint16_t*>(stage_lds) + wave * (64 * 128);
    float wsc[4][4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                int64_t n = n0 + wn * 128 + a * 32 + q4 * 8 + 4 * g + e;
                n = n < N ? n : N - 1;
                wsc[a][q4][e] = ws[n];
            }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const float sx = row_scale(wm * 64 + b * 32 + l32);
        const int ml = b * 32 + l32;           // row of the staging block
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int nl = a * 32 + q4 * 8 + 4 * g;   // column of the staging block (multiple of 4)
                const f32x16& c = acc[a][b];
                const uint2 w2 = make_uint2(
                    pack_bf16x2((c[4 * q4 + 0] * sx) * wsc[a][q4][0], (c[4 * q4 + 1] * sx) * wsc[a][q4][1]),
                    pack_bf16x2((c[4 * q4 + 2] * sx) * wsc[a][q4][2], (c[4 * q4 + 3] * sx) * wsc[a][q4][3]));
                // 16-byte chunks of a staging row are rotated by the row index to spread banks.
                const int chunk = ((nl >> 3) + ml) & 15;
                *reinterpret_cast<uint2*>(stg + ml * 128 + chunk * 8 + (nl & 7)) = w2;
            }
    }
    __syncthreads();
    // 64 rows x 16 chunks of 16 bytes: each instruction writes 4 whole rows, with streaming
    // stores, so no dirty lines are left for the end-of-kernel write-back.
    const int64_t nbase = n0 + wn * 128;
#pragma unroll
    for (int it = 0; it < 16; ++it) {
        const int ml = it * 4 + (lane >> 4);
        const int ch = lane & 15;
        const int64_t m = m0 + wm * 64 + ml;
        const int64_t n = nbase + ch * 8;
        const u32x4 v = *reinterpret_cast<const u32x4*>(stg + ml * 128 + (((ch + ml) & 15) * 8));
        if (m < M) {
            uint16_t* dst = y + m * N + n;
            if (n + 7 < N && ((N & 7) == 0)) {
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst));
            } else {
                const uint16_t* hv = reinterpret_cast<const uint16_t*>(&v);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (n + e < N) dst[e] = hv[e];
            }
        }
    }
}

__global__ __launch_bounds__(GT) void fp8_gemm_kernel(const uint8_t* __restrict__ xq, const uint8_t* __restrict__ wq,
                                                      const float* __restrict__ xs, const float* __restrict__ ws,
                                                      int64_t M, int64_t N, int64_t K, int tiles_m, int tiles_n,
                                                      uint16_t* __restrict__ y) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[2][2][TILE_BYTES];   // [stage][W, X]

    int64_t tn, tm;
    tile_of(blockIdx.x, int64_t(gridDim.x), tiles_m, tiles_n, tn, tm);
    const int64_t n0 = tn * BT, m0 = tm * BT;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, g = lane >> 5;
    const int wn = wave >> 2;      // 0..1 : 128 rows of N each
    const int wm = wave & 3;       // 0..3 : 64 columns of M each

    // Global -> LDS without registers (global_load_lds_dwordx4): one wave instruction
    // fills 1 KiB of LDS = 8 rows of 128 bytes, lane i landing in row i/8, physical
    // chunk i%8; the lane therefore fetches logical chunk (i%8) ^ ((row >> 1) & 7).
    // Waves 0-3 fill the W tile, waves 4-7 the X tile, 8 instructions each.
    const int which = wave >> 2;
    const uint8_t* gsrc = which ? xq : wq;
    const int64_t lim = which ? M : N;
    const int64_t base_row = which ? m0 : n0;
    auto load = [&](int64_t k0, int st) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int r0 = ((wave & 3) * 8 + j) * 8;
            const int r = r0 + (lane >> 3);
            const int ch = (lane & 7) ^ ((r >> 1) & 7);
            int64_t gr = base_row + r;
            gr = gr < lim ? gr : lim - 1;
            __builtin_amdgcn_global_load_lds(
                (const void*)(gsrc + gr * K + k0 + ch * 16),
                (__attribute__((address_space(3))) void*)(&smem[st][which][r0 * BK]), 16, 0, 0);
        }
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};

    auto read_slice = [&](int st, int p, SliceRegs& r) {
        const uint8_t* sw = smem[st][0];
        const uint8_t* sx = smem[st][1];
#pragma unroll
        for (int a = 0; a < 4; ++a)
            r.a[a] = *reinterpret_cast<const u32x4*>(sw + swz(wn * 128 + a * 32 + l32, 2 * p + g));
#pragma unroll
        for (int b = 0; b < 2; ++b)
            r.b[b] = *reinterpret_cast<const u32x4*>(sx + swz(wm * 64 + b * 32 + l32, 2 * p + g));
    };

    // Software pipeline: the LDS reads of slice p+1 are issued before the MFMAs of slice p,
    // and the step's barrier sits between the last slice's conversion and its MFMAs, so the
    // first slice of the next stage is read while those MFMAs run. The stage a step's loads
    // overwrite was last read before the previous step's barrier.
    const int64_t nk = K / BK;
    load(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    SliceRegs cur;
    read_slice(0, 0, cur);
    for (int64_t t = 0; t < nk; ++t) {
        const int st = int(t & 1);
        if (t + 1 < nk) load((t + 1) * BK, st ^ 1);
#pragma unroll
        for (int p = 0; p < BK / 32 - 1; ++p) {
            SliceRegs nxt;
            read_slice(st, p + 1, nxt);
            Operands o;
            convert(cur, o);
            mfmas(o, acc);
            cur = nxt;
        }
        Operands o;
        convert(cur, o);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (t + 1 < nk) read_slice(st ^ 1, 0, cur);
        mfmas(o, acc);
    }
    store_tile(acc, &smem[0][0][0], [&](int r) { const int64_t m = m0 + r; return xs[m < M ? m : M - 1]; }, ws, M, N,
               m0, n0, y);
}

// ------------------------------------------------------------------ 3. one-launch form
//
// The whole cascade in one launch (the explainer's single-kernel level): each 256 x 256
// tile first reduces the absolute maxima of its own 256 X rows (every tile of a tile row
// repeats that reduction: there is no exchange between workgroups), then streams bf16 X
// through LDS and quantises it there, a K step ahead of the matrix products, into the same
// code layout the two-launch form loads. Codes and scales come from the same quantiser
// (codes8) and the products run in the same order, so Y, the scales and the codes are
// bit-identical to the two-launch form. The price is the X traffic: every tile reads its
// X rows in bf16 twice (absolute maxima, then the operand), against one read of 8-bit
// codes per tile in the two-launch form.
constexpr int FBK = 64;                 // code bytes of K per step
constexpr int FCODE = BT * FBK;         // 16 KiB: one operand's codes per stage
constexpr int FSTG = BT * FBK * 2;      // 32 KiB: bf16 X of one step

// Code rows of 64 bytes = 4 chunks of 16 bytes. A read group of 16 lanes takes 16
// consecutive rows at one logical chunk: rows r..r+3 fill one 256-byte bank row, and the
// XOR with (row >> 2) & 3 gives the four rows sharing a bank-row position four distinct
// chunks, so the 16 reads hit 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz64(int row, int chunk) { return row * FBK + ((chunk ^ ((row >> 2) & 3)) << 4); }

__global__ __launch_bounds__(GT) void fp8_gemm_fused_kernel(const uint16_t* __restrict__ x,
                                                            const uint8_t* __restrict__ wq,
                                                            const float* __restrict__ ws, int64_t M, int64_t N,
                                                            int64_t K, int tiles_m, int tiles_n,
                                                            uint16_t* __restrict__ y, float* __restrict__ xs_out,
                                                            uint8_t* __restrict__ xq_out) {
    // [0, 64 KiB): codes, stage s at s * 2 * FCODE (W, then X); [64, 128 KiB): two bf16 X
    // staging buffers. The epilogue reuses all 128 KiB.
    __shared__ __attribute__((aligned(16))) uint8_t smem[4 * FCODE + 2 * FSTG];
    __shared__ float sig[BT], rcp[BT];
    uint8_t* const codes = smem;
    uint8_t* const stage = smem + 4 * FCODE;

    int64_t tn, tm;
    tile_of(blockIdx.x, int64_t(gridDim.x), tiles_m, tiles_n, tn, tm);
    const int64_t n0 = tn * BT, m0 = tm * BT;
    const bool owner = tn == 0;        // the tile that writes x_scale and the codes of its rows

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, g = lane >> 5;
    const int wn = wave >> 2, wm = wave & 3;

    // 1. Row scales. Wave w reduces rows 32w..32w+31, four rows at a time with four 16-byte
    //    loads per row in flight per lane; rows past M get sigma = 0.
    const int nch = int(K / 8);
    for (int rg = 0; rg < 32; rg += 4) {
        uint32_t am[4] = {0u, 0u, 0u, 0u};
        const u32x4* rp[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t m = m0 + wave * 32 + rg + q;
            rp[q] = reinterpret_cast<const u32x4*>(x + (m < M ? m : M - 1) * K);
        }
        for (int ch = lane; ch < nch; ch += 256) {
            u32x4 v[4][4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int c = ch + 64 * u;
                    v[q][u] = c < nch ? rp[q][c] : u32x4{0u, 0u, 0u, 0u};
                }
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int u = 0; u < 4; ++u) am[q] = absmax8(v[q][u], am[q]);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) am[q] = max(am[q], uint32_t(__shfl_xor(int(am[q]), d, 64)));
            const int r = wave * 32 + rg + q;
            const int64_t m = m0 + r;
            const float sigma = m < M ? bf16_to_f32(am[q]) / 448.0f : 0.0f;   // IEEE fp32 division
            if (lane == 0) {
                sig[r] = sigma;
                rcp[r] = 1.0f / sigma;                                          // inf for a zero row; unused then
                if (owner && m < M) xs_out[m] = sigma;
            }
        }
    }

    // 2. W codes by direct global -> LDS loads: 16 KiB per step, two instructions per wave,
    //    each 16 rows x 64 bytes (lane i: row i/4, physical chunk i%4). They are issued from
    //    inline assembly (lds_dma16): a load the compiler tracks would make it wait for the
    //    loads into the staging buffer before every LDS read of the step. The explicit
    //    vmcnt wait before each barrier orders them.
    auto load_w = [&](int64_t k0, int s) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int r0 = (wave * 2 + j) * 16;
            const int r = r0 + (lane >> 2);
            const int ch = (lane & 3) ^ ((r >> 2) & 3);
            int64_t gr = n0 + r;
            gr = gr < N ? gr : N - 1;
            lds_dma16(wq + gr * K + k0 + ch * 16, &codes[s * 2 * FCODE + r0 * FBK]);
        }
    };
    //    bf16 X by direct loads into a staging buffer: 32 KiB per step, four instructions per
    //    wave, each 8 rows x 128 bytes, unswizzled.
    auto load_x = [&](int64_t k0, int b) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r0 = (wave * 4 + j) * 8;
            const int r = r0 + (lane >> 3);
            int64_t gr = m0 + r;
            gr = gr < M ? gr : M - 1;
            lds_dma16(x + gr * K + k0 + (lane & 7) * 8, &stage[b * FSTG + r0 * 128]);
        }
    };
    //    Staging buffer b -> X codes of stage s: 2048 chunks of 8 values, four per thread;
    //    a wave reads 1 KiB of consecutive chunks and writes 8-byte code pairs.
    auto quantize = [&](int64_t k0, int b, int s) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int idx = j * GT + tid;
            const int r = idx >> 3, c = idx & 7;
            const u32x4 v = *reinterpret_cast<const u32x4*>(&stage[b * FSTG + r * 128 + c * 16]);
            const uint2 q = codes8(v, sig[r], rcp[r]);
            *reinterpret_cast<uint2*>(&codes[s * 2 * FCODE + FCODE + swz64(r, c >> 1) + 8 * (c & 1)]) = q;
            if (owner && xq_out != nullptr && m0 + r < M)
                *reinterpret_cast<uint2*>(xq_out + (m0 + r) * K + k0 + c * 8) = q;
        }
    };
    auto read_slice = [&](int s, int p, SliceRegs& rr) {
        const uint8_t* sw = codes + s * 2 * FCODE;
        const uint8_t* sx = sw + FCODE;
#pragma unroll
        for (int a = 0; a < 4; ++a)
            rr.a[a] = *reinterpret_cast<const u32x4*>(sw + swz64(wn * 128 + a * 32 + l32, 2 * p + g));
#pragma unroll
        for (int b = 0; b < 2; ++b)
            rr.b[b] = *reinterpret_cast<const u32x4*>(sx + swz64(wm * 64 + b * 32 + l32, 2 * p + g));
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};

    // 3. Pipeline. At the top of step t the codes of stage t&1 are complete and staging
    //    buffer (t+1)&1 holds bf16 X of step t+1. Step t loads W of step t+1 into the other
    //    code stage and bf16 X of step t+2 into staging buffer t&1 (quantised during step
    //    t-1), quantises staging buffer (t+1)&1 into the other code stage, and multiplies
    //    the two 32-byte slices of stage t&1.
    const int64_t nk = K / FBK;
    load_w(0, 0);
    load_x(0, 0);
    if (nk > 1) load_x(FBK, 1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();                   // also publishes sig / rcp
    quantize(0, 0, 0);
    __syncthreads();
    SliceRegs cur;
    read_slice(0, 0, cur);
    for (int64_t t = 0; t < nk; ++t) {
        const int st = int(t & 1);
        if (t + 1 < nk) load_w((t + 1) * FBK, st ^ 1);
        if (t + 2 < nk) load_x((t + 2) * FBK, st);
        {
            SliceRegs nxt;
            read_slice(st, 1, nxt);
            Operands o;
            convert(cur, o);
            mfmas(o, acc);
            cur = nxt;
        }
        if (t + 1 < nk) quantize((t + 1) * FBK, st ^ 1, st ^ 1);
        Operands o;
        convert(cur, o);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (t + 1 < nk) read_slice(st ^ 1, 0, cur);
        mfmas(o, acc);
    }
    store_tile(acc, smem, [&](int r) { return sig[r]; }, ws, M, N, m0, n0, y);
}

}  // namespace

hipError_t launch_quant_rows(const uint16_t* x, int64_t M, int64_t K, uint8_t* codes, float* x_scale,
                             hipStream_t stream) {
    if (ceil_div(M, QROWS) > INT32_MAX || K / 8 > INT32_MAX) return hipErrorInvalidValue;
    const int64_t nct = ceil_div(K / 8, 64);   // chunks of 8 values per lane
    const dim3 grid{unsigned(ceil_div(M, QROWS)), 1u, 1u};
    if (nct <= 1) hipLaunchKernelGGL(quant_rows_kernel<1>, grid, dim3(QT), 0, stream, x, M, K, codes, x_scale);
    else if (nct <= 2) hipLaunchKernelGGL(quant_rows_kernel<2>, grid, dim3(QT), 0, stream, x, M, K, codes, x_scale);
    else if (nct <= 4) hipLaunchKernelGGL(quant_rows_kernel<4>, grid, dim3(QT), 0, stream, x, M, K, codes, x_scale);
    else if (nct <= 8) hipLaunchKernelGGL(quant_rows_kernel<8>, grid, dim3(QT), 0, stream, x, M, K, codes, x_scale);
    else if (nct <= 16) hipLaunchKernelGGL(quant_rows_kernel<16>, grid, dim3(QT), 0, stream, x, M, K, codes, x_scale);
    else hipLaunchKernelGGL(quant_rows_kernel<0>, grid, dim3(QT), 0, stream, x, M, K, codes, x_scale);
    return hipGetLastError();
}

hipError_t launch_quant_gemm_fused(const uint16_t* x, const uint8_t* wq, const float* w_scale, int64_t M, int64_t N,
                                   int64_t K, uint16_t* y, float* x_scale, uint8_t* xq, hipStream_t stream) {
    const int64_t tm = ceil_div(M, BT), tn = ceil_div(N, BT);
    const int64_t blocks = tm * tn;
    if (blocks > INT32_MAX || K % FBK != 0 || K / 8 > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fp8_gemm_fused_kernel, dim3(unsigned(blocks)), dim3(GT), 0, stream, x, wq, w_scale, M, N, K,
                       int(tm), int(tn), y, x_scale, xq);
    return hipGetLastError();
}

hipError_t launch_fp8_gemm(const uint8_t* a, const uint8_t* b, const float* sa, const float* sb, int64_t M,
                           int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
    const int64_t tm = ceil_div(M, BT), tn = ceil_div(N, BT);
    const int64_t blocks = tm * tn;
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fp8_gemm_kernel, dim3(unsigned(blocks)), dim3(GT), 0, stream, a, b, sa, sb, M, N, K, int(tm),
                       int(tn), y);
    return hipGetLastError();
}

}  // namespace rf
