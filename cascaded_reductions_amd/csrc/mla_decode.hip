// Multi-head latent attention (MLA) decode: the multi-segment split kernel.
//
// MLA (named among the workloads of the technical summary "RedFuser: An
// Automatic Operator Fusion Framework for Cascaded Reductions on AI
// Accelerators", Resultaten) caches one compressed latent per token: a row of
// DQK = 576 values whose first DV = 512 are the latent c_kv and whose last 64
// are the shared rotary key. With the key projection absorbed into the query,
// every head h scores token j as x_hj = scale * <q_h, row_j> (576 values) and
// reads back o_h = sum_j softmax_j(x_hj) row_j[0 .. 512). It is the softmax ->
// GEMM cascade of the explainer "RedFuser框架：AI加速器中的算子融合技术解析"
// (section 4.1) with all heads sharing one key/value row, evaluated per key
// segment in the incremental form (Multi-Segment strategy, Methodologie 3);
// the segments are combined by rf_segment_merge (D = 512).
//
// Because the heads share the cache row, the per-token work is a small GEMM
// and runs on the matrix cores: a workgroup owns one batch entry, 64 heads and
// one key segment, and walks the segment in tiles of 32 tokens staged in LDS (a
// 4-slot ring filled by direct global-to-LDS loads three tiles ahead). Its four
// waves are two head blocks of 32 x two halves: half e of a head block forms the
// scores over key values [288 e, 288 e + 288) and the output over latent values
// [256 e, 256 e + 256), so a wave holds half of Q (72 registers) and half of the
// accumulator (128). Per tile and wave:
//   * partial S^T (32 tokens x 32 heads) = K Q^T on v_mfma_f32_32x32x16_bf16,
//     18 K-steps; the two halves swap partial scores through LDS and add them
//     (a + b = b + a exactly, so both hold identical scores and take identical
//     decisions below);
//   * the probabilities, packed to bf16, are the B operand of O^T += V^T P^T
//     (8 blocks of 32 latent values; V^T read with ds_read_b64_tr_b16), and the
//     row sum is taken from the same packed values;
//   * the reference maximum is lazy, as in the prefill kernel: a lane whose tile
//     probabilities sum to at most 2^8 needs no rescale; otherwise the exact row
//     maximum moves the reference (first tile included).
// The tiles are software-pipelined: the score MFMAs of tile j + 1 are issued while
// the vector ALUs form tile j's probabilities, and tile j's PV MFMAs run while the
// halves swap tile j + 1's partial scores. The output accumulators stay in AGPRs.
// Partials: part_m holds each segment's reference in natural units, part_s and
// part_o the sum and the unnormalised accumulator relative to it -- the same
// triple the merge combines exactly whatever the reference is.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace rf {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int DQK = 576;                 // latent + rotary key width
constexpr int DV = 512;                  // latent width (the value)
constexpr int KT = 32;                   // tokens per tile
constexpr int RCH = DQK / 8;             // 16-byte chunks per cache row (72)
constexpr int TILE_CHUNKS = KT * RCH;    // 2304
constexpr int TILE_ELEMS = KT * DQK;     // 18432 bf16 = 36 KiB
constexpr int NCQ = DQK / 32;            // K=16 steps of one half's partial scores (18)
constexpr int DBV = DV / 64;             // 32-wide latent blocks of one half's output (8)
constexpr int STAGES = 4;                // ring slots: 4 x 36 KiB + 16 KiB of score exchange = 160 KiB
constexpr int NW = 4;                    // waves: 2 head blocks x 2 halves
constexpr int HPW = 64;                  // heads per workgroup

__device__ __forceinline__ uint32_t pack2(float a, float b) {
    bf16x2_t t = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, t);
}

__device__ __forceinline__ bf16x4_t read_tr16(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)(p));
}

// O^T += V^T P^T on an accumulator kept in AGPRs (the matrix instruction reads and writes
// them directly; the compiler would otherwise copy the 128 accumulator registers of a
// wave between AGPRs and VGPRs on every tile). As inline assembly the instruction is
// outside the compiler's hazard tracking, so the required wait states are explicit:
// FIRST puts 5 before the instruction, covering a vector ALU write of the P operand (or
// of the accumulator, by a rescale) just before it; accumulator chains on the same
// registers need none; reads of the accumulator after the last one wait in agpr_settle.
template <bool FIRST>
__device__ __forceinline__ void mfma_pv(f32x16& acc, const bf16x8& a, const bf16x8& b) {
    if constexpr (FIRST)
        asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
    else
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// 24 wait states before any other instruction touches the accumulators written by mfma_pv
// (more than the 18 a 16-pass matrix instruction needs before a vector read).
__device__ __forceinline__ void agpr_settle(f32x16 (&acc)[8]) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3]), "+a"(acc[4]), "+a"(acc[5]),
                   "+a"(acc[6]), "+a"(acc[7]));
}

// Element offset of logical 8-element chunk c of token row r inside a tile: the chunk
// index is XOR-swizzled with r & 7 (it stays inside its aligned group of 8 chunks).
__device__ __forceinline__ int tile_off(int r, int c) { return r * DQK + ((c ^ (r & 7)) << 3); }

__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_split_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, int64_t H, int64_t L,
                      int64_t nseg, int64_t seglen, int nhb, float sl2, uint32_t qsign, float* __restrict__ part_m,
                      float* __restrict__ part_s, float* __restrict__ part_o) {
    constexpr int WLT = TILE_CHUNKS / 64 / NW;   // wave loads per tile and wave
    __shared__ __attribute__((aligned(16))) uint16_t ring[STAGES * TILE_ELEMS];
    __shared__ __attribute__((aligned(16))) f32x4 xbuf[NW][4][64];    // partial scores, [reg/4][lane][4]

    // Workgroup -> (batch b, segment t, head block hb). Workgroups are dispatched round-robin
    // over the 8 XCDs; renumbering gives each XCD a contiguous range of logical ids, and the
    // head blocks of one (b, t) are consecutive ids, so they read the same cache tiles
    // through one L2.
    int64_t bid = blockIdx.x;
    const int64_t total = int64_t(gridDim.x);
    if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
    const int64_t hb = bid % nhb;
    const int64_t rest = bid / nhb;
    const int64_t t = rest % nseg;
    const int64_t b = rest / nseg;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, h = lane >> 5;
    const int blk = wave >> 1;               // head block (32 heads)
    const int half = wave & 1;               // key/latent half

    const int64_t s0 = t * seglen;
    const int64_t s1 = s0 + seglen < L ? s0 + seglen : L;
    const int ntiles = s1 > s0 ? int((s1 - s0 + KT - 1) / KT) : 0;
    const uint16_t* kvb = kv + b * L * DQK;

    // Tile j of the segment into ring slot `slot`: wave load i (i = wave + NW * w) covers
    // physical chunks [64 i, 64 i + 64) of the tile, so lane `lane` lands in token row
    // r = (64 i + lane) / RCH at physical chunk pc and fetches the logical chunk pc ^ (r & 7)
    // that the read side expects there. The byte offsets inside a tile do not depend on
    // the tile and are formed once; a tile that runs past the segment re-reads its last
    // token for the rows beyond it (their scores are masked).
    uint32_t goff[WLT];
#pragma unroll
    for (int w = 0; w < WLT; ++w) {
        const int p = (wave + NW * w) * 64 + lane;
        const int r = p / RCH;
        const int lc = (p - r * RCH) ^ (r & 7);
        goff[w] = uint32_t(r * DQK + lc * 8) * 2u;
    }
    const uint32_t ring_lds = lds_addr(ring);
    auto issue = [&](int j, int slot) {
        const int64_t k0 = s0 + int64_t(j) * KT;
        const uint16_t* gbase = kvb + k0 * DQK;                       // wave-uniform
        const uint32_t lbase = ring_lds + uint32_t(slot * TILE_ELEMS * 2);
        if (k0 + KT <= s1) {
#pragma unroll
            for (int w = 0; w < WLT; ++w) lds_dma16_sb(gbase, goff[w], lbase + uint32_t((wave + NW * w) * 1024));
        } else {
            const int rmax = int(s1 - 1 - k0);
#pragma unroll
            for (int w = 0; w < WLT; ++w) {
                const int r = ((wave + NW * w) * 64 + lane) / RCH;
                const int dr = r > rmax ? r - rmax : 0;              // rows past the end move back
                lds_dma16_sb(gbase, goff[w] - uint32_t(dr * DQK * 2), lbase + uint32_t((wave + NW * w) * 1024));
            }
        }
    };

    // Q^T operand: lane (head l32 of the block, lane half h) holds
    // Q[head][288 half + 16c + 8h .. +7].
    const int64_t head = hb * HPW + 32 * blk + l32;
    bf16x8 qf[NCQ];
    {
        const int64_t hq = head < H ? head : H - 1;
        const uint16_t* src = q + (b * H + hq) * DQK + 288 * half + 8 * h;
#pragma unroll
        for (int c = 0; c < NCQ; ++c) {
            u32x4 v4 = *reinterpret_cast<const u32x4*>(src + 16 * c);
            v4 ^= qsign;
            qf[c] = __builtin_bit_cast(bf16x8, v4);
        }
    }

    f32x16 acc_o[DBV];
#pragma unroll
    for (int d = 0; d < DBV; ++d) acc_o[d] = f32x16{};
    float m_ref = kNegInf, s_part = 0.f;
    const bf16x2_t ones = {(__bf16)1.f, (__bf16)1.f};

    // p = 2^(x sl2 - ref) for the 16 scores of the lane, packed to bf16. Returns the lane's
    // sum of the packed values.
    auto probs = [&](const f32x16& sc, uint32_t (&pk)[8]) {
        float t0 = 0.f, t1 = 0.f;
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const float p0 = exp2_fast(fmaf(sc[r], sl2, -m_ref));
            const float p1 = exp2_fast(fmaf(sc[r + 1], sl2, -m_ref));
            const uint32_t w = pack2(p0, p1);
            pk[r >> 1] = w;
            if (r & 2) t1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), ones, t1, false);
            else t0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), ones, t0, false);
        }
        return t0 + t1;
    };
    // Tail tiles: zero the probabilities of tokens at or past kvalid and return the new sum.
    // (Rows past the segment hold copies of its last token, so their scores are finite and
    // never exceed the valid maximum; only their weights must go.)
    auto mask_tail = [&](int kvalid, uint32_t (&pk)[8]) {
        float t = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int key = (i >> 1) * 8 + 4 * h + 2 * (i & 1);
            const uint32_t keep = (key < kvalid ? 0x0000FFFFu : 0u) | (key + 1 < kvalid ? 0xFFFF0000u : 0u);
            pk[i] &= keep;
            t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[i]), ones, t, false);
        }
        return t;
    };

    // Read-side LDS element offsets inside a tile, formed once. The swizzle only touches
    // the low three bits of a chunk index, so chunks 8 apart (and rows 8 apart) stay a
    // constant distance apart and every other read is an immediate offset from these.
    const int j16 = lane & 15;
    int kbase[4];                            // S: row l32, chunk 36 half + 2 cc + h (+8 per 4 K-steps)
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) kbase[cc] = tile_off(l32, 36 * half + 2 * cc + h);
    int vbase[2];                            // PV: token 4h + j/4, latent 256 half + 32 e + ...
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int col = 256 * half + 32 * e + 16 * (l32 >> 4) + 4 * (j16 & 3);
        const int key0 = 4 * h + (j16 >> 2);
        vbase[e] = tile_off(key0, col >> 3) + (col & 7);
    }

    // Partial S^T = K Q^T of one tile over this half's 288 key values. Two accumulators (even
    // and odd K-steps) halve the dependent MFMA chain; their sum is formed in a fixed order,
    // so both halves of a pair agree bit for bit once the partner's part is added.
    auto scores = [&](const uint16_t* tl) {
        f32x16 sc0 = f32x16{}, sc1 = f32x16{};
#pragma unroll
        for (int c = 0; c < NCQ; c += 2) {
            const u32x4 kf0 = *reinterpret_cast<const u32x4*>(tl + kbase[c & 3] + (c >> 2) * 64);
            const u32x4 kf1 = *reinterpret_cast<const u32x4*>(tl + kbase[(c + 1) & 3] + ((c + 1) >> 2) * 64);
            sc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf0), qf[c], sc0, 0, 0, 0);
            sc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf1), qf[c + 1], sc1, 0, 0, 0);
        }
        return sc0 + sc1;
    };
    // The two halves of a head block swap partial scores through LDS (one barrier).
    auto exchange = [&](f32x16 sc) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            xbuf[wave][q4][lane] = f32x4{sc[4 * q4], sc[4 * q4 + 1], sc[4 * q4 + 2], sc[4 * q4 + 3]};
        __syncthreads();
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 o = xbuf[wave ^ 1][q4][lane];
#pragma unroll
            for (int e = 0; e < 4; ++e) sc[4 * q4 + e] += o[e];
        }
        return sc;
    };
    // Probabilities of one tile's full scores (lazy reference; the exact path when a lane's
    // sum exceeds 2^8), accumulated into s_part.
    auto softmax = [&](const f32x16& sc, int kvalid, uint32_t (&pk)[8]) {
        float tsum = probs(sc, pk);
        if (kvalid < KT) tsum = mask_tail(kvalid, pk);
        if (__any(!(tsum <= 256.f))) {
            float mx = kNegInf;
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[r]);
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
            const float mx2 = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * sl2;
            if (mx2 > m_ref) {
                const float alpha = exp2_fast(m_ref - mx2);   // 0 on the first tile
                agpr_settle(acc_o);
                s_part *= alpha;
#pragma unroll
                for (int d = 0; d < DBV; ++d) acc_o[d] *= alpha;
                m_ref = mx2;
            }
            tsum = probs(sc, pk);
            if (kvalid < KT) tsum = mask_tail(kvalid, pk);
        }
        s_part += tsum;
    };
    // O^T += V^T P^T over the tile's two 16-token chunks; block d of 32 latent values
    // reads tokens key0 and key0 + 8 (16-lane group layout of the transposing read).
    auto pv = [&](const uint16_t* tl, const uint32_t (&pk)[8]) {
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            const u32x4 pb = {pk[kc * 4 + 0], pk[kc * 4 + 1], pk[kc * 4 + 2], pk[kc * 4 + 3]};
#pragma unroll
            for (int d = 0; d < DBV; ++d) {
                const uint16_t* vp = tl + vbase[d & 1] + kc * 16 * DQK + (d >> 1) * 64;
                const bf16x4_t lo = read_tr16(vp);
                const bf16x4_t hi = read_tr16(vp + 8 * DQK);
                const bf16x8_t va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                if (d == 0) mfma_pv<true>(acc_o[d], __builtin_bit_cast(bf16x8, va), __builtin_bit_cast(bf16x8, pb));
                else mfma_pv<false>(acc_o[d], __builtin_bit_cast(bf16x8, va), __builtin_bit_cast(bf16x8, pb));
            }
        }
    };
    auto kvalid_of = [&](int j) {
        const int64_t kleft = s1 - (s0 + int64_t(j) * KT);
        return kleft < KT ? int(kleft) : KT;
    };

    // Software pipeline over tiles: iteration j forms tile j + 1's scores on the matrix cores
    // while the vector ALUs form tile j's probabilities, then runs tile j's PV and swaps tile
    // j + 1's partial scores. Ring protocol (4 slots): tile t lives in slot t % 4 and is
    // issued three tiles before its scores are formed; at the first barrier of iteration j,
    // tile j + 1 has landed and tile j - 1's slot (last read by the PV of iteration j - 1)
    // is free for tile j + 3.
    if (ntiles > 0) {
        issue(0, 0);
        if (ntiles > 1) issue(1, 1);
        if (ntiles > 2) issue(2, 2);
        if (ntiles > 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * WLT) : "memory");   // tile 0 is in
        else if (ntiles > 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(WLT) : "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        f32x16 sc = exchange(scores(ring));
        int j = 0;
        for (; j + 1 < ntiles; ++j) {
            if (j + 2 < ntiles) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(WLT) : "memory");   // tile j + 1 is in
            else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (j + 3 < ntiles) issue(j + 3, (j + 3) % STAGES);
            const f32x16 nxt = scores(ring + ((j + 1) % STAGES) * TILE_ELEMS);
            uint32_t pk[8];
            softmax(sc, kvalid_of(j), pk);
            pv(ring + (j % STAGES) * TILE_ELEMS, pk);
            sc = exchange(nxt);
        }
        uint32_t pk[8];
        softmax(sc, kvalid_of(j), pk);
        pv(ring + (j % STAGES) * TILE_ELEMS, pk);
    }

    agpr_settle(acc_o);
    // Partials of (row = b * H + head, segment t); both halves hold the same m and s.
    const float s_row = s_part + __shfl_xor(s_part, 32, 64);
    if (head < H) {
        const int64_t pr = (b * H + head) * nseg + t;
        if (h == 0 && half == 0) {
            part_m[pr] = m_ref == kNegInf ? kNegInf : m_ref * kLn2;
            part_s[pr] = s_row;
        }
        float* po = part_o + pr * DV + 256 * half;
#pragma unroll
        for (int d = 0; d < DBV; ++d)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                // acc_o[d][4 g4 + e] = O^T[32 d + 8 g4 + 4 h + e][head].
                const float4 w = make_float4(acc_o[d][4 * g4], acc_o[d][4 * g4 + 1], acc_o[d][4 * g4 + 2],
                                             acc_o[d][4 * g4 + 3]);
                *reinterpret_cast<float4*>(po + 32 * d + 8 * g4 + 4 * h) = w;
            }
    }
}

hipError_t launch_blocks(const uint16_t* q, const uint16_t* kv, int64_t B, int64_t H, int64_t L, int64_t nseg,
                        float scale, float* part_m, float* part_s, float* part_o, hipStream_t stream) {
    const int64_t nhb = ceil_div(H, int64_t(HPW));
    const int64_t blocks = B * nhb * nseg;
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    const int64_t seglen = ceil_div(L, nseg);
    const float sl2 = (scale < 0.f ? -scale : scale) * kLog2e;
    const uint32_t qsign = scale < 0.f ? 0x80008000u : 0u;
    hipLaunchKernelGGL(mla_split_kernel, dim3(unsigned(blocks)), dim3(NW * 64), 0, stream, q, kv, H, L, nseg, seglen,
                       int(nhb), sl2, qsign, part_m, part_s, part_o);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mla_decode_split(const uint16_t* q, const uint16_t* kv, int64_t B, int64_t H, int64_t L,
                                   int64_t nseg, float scale, float* part_m, float* part_s, float* part_o,
                                   hipStream_t stream) {
    return launch_blocks(q, kv, B, H, L, nseg, scale, part_m, part_s, part_o, stream);
}

}  // namespace rf
