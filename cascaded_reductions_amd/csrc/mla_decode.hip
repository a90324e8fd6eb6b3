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
// 4-slot ring filled by direct global-to-LDS loads three tiles ahead). Its eight
// waves are four head blocks of 16 x two halves: half e of a head block forms
// the scores over key values [288 e, 288 e + 288) and the output over latent
// values [256 e, 256 e + 256), so a wave holds 36 registers of Q and 64 of
// accumulator, and two waves share each SIMD. Per tile and wave, on
// v_mfma_f32_16x16x32_bf16:
//   * partial S^T (two blocks of 16 tokens x 16 heads) = K Q^T, 9 K-steps each;
//     the two halves swap partial scores through LDS and add them (a + b = b + a
//     exactly, so both hold identical scores and take identical decisions);
//   * the score MFMAs take the tile's tokens in an order that leaves each lane
//     group holding eight consecutive tokens, so the probabilities, packed to
//     bf16, are directly the B operand of O^T += V^T P^T (16 blocks of 16 latent
//     values, the 32 tokens as K; V^T read with ds_read_b64_tr_b16), and the row
//     sum is taken from the same packed values;
//   * the reference maximum is lazy, as in the prefill kernel: a lane whose tile
//     probabilities sum to at most 2^8 needs no rescale; otherwise the exact row
//     maximum moves the reference (first tile included).
// The tiles are software-pipelined: the score MFMAs of tile j + 1 are issued while
// the vector ALUs form tile j's probabilities, and tile j's PV MFMAs run while the
// halves swap tile j + 1's partial scores.
// Partials: part_m holds each segment's reference in natural units, part_s and
// part_o the sum and the unnormalised accumulator relative to it -- the same
// triple the merge combines exactly whatever the reference is.
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
constexpr int NCQ = DQK / 2 / 32;        // K=32 steps of one half's partial scores (9)
constexpr int DBV = DV / 2 / 16;         // 16-wide latent blocks of one half's output (16)
constexpr int STAGES = 4;                // ring slots: 4 x 36 KiB + 16 KiB of score exchange = 160 KiB
constexpr int NW = 8;                    // waves: 4 head blocks of 16 x 2 halves
constexpr int HPW = 64;                  // heads per workgroup
constexpr int NLD = 4;                   // waves 0-3 fill the ring
constexpr int WLT = TILE_CHUNKS / 64 / NLD;   // wave loads per tile and loading wave (9)


__device__ __forceinline__ uint32_t pack2(float a, float b) {
    bf16x2_t t = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, t);
}

__device__ __forceinline__ bf16x4_t read_tr16(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)(p));
}

// Element offset of logical 8-element chunk c of token row r inside a tile: the chunk
// index is XOR-swizzled with row_swz(r) < 8 (it stays inside its aligned group of 8
// chunks). The LDS serves 256 bytes per cycle, and a row is 1152 bytes, so rows of one
// parity share the 128-byte bank halves. The score reads of a 16-lane group take rows
// 8a + 4tb + b (a, b in 0..3) at one chunk, and the transposed V reads of a 32-lane group
// take rows 8a' + b + 4hi at two adjacent chunks, with a' in {0, 1} or {0, 2} depending
// on how the hardware pairs the lane groups. Chunk bit 0 = row bit 3, bit 1 = row bit 1,
// bit 2 = row bit 3 ^ row bit 4 gives every row of one parity its own banks in each of
// these groups (an XOR with r & 7 would put rows 8 apart on the same ones).
__device__ __forceinline__ int row_swz(int r) {
    return ((r >> 3) & 1) | (((r >> 1) & 1) << 1) | ((((r >> 3) ^ (r >> 4)) & 1) << 2);
}
__device__ __forceinline__ int tile_off(int r, int c) { return r * DQK + ((c ^ row_swz(r)) << 3); }

__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mla_split_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, int64_t H, int64_t L,
                      int64_t nseg, int64_t seglen, int nhb, float sl2, uint32_t qsign, float* __restrict__ part_m,
                      float* __restrict__ part_s, float* __restrict__ part_o) {
    __shared__ __attribute__((aligned(16))) uint16_t ring[STAGES * TILE_ELEMS];
    __shared__ __attribute__((aligned(16))) f32x4 xbuf[NW][2][64];    // partial scores, [token block][lane]

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
    const int l16 = lane & 15, g = lane >> 4;
    const int blk = wave >> 1;               // head block (16 heads)
    const int half = wave & 1;               // key/latent half

    const int64_t s0 = t * seglen;
    const int64_t s1 = s0 + seglen < L ? s0 + seglen : L;
    const int ntiles = s1 > s0 ? int((s1 - s0 + KT - 1) / KT) : 0;
    const uint16_t* kvb = kv + b * L * DQK;

    // Tile j of the segment into ring slot `slot`, by waves 0-3: wave load i (i = wave +
    // NLD * w) covers physical chunks [64 i, 64 i + 64) of the tile, so lane `lane` lands in
    // token row r = (64 i + lane) / RCH at physical chunk pc and fetches the logical chunk
    // pc ^ row_swz(r) that the read side expects there. A tile that runs past the segment
    // re-reads its last token for the rows beyond it (their weights are zeroed).
    const bool loader = wave < NLD;
    uint32_t goff[WLT];
#pragma unroll
    for (int w = 0; w < WLT; ++w) {
        const int p = (wave % NLD + NLD * w) * 64 + lane;
        const int r = p / RCH;
        const int lc = (p - r * RCH) ^ row_swz(r);
        goff[w] = uint32_t(r * DQK + lc * 8) * 2u;
    }
    const uint32_t ring_lds = lds_addr(ring);
    auto issue = [&](int j, int slot) {
        if (!loader) return;
        const int64_t k0 = s0 + int64_t(j) * KT;
        const uint16_t* gbase = kvb + k0 * DQK;                       // wave-uniform
        const uint32_t lbase = ring_lds + uint32_t(slot * TILE_ELEMS * 2);
        if (k0 + KT <= s1) {
#pragma unroll
            for (int w = 0; w < WLT; ++w) lds_dma16_sb(gbase, goff[w], lbase + uint32_t((wave + NLD * w) * 1024));
        } else {
            const int rmax = int(s1 - 1 - k0);
#pragma unroll
            for (int w = 0; w < WLT; ++w) {
                const int r = ((wave + NLD * w) * 64 + lane) / RCH;
                const int dr = r > rmax ? r - rmax : 0;              // rows past the end move back
                lds_dma16_sb(gbase, goff[w] - uint32_t(dr * DQK * 2), lbase + uint32_t((wave + NLD * w) * 1024));
            }
        }
    };

    // Q^T operand (B of S^T = K Q^T on v_mfma_f32_16x16x32_bf16): lane (head l16 of the
    // block, group g) holds Q[head][288 half + 32 c + 8 g .. +7].
    const int64_t head = hb * HPW + 16 * blk + l16;
    bf16x8 qf[NCQ];
    {
        const int64_t hq = head < H ? head : H - 1;
        const uint16_t* src = q + (b * H + hq) * DQK + 288 * half + 8 * g;
#pragma unroll
        for (int c = 0; c < NCQ; ++c) {
            u32x4 v4 = *reinterpret_cast<const u32x4*>(src + 32 * c);
            v4 ^= qsign;
            qf[c] = __builtin_bit_cast(bf16x8, v4);
        }
    }

    // acc_o[d][r] = O^T[256 half + 16 d + 4 g + r][head].
    f32x4 acc_o[DBV];
#pragma unroll
    for (int d = 0; d < DBV; ++d) acc_o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_ref = kNegInf, s_part = 0.f;
    const bf16x2_t ones = {(__bf16)1.f, (__bf16)1.f};

    // Token order of the score MFMAs: row i of token block tb is token 8 (i / 4) + 4 tb + i % 4,
    // so the accumulator rows a lane holds (4 g + r of blocks 0 and 1) are tokens 8 g .. 8 g + 7,
    // exactly the eight consecutive tokens the P^T operand of PV takes from lane group g.
    // p = 2^(x sl2 - ref) for the lane's 8 scores, packed to bf16 in token order.
    auto probs = [&](const f32x4 (&sc)[2], uint32_t (&pk)[4]) {
        float t0 = 0.f, t1 = 0.f;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const float p0 = exp2_fast(fmaf(sc[tb][0], sl2, -m_ref));
            const float p1 = exp2_fast(fmaf(sc[tb][1], sl2, -m_ref));
            const float p2 = exp2_fast(fmaf(sc[tb][2], sl2, -m_ref));
            const float p3 = exp2_fast(fmaf(sc[tb][3], sl2, -m_ref));
            const uint32_t w0 = pack2(p0, p1), w1 = pack2(p2, p3);
            pk[2 * tb] = w0;
            pk[2 * tb + 1] = w1;
            t0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w0), ones, t0, false);
            t1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w1), ones, t1, false);
        }
        return t0 + t1;
    };
    // Tail tiles: zero the weights of tokens at or past kvalid and return the new sum. (Rows
    // past the segment hold copies of its last token, so their scores are finite and never
    // exceed the valid maximum; only their weights must go.)
    auto mask_tail = [&](int kvalid, uint32_t (&pk)[4]) {
        float tt = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = 8 * g + 2 * i;
            const uint32_t keep = (key < kvalid ? 0x0000FFFFu : 0u) | (key + 1 < kvalid ? 0xFFFF0000u : 0u);
            pk[i] &= keep;
            tt = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[i]), ones, tt, false);
        }
        return tt;
    };

    // Read-side LDS element offsets inside a tile, formed once. The swizzle only touches
    // the low three bits of a chunk index, so chunks 8 apart stay a constant distance apart.
    int kbase[2][2];                         // S: token row of (tb, lane), chunk 36 half + g + 4 (c & 1)
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int e = 0; e < 2; ++e) kbase[tb][e] = tile_off(8 * (l16 >> 2) + 4 * tb + (l16 & 3), 36 * half + g + 4 * e);
    int vbase[4][2];                         // PV: tokens 8 g + l16 / 4 (+4), latent 256 half + 16 d + 4 (l16 % 4)
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int hi = 0; hi < 2; ++hi) {
            const int col = 256 * half + 16 * e + 4 * (l16 & 3);
            const int key = 8 * g + (l16 >> 2) + 4 * hi;
            vbase[e][hi] = tile_off(key, col >> 3) + (col & 7);
        }

    // Partial S^T of one tile over this half's 288 key values: two token blocks of 16.
    auto scores = [&](const uint16_t* tl, f32x4 (&sc)[2]) {
        sc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
        sc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NCQ; ++c)
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                const u32x4 kf = *reinterpret_cast<const u32x4*>(tl + kbase[tb][c & 1] + (c >> 1) * 64);
                sc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf), qf[c], sc[tb], 0, 0, 0);
            }
    };
    // The two halves of a head block swap partial scores through LDS (one barrier); the sum
    // is formed in a fixed order, so both halves hold identical scores.
    auto exchange = [&](f32x4 (&sc)[2]) {
        xbuf[wave][0][lane] = sc[0];
        xbuf[wave][1][lane] = sc[1];
        __syncthreads();
        const f32x4 o0 = xbuf[wave ^ 1][0][lane];
        const f32x4 o1 = xbuf[wave ^ 1][1][lane];
        if (half == 0) {
            sc[0] = sc[0] + o0;
            sc[1] = sc[1] + o1;
        } else {
            sc[0] = o0 + sc[0];
            sc[1] = o1 + sc[1];
        }
    };
    auto softmax = [&](const f32x4 (&sc)[2], int kvalid, uint32_t (&pk)[4]) {
        float tsum = probs(sc, pk);
        if (kvalid < KT) tsum = mask_tail(kvalid, pk);
        if (__any(!(tsum <= 256.f))) {
            float mx = kNegInf;
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[tb][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float mx2 = mx * sl2;
            if (mx2 > m_ref) {
                const float alpha = exp2_fast(m_ref - mx2);   // 0 on the first tile
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
    // O^T += V^T P^T: 16 blocks of 16 latent values, the tile's 32 tokens as K.
    auto pv = [&](const uint16_t* tl, const uint32_t (&pk)[4]) {
        const u32x4 pb = {pk[0], pk[1], pk[2], pk[3]};
#pragma unroll
        for (int d = 0; d < DBV; ++d) {
            const bf16x4_t lo = read_tr16(tl + vbase[d & 3][0] + (d >> 2) * 64);
            const bf16x4_t hi = read_tr16(tl + vbase[d & 3][1] + (d >> 2) * 64);
            const bf16x8_t va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            acc_o[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va),
                                                                __builtin_bit_cast(bf16x8, pb), acc_o[d], 0, 0, 0);
        }
    };
    auto kvalid_of = [&](int j) {
        const int64_t kleft = s1 - (s0 + int64_t(j) * KT);
        return kleft < KT ? int(kleft) : KT;
    };

    // Software pipeline over tiles (as in the 32-head form): iteration j forms tile j + 1's
    // scores while the vector ALUs form tile j's probabilities, then runs tile j's PV and
    // swaps tile j + 1's partial scores. Ring protocol (4 slots): tile t lives in slot t % 4
    // and is issued three tiles before its scores are formed.
    if (ntiles > 0) {
        issue(0, 0);
        if (ntiles > 1) issue(1, 1);
        if (ntiles > 2) issue(2, 2);
        if (ntiles > 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * WLT) : "memory");   // tile 0 is in
        else if (ntiles > 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(WLT) : "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        f32x4 sc[2];
        scores(ring, sc);
        exchange(sc);
        int j = 0;
        for (; j + 1 < ntiles; ++j) {
            if (j + 2 < ntiles) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(WLT) : "memory");   // tile j + 1 is in
            else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (j + 3 < ntiles) issue(j + 3, (j + 3) % STAGES);
            f32x4 nxt[2];
            scores(ring + ((j + 1) % STAGES) * TILE_ELEMS, nxt);
            uint32_t pk[4];
            softmax(sc, kvalid_of(j), pk);
            pv(ring + (j % STAGES) * TILE_ELEMS, pk);
            exchange(nxt);
            sc[0] = nxt[0];
            sc[1] = nxt[1];
        }
        uint32_t pk[4];
        softmax(sc, kvalid_of(j), pk);
        pv(ring + (j % STAGES) * TILE_ELEMS, pk);
    }

    // Partials of (row = b * H + head, segment t); the four lane groups of a head hold a
    // quarter of its tokens each, and both halves hold the same m and s.
    float s_row = s_part + __shfl_xor(s_part, 16, 64);
    s_row = s_row + __shfl_xor(s_row, 32, 64);
    if (head < H) {
        const int64_t pr = (b * H + head) * nseg + t;
        if (g == 0 && half == 0) {
            part_m[pr] = m_ref == kNegInf ? kNegInf : m_ref * kLn2;
            part_s[pr] = s_row;
        }
        float* po = part_o + pr * DV + 256 * half + 4 * g;
#pragma unroll
        for (int d = 0; d < DBV; ++d)
            *reinterpret_cast<float4*>(po + 16 * d) = make_float4(acc_o[d][0], acc_o[d][1], acc_o[d][2], acc_o[d][3]);
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
