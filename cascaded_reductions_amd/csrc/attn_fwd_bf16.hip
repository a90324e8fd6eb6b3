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
// gfx950 mapping (wave64, v_mfma_f32_32x32x16_bf16):
//  * A workgroup is 4 waves: 2 blocks of 32 query rows x 2 halves of the key
//    axis. Each wave runs the incremental loop over its half; the two halves'
//    states are combined through LDS at the end with the same (max, sum,
//    partial-O) merge that joins segments (an intra-block use of the merge).
//    With 64 query rows per workgroup, the 8 x 12 x 512 prefill has 768
//    workgroups: exactly 3 per CU and 3 waves per SIMD.
//  * S^T = K Q^T: the Q^T operand stays in registers; in the 32x32 accumulator
//    layout each lane owns one query row (lane % 32) and 16 of every 32 keys,
//    so the row maximum needs one cross-lane step (lanes l and l ^ 32).
//  * O^T += V^T P^T: the probabilities, packed to bf16 in registers, are the B
//    operand as they stand; V^T comes from LDS through the transposing read
//    (ds_read_b64_tr_b16), so V is never transposed in memory. The row sum is
//    taken from the same packed bf16 values with v_dot2_f32_bf16, so numerator
//    and denominator see identical probabilities.
//  * K/V tiles of 32 keys per half go to LDS with direct global-to-LDS loads
//    (no registers) into a 3-slot K ring and a 3-slot V ring, issued two loop
//    iterations before their first use; 16-byte chunks are XOR-swizzled per
//    key row so the K reads and the transposed V reads avoid bank conflicts.
//  * The loop is software-pipelined: the scores of step j + 1 go to the matrix
//    cores before the softmax (vector ALU) and PV of step j, so both units work
//    at once within each wave, on top of the overlap between the 3 waves that
//    share a SIMD.
//  * The reference maximum moves (and the state is rescaled) only when a tile's
//    maximum exceeds it by more than 2^8; exponentials up to 2^8 are otherwise
//    accumulated against the stale reference. This is exact in exact arithmetic
//    (the reference cancels in o~ / s and in lse = ref + log s).
//  * Workgroups of one head are placed on one XCD (workgroups are dispatched
//    round-robin over the 8 XCDs), so the head's K and V are fetched into that
//    XCD's L2 once.
//  * The output leaves through an LDS staging tile as whole 128-byte lines with
//    streaming stores, so no dirty lines wait in L2 for the end-of-kernel write-back.
#include <type_traits>

#include "attn_tiles.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace rf {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

constexpr int KT = 32;              // keys per tile (per key half)
constexpr float kRescaleSlack = 8.f;

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    bf16x2_t t = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, t);
}

__device__ __forceinline__ bf16x4_t lds_read_tr16(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)(p));
}


template <int D, int STAGES, bool EXACT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 64 ? 3 : 1)))
void attn_fwd_bf16_kernel(const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ k,
                                                            const uint16_t* __restrict__ v,
                                                            uint16_t* __restrict__ o, float* __restrict__ lse,
                                                            int64_t Sq, int64_t Sk, int nqb, float sl2,
                                                            uint32_t qsign) {
    constexpr int CH = D / 8;                 // 16-byte chunks per key row
    constexpr int TILE = KT * D;              // elements of one K (or V) tile
    constexpr int SLOT = 2 * TILE;            // one ring slot: the tile of both key halves
    constexpr int STEP = 2 * SLOT;            // LDS per step of ring depth (a K slot and a V slot)
    constexpr int WL = TILE * 2 / 1024;       // 1 KiB wave loads per tile
    constexpr int RPW = 64 / CH;              // key rows per wave load
    constexpr int NC = D / 16;                // K=16 slices of the head dimension
    constexpr int DB = D / 32;                // 32-wide output column blocks
    static_assert(STAGES * STEP * 2 >= 2 * (DB * 16 + 2) * 64 * 4 + 2 * 32 * (D + 8) * 2,
                  "LDS must also hold the merge buffers and the output staging tile");

    // A ring of STAGES K slots followed by a ring of STAGES V slots.
    __shared__ __attribute__((aligned(16))) uint16_t smem[STAGES * STEP];
    uint16_t* const kring = smem;
    uint16_t* const vring = smem + STAGES * SLOT;

    // Workgroup -> (head, block of 64 queries); heads stay on one XCD when the grid divides by 8.
    int64_t bid = blockIdx.x;
    const int64_t total = int64_t(gridDim.x);
    if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
    const int64_t bh = bid / nqb;
    const int64_t q0 = (bid - bh * nqb) * 64;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // scalar: derived values live in SGPRs
    const int l32 = lane & 31, h = lane >> 5;
    const int qh = wave & 1;                  // query block of this wave
    const int kh = wave >> 1;                 // key half of this wave

    // Per-head bases in 64-bit once; all offsets inside a head are 32-bit (the host
    // guarantees Sk * D < 2^30).
    const uint16_t* kh_ptr = k + bh * Sk * D;
    const uint16_t* vh_ptr = v + bh * Sk * D;
    const int sk = int(Sk);

    // Q^T operand: lane (query l32, half h) holds Q[row][16c + 8h .. +7]; the sign of
    // Q is flipped for a negative scale so that sl2 = |scale| log2(e) >= 0.
    const int64_t qrow = q0 + 32 * qh + l32;
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

    const int nt = (sk + KT - 1) / KT;        // tiles over the whole key axis
    const int half0 = (nt + 1) / 2;           // tiles of key half 0; half 1 has nt - half0
    const int nsteps = half0;
    const int my_first = kh ? half0 : 0;      // first tile of this wave's key half
    const int my_tiles = kh ? nt - half0 : half0;

    // Wave w fills tile (half w>>1, K if w even else V) of a step: WL wave loads of 1 KiB;
    // lane i lands in row l*RPW + i/CH, physical chunk i%CH, and fetches the logical chunk
    // that the read-side swizzle maps there. Tiles past the end re-read the last tile, so
    // every wave issues the same number of loads per step (the wait counts rely on it).
    const int ld_half = wave >> 1, ld_kind = wave & 1;
    const uint16_t* ld_src = ld_kind ? vh_ptr : kh_ptr;
    const int ld_first = ld_half ? half0 : 0;
    uint32_t ld_off[WL];                      // byte offset of this lane's chunk within a tile
#pragma unroll
    for (int l = 0; l < WL; ++l) {
        const int row = l * RPW + lane / CH;
        const int pc = lane % CH;
        const int lc = ld_kind ? (pc ^ attn_v_swz<D>(row)) : (pc ^ attn_k_swz<D>(row));
        ld_off[l] = uint32_t(row * D + lc * 8) * 2u;
    }
    const uint32_t ld_lds0 = lds_addr(smem) + uint32_t(((ld_kind ? STAGES * SLOT : 0) + ld_half * TILE) * 2);
    auto issue = [&](int step, int stage) {
        int t = ld_first + step;
        t = t < nt ? t : nt - 1;
        const uint16_t* gbase = ld_src + int64_t(t) * KT * D;   // scalar
        const uint32_t lbase = ld_lds0 + uint32_t(stage * SLOT * 2);
        if (EXACT || t * KT + KT <= sk) {
#pragma unroll
            for (int l = 0; l < WL; ++l) lds_dma16_sb(gbase, ld_off[l], lbase + l * 1024);
        } else {                              // the last tile runs past the key axis: clamp rows
            const uint32_t last = uint32_t((sk - 1 - t * KT) * D * 2);
#pragma unroll
            for (int l = 0; l < WL; ++l) {
                const uint32_t col = ld_off[l] & uint32_t(D * 2 - 1);
                const uint32_t off = ld_off[l] - col > last ? last + col : ld_off[l];
                lds_dma16_sb(gbase, off, lbase + l * 1024);
            }
        }
    };

    f32x16 acc_o[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) acc_o[b] = f32x16{};
    float m_ref = kNegInf, s_part = 0.f;
    const bf16x2_t ones = {(__bf16)1.f, (__bf16)1.f};

    // Read-side LDS element offsets (constant across steps).
    int k_off[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) k_off[c] = l32 * D + (((2 * c + h) ^ attn_k_swz<D>(l32)) << 3);
    int v_off[2][DB][2];
    {
        const int j16 = lane & 15;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int b = 0; b < DB; ++b) {
                // 16-lane group: rows kc*16 + 4h + j/4 (+8), columns 32b + 16*(l32/16) + 4*(j%4).
                const int d = 32 * b + 16 * (l32 >> 4) + 4 * (j16 & 3);
                const int key0 = kc * 16 + 4 * h + (j16 >> 2);
                const int key1 = key0 + 8;
                v_off[kc][b][0] = key0 * D + (((d >> 3) ^ attn_v_swz<D>(key0)) << 3) + (d & 7);
                v_off[kc][b][1] = key1 * D + (((d >> 3) ^ attn_v_swz<D>(key1)) << 3) + (d & 7);
            }
    }

    // ---- building blocks of one step ------------------------------------------------

    // S^T (32 keys x 32 queries) of one step: K fragments from LDS, then the MFMA chain.
    auto load_k = [&](int stage, u32x4 (&kf)[NC]) {
        const uint16_t* ks = kring + stage * SLOT + kh * TILE;
#pragma unroll
        for (int c = 0; c < NC; ++c) kf[c] = *reinterpret_cast<const u32x4*>(ks + k_off[c]);
    };
    auto mfma_s = [&](const u32x4 (&kf)[NC]) {
        f32x16 acc = f32x16{};
#pragma unroll
        for (int c = 0; c < NC; ++c)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[c]), qf[c], acc, 0, 0, 0);
        return acc;
    };
    auto scores = [&](int stage) {
        u32x4 kf[NC];
        load_k(stage, kf);
        return mfma_s(kf);
    };
    // Keys of the lane's 16 accumulator entries at or past kvalid become -inf.
    auto mask_tail = [&](f32x16& acc_s, int kvalid) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = (r >> 2) * 8 + 4 * h + (r & 3);
            if (key >= kvalid) acc_s[r] = kNegInf;
        }
    };
    // Row maximum in base-2 units: lanes l and l ^ 32 hold the two halves of the row's keys.
    auto rowmax2 = [&](const f32x16& acc_s) {
        float mx = fmaxf(fmaxf(acc_s[0], acc_s[1]), acc_s[2]);
#pragma unroll
        for (int r = 3; r < 15; r += 2) mx = fmaxf(fmaxf(mx, acc_s[r]), acc_s[r + 1]);
        mx = fmaxf(mx, acc_s[15]);
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * sl2;
    };
    // Move the reference maximum if the step's maximum exceeds it by more than the slack.
    auto rescale = [&](float mx2) {
        const bool need = mx2 > m_ref + kRescaleSlack;
        if (__any(need)) {
            const float ref = need ? mx2 : m_ref;
            const float alpha = exp2_fast(m_ref - ref);   // -inf -> 0 on the first tile
            s_part *= alpha;
#pragma unroll
            for (int b = 0; b < DB; ++b) acc_o[b] *= alpha;
            m_ref = ref;
        }
    };
    // p = 2^(x - ref) packed to bf16 (the P^T operand); the row sum reads the packed pairs.
    // MASK: zero the probabilities of keys past kvalid (with a zero scale a masked -inf
    // score would give NaN).
    auto probs = [&](auto mask_tag, const f32x16& acc_s, int kvalid, uint32_t (&pk)[8]) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            float p0 = exp2_fast(fmaf(acc_s[r], sl2, -m_ref));
            float p1 = exp2_fast(fmaf(acc_s[r + 1], sl2, -m_ref));
            if constexpr (decltype(mask_tag)::value) {
                const int key = (r >> 2) * 8 + 4 * h + (r & 3);
                p0 = key < kvalid ? p0 : 0.f;
                p1 = key + 1 < kvalid ? p1 : 0.f;
            }
            pk[r >> 1] = pack_bf16(p0, p1);
            s_part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[r >> 1]), ones, s_part, false);
        }
    };
    // O^T += V^T P^T over two 16-key chunks.
    auto pv = [&](int stage, const auto& pk) {
        const uint16_t* vs = vring + stage * SLOT + kh * TILE;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            const u32x4 pb = {pk[kc * 4 + 0], pk[kc * 4 + 1], pk[kc * 4 + 2], pk[kc * 4 + 3]};
#pragma unroll
            for (int b = 0; b < DB; ++b) {
                const bf16x4_t lo = lds_read_tr16(vs + v_off[kc][b][0]);
                const bf16x4_t hi = lds_read_tr16(vs + v_off[kc][b][1]);
                const bf16x8_t va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                acc_o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va),
                                                                    __builtin_bit_cast(bf16x8, pb), acc_o[b], 0, 0,
                                                                    0);
            }
        }
    };

    if constexpr (EXACT) {
        // ---- key axis a multiple of 2 * KT: every tile full, nsteps per key half -----------
        // Step j (of a key half) issues the score MFMAs of tile j + 1 and the PV MFMAs of
        // tile j - 1 while the vector ALUs form tile j's probabilities, so all eight MFMAs
        // of a step overlap the softmax work of the same wave. Ring protocol (3 K slots,
        // 3 V slots): at the top of step j, K(j + 1) and V(j - 1) have landed; the K
        // loaders then refill K(j)'s slot with K(j + 3) and the V loaders V(j - 2)'s slot
        // with V(j + 1) (both read for the last time in step j - 1), so every tile is issued
        // two steps before its first use. Ring slots repeat every 3 steps and the score and
        // probability buffers every 2, so the loop is unrolled 6 times and no buffer is
        // ever copied.
        //
        // The reference maximum starts at the first tile's maximum; afterwards a tile's row
        // maximum is only formed when needed: a lane whose probabilities (against the
        // current reference) sum to at most 2^8 has every probability at most 2^8, which is
        // all the lazy reference requires, so only a larger or non-finite sum sends the
        // wave through the exact path (row maximum, move of the reference if the maximum is
        // above it, probabilities again).
        const bool k_loader = ld_kind == 0;
        if (k_loader) {
            // K tiles are issued only up to the half's last one, so no load is left in flight
            // past the end of the loop; the waits below count what is actually in flight.
            issue(0, 0);
            if (nsteps > 1) issue(1, 1);
            if (nsteps > 2) issue(2, 2);
            if (nsteps > 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * WL) : "memory");   // K(0) is in
            else if (nsteps > 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(WL) : "memory");
            else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        } else {
            issue(0, 0);
        }
        __syncthreads();
        f32x16 sa = scores(0), sb;
        m_ref = rowmax2(sa);
        auto probs_sum = [&](const f32x16& sc, u32x8& pk) {
            float t0 = 0.f, t1 = 0.f;
#pragma unroll
            for (int r = 0; r < 16; r += 4) {
                const float p0 = exp2_fast(fmaf(sc[r], sl2, -m_ref));
                const float p1 = exp2_fast(fmaf(sc[r + 1], sl2, -m_ref));
                const float p2 = exp2_fast(fmaf(sc[r + 2], sl2, -m_ref));
                const float p3 = exp2_fast(fmaf(sc[r + 3], sl2, -m_ref));
                // (Packed words go through scalars: a bit cast of a vector element reads element 0.)
                const uint32_t w0 = pack_bf16(p0, p1), w1 = pack_bf16(p2, p3);
                pk[r >> 1] = w0;
                pk[(r >> 1) + 1] = w1;
                t0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w0), ones, t0, false);
                t1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w1), ones, t1, false);
            }
            return t0 + t1;
        };
        auto settle = [&](const f32x16& sc, u32x8& pk, float t) {
            if (__any(!(t <= 256.f))) {
                const float mx2 = rowmax2(sc);
                if (mx2 > m_ref) {
                    const float alpha = exp2_fast(m_ref - mx2);
                    s_part *= alpha;
#pragma unroll
                    for (int b = 0; b < DB; ++b) acc_o[b] *= alpha;
                    m_ref = mx2;
                }
                t = probs_sum(sc, pk);
            }
            s_part += t;
        };
        // One step with a successor tile. J = j mod 3 (compile time).
        auto step = [&](int j, auto j_tag, auto first_tag, const f32x16& s_cur, f32x16& s_next,
                        const u32x8& pk_prev, u32x8& pk_cur) {
            constexpr int J = decltype(j_tag)::value % 3;
            constexpr bool FIRST = decltype(first_tag)::value;
            constexpr int KS1 = (J + 1) % 3;     // K(j + 1)
            constexpr int VP = (J + 2) % 3;      // V(j - 1)
            u32x4 kf[NC];
            // K(j + 1) / V(j - 1) are in (a K loader with no K(j + 2) in flight waits for all).
            if (k_loader && j + 2 >= nsteps) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(WL) : "memory");
            __syncthreads();
            if (k_loader) {
                if (j + 3 < nsteps) issue(j + 3, J);   // into K(j)'s slot
            } else {
                issue(j + 1, KS1);                  // into V(j - 2)'s slot
            }
            load_k(KS1, kf);
            s_next = mfma_s(kf);
            if constexpr (!FIRST) pv(VP, pk_prev);
            const float t = probs_sum(s_cur, pk_cur);
            if constexpr (FIRST) {
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x402, 12, 0);   // then VALU work
                }
            } else {
                __builtin_amdgcn_sched_group_barrier(0x100, NC + 4 * DB, 0);   // K and V reads
#pragma unroll
                for (int c = 0; c < NC + 2 * DB; ++c) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x402, 6, 0);
                }
            }
            settle(s_cur, pk_cur, t);
        };
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using I2 = std::integral_constant<int, 2>;
        using I3 = std::integral_constant<int, 3>;
        using I4 = std::integral_constant<int, 4>;
        using I5 = std::integral_constant<int, 5>;
        using F = std::false_type;
        u32x8 pka{}, pkb{};                      // probabilities of even / odd tiles
        const int nst = nsteps - 1;              // steps with a successor
        if (nst > 0) step(0, I0{}, std::true_type{}, sa, sb, pkb, pka);
        int j = 1;
        for (; j + 6 <= nst; j += 6) {
            step(j, I1{}, F{}, sb, sa, pka, pkb);
            step(j + 1, I2{}, F{}, sa, sb, pkb, pka);
            step(j + 2, I3{}, F{}, sb, sa, pka, pkb);
            step(j + 3, I4{}, F{}, sa, sb, pkb, pka);
            step(j + 4, I5{}, F{}, sb, sa, pka, pkb);
            step(j + 5, I0{}, F{}, sa, sb, pkb, pka);
        }
        if (j < nst) {
            step(j, I1{}, F{}, sb, sa, pka, pkb);
            if (j + 1 < nst) {
                step(j + 1, I2{}, F{}, sa, sb, pkb, pka);
                if (j + 2 < nst) {
                    step(j + 2, I3{}, F{}, sb, sa, pka, pkb);
                    if (j + 3 < nst) {
                        step(j + 3, I4{}, F{}, sa, sb, pkb, pka);
                        if (j + 4 < nst) step(j + 4, I5{}, F{}, sb, sa, pka, pkb);
                    }
                }
            }
        }
        {   // The last tile: PV of the one before, its own probabilities, then its PV once
            // V(nst) has landed. Its scores sit in sa (nst even) or sb.
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(WL) : "memory");   // V(nst - 1) is in
            __syncthreads();
            const bool odd = nst & 1;
            const f32x16 sl = odd ? sb : sa;
            const u32x8 pp = odd ? pka : pkb;
            u32x8 pl;
            if (nst > 0) pv((nst + 2) % 3, pp);
            const float t = probs_sum(sl, pl);
            settle(sl, pl, t);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // V(nst) is in
            __syncthreads();
            pv(nst % 3, pl);
        }
    } else {
    // ---- the pipelined loop ------------------------------------------------------------
    // Iteration j works on step j (scores s_cur and row maximum mx_cur already known) and
    // prepares step j + 1:
    //   top     wait for K(j + 1) and V(j), barrier, issue K(j + 3) and V(j + 2) into the
    //           ring slots K(j) and V(j - 1) used (every wave has passed the barrier, so
    //           none still reads them), and read step j + 1's K fragments;
    //   block A the score MFMAs of step j + 1, interleaved with step j's exponentials;
    //   block B step j's PV MFMAs, interleaved with step j + 1's row maximum.
    // Every load is thus issued two iterations before its first use, and matrix cores
    // and vector ALUs work at once inside every wave. Waves that fill K slots issue K
    // loads and waves that fill V slots V loads, WL per iteration each, so one wait count
    // serves both. Only the last step of a key half can run past the key axis, and it
    // has no successor, so the interleaved path never masks.
    const bool k_loader = ld_kind == 0;
    // Prologue: K(0), K(1), K(2) / V(0), V(1) in flight.
    issue(0, 0);
    issue(1, 1);
    if (k_loader) issue(2, 2);
    if (k_loader) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * WL) : "memory");   // K(0) is in
    __syncthreads();
    f32x16 s_cur = f32x16{};
    float mx_cur = kNegInf;
    if (0 < my_tiles) {
        s_cur = scores(0);
        const int kv0 = sk - my_first * KT;
        if (kv0 < KT) mask_tail(s_cur, kv0);
        mx_cur = rowmax2(s_cur);
    }
    // One iteration; KS1 (the K slot of step j + 1) and VS0 (the V slot of step j) are
    // compile-time so every LDS address is a per-lane base plus an immediate. K(j) sits in
    // slot VS0 as well (both rings advance together), V(j - 1) in slot VS0 - 1.
    auto iteration = [&](int j, auto ks1_tag, auto vs0_tag) {
        constexpr int KS1 = decltype(ks1_tag)::value;
        constexpr int VS0 = decltype(vs0_tag)::value;
        constexpr int VFREE = (VS0 + STAGES - 1) % STAGES;
        u32x4 kf[NC];
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(WL) : "memory");   // K(j + 1) / V(j) are in
        __syncthreads();
        if (k_loader) issue(j + 3, VS0);      // into K(j)'s slot
        else issue(j + 2, VFREE);             // into V(j - 1)'s slot
        if (j + 1 < my_tiles) load_k(KS1, kf);   // step j + 1's K fragments, early
        if (j < my_tiles) {
            rescale(mx_cur);
            uint32_t pk[8];
            if (j + 1 < my_tiles) {
                // Steady state (step j is a full tile).
                f32x16 s_next;
                {   // block A
                    s_next = mfma_s(kf);
                    probs(std::false_type{}, s_cur, KT, pk);
#pragma unroll
                    for (int c = 0; c < NC; ++c) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // one MFMA
                        __builtin_amdgcn_sched_group_barrier(0x402, 12, 0);   // then VALU work
                    }
                }
                const int kvn = sk - (my_first + j + 1) * KT;
                if (kvn < KT) {                // the next step is the half's last, partial tile
                    pv(VS0, pk);
                    mask_tail(s_next, kvn);
                    mx_cur = rowmax2(s_next);
                } else {                       // block B
                    pv(VS0, pk);
                    mx_cur = rowmax2(s_next);
                    __builtin_amdgcn_sched_group_barrier(0x100, 4 * DB, 0);   // V reads
#pragma unroll
                    for (int c = 0; c < 2 * DB; ++c) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x402, 5, 0);
                    }
                }
                s_cur = s_next;
            } else {
                // Last step of this key half (possibly a partial tile).
                const int kv = sk - (my_first + j) * KT;
                if (kv < KT) probs(std::true_type{}, s_cur, kv, pk);
                else probs(std::false_type{}, s_cur, KT, pk);
                pv(VS0, pk);
            }
        }
    };
    static_assert(STAGES == 3, "the loop is unrolled over the 3 ring slots");
    for (int j = 0; j < nsteps; j += 3) {
        iteration(j, std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{});
        if (j + 1 < nsteps) iteration(j + 1, std::integral_constant<int, 2>{}, std::integral_constant<int, 1>{});
        if (j + 2 < nsteps) iteration(j + 2, std::integral_constant<int, 0>{}, std::integral_constant<int, 2>{});
    }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // retire the trailing (unused) loads

    // Merge the two key halves of each query block: half 1 publishes (ref, s, o~) in
    // its lane layout, half 0 combines and writes. The stages are free after the barrier.
    const float s_row = s_part + __shfl_xor(s_part, 32, 64);
    float* mb = reinterpret_cast<float*>(smem);           // [qh][DB*16 + 2][64]
    constexpr int NR = DB * 16 + 2;
    __syncthreads();
    if (kh == 1) {
        float* dst = mb + qh * NR * 64;
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) dst[(b * 16 + r) * 64 + lane] = acc_o[b][r];
        dst[(DB * 16) * 64 + lane] = m_ref;
        dst[(DB * 16 + 1) * 64 + lane] = s_row;
    }
    __syncthreads();
    if (kh == 0) {
        const float* src = mb + qh * NR * 64;
        const float m2 = src[(DB * 16) * 64 + lane];
        const float s2 = src[(DB * 16 + 1) * 64 + lane];
        const float M = fmaxf(m_ref, m2);
        const float w1 = m_ref == kNegInf ? 0.f : exp2_fast(m_ref - M);
        const float w2 = m2 == kNegInf ? 0.f : exp2_fast(m2 - M);
        const float s = w1 * s_row + w2 * s2;
        {
            // The normalised rows go to an LDS staging tile (rows padded by 16 bytes), then out
            // as whole 128-byte lines, 16 bytes per lane, with streaming stores: written through
            // while the kernel runs, they leave no dirty lines for the end-of-kernel write-back,
            // which otherwise holds the kernel's end (0.7 us at 8 x 12 x 512 x 512 x 64).
            constexpr int SRW = D + 8;
            uint16_t* stg = reinterpret_cast<uint16_t*>(mb + 2 * NR * 64) + qh * 32 * SRW;
            const float inv = 1.f / s;
            const float a1 = w1 * inv, a2 = w2 * inv;
#pragma unroll
            for (int b = 0; b < DB; ++b)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int d = 32 * b + g4 * 8 + 4 * h;
                    float ov[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        ov[e] = acc_o[b][4 * g4 + e] * a1 + src[(b * 16 + 4 * g4 + e) * 64 + lane] * a2;
                    const u32x2 w = {pack_bf16(ov[0], ov[1]), pack_bf16(ov[2], ov[3])};
                    *reinterpret_cast<u32x2*>(stg + l32 * SRW + d) = w;
                }
            if (lse && h == 0 && qrow < Sq) lse[bh * Sq + qrow] = (M + __log2f(s)) * kLn2;
            asm volatile("" ::: "memory");   // the wave reads back its own staging writes
            constexpr int PPR = D / 8;               // 16-byte pieces per row
#pragma unroll
            for (int it = 0; it < 32 * PPR / 64; ++it) {
                const int idx = it * 64 + lane;
                const int row = idx / PPR, piece = idx % PPR;
                const u32x4 val = *reinterpret_cast<const u32x4*>(stg + row * SRW + piece * 8);
                const int64_t grow = q0 + 32 * qh + row;
                if (grow < Sq) __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(o + (bh * Sq + grow) * D + piece * 8));
            }
        }
    }
}

template <int D, int STAGES, bool EXACT>
hipError_t launch_t(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse, int64_t BH,
                    int64_t Sq, int64_t Sk, float scale, hipStream_t stream) {
    const int64_t nqb = ceil_div(Sq, 64);
    const int64_t blocks = BH * nqb;
    if (blocks > INT32_MAX || nqb > INT32_MAX) return hipErrorInvalidValue;
    const float sl2 = (scale < 0.f ? -scale : scale) * kLog2e;
    const uint32_t qsign = scale < 0.f ? 0x80008000u : 0u;
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, STAGES, EXACT>), dim3(unsigned(blocks)), dim3(256), 0, stream, q, k,
                       v, o, lse, Sq, Sk, int(nqb), sl2, qsign);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
                                int64_t BH, int64_t Sq, int64_t Sk, int D, float scale, hipStream_t stream) {
    const bool exact = Sk % (2 * KT) == 0;
    if (D == 64)
        return exact ? launch_t<64, 3, true>(q, k, v, o, lse, BH, Sq, Sk, scale, stream)
                     : launch_t<64, 3, false>(q, k, v, o, lse, BH, Sq, Sk, scale, stream);
    return exact ? launch_t<128, 3, true>(q, k, v, o, lse, BH, Sq, Sk, scale, stream)
                 : launch_t<128, 3, false>(q, k, v, o, lse, BH, Sq, Sk, scale, stream);
}

}  // namespace rf
