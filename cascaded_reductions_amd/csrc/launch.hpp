// Internal launchers: one per kernel family. Each one enqueues its kernel(s)
// on `stream` and returns hipGetLastError(). Arguments have been validated by
// the C-ABI layer (abi.cpp) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rf {

// Single-segment attention; q/k/v/o are [BH, S, D] row-major.
hipError_t launch_attn_fwd_f32(const float* q, const float* k, const float* v, float* o,
                               float* lse, int64_t BH, int64_t Sq, int64_t Sk, int D,
                               float scale, hipStream_t stream);
hipError_t launch_attn_fwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                uint16_t* o, float* lse, int64_t BH, int64_t Sq, int64_t Sk,
                                int D, float scale, hipStream_t stream);

// Whole-row (non-incremental) bf16 attention for short key axes, 1 <= Sk <= kWholeRowMaxKeys.
constexpr int64_t kWholeRowMaxKeys = 256;
hipError_t launch_attn_whole_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
                                  int64_t BH, int64_t Sq, int64_t Sk, int D, float scale, hipStream_t stream);

// Multi-segment decode split: q [R, D], k/v [R, L, D] bf16, R = B*H rows.
hipError_t launch_decode_split(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                               int64_t R, int64_t L, int D, int64_t nseg, float scale,
                               float* part_m, float* part_s, float* part_o, hipStream_t stream);

// Multi-head latent attention decode split: q [B, H, 576], kv [B, L, 576] bf16 (value = the
// first 512 entries of each cache row); partials for rows b * H + h, D = 512.
hipError_t launch_mla_decode_split(const uint16_t* q, const uint16_t* kv, int64_t B, int64_t H, int64_t L,
                                   int64_t nseg, float scale, float* part_m, float* part_s, float* part_o,
                                   hipStream_t stream);

// Row cascades from the generic incremental template: kind 0 logsumexp, 1 softmax-weighted
// sum (P payload values per element), 2 top-k then softmax, 3 mean and variance.
hipError_t launch_row_cascade(int kind, const float* x, const float* payload, int64_t R, int64_t N, int P, int k,
                              float* out, int32_t* out_idx, hipStream_t stream);

// Single-segment decode: each wave reduces a whole row and writes o [R, D] (bf16 or fp32) and lse.
hipError_t launch_decode_direct(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t R, int64_t L, int D,
                                float scale, bool out_bf16, void* o, float* lse, hipStream_t stream);

// Merge of per-segment partials into o [rows, D] (fp32 or bf16) and lse.
hipError_t launch_segment_merge(const float* part_m, const float* part_s, const float* part_o,
                                int64_t rows, int64_t nseg, int D, bool out_bf16, void* o,
                                float* lse, hipStream_t stream);

// MoE gate in one launch: x [T, Hd] bf16, w [Hd, E] bf16 -> idx/w [T, k], optional scores [T, E].
hipError_t launch_moe_route(const uint16_t* x, const uint16_t* w_gate, int64_t T, int64_t Hd,
                            int E, int k, int32_t* idx, float* w, float* scores, hipStream_t stream);
// The same in two launches over a split hidden axis; the workspace holds the partial score
// blocks of the hidden ranges.
size_t moe_split_workspace_bytes(int64_t T, int64_t Hd, int64_t E);
hipError_t launch_moe_route_split(const uint16_t* x, const uint16_t* w_gate, int64_t T, int64_t Hd, int E, int k,
                                  int32_t* idx, float* w, float* scores, void* workspace, hipStream_t stream);

// Row-scaled GEMM cascades from the generic template: kind 0 y = softmax(x) w with stat = lse,
// kind 1 y = (x / max|x|) w with stat = max|x|; x [M, K] fp32, w [K, N] bf16, y [M, N] fp32.
hipError_t launch_cascade_gemm(int kind, const float* x, const uint16_t* w, int64_t M, int64_t K, int N, float* y,
                               float* stat, hipStream_t stream);

// Per-row dynamic E4M3FN quantisation of x [M, K] bf16 -> codes [M, K], scale [M].
hipError_t launch_quant_rows(const uint16_t* x, int64_t M, int64_t K, uint8_t* codes,
                             float* x_scale, hipStream_t stream);
// FP8 GEMM with per-row / per-column dequantisation: y[M,N] bf16 = (a[M,K] . b[N,K]^T) * sa[m] * sb[n].
hipError_t launch_fp8_gemm(const uint8_t* a, const uint8_t* b, const float* sa, const float* sb,
                           int64_t M, int64_t N, int64_t K, uint16_t* y, hipStream_t stream);
// Both steps in one launch: x [M, K] bf16 -> y, x_scale [M] and (when xq is not null) the codes.
hipError_t launch_quant_gemm_fused(const uint16_t* x, const uint8_t* wq, const float* w_scale, int64_t M, int64_t N,
                                   int64_t K, uint16_t* y, float* x_scale, uint8_t* xq, hipStream_t stream);

}  // namespace rf
