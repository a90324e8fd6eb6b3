/*
 * librf: fused cascaded reductions for AMD Instinct MI355X (gfx950).
 *
 * A cascaded reduction is a chain of reductions in which each one depends on
 * the results of the earlier ones (the safe softmax followed by a GEMM being
 * the standard case). The library evaluates each chain in a single pass over
 * its input, keeping only a small running state that is rescaled as new data
 * arrives (the incremental form), as described on the pages about RedFuser
 * ("RedFuser: An Automatic Operator Fusion Framework for Cascaded Reductions
 * on AI Accelerators", ASPLOS 2026): its abstract; the Chinese explainer
 * "RedFuser框架：AI加速器中的算子融合技术解析" sections 2.2, 2.3, 3.3 and 4.1-4.3;
 * and the Dutch technical summary ("Technische samenvatting", Methodologie
 * items 1-3).
 *
 * Conventions for every call
 * --------------------------
 *  - Tensor pointers are DEVICE pointers owned by the caller. The library
 *    allocates nothing, frees nothing and keeps no pointer after it returns.
 *  - Every call only enqueues work on `stream` (a hipStream_t; NULL means the
 *    null stream) and returns; it never synchronises. Results are valid once
 *    the caller has synchronised with the stream.
 *  - Sizes are int64_t element counts. Tensors are dense and row-major in the
 *    layouts stated per call. Every tensor pointer must be 16-byte aligned.
 *  - Outputs must not alias inputs or each other.
 *  - Results are deterministic: fixed reduction order, no floating-point atomics.
 *  - All arguments are validated on the host before any HIP call; an invalid
 *    call returns an error status, launches nothing and sets rf_last_error().
 *    A launch failure returns RF_ERR_DEVICE. Faults inside a kernel surface at
 *    the caller's next synchronisation, as for any HIP kernel.
 *  - Thread-safe: the only state is a thread-local error message, plus the
 *    per-device address of rf_attn_decode_noalloc's static scratch.
 *  - No call throws across the ABI or aborts the process.
 */
#ifndef LIBRF_H
#define LIBRF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RF_ABI_VERSION 5

/* Exported symbols (the library is built with hidden visibility by default). */
#if defined(__GNUC__) || defined(__clang__)
#define RF_API __attribute__((visibility("default")))
#else
#define RF_API
#endif

typedef enum rf_status {
    RF_OK = 0,
    RF_ERR_INVALID_ARGUMENT = 1, /* NULL pointer, bad size, misalignment, aliasing  */
    RF_ERR_UNSUPPORTED = 2,      /* well-formed but outside what this build implements */
    RF_ERR_BUFFER_TOO_SMALL = 3, /* a caller-provided workspace is too small        */
    RF_ERR_DEVICE = 4            /* the HIP runtime reported an error              */
} rf_status;

typedef enum rf_dtype {
    RF_F32 = 0,  /* IEEE binary32                                   */
    RF_BF16 = 1  /* bfloat16 (upper half of a binary32), RNE rounding */
} rf_dtype;

/* A hipStream_t passed as an opaque pointer; NULL is the null stream. */
typedef void* rf_stream;

/* RF_ABI_VERSION of the loaded library. */
RF_API int rf_abi_version(void);

/* Static text for a status code. Never NULL. */
RF_API const char* rf_status_string(rf_status s);

/* Detail of the last error on the calling thread ("" if none). The string is
 * owned by the library and valid until the thread's next librf call. */
RF_API const char* rf_last_error(void);

/*
 * rf_softmax_gemm_fused -- single-segment fused attention, O = softmax(scale * Q K^T) V.
 *
 * The softmax -> GEMM cascade of the explainer's sections 2.2 and 4.1: the
 * running maximum, running sum of exponentials and output accumulator of each
 * query row are updated once per key tile (rescaled by exp(m_old - m_new)),
 * and O is normalised once at the end. One workgroup owns a block of query
 * rows and walks the whole key axis (the Single-Segment strategy of the
 * technical summary, Methodologie 3). Non-causal, no mask.
 *
 *   dt     RF_F32 or RF_BF16: the element type of q, k, v and o.
 *   q      [B, H, Sq, D]   queries.
 *   k, v   [B, H, Sk, D]   keys and values.
 *   o      [B, H, Sq, D]   output (written), same dtype as q.
 *   lse    [B, H, Sq] fp32 natural-log logsumexp of the scaled scores,
 *          m + ln(s); may be NULL.
 *   scale  the softmax scale applied to Q K^T before the maximum.
 *   Supported: B, H, Sq, Sk >= 1; D in {64, 128}; B*H*Sq*D and B*H*Sk*D below 2^40;
 *   for RF_BF16 also Sk*D below 2^30.
 *   Accumulation is fp32. bf16 outputs are rounded to nearest even.
 */
RF_API rf_status rf_softmax_gemm_fused(rf_dtype dt, const void* q, const void* k, const void* v,
                                void* o, float* lse, int64_t B, int64_t H, int64_t Sq,
                                int64_t Sk, int64_t D, float scale, rf_stream stream);

/* How rf_softmax_gemm_fused_mode evaluates the cascade. */
typedef enum rf_attn_mode {
    RF_ATTN_AUTO = 0,        /* whole-row for bf16 rows shorter than 256 keys (D = 64: at most
                                224), else incremental                                         */
    RF_ATTN_INCREMENTAL = 1, /* running maximum, rescaled running sum and accumulator           */
    RF_ATTN_WHOLE_ROW = 2    /* every score of a row on chip, the exact maximum, no rescaling   */
} rf_attn_mode;

/*
 * rf_softmax_gemm_fused_mode -- rf_softmax_gemm_fused with the evaluation chosen
 * explicitly. The explainer's section 5.2 recommends the non-incremental form for
 * sequences shorter than 256 and the incremental form from 256 on; RF_ATTN_AUTO
 * applies that threshold, except that D = 64 rows of more than 224 keys stay
 * incremental (the whole-row kernel measured slower there on MI355X).
 * rf_softmax_gemm_fused is RF_ATTN_AUTO. The whole-row
 * form keeps the head's entire K and V in LDS and every score of the row block in
 * registers, then takes the exact maximum, the exponentials, their sum and P V
 * (the three passes of the explainer's section 2.1, on chip).
 *
 *   mode   RF_ATTN_AUTO, RF_ATTN_INCREMENTAL or RF_ATTN_WHOLE_ROW.
 *   Other arguments as for rf_softmax_gemm_fused.
 *   RF_ATTN_WHOLE_ROW supports RF_BF16 with 1 <= Sk <= 256 (RF_ERR_UNSUPPORTED otherwise).
 */
RF_API rf_status rf_softmax_gemm_fused_mode(rf_attn_mode mode, rf_dtype dt, const void* q, const void* k,
                                     const void* v, void* o, float* lse, int64_t B, int64_t H,
                                     int64_t Sq, int64_t Sk, int64_t D, float scale, rf_stream stream);

/*
 * rf_attn_decode_split -- multi-segment decode attention, first kernel of two.
 *
 * One query token per (batch, head). The key axis L is split into nseg
 * contiguous segments of ceil(L/nseg) keys (trailing segments may be shorter
 * or empty), and each segment is reduced independently in the incremental
 * form (the Multi-Segment strategy of the technical summary, Methodologie 3;
 * the inter-block level of the explainer's section 3.3). For segment t of row
 * r = b*H + h it writes
 *     part_m[r*nseg + t]        = max_j x_j over the segment           (or -inf if empty)
 *     part_s[r*nseg + t]        = sum_j exp(x_j - part_m)              (or 0)
 *     part_o[(r*nseg + t)*D + d] = sum_j exp(x_j - part_m) v_j[d]     (or 0), unnormalised,
 * with x_j = scale * <q, k_j>. Combine the partials with rf_segment_merge.
 *
 *   q        [B, H, D] bf16.     k, v  [B, H, L, D] bf16.
 *   part_m, part_s  fp32, B*H*nseg elements each.  part_o  fp32, B*H*nseg*D elements.
 *   Supported: B, H >= 1; 1 <= nseg <= L; D in {64, 128}; B*H*nseg <= 2^31 - 1.
 */
RF_API rf_status rf_attn_decode_split(const void* q, const void* k, const void* v, int64_t B,
                               int64_t H, int64_t L, int64_t D, int64_t nseg, float scale,
                               float* part_m, float* part_s, float* part_o, rf_stream stream);

/*
 * rf_attn_decode_segments -- segment count for rf_attn_decode_split.
 *
 * A host-side rule (no device work) for how finely to split the key axis. The
 * explainer's section 5.2 asks for a launch whose waves per compute unit are
 * close to a whole number, and its sections 5.3 and 6 for enough parallelism
 * on long sequences (split the key axis). The split kernel streams each
 * segment with one wave and saturates HBM once every SIMD runs one wave, so
 * the rule asks for the fewest segments that give rows * nseg >= 4 * num_cus
 * waves (one per SIMD, a whole number of waves per compute unit), with
 * segments of at least 128 keys; more segments only add partial traffic and
 * merge work.
 *
 *   rows     B * H query rows (>= 1).   L  keys per row (>= 1).
 *   num_cus  compute units of the device (256 on MI355X); <= 0 queries the
 *            current HIP device.
 *   Returns  nseg in [1, min(L, 1024)], or 0 if rows or L < 1 (see rf_last_error).
 */
RF_API int64_t rf_attn_decode_segments(int64_t rows, int64_t L, int64_t num_cus);

/*
 * rf_segment_merge -- merge of per-segment (max, sum, partial-O) triples.
 *
 * For each row r: m = max_t part_m, w_t = exp(part_m[t] - m) (0 for a segment
 * whose maximum is -inf), s = sum_t w_t part_s[t], o = sum_t w_t part_o[t] / s,
 * lse = m + ln(s). This is the commutative-monoid combination that the fusion
 * conditions of the technical summary (Methodologie 1) make exact; a row whose
 * segments are all empty gives o = 0 and lse = -inf.
 *
 *   part_m, part_s  [rows, nseg] fp32.  part_o  [rows, nseg, D] fp32.
 *   out_dt  RF_F32 or RF_BF16 (RNE): the dtype of o.   o  [rows, D].
 *   lse     [rows] fp32, may be NULL.
 *   Supported: rows >= 1, 1 <= nseg <= 1024, D in {64, 128, 512} (512: the latent
 *   width of rf_mla_decode_split).
 */
RF_API rf_status rf_segment_merge(const float* part_m, const float* part_s, const float* part_o,
                           int64_t rows, int64_t nseg, int64_t D, rf_dtype out_dt, void* o,
                           float* lse, rf_stream stream);

/*
 * rf_attn_decode_workspace_size -- bytes of device workspace rf_attn_decode needs for the
 * partials of nseg segments (nseg = 0: the rf_attn_decode_segments choice on the current
 * device); 0 when one segment is used. Returns 0 for invalid sizes as well.
 */
RF_API size_t rf_attn_decode_workspace_size(int64_t B, int64_t H, int64_t L, int64_t D, int64_t nseg);

/*
 * rf_attn_decode -- decode attention in one call: o = softmax(scale * q K^T) V per (b, h).
 *
 * With one segment (the Single-Segment strategy of the technical summary,
 * Methodologie 3) each row is reduced by one wave in the incremental form and
 * normalised in place: one launch, no partials. With nseg > 1 it runs
 * rf_attn_decode_split into `workspace` and then rf_segment_merge (the
 * Multi-Segment strategy). nseg = 0 asks rf_attn_decode_segments, which picks one
 * segment whenever the rows alone give every SIMD a wave.
 *
 *   q [B, H, D], k, v [B, H, L, D] bf16.   out_dt RF_F32 or RF_BF16: o [B, H, D].
 *   lse [B, H] fp32 or NULL.   workspace: rf_attn_decode_workspace_size bytes (NULL if 0).
 *   Supported: as rf_attn_decode_split; 0 <= nseg <= min(L, 1024).
 */
RF_API rf_status rf_attn_decode(const void* q, const void* k, const void* v, int64_t B, int64_t H, int64_t L,
                                int64_t D, int64_t nseg, float scale, rf_dtype out_dt, void* o, float* lse,
                                void* workspace, size_t ws_bytes, rf_stream stream);

/* Bytes of device scratch that rf_attn_decode_noalloc holds per GPU (32 MiB). */
#define RF_DECODE_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * rf_attn_decode_noalloc -- rf_attn_decode for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments, results and kernels as rf_attn_decode, without the workspace: the
 * segment partials go to a static device array of RF_DECODE_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends (its address is looked up
 * once per device, on the first call made with that device current). The call allocates
 * nothing and frees nothing.
 *
 *   Arguments as for rf_attn_decode, minus workspace and ws_bytes.
 *   The partials need rf_attn_decode_workspace_size(B, H, L, D, nseg) bytes; a split whose
 *   partials exceed RF_DECODE_SCRATCH_BYTES returns RF_ERR_UNSUPPORTED (one segment needs
 *   no scratch at all).
 *   Every call on one GPU shares that GPU's scratch (no initial contents are needed; it
 *   keeps whatever the last call left): calls that may run concurrently on one GPU (on
 *   different streams, or from different threads) race on it and must be serialised by
 *   the caller.
 */
RF_API rf_status rf_attn_decode_noalloc(const void* q, const void* k, const void* v, int64_t B, int64_t H,
                                        int64_t L, int64_t D, int64_t nseg, float scale, rf_dtype out_dt, void* o,
                                        float* lse, rf_stream stream);

/*
 * rf_mla_decode_split -- multi-head latent attention (MLA) decode, first kernel of two.
 *
 * MLA (named among the workloads of the technical summary's "Resultaten") caches
 * one compressed row per token: d_qk = 576 values, of which the first d_v = 512
 * are the latent and the rest the shared rotary key. With the key projection
 * absorbed into the query, head h of batch entry b scores token j as
 * x_hj = scale * <q[b,h,:], kv[b,j,:]> and reads back sum_j softmax_j(x) kv[b,j,0:d_v]:
 * the softmax -> GEMM cascade with every head sharing the cache rows. The key
 * axis is split into nseg segments of ceil(L/nseg) tokens (as in
 * rf_attn_decode_split); for row r = b*H + h and segment t it writes a triple
 * that rf_segment_merge (D = 512) combines:
 *     part_m[r*nseg + t]          a reference value m_t (natural units, -inf if empty),
 *     part_s[r*nseg + t]          sum_j exp(x_j - m_t),
 *     part_o[(r*nseg + t)*512 + d] sum_j exp(x_j - m_t) kv[b,j,d]  (unnormalised).
 * m_t is at most the segment maximum plus 8 ln 2 (a lazily moved reference); the
 * triple represents the segment exactly whatever m_t is, and the merge result
 * does not depend on it.
 *
 *   q        [B, H, 576] bf16.   kv  [B, L, 576] bf16.
 *   d_qk, d_v  must be 576 and 512.
 *   part_m, part_s  fp32, B*H*nseg elements each.  part_o  fp32, B*H*nseg*512 elements.
 *   Supported: B, H, L >= 1; H a multiple of 32; 1 <= nseg <= L; B*ceil(H/64)*nseg <= 2^31 - 1.
 */
RF_API rf_status rf_mla_decode_split(const void* q, const void* kv, int64_t B, int64_t H, int64_t L,
                                     int64_t d_qk, int64_t d_v, int64_t nseg, float scale, float* part_m,
                                     float* part_s, float* part_o, rf_stream stream);

/* The cascades rf_row_cascade instantiates from one incremental template. */
typedef enum rf_cascade {
    RF_CASCADE_LOGSUMEXP = 0,        /* out[r] = m + ln sum_j exp(x_rj - m), m = max_j x_rj        */
    RF_CASCADE_SOFTMAX_WEIGHTED = 1, /* out[r, :] = sum_j softmax(x_r)_j payload[r, j, :]         */
    RF_CASCADE_TOPK_SOFTMAX = 2,     /* out[r, :] = softmax of the k best, out_idx[r, :] = indices */
    RF_CASCADE_MEAN_VAR = 3          /* out[r, 0] = mean, out[r, 1] = population variance         */
} rf_cascade;

/*
 * rf_row_cascade -- a cascaded reduction over each row of x, from a generic
 * incremental template.
 *
 * The fusion conditions of the technical summary (Methodologie 1-2) and the
 * explainer's sections 2.2-2.3 reduce any chain d_i = (+)_j G_i(x_j, d_<i) whose
 * terms factor as H_i(d) G'_i(x) to one loop that keeps running values of every
 * d_i and corrects them by H_i(d_new) H_i^-1(d_old) when an earlier d moves. The
 * library's template takes such a cascade as (state, incremental update, merge of
 * partial states) and folds each row with a group of 4 to 64 lanes (chosen from the
 * row length) whose states are merged in a fixed order; this entry point exposes four
 * instances:
 *   RF_CASCADE_LOGSUMEXP        max, then the sum of exp(x - max) (safe softmax's head);
 *   RF_CASCADE_SOFTMAX_WEIGHTED max, sum of exp, then the exp-weighted sum of the payload
 *                               (the attention chain with given scores);
 *   RF_CASCADE_TOPK_SOFTMAX     the k best (score descending, index ascending), then the
 *                               softmax over them (the MoE gate's tail, any k <= 8);
 *   RF_CASCADE_MEAN_VAR         the mean, then the sum of squared deviations from it
 *                               (Welford's update, Chan-Golub-LeVeque merge).
 * Results are deterministic (fixed merge order); accumulation is fp32.
 *
 *   x        [R, N] fp32.   payload  [R, N, P] fp32 for RF_CASCADE_SOFTMAX_WEIGHTED, else NULL.
 *   P        payload values per element: 1, 2, 4, 8 or 16 (softmax-weighted), else 0.
 *   k        1 <= k <= min(8, N) for RF_CASCADE_TOPK_SOFTMAX, else ignored.
 *   out      fp32: [R] (logsumexp), [R, P] (softmax-weighted), [R, k] (top-k weights),
 *            [R, 2] (mean, variance).   out_idx  [R, k] int32 for top-k, else NULL.
 *   Supported: R, N >= 1; R*N*max(P,1) below 2^40; N < 2^31.
 */
RF_API rf_status rf_row_cascade(rf_cascade kind, const float* x, const float* payload, int64_t R, int64_t N,
                                int64_t P, int64_t k, float* out, int32_t* out_idx, rf_stream stream);

/* The row-scaled GEMM cascades rf_cascade_gemm instantiates from the same template. */
typedef enum rf_cascade_gemm_kind {
    RF_CASCADE_GEMM_SOFTMAX = 0, /* y = softmax(x) w,        stat = ln sum_k exp(x_k)  */
    RF_CASCADE_GEMM_ABSMAX = 1   /* y = (x / max|x|) w,      stat = max_k |x_k|        */
} rf_cascade_gemm_kind;

/*
 * rf_cascade_gemm -- a row-scaled GEMM cascade on the matrix cores, from the generic template.
 *
 * For every row x of X, a cascade whose leading reduction scales the row and whose last
 * reduction is a contraction with the weight W (technical summary, Methodologie 1-2; the
 * explainer's sections 2.2-2.3):
 *   RF_CASCADE_GEMM_SOFTMAX  d1 = max_k x_k, d2 = sum_k exp(x_k - d1),
 *                            y = sum_k exp(x_k - d1) W[k, :] / d2, stat = d1 + ln d2
 *                            (the softmax -> GEMM cascade of section 4.1 with the scores
 *                            given; -inf entries are masked; a row must have a finite entry);
 *   RF_CASCADE_GEMM_ABSMAX   d1 = max_k |x_k|, y = sum_k (x_k / d1) W[k, :], stat = d1
 *                            (the row scaling of section 4.3's quantisation cascade, without
 *                            the rounding; a zero row gives y = 0 and stat = 0).
 * The template keeps the lead, corrects the running output by H(d_new) H^-1(d_old) when it
 * moves (exp(d1_old - d1_new), or d1_old / d1_new), and forms the contraction on the bf16
 * matrix cores with fp32 accumulation, each per-element weight split into a bf16 head and
 * a bf16 tail (about 2^-17 relative; the softmax's sum reads the same two parts).
 *
 *   x     [M, K] fp32.   w  [K, N] bf16 (N contiguous).   y  [M, N] fp32.
 *   stat  [M] fp32, may be NULL.
 *   Supported: M >= 1; 4 <= K < 2^24 and K % 4 == 0; N in {64, 128}; M*K below 2^40.
 */
RF_API rf_status rf_cascade_gemm(rf_cascade_gemm_kind kind, const float* x, const void* w, int64_t M, int64_t K,
                                 int64_t N, float* y, float* stat, rf_stream stream);

/*
 * rf_moe_route -- fused MoE gate: scores = X W_gate -> top-k -> softmax over the k.
 *
 * The cascade of the explainer's section 4.2 in a single kernel: the score matrix
 * never reaches memory (unless the optional debug output is requested). Experts are
 * ordered by descending score, equal scores by the lower expert index. The
 * weights are the softmax of the k selected scores:
 * w_r = exp(s_r - s_1) / sum_r' exp(s_r' - s_1). Scores accumulate in fp32.
 *
 * Each workgroup owns 8 tokens and every expert: its waves split the hidden axis
 * (the Multi-Segment strategy of the technical summary, Methodologie 3, inside one
 * workgroup), add their partial scores on chip in a fixed order (deterministic) and
 * select and normalise the k best. No workspace is needed. Every workgroup reads all of
 * W_gate from L2; rf_moe_route_split gives each workgroup one range of it instead and
 * exchanges partial scores through a workspace in two launches (measured beside it).
 *
 *   x       [T, Hd] bf16 tokens.   w_gate  [Hd, E] bf16 (expert index contiguous).
 *   idx     [T, k] int32 expert indices.   w  [T, k] fp32 weights.
 *   scores  [T, E] fp32 debug copy of the gate scores, or NULL.
 *   Supported: T >= 1; 32 <= Hd < 2^26 and Hd % 32 == 0; 16 <= E <= 256 and E % 16 == 0;
 *   1 <= k <= min(8, E).
 */
RF_API rf_status rf_moe_route(const void* x, const void* w_gate, int64_t T, int64_t Hd, int64_t E,
                              int64_t k, int32_t* idx, float* w, float* scores, rf_stream stream);

/*
 * rf_moe_route_split_workspace_size -- bytes of device workspace rf_moe_route_split needs.
 */
RF_API size_t rf_moe_route_split_workspace_size(int64_t T, int64_t Hd, int64_t E);

/*
 * rf_moe_route_split -- rf_moe_route in two launches over a split hidden axis (the
 * Multi-Segment strategy of the technical summary, Methodologie 3, across workgroups and
 * the multi-kernel level of the explainer's section 3.3), for comparison with the
 * one-launch form: a first launch writes one partial score block per (64-token block,
 * hidden range) to `workspace`, a second adds each token's partials in a fixed order
 * (deterministic) and performs the top-k and the softmax. Each workgroup reads only its
 * range of W_gate, which on MI355X outweighs the partials' round trip: see rf_moe_route.
 *
 *   Arguments and results as for rf_moe_route, plus:
 *   workspace, ws_bytes  device scratch of at least rf_moe_route_split_workspace_size(T, Hd, E)
 *           bytes (RF_ERR_BUFFER_TOO_SMALL otherwise); no initial contents are required.
 *           Calls that share a workspace must not run concurrently.
 */
RF_API rf_status rf_moe_route_split(const void* x, const void* w_gate, int64_t T, int64_t Hd, int64_t E,
                                    int64_t k, int32_t* idx, float* w, float* scores, void* workspace,
                                    size_t ws_bytes, rf_stream stream);

/*
 * rf_quant_gemm_workspace_size -- bytes of device workspace rf_quant_gemm needs
 * for this shape when xq is NULL (0 when it needs none). With xq non-NULL no
 * workspace is needed.
 */
RF_API size_t rf_quant_gemm_workspace_size(int64_t M, int64_t N, int64_t K);

/*
 * rf_quant_gemm -- dynamic per-row FP8 quantisation fused with an FP8 GEMM.
 *
 * The cascade of the explainer's section 4.3 with one scale per row of X:
 *     a_i      = max_k |x_ik|
 *     sigma_i  = fl32(a_i / 448)                (x_scale[i], IEEE fp32 division)
 *     c_ik     = E4M3FN_RNE(fl32(x_ik / sigma_i))  (OCP FP8 E4M3FN, ties to even,
 *                                                  sign of zero kept; all 0 if a_i = 0)
 *     y_ij     = bf16_RNE(sigma_i * w_scale_j * sum_k dec(c_ik) dec(wq_jk))
 * The sum is accumulated in fp32 on the matrix cores: the codes stay 8-bit in
 * memory and are converted exactly to bf16 in registers for the bf16 MFMA,
 * because gfx950's FP8 matrix instructions keep only about 13 bits below the
 * largest product of each instruction, short of fp32 accumulation.
 *
 *   x        [M, K] bf16.
 *   wq       [N, K] E4M3FN codes: row j holds column j of the K x N weight.
 *   w_scale  [N] fp32 per-column weight scale.
 *   y        [M, N] bf16 output.   x_scale [M] fp32 output (required).
 *   xq       [M, K] E4M3FN codes output, or NULL.
 *   workspace, ws_bytes  device scratch of at least
 *            rf_quant_gemm_workspace_size(M, N, K) bytes when xq is NULL
 *            (RF_ERR_BUFFER_TOO_SMALL otherwise); may be NULL when that is 0.
 *   Supported: M, N >= 1; K >= 128 and K % 128 == 0; M*K, N*K, M*N below 2^40.
 */
RF_API rf_status rf_quant_gemm(const void* x, const uint8_t* wq, const float* w_scale, int64_t M,
                        int64_t N, int64_t K, void* y, float* x_scale, uint8_t* xq,
                        void* workspace, size_t ws_bytes, rf_stream stream);

/*
 * rf_quant_gemm_fused -- the same cascade as rf_quant_gemm in ONE launch (the
 * explainer's single-kernel fusion level, section 3.3, applied to the
 * quantisation cascade of section 4.3), with no workspace.
 *
 * Each 256 x 256 output tile reduces the absolute maxima of its own 256 rows of
 * X, then quantises bf16 X into LDS a K step ahead of the matrix products. No
 * workgroup waits for another, so the maxima are recomputed by every tile of a
 * row of tiles, and X is read in bf16 by every tile instead of once as codes.
 * The explainer's section 6 warns that fusion can lose to the unfused form; this
 * form exists to measure that (rf_quant_gemm is the faster one on the workloads
 * measured here). y, x_scale and xq are bit-identical to rf_quant_gemm's.
 *
 *   Arguments, layouts and limits as rf_quant_gemm; xq [M, K] may be NULL (the
 *   codes are then not stored anywhere). Outputs must not alias the inputs or
 *   each other (RF_ERR_INVALID_ARGUMENT).
 */
RF_API rf_status rf_quant_gemm_fused(const void* x, const uint8_t* wq, const float* w_scale, int64_t M,
                              int64_t N, int64_t K, void* y, float* x_scale, uint8_t* xq,
                              rf_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBRF_H */
