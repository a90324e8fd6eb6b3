// The C ABI of librf: argument validation (pure host code, no HIP call before
// it has passed), status text, the thread-local error message, and dispatch to
// the kernel launchers.
#include "librf.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "launch.hpp"

namespace {

thread_local std::string t_err;

rf_status fail(rf_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    t_err = buf;
    return s;
}

rf_status ok() {
    t_err.clear();
    return RF_OK;
}

rf_status device_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(RF_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Byte ranges [a, a+na) and [b, b+nb) intersect.
bool overlap(const void* a, uint64_t na, const void* b, uint64_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

constexpr int64_t kMaxElems = int64_t(1) << 40;

// a*b*... without overflow for the (positive, bounded) sizes accepted here.
bool mul_ok(int64_t a, int64_t b, int64_t* out) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > INT64_MAX / a) return false;
    *out = a * b;
    return true;
}

bool prod(std::initializer_list<int64_t> xs, int64_t* out) {
    int64_t p = 1;
    for (int64_t x : xs)
        if (!mul_ok(p, x, &p)) return false;
    *out = p;
    return true;
}

#define RF_REQUIRE(cond, status, ...)                     \
    do {                                                  \
        if (!(cond)) return fail((status), __VA_ARGS__);  \
    } while (0)

#define RF_PTR(p, name)                                                                        \
    do {                                                                                       \
        RF_REQUIRE((p) != nullptr, RF_ERR_INVALID_ARGUMENT, "%s must not be NULL", name);      \
        RF_REQUIRE(aligned16(p), RF_ERR_INVALID_ARGUMENT, "%s must be 16-byte aligned", name); \
    } while (0)

#define RF_OPT_PTR(p, name)                                                                    \
    do {                                                                                       \
        if (p) RF_REQUIRE(aligned16(p), RF_ERR_INVALID_ARGUMENT, "%s must be 16-byte aligned", name); \
    } while (0)

}  // namespace

extern "C" {

int rf_abi_version(void) { return RF_ABI_VERSION; }

const char* rf_status_string(rf_status s) {
    switch (s) {
        case RF_OK: return "RF_OK";
        case RF_ERR_INVALID_ARGUMENT: return "RF_ERR_INVALID_ARGUMENT";
        case RF_ERR_UNSUPPORTED: return "RF_ERR_UNSUPPORTED";
        case RF_ERR_BUFFER_TOO_SMALL: return "RF_ERR_BUFFER_TOO_SMALL";
        case RF_ERR_DEVICE: return "RF_ERR_DEVICE";
    }
    return "RF_STATUS_UNKNOWN";
}

const char* rf_last_error(void) { return t_err.c_str(); }

rf_status rf_softmax_gemm_fused(rf_dtype dt, const void* q, const void* k, const void* v,
                                void* o, float* lse, int64_t B, int64_t H, int64_t Sq,
                                int64_t Sk, int64_t D, float scale, rf_stream stream) {
    return rf_softmax_gemm_fused_mode(RF_ATTN_AUTO, dt, q, k, v, o, lse, B, H, Sq, Sk, D, scale, stream);
}

rf_status rf_softmax_gemm_fused_mode(rf_attn_mode mode, rf_dtype dt, const void* q, const void* k,
                                     const void* v, void* o, float* lse, int64_t B, int64_t H,
                                     int64_t Sq, int64_t Sk, int64_t D, float scale, rf_stream stream) {
    RF_REQUIRE(mode == RF_ATTN_AUTO || mode == RF_ATTN_INCREMENTAL || mode == RF_ATTN_WHOLE_ROW,
               RF_ERR_INVALID_ARGUMENT, "mode must be RF_ATTN_AUTO, RF_ATTN_INCREMENTAL or RF_ATTN_WHOLE_ROW");
    RF_REQUIRE(dt == RF_F32 || dt == RF_BF16, RF_ERR_INVALID_ARGUMENT, "dt must be RF_F32 or RF_BF16");
    RF_PTR(q, "q");
    RF_PTR(k, "k");
    RF_PTR(v, "v");
    RF_PTR(o, "o");
    RF_OPT_PTR(lse, "lse");
    RF_REQUIRE(B >= 1 && H >= 1 && Sq >= 1 && Sk >= 1, RF_ERR_INVALID_ARGUMENT,
               "B, H, Sq and Sk must be >= 1 (got %lld, %lld, %lld, %lld)", (long long)B,
               (long long)H, (long long)Sq, (long long)Sk);
    RF_REQUIRE(D >= 1, RF_ERR_INVALID_ARGUMENT, "D must be >= 1");
    RF_REQUIRE(D == 64 || D == 128, RF_ERR_UNSUPPORTED, "D must be 64 or 128 (got %lld)", (long long)D);
    RF_REQUIRE(scale == scale && scale - scale == 0.0f, RF_ERR_INVALID_ARGUMENT, "scale must be finite");
    int64_t nq, nk, nl;
    RF_REQUIRE(prod({B, H, Sq, D}, &nq) && nq < kMaxElems && prod({B, H, Sk, D}, &nk) &&
                   nk < kMaxElems && prod({B, H, Sq}, &nl),
               RF_ERR_UNSUPPORTED, "tensor too large");
    RF_REQUIRE(dt == RF_F32 || Sk * D < (int64_t(1) << 30), RF_ERR_UNSUPPORTED,
               "bf16 path needs Sk * D < 2^30 (got Sk=%lld, D=%lld)", (long long)Sk, (long long)D);
    const uint64_t es = dt == RF_F32 ? 4 : 2;
    RF_REQUIRE(!overlap(o, nq * es, q, nq * es) && !overlap(o, nq * es, k, nk * es) &&
                   !overlap(o, nq * es, v, nk * es) && !overlap(lse, nl * 4, q, nq * es) &&
                   !overlap(lse, nl * 4, k, nk * es) && !overlap(lse, nl * 4, v, nk * es) &&
                   !overlap(lse, nl * 4, o, nq * es),
               RF_ERR_INVALID_ARGUMENT, "outputs must not alias inputs or each other");
    RF_REQUIRE(mode != RF_ATTN_WHOLE_ROW || (dt == RF_BF16 && Sk <= rf::kWholeRowMaxKeys), RF_ERR_UNSUPPORTED,
               "RF_ATTN_WHOLE_ROW needs RF_BF16 and Sk <= %lld (got Sk=%lld)", (long long)rf::kWholeRowMaxKeys,
               (long long)Sk);
    // The automatic choice takes the explainer's threshold (whole-row below 256 keys) except
    // where the whole-row kernel measured slower on MI355X: D = 64 rows of 8 tiles (225..255 keys).
    const bool auto_whole = Sk < 256 && (D == 128 || Sk <= 224);
    const bool whole = dt == RF_BF16 && (mode == RF_ATTN_WHOLE_ROW || (mode == RF_ATTN_AUTO && auto_whole));
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (whole)
        e = rf::launch_attn_whole_bf16(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                       static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, B * H, Sq,
                                       Sk, int(D), scale, s);
    else if (dt == RF_F32)
        e = rf::launch_attn_fwd_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                                    static_cast<const float*>(v), static_cast<float*>(o), lse,
                                    B * H, Sq, Sk, int(D), scale, s);
    else
        e = rf::launch_attn_fwd_bf16(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                     static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse,
                                     B * H, Sq, Sk, int(D), scale, s);
    return device_status(e, "rf_softmax_gemm_fused launch");
}

rf_status rf_attn_decode_split(const void* q, const void* k, const void* v, int64_t B,
                               int64_t H, int64_t L, int64_t D, int64_t nseg, float scale,
                               float* part_m, float* part_s, float* part_o, rf_stream stream) {
    RF_PTR(q, "q");
    RF_PTR(k, "k");
    RF_PTR(v, "v");
    RF_PTR(part_m, "part_m");
    RF_PTR(part_s, "part_s");
    RF_PTR(part_o, "part_o");
    RF_REQUIRE(B >= 1 && H >= 1 && L >= 1, RF_ERR_INVALID_ARGUMENT,
               "B, H and L must be >= 1 (got %lld, %lld, %lld)", (long long)B, (long long)H, (long long)L);
    RF_REQUIRE(nseg >= 1 && nseg <= L, RF_ERR_INVALID_ARGUMENT, "need 1 <= nseg <= L (nseg=%lld, L=%lld)",
               (long long)nseg, (long long)L);
    RF_REQUIRE(D >= 1, RF_ERR_INVALID_ARGUMENT, "D must be >= 1");
    RF_REQUIRE(D == 64 || D == 128, RF_ERR_UNSUPPORTED, "D must be 64 or 128 (got %lld)", (long long)D);
    RF_REQUIRE(scale == scale && scale - scale == 0.0f, RF_ERR_INVALID_ARGUMENT, "scale must be finite");
    int64_t rows, kv, np, npo;
    RF_REQUIRE(prod({B, H}, &rows) && prod({rows, L, D}, &kv) && kv < (int64_t(1) << 46) &&
                   prod({rows, nseg}, &np) && np <= INT32_MAX && prod({np, D}, &npo),
               RF_ERR_UNSUPPORTED, "tensor too large");
    RF_REQUIRE(!overlap(part_m, np * 4, part_s, np * 4) && !overlap(part_m, np * 4, part_o, npo * 4) &&
                   !overlap(part_s, np * 4, part_o, npo * 4) && !overlap(part_o, npo * 4, k, kv * 2) &&
                   !overlap(part_o, npo * 4, v, kv * 2) && !overlap(part_o, npo * 4, q, rows * D * 2) &&
                   !overlap(part_m, np * 4, k, kv * 2) && !overlap(part_m, np * 4, v, kv * 2) &&
                   !overlap(part_s, np * 4, k, kv * 2) && !overlap(part_s, np * 4, v, kv * 2) &&
                   !overlap(part_m, np * 4, q, rows * D * 2) && !overlap(part_s, np * 4, q, rows * D * 2),
               RF_ERR_INVALID_ARGUMENT, "outputs must not alias inputs or each other");
    hipError_t e = rf::launch_decode_split(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                           static_cast<const uint16_t*>(v), rows, L, int(D), nseg, scale,
                                           part_m, part_s, part_o, static_cast<hipStream_t>(stream));
    return device_status(e, "rf_attn_decode_split launch");
}

namespace {
// Partials of rf_attn_decode: part_m, part_s [rows * nseg] and part_o [rows * nseg * D] fp32,
// each section starting on a 256-byte boundary.
size_t round256(size_t x) { return (x + 255) & ~size_t(255); }
size_t decode_ws_bytes(int64_t rows, int64_t D, int64_t nseg) {
    if (nseg <= 1) return 0;
    const size_t n = size_t(rows) * size_t(nseg);
    return 2 * round256(n * 4) + round256(n * size_t(D) * 4);
}
}  // namespace

size_t rf_attn_decode_workspace_size(int64_t B, int64_t H, int64_t L, int64_t D, int64_t nseg) {
    int64_t rows;
    if (B < 1 || H < 1 || L < 1 || (D != 64 && D != 128) || nseg < 0 || !prod({B, H}, &rows)) return 0;
    if (nseg == 0) nseg = rf_attn_decode_segments(rows, L, 0);
    if (nseg > L || nseg > 1024) return 0;
    return decode_ws_bytes(rows, D, nseg);
}

}  // extern "C"

namespace {

// Device scratch of rf_attn_decode_noalloc: the segment partials live in this file-scope
// array instead of a caller workspace. Host code never uses the array's name as an address
// (on the host it is only a stand-in); the device address comes from hipGetSymbolAddress,
// taken once per device with that device current, and is kept per device.
constexpr size_t kDecodeScratchBytes = RF_DECODE_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The calling thread's current device's copy of `scratch`, or an error status.
rf_status decode_scratch(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return device_status(e, "rf_attn_decode_noalloc: hipGetDevice");
    RF_REQUIRE(dev >= 0 && dev < kMaxDevices, RF_ERR_UNSUPPORTED, "device index %d is beyond the %d supported", dev,
               kMaxDevices);
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p)
                return device_status(e != hipSuccess ? e : hipErrorInvalidSymbol,
                                     "rf_attn_decode_noalloc: hipGetSymbolAddress(scratch)");
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return RF_OK;
}

// The body shared by rf_attn_decode (caller workspace) and rf_attn_decode_noalloc (the
// static scratch, use_scratch = true).
rf_status attn_decode_impl(const void* q, const void* k, const void* v, int64_t B, int64_t H, int64_t L, int64_t D,
                           int64_t nseg, float scale, rf_dtype out_dt, void* o, float* lse, void* workspace,
                           size_t ws_bytes, bool use_scratch, rf_stream stream) {
    RF_PTR(q, "q");
    RF_PTR(k, "k");
    RF_PTR(v, "v");
    RF_PTR(o, "o");
    RF_OPT_PTR(lse, "lse");
    RF_REQUIRE(out_dt == RF_F32 || out_dt == RF_BF16, RF_ERR_INVALID_ARGUMENT, "out_dt must be RF_F32 or RF_BF16");
    RF_REQUIRE(B >= 1 && H >= 1 && L >= 1, RF_ERR_INVALID_ARGUMENT, "B, H and L must be >= 1");
    RF_REQUIRE(D == 64 || D == 128, RF_ERR_UNSUPPORTED, "D must be 64 or 128 (got %lld)", (long long)D);
    RF_REQUIRE(nseg >= 0 && nseg <= L && nseg <= 1024, RF_ERR_INVALID_ARGUMENT,
               "nseg must be in [0, min(L, 1024)] (got %lld)", (long long)nseg);
    RF_REQUIRE(scale == scale && scale - scale == 0.0f, RF_ERR_INVALID_ARGUMENT, "scale must be finite");
    int64_t rows, nkv, nq;
    RF_REQUIRE(prod({B, H}, &rows) && prod({rows, L, D}, &nkv) && nkv < kMaxElems && prod({rows, D}, &nq) &&
                   rows <= INT32_MAX,
               RF_ERR_UNSUPPORTED, "tensor too large");
    if (nseg == 0) nseg = rf_attn_decode_segments(rows, L, 0);
    int64_t nparts;
    RF_REQUIRE(nseg == 1 || (prod({rows, nseg}, &nparts) && nparts <= INT32_MAX), RF_ERR_UNSUPPORTED,
               "B*H*nseg must be <= 2^31 - 1 when the key axis is split (got %lld rows x %lld segments)",
               (long long)rows, (long long)nseg);
    const uint64_t oes = out_dt == RF_F32 ? 4 : 2;
    RF_REQUIRE(!overlap(o, nq * oes, q, nq * 2) && !overlap(o, nq * oes, k, nkv * 2) &&
                   !overlap(o, nq * oes, v, nkv * 2) && !overlap(lse, rows * 4, q, nq * 2) &&
                   !overlap(lse, rows * 4, k, nkv * 2) && !overlap(lse, rows * 4, v, nkv * 2) &&
                   !overlap(lse, rows * 4, o, nq * oes),
               RF_ERR_INVALID_ARGUMENT, "outputs must not alias inputs or each other");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (nseg == 1) {
        const hipError_t e = rf::launch_decode_direct(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                                      static_cast<const uint16_t*>(v), rows, L, int(D), scale,
                                                      out_dt == RF_BF16, o, lse, s);
        return device_status(e, "rf_attn_decode launch");
    }
    const size_t need = decode_ws_bytes(rows, D, nseg);
    if (use_scratch) {
        RF_REQUIRE(need <= kDecodeScratchBytes, RF_ERR_UNSUPPORTED,
                   "%lld rows x %lld segments need %zu bytes of partials, beyond the %zu-byte static scratch "
                   "(use fewer segments, or rf_attn_decode with a workspace)",
                   (long long)rows, (long long)nseg, need, kDecodeScratchBytes);
        const rf_status st = decode_scratch(&workspace);
        if (st != RF_OK) return st;
        ws_bytes = kDecodeScratchBytes;
    }
    RF_REQUIRE(ws_bytes >= need, RF_ERR_BUFFER_TOO_SMALL, "workspace too small: %zu bytes, need %zu", ws_bytes, need);
    RF_PTR(workspace, "workspace");
    const uint64_t n = uint64_t(rows) * uint64_t(nseg);
    RF_REQUIRE(!overlap(workspace, need, q, nq * 2) && !overlap(workspace, need, k, nkv * 2) &&
                   !overlap(workspace, need, v, nkv * 2) && !overlap(workspace, need, o, nq * oes) &&
                   !overlap(workspace, need, lse, rows * 4),
               RF_ERR_INVALID_ARGUMENT, "workspace must not alias the tensors");
    float* pm = static_cast<float*>(workspace);
    float* ps = reinterpret_cast<float*>(static_cast<char*>(workspace) + round256(n * 4));
    float* po = reinterpret_cast<float*>(static_cast<char*>(workspace) + 2 * round256(n * 4));
    hipError_t e = rf::launch_decode_split(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                           static_cast<const uint16_t*>(v), rows, L, int(D), nseg, scale, pm, ps, po,
                                           s);
    if (e == hipSuccess) e = rf::launch_segment_merge(pm, ps, po, rows, nseg, int(D), out_dt == RF_BF16, o, lse, s);
    return device_status(e, "rf_attn_decode launch");
}

}  // namespace

extern "C" {

rf_status rf_attn_decode(const void* q, const void* k, const void* v, int64_t B, int64_t H, int64_t L, int64_t D,
                         int64_t nseg, float scale, rf_dtype out_dt, void* o, float* lse, void* workspace,
                         size_t ws_bytes, rf_stream stream) {
    return attn_decode_impl(q, k, v, B, H, L, D, nseg, scale, out_dt, o, lse, workspace, ws_bytes, false, stream);
}

rf_status rf_attn_decode_noalloc(const void* q, const void* k, const void* v, int64_t B, int64_t H, int64_t L,
                                 int64_t D, int64_t nseg, float scale, rf_dtype out_dt, void* o, float* lse,
                                 rf_stream stream) {
    return attn_decode_impl(q, k, v, B, H, L, D, nseg, scale, out_dt, o, lse, nullptr, 0, true, stream);
}

rf_status rf_mla_decode_split(const void* q, const void* kv, int64_t B, int64_t H, int64_t L, int64_t d_qk,
                              int64_t d_v, int64_t nseg, float scale, float* part_m, float* part_s,
                              float* part_o, rf_stream stream) {
    RF_PTR(q, "q");
    RF_PTR(kv, "kv");
    RF_PTR(part_m, "part_m");
    RF_PTR(part_s, "part_s");
    RF_PTR(part_o, "part_o");
    RF_REQUIRE(B >= 1 && H >= 1 && L >= 1, RF_ERR_INVALID_ARGUMENT, "B, H and L must be >= 1");
    RF_REQUIRE(d_qk == 576 && d_v == 512, RF_ERR_UNSUPPORTED, "d_qk must be 576 and d_v 512 (got %lld, %lld)",
               (long long)d_qk, (long long)d_v);
    RF_REQUIRE(H % 32 == 0, RF_ERR_UNSUPPORTED, "H must be a multiple of 32 (got %lld)", (long long)H);
    RF_REQUIRE(nseg >= 1 && nseg <= L, RF_ERR_INVALID_ARGUMENT, "nseg must be in [1, L] (got %lld)",
               (long long)nseg);
    RF_REQUIRE(scale == scale && scale - scale == 0.0f, RF_ERR_INVALID_ARGUMENT, "scale must be finite");
    int64_t nq, nkv, np, npo, nblk;
    RF_REQUIRE(prod({B, H, d_qk}, &nq) && prod({B, L, d_qk}, &nkv) && nkv < kMaxElems && prod({B, H, nseg}, &np) &&
                   prod({np, d_v}, &npo) && npo < kMaxElems && prod({B, (H + 63) / 64, nseg}, &nblk) &&
                   nblk <= INT32_MAX,
               RF_ERR_UNSUPPORTED, "problem too large");
    RF_REQUIRE(!overlap(part_m, np * 4, q, nq * 2) && !overlap(part_m, np * 4, kv, nkv * 2) &&
                   !overlap(part_s, np * 4, q, nq * 2) && !overlap(part_s, np * 4, kv, nkv * 2) &&
                   !overlap(part_o, npo * 4, q, nq * 2) && !overlap(part_o, npo * 4, kv, nkv * 2) &&
                   !overlap(part_m, np * 4, part_s, np * 4) && !overlap(part_m, np * 4, part_o, npo * 4) &&
                   !overlap(part_s, np * 4, part_o, npo * 4),
               RF_ERR_INVALID_ARGUMENT, "outputs must not alias inputs or each other");
    hipError_t e = rf::launch_mla_decode_split(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kv), B,
                                               H, L, nseg, scale, part_m, part_s, part_o,
                                               static_cast<hipStream_t>(stream));
    return device_status(e, "rf_mla_decode_split launch");
}

rf_status rf_row_cascade(rf_cascade kind, const float* x, const float* payload, int64_t R, int64_t N, int64_t P,
                         int64_t k, float* out, int32_t* out_idx, rf_stream stream) {
    RF_REQUIRE(kind >= RF_CASCADE_LOGSUMEXP && kind <= RF_CASCADE_MEAN_VAR, RF_ERR_INVALID_ARGUMENT,
               "unknown cascade kind %d", int(kind));
    RF_PTR(x, "x");
    RF_PTR(out, "out");
    RF_REQUIRE(R >= 1 && N >= 1, RF_ERR_INVALID_ARGUMENT, "R and N must be >= 1");
    RF_REQUIRE(N < (int64_t(1) << 31), RF_ERR_UNSUPPORTED, "N must be below 2^31");
    const bool weighted = kind == RF_CASCADE_SOFTMAX_WEIGHTED, topk = kind == RF_CASCADE_TOPK_SOFTMAX;
    if (weighted) {
        RF_PTR(payload, "payload");
        RF_REQUIRE(P == 1 || P == 2 || P == 4 || P == 8 || P == 16, RF_ERR_UNSUPPORTED,
                   "P must be 1, 2, 4, 8 or 16 (got %lld)", (long long)P);
    } else {
        RF_REQUIRE(P == 0, RF_ERR_INVALID_ARGUMENT, "P must be 0 for this cascade");
    }
    if (topk) {
        RF_PTR(out_idx, "out_idx");
        RF_REQUIRE(k >= 1 && k <= 8 && k <= N, RF_ERR_UNSUPPORTED, "k must be in [1, min(8, N)] (got %lld)",
                   (long long)k);
    }
    int64_t nx, np = 0, no;
    const int64_t ow = weighted ? P : topk ? k : kind == RF_CASCADE_MEAN_VAR ? 2 : 1;
    RF_REQUIRE(prod({R, N}, &nx) && nx < kMaxElems && (!weighted || (prod({nx, P}, &np) && np < kMaxElems)) &&
                   prod({R, ow}, &no),
               RF_ERR_UNSUPPORTED, "problem too large");
    RF_REQUIRE(!overlap(out, no * 4, x, nx * 4) && !overlap(out, no * 4, payload, np * 4) &&
                   (!topk || (!overlap(out_idx, no * 4, x, nx * 4) && !overlap(out_idx, no * 4, out, no * 4))),
               RF_ERR_INVALID_ARGUMENT, "outputs must not alias inputs or each other");
    const hipError_t e = rf::launch_row_cascade(int(kind), x, weighted ? payload : nullptr, R, N, int(P), int(k),
                                                out, topk ? out_idx : nullptr, static_cast<hipStream_t>(stream));
    return device_status(e, "rf_row_cascade launch");
}

rf_status rf_cascade_gemm(rf_cascade_gemm_kind kind, const float* x, const void* w, int64_t M, int64_t K, int64_t N,
                          float* y, float* stat, rf_stream stream) {
    RF_REQUIRE(kind == RF_CASCADE_GEMM_SOFTMAX || kind == RF_CASCADE_GEMM_ABSMAX, RF_ERR_INVALID_ARGUMENT,
               "unknown cascade GEMM kind %d", int(kind));
    RF_PTR(x, "x");
    RF_PTR(w, "w");
    RF_PTR(y, "y");
    RF_OPT_PTR(stat, "stat");
    RF_REQUIRE(M >= 1 && K >= 1 && N >= 1, RF_ERR_INVALID_ARGUMENT, "M, K and N must be >= 1");
    RF_REQUIRE(N == 64 || N == 128, RF_ERR_UNSUPPORTED, "N must be 64 or 128 (got %lld)", (long long)N);
    RF_REQUIRE(K % 4 == 0 && K < (int64_t(1) << 24), RF_ERR_UNSUPPORTED,
               "K must be a multiple of 4 below 2^24 (got %lld)", (long long)K);
    int64_t nx, nw, ny;
    RF_REQUIRE(prod({M, K}, &nx) && nx < kMaxElems && prod({K, N}, &nw) && prod({M, N}, &ny) && ny < kMaxElems,
               RF_ERR_UNSUPPORTED, "problem too large");
    RF_REQUIRE(!overlap(y, ny * 4, x, nx * 4) && !overlap(y, ny * 4, w, nw * 2) && !overlap(stat, M * 4, x, nx * 4) &&
                   !overlap(stat, M * 4, w, nw * 2) && !overlap(stat, M * 4, y, ny * 4),
               RF_ERR_INVALID_ARGUMENT, "outputs must not alias inputs or each other");
    const hipError_t e = rf::launch_cascade_gemm(int(kind), x, static_cast<const uint16_t*>(w), M, K, int(N), y, stat,
                                                 static_cast<hipStream_t>(stream));
    return device_status(e, "rf_cascade_gemm launch");
}

int64_t rf_attn_decode_segments(int64_t rows, int64_t L, int64_t num_cus) {
    if (rows < 1 || L < 1) {
        fail(RF_ERR_INVALID_ARGUMENT, "rows and L must be >= 1 (got %lld, %lld)", (long long)rows, (long long)L);
        return 0;
    }
    if (num_cus <= 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        num_cus = n;
    }
    constexpr int64_t kMinSegKeys = 128;   // shortest segment worth a wave
    constexpr int64_t kMaxSeg = 1024;      // the merge kernel's limit
    const int64_t waves = 4 * num_cus;     // one wave per SIMD
    int64_t n = rows >= waves ? 1 : (waves + rows - 1) / rows;
    const int64_t by_len = L / kMinSegKeys > 1 ? L / kMinSegKeys : 1;
    if (n > by_len) n = by_len;
    if (n > kMaxSeg) n = kMaxSeg;
    if (n > L) n = L;
    ok();
    return n;
}

rf_status rf_segment_merge(const float* part_m, const float* part_s, const float* part_o,
                           int64_t rows, int64_t nseg, int64_t D, rf_dtype out_dt, void* o,
                           float* lse, rf_stream stream) {
    RF_PTR(part_m, "part_m");
    RF_PTR(part_s, "part_s");
    RF_PTR(part_o, "part_o");
    RF_PTR(o, "o");
    RF_OPT_PTR(lse, "lse");
    RF_REQUIRE(out_dt == RF_F32 || out_dt == RF_BF16, RF_ERR_INVALID_ARGUMENT, "out_dt must be RF_F32 or RF_BF16");
    RF_REQUIRE(rows >= 1 && nseg >= 1, RF_ERR_INVALID_ARGUMENT, "rows and nseg must be >= 1");
    RF_REQUIRE(nseg <= 1024, RF_ERR_UNSUPPORTED, "nseg must be <= 1024 (got %lld)", (long long)nseg);
    RF_REQUIRE(D >= 1, RF_ERR_INVALID_ARGUMENT, "D must be >= 1");
    RF_REQUIRE(D == 64 || D == 128 || D == 512, RF_ERR_UNSUPPORTED, "D must be 64, 128 or 512 (got %lld)",
               (long long)D);
    int64_t np, npo, no;
    RF_REQUIRE(prod({rows, nseg}, &np) && np <= INT32_MAX && prod({np, D}, &npo) && prod({rows, D}, &no) &&
                   npo < kMaxElems,
               RF_ERR_UNSUPPORTED, "tensor too large");
    const uint64_t oes = out_dt == RF_F32 ? 4 : 2;
    RF_REQUIRE(!overlap(o, no * oes, part_m, np * 4) && !overlap(o, no * oes, part_s, np * 4) &&
                   !overlap(o, no * oes, part_o, npo * 4) && !overlap(lse, rows * 4, part_m, np * 4) &&
                   !overlap(lse, rows * 4, part_s, np * 4) && !overlap(lse, rows * 4, part_o, npo * 4) &&
                   !overlap(lse, rows * 4, o, no * oes),
               RF_ERR_INVALID_ARGUMENT, "outputs must not alias inputs or each other");
    hipError_t e = rf::launch_segment_merge(part_m, part_s, part_o, rows, nseg, int(D), out_dt == RF_BF16, o,
                                            lse, static_cast<hipStream_t>(stream));
    return device_status(e, "rf_segment_merge launch");
}

}  // extern "C"

namespace {
// Arguments shared by both forms of the MoE gate; RF_OK when they are valid.
rf_status moe_check(const void* x, const void* w_gate, int64_t T, int64_t Hd, int64_t E, int64_t k, int32_t* idx,
                    float* w, float* scores) {
    RF_PTR(x, "x");
    RF_PTR(w_gate, "w_gate");
    RF_PTR(idx, "idx");
    RF_PTR(w, "w");
    RF_OPT_PTR(scores, "scores");
    RF_REQUIRE(T >= 1 && Hd >= 1 && E >= 1, RF_ERR_INVALID_ARGUMENT, "T, Hd and E must be >= 1");
    RF_REQUIRE(k >= 1 && k <= E, RF_ERR_INVALID_ARGUMENT, "need 1 <= k <= E (k=%lld, E=%lld)", (long long)k,
               (long long)E);
    RF_REQUIRE(Hd % 32 == 0, RF_ERR_UNSUPPORTED, "Hd must be a multiple of 32 (got %lld)", (long long)Hd);
    RF_REQUIRE(Hd < (int64_t(1) << 26), RF_ERR_UNSUPPORTED, "Hd must be below 2^26 (got %lld)", (long long)Hd);
    RF_REQUIRE(E >= 16 && E <= 256 && E % 16 == 0, RF_ERR_UNSUPPORTED,
               "E must be a multiple of 16 in [16, 256] (got %lld)", (long long)E);
    RF_REQUIRE(k <= 8, RF_ERR_UNSUPPORTED, "k must be <= 8 (got %lld)", (long long)k);
    int64_t nx, ns;
    RF_REQUIRE(prod({T, Hd}, &nx) && nx < kMaxElems && prod({T, E}, &ns) && T <= INT32_MAX,
               RF_ERR_UNSUPPORTED, "tensor too large");
    RF_REQUIRE(!overlap(idx, T * k * 4, x, nx * 2) && !overlap(idx, T * k * 4, w_gate, Hd * E * 2) &&
                   !overlap(w, T * k * 4, x, nx * 2) && !overlap(w, T * k * 4, w_gate, Hd * E * 2) &&
                   !overlap(idx, T * k * 4, w, T * k * 4) && !overlap(scores, ns * 4, x, nx * 2) &&
                   !overlap(scores, ns * 4, w_gate, Hd * E * 2) && !overlap(scores, ns * 4, idx, T * k * 4) &&
                   !overlap(scores, ns * 4, w, T * k * 4),
               RF_ERR_INVALID_ARGUMENT, "outputs must not alias inputs or each other");
    return RF_OK;
}
}  // namespace

extern "C" {

rf_status rf_moe_route(const void* x, const void* w_gate, int64_t T, int64_t Hd, int64_t E, int64_t k, int32_t* idx,
                       float* w, float* scores, rf_stream stream) {
    const rf_status st = moe_check(x, w_gate, T, Hd, E, k, idx, w, scores);
    if (st != RF_OK) return st;
    const hipError_t e = rf::launch_moe_route(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_gate),
                                              T, Hd, int(E), int(k), idx, w, scores, static_cast<hipStream_t>(stream));
    return device_status(e, "rf_moe_route launch");
}

size_t rf_moe_route_split_workspace_size(int64_t T, int64_t Hd, int64_t E) {
    if (T < 1 || Hd < 1 || E < 1 || T > INT32_MAX || Hd > INT32_MAX || E > 256) return 0;
    return rf::moe_split_workspace_bytes(T, Hd, E);
}

rf_status rf_moe_route_split(const void* x, const void* w_gate, int64_t T, int64_t Hd, int64_t E, int64_t k,
                             int32_t* idx, float* w, float* scores, void* workspace, size_t ws_bytes,
                             rf_stream stream) {
    const rf_status st = moe_check(x, w_gate, T, Hd, E, k, idx, w, scores);
    if (st != RF_OK) return st;
    RF_OPT_PTR(workspace, "workspace");
    const size_t need = rf_moe_route_split_workspace_size(T, Hd, E);
    RF_REQUIRE(workspace != nullptr && ws_bytes >= need, RF_ERR_BUFFER_TOO_SMALL,
               "workspace of %zu bytes needed (got %zu)", need, workspace ? ws_bytes : size_t(0));
    const uint64_t nx = uint64_t(T) * uint64_t(Hd), ns = uint64_t(T) * uint64_t(E);
    RF_REQUIRE(!overlap(workspace, need, x, nx * 2) && !overlap(workspace, need, w_gate, Hd * E * 2) &&
                   !overlap(workspace, need, idx, T * k * 4) && !overlap(workspace, need, w, T * k * 4) &&
                   !overlap(workspace, need, scores, ns * 4),
               RF_ERR_INVALID_ARGUMENT, "the workspace must not alias the tensors");
    const hipError_t e = rf::launch_moe_route_split(static_cast<const uint16_t*>(x),
                                                    static_cast<const uint16_t*>(w_gate), T, Hd, int(E), int(k), idx,
                                                    w, scores, workspace, static_cast<hipStream_t>(stream));
    return device_status(e, "rf_moe_route_split launch");
}

size_t rf_quant_gemm_workspace_size(int64_t M, int64_t N, int64_t K) {
    (void)N;
    int64_t n;
    if (M < 1 || K < 1 || !prod({M, K}, &n)) return 0;
    return size_t(n);  // the E4M3FN codes of X, when the caller does not ask for them
}

rf_status rf_quant_gemm(const void* x, const uint8_t* wq, const float* w_scale, int64_t M,
                        int64_t N, int64_t K, void* y, float* x_scale, uint8_t* xq,
                        void* workspace, size_t ws_bytes, rf_stream stream) {
    RF_PTR(x, "x");
    RF_PTR(wq, "wq");
    RF_PTR(w_scale, "w_scale");
    RF_PTR(y, "y");
    RF_PTR(x_scale, "x_scale");
    RF_OPT_PTR(xq, "xq");
    RF_OPT_PTR(workspace, "workspace");
    RF_REQUIRE(M >= 1 && N >= 1 && K >= 1, RF_ERR_INVALID_ARGUMENT, "M, N and K must be >= 1");
    RF_REQUIRE(K % 128 == 0, RF_ERR_UNSUPPORTED, "K must be a multiple of 128 (got %lld)", (long long)K);
    int64_t nx, nw, ny;
    RF_REQUIRE(prod({M, K}, &nx) && nx < kMaxElems && prod({N, K}, &nw) && nw < kMaxElems &&
                   prod({M, N}, &ny) && ny < kMaxElems && M <= INT32_MAX && N <= INT32_MAX,
               RF_ERR_UNSUPPORTED, "tensor too large");
    uint8_t* codes = xq;
    if (!codes) {
        const size_t need = rf_quant_gemm_workspace_size(M, N, K);
        RF_REQUIRE(workspace != nullptr && ws_bytes >= need, RF_ERR_BUFFER_TOO_SMALL,
                   "workspace of %zu bytes needed when xq is NULL (got %zu)", need,
                   workspace ? ws_bytes : size_t(0));
        codes = static_cast<uint8_t*>(workspace);
    }
    RF_REQUIRE(!overlap(y, ny * 2, x, nx * 2) && !overlap(y, ny * 2, wq, nw) && !overlap(y, ny * 2, w_scale, N * 4) &&
                   !overlap(x_scale, M * 4, x, nx * 2) && !overlap(x_scale, M * 4, wq, nw) &&
                   !overlap(x_scale, M * 4, y, ny * 2) && !overlap(x_scale, M * 4, w_scale, N * 4) &&
                   !overlap(codes, nx, x, nx * 2) && !overlap(codes, nx, wq, nw) && !overlap(codes, nx, y, ny * 2) &&
                   !overlap(codes, nx, x_scale, M * 4) && !overlap(codes, nx, w_scale, N * 4),
               RF_ERR_INVALID_ARGUMENT, "outputs and workspace must not alias inputs or each other");
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = rf::launch_quant_rows(static_cast<const uint16_t*>(x), M, K, codes, x_scale, s);
    if (e != hipSuccess) return device_status(e, "rf_quant_gemm quantise launch");
    e = rf::launch_fp8_gemm(codes, wq, x_scale, w_scale, M, N, K, static_cast<uint16_t*>(y), s);
    return device_status(e, "rf_quant_gemm GEMM launch");
}

rf_status rf_quant_gemm_fused(const void* x, const uint8_t* wq, const float* w_scale, int64_t M, int64_t N,
                              int64_t K, void* y, float* x_scale, uint8_t* xq, rf_stream stream) {
    RF_PTR(x, "x");
    RF_PTR(wq, "wq");
    RF_PTR(w_scale, "w_scale");
    RF_PTR(y, "y");
    RF_PTR(x_scale, "x_scale");
    RF_OPT_PTR(xq, "xq");
    RF_REQUIRE(M >= 1 && N >= 1 && K >= 1, RF_ERR_INVALID_ARGUMENT, "M, N and K must be >= 1");
    RF_REQUIRE(K % 128 == 0, RF_ERR_UNSUPPORTED, "K must be a multiple of 128 (got %lld)", (long long)K);
    int64_t nx, nw, ny;
    RF_REQUIRE(prod({M, K}, &nx) && nx < kMaxElems && prod({N, K}, &nw) && nw < kMaxElems &&
                   prod({M, N}, &ny) && ny < kMaxElems && M <= INT32_MAX && N <= INT32_MAX,
               RF_ERR_UNSUPPORTED, "tensor too large");
    const size_t nq = xq ? size_t(nx) : 0;
    RF_REQUIRE(!overlap(y, ny * 2, x, nx * 2) && !overlap(y, ny * 2, wq, nw) && !overlap(y, ny * 2, w_scale, N * 4) &&
                   !overlap(x_scale, M * 4, x, nx * 2) && !overlap(x_scale, M * 4, wq, nw) &&
                   !overlap(x_scale, M * 4, y, ny * 2) && !overlap(x_scale, M * 4, w_scale, N * 4) &&
                   !overlap(xq, nq, x, nx * 2) && !overlap(xq, nq, wq, nw) && !overlap(xq, nq, y, ny * 2) &&
                   !overlap(xq, nq, x_scale, M * 4) && !overlap(xq, nq, w_scale, N * 4),
               RF_ERR_INVALID_ARGUMENT, "outputs must not alias inputs or each other");
    hipError_t e = rf::launch_quant_gemm_fused(static_cast<const uint16_t*>(x), wq, w_scale, M, N, K,
                                               static_cast<uint16_t*>(y), x_scale, xq, static_cast<hipStream_t>(stream));
    return device_status(e, "rf_quant_gemm_fused launch");
}

}  // extern "C"
