// C ABI of the library (declared in include/linattn.h): argument validation,
// launch planning and dispatch to the gfx950 kernels.  Validation runs before
// any HIP call, so an invalid call touches neither the device nor a buffer.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <atomic>
#include <chrono>
#include <random>

#include <hip/hip_runtime.h>

#include "kernels.hpp"
#include "linattn.h"

namespace {

thread_local char g_err[512] = "";

la_status fail(la_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

la_status ok() {
    g_err[0] = '\0';
    return LA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool supported_dim(int d) { return d == 64 || d == 128; }

// Segments per head: enough (head, segment) workgroups to give every one of
// the 256 compute units about four, never more segments than chunks.
la::LaPlan plan_segments(int HT, int T, int chunk, int target_groups) {
    const int nch = (T + chunk - 1) / chunk;
    long want = (target_groups + (long)HT - 1) / HT;
    if (want > nch) want = nch;
    if (want < 1) want = 1;
    const int cps = (int)((nch + want - 1) / want);
    la::LaPlan p;
    p.L = cps * chunk;
    p.G = (T + p.L - 1) / p.L;
    return p;
}

constexpr int kDeltaTargetGroups = 256;  // one 8-wave workgroup per CU (LDS and registers allow one)

// Shared shape checks of the two prefill calls.  Returns LA_OK or a status.
la_status check_prefill(const char* fn, int B, int H, int T, int dk, int dv, int dtype, int chunk) {
    if (B < 1 || H < 1 || T < 1 || dk < 1 || dv < 1)
        return fail(LA_ERR_INVALID_ARG, "%s: sizes must be >= 1 (B=%d H=%d T=%d dk=%d dv=%d)", fn, B,
                    H, T, dk, dv);
    if (chunk < 1) return fail(LA_ERR_INVALID_ARG, "%s: chunk must be positive (got %d)", fn, chunk);
    if (dtype != LA_F32 && dtype != LA_BF16)
        return fail(LA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
    if ((long)B * H > (1L << 24))
        return fail(LA_ERR_UNSUPPORTED, "%s: B*H = %ld heads exceeds 2^24", fn, (long)B * H);
    if (!supported_dim(dk) || !supported_dim(dv))
        return fail(LA_ERR_UNSUPPORTED, "%s: dk=%d dv=%d not in {64, 128}", fn, dk, dv);
    if (chunk != la::kChunk)
        return fail(LA_ERR_UNSUPPORTED, "%s: chunk=%d not supported (only %d)", fn, chunk, la::kChunk);
    const long elem = dtype == LA_BF16 ? 2 : 4;
    if (((long)T + la::kChunk) * (dk > dv ? dk : dv) * elem >= (1L << 31))
        return fail(LA_ERR_UNSUPPORTED, "%s: T=%d too long (one head's rows must span < 2 GiB)", fn, T);
    return LA_OK;
}

size_t la_ws_bytes(int B, int H, int T, int dk, int dv, int) {
    return sizeof(float) * la::la_ws_floats(B * H, T, dk, dv);
}

size_t ssd_ws_bytes(int B, int H, int T, int dk, int dv, int) {
    const int HT = B * H;
    return sizeof(float) * la::ssd_ws_floats(HT, dk, dv, la::la_plan(HT, T, dk, dv));
}

size_t delta_ws_bytes(int B, int H, int T, int dk, int dv, int chunk) {
    const int HT = B * H;
    const la::LaPlan p = plan_segments(HT, T, chunk, kDeltaTargetGroups);
    return sizeof(float) * la::delta_ws_floats(HT, dk, dv, p);
}

// Tags for the look-back flags of la_forward: a process-wide counter from a
// random 62-bit start, so a flag word left in a reused workspace by any
// earlier call (or found there as leftover data) does not carry the tag of
// the current call.  Zero is never used (a cleared word is absent).
unsigned long long next_tag() {
    static std::atomic<unsigned long long> counter{[] {
        std::random_device rd;
        const unsigned long long t = (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count();
        return ((unsigned long long)rd() << 32) ^ (unsigned long long)rd() ^ (t * 0x9E3779B97F4A7C15ull);
    }()};
    constexpr unsigned long long mask = (1ull << 62) - 1;
    unsigned long long t;
    do t = counter.fetch_add(1, std::memory_order_relaxed) & mask;
    while (t == 0 || t == mask);  // an all-ones word (e.g. 0xFF fill) never matches
    return t;
}

// A launch recorded into a graph is replayed with the same tag, so such
// launches clear the flags first.  If the capture state cannot be read, clear.
bool stream_capturing(hipStream_t s) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &st) != hipSuccess) return true;
    return st != hipStreamCaptureStatusNone;
}

la_status hip_status(const char* fn, hipError_t e) {
    if (e == hipSuccess) return ok();
    return fail(LA_ERR_HIP, "%s: HIP error %d: %s", fn, (int)e, hipGetErrorString(e));
}

}  // namespace

extern "C" {

const char* la_status_string(int status) {
    switch (status) {
        case LA_OK: return "LA_OK";
        case LA_ERR_INVALID_ARG: return "LA_ERR_INVALID_ARG";
        case LA_ERR_UNSUPPORTED: return "LA_ERR_UNSUPPORTED";
        case LA_ERR_WORKSPACE: return "LA_ERR_WORKSPACE";
        case LA_ERR_HIP: return "LA_ERR_HIP";
        default: return "LA_ERR_UNKNOWN";
    }
}

const char* la_last_error(void) { return g_err; }

size_t la_forward_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk) {
    if (check_prefill("la_forward_workspace_bytes", B, H, T, dk, dv, LA_BF16, chunk) != LA_OK) return 0;
    return la_ws_bytes(B, H, T, dk, dv, chunk);
}

size_t delta_forward_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk) {
    if (check_prefill("delta_forward_workspace_bytes", B, H, T, dk, dv, LA_BF16, chunk) != LA_OK) return 0;
    return delta_ws_bytes(B, H, T, dk, dv, chunk);
}

size_t ssd_forward_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk) {
    if (check_prefill("ssd_forward_workspace_bytes", B, H, T, dk, dv, LA_BF16, chunk) != LA_OK) return 0;
    return ssd_ws_bytes(B, H, T, dk, dv, chunk);
}

la_status la_forward(const void* q, const void* k, const void* v, const float* S0, const float* z0,
                     void* o, float* S_out, float* z_out, int B, int H, int T, int dk, int dv,
                     int dtype, float eps, int chunk, void* workspace, size_t workspace_bytes,
                     void* stream) {
    const char* fn = "la_forward";
    if (!q || !k || !v || !o) return fail(LA_ERR_INVALID_ARG, "%s: q, k, v and o must be non-NULL", fn);
    if (!(eps > 0.f) || !isfinite(eps))
        return fail(LA_ERR_INVALID_ARG, "%s: eps must be finite and > 0 (got %g)", fn, (double)eps);
    la_status st = check_prefill(fn, B, H, T, dk, dv, dtype, chunk);
    if (st != LA_OK) return st;
    if (dtype == LA_F32 && la::la_lds_bytes(dk, dv, dtype) > 160 * 1024)
        return fail(LA_ERR_UNSUPPORTED, "%s: fp32 with dk=%d dv=%d exceeds the 160 KiB LDS", fn, dk, dv);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return fail(LA_ERR_INVALID_ARG, "%s: q, k, v and o must be 16-byte aligned", fn);
    const size_t need = la_ws_bytes(B, H, T, dk, dv, chunk);
    if (!workspace || workspace_bytes < need || !aligned16(workspace))
        return fail(LA_ERR_WORKSPACE, "%s: workspace of %zu bytes (16-byte aligned) required, got %zu", fn,
                    need, workspace ? workspace_bytes : (size_t)0);
    const la::LaPlan plan = la::la_plan(B * H, T, dk, dv);
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    return hip_status(fn, la::launch_la_forward(q, k, v, S0, z0, o, S_out, z_out, B * H, T, dk, dv, dtype,
                                                eps, plan, static_cast<float*>(workspace), next_tag(),
                                                stream_capturing(hs), hs));
}

}  // extern "C"

namespace {

constexpr int kKnownFlags = LA_NORMALIZE_QK | LA_BETA_SIGMOID;
static_assert(LA_NORMALIZE_QK == la::kNormQK && LA_BETA_SIGMOID == la::kBetaSigmoid, "flag values");

// The delta-rule prefills: alpha NULL selects the ungated rule.
la_status delta_forward_impl(const char* fn, const void* q, const void* k, const void* v, const void* beta,
                             const float* alpha, const float* S0, void* o, float* S_out, void* pred, int flags,
                             int B, int H, int T, int dk, int dv, int dtype, int chunk, void* workspace,
                             size_t workspace_bytes, void* stream) {
    if (flags & ~kKnownFlags) return fail(LA_ERR_INVALID_ARG, "%s: unknown flags 0x%x", fn, flags);
    la_status st = check_prefill(fn, B, H, T, dk, dv, dtype, chunk);
    if (st != LA_OK) return st;
    if (dtype != LA_BF16) return fail(LA_ERR_UNSUPPORTED, "%s: only bf16 inputs are supported", fn);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return fail(LA_ERR_INVALID_ARG, "%s: q, k, v and o must be 16-byte aligned", fn);
    if ((reinterpret_cast<uintptr_t>(beta) & 1u) || (reinterpret_cast<uintptr_t>(alpha) & 3u) ||
        (reinterpret_cast<uintptr_t>(pred) & 1u))
        return fail(LA_ERR_INVALID_ARG, "%s: beta, alpha and pred must be aligned to their element size", fn);
    const size_t need = delta_ws_bytes(B, H, T, dk, dv, chunk);
    if (!workspace || workspace_bytes < need || !aligned16(workspace))
        return fail(LA_ERR_WORKSPACE, "%s: workspace of %zu bytes (16-byte aligned) required, got %zu", fn,
                    need, workspace ? workspace_bytes : (size_t)0);
    const la::LaPlan plan = plan_segments(B * H, T, chunk, kDeltaTargetGroups);
    return hip_status(fn, la::launch_delta_forward(q, k, v, beta, alpha, S0, o, S_out, pred, flags, B * H, T, dk,
                                                   dv, dtype, plan, static_cast<float*>(workspace),
                                                   static_cast<hipStream_t>(stream)));
}

// The decode steps of the three rules: alpha NULL = delta, beta NULL = scalar decay.
la_status delta_decode_impl(const char* fn, const void* q, const void* k, const void* v, const void* beta,
                            const float* alpha, float* S, void* o, void* pred, int flags, int N, int H, int dk,
                            int dv, int dtype, void* stream) {
    if (flags & ~kKnownFlags) return fail(LA_ERR_INVALID_ARG, "%s: unknown flags 0x%x", fn, flags);
    if (N < 1 || H < 1 || dk < 1 || dv < 1)
        return fail(LA_ERR_INVALID_ARG, "%s: sizes must be >= 1 (N=%d H=%d dk=%d dv=%d)", fn, N, H, dk, dv);
    if (dtype != LA_F32 && dtype != LA_BF16) return fail(LA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
    if (!supported_dim(dk) || !supported_dim(dv))
        return fail(LA_ERR_UNSUPPORTED, "%s: dk=%d dv=%d not in {64, 128}", fn, dk, dv);
    if ((long)N * H > 0x7fffffffL) return fail(LA_ERR_UNSUPPORTED, "%s: N*H exceeds 2^31-1", fn);
    if (!aligned16(S)) return fail(LA_ERR_INVALID_ARG, "%s: S must be 16-byte aligned", fn);
    return hip_status(fn, la::launch_delta_decode(q, k, v, beta, alpha, S, o, pred, flags, N * H, dk, dv, dtype,
                                                  static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

la_status delta_forward(const void* q, const void* k, const void* v, const void* beta, const float* S0,
                        void* o, float* S_out, int B, int H, int T, int dk, int dv, int dtype, int chunk,
                        void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "delta_forward";
    if (!q || !k || !v || !beta || !o)
        return fail(LA_ERR_INVALID_ARG, "%s: q, k, v, beta and o must be non-NULL", fn);
    return delta_forward_impl(fn, q, k, v, beta, nullptr, S0, o, S_out, nullptr, 0, B, H, T, dk, dv, dtype, chunk,
                              workspace, workspace_bytes, stream);
}

la_status gated_delta_forward(const void* q, const void* k, const void* v, const void* beta, const float* alpha,
                              const float* S0, void* o, float* S_out, int B, int H, int T, int dk, int dv,
                              int dtype, int chunk, void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "gated_delta_forward";
    if (!q || !k || !v || !beta || !alpha || !o)
        return fail(LA_ERR_INVALID_ARG, "%s: q, k, v, beta, alpha and o must be non-NULL", fn);
    return delta_forward_impl(fn, q, k, v, beta, alpha, S0, o, S_out, nullptr, 0, B, H, T, dk, dv, dtype, chunk,
                              workspace, workspace_bytes, stream);
}

la_status delta_forward_ex(const void* q, const void* k, const void* v, const void* beta, const float* alpha,
                           const float* S0, void* o, float* S_out, void* pred, int flags, int B, int H, int T, int dk,
                           int dv, int dtype, int chunk, void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "delta_forward_ex";
    if (!q || !k || !v || !beta || !o)
        return fail(LA_ERR_INVALID_ARG, "%s: q, k, v, beta and o must be non-NULL", fn);
    return delta_forward_impl(fn, q, k, v, beta, alpha, S0, o, S_out, pred, flags, B, H, T, dk, dv, dtype, chunk,
                              workspace, workspace_bytes, stream);
}

la_status la_decode_step(const void* q, const void* k, const void* v, float* S, float* z, void* o, int N,
                         int H, int dk, int dv, int dtype, float eps, void* stream) {
    const char* fn = "la_decode_step";
    if (!q || !k || !v || !S || !z || !o)
        return fail(LA_ERR_INVALID_ARG, "%s: q, k, v, S, z and o must be non-NULL", fn);
    if (N < 1 || H < 1 || dk < 1 || dv < 1)
        return fail(LA_ERR_INVALID_ARG, "%s: sizes must be >= 1 (N=%d H=%d dk=%d dv=%d)", fn, N, H, dk, dv);
    if (!(eps > 0.f) || !isfinite(eps))
        return fail(LA_ERR_INVALID_ARG, "%s: eps must be finite and > 0 (got %g)", fn, (double)eps);
    if (dtype != LA_F32 && dtype != LA_BF16) return fail(LA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
    if (!supported_dim(dk) || !supported_dim(dv))
        return fail(LA_ERR_UNSUPPORTED, "%s: dk=%d dv=%d not in {64, 128}", fn, dk, dv);
    if ((long)N * H > 0x7fffffffL) return fail(LA_ERR_UNSUPPORTED, "%s: N*H exceeds 2^31-1", fn);
    if (!aligned16(S)) return fail(LA_ERR_INVALID_ARG, "%s: S must be 16-byte aligned", fn);
    return hip_status(fn, la::launch_la_decode(q, k, v, S, z, o, N * H, dk, dv, dtype, eps,
                                               static_cast<hipStream_t>(stream)));
}

la_status delta_decode_step(const void* q, const void* k, const void* v, const void* beta, float* S, void* o,
                            int N, int H, int dk, int dv, int dtype, void* stream) {
    const char* fn = "delta_decode_step";
    if (!q || !k || !v || !beta || !S || !o)
        return fail(LA_ERR_INVALID_ARG, "%s: q, k, v, beta, S and o must be non-NULL", fn);
    return delta_decode_impl(fn, q, k, v, beta, nullptr, S, o, nullptr, 0, N, H, dk, dv, dtype, stream);
}

la_status gated_delta_decode_step(const void* q, const void* k, const void* v, const void* beta,
                                  const float* alpha, float* S, void* o, int N, int H, int dk, int dv, int dtype,
                                  void* stream) {
    const char* fn = "gated_delta_decode_step";
    if (!q || !k || !v || !beta || !alpha || !S || !o)
        return fail(LA_ERR_INVALID_ARG, "%s: q, k, v, beta, alpha, S and o must be non-NULL", fn);
    return delta_decode_impl(fn, q, k, v, beta, alpha, S, o, nullptr, 0, N, H, dk, dv, dtype, stream);
}

la_status delta_decode_step_ex(const void* q, const void* k, const void* v, const void* beta, const float* alpha,
                               float* S, void* o, void* pred, int flags, int N, int H, int dk, int dv, int dtype,
                               void* stream) {
    const char* fn = "delta_decode_step_ex";
    if (!q || !k || !v || !beta || !S || !o)
        return fail(LA_ERR_INVALID_ARG, "%s: q, k, v, beta, S and o must be non-NULL", fn);
    return delta_decode_impl(fn, q, k, v, beta, alpha, S, o, pred, flags, N, H, dk, dv, dtype, stream);
}

la_status ssd_forward(const void* q, const void* k, const void* v, const float* alpha, const float* S0, void* o,
                      float* S_out, int B, int H, int T, int dk, int dv, int dtype, int chunk, void* workspace,
                      size_t workspace_bytes, void* stream) {
    const char* fn = "ssd_forward";
    if (!q || !k || !v || !alpha || !o)
        return fail(LA_ERR_INVALID_ARG, "%s: q, k, v, alpha and o must be non-NULL", fn);
    la_status st = check_prefill(fn, B, H, T, dk, dv, dtype, chunk);
    if (st != LA_OK) return st;
    if (dtype != LA_BF16) return fail(LA_ERR_UNSUPPORTED, "%s: only bf16 inputs are supported", fn);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return fail(LA_ERR_INVALID_ARG, "%s: q, k, v and o must be 16-byte aligned", fn);
    if ((reinterpret_cast<uintptr_t>(alpha) & 3u) || !aligned16(S0))
        return fail(LA_ERR_INVALID_ARG, "%s: alpha must be 4-byte and S0 16-byte aligned", fn);
    const size_t need = ssd_ws_bytes(B, H, T, dk, dv, chunk);
    if (!workspace || workspace_bytes < need || !aligned16(workspace))
        return fail(LA_ERR_WORKSPACE, "%s: workspace of %zu bytes (16-byte aligned) required, got %zu", fn,
                    need, workspace ? workspace_bytes : (size_t)0);
    const la::LaPlan plan = la::la_plan(B * H, T, dk, dv);
    return hip_status(fn, la::launch_ssd_forward(q, k, v, alpha, S0, o, S_out, B * H, T, dk, dv, dtype, plan,
                                                 static_cast<float*>(workspace), static_cast<hipStream_t>(stream)));
}

la_status ssd_decode_step(const void* q, const void* k, const void* v, const float* alpha, float* S, void* o,
                          int N, int H, int dk, int dv, int dtype, void* stream) {
    const char* fn = "ssd_decode_step";
    if (!q || !k || !v || !alpha || !S || !o)
        return fail(LA_ERR_INVALID_ARG, "%s: q, k, v, alpha, S and o must be non-NULL", fn);
    return delta_decode_impl(fn, q, k, v, nullptr, alpha, S, o, nullptr, 0, N, H, dk, dv, dtype, stream);
}

}  // extern "C"
