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

#include "api_internal.hpp"
#include "kernels.hpp"
#include "la_chunked.hpp"
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

// ---------------------------------------------------------------- planning
//
// A prefill call's batch: uniform (B sequences of T tokens, inputs
// [B][H][T][d]) or packed (N sequences of cu[n+1] - cu[n] tokens, inputs
// [H][T_total][d], offsets on the device in cu_dev and on the host in
// cu_host).
struct Batch {
    const int* cu_dev = nullptr;
    const int* cu_host = nullptr;
    int N = 0;  // sequences (B for a uniform batch)
    int H = 0;
    int T = 0;  // tokens per sequence (uniform) or T_total (packed)
    bool packed() const { return cu_host != nullptr; }
};

enum Family { kFamLA, kFamDelta, kFamSsd };

constexpr int kDeltaTargetGroups = 256;  // one 8-wave workgroup per CU (LDS and registers allow one)

// Chunks per segment.  LA and SSD: enough (head, segment) workgroups for two
// per compute unit, and segments short enough that the keys and values of
// all resident workgroups (read twice) stay within the Infinity Cache.
// Delta: one 8-wave workgroup per compute unit.  `work` = chunks summed over
// the sequences of one head; `longest` = chunks of the longest sequence.
int chunks_per_segment(Family f, long work, long longest, int H, int dk, int dv) {
    long cps;
    if (f == kFamDelta) {
        cps = (work * H + kDeltaTargetGroups - 1) / kDeltaTargetGroups;
    } else {
        const long occ = work * H / 512;
        const long cap = (256L * 1024) / ((long)(dk + dv) * 2 * la::kChunk);
        cps = occ < cap ? occ : cap;
    }
    if (cps > longest) cps = longest;
    return cps < 1 ? 1 : (int)cps;
}

// The segment map (device arrays filled in at launch) and the workspace layout.
struct Plan {
    la::SegMap sm{};
    size_t sp_floats = 0;   // packed: the segment prefix, at the workspace start
    size_t fam_floats = 0;  // the family's per-slot arrays after it
    size_t bytes() const { return sizeof(float) * (sp_floats + fam_floats); }
};

Plan make_plan(Family f, const Batch& b, int dk, int dv, int chunk = la::kChunk) {
    Plan p;
    la::SegMap& sm = p.sm;
    sm.N = b.N;
    sm.H = b.H;
    sm.T = b.T;
    sm.hs = b.T;
    if (!b.packed()) {
        const int nch = (b.T + la::kChunk - 1) / la::kChunk;
        if (f == kFamDelta) {
            // segments per sequence: enough workgroups for about one per CU
            const int HT = b.N * b.H;
            long want = (kDeltaTargetGroups + (long)HT - 1) / HT;
            if (want > nch) want = nch;
            if (want < 1) want = 1;
            sm.L = (int)((nch + want - 1) / want) * la::kChunk;
        } else {
            sm.L = la::la_plan(b.N * b.H, b.T, dk, dv).L;
        }
        // the blocked paths (chunk != 64) need whole chunks per segment
        if (chunk > la::kChunk) sm.L = (sm.L + chunk - 1) / chunk * chunk;
        sm.G = (b.T + sm.L - 1) / sm.L;
        sm.NS = b.N * sm.G;
    } else {
        long work = 0, longest = 0;
        for (int n = 0; n < b.N; ++n) {
            const long c = (b.cu_host[n + 1] - b.cu_host[n] + la::kChunk - 1) / la::kChunk;
            work += c;
            longest = c > longest ? c : longest;
        }
        sm.L = chunks_per_segment(f, work, longest, b.H, dk, dv) * la::kChunk;
        long ns = 0;
        for (int n = 0; n < b.N; ++n) ns += (b.cu_host[n + 1] - b.cu_host[n] + sm.L - 1) / sm.L;
        sm.NS = (int)ns;
        p.sp_floats = ((size_t)b.N + 1 + 63) / 64 * 64;
    }
    const long slots = (long)sm.H * sm.NS;
    p.fam_floats = f == kFamLA ? (chunk == la::kChunk ? la::la_ws_floats(slots, (long)b.N * b.H, dk, dv)
                                                      : la::la_chunked_ws_floats(slots, dk, dv))
                 : f == kFamDelta ? (chunk == la::kChunk
                                         ? la::delta_ws_floats(slots, (long)sm.H * sm.chunk_recs_per_head(la::kChunk), dk, dv)
                                         : la::delta_chunked_ws_floats(slots, dk, dv))
                                  : la::ssd_ws_floats(slots, dk, dv);
    return p;
}

// Shape checks shared by every prefill call.  Returns LA_OK or a status.
// blocked: the caller also runs a blocked path (uniform batches, chunk sizes
// other than 64: la_forward, and delta_forward without gates, transforms or
// predictions).
la_status check_batch(const char* fn, const Batch& b, int dk, int dv, int dtype, int chunk, bool blocked = false) {
    if (b.N < 1 || b.H < 1 || b.T < 1 || dk < 1 || dv < 1)
        return fail(LA_ERR_INVALID_ARG, "%s: sizes must be >= 1 (%s=%d H=%d T=%d dk=%d dv=%d)", fn,
                    b.packed() ? "N" : "B", b.N, b.H, b.T, dk, dv);
    if (chunk < 1) return fail(LA_ERR_INVALID_ARG, "%s: chunk must be positive (got %d)", fn, chunk);
    if (dtype != LA_F32 && dtype != LA_BF16)
        return fail(LA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
    if (b.packed()) {
        if (!b.cu_dev) return fail(LA_ERR_INVALID_ARG, "%s: the device sequence offsets must be non-NULL", fn);
        if (reinterpret_cast<uintptr_t>(b.cu_dev) & 3u)
            return fail(LA_ERR_INVALID_ARG, "%s: the device sequence offsets must be 4-byte aligned", fn);
        if (b.cu_host[0] != 0 || b.cu_host[b.N] != b.T)
            return fail(LA_ERR_INVALID_ARG, "%s: sequence offsets must run from 0 to T_total=%d (got %d .. %d)", fn,
                        b.T, b.cu_host[0], b.cu_host[b.N]);
        for (int n = 0; n < b.N; ++n)
            if (b.cu_host[n + 1] <= b.cu_host[n])
                return fail(LA_ERR_INVALID_ARG, "%s: sequence %d is empty or offsets decrease (%d, %d)", fn, n,
                            b.cu_host[n], b.cu_host[n + 1]);
    }
    if ((long)b.N * b.H > (1L << 24))
        return fail(LA_ERR_UNSUPPORTED, "%s: %ld (sequence, head) pairs exceed 2^24", fn, (long)b.N * b.H);
    if (!supported_dim(dk) || !supported_dim(dv))
        return fail(LA_ERR_UNSUPPORTED, "%s: dk=%d dv=%d not in {64, 128}", fn, dk, dv);
    if (chunk != la::kChunk) {
        if (!blocked || b.packed())
            return fail(LA_ERR_UNSUPPORTED, "%s: chunk=%d not supported (only %d)", fn, chunk, la::kChunk);
        if (!la::la_chunked_supported(chunk, dtype == LA_BF16 ? 1 : 0))
            return fail(LA_ERR_UNSUPPORTED,
                        "%s: chunk=%d not supported (bf16: 16, 32, 64, 128; fp32: 16, 32, 64)", fn, chunk);
    }
    // The kernels address one (sequence, head)'s rows through buffer
    // resources of 32-bit size with 32-bit signed byte offsets, and read up
    // to four chunks ahead of the row being processed: every such offset must
    // stay below 2 GiB (fp32 gates and 8-byte per-token records are smaller).
    const long elem = dtype == LA_BF16 ? 2 : 4;
    if (((long)b.T + 4 * la::kChunk) * (dk > dv ? dk : dv) * elem >= (1L << 31))
        return fail(LA_ERR_UNSUPPORTED, "%s: T=%d too long (one head's rows must span < 2 GiB)", fn, b.T);
    return LA_OK;
}

// The launch grids number (head, segment) units and chunk records with 32-bit
// indices.
la_status check_plan(const char* fn, const Plan& p) {
    const long units = (long)p.sm.H * p.sm.NS;
    const long recs = (long)p.sm.H * p.sm.chunk_recs_per_head(la::kChunk);
    if (units > 0x7fffffffL || recs > 0x7fffffffL)
        return fail(LA_ERR_UNSUPPORTED, "%s: %ld (head, segment) units or %ld chunks exceed 2^31-1", fn, units, recs);
    return LA_OK;
}

la_status check_workspace(const char* fn, const Plan& p, const void* workspace, size_t workspace_bytes) {
    const size_t need = p.bytes();
    if (!workspace || workspace_bytes < need || !aligned16(workspace))
        return fail(LA_ERR_WORKSPACE, "%s: workspace of %zu bytes (16-byte aligned) required, got %zu", fn, need,
                    workspace ? workspace_bytes : (size_t)0);
    return LA_OK;
}

// The workspace's family part; for a packed batch, first builds the segment
// prefix on the device and points the map at it.
hipError_t bind_workspace(Plan& p, const Batch& b, void* workspace, hipStream_t stream, float** fam) {
    float* ws = static_cast<float*>(workspace);
    if (b.packed()) {
        int* sp = reinterpret_cast<int*>(ws);
        const hipError_t e = la::launch_segment_prefix(b.cu_dev, b.N, b.T, p.sm.L, sp, stream);
        if (e != hipSuccess) return e;
        p.sm.cu = b.cu_dev;
        p.sm.sp = sp;
    }
    *fam = ws + p.sp_floats;
    return hipSuccess;
}

size_t workspace_query(const char* fn, Family f, const Batch& b, int dk, int dv, int chunk) {
    if (b.packed() && b.N < 1) return 0;
    Batch bb = b;
    if (b.packed() && !bb.cu_dev) bb.cu_dev = b.cu_host;  // only its presence is checked here
    if (check_batch(fn, bb, dk, dv, LA_BF16, chunk, f == kFamLA || f == kFamDelta) != LA_OK) return 0;
    return make_plan(f, b, dk, dv, chunk).bytes();
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

Batch uniform(int B, int H, int T) {
    Batch b;
    b.N = B;
    b.H = H;
    b.T = T;
    return b;
}

Batch packed(const int* cu_dev, const int* cu_host, int N, int H, int T_total) {
    Batch b;
    b.cu_dev = cu_dev;
    b.cu_host = cu_host;
    b.N = N;
    b.H = H;
    b.T = T_total;
    return b;
}

la_status la_forward_impl(const char* fn, const void* q, const void* k, const void* v, const float* S0,
                          const float* z0, void* o, float* S_out, float* z_out, const Batch& b, int dk, int dv,
                          int dtype, float eps, int chunk, void* workspace, size_t workspace_bytes, void* stream,
                          int poll_limit = la::kLaPollLimit) {
    if (!q || !k || !v || !o) return fail(LA_ERR_INVALID_ARG, "%s: q, k, v and o must be non-NULL", fn);
    if (!(eps > 0.f) || !isfinite(eps))
        return fail(LA_ERR_INVALID_ARG, "%s: eps must be finite and > 0 (got %g)", fn, (double)eps);
    la_status st = check_batch(fn, b, dk, dv, dtype, chunk, true);
    if (st != LA_OK) return st;
    if (chunk == la::kChunk && dtype == LA_F32 && la::la_lds_bytes(dk, dv, dtype) > 160 * 1024)
        return fail(LA_ERR_UNSUPPORTED, "%s: fp32 with dk=%d dv=%d exceeds the 160 KiB LDS", fn, dk, dv);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return fail(LA_ERR_INVALID_ARG, "%s: q, k, v and o must be 16-byte aligned", fn);
    Plan plan = make_plan(kFamLA, b, dk, dv, chunk);
    if ((st = check_plan(fn, plan)) != LA_OK) return st;
    if ((st = check_workspace(fn, plan, workspace, workspace_bytes)) != LA_OK) return st;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    float* ws = nullptr;
    hipError_t e = bind_workspace(plan, b, workspace, hs, &ws);
    if (e == hipSuccess) {
        if (chunk == la::kChunk)
            e = la::launch_la_forward(q, k, v, S0, z0, o, S_out, z_out, plan.sm, dk, dv, dtype, eps, ws, next_tag(),
                                      stream_capturing(hs), poll_limit, hs);
        else  // the blocked path: segment sums, their prefix, chunk loops of `chunk` tokens
            e = la::launch_la_forward_chunked(q, k, v, S0, z0, o, S_out, z_out, plan.sm, dk, dv,
                                              dtype == LA_BF16 ? 1 : 0, eps, chunk, ws, hs);
    }
    return hip_status(fn, e);
}

constexpr int kKnownFlags = LA_NORMALIZE_QK | LA_BETA_SIGMOID;
static_assert(LA_NORMALIZE_QK == la::kNormQK && LA_BETA_SIGMOID == la::kBetaSigmoid, "flag values");

// The delta-rule prefills: alpha NULL selects the ungated rule.
la_status delta_forward_impl(const char* fn, const void* q, const void* k, const void* v, const void* beta,
                             const float* alpha, const float* S0, void* o, float* S_out, void* pred, int flags,
                             const Batch& b, int dk, int dv, int dtype, int chunk, void* workspace,
                             size_t workspace_bytes, void* stream) {
    if (flags & ~kKnownFlags) return fail(LA_ERR_INVALID_ARG, "%s: unknown flags 0x%x", fn, flags);
    la_status st = check_batch(fn, b, dk, dv, dtype, chunk, true);
    if (st != LA_OK) return st;
    if (dtype != LA_BF16) return fail(LA_ERR_UNSUPPORTED, "%s: only bf16 inputs are supported", fn);
    if (chunk != la::kChunk && (alpha || flags || pred))
        return fail(LA_ERR_UNSUPPORTED, "%s: chunk=%d is for the plain rule without transforms (only %d here)", fn,
                    chunk, la::kChunk);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return fail(LA_ERR_INVALID_ARG, "%s: q, k, v and o must be 16-byte aligned", fn);
    if ((reinterpret_cast<uintptr_t>(beta) & 1u) || (reinterpret_cast<uintptr_t>(alpha) & 3u) ||
        (reinterpret_cast<uintptr_t>(pred) & 1u))
        return fail(LA_ERR_INVALID_ARG, "%s: beta, alpha and pred must be aligned to their element size", fn);
    Plan plan = make_plan(kFamDelta, b, dk, dv, chunk);
    if ((st = check_plan(fn, plan)) != LA_OK) return st;
    if ((st = check_workspace(fn, plan, workspace, workspace_bytes)) != LA_OK) return st;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    float* ws = nullptr;
    hipError_t e = bind_workspace(plan, b, workspace, hs, &ws);
    if (e == hipSuccess) {
        if (chunk == la::kChunk)
            e = la::launch_delta_forward(q, k, v, beta, alpha, S0, o, S_out, pred, flags, plan.sm, dk, dv, dtype, ws,
                                         hs);
        else  // the blocked path: segment maps, their composition, chunk loops of `chunk` tokens
            e = la::launch_delta_forward_chunked(q, k, v, beta, S0, o, S_out, plan.sm, dk, dv, chunk, ws, hs);
    }
    return hip_status(fn, e);
}

la_status ssd_forward_impl(const char* fn, const void* q, const void* k, const void* v, const float* alpha,
                           const float* S0, void* o, float* S_out, const Batch& b, int dk, int dv, int dtype,
                           int chunk, void* workspace, size_t workspace_bytes, void* stream) {
    if (!q || !k || !v || !alpha || !o)
        return fail(LA_ERR_INVALID_ARG, "%s: q, k, v, alpha and o must be non-NULL", fn);
    la_status st = check_batch(fn, b, dk, dv, dtype, chunk);
    if (st != LA_OK) return st;
    if (dtype != LA_BF16) return fail(LA_ERR_UNSUPPORTED, "%s: only bf16 inputs are supported", fn);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return fail(LA_ERR_INVALID_ARG, "%s: q, k, v and o must be 16-byte aligned", fn);
    if ((reinterpret_cast<uintptr_t>(alpha) & 3u) || !aligned16(S0))
        return fail(LA_ERR_INVALID_ARG, "%s: alpha must be 4-byte and S0 16-byte aligned", fn);
    Plan plan = make_plan(kFamSsd, b, dk, dv);
    if ((st = check_plan(fn, plan)) != LA_OK) return st;
    if ((st = check_workspace(fn, plan, workspace, workspace_bytes)) != LA_OK) return st;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    float* ws = nullptr;
    hipError_t e = bind_workspace(plan, b, workspace, hs, &ws);
    if (e == hipSuccess) e = la::launch_ssd_forward(q, k, v, alpha, S0, o, S_out, plan.sm, dk, dv, dtype, ws, hs);
    return hip_status(fn, e);
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

namespace la_api {
// la_forward for other translation units of the library (the no-allocation
// variant): the same validation and launch, a caller-chosen workspace, and
// workspace_query's answer for the size.
la_status la_forward_ws(const char* fn, const void* q, const void* k, const void* v, const float* S0,
                        const float* z0, void* o, float* S_out, float* z_out, int B, int H, int T, int dk, int dv,
                        int dtype, float eps, int chunk, void* workspace, size_t workspace_bytes, void* stream) {
    return la_forward_impl(fn, q, k, v, S0, z0, o, S_out, z_out, uniform(B, H, T), dk, dv, dtype, eps, chunk,
                           workspace, workspace_bytes, stream);
}
size_t la_forward_ws_bytes(const char* fn, int B, int H, int T, int dk, int dv, int chunk) {
    return workspace_query(fn, kFamLA, uniform(B, H, T), dk, dv, chunk);
}
la_status set_error(la_status st, const char* msg) { return fail(st, "%s", msg); }
}  // namespace la_api

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

// ---------------------------------------------------------------- workspace queries

size_t la_forward_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk) {
    return workspace_query("la_forward_workspace_bytes", kFamLA, uniform(B, H, T), dk, dv, chunk);
}

size_t delta_forward_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk) {
    return workspace_query("delta_forward_workspace_bytes", kFamDelta, uniform(B, H, T), dk, dv, chunk);
}

size_t ssd_forward_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk) {
    return workspace_query("ssd_forward_workspace_bytes", kFamSsd, uniform(B, H, T), dk, dv, chunk);
}

size_t la_forward_packed_workspace_bytes(const int* cu_seqlens_host, int N, int H, int T_total, int dk, int dv,
                                         int chunk) {
    if (!cu_seqlens_host) return 0;
    return workspace_query("la_forward_packed_workspace_bytes", kFamLA,
                           packed(nullptr, cu_seqlens_host, N, H, T_total), dk, dv, chunk);
}

size_t delta_forward_packed_workspace_bytes(const int* cu_seqlens_host, int N, int H, int T_total, int dk, int dv,
                                            int chunk) {
    if (!cu_seqlens_host) return 0;
    return workspace_query("delta_forward_packed_workspace_bytes", kFamDelta,
                           packed(nullptr, cu_seqlens_host, N, H, T_total), dk, dv, chunk);
}

size_t ssd_forward_packed_workspace_bytes(const int* cu_seqlens_host, int N, int H, int T_total, int dk, int dv,
                                          int chunk) {
    if (!cu_seqlens_host) return 0;
    return workspace_query("ssd_forward_packed_workspace_bytes", kFamSsd,
                           packed(nullptr, cu_seqlens_host, N, H, T_total), dk, dv, chunk);
}

// ---------------------------------------------------------------- prefill

la_status la_forward(const void* q, const void* k, const void* v, const float* S0, const float* z0,
                     void* o, float* S_out, float* z_out, int B, int H, int T, int dk, int dv,
                     int dtype, float eps, int chunk, void* workspace, size_t workspace_bytes,
                     void* stream) {
    return la_forward_impl("la_forward", q, k, v, S0, z0, o, S_out, z_out, uniform(B, H, T), dk, dv, dtype, eps,
                           chunk, workspace, workspace_bytes, stream);
}

la_status la_forward_lookback_polls(const void* q, const void* k, const void* v, const float* S0, const float* z0,
                                    void* o, float* S_out, float* z_out, int B, int H, int T, int dk, int dv,
                                    int dtype, float eps, int chunk, void* workspace, size_t workspace_bytes,
                                    void* stream, int lookback_polls) {
    return la_forward_impl("la_forward_lookback_polls", q, k, v, S0, z0, o, S_out, z_out, uniform(B, H, T), dk, dv,
                           dtype, eps, chunk, workspace, workspace_bytes, stream, lookback_polls);
}

la_status la_forward_packed(const void* q, const void* k, const void* v, const int* cu_seqlens,
                            const int* cu_seqlens_host, int N, const float* S0, const float* z0, void* o,
                            float* S_out, float* z_out, int H, int T_total, int dk, int dv, int dtype, float eps,
                            int chunk, void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "la_forward_packed";
    if (!cu_seqlens_host) return fail(LA_ERR_INVALID_ARG, "%s: the host sequence offsets must be non-NULL", fn);
    return la_forward_impl(fn, q, k, v, S0, z0, o, S_out, z_out,
                           packed(cu_seqlens, cu_seqlens_host, N, H, T_total), dk, dv, dtype, eps, chunk, workspace,
                           workspace_bytes, stream);
}

la_status delta_forward(const void* q, const void* k, const void* v, const void* beta, const float* S0,
                        void* o, float* S_out, int B, int H, int T, int dk, int dv, int dtype, int chunk,
                        void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "delta_forward";
    if (!q || !k || !v || !beta || !o)
        return fail(LA_ERR_INVALID_ARG, "%s: q, k, v, beta and o must be non-NULL", fn);
    return delta_forward_impl(fn, q, k, v, beta, nullptr, S0, o, S_out, nullptr, 0, uniform(B, H, T), dk, dv, dtype,
                              chunk, workspace, workspace_bytes, stream);
}

la_status gated_delta_forward(const void* q, const void* k, const void* v, const void* beta, const float* alpha,
                              const float* S0, void* o, float* S_out, int B, int H, int T, int dk, int dv,
                              int dtype, int chunk, void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "gated_delta_forward";
    if (!q || !k || !v || !beta || !alpha || !o)
        return fail(LA_ERR_INVALID_ARG, "%s: q, k, v, beta, alpha and o must be non-NULL", fn);
    return delta_forward_impl(fn, q, k, v, beta, alpha, S0, o, S_out, nullptr, 0, uniform(B, H, T), dk, dv, dtype,
                              chunk, workspace, workspace_bytes, stream);
}

la_status delta_forward_ex(const void* q, const void* k, const void* v, const void* beta, const float* alpha,
                           const float* S0, void* o, float* S_out, void* pred, int flags, int B, int H, int T, int dk,
                           int dv, int dtype, int chunk, void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "delta_forward_ex";
    if (!q || !k || !v || !beta || !o)
        return fail(LA_ERR_INVALID_ARG, "%s: q, k, v, beta and o must be non-NULL", fn);
    return delta_forward_impl(fn, q, k, v, beta, alpha, S0, o, S_out, pred, flags, uniform(B, H, T), dk, dv, dtype,
                              chunk, workspace, workspace_bytes, stream);
}

la_status delta_forward_packed(const void* q, const void* k, const void* v, const void* beta, const float* alpha,
                               const int* cu_seqlens, const int* cu_seqlens_host, int N, const float* S0, void* o,
                               float* S_out, void* pred, int flags, int H, int T_total, int dk, int dv, int dtype,
                               int chunk, void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "delta_forward_packed";
    if (!q || !k || !v || !beta || !o)
        return fail(LA_ERR_INVALID_ARG, "%s: q, k, v, beta and o must be non-NULL", fn);
    if (!cu_seqlens_host) return fail(LA_ERR_INVALID_ARG, "%s: the host sequence offsets must be non-NULL", fn);
    return delta_forward_impl(fn, q, k, v, beta, alpha, S0, o, S_out, pred, flags,
                              packed(cu_seqlens, cu_seqlens_host, N, H, T_total), dk, dv, dtype, chunk, workspace,
                              workspace_bytes, stream);
}

la_status ssd_forward(const void* q, const void* k, const void* v, const float* alpha, const float* S0, void* o,
                      float* S_out, int B, int H, int T, int dk, int dv, int dtype, int chunk, void* workspace,
                      size_t workspace_bytes, void* stream) {
    return ssd_forward_impl("ssd_forward", q, k, v, alpha, S0, o, S_out, uniform(B, H, T), dk, dv, dtype, chunk,
                            workspace, workspace_bytes, stream);
}

la_status ssd_forward_packed(const void* q, const void* k, const void* v, const float* alpha, const int* cu_seqlens,
                             const int* cu_seqlens_host, int N, const float* S0, void* o, float* S_out, int H,
                             int T_total, int dk, int dv, int dtype, int chunk, void* workspace,
                             size_t workspace_bytes, void* stream) {
    const char* fn = "ssd_forward_packed";
    if (!cu_seqlens_host) return fail(LA_ERR_INVALID_ARG, "%s: the host sequence offsets must be non-NULL", fn);
    return ssd_forward_impl(fn, q, k, v, alpha, S0, o, S_out, packed(cu_seqlens, cu_seqlens_host, N, H, T_total), dk,
                            dv, dtype, chunk, workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------- backward

size_t la_backward_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk) {
    if (check_batch("la_backward_workspace_bytes", uniform(B, H, T), dk, dv, LA_BF16, chunk) != LA_OK) return 0;
    return sizeof(float) * la::la_backward_ws_floats(B * H, T, dk, dv, la::la_plan(B * H, T, dk, dv));
}

la_status la_backward(const void* q, const void* k, const void* v, const float* S0, const float* z0, const void* dO,
                      const float* dS_T, const float* dz_T, void* dq, void* dk_out, void* dv_out, float* dS0,
                      float* dz0, int B, int H, int T, int dk, int dv, int dtype, float eps, int chunk,
                      void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "la_backward";
    if (!q || !k || !v || !dO || !dq || !dk_out || !dv_out)
        return fail(LA_ERR_INVALID_ARG, "%s: q, k, v, dO, dq, dk and dv must be non-NULL", fn);
    if (!(eps > 0.f) || !isfinite(eps))
        return fail(LA_ERR_INVALID_ARG, "%s: eps must be finite and > 0 (got %g)", fn, (double)eps);
    const Batch b = uniform(B, H, T);
    la_status st = check_batch(fn, b, dk, dv, dtype, chunk);
    if (st != LA_OK) return st;
    if (dtype != LA_BF16) return fail(LA_ERR_UNSUPPORTED, "%s: only bf16 inputs are supported", fn);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dO) || !aligned16(dq) || !aligned16(dk_out) ||
        !aligned16(dv_out))
        return fail(LA_ERR_INVALID_ARG, "%s: q, k, v, dO, dq, dk and dv must be 16-byte aligned", fn);
    const la::LaPlan plan = la::la_plan(B * H, T, dk, dv);
    if ((long)B * H * plan.G > 0x7fffffffL)
        return fail(LA_ERR_UNSUPPORTED, "%s: %ld (head, segment) units exceed 2^31-1", fn, (long)B * H * plan.G);
    const size_t need = sizeof(float) * la::la_backward_ws_floats(B * H, T, dk, dv, plan);
    if (!workspace || workspace_bytes < need || !aligned16(workspace))
        return fail(LA_ERR_WORKSPACE, "%s: workspace of %zu bytes (16-byte aligned) required, got %zu", fn, need,
                    workspace ? workspace_bytes : (size_t)0);
    return hip_status(fn, la::launch_la_backward(q, k, v, S0, z0, dO, dS_T, dz_T, dq, dk_out, dv_out, dS0, dz0,
                                                 B * H, T, dk, dv, dtype, eps, plan, static_cast<float*>(workspace),
                                                 static_cast<hipStream_t>(stream)));
}

size_t delta_backward_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk) {
    const Batch b = uniform(B, H, T);
    if (check_batch("delta_backward_workspace_bytes", b, dk, dv, LA_BF16, chunk) != LA_OK) return 0;
    const Plan p = make_plan(kFamDelta, b, dk, dv);
    return sizeof(float) * la::delta_backward_ws_floats((long)p.sm.H * p.sm.NS,
                                                        (long)p.sm.H * p.sm.chunk_recs_per_head(la::kChunk), B * H, T,
                                                        dk, dv);
}

}  // extern "C"

namespace {

// delta_backward's checks and launch; after_forward: the workspace holds the
// context of delta_forward_train on the same inputs.
la_status delta_backward_impl(const char* fn, const void* q, const void* k, const void* v, const void* beta,
                              const float* alpha, const float* S0, const void* dO, const float* dS_T, void* dq,
                              void* dk_out, void* dv_out, float* dbeta, float* dalpha, float* dS0, int B, int H,
                              int T, int dk, int dv, int dtype, int chunk, void* workspace, size_t workspace_bytes,
                              void* stream, bool after_forward) {
    if (!q || !k || !v || !beta || !dO || !dq || !dk_out || !dv_out || !dbeta)
        return fail(LA_ERR_INVALID_ARG, "%s: q, k, v, beta, dO, dq, dk, dv and dbeta must be non-NULL", fn);
    if (!alpha != !dalpha)
        return fail(LA_ERR_INVALID_ARG, "%s: dalpha must be given exactly when alpha is (the gated rule)", fn);
    const Batch b = uniform(B, H, T);
    la_status st = check_batch(fn, b, dk, dv, dtype, chunk);
    if (st != LA_OK) return st;
    if (dtype != LA_BF16) return fail(LA_ERR_UNSUPPORTED, "%s: only bf16 inputs are supported", fn);
    if ((long)B * H * ((T + la::kChunk - 1) / la::kChunk) > 0x7fffffffL)
        return fail(LA_ERR_UNSUPPORTED, "%s: B*H*ceil(T/%d) exceeds 2^31-1", fn, la::kChunk);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dO) || !aligned16(dq) || !aligned16(dk_out) ||
        !aligned16(dv_out))
        return fail(LA_ERR_INVALID_ARG, "%s: q, k, v, dO, dq, dk and dv must be 16-byte aligned", fn);
    if ((reinterpret_cast<uintptr_t>(beta) & 1u) || ((reinterpret_cast<uintptr_t>(alpha) |
         reinterpret_cast<uintptr_t>(dbeta) | reinterpret_cast<uintptr_t>(dalpha) | reinterpret_cast<uintptr_t>(S0) |
         reinterpret_cast<uintptr_t>(dS_T) | reinterpret_cast<uintptr_t>(dS0)) & 3u))
        return fail(LA_ERR_INVALID_ARG, "%s: beta must be 2-byte and the fp32 arrays 4-byte aligned", fn);
    const Plan plan = make_plan(kFamDelta, b, dk, dv);
    const size_t need = sizeof(float) * la::delta_backward_ws_floats((long)plan.sm.H * plan.sm.NS,
                                                                     (long)plan.sm.H * plan.sm.chunk_recs_per_head(la::kChunk),
                                                                     B * H, T, dk, dv);
    if (!workspace || workspace_bytes < need || !aligned16(workspace))
        return fail(LA_ERR_WORKSPACE, "%s: workspace of %zu bytes (16-byte aligned) required, got %zu", fn, need,
                    workspace ? workspace_bytes : (size_t)0);
    return hip_status(fn, la::launch_delta_backward(q, k, v, beta, alpha, S0, dO, dS_T, dq, dk_out, dv_out, dbeta,
                                                    dalpha, dS0, plan.sm, dk, dv, dtype,
                                                    static_cast<float*>(workspace), static_cast<hipStream_t>(stream),
                                                    after_forward));
}

}  // namespace

extern "C" {

la_status delta_backward(const void* q, const void* k, const void* v, const void* beta, const float* alpha,
                         const float* S0, const void* dO, const float* dS_T, void* dq, void* dk_out, void* dv_out,
                         float* dbeta, float* dalpha, float* dS0, int B, int H, int T, int dk, int dv, int dtype,
                         int chunk, void* workspace, size_t workspace_bytes, void* stream) {
    return delta_backward_impl("delta_backward", q, k, v, beta, alpha, S0, dO, dS_T, dq, dk_out, dv_out, dbeta,
                               dalpha, dS0, B, H, T, dk, dv, dtype, chunk, workspace, workspace_bytes, stream, false);
}

la_status delta_backward_after_forward(const void* q, const void* k, const void* v, const void* beta,
                                       const float* alpha, const float* S0, const void* dO, const float* dS_T,
                                       void* dq, void* dk_out, void* dv_out, float* dbeta, float* dalpha,
                                       float* dS0, int B, int H, int T, int dk, int dv, int dtype, int chunk,
                                       void* workspace, size_t workspace_bytes, void* stream) {
    return delta_backward_impl("delta_backward_after_forward", q, k, v, beta, alpha, S0, dO, dS_T, dq, dk_out,
                               dv_out, dbeta, dalpha, dS0, B, H, T, dk, dv, dtype, chunk, workspace, workspace_bytes,
                               stream, true);
}

la_status delta_forward_train(const void* q, const void* k, const void* v, const void* beta, const float* alpha,
                              const float* S0, void* o, float* S_out, int B, int H, int T, int dk, int dv, int dtype,
                              int chunk, void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "delta_forward_train";
    if (!q || !k || !v || !beta || !o) return fail(LA_ERR_INVALID_ARG, "%s: q, k, v, beta and o must be non-NULL", fn);
    const Batch b = uniform(B, H, T);
    la_status st = check_batch(fn, b, dk, dv, dtype, chunk);
    if (st != LA_OK) return st;
    if (dtype != LA_BF16) return fail(LA_ERR_UNSUPPORTED, "%s: only bf16 inputs are supported", fn);
    if ((long)B * H * ((T + la::kChunk - 1) / la::kChunk) > 0x7fffffffL)
        return fail(LA_ERR_UNSUPPORTED, "%s: B*H*ceil(T/%d) exceeds 2^31-1", fn, la::kChunk);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return fail(LA_ERR_INVALID_ARG, "%s: q, k, v and o must be 16-byte aligned", fn);
    if ((reinterpret_cast<uintptr_t>(beta) & 1u) ||
        ((reinterpret_cast<uintptr_t>(alpha) | reinterpret_cast<uintptr_t>(S0) | reinterpret_cast<uintptr_t>(S_out)) & 3u))
        return fail(LA_ERR_INVALID_ARG, "%s: beta must be 2-byte and the fp32 arrays 4-byte aligned", fn);
    const Plan plan = make_plan(kFamDelta, b, dk, dv);
    if ((st = check_plan(fn, plan)) != LA_OK) return st;
    const size_t need = delta_backward_workspace_bytes(B, H, T, dk, dv, chunk);
    if (!workspace || workspace_bytes < need || !aligned16(workspace))
        return fail(LA_ERR_WORKSPACE, "%s: workspace of %zu bytes (16-byte aligned; delta_backward_workspace_bytes) "
                    "required, got %zu", fn, need, workspace ? workspace_bytes : (size_t)0);
    float* ws = static_cast<float*>(workspace);
    return hip_status(fn, la::launch_delta_forward_train(q, k, v, beta, alpha, S0, o, S_out,
                                                         la::delta_backward_states(ws, plan.sm, dk, dv), plan.sm, dk,
                                                         dv, ws, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------- decode

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

la_status ssd_decode_step(const void* q, const void* k, const void* v, const float* alpha, float* S, void* o,
                          int N, int H, int dk, int dv, int dtype, void* stream) {
    const char* fn = "ssd_decode_step";
    if (!q || !k || !v || !alpha || !S || !o)
        return fail(LA_ERR_INVALID_ARG, "%s: q, k, v, alpha, S and o must be non-NULL", fn);
    return delta_decode_impl(fn, q, k, v, nullptr, alpha, S, o, nullptr, 0, N, H, dk, dv, dtype, stream);
}

}  // extern "C"
