// Internal launcher interface between the C ABI (api.hip) and the kernels.
// Not installed; the public interface is include/linattn.h.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

#include "segments.hpp"

namespace la {

constexpr int kChunk = 64;  // tokens per chunk in every prefill kernel

struct LaPlan {
    int G;  // segments per sequence (uniform batches)
    int L;  // tokens per segment (a multiple of kChunk); the last may be ragged
};

// Every prefill launcher takes the (head, sequence, segment) decomposition
// of segments.hpp; its workspaces hold one entry per (head, segment) slot,
// H * NS slots in all.

// Linear attention prefill: one fused launch (segment aggregate, look-back,
// chunked outputs).  dtype 0 = fp32, 1 = bf16 (raw bits).  ws holds
// la_ws_floats(...) floats: the look-back flags, per-slot aggregate and
// inclusive states, then room for a copy of S0, z0 (used when S_out, z_out
// alias them).  tag (nonzero, < 2^62) must differ from the tag of every
// earlier call that used ws, unless clear_flags is set (a flag-clearing
// launch first, for launches recorded into a graph).  poll_limit bounds the
// look-back's polls per window (kLaPollLimit in production; a negative
// value makes every later segment recompute its incoming state instead).
constexpr int kLaPollLimit = 4000;
hipError_t launch_la_forward(const void* q, const void* k, const void* v,
                             const float* S0, const float* z0, void* o,
                             float* S_out, float* z_out, const SegMap& sm, int dk,
                             int dv, int dtype, float eps, float* ws,
                             unsigned long long tag, bool clear_flags, int poll_limit, hipStream_t stream);
size_t la_lds_bytes(int dk, int dv, int dtype);
LaPlan la_plan(int HT, int T, int dk, int dv);
size_t la_flag_words(long slots);
// slots = H * NS (head, segment) units; states = N * H (sequence, head) pairs.
size_t la_ws_floats(long slots, long states, int dk, int dv);

// Packed batches: sp[n] = segments of sequences 0..n-1 (L tokens per
// segment, lengths from the clamped offsets cu), n = 0..N, on the device.
hipError_t launch_segment_prefix(const int* cu, int N, int T_total, int L, int* sp, hipStream_t stream);

// Input-transform flags of the delta-rule kernels (same values as the ABI's).
constexpr int kNormQK = 1;        // q, k rows scaled to unit L2 norm in the kernel
constexpr int kBetaSigmoid = 2;   // beta holds logits; the kernel applies a sigmoid

// Delta-rule prefill: every chunk's T = (I + A)^{-1} (a parallel pass) ->
// segment affine maps -> serial composition -> chunked outputs.  alpha (fp32
// [HT][T]) selects the gated rule; NULL = ungated.
// pred (optional, [HT][T][dv] in the input dtype) receives the prediction
// made before each write.
hipError_t launch_delta_forward(const void* q, const void* k, const void* v,
                                const void* beta, const float* alpha, const float* S0,
                                void* o, float* S_out, void* pred, int flags, const SegMap& sm,
                                int dk, int dv, int dtype, float* ws, hipStream_t stream);
// recs = H * sm.chunk_recs_per_head(kChunk) chunk records.
size_t delta_ws_floats(long slots, long recs, int dk, int dv);

// The backward pass's forward sweep (uniform batches, bf16): every chunk's
// entering state as bf16 tiles in `states` (layout in delta_chunk.hpp);
// ws as for launch_delta_forward.
hipError_t launch_delta_states(const void* q, const void* k, const void* v, const void* beta, const float* alpha,
                               const float* S0, void* states, const SegMap& sm, int dk, int dv, float* ws,
                               hipStream_t stream);
// The segment composition run backwards: g_end[last] = G_last (or 0),
// g_end[g-1] = map_mt[g] g_end[g] + map_c[g].
hipError_t launch_delta_compose_rev(const float* map_c, const float* map_mt, const float* G_last, float* g_end,
                                    const SegMap& sm, int dk, int dv, hipStream_t stream);

// A training forward of the delta rule (uniform batches, bf16, gated when
// alpha is non-NULL): delta_forward's outputs, and the backward pass's
// context left in ws (delta_backward_ws_floats(...) floats): the chunk
// records, every segment's maps and entering state, and every chunk's
// entering state as bf16 tiles at `states` (= the tiles region of ws).
hipError_t launch_delta_forward_train(const void* q, const void* k, const void* v, const void* beta,
                                      const float* alpha, const float* S0, void* o, float* S_out, void* states,
                                      const SegMap& sm, int dk, int dv, float* ws, hipStream_t stream);

// Backward pass of the delta rule (gated when alpha is non-NULL; uniform
// batches, bf16): dq, dk, dv (bf16), dbeta, dalpha (fp32 [HT][T]) and
// optionally dS0 (fp32) for the loss sum dO . o + <dS_T, S_T>.  ws holds
// delta_backward_ws_floats(...) floats.  after_forward: ws already holds the
// context a training forward on the same inputs left; the forward sweep
// (T records, maps, composition, chunk states) is not run again.
hipError_t launch_delta_backward(const void* q, const void* k, const void* v, const void* beta, const float* alpha,
                                 const float* S0, const void* dO, const float* dS_T, void* dq, void* dk_, void* dv_,
                                 float* dbeta, float* dalpha, float* dS0, const SegMap& sm, int dk, int dv, int dtype,
                                 float* ws, hipStream_t stream, bool after_forward = false);
// The bf16 chunk-state tiles region of a delta_backward workspace.
void* delta_backward_states(float* ws, const SegMap& sm, int dk, int dv);
size_t delta_backward_ws_floats(long slots, long recs, int HT, int T, int dk, int dv);

// Scalar-decay (Mamba-2 / SSD) prefill: segment maps -> elementwise
// composition -> chunked outputs.  alpha fp32 [HT][T].  Segments as la_plan.
hipError_t launch_ssd_forward(const void* q, const void* k, const void* v, const float* alpha,
                              const float* S0, void* o, float* S_out, const SegMap& sm, int dk, int dv,
                              int dtype, float* ws, hipStream_t stream);
size_t ssd_ws_floats(long slots, int dk, int dv);

// Backward pass of LA prefill (bf16, uniform batches): dq, dk, dv (bf16)
// and optionally dS0, dz0 (fp32) for the loss sum dO . o + <dS_T, S_T> +
// <dz_T, z_T>; recomputes the forward states.  ws holds
// la_backward_ws_floats(...) floats.
hipError_t launch_la_backward(const void* q, const void* k, const void* v, const float* S0, const float* z0,
                              const void* dO, const float* dS_T, const float* dz_T, void* dq, void* dk, void* dv,
                              float* dS0, float* dz0, int HT, int T, int dk_, int dv_, int dtype, float eps,
                              const LaPlan& plan, float* ws, hipStream_t stream);
size_t la_backward_ws_floats(int HT, int T, int dk, int dv, const LaPlan& plan);
size_t la_backward_lds_bytes(int dk, int dv);

// Delta-rule decode step on a resident fp32 state (in place); alpha (fp32
// [NH]) selects the gated rule, NULL = ungated; beta NULL with alpha given
// selects the scalar-decay rule (no correction).
hipError_t launch_delta_decode(const void* q, const void* k, const void* v, const void* beta,
                               const float* alpha, float* S, void* o, void* pred, int flags, int NH, int dk,
                               int dv, int dtype, hipStream_t stream);

// Linear attention decode step on a resident fp32 state (in place).
hipError_t launch_la_decode(const void* q, const void* k, const void* v, float* S,
                            float* z, void* o, int NH, int dk, int dv, int dtype,
                            float eps, hipStream_t stream);

}  // namespace la
