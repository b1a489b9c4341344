// Launchers of the prefills for chunk sizes other than the main kernels' 64
// tokens: linear attention (la_chunked.hip) and the plain delta rule
// (delta_chunked.hip).  Internal; the public interface is include/linattn.h.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

#include "segments.hpp"

namespace la {

// Chunk sizes the blocked path takes: 16, 32 and 128 tokens (fp32 inputs:
// 16 and 32; a 128-token fp32 chunk does not fit the LDS).
bool la_chunked_supported(int chunk, int dtype);

// Uniform batches only.  Three launches: every segment's sum of
// phi(K)^T [V | 1] but the last (sm.L tokens a segment, a multiple of the
// chunk), their prefix from S0, z0 (or zero) as each segment's entering
// state, and the chunk loop of every segment writing o (and S_out, z_out
// from the last segment of each sequence).  ws holds
// la_chunked_ws_floats(H * NS, dk, dv) floats.  dtype 0 = fp32, 1 = bf16.
hipError_t launch_la_forward_chunked(const void* q, const void* k, const void* v, const float* S0,
                                     const float* z0, void* o, float* S_out, float* z_out, const SegMap& sm,
                                     int dk, int dv, int dtype, float eps, int chunk, float* ws,
                                     hipStream_t stream);
size_t la_chunked_ws_floats(long slots, int dk, int dv);

// The delta rule (ungated, bf16 inputs, no in-kernel transforms), uniform
// batches, chunk 16, 32 or 128: every segment's affine map (M_g, N_g) but
// the last's by a chunk loop of `chunk` tokens, their composition from S0
// (launch_delta_compose), then every segment's chunk loop writing o (and
// S_out from the last segment of each sequence).  ws holds
// delta_chunked_ws_floats(H * NS, dk, dv) floats.
bool delta_chunked_supported(int chunk);
hipError_t launch_delta_forward_chunked(const void* q, const void* k, const void* v, const void* beta,
                                        const float* S0, void* o, float* S_out, const SegMap& sm, int dk, int dv,
                                        int chunk, float* ws, hipStream_t stream);
size_t delta_chunked_ws_floats(long slots, int dk, int dv);

// S_in(0) = S0 (or 0), S_in(g+1) = M_g S_in(g) + N_g over each sequence's
// segments (delta_prefill.hip; uniform batches): maps N_g ([dk][dv]) and
// M_g ([dk][dk]) per slot, states [dk][dv] per slot.
hipError_t launch_delta_compose(const float* map_n, const float* map_m, const float* S0, float* state_in,
                                const SegMap& sm, int dk, int dv, hipStream_t stream);

}  // namespace la
