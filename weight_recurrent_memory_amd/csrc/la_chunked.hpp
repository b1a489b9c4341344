// Launcher of the linear-attention prefill for chunk sizes other than the
// fused kernel's 64 tokens (internal; the public interface is
// include/linattn.h).
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

}  // namespace la
