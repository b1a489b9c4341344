// Entry points of api.hip for the library's other translation units.  Not
// installed; the public interface is include/linattn.h.
#pragma once
#include <stddef.h>

#include "linattn.h"

namespace la_api {

// la_forward's validation and launch with a caller-chosen workspace; fn
// names the public call in error messages.
la_status la_forward_ws(const char* fn, const void* q, const void* k, const void* v, const float* S0,
                        const float* z0, void* o, float* S_out, float* z_out, int B, int H, int T, int dk, int dv,
                        int dtype, float eps, int chunk, void* workspace, size_t workspace_bytes, void* stream);
// la_forward_workspace_bytes for these sizes (0 if they are invalid).
size_t la_forward_ws_bytes(const char* fn, int B, int H, int T, int dk, int dv, int chunk);
// Records msg as the calling thread's la_last_error() and returns st.
la_status set_error(la_status st, const char* msg);

}  // namespace la_api
