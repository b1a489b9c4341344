"""MI355X-native causal linear attention (ELU+1) and delta-rule fast-weight memory.

Public API (same names as the C ABI in include/linattn.h):
    la_forward(q, k, v, S0=None, z0=None, eps=1e-6) -> (o, S_T, z_T)
    delta_forward(q, k, v, beta, S0=None) -> (o, S_T)
    la_decode_step(q, k, v, S, z, eps=1e-6) -> o        (S, z updated in place)
    delta_decode_step(q, k, v, beta, S) -> o             (S updated in place)
    gated_delta_forward(q, k, v, beta, alpha, S0=None) -> (o, S_T)
    gated_delta_decode_step(q, k, v, beta, alpha, S) -> o (S updated in place)
    ssd_forward(q, k, v, alpha, S0=None) -> (o, S_T)
    ssd_decode_step(q, k, v, alpha, S) -> o               (S updated in place)
    delta_forward_ex / delta_decode_step_ex: the delta rules with in-kernel q/k
        L2 normalisation, beta = sigmoid(logit) and the read-then-write predictions
    la_backward(q, k, v, dO, S0=None, z0=None, dS_T=None, dz_T=None) -> (dq, dk, dv, dS0, dz0)
    delta_backward(q, k, v, beta, dO, alpha=None, S0=None, dS_T=None) -> (dq, dk, dv, dbeta, dalpha, dS0)
    la_forward_packed / delta_forward_packed / ssd_forward_packed: packed batches of
        variable-length sequences ([H][T_total][d], offsets cu_seqlens), each
        sequence with its own initial and final state
"""
from .binding import (  # noqa: F401
    CHUNK, LA_BETA_SIGMOID, LA_BF16, LA_F32, LA_NORMALIZE_QK, LinAttnError, UnsupportedError, delta_backward,
    delta_backward_workspace_bytes, delta_decode_step_ex,
    delta_forward, delta_forward_ex, delta_forward_packed, delta_forward_packed_workspace_bytes,
    delta_decode_step, delta_forward_workspace_bytes, gated_delta_decode_step, gated_delta_forward,
    la_backward, la_backward_workspace_bytes, la_decode_step, la_forward, la_forward_packed, la_forward_packed_workspace_bytes, la_forward_workspace_bytes,
    lib, ssd_decode_step, ssd_forward, ssd_forward_packed, ssd_forward_packed_workspace_bytes,
    ssd_forward_workspace_bytes)
