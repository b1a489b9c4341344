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
"""
from .binding import (  # noqa: F401
    CHUNK, LA_BF16, LA_F32, LinAttnError, UnsupportedError, delta_forward,
    delta_decode_step, delta_forward_workspace_bytes, gated_delta_decode_step, gated_delta_forward,
    la_decode_step, la_forward, la_forward_workspace_bytes, lib, ssd_decode_step, ssd_forward,
    ssd_forward_workspace_bytes)
