"""Thin Python binding of the C ABI in include/linattn.h.

The functions carry the ABI's names and do argument marshalling only:
shape/dtype bookkeeping, output and workspace allocation with torch (device
memory), the current HIP stream, and status -> exception mapping.  Every step
of the computation runs in the HIP library; if ``liblinattn.so`` is missing
or fails to load, every call raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblinattn.so")

LA_F32, LA_BF16 = 0, 1
LA_NORMALIZE_QK, LA_BETA_SIGMOID = 1, 2
LA_OK, LA_ERR_INVALID_ARG, LA_ERR_UNSUPPORTED, LA_ERR_WORKSPACE, LA_ERR_HIP = range(5)
CHUNK = 64

_lock = threading.Lock()
_lib = None


class LinAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class UnsupportedError(LinAttnError, NotImplementedError):
    pass


def lib():
    """The loaded HIP library (ctypes).  Raises if it is not built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with "
                    "`python -m weight_recurrent_memory_amd.build_lib` (hipcc, gfx950)")
            L = ctypes.CDLL(LIB_PATH)
            vp, fp, i, sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
            L.la_forward_workspace_bytes.argtypes = [i, i, i, i, i, i]
            L.la_forward_workspace_bytes.restype = sz
            L.delta_forward_workspace_bytes.argtypes = [i, i, i, i, i, i]
            L.delta_forward_workspace_bytes.restype = sz
            L.la_forward.argtypes = [vp, vp, vp, fp, fp, vp, fp, fp, i, i, i, i, i, i,
                                     ctypes.c_float, i, vp, sz, vp]
            L.la_forward.restype = i
            L.la_forward_lookback_polls.argtypes = L.la_forward.argtypes + [i]
            L.la_forward_lookback_polls.restype = i
            L.la_forward_noalloc.argtypes = [vp, vp, vp, fp, fp, vp, fp, fp, i, i, i, i, i, i, ctypes.c_float, i, vp]
            L.la_forward_noalloc.restype = i
            L.delta_forward.argtypes = [vp, vp, vp, vp, fp, vp, fp, i, i, i, i, i, i, i, vp, sz, vp]
            L.delta_forward.restype = i
            L.la_decode_step.argtypes = [vp, vp, vp, fp, fp, vp, i, i, i, i, i, ctypes.c_float, vp]
            L.la_decode_step.restype = i
            L.delta_decode_step.argtypes = [vp, vp, vp, vp, fp, vp, i, i, i, i, i, vp]
            L.delta_decode_step.restype = i
            L.gated_delta_forward.argtypes = [vp, vp, vp, vp, fp, fp, vp, fp, i, i, i, i, i, i, i, vp, sz, vp]
            L.gated_delta_forward.restype = i
            L.gated_delta_decode_step.argtypes = [vp, vp, vp, vp, fp, fp, vp, i, i, i, i, i, vp]
            L.gated_delta_decode_step.restype = i
            L.ssd_forward_workspace_bytes.argtypes = [i, i, i, i, i, i]
            L.ssd_forward_workspace_bytes.restype = sz
            L.ssd_forward.argtypes = [vp, vp, vp, fp, fp, vp, fp, i, i, i, i, i, i, i, vp, sz, vp]
            L.ssd_forward.restype = i
            L.ssd_decode_step.argtypes = [vp, vp, vp, fp, fp, vp, i, i, i, i, i, vp]
            L.ssd_decode_step.restype = i
            L.delta_forward_ex.argtypes = [vp, vp, vp, vp, fp, fp, vp, fp, vp, i, i, i, i, i, i, i, i, vp, sz, vp]
            L.delta_forward_ex.restype = i
            L.delta_decode_step_ex.argtypes = [vp, vp, vp, vp, fp, fp, vp, vp, i, i, i, i, i, i, vp]
            L.delta_decode_step_ex.restype = i
            L.la_forward_packed_workspace_bytes.argtypes = [vp, i, i, i, i, i, i]
            L.la_forward_packed_workspace_bytes.restype = sz
            L.delta_forward_packed_workspace_bytes.argtypes = [vp, i, i, i, i, i, i]
            L.delta_forward_packed_workspace_bytes.restype = sz
            L.ssd_forward_packed_workspace_bytes.argtypes = [vp, i, i, i, i, i, i]
            L.ssd_forward_packed_workspace_bytes.restype = sz
            L.la_forward_packed.argtypes = [vp, vp, vp, vp, vp, i, fp, fp, vp, fp, fp, i, i, i, i, i,
                                            ctypes.c_float, i, vp, sz, vp]
            L.la_forward_packed.restype = i
            L.delta_forward_packed.argtypes = [vp, vp, vp, vp, fp, vp, vp, i, fp, vp, fp, vp, i, i, i, i, i, i, i,
                                               vp, sz, vp]
            L.delta_forward_packed.restype = i
            L.ssd_forward_packed.argtypes = [vp, vp, vp, fp, vp, vp, i, fp, vp, fp, i, i, i, i, i, i, vp, sz, vp]
            L.ssd_forward_packed.restype = i
            L.la_backward_workspace_bytes.argtypes = [i, i, i, i, i, i]
            L.la_backward_workspace_bytes.restype = sz
            L.la_backward.argtypes = [vp, vp, vp, fp, fp, vp, fp, fp, vp, vp, vp, fp, fp, i, i, i, i, i, i,
                                      ctypes.c_float, i, vp, sz, vp]
            L.la_backward.restype = i
            L.delta_backward_workspace_bytes.argtypes = [i, i, i, i, i, i]
            L.delta_backward_workspace_bytes.restype = sz
            L.delta_backward.argtypes = [vp, vp, vp, vp, fp, fp, vp, fp, vp, vp, vp, fp, fp, fp, i, i, i, i, i, i,
                                         i, vp, sz, vp]
            L.delta_backward.restype = i
            L.delta_forward_train.argtypes = [vp, vp, vp, vp, fp, fp, vp, fp, i, i, i, i, i, i, i, vp, sz, vp]
            L.delta_forward_train.restype = i
            L.delta_backward_after_forward.argtypes = L.delta_backward.argtypes
            L.delta_backward_after_forward.restype = i
            L.la_status_string.argtypes = [i]
            L.la_status_string.restype = ctypes.c_char_p
            L.la_last_error.argtypes = []
            L.la_last_error.restype = ctypes.c_char_p
            _lib = L
    return _lib


def _check(status: int):
    if status == LA_OK:
        return
    L = lib()
    msg = "%s: %s" % (L.la_status_string(status).decode(), L.la_last_error().decode())
    if status == LA_ERR_INVALID_ARG:
        raise ValueError(msg)
    if status == LA_ERR_UNSUPPORTED:
        raise UnsupportedError(status, msg)
    raise LinAttnError(status, msg)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return LA_BF16
    if t.dtype == torch.float32:
        return LA_F32
    raise ValueError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype, shape, device):
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def la_forward_workspace_bytes(B, H, T, dk, dv, chunk=CHUNK) -> int:
    return int(lib().la_forward_workspace_bytes(B, H, T, dk, dv, chunk))


def delta_forward_workspace_bytes(B, H, T, dk, dv, chunk=CHUNK) -> int:
    return int(lib().delta_forward_workspace_bytes(B, H, T, dk, dv, chunk))


def _workspace(nbytes, device, workspace):
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def la_forward(q, k, v, S0=None, z0=None, eps=1e-6, chunk=CHUNK, *, o=None, S_out=None,
               z_out=None, workspace=None, return_state=True, lookback_polls=None):
    """Causal ELU+1 linear attention prefill.  q, k: [B,H,T,dk]; v: [B,H,T,dv]
    (bf16 or fp32, CUDA/HIP tensors).  Returns (o, S_T, z_T); S_T/z_T are fp32
    and None when return_state is False.  S_out/z_out may be S0/z0.
    lookback_polls (tests only) calls la_forward_lookback_polls with that
    wait bound instead of la_forward."""
    code = _dtype_code(q)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    _need(k, "k", q.dtype, (B, H, T, dk), dev)
    _need(v, "v", q.dtype, (B, H, T, dv), dev)
    _need(q, "q", q.dtype, (B, H, T, dk), dev)
    if S0 is not None:
        _need(S0, "S0", torch.float32, (B, H, dk, dv), dev)
    if z0 is not None:
        _need(z0, "z0", torch.float32, (B, H, dk), dev)
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=q.dtype, device=dev)
    _need(o, "o", q.dtype, (B, H, T, dv), dev)
    if return_state:
        if S_out is None:
            S_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
        if z_out is None:
            z_out = torch.empty((B, H, dk), dtype=torch.float32, device=dev)
        _need(S_out, "S_out", torch.float32, (B, H, dk, dv), dev)
        _need(z_out, "z_out", torch.float32, (B, H, dk), dev)
    ws, wsb = _workspace(la_forward_workspace_bytes(B, H, T, dk, dv, chunk), dev, workspace)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(S0), _ptr(z0), _ptr(o), _ptr(S_out), _ptr(z_out),
            B, H, T, dk, dv, code, float(eps), int(chunk), _ptr(ws), wsb, _stream(dev))
    if lookback_polls is None:
        _check(lib().la_forward(*args))
    else:
        _check(lib().la_forward_lookback_polls(*args, int(lookback_polls)))
    return o, S_out, z_out


def la_forward_noalloc(q, k, v, S0=None, z0=None, eps=1e-6, chunk=CHUNK, *, o=None, S_out=None, z_out=None):
    """la_forward on the library's fixed per-GPU scratch instead of a
    workspace: the call allocates nothing when o, S_out and z_out are given.
    Returns (o, S_T, z_T)."""
    code = _dtype_code(q)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    _need(k, "k", q.dtype, (B, H, T, dk), dev)
    _need(v, "v", q.dtype, (B, H, T, dv), dev)
    if S0 is not None:
        _need(S0, "S0", torch.float32, (B, H, dk, dv), dev)
    if z0 is not None:
        _need(z0, "z0", torch.float32, (B, H, dk), dev)
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=q.dtype, device=dev)
    if S_out is None:
        S_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if z_out is None:
        z_out = torch.empty((B, H, dk), dtype=torch.float32, device=dev)
    _need(o, "o", q.dtype, (B, H, T, dv), dev)
    _need(S_out, "S_out", torch.float32, (B, H, dk, dv), dev)
    _need(z_out, "z_out", torch.float32, (B, H, dk), dev)
    _check(lib().la_forward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(S0), _ptr(z0), _ptr(o), _ptr(S_out),
                                    _ptr(z_out), B, H, T, dk, dv, code, float(eps), int(chunk), _stream(dev)))
    return o, S_out, z_out


def delta_forward(q, k, v, beta, S0=None, chunk=CHUNK, *, o=None, S_out=None, workspace=None,
                  return_state=True):
    """Delta-rule prefill.  q, k: [B,H,T,dk]; v: [B,H,T,dv]; beta: [B,H,T].
    Returns (o, S_T)."""
    return _delta_forward(q, k, v, beta, None, S0, chunk, o, S_out, workspace, return_state)


def gated_delta_forward(q, k, v, beta, alpha, S0=None, chunk=CHUNK, *, o=None, S_out=None, workspace=None,
                        return_state=True):
    """Gated delta-rule prefill: alpha [B,H,T] fp32 forgetting factors in
    (0, 1], applied to the state before each correction.  Returns (o, S_T)."""
    return _delta_forward(q, k, v, beta, alpha, S0, chunk, o, S_out, workspace, return_state)


def _delta_forward(q, k, v, beta, alpha, S0, chunk, o, S_out, workspace, return_state):
    code = _dtype_code(q)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    _need(k, "k", q.dtype, (B, H, T, dk), dev)
    _need(v, "v", q.dtype, (B, H, T, dv), dev)
    _need(beta, "beta", q.dtype, (B, H, T), dev)
    _need(q, "q", q.dtype, (B, H, T, dk), dev)
    if alpha is not None:
        _need(alpha, "alpha", torch.float32, (B, H, T), dev)
    if S0 is not None:
        _need(S0, "S0", torch.float32, (B, H, dk, dv), dev)
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=q.dtype, device=dev)
    _need(o, "o", q.dtype, (B, H, T, dv), dev)
    if return_state:
        if S_out is None:
            S_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
        _need(S_out, "S_out", torch.float32, (B, H, dk, dv), dev)
    ws, wsb = _workspace(delta_forward_workspace_bytes(B, H, T, dk, dv, chunk), dev, workspace)
    if alpha is None:
        _check(lib().delta_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(S0), _ptr(o), _ptr(S_out),
                                   B, H, T, dk, dv, code, int(chunk), _ptr(ws), wsb, _stream(dev)))
    else:
        _check(lib().gated_delta_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(alpha), _ptr(S0), _ptr(o),
                                         _ptr(S_out), B, H, T, dk, dv, code, int(chunk), _ptr(ws), wsb,
                                         _stream(dev)))
    return o, S_out


def la_decode_step(q, k, v, S, z, eps=1e-6, *, o=None):
    """One decode step; S [N,H,dk,dv] and z [N,H,dk] (fp32) are updated in
    place.  q, k: [N,H,dk]; v: [N,H,dv].  Returns o [N,H,dv]."""
    code = _dtype_code(q)
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    _need(k, "k", q.dtype, (N, H, dk), dev)
    _need(v, "v", q.dtype, (N, H, dv), dev)
    _need(S, "S", torch.float32, (N, H, dk, dv), dev)
    _need(z, "z", torch.float32, (N, H, dk), dev)
    if o is None:
        o = torch.empty((N, H, dv), dtype=q.dtype, device=dev)
    _need(o, "o", q.dtype, (N, H, dv), dev)
    _check(lib().la_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(S), _ptr(z), _ptr(o), N, H, dk, dv,
                                code, float(eps), _stream(dev)))
    return o


def delta_decode_step(q, k, v, beta, S, *, o=None):
    """One delta-rule decode step; S [N,H,dk,dv] (fp32) is updated in place.
    q, k: [N,H,dk]; v: [N,H,dv]; beta: [N,H] (same dtype as q).  Returns
    o [N,H,dv] = S_new^T q."""
    return _delta_decode(q, k, v, beta, None, S, o)


def gated_delta_decode_step(q, k, v, beta, alpha, S, *, o=None):
    """One gated delta-rule decode step: S (fp32, in place) is decayed by
    alpha [N,H] (fp32) before the correction.  Returns o [N,H,dv]."""
    return _delta_decode(q, k, v, beta, alpha, S, o)


def _delta_decode(q, k, v, beta, alpha, S, o):
    code = _dtype_code(q)
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    _need(k, "k", q.dtype, (N, H, dk), dev)
    _need(v, "v", q.dtype, (N, H, dv), dev)
    _need(beta, "beta", q.dtype, (N, H), dev)
    _need(S, "S", torch.float32, (N, H, dk, dv), dev)
    if alpha is not None:
        _need(alpha, "alpha", torch.float32, (N, H), dev)
    if o is None:
        o = torch.empty((N, H, dv), dtype=q.dtype, device=dev)
    _need(o, "o", q.dtype, (N, H, dv), dev)
    if alpha is None:
        _check(lib().delta_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(S), _ptr(o), N, H, dk, dv,
                                       code, _stream(dev)))
    else:
        _check(lib().gated_delta_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(alpha), _ptr(S), _ptr(o),
                                             N, H, dk, dv, code, _stream(dev)))
    return o


def ssd_forward_workspace_bytes(B, H, T, dk, dv, chunk=CHUNK) -> int:
    return int(lib().ssd_forward_workspace_bytes(B, H, T, dk, dv, chunk))


def ssd_forward(q, k, v, alpha, S0=None, chunk=CHUNK, *, o=None, S_out=None, workspace=None, return_state=True):
    """Scalar-decay (Mamba-2 / SSD form) prefill: S_t = alpha_t S_{t-1} + k_t v_t^T,
    o_t = S_t^T q_t.  q, k: [B,H,T,dk]; v: [B,H,T,dv] (bf16); alpha: [B,H,T]
    fp32.  Returns (o, S_T)."""
    code = _dtype_code(q)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    _need(k, "k", q.dtype, (B, H, T, dk), dev)
    _need(v, "v", q.dtype, (B, H, T, dv), dev)
    _need(alpha, "alpha", torch.float32, (B, H, T), dev)
    if S0 is not None:
        _need(S0, "S0", torch.float32, (B, H, dk, dv), dev)
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=q.dtype, device=dev)
    _need(o, "o", q.dtype, (B, H, T, dv), dev)
    if return_state:
        if S_out is None:
            S_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
        _need(S_out, "S_out", torch.float32, (B, H, dk, dv), dev)
    ws, wsb = _workspace(ssd_forward_workspace_bytes(B, H, T, dk, dv, chunk), dev, workspace)
    _check(lib().ssd_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(S0), _ptr(o), _ptr(S_out), B, H, T, dk,
                             dv, code, int(chunk), _ptr(ws), wsb, _stream(dev)))
    return o, S_out


def ssd_decode_step(q, k, v, alpha, S, *, o=None):
    """One scalar-decay decode step; S [N,H,dk,dv] (fp32) is updated in place:
    S <- alpha S + k v^T.  q, k: [N,H,dk]; v: [N,H,dv]; alpha: [N,H] fp32.
    Returns o [N,H,dv] = S_new^T q."""
    code = _dtype_code(q)
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    _need(k, "k", q.dtype, (N, H, dk), dev)
    _need(v, "v", q.dtype, (N, H, dv), dev)
    _need(alpha, "alpha", torch.float32, (N, H), dev)
    _need(S, "S", torch.float32, (N, H, dk, dv), dev)
    if o is None:
        o = torch.empty((N, H, dv), dtype=q.dtype, device=dev)
    _need(o, "o", q.dtype, (N, H, dv), dev)
    _check(lib().ssd_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(S), _ptr(o), N, H, dk, dv, code,
                                 _stream(dev)))
    return o


def _flags(normalize_qk, beta_logits):
    return (LA_NORMALIZE_QK if normalize_qk else 0) | (LA_BETA_SIGMOID if beta_logits else 0)


def delta_forward_ex(q, k, v, beta, alpha=None, S0=None, chunk=CHUNK, *, normalize_qk=False, beta_logits=False,
                     return_pred=False, o=None, S_out=None, pred=None, workspace=None):
    """Delta-rule prefill with serving options: gated when alpha ([B,H,T]
    fp32) is given; q/k L2-normalised in the kernel with normalize_qk; beta
    read as logits with beta_logits; with return_pred the read-then-write
    predictions [B,H,T,dv] are returned too.  Returns (o, S_T[, pred])."""
    code = _dtype_code(q)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    _need(k, "k", q.dtype, (B, H, T, dk), dev)
    _need(v, "v", q.dtype, (B, H, T, dv), dev)
    _need(beta, "beta", q.dtype, (B, H, T), dev)
    if alpha is not None:
        _need(alpha, "alpha", torch.float32, (B, H, T), dev)
    if S0 is not None:
        _need(S0, "S0", torch.float32, (B, H, dk, dv), dev)
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=q.dtype, device=dev)
    _need(o, "o", q.dtype, (B, H, T, dv), dev)
    if S_out is None:
        S_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    _need(S_out, "S_out", torch.float32, (B, H, dk, dv), dev)
    if return_pred:
        if pred is None:
            pred = torch.empty((B, H, T, dv), dtype=q.dtype, device=dev)
        _need(pred, "pred", q.dtype, (B, H, T, dv), dev)
    else:
        pred = None
    ws, wsb = _workspace(delta_forward_workspace_bytes(B, H, T, dk, dv, chunk), dev, workspace)
    _check(lib().delta_forward_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(alpha), _ptr(S0), _ptr(o),
                                  _ptr(S_out), _ptr(pred), _flags(normalize_qk, beta_logits), B, H, T, dk, dv, code,
                                  int(chunk), _ptr(ws), wsb, _stream(dev)))
    return (o, S_out, pred) if return_pred else (o, S_out)


def delta_decode_step_ex(q, k, v, beta, S, alpha=None, *, normalize_qk=False, beta_logits=False,
                         return_pred=False, o=None, pred=None):
    """One delta-rule decode step with serving options (see delta_forward_ex);
    S is updated in place.  Returns o, or (o, pred) with return_pred."""
    code = _dtype_code(q)
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    _need(k, "k", q.dtype, (N, H, dk), dev)
    _need(v, "v", q.dtype, (N, H, dv), dev)
    _need(beta, "beta", q.dtype, (N, H), dev)
    _need(S, "S", torch.float32, (N, H, dk, dv), dev)
    if alpha is not None:
        _need(alpha, "alpha", torch.float32, (N, H), dev)
    if o is None:
        o = torch.empty((N, H, dv), dtype=q.dtype, device=dev)
    _need(o, "o", q.dtype, (N, H, dv), dev)
    if return_pred:
        if pred is None:
            pred = torch.empty((N, H, dv), dtype=q.dtype, device=dev)
        _need(pred, "pred", q.dtype, (N, H, dv), dev)
    else:
        pred = None
    _check(lib().delta_decode_step_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(alpha), _ptr(S), _ptr(o),
                                      _ptr(pred), _flags(normalize_qk, beta_logits), N, H, dk, dv, code,
                                      _stream(dev)))
    return (o, pred) if return_pred else o


# ------------------------------------------------------------ packed batches

def _offsets(cu_seqlens, cu_seqlens_host, dev):
    """(N, device offsets, host offsets) of a packed batch.  cu_seqlens is an
    int32 device tensor [N+1]; the host copy is taken from cu_seqlens_host
    (any int sequence) or, if None, copied from the device."""
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.device != dev:
        raise ValueError(f"cu_seqlens must be a 1-D int32 tensor on {dev}")
    if not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be contiguous")
    host = cu_seqlens.cpu() if cu_seqlens_host is None else torch.as_tensor(cu_seqlens_host, dtype=torch.int32)
    host = host.contiguous()
    if host.numel() != cu_seqlens.numel():
        raise ValueError("cu_seqlens_host and cu_seqlens differ in length")
    return cu_seqlens.numel() - 1, host


def la_forward_packed_workspace_bytes(cu_seqlens_host, H, dk, dv, chunk=CHUNK) -> int:
    host = torch.as_tensor(cu_seqlens_host, dtype=torch.int32).contiguous()
    return int(lib().la_forward_packed_workspace_bytes(_ptr(host), host.numel() - 1, H, int(host[-1]), dk, dv, chunk))


def delta_forward_packed_workspace_bytes(cu_seqlens_host, H, dk, dv, chunk=CHUNK) -> int:
    host = torch.as_tensor(cu_seqlens_host, dtype=torch.int32).contiguous()
    return int(lib().delta_forward_packed_workspace_bytes(_ptr(host), host.numel() - 1, H, int(host[-1]), dk, dv,
                                                          chunk))


def ssd_forward_packed_workspace_bytes(cu_seqlens_host, H, dk, dv, chunk=CHUNK) -> int:
    host = torch.as_tensor(cu_seqlens_host, dtype=torch.int32).contiguous()
    return int(lib().ssd_forward_packed_workspace_bytes(_ptr(host), host.numel() - 1, H, int(host[-1]), dk, dv,
                                                        chunk))


def la_forward_packed(q, k, v, cu_seqlens, S0=None, z0=None, eps=1e-6, chunk=CHUNK, *, cu_seqlens_host=None,
                      o=None, S_out=None, z_out=None, workspace=None):
    """LA prefill over a packed batch: q, k [H,T_total,dk]; v [H,T_total,dv];
    sequence n is rows cu_seqlens[n]..cu_seqlens[n+1]-1 and has its own
    initial/final state S [N,H,dk,dv], z [N,H,dk].  Returns (o, S_out, z_out)."""
    code = _dtype_code(q)
    H, T, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    N, host = _offsets(cu_seqlens, cu_seqlens_host, dev)
    _need(k, "k", q.dtype, (H, T, dk), dev)
    _need(v, "v", q.dtype, (H, T, dv), dev)
    _need(q, "q", q.dtype, (H, T, dk), dev)
    if S0 is not None:
        _need(S0, "S0", torch.float32, (N, H, dk, dv), dev)
    if z0 is not None:
        _need(z0, "z0", torch.float32, (N, H, dk), dev)
    o = torch.empty((H, T, dv), dtype=q.dtype, device=dev) if o is None else o
    S_out = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev) if S_out is None else S_out
    z_out = torch.empty((N, H, dk), dtype=torch.float32, device=dev) if z_out is None else z_out
    _need(o, "o", q.dtype, (H, T, dv), dev)
    _need(S_out, "S_out", torch.float32, (N, H, dk, dv), dev)
    _need(z_out, "z_out", torch.float32, (N, H, dk), dev)
    nb = int(lib().la_forward_packed_workspace_bytes(_ptr(host), N, H, T, dk, dv, chunk))
    ws, wsb = _workspace(nb, dev, workspace)
    _check(lib().la_forward_packed(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), _ptr(host), N, _ptr(S0), _ptr(z0),
                                   _ptr(o), _ptr(S_out), _ptr(z_out), H, T, dk, dv, code, float(eps), int(chunk),
                                   _ptr(ws), wsb, _stream(dev)))
    return o, S_out, z_out


def delta_forward_packed(q, k, v, beta, cu_seqlens, alpha=None, S0=None, chunk=CHUNK, *, normalize_qk=False,
                         beta_logits=False, return_pred=False, cu_seqlens_host=None, o=None, S_out=None, pred=None,
                         workspace=None):
    """Delta-rule (gated when alpha [H,T_total] fp32 is given) prefill over a
    packed batch; options as delta_forward_ex.  beta [H,T_total].  Returns
    (o, S_out[, pred]) with S_out [N,H,dk,dv]."""
    code = _dtype_code(q)
    H, T, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    N, host = _offsets(cu_seqlens, cu_seqlens_host, dev)
    _need(k, "k", q.dtype, (H, T, dk), dev)
    _need(v, "v", q.dtype, (H, T, dv), dev)
    _need(beta, "beta", q.dtype, (H, T), dev)
    _need(q, "q", q.dtype, (H, T, dk), dev)
    if alpha is not None:
        _need(alpha, "alpha", torch.float32, (H, T), dev)
    if S0 is not None:
        _need(S0, "S0", torch.float32, (N, H, dk, dv), dev)
    o = torch.empty((H, T, dv), dtype=q.dtype, device=dev) if o is None else o
    S_out = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev) if S_out is None else S_out
    _need(o, "o", q.dtype, (H, T, dv), dev)
    _need(S_out, "S_out", torch.float32, (N, H, dk, dv), dev)
    if return_pred:
        pred = torch.empty((H, T, dv), dtype=q.dtype, device=dev) if pred is None else pred
        _need(pred, "pred", q.dtype, (H, T, dv), dev)
    else:
        pred = None
    nb = int(lib().delta_forward_packed_workspace_bytes(_ptr(host), N, H, T, dk, dv, chunk))
    ws, wsb = _workspace(nb, dev, workspace)
    _check(lib().delta_forward_packed(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(alpha), _ptr(cu_seqlens),
                                      _ptr(host), N, _ptr(S0), _ptr(o), _ptr(S_out), _ptr(pred),
                                      _flags(normalize_qk, beta_logits), H, T, dk, dv, code, int(chunk), _ptr(ws), wsb,
                                      _stream(dev)))
    return (o, S_out, pred) if return_pred else (o, S_out)


def ssd_forward_packed(q, k, v, alpha, cu_seqlens, S0=None, chunk=CHUNK, *, cu_seqlens_host=None, o=None,
                       S_out=None, workspace=None):
    """Scalar-decay prefill over a packed batch: alpha [H,T_total] fp32.
    Returns (o, S_out) with S_out [N,H,dk,dv]."""
    code = _dtype_code(q)
    H, T, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    N, host = _offsets(cu_seqlens, cu_seqlens_host, dev)
    _need(k, "k", q.dtype, (H, T, dk), dev)
    _need(v, "v", q.dtype, (H, T, dv), dev)
    _need(alpha, "alpha", torch.float32, (H, T), dev)
    _need(q, "q", q.dtype, (H, T, dk), dev)
    if S0 is not None:
        _need(S0, "S0", torch.float32, (N, H, dk, dv), dev)
    o = torch.empty((H, T, dv), dtype=q.dtype, device=dev) if o is None else o
    S_out = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev) if S_out is None else S_out
    _need(o, "o", q.dtype, (H, T, dv), dev)
    _need(S_out, "S_out", torch.float32, (N, H, dk, dv), dev)
    nb = int(lib().ssd_forward_packed_workspace_bytes(_ptr(host), N, H, T, dk, dv, chunk))
    ws, wsb = _workspace(nb, dev, workspace)
    _check(lib().ssd_forward_packed(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(cu_seqlens), _ptr(host), N,
                                    _ptr(S0), _ptr(o), _ptr(S_out), H, T, dk, dv, code, int(chunk), _ptr(ws), wsb,
                                    _stream(dev)))
    return o, S_out


def la_backward_workspace_bytes(B, H, T, dk, dv, chunk=CHUNK) -> int:
    return int(lib().la_backward_workspace_bytes(B, H, T, dk, dv, chunk))


def la_backward(q, k, v, dO, S0=None, z0=None, dS_T=None, dz_T=None, eps=1e-6, chunk=CHUNK, *, dq=None, dk=None,
                dv=None, return_state_grads=True, workspace=None):
    """Gradients of L = sum dO . o + <dS_T, S_T> + <dz_T, z_T> for la_forward
    (bf16).  Returns (dq, dk, dv, dS0, dz0); dS0/dz0 are None when
    return_state_grads is False."""
    code = _dtype_code(q)
    B, H, T, dkk = q.shape
    dvv = v.shape[-1]
    dev = q.device
    _need(k, "k", q.dtype, (B, H, T, dkk), dev)
    _need(v, "v", q.dtype, (B, H, T, dvv), dev)
    _need(dO, "dO", q.dtype, (B, H, T, dvv), dev)
    for t, name, shape in ((S0, "S0", (B, H, dkk, dvv)), (z0, "z0", (B, H, dkk)), (dS_T, "dS_T", (B, H, dkk, dvv)),
                           (dz_T, "dz_T", (B, H, dkk))):
        if t is not None:
            _need(t, name, torch.float32, shape, dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _need(dq, "dq", q.dtype, (B, H, T, dkk), dev)
    _need(dk, "dk", q.dtype, (B, H, T, dkk), dev)
    _need(dv, "dv", q.dtype, (B, H, T, dvv), dev)
    dS0 = torch.empty((B, H, dkk, dvv), dtype=torch.float32, device=dev) if return_state_grads else None
    dz0 = torch.empty((B, H, dkk), dtype=torch.float32, device=dev) if return_state_grads else None
    ws, wsb = _workspace(la_backward_workspace_bytes(B, H, T, dkk, dvv, chunk), dev, workspace)
    _check(lib().la_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(S0), _ptr(z0), _ptr(dO), _ptr(dS_T), _ptr(dz_T), _ptr(dq),
                             _ptr(dk), _ptr(dv), _ptr(dS0), _ptr(dz0), B, H, T, dkk, dvv, code, float(eps), int(chunk),
                             _ptr(ws), wsb, _stream(dev)))
    return dq, dk, dv, dS0, dz0


def delta_backward_workspace_bytes(B, H, T, dk, dv, chunk=CHUNK) -> int:
    return int(lib().delta_backward_workspace_bytes(B, H, T, dk, dv, chunk))


def delta_backward(q, k, v, beta, dO, alpha=None, S0=None, dS_T=None, chunk=CHUNK, *, dq=None, dk=None, dv=None,
                   return_state_grad=True, workspace=None):
    """Gradients of L = sum dO . o + <dS_T, S_T> for delta_forward (alpha
    None) or gated_delta_forward (bf16).  Returns (dq, dk, dv, dbeta,
    dalpha, dS0); dbeta and dalpha are fp32 [B,H,T] (dalpha None for the
    plain rule), dS0 None when return_state_grad is False."""
    return _delta_backward("delta_backward", q, k, v, beta, dO, alpha, S0, dS_T, chunk, dq, dk, dv,
                           return_state_grad, workspace)


def delta_forward_train(q, k, v, beta, alpha=None, S0=None, chunk=CHUNK, *, o=None, S_out=None, workspace=None,
                        return_state=True):
    """delta_forward (alpha None) or gated_delta_forward that also leaves the
    backward pass's context in its workspace (a delta_backward workspace,
    allocated when None).  Returns (o, S_T, workspace); hand the workspace to
    delta_backward_after_forward with the same inputs."""
    code = _dtype_code(q)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    _need(k, "k", q.dtype, (B, H, T, dk), dev)
    _need(v, "v", q.dtype, (B, H, T, dv), dev)
    _need(beta, "beta", q.dtype, (B, H, T), dev)
    _need(q, "q", q.dtype, (B, H, T, dk), dev)
    if alpha is not None:
        _need(alpha, "alpha", torch.float32, (B, H, T), dev)
    if S0 is not None:
        _need(S0, "S0", torch.float32, (B, H, dk, dv), dev)
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=q.dtype, device=dev)
    _need(o, "o", q.dtype, (B, H, T, dv), dev)
    if return_state:
        if S_out is None:
            S_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
        _need(S_out, "S_out", torch.float32, (B, H, dk, dv), dev)
    ws, wsb = _workspace(delta_backward_workspace_bytes(B, H, T, dk, dv, chunk), dev, workspace)
    _check(lib().delta_forward_train(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(alpha), _ptr(S0), _ptr(o),
                                     _ptr(S_out), B, H, T, dk, dv, code, int(chunk), _ptr(ws), wsb, _stream(dev)))
    return o, S_out, ws


def delta_backward_after_forward(q, k, v, beta, dO, workspace, alpha=None, S0=None, dS_T=None, chunk=CHUNK, *,
                                 dq=None, dk=None, dv=None, return_state_grad=True):
    """delta_backward on the workspace a delta_forward_train call with the
    same inputs filled (its forward sweep is not run again; the workspace's
    context is consumed).  Returns what delta_backward returns."""
    if workspace is None:
        raise ValueError("delta_backward_after_forward needs the workspace of delta_forward_train")
    return _delta_backward("delta_backward_after_forward", q, k, v, beta, dO, alpha, S0, dS_T, chunk, dq, dk, dv,
                           return_state_grad, workspace)


def _delta_backward(entry, q, k, v, beta, dO, alpha, S0, dS_T, chunk, dq, dk, dv, return_state_grad, workspace):
    code = _dtype_code(q)
    B, H, T, dkk = q.shape
    dvv = v.shape[-1]
    dev = q.device
    _need(k, "k", q.dtype, (B, H, T, dkk), dev)
    _need(v, "v", q.dtype, (B, H, T, dvv), dev)
    _need(beta, "beta", q.dtype, (B, H, T), dev)
    _need(dO, "dO", q.dtype, (B, H, T, dvv), dev)
    if alpha is not None:
        _need(alpha, "alpha", torch.float32, (B, H, T), dev)
    for t, name in ((S0, "S0"), (dS_T, "dS_T")):
        if t is not None:
            _need(t, name, torch.float32, (B, H, dkk, dvv), dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _need(dq, "dq", q.dtype, (B, H, T, dkk), dev)
    _need(dk, "dk", q.dtype, (B, H, T, dkk), dev)
    _need(dv, "dv", q.dtype, (B, H, T, dvv), dev)
    dbeta = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    dalpha = torch.empty((B, H, T), dtype=torch.float32, device=dev) if alpha is not None else None
    dS0 = torch.empty((B, H, dkk, dvv), dtype=torch.float32, device=dev) if return_state_grad else None
    ws, wsb = _workspace(delta_backward_workspace_bytes(B, H, T, dkk, dvv, chunk), dev, workspace)
    _check(getattr(lib(), entry)(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(alpha), _ptr(S0), _ptr(dO), _ptr(dS_T),
                                 _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbeta), _ptr(dalpha), _ptr(dS0), B, H, T, dkk,
                                 dvv, code, int(chunk), _ptr(ws), wsb, _stream(dev)))
    return dq, dk, dv, dbeta, dalpha, dS0
