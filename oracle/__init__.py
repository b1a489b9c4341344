"""TEST INFRASTRUCTURE ONLY: the fp64 CPU oracle.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports it, and it imports nothing from them.

The arithmetic lives in ``linattn_oracle.c`` (plain C, double precision,
sequential token loops, OpenMP only across independent heads).  This module
builds it with gcc when ``liboracle.so`` is missing and marshals arrays.

Functions and what pins them (the pins are in ``tests/test_oracle_pins.py``):

``la_forward``   -- normalized causal ELU+1 linear attention, write-then-read.
    Pinned by the seed-7 run printed on the LinearMem page (§04), the
    quadratic masked form on small inputs (brute force), the T = 1 and
    identical-key closed forms, the LA-SSM page's 4-token additive example
    and the memory-capacity page's two-entry example (identity feature map,
    no normaliser), causality and resume invariants.
``delta_forward`` -- delta-rule fast weight.  Pinned by the LA-SSM page's
    4-token delta example (every intermediate state), the LinearMem memory
    experiment (same key, half beta, crosstalk), the exact-overwrite
    invariant, the EMA closed form, the dense triangular-solve form via
    LAPACK, the orthonormal-key reduction to the additive memory and the
    Kaczmarz limit equal to the memory-capacity page's least-squares W*.
    The per-token query read o_t = S_t^T q_t is a reading taken here (the
    pages print no such sequence): parity of that read is pinned only by the
    dense form and the orthonormal-key reduction.
``la_backward`` -- the gradients of la_forward for a linear loss
    sum dO . o + <dS_T, S_T> + <dz_T, z_T> (reverse-mode differentiation of
    the same recurrence, per-token scalars kept, states recomputed).  Pinned
    by central finite differences of la_forward for every input element, the
    adjoint of the additive memory's linear map v -> o (brute force), and the
    single-token closed forms of dv, dS0 and dz0.
``delta_backward`` -- the gradients of the (gated) delta rule for a linear
    loss sum dO . o + <dS_T, S_T>, by reverse-mode differentiation of the
    token recurrence with states recomputed from 64-token checkpoints.
    Pinned by central finite differences of the forward oracle for every
    element of q, k, v, beta, alpha and S0, and by the orthonormal-key case,
    where the rule is the additive memory and the value gradient is the
    additive memory's adjoint.
``la_decode_step`` -- one in-place step; pinned by equality with one token of
    ``la_forward`` continued from the same state.
``gated_delta_forward`` / ``gated_delta_decode_step`` -- the delta rule with a
    forgetting gate applied before the correction (LinearMem §03, the
    Gated DeltaNet rule).  Pinned by the LinearMem gate reads (identity
    state, key (1, 0) written with beta = 1: the orthogonal key reads [0, 0.8]
    with alpha = 0.8, §06, and [0, 1] with alpha = 1, §09), alpha = 1 equal to the ungated functions bit for
    bit, beta = 0 reducing to pure decay (S_T = prod(alpha) S_0), a dense
    form with decay products solved by LAPACK, the exact overwrite after the
    decay, the step chain equal to the sequence form, and the order check
    (decaying after the correction gives a different, wrong state).
``ssd_forward`` / ``ssd_decode_step`` -- scalar-decay memory, the Mamba-2 /
    SSD form (LA-SSM §3): S_t = alpha_t S_{t-1} + k_t v_t^T, o_t = S_t^T q_t.
    Pinned by the Recurrence page's explicit mixing matrix of the selective
    scan (d_k = d_v = 1: M[j][i] = c_j b_i prod_{i<s<=j} a_s), a brute-force
    sum of decayed outer products at larger sizes, alpha = 1 equal bit for
    bit to the additive memory (identity map, no normaliser), the page's
    chunked scan (state handed across chunk boundaries) equal to one pass,
    the LinearMem decay read ([0, 0.8] at alpha = 0.8 on an identity state
    for an orthogonal key, §06), and the step chain equal to the sequence
    form.
``delta_forward_ex`` / ``delta_decode_step_ex`` -- either delta rule with
    the input transforms of a serving stack (LinearMem §05 and §08: q/k L2
    normalisation and beta = sigmoid(logit) in the kernel) and the
    Recurrence page's read-then-write prediction k_t^T S~_{t-1} as an extra
    output.  Pinned by closed forms of the transforms (a 3-4-5 row, unit
    norms, a zero row, sigmoid(0) = 1/2 and its symmetry), the LA-SSM
    four-token delta example's predictions read off its printed states, the
    exact recall of a basis key's stored value, pred + correction = v, and
    the flags reducing to the plain functions on pre-transformed inputs.
``delta_decode_step`` -- one in-place delta-rule step.  Pinned by the LA-SSM
    page's 4-token delta example replayed one step at a time (every
    intermediate state and the final read of k_1), the bit-exact overwrite
    with basis keys and beta = 1, beta = 0 leaving the state unchanged, and
    a step chain equal to ``delta_forward`` over the same tokens.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "linattn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

PHI_ELU1 = 0
PHI_IDENTITY = 1


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
           "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build()
            lib = ctypes.CDLL(_LIB_PATH)
            dp = ctypes.POINTER(ctypes.c_double)
            i = ctypes.c_int
            lib.la_ref_forward.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp,
                                           i, i, i, i, i, ctypes.c_double, i, i]
            lib.la_ref_forward.restype = None
            lib.delta_ref_forward.argtypes = [dp, dp, dp, dp, dp, dp, dp,
                                              i, i, i, i, i]
            lib.delta_ref_forward.restype = None
            lib.la_ref_decode_step.argtypes = [dp, dp, dp, dp, dp, dp,
                                               i, i, i, i, ctypes.c_double]
            lib.la_ref_decode_step.restype = None
            lib.delta_ref_decode_step.argtypes = [dp, dp, dp, dp, dp, dp, i, i, i, i]
            lib.delta_ref_decode_step.restype = None
            lib.gated_delta_ref_forward.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, i, i, i, i, i]
            lib.gated_delta_ref_forward.restype = None
            lib.gated_delta_ref_decode_step.argtypes = [dp, dp, dp, dp, dp, dp, dp, i, i, i, i]
            lib.gated_delta_ref_decode_step.restype = None
            lib.ssd_ref_forward.argtypes = [dp, dp, dp, dp, dp, dp, dp, i, i, i, i, i]
            lib.ssd_ref_forward.restype = None
            lib.ssd_ref_decode_step.argtypes = [dp, dp, dp, dp, dp, dp, i, i, i, i]
            lib.ssd_ref_decode_step.restype = None
            lib.delta_ref_forward_ex.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, dp, i, i, i, i, i]
            lib.delta_ref_forward_ex.restype = None
            lib.delta_ref_decode_step_ex.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, i, i, i, i]
            lib.delta_ref_decode_step_ex.restype = None
            lib.oracle_l2_normalize_rows.argtypes = [dp, dp, ctypes.c_long, i]
            lib.oracle_l2_normalize_rows.restype = None
            lib.oracle_sigmoid.argtypes = [dp, dp, ctypes.c_long]
            lib.oracle_sigmoid.restype = None
            lib.la_ref_backward.argtypes = [dp] * 13 + [i, i, i, i, i, ctypes.c_double, i, i]
            lib.la_ref_backward.restype = None
            lib.delta_ref_backward.argtypes = [dp] * 14 + [i, i, i, i, i]
            lib.delta_ref_backward.restype = None
            lib.oracle_phi.argtypes = [dp, dp, ctypes.c_long]
            lib.oracle_phi.restype = None
            lib.oracle_num_threads.argtypes = []
            lib.oracle_num_threads.restype = ctypes.c_int
            _lib = lib
    return _lib


def _f64(x):
    """Exact upcast to a contiguous float64 array (torch or numpy input)."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: bf16/fp32 -> fp64 is exact
        x = x.detach().to("cpu").double().contiguous().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def phi(x):
    x = _f64(x)
    y = np.empty_like(x)
    _load().oracle_phi(_ptr(x), _ptr(y), x.size)
    return y


def la_forward(q, k, v, S0=None, z0=None, eps=1e-6,
               feature=PHI_ELU1, normalize=True):
    """q, k: [B,H,T,dk]; v: [B,H,T,dv] -> (o [B,H,T,dv], S [B,H,dk,dv], z [B,H,dk])."""
    q, k, v, S0, z0 = map(_f64, (q, k, v, S0, z0))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and v.shape[:3] == (B, H, T)
    if S0 is not None:
        assert S0.shape == (B, H, dk, dv)
    if z0 is not None:
        assert z0.shape == (B, H, dk)
    o = np.empty((B, H, T, dv))
    S = np.empty((B, H, dk, dv))
    z = np.empty((B, H, dk))
    _load().la_ref_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(S0), _ptr(z0),
                           _ptr(o), _ptr(S), _ptr(z), B, H, T, dk, dv,
                           float(eps), int(feature), 1 if normalize else 0)
    return o, S, z


def delta_forward(q, k, v, beta, S0=None):
    """q, k: [B,H,T,dk]; v: [B,H,T,dv]; beta: [B,H,T] -> (o [B,H,T,dv], S [B,H,dk,dv])."""
    q, k, v, beta, S0 = map(_f64, (q, k, v, beta, S0))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and v.shape[:3] == (B, H, T) and beta.shape == (B, H, T)
    if S0 is not None:
        assert S0.shape == (B, H, dk, dv)
    o = np.empty((B, H, T, dv))
    S = np.empty((B, H, dk, dv))
    _load().delta_ref_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(S0),
                              _ptr(o), _ptr(S), B, H, T, dk, dv)
    return o, S


def la_decode_step(q, k, v, S, z, eps=1e-6):
    """One step on copies of (S, z).  q, k: [N,H,dk]; v: [N,H,dv];
    S: [N,H,dk,dv]; z: [N,H,dk] -> (o [N,H,dv], S_new, z_new)."""
    q, k, v = map(_f64, (q, k, v))
    S = _f64(S).copy()
    z = _f64(z).copy()
    N, H, dk = q.shape
    dv = v.shape[-1]
    assert S.shape == (N, H, dk, dv) and z.shape == (N, H, dk)
    o = np.empty((N, H, dv))
    _load().la_ref_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(S), _ptr(z),
                               _ptr(o), N, H, dk, dv, float(eps))
    return o, S, z


def delta_decode_step(q, k, v, beta, S):
    """One delta-rule step on a copy of S.  q, k: [N,H,dk]; v: [N,H,dv];
    beta: [N,H]; S: [N,H,dk,dv] -> (o [N,H,dv], S_new)."""
    q, k, v, beta = map(_f64, (q, k, v, beta))
    S = _f64(S).copy()
    N, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and v.shape == (N, H, dv) and beta.shape == (N, H)
    assert S.shape == (N, H, dk, dv)
    o = np.empty((N, H, dv))
    _load().delta_ref_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(S), _ptr(o),
                                  N, H, dk, dv)
    return o, S


def gated_delta_forward(q, k, v, beta, alpha, S0=None):
    """The gated delta rule.  q, k: [B,H,T,dk]; v: [B,H,T,dv]; beta, alpha:
    [B,H,T] -> (o [B,H,T,dv], S [B,H,dk,dv])."""
    q, k, v, beta, alpha, S0 = map(_f64, (q, k, v, beta, alpha, S0))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and v.shape[:3] == (B, H, T)
    assert beta.shape == (B, H, T) and alpha.shape == (B, H, T)
    if S0 is not None:
        assert S0.shape == (B, H, dk, dv)
    o = np.empty((B, H, T, dv))
    S = np.empty((B, H, dk, dv))
    _load().gated_delta_ref_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(alpha), _ptr(S0),
                                    _ptr(o), _ptr(S), B, H, T, dk, dv)
    return o, S


def gated_delta_decode_step(q, k, v, beta, alpha, S):
    """One gated delta step on a copy of S.  q, k: [N,H,dk]; v: [N,H,dv];
    beta, alpha: [N,H]; S: [N,H,dk,dv] -> (o [N,H,dv], S_new)."""
    q, k, v, beta, alpha = map(_f64, (q, k, v, beta, alpha))
    S = _f64(S).copy()
    N, H, dk = q.shape
    dv = v.shape[-1]
    assert beta.shape == (N, H) and alpha.shape == (N, H) and S.shape == (N, H, dk, dv)
    o = np.empty((N, H, dv))
    _load().gated_delta_ref_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(alpha), _ptr(S),
                                        _ptr(o), N, H, dk, dv)
    return o, S


def ssd_forward(q, k, v, alpha, S0=None):
    """Scalar-decay memory (Mamba-2 / SSD form).  q, k: [B,H,T,dk]; v: [B,H,T,dv];
    alpha: [B,H,T] -> (o [B,H,T,dv], S [B,H,dk,dv])."""
    q, k, v, alpha, S0 = map(_f64, (q, k, v, alpha, S0))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and v.shape[:3] == (B, H, T) and alpha.shape == (B, H, T)
    if S0 is not None:
        assert S0.shape == (B, H, dk, dv)
    o = np.empty((B, H, T, dv))
    S = np.empty((B, H, dk, dv))
    _load().ssd_ref_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(S0), _ptr(o), _ptr(S),
                            B, H, T, dk, dv)
    return o, S


def ssd_decode_step(q, k, v, alpha, S):
    """One scalar-decay step on a copy of S.  q, k: [N,H,dk]; v: [N,H,dv];
    alpha: [N,H]; S: [N,H,dk,dv] -> (o [N,H,dv], S_new)."""
    q, k, v, alpha = map(_f64, (q, k, v, alpha))
    S = _f64(S).copy()
    N, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and v.shape == (N, H, dv) and alpha.shape == (N, H)
    assert S.shape == (N, H, dk, dv)
    o = np.empty((N, H, dv))
    _load().ssd_ref_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(S), _ptr(o), N, H, dk, dv)
    return o, S


def l2_normalize_rows(x):
    """x / ||x|| over the last axis (a zero row stays zero)."""
    x = _f64(x)
    y = np.empty_like(x)
    _load().oracle_l2_normalize_rows(_ptr(x), _ptr(y), x.size // x.shape[-1], x.shape[-1])
    return y


def sigmoid(x):
    x = _f64(x)
    y = np.empty_like(x)
    _load().oracle_sigmoid(_ptr(x), _ptr(y), x.size)
    return y


def _pre(q, k, beta, normalize_qk, beta_logits):
    q, k, beta = map(_f64, (q, k, beta))
    if normalize_qk:
        q, k = l2_normalize_rows(q), l2_normalize_rows(k)
    if beta_logits:
        beta = sigmoid(beta)
    return q, k, beta


def delta_forward_ex(q, k, v, beta, alpha=None, S0=None, normalize_qk=False, beta_logits=False):
    """The delta rule, gated when alpha is given, after the optional input
    transforms; returns (o, S_T, pred) with pred the read-then-write
    predictions [B,H,T,dv]."""
    q, k, beta = _pre(q, k, beta, normalize_qk, beta_logits)
    v, alpha, S0 = map(_f64, (v, alpha, S0))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and v.shape[:3] == (B, H, T) and beta.shape == (B, H, T)
    if alpha is not None:
        assert alpha.shape == (B, H, T)
    if S0 is not None:
        assert S0.shape == (B, H, dk, dv)
    o = np.empty((B, H, T, dv))
    S = np.empty((B, H, dk, dv))
    pred = np.empty((B, H, T, dv))
    _load().delta_ref_forward_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(alpha), _ptr(S0), _ptr(o), _ptr(S),
                                 _ptr(pred), B, H, T, dk, dv)
    return o, S, pred


def delta_decode_step_ex(q, k, v, beta, S, alpha=None, normalize_qk=False, beta_logits=False):
    """One delta step (gated when alpha is given) on a copy of S after the
    optional input transforms; returns (o, S_new, pred)."""
    q, k, beta = _pre(q, k, beta, normalize_qk, beta_logits)
    v, alpha = map(_f64, (v, alpha))
    S = _f64(S).copy()
    N, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and v.shape == (N, H, dv) and beta.shape == (N, H) and S.shape == (N, H, dk, dv)
    o = np.empty((N, H, dv))
    pred = np.empty((N, H, dv))
    _load().delta_ref_decode_step_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(alpha), _ptr(S), _ptr(o), _ptr(pred),
                                     N, H, dk, dv)
    return o, S, pred


def la_backward(q, k, v, dO, S0=None, z0=None, dS_T=None, dz_T=None, eps=1e-6, feature=PHI_ELU1, normalize=True):
    """Gradients of L = sum dO . o + <dS_T, S_T> + <dz_T, z_T> for la_forward:
    returns (dq, dk, dv, dS0, dz0)."""
    q, k, v, dO, S0, z0, dS_T, dz_T = map(_f64, (q, k, v, dO, S0, z0, dS_T, dz_T))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and v.shape == (B, H, T, dv) and dO.shape == v.shape
    dq, dkk, dvv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    dS0, dz0 = np.empty((B, H, dk, dv)), np.empty((B, H, dk))
    _load().la_ref_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(S0), _ptr(z0), _ptr(dO), _ptr(dS_T), _ptr(dz_T),
                            _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(dS0), _ptr(dz0), B, H, T, dk, dv, float(eps),
                            int(feature), 1 if normalize else 0)
    return dq, dkk, dvv, dS0, dz0


def delta_backward(q, k, v, beta, dO, alpha=None, S0=None, dS_T=None):
    """Gradients of L = sum dO . o + <dS_T, S_T> for the delta rule (gated
    when alpha is given): returns (dq, dk, dv, dbeta, dalpha or None, dS0)."""
    q, k, v, beta, dO, alpha, S0, dS_T = map(_f64, (q, k, v, beta, dO, alpha, S0, dS_T))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and v.shape == (B, H, T, dv) and dO.shape == v.shape and beta.shape == (B, H, T)
    dq, dkk, dvv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    dbeta = np.empty((B, H, T))
    dalpha = np.empty((B, H, T)) if alpha is not None else None
    dS0 = np.empty((B, H, dk, dv))
    _load().delta_ref_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(alpha), _ptr(S0), _ptr(dO), _ptr(dS_T),
                               _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(dbeta), _ptr(dalpha), _ptr(dS0), B, H, T, dk, dv)
    return dq, dkk, dvv, dbeta, dalpha, dS0
