"""Independent fp64 evaluation forms used to pin the oracle (test helpers).

None of these is the oracle's sequential token loop; each reaches the same
function by a different route, so a dropped term, a swapped order or a
transposed operand in the oracle shows up as a mismatch.

* ``la_quadratic`` -- the ratio-of-sums definition of o_t taken term by
  term ("AIGC 基本功｜线性、循环与记忆架构-LinearMem", §03): for every query
  t, a loop over the history i <= t adds w_ti v_i to the numerator and w_ti
  to the denominator, w_ti = phi(q_t) . phi(k_i), then divides.  No matrix of
  all pairs is formed and no mask is applied.
* ``delta_dense`` -- the delta rule solved in one shot.  Unrolling
  S_{t-1} = S_0 + sum_{i<t} beta_i k_i u_i^T in u_t = v_t - S_{t-1}^T k_t gives
  the unit lower-triangular system (I + A) U = V - K S_0 with
  A[t, i] = beta_i (k_t . k_i) for i < t; it is solved with LAPACK
  (numpy.linalg.solve).  Then O = Q S_0 + tril(Q K^T) diag(beta) U and
  S_T = S_0 + K^T diag(beta) U.  (Same page, §03 "从累加改成纠错".)
* ``la_chunked`` / ``delta_chunked`` -- the chunked forms with state passing
  between chunks (only the final state crosses a chunk boundary:
  "手撕：递推与记忆模型", "Chunked scan"); these are the forms the HIP
  kernels evaluate, checked here in fp64 for every chunk size.
"""
import numpy as np


def phi(x):
    """ELU+1 written as ELU(x) + 1, with ELU(x) = x (x > 0), e^x - 1 (x <= 0)
    through expm1: the same function as the oracle's exp form, another
    rounding path (they differ by at most an ulp near 0-)."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0, x, np.expm1(np.minimum(x, 0.0))) + 1.0


def la_quadratic(q, k, v, S0=None, z0=None, eps=1e-6):
    """Single head: q, k [T, dk]; v [T, dv].  For each t,
    o_t = (phi(q_t)^T S0 + sum_{i<=t} w_ti v_i) / (phi(q_t)^T z0 + sum_{i<=t} w_ti + eps)
    with w_ti = phi(q_t) . phi(k_i), accumulated one history term at a time."""
    T, dv = q.shape[0], v.shape[1]
    fk = [phi(k[i]) for i in range(T)]
    out = np.empty((T, dv))
    for t in range(T):
        fq = phi(q[t])
        num = np.zeros(dv) if S0 is None else fq @ S0
        den = eps if z0 is None else eps + float(fq @ z0)
        for i in range(t + 1):
            w = float(np.dot(fq, fk[i]))
            num = num + w * v[i]
            den += w
        out[t] = num / den
    return out


def delta_dense(q, k, v, beta, S0=None):
    T, dk = k.shape
    dv = v.shape[1]
    S0 = np.zeros((dk, dv)) if S0 is None else S0
    A = np.tril(k @ k.T, -1) * beta[None, :]
    U = np.linalg.solve(np.eye(T) + A, v - k @ S0)
    O = q @ S0 + (np.tril(q @ k.T) * beta[None, :]) @ U
    S = S0 + k.T @ (beta[:, None] * U)
    return O, S


def gated_delta_dense(q, k, v, beta, alpha, S0=None):
    """The gated delta rule over a whole sequence as one linear system.
    With g_t = alpha_1 ... alpha_t, unrolling decay-then-correct gives
    (I + A) U = V - diag(g) K S0 with A[t][i] = (g_t / g_i) beta_i k_t . k_i
    (i < t); then o_t = g_t S0^T q_t + sum_{i<=t} (g_t / g_i) beta_i (k_i . q_t) u_i
    and S_T = g_T S0 + sum_i (g_T / g_i) beta_i k_i u_i^T."""
    T, dk = k.shape
    dv = v.shape[1]
    S0 = np.zeros((dk, dv)) if S0 is None else S0
    g = np.cumprod(alpha)
    ratio = g[:, None] / g[None, :]                       # g_t / g_i
    A = np.tril(ratio * (k @ k.T), -1) * beta[None, :]
    U = np.linalg.solve(np.eye(T) + A, v - g[:, None] * (k @ S0))
    O = g[:, None] * (q @ S0) + (np.tril(ratio * (q @ k.T)) * beta[None, :]) @ U
    S = g[-1] * S0 + k.T @ ((g[-1] / g * beta)[:, None] * U)
    return O, S


def la_chunked(q, k, v, C, S0=None, z0=None, eps=1e-6):
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else S0.copy()
    z = np.zeros(dk) if z0 is None else z0.copy()
    out = np.empty((T, dv))
    for s in range(0, T, C):
        e = min(s + C, T)
        fq, fk, vc = phi(q[s:e]), phi(k[s:e]), v[s:e]
        P = np.tril(fq @ fk.T)
        num = P @ vc + fq @ S
        den = P.sum(axis=1) + fq @ z + eps
        out[s:e] = num / den[:, None]
        S = S + fk.T @ vc
        z = z + fk.sum(axis=0)
    return out, S, z


def delta_chunked(q, k, v, beta, C, S0=None):
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else S0.copy()
    out = np.empty((T, dv))
    for s in range(0, T, C):
        e = min(s + C, T)
        kc, qc, vc, bc = k[s:e], q[s:e], v[s:e], beta[s:e]
        n = e - s
        A = np.tril(kc @ kc.T, -1) * bc[None, :]
        # (I + A)^{-1} by forward substitution, written out
        Tm = np.eye(n)
        for r in range(n):
            for c in range(r):
                Tm[r, c] = -A[r, c:r] @ Tm[c:r, c]
        W = Tm @ kc
        Uv = Tm @ vc
        U = Uv - W @ S
        out[s:e] = qc @ S + (np.tril(qc @ kc.T) * bc[None, :]) @ U
        S = S + kc.T @ (bc[:, None] * U)
    return out, S
