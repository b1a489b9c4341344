"""GPU parity tests of gated_delta_forward and gated_delta_decode_step (through
the C ABI): the delta rule with a forgetting gate applied before the
correction."""
import numpy as np
import pytest
import torch

import oracle
from tests.parity import TOL, assert_parity, to64
from weight_recurrent_memory_amd import binding as lin
from weight_recurrent_memory_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run(q, k, v, beta, alpha, S0=None):
    o, S = lin.gated_delta_forward(q, k, v, beta, alpha, S0)
    torch.cuda.synchronize()
    return o, S


def _check(q, k, v, beta, alpha, o, S, S0=None, heads=None):
    tol = TOL[q.dtype]
    B, H = q.shape[:2]
    flat = lambda t: None if t is None else t.reshape(B * H, *t.shape[2:])
    qf, kf, vf, bf, af, of, Sf, S0f = map(flat, (q, k, v, beta, alpha, o, S, S0))
    idx = list(range(B * H)) if heads is None else list(heads)
    sel = lambda t: None if t is None else t[idx][None]
    ro, rS = oracle.gated_delta_forward(sel(qf), sel(kf), sel(vf), sel(bf), sel(af), sel(S0f))
    e1 = assert_parity(sel(of), ro, tol, "o", rows=True)
    e2 = assert_parity(sel(Sf), rS, tol, "S_T")
    print(f"worst slice errors: o {e1:.2e}  S {e2:.2e}")


SHAPES = [
    # B, H, T, dk, dv, with initial state, gate rate
    (1, 1, 1, 128, 128, True, 1 / 16),
    (1, 2, 2, 64, 64, True, 1 / 16),
    (2, 1, 63, 128, 128, True, 1 / 4),
    (1, 1, 64, 64, 128, False, 1 / 16),
    (1, 3, 65, 128, 64, True, 1 / 16),
    (1, 1, 200, 128, 128, False, 1),
    (2, 2, 1000, 64, 64, True, 1 / 16),
    (1, 2, 3000, 128, 128, True, 1 / 64),
    (1, 1, 2500, 128, 64, False, 1 / 16),
    (1, 1, 2049, 64, 128, True, 1 / 4),
]


@pytest.mark.parametrize("B,H,T,dk,dv,init,rate", SHAPES)
def test_gated_delta_small_shapes(B, H, T, dk, dv, init, rate):
    print(f"gated_delta_forward B={B} H={H} T={T} dk={dk} dv={dv} init={init} rate={rate}", flush=True)
    q, k, v, beta = wl.delta_inputs(B, H, T, dk, dv, torch.bfloat16, seed=3000 + T, device=DEV)
    alpha = wl.gates((B, H, T), seed=T, device=DEV, rate=rate)
    S0 = None
    if init:
        S0, _ = wl.decode_state(B, H, dk, dv, seed=79, device=DEV, std=0.5)
    o, S = _run(q, k, v, beta, alpha, S0)
    _check(q, k, v, beta, alpha, o, S, S0)


def test_gated_delta_config_all_heads():
    w = wl.GATED_DELTA_BF16_PREFILL
    print(f"gated_delta_forward {w.name}", flush=True)
    q, k, v, beta, alpha = wl.make(w, DEV)
    o, S = _run(q, k, v, beta, alpha)
    _check(q, k, v, beta, alpha, o, S)


def test_gated_delta_alpha_one_is_delta_forward():
    """alpha = 1: every gate factor is exactly 1.0, so the result is the
    ungated kernel's, bit for bit."""
    q, k, v, beta = wl.delta_inputs(1, 4, 2500, 128, 128, torch.bfloat16, seed=31, device=DEV)
    S0, _ = wl.decode_state(1, 4, 128, 128, seed=32, device=DEV, std=0.3)
    ones = torch.ones((1, 4, 2500), dtype=torch.float32, device=DEV)
    og, Sg = _run(q, k, v, beta, ones, S0)
    od, Sd = lin.delta_forward(q, k, v, beta, S0)
    torch.cuda.synchronize()
    assert torch.equal(og, od) and torch.equal(Sg, Sd)


def test_gated_delta_zero_beta_is_pure_decay():
    """beta = 0: no writes, so S_T = prod(alpha) S_0 and o_t = gamma_t S_0^T q_t."""
    B, H, T, d = 1, 2, 700, 128
    q, k, v, _ = wl.delta_inputs(B, H, T, d, d, torch.bfloat16, seed=33, device=DEV)
    beta = torch.zeros((B, H, T), dtype=torch.bfloat16, device=DEV)
    alpha = wl.gates((B, H, T), seed=34, device=DEV, rate=1 / 64)
    S0, _ = wl.decode_state(B, H, d, d, seed=35, device=DEV, std=0.5)
    o, S = _run(q, k, v, beta, alpha, S0)
    _check(q, k, v, beta, alpha, o, S, S0)


def test_gated_delta_resets_and_tiny_gates():
    """alpha = 0 tokens (an effective reset) and gates down to 1e-6 inside a
    chunk, against the oracle's exact alpha."""
    B, H, T, d = 1, 2, 1000, 128
    q, k, v, beta = wl.delta_inputs(B, H, T, d, d, torch.bfloat16, seed=36, device=DEV)
    alpha = wl.gates((B, H, T), seed=37, device=DEV)
    alpha[:, :, 100] = 0.0
    alpha[:, 1, 130:140] = 1e-6
    alpha[:, 0, 640] = 0.0
    S0, _ = wl.decode_state(B, H, d, d, seed=38, device=DEV, std=0.5)
    o, S = _run(q, k, v, beta, alpha, S0)
    _check(q, k, v, beta, alpha, o, S, S0)


def test_gated_delta_causality_bitwise():
    q, k, v, beta = wl.delta_inputs(1, 2, 300, 128, 128, torch.bfloat16, seed=39, device=DEV)
    alpha = wl.gates((1, 2, 300), seed=40, device=DEV, rate=1 / 4)
    S0, _ = wl.decode_state(1, 2, 128, 128, seed=41, device=DEV, std=0.5)
    o, _ = _run(q, k, v, beta, alpha, S0)
    for s in (0, 63, 64, 100, 299):
        pert = alpha.clone()
        pert[:, :, s] *= 0.5
        o2, _ = _run(q, k, v, beta, pert, S0)
        assert torch.equal(o2[:, :, :s], o[:, :, :s]), s
        assert not torch.equal(o2[:, :, s:], o[:, :, s:]), s


def test_gated_delta_deterministic_and_resume():
    q, k, v, beta = wl.delta_inputs(1, 4, 2500, 128, 128, torch.bfloat16, seed=42, device=DEV)
    alpha = wl.gates((1, 4, 2500), seed=43, device=DEV, rate=1 / 64)
    a = _run(q, k, v, beta, alpha)
    b = _run(q, k, v, beta, alpha)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    T1 = 1000
    cut = lambda x, s: x[:, :, s].contiguous()
    h1, h2 = slice(0, T1), slice(T1, None)
    oa, Sa = _run(cut(q, h1), cut(k, h1), cut(v, h1), cut(beta, h1), cut(alpha, h1))
    ob, Sb = _run(cut(q, h2), cut(k, h2), cut(v, h2), cut(beta, h2), cut(alpha, h2), Sa)
    tol = TOL[torch.bfloat16]
    assert_parity(torch.cat([oa, ob], 2), to64(a[0]), tol, "o", rows=True)
    assert_parity(Sb, to64(a[1]), tol, "S")


# ------------------------------------------------------------------ decode

@pytest.mark.parametrize("N,H,dk,dv,dtype", [
    (1, 1, 64, 64, torch.bfloat16), (3, 5, 64, 128, torch.bfloat16), (2, 2, 128, 64, torch.float32),
    (7, 3, 128, 128, torch.bfloat16), (4, 4, 128, 128, torch.float32), (5, 1, 64, 64, torch.float32)])
def test_gated_delta_decode_step_shapes(N, H, dk, dv, dtype):
    print(f"gated_delta_decode_step N={N} H={H} dk={dk} dv={dv} {dtype}", flush=True)
    S, _ = wl.decode_state(N, H, dk, dv, seed=15, device=DEV, std=0.3)
    q, k, v, beta = (t[0] for t in wl.delta_decode_tokens(1, N, H, dk, dv, dtype, seed=16, device=DEV))
    alpha = wl.gates((N, H), seed=17, device=DEV, rate=1 / 2)
    S_ref = to64(S)
    o = lin.gated_delta_decode_step(q, k, v, beta, alpha, S)
    torch.cuda.synchronize()
    ro, rS = oracle.gated_delta_decode_step(q, k, v, beta, alpha, S_ref)
    assert_parity(o, ro, TOL[dtype], "o", rows=True)
    assert_parity(S, rS, 1e-5, "S")  # fp32 state: a dk-term dot product, then two products and a sum


def test_gated_delta_decode_zero_alpha_resets():
    """alpha = 0 wipes the state exactly: S_new = beta k v^T and o = beta (k.q) v."""
    N, H, d = 3, 2, 128
    S, _ = wl.decode_state(N, H, d, d, seed=18, device=DEV, std=0.3)
    q, k, v, beta = (t[0] for t in wl.delta_decode_tokens(1, N, H, d, d, torch.float32, seed=19, device=DEV))
    alpha = torch.zeros((N, H), dtype=torch.float32, device=DEV)
    o = lin.gated_delta_decode_step(q, k, v, beta, alpha, S)
    torch.cuda.synchronize()
    ro, rS = oracle.gated_delta_decode_step(q, k, v, beta, alpha, np.zeros((N, H, d, d)))
    assert_parity(S, rS, 1e-6, "S")
    assert_parity(o, ro, 1e-5, "o", rows=True)


def test_gated_delta_decode_config_chain_sampled_states():
    """The 256 x 32 x d128 states for 200 gated steps on the GPU; the oracle
    follows 8 sampled (sequence, head) states through every step."""
    w = wl.GATED_DELTA_DECODE_BF16
    steps = 200
    print(f"gated_delta_decode_step {w.name} ({steps} steps)", flush=True)
    S, Q, K, V, Bt, At = wl.make(w, DEV)
    picks = [(0, 0), (17, 3), (100, 31), (128, 16), (200, 7), (255, 31), (64, 0), (3, 29)]
    n_idx = torch.tensor([p[0] for p in picks], device=DEV)
    h_idx = torch.tensor([p[1] for p in picks], device=DEV)
    S_ref = to64(S[n_idx, h_idx])[None]
    outs = torch.empty((steps, len(picks), w.dv), dtype=w.dtype, device=DEV)
    o = torch.empty((w.B, w.H, w.dv), dtype=w.dtype, device=DEV)
    for t in range(steps):
        lin.gated_delta_decode_step(Q[t], K[t], V[t], Bt[t], At[t], S, o=o)
        outs[t] = o[n_idx, h_idx]
    torch.cuda.synchronize()
    qs, ks, vs, bs, als = (to64(X[:steps, n_idx, h_idx]) for X in (Q, K, V, Bt, At))
    tol = TOL[w.dtype]
    worst = 0.0
    for t in range(steps):
        ro, S_ref = oracle.gated_delta_decode_step(qs[t][None], ks[t][None], vs[t][None], bs[t][None],
                                                   als[t][None], S_ref)
        worst = max(worst, assert_parity(outs[t][None], ro, tol, f"o step {t}", axes=(2,), rows=True))
    assert_parity(S[n_idx, h_idx][None], S_ref, tol, "S final")
    print(f"worst per-step slice error of o: {worst:.2e}")


def test_gated_delta_decode_chain_equals_prefill():
    N, H, d, steps = 2, 3, 128, 256
    S, _ = wl.decode_state(N, H, d, d, seed=23, device=DEV, std=0.1)
    Q, K, V, Bt = wl.delta_decode_tokens(steps, N, H, d, d, torch.bfloat16, seed=24, device=DEV)
    At = wl.gates((steps, N, H), seed=25, device=DEV, rate=1 / 4)
    S0 = S.clone()
    outs = torch.stack([lin.gated_delta_decode_step(Q[t], K[t], V[t], Bt[t], At[t], S) for t in range(steps)], 2)
    seq = lambda X: X.permute(1, 2, 0, 3).contiguous()
    seq3 = lambda X: X.permute(1, 2, 0).contiguous()
    o, Sf = lin.gated_delta_forward(seq(Q), seq(K), seq(V), seq3(Bt), seq3(At), S0)
    torch.cuda.synchronize()
    tol = TOL[torch.bfloat16]
    assert_parity(outs, to64(o), tol, "o", rows=True)
    assert_parity(S, to64(Sf), tol, "S")
