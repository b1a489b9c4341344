"""GPU parity tests of ssd_forward and ssd_decode_step (through the C ABI):
the scalar-decay memory S_t = alpha_t S_{t-1} + k_t v_t^T, o_t = S_t^T q_t."""
import numpy as np
import pytest
import torch

import oracle
from tests.parity import TOL, assert_parity, to64
from weight_recurrent_memory_amd import binding as lin
from weight_recurrent_memory_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run(q, k, v, alpha, S0=None):
    o, S = lin.ssd_forward(q, k, v, alpha, S0)
    torch.cuda.synchronize()
    return o, S


def _check(q, k, v, alpha, o, S, S0=None, heads=None):
    tol = TOL[q.dtype]
    B, H = q.shape[:2]
    flat = lambda t: None if t is None else t.reshape(B * H, *t.shape[2:])
    qf, kf, vf, af, of, Sf, S0f = map(flat, (q, k, v, alpha, o, S, S0))
    idx = list(range(B * H)) if heads is None else list(heads)
    sel = lambda t: None if t is None else t[idx][None]
    ro, rS = oracle.ssd_forward(sel(qf), sel(kf), sel(vf), sel(af), sel(S0f))
    e1 = assert_parity(sel(of), ro, tol, "o", rows=True)
    e2 = assert_parity(sel(Sf), rS, tol, "S_T")
    print(f"worst slice errors: o {e1:.2e}  S {e2:.2e}")


SHAPES = [
    # B, H, T, dk, dv, with initial state, gate rate
    (1, 1, 1, 64, 64, True, 1 / 16),
    (1, 2, 2, 128, 128, True, 1 / 16),
    (2, 1, 63, 64, 128, True, 1 / 4),
    (1, 1, 64, 128, 64, False, 1 / 16),
    (1, 3, 65, 64, 64, True, 1 / 16),
    (1, 1, 200, 128, 128, False, 1),
    (2, 2, 1000, 64, 64, True, 1 / 16),
    (1, 2, 3000, 128, 128, True, 1 / 64),
    (1, 1, 2500, 128, 64, False, 1 / 16),
    (1, 1, 4100, 64, 128, True, 1 / 4),
]


@pytest.mark.parametrize("B,H,T,dk,dv,init,rate", SHAPES)
def test_ssd_small_shapes(B, H, T, dk, dv, init, rate):
    print(f"ssd_forward B={B} H={H} T={T} dk={dk} dv={dv} init={init} rate={rate}", flush=True)
    q, k, v = wl.la_inputs(B, H, T, dk, dv, torch.bfloat16, seed=4000 + T, device=DEV)
    alpha = wl.gates((B, H, T), seed=T + 1, device=DEV, rate=rate)
    S0 = None
    if init:
        S0, _ = wl.decode_state(B, H, dk, dv, seed=80, device=DEV, std=0.5)
    o, S = _run(q, k, v, alpha, S0)
    _check(q, k, v, alpha, o, S, S0)


def test_ssd_config_all_heads():
    w = wl.SSD_BF16_PREFILL
    print(f"ssd_forward {w.name}", flush=True)
    q, k, v, alpha = wl.make(w, DEV)
    o, S = _run(q, k, v, alpha)
    _check(q, k, v, alpha, o, S)


def test_ssd_d128_long_all_heads():
    B, H, T, d = 2, 16, 16384, 128
    print(f"ssd_forward B={B} H={H} T={T} d={d}", flush=True)
    q, k, v = wl.la_inputs(B, H, T, d, d, torch.bfloat16, seed=41, device=DEV)
    alpha = wl.gates((B, H, T), seed=42, device=DEV, rate=1 / 64)
    o, S = _run(q, k, v, alpha)
    _check(q, k, v, alpha, o, S)


def test_ssd_resets_and_tiny_gates():
    B, H, T, d = 1, 2, 1000, 64
    q, k, v = wl.la_inputs(B, H, T, d, d, torch.bfloat16, seed=43, device=DEV)
    alpha = wl.gates((B, H, T), seed=44, device=DEV)
    alpha[:, :, 100] = 0.0
    alpha[:, 1, 130:140] = 1e-6
    alpha[:, 0, 640] = 0.0
    S0, _ = wl.decode_state(B, H, d, d, seed=45, device=DEV, std=0.5)
    o, S = _run(q, k, v, alpha, S0)
    _check(q, k, v, alpha, o, S, S0)


def test_ssd_causality_bitwise():
    q, k, v = wl.la_inputs(1, 2, 300, 64, 64, torch.bfloat16, seed=46, device=DEV)
    alpha = wl.gates((1, 2, 300), seed=47, device=DEV, rate=1 / 4)
    S0, _ = wl.decode_state(1, 2, 64, 64, seed=48, device=DEV, std=0.5)
    o, _ = _run(q, k, v, alpha, S0)
    for s in (0, 63, 64, 100, 299):
        for name in ("k", "v", "alpha"):
            t = {"k": k, "v": v, "alpha": alpha}
            pert = t[name].clone()
            pert[:, :, s] = pert[:, :, s] * 0.5
            t = dict(t, **{name: pert})
            o2, _ = _run(q, t["k"], t["v"], t["alpha"], S0)
            assert torch.equal(o2[:, :, :s], o[:, :, :s]), (name, s)
            assert not torch.equal(o2[:, :, s:], o[:, :, s:]), (name, s)


def test_ssd_deterministic_resume_and_alias():
    q, k, v = wl.la_inputs(1, 4, 2500, 64, 64, torch.bfloat16, seed=49, device=DEV)
    alpha = wl.gates((1, 4, 2500), seed=50, device=DEV, rate=1 / 64)
    a = _run(q, k, v, alpha)
    b = _run(q, k, v, alpha)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    T1 = 1000
    cut = lambda x, s: x[:, :, s].contiguous()
    h1, h2 = slice(0, T1), slice(T1, None)
    oa, Sa = _run(cut(q, h1), cut(k, h1), cut(v, h1), cut(alpha, h1))
    ref = _run(cut(q, h2), cut(k, h2), cut(v, h2), cut(alpha, h2), Sa.clone())
    S = Sa.clone()
    ob, _ = lin.ssd_forward(cut(q, h2), cut(k, h2), cut(v, h2), cut(alpha, h2), S, S_out=S)
    torch.cuda.synchronize()
    assert torch.equal(ob, ref[0]) and torch.equal(S, ref[1])
    tol = TOL[torch.bfloat16]
    assert_parity(torch.cat([oa, ob], 2), to64(a[0]), tol, "o", rows=True)
    assert_parity(S, to64(a[1]), tol, "S")


# ------------------------------------------------------------------ decode

@pytest.mark.parametrize("N,H,dk,dv,dtype", [
    (1, 1, 64, 64, torch.bfloat16), (3, 5, 64, 128, torch.bfloat16), (2, 2, 128, 64, torch.float32),
    (7, 3, 128, 128, torch.bfloat16), (4, 4, 128, 128, torch.float32), (5, 1, 64, 64, torch.float32)])
def test_ssd_decode_step_shapes(N, H, dk, dv, dtype):
    print(f"ssd_decode_step N={N} H={H} dk={dk} dv={dv} {dtype}", flush=True)
    S, _ = wl.decode_state(N, H, dk, dv, seed=26, device=DEV, std=0.3)
    q, k, v = (t[0] for t in wl.decode_tokens(1, N, H, dk, dv, dtype, seed=27, device=DEV))
    alpha = wl.gates((N, H), seed=28, device=DEV, rate=1 / 2)
    S_ref = to64(S)
    o = lin.ssd_decode_step(q, k, v, alpha, S)
    torch.cuda.synchronize()
    ro, rS = oracle.ssd_decode_step(q, k, v, alpha, S_ref)
    assert_parity(o, ro, TOL[dtype], "o", rows=True)
    assert_parity(S, rS, 1e-6, "S")  # fp32 state: one product and one fma per element


def test_ssd_decode_zero_alpha_resets():
    N, H, d = 3, 2, 128
    S, _ = wl.decode_state(N, H, d, d, seed=29, device=DEV, std=0.3)
    q, k, v = (t[0] for t in wl.decode_tokens(1, N, H, d, d, torch.float32, seed=30, device=DEV))
    alpha = torch.zeros((N, H), dtype=torch.float32, device=DEV)
    o = lin.ssd_decode_step(q, k, v, alpha, S)
    torch.cuda.synchronize()
    assert torch.equal(S, k[..., :, None] * v[..., None, :])
    ro, _ = oracle.ssd_decode_step(q, k, v, alpha, np.zeros((N, H, d, d)))
    assert_parity(o, ro, 1e-5, "o", rows=True)


def test_ssd_decode_config_chain_sampled_states():
    w = wl.SSD_DECODE_BF16
    steps = 200
    print(f"ssd_decode_step {w.name} ({steps} steps)", flush=True)
    S, Q, K, V, At = wl.make(w, DEV)
    picks = [(0, 0), (17, 3), (100, 31), (128, 16), (200, 7), (255, 31), (64, 0), (3, 29)]
    n_idx = torch.tensor([p[0] for p in picks], device=DEV)
    h_idx = torch.tensor([p[1] for p in picks], device=DEV)
    S_ref = to64(S[n_idx, h_idx])[None]
    outs = torch.empty((steps, len(picks), w.dv), dtype=w.dtype, device=DEV)
    o = torch.empty((w.B, w.H, w.dv), dtype=w.dtype, device=DEV)
    for t in range(steps):
        lin.ssd_decode_step(Q[t], K[t], V[t], At[t], S, o=o)
        outs[t] = o[n_idx, h_idx]
    torch.cuda.synchronize()
    qs, ks, vs, als = (to64(X[:steps, n_idx, h_idx]) for X in (Q, K, V, At))
    tol = TOL[w.dtype]
    worst = 0.0
    for t in range(steps):
        ro, S_ref = oracle.ssd_decode_step(qs[t][None], ks[t][None], vs[t][None], als[t][None], S_ref)
        worst = max(worst, assert_parity(outs[t][None], ro, tol, f"o step {t}", axes=(2,), rows=True))
    assert_parity(S[n_idx, h_idx][None], S_ref, tol, "S final")
    print(f"worst per-step slice error of o: {worst:.2e}")


def test_ssd_decode_chain_equals_prefill():
    N, H, d, steps = 2, 3, 128, 256
    S, _ = wl.decode_state(N, H, d, d, seed=31, device=DEV, std=0.1)
    Q, K, V = wl.decode_tokens(steps, N, H, d, d, torch.bfloat16, seed=32, device=DEV)
    At = wl.gates((steps, N, H), seed=33, device=DEV, rate=1 / 4)
    S0 = S.clone()
    outs = torch.stack([lin.ssd_decode_step(Q[t], K[t], V[t], At[t], S) for t in range(steps)], 2)
    seq = lambda X: X.permute(1, 2, 0, 3).contiguous()
    o, Sf = lin.ssd_forward(seq(Q), seq(K), seq(V), At.permute(1, 2, 0).contiguous(), S0)
    torch.cuda.synchronize()
    tol = TOL[torch.bfloat16]
    assert_parity(outs, to64(o), tol, "o", rows=True)
    assert_parity(S, to64(Sf), tol, "S")
