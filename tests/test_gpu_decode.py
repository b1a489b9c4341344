"""GPU parity tests of la_decode_step (through the C ABI)."""
import numpy as np
import pytest
import torch

import oracle
from tests.parity import EPS, TOL, assert_parity, to64
from weight_recurrent_memory_amd import binding as lin
from weight_recurrent_memory_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("N,H,dk,dv,dtype", [
    (1, 1, 64, 64, torch.bfloat16), (3, 5, 64, 128, torch.bfloat16), (2, 2, 128, 64, torch.float32),
    (7, 3, 128, 128, torch.bfloat16), (4, 4, 128, 128, torch.float32), (5, 1, 64, 64, torch.float32)])
def test_decode_step_shapes(N, H, dk, dv, dtype):
    print(f"la_decode_step N={N} H={H} dk={dk} dv={dv} {dtype}", flush=True)
    S, z = wl.decode_state(N, H, dk, dv, seed=3, device=DEV)
    q, k, v = (t[0] for t in wl.decode_tokens(1, N, H, dk, dv, dtype, seed=4, device=DEV))
    S_ref, z_ref = to64(S), to64(z)
    o = lin.la_decode_step(q, k, v, S, z, eps=EPS)
    torch.cuda.synchronize()
    ro, rS, rz = oracle.la_decode_step(q, k, v, S_ref, z_ref, eps=EPS)
    tol = TOL[dtype]
    assert_parity(o, ro, tol, "o", rows=True)
    assert_parity(S, rS, 1e-6, "S")   # fp32 state: one fma per element
    assert_parity(z, rz, 1e-6, "z")


def test_decode_config_chain_sampled_states():
    """The full 256 x 32 x d128 workload for all 1000 steps on the GPU; the
    oracle follows 8 sampled (sequence, head) states through every step."""
    w = wl.DECODE_BF16
    print(f"la_decode_step {w.name}", flush=True)
    S, z, Q, K, V = wl.make(w, DEV)
    picks = [(0, 0), (17, 3), (100, 31), (128, 16), (200, 7), (255, 31), (64, 0), (3, 29)]
    n_idx = torch.tensor([p[0] for p in picks], device=DEV)
    h_idx = torch.tensor([p[1] for p in picks], device=DEV)
    S_ref = to64(S[n_idx, h_idx])[None]
    z_ref = to64(z[n_idx, h_idx])[None]
    outs = torch.empty((w.T, len(picks), w.dv), dtype=w.dtype, device=DEV)
    o = torch.empty((w.B, w.H, w.dv), dtype=w.dtype, device=DEV)
    for t in range(w.T):
        lin.la_decode_step(Q[t], K[t], V[t], S, z, eps=EPS, o=o)
        outs[t] = o[n_idx, h_idx]
    torch.cuda.synchronize()
    qs, ks, vs = (to64(X[:, n_idx, h_idx]) for X in (Q, K, V))
    tol = TOL[w.dtype]
    worst = 0.0
    for t in range(w.T):
        ro, S_ref, z_ref = oracle.la_decode_step(qs[t][None], ks[t][None], vs[t][None], S_ref, z_ref, eps=EPS)
        worst = max(worst, assert_parity(outs[t][None], ro, tol, f"o step {t}", axes=(2,), rows=True))
    assert_parity(S[n_idx, h_idx][None], S_ref, tol, "S final")
    assert_parity(z[n_idx, h_idx][None], z_ref, tol, "z final")
    print(f"worst per-step slice error of o: {worst:.2e}")


def test_decode_chain_equals_prefill():
    N, H, d, steps = 2, 3, 64, 300
    S, z = wl.decode_state(N, H, d, d, seed=11, device=DEV)
    z = z.abs() + 1.0
    Q, K, V = wl.decode_tokens(steps, N, H, d, d, torch.float32, seed=12, device=DEV)
    S0, z0 = S.clone(), z.clone()
    outs = torch.stack([lin.la_decode_step(Q[t], K[t], V[t], S, z, eps=EPS) for t in range(steps)], 2)
    seq = lambda X: X.permute(1, 2, 0, 3).contiguous()
    o, Sf, zf = lin.la_forward(seq(Q), seq(K), seq(V), S0, z0, eps=EPS)
    torch.cuda.synchronize()
    tol = TOL[torch.float32]
    assert_parity(outs, to64(o), tol, "o", rows=True)
    assert_parity(S, to64(Sf), tol, "S")
    assert_parity(z, to64(zf), tol, "z")
