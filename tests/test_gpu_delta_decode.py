"""GPU parity tests of delta_decode_step (through the C ABI)."""
import numpy as np
import pytest
import torch

import oracle
from tests.parity import TOL, assert_parity, to64
from weight_recurrent_memory_amd import binding as lin
from weight_recurrent_memory_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("N,H,dk,dv,dtype", [
    (1, 1, 64, 64, torch.bfloat16), (3, 5, 64, 128, torch.bfloat16), (2, 2, 128, 64, torch.float32),
    (7, 3, 128, 128, torch.bfloat16), (4, 4, 128, 128, torch.float32), (5, 1, 64, 64, torch.float32)])
def test_delta_decode_step_shapes(N, H, dk, dv, dtype):
    print(f"delta_decode_step N={N} H={H} dk={dk} dv={dv} {dtype}", flush=True)
    S, _ = wl.decode_state(N, H, dk, dv, seed=13, device=DEV, std=0.3)
    q, k, v, beta = (t[0] for t in wl.delta_decode_tokens(1, N, H, dk, dv, dtype, seed=14, device=DEV))
    S_ref = to64(S)
    o = lin.delta_decode_step(q, k, v, beta, S)
    torch.cuda.synchronize()
    ro, rS = oracle.delta_decode_step(q, k, v, beta, S_ref)
    assert_parity(o, ro, TOL[dtype], "o", rows=True)
    assert_parity(S, rS, 1e-5, "S")  # fp32 state: a dk-term dot product, then one fma


def test_delta_decode_exact_overwrite_basis_keys():
    """Unit basis keys, beta = 1 and dyadic values: the read of the key just
    written returns the new value exactly, in fp32 and in bf16."""
    for dtype in (torch.float32, torch.bfloat16):
        N, H, d = 3, 4, 64
        g = torch.Generator(device="cpu").manual_seed(5)
        S = (torch.randint(-64, 64, (N, H, d, d), generator=g).float() / 16).to(DEV)
        idx = torch.randint(0, d, (N, H), generator=g)
        k = torch.nn.functional.one_hot(idx, d).to(dtype).to(DEV)
        v = (torch.randint(-64, 64, (N, H, d), generator=g).float() / 8).to(dtype).to(DEV)
        beta = torch.ones((N, H), dtype=dtype, device=DEV)
        o = lin.delta_decode_step(k, k, v, beta, S)
        torch.cuda.synchronize()
        assert torch.equal(o, v), dtype


def test_delta_decode_config_chain_sampled_states():
    """The 256 x 32 x d128 states for 200 steps on the GPU; the oracle follows
    8 sampled (sequence, head) states through every step."""
    w = wl.DELTA_DECODE_BF16
    steps = 200
    print(f"delta_decode_step {w.name} ({steps} steps)", flush=True)
    S, Q, K, V, Bt = wl.make(w, DEV)
    picks = [(0, 0), (17, 3), (100, 31), (128, 16), (200, 7), (255, 31), (64, 0), (3, 29)]
    n_idx = torch.tensor([p[0] for p in picks], device=DEV)
    h_idx = torch.tensor([p[1] for p in picks], device=DEV)
    S_ref = to64(S[n_idx, h_idx])[None]
    outs = torch.empty((steps, len(picks), w.dv), dtype=w.dtype, device=DEV)
    o = torch.empty((w.B, w.H, w.dv), dtype=w.dtype, device=DEV)
    for t in range(steps):
        lin.delta_decode_step(Q[t], K[t], V[t], Bt[t], S, o=o)
        outs[t] = o[n_idx, h_idx]
    torch.cuda.synchronize()
    qs, ks, vs, bs = (to64(X[:steps, n_idx, h_idx]) for X in (Q, K, V, Bt))
    tol = TOL[w.dtype]
    worst = 0.0
    for t in range(steps):
        ro, S_ref = oracle.delta_decode_step(qs[t][None], ks[t][None], vs[t][None], bs[t][None], S_ref)
        worst = max(worst, assert_parity(outs[t][None], ro, tol, f"o step {t}", axes=(2,), rows=True))
    assert_parity(S[n_idx, h_idx][None], S_ref, tol, "S final")
    print(f"worst per-step slice error of o: {worst:.2e}")


def test_delta_decode_chain_equals_prefill():
    N, H, d, steps = 2, 3, 128, 256
    S, _ = wl.decode_state(N, H, d, d, seed=21, device=DEV, std=0.1)
    Q, K, V, Bt = wl.delta_decode_tokens(steps, N, H, d, d, torch.bfloat16, seed=22, device=DEV)
    S0 = S.clone()
    outs = torch.stack([lin.delta_decode_step(Q[t], K[t], V[t], Bt[t], S) for t in range(steps)], 2)
    seq = lambda X: X.permute(1, 2, 0, 3).contiguous()
    o, Sf = lin.delta_forward(seq(Q), seq(K), seq(V), Bt.permute(1, 2, 0).contiguous(), S0)
    torch.cuda.synchronize()
    tol = TOL[torch.bfloat16]
    assert_parity(outs, to64(o), tol, "o", rows=True)
    assert_parity(S, to64(Sf), tol, "S")
