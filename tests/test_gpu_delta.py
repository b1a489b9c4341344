"""GPU parity and structure tests of delta_forward (through the C ABI)."""
import numpy as np
import pytest
import torch

import oracle
from tests.parity import TOL, assert_parity, to64
from weight_recurrent_memory_amd import binding as lin
from weight_recurrent_memory_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run(q, k, v, beta, S0=None):
    o, S = lin.delta_forward(q, k, v, beta, S0)
    torch.cuda.synchronize()
    return o, S


def _check(q, k, v, beta, o, S, S0=None, heads=None):
    tol = TOL[q.dtype]
    B, H = q.shape[:2]
    flat = lambda t: None if t is None else t.reshape(B * H, *t.shape[2:])
    qf, kf, vf, bf, of, Sf, S0f = map(flat, (q, k, v, beta, o, S, S0))
    idx = list(range(B * H)) if heads is None else list(heads)
    sel = lambda t: None if t is None else t[idx][None]
    ro, rS = oracle.delta_forward(sel(qf), sel(kf), sel(vf), sel(bf), sel(S0f))
    e1 = assert_parity(sel(of), ro, tol, "o", rows=True)
    e2 = assert_parity(sel(Sf), rS, tol, "S_T")
    print(f"worst slice errors: o {e1:.2e}  S {e2:.2e}")


SHAPES = [
    # B, H, T, dk, dv, with initial state
    (1, 1, 1, 128, 128, False),
    (1, 2, 2, 64, 64, True),
    (2, 1, 63, 128, 128, True),
    (1, 1, 64, 64, 128, False),
    (1, 3, 65, 128, 64, True),
    (1, 1, 200, 128, 128, False),
    (2, 2, 1000, 64, 64, True),
    (1, 2, 3000, 128, 128, True),
    (1, 1, 2500, 128, 64, False),
    (1, 1, 2049, 64, 128, True),
    (2, 160, 300, 128, 128, True),   # 320 heads: one segment per sequence, no map pass
    (1, 64, 1000, 128, 128, True),   # four segments per head: the sixteen-wave map pass
]


@pytest.mark.parametrize("B,H,T,dk,dv,init", SHAPES)
def test_delta_small_shapes(B, H, T, dk, dv, init):
    print(f"delta_forward B={B} H={H} T={T} dk={dk} dv={dv} init={init}", flush=True)
    q, k, v, beta = wl.delta_inputs(B, H, T, dk, dv, torch.bfloat16, seed=2000 + T, device=DEV)
    S0 = None
    if init:
        S0, _ = wl.decode_state(B, H, dk, dv, seed=78, device=DEV, std=0.5)
    o, S = _run(q, k, v, beta, S0)
    _check(q, k, v, beta, o, S, S0)


def test_delta_config_all_heads():
    w = wl.DELTA_BF16_PREFILL
    print(f"delta_forward {w.name}", flush=True)
    q, k, v, beta = wl.make(w, DEV)
    o, S = _run(q, k, v, beta)
    _check(q, k, v, beta, o, S)


def test_delta_exact_overwrite_basis_keys():
    """Unit (basis) keys, beta = 1, dyadic values: reading k_t right after the
    write returns v_t exactly, through the chunked MFMA path."""
    B, H, T, d = 1, 2, 300, 128
    g = torch.Generator().manual_seed(5)
    idx = torch.randint(0, d, (B, H, T), generator=g)
    k = torch.nn.functional.one_hot(idx, d).to(torch.bfloat16)
    v = (torch.randint(-64, 64, (B, H, T, d), generator=g) / 8.0).to(torch.bfloat16)
    beta = torch.ones((B, H, T), dtype=torch.bfloat16)
    k, v, beta = k.to(DEV), v.to(DEV), beta.to(DEV)
    o, _ = _run(k, k, v, beta)
    assert torch.equal(o, v)


def test_delta_causality_bitwise():
    q, k, v, beta = wl.delta_inputs(1, 2, 300, 128, 128, torch.bfloat16, seed=5, device=DEV)
    o, _ = _run(q, k, v, beta)
    for s in (0, 63, 64, 100, 299):
        for name in ("k", "v", "beta"):
            t = {"k": k, "v": v, "beta": beta}
            pert = t[name].clone()
            pert[:, :, s] = pert[:, :, s] * 0.5 + 0.25
            t = dict(t, **{name: pert})
            o2, _ = _run(q, t["k"], t["v"], t["beta"])
            assert torch.equal(o2[:, :, :s], o[:, :, :s]), (name, s)
            assert not torch.equal(o2[:, :, s:], o[:, :, s:]), (name, s)


def test_delta_deterministic_and_resume():
    q, k, v, beta = wl.delta_inputs(1, 4, 2500, 128, 128, torch.bfloat16, seed=6, device=DEV)
    a = _run(q, k, v, beta)
    b = _run(q, k, v, beta)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    T1 = 1000
    cut = lambda x, s: x[:, :, s].contiguous()
    oa, Sa = _run(cut(q, slice(0, T1)), cut(k, slice(0, T1)), cut(v, slice(0, T1)), cut(beta, slice(0, T1)))
    ob, Sb = _run(cut(q, slice(T1, None)), cut(k, slice(T1, None)), cut(v, slice(T1, None)),
                  cut(beta, slice(T1, None)), Sa)
    tol = TOL[torch.bfloat16]
    assert_parity(torch.cat([oa, ob], 2), to64(a[0]), tol, "o", rows=True)
    assert_parity(Sb, to64(a[1]), tol, "S")


def test_delta_state_alias_and_head_isolation():
    q, k, v, beta = wl.delta_inputs(1, 8, 1500, 128, 128, torch.bfloat16, seed=7, device=DEV)
    S0, _ = wl.decode_state(1, 8, 128, 128, seed=8, device=DEV, std=0.3)
    ref = _run(q, k, v, beta, S0.clone())
    S = S0.clone()
    o, _ = lin.delta_forward(q, k, v, beta, S, S_out=S)
    torch.cuda.synchronize()
    assert torch.equal(o, ref[0]) and torch.equal(S, ref[1])
    v2 = v.clone()
    v2[:, 3] += 1.0
    o2, S2 = _run(q, k, v2, beta, S0.clone())
    assert torch.equal(o2[:, :3], ref[0][:, :3]) and torch.equal(o2[:, 4:], ref[0][:, 4:])
    assert torch.equal(S2[:, :3], ref[1][:, :3])
