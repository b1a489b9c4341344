"""GPU tests of the delta rule's training pair, through the C ABI:
delta_forward_train keeps the context the backward pass needs (the states at
chunk boundaries, "AIGC 基本功｜线性、循环与记忆架构-LinearMem" §03 on
training by chunks), and delta_backward_after_forward reads it instead of
recomputing it.  Both must return, bit for bit, what delta_forward /
gated_delta_forward and delta_backward return on the same inputs; one case
is also held against the oracle's gradients directly."""
import pytest
import torch

import oracle
from tests.parity import TOL, assert_parity
from weight_recurrent_memory_amd import binding as lin
from weight_recurrent_memory_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(B, H, T, dk, dv, seed, init, gated):
    q, k, v, beta = wl.delta_inputs(B, H, T, dk, dv, torch.bfloat16, seed=seed, device=DEV)
    dO = wl.la_inputs(B, H, T, dv, dv, torch.bfloat16, seed=seed + 1, device=DEV)[0]
    alpha = wl.gates((B, H, T), seed=seed, device=DEV) if gated else None
    S0 = dS_T = None
    if init:
        S0, _ = wl.decode_state(B, H, dk, dv, seed=seed + 2, device=DEV, std=0.5)
        dS_T, _ = wl.decode_state(B, H, dk, dv, seed=seed + 3, device=DEV, std=0.1)
    return q, k, v, beta, dO, alpha, S0, dS_T


def _plain(q, k, v, beta, dO, alpha, S0, dS_T):
    fwd = (lin.gated_delta_forward(q, k, v, beta, alpha, S0) if alpha is not None
           else lin.delta_forward(q, k, v, beta, S0))
    bwd = lin.delta_backward(q, k, v, beta, dO, alpha, S0, dS_T)
    return fwd, bwd


def _train(q, k, v, beta, dO, alpha, S0, dS_T, workspace=None):
    o, S, ws = lin.delta_forward_train(q, k, v, beta, alpha, S0, workspace=workspace)
    bwd = lin.delta_backward_after_forward(q, k, v, beta, dO, ws, alpha, S0, dS_T)
    return (o, S), bwd, ws


def _same(a, b, names):
    for name, x, y in zip(names, a, b):
        if x is None or y is None:
            assert x is None and y is None, name
            continue
        assert torch.equal(x, y), f"{name}: max |diff| {(x.float() - y.float()).abs().max().item():.3e}"


FWD = ("o", "S_T")
BWD = ("dq", "dk", "dv", "dbeta", "dalpha", "dS0")

SHAPES = [
    # B, H, T, dk, dv, with states, gated
    (1, 1, 1, 64, 64, True, False),
    (1, 2, 63, 128, 128, False, True),
    (2, 1, 65, 128, 128, True, False),
    (1, 3, 700, 64, 128, True, True),
    (2, 2, 1000, 128, 64, False, False),
    (1, 2, 3000, 128, 128, True, True),
    (1, 1, 4100, 64, 64, True, False),
    (1, 256, 130, 64, 64, True, True),   # one segment per sequence
    (1, 64, 1000, 128, 128, True, False),  # four segments per sequence
]


@pytest.mark.parametrize("B,H,T,dk,dv,init,gated", SHAPES)
def test_training_pair_equals_the_separate_calls(B, H, T, dk, dv, init, gated):
    print(f"delta training pair B={B} H={H} T={T} dk={dk} dv={dv} init={init} gated={gated}", flush=True)
    args = _inputs(B, H, T, dk, dv, seed=9000 + T + H, init=init, gated=gated)
    fwd, bwd = _plain(*args)
    fwd_t, bwd_t, _ = _train(*args)
    torch.cuda.synchronize()
    _same(fwd_t, fwd, FWD)
    _same(bwd_t, bwd, BWD)


@pytest.mark.parametrize("gated", [False, True])
def test_training_pair_on_the_bench_shape(gated):
    w = wl.DELTA_BF16_PREFILL
    print(f"delta training pair {w.name} gated={gated}", flush=True)
    args = _inputs(w.B, w.H, w.T, w.dk, w.dv, seed=91, init=False, gated=gated)
    fwd, bwd = _plain(*args)
    fwd_t, bwd_t, _ = _train(*args)
    torch.cuda.synchronize()
    _same(fwd_t, fwd, FWD)
    _same(bwd_t, bwd, BWD)


def test_training_pair_matches_the_oracle():
    args = _inputs(1, 2, 900, 128, 128, seed=92, init=True, gated=True)
    q, k, v, beta, dO, alpha, S0, dS_T = args
    (o, S), res, _ = _train(*args)
    torch.cuda.synchronize()
    flat = lambda t: None if t is None else t.reshape(1, 2, *t.shape[2:])
    ro, rS = oracle.gated_delta_forward(flat(q), flat(k), flat(v), flat(beta), flat(alpha), flat(S0))
    tol = TOL[torch.bfloat16]
    assert_parity(o, ro, tol, "o", rows=True)
    assert_parity(S, rS, tol, "S_T")
    ref = oracle.delta_backward(q, k, v, beta, dO, alpha, S0, dS_T)
    for name, x, r in zip(BWD, res, ref):
        axes = (2,) if x.dim() == 3 else None
        assert_parity(x, r, tol, name, axes=axes, rows=name in ("dq", "dk", "dv"), row_floor=1 / 4)


def test_workspace_reused_by_a_second_pair():
    # one workspace for two training steps of different inputs: the second
    # pair's context replaces the first's entirely
    a1 = _inputs(1, 4, 2500, 128, 128, seed=93, init=True, gated=True)
    a2 = _inputs(1, 4, 2500, 128, 128, seed=94, init=False, gated=True)
    _, _, ws = _train(*a1)
    fwd_t, bwd_t, ws2 = _train(*a2, workspace=ws)
    assert ws2.data_ptr() == ws.data_ptr()
    fwd, bwd = _plain(*a2)
    torch.cuda.synchronize()
    _same(fwd_t, fwd, FWD)
    _same(bwd_t, bwd, BWD)
