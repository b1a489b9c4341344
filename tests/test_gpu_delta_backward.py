"""GPU parity tests of delta_backward (through the C ABI) against the oracle's
reverse-mode gradients of the delta rule and its gated form (themselves
pinned by finite differences and closed forms)."""
import pytest
import torch

import oracle
from tests.parity import TOL, assert_parity
from weight_recurrent_memory_amd import binding as lin
from weight_recurrent_memory_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(B, H, T, dk, dv, seed, init, gated, rate=wl.GATE_RATE):
    q, k, v, beta = wl.delta_inputs(B, H, T, dk, dv, torch.bfloat16, seed=seed, device=DEV)
    dO = wl.la_inputs(B, H, T, dv, dv, torch.bfloat16, seed=seed + 1, device=DEV)[0]
    alpha = wl.gates((B, H, T), seed=seed, device=DEV, rate=rate) if gated else None
    S0 = dS_T = None
    if init:
        S0, _ = wl.decode_state(B, H, dk, dv, seed=seed + 2, device=DEV, std=0.5)
        dS_T, _ = wl.decode_state(B, H, dk, dv, seed=seed + 3, device=DEV, std=0.1)
    return q, k, v, beta, dO, alpha, S0, dS_T


# Row check of dq, dk, dv: each token's row against its own norm, floored at a
# quarter of the median row norm of its (batch, head).  Rows far below the
# median are single inner products that bf16 operands cannot resolve to 2 %
# of their own size -- the last token's dk, for one, has only its own output
# to come from (no dS_T), at about a hundredth of the median row.
ROW_FLOOR = 1 / 4


def _check(args, res, heads=None, row_floor=ROW_FLOOR):
    q, k, v, beta, dO, alpha, S0, dS_T = args
    B, H = q.shape[:2]
    flat = lambda t: None if t is None else t.reshape(B * H, *t.shape[2:])
    idx = list(range(B * H)) if heads is None else list(heads)
    sel = lambda t: None if t is None else flat(t)[idx][None]
    ref = oracle.delta_backward(sel(q), sel(k), sel(v), sel(beta), sel(dO), sel(alpha), sel(S0), sel(dS_T))
    tol = TOL[torch.bfloat16]
    worst = {}
    for name, x, r in zip(("dq", "dk", "dv", "dbeta", "dalpha", "dS0"), res, ref):
        if r is None:
            assert x is None, name
            continue
        axes = (2,) if x.dim() == 3 else None  # dbeta, dalpha: one slice per (batch, head)
        worst[name] = assert_parity(sel(x), r, tol, name, axes=axes, rows=name in ("dq", "dk", "dv"),
                                    row_floor=row_floor)
    print("worst slice errors:", {n: f"{e:.2e}" for n, e in worst.items()})


SHAPES = [
    # B, H, T, dk, dv, with states, gated
    (1, 1, 1, 64, 64, True, False),
    (1, 1, 1, 128, 128, True, True),
    (1, 2, 63, 64, 64, False, True),
    (2, 1, 65, 128, 128, True, False),
    (1, 1, 200, 64, 128, True, True),
    (1, 3, 700, 128, 64, False, False),
    (2, 2, 1000, 64, 64, True, True),
    (1, 2, 3000, 128, 128, True, False),
    (1, 2, 3000, 128, 128, True, True),
    (1, 1, 4100, 64, 64, False, True),
    (1, 256, 130, 64, 64, True, True),   # one segment per sequence
]


@pytest.mark.parametrize("B,H,T,dk,dv,init,gated", SHAPES)
def test_delta_backward_shapes(B, H, T, dk, dv, init, gated):
    print(f"delta_backward B={B} H={H} T={T} dk={dk} dv={dv} init={init} gated={gated}", flush=True)
    args = _inputs(B, H, T, dk, dv, seed=7000 + T, init=init, gated=gated)
    q, k, v, beta, dO, alpha, S0, dS_T = args
    res = lin.delta_backward(q, k, v, beta, dO, alpha, S0, dS_T)
    torch.cuda.synchronize()
    _check(args, res)


def test_delta_backward_strong_gates():
    # Gates well below one (rate 1: alpha down to about e^-5 per token), so
    # chunk-local products span many orders of magnitude.  The state then
    # holds little more than the last write, beta k u^T, and dq_t = S_t dO_t
    # nearly cancels on tokens where u_t . dO_t is small: rounding S to the
    # bf16 MFMA operand alone (all else exact, fp64) gives those rows errors
    # of 3-4 % of their own norm, at about a tenth of the median row norm.
    # Here the row check's floor is half the median row norm.
    print("delta_backward strong gates", flush=True)
    args = _inputs(1, 2, 600, 128, 128, seed=71, init=True, gated=True, rate=1.0)
    res = lin.delta_backward(*args[:5], alpha=args[5], S0=args[6], dS_T=args[7])
    torch.cuda.synchronize()
    _check(args, res, row_floor=1 / 2)


@pytest.mark.parametrize("gated", [False, True])
def test_delta_backward_config_all_heads(gated):
    w = wl.DELTA_BF16_PREFILL
    print(f"delta_backward {w.name} gated={gated}", flush=True)
    args = _inputs(w.B, w.H, w.T, w.dk, w.dv, seed=72, init=False, gated=gated)
    res = lin.delta_backward(*args[:5], alpha=args[5])
    torch.cuda.synchronize()
    _check(args, res)


def test_delta_backward_deterministic():
    args = _inputs(1, 4, 2500, 128, 128, seed=73, init=True, gated=True)
    a = lin.delta_backward(*args[:5], alpha=args[5], S0=args[6], dS_T=args[7])
    b = lin.delta_backward(*args[:5], alpha=args[5], S0=args[6], dS_T=args[7])
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
