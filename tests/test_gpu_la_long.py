"""GPU parity of la_forward (bf16, dk = dv = 64) on the shapes where
segments are long and sequences many, through the C ABI: ragged last
segments, sequences shorter than one segment, the look-back's give-up path
with many segments per sequence, and in-place continuation.

The chunked form with its state handed between segments equals the
sequential recurrence ("AIGC 基本功｜线性、循环与记忆架构-LinearMem" §03;
"手撕：递推与记忆模型", "Chunked scan")."""
import pytest
import torch

import oracle
from tests.parity import EPS, TOL, assert_parity
from weight_recurrent_memory_amd import binding as lin
from weight_recurrent_memory_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _state(B, H, seed):
    S0, z0 = wl.decode_state(B, H, 64, 64, seed=seed, device=DEV, std=0.5)
    return S0, z0.abs() + 1.0


def _check(q, k, v, o, S, z, S0=None, z0=None):
    tol = TOL[q.dtype]
    B, H = q.shape[:2]
    flat = lambda t: None if t is None else t.reshape(1, B * H, *t.shape[2:])
    ro, rS, rz = oracle.la_forward(flat(q), flat(k), flat(v), flat(S0), flat(z0), eps=EPS)
    e1 = assert_parity(flat(o), ro, tol, "o", rows=True)
    e2 = assert_parity(flat(S), rS, tol, "S_T")
    e3 = assert_parity(flat(z), rz, tol, "z_T")
    print(f"worst errors: o {e1:.2e}  S {e2:.2e}  z {e3:.2e}")


@pytest.mark.parametrize("B,H,T,init", [
    (2, 16, 8193, True),    # the last segment one token long
    (2, 16, 9000, False),   # a ragged last chunk
    (1, 32, 16383, True),   # the last chunk one token short
    (1, 512, 600, True),    # many short sequences
    (4, 16, 4100, False),   # the last segment 4 tokens
])
def test_la_long_segments_match_oracle(B, H, T, init):
    print(f"la_forward B={B} H={H} T={T} init={init}", flush=True)
    q, k, v = wl.la_inputs(B, H, T, 64, 64, torch.bfloat16, seed=6000 + T + H, device=DEV)
    S0 = z0 = None
    if init:
        S0, z0 = _state(B, H, 61)
    o, S, z = lin.la_forward(q, k, v, S0, z0, eps=EPS)
    torch.cuda.synchronize()
    _check(q, k, v, o, S, z, S0, z0)


@pytest.mark.parametrize("polls", [-1, 0, 1])
@pytest.mark.parametrize("init,alias", [(False, False), (True, False), (True, True)])
def test_la_give_up_path_with_many_segments_is_bitwise_equal(polls, init, alias):
    """With the look-back's wait bound forced to (almost) nothing, later
    segments recompute their incoming state from the inputs in the
    look-back's own order: every output equals the normal call bit for bit,
    also when S_out, z_out alias S0, z0."""
    B, H, T = 2, 16, 9000
    print(f"la_forward give-up path B=2 H=16 T=9000 polls={polls} init={init} alias={alias}", flush=True)
    q, k, v = wl.la_inputs(B, H, T, 64, 64, torch.bfloat16, seed=95, device=DEV)
    S0 = z0 = None
    if init:
        S0, z0 = _state(B, H, 96)
    ref = lin.la_forward(q, k, v, None if S0 is None else S0.clone(), None if z0 is None else z0.clone(), eps=EPS)
    if alias:
        S, z = S0.clone(), z0.clone()
        o, _, _ = lin.la_forward(q, k, v, S, z, eps=EPS, S_out=S, z_out=z, lookback_polls=polls)
    else:
        o, S, z = lin.la_forward(q, k, v, S0, z0, eps=EPS, lookback_polls=polls)
    torch.cuda.synchronize()
    assert torch.equal(o, ref[0]) and torch.equal(S, ref[1]) and torch.equal(z, ref[2])
    if polls == 0 and not alias:
        _check(q, k, v, o, S, z, S0, z0)


def test_la_long_stream_continues_in_place():
    # the second call starts from the first call's final state, in the same buffers
    B, H, T1, T2 = 1, 32, 8192, 8300
    q, k, v = wl.la_inputs(B, H, T1 + T2, 64, 64, torch.bfloat16, seed=97, device=DEV)
    part = lambda t, a, b: t[:, :, a:b].contiguous()
    S = torch.empty((B, H, 64, 64), dtype=torch.float32, device=DEV)
    z = torch.empty((B, H, 64), dtype=torch.float32, device=DEV)
    o1, _, _ = lin.la_forward(part(q, 0, T1), part(k, 0, T1), part(v, 0, T1), eps=EPS, S_out=S, z_out=z)
    o2, _, _ = lin.la_forward(part(q, T1, T1 + T2), part(k, T1, T1 + T2), part(v, T1, T1 + T2), S, z, eps=EPS,
                              S_out=S, z_out=z)
    torch.cuda.synchronize()
    _check(q, k, v, torch.cat([o1, o2], dim=2), S, z)


def test_la_long_stream_is_bitwise_repeatable():
    q, k, v = wl.la_inputs(2, 16, 12000, 64, 64, torch.bfloat16, seed=98, device=DEV)
    a = lin.la_forward(q, k, v, eps=EPS)
    b = lin.la_forward(q, k, v, eps=EPS)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
