"""GPU parity of delta_forward at chunk sizes other than 64 (the blocked
path: segment maps by chunk loops of C tokens, their composition, then the
chunk loops writing the outputs), through the C ABI.

The rule's chunked form -- corrections solved per chunk, the state handed
from chunk to chunk -- gives the same outputs and final state for every
chunk size up to rounding ("手撕：递推与记忆模型", "Chunked scan"; the
Delta-rule fast weight section for the rule): every case is checked
against the sequential fp64 oracle, and C = 16, 32, 128 against the 64-token
kernels' result."""
import pytest
import torch

import oracle
from tests.parity import TOL, assert_parity, to64
from weight_recurrent_memory_amd import binding as lin
from weight_recurrent_memory_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _check(q, k, v, beta, o, S, S0=None):
    tol = TOL[q.dtype]
    B, H = q.shape[:2]
    flat = lambda t: None if t is None else t.reshape(1, B * H, *t.shape[2:])
    ro, rS = oracle.delta_forward(flat(q), flat(k), flat(v), flat(beta), flat(S0))
    e1 = assert_parity(flat(o), ro, tol, "o", rows=True)
    e2 = assert_parity(flat(S), rS, tol, "S_T")
    print(f"worst errors: o {e1:.2e}  S {e2:.2e}")


CASES = [
    # C, B, H, T, dk, dv, with initial state
    (16, 1, 1, 1, 128, 128, False),
    (16, 1, 2, 17, 64, 64, True),
    (16, 2, 1, 1000, 128, 128, True),     # 128 segments of 64 tokens per sequence
    (16, 1, 3, 555, 64, 128, False),
    (32, 1, 1, 31, 128, 64, True),
    (32, 2, 2, 2049, 128, 128, True),
    (32, 1, 4, 700, 64, 64, False),
    (128, 1, 1, 100, 128, 128, True),
    (128, 1, 2, 129, 64, 128, False),
    (128, 2, 2, 3000, 128, 128, True),    # segments of 128 tokens: twice the 64-token plan's length
    (128, 1, 3, 1500, 128, 64, True),
    (128, 1, 64, 1000, 128, 128, True),   # four segments per head
]


@pytest.mark.parametrize("C,B,H,T,dk,dv,init", CASES)
def test_delta_chunk_size_matches_oracle(C, B, H, T, dk, dv, init):
    print(f"delta_forward chunk={C} B={B} H={H} T={T} dk={dk} dv={dv} init={init}", flush=True)
    q, k, v, beta = wl.delta_inputs(B, H, T, dk, dv, torch.bfloat16, seed=8000 + T + C, device=DEV)
    S0 = None
    if init:
        S0, _ = wl.decode_state(B, H, dk, dv, seed=81, device=DEV, std=0.5)
    o, S = lin.delta_forward(q, k, v, beta, S0, chunk=C)
    torch.cuda.synchronize()
    _check(q, k, v, beta, o, S, S0)


@pytest.mark.parametrize("C", [16, 32, 128])
def test_delta_chunk_size_independent_of_the_64_token_kernels(C):
    # the bench shape's heads (d = 128) at 4096 tokens
    B, H, T = 2, 16, 4096
    print(f"delta_forward chunk={C} vs 64, B={B} H={H} T={T}", flush=True)
    q, k, v, beta = wl.delta_inputs(B, H, T, 128, 128, torch.bfloat16, seed=8100, device=DEV)
    o64, S64 = lin.delta_forward(q, k, v, beta)
    oc, Sc = lin.delta_forward(q, k, v, beta, chunk=C)
    torch.cuda.synchronize()
    tol = TOL[torch.bfloat16]
    assert_parity(oc, to64(o64), tol, f"o(C={C}) vs o(C=64)", rows=True)
    assert_parity(Sc, to64(S64), tol, f"S(C={C}) vs S(C=64)")
    for hh in (0, 31):
        b, h = divmod(hh, H)
        sl = lambda t: t[b:b + 1, h:h + 1]
        ro, rS = oracle.delta_forward(sl(q), sl(k), sl(v), sl(beta))
        assert_parity(sl(oc), ro, tol, f"o(C={C}) head {hh}", rows=True)
        assert_parity(sl(Sc), rS, tol, f"S(C={C}) head {hh}")


def test_delta_chunk_size_exact_overwrite_basis_keys():
    # unit basis keys with beta = 1 overwrite their slot exactly, and a read
    # right after returns the value written (LinearMem §03 overwrite)
    C, B, H, T, d = 16, 1, 1, 48, 64
    eye = torch.eye(d, dtype=torch.float32)
    k = eye[torch.arange(T) % d][None, None].to(torch.bfloat16).to(DEV)
    v = (torch.arange(T * d, dtype=torch.float32).reshape(1, 1, T, d) % 7 - 3).to(torch.bfloat16).to(DEV)
    beta = torch.ones((B, H, T), dtype=torch.bfloat16, device=DEV)
    o, S = lin.delta_forward(k, k, v, beta, chunk=C)
    torch.cuda.synchronize()
    assert torch.equal(o.float().cpu(), v.float().cpu())


@pytest.mark.parametrize("C", [16, 32, 128])
def test_delta_chunk_size_is_bitwise_repeatable(C):
    q, k, v, beta = wl.delta_inputs(2, 4, 2500, 128, 128, torch.bfloat16, seed=8200 + C, device=DEV)
    S0, _ = wl.decode_state(2, 4, 128, 128, seed=82, device=DEV, std=0.5)
    a = lin.delta_forward(q, k, v, beta, S0, chunk=C)
    b = lin.delta_forward(q, k, v, beta, S0, chunk=C)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
