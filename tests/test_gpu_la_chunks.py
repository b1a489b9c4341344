"""GPU parity of la_forward at chunk sizes other than 64 (the blocked path:
segment sums, their prefix, chunk loops of C tokens), through the C ABI.

The chunked form gives the same outputs and final state for every chunk
size up to rounding ("手撕：递推与记忆模型", "Chunked scan": a scan handed its
state every few tokens equals one pass; "线性注意力与 SSM:两条技术路线的完整
推导" §3, the chunkwise form): every case is checked against the sequential
fp64 oracle, and the C = 16, 32, 128 results against the fused 64-token
kernel's."""
import pytest
import torch

import oracle
from tests.parity import EPS, TOL, assert_parity, to64
from weight_recurrent_memory_amd import binding as lin
from weight_recurrent_memory_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _check(q, k, v, o, S, z, S0=None, z0=None):
    tol = TOL[q.dtype]
    B, H = q.shape[:2]
    flat = lambda t: None if t is None else t.reshape(1, B * H, *t.shape[2:])
    ro, rS, rz = oracle.la_forward(flat(q), flat(k), flat(v), flat(S0), flat(z0), eps=EPS)
    e1 = assert_parity(flat(o), ro, tol, "o", rows=True)
    e2 = assert_parity(flat(S), rS, tol, "S_T")
    e3 = assert_parity(flat(z), rz, tol, "z_T")
    print(f"worst errors: o {e1:.2e}  S {e2:.2e}  z {e3:.2e}")


CASES = [
    # C, B, H, T, dk, dv, dtype, with initial state
    (16, 1, 1, 1, 64, 64, torch.bfloat16, False),
    (16, 1, 2, 15, 64, 64, torch.bfloat16, True),
    (16, 2, 2, 1000, 64, 128, torch.bfloat16, True),
    (16, 1, 3, 777, 128, 64, torch.float32, True),
    (32, 1, 1, 33, 128, 128, torch.bfloat16, False),
    (32, 2, 3, 2049, 64, 64, torch.bfloat16, True),
    (32, 1, 2, 1000, 128, 128, torch.float32, False),
    (32, 2, 2, 333, 64, 128, torch.float32, True),
    (128, 1, 1, 127, 64, 64, torch.bfloat16, True),
    (128, 1, 2, 129, 128, 128, torch.bfloat16, False),
    (128, 2, 4, 3000, 64, 64, torch.bfloat16, True),
    (128, 1, 3, 1500, 128, 64, torch.bfloat16, True),
]


@pytest.mark.parametrize("C,B,H,T,dk,dv,dtype,init", CASES)
def test_la_chunk_size_matches_oracle(C, B, H, T, dk, dv, dtype, init):
    print(f"la_forward chunk={C} B={B} H={H} T={T} dk={dk} dv={dv} {dtype} init={init}", flush=True)
    q, k, v = wl.la_inputs(B, H, T, dk, dv, dtype, seed=7000 + T + C, device=DEV)
    S0 = z0 = None
    if init:
        S0, z0 = wl.decode_state(B, H, dk, dv, seed=79, device=DEV, std=0.5)
        z0 = z0.abs() + 1.0
    o, S, z = lin.la_forward(q, k, v, S0, z0, eps=EPS, chunk=C)
    torch.cuda.synchronize()
    _check(q, k, v, o, S, z, S0, z0)


@pytest.mark.parametrize("C", [16, 32, 128])
def test_la_chunk_size_independent_of_the_fused_kernel(C):
    # 32 (sequence, head) pairs of 6000 tokens: several segments of each
    B, H, T = 2, 16, 6000
    print(f"la_forward chunk={C} vs 64, B={B} H={H} T={T}", flush=True)
    q, k, v = wl.la_inputs(B, H, T, 64, 64, torch.bfloat16, seed=7100, device=DEV)
    o64, S64, z64 = lin.la_forward(q, k, v, eps=EPS)
    oc, Sc, zc = lin.la_forward(q, k, v, eps=EPS, chunk=C)
    torch.cuda.synchronize()
    tol = TOL[torch.bfloat16]
    assert_parity(oc, to64(o64), tol, f"o(C={C}) vs o(C=64)", rows=True)
    assert_parity(Sc, to64(S64), tol, f"S(C={C}) vs S(C=64)")
    assert_parity(zc, to64(z64), tol, f"z(C={C}) vs z(C=64)")
    # and both against the oracle on two heads (the whole length)
    for hh in (0, 31):
        b, h = divmod(hh, H)
        sl = lambda t: t[b:b + 1, h:h + 1]
        ro, rS, rz = oracle.la_forward(sl(q), sl(k), sl(v), eps=EPS)
        assert_parity(sl(oc), ro, tol, f"o(C={C}) head {hh}", rows=True)
        assert_parity(sl(Sc), rS, tol, f"S(C={C}) head {hh}")


@pytest.mark.parametrize("C", [16, 128])
def test_la_chunk_size_continues_in_place(C):
    # the second call's S0, z0 are the first call's S_out, z_out (the same
    # buffers): the prefix reads them before the chunk loops write them
    B, H, T1, T2 = 1, 4, 700, 900
    q, k, v = wl.la_inputs(B, H, T1 + T2, 64, 64, torch.bfloat16, seed=7200 + C, device=DEV)
    S = torch.empty((B, H, 64, 64), dtype=torch.float32, device=DEV)
    z = torch.empty((B, H, 64), dtype=torch.float32, device=DEV)
    o1 = torch.empty((B, H, T1, 64), dtype=torch.bfloat16, device=DEV)
    o2 = torch.empty((B, H, T2, 64), dtype=torch.bfloat16, device=DEV)
    part = lambda t, a, b: t[:, :, a:b].contiguous()
    lin.la_forward(part(q, 0, T1), part(k, 0, T1), part(v, 0, T1), eps=EPS, chunk=C, o=o1, S_out=S, z_out=z)
    lin.la_forward(part(q, T1, T1 + T2), part(k, T1, T1 + T2), part(v, T1, T1 + T2), S, z, eps=EPS, chunk=C,
                   o=o2, S_out=S, z_out=z)
    torch.cuda.synchronize()
    _check(q, k, v, torch.cat([o1, o2], dim=2), S, z)


@pytest.mark.parametrize("C,dtype", [(16, torch.float32), (32, torch.bfloat16), (128, torch.bfloat16)])
def test_la_chunk_size_is_bitwise_repeatable(C, dtype):
    # fixed summation order, no atomics: the same inputs give the same bits
    q, k, v = wl.la_inputs(2, 4, 3000, 64, 64, dtype, seed=7300 + C, device=DEV)
    a = lin.la_forward(q, k, v, eps=EPS, chunk=C)
    b = lin.la_forward(q, k, v, eps=EPS, chunk=C)
    torch.cuda.synchronize()
    for name, x, y in zip(("o", "S", "z"), a, b):
        assert torch.equal(x, y), name
