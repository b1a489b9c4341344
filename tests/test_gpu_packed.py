"""GPU tests of the packed-batch prefills (through the C ABI): variable-length
sequences concatenated along the token axis, each with its own initial and
final state; every sequence is checked against the oracle run on it alone."""
import numpy as np
import pytest
import torch

import oracle
from tests.parity import TOL, EPS, assert_parity
from weight_recurrent_memory_amd import binding as lin
from weight_recurrent_memory_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _packed_inputs(lengths, H, dk, dv, dtype, seed, unit=False):
    T = int(sum(lengths))
    q, k, v = (x[0] for x in wl.la_inputs(1, H, T, dk, dv, dtype, seed=seed, device=DEV))
    if unit:
        q, k = wl.unit_rows(q.float()).to(dtype), wl.unit_rows(k.float()).to(dtype)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32)
    return q, k, v, cu


def _seq(x, cu, n):
    """Sequence n of a packed [H][T_total][...] tensor as a [1][H][T_n][...] one."""
    return x[:, int(cu[n]):int(cu[n + 1])][None]


LENGTHS = [
    [1],
    [64, 64, 64],
    [1, 63, 64, 65, 700, 3, 2000],
    [5000, 17, 900],
]


@pytest.mark.parametrize("lengths", LENGTHS)
@pytest.mark.parametrize("dk,dv,dtype", [(64, 64, torch.bfloat16), (128, 128, torch.bfloat16), (64, 64, torch.float32)])
def test_la_forward_packed_per_sequence(lengths, dk, dv, dtype):
    H, N = 2, len(lengths)
    print(f"la_forward_packed lengths={lengths} dk={dk} dv={dv} {dtype}", flush=True)
    q, k, v, cu = _packed_inputs(lengths, H, dk, dv, dtype, seed=sum(lengths))
    S0, z0 = wl.decode_state(N, H, dk, dv, seed=3, device=DEV, std=0.5)
    z0 = z0.abs()
    o, S, z = lin.la_forward_packed(q, k, v, cu.to(DEV), S0, z0, eps=EPS, cu_seqlens_host=cu)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    for n in range(N):
        ro, rS, rz = oracle.la_forward(_seq(q, cu, n), _seq(k, cu, n), _seq(v, cu, n), S0[n][None], z0[n][None], EPS)
        assert_parity(_seq(o, cu, n), ro, tol, f"o[{n}]", rows=True)
        assert_parity(S[n][None], rS, tol, f"S[{n}]")
        assert_parity(z[n][None], rz, tol, f"z[{n}]")


def test_la_forward_packed_isolation_and_many_sequences():
    """1500 sequences (the device segment table spans two scan tiles); a
    change inside one sequence changes nothing outside it, bit for bit."""
    rng = np.random.default_rng(7)
    lengths = rng.integers(1, 200, size=1500)
    H, d = 2, 64
    q, k, v, cu = _packed_inputs(lengths, H, d, d, torch.bfloat16, seed=8)
    o, S, z = lin.la_forward_packed(q, k, v, cu.to(DEV), eps=EPS, cu_seqlens_host=cu)
    v2 = v.clone()
    m = 777
    v2[:, int(cu[m]):int(cu[m + 1])] += 1.0
    o2, S2, z2 = lin.la_forward_packed(q, k, v2, cu.to(DEV), eps=EPS, cu_seqlens_host=cu)
    torch.cuda.synchronize()
    a, b = int(cu[m]), int(cu[m + 1])
    assert torch.equal(o2[:, :a], o[:, :a]) and torch.equal(o2[:, b:], o[:, b:])
    assert not torch.equal(o2[:, a:b], o[:, a:b])
    keep = [n for n in range(len(lengths)) if n != m]
    assert torch.equal(S2[keep], S[keep]) and torch.equal(z2[keep], z[keep])
    tol = TOL[torch.bfloat16]
    for n in (0, 1023, 1024, 1499, m):
        ro, rS, rz = oracle.la_forward(_seq(q, cu, n), _seq(k, cu, n), _seq(v, cu, n), eps=EPS)
        assert_parity(_seq(o, cu, n), ro, tol, f"o[{n}]", rows=True)
        assert_parity(S[n][None], rS, tol, f"S[{n}]")


@pytest.mark.parametrize("lengths", [[1, 63, 64, 65, 700, 3, 2000], [3000, 1, 129]])
@pytest.mark.parametrize("gated,norm,logits,pred", [(False, False, False, False), (True, True, True, True)])
def test_delta_forward_packed_per_sequence(lengths, gated, norm, logits, pred):
    H, d, N = 2, 128, len(lengths)
    print(f"delta_forward_packed lengths={lengths} gated={gated} options={norm, logits, pred}", flush=True)
    q, k, v, cu = _packed_inputs(lengths, H, d, d, torch.bfloat16, seed=11 + sum(lengths), unit=not norm)
    T = int(cu[-1])
    b = wl.la_inputs(1, H, T, 1, 1, torch.float32, seed=12, device=DEV)[0][0, ..., 0]
    b = (b if logits else torch.sigmoid(b)).to(torch.bfloat16)
    alpha = wl.gates((H, T), seed=13, device=DEV, rate=1 / 4) if gated else None
    S0, _ = wl.decode_state(N, H, d, d, seed=14, device=DEV, std=0.5)
    res = lin.delta_forward_packed(q, k, v, b, cu.to(DEV), alpha, S0, normalize_qk=norm, beta_logits=logits,
                                   return_pred=pred, cu_seqlens_host=cu)
    torch.cuda.synchronize()
    o, S = res[0], res[1]
    tol = TOL[torch.bfloat16]
    for n in range(N):
        sl = lambda x: x[:, int(cu[n]):int(cu[n + 1])][None]
        ro, rS, rp = oracle.delta_forward_ex(sl(q), sl(k), sl(v), sl(b), None if alpha is None else sl(alpha),
                                             S0[n][None], normalize_qk=norm, beta_logits=logits)
        assert_parity(sl(o), ro, tol, f"o[{n}]", rows=True, row_floor=1 / 8 if norm else 0.0)
        assert_parity(S[n][None], rS, tol, f"S[{n}]")
        if pred:
            # slice check only: the prediction is v - u (see test_gpu_delta_ex.PRED_NOTE)
            assert_parity(sl(res[2]), rp, tol, f"pred[{n}]")


@pytest.mark.parametrize("lengths", [[1, 63, 64, 65, 700, 3, 2000], [5000, 17]])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128)])
def test_ssd_forward_packed_per_sequence(lengths, dk, dv):
    H, N = 2, len(lengths)
    print(f"ssd_forward_packed lengths={lengths} dk={dk} dv={dv}", flush=True)
    q, k, v, cu = _packed_inputs(lengths, H, dk, dv, torch.bfloat16, seed=21 + sum(lengths))
    T = int(cu[-1])
    alpha = wl.gates((H, T), seed=22, device=DEV, rate=1 / 8)
    S0, _ = wl.decode_state(N, H, dk, dv, seed=23, device=DEV, std=0.5)
    o, S = lin.ssd_forward_packed(q, k, v, alpha, cu.to(DEV), S0, cu_seqlens_host=cu)
    torch.cuda.synchronize()
    tol = TOL[torch.bfloat16]
    for n in range(N):
        sl = lambda x: x[:, int(cu[n]):int(cu[n + 1])][None]
        ro, rS = oracle.ssd_forward(sl(q), sl(k), sl(v), sl(alpha), S0[n][None])
        assert_parity(sl(o), ro, tol, f"o[{n}]", rows=True)
        assert_parity(S[n][None], rS, tol, f"S[{n}]")


def test_packed_equal_lengths_match_the_uniform_calls():
    """Equal lengths: the packed call and the uniform call compute the same
    thing (their segment plans may differ, so within rounding)."""
    N, H, T, d = 3, 2, 1000, 64
    q, k, v = wl.la_inputs(N, H, T, d, d, torch.bfloat16, seed=31, device=DEV)
    pk = lambda x: x.permute(1, 0, 2, 3).reshape(H, N * T, x.shape[-1]).contiguous()
    cu = torch.arange(0, N * T + 1, T, dtype=torch.int32)
    o1, S1, z1 = lin.la_forward(q, k, v, eps=EPS)
    o2, S2, z2 = lin.la_forward_packed(pk(q), pk(k), pk(v), cu.to(DEV), eps=EPS, cu_seqlens_host=cu)
    torch.cuda.synchronize()
    tol = TOL[torch.bfloat16]
    assert_parity(o2[None], pk(o1).double().cpu().numpy()[None], tol, "o", rows=True)
    assert_parity(S2, S1.double().cpu().numpy(), tol, "S")
