"""GPU parity and structure tests of la_forward (through the C ABI)."""
import numpy as np
import pytest
import torch

import oracle
from tests.parity import EPS, TOL, assert_parity, to64
from weight_recurrent_memory_amd import binding as lin
from weight_recurrent_memory_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run(q, k, v, S0=None, z0=None):
    o, S, z = lin.la_forward(q, k, v, S0, z0, eps=EPS)
    torch.cuda.synchronize()
    return o, S, z


def _check(q, k, v, o, S, z, S0=None, z0=None, heads=None):
    """Oracle on (a sample of) the heads; compare o, S_T, z_T."""
    tol = TOL[q.dtype]
    B, H = q.shape[:2]
    flat = lambda t: None if t is None else t.reshape(B * H, *t.shape[2:])
    qf, kf, vf, of, Sf, zf, S0f, z0f = map(flat, (q, k, v, o, S, z, S0, z0))
    idx = list(range(B * H)) if heads is None else list(heads)
    sel = lambda t: None if t is None else t[idx][None]
    ro, rS, rz = oracle.la_forward(sel(qf), sel(kf), sel(vf), sel(S0f), sel(z0f), eps=EPS)
    e1 = assert_parity(sel(of), ro, tol, "o", rows=True)
    e2 = assert_parity(sel(Sf), rS, tol, "S_T")
    e3 = assert_parity(sel(zf), rz, tol, "z_T")
    print(f"worst slice errors: o {e1:.2e}  S {e2:.2e}  z {e3:.2e}")


SHAPES = [
    # B, H, T, dk, dv, dtype, with initial state
    (1, 1, 1, 64, 64, torch.bfloat16, False),
    (1, 2, 2, 64, 64, torch.float32, False),
    (2, 1, 63, 64, 64, torch.bfloat16, True),
    (1, 1, 64, 64, 128, torch.bfloat16, False),
    (1, 3, 65, 128, 64, torch.bfloat16, True),
    (1, 1, 200, 128, 128, torch.bfloat16, True),
    (2, 2, 1000, 64, 64, torch.float32, True),
    (1, 1, 777, 64, 128, torch.float32, False),
    (1, 1, 333, 128, 64, torch.float32, True),
    (3, 5, 4099, 64, 64, torch.bfloat16, True),
]


@pytest.mark.parametrize("B,H,T,dk,dv,dtype,init", SHAPES)
def test_la_small_shapes(B, H, T, dk, dv, dtype, init):
    print(f"la_forward B={B} H={H} T={T} dk={dk} dv={dv} {dtype} init={init}", flush=True)
    q, k, v = wl.la_inputs(B, H, T, dk, dv, dtype, seed=1000 + T, device=DEV)
    S0 = z0 = None
    if init:
        S0, z0 = wl.decode_state(B, H, dk, dv, seed=77, device=DEV, std=0.5)
        z0 = z0.abs() + 1.0
    o, S, z = _run(q, k, v, S0, z0)
    _check(q, k, v, o, S, z, S0, z0)


# 32 (sequence, head) pairs with lengths that give segments of 2, 3, 5, 6 and 7
# chunks (the plan takes chunks x heads / 512 chunks per segment): the
# aggregate pass takes whole groups of four chunks from the segment end, the
# first four chunks stay in registers for the output pass, and the last
# segment of each sequence is shorter still.
@pytest.mark.parametrize("T,init", [(2500, False), (3500, True), (5100, False), (6500, True), (7900, False)])
def test_la_segment_lengths(T, init):
    B, H = 2, 16
    print(f"la_forward B={B} H={H} T={T} init={init}", flush=True)
    q, k, v = wl.la_inputs(B, H, T, 64, 64, torch.bfloat16, seed=4000 + T, device=DEV)
    S0 = z0 = None
    if init:
        S0, z0 = wl.decode_state(B, H, 64, 64, seed=78, device=DEV, std=0.5)
        z0 = z0.abs() + 1.0
    o, S, z = _run(q, k, v, S0, z0)
    _check(q, k, v, o, S, z, S0, z0)


def test_la_fp32_config_full():
    w = wl.LA_FP32_SMALL
    print(f"la_forward {w.name}", flush=True)
    q, k, v = wl.make(w, DEV)
    o, S, z = _run(q, k, v)
    _check(q, k, v, o, S, z)


@pytest.mark.parametrize("w", [wl.LA_BF16_PREFILL, wl.LA_BF16_LONG])
def test_la_bf16_configs_all_heads(w):
    print(f"la_forward {w.name}, every head", flush=True)
    q, k, v = wl.make(w, DEV)
    o, S, z = _run(q, k, v)
    _check(q, k, v, o, S, z)


def test_la_causality_bitwise():
    q, k, v = wl.la_inputs(1, 2, 300, 64, 64, torch.bfloat16, seed=5, device=DEV)
    o, _, _ = _run(q, k, v)
    for s in (0, 63, 64, 100, 299):
        for name in ("q", "k", "v"):
            t = {"q": q, "k": k, "v": v}
            pert = t[name].clone()
            pert[:, :, s] += 3.0
            t = dict(t, **{name: pert})
            o2, _, _ = _run(t["q"], t["k"], t["v"])
            assert torch.equal(o2[:, :, :s], o[:, :, :s]), (name, s)
            if not (name == "q" and s == 0):  # o_0 = v_0 w / (w + eps) barely depends on q_0
                assert not torch.equal(o2[:, :, s:], o[:, :, s:]), (name, s)


def test_la_deterministic():
    # Segments find their incoming state by look-back over whatever their
    # predecessors have published so far; the sum order is fixed regardless,
    # so repeated runs are bitwise identical.
    for shape in ((2, 4, 3000), (1, 32, 8192)):
        q, k, v = wl.la_inputs(*shape, 64, 64, torch.bfloat16, seed=6, device=DEV)
        a = _run(q, k, v)
        for _ in range(4):
            b = _run(q, k, v)
            for x, y in zip(a, b):
                assert torch.equal(x, y)


def test_la_resume_matches_single_call():
    q, k, v = wl.la_inputs(1, 4, 2000, 64, 64, torch.float32, seed=7, device=DEV)
    o, S, z = _run(q, k, v)
    T1 = 777
    oa, Sa, za = _run(q[:, :, :T1].contiguous(), k[:, :, :T1].contiguous(), v[:, :, :T1].contiguous())
    ob, Sb, zb = _run(q[:, :, T1:].contiguous(), k[:, :, T1:].contiguous(), v[:, :, T1:].contiguous(), Sa, za)
    tol = TOL[torch.float32]
    assert_parity(torch.cat([oa, ob], 2), to64(o), tol, "o", rows=True)
    assert_parity(Sb, to64(S), tol, "S")
    assert_parity(zb, to64(z), tol, "z")


def test_la_state_out_may_alias_state_in():
    q, k, v = wl.la_inputs(1, 2, 500, 64, 64, torch.bfloat16, seed=8, device=DEV)
    S0, z0 = wl.decode_state(1, 2, 64, 64, seed=9, device=DEV)
    z0 = z0.abs() + 1.0
    ref = _run(q, k, v, S0.clone(), z0.clone())
    S, z = S0.clone(), z0.clone()
    o, _, _ = lin.la_forward(q, k, v, S, z, eps=EPS, S_out=S, z_out=z)
    torch.cuda.synchronize()
    assert torch.equal(o, ref[0]) and torch.equal(S, ref[1]) and torch.equal(z, ref[2])


def test_la_heads_isolated_and_plan_independent():
    # the same head alone (one head: many segments) and among 32 heads (fewer
    # segments per head) gives the same answer within tolerance; perturbing
    # another head changes nothing in it.
    q, k, v = wl.la_inputs(1, 32, 4096, 64, 64, torch.bfloat16, seed=10, device=DEV)
    o, S, z = _run(q, k, v)
    o1, S1, z1 = _run(q[:, 5:6].contiguous(), k[:, 5:6].contiguous(), v[:, 5:6].contiguous())
    tol = TOL[torch.bfloat16]
    assert_parity(o1, to64(o[:, 5:6]), tol, "o", rows=True)
    assert_parity(S1, to64(S[:, 5:6]), tol, "S")
    v2 = v.clone()
    v2[:, 6] += 1.0
    o2, S2, _ = _run(q, k, v2)
    assert torch.equal(o2[:, :6], o[:, :6]) and torch.equal(o2[:, 7:], o[:, 7:])
    assert torch.equal(S2[:, :6], S[:, :6])


def test_la_workspace_leftovers_ignored():
    """Look-back flags carry a per-call tag: whatever an earlier call (or other
    data) left in the workspace must not change the result."""
    B, H, T, dk, dv = 2, 3, 5000, 64, 64
    print(f"la_forward workspace reuse B={B} H={H} T={T}", flush=True)
    qa, ka, va = wl.la_inputs(B, H, T, dk, dv, torch.bfloat16, seed=31, device=DEV)
    qb, kb, vb = wl.la_inputs(B, H, T, dk, dv, torch.bfloat16, seed=32, device=DEV)
    nb = lin.la_forward_workspace_bytes(B, H, T, dk, dv)
    ref = lin.la_forward(qb, kb, vb, eps=EPS, workspace=torch.zeros(nb, dtype=torch.uint8, device=DEV))
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    for fill in (0xFF, 0x01, None):
        if fill is None:
            ws.copy_(torch.randint(0, 256, (nb,), dtype=torch.uint8, device=DEV))
        else:
            ws.fill_(fill)
        lin.la_forward(qa, ka, va, eps=EPS, workspace=ws)  # leaves its flags and states
        got = lin.la_forward(qb, kb, vb, eps=EPS, workspace=ws)
        torch.cuda.synchronize()
        for g, r in zip(got, ref):
            assert torch.equal(g, r)


def test_la_graph_replays_match_eager():
    """A la_forward recorded into a graph (one tag for every replay) clears its
    flags in-graph; each replay, with eager calls on the same workspace in
    between, must equal the eager result for its inputs."""
    B, H, T, dk, dv = 1, 4, 3000, 64, 64
    print(f"la_forward graph replay B={B} H={H} T={T}", flush=True)
    sets = [wl.la_inputs(B, H, T, dk, dv, torch.bfloat16, seed=40 + i, device=DEV) for i in range(3)]
    nb = lin.la_forward_workspace_bytes(B, H, T, dk, dv)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    sq, sk, sv = (t.clone() for t in sets[0])
    o = torch.empty((B, H, T, dv), dtype=torch.bfloat16, device=DEV)
    S = torch.empty((B, H, dk, dv), dtype=torch.float32, device=DEV)
    z = torch.empty((B, H, dk), dtype=torch.float32, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside capture
        lin.la_forward(sq, sk, sv, eps=EPS, o=o, S_out=S, z_out=z, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lin.la_forward(sq, sk, sv, eps=EPS, o=o, S_out=S, z_out=z, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(6):
        q, k, v = sets[rep % 3]
        want = lin.la_forward(q, k, v, eps=EPS, workspace=torch.empty(nb, dtype=torch.uint8, device=DEV))
        lin.la_forward(*sets[(rep + 1) % 3], eps=EPS, workspace=ws)  # eager use of the graph's workspace
        sq.copy_(q), sk.copy_(k), sv.copy_(v)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, ref in zip((o, S, z), want):
            assert torch.equal(got, ref), f"replay {rep}"


@pytest.mark.parametrize("polls", [-1, 0, 1])
@pytest.mark.parametrize("init,alias", [(False, False), (True, False), (True, True)])
def test_la_lookback_give_up_path_is_bitwise_equal(polls, init, alias):
    """With the look-back's wait bound forced to (almost) nothing, later
    segments recompute their incoming state from the inputs; the sum is taken
    in the look-back's own order, so every output and the final state must
    equal the normal call bit for bit -- also when S_out, z_out alias S0, z0
    (the recomputation reads the initial state while the last segment may be
    writing the final one)."""
    B, H, T = 2, 16, 5100  # 16 segments of 5 chunks per sequence
    print(f"la_forward give-up path polls={polls} init={init} alias={alias}", flush=True)
    q, k, v = wl.la_inputs(B, H, T, 64, 64, torch.bfloat16, seed=90, device=DEV)
    S0 = z0 = None
    if init:
        S0, z0 = wl.decode_state(B, H, 64, 64, seed=91, device=DEV, std=0.5)
        z0 = z0.abs() + 1.0
    ref = _run(q, k, v, None if S0 is None else S0.clone(), None if z0 is None else z0.clone())
    if alias:
        S, z = S0.clone(), z0.clone()
        o, _, _ = lin.la_forward(q, k, v, S, z, eps=EPS, S_out=S, z_out=z, lookback_polls=polls)
    else:
        o, S, z = lin.la_forward(q, k, v, S0, z0, eps=EPS, lookback_polls=polls)
    torch.cuda.synchronize()
    assert torch.equal(o, ref[0]) and torch.equal(S, ref[1]) and torch.equal(z, ref[2])
    if polls == -1 and not alias:
        _check(q, k, v, o, S, z, S0, z0)
