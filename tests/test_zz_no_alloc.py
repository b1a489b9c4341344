"""la_forward_noalloc (the fixed per-GPU scratch in place of a workspace)
through the C ABI: its results must equal la_forward's bit for bit (same
kernels, same plan), on consecutive calls that reuse the scratch, the second
smaller than the first."""
import pytest
import torch

from tests.parity import EPS
from weight_recurrent_memory_amd import binding as lin
from weight_recurrent_memory_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(B, H, T, seed, init):
    q, k, v = wl.la_inputs(B, H, T, 64, 64, torch.bfloat16, seed=seed, device=DEV)
    S0 = z0 = None
    if init:
        S0, z0 = wl.decode_state(B, H, 64, 64, seed=seed + 1, device=DEV, std=0.5)
        z0 = z0.abs() + 1.0
    return q, k, v, S0, z0


@pytest.mark.parametrize("shapes", [[(1, 32, 65536, False), (2, 3, 5000, True)],
                                    [(4, 8, 8192, True), (1, 1, 130, False)]])
def test_noalloc_equals_la_forward_on_consecutive_calls(shapes):
    for B, H, T, init in shapes:
        print(f"la_forward_noalloc B={B} H={H} T={T} init={init}", flush=True)
        q, k, v, S0, z0 = _inputs(B, H, T, seed=B * 100 + H + T, init=init)
        ref = lin.la_forward(q, k, v, S0, z0, eps=EPS)
        got = lin.la_forward_noalloc(q, k, v, S0, z0, eps=EPS)
        torch.cuda.synchronize()
        for name, g, r in zip(("o", "S", "z"), got, ref):
            assert torch.equal(g, r), name


@pytest.mark.parametrize("chunk", [16, 128])
def test_noalloc_equals_la_forward_at_other_chunk_sizes(chunk):
    # the blocked path on the scratch: segment sums and entering states
    q, k, v, S0, z0 = _inputs(2, 3, 5000, seed=chunk, init=True)
    ref = lin.la_forward(q, k, v, S0, z0, eps=EPS, chunk=chunk)
    got = lin.la_forward_noalloc(q, k, v, S0, z0, eps=EPS, chunk=chunk)
    torch.cuda.synchronize()
    for name, g, r in zip(("o", "S", "z"), got, ref):
        assert torch.equal(g, r), name


def test_noalloc_in_place_continuation():
    q, k, v, S0, z0 = _inputs(2, 16, 5100, seed=5, init=True)
    ref = lin.la_forward(q, k, v, S0.clone(), z0.clone(), eps=EPS)
    S, z = S0.clone(), z0.clone()
    o, _, _ = lin.la_forward_noalloc(q, k, v, S, z, eps=EPS, S_out=S, z_out=z)
    torch.cuda.synchronize()
    assert torch.equal(o, ref[0]) and torch.equal(S, ref[1]) and torch.equal(z, ref[2])


def test_noalloc_refuses_sizes_beyond_the_scratch():
    q = torch.zeros((1, 64, 65536, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(lin.UnsupportedError, match="scratch"):
        lin.la_forward_noalloc(q, q, q, eps=EPS)
