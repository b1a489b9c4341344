"""Pins for the fp64 oracle (CPU only).

Each test ties the oracle to something other than itself: values the pages
print (fixtures under tests/golden/, each with its citation), closed forms,
brute-force forms on tiny inputs, and invariants.  Together they are chosen
so that a plausible mistake (dropped eps or z, read-before-write, a wrong
branch of the feature map, a transposed state, a wrong sign or a misplaced
beta in the delta correction) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from tests import forms

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def _h(x):
    """Add the batch and head axes: [T, d] -> [1, 1, T, d]."""
    return np.asarray(x, dtype=np.float64)[None, None]


def _la1(q, k, v, **kw):
    o, S, z = oracle.la_forward(_h(q), _h(k), _h(v), **kw)
    return o[0, 0], S[0, 0], z[0, 0]


def _delta1(q, k, v, beta, S0=None):
    o, S = oracle.delta_forward(_h(q), _h(k), _h(v), np.asarray(beta, dtype=np.float64)[None, None],
                                None if S0 is None else S0[None, None])
    return o[0, 0], S[0, 0]


# ----------------------------------------------------------------- feature map

def test_phi_values_printed_on_lassm_page():
    # "线性注意力与 SSM" §1.2: ELU(0)+1 = 1 and ELU(-3)+1 = e^-3 (about 0.05).
    y = oracle.phi([0.0, -3.0, 2.5, -0.0])
    assert y[0] == 1.0
    assert y[1] == math.exp(-3.0) and abs(y[1] - 0.05) < 0.001
    assert y[2] == 3.5          # positive branch: u + 1
    assert y[3] == 1.0


def test_phi_positive_everywhere():
    x = np.linspace(-700.0, 50.0, 10001)
    y = oracle.phi(x)
    assert np.all(y > 0)
    assert np.all(np.diff(y) > 0)  # strictly increasing through the branch change


# ------------------------------------------------- LinearMem printed seed-7 run

def _seed7_inputs():
    rng = np.random.default_rng(7)
    q = rng.normal(size=(8, 4))
    k = rng.normal(size=(8, 4))
    v = rng.normal(size=(8, 3))
    return q, k, v


def test_seed7_printed_run():
    g = _golden("linearmem_seed7_run.json")
    q, k, v = _seed7_inputs()
    o, S, z = _la1(q, k, v, eps=1e-6)
    assert list(o.shape) == g["output_shape"]
    assert list(S.shape) == g["state_shape"]
    assert list(z.shape) == g["normalizer_shape"]
    np.testing.assert_allclose(o[:2], np.array(g["first_two_outputs_8dp"]), rtol=0, atol=5.1e-9)
    assert abs(o.min() - g["output_min"]) <= 1e-14
    assert abs(o.max() - g["output_max"]) <= 1e-14
    # the page's own acceptance: explicit and recurrent agree below 1e-12
    assert np.max(np.abs(forms.la_quadratic(q, k, v) - o)) < 1e-12


def test_seed7_future_leak():
    g = _golden("linearmem_seed7_run.json")
    q, k, v = _seed7_inputs()
    o, _, _ = _la1(q, k, v)
    v2 = v.copy()
    v2[-1] += 100.0
    o2, _, _ = _la1(q, k, v2)
    assert float(np.max(np.abs(o2[:-1] - o[:-1]))) == g["future_leak_error"]
    assert np.max(np.abs(o2[-1] - o[-1])) > 1.0


# ------------------------------------------------------- LA brute force / forms

@pytest.mark.parametrize("T,dk,dv,seed,init", [
    (1, 4, 3, 0, False), (2, 3, 5, 1, False), (17, 8, 4, 2, False),
    (64, 16, 16, 3, False), (33, 5, 7, 4, True), (64, 8, 12, 5, True)])
def test_la_matches_quadratic_masked_form(T, dk, dv, seed, init):
    rng = np.random.default_rng(seed)
    q, k = rng.normal(size=(T, dk)), rng.normal(size=(T, dk))
    v = rng.normal(size=(T, dv))
    S0 = rng.normal(size=(dk, dv)) if init else None
    z0 = rng.uniform(0.5, 2.0, size=dk) if init else None
    o, S, z = _la1(q, k, v, S0=None if S0 is None else S0[None, None],
                   z0=None if z0 is None else z0[None, None])
    ref = forms.la_quadratic(q, k, v, S0, z0)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
    fk = forms.phi(k)
    S_ref = fk.T @ v + (0 if S0 is None else S0)
    z_ref = fk.sum(axis=0) + (0 if z0 is None else z0)
    np.testing.assert_allclose(S, S_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(z, z_ref, rtol=1e-12, atol=1e-12)


def test_la_single_token_closed_form_exposes_eps():
    # T = 1: o_1 = v_1 * w / (w + eps) with w = phi(q).phi(k).  With very
    # negative q and k, w is ~1e-10 and eps dominates the denominator.
    dk = 4
    q = np.full((1, dk), -12.0)
    k = np.full((1, dk), -12.0)
    v = np.array([[1.5, -2.0, 0.25]])
    w = dk * math.exp(-12.0) * math.exp(-12.0)
    o, _, _ = _la1(q, k, v, eps=1e-6)
    np.testing.assert_allclose(o[0], v[0] * w / (w + 1e-6), rtol=1e-13)
    assert abs(o[0, 0]) < 1e-3  # would be 1.5 without eps


def test_la_identical_keys_running_mean():
    # All keys equal: o_t = (sum_{i<=t} v_i) w / (t w + eps), w = phi(q_t).phi(k).
    rng = np.random.default_rng(11)
    T, dk, dv = 20, 6, 5
    q = rng.normal(size=(T, dk))
    k = np.tile(rng.normal(size=(1, dk)), (T, 1))
    v = rng.normal(size=(T, dv))
    o, _, _ = _la1(q, k, v)
    fk = np.array([x + 1 if x > 0 else math.exp(x) for x in k[0]])
    for t in range(T):
        fq = np.array([x + 1 if x > 0 else math.exp(x) for x in q[t]])
        w = float(fq @ fk)
        ref = v[:t + 1].sum(axis=0) * w / ((t + 1) * w + 1e-6)
        np.testing.assert_allclose(o[t], ref, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("T", [1, 7, 37])
def test_la_chunked_equals_recurrent_every_chunk_size(T):
    rng = np.random.default_rng(100 + T)
    dk, dv = 6, 5
    q, k = rng.normal(size=(T, dk)), rng.normal(size=(T, dk))
    v = rng.normal(size=(T, dv))
    S0, z0 = rng.normal(size=(dk, dv)), rng.uniform(0.5, 2.0, size=dk)
    o, S, z = _la1(q, k, v, S0=S0[None, None], z0=z0[None, None])
    for C in range(1, T + 1):
        oc, Sc, zc = forms.la_chunked(q, k, v, C, S0, z0)
        np.testing.assert_allclose(oc, o, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(Sc, S, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(zc, z, rtol=1e-12, atol=1e-12)


def test_la_causality_every_position():
    rng = np.random.default_rng(12)
    T, dk, dv = 24, 4, 3
    q, k, v = rng.normal(size=(T, dk)), rng.normal(size=(T, dk)), rng.normal(size=(T, dv))
    o, _, _ = _la1(q, k, v)
    for s in (0, 5, 23):
        for which in ("q", "k", "v"):
            qq, kk, vv = q.copy(), k.copy(), v.copy()
            {"q": qq, "k": kk, "v": vv}[which][s] += 100.0
            o2, _, _ = _la1(qq, kk, vv)
            assert np.array_equal(o2[:s], o[:s])
            assert not np.array_equal(o2[s], o[s])


def test_la_resume_equals_one_call():
    rng = np.random.default_rng(13)
    T, T1, dk, dv = 40, 17, 5, 6
    q, k, v = rng.normal(size=(T, dk)), rng.normal(size=(T, dk)), rng.normal(size=(T, dv))
    o, S, z = _la1(q, k, v)
    oa, Sa, za = _la1(q[:T1], k[:T1], v[:T1])
    ob, Sb, zb = _la1(q[T1:], k[T1:], v[T1:], S0=Sa[None, None], z0=za[None, None])
    np.testing.assert_allclose(np.concatenate([oa, ob]), o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(Sb, S, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(zb, z, rtol=1e-13, atol=1e-13)


def test_la_heads_are_independent():
    rng = np.random.default_rng(14)
    B, H, T, dk, dv = 2, 3, 9, 4, 5
    q, k = rng.normal(size=(B, H, T, dk)), rng.normal(size=(B, H, T, dk))
    v = rng.normal(size=(B, H, T, dv))
    o, S, z = oracle.la_forward(q, k, v)
    for b in range(B):
        for h in range(H):
            oh, Sh, zh = _la1(q[b, h], k[b, h], v[b, h])
            assert np.array_equal(oh, o[b, h]) and np.array_equal(Sh, S[b, h])
            assert np.array_equal(zh, z[b, h])


# ------------------------------------ additive memory worked examples (pages)

def test_additive_four_token_example_lassm():
    g = _golden("lassm_four_token_example.json")
    keys, values = np.array(g["keys"]), np.array(g["values"])
    for t in range(1, 5):
        _, S, _ = _la1(keys[:t], keys[:t], values[:t], feature=oracle.PHI_IDENTITY, normalize=False)
        np.testing.assert_allclose(S, np.array(g["additive_states_value_first"][t - 1]).T, atol=1e-15)
    # query with k_1 after all four writes
    q = keys.copy()
    q[-1] = keys[0]
    o, _, _ = _la1(q, keys, values, feature=oracle.PHI_IDENTITY, normalize=False)
    np.testing.assert_allclose(o[-1], g["additive_read_k1"], atol=1e-15)


def test_two_entry_example_memory_capacity():
    g = _golden("memory_capacity_two_entry.json")
    keys, values = np.array(g["keys"]), np.array(g["values"])
    q = np.array([keys[0], keys[0]])
    o, S, _ = _la1(q, keys, values, feature=oracle.PHI_IDENTITY, normalize=False)
    np.testing.assert_allclose(S, np.array(g["W_value_first"]).T, atol=1e-15)
    np.testing.assert_allclose(o[-1], g["read_A"], atol=1e-15)
    q = np.array([keys[1], keys[1]])
    o, _, _ = _la1(q, keys, values, feature=oracle.PHI_IDENTITY, normalize=False)
    np.testing.assert_allclose(o[-1], g["read_B"], atol=1e-15)


def test_memory_experiment_additive_same_key():
    g = _golden("linearmem_memory_experiment.json")
    key, values = np.array(g["key"]), np.array(g["values"])
    keys = np.array([key, key])
    o, _, _ = _la1(keys, keys, values, feature=oracle.PHI_IDENTITY, normalize=False)
    np.testing.assert_allclose(o[-1] / 2.0, g["additive_same_key_read_divided_by_writes"], atol=1e-15)


# ---------------------------------------------------------------- delta rule

def test_delta_four_token_example_lassm():
    g = _golden("lassm_four_token_example.json")
    keys, values = np.array(g["keys"]), np.array(g["values"])
    ones = np.ones(4)
    for t in range(1, 5):
        _, S = _delta1(keys[:t], keys[:t], values[:t], ones[:t])
        np.testing.assert_allclose(S, np.array(g["delta_states_value_first"][t - 1]).T, atol=1e-14)
    q = keys.copy()
    q[-1] = keys[0]
    o, _ = _delta1(q, keys, values, ones)
    np.testing.assert_allclose(o[-1], g["delta_read_k1"], atol=1e-14)


def test_memory_experiment_delta_same_key_and_half_beta():
    g = _golden("linearmem_memory_experiment.json")
    key, values = np.array(g["key"]), np.array(g["values"])
    keys = np.array([key, key])
    o, _ = _delta1(keys, keys, values, [1.0, 1.0])
    assert o[-1].tolist() == g["delta_same_key_read_beta1"]
    o, _ = _delta1(keys, keys, values, [0.5, 0.5])
    assert o[-1].tolist() == g["delta_same_key_read_beta_half"]


def test_memory_experiment_crosstalk():
    g = _golden("linearmem_memory_experiment.json")
    key, values = np.array(g["key"]), np.array(g["values"])
    for rho in g["crosstalk_rhos"]:
        k2 = np.array([rho, math.sqrt(1.0 - rho ** 2)])
        keys = np.array([key, k2])
        q = np.array([key, key])  # read the old key after both writes
        o, _ = _delta1(q, keys, values, [1.0, 1.0])
        np.testing.assert_allclose(o[-1], [1.0 - rho ** 2, rho], rtol=0, atol=2e-16)
        if rho == 0.9:
            assert o[-1][0] == g["crosstalk_rho_0.9_raw_first_component"]


def test_delta_exact_overwrite_bitwise_basis_keys():
    # LinearMem §03: with a unit key and beta = 1 the read of k_t right after the
    # write returns v_t.  Basis keys and dyadic values make it bit-exact.
    rng = np.random.default_rng(21)
    T, dk, dv = 32, 8, 6
    idx = rng.integers(0, dk, size=T)
    keys = np.eye(dk)[idx]
    values = rng.integers(-64, 64, size=(T, dv)) / 8.0
    S0 = rng.integers(-64, 64, size=(dk, dv)) / 16.0
    o, _ = _delta1(keys, keys, values, np.ones(T), S0=S0)
    assert np.array_equal(o, values)


def test_delta_overwrite_invariant_general_beta():
    # k_t^T S_t = (1 - beta_t) k_t^T S_{t-1} + beta_t v_t^T for unit k_t.
    rng = np.random.default_rng(22)
    T, dk, dv = 12, 5, 4
    k = rng.normal(size=(T, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    q, v = rng.normal(size=(T, dk)), rng.normal(size=(T, dv))
    beta = rng.uniform(0.05, 1.0, size=T)
    S0 = rng.normal(size=(dk, dv))
    prev = S0
    for t in range(1, T + 1):
        _, S = _delta1(q[:t], k[:t], v[:t], beta[:t], S0=S0)
        lhs = k[t - 1] @ S
        rhs = (1 - beta[t - 1]) * (k[t - 1] @ prev) + beta[t - 1] * v[t - 1]
        np.testing.assert_allclose(lhs, rhs, rtol=1e-13, atol=1e-14)
        prev = S
    o, _ = _delta1(k, k, v, np.ones(T), S0=S0)  # beta = 1: read returns v_t
    np.testing.assert_allclose(o, v, rtol=1e-13, atol=1e-13)


def test_delta_identical_key_is_ema():
    rng = np.random.default_rng(23)
    T, dk, dv, b = 30, 6, 3, 0.3
    key = rng.normal(size=dk)
    key /= np.linalg.norm(key)
    keys = np.tile(key, (T, 1))
    v = rng.normal(size=(T, dv))
    o, _ = _delta1(keys, keys, v, np.full(T, b))
    ema = np.zeros(dv)
    for t in range(T):
        ema = (1 - b) * ema + b * v[t]
        np.testing.assert_allclose(o[t], ema, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("T,dk,dv,seed,init", [
    (1, 4, 3, 0, False), (9, 3, 5, 1, True), (64, 16, 8, 2, False), (48, 8, 8, 3, True)])
def test_delta_matches_dense_triangular_solve(T, dk, dv, seed, init):
    rng = np.random.default_rng(seed)
    k = rng.normal(size=(T, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    q, v = rng.normal(size=(T, dk)), rng.normal(size=(T, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.normal(size=T)))
    S0 = rng.normal(size=(dk, dv)) if init else None
    o, S = _delta1(q, k, v, beta, S0=S0)
    O_ref, S_ref = forms.delta_dense(q, k, v, beta, S0)
    np.testing.assert_allclose(o, O_ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(S, S_ref, rtol=1e-11, atol=1e-12)


def test_delta_orthonormal_keys_reduce_to_additive():
    rng = np.random.default_rng(24)
    dk, dv, T = 8, 5, 8
    Qm, _ = np.linalg.qr(rng.normal(size=(dk, dk)))
    keys = Qm.T[:T]
    q, v = rng.normal(size=(T, dk)), rng.normal(size=(T, dv))
    od, Sd = _delta1(q, keys, v, np.ones(T))
    oa, Sa, _ = _la1(q, keys, v, feature=oracle.PHI_IDENTITY, normalize=False)
    np.testing.assert_allclose(Sd, Sa, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(od, oa, rtol=1e-12, atol=1e-13)


def test_delta_repeated_sweeps_reach_least_squares_w_star():
    # memory-capacity page: for the two-entry example the least-squares write is
    # W* = [[1, -0.75], [0, 1.25]]; repeated beta = 1 delta sweeps over the two
    # pairs (Kaczmarz projections) converge to it.
    g = _golden("memory_capacity_two_entry.json")
    keys, values = np.array(g["keys"]), np.array(g["values"])
    sweeps = 200
    K = np.tile(keys, (sweeps, 1))
    V = np.tile(values, (sweeps, 1))
    _, S = _delta1(K, K, V, np.ones(2 * sweeps))
    np.testing.assert_allclose(S, np.array(g["least_squares_W_star_value_first"]).T, atol=1e-12)


@pytest.mark.parametrize("T", [1, 6, 29])
def test_delta_chunked_equals_recurrent_every_chunk_size(T):
    rng = np.random.default_rng(200 + T)
    dk, dv = 6, 4
    k = rng.normal(size=(T, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    q, v = rng.normal(size=(T, dk)), rng.normal(size=(T, dv))
    beta = rng.uniform(0.0, 1.0, size=T)
    S0 = rng.normal(size=(dk, dv))
    o, S = _delta1(q, k, v, beta, S0=S0)
    for C in range(1, T + 1):
        oc, Sc = forms.delta_chunked(q, k, v, beta, C, S0)
        np.testing.assert_allclose(oc, o, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(Sc, S, rtol=1e-11, atol=1e-12)


def test_delta_causality_and_resume():
    rng = np.random.default_rng(25)
    T, dk, dv = 20, 4, 3
    k = rng.normal(size=(T, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    q, v, beta = rng.normal(size=(T, dk)), rng.normal(size=(T, dv)), rng.uniform(size=T)
    o, S = _delta1(q, k, v, beta)
    for s in (0, 9, 19):
        vv = v.copy()
        vv[s] += 100.0
        o2, _ = _delta1(q, k, vv, beta)
        assert np.array_equal(o2[:s], o[:s]) and not np.array_equal(o2[s], o[s])
    T1 = 7
    oa, Sa = _delta1(q[:T1], k[:T1], v[:T1], beta[:T1])
    ob, Sb = _delta1(q[T1:], k[T1:], v[T1:], beta[T1:], S0=Sa)
    np.testing.assert_allclose(np.concatenate([oa, ob]), o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(Sb, S, rtol=1e-13, atol=1e-14)


# -------------------------------------------------------------------- decode

def test_decode_step_equals_one_token_of_forward():
    rng = np.random.default_rng(31)
    N, H, dk, dv = 3, 2, 8, 6
    S0 = rng.normal(scale=0.01, size=(N, H, dk, dv))
    z0 = rng.normal(scale=0.01, size=(N, H, dk))
    q, k, v = rng.normal(size=(N, H, dk)), rng.normal(size=(N, H, dk)), rng.normal(size=(N, H, dv))
    o, S, z = oracle.la_decode_step(q, k, v, S0, z0)
    of, Sf, zf = oracle.la_forward(q[:, :, None], k[:, :, None], v[:, :, None], S0=S0, z0=z0)
    np.testing.assert_allclose(o, of[:, :, 0], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(S, Sf, rtol=1e-15, atol=1e-16)
    np.testing.assert_allclose(z, zf, rtol=1e-15, atol=1e-16)


def test_decode_chain_equals_forward_over_the_same_tokens():
    rng = np.random.default_rng(32)
    N, H, dk, dv, steps = 2, 2, 4, 3, 25
    S = rng.normal(scale=0.01, size=(N, H, dk, dv))
    z = rng.normal(scale=0.01, size=(N, H, dk))
    q, k = rng.normal(size=(steps, N, H, dk)), rng.normal(size=(steps, N, H, dk))
    v = rng.normal(size=(steps, N, H, dv))
    of, Sf, zf = oracle.la_forward(q.transpose(1, 2, 0, 3), k.transpose(1, 2, 0, 3),
                                   v.transpose(1, 2, 0, 3), S0=S, z0=z)
    outs = []
    for t in range(steps):
        o, S, z = oracle.la_decode_step(q[t], k[t], v[t], S, z)
        outs.append(o)
    np.testing.assert_allclose(np.stack(outs, 2), of, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S, Sf, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(z, zf, rtol=1e-12, atol=1e-13)


def _dstep(q, k, v, beta, S):
    """One delta decode step on a single state: vectors -> (o, S)."""
    o, S = oracle.delta_decode_step(np.asarray(q, float)[None, None], np.asarray(k, float)[None, None],
                                    np.asarray(v, float)[None, None], np.array([[beta]], float),
                                    np.asarray(S, float)[None, None])
    return o[0, 0], S[0, 0]


def test_delta_decode_four_token_example_lassm():
    # LA-SSM page §1.3: the delta rule with beta = 1 over four tokens, every
    # intermediate state printed (value-first there, hence the transposes).
    g = _golden("lassm_four_token_example.json")
    keys, values = np.array(g["keys"]), np.array(g["values"])
    S = np.zeros((2, 2))
    for t in range(4):
        q = keys[0] if t == 3 else keys[t]
        o, S = _dstep(q, keys[t], values[t], 1.0, S)
        np.testing.assert_allclose(S, np.array(g["delta_states_value_first"][t]).T, atol=1e-14)
    np.testing.assert_allclose(o, g["delta_read_k1"], atol=1e-14)


def test_delta_decode_exact_overwrite_and_zero_beta():
    # Unit (basis) key with beta = 1: reading the same key right after the
    # write returns the new value exactly; beta = 0 leaves the state alone.
    rng = np.random.default_rng(41)
    dk, dv = 8, 5
    S0 = rng.integers(-64, 64, size=(dk, dv)) / 16.0
    for i in range(dk):
        key = np.eye(dk)[i]
        val = rng.integers(-64, 64, size=dv) / 8.0
        o, S1 = _dstep(key, key, val, 1.0, S0)
        assert np.array_equal(o, val)
        assert np.array_equal(np.delete(S1, i, axis=0), np.delete(S0, i, axis=0))
        q = rng.normal(size=dk)
        o0, S2 = _dstep(q, rng.normal(size=dk), rng.normal(size=dv), 0.0, S0)
        assert np.array_equal(S2, S0)
        np.testing.assert_allclose(o0, S0.T @ q, rtol=1e-15, atol=1e-15)


def test_delta_decode_chain_equals_forward_over_the_same_tokens():
    rng = np.random.default_rng(42)
    N, H, dk, dv, steps = 2, 3, 5, 4, 30
    S = rng.normal(scale=0.1, size=(N, H, dk, dv))
    k = rng.normal(size=(steps, N, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q, v = rng.normal(size=(steps, N, H, dk)), rng.normal(size=(steps, N, H, dv))
    beta = rng.uniform(0.0, 1.0, size=(steps, N, H))
    of, Sf = oracle.delta_forward(q.transpose(1, 2, 0, 3), k.transpose(1, 2, 0, 3), v.transpose(1, 2, 0, 3),
                                  beta.transpose(1, 2, 0), S0=S)
    outs = []
    for t in range(steps):
        o, S = oracle.delta_decode_step(q[t], k[t], v[t], beta[t], S)
        outs.append(o)
    np.testing.assert_allclose(np.stack(outs, 2), of, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S, Sf, rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------- gated delta

def _gdelta1(q, k, v, beta, alpha, S0=None):
    o, S = oracle.gated_delta_forward(_h(q), _h(k), _h(v), np.asarray(beta, dtype=np.float64)[None, None],
                                      np.asarray(alpha, dtype=np.float64)[None, None],
                                      None if S0 is None else S0[None, None])
    return o[0, 0], S[0, 0]


def test_gated_delta_gate_reads_printed_on_linearmem():
    # LinearMem §06 / §09: identity state, write key (1, 0) -> value (0, 1)
    # with beta = 1 and forgetting factor alpha, then read the orthogonal key
    # (0, 1): [0, 0.8] for alpha = 0.8, [0, 1] for alpha = 1.
    g = _golden("linearmem_memory_experiment.json")
    key, values = np.array(g["key"]), np.array(g["values"])
    q = np.array([0.0, 1.0])
    for alpha, want in ((0.8, g["gated_unrelated_key_read_alpha_0.8"]), (1.0, g["gated_unrelated_key_read_alpha_1"])):
        o, _ = _gdelta1([q], [key], [values[1]], [1.0], [alpha], S0=np.eye(2))
        np.testing.assert_allclose(o[0], want, atol=1e-15)
        od, _ = oracle.gated_delta_decode_step(q[None, None], key[None, None], values[1][None, None],
                                               np.ones((1, 1)), np.full((1, 1), alpha), np.eye(2)[None, None])
        np.testing.assert_allclose(od[0, 0], want, atol=1e-15)


def test_gated_delta_alpha_one_is_the_delta_rule_bitwise():
    rng = np.random.default_rng(51)
    B, H, T, dk, dv = 2, 2, 40, 6, 5
    q, k, v = rng.normal(size=(B, H, T, dk)), rng.normal(size=(B, H, T, dk)), rng.normal(size=(B, H, T, dv))
    beta = rng.uniform(size=(B, H, T))
    S0 = rng.normal(size=(B, H, dk, dv))
    o1, S1 = oracle.delta_forward(q, k, v, beta, S0)
    o2, S2 = oracle.gated_delta_forward(q, k, v, beta, np.ones((B, H, T)), S0)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


def test_gated_delta_zero_beta_is_pure_decay():
    rng = np.random.default_rng(52)
    T, dk, dv = 20, 4, 3
    q, k, v = rng.normal(size=(T, dk)), rng.normal(size=(T, dk)), rng.normal(size=(T, dv))
    alpha = rng.uniform(0.5, 1.0, size=T)
    S0 = rng.normal(size=(dk, dv))
    o, S = _gdelta1(q, k, v, np.zeros(T), alpha, S0=S0)
    g = np.cumprod(alpha)
    np.testing.assert_allclose(S, g[-1] * S0, rtol=1e-13)
    np.testing.assert_allclose(o, g[:, None] * (q @ S0), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("T,dk,dv,seed,init", [(1, 3, 2, 1, False), (17, 5, 4, 2, True), (64, 8, 8, 3, True)])
def test_gated_delta_matches_dense_form(T, dk, dv, seed, init):
    rng = np.random.default_rng(60 + seed)
    k = rng.normal(size=(T, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    q, v = rng.normal(size=(T, dk)), rng.normal(size=(T, dv))
    beta, alpha = rng.uniform(size=T), rng.uniform(0.6, 1.0, size=T)
    S0 = rng.normal(size=(dk, dv)) if init else None
    o, S = _gdelta1(q, k, v, beta, alpha, S0=S0)
    rO, rS = forms.gated_delta_dense(q, k, v, beta, alpha, S0)
    np.testing.assert_allclose(o, rO, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(S, rS, rtol=1e-10, atol=1e-12)


def test_gated_delta_decay_comes_before_the_correction():
    # The page: decay first, then the error against the decayed state; the
    # other order is a different rule.  Exact overwrite holds only for the
    # page's order: with a unit basis key and beta = 1 the key reads back its
    # new value whatever alpha is (dyadic values, bit-exact).
    rng = np.random.default_rng(53)
    dk, dv = 6, 4
    S0 = rng.integers(-64, 64, size=(dk, dv)) / 16.0
    key = np.eye(dk)[2]
    val = rng.integers(-64, 64, size=dv) / 8.0
    o, S = _gdelta1([key], [key], [val], [1.0], [0.5], S0=S0)
    assert np.array_equal(o[0], val)
    other = 0.5 * (S0 + np.outer(key, val - key @ S0))  # correct first, then decay
    assert not np.allclose(S, other)


def test_gated_delta_decode_chain_equals_forward():
    rng = np.random.default_rng(54)
    N, H, dk, dv, steps = 2, 2, 5, 4, 30
    S = rng.normal(scale=0.1, size=(N, H, dk, dv))
    k = rng.normal(size=(steps, N, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q, v = rng.normal(size=(steps, N, H, dk)), rng.normal(size=(steps, N, H, dv))
    beta, alpha = rng.uniform(size=(steps, N, H)), rng.uniform(0.7, 1.0, size=(steps, N, H))
    tr = lambda x: x.transpose(1, 2, 0, 3) if x.ndim == 4 else x.transpose(1, 2, 0)
    of, Sf = oracle.gated_delta_forward(tr(q), tr(k), tr(v), tr(beta), tr(alpha), S0=S)
    outs = []
    for t in range(steps):
        o, S = oracle.gated_delta_decode_step(q[t], k[t], v[t], beta[t], alpha[t], S)
        outs.append(o)
    np.testing.assert_allclose(np.stack(outs, 2), of, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S, Sf, rtol=1e-12, atol=1e-13)


# ------------------------------------------------------- scalar decay (SSD)

def _ssd1(q, k, v, alpha, S0=None):
    o, S = oracle.ssd_forward(_h(q), _h(k), _h(v), np.asarray(alpha, dtype=np.float64)[None, None],
                              None if S0 is None else S0[None, None])
    return o[0, 0], S[0, 0]


def test_ssd_scalar_case_is_the_explicit_mixing_matrix():
    # "手撕：递推与记忆模型" "Selective scan": with h_t = a_t h_{t-1} + b_t x_t and
    # y_t = c_t h_t, output j weighs input i (i <= j) by c_j b_i prod_{i<s<=j} a_s.
    # d_k = d_v = 1 maps a -> alpha, b -> k, x -> v, c -> q.
    rng = np.random.default_rng(70)
    T = 6
    a = 1.0 / (1.0 + np.exp(-rng.normal(size=T)))
    b, c, x = rng.normal(size=T), rng.normal(size=T), rng.normal(size=T)
    M = np.zeros((T, T))
    for j in range(T):
        for i in range(j + 1):
            w = c[j] * b[i]
            for s in range(i + 1, j + 1):
                w *= a[s]
            M[j, i] = w
    o, S = _ssd1(c[:, None], b[:, None], x[:, None], a)
    np.testing.assert_allclose(o[:, 0], M @ x, rtol=1e-13, atol=1e-15)
    # the final state is the last output divided by its read weight
    np.testing.assert_allclose(S[0, 0] * c[-1], (M @ x)[-1], rtol=1e-13)


@pytest.mark.parametrize("T,dk,dv,seed", [(1, 3, 2, 1), (9, 4, 5, 2), (40, 6, 3, 3)])
def test_ssd_is_the_sum_of_decayed_outer_products(T, dk, dv, seed):
    # S_t = (prod_{s<=t} alpha_s) S_0 + sum_{i<=t} (prod_{i<s<=t} alpha_s) k_i v_i^T
    rng = np.random.default_rng(80 + seed)
    q, k, v = rng.normal(size=(T, dk)), rng.normal(size=(T, dk)), rng.normal(size=(T, dv))
    alpha = rng.uniform(0.3, 1.0, size=T)
    S0 = rng.normal(size=(dk, dv))
    o, S = _ssd1(q, k, v, alpha, S0=S0)
    for t in range(T):
        St = np.prod(alpha[:t + 1]) * S0
        for i in range(t + 1):
            St = St + np.prod(alpha[i + 1:t + 1]) * np.outer(k[i], v[i])
        np.testing.assert_allclose(o[t], q[t] @ St, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S, St, rtol=1e-12, atol=1e-13)


def test_ssd_alpha_one_is_the_additive_memory_bitwise():
    rng = np.random.default_rng(71)
    B, H, T, dk, dv = 2, 2, 30, 5, 4
    q, k, v = rng.normal(size=(B, H, T, dk)), rng.normal(size=(B, H, T, dk)), rng.normal(size=(B, H, T, dv))
    S0 = rng.normal(size=(B, H, dk, dv))
    o1, S1 = oracle.ssd_forward(q, k, v, np.ones((B, H, T)), S0)
    o2, S2, _ = oracle.la_forward(q, k, v, S0=S0, feature=oracle.PHI_IDENTITY, normalize=False)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


def test_ssd_chunked_scan_equals_one_pass():
    # "手撕：递推与记忆模型" "Chunked scan": only the final state crosses a chunk
    # boundary; the chunked run equals the full run.
    rng = np.random.default_rng(72)
    B, H, T, dk, dv = 1, 3, 23, 4, 4
    q, k, v = rng.normal(size=(B, H, T, dk)), rng.normal(size=(B, H, T, dk)), rng.normal(size=(B, H, T, dv))
    alpha = rng.uniform(0.2, 1.0, size=(B, H, T))
    full, Sf = oracle.ssd_forward(q, k, v, alpha)
    outs, S = [], None
    for s in range(0, T, 4):
        o, S = oracle.ssd_forward(q[:, :, s:s + 4], k[:, :, s:s + 4], v[:, :, s:s + 4], alpha[:, :, s:s + 4], S)
        outs.append(o)
    assert np.array_equal(np.concatenate(outs, 2), full) and np.array_equal(S, Sf)


def test_ssd_decay_reaches_an_orthogonal_key_linearmem():
    # LinearMem §06: decay scales the whole state, including maps of keys
    # orthogonal to the one written: identity state, alpha = 0.8, write key
    # (1, 0) -> (0, 1), read (0, 1) -> [0, 0.8].  The write term adds
    # (k . q) v = 0, so the scalar-decay rule gives the page's read too.
    g = _golden("linearmem_memory_experiment.json")
    o, S = _ssd1([[0.0, 1.0]], [g["key"]], [g["values"][1]], [0.8], S0=np.eye(2))
    np.testing.assert_allclose(o[0], g["gated_unrelated_key_read_alpha_0.8"], atol=1e-15)


def test_ssd_decode_chain_equals_forward_and_zero_alpha_resets():
    rng = np.random.default_rng(73)
    N, H, dk, dv, steps = 2, 2, 4, 3, 25
    S = rng.normal(size=(N, H, dk, dv))
    q, k, v = rng.normal(size=(steps, N, H, dk)), rng.normal(size=(steps, N, H, dk)), rng.normal(size=(steps, N, H, dv))
    alpha = rng.uniform(0.5, 1.0, size=(steps, N, H))
    tr = lambda x: x.transpose(1, 2, 0, 3) if x.ndim == 4 else x.transpose(1, 2, 0)
    of, Sf = oracle.ssd_forward(tr(q), tr(k), tr(v), tr(alpha), S0=S)
    outs = []
    for t in range(steps):
        o, S = oracle.ssd_decode_step(q[t], k[t], v[t], alpha[t], S)
        outs.append(o)
    np.testing.assert_allclose(np.stack(outs, 2), of, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S, Sf, rtol=1e-12, atol=1e-13)
    o, S2 = oracle.ssd_decode_step(q[0], k[0], v[0], np.zeros((N, H)), S)
    assert np.array_equal(S2, k[0][..., :, None] * v[0][..., None, :])


# ------------------------------------------- input transforms and predictions

def test_l2_normalize_rows_closed_forms():
    y = oracle.l2_normalize_rows(np.array([[3.0, 4.0], [0.0, 0.0], [-5.0, 12.0]]))
    np.testing.assert_allclose(y, [[0.6, 0.8], [0.0, 0.0], [-5 / 13, 12 / 13]], rtol=1e-15, atol=0)
    x = np.random.default_rng(90).normal(size=(50, 17)) * np.arange(1, 51)[:, None]
    y = oracle.l2_normalize_rows(x)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), 1.0, rtol=1e-14)
    assert np.all(np.sign(y) == np.sign(x))


def test_sigmoid_closed_forms():
    x = np.array([0.0, math.log(3.0), -math.log(3.0), 40.0, -40.0])
    y = oracle.sigmoid(x)
    np.testing.assert_allclose(y[:3], [0.5, 0.75, 0.25], rtol=1e-15)
    assert abs(y[3] - 1.0) < 1e-16 and 0.0 < y[4] < 1e-17
    xs = np.random.default_rng(91).normal(size=100) * 5
    np.testing.assert_allclose(oracle.sigmoid(xs) + oracle.sigmoid(-xs), 1.0, rtol=1e-15)
    assert np.all(np.diff(oracle.sigmoid(np.sort(xs))) >= 0)


def test_delta_predictions_printed_lassm():
    # LA-SSM §1.3: before each write the walk-through prints the prediction
    # S_{t-1} k_t and the correction u_t (beta = 1, four tokens).
    g = _golden("lassm_four_token_example.json")
    keys, values = np.array(g["keys"]), np.array(g["values"])
    o, S, pred = oracle.delta_forward_ex(_h(keys), _h(keys), _h(values), np.ones((1, 1, 4)))
    np.testing.assert_allclose(pred[0, 0], g["delta_predictions"], atol=1e-14)
    np.testing.assert_allclose(values - pred[0, 0], g["delta_corrections"], atol=1e-14)
    # the same through the step form
    St = np.zeros((1, 1, 2, 2))
    for t in range(4):
        _, St, p = oracle.delta_decode_step_ex(keys[t][None, None], keys[t][None, None], values[t][None, None],
                                               np.ones((1, 1)), St)
        np.testing.assert_allclose(p[0, 0], g["delta_predictions"][t], atol=1e-14)


def test_delta_prediction_recalls_a_basis_key_exactly():
    # A basis key written with beta = 1 stores its value exactly; writing the
    # same key later first predicts that value, bit for bit.
    rng = np.random.default_rng(92)
    dk, dv = 6, 4
    keys = np.eye(dk)[[2, 4, 2]]
    values = rng.integers(-64, 64, size=(3, dv)) / 8.0
    _, _, pred = oracle.delta_forward_ex(_h(keys), _h(keys), _h(values), np.ones((1, 1, 3)))
    assert np.array_equal(pred[0, 0, 2], values[0])
    assert np.array_equal(pred[0, 0, 1], np.zeros(dv))


def test_gated_prediction_reads_the_decayed_state():
    # LinearMem gate setup: identity state, alpha = 0.8, key (1, 0): the
    # prediction is taken from the decayed state, 0.8 k^T I = [0.8, 0].
    g = _golden("linearmem_memory_experiment.json")
    k = np.array(g["key"])[None, None, None]
    v = np.array(g["values"][1])[None, None, None]
    _, _, pred = oracle.delta_forward_ex(k, k, v, np.ones((1, 1, 1)), alpha=np.full((1, 1, 1), 0.8),
                                         S0=np.eye(2)[None, None])
    np.testing.assert_allclose(pred[0, 0, 0], [0.8, 0.0], rtol=1e-15)


def test_transform_flags_reduce_to_the_plain_rule():
    rng = np.random.default_rng(93)
    B, H, T, dk, dv = 1, 2, 20, 5, 3
    q, k, v = rng.normal(size=(B, H, T, dk)) * 3, rng.normal(size=(B, H, T, dk)) * 2, rng.normal(size=(B, H, T, dv))
    logits = rng.normal(size=(B, H, T))
    alpha = rng.uniform(0.5, 1.0, size=(B, H, T))
    o, S, pred = oracle.delta_forward_ex(q, k, v, logits, alpha=alpha, normalize_qk=True, beta_logits=True)
    qn, kn = oracle.l2_normalize_rows(q), oracle.l2_normalize_rows(k)
    o2, S2 = oracle.gated_delta_forward(qn, kn, v, oracle.sigmoid(logits), alpha)
    assert np.array_equal(o, o2) and np.array_equal(S, S2)
    # from a zero state the first prediction is zero
    _, _, p3 = oracle.delta_forward_ex(qn[:, :, :1], kn[:, :, :1], v[:, :, :1], np.ones((B, H, 1)))
    assert np.array_equal(p3, np.zeros_like(p3))


# ------------------------------------------------------------------- backward

def _la_loss(q, k, v, S0, z0, dO, dS_T, dz_T, feature, normalize, eps=1e-6):
    o, S, z = oracle.la_forward(q, k, v, S0, z0, eps, feature=feature, normalize=normalize)
    return float(np.sum(dO * o) + np.sum(dS_T * S) + np.sum(dz_T * z))


@pytest.mark.parametrize("feature,normalize", [(oracle.PHI_ELU1, True), (oracle.PHI_IDENTITY, False),
                                               (oracle.PHI_ELU1, False)])
def test_la_backward_matches_central_differences(feature, normalize):
    # Every gradient entry against (L(x + h) - L(x - h)) / 2h of the forward
    # oracle, with a random linear loss on o, S_T and z_T.
    rng = np.random.default_rng(100 + feature + 2 * normalize)
    B, H, T, dk, dv = 1, 2, 9, 3, 4
    q, k, v = rng.normal(size=(B, H, T, dk)), rng.normal(size=(B, H, T, dk)), rng.normal(size=(B, H, T, dv))
    S0, z0 = rng.normal(size=(B, H, dk, dv)), rng.uniform(0.1, 1.0, size=(B, H, dk))
    dO, dS_T, dz_T = rng.normal(size=(B, H, T, dv)), rng.normal(size=(B, H, dk, dv)), rng.normal(size=(B, H, dk))
    grads = oracle.la_backward(q, k, v, dO, S0, z0, dS_T, dz_T, feature=feature, normalize=normalize)
    inputs = [q, k, v, S0, z0]
    h = 1e-6
    for which, (x, g) in enumerate(zip(inputs, grads)):
        fd = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + h
            lp = _la_loss(*inputs, dO, dS_T, dz_T, feature, normalize)
            x[idx] = keep - h
            lm = _la_loss(*inputs, dO, dS_T, dz_T, feature, normalize)
            x[idx] = keep
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-7, err_msg=f"input {which}")


def test_la_backward_value_gradient_is_the_adjoint_of_the_additive_map():
    # Identity map, no normaliser: o_t = S0^T q_t + sum_{i<=t} (q_t . k_i) v_i,
    # a linear map of v, so dv_i = sum_{t>=i} (q_t . k_i) dO_t (brute force).
    rng = np.random.default_rng(104)
    T, dk, dv = 15, 5, 3
    q, k, v, dO = rng.normal(size=(T, dk)), rng.normal(size=(T, dk)), rng.normal(size=(T, dv)), rng.normal(size=(T, dv))
    _, _, dvv, _, _ = oracle.la_backward(_h(q), _h(k), _h(v), _h(dO), feature=oracle.PHI_IDENTITY, normalize=False)
    want = np.zeros((T, dv))
    for i in range(T):
        for t in range(i, T):
            want[i] += (q[t] @ k[i]) * dO[t]
    np.testing.assert_allclose(dvv[0, 0], want, rtol=1e-12, atol=1e-13)


def test_la_backward_single_token_closed_form():
    # T = 1, normalised: o = phi(q)^T (S0 + phi(k) v^T) / (phi(q) . (z0 + phi(k)) + eps),
    # so dv_j = (phi(q) . phi(k)) dO_j / den, dS0 = phi(q) dO^T / den and
    # dz0 = -phi(q) (dO . num) / den^2.
    rng = np.random.default_rng(105)
    dk, dv, eps = 4, 3, 1e-6
    q, k, v, dO = rng.normal(size=dk), rng.normal(size=dk), rng.normal(size=dv), rng.normal(size=dv)
    S0, z0 = rng.normal(size=(dk, dv)), rng.uniform(0.2, 1.0, size=dk)
    fq, fk = oracle.phi(q), oracle.phi(k)
    den = fq @ (z0 + fk) + eps
    _, _, dvv, dS0, dz0 = oracle.la_backward(_h([q]), _h([k]), _h([v]), _h([dO]), S0[None, None], z0[None, None], eps=eps)
    np.testing.assert_allclose(dvv[0, 0, 0], (fq @ fk) * dO / den, rtol=1e-13)
    num = fq @ (S0 + np.outer(fk, v))
    np.testing.assert_allclose(dS0[0, 0], np.outer(fq, dO) / den, rtol=1e-13)
    np.testing.assert_allclose(dz0[0, 0], -fq * (dO @ num) / den ** 2, rtol=1e-12)


def _delta_loss(q, k, v, beta, alpha, S0, dO, dS_T):
    if alpha is None:
        o, S = oracle.delta_forward(q, k, v, beta, S0)
    else:
        o, S = oracle.gated_delta_forward(q, k, v, beta, alpha, S0)
    return float(np.sum(dO * o) + np.sum(dS_T * S))


def _unit_rows(x, norm):
    return norm * x / np.linalg.norm(x, axis=-1, keepdims=True)


@pytest.mark.parametrize("gated", [False, True])
def test_delta_backward_matches_central_differences(gated):
    # Every gradient entry against (L(x + h) - L(x - h)) / 2h of the forward
    # oracle; T = 70 crosses the backward's 64-token recomputation blocks.
    rng = np.random.default_rng(110 + gated)
    B, H, T, dk, dv = 1, 2, 70, 3, 4
    q = rng.normal(size=(B, H, T, dk))
    k = _unit_rows(rng.normal(size=(B, H, T, dk)), 0.9)
    v = rng.normal(size=(B, H, T, dv))
    beta = rng.uniform(0.1, 0.9, size=(B, H, T))
    alpha = rng.uniform(0.8, 1.0, size=(B, H, T)) if gated else None
    S0 = rng.normal(size=(B, H, dk, dv))
    dO, dS_T = rng.normal(size=(B, H, T, dv)), rng.normal(size=(B, H, dk, dv))
    dq, dkk, dvv, dbeta, dalpha, dS0 = oracle.delta_backward(q, k, v, beta, dO, alpha, S0, dS_T)
    assert (dalpha is None) == (not gated)
    cases = [(q, dq), (k, dkk), (v, dvv), (beta, dbeta), (S0, dS0)] + ([(alpha, dalpha)] if gated else [])
    h = 1e-6
    for which, (x, g) in enumerate(cases):
        fd = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + h
            lp = _delta_loss(q, k, v, beta, alpha, S0, dO, dS_T)
            x[idx] = keep - h
            lm = _delta_loss(q, k, v, beta, alpha, S0, dO, dS_T)
            x[idx] = keep
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g, fd, rtol=1e-5, atol=1e-6, err_msg=f"input {which}")


def test_delta_backward_orthonormal_keys_value_gradient_is_the_additive_adjoint():
    # Orthonormal keys from a zero state: every correction reads zero, so
    # o_t = sum_{i<=t} beta_i (q_t . k_i) v_i and dv_i = beta_i sum_{t>=i} (q_t . k_i) dO_t.
    rng = np.random.default_rng(112)
    T, dk, dv = 6, 6, 3
    k, _ = np.linalg.qr(rng.normal(size=(dk, dk)))
    k = k.T[:T]
    q, v, dO = rng.normal(size=(T, dk)), rng.normal(size=(T, dv)), rng.normal(size=(T, dv))
    beta = rng.uniform(0.2, 1.0, size=T)
    _, _, dvv, dbeta, _, _ = oracle.delta_backward(_h(q), _h(k), _h(v), beta[None, None], _h(dO))
    want = np.zeros((T, dv))
    for i in range(T):
        for t in range(i, T):
            want[i] += beta[i] * (q[t] @ k[i]) * dO[t]
    np.testing.assert_allclose(dvv[0, 0], want, rtol=1e-12, atol=1e-13)
    # and dbeta_i = sum_{t>=i} (q_t . k_i) (v_i . dO_t)
    wb = np.array([sum((q[t] @ k[i]) * (v[i] @ dO[t]) for t in range(i, T)) for i in range(T)])
    np.testing.assert_allclose(dbeta[0, 0], wb, rtol=1e-12, atol=1e-13)


def test_delta_backward_single_token_closed_form():
    # T = 1: S_1 = a (I - b k k^T) S0 + b k v^T, o = S_1^T q, L = dO . o.
    rng = np.random.default_rng(113)
    dk, dv = 4, 3
    q, k, v, dO = rng.normal(size=dk), rng.normal(size=dk), rng.normal(size=dv), rng.normal(size=dv)
    S0 = rng.normal(size=(dk, dv))
    a, b = 0.7, 0.4
    P = np.eye(dk) - b * np.outer(k, k)
    S1 = a * P @ S0 + b * np.outer(k, v)
    u = v - a * S0.T @ k
    dq, _, dvv, dbeta, dalpha, dS0 = oracle.delta_backward(
        _h([q]), _h([k]), _h([v]), np.array([[[b]]]), _h([dO]), np.array([[[a]]]), S0[None, None])
    np.testing.assert_allclose(dq[0, 0, 0], S1 @ dO, rtol=1e-13)
    np.testing.assert_allclose(dvv[0, 0, 0], b * (q @ k) * dO, rtol=1e-13)
    np.testing.assert_allclose(dbeta[0, 0, 0], (q @ k) * (u @ dO), rtol=1e-12)
    np.testing.assert_allclose(dalpha[0, 0, 0], q @ P @ S0 @ dO, rtol=1e-12)
    np.testing.assert_allclose(dS0[0, 0], a * np.outer(P @ q, dO), rtol=1e-12, atol=1e-14)
