"""The C ABI on the CPU: the library loads, exports every symbol the header
declares, and rejects invalid arguments before touching the device.

No case here reaches a kernel launch: each call carries at least one argument
that validation rejects (fake but aligned pointers are never dereferenced).
"""
import ctypes
import os
import re

import pytest

from weight_recurrent_memory_amd import binding as lin

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "linattn.h")
P = ctypes.c_void_p(0x10000)  # aligned, never dereferenced
ST = {n: i for i, n in enumerate(["OK", "INVALID_ARG", "UNSUPPORTED", "WORKSPACE", "HIP"])}


def _declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)))


def test_header_declares_the_operations():
    fns = _declared_functions()
    for name in ("la_forward", "delta_forward", "la_decode_step", "delta_decode_step", "gated_delta_forward",
                 "gated_delta_decode_step", "ssd_forward", "ssd_decode_step", "delta_forward_ex",
                 "delta_decode_step_ex", "la_forward_packed", "delta_forward_packed", "ssd_forward_packed",
                 "la_backward", "delta_backward", "delta_forward_train", "delta_backward_after_forward"):
        assert name in fns


def test_library_exports_every_declared_symbol():
    L = lin.lib()
    for name in _declared_functions():
        assert hasattr(L, name), name


def _la(**kw):
    a = dict(q=P, k=P, v=P, S0=None, z0=None, o=P, S_out=None, z_out=None, B=1, H=1, T=8, dk=64, dv=64,
             dtype=1, eps=1e-6, chunk=64, ws=P, wsb=1 << 30, stream=None)
    a.update(kw)
    return lin.lib().la_forward(a["q"], a["k"], a["v"], a["S0"], a["z0"], a["o"], a["S_out"], a["z_out"],
                                a["B"], a["H"], a["T"], a["dk"], a["dv"], a["dtype"], a["eps"], a["chunk"],
                                a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), "INVALID_ARG"), (dict(o=None), "INVALID_ARG"), (dict(T=0), "INVALID_ARG"),
    (dict(B=-1), "INVALID_ARG"), (dict(dk=0), "INVALID_ARG"), (dict(chunk=0), "INVALID_ARG"),
    (dict(eps=0.0), "INVALID_ARG"), (dict(eps=-1.0), "INVALID_ARG"), (dict(eps=float("nan")), "INVALID_ARG"),
    (dict(eps=float("inf")), "INVALID_ARG"), (dict(dtype=7), "INVALID_ARG"),
    (dict(dk=96), "UNSUPPORTED"), (dict(dv=32), "UNSUPPORTED"), (dict(chunk=48), "UNSUPPORTED"),
    (dict(chunk=256), "UNSUPPORTED"), (dict(chunk=8), "UNSUPPORTED"), (dict(chunk=128, dtype=0), "UNSUPPORTED"),
    (dict(dtype=0, dk=128, dv=128), "UNSUPPORTED"),
    (dict(q=ctypes.c_void_p(0x10002)), "INVALID_ARG"),
    (dict(ws=None), "WORKSPACE"), (dict(wsb=16), "WORKSPACE"), (dict(ws=ctypes.c_void_p(0x10004)), "WORKSPACE"),
])
def test_la_forward_rejects(kw, status):
    assert _la(**kw) == ST[status]
    assert lin.lib().la_last_error().decode()


def _delta(**kw):
    a = dict(q=P, k=P, v=P, beta=P, S0=None, o=P, S_out=None, B=1, H=1, T=8, dk=128, dv=128, dtype=1,
             chunk=64, ws=P, wsb=1 << 30, stream=None)
    a.update(kw)
    return lin.lib().delta_forward(a["q"], a["k"], a["v"], a["beta"], a["S0"], a["o"], a["S_out"], a["B"],
                                   a["H"], a["T"], a["dk"], a["dv"], a["dtype"], a["chunk"], a["ws"],
                                   a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(beta=None), "INVALID_ARG"), (dict(T=0), "INVALID_ARG"), (dict(chunk=-3), "INVALID_ARG"),
    (dict(dtype=3), "INVALID_ARG"), (dict(dk=100), "UNSUPPORTED"), (dict(dtype=0), "UNSUPPORTED"),
    (dict(chunk=48), "UNSUPPORTED"), (dict(chunk=256), "UNSUPPORTED"),
    (dict(ws=None), "WORKSPACE"), (dict(wsb=0), "WORKSPACE"),
])
def test_delta_forward_rejects(kw, status):
    assert _delta(**kw) == ST[status]


def _dec(**kw):
    a = dict(q=P, k=P, v=P, S=P, z=P, o=P, N=4, H=2, dk=128, dv=128, dtype=1, eps=1e-6, stream=None)
    a.update(kw)
    if "eps_only" in a:
        a["eps"] = a.pop("eps_only")
    return lin.lib().la_decode_step(a["q"], a["k"], a["v"], a["S"], a["z"], a["o"], a["N"], a["H"], a["dk"],
                                    a["dv"], a["dtype"], a["eps"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(S=None), "INVALID_ARG"), (dict(z=None), "INVALID_ARG"), (dict(N=0), "INVALID_ARG"),
    (dict(eps=0.0), "INVALID_ARG"), (dict(dtype=2), "INVALID_ARG"), (dict(dk=48), "UNSUPPORTED"),
    (dict(S=ctypes.c_void_p(0x10008)), "INVALID_ARG"),
])
def test_decode_rejects(kw, status):
    assert _dec(**kw) == ST[status]


def _ddec(**kw):
    a = dict(q=P, k=P, v=P, beta=P, S=P, o=P, N=4, H=2, dk=128, dv=128, dtype=1, stream=None)
    a.update(kw)
    return lin.lib().delta_decode_step(a["q"], a["k"], a["v"], a["beta"], a["S"], a["o"], a["N"], a["H"],
                                       a["dk"], a["dv"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(beta=None), "INVALID_ARG"), (dict(S=None), "INVALID_ARG"), (dict(o=None), "INVALID_ARG"),
    (dict(H=0), "INVALID_ARG"), (dict(dtype=5), "INVALID_ARG"), (dict(dv=96), "UNSUPPORTED"),
    (dict(S=ctypes.c_void_p(0x10004)), "INVALID_ARG"),
])
def test_delta_decode_rejects(kw, status):
    assert _ddec(**kw) == ST[status]
    assert lin.lib().la_last_error().decode()


def _gdelta(**kw):
    a = dict(q=P, k=P, v=P, beta=P, alpha=P, S0=None, o=P, S_out=None, B=1, H=1, T=8, dk=128, dv=128, dtype=1,
             chunk=64, ws=P, wsb=1 << 30, stream=None)
    a.update(kw)
    return lin.lib().gated_delta_forward(a["q"], a["k"], a["v"], a["beta"], a["alpha"], a["S0"], a["o"],
                                         a["S_out"], a["B"], a["H"], a["T"], a["dk"], a["dv"], a["dtype"],
                                         a["chunk"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(alpha=None), "INVALID_ARG"), (dict(beta=None), "INVALID_ARG"), (dict(T=0), "INVALID_ARG"),
    (dict(alpha=ctypes.c_void_p(0x10002)), "INVALID_ARG"), (dict(dk=100), "UNSUPPORTED"),
    (dict(dtype=0), "UNSUPPORTED"), (dict(chunk=32), "UNSUPPORTED"),  # other chunk sizes: the plain rule only
    (dict(ws=None), "WORKSPACE"), (dict(wsb=0), "WORKSPACE"),
])
def test_gated_delta_forward_rejects(kw, status):
    assert _gdelta(**kw) == ST[status]
    assert lin.lib().la_last_error().decode().startswith("gated_delta_forward")


def _gddec(**kw):
    a = dict(q=P, k=P, v=P, beta=P, alpha=P, S=P, o=P, N=4, H=2, dk=128, dv=128, dtype=1, stream=None)
    a.update(kw)
    return lin.lib().gated_delta_decode_step(a["q"], a["k"], a["v"], a["beta"], a["alpha"], a["S"], a["o"],
                                             a["N"], a["H"], a["dk"], a["dv"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(alpha=None), "INVALID_ARG"), (dict(S=None), "INVALID_ARG"), (dict(N=0), "INVALID_ARG"),
    (dict(dtype=5), "INVALID_ARG"), (dict(dk=32), "UNSUPPORTED"), (dict(S=ctypes.c_void_p(0x10004)), "INVALID_ARG"),
])
def test_gated_delta_decode_rejects(kw, status):
    assert _gddec(**kw) == ST[status]
    assert lin.lib().la_last_error().decode().startswith("gated_delta_decode_step")


def _ssd(**kw):
    a = dict(q=P, k=P, v=P, alpha=P, S0=None, o=P, S_out=None, B=1, H=1, T=8, dk=64, dv=64, dtype=1, chunk=64,
             ws=P, wsb=1 << 30, stream=None)
    a.update(kw)
    return lin.lib().ssd_forward(a["q"], a["k"], a["v"], a["alpha"], a["S0"], a["o"], a["S_out"], a["B"], a["H"],
                                 a["T"], a["dk"], a["dv"], a["dtype"], a["chunk"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(alpha=None), "INVALID_ARG"), (dict(q=None), "INVALID_ARG"), (dict(H=0), "INVALID_ARG"),
    (dict(alpha=ctypes.c_void_p(0x10002)), "INVALID_ARG"), (dict(S0=ctypes.c_void_p(0x10004)), "INVALID_ARG"),
    (dict(dv=100), "UNSUPPORTED"), (dict(dtype=0), "UNSUPPORTED"), (dict(chunk=128), "UNSUPPORTED"),
    (dict(ws=None), "WORKSPACE"), (dict(wsb=8), "WORKSPACE"),
])
def test_ssd_forward_rejects(kw, status):
    assert _ssd(**kw) == ST[status]
    assert lin.lib().la_last_error().decode().startswith("ssd_forward")


def _ssd_dec(**kw):
    a = dict(q=P, k=P, v=P, alpha=P, S=P, o=P, N=4, H=2, dk=128, dv=128, dtype=1, stream=None)
    a.update(kw)
    return lin.lib().ssd_decode_step(a["q"], a["k"], a["v"], a["alpha"], a["S"], a["o"], a["N"], a["H"], a["dk"],
                                     a["dv"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(alpha=None), "INVALID_ARG"), (dict(S=None), "INVALID_ARG"), (dict(N=0), "INVALID_ARG"),
    (dict(dtype=9), "INVALID_ARG"), (dict(dk=256), "UNSUPPORTED"), (dict(S=ctypes.c_void_p(0x10008)), "INVALID_ARG"),
])
def test_ssd_decode_rejects(kw, status):
    assert _ssd_dec(**kw) == ST[status]
    assert lin.lib().la_last_error().decode().startswith("ssd_decode_step")


def _dex(**kw):
    a = dict(q=P, k=P, v=P, beta=P, alpha=None, S0=None, o=P, S_out=None, pred=None, flags=3, B=1, H=1, T=8, dk=128,
             dv=128, dtype=1, chunk=64, ws=P, wsb=1 << 30, stream=None)
    a.update(kw)
    return lin.lib().delta_forward_ex(a["q"], a["k"], a["v"], a["beta"], a["alpha"], a["S0"], a["o"], a["S_out"],
                                      a["pred"], a["flags"], a["B"], a["H"], a["T"], a["dk"], a["dv"], a["dtype"],
                                      a["chunk"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(flags=4), "INVALID_ARG"), (dict(flags=-1), "INVALID_ARG"), (dict(beta=None), "INVALID_ARG"),
    (dict(pred=ctypes.c_void_p(0x10001)), "INVALID_ARG"), (dict(T=0), "INVALID_ARG"), (dict(dk=32), "UNSUPPORTED"),
    (dict(dtype=0), "UNSUPPORTED"), (dict(chunk=16), "UNSUPPORTED"), (dict(chunk=128, flags=0, pred=P), "UNSUPPORTED"),
    (dict(ws=None), "WORKSPACE"),
])
def test_delta_forward_ex_rejects(kw, status):
    assert _dex(**kw) == ST[status]
    assert lin.lib().la_last_error().decode().startswith("delta_forward_ex")


def _ddex(**kw):
    a = dict(q=P, k=P, v=P, beta=P, alpha=None, S=P, o=P, pred=None, flags=1, N=4, H=2, dk=128, dv=128, dtype=1,
             stream=None)
    a.update(kw)
    return lin.lib().delta_decode_step_ex(a["q"], a["k"], a["v"], a["beta"], a["alpha"], a["S"], a["o"], a["pred"],
                                          a["flags"], a["N"], a["H"], a["dk"], a["dv"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(flags=8), "INVALID_ARG"), (dict(beta=None), "INVALID_ARG"), (dict(S=None), "INVALID_ARG"),
    (dict(N=0), "INVALID_ARG"), (dict(dv=48), "UNSUPPORTED"),
])
def test_delta_decode_step_ex_rejects(kw, status):
    assert _ddex(**kw) == ST[status]
    assert lin.lib().la_last_error().decode().startswith("delta_decode_step_ex")


def _packed_la(cu_host, **kw):
    host = (ctypes.c_int * len(cu_host))(*cu_host)
    a = dict(q=P, k=P, v=P, cu=P, N=len(cu_host) - 1, S0=None, z0=None, o=P, S_out=None, z_out=None, H=2,
             T=cu_host[-1], dk=64, dv=64, dtype=1, eps=1e-6, chunk=64, ws=P, wsb=1 << 30, stream=None)
    a.update(kw)
    return lin.lib().la_forward_packed(a["q"], a["k"], a["v"], a["cu"], ctypes.cast(host, ctypes.c_void_p), a["N"],
                                       a["S0"], a["z0"], a["o"], a["S_out"], a["z_out"], a["H"], a["T"], a["dk"],
                                       a["dv"], a["dtype"], a["eps"], a["chunk"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("cu_host,kw,status", [
    ([1, 5, 9], {}, "INVALID_ARG"),              # does not start at 0
    ([0, 5, 5, 9], {}, "INVALID_ARG"),           # an empty sequence
    ([0, 6, 4, 9], {}, "INVALID_ARG"),           # decreasing
    ([0, 5, 9], dict(T=10), "INVALID_ARG"),      # last offset is not T_total
    ([0, 5, 9], dict(cu=None), "INVALID_ARG"),   # no device offsets
    ([0, 5, 9], dict(cu=ctypes.c_void_p(0x10002)), "INVALID_ARG"),
    ([0, 5, 9], dict(N=0), "INVALID_ARG"),
    ([0, 5, 9], dict(dk=96), "UNSUPPORTED"),
    ([0, 5, 9], dict(chunk=32), "UNSUPPORTED"),  # other chunk sizes: uniform batches only
    ([0, 5, 9], dict(ws=None), "WORKSPACE"),
])
def test_la_forward_packed_rejects(cu_host, kw, status):
    assert _packed_la(cu_host, **kw) == ST[status]
    assert lin.lib().la_last_error().decode().startswith("la_forward_packed")


def test_packed_workspace_queries_and_rejects():
    L = lin.lib()
    for fn in (L.la_forward_packed_workspace_bytes, L.delta_forward_packed_workspace_bytes,
               L.ssd_forward_packed_workspace_bytes):
        good = (ctypes.c_int * 4)(0, 100, 3000, 3001)
        assert fn(ctypes.cast(good, ctypes.c_void_p), 3, 8, 3001, 128, 128, 64) > 0
        bad = (ctypes.c_int * 4)(0, 100, 100, 3001)
        assert fn(ctypes.cast(bad, ctypes.c_void_p), 3, 8, 3001, 128, 128, 64) == 0
        assert fn(None, 3, 8, 3001, 128, 128, 64) == 0
    cu = (ctypes.c_int * 3)(0, 5, 9)
    h = ctypes.cast(cu, ctypes.c_void_p)
    assert L.delta_forward_packed(P, P, P, P, None, P, h, 2, None, P, None, None, 4, 2, 9, 128, 128, 1, 64, P,
                                  1 << 30, None) == ST["INVALID_ARG"]  # unknown flags
    assert L.ssd_forward_packed(P, P, P, None, P, h, 2, None, P, None, 2, 9, 64, 64, 1, 64, P, 1 << 30,
                                None) == ST["INVALID_ARG"]  # alpha NULL


def _lab(**kw):
    a = dict(q=P, k=P, v=P, S0=None, z0=None, dO=P, dS_T=None, dz_T=None, dq=P, dk_out=P, dv_out=P, dS0=None,
             dz0=None, B=1, H=1, T=8, dk=64, dv=64, dtype=1, eps=1e-6, chunk=64, ws=P, wsb=1 << 30, stream=None)
    a.update(kw)
    return lin.lib().la_backward(a["q"], a["k"], a["v"], a["S0"], a["z0"], a["dO"], a["dS_T"], a["dz_T"], a["dq"],
                                 a["dk_out"], a["dv_out"], a["dS0"], a["dz0"], a["B"], a["H"], a["T"], a["dk"],
                                 a["dv"], a["dtype"], a["eps"], a["chunk"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(dO=None), "INVALID_ARG"), (dict(dq=None), "INVALID_ARG"), (dict(T=0), "INVALID_ARG"),
    (dict(eps=0.0), "INVALID_ARG"), (dict(dtype=5), "INVALID_ARG"), (dict(dtype=0), "UNSUPPORTED"),
    (dict(dk=96), "UNSUPPORTED"), (dict(dv_out=ctypes.c_void_p(0x10002)), "INVALID_ARG"),
    (dict(ws=None), "WORKSPACE"), (dict(wsb=64), "WORKSPACE"),
])
def test_la_backward_rejects(kw, status):
    assert _lab(**kw) == ST[status]
    assert lin.lib().la_last_error().decode().startswith("la_backward")


def _dlb(entry="delta_backward", **kw):
    a = dict(q=P, k=P, v=P, beta=P, alpha=None, S0=None, dO=P, dS_T=None, dq=P, dk_out=P, dv_out=P, dbeta=P,
             dalpha=None, dS0=None, B=1, H=1, T=8, dk=128, dv=128, dtype=1, chunk=64, ws=P, wsb=1 << 30,
             stream=None)
    a.update(kw)
    return getattr(lin.lib(), entry)(a["q"], a["k"], a["v"], a["beta"], a["alpha"], a["S0"], a["dO"], a["dS_T"],
                                    a["dq"], a["dk_out"], a["dv_out"], a["dbeta"], a["dalpha"], a["dS0"], a["B"],
                                    a["H"], a["T"], a["dk"], a["dv"], a["dtype"], a["chunk"], a["ws"], a["wsb"],
                                    a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(beta=None), "INVALID_ARG"), (dict(dbeta=None), "INVALID_ARG"), (dict(dO=None), "INVALID_ARG"),
    (dict(alpha=P), "INVALID_ARG"),                      # alpha without dalpha
    (dict(dalpha=P), "INVALID_ARG"),                     # dalpha without alpha
    (dict(T=0), "INVALID_ARG"), (dict(dtype=4), "INVALID_ARG"), (dict(dtype=0), "UNSUPPORTED"),
    (dict(dk=32), "UNSUPPORTED"), (dict(chunk=128), "UNSUPPORTED"),
    (dict(beta=ctypes.c_void_p(0x10001)), "INVALID_ARG"), (dict(dbeta=ctypes.c_void_p(0x10002)), "INVALID_ARG"),
    (dict(dq=ctypes.c_void_p(0x10008)), "INVALID_ARG"),
    (dict(ws=None), "WORKSPACE"), (dict(wsb=1024), "WORKSPACE"),
])
def test_delta_backward_rejects(kw, status):
    assert _dlb(**kw) == ST[status]
    assert lin.lib().la_last_error().decode().startswith("delta_backward")
    # the variant that reads a training forward's context checks the same
    assert _dlb("delta_backward_after_forward", **kw) == ST[status]
    assert lin.lib().la_last_error().decode().startswith("delta_backward_after_forward")


def _dft(**kw):
    a = dict(q=P, k=P, v=P, beta=P, alpha=None, S0=None, o=P, S_out=None, B=1, H=1, T=8, dk=128, dv=128, dtype=1,
             chunk=64, ws=P, wsb=1 << 30, stream=None)
    a.update(kw)
    return lin.lib().delta_forward_train(a["q"], a["k"], a["v"], a["beta"], a["alpha"], a["S0"], a["o"],
                                         a["S_out"], a["B"], a["H"], a["T"], a["dk"], a["dv"], a["dtype"],
                                         a["chunk"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), "INVALID_ARG"), (dict(beta=None), "INVALID_ARG"), (dict(o=None), "INVALID_ARG"),
    (dict(T=0), "INVALID_ARG"), (dict(H=-1), "INVALID_ARG"), (dict(dtype=3), "INVALID_ARG"),
    (dict(dtype=0), "UNSUPPORTED"), (dict(dk=96), "UNSUPPORTED"), (dict(chunk=32), "UNSUPPORTED"),
    (dict(o=ctypes.c_void_p(0x10008)), "INVALID_ARG"), (dict(beta=ctypes.c_void_p(0x10001)), "INVALID_ARG"),
    (dict(alpha=ctypes.c_void_p(0x10002)), "INVALID_ARG"), (dict(S_out=ctypes.c_void_p(0x10002)), "INVALID_ARG"),
    (dict(ws=None), "WORKSPACE"), (dict(ws=ctypes.c_void_p(0x10008)), "WORKSPACE"),
])
def test_delta_forward_train_rejects(kw, status):
    assert _dft(**kw) == ST[status]
    assert lin.lib().la_last_error().decode().startswith("delta_forward_train")


def test_delta_forward_train_needs_the_backward_workspace():
    # a forward-sized workspace is too small: the training forward also
    # keeps every chunk's entering state for the backward
    L = lin.lib()
    B, H, T = 2, 4, 1000
    fwd = L.delta_forward_workspace_bytes(B, H, T, 128, 128, 64)
    bwd = L.delta_backward_workspace_bytes(B, H, T, 128, 128, 64)
    assert 0 < fwd < bwd
    assert _dft(B=B, H=H, T=T, wsb=fwd) == ST["WORKSPACE"]
    assert str(bwd) in L.la_last_error().decode()


@pytest.mark.parametrize("dk,dv,dtype", [(128, 128, 1), (64, 64, 1), (64, 128, 0)])
def test_rows_beyond_32_bit_offsets_are_unsupported(dk, dv, dtype):
    # one (sequence, head)'s rows, plus four chunks of read-ahead, must span
    # < 2 GiB: the kernels address them with 32-bit buffer offsets
    el = 2 if dtype == 1 else 4
    t_max = (1 << 31) // (max(dk, dv) * el) - 4 * 64 - 1  # the longest accepted T
    assert _la(T=t_max + 1, dk=dk, dv=dv, dtype=dtype) == ST["UNSUPPORTED"]
    assert "too long" in lin.lib().la_last_error().decode()
    assert _la(T=t_max, dk=dk, dv=dv, dtype=dtype, wsb=16) == ST["WORKSPACE"]  # passes the size check
    if dtype == 1:
        assert _delta(T=t_max + 1, dk=dk, dv=dv) == ST["UNSUPPORTED"]
        assert _delta(T=t_max, dk=dk, dv=dv, wsb=16) == ST["WORKSPACE"]
    assert lin.lib().la_forward_workspace_bytes(1, 1, t_max + 1, dk, dv, 64) == 0 or dtype == 0


def test_lookback_test_hook_validates_like_la_forward():
    L = lin.lib()
    args = [P, P, P, None, None, P, None, None, 1, 1, 8, 64, 64, 1, 1e-6, 64, P, 16, None]
    assert L.la_forward_lookback_polls(*args, -1) == ST["WORKSPACE"]
    args[10] = 0
    assert L.la_forward_lookback_polls(*args, 5) == ST["INVALID_ARG"]
    assert lin.lib().la_last_error().decode().startswith("la_forward_lookback_polls")


def test_noalloc_refuses_beyond_its_scratch_before_touching_the_device():
    L = lin.lib()
    args = [P, P, P, None, None, P, None, None, 1, 64, 65536, 64, 64, 1, 1e-6, 64, None]
    assert L.la_forward_workspace_bytes(1, 64, 65536, 64, 64, 64) > (96 << 20)
    assert L.la_forward_noalloc(*args) == ST["UNSUPPORTED"]
    assert "scratch" in L.la_last_error().decode()
    args[10] = 0  # invalid sizes are reported as such
    assert L.la_forward_noalloc(*args) == ST["INVALID_ARG"]
    assert L.la_forward_workspace_bytes(1, 32, 65536, 64, 64, 64) <= (96 << 20)  # the long-stream size fits


def test_workspace_queries():
    L = lin.lib()
    assert L.la_forward_workspace_bytes(0, 1, 8, 64, 64, 64) == 0
    assert L.la_forward_workspace_bytes(1, 1, 8, 96, 64, 64) == 0
    n = L.la_forward_workspace_bytes(4, 8, 8192, 64, 64, 64)
    assert n > 0 and n % 16 == 0
    assert L.delta_forward_workspace_bytes(2, 16, 16384, 128, 128, 64) > 0
    assert L.ssd_forward_workspace_bytes(4, 8, 8192, 64, 64, 64) > 0
    assert L.ssd_forward_workspace_bytes(4, 8, 8192, 64, 32, 64) == 0
    # the backward holds two bf16 tiles per chunk beyond the forward's arrays
    nb = L.delta_backward_workspace_bytes(2, 16, 16384, 128, 128, 64)
    assert nb == L.delta_forward_workspace_bytes(2, 16, 16384, 128, 128, 64) + 4 * 32 * 256 * 128 * 128
    assert L.delta_backward_workspace_bytes(2, 16, 16384, 128, 96, 64) == 0


def test_chunk_size_workspace_queries():
    # la_forward, uniform batches: chunks of 16, 32, 64 and 128 tokens; the
    # blocked path (not 64) holds two [S | z] states per (head, segment)
    L = lin.lib()
    for C in (16, 32, 64, 128):
        n = L.la_forward_workspace_bytes(2, 16, 6000, 64, 128, C)
        assert n > 0 and n % 16 == 0, C
    for C in (0, 8, 48, 96, 256):
        assert L.la_forward_workspace_bytes(2, 16, 6000, 64, 64, C) == 0, C
    # a 128-token chunk rounds the segments up to whole chunks; 16 and 32 keep
    # the 64-token plan's segments
    E = 64 * 128 + 64
    n16 = L.la_forward_workspace_bytes(1, 1, 100000, 64, 128, 16)
    assert n16 % (2 * 4 * E) == 0 and n16 == L.la_forward_workspace_bytes(1, 1, 100000, 64, 128, 32)
    # delta_forward too (three per-slot arrays, no chunk records); the
    # scalar-decay rule and the packed batches take 64 only
    for C in (16, 32, 128):
        n = L.delta_forward_workspace_bytes(2, 16, 16384, 128, 128, C)
        assert n > 0 and n % (4 * (2 * 128 * 128 + 128 * 128)) == 0, C
        assert L.ssd_forward_workspace_bytes(4, 8, 8192, 64, 64, C) == 0
        cu = (ctypes.c_int * 3)(0, 5, 9)
        assert L.la_forward_packed_workspace_bytes(ctypes.cast(cu, ctypes.c_void_p), 2, 2, 9, 64, 64, C) == 0


def test_status_strings():
    L = lin.lib()
    assert [L.la_status_string(i).decode() for i in range(5)] == [
        "LA_OK", "LA_ERR_INVALID_ARG", "LA_ERR_UNSUPPORTED", "LA_ERR_WORKSPACE", "LA_ERR_HIP"]


def test_python_binding_raises_value_error():
    import torch
    q = torch.zeros((1, 1, 4, 64), dtype=torch.float16)
    with pytest.raises(ValueError):
        lin.la_forward(q, q, q)
