"""Seeded synthetic workloads (input generation only; none of the method's
arithmetic lives here).  Tests, the benchmark and the oracle's callers all
draw their inputs from this module.

Distributions follow the pages' settings: N(0, 1) draws for q, k, v
("AIGC 基本功｜线性、循环与记忆架构-LinearMem", §04 script), unit keys
(Gaussian, then normalised per token: same page §03, the delta rule assumes
unit keys), beta through a sigmoid (same page §08: the final per-token step
size after the model's transform), d = 64 / 128 with lengths up to 65536
(same page §01 ledger).  Forgetting gates take the Mamba-2 form of the
"线性注意力与 SSM" page (§2.9, and §3 on Mamba-2), alpha = exp(-Delta a)
with Delta = softplus(N(0, 1)) and a = 1/16: alpha lies in about (0.83,
0.997), median about 0.96.  bf16 inputs are fp32 draws rounded to nearest even.
Generation runs on the device the tensors are wanted on, with a
torch.Generator seeded per workload.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str        # "la", "delta", "gated_delta", "ssd", or one of those + "_decode" ("decode" = LA)
    B: int           # batch (decode: sequences N)
    H: int
    T: int           # tokens (decode: number of steps)
    dk: int
    dv: int
    dtype: torch.dtype
    seed: int


# The five configurations the measurements and parity tests are quoted on.
LA_FP32_SMALL = Workload("la_fp32_b1_h1_t1024_d64", "la", 1, 1, 1024, 64, 64, torch.float32, 1)
LA_BF16_PREFILL = Workload("la_bf16_b4_h8_t8192_d64", "la", 4, 8, 8192, 64, 64, torch.bfloat16, 2)
DELTA_BF16_PREFILL = Workload("delta_bf16_b2_h16_t16384_d128", "delta", 2, 16, 16384, 128, 128,
                              torch.bfloat16, 3)
LA_BF16_LONG = Workload("la_bf16_b1_h32_t65536_d64", "la", 1, 32, 65536, 64, 64, torch.bfloat16, 4)
DECODE_BF16 = Workload("decode_bf16_n256_h32_d128_1000steps", "decode", 256, 32, 1000, 128, 128,
                       torch.bfloat16, 5)
ALL = (LA_FP32_SMALL, LA_BF16_PREFILL, DELTA_BF16_PREFILL, LA_BF16_LONG, DECODE_BF16)
# The delta-rule decode step on the decode configuration's states and steps.
DELTA_DECODE_BF16 = Workload("delta_decode_bf16_n256_h32_d128_1000steps", "delta_decode", 256, 32, 1000, 128,
                             128, torch.bfloat16, 6)
# The gated delta rule on the delta prefill and decode configurations.
GATED_DELTA_BF16_PREFILL = Workload("gated_delta_bf16_b2_h16_t16384_d128", "gated_delta", 2, 16, 16384, 128, 128,
                                    torch.bfloat16, 7)
GATED_DELTA_DECODE_BF16 = Workload("gated_delta_decode_bf16_n256_h32_d128_1000steps", "gated_delta_decode", 256,
                                   32, 1000, 128, 128, torch.bfloat16, 8)
# The scalar-decay (Mamba-2 / SSD form) rule on the LA prefill configuration.
SSD_BF16_PREFILL = Workload("ssd_bf16_b4_h8_t8192_d64", "ssd", 4, 8, 8192, 64, 64, torch.bfloat16, 9)
SSD_DECODE_BF16 = Workload("ssd_decode_bf16_n256_h32_d128_1000steps", "ssd_decode", 256, 32, 1000, 128, 128,
                           torch.bfloat16, 10)
GATE_RATE = 1.0 / 16
# A packed serving batch with the LA prefill configuration's token total
# (4 x 8192 per head, 8 heads, d = 64): 48 requests of mixed lengths.
PACKED_LA_BF16 = Workload("la_packed_bf16_h8_48req_32768tok_d64", "la_packed", 48, 8, 32768, 64, 64,
                          torch.bfloat16, 12)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(seed)
    return g


def _normal(shape, g, device, std=1.0):
    x = torch.empty(shape, dtype=torch.float32, device=device)
    x.normal_(mean=0.0, std=std, generator=g)
    return x


def la_inputs(B, H, T, dk, dv, dtype, seed, device="cpu"):
    """q, k, v ~ N(0, 1), rounded to `dtype`."""
    g = _gen(seed, device)
    q = _normal((B, H, T, dk), g, device).to(dtype)
    k = _normal((B, H, T, dk), g, device).to(dtype)
    v = _normal((B, H, T, dv), g, device).to(dtype)
    return q, k, v


def unit_rows(x: torch.Tensor) -> torch.Tensor:
    """Scale each last-axis vector to unit L2 norm (input preparation)."""
    return x / x.norm(dim=-1, keepdim=True)


def delta_inputs(B, H, T, dk, dv, dtype, seed, device="cpu"):
    """q, k: N(0, 1) normalised per token; v ~ N(0, 1); beta = sigmoid(N(0, 1))."""
    g = _gen(seed, device)
    k = unit_rows(_normal((B, H, T, dk), g, device)).to(dtype)
    q = unit_rows(_normal((B, H, T, dk), g, device)).to(dtype)
    v = _normal((B, H, T, dv), g, device).to(dtype)
    beta = torch.sigmoid(_normal((B, H, T), g, device)).to(dtype)
    return q, k, v, beta


def decode_state(N, H, dk, dv, seed, device="cpu", std=0.01):
    """Resident fp32 state S, z ~ N(0, std^2)."""
    g = _gen(seed, device)
    S = _normal((N, H, dk, dv), g, device, std)
    z = _normal((N, H, dk), g, device, std)
    return S, z


def decode_tokens(steps, N, H, dk, dv, dtype, seed, device="cpu"):
    """Per-step q, k [steps, N, H, dk] and v [steps, N, H, dv] ~ N(0, 1)."""
    g = _gen(seed + 1000003, device)
    q = _normal((steps, N, H, dk), g, device).to(dtype)
    k = _normal((steps, N, H, dk), g, device).to(dtype)
    v = _normal((steps, N, H, dv), g, device).to(dtype)
    return q, k, v


def delta_decode_tokens(steps, N, H, dk, dv, dtype, seed, device="cpu"):
    """Per-step q, k [steps, N, H, dk] (N(0, 1) normalised per token),
    v [steps, N, H, dv] ~ N(0, 1) and beta [steps, N, H] = sigmoid(N(0, 1))."""
    g = _gen(seed + 1000003, device)
    k = unit_rows(_normal((steps, N, H, dk), g, device)).to(dtype)
    q = unit_rows(_normal((steps, N, H, dk), g, device)).to(dtype)
    v = _normal((steps, N, H, dv), g, device).to(dtype)
    beta = torch.sigmoid(_normal((steps, N, H), g, device)).to(dtype)
    return q, k, v, beta


def gates(shape, seed, device="cpu", rate=GATE_RATE):
    """Forgetting factors alpha = exp(-softplus(N(0, 1)) * rate), fp32."""
    g = _gen(seed + 2000003, device)
    return torch.exp(-torch.nn.functional.softplus(_normal(shape, g, device)) * rate)


def packed_lengths(n, total, seed):
    """n request lengths >= 1 summing to `total`: log-normal shares (sigma
    1), so a few long prompts and many short ones, rounded with the remainder
    spread over the first requests."""
    g = _gen(seed + 3000017, "cpu")
    w = torch.exp(torch.empty(n, dtype=torch.float64).normal_(0.0, 1.0, generator=g))
    share = (w / w.sum() * (total - n)).floor().to(torch.int64) + 1
    rest = total - int(share.sum())
    share[:rest] += 1
    return share


def packed_offsets(lengths):
    """Sequence offsets [0, l0, l0 + l1, ...] (int32, host)."""
    return torch.cat([torch.zeros(1, dtype=torch.int64), torch.cumsum(lengths, 0)]).to(torch.int32)


def make(w: Workload, device="cpu"):
    """All inputs of a workload on `device`."""
    if w.kind == "la":
        return la_inputs(w.B, w.H, w.T, w.dk, w.dv, w.dtype, w.seed, device)
    if w.kind == "delta":
        return delta_inputs(w.B, w.H, w.T, w.dk, w.dv, w.dtype, w.seed, device)
    if w.kind == "decode":
        S, z = decode_state(w.B, w.H, w.dk, w.dv, w.seed, device)
        return (S, z) + decode_tokens(w.T, w.B, w.H, w.dk, w.dv, w.dtype, w.seed, device)
    if w.kind == "delta_decode":
        S, _ = decode_state(w.B, w.H, w.dk, w.dv, w.seed, device, std=0.1)
        return (S,) + delta_decode_tokens(w.T, w.B, w.H, w.dk, w.dv, w.dtype, w.seed, device)
    if w.kind == "gated_delta":
        return delta_inputs(w.B, w.H, w.T, w.dk, w.dv, w.dtype, w.seed, device) + (
            gates((w.B, w.H, w.T), w.seed, device),)
    if w.kind == "ssd":
        return la_inputs(w.B, w.H, w.T, w.dk, w.dv, w.dtype, w.seed, device) + (
            gates((w.B, w.H, w.T), w.seed, device),)
    if w.kind == "ssd_decode":
        S, _ = decode_state(w.B, w.H, w.dk, w.dv, w.seed, device, std=0.1)
        return (S,) + decode_tokens(w.T, w.B, w.H, w.dk, w.dv, w.dtype, w.seed, device) + (
            gates((w.T, w.B, w.H), w.seed, device),)
    if w.kind == "la_packed":
        q, k, v = (x[0] for x in la_inputs(1, w.H, w.T, w.dk, w.dv, w.dtype, w.seed, device))
        return q, k, v, packed_offsets(packed_lengths(w.B, w.T, w.seed))
    if w.kind == "gated_delta_decode":
        S, _ = decode_state(w.B, w.H, w.dk, w.dv, w.seed, device, std=0.1)
        return (S,) + delta_decode_tokens(w.T, w.B, w.H, w.dk, w.dv, w.dtype, w.seed, device) + (
            gates((w.T, w.B, w.H), w.seed, device),)
    raise ValueError(w.kind)
