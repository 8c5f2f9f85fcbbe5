"""Seeded synthetic inputs for the KDA forward (prefill and decode).

This module draws random tensors only; it holds none of the attention
arithmetic.  The same generators feed the HIP library, the CPU oracle, the
tests and the benchmark.

Recipe (one torch.Generator on the target device, seeded, draws in the order
listed; fp32 draws, transformed, then cast):
  prefill: q, k ~ N(0,1) then unit-L2-normalised per (token, head) row
           (torch.nn.functional.normalize), v ~ N(0,1),
           g = lower * sigmoid(N(0,1)) per (token, value head, key channel),
           beta = sigmoid(N(0,1)), then optionally S0 ~ N(0, s0_std^2) last.
           q, k, v are cast to the working dtype after the transform.
  decode:  parameters first: conv_w [C, KW], dt_bias [HV*K], A_log [HV] ~ N(0,1);
           then a pool of P step inputs, each x [B, C], z [B, HV*K],
           beta logits [B, HV] ~ N(0,1), where C = 2*H*K + HV*V.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch
import torch.nn.functional as F


@dataclass(frozen=True)
class PrefillShape:
    B: int
    T: int
    H: int
    HV: int
    K: int
    V: int
    dtype: torch.dtype = torch.bfloat16
    s0: str = "none"          # "none" | "zeros" | "normal"
    s0_std: float = 0.02
    g_lower: float = -5.0     # g = g_lower * sigmoid(N(0,1))
    chunk: int = 32


@dataclass(frozen=True)
class DecodeShape:
    B: int
    H: int
    HV: int
    K: int
    V: int
    KW: int = 4
    pool: int = 8
    steps: int = 1000
    lower_bound: float = -5.0


# The workloads, by what they are.
PREFILL_TINY_F32 = PrefillShape(1, 64, 2, 2, 32, 32, torch.float32, "none")
PREFILL_TWIN_BF16 = PrefillShape(4, 2048, 8, 8, 32, 32, torch.bfloat16, "none")
PREFILL_HV96_BF16 = PrefillShape(1, 8192, 96, 96, 128, 128, torch.bfloat16, "zeros")
PREFILL_GQA_BF16 = PrefillShape(8, 4096, 16, 64, 128, 128, torch.bfloat16, "normal")
DECODE_B256_HV96 = DecodeShape(256, 96, 96, 128, 128)


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def make_prefill_inputs(shape: PrefillShape, device="cpu", seed: int = 0,
                        g_lower: float | None = None, g_heavy: bool = False):
    """Return dict(q, k, v, g, beta, S0) on ``device`` following the recipe above.
    ``g_heavy`` draws g = -exp(1.5 N(0,1)) instead (no lower bound: median -1,
    about 5 % below -12, 0.1 % below -100), the range of an unbounded gate."""
    B, T, H, HV, K, V = shape.B, shape.T, shape.H, shape.HV, shape.K, shape.V
    lower = shape.g_lower if g_lower is None else g_lower
    gen = _gen(device, seed)
    f32 = dict(dtype=torch.float32, device=device, generator=gen)
    q = F.normalize(torch.randn(B, T, H, K, **f32), dim=-1)
    k = F.normalize(torch.randn(B, T, H, K, **f32), dim=-1)
    v = torch.randn(B, T, HV, V, **f32)
    g = lower * torch.sigmoid(torch.randn(B, T, HV, K, **f32))
    if g_heavy:
        g = -torch.exp(1.5 * torch.randn(B, T, HV, K, **f32))
    beta = torch.sigmoid(torch.randn(B, T, HV, **f32))
    if shape.s0 == "normal":
        S0 = shape.s0_std * torch.randn(B, HV, K, V, **f32)
    elif shape.s0 == "zeros":
        S0 = torch.zeros(B, HV, K, V, dtype=torch.float32, device=device)
    else:
        S0 = None
    dt = shape.dtype
    return dict(q=q.to(dt).contiguous(), k=k.to(dt).contiguous(), v=v.to(dt).contiguous(),
                g=g.contiguous(), beta=beta.contiguous(), S0=S0)


def make_decode_params(shape: DecodeShape, device="cpu", seed: int = 0):
    """Parameters and the pool of per-step inputs, following the recipe above."""
    B, H, HV, K, V, KW = shape.B, shape.H, shape.HV, shape.K, shape.V, shape.KW
    C = 2 * H * K + HV * V
    gen = _gen(device, seed)
    f32 = dict(dtype=torch.float32, device=device, generator=gen)
    conv_w = torch.randn(C, KW, **f32)
    dt_bias = torch.randn(HV * K, **f32)
    A_log = torch.randn(HV, **f32)
    pool = []
    for _ in range(shape.pool):
        x = torch.randn(B, C, **f32)
        z = torch.randn(B, HV * K, **f32)
        bl = torch.randn(B, HV, **f32)
        pool.append((x, z, bl))
    return dict(conv_w=conv_w, dt_bias=dt_bias, A_log=A_log, pool=pool)
