"""The ring layout of the conv registers ([W, B, C] slot arrays, the oldest
register in slot conv_pos) against the shifted layout ([B, C, W], oldest
first) on the GPU: the decode step and the prefill prologue must give
bit-identical outputs and states, and registers that map onto each other
slot for slot.  The shifted layout is pinned to the oracle by
test_decode_parity.py and test_prologue_parity.py; one case here also goes to
the oracle directly."""
import sys

import numpy as np
import pytest
import torch

import oracle
import gated_delta_rule_kda_amd as kda
from gated_delta_rule_kda_amd import synth
from kda_testutil import assert_close, gpu_available, np64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def ring_from_rows(rows, pos):
    """[B, C, W] registers (oldest first) -> the [W, B, C] ring with the
    oldest register in slot pos."""
    W = rows.shape[-1]
    ring = torch.empty(W, rows.shape[0], rows.shape[1], dtype=rows.dtype, device=rows.device)
    for j in range(W):
        ring[(pos + j) % W] = rows[..., j]
    return ring.contiguous()


def rows_from_ring(ring, pos):
    W = ring.shape[0]
    return torch.stack([ring[(pos + j) % W] for j in range(W)], dim=-1)


DECODE_CASES = [
    # B, H, HV, K, V, KW, dtype, steps
    (3, 2, 2, 32, 32, 4, torch.float32, 11),
    (2, 2, 8, 64, 128, 3, torch.bfloat16, 7),
    (2, 1, 2, 128, 128, 8, torch.float32, 10),
    (1, 1, 1, 32, 64, 1, torch.float32, 3),
    (4, 4, 4, 128, 128, 4, torch.bfloat16, 9),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: "B%dH%dHV%dK%dV%dKW%d-%s-%d" % (
    c[:6] + (str(c[6]).split(".")[-1], c[7])))
def test_decode_ring_equals_shifted(case):
    """Steps past one full turn of the ring, from random registers and a
    nonzero start slot: out and state bitwise equal to the shifted layout's
    after every step, and the registers equal slot for slot."""
    B, H, HV, K, V, KW, dt, steps = case
    say("decode ring", case)
    shape = synth.DecodeShape(B=B, H=H, HV=HV, K=K, V=V, KW=KW)
    C = 2 * H * K + HV * V
    prm = synth.make_decode_params(shape, DEV, 11)
    gen = torch.Generator(device=DEV).manual_seed(12)
    rows = torch.randn(B, C, KW, device=DEV, generator=gen)
    pos = 1 % KW
    ring = ring_from_rows(rows, pos)
    s_rows = torch.randn(B, HV, K, V, device=DEV, generator=gen) * 0.3
    s_ring = s_rows.clone()
    kw = dict(H=H, HV=HV, K=K, V=V, conv_weight=prm["conv_w"], l2norm_qk=True, l2_eps=1e-6,
              gate_mode=kda.GATE_BOUNDED, A_log=prm["A_log"], dt_bias=prm["dt_bias"],
              beta_is_logit=True)
    for t in range(steps):
        x, z, bl = prm["pool"][t % shape.pool]
        x = x.to(dt)
        y_rows = kda.decode_step(x, z.view(B, HV, K), bl, s_rows, conv_state=rows, **kw)
        y_ring = kda.decode_step(x, z.view(B, HV, K), bl, s_ring, conv_state=ring, conv_ring=True,
                                 conv_pos=pos, **kw)
        pos = (pos + 1) % KW
        torch.cuda.synchronize()
        assert torch.equal(y_ring, y_rows), ("out", t)
        assert torch.equal(s_ring, s_rows), ("state", t)
        assert torch.equal(rows_from_ring(ring, pos), rows), ("registers", t)


def test_decode_ring_against_oracle():
    """Ring-layout decode steps against the oracle's decode (which keeps the
    registers oldest first), from zero registers."""
    shape = synth.DecodeShape(B=2, H=2, HV=4, K=64, V=64, KW=4)
    B, H, HV, K, V, KW = shape.B, shape.H, shape.HV, shape.K, shape.V, shape.KW
    C = 2 * H * K + HV * V
    say("decode ring vs oracle", shape)
    prm = synth.make_decode_params(shape, DEV, 21)
    state = torch.zeros(B, HV, K, V, device=DEV)
    ring = torch.zeros(KW, B, C, device=DEV)
    st_ref = np.zeros((B, HV, K, V))
    cv_ref = np.zeros((B, C, KW))
    pos = 0
    for t in range(9):
        x, z, bl = prm["pool"][t % shape.pool]
        out = kda.decode_step(x, z.view(B, HV, K), bl, state, H=H, HV=HV, K=K, V=V,
                              conv_weight=prm["conv_w"], conv_state=ring, conv_ring=True, conv_pos=pos,
                              l2norm_qk=True, l2_eps=1e-6, gate_mode=kda.GATE_BOUNDED,
                              A_log=prm["A_log"], dt_bias=prm["dt_bias"], beta_is_logit=True)
        pos = (pos + 1) % KW
        oref = oracle.kda_decode_step(x, st_ref, H, HV, K, V, conv_w=prm["conv_w"], conv_state=cv_ref,
                                      l2norm_qk=True, eps=1e-6, gate_in=z, A_log=prm["A_log"],
                                      dt_bias=prm["dt_bias"], gate_bounded=True, lower_bound=-5.0,
                                      beta=bl, beta_is_logit=True)
        assert_close(out, oref, torch.float32, True, "ring step %d out" % t)
    assert_close(state, st_ref, torch.float32, False, "ring final state")
    np.testing.assert_array_equal(np64(rows_from_ring(ring, pos)), cv_ref)


PROLOGUE_CASES = [
    # B, T, H, HV, K, V, KW, dtype, pos
    (2, 1, 2, 2, 32, 32, 4, torch.float32, 3),
    (2, 2, 1, 2, 64, 64, 4, torch.bfloat16, 1),
    (1, 3, 2, 2, 128, 128, 4, torch.bfloat16, 2),
    (1, 4, 2, 2, 128, 128, 4, torch.bfloat16, 2),
    (2, 37, 1, 3, 64, 32, 3, torch.float32, 1),
    (1, 300, 2, 2, 128, 128, 4, torch.bfloat16, 0),
    (1, 5, 1, 1, 32, 32, 8, torch.float32, 6),
    (1, 9, 1, 1, 32, 32, 1, torch.float32, 0),
]


def _prologue(x, z, bl, prm, H, HV, K, V, conv_state, **kw):
    return kda.prefill_prologue(x, z, bl, H=H, HV=HV, K=K, V=V, conv_weight=prm["conv_w"],
                                conv_state=conv_state, l2norm_qk=True, l2_eps=1e-6,
                                gate_mode=kda.GATE_BOUNDED, A_log=prm["A_log"], dt_bias=prm["dt_bias"],
                                gate_lower_bound=-5.0, beta_is_logit=True, **kw)


@pytest.mark.parametrize("case", PROLOGUE_CASES, ids=lambda c: "B%dT%dH%dHV%dK%dV%dKW%d-%s-p%d" % (
    c[:7] + (str(c[7]).split(".")[-1], c[8])))
def test_prologue_ring_equals_shifted(case):
    """The prefill prologue from random registers in either layout (T below,
    at and above the conv width): q, k, v, g and beta bitwise equal, the
    registers after the last token equal slot for slot; then decode steps
    continue from both (the ring's position advanced by T) and stay equal."""
    B, T, H, HV, K, V, KW, dt, pos = case
    say("prologue ring", case)
    C = 2 * H * K + HV * V
    gen = torch.Generator(device="cpu").manual_seed(31 + T)
    r = lambda *s: torch.randn(*s, generator=gen).to(DEV)
    x = r(B, T, C).to(dt)
    z = r(B, T, HV, K)
    bl = r(B, T, HV)
    prm = dict(conv_w=r(C, KW) * 0.5, A_log=r(HV) * 0.5, dt_bias=r(HV * K) * 0.5)
    rows = r(B, C, KW)
    ring = ring_from_rows(rows, pos)
    got_rows = _prologue(x, z, bl, prm, H, HV, K, V, rows)
    got_ring = _prologue(x, z, bl, prm, H, HV, K, V, ring, conv_ring=True, conv_pos=pos)
    torch.cuda.synchronize()
    for name, a, b in zip(("q", "k", "v", "g", "beta"), got_ring, got_rows):
        assert torch.equal(a, b), name
    pos = (pos + T) % KW
    assert torch.equal(rows_from_ring(ring, pos), rows), "registers after the prefill"
    # decode continues from both
    s_rows = torch.zeros(B, HV, K, V, device=DEV)
    s_ring = s_rows.clone()
    kw = dict(H=H, HV=HV, K=K, V=V, conv_weight=prm["conv_w"], l2norm_qk=True, l2_eps=1e-6,
              gate_mode=kda.GATE_BOUNDED, A_log=prm["A_log"], dt_bias=prm["dt_bias"], beta_is_logit=True)
    for t in range(KW + 1):
        xd = r(B, C).to(dt)
        zd = r(B, HV, K)
        bd = r(B, HV)
        y_rows = kda.decode_step(xd, zd, bd, s_rows, conv_state=rows, **kw)
        y_ring = kda.decode_step(xd, zd, bd, s_ring, conv_state=ring, conv_ring=True, conv_pos=pos, **kw)
        pos = (pos + 1) % KW
        torch.cuda.synchronize()
        assert torch.equal(y_ring, y_rows), ("decode out", t)
        assert torch.equal(s_ring, s_rows), ("decode state", t)
    assert torch.equal(rows_from_ring(ring, pos), rows), "registers after decoding"


def test_prologue_ring_without_registers():
    """No conv_state: both layouts start from zero registers and write none."""
    B, T, H, HV, K, V, KW = 1, 6, 1, 2, 32, 32, 4
    C = 2 * H * K + HV * V
    gen = torch.Generator(device="cpu").manual_seed(41)
    r = lambda *s: torch.randn(*s, generator=gen).to(DEV)
    x, z, bl = r(B, T, C), r(B, T, HV, K), r(B, T, HV)
    prm = dict(conv_w=r(C, KW), A_log=r(HV), dt_bias=r(HV * K))
    a = _prologue(x, z, bl, prm, H, HV, K, V, None)
    b = _prologue(x, z, bl, prm, H, HV, K, V, None, conv_ring=True, conv_pos=2)
    torch.cuda.synchronize()
    for name, u, w in zip(("q", "k", "v", "g", "beta"), a, b):
        assert torch.equal(u, w), name
