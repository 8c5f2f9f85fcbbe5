"""GPU parity of kda_chunk_fwd_unbounded (the chunked prefill for gates without
a lower bound: in-chunk matrices from blocks with a reference row of their
own, each token's g floored at -17) against the fp64 oracle, whose recurrence
takes every gate as given."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import gated_delta_rule_kda_amd as kda
from gated_delta_rule_kda_amd import synth
from kda_testutil import assert_close, gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def unbounded_gate(B, T, HV, K, seed, a_scale=1.0, z_scale=2.0):
    """g = -exp(A_log) * softplus(z + dt_bias): the bounded_gate of the kda.rs
    page with no lower bound; A_log, dt_bias, z drawn N(0,1), z scaled."""
    gen = torch.Generator(device="cpu").manual_seed(seed)
    A_log = torch.randn(HV, generator=gen) * a_scale
    dt = torch.randn(HV * K, generator=gen)
    z = torch.randn(B, T, HV * K, generator=gen) * z_scale
    g = -torch.exp(A_log).repeat_interleave(K) * torch.nn.functional.softplus(z + dt)
    return g.view(B, T, HV, K).contiguous()


def gates(shape, seed, kind):
    if kind == "unbounded":
        return unbounded_gate(shape.B, shape.T, shape.HV, shape.K, seed + 1).to(DEV)
    if kind == "extreme":
        g = unbounded_gate(shape.B, shape.T, shape.HV, shape.K, seed + 1, a_scale=3.0, z_scale=4.0)
        g[:, ::7] = -1.0e4           # tokens that forget everything
        return g.to(DEV)
    if kind == "heavy":              # g = -exp(1.5 N(0,1))
        return synth.make_prefill_inputs(shape, DEV, seed + 2, g_heavy=True)["g"]
    if kind == "near_floor":         # every token within a few units of the floor
        gen = torch.Generator(device="cpu").manual_seed(seed + 3)
        g = -17.0 + 4.0 * (torch.rand(shape.B, shape.T, shape.HV, shape.K, generator=gen) - 0.5)
        return g.to(DEV)
    raise ValueError(kind)


def run(shape, seed, kind="unbounded", label=""):
    say("unbounded chunk case", label, shape, "seed", seed, "gate", kind)
    inp = synth.make_prefill_inputs(shape, DEV, seed)
    inp["g"] = gates(shape, seed, kind)
    say("   g range", float(inp["g"].min()), float(inp["g"].max()))
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    o, S = kda.chunk_fwd_unbounded(*args, initial_state=inp["S0"], output_final_state=True)
    torch.cuda.synchronize()
    oref, Sref = oracle.kda_fwd(*args, initial_state=inp["S0"])
    mo = assert_close(o, oref, shape.dtype, True, "o " + label)
    ms = assert_close(S, Sref, shape.dtype, False, "S_T " + label)
    say("   o", mo)
    say("   S", ms)
    return inp, o, S


CASES = [
    # B, T, H, HV, K, V  (bf16): several chunks and a ragged tail, GQA, every K, V
    (2, 100, 2, 4, 128, 64),
    (1, 257, 1, 2, 128, 128),
    (3, 33, 1, 3, 64, 32),
    (2, 65, 2, 2, 32, 64),
    (1, 1, 1, 1, 32, 32),
    (1, 16, 2, 8, 64, 128),
    (1, 96, 1, 1, 128, 32),
    (2, 160, 1, 2, 32, 128),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dT%dH%dHV%dK%dV%d" % c)
@pytest.mark.parametrize("kind", ["unbounded", "extreme", "heavy"])
def test_unbounded_chunk_gates(case, kind):
    B, T, H, HV, K, V = case
    run(synth.PrefillShape(B, T, H, HV, K, V, torch.bfloat16, "normal", s0_std=0.3), seed=T + K,
        kind=kind, label=str(case))


def test_unbounded_chunk_near_floor():
    """Every token's g within 2 of the floor (-17): the F3 factors at their
    widest, and the floor itself active on about half the tokens."""
    run(synth.PrefillShape(2, 130, 2, 2, 128, 64, torch.bfloat16, "normal", s0_std=0.3), seed=5,
        kind="near_floor", label="near floor")


def test_unbounded_chunk_long_memory():
    """Slow decay (g = -0.05 sigmoid(N(0,1))) over 2048 tokens: the state
    carried over 64 chunks with the forward-only factors."""
    shape = synth.PrefillShape(1, 2048, 1, 2, 128, 128, torch.bfloat16, "normal", s0_std=0.3)
    inp = synth.make_prefill_inputs(shape, DEV, 21, g_lower=-0.05)
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    o, S = kda.chunk_fwd_unbounded(*args, initial_state=inp["S0"], output_final_state=True)
    torch.cuda.synchronize()
    oref, Sref = oracle.kda_fwd(*args, initial_state=inp["S0"])
    say("   o", assert_close(o, oref, torch.bfloat16, True, "long memory o"))
    say("   S", assert_close(S, Sref, torch.bfloat16, False, "long memory S"))


def test_unbounded_chunk_matches_bounded_chunked():
    """Inside the bounded range (-5 <= g <= 0) the bounded and the unbounded
    chunked paths both agree with the oracle, and so with each other."""
    shape = synth.PrefillShape(2, 200, 2, 4, 64, 64, torch.bfloat16, "normal", s0_std=0.3)
    inp = synth.make_prefill_inputs(shape, DEV, 3)
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    o, S = kda.chunk_fwd_unbounded(*args, initial_state=inp["S0"], output_final_state=True)
    oc, Sc = kda.chunk_fwd(*args, initial_state=inp["S0"], output_final_state=True)
    torch.cuda.synchronize()
    oref, Sref = oracle.kda_fwd(*args, initial_state=inp["S0"])
    assert_close(o, oref, torch.bfloat16, True, "unbounded o (bounded gates)")
    assert_close(S, Sref, torch.bfloat16, False, "unbounded S (bounded gates)")
    assert_close(o, oc.double().cpu().numpy(), torch.bfloat16, True, "unbounded vs bounded chunked o")


def test_unbounded_chunk_forget_everything_closed_form():
    """g = -1e4 at every token (floored to -17, so e^-17 of the state
    survives each step): o_t = s (q_t . k_t) beta_t v_t up to that remainder."""
    shape = synth.PrefillShape(1, 70, 1, 2, 32, 32, torch.bfloat16, "normal", s0_std=1.0)
    inp = synth.make_prefill_inputs(shape, DEV, 8)
    inp["g"].fill_(-1.0e4)
    o, _ = kda.chunk_fwd_unbounded(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                   initial_state=inp["S0"])
    torch.cuda.synchronize()
    s = 1 / math.sqrt(32)
    qk = (inp["q"].double() * inp["k"].double()).sum(-1)            # [B,T,H]
    qk = qk.repeat_interleave(2, dim=2)
    want = s * qk[..., None] * inp["beta"].double()[..., None] * inp["v"].double()
    assert_close(o, want.cpu().numpy(), torch.bfloat16, True, "forget-everything closed form")


def test_unbounded_chunk_agrees_with_recurrent():
    """The chunked and the token-recurrent unbounded paths on the same
    extreme gates: both within the oracle's tolerance, and within it of each
    other."""
    shape = synth.PrefillShape(2, 190, 2, 4, 128, 64, torch.bfloat16, "normal", s0_std=0.3)
    inp, o, S = run(shape, seed=9, kind="extreme", label="vs recurrent")
    orr, Sr = kda.recurrent_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                initial_state=inp["S0"], output_final_state=True)
    torch.cuda.synchronize()
    assert_close(o, orr.double().cpu().numpy(), torch.bfloat16, True, "chunked vs recurrent o")


def test_unbounded_chunk_caller_workspace_and_empty():
    """A caller-given workspace (larger than needed, stale contents) gives the
    same bits as the library-sized one; T = 0 leaves the final state equal to
    the initial state."""
    shape = synth.PrefillShape(1, 75, 1, 2, 64, 64, torch.bfloat16, "normal", s0_std=0.3)
    inp = synth.make_prefill_inputs(shape, DEV, 4)
    inp["g"] = gates(shape, 4, "heavy")
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    o1, S1 = kda.chunk_fwd_unbounded(*args, initial_state=inp["S0"], output_final_state=True)
    n = kda.chunk_fwd_unbounded_workspace_size(1, 75, 1, 2, 64, 64)
    assert n == 1 * 2 * 3 * 7168
    ws = torch.full((n + 4096,), 0x7f, dtype=torch.uint8, device=DEV)
    o2, S2 = kda.chunk_fwd_unbounded(*args, initial_state=inp["S0"], output_final_state=True, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    e = lambda x: x[:, :0].contiguous()
    o0, S0 = kda.chunk_fwd_unbounded(e(inp["q"]), e(inp["k"]), e(inp["v"]), e(inp["g"]), e(inp["beta"]),
                                     initial_state=inp["S0"], output_final_state=True)
    torch.cuda.synchronize()
    assert o0.numel() == 0 and torch.equal(S0, inp["S0"])


def test_full_size_hv96_unbounded_chunk_sampled():
    """The HV96 shape (B1 T8192 H=HV=96 K=V=128 bf16) with g = -exp(1.5 N(0,1)),
    in the launch the bench times: heads 0, 47 and 95 against the oracle."""
    shape = synth.PREFILL_HV96_BF16
    say("full-size unbounded chunked", shape)
    inp = synth.make_prefill_inputs(shape, DEV, 0, g_heavy=True)
    o, S = kda.chunk_fwd_unbounded(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                   initial_state=inp["S0"], output_final_state=True)
    torch.cuda.synchronize()
    for hv in (0, 47, 95):
        sub = lambda x: x[:, :, hv:hv + 1]
        oref, Sref = oracle.kda_fwd(sub(inp["q"]), sub(inp["k"]), sub(inp["v"]), sub(inp["g"]),
                                    inp["beta"][:, :, hv:hv + 1],
                                    initial_state=inp["S0"][:, hv:hv + 1])
        say("   head", hv, assert_close(o[:, :, hv:hv + 1], oref, torch.bfloat16, True,
                                       "HV96 unbounded chunked o head %d" % hv))
        assert_close(S[:, hv:hv + 1], Sref, torch.bfloat16, False, "HV96 unbounded chunked S head %d" % hv)


def test_autograd_unbounded_gate():
    """kda.kda(..., bounded_gate=False): the chunked unbounded forward under
    torch.autograd with the token-recurrent backward; outputs and gradients
    of L = sum(o * Wo) + sum(S_T * WS) against the oracle, with g = -exp(1.5 N(0,1))."""
    shape = synth.PrefillShape(2, 45, 1, 2, 64, 64, torch.bfloat16, "normal", s0_std=0.3)
    inp = synth.make_prefill_inputs(shape, DEV, 31)
    inp["g"] = gates(shape, 31, "heavy")
    gen = torch.Generator(device="cpu").manual_seed(32)
    Wo = torch.randn(2, 45, 2, 64, generator=gen).to(torch.bfloat16).to(DEV)
    WS = (torch.randn(2, 2, 64, 64, generator=gen) * 0.1).to(DEV)
    leaves = {n: inp[n].clone().requires_grad_(True) for n in ("q", "k", "v", "g", "beta", "S0")}
    o, S = kda.kda(leaves["q"], leaves["k"], leaves["v"], leaves["g"], leaves["beta"],
                   initial_state=leaves["S0"], output_final_state=True, bounded_gate=False)
    ((o.float() * Wo.float()).sum() + (S * WS).sum()).backward()
    torch.cuda.synchronize()
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    oref, Sref = oracle.kda_fwd(*args, initial_state=inp["S0"])
    assert_close(o, oref, torch.bfloat16, True, "autograd unbounded o")
    ref = oracle.kda_bwd(*args, Wo, WS, initial_state=inp["S0"])
    for name, want, st in zip(("q", "k", "v", "g", "beta", "S0"), ref, (True, True, True, False, False, False)):
        assert leaves[name].grad is not None, name
        assert_close(leaves[name].grad, want, torch.bfloat16, st, "autograd unbounded d%s" % name)
