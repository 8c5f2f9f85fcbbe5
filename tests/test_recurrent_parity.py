"""GPU parity of kda_recurrent_fwd (the token-recurrent prefill for gates
without a lower bound) against the fp64 oracle, including gates far below the
chunked kernels' -5 bound."""
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


def run(shape, seed, gate="unbounded", label=""):
    say("recurrent case", label, shape, "seed", seed, "gate", gate)
    inp = synth.make_prefill_inputs(shape, DEV, seed)
    if gate == "unbounded":
        inp["g"] = unbounded_gate(shape.B, shape.T, shape.HV, shape.K, seed + 1).to(DEV)
    elif gate == "extreme":
        g = unbounded_gate(shape.B, shape.T, shape.HV, shape.K, seed + 1, a_scale=3.0, z_scale=4.0)
        g[:, ::7] = -1.0e4           # tokens that forget everything
        inp["g"] = g.to(DEV)
    say("   g range", float(inp["g"].min()), float(inp["g"].max()))
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    o, S = kda.recurrent_fwd(*args, initial_state=inp["S0"], output_final_state=True)
    torch.cuda.synchronize()
    oref, Sref = oracle.kda_fwd(*args, initial_state=inp["S0"])
    mo = assert_close(o, oref, shape.dtype, True, "o " + label)
    ms = assert_close(S, Sref, shape.dtype, False, "S_T " + label)
    say("   o", mo)
    say("   S", ms)
    return inp, o, S


CASES = [
    # B, T, H, HV, K, V, dtype
    (2, 100, 2, 4, 128, 64, torch.bfloat16),
    (1, 257, 1, 2, 128, 128, torch.float32),
    (3, 33, 1, 3, 64, 32, torch.bfloat16),
    (2, 65, 2, 2, 32, 64, torch.float32),
    (1, 1, 1, 1, 32, 32, torch.bfloat16),
    (1, 16, 2, 8, 64, 128, torch.float32),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dT%dH%dHV%dK%dV%d-%s" % (
    c[:6] + (str(c[6]).split(".")[-1],)))
@pytest.mark.parametrize("gate", ["unbounded", "extreme"])
def test_recurrent_unbounded_gates(case, gate):
    B, T, H, HV, K, V, dt = case
    run(synth.PrefillShape(B, T, H, HV, K, V, dt, "normal", s0_std=0.3), seed=T + K, gate=gate,
        label=str(case))


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_recurrent_bounded_matches_chunked(dt):
    """Inside the bounded range both prefill paths agree with the oracle (and
    so with each other)."""
    shape = synth.PrefillShape(2, 200, 2, 4, 64, 64, dt, "normal", s0_std=0.3)
    inp, o, S = run(shape, seed=3, gate="bounded", label="bounded")
    oc, Sc = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                           initial_state=inp["S0"], output_final_state=True)
    torch.cuda.synchronize()
    assert_close(o, oc.double().cpu().numpy(), dt, True, "recurrent vs chunked o")


def test_recurrent_forget_everything_closed_form():
    """g = -inf in effect (exp(g) = 0) at every token: S_t = beta_t k_t v_t^T,
    so o_t = s (q_t . k_t) beta_t v_t whatever came before."""
    shape = synth.PrefillShape(1, 40, 1, 2, 32, 32, torch.float32, "normal", s0_std=1.0)
    inp = synth.make_prefill_inputs(shape, DEV, 8)
    inp["g"].fill_(-1.0e4)
    o, _ = kda.recurrent_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                             initial_state=inp["S0"])
    torch.cuda.synchronize()
    s = 1 / math.sqrt(32)
    qk = (inp["q"].double() * inp["k"].double()).sum(-1)            # [B,T,H]
    qk = qk.repeat_interleave(2, dim=2)
    want = s * qk[..., None] * inp["beta"].double()[..., None] * inp["v"].double()
    assert_close(o, want.cpu().numpy(), torch.float32, True, "forget-everything closed form")


def test_full_size_hv96_unbounded_sampled():
    """The HV96 shape (B1 T8192 H=HV=96 K=V=128 bf16) with the unbounded gate:
    heads 0, 47 and 95 against the oracle."""
    shape = synth.PREFILL_HV96_BF16
    say("full-size unbounded", shape)
    inp = synth.make_prefill_inputs(shape, DEV, 0)
    inp["g"] = unbounded_gate(1, shape.T, shape.HV, shape.K, 1).to(DEV)
    o, S = kda.recurrent_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                             initial_state=inp["S0"], output_final_state=True)
    torch.cuda.synchronize()
    for hv in (0, 47, 95):
        sub = lambda x: x[:, :, hv:hv + 1]
        oref, Sref = oracle.kda_fwd(sub(inp["q"]), sub(inp["k"]), sub(inp["v"]), sub(inp["g"]),
                                    inp["beta"][:, :, hv:hv + 1],
                                    initial_state=inp["S0"][:, hv:hv + 1])
        assert_close(o[:, :, hv:hv + 1], oref, torch.bfloat16, True, "HV96 unbounded o head %d" % hv)
        assert_close(S[:, hv:hv + 1], Sref, torch.bfloat16, False, "HV96 unbounded S head %d" % hv)
        say("   head", hv, "ok")


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_recurrent_prefix_and_resume_bitwise(dt):
    """Each token's step depends on earlier tokens only, and tokens past the
    end of a sequence are exact no-ops, so (a) the outputs of a prefix do not
    change when later tokens are appended, and (b) running a sequence in two
    calls, the second resuming from the first one's final state, reproduces
    the single call bit for bit (outputs and final state), whatever the split
    point."""
    shape = synth.PrefillShape(2, 53, 2, 4, 64, 32, dt, "normal", s0_std=0.3)
    inp = synth.make_prefill_inputs(shape, DEV, 11)
    inp["g"] = unbounded_gate(shape.B, shape.T, shape.HV, shape.K, 12).to(DEV)
    sl = lambda x, a, b: x[:, a:b].contiguous()
    args = lambda a, b: (sl(inp["q"], a, b), sl(inp["k"], a, b), sl(inp["v"], a, b),
                         sl(inp["g"], a, b), sl(inp["beta"], a, b))
    o_full, S_full = kda.recurrent_fwd(*args(0, 53), initial_state=inp["S0"], output_final_state=True)
    for split in (1, 16, 21, 32, 52):
        say("   split at", split)
        o1, S1 = kda.recurrent_fwd(*args(0, split), initial_state=inp["S0"], output_final_state=True)
        o2, S2 = kda.recurrent_fwd(*args(split, 53), initial_state=S1, output_final_state=True)
        torch.cuda.synchronize()
        assert torch.equal(o1, o_full[:, :split]), "prefix outputs changed (split %d)" % split
        assert torch.equal(o2, o_full[:, split:]), "resumed outputs differ (split %d)" % split
        assert torch.equal(S2, S_full), "resumed final state differs (split %d)" % split
