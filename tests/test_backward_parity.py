"""GPU parity of kda_recurrent_bwd (the backward of the forward pass) against
the fp64 oracle's back-propagation through time, which the CPU suite checks
against finite differences."""
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
NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dS0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def unbounded_gate(B, T, HV, K, seed):
    """g = -exp(A_log) * softplus(z + dt_bias), no lower bound (the kda.rs
    page's bounded_gate without its bound), A_log, dt_bias, z ~ N(0,1)."""
    gen = torch.Generator(device="cpu").manual_seed(seed)
    A_log = torch.randn(HV, generator=gen)
    dt = torch.randn(HV * K, generator=gen)
    z = torch.randn(B, T, HV * K, generator=gen) * 2.0
    g = -torch.exp(A_log).repeat_interleave(K) * torch.nn.functional.softplus(z + dt)
    return g.view(B, T, HV, K).contiguous()


def run(shape, seed, gate="bounded", with_dst=True, label=""):
    say("backward case", label, shape, "seed", seed, "gate", gate, "dS_T", with_dst)
    inp = synth.make_prefill_inputs(shape, DEV, seed)
    if gate == "unbounded":
        inp["g"] = unbounded_gate(shape.B, shape.T, shape.HV, shape.K, seed + 1).to(DEV)
    gen = torch.Generator(device="cpu").manual_seed(seed + 2)
    dout = torch.randn(shape.B, shape.T, shape.HV, shape.V, generator=gen).to(shape.dtype).to(DEV)
    dST = (torch.randn(shape.B, shape.HV, shape.K, shape.V, generator=gen) * 0.1).to(DEV) if with_dst else None
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    got = kda.recurrent_bwd(*args, dout, dST, initial_state=inp["S0"])
    torch.cuda.synchronize()
    ref = oracle.kda_bwd(*args, dout, dST, initial_state=inp["S0"])
    stored = (True, True, True, False, False, False)
    for name, gpu, want, st in zip(NAMES, got, ref, stored):
        m = assert_close(gpu, want, shape.dtype, st, "%s %s" % (name, label))
        say("   %-6s max_rel %.2e  excess/rms %.2e" % (name, m["max_rel"], m["excess_over_rms"]))
    return inp, dout, dST, got


CASES = [
    # B, T, H, HV, K, V, dtype
    (2, 37, 1, 2, 32, 32, torch.float32),
    (1, 70, 2, 4, 64, 64, torch.bfloat16),
    (2, 100, 2, 2, 128, 128, torch.float32),
    (1, 45, 1, 3, 128, 64, torch.bfloat16),
    (1, 1, 1, 1, 32, 32, torch.float32),
    (3, 9, 2, 2, 64, 128, torch.bfloat16),
    (2, 33, 2, 2, 64, 128, torch.float32),
    (1, 24, 1, 4, 32, 128, torch.bfloat16),
    (1, 19, 1, 1, 128, 32, torch.float32),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dT%dH%dHV%dK%dV%d-%s" % (
    c[:6] + (str(c[6]).split(".")[-1],)))
@pytest.mark.parametrize("gate,with_dst", [("bounded", True), ("unbounded", False)])
def test_backward_matches_oracle(case, gate, with_dst):
    B, T, H, HV, K, V, dt = case
    shape = synth.PrefillShape(B, T, H, HV, K, V, dt, "normal", s0_std=0.3)
    run(shape, seed=T + K + V, gate=gate, with_dst=with_dst, label=str(case))


def test_backward_empty_sequence():
    """T = 0: dS0 = dL/dS_T, and nothing else is written."""
    B, H, HV, K, V = 2, 1, 2, 64, 32
    z = lambda *s, dt=torch.float32: torch.zeros(*s, dtype=dt, device=DEV)
    dST = torch.randn(B, HV, K, V, device=DEV)
    got = kda.recurrent_bwd(z(B, 0, H, K), z(B, 0, H, K), z(B, 0, HV, V), z(B, 0, HV, K), z(B, 0, HV),
                            z(B, 0, HV, V), dST)
    torch.cuda.synchronize()
    assert torch.equal(got[5], dST)
    got = kda.recurrent_bwd(z(B, 0, H, K), z(B, 0, H, K), z(B, 0, HV, V), z(B, 0, HV, K), z(B, 0, HV),
                            z(B, 0, HV, V), None)
    torch.cuda.synchronize()
    assert torch.count_nonzero(got[5]) == 0


def test_backward_workspace_reuse_and_determinism():
    """The same call twice through one workspace (with other sizes in between)
    gives bitwise equal gradients."""
    shape = synth.PrefillShape(2, 50, 2, 4, 64, 64, torch.bfloat16, "normal", s0_std=0.3)
    inp = synth.make_prefill_inputs(shape, DEV, 5)
    dout = torch.randn(2, 50, 4, 64, device=DEV).to(torch.bfloat16)
    nbytes = kda.recurrent_bwd_workspace_size(2, 50, 2, 4, 64, 64)
    ws = torch.full((nbytes,), 0x7f, dtype=torch.uint8, device=DEV)
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], dout)
    a = kda.recurrent_bwd(*args, initial_state=inp["S0"], workspace=ws)
    small = synth.make_prefill_inputs(synth.PrefillShape(1, 7, 1, 1, 32, 32, torch.bfloat16, "normal"), DEV, 6)
    kda.recurrent_bwd(small["q"], small["k"], small["v"], small["g"], small["beta"],
                      torch.ones(1, 7, 1, 32, device=DEV, dtype=torch.bfloat16), workspace=ws)
    b = kda.recurrent_bwd(*args, initial_state=inp["S0"], workspace=ws)
    torch.cuda.synchronize()
    for name, x, y in zip(NAMES, a, b):
        assert torch.equal(x, y), name


def test_full_size_hv96_backward_sampled():
    """The HV96 workload at its full length, as the benchmark times it (B1
    T8192 H=HV=96 K=V=128 bf16, bounded gate, dL/dS_T given): heads 0 and 95
    against the oracle run on just those heads."""
    shape = synth.PrefillShape(1, 8192, 96, 96, 128, 128, torch.bfloat16, "none")
    say("full-width backward", shape)
    inp = synth.make_prefill_inputs(shape, DEV, 0)
    gen = torch.Generator(device="cpu").manual_seed(3)
    dout = torch.randn(1, 8192, 96, 128, generator=gen).to(torch.bfloat16).to(DEV)
    dST = (torch.randn(1, 96, 128, 128, generator=gen) * 0.1).to(DEV)
    got = kda.recurrent_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], dout, dST)
    torch.cuda.synchronize()
    for hv in (0, 95):
        sub = lambda x: x[:, :, hv:hv + 1]
        ref = oracle.kda_bwd(sub(inp["q"]), sub(inp["k"]), sub(inp["v"]), sub(inp["g"]),
                             inp["beta"][:, :, hv:hv + 1], sub(dout), dST[:, hv:hv + 1])
        part = (got[0][:, :, hv:hv + 1], got[1][:, :, hv:hv + 1], got[2][:, :, hv:hv + 1],
                got[3][:, :, hv:hv + 1], got[4][:, :, hv:hv + 1], got[5][:, hv:hv + 1])
        for name, gpu, want, st in zip(NAMES, part, ref, (True, True, True, False, False, False)):
            m = assert_close(gpu, want, torch.bfloat16, st, "HV96 %s head %d" % (name, hv))
            say("   head %d %-6s max_rel %.2e  excess/rms %.2e" % (hv, name, m["max_rel"],
                                                                 m["excess_over_rms"]))


LONG_MEMORY = [
    # B, T, H, HV, K, V, dtype: g = -0.05 sigmoid(N(0,1)), so the state keeps
    # most of its past over the whole sequence and dg sums over hundreds of
    # tokens of slowly decaying terms
    (1, 1024, 2, 2, 128, 128, torch.bfloat16),
    (1, 2048, 1, 1, 128, 128, torch.float32),
    (2, 512, 1, 2, 64, 64, torch.float32),
    (1, 600, 1, 2, 128, 64, torch.bfloat16),
]


@pytest.mark.parametrize("case", LONG_MEMORY, ids=lambda c: "B%dT%dH%dHV%dK%dV%d-%s" % (
    c[:6] + (str(c[6]).split(".")[-1],)))
def test_backward_long_memory(case):
    B, T, H, HV, K, V, dt = case
    shape = synth.PrefillShape(B, T, H, HV, K, V, dt, "normal", s0_std=0.3, g_lower=-0.05)
    run(shape, seed=T + 1, gate="bounded", with_dst=True, label="long memory " + str(case))


SLABS = [
    # B, T, H, HV, K, V, dtype: sequences longer than one slab of 1024 tokens,
    # so the state gradient, the forward states and the dg sum cross slab
    # boundaries (a last slab of 76 tokens; of 1 token; three slabs with GQA)
    (2, 1100, 1, 2, 64, 64, torch.bfloat16),
    (1, 1025, 2, 2, 32, 32, torch.float32),
    (1, 2100, 1, 4, 128, 32, torch.float32),
]


@pytest.mark.parametrize("case", SLABS, ids=lambda c: "B%dT%dH%dHV%dK%dV%d-%s" % (
    c[:6] + (str(c[6]).split(".")[-1],)))
@pytest.mark.parametrize("gate", ["bounded", "unbounded"])
def test_backward_across_slabs(case, gate):
    B, T, H, HV, K, V, dt = case
    shape = synth.PrefillShape(B, T, H, HV, K, V, dt, "normal", s0_std=0.3, g_lower=-1.0)
    run(shape, seed=T + 7, gate=gate, with_dst=True, label="slabs " + str(case))


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_backward_beta_zero(dt):
    """beta = 0: nothing is written, so dL/dv = 0 exactly and
    dS0 = exp(G_T) (.) dS_T + sum_t exp(G_t) (.) (s q_t (x) dout_t)
    (the state only decays; G_t the cumulative sum of g up to t); all six
    gradients also against the oracle."""
    B, T, H, HV, K, V = 1, 300, 1, 2, 64, 64
    shape = synth.PrefillShape(B, T, H, HV, K, V, dt, "normal", s0_std=0.3, g_lower=-0.2)
    inp = synth.make_prefill_inputs(shape, DEV, 31)
    inp["beta"].zero_()
    gen = torch.Generator(device="cpu").manual_seed(32)
    dout = torch.randn(B, T, HV, V, generator=gen).to(dt).to(DEV)
    dST = (torch.randn(B, HV, K, V, generator=gen) * 0.1).to(DEV)
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    got = kda.recurrent_bwd(*args, dout, dST, initial_state=inp["S0"])
    torch.cuda.synchronize()
    assert torch.count_nonzero(got[2]) == 0, "dv must vanish when nothing is written"
    s = 1.0 / np.sqrt(K)
    q, g, do = np64(inp["q"])[0, :, 0], np64(inp["g"])[0], np64(dout)[0]
    for hv in range(HV):
        G = np.cumsum(g[:, hv], axis=0)                                  # [T, K]
        want = np.exp(G[-1])[:, None] * np64(dST)[0, hv]
        want = want + (np.exp(G) * (s * q)).T @ do[:, hv]                 # [K, V]
        assert_close(got[5][0, hv], want, dt, False, "beta=0 dS0 head %d" % hv)
    ref = oracle.kda_bwd(*args, dout, dST, initial_state=inp["S0"])
    for name, gpu, want, st in zip(NAMES, got, ref, (True, True, True, False, False, False)):
        m = assert_close(gpu, want, dt, st, "beta=0 %s" % name)
        say("   beta=0 %-6s max_rel %.2e  excess/rms %.2e" % (name, m["max_rel"], m["excess_over_rms"]))


@pytest.mark.parametrize("chunked,dt", [(True, torch.bfloat16), (False, torch.float32)])
def test_autograd_function_matches_oracle(chunked, dt):
    """kda.kda (forward kernel + kda_recurrent_bwd under torch.autograd): the
    gradients of L = sum(o * Wo) + sum(S_T * WS) reach every input and equal
    the oracle's."""
    shape = synth.PrefillShape(2, 41, 1, 2, 64, 64, dt, "normal", s0_std=0.3)
    inp = synth.make_prefill_inputs(shape, DEV, 17)
    gen = torch.Generator(device="cpu").manual_seed(18)
    Wo = torch.randn(2, 41, 2, 64, generator=gen).to(dt).to(DEV)
    WS = (torch.randn(2, 2, 64, 64, generator=gen) * 0.1).to(DEV)
    leaves = {n: inp[n].clone().requires_grad_(True) for n in ("q", "k", "v", "g", "beta", "S0")}
    o, S = kda.kda(leaves["q"], leaves["k"], leaves["v"], leaves["g"], leaves["beta"],
                   initial_state=leaves["S0"], output_final_state=True, chunked=chunked)
    ((o.float() * Wo.float()).sum() + (S * WS).sum()).backward()
    torch.cuda.synchronize()
    ref = oracle.kda_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], Wo, WS, initial_state=inp["S0"])
    for name, want, st in zip(("q", "k", "v", "g", "beta", "S0"), ref, (True, True, True, False, False, False)):
        assert leaves[name].grad is not None, name
        assert_close(leaves[name].grad, want, dt, st, "autograd d%s" % name)
