"""An explicit output scale, not the default 1/sqrt(K), through every entry
point that takes one, each against the oracle given the same scale: the
chunked forward (bf16 and fp32), its snapshot form, the chunked unbounded
form and the token recurrence, both backward forms and the saved-states
backward, and the decode step.  The scale multiplies every output row
(o = s q S) and enters dq and, through dA_qk, dk."""
import sys

import pytest
import torch

import gated_delta_rule_kda_amd as kda
import oracle
from gated_delta_rule_kda_amd import synth
from kda_testutil import assert_close, gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda"
S = 0.37          # K = 64 below: 1/sqrt(K) would be 0.125
NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dS0")
STORED = (True, True, True, False, False, False)   # gradients stored in the input dtype


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def shape_of(dt, T=70):
    return synth.PrefillShape(1, T, 1, 2, 64, 32, dt, "normal", s0_std=0.3)


def check_fwd(o, St, inp, dt, label, snaps=None, every=None):
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    ref = oracle.kda_fwd(*args, scale=S, initial_state=inp["S0"], snapshot_every=every)
    assert_close(o, ref[0], dt, True, "o " + label)
    assert_close(St, ref[1], dt, False, "S_T " + label)
    if snaps is not None:
        assert_close(snaps, ref[2], dt, False, "snapshots " + label)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_scale_chunk_fwd(dt):
    say("chunk_fwd scale", S, dt)
    inp = synth.make_prefill_inputs(shape_of(dt), DEV, 1)
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    o, St = kda.chunk_fwd(*args, scale=S, initial_state=inp["S0"], output_final_state=True)
    torch.cuda.synchronize()
    check_fwd(o, St, inp, dt, "chunk_fwd")
    o, St, sn = kda.chunk_fwd_snapshots(*args, 32, scale=S, initial_state=inp["S0"], output_final_state=True)
    torch.cuda.synchronize()
    check_fwd(o, St, inp, dt, "chunk_fwd_snapshots", sn, 32)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_scale_unbounded_forms(dt):
    say("unbounded forms scale", S, dt)
    inp = synth.make_prefill_inputs(shape_of(dt), DEV, 2, g_heavy=True)
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    o, St = kda.recurrent_fwd(*args, scale=S, initial_state=inp["S0"], output_final_state=True)
    torch.cuda.synchronize()
    check_fwd(o, St, inp, dt, "recurrent_fwd")
    if dt == torch.bfloat16:
        o, St = kda.chunk_fwd_unbounded(*args, scale=S, initial_state=inp["S0"], output_final_state=True)
        torch.cuda.synchronize()
        check_fwd(o, St, inp, dt, "chunk_fwd_unbounded")


def check_bwd(got, inp, dout, dST, dt, label):
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    ref = oracle.kda_bwd(*args, dout, dST, scale=S, initial_state=inp["S0"])
    for name, gpu, want, st in zip(NAMES, got, ref, STORED):
        m = assert_close(gpu, want, dt, st, "%s %s" % (name, label))
        say("   %-6s %s" % (name, {k: m[k] for k in ("max_rel", "excess_over_rms")}))


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_scale_backward(dt):
    say("backward scale", S, dt)
    shape = shape_of(dt)
    inp = synth.make_prefill_inputs(shape, DEV, 3)
    gen = torch.Generator(device="cpu").manual_seed(4)
    dout = torch.randn(shape.B, shape.T, shape.HV, shape.V, generator=gen).to(dt).to(DEV)
    dST = (0.1 * torch.randn(shape.B, shape.HV, shape.K, shape.V, generator=gen)).to(DEV)
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    got = kda.recurrent_bwd(*args, dout, dST, scale=S, initial_state=inp["S0"])
    torch.cuda.synchronize()
    check_bwd(got, inp, dout, dST, dt, "recurrent_bwd")
    if dt == torch.bfloat16:
        got = kda.chunk_bwd(*args, dout, dST, scale=S, initial_state=inp["S0"])
        torch.cuda.synchronize()
        check_bwd(got, inp, dout, dST, dt, "chunk_bwd")


def test_scale_chunk_bwd_saved_two_slabs():
    """Two slabs of 1024 tokens: the saved states from the snapshot form with
    the same scale (the states themselves do not depend on it)."""
    dt = torch.bfloat16
    say("chunk_bwd_saved scale", S, "T 1100")
    shape = shape_of(dt, T=1100)
    inp = synth.make_prefill_inputs(shape, DEV, 5)
    gen = torch.Generator(device="cpu").manual_seed(6)
    dout = torch.randn(shape.B, shape.T, shape.HV, shape.V, generator=gen).to(dt).to(DEV)
    dST = (0.1 * torch.randn(shape.B, shape.HV, shape.K, shape.V, generator=gen)).to(DEV)
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    _, St, sn = kda.chunk_fwd_snapshots(*args, 1024, scale=S, initial_state=inp["S0"], output_final_state=True)
    got = kda.chunk_bwd(*args, dout, dST, scale=S, initial_state=inp["S0"], saved_states=sn, final_state=St)
    torch.cuda.synchronize()
    check_bwd(got, inp, dout, dST, dt, "chunk_bwd_saved")


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_scale_decode(dt):
    """Plain decode steps (g, beta given) against the oracle's forward over the
    same tokens."""
    say("decode scale", S, dt)
    shape = synth.PrefillShape(3, 10, 1, 2, 64, 32, dt, "normal", s0_std=0.3)
    inp = synth.make_prefill_inputs(shape, DEV, 7)
    B, T = shape.B, shape.T
    state = inp["S0"].clone()
    outs = []
    for t in range(T):
        x = torch.cat([inp["q"][:, t].reshape(B, -1), inp["k"][:, t].reshape(B, -1),
                       inp["v"][:, t].reshape(B, -1)], dim=1).contiguous()
        outs.append(kda.decode_step(x, inp["g"][:, t].contiguous(), inp["beta"][:, t].contiguous(), state,
                                    H=shape.H, HV=shape.HV, K=shape.K, V=shape.V, scale=S))
    torch.cuda.synchronize()
    check_fwd(torch.stack(outs, 1), state, inp, dt, "decode")
