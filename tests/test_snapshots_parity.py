"""GPU parity of kda_chunk_fwd_snapshots (prefix snapshots of the state)
against the fp64 oracle's snapshots, plus the properties that tie them to the
rest of the library: o and the final state are bit-identical to
kda_chunk_fwd's, and decoding from a snapshot continues the sequence."""
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


def run_snap(shape, every, seed=0, g_lower=None, label=""):
    say("snapshot case", label, shape, "every", every, "seed", seed)
    inp = synth.make_prefill_inputs(shape, DEV, seed, g_lower=g_lower)
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    o, S, snaps = kda.chunk_fwd_snapshots(*args, every, initial_state=inp["S0"],
                                          output_final_state=True)
    o_plain, S_plain = kda.chunk_fwd(*args, initial_state=inp["S0"], output_final_state=True)
    torch.cuda.synchronize()
    assert snaps.shape == (shape.B, shape.T // every, shape.HV, shape.K, shape.V)
    # taking snapshots changes nothing else, bit for bit
    assert torch.equal(o, o_plain) and torch.equal(S, S_plain)
    _, Sref, snref = oracle.kda_fwd(*args, initial_state=inp["S0"], snapshot_every=every)
    for j in range(snaps.shape[1]):
        m = assert_close(snaps[:, j], snref[:, j], shape.dtype, False, "snapshot %d %s" % (j, label))
        if j == 0 or j == snaps.shape[1] - 1:
            say("   snapshot", j, m)
    if shape.T % every == 0 and shape.T > 0:
        assert torch.equal(snaps[:, -1], S)
    return inp, o, S, snaps


CASES = [
    # B, T, H, HV, K, V, dtype, every
    (2, 200, 2, 4, 128, 64, torch.bfloat16, 32),      # ragged tail, 6 snapshots, VT 32 x 2
    (1, 256, 1, 2, 128, 128, torch.bfloat16, 64),     # T a multiple: last snapshot = S_T
    (3, 191, 1, 3, 64, 64, torch.bfloat16, 96),
    (2, 100, 2, 2, 32, 32, torch.bfloat16, 32),
    (1, 320, 4, 160, 128, 128, torch.bfloat16, 128),  # 160 chains: VT = V = 128 workgroups
    (2, 150, 2, 4, 128, 64, torch.float32, 32),
    (1, 96, 1, 1, 32, 32, torch.float32, 64),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dT%dH%dHV%dK%dV%d-%s-e%d" % (
    c[:6] + (str(c[6]).split(".")[-1], c[7])))
def test_snapshots_match_oracle(case):
    B, T, H, HV, K, V, dt, every = case
    shape = synth.PrefillShape(B, T, H, HV, K, V, dt, "normal", s0_std=0.3)
    run_snap(shape, every, seed=B * 7 + T, label=str(case))


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_snapshots_long_memory(dt):
    """g = -0.05 sigmoid(N(0,1)): the state carries over many chunks."""
    shape = synth.PrefillShape(2, 500, 2, 4, 64, 64, dt, "normal", s0_std=0.3)
    run_snap(shape, 64, seed=3, g_lower=-0.05, label="long " + str(dt))


def test_snapshots_shorter_than_interval():
    """T < snapshot_every: no snapshots, everything else as kda_chunk_fwd."""
    shape = synth.PrefillShape(1, 50, 1, 2, 64, 64, torch.bfloat16, "normal")
    _, _, _, snaps = run_snap(shape, 64, label="none")
    assert snaps.shape[1] == 0


def test_decode_resumes_from_snapshot():
    """The prefix cache use: decode the tokens after snapshot j from it, and
    compare with the prefill's outputs for those tokens (and the oracle)."""
    shape = synth.PrefillShape(2, 160, 2, 4, 64, 64, torch.float32, "normal", s0_std=0.3)
    inp = synth.make_prefill_inputs(shape, DEV, 11)
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    o, S, snaps = kda.chunk_fwd_snapshots(*args, 64, initial_state=inp["S0"],
                                          output_final_state=True)
    j, every = 1, 64
    t0 = (j + 1) * every
    state = snaps[:, j].clone()
    B, H, HV, K, V = shape.B, shape.H, shape.HV, shape.K, shape.V
    outs = []
    for t in range(t0, shape.T):
        qkv = torch.cat([inp["q"][:, t].reshape(B, H * K), inp["k"][:, t].reshape(B, H * K),
                         inp["v"][:, t].reshape(B, HV * V)], dim=1).contiguous()
        outs.append(kda.decode_step(qkv, inp["g"][:, t].contiguous(), inp["beta"][:, t].contiguous(),
                                    state, H=H, HV=HV, K=K, V=V))
    torch.cuda.synchronize()
    o_dec = torch.stack(outs, 1)
    oref, Sref = oracle.kda_fwd(*args, initial_state=inp["S0"])
    assert_close(o_dec, oref[:, t0:], torch.float32, True, "decode from snapshot")
    assert_close(state, Sref, torch.float32, False, "state after decode from snapshot")
    assert_close(o[:, t0:], oref[:, t0:], torch.float32, True, "prefill tail")


def test_full_size_hv96_snapshots_sampled():
    """B1 T8192 H=HV=96 K=V=128 bf16 in the benchmark's launch configuration,
    a snapshot every 1024 tokens; whole chains checked against the oracle."""
    shape = synth.PREFILL_HV96_BF16
    every = 1024
    say("full-size snapshots", shape, "every", every)
    inp = synth.make_prefill_inputs(shape, DEV, 0)
    o, S, snaps = kda.chunk_fwd_snapshots(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                          every, initial_state=inp["S0"], output_final_state=True)
    torch.cuda.synchronize()
    assert torch.equal(snaps[:, -1], S)
    for hv in (3, 50, 95):
        sub = lambda x: x[:, :, hv:hv + 1]
        _, _, snref = oracle.kda_fwd(sub(inp["q"]), sub(inp["k"]), sub(inp["v"]), sub(inp["g"]),
                                     inp["beta"][:, :, hv:hv + 1],
                                     initial_state=inp["S0"][:, hv:hv + 1], snapshot_every=every)
        for j in range(snaps.shape[1]):
            assert_close(snaps[:, j, hv:hv + 1], snref[:, j], torch.bfloat16, False,
                         "HV96 snapshot %d hv %d" % (j, hv))
        say("   hv", hv, "ok")
