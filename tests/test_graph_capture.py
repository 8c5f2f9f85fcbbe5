"""HIP graph capture of the entry points a serving or training loop would
capture: kda_chunk_fwd, kda_chunk_fwd_unbounded (its two kernels), and
kda_chunk_bwd / kda_chunk_bwd_saved (eagerly on three streams joined by
events; while captured, every pass in order on the captured stream).  Each graph is replayed several times, with new input values written
in place and the program's own eager work and synchronizations between the
replays, and every replay must give the eager call's bits on those inputs."""
import sys

import pytest
import torch

import gated_delta_rule_kda_amd as kda
from gated_delta_rule_kda_amd import synth
from kda_testutil import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def refill(inp, shape, seed, heavy=False):
    """New input values, written into the captured tensors in place."""
    fresh = synth.make_prefill_inputs(shape, DEV, seed, g_heavy=heavy)
    for n in ("q", "k", "v", "g", "beta"):
        inp[n].copy_(fresh[n])
    if inp["S0"] is not None:
        inp["S0"].copy_(fresh["S0"])


def replay_and_check(capture, eager, refill_fn, n=3):
    """Capture `capture` into a graph, then per replay: new inputs, an eager
    call (the reference), a replay, and a bitwise comparison."""
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say("   capture")
    with torch.cuda.graph(g):
        outs = capture()
    torch.cuda.synchronize()
    for r in range(n):
        say("   replay", r, ": new inputs, eager call")
        refill_fn(100 + r)
        torch.cuda.synchronize()
        want = [t.clone() for t in eager() if t is not None]
        torch.cuda.synchronize()
        say("   replay", r, ": graph")
        g.replay()
        torch.cuda.synchronize()
        got = [t for t in outs if t is not None]
        for i, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a, b), "replay %d output %d differs from the eager call" % (r, i)
        say("   replay", r, "ok")


def test_graph_chunk_fwd():
    shape = synth.PrefillShape(2, 200, 2, 4, 64, 64, torch.bfloat16, "normal", s0_std=0.3)
    inp = synth.make_prefill_inputs(shape, DEV, 1)
    out = torch.empty(2, 200, 4, 64, dtype=torch.bfloat16, device=DEV)
    ST = torch.empty(2, 4, 64, 64, device=DEV)
    args = lambda: (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    run = lambda o, s: kda.chunk_fwd(*args(), initial_state=inp["S0"], out=o, final_state=s)
    say("chunk_fwd B2 T200 H2 HV4 K64 V64: eager")
    run(out, ST)   # eager first
    replay_and_check(lambda: run(out, ST), lambda: run(torch.empty_like(out), torch.empty_like(ST)),
                     lambda seed: refill(inp, shape, seed))


def test_graph_chunk_fwd_unbounded():
    shape = synth.PrefillShape(1, 300, 1, 2, 128, 64, torch.bfloat16, "normal", s0_std=0.3)
    inp = synth.make_prefill_inputs(shape, DEV, 2, g_heavy=True)
    out = torch.empty(1, 300, 2, 64, dtype=torch.bfloat16, device=DEV)
    ST = torch.empty(1, 2, 128, 64, device=DEV)
    ws = torch.empty(kda.chunk_fwd_unbounded_workspace_size(1, 300, 1, 2, 128, 64), dtype=torch.uint8, device=DEV)
    ws2 = torch.empty_like(ws)
    args = lambda: (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    run = lambda o, s, w: kda.chunk_fwd_unbounded(*args(), initial_state=inp["S0"], out=o, final_state=s,
                                                  workspace=w)
    say("chunk_fwd_unbounded B1 T300 H1 HV2 K128 V64: eager")
    run(out, ST, ws)
    replay_and_check(lambda: run(out, ST, ws), lambda: run(torch.empty_like(out), torch.empty_like(ST), ws2),
                     lambda seed: refill(inp, shape, seed, heavy=True))


@pytest.mark.parametrize("saved", [False, True])
def test_graph_chunk_bwd(saved):
    """Three slabs (T = 2100): the library's two side streams fork from and
    join the captured stream through its events."""
    B, T, H, HV, K, V = 1, 2100, 1, 2, 64, 64
    shape = synth.PrefillShape(B, T, H, HV, K, V, torch.bfloat16, "normal", s0_std=0.3, g_lower=-1.0)
    inp = synth.make_prefill_inputs(shape, DEV, 3)
    gen = torch.Generator(device="cpu").manual_seed(4)
    dout = torch.randn(B, T, HV, V, generator=gen).to(torch.bfloat16).to(DEV)
    dST = (torch.randn(B, HV, K, V, generator=gen) * 0.1).to(DEV)
    ws = torch.empty(kda.chunk_bwd_workspace_size(B, T, H, HV, K, V), dtype=torch.uint8, device=DEV)
    ws2 = torch.empty_like(ws)
    snaps = torch.empty(B, T // 1024, HV, K, V, device=DEV)
    ST = torch.empty(B, HV, K, V, device=DEV)
    fo = torch.empty(B, T, HV, V, dtype=torch.bfloat16, device=DEV)
    args = lambda: (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])

    def mk_outs():
        return (torch.empty(B, T, H, K, dtype=torch.bfloat16, device=DEV),
                torch.empty(B, T, H, K, dtype=torch.bfloat16, device=DEV),
                torch.empty(B, T, HV, V, dtype=torch.bfloat16, device=DEV),
                torch.empty(B, T, HV, K, device=DEV), torch.empty(B, T, HV, device=DEV),
                torch.empty(B, HV, K, V, device=DEV))
    outs = mk_outs()

    def run(o, w):
        if saved:
            kda.chunk_fwd_snapshots(*args(), 1024, initial_state=inp["S0"], out=fo, final_state=ST,
                                    snapshots=snaps)
            return kda.chunk_bwd(*args(), dout, dST, initial_state=inp["S0"], workspace=w, out=o,
                                 saved_states=snaps, final_state=ST)
        return kda.chunk_bwd(*args(), dout, dST, initial_state=inp["S0"], workspace=w, out=o)
    say("chunk_bwd saved=%s B1 T2100 H1 HV2 K64 V64: eager" % saved)
    run(outs, ws)
    replay_and_check(lambda: run(outs, ws), lambda: run(mk_outs(), ws2),
                     lambda seed: refill(inp, shape, seed))
