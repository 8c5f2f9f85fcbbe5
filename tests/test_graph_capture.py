"""HIP graph capture of the entry points a serving or training loop would
capture: kda_chunk_fwd, kda_chunk_fwd_unbounded (its two kernels), and
kda_chunk_bwd / kda_chunk_bwd_saved (eagerly on four streams joined by
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
    """Three slabs (T = 2100): captured, the passes run in order on the
    captured stream; each replay must give the eager call's bits, which runs
    them on four streams joined by events."""
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


def test_graph_decode_steps():
    """Two fused decode steps (conv width 4 + SiLU, L2 norm, bounded gate,
    beta logits) in one graph; state and conv registers updated in place."""
    B, H, HV, K, V, KW = 4, 2, 4, 64, 64, 4
    C = 2 * H * K + HV * V
    say("decode B4 H2 HV4 K64 V64 KW4, two steps: eager")
    gen = torch.Generator(device="cpu").manual_seed(11)
    r = lambda *s_: torch.randn(*s_, generator=gen).to(DEV)
    conv_w, A_log, dt_bias = r(C, KW), r(HV), r(HV * K)
    xs = [torch.empty(B, C, dtype=torch.bfloat16, device=DEV) for _ in range(2)]
    zs = [torch.empty(B, HV, K, device=DEV) for _ in range(2)]
    bls = [torch.empty(B, HV, device=DEV) for _ in range(2)]
    state = torch.empty(B, HV, K, V, device=DEV)
    conv = torch.empty(B, C, KW, device=DEV)
    outs = [torch.empty(B, HV, V, dtype=torch.bfloat16, device=DEV) for _ in range(2)]

    def refill_fn(seed):
        g2 = torch.Generator(device="cpu").manual_seed(seed)
        rr = lambda *s_: torch.randn(*s_, generator=g2).to(DEV)
        for i in range(2):
            xs[i].copy_(rr(B, C))
            zs[i].copy_(rr(B, HV, K))
            bls[i].copy_(rr(B, HV))
        state.copy_(0.1 * rr(B, HV, K, V))
        conv.copy_(rr(B, C, KW))

    def steps(st, cv, o):
        for i in range(2):
            kda.decode_step(xs[i], zs[i], bls[i], st, H=H, HV=HV, K=K, V=V, out=o[i], conv_weight=conv_w,
                            conv_state=cv, l2norm_qk=True, l2_eps=1e-6, gate_mode=kda.GATE_BOUNDED,
                            A_log=A_log, dt_bias=dt_bias, gate_lower_bound=-5.0, beta_is_logit=True)
        return list(o) + [st, cv]

    def eager():
        return steps(state.clone(), conv.clone(), [torch.empty_like(o) for o in outs])

    refill_fn(1)
    eager()
    replay_and_check(lambda: steps(state, conv, outs), eager, refill_fn)


def test_graph_decode_ring_rotation():
    """The ring layout of the conv registers under capture: the slot of the
    oldest register is an argument of the call, so a loop captures one graph
    per slot (KW of them) and replays them in turn.  Nine steps through the
    three graphs of a width-3 ring against the same steps eagerly, every step
    bit for bit (outputs, state and the ring)."""
    B, H, HV, K, V, KW = 2, 2, 2, 64, 64, 3
    C = 2 * H * K + HV * V
    say("decode ring B2 H2 HV2 K64 V64 KW3: one graph per slot")
    gen = torch.Generator(device="cpu").manual_seed(13)
    r = lambda *s_: torch.randn(*s_, generator=gen).to(DEV)
    conv_w, A_log, dt_bias = r(C, KW), r(HV), r(HV * K)
    x = torch.empty(B, C, device=DEV)
    z = torch.empty(B, HV, K, device=DEV)
    bl = torch.empty(B, HV, device=DEV)
    out = torch.empty(B, HV, V, device=DEV)
    state = 0.1 * r(B, HV, K, V)
    ring = r(KW, B, C)
    st_e, ring_e = state.clone(), ring.clone()
    kw = dict(H=H, HV=HV, K=K, V=V, conv_weight=conv_w, l2norm_qk=True, l2_eps=1e-6,
              gate_mode=kda.GATE_BOUNDED, A_log=A_log, dt_bias=dt_bias, gate_lower_bound=-5.0,
              beta_is_logit=True, conv_ring=True)
    torch.cuda.synchronize()
    # capturing records the work without running it: state and ring stay as they are
    graphs = []
    for pos in range(KW):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            kda.decode_step(x, z, bl, state, out=out, conv_state=ring, conv_pos=pos, **kw)
        graphs.append(g)
    torch.cuda.synchronize()
    for t in range(3 * KW):
        x.copy_(r(B, C))
        z.copy_(r(B, HV, K))
        bl.copy_(r(B, HV))
        want = kda.decode_step(x, z, bl, st_e, conv_state=ring_e, conv_pos=t % KW, **kw)
        torch.cuda.synchronize()
        graphs[t % KW].replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), ("out", t)
        assert torch.equal(state, st_e), ("state", t)
        assert torch.equal(ring, ring_e), ("ring", t)
        say("   step", t, "slot", t % KW, "ok")


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_graph_recurrent_fwd_bwd(dt):
    """kda_recurrent_fwd, then kda_recurrent_bwd and kda_recurrent_bwd_noalloc
    (the library's scratch array in place of a workspace) on its inputs, in
    one graph."""
    B, T, H, HV, K, V = 1, 150, 1, 2, 64, 32
    say("recurrent fwd + bwd B1 T150 H1 HV2 K64 V32 %s: eager" % dt)
    shape = synth.PrefillShape(B, T, H, HV, K, V, dt, "normal", s0_std=0.3)
    inp = synth.make_prefill_inputs(shape, DEV, 5, g_heavy=True)
    dout = torch.empty(B, T, HV, V, dtype=dt, device=DEV)
    dST = torch.empty(B, HV, K, V, device=DEV)
    ws = torch.empty(kda.recurrent_bwd_workspace_size(B, T, H, HV, K, V), dtype=torch.uint8, device=DEV)
    ws2 = torch.empty_like(ws)

    def grads():
        return (torch.empty(B, T, H, K, dtype=dt, device=DEV), torch.empty(B, T, H, K, dtype=dt, device=DEV),
                torch.empty(B, T, HV, V, dtype=dt, device=DEV), torch.empty(B, T, HV, K, device=DEV),
                torch.empty(B, T, HV, device=DEV), torch.empty(B, HV, K, V, device=DEV))

    def mk():
        return (torch.empty(B, T, HV, V, dtype=dt, device=DEV), torch.empty(B, HV, K, V, device=DEV),
                grads(), grads())
    cap = mk()

    def refill_fn(seed):
        refill(inp, shape, seed, heavy=True)
        g2 = torch.Generator(device="cpu").manual_seed(seed)
        dout.copy_(torch.randn(B, T, HV, V, generator=g2).to(dt))
        dST.copy_(0.1 * torch.randn(B, HV, K, V, generator=g2))

    def run(o, w):
        a = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
        kda.recurrent_fwd(*a, initial_state=inp["S0"], out=o[0], final_state=o[1])
        kda.recurrent_bwd(*a, dout, dST, initial_state=inp["S0"], workspace=w, out=o[2])
        kda.recurrent_bwd_noalloc(*a, dout, dST, initial_state=inp["S0"], out=o[3])
        return [o[0], o[1]] + list(o[2]) + list(o[3])

    refill_fn(6)
    run(mk(), ws2)
    replay_and_check(lambda: run(cap, ws), lambda: run(mk(), ws2), refill_fn)


def test_graph_layer_paths():
    """The layer's per-token stages around the chunk kernel, both ways:
    kda_prefill_prologue (gate stage) -> kda_chunk_fwd_snapshots ->
    kda_output_gate, and kda_prefill_prologue (no gate stage) ->
    kda_chunk_fwd_gated with the output gate; conv registers in place."""
    B, T, H, HV, K, V, KW = 1, 200, 2, 4, 128, 128, 4
    C = 2 * H * K + HV * V
    say("layer paths B1 T200 H2 HV4 K128 V128 KW4: eager")
    gen = torch.Generator(device="cpu").manual_seed(21)
    r = lambda *s_: torch.randn(*s_, generator=gen).to(DEV)
    conv_w, A_log, dt_bias = 0.5 * r(C, KW), r(HV), r(HV * K)
    x = torch.empty(B, T, C, dtype=torch.bfloat16, device=DEV)
    z = torch.empty(B, T, HV, K, device=DEV)
    bl = torch.empty(B, T, HV, device=DEV)
    og = torch.empty(B, T, HV, V, dtype=torch.bfloat16, device=DEV)
    cs = [torch.empty(B, C, KW, device=DEV) for _ in range(2)]
    common = dict(H=H, HV=HV, K=K, V=V, conv_weight=conv_w, l2norm_qk=True, l2_eps=1e-6)

    def refill_fn(seed):
        g2 = torch.Generator(device="cpu").manual_seed(seed)
        rr = lambda *s_: torch.randn(*s_, generator=g2).to(DEV)
        x.copy_(rr(B, T, C))
        z.copy_(2 * rr(B, T, HV, K))
        bl.copy_(rr(B, T, HV))
        og.copy_(rr(B, T, HV, V))
        st = rr(B, C, KW)
        for c in cs:
            c.copy_(st)

    def mk():
        bf = dict(dtype=torch.bfloat16, device=DEV)
        pro = lambda gate: (torch.empty(B, T, H, K, **bf), torch.empty(B, T, H, K, **bf),
                            torch.empty(B, T, HV, V, **bf),
                            torch.empty(B, T, HV, K, device=DEV) if gate else None,
                            torch.empty(B, T, HV, device=DEV) if gate else None)
        return dict(p1=pro(True), p2=pro(False), o1=torch.empty(B, T, HV, V, **bf),
                    S1=torch.empty(B, HV, K, V, device=DEV), sn=torch.empty(B, T // 64, HV, K, V, device=DEV),
                    y1=torch.empty(B, T, HV, V, **bf), y2=torch.empty(B, T, HV, V, **bf),
                    S2=torch.empty(B, HV, K, V, device=DEV))

    def run(o, c1, c2):
        q, k, v, g, beta = kda.prefill_prologue(x, z, bl, conv_state=c1, gate_mode=kda.GATE_BOUNDED,
                                                A_log=A_log, dt_bias=dt_bias, gate_lower_bound=-5.0,
                                                beta_is_logit=True, out=o["p1"], **common)
        kda.chunk_fwd_snapshots(q, k, v, g, beta, 64, out=o["o1"], final_state=o["S1"], snapshots=o["sn"])
        kda.output_gate(o["o1"], og, 1e-6, out=o["y1"])
        q2, k2, v2, _, _ = kda.prefill_prologue(x, None, None, conv_state=c2, out=o["p2"], **common)
        kda.chunk_fwd_gated(q2, k2, v2, z, bl, A_log, dt_bias, -5.0, out_gate=og, out_gate_eps=1e-6,
                            out=o["y2"], final_state=o["S2"])
        return [o["o1"], o["S1"], o["sn"], o["y1"], o["y2"], o["S2"], c1, c2] + [t for t in o["p1"]] + \
            [t for t in o["p2"] if t is not None]

    cap = mk()
    refill_fn(22)
    run(mk(), cs[0].clone(), cs[1].clone())
    replay_and_check(lambda: run(cap, cs[0], cs[1]), lambda: run(mk(), cs[0].clone(), cs[1].clone()),
                     refill_fn)
