"""GPU parity of kda_chunk_fwd_gated (the gate, beta and output gate fused
into the chunk kernel) against the fp64 oracle: the gate stage of the
"kda.rs" host layer (bounded_gate), the token-loop recurrence, and
full_rank_output_gate, each pinned in the CPU suite."""
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


def gate_inputs(B, T, HV, K, V, seed, og=True):
    """z ~ N(0,1) (scaled by 2 for a wide gate range), beta logits ~ N(0,1),
    A_log, dt_bias ~ N(0,1), output-gate values ~ N(0,1) (bf16)."""
    gen = torch.Generator(device="cpu").manual_seed(seed)
    z = torch.randn(B, T, HV, K, generator=gen) * 2.0
    bl = torch.randn(B, T, HV, generator=gen)
    A_log = torch.randn(HV, generator=gen)
    dt = torch.randn(HV * K, generator=gen)
    ogate = torch.randn(B, T, HV, V, generator=gen).to(torch.bfloat16) if og else None
    to = lambda x: None if x is None else x.to(DEV).contiguous()
    return to(z), to(bl), to(A_log), to(dt), to(ogate)


def reference(q, k, v, z, bl, A_log, dt, lb, S0, ogate, eps, heads=None):
    """The oracle's chain: g from bounded_gate, beta = sigmoid(logit), the token
    loop, then the output gate on o.  heads = (b, hv) limits it to one chain."""
    B, T, H, K = q.shape
    HV = v.shape[2]
    if heads is not None:
        b, hv = heads
        h = hv // (HV // H)
        q, k = q[b:b + 1, :, h:h + 1], k[b:b + 1, :, h:h + 1]
        v, z, bl = v[b:b + 1, :, hv:hv + 1], z[b:b + 1, :, hv:hv + 1], bl[b:b + 1, :, hv:hv + 1]
        A_log, dt = A_log[hv:hv + 1], dt[hv * K:(hv + 1) * K]
        S0 = S0[b:b + 1, hv:hv + 1] if S0 is not None else None
        ogate = ogate[b:b + 1, :, hv:hv + 1] if ogate is not None else None
        HV = 1
    g = oracle.gate(np64(z).reshape(-1, HV * K), np64(A_log), np64(dt), HV, K, bounded=True,
                    lower_bound=lb).reshape(z.shape)
    beta = 1.0 / (1.0 + np.exp(-np64(bl)))
    o, S = oracle.kda_fwd(q, k, v, g, beta, initial_state=S0)
    if ogate is not None:
        o = oracle.output_gate(o, np64(ogate), eps)
    return o, S


CASES = [
    # B, T, H, HV, K, V, s0, out gate: the first three run one workgroup per
    # whole V row (the output gate in the o stores), the rest split V (the
    # output gate as a pass after the kernel) or have none
    (2, 77, 16, 96, 128, 128, "normal", True),
    (3, 45, 64, 64, 64, 64, "none", True),
    (5, 33, 32, 32, 128, 32, "normal", True),
    (1, 70, 2, 4, 128, 128, "normal", True),
    (2, 45, 1, 2, 64, 32, "none", True),
    (1, 97, 2, 2, 128, 64, "normal", False),
    (1, 1, 1, 1, 32, 32, "normal", True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dT%dH%dHV%dK%dV%d-%s-og%d" % (c[:7] + (int(c[7]),)))
def test_gated_matches_oracle(case):
    B, T, H, HV, K, V, s0, og = case
    shape = synth.PrefillShape(B, T, H, HV, K, V, torch.bfloat16, s0, s0_std=0.3)
    say("gated case", case)
    inp = synth.make_prefill_inputs(shape, DEV, T + HV)
    z, bl, A_log, dt, ogate = gate_inputs(B, T, HV, K, V, T + HV + 1, og)
    for lb in (-5.0, -0.5):
        y, S = kda.chunk_fwd_gated(inp["q"], inp["k"], inp["v"], z, bl, A_log, dt, lb,
                                   initial_state=inp["S0"], output_final_state=True, out_gate=ogate,
                                   out_gate_eps=1e-6)
        torch.cuda.synchronize()
        yref, Sref = reference(inp["q"], inp["k"], inp["v"], z, bl, A_log, dt, lb, inp["S0"], ogate, 1e-6)
        my = assert_close(y, yref, torch.bfloat16, True, "y lb=%g %s" % (lb, case))
        ms = assert_close(S, Sref, torch.bfloat16, False, "S_T lb=%g %s" % (lb, case))
        say("   lb %g  y excess/rms %.2e  S excess/rms %.2e" % (lb, my["excess_over_rms"], ms["excess_over_rms"]))


def test_gated_equals_unfused_layer_path():
    """prologue (conv + SiLU, L2 norm; no gate stage) + kda_chunk_fwd_gated
    against the unfused path prologue (with the gate) + kda_chunk_fwd +
    kda_output_gate: the same inputs give the same outputs within the bf16
    rule, and both match the oracle's prologue, token loop and output gate."""
    B, T, H, HV, K, V, KW = 1, 150, 2, 4, 128, 128, 4
    C = 2 * H * K + HV * V
    gen = torch.Generator(device="cpu").manual_seed(77)
    r = lambda *s_: torch.randn(*s_, generator=gen)
    x = r(B, T, C).to(torch.bfloat16).to(DEV)
    conv_w = (r(C, KW) * 0.5).to(DEV)
    z, bl = (r(B, T, HV, K) * 2).to(DEV), r(B, T, HV).to(DEV)
    A_log, dt = r(HV).to(DEV), r(HV * K).to(DEV)
    ogate = r(B, T, HV, V).to(torch.bfloat16).to(DEV)
    common = dict(H=H, HV=HV, K=K, V=V, conv_weight=conv_w, l2norm_qk=True, l2_eps=1e-6)
    cs1 = torch.zeros(B, C, KW, device=DEV)
    q, k, v, g, beta = kda.prefill_prologue(x, z, bl, conv_state=cs1, gate_mode=kda.GATE_BOUNDED, A_log=A_log,
                                            dt_bias=dt, gate_lower_bound=-5.0, beta_is_logit=True, **common)
    o, S = kda.chunk_fwd(q, k, v, g, beta, output_final_state=True)
    y_unf = kda.output_gate(o, ogate, 1e-6)
    cs2 = torch.zeros(B, C, KW, device=DEV)
    q2, k2, v2, g2, b2 = kda.prefill_prologue(x, None, None, conv_state=cs2, **common)
    assert g2 is None and b2 is None
    y_fus, S2 = kda.chunk_fwd_gated(q2, k2, v2, z, bl, A_log, dt, -5.0, output_final_state=True,
                                    out_gate=ogate, out_gate_eps=1e-6)
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(k, k2) and torch.equal(v, v2) and torch.equal(cs1, cs2)
    # against the oracle's stages
    cso = np.zeros((B, C, KW))
    qo, ko, vo, go, bo = oracle.prefill_prologue(x, H, HV, K, V, conv_w=conv_w, conv_state=cso,
                                                 l2norm_qk=True, eps=1e-6, gate_in=z, A_log=A_log,
                                                 dt_bias=dt, gate_bounded=True, lower_bound=-5.0,
                                                 beta=bl, beta_is_logit=True)
    # the layer stores q, k, v in bf16 between the stages: the reference rounds
    # the oracle's prologue outputs the same way before the recurrence
    rb = lambda a: torch.from_numpy(a).to(torch.bfloat16).double().numpy()
    oref, Sref = oracle.kda_fwd(rb(qo), rb(ko), rb(vo), go, bo)
    yref = oracle.output_gate(oref, np64(ogate), 1e-6)
    for name, got in (("unfused", y_unf), ("fused", y_fus)):
        m = assert_close(got, yref, torch.bfloat16, True, "layer y " + name)
        say("   layer %s y excess/rms %.2e" % (name, m["excess_over_rms"]))
    assert_close(S2, Sref, torch.bfloat16, False, "layer S fused")
    assert_close(y_fus, np64(y_unf), torch.bfloat16, True, "fused vs unfused")


@pytest.mark.parametrize("which", ["hv96", "gqa"])
def test_gated_full_size_sampled(which):
    """The HV96 shape (V split over two workgroups: the output gate as its own
    pass) and the GQA shape (whole rows per workgroup: the output gate in the
    o stores) at full size, in the launch configuration the benchmark times;
    chains checked against the oracle."""
    shape = synth.PREFILL_HV96_BF16 if which == "hv96" else synth.PREFILL_GQA_BF16
    chains = [(0, 0), (0, 95)] if which == "hv96" else [(0, 1), (7, 62)]
    B, T, H, HV, K, V = shape.B, shape.T, shape.H, shape.HV, shape.K, shape.V
    say("gated full size", which)
    inp = synth.make_prefill_inputs(shape, DEV, 3)
    z, bl, A_log, dt, ogate = gate_inputs(B, T, HV, K, V, 4)
    y, S = kda.chunk_fwd_gated(inp["q"], inp["k"], inp["v"], z, bl, A_log, dt, -5.0,
                               initial_state=inp["S0"], output_final_state=True, out_gate=ogate)
    torch.cuda.synchronize()
    for (b, hv) in chains:
        yref, Sref = reference(inp["q"], inp["k"], inp["v"], z, bl, A_log, dt, -5.0, inp["S0"], ogate, 1e-6,
                               heads=(b, hv))
        assert_close(y[b:b + 1, :, hv:hv + 1], yref, torch.bfloat16, True, "y chain %s" % ((b, hv),))
        assert_close(S[b:b + 1, hv:hv + 1], Sref, torch.bfloat16, False, "S chain %s" % ((b, hv),))
        say("   chain", (b, hv), "ok")
