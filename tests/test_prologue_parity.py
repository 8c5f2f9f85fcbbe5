"""GPU parity of kda_prefill_prologue and kda_output_gate against the fp64
oracle, and of the whole layer path (prologue -> chunk_fwd -> output gate,
then decode continuing from the prologue's conv registers and the final
state)."""
import sys

import numpy as np
import pytest
import torch

import oracle
import gated_delta_rule_kda_amd as kda
from kda_testutil import assert_close, gpu_available, np64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def make_layer_inputs(B, T, H, HV, K, V, KW, dtype, seed, state_in=True):
    """Raw projections and prologue parameters, N(0,1) unless stated."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    C = 2 * H * K + HV * V
    r = lambda *s: torch.randn(*s, generator=g)
    p = dict(
        x=r(B, T, C).to(dtype),
        conv_w=r(C, KW) * 0.5 if KW else None,
        conv_state=r(B, C, KW) if (KW and state_in) else None,
        z=r(B, T, HV, K),
        A_log=r(HV) * 0.5,
        dt_bias=r(HV * K) * 0.5,
        beta=r(B, T, HV),
        ogate=r(B, T, HV, V).to(dtype),
    )
    return {k: (v.to(DEV) if v is not None else None) for k, v in p.items()}


MODES = {"direct": kda.GATE_DIRECT, "bounded": kda.GATE_BOUNDED, "softplus": kda.GATE_SOFTPLUS}


def run_prologue(B, T, H, HV, K, V, KW, dtype, gate="bounded", l2=True, logit=True,
                 state_in=True, seed=0):
    say("prologue case", (B, T, H, HV, K, V, KW, str(dtype), gate, l2, logit, state_in))
    p = make_layer_inputs(B, T, H, HV, K, V, KW, dtype, seed, state_in)
    if gate == "direct":
        p["z"] = -5.0 * torch.sigmoid(p["z"])
    cs = p["conv_state"].clone() if p["conv_state"] is not None else None
    out = kda.prefill_prologue(p["x"], p["z"], p["beta"], H=H, HV=HV, K=K, V=V,
                               conv_weight=p["conv_w"], conv_state=cs, l2norm_qk=l2,
                               l2_eps=1e-6, gate_mode=MODES[gate], A_log=p["A_log"],
                               dt_bias=p["dt_bias"], gate_lower_bound=-5.0, beta_is_logit=logit)
    torch.cuda.synchronize()
    cs_ref = np64(p["conv_state"]) if p["conv_state"] is not None else (
        np.zeros((B, 2 * H * K + HV * V, KW)) if KW else None)
    ref = oracle.prefill_prologue(
        p["x"], H, HV, K, V, conv_w=p["conv_w"], conv_state=cs_ref, l2norm_qk=l2, eps=1e-6,
        gate_in=p["z"], A_log=p["A_log"] if gate != "direct" else None,
        dt_bias=p["dt_bias"] if gate != "direct" else None, gate_bounded=(gate == "bounded"),
        lower_bound=-5.0, beta=p["beta"], beta_is_logit=logit)
    for name, got, want, io in zip(("q", "k", "v", "g", "beta"), out, ref,
                                   (dtype, dtype, dtype, torch.float32, torch.float32)):
        assert_close(got, want, io, True, "prologue %s" % name)
    if cs is not None:
        # the registers after the last token are copies of inputs: exact
        np.testing.assert_array_equal(np64(cs), cs_ref)
    return p, out


CASES = [
    # B, T, H, HV, K, V, KW, dtype
    (1, 300, 2, 2, 128, 128, 4, torch.bfloat16),
    (2, 100, 1, 3, 64, 32, 4, torch.bfloat16),
    (1, 3, 2, 4, 32, 64, 4, torch.float32),
    (2, 257, 1, 2, 128, 64, 8, torch.float32),
    (1, 1, 1, 1, 32, 32, 2, torch.bfloat16),
    (1, 70, 2, 2, 64, 64, 1, torch.float32),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dT%dH%dHV%dK%dV%dKW%d-%s" % (
    c[:7] + (str(c[7]).split(".")[-1],)))
def test_prologue_matches_oracle(case):
    run_prologue(*case, seed=sum(case[:7]))


@pytest.mark.parametrize("gate", ["direct", "bounded", "softplus"])
@pytest.mark.parametrize("l2,logit,state_in", [(True, True, True), (False, False, False)])
def test_prologue_options(gate, l2, logit, state_in):
    run_prologue(2, 90, 2, 4, 64, 64, 4, torch.float32, gate=gate, l2=l2, logit=logit,
                 state_in=state_in, seed=5)


def test_prologue_without_conv():
    run_prologue(1, 40, 1, 2, 32, 32, 0, torch.bfloat16, state_in=False)


@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_output_gate_matches_oracle(D, dtype):
    g = torch.Generator(device="cpu").manual_seed(D)
    for rows in (1, 37, 1000):
        o = (torch.randn(rows, D, generator=g) * 3).to(dtype).to(DEV)
        gt = torch.randn(rows, D, generator=g).to(dtype).to(DEV)
        y = kda.output_gate(o, gt, 1e-6)
        y2 = o.clone()
        kda.output_gate(y2, gt, 1e-6, out=y2)        # in place
        torch.cuda.synchronize()
        ref = oracle.output_gate(o, gt, 1e-6)
        assert_close(y, ref, dtype, True, "output gate D%d rows %d" % (D, rows))
        assert torch.equal(y, y2)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_layer_path_and_decode_continuation(dtype):
    """prologue -> chunk_fwd -> output gate over T tokens, then 5 decode steps
    from the prologue's conv registers and the chunk's final state, against
    the oracle doing the same (its decode steps run the same prologue)."""
    B, T, H, HV, K, V, KW = 2, 130, 1, 2, 64, 64, 4
    Td = 5
    p = make_layer_inputs(B, T + Td, H, HV, K, V, KW, dtype, 21)
    C = 2 * H * K + HV * V
    cs = p["conv_state"].clone()
    kw = dict(H=H, HV=HV, K=K, V=V)
    pro = dict(conv_weight=p["conv_w"], l2norm_qk=True, l2_eps=1e-6, gate_mode=kda.GATE_BOUNDED,
               A_log=p["A_log"], dt_bias=p["dt_bias"], gate_lower_bound=-5.0, beta_is_logit=True)
    x = p["x"][:, :T].contiguous()
    q, k, v, gg, bb = kda.prefill_prologue(x, p["z"][:, :T].contiguous(), p["beta"][:, :T].contiguous(),
                                           conv_state=cs, **kw, **pro)
    o, S = kda.chunk_fwd(q, k, v, gg, bb, output_final_state=True)
    y = kda.output_gate(o, p["ogate"][:, :T].contiguous(), 1e-6)
    dec = []
    for t in range(T, T + Td):
        od = kda.decode_step(p["x"][:, t].contiguous(), p["z"][:, t].contiguous(),
                             p["beta"][:, t].contiguous(), S, conv_state=cs, **kw, **pro)
        dec.append(kda.output_gate(od, p["ogate"][:, t].contiguous(), 1e-6))
    torch.cuda.synchronize()

    cs_ref = np64(p["conv_state"])
    opt = dict(conv_w=p["conv_w"], l2norm_qk=True, eps=1e-6, A_log=p["A_log"], dt_bias=p["dt_bias"],
               gate_bounded=True, lower_bound=-5.0, beta_is_logit=True)
    rq, rk, rv, rg, rb = oracle.prefill_prologue(x, H, HV, K, V, conv_state=cs_ref,
                                                 gate_in=p["z"][:, :T], beta=p["beta"][:, :T], **opt)
    # the chunk step of the oracle sees the GPU's own (rounded) prologue outputs,
    # so each stage is checked against its own error
    ro, rS = oracle.kda_fwd(q, k, v, gg, bb)
    assert_close(q, rq, dtype, True, "layer q")
    assert_close(o, ro, dtype, True, "layer o")
    assert_close(y, oracle.output_gate(o, p["ogate"][:, :T], 1e-6), dtype, True, "layer y")
    st = rS.copy()
    for i, t in enumerate(range(T, T + Td)):
        od = oracle.kda_decode_step(p["x"][:, t], st, H, HV, K, V, conv_state=cs_ref,
                                    gate_in=p["z"][:, t], beta=p["beta"][:, t], **opt)
        yd = oracle.output_gate(od, p["ogate"][:, t], 1e-6)
        assert_close(dec[i], yd, dtype, True, "decode step %d after prefill" % i)
    assert_close(S, st, dtype, False, "state after decode")
    np.testing.assert_allclose(np64(cs), cs_ref, rtol=0, atol=0)


def test_full_size_hv96_prologue_sampled():
    """The HV96 layer shape (B1 T8192 H=HV=96 K=V=128, conv width 4, bf16),
    the launch the benchmark times; heads 0, 41 and 95 (their q, k, v channel
    rows) against the oracle run on just those channels."""
    B, T, H, HV, K, V, KW = 1, 8192, 96, 96, 128, 128, 4
    p = make_layer_inputs(B, T, H, HV, K, V, KW, torch.bfloat16, 0)
    cs = p["conv_state"].clone()
    q, k, v, gg, bb = kda.prefill_prologue(
        p["x"], p["z"], p["beta"], H=H, HV=HV, K=K, V=V, conv_weight=p["conv_w"], conv_state=cs,
        l2norm_qk=True, l2_eps=1e-6, gate_mode=kda.GATE_BOUNDED, A_log=p["A_log"],
        dt_bias=p["dt_bias"], gate_lower_bound=-5.0, beta_is_logit=True)
    torch.cuda.synchronize()
    for h in (0, 41, 95):
        ch = np.concatenate([np.arange(h * K, (h + 1) * K), H * K + np.arange(h * K, (h + 1) * K),
                             2 * H * K + np.arange(h * V, (h + 1) * V)])
        chi = torch.as_tensor(ch, device=DEV)
        cs_ref = np64(p["conv_state"][:, chi])
        rq, rk, rv, rg, rb = oracle.prefill_prologue(
            p["x"][:, :, chi], 1, 1, K, V, conv_w=p["conv_w"][chi], conv_state=cs_ref,
            l2norm_qk=True, eps=1e-6, gate_in=p["z"][:, :, h:h + 1], A_log=p["A_log"][h:h + 1],
            dt_bias=p["dt_bias"][h * K:(h + 1) * K], gate_bounded=True, lower_bound=-5.0,
            beta=p["beta"][:, :, h:h + 1], beta_is_logit=True)
        assert_close(q[:, :, h:h + 1], rq, torch.bfloat16, True, "HV96 q head %d" % h)
        assert_close(k[:, :, h:h + 1], rk, torch.bfloat16, True, "HV96 k head %d" % h)
        assert_close(v[:, :, h:h + 1], rv, torch.bfloat16, True, "HV96 v head %d" % h)
        assert_close(gg[:, :, h:h + 1], rg, torch.float32, True, "HV96 g head %d" % h)
        assert_close(bb[:, :, h:h + 1], rb, torch.float32, True, "HV96 beta head %d" % h)
        np.testing.assert_array_equal(np64(cs[:, chi]), cs_ref)
        say("   head", h, "ok")
