"""GPU parity of kda_decode_step against the fp64 oracle."""
import dataclasses
import json
import math
import os
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
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("H,HV,K,V", [(2, 2, 32, 32), (1, 4, 64, 128), (2, 4, 128, 64), (3, 3, 128, 128)])
def test_plain_steps_equal_prefill_oracle(dt, H, HV, K, V):
    """T plain decode steps (g, beta given; no prologue) against the oracle's
    forward over the same T tokens."""
    B, T = 3, 12
    shape = synth.PrefillShape(B, T, H, HV, K, V, dt, "normal", s0_std=0.5)
    say("decode plain", shape)
    inp = synth.make_prefill_inputs(shape, DEV, K + V)
    state = inp["S0"].clone()
    outs = []
    for t in range(T):
        x = torch.cat([inp["q"][:, t].reshape(B, -1), inp["k"][:, t].reshape(B, -1),
                       inp["v"][:, t].reshape(B, -1)], dim=1).contiguous()
        outs.append(kda.decode_step(x, inp["g"][:, t].contiguous(), inp["beta"][:, t].contiguous(),
                                    state, H=H, HV=HV, K=K, V=V))
    oref, Sref = oracle.kda_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                initial_state=inp["S0"])
    assert_close(torch.stack(outs, 1), oref, dt, True, "decode o")
    # the state is fp32 and updated in fp32 arithmetic: fp32 rule for both dtypes
    assert_close(state, Sref, torch.float32, False, "decode S")


def _prologue_run(shape: synth.DecodeShape, steps, seed=0, dt=torch.float32, check_b=None, ring=False):
    """Run `steps` fused decode steps with the full prologue (conv + SiLU,
    L2 norm, bounded gate, sigmoid beta) and compare against the oracle.
    ring: the conv registers as the [KW, B, C] ring (the oracle keeps rows)."""
    B, H, HV, K, V, KW = shape.B, shape.H, shape.HV, shape.K, shape.V, shape.KW
    C = 2 * H * K + HV * V
    say("decode prologue", shape, "steps", steps, "dtype", dt, "ring" if ring else "rows")
    prm = synth.make_decode_params(shape, DEV, seed)
    state = torch.zeros(B, HV, K, V, device=DEV)
    conv = torch.zeros(KW, B, C, device=DEV) if ring else torch.zeros(B, C, KW, device=DEV)
    bs = list(range(B)) if check_b is None else check_b
    st_ref = np.zeros((len(bs), HV, K, V))
    cv_ref = np.zeros((len(bs), C, KW))
    for t in range(steps):
        x, z, bl = prm["pool"][t % shape.pool]
        x = x.to(dt)
        out = kda.decode_step(x, z.view(B, HV, K), bl, state, H=H, HV=HV, K=K, V=V,
                              conv_weight=prm["conv_w"], conv_state=conv, l2norm_qk=True,
                              l2_eps=1e-6, gate_mode=kda.GATE_BOUNDED, A_log=prm["A_log"],
                              dt_bias=prm["dt_bias"], gate_lower_bound=shape.lower_bound,
                              beta_is_logit=True, conv_ring=ring, conv_pos=t % KW)
        oref = oracle.kda_decode_step(x[bs], st_ref, H, HV, K, V, conv_w=prm["conv_w"],
                                      conv_state=cv_ref, l2norm_qk=True, eps=1e-6,
                                      gate_in=z[bs], A_log=prm["A_log"], dt_bias=prm["dt_bias"],
                                      gate_bounded=True, lower_bound=shape.lower_bound,
                                      beta=bl[bs], beta_is_logit=True)
        assert_close(out[bs], oref, dt, True, "step %d out" % t)
    assert_close(state[bs], st_ref, torch.float32, False, "final state")
    if ring:
        # register j (oldest first) of the ring after `steps` steps sits in slot (steps + j) % KW
        conv = torch.stack([conv[(steps + j) % KW] for j in range(KW)], dim=-1)
    assert_close(conv[bs], cv_ref, torch.float32, False, "conv state")


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_prologue_small(dt):
    shape = synth.DecodeShape(B=3, H=2, HV=2, K=32, V=32, KW=4)
    _prologue_run(shape, steps=12, dt=dt)


def test_prologue_gqa_conv3():
    shape = synth.DecodeShape(B=2, H=2, HV=8, K=64, V=128, KW=3)
    _prologue_run(shape, steps=10)


def test_prologue_production_geometry_sampled():
    """The B256 HV96 K=V=128 decode workload (fp32, conv 4, bounded gate -5,
    L2 norm eps 1e-6, beta logits) for 40 steps; all 256 sequences run on the
    GPU, four of them are followed by the oracle."""
    _prologue_run(synth.DECODE_B256_HV96, steps=40, check_b=[0, 77, 128, 255])


def test_prologue_production_geometry_ring_sampled():
    """The same workload with the conv registers as the [4, B, C] ring, as
    the decode bench runs it: 41 steps (ten turns of the ring and one slot),
    four sequences followed by the oracle."""
    _prologue_run(synth.DECODE_B256_HV96, steps=41, check_b=[1, 64, 200, 254], ring=True)


def test_softplus_gate_mode():
    """The unbounded gate -exp(A_log) softplus(z + dt_bias)."""
    B, H, HV, K, V = 2, 2, 2, 64, 64
    C = 2 * H * K + HV * V
    gen = torch.Generator(device=DEV).manual_seed(5)
    x = torch.randn(B, C, device=DEV, generator=gen)
    z = torch.randn(B, HV, K, device=DEV, generator=gen)
    bl = torch.randn(B, HV, device=DEV, generator=gen)
    A_log = torch.randn(HV, device=DEV, generator=gen)
    dtb = torch.randn(HV * K, device=DEV, generator=gen)
    state = torch.randn(B, HV, K, V, device=DEV, generator=gen)
    st_ref = np64(state)
    out = kda.decode_step(x, z, bl, state, H=H, HV=HV, K=K, V=V, l2norm_qk=True,
                          gate_mode=kda.GATE_SOFTPLUS, A_log=A_log, dt_bias=dtb, beta_is_logit=True)
    oref = oracle.kda_decode_step(x, st_ref, H, HV, K, V, l2norm_qk=True, gate_in=z, A_log=A_log,
                                  dt_bias=dtb, gate_bounded=False, beta=bl, beta_is_logit=True)
    assert_close(out, oref, torch.float32, True, "softplus out")
    assert_close(state, st_ref, torch.float32, False, "softplus state")


def test_beta_logit_zero_still_writes():
    """The page's beta_zero_is_sigmoid_half_not_zero example on the GPU."""
    d = json.load(open(os.path.join(GOLDEN, "kda_rs_unit_examples.json")))["beta_logit_step"]
    # the library needs K, V >= 32: embed the 2-dim example in 32 dims (zeros elsewhere)
    K = V = 32
    q = torch.zeros(K); k = torch.zeros(K); v = torch.zeros(V)
    q[:2] = torch.tensor(d["qkv"][0:2]); k[:2] = torch.tensor(d["qkv"][2:4]); v[:2] = torch.tensor(d["qkv"][4:6])
    x = torch.cat([q, k, v])[None].to(DEV)
    gate = torch.full((1, 1, K), d["gate"][0], device=DEV)
    outs = []
    for logit in d["logits"]:
        state = torch.zeros(1, 1, K, V, device=DEV)
        o = kda.decode_step(x, gate, torch.tensor([[logit]], device=DEV), state, H=1, HV=1, K=K, V=V,
                            scale=1 / math.sqrt(2), l2norm_qk=True, l2_eps=d["eps"], beta_is_logit=True)
        beta = 1 / (1 + math.exp(-logit))
        expect = beta / (1 + d["eps"]) / math.sqrt(2) * np.array([1.0, 0.5])
        np.testing.assert_allclose(np64(o)[0, 0, :2], expect, rtol=1e-5)
        outs.append(o)
    assert float(outs[0].abs().max()) > 1e-6
    assert not torch.equal(outs[0], outs[1])


def test_snapshot_restore_bitwise():
    """Decoding from a restored copy of (state, conv state) equals sequential
    decoding bit for bit; a wrong snapshot diverges (the page's
    prefix_hit_wrong_slot_diverges, on production-shaped heads)."""
    shape = synth.DecodeShape(B=2, H=4, HV=4, K=128, V=128)
    B, H, HV, K, V, KW = shape.B, shape.H, shape.HV, shape.K, shape.V, shape.KW
    C = 2 * H * K + HV * V
    prm = synth.make_decode_params(shape, DEV, 3)
    kw = dict(H=H, HV=HV, K=K, V=V, conv_weight=prm["conv_w"], l2norm_qk=True,
              gate_mode=kda.GATE_BOUNDED, A_log=prm["A_log"], dt_bias=prm["dt_bias"],
              beta_is_logit=True)
    state = torch.zeros(B, HV, K, V, device=DEV)
    conv = torch.zeros(B, C, KW, device=DEV)
    snaps = []
    for t in range(3):
        x, z, bl = prm["pool"][t]
        kda.decode_step(x, z.view(B, HV, K), bl, state, conv_state=conv, **kw)
        snaps.append((state.clone(), conv.clone()))
    x, z, bl = prm["pool"][3]
    y_seq = kda.decode_step(x, z.view(B, HV, K), bl, state, conv_state=conv, **kw)
    s2, c2 = snaps[2][0].clone(), snaps[2][1].clone()
    y_hit = kda.decode_step(x, z.view(B, HV, K), bl, s2, conv_state=c2, **kw)
    assert torch.equal(y_hit, y_seq) and torch.equal(s2, state) and torch.equal(c2, conv)
    s1, c1 = snaps[1][0].clone(), snaps[1][1].clone()
    y_wrong = kda.decode_step(x, z.view(B, HV, K), bl, s1, conv_state=c1, **kw)
    assert float((y_hit - y_wrong).abs().max()) > 1e-4


def test_decode_matches_chunk_prefill():
    """Decoding T tokens one by one and the chunk prefill over the same tokens
    agree (two different kernels, one recurrence)."""
    shape = synth.PrefillShape(2, 70, 2, 4, 128, 128, torch.float32, "normal", s0_std=0.3)
    inp = synth.make_prefill_inputs(shape, DEV, 8, g_lower=-0.3)
    B, T, H, HV, K, V = shape.B, shape.T, shape.H, shape.HV, shape.K, shape.V
    o_pf, S_pf = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                               initial_state=inp["S0"], output_final_state=True)
    state = inp["S0"].clone()
    outs = []
    for t in range(T):
        x = torch.cat([inp["q"][:, t].reshape(B, -1), inp["k"][:, t].reshape(B, -1),
                       inp["v"][:, t].reshape(B, -1)], dim=1).contiguous()
        outs.append(kda.decode_step(x, inp["g"][:, t].contiguous(), inp["beta"][:, t].contiguous(),
                                    state, H=H, HV=HV, K=K, V=V))
    assert_close(torch.stack(outs, 1), o_pf.double(), torch.float32, True, "decode vs prefill o")
    assert_close(state, S_pf.double(), torch.float32, False, "decode vs prefill S")
