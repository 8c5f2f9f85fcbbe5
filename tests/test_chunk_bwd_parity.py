"""GPU parity of kda_chunk_bwd (the chunked backward, bf16 inputs, bounded
gate) against the fp64 oracle's back-propagation through time, which the CPU
suite checks against finite differences."""
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
STORED = (True, True, True, False, False, False)   # outputs stored in bf16


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def grads_in(shape, seed, with_dst=True):
    gen = torch.Generator(device="cpu").manual_seed(seed + 2)
    dout = torch.randn(shape.B, shape.T, shape.HV, shape.V, generator=gen).to(torch.bfloat16).to(DEV)
    dST = (torch.randn(shape.B, shape.HV, shape.K, shape.V, generator=gen) * 0.1).to(DEV) if with_dst else None
    return dout, dST


def run(shape, seed, with_dst=True, label=""):
    say("chunked backward case", label, shape, "seed", seed, "dS_T", with_dst)
    inp = synth.make_prefill_inputs(shape, DEV, seed)
    dout, dST = grads_in(shape, seed, with_dst)
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    got = kda.chunk_bwd(*args, dout, dST, initial_state=inp["S0"])
    torch.cuda.synchronize()
    ref = oracle.kda_bwd(*args, dout, dST, initial_state=inp["S0"])
    for name, gpu, want, st in zip(NAMES, got, ref, STORED):
        if want is None:
            continue
        m = assert_close(gpu, want, torch.bfloat16, st, "%s %s" % (name, label))
        say("   %-6s max_rel %.2e  excess/rms %.2e" % (name, m["max_rel"], m["excess_over_rms"]))
    return inp, dout, dST, got


CASES = [
    # B, T, H, HV, K, V: ragged tails, one to several chunks, GQA, every K and V
    (1, 1, 1, 1, 32, 32),
    (2, 31, 1, 2, 32, 32),
    (1, 33, 2, 2, 64, 64),
    (2, 64, 1, 1, 128, 128),
    (1, 65, 1, 3, 128, 64),
    (1, 70, 2, 4, 64, 64),
    (3, 9, 2, 2, 64, 128),
    (1, 24, 1, 4, 32, 128),
    (2, 100, 2, 2, 128, 128),
    (1, 45, 1, 3, 128, 32),
    (1, 200, 2, 8, 128, 128),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dT%dH%dHV%dK%dV%d" % c)
@pytest.mark.parametrize("with_dst", [True, False])
def test_chunk_bwd_matches_oracle(case, with_dst):
    B, T, H, HV, K, V = case
    shape = synth.PrefillShape(B, T, H, HV, K, V, torch.bfloat16, "normal", s0_std=0.3)
    run(shape, seed=T + K + V, with_dst=with_dst, label=str(case))


def test_chunk_bwd_no_initial_state():
    """S0 absent: the forward starts from zeros and dS0 is not requested."""
    shape = synth.PrefillShape(2, 77, 1, 2, 64, 64, torch.bfloat16, "none")
    inp = synth.make_prefill_inputs(shape, DEV, 3)
    dout, dST = grads_in(shape, 3)
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    got = kda.chunk_bwd(*args, dout, dST, need_d_initial_state=False)
    torch.cuda.synchronize()
    assert got[5] is None
    ref = oracle.kda_bwd(*args, dout, dST)
    for name, gpu, want, st in zip(NAMES[:5], got[:5], ref[:5], STORED):
        assert_close(gpu, want, torch.bfloat16, st, "no S0 %s" % name)


LONG_MEMORY = [
    # g = -0.05 sigmoid(N(0,1)): the state keeps most of its past, dg sums
    # slowly decaying terms over the whole sequence
    (1, 1024, 2, 2, 128, 128),
    (1, 600, 1, 2, 128, 64),
    (2, 512, 1, 2, 64, 64),
]


@pytest.mark.parametrize("case", LONG_MEMORY, ids=lambda c: "B%dT%dH%dHV%dK%dV%d" % c)
def test_chunk_bwd_long_memory(case):
    B, T, H, HV, K, V = case
    shape = synth.PrefillShape(B, T, H, HV, K, V, torch.bfloat16, "normal", s0_std=0.3, g_lower=-0.05)
    run(shape, seed=T + 1, label="long memory " + str(case))


SLABS = [
    # longer than one slab of 1024 tokens: the state gradient, the slab-start
    # states and the dg sum cross slab boundaries (a last slab of 76 tokens, of
    # 1 token, three slabs with GQA)
    (2, 1100, 1, 2, 64, 64),
    (1, 1025, 2, 2, 32, 32),
    (1, 2100, 1, 4, 128, 32),
]


@pytest.mark.parametrize("case", SLABS, ids=lambda c: "B%dT%dH%dHV%dK%dV%d" % c)
def test_chunk_bwd_across_slabs(case):
    B, T, H, HV, K, V = case
    shape = synth.PrefillShape(B, T, H, HV, K, V, torch.bfloat16, "normal", s0_std=0.3, g_lower=-1.0)
    run(shape, seed=T + 7, label="slabs " + str(case))


def test_chunk_bwd_gate_at_its_bound():
    """g = -5 everywhere (the strongest decay the chunk form takes) and
    g = 0 everywhere (no decay): the reference-row factors at their extremes."""
    for gval in (-5.0, 0.0):
        shape = synth.PrefillShape(1, 96, 1, 2, 64, 64, torch.bfloat16, "normal", s0_std=0.3)
        inp = synth.make_prefill_inputs(shape, DEV, 11)
        inp["g"].fill_(gval)
        dout, dST = grads_in(shape, 11)
        args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
        got = kda.chunk_bwd(*args, dout, dST, initial_state=inp["S0"])
        torch.cuda.synchronize()
        ref = oracle.kda_bwd(*args, dout, dST, initial_state=inp["S0"])
        for name, gpu, want, st in zip(NAMES, got, ref, STORED):
            assert_close(gpu, want, torch.bfloat16, st, "g=%g %s" % (gval, name))


def test_chunk_bwd_beta_zero():
    """beta = 0: nothing is written, so dL/dv = 0 exactly and
    dS0 = exp(G_T) (.) dS_T + sum_t exp(G_t) (.) (s q_t (x) dout_t); all six
    gradients also against the oracle."""
    B, T, H, HV, K, V = 1, 300, 1, 2, 64, 64
    shape = synth.PrefillShape(B, T, H, HV, K, V, torch.bfloat16, "normal", s0_std=0.3, g_lower=-0.2)
    inp = synth.make_prefill_inputs(shape, DEV, 31)
    inp["beta"].zero_()
    dout, dST = grads_in(shape, 31)
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    got = kda.chunk_bwd(*args, dout, dST, initial_state=inp["S0"])
    torch.cuda.synchronize()
    assert torch.count_nonzero(got[2]) == 0, "dv must vanish when nothing is written"
    s = 1.0 / np.sqrt(K)
    q, g, do = np64(inp["q"])[0, :, 0], np64(inp["g"])[0], np64(dout)[0]
    for hv in range(HV):
        G = np.cumsum(g[:, hv], axis=0)
        want = np.exp(G[-1])[:, None] * np64(dST)[0, hv] + (np.exp(G) * (s * q)).T @ do[:, hv]
        assert_close(got[5][0, hv], want, torch.bfloat16, False, "beta=0 dS0 head %d" % hv)
    ref = oracle.kda_bwd(*args, dout, dST, initial_state=inp["S0"])
    for name, gpu, want, st in zip(NAMES, got, ref, STORED):
        assert_close(gpu, want, torch.bfloat16, st, "beta=0 %s" % name)


def test_chunk_bwd_empty_sequence():
    """T = 0: dS0 = dL/dS_T (zeros without it), nothing else written."""
    B, H, HV, K, V = 2, 1, 2, 64, 32
    z = lambda *s, dt=torch.bfloat16: torch.zeros(*s, dtype=dt, device=DEV)
    zf = lambda *s: torch.zeros(*s, dtype=torch.float32, device=DEV)
    dST = torch.randn(B, HV, K, V, device=DEV)
    got = kda.chunk_bwd(z(B, 0, H, K), z(B, 0, H, K), z(B, 0, HV, V), zf(B, 0, HV, K), zf(B, 0, HV),
                        z(B, 0, HV, V), dST)
    torch.cuda.synchronize()
    assert torch.equal(got[5], dST)
    # the zeros are written, over whatever dS0 held
    outs = (z(B, 0, H, K), z(B, 0, H, K), z(B, 0, HV, V), zf(B, 0, HV, K), zf(B, 0, HV),
            torch.full((B, HV, K, V), float("nan"), device=DEV))
    got = kda.chunk_bwd(z(B, 0, H, K), z(B, 0, H, K), z(B, 0, HV, V), zf(B, 0, HV, K), zf(B, 0, HV),
                        z(B, 0, HV, V), None, out=outs)
    torch.cuda.synchronize()
    assert torch.count_nonzero(got[5]) == 0 and not torch.isnan(got[5]).any()


def test_chunk_bwd_workspace_reuse_and_determinism():
    """The same call twice through one workspace (another size in between, the
    workspace filled with garbage first) gives bitwise equal gradients."""
    shape = synth.PrefillShape(2, 150, 2, 4, 64, 64, torch.bfloat16, "normal", s0_std=0.3)
    inp = synth.make_prefill_inputs(shape, DEV, 5)
    dout, dST = grads_in(shape, 5)
    nbytes = kda.chunk_bwd_workspace_size(2, 150, 2, 4, 64, 64)
    ws = torch.full((nbytes,), 0x7f, dtype=torch.uint8, device=DEV)
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], dout, dST)
    a = kda.chunk_bwd(*args, initial_state=inp["S0"], workspace=ws)
    small = synth.make_prefill_inputs(synth.PrefillShape(1, 7, 1, 1, 32, 32, torch.bfloat16, "normal"), DEV, 6)
    kda.chunk_bwd(small["q"], small["k"], small["v"], small["g"], small["beta"],
                  torch.ones(1, 7, 1, 32, device=DEV, dtype=torch.bfloat16), workspace=ws)
    b = kda.chunk_bwd(*args, initial_state=inp["S0"], workspace=ws)
    torch.cuda.synchronize()
    for name, x, y in zip(NAMES, a, b):
        assert torch.equal(x, y), name


def test_chunk_bwd_agrees_with_recurrent_bwd():
    """The two GPU backward paths on one input (GQA, three slabs): within the
    bf16 bar of each other as well as of the oracle."""
    shape = synth.PrefillShape(1, 2500, 2, 4, 128, 64, torch.bfloat16, "normal", s0_std=0.3, g_lower=-2.0)
    inp = synth.make_prefill_inputs(shape, DEV, 41)
    dout, dST = grads_in(shape, 41)
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], dout, dST)
    a = kda.chunk_bwd(*args, initial_state=inp["S0"])
    b = kda.recurrent_bwd(*args, initial_state=inp["S0"])
    torch.cuda.synchronize()
    for name, x, y, st in zip(NAMES, a, b, STORED):
        assert_close(x, y, torch.bfloat16, st, "chunked vs recurrent %s" % name)


def test_full_size_hv96_chunk_bwd_sampled():
    """The HV96 workload at its full length, as the benchmark times it (B1
    T8192 H=HV=96 K=V=128 bf16, bounded gate, dL/dS_T given): heads 0 and 95
    against the oracle run on just those heads."""
    shape = synth.PrefillShape(1, 8192, 96, 96, 128, 128, torch.bfloat16, "none")
    say("full-width chunked backward", shape)
    inp = synth.make_prefill_inputs(shape, DEV, 0)
    gen = torch.Generator(device="cpu").manual_seed(3)
    dout = torch.randn(1, 8192, 96, 128, generator=gen).to(torch.bfloat16).to(DEV)
    dST = (torch.randn(1, 96, 128, 128, generator=gen) * 0.1).to(DEV)
    got = kda.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], dout, dST)
    torch.cuda.synchronize()
    for hv in (0, 95):
        sub = lambda x: x[:, :, hv:hv + 1]
        ref = oracle.kda_bwd(sub(inp["q"]), sub(inp["k"]), sub(inp["v"]), sub(inp["g"]),
                             inp["beta"][:, :, hv:hv + 1], sub(dout), dST[:, hv:hv + 1])
        part = [x[:, :, hv:hv + 1] for x in got[:5]] + [got[5][:, hv:hv + 1]]
        for name, gpu, want, st in zip(NAMES, part, ref, STORED):
            m = assert_close(gpu, want, torch.bfloat16, st, "HV96 %s head %d" % (name, hv))
            say("   head %d %-6s max_rel %.2e  excess/rms %.2e" % (hv, name, m["max_rel"], m["excess_over_rms"]))


def test_full_size_gqa_chunk_bwd_sampled():
    """The GQA workload (B8 T4096 H16 HV64 K=V=128 bf16, S0 ~ N(0, 0.02^2)):
    sequence 7, q/k head 15 (value heads 60-63, whose dq and dk sum) against
    the oracle on just those heads."""
    shape = synth.PREFILL_GQA_BF16
    say("full-width chunked backward", shape)
    inp = synth.make_prefill_inputs(shape, DEV, 0)
    gen = torch.Generator(device="cpu").manual_seed(4)
    dout = torch.randn(8, 4096, 64, 128, generator=gen).to(torch.bfloat16).to(DEV)
    dST = (torch.randn(8, 64, 128, 128, generator=gen) * 0.1).to(DEV)
    got = kda.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], dout, dST,
                        initial_state=inp["S0"])
    torch.cuda.synchronize()
    b, h = 7, 15
    hv = slice(4 * h, 4 * h + 4)
    ref = oracle.kda_bwd(inp["q"][b:b + 1, :, h:h + 1], inp["k"][b:b + 1, :, h:h + 1],
                         inp["v"][b:b + 1, :, hv], inp["g"][b:b + 1, :, hv], inp["beta"][b:b + 1, :, hv],
                         dout[b:b + 1, :, hv], dST[b:b + 1, hv], initial_state=inp["S0"][b:b + 1, hv])
    part = (got[0][b:b + 1, :, h:h + 1], got[1][b:b + 1, :, h:h + 1], got[2][b:b + 1, :, hv],
            got[3][b:b + 1, :, hv], got[4][b:b + 1, :, hv], got[5][b:b + 1, hv])
    for name, gpu, want, st in zip(NAMES, part, ref, STORED):
        m = assert_close(gpu, want, torch.bfloat16, st, "GQA %s" % name)
        say("   %-6s max_rel %.2e  excess/rms %.2e" % (name, m["max_rel"], m["excess_over_rms"]))


SAVED = [
    # B, T, H, HV, K, V: one slab, a ragged last slab, T a multiple of the slab, GQA
    (1, 300, 1, 2, 64, 64),
    (1, 2100, 1, 2, 64, 64),
    (2, 2048, 1, 2, 32, 64),
    (1, 1100, 2, 4, 128, 128),
]


@pytest.mark.parametrize("case", SAVED, ids=lambda c: "B%dT%dH%dHV%dK%dV%d" % c)
@pytest.mark.parametrize("with_dst", [True, False])
def test_chunk_bwd_saved_states(case, with_dst):
    """kda_chunk_bwd_saved with the states kda_chunk_fwd_snapshots keeps every
    1024 tokens and its final state: the gradients of kda_chunk_bwd (within
    the tolerance of each other) and the oracle's."""
    B, T, H, HV, K, V = case
    shape = synth.PrefillShape(B, T, H, HV, K, V, torch.bfloat16, "normal", s0_std=0.3)
    say("saved-states backward", case, "dS_T", with_dst)
    inp = synth.make_prefill_inputs(shape, DEV, T + 5)
    dout, dST = grads_in(shape, T + 5, with_dst)
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    _, ST, snaps = kda.chunk_fwd_snapshots(*args, 1024, initial_state=inp["S0"], output_final_state=True)
    got = kda.chunk_bwd(*args, dout, dST, initial_state=inp["S0"], saved_states=snaps if T > 1024 else None,
                        final_state=ST)
    plain = kda.chunk_bwd(*args, dout, dST, initial_state=inp["S0"])
    torch.cuda.synchronize()
    ref = oracle.kda_bwd(*args, dout, dST, initial_state=inp["S0"])
    for name, gpu, p, want, st in zip(NAMES, got, plain, ref, STORED):
        assert_close(gpu, want, torch.bfloat16, st, "saved %s %s" % (name, case))
        assert_close(gpu, p.double().cpu().numpy(), torch.bfloat16, st, "saved vs plain %s %s" % (name, case))


def test_chunk_bwd_concurrent_host_threads():
    """Two host threads, each with its own stream, call the chunked backward
    at the same time (the library's side streams are shared per device and a
    call's enqueue is serialized): each result has the bits of a call made
    alone."""
    import threading
    shape = synth.PrefillShape(1, 1100, 1, 2, 64, 64, torch.bfloat16, "normal", s0_std=0.3, g_lower=-1.0)
    inp = synth.make_prefill_inputs(shape, DEV, 41)
    dout, dST = grads_in(shape, 41)
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    alone = kda.chunk_bwd(*args, dout, dST, initial_state=inp["S0"])
    torch.cuda.synchronize()
    results, errors = [None, None], []

    def worker(i):
        try:
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                for _ in range(3):
                    results[i] = kda.chunk_bwd(*args, dout, dST, initial_state=inp["S0"])
            st.synchronize()
        except Exception as e:   # reported below, on the main thread
            errors.append(e)
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(2):
        for name, a, b in zip(NAMES, results[i], alone):
            assert torch.equal(a, b), "thread %d: %s differs from the call made alone" % (i, name)
