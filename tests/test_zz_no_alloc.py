"""kda_recurrent_bwd_noalloc (the backward over the library's own scratch
array, for callers that cannot allocate) against kda_recurrent_bwd with a
caller workspace: the same kernels, so the gradients must be bitwise equal.
Two calls in a row, the second smaller; the size limit on the GPU."""
import sys

import pytest
import torch

import gated_delta_rule_kda_amd as kda
from gated_delta_rule_kda_amd import synth
from kda_testutil import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda"
NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dS0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _case(shape, seed):
    inp = synth.make_prefill_inputs(shape, DEV, seed)
    gen = torch.Generator(device="cpu").manual_seed(seed + 1)
    dout = torch.randn(shape.B, shape.T, shape.HV, shape.V, generator=gen).to(shape.dtype).to(DEV)
    dST = (torch.randn(shape.B, shape.HV, shape.K, shape.V, generator=gen) * 0.1).to(DEV)
    return (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], dout, dST), inp["S0"]


def test_noalloc_backward_matches_workspace_backward():
    shapes = [synth.PrefillShape(1, 300, 2, 4, 128, 128, torch.bfloat16, "normal", s0_std=0.3),
              synth.PrefillShape(1, 70, 1, 2, 64, 64, torch.float32, "normal", s0_std=0.3)]
    for i, shape in enumerate(shapes):
        say("no-alloc backward call", i, shape)
        args, S0 = _case(shape, 40 + i)
        assert kda.recurrent_bwd_workspace_size(shape.B, shape.T, shape.H, shape.HV, shape.K,
                                                shape.V) <= kda.NOALLOC_SCRATCH_BYTES
        want = kda.recurrent_bwd(*args, initial_state=S0)
        got = kda.recurrent_bwd_noalloc(*args, initial_state=S0)
        torch.cuda.synchronize()
        for name, x, y in zip(NAMES, got, want):
            assert torch.equal(x, y), (i, name)
        say("   bitwise equal")


def test_noalloc_backward_rejects_sizes_past_the_scratch():
    shape = synth.PrefillShape(1, 8192, 16, 16, 128, 128, torch.bfloat16, "none")
    args, S0 = _case(shape, 50)
    with pytest.raises(kda.KDAError) as e:
        kda.recurrent_bwd_noalloc(*args, initial_state=S0)
    assert "scratch" in str(e.value)
