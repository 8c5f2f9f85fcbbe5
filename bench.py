#!/usr/bin/env python3
"""KDA forward benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Headline workload (one JSON line on stdout):
  * prefill: kda_chunk_fwd on B=1, T=8192, H=HV=96, K=V=128, bf16 q/k/v, fp32
    g/beta, explicit zero fp32 initial state, final state returned, chunk 32.
    One timed step = one call over that batch.  value = tokens/s.
  * decode: 1000 kda_decode_step calls on B=256 sequences, H=HV=96, K=V=128,
    fp32 everywhere, fused short conv (width 4) + SiLU (its registers as a
    ring of 4 slot arrays; the shifted [B, C, 4] rows timed beside), L2 norm of q/k
    (eps 1e-6), bounded gate -5*sigmoid(exp(A_log)(z+dt_bias)), beta logits;
    state resident in HBM and updated in place.  Reported as GB/s against the
    HBM peak.
  * secondary lines: the GQA prefill (B8 T4096 H16 HV64), and the HV96 prefill
    with prefix snapshots of the state every 1024 and every 32 tokens
    (kda_chunk_fwd_snapshots; the snapshot stores count in the bytes), and the
    layer's per-token stages on the HV96 shape (kda_prefill_prologue,
    kda_output_gate) against the HBM peak, the HV96 workload with an
    unbounded gate (kda_chunk_fwd_unbounded against the HBM peak, and
    kda_recurrent_fwd against the fp32 vector peak), and the
    backward on the HV96 workload: kda_chunk_bwd (matrix cores: fp32, and bf16
    pairs in its reverse chain) and
    kda_recurrent_bwd (fp32 vector ALUs).
Inputs are seeded synthetic tensors (gated_delta_rule_kda_amd.synth) created on
the GPU before the timed region.  Kernel durations come from HIP events
recorded on the stream the kernels are launched on.  The CPU baseline runs the
fp64 oracle on the host's cores over a bounded sample of the prefill workload.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK = 2.5e15        # MI355X dense bf16 MFMA, FLOP/s
FP32_VALU_PEAK = 157.3e12      # MI355X fp32 vector, FLOP/s, counting packed (2-wide) FP32
# The same without packed FP32 (256 CU x 4 SIMD x 16 lanes x 2 flops x 2.4 GHz):
# the ceiling for code built, as this library is, without packed FP32 instructions.
FP32_VALU_PEAK_NONPACKED = 78.6e12
FP32_MFMA_PEAK = 157.3e12      # MI355X dense fp32 matrix cores, FLOP/s
COUNTERS = os.path.join(ROOT, "profiles", "counters.json")
N_CU = 256                     # MI355X compute units, 4 SIMDs each


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# The sources each profiled kernel is built from: its counters stay valid
# while these files are unchanged.
KERNEL_SOURCES = {
    "prefill_hv96": ["kda_prefill_bf16.hip", "kda_internal.h"],
    "prefill_gqa": ["kda_prefill_bf16.hip", "kda_internal.h"],
    "decode_b256": ["kda_decode.hip", "kda_internal.h"],
    "decode_b256_ring": ["kda_decode.hip", "kda_internal.h"],
}


def kernel_source_hash(kernel_key=None) -> str:
    """sha256 (first 16 hex digits) of the kernel's source files, or of every
    file under csrc/ when the kernel is not listed."""
    csrc = os.path.join(ROOT, "gated_delta_rule_kda_amd", "csrc")
    names = KERNEL_SOURCES.get(kernel_key)
    paths = ([os.path.join(csrc, n) for n in names] if names
             else sorted(glob.glob(os.path.join(csrc, "*"))))
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def prefill_alg_bytes(B, T, H, HV, K, V, esz):
    """Algorithmic HBM bytes of one prefill call: every input read once, every
    output written once (q,k per q/k head; v,g,beta,o per value head; S0 and S_T)."""
    per_tok = H * 2 * K * esz + HV * (V * esz + K * 4 + 4 + V * esz)
    return B * T * per_tok + 2 * B * HV * K * V * 4


def prefill_alg_flops(B, T, HV, K, V, C=32):
    """Algorithmic flops: 6KV + 2C(K+V) per token per value head at C = 32."""
    return B * T * HV * (6 * K * V + 2 * C * (K + V))


def decode_alg_bytes(B, H, HV, K, V, KW):
    """Algorithmic HBM bytes of one fused decode step: fp32 state read and
    written once, conv state one 16-byte pass per channel, the token's qkv,
    z, beta, the output, and the parameters (conv weights, dt_bias, A_log)."""
    C = 2 * H * K + HV * V
    per_seq = 2 * HV * K * V * 4 + C * KW * 4 + C * 4 + HV * K * 4 + HV * 4 + HV * V * 4
    params = C * KW * 4 + HV * K * 4 + HV * 4
    return B * per_seq + params


def counter_entry(kernel_key):
    """The committed rocprofv3 counter record of a kernel, if it was taken on
    the kernel sources as they are now; else None."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    e = c.get(kernel_key)
    if not e or e.get("source_hash") != kernel_source_hash(kernel_key):
        return None
    return e


def load_counters(kernel_key):
    """HBM traffic per launch from the committed counter runs (see
    counter_entry), or None."""
    e = counter_entry(kernel_key)
    return e.get("traffic_bytes") if e else None


def mfma_busy(kernel_key, avg_launch_ms):
    """The matrix cores' busy fraction from the committed SQ counters of one
    launch: SQ_VALU_MFMA_BUSY_CYCLES (summed over SIMDs) over the SIMD-cycles
    of the CUs the kernel kept busy (4 x SQ_BUSY_CU_CYCLES), and over the
    SIMD-cycles of the whole GPU for the launch (4 x 256 CUs x duration x the
    clock those counters imply).  The cross-check: SQ_INSTS_VALU_MFMA_MOPS_BF16
    (units of 512 flops) at 1024 bf16 flops per SIMD-cycle gives the busy
    cycles the instructions alone need.  None without counters."""
    e = counter_entry(kernel_key)
    if not e or "sq_valu_mfma_busy_cycles" not in e:
        return None
    busy, cu = e["sq_valu_mfma_busy_cycles"], e["sq_busy_cu_cycles"]
    clock_hz = cu / (e["busy_cus"] * e["kernel_avg_ns"] * 1e-9)
    gpu_simd_cycles = 4 * N_CU * avg_launch_ms * 1e-3 * clock_hz
    return {"busy_frac": busy / (4.0 * cu), "busy_frac_whole_gpu": busy / gpu_simd_cycles,
            "mfma_busy_cycles": busy, "busy_cu_cycles": cu, "busy_cus": e["busy_cus"],
            "implied_clock_ghz": clock_hz / 1e9,
            "mops_bf16": e["sq_insts_valu_mfma_mops_bf16"],
            "cycles_from_mops": e["sq_insts_valu_mfma_mops_bf16"] * 512 / 1024.0,
            "executed_bf16_flops": e["sq_insts_valu_mfma_mops_bf16"] * 512,
            "source": "profiles/counters.json (rocprofv3 --pmc on the current kernel sources)"}


def measure_copy_bandwidth(nbytes=1 << 30, reps=10):
    """HBM bandwidth a plain device copy (torch copy_) and an in-place
    read-modify-write (mul_) reach on this GPU, in GB/s counting every byte
    read and written once: the practical ceilings beside the 8 TB/s peak."""
    import torch
    n = nbytes // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    res = {}
    for name, fn in (("copy", lambda: b.copy_(a)), ("rmw_in_place", lambda: a.mul_(1.0000001))):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        s_ = torch.cuda.Event(enable_timing=True)
        e_ = torch.cuda.Event(enable_timing=True)
        s_.record()
        for _ in range(reps):
            fn()
        e_.record()
        torch.cuda.synchronize()
        ms = s_.elapsed_time(e_) / reps
        res[name] = 2 * n * 4 / (ms * 1e-3) / 1e9
        log("[%s] %.1f GB/s (%d MiB each way)" % (name, res[name], nbytes >> 20))
    del a, b
    return res


def time_calls(fn, n, stream):
    """Average event time (ms) of n calls of fn, events on `stream`."""
    import torch
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for i in range(n):
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    return starts, ends


def cpu_baseline(inp, shape, budget_heads=None):
    """The fp64 oracle on host cores over a bounded sample of the prefill
    workload: every token of the first `budget_heads` value heads (all heads
    by default).  Returns the dict for the JSON line."""
    import numpy as np
    import oracle
    import torch
    B, T, H, HV, K, V = shape.B, shape.T, shape.H, shape.HV, shape.K, shape.V
    nh = HV if budget_heads is None else min(HV, budget_heads)
    G = HV // H
    nq = max(1, nh // G)
    q = inp["q"][:, :, :nq].to("cpu")
    k = inp["k"][:, :, :nq].to("cpu")
    v = inp["v"][:, :, :nh].to("cpu")
    g = inp["g"][:, :, :nh].to("cpu")
    beta = inp["beta"][:, :, :nh].to("cpu")
    S0 = inp["S0"][:, :nh].to("cpu") if inp["S0"] is not None else None
    args = [oracle.f64(x) for x in (q, k, v, g, beta)]
    S0 = oracle.f64(S0)
    threads = oracle.omp_threads()
    t0 = time.perf_counter()
    oracle.kda_fwd(*args, initial_state=S0)
    dt = time.perf_counter() - t0
    # tokens/s of the whole workload: the sample did nh/HV of every token's work
    value = B * T * (nh / HV) / dt
    return {"value": value, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "fp64 token loop over all %d tokens of %d of the %d value heads "
                      "(B=%d), %.2f s on the host; value scaled to all %d heads"
                      % (T, nh, HV, B, dt, HV),
            "seconds": dt}


def bench_prefill(shape, steps, warmup, tag, snapshot_every=None, inp=None, recurrent=False,
                  unbounded=False):
    import torch
    import gated_delta_rule_kda_amd as kda
    from gated_delta_rule_kda_amd import synth
    dev = torch.device("cuda:0")
    if inp is None:
        inp = synth.make_prefill_inputs(shape, dev, 0)
    out = torch.empty(shape.B, shape.T, shape.HV, shape.V, dtype=shape.dtype, device=dev)
    ST = torch.empty(shape.B, shape.HV, shape.K, shape.V, dtype=torch.float32, device=dev)
    snap_bytes = 0
    if snapshot_every:
        snaps = torch.empty(shape.B, shape.T // snapshot_every, shape.HV, shape.K, shape.V,
                            dtype=torch.float32, device=dev)
        snap_bytes = snaps.numel() * 4

        def call():
            kda.chunk_fwd_snapshots(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                    snapshot_every, initial_state=inp["S0"], out=out,
                                    final_state=ST, snapshots=snaps)
    elif recurrent:
        def call():
            kda.recurrent_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                              initial_state=inp["S0"], out=out, final_state=ST)
    elif unbounded:
        ws = torch.empty(kda.chunk_fwd_unbounded_workspace_size(shape.B, shape.T, shape.H, shape.HV,
                                                                shape.K, shape.V),
                         dtype=torch.uint8, device=dev)

        def call():
            kda.chunk_fwd_unbounded(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                    initial_state=inp["S0"], out=out, final_state=ST, workspace=ws)
    else:
        def call():
            kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                          initial_state=inp["S0"], out=out, final_state=ST)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    t0 = time.perf_counter()
    starts, ends = time_calls(call, steps, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    total_ms = starts[0].elapsed_time(ends[-1])
    esz = 2 if shape.dtype == torch.bfloat16 else 4
    nbytes = prefill_alg_bytes(shape.B, shape.T, shape.H, shape.HV, shape.K, shape.V, esz) + snap_bytes
    flops = prefill_alg_flops(shape.B, shape.T, shape.HV, shape.K, shape.V)
    avg_ms = sum(ev_ms) / len(ev_ms)
    log("[%s] prefill avg %.4f ms (min %.4f, max %.4f), span %.3f ms, wall %.3f s" % (
        tag, avg_ms, min(ev_ms), max(ev_ms), total_ms, wall))
    return dict(inp=inp, avg_ms=avg_ms, min_ms=min(ev_ms), span_ms=total_ms,
                bytes=nbytes, flops=flops, tokens=shape.B * shape.T,
                workspace=ws.numel() if unbounded else 0)


def bench_decode(shape, steps, warmup, ring=True):
    """ring: the conv registers as the [KW, B, C] ring (each step reads the
    KW - 1 newest slots and writes one); else the [B, C, KW] rows that each
    step shifts and rewrites whole."""
    import torch
    import gated_delta_rule_kda_amd as kda
    from gated_delta_rule_kda_amd import synth
    dev = torch.device("cuda:0")
    B, H, HV, K, V, KW = shape.B, shape.H, shape.HV, shape.K, shape.V, shape.KW
    C = 2 * H * K + HV * V
    prm = synth.make_decode_params(shape, dev, 0)
    state = torch.zeros(B, HV, K, V, device=dev)
    conv = torch.zeros(KW, B, C, device=dev) if ring else torch.zeros(B, C, KW, device=dev)
    out = torch.empty(B, HV, V, device=dev)
    pool = [(x, z.view(B, HV, K), bl) for (x, z, bl) in prm["pool"]]

    def call(t):
        x, z, bl = pool[t % len(pool)]
        kda.decode_step(x, z, bl, state, H=H, HV=HV, K=K, V=V, out=out,
                        conv_weight=prm["conv_w"], conv_state=conv, l2norm_qk=True, l2_eps=1e-6,
                        gate_mode=kda.GATE_BOUNDED, A_log=prm["A_log"], dt_bias=prm["dt_bias"],
                        gate_lower_bound=shape.lower_bound, beta_is_logit=True,
                        conv_ring=ring, conv_pos=t % KW)

    for t in range(warmup):
        call(t)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record(stream)
    for t in range(steps):
        call(t)
    e.record(stream)
    torch.cuda.synchronize()
    span_ms = s.elapsed_time(e)
    nbytes = decode_alg_bytes(B, H, HV, K, V, KW)
    per_ms = span_ms / steps
    gbs = nbytes / (per_ms * 1e-3) / 1e9
    log("[decode%s] %d steps: %.3f ms total, %.4f ms/step, %.1f GB/s"
        % (" ring" if ring else " rows", steps, span_ms, per_ms, gbs))
    return dict(span_ms=span_ms, per_ms=per_ms, bytes=nbytes, gbs=gbs)


def prologue_alg_bytes(B, T, H, HV, K, V, KW, esz):
    """Bytes of kda_prefill_prologue read or written once: x, z, beta in; q, k,
    v, g, beta out; conv weights, conv registers in and out, A_log, dt_bias."""
    C = 2 * H * K + HV * V
    return (B * T * C * esz * 2 + B * T * HV * K * 4 * 2 + B * T * HV * 4 * 2
            + C * KW * 4 + B * C * KW * 4 * 2 + HV * 4 + HV * K * 4)


def bench_layer_stages(steps, warmup):
    """kda_prefill_prologue and kda_output_gate on the HV96 layer shape."""
    import torch
    import gated_delta_rule_kda_amd as kda
    dev = torch.device("cuda:0")
    B, T, H, HV, K, V, KW = 1, 8192, 96, 96, 128, 128, 4
    C = 2 * H * K + HV * V
    gen = torch.Generator(device=dev).manual_seed(0)
    r = lambda *s_: torch.randn(*s_, generator=gen, device=dev)
    x = r(B, T, C).to(torch.bfloat16)
    conv_w, conv_state = r(C, KW) * 0.5, r(B, C, KW)
    z, A_log, dt_bias, bl = r(B, T, HV, K), r(HV) * 0.5, r(HV * K) * 0.5, r(B, T, HV)
    outs = (torch.empty(B, T, H, K, dtype=torch.bfloat16, device=dev),
            torch.empty(B, T, H, K, dtype=torch.bfloat16, device=dev),
            torch.empty(B, T, HV, V, dtype=torch.bfloat16, device=dev),
            torch.empty(B, T, HV, K, device=dev), torch.empty(B, T, HV, device=dev))
    o = r(B, T, HV, V).to(torch.bfloat16)
    og = r(B, T, HV, V).to(torch.bfloat16)
    y = torch.empty_like(o)

    def pro():
        kda.prefill_prologue(x, z, bl, H=H, HV=HV, K=K, V=V, conv_weight=conv_w,
                             conv_state=conv_state, l2norm_qk=True, l2_eps=1e-6,
                             gate_mode=kda.GATE_BOUNDED, A_log=A_log, dt_bias=dt_bias,
                             gate_lower_bound=-5.0, beta_is_logit=True, out=outs)

    def gate():
        kda.output_gate(o, og, 1e-6, out=y)

    res = {}
    stream = torch.cuda.current_stream(dev)
    for name, fn, nbytes in (("prologue", pro, prologue_alg_bytes(B, T, H, HV, K, V, KW, 2)),
                             ("output_gate", gate, 3 * o.numel() * 2)):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        starts, ends = time_calls(fn, steps, stream)
        torch.cuda.synchronize()
        ms = sum(s_.elapsed_time(e_) for s_, e_ in zip(starts, ends)) / steps
        gbs = nbytes / (ms * 1e-3) / 1e9
        log("[%s] avg %.4f ms, %.1f GB/s" % (name, ms, gbs))
        res[name] = dict(avg_ms=ms, bytes=nbytes, gbs=gbs)
    return res


def bench_layer_path(shape, steps, warmup, tag):
    """The layer around the prefill, end to end, two ways on the same inputs:
    unfused = kda_prefill_prologue (conv width 4 + SiLU, L2 norm, bounded gate
    into g, beta logits) -> kda_chunk_fwd -> kda_output_gate; fused =
    kda_prefill_prologue without its gate stage -> kda_chunk_fwd_gated (gate,
    beta and output gate in the chunk kernel).  Outputs preallocated; each
    timed step is the whole sequence of calls."""
    import torch
    import gated_delta_rule_kda_amd as kda
    dev = torch.device("cuda:0")
    B, T, H, HV, K, V, KW = shape.B, shape.T, shape.H, shape.HV, shape.K, shape.V, 4
    C = 2 * H * K + HV * V
    gen = torch.Generator(device=dev).manual_seed(0)
    r = lambda *s_: torch.randn(*s_, generator=gen, device=dev)
    x = r(B, T, C).to(torch.bfloat16)
    conv_w, conv_state = r(C, KW) * 0.5, torch.zeros(B, C, KW, device=dev)
    z, A_log, dt_bias, bl = r(B, T, HV, K), r(HV) * 0.5, r(HV * K) * 0.5, r(B, T, HV)
    ogate = r(B, T, HV, V).to(torch.bfloat16)
    bf = dict(dtype=torch.bfloat16, device=dev)
    q, k, v = torch.empty(B, T, H, K, **bf), torch.empty(B, T, H, K, **bf), torch.empty(B, T, HV, V, **bf)
    g, beta = torch.empty(B, T, HV, K, device=dev), torch.empty(B, T, HV, device=dev)
    o, y = torch.empty(B, T, HV, V, **bf), torch.empty(B, T, HV, V, **bf)
    ST = torch.empty(B, HV, K, V, device=dev)
    pro = dict(H=H, HV=HV, K=K, V=V, conv_weight=conv_w, conv_state=conv_state, l2norm_qk=True, l2_eps=1e-6)

    def unfused():
        kda.prefill_prologue(x, z, bl, gate_mode=kda.GATE_BOUNDED, A_log=A_log, dt_bias=dt_bias,
                             gate_lower_bound=-5.0, beta_is_logit=True, out=(q, k, v, g, beta), **pro)
        kda.chunk_fwd(q, k, v, g, beta, out=o, final_state=ST)
        kda.output_gate(o, ogate, 1e-6, out=y)

    def fused():
        kda.prefill_prologue(x, None, None, out=(q, k, v, None, None), **pro)
        kda.chunk_fwd_gated(q, k, v, z, bl, A_log, dt_bias, -5.0, out_gate=ogate, out_gate_eps=1e-6,
                            out=y, final_state=ST)

    res = {}
    stream = torch.cuda.current_stream(dev)
    for name, fn in (("unfused", unfused), ("fused", fused)):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        starts, ends = time_calls(fn, steps, stream)
        torch.cuda.synchronize()
        ms = sum(s_.elapsed_time(e_) for s_, e_ in zip(starts, ends)) / steps
        log("[layer %s %s] %.4f ms" % (tag, name, ms))
        res[name + "_ms"] = ms
    return res


def backward_alg_flops(B, T, HV, K, V):
    """The gradient's own arithmetic per token and value head, as the
    back-propagation through time forms it: D += qs dout^T, S_t dout, D r,
    a^T D, D - k dr^T, S_dec dr, rowsum(S_dec * D_dec) (2KV each) and the
    decay (KV): 15KV (the forward recompute not counted)."""
    return 15 * K * V * B * T * HV


def bench_backward(shape, steps, warmup, inp=None, chunked=True, saved=False):
    """kda_chunk_bwd (chunked) or kda_recurrent_bwd on `shape` with dL/do ~
    N(0,1) and dL/dS_T ~ 0.1 N(0,1); workspace and outputs allocated before the
    timed region.  saved: kda_chunk_bwd_saved, given the states every 1024
    tokens and the final state of a kda_chunk_fwd_snapshots call made before
    the timed region (the forward a training step has already run)."""
    import torch
    import gated_delta_rule_kda_amd as kda
    from gated_delta_rule_kda_amd import synth
    dev = torch.device("cuda:0")
    if inp is None:
        inp = synth.make_prefill_inputs(shape, dev, 0)
    B, T, H, HV, K, V = shape.B, shape.T, shape.H, shape.HV, shape.K, shape.V
    gen = torch.Generator(device=dev).manual_seed(1)
    dout = torch.randn(B, T, HV, V, generator=gen, device=dev).to(shape.dtype)
    dST = torch.randn(B, HV, K, V, generator=gen, device=dev) * 0.1
    nbytes = (kda.chunk_bwd_workspace_size(B, T, H, HV, K, V, shape.dtype) if chunked
              else kda.recurrent_bwd_workspace_size(B, T, H, HV, K, V))
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    bwd = kda.chunk_bwd if chunked else kda.recurrent_bwd
    outs = (torch.empty(B, T, H, K, dtype=shape.dtype, device=dev),
            torch.empty(B, T, H, K, dtype=shape.dtype, device=dev),
            torch.empty(B, T, HV, V, dtype=shape.dtype, device=dev),
            torch.empty(B, T, HV, K, device=dev), torch.empty(B, T, HV, device=dev),
            torch.empty(B, HV, K, V, device=dev))
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], dout, dST)
    kw = {}
    if saved:
        _, ST, snaps = kda.chunk_fwd_snapshots(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], 1024,
                                               initial_state=inp["S0"], output_final_state=True)
        kw = dict(saved_states=snaps, final_state=ST)

    def call():
        bwd(*args, initial_state=inp["S0"], workspace=ws, out=outs, **kw)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    starts, ends = time_calls(call, steps, stream)
    torch.cuda.synchronize()
    ms = sum(s_.elapsed_time(e_) for s_, e_ in zip(starts, ends)) / steps
    flops = backward_alg_flops(B, T, HV, K, V)
    log("[backward %s] avg %.3f ms, %.1f TFLOP/s (15KV per token-head), workspace %.2f GB"
        % (("chunked, saved states" if saved else "chunked") if chunked else "recurrent", ms,
           flops / (ms * 1e-3) / 1e12, ws.numel() / 1e9))
    return dict(avg_ms=ms, flops=flops, tokens=B * T, workspace=ws.numel())


def bench_train_step(shape, steps, warmup, inp=None):
    """One layer's forward and backward as a training step runs them: kda.kda
    under torch.autograd (chunked bf16: kda_chunk_fwd_snapshots keeping a
    state every 1024 tokens, then kda_chunk_bwd_saved), the backward driven by
    given dL/do ~ N(0,1) and dL/dS_T ~ 0.1 N(0,1)."""
    import torch
    import gated_delta_rule_kda_amd as kda
    from gated_delta_rule_kda_amd import synth
    dev = torch.device("cuda:0")
    if inp is None:
        inp = synth.make_prefill_inputs(shape, dev, 0)
    B, T, H, HV, K, V = shape.B, shape.T, shape.H, shape.HV, shape.K, shape.V
    gen = torch.Generator(device=dev).manual_seed(2)
    dout = torch.randn(B, T, HV, V, generator=gen, device=dev).to(shape.dtype)
    dST = torch.randn(B, HV, K, V, generator=gen, device=dev) * 0.1
    leaves = {n: inp[n].detach().clone().requires_grad_(True) for n in ("q", "k", "v", "g", "beta", "S0")}

    def call():
        for t in leaves.values():
            t.grad = None
        o, S = kda.kda(leaves["q"], leaves["k"], leaves["v"], leaves["g"], leaves["beta"],
                       initial_state=leaves["S0"], output_final_state=True)
        torch.autograd.backward([o, S], [dout, dST])

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    starts, ends = time_calls(call, steps, stream)
    torch.cuda.synchronize()
    ms = sum(s_.elapsed_time(e_) for s_, e_ in zip(starts, ends)) / steps
    log("[train step] forward + backward avg %.3f ms" % ms)
    return dict(avg_ms=ms, tokens=B * T)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed prefill calls")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-gqa", action="store_true")
    ap.add_argument("--no-snapshots", action="store_true")
    ap.add_argument("--no-layer-stages", action="store_true")
    ap.add_argument("--no-unbounded", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--only", choices=["prefill", "gqa", "decode", "decode_rows", "copy", "snap", "stages", "unbounded",
                                       "backward", "bandwidth", "layer"],
                    default=None,
                    help="run one workload only (for profiler runs); prints no JSON line")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from gated_delta_rule_kda_amd import synth

    if args.only == "bandwidth":
        measure_copy_bandwidth()
        return
    if args.only == "copy":
        # A plain copy of a known size, for scaling the HBM byte counters.
        n = 256 * 1024 * 1024
        a = torch.empty(n, dtype=torch.float32, device="cuda:0").fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        log("[copy] 5 copies of %d bytes" % (n * 4))
        return
    if args.only == "prefill":
        bench_prefill(synth.PREFILL_HV96_BF16, args.steps, args.warmup, "hv96")
        return
    if args.only == "gqa":
        bench_prefill(synth.PREFILL_GQA_BF16, args.steps, args.warmup, "gqa")
        return
    if args.only == "decode":
        bench_decode(synth.DECODE_B256_HV96, args.decode_steps, args.warmup)
        return
    if args.only == "decode_rows":
        bench_decode(synth.DECODE_B256_HV96, args.decode_steps, args.warmup, ring=False)
        return
    if args.only == "unbounded":
        sh = synth.PREFILL_HV96_BF16
        uinp = synth.make_prefill_inputs(sh, "cuda:0", 0, g_heavy=True)
        bench_prefill(sh, args.steps, args.warmup, "hv96 unbounded gate, chunked", inp=uinp, unbounded=True)
        bench_prefill(sh, args.steps, args.warmup, "hv96 unbounded gate, recurrent", inp=uinp, recurrent=True)
        return
    if args.only == "stages":
        bench_layer_stages(args.steps, args.warmup)
        return
    if args.only == "layer":
        bench_layer_path(synth.PREFILL_HV96_BF16, args.steps, args.warmup, "hv96")
        bench_layer_path(synth.PREFILL_GQA_BF16, args.steps, args.warmup, "gqa")
        return
    if args.only == "backward":
        bench_backward(synth.PREFILL_HV96_BF16, args.steps, args.warmup, chunked=True)
        bench_backward(synth.PREFILL_HV96_BF16, args.steps, args.warmup, chunked=False)
        bench_backward(synth.PREFILL_HV96_BF16, args.steps, args.warmup, chunked=True, saved=True)
        bench_train_step(synth.PREFILL_HV96_BF16, args.steps, args.warmup)
        return
    if args.only == "snap":
        bench_prefill(synth.PREFILL_HV96_BF16, args.steps, args.warmup, "hv96 snapshots/1024", 1024)
        return

    shape = synth.PREFILL_HV96_BF16
    torch.cuda.synchronize()
    p = bench_prefill(shape, args.steps, args.warmup, "hv96")
    ms_per_step = p["span_ms"] / args.steps
    value = p["tokens"] / (ms_per_step * 1e-3)
    achieved = p["bytes"] / (p["avg_ms"] * 1e-3) / 1e9
    traffic = load_counters("prefill_hv96")
    line = {
        "metric": "prefill tokens/s (HV=96,K=V=128) + decode GB/s vs HBM peak, 1 GPU",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "KDA chunked prefill B1 T8192 H=HV=96 K=V=128 bf16 q/k/v, "
                               "fp32 g/beta/state, zero S0, final state returned, chunk 32",
                   "B": shape.B, "T": shape.T, "H": shape.H, "HV": shape.HV, "K": shape.K,
                   "V": shape.V, "chunk": 32, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "prefill_bf16_kernel<128,64>",
                     "alg_bytes_per_launch": p["bytes"], "avg_launch_ms": p["avg_ms"]},
        "mfma": {"alg_flops_per_launch": p["flops"],
                 "achieved_tflops": p["flops"] / (p["avg_ms"] * 1e-3) / 1e12,
                 "peak_tflops": BF16_MFMA_PEAK / 1e12,
                 "frac": p["flops"] / (p["avg_ms"] * 1e-3) / BF16_MFMA_PEAK,
                 "counters": mfma_busy("prefill_hv96", p["avg_ms"])},
    }
    if not args.no_gqa:
        gshape = synth.PREFILL_GQA_BF16
        gq = bench_prefill(gshape, max(3, args.steps // 2), args.warmup, "gqa")
        line["prefill_gqa"] = {
            "workload": "KDA chunked prefill with GQA B8 T4096 H16 HV64 K=V=128 bf16, S0~N(0,0.02^2)",
            "tokens_per_s": gq["tokens"] / (gq["avg_ms"] * 1e-3), "avg_launch_ms": gq["avg_ms"],
            "achieved_gbs": gq["bytes"] / (gq["avg_ms"] * 1e-3) / 1e9,
            "frac_hbm": gq["bytes"] / (gq["avg_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "alg_bytes_per_launch": gq["bytes"]}
        del gq
    if not args.no_snapshots:
        line["prefill_snapshots"] = []
        for every in (1024, 32):
            sp = bench_prefill(shape, max(3, args.steps // 2), args.warmup,
                               "hv96 snapshots/%d" % every, every, inp=p["inp"])
            line["prefill_snapshots"].append({
                "workload": "kda_chunk_fwd_snapshots on the HV96 workload, a state snapshot "
                            "every %d tokens" % every,
                "snapshot_every": every, "tokens_per_s": sp["tokens"] / (sp["avg_ms"] * 1e-3),
                "avg_launch_ms": sp["avg_ms"],
                "alg_bytes_per_launch": sp["bytes"],
                "achieved_gbs": sp["bytes"] / (sp["avg_ms"] * 1e-3) / 1e9,
                "frac_hbm": sp["bytes"] / (sp["avg_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS})
            del sp
    if not args.no_unbounded:
        uinp = dict(p["inp"])
        uinp["g"] = synth.make_prefill_inputs(shape, "cuda:0", 0, g_heavy=True)["g"]
        uc = bench_prefill(shape, max(3, args.steps // 2), args.warmup, "hv96 unbounded gate, chunked",
                           inp=uinp, unbounded=True)
        ub = bench_prefill(shape, max(3, args.steps // 4), min(args.warmup, 3), "hv96 unbounded gate, recurrent",
                           inp=uinp, recurrent=True)
        del uinp
        gc = uc["bytes"] / (uc["avg_ms"] * 1e-3) / 1e9
        tf = ub["flops"] / (ub["avg_ms"] * 1e-3) / 1e12
        line["prefill_unbounded_gate"] = {
            "workload": "kda_chunk_fwd_unbounded on the HV96 workload with g = -exp(1.5 N(0,1)) (no lower "
                        "bound; outside kda_chunk_fwd's -5 <= g <= 0): the in-chunk matrix pass, then the "
                        "bf16 chunk kernel",
            "tokens_per_s": uc["tokens"] / (uc["avg_ms"] * 1e-3), "avg_call_ms": uc["avg_ms"],
            "workspace_bytes": uc["workspace"],
            "roofline": {"bound": "hbm", "achieved": gc, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gc / HBM_PEAK_GBS, "alg_bytes_per_call": uc["bytes"],
                         "kernels": "unb_prep_kernel<128> + prefill_bf16_kernel<128,64> (unbounded)"},
            "mfma": {"alg_flops_per_call": uc["flops"],
                     "achieved_tflops": uc["flops"] / (uc["avg_ms"] * 1e-3) / 1e12,
                     "peak_tflops": BF16_MFMA_PEAK / 1e12,
                     "frac": uc["flops"] / (uc["avg_ms"] * 1e-3) / BF16_MFMA_PEAK},
            "recurrent": {
                "workload": "kda_recurrent_fwd (token recurrence on the vector ALUs) on the same inputs",
                "tokens_per_s": ub["tokens"] / (ub["avg_ms"] * 1e-3), "avg_launch_ms": ub["avg_ms"],
                "roofline": {"bound": "alu", "achieved": tf, "peak": FP32_VALU_PEAK / 1e12, "unit": "TFLOP/s",
                             "frac": tf * 1e12 / FP32_VALU_PEAK,
                             "peak_nonpacked": FP32_VALU_PEAK_NONPACKED / 1e12,
                             "frac_nonpacked": tf * 1e12 / FP32_VALU_PEAK_NONPACKED,
                             "flops_per_launch": ub["flops"]}}}
        del ub, uc
    if not args.no_backward:
        bw = bench_backward(shape, max(3, args.steps // 4), min(args.warmup, 3), inp=p["inp"], chunked=True)
        tf = bw["flops"] / (bw["avg_ms"] * 1e-3) / 1e12
        br = bench_backward(shape, max(3, args.steps // 4), min(args.warmup, 3), inp=p["inp"], chunked=False)
        tr = br["flops"] / (br["avg_ms"] * 1e-3) / 1e12
        bs = bench_backward(shape, max(3, args.steps // 4), min(args.warmup, 3), inp=p["inp"], chunked=True,
                            saved=True)
        ts = bs["flops"] / (bs["avg_ms"] * 1e-3) / 1e12
        line["backward"] = {
            "workload": "kda_chunk_bwd on the HV96 workload (B1 T8192 H=HV=96 K=V=128 bf16, bounded "
                        "gate), dL/do ~ N(0,1), dL/dS_T ~ 0.1 N(0,1): dq, dk, dv, dg, dbeta, dS0",
            "tokens_per_s": bw["tokens"] / (bw["avg_ms"] * 1e-3), "avg_call_ms": bw["avg_ms"],
            "workspace_bytes": bw["workspace"],
            "roofline": {"bound": "mfma", "achieved": tf, "peak": FP32_MFMA_PEAK / 1e12, "unit": "TFLOP/s",
                         "frac": tf * 1e12 / FP32_MFMA_PEAK, "flops_per_call": bw["flops"],
                         "what": "the gradient's own arithmetic (15KV per token and value head) against "
                                 "the fp32 matrix-core peak (the gradient and operand passes multiply fp32 "
                                 "operands; the reverse chain bf16 pairs)"},
            "saved_states": {
                "workload": "kda_chunk_bwd_saved on the same inputs, given the forward's states every 1024 "
                            "tokens and its final state (kda_chunk_fwd_snapshots, run before the timed "
                            "region, as a training step's forward has): no forward over the whole sequence",
                "avg_call_ms": bs["avg_ms"], "tokens_per_s": bs["tokens"] / (bs["avg_ms"] * 1e-3),
                "roofline": {"bound": "mfma", "achieved": ts, "peak": FP32_MFMA_PEAK / 1e12, "unit": "TFLOP/s",
                             "frac": ts * 1e12 / FP32_MFMA_PEAK, "flops_per_call": bs["flops"]}},
            "recurrent": {
                "workload": "kda_recurrent_bwd (token recurrence on the vector ALUs, any finite g) on the "
                            "same inputs",
                "avg_call_ms": br["avg_ms"], "workspace_bytes": br["workspace"],
                "roofline": {"bound": "alu", "achieved": tr, "peak": FP32_VALU_PEAK / 1e12,
                             "unit": "TFLOP/s", "frac": tr * 1e12 / FP32_VALU_PEAK,
                             "peak_nonpacked": FP32_VALU_PEAK_NONPACKED / 1e12,
                             "frac_nonpacked": tr * 1e12 / FP32_VALU_PEAK_NONPACKED,
                             "flops_per_call": br["flops"]}}}
        ts_ = bench_train_step(shape, max(3, args.steps // 4), min(args.warmup, 3), inp=p["inp"])
        line["backward"]["train_step"] = {
            "workload": "one layer's forward and backward under torch.autograd (kda.kda, chunked bf16: "
                        "kda_chunk_fwd_snapshots keeping a state every 1024 tokens, then kda_chunk_bwd_saved), "
                        "driven by given dL/do and dL/dS_T",
            "avg_step_ms": ts_["avg_ms"], "tokens_per_s": ts_["tokens"] / (ts_["avg_ms"] * 1e-3)}
        del bw, br, bs, ts_
    if not args.no_layer_stages:
        st = bench_layer_stages(args.steps, args.warmup)
        line["layer_stages"] = {
            "workload": "the HV96 layer's per-token stages, B1 T8192 H=HV=96 K=V=128 bf16: "
                        "kda_prefill_prologue (conv width 4 + SiLU, L2 norm, bounded gate, beta "
                        "logits, conv registers in and out) and kda_output_gate on o",
            "prologue": {"avg_launch_ms": st["prologue"]["avg_ms"],
                         "alg_bytes_per_launch": st["prologue"]["bytes"],
                         "achieved_gbs": st["prologue"]["gbs"],
                         "frac_hbm": st["prologue"]["gbs"] / HBM_PEAK_GBS},
            "output_gate": {"avg_launch_ms": st["output_gate"]["avg_ms"],
                            "alg_bytes_per_launch": st["output_gate"]["bytes"],
                            "achieved_gbs": st["output_gate"]["gbs"],
                            "frac_hbm": st["output_gate"]["gbs"] / HBM_PEAK_GBS}}
    if not args.no_layer_stages:
        lp = {}
        for tag, sh in (("hv96", synth.PREFILL_HV96_BF16), ("gqa", synth.PREFILL_GQA_BF16)):
            r_ = bench_layer_path(sh, max(3, args.steps // 2), min(args.warmup, 5), tag)
            lp[tag] = {"unfused_ms": r_["unfused_ms"], "fused_ms": r_["fused_ms"],
                       "fused_speedup": r_["unfused_ms"] / r_["fused_ms"]}
        line["layer_path"] = {
            "workload": "prologue (conv width 4 + SiLU, L2 norm) + gate/beta + chunked prefill + output gate, "
                        "end to end: unfused = kda_prefill_prologue -> kda_chunk_fwd -> kda_output_gate, "
                        "fused = kda_prefill_prologue (no gate stage) -> kda_chunk_fwd_gated",
            **lp}
    if not args.no_decode:
        d = bench_decode(synth.DECODE_B256_HV96, args.decode_steps, args.warmup)
        dr = bench_decode(synth.DECODE_B256_HV96, args.decode_steps, args.warmup, ring=False)
        bw_meas = measure_copy_bandwidth()
        line["decode"] = {
            "workload": "KDA recurrent decode, %d steps, B256 H=HV=96 K=V=128 fp32, fused conv4+SiLU "
                        "(conv registers as a [4, B, C] ring), L2 norm, bounded gate -5, beta logits"
                        % args.decode_steps,
            "value": d["gbs"], "unit": "GB/s", "ms_per_token_step": d["per_ms"],
            "steps": args.decode_steps, "seconds_total": d["span_ms"] * 1e-3, "dtype": "f32",
            "roofline": {"bound": "hbm", "achieved": d["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": d["gbs"] / HBM_PEAK_GBS, "traffic": load_counters("decode_b256_ring"),
                         "kernel": "decode_kernel<128,128>", "alg_bytes_per_launch": d["bytes"],
                         "avg_launch_ms": d["per_ms"]},
            "rows_layout": {"what": "the same steps with the conv registers as [B, C, 4] rows, shifted "
                                    "and rewritten whole each step",
                            "ms_per_token_step": dr["per_ms"], "achieved_gbs": dr["gbs"],
                            "frac_hbm": dr["gbs"] / HBM_PEAK_GBS, "traffic": load_counters("decode_b256")},
            "measured_ceilings": {"copy_gbs": bw_meas["copy"], "rmw_in_place_gbs": bw_meas["rmw_in_place"],
                                  "frac_of_copy": d["gbs"] / bw_meas["copy"],
                                  "frac_of_rmw_in_place": d["gbs"] / bw_meas["rmw_in_place"],
                                  "what": "torch copy_ and in-place mul_ over 1 GiB fp32, bytes read + "
                                          "written per second on this GPU"}}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(p["inp"], shape)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
