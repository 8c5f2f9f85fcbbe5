"""KDA (Kimi Delta Attention) forward for AMD Instinct MI355X (gfx950).

A thin Python binding over libkda.so, the HIP library whose C ABI is declared
in include/kda.h.  This module only marshals arguments (device pointers,
sizes, the current HIP stream); every step of the computation runs in the
library's kernels.  torch supplies device memory and streams.

    o, S_T = chunk_fwd(q, k, v, g, beta, scale=None, initial_state=None,
                       output_final_state=False)
    o, S_T, snaps = chunk_fwd_snapshots(q, k, v, g, beta, snapshot_every, ...)
    o, S_T = recurrent_fwd(q, k, v, g, beta, ...)        # any g (unbounded gate)
    q, k, v, g, beta = prefill_prologue(x, z, beta_logits, H=..., ...)
    y = output_gate(o, gate, eps)
    out = decode_step(qkv, gate, beta, state, H=..., ...)   # state updated in place

There is no CPU fallback: calling an op without the built library, or with
tensors that are not on a GPU, raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = ["kda", "chunk_fwd", "chunk_fwd_gated", "chunk_fwd_workspace_size", "recurrent_bwd", "recurrent_bwd_noalloc", "recurrent_bwd_workspace_size", "chunk_bwd", "chunk_bwd_workspace_size", "chunk_fwd_snapshots", "recurrent_fwd", "prefill_prologue", "output_gate", "decode_step", "abi_version", "library_path", "KDAError",
           "GATE_DIRECT", "GATE_BOUNDED", "GATE_SOFTPLUS"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libkda.so")
_lock = threading.Lock()
_lib = None

KDA_OK, KDA_EINVAL, KDA_EUNSUPPORTED, KDA_EHIP = 0, 1, 2, 3
DTYPE_F32, DTYPE_BF16 = 0, 1
GATE_DIRECT, GATE_BOUNDED, GATE_SOFTPLUS = 0, 1, 2
ABI_VERSION = 6


class KDAError(RuntimeError):
    """A non-zero status from libkda, with the library's message."""

    def __init__(self, status: int, message: str):
        super().__init__("libkda status %d: %s" % (status, message))
        self.status = status


class DecodePrologue(ctypes.Structure):
    """Mirror of `kda_decode_prologue` in include/kda.h."""
    _fields_ = [
        ("conv_weight", ctypes.c_void_p),
        ("conv_state", ctypes.c_void_p),
        ("conv_kernel", ctypes.c_int),
        ("l2norm_qk", ctypes.c_int),
        ("l2_eps", ctypes.c_float),
        ("gate_mode", ctypes.c_int),
        ("A_log", ctypes.c_void_p),
        ("dt_bias", ctypes.c_void_p),
        ("gate_lower_bound", ctypes.c_float),
        ("beta_is_logit", ctypes.c_int),
        ("conv_ring", ctypes.c_int),
        ("conv_pos", ctypes.c_int),
    ]


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                raise ImportError(
                    "libkda.so is not built; run `python -m gated_delta_rule_kda_amd.build` "
                    "(expected at %s)" % _LIB_PATH)
            lib = ctypes.CDLL(_LIB_PATH)
            P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
            lib.kda_abi_version.argtypes = []
            lib.kda_abi_version.restype = I
            lib.kda_last_error.argtypes = []
            lib.kda_last_error.restype = ctypes.c_char_p
            lib.kda_chunk_fwd_workspace_size.argtypes = [I] * 8
            lib.kda_chunk_fwd_workspace_size.restype = ctypes.c_longlong
            lib.kda_chunk_fwd.argtypes = [P] * 8 + [I] * 6 + [F, I, I, P, ctypes.c_longlong, P]
            lib.kda_chunk_fwd.restype = I
            lib.kda_chunk_fwd_gated.argtypes = ([P] * 7 + [F, P, P, F, P, P] + [I] * 6 + [F, I, I, P,
                                                ctypes.c_longlong, P])
            lib.kda_chunk_fwd_gated.restype = I
            lib.kda_recurrent_fwd.argtypes = [P] * 8 + [I] * 6 + [F, I, P]
            lib.kda_recurrent_fwd.restype = I
            lib.kda_chunk_fwd_unbounded_workspace_size.argtypes = [I] * 7
            lib.kda_chunk_fwd_unbounded_workspace_size.restype = ctypes.c_longlong
            lib.kda_chunk_fwd_unbounded.argtypes = [P] * 8 + [I] * 6 + [F, I, P, ctypes.c_longlong, P]
            lib.kda_chunk_fwd_unbounded.restype = I
            lib.kda_recurrent_bwd_workspace_size.argtypes = [I] * 6
            lib.kda_recurrent_bwd_workspace_size.restype = ctypes.c_longlong
            lib.kda_recurrent_bwd.argtypes = ([P] * 14 + [I] * 6 + [F, I, P, ctypes.c_longlong, P])
            lib.kda_recurrent_bwd.restype = I
            lib.kda_recurrent_bwd_noalloc.argtypes = ([P] * 14 + [I] * 6 + [F, I, P])
            lib.kda_recurrent_bwd_noalloc.restype = I
            lib.kda_chunk_bwd_workspace_size.argtypes = [I] * 7
            lib.kda_chunk_bwd_workspace_size.restype = ctypes.c_longlong
            lib.kda_chunk_bwd.argtypes = ([P] * 14 + [I] * 6 + [F, I, P, ctypes.c_longlong, P])
            lib.kda_chunk_bwd.restype = I
            lib.kda_chunk_bwd_saved.argtypes = ([P] * 16 + [I] * 6 + [F, I, P, ctypes.c_longlong, P])
            lib.kda_chunk_bwd_saved.restype = I
            lib.kda_chunk_fwd_snapshots.argtypes = [P] * 9 + [I] * 7 + [F, I, I, P, ctypes.c_longlong, P]
            lib.kda_chunk_fwd_snapshots.restype = I
            lib.kda_prefill_prologue.argtypes = ([P, P, P, ctypes.POINTER(DecodePrologue)] + [P] * 5
                                                 + [I] * 6 + [I, P])
            lib.kda_prefill_prologue.restype = I
            lib.kda_output_gate.argtypes = [P, P, P, ctypes.c_longlong, I, F, I, P]
            lib.kda_output_gate.restype = I
            lib.kda_decode_step.argtypes = [P] * 5 + [ctypes.POINTER(DecodePrologue)] + [I] * 5 + [F, I, P]
            lib.kda_decode_step.restype = I
            if lib.kda_abi_version() != ABI_VERSION:
                raise ImportError("libkda ABI %d, binding expects %d" % (lib.kda_abi_version(), ABI_VERSION))
            _lib = lib
    return _lib


def abi_version() -> int:
    return _load().kda_abi_version()


def _check(status: int):
    if status != KDA_OK:
        raise KDAError(status, _load().kda_last_error().decode(errors="replace"))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return DTYPE_BF16
    if dt == torch.float32:
        return DTYPE_F32
    raise TypeError("q/k/v must be bfloat16 or float32, got %s" % dt)


def _stream_handle(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype=None, shape=None, device=None):
    if t is None:
        raise ValueError("%s is required" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor (libkda has no CPU path)" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))


def _prefill_args(q, k, v, g, beta, initial_state, output_final_state, out, final_state):
    _need(q, "q")
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    dt = q.dtype
    dev = q.device
    _need(k, "k", dt, (B, T, H, K), dev)
    _need(v, "v", dt, (B, T, HV, V), dev)
    _need(g, "g", torch.float32, (B, T, HV, K), dev)
    _need(beta, "beta", torch.float32, (B, T, HV), dev)
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (B, HV, K, V), dev)
    if out is None:
        out = torch.empty(B, T, HV, V, dtype=dt, device=dev)
    else:
        _need(out, "out", dt, (B, T, HV, V), dev)
    if final_state is None and output_final_state:
        final_state = torch.empty(B, HV, K, V, dtype=torch.float32, device=dev)
    elif final_state is not None:
        _need(final_state, "final_state", torch.float32, (B, HV, K, V), dev)
    return (B, T, H, HV, K, V), out, final_state


def chunk_fwd_workspace_size(B, T, H, HV, K, V, chunk_size=32, dtype=torch.bfloat16) -> int:
    """Bytes of workspace ``kda_chunk_fwd`` (and ``kda_chunk_fwd_snapshots``)
    needs for these sizes (0 for the fused kernels built here)."""
    n = _load().kda_chunk_fwd_workspace_size(B, T, H, HV, K, V, int(chunk_size), _dtype_code(dtype))
    if n < 0:
        raise KDAError(KDA_EINVAL, _load().kda_last_error().decode(errors="replace"))
    return n


def _prefill_workspace(workspace, shape, chunk_size, dtype, dev):
    """The caller's workspace (a uint8 GPU tensor), or one of the size the
    library asks for (None when it needs none)."""
    B, T, H, HV, K, V = shape
    nbytes = chunk_fwd_workspace_size(B, T, H, HV, K, V, chunk_size, dtype)
    if workspace is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes > 0 else None
    _need(workspace, "workspace", torch.uint8, None, dev)
    return workspace


def chunk_fwd_snapshots(q, k, v, g, beta, snapshot_every, scale=None, initial_state=None,
                        output_final_state=False, *, chunk_size=32, out=None,
                        final_state=None, snapshots=None, workspace=None):
    """``kda_chunk_fwd_snapshots``: :func:`chunk_fwd` that also returns prefix
    snapshots [B, T // snapshot_every, HV, K, V] fp32, snapshot j being the
    state after the first (j+1)*snapshot_every tokens (a positive multiple of
    32).  Returns (o, final state or None, snapshots)."""
    (B, T, H, HV, K, V), out, final_state = _prefill_args(
        q, k, v, g, beta, initial_state, output_final_state, out, final_state)
    dev = q.device
    every = int(snapshot_every)
    if every < 32 or every % 32 != 0:
        raise ValueError("snapshot_every=%d must be a positive multiple of the chunk size 32" % every)
    NS = T // every
    if snapshots is None:
        snapshots = torch.empty(B, NS, HV, K, V, dtype=torch.float32, device=dev)
    else:
        _need(snapshots, "snapshots", torch.float32, (B, NS, HV, K, V), dev)
    ws = _prefill_workspace(workspace, (B, T, H, HV, K, V), chunk_size, q.dtype, dev)
    with torch.cuda.device(dev):
        _check(_load().kda_chunk_fwd_snapshots(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(out),
            _ptr(final_state), _ptr(snapshots), every, B, T, H, HV, K, V,
            float(scale) if scale else 0.0, int(chunk_size), _dtype_code(q.dtype),
            _ptr(ws), ws.numel() if ws is not None else 0, _stream_handle(dev)))
    return out, final_state, snapshots


def recurrent_fwd(q, k, v, g, beta, scale=None, initial_state=None, output_final_state=False,
                  *, out=None, final_state=None):
    """``kda_recurrent_fwd``: :func:`chunk_fwd`'s computation for gates without
    a lower bound (any finite g), token by token with the state on chip."""
    (B, T, H, HV, K, V), out, final_state = _prefill_args(
        q, k, v, g, beta, initial_state, output_final_state, out, final_state)
    dev = q.device
    with torch.cuda.device(dev):
        _check(_load().kda_recurrent_fwd(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(out),
            _ptr(final_state), B, T, H, HV, K, V, float(scale) if scale else 0.0,
            _dtype_code(q.dtype), _stream_handle(dev)))
    return out, final_state


def chunk_fwd_unbounded_workspace_size(B, T, H, HV, K, V, dtype=torch.bfloat16) -> int:
    """Bytes of workspace ``kda_chunk_fwd_unbounded`` needs for these sizes
    (bf16 only)."""
    n = _load().kda_chunk_fwd_unbounded_workspace_size(B, T, H, HV, K, V, _dtype_code(dtype))
    if n < 0:
        raise KDAError(KDA_EINVAL, _load().kda_last_error().decode(errors="replace"))
    return n


def chunk_fwd_unbounded(q, k, v, g, beta, scale=None, initial_state=None, output_final_state=False,
                        *, out=None, final_state=None, workspace=None):
    """``kda_chunk_fwd_unbounded``: :func:`chunk_fwd` for gates with no lower
    bound (any g <= 0; each token's g floored at -17), on the matrix cores.
    bf16 inputs only.  ``workspace``: a uint8 GPU tensor of at least
    :func:`chunk_fwd_unbounded_workspace_size` bytes, else one is allocated."""
    (B, T, H, HV, K, V), out, final_state = _prefill_args(
        q, k, v, g, beta, initial_state, output_final_state, out, final_state)
    dev = q.device
    if workspace is None:
        n = chunk_fwd_unbounded_workspace_size(B, T, H, HV, K, V, q.dtype)
        workspace = torch.empty(n, dtype=torch.uint8, device=dev) if n > 0 else None
    else:
        _need(workspace, "workspace", torch.uint8, None, dev)
    with torch.cuda.device(dev):
        _check(_load().kda_chunk_fwd_unbounded(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(out),
            _ptr(final_state), B, T, H, HV, K, V, float(scale) if scale else 0.0,
            _dtype_code(q.dtype), _ptr(workspace), workspace.numel() if workspace is not None else 0,
            _stream_handle(dev)))
    return out, final_state


def recurrent_bwd_workspace_size(B, T, H, HV, K, V) -> int:
    """Bytes of workspace ``kda_recurrent_bwd`` needs for these sizes."""
    n = _load().kda_recurrent_bwd_workspace_size(B, T, H, HV, K, V)
    if n < 0:
        raise KDAError(KDA_EINVAL, _load().kda_last_error().decode(errors="replace"))
    return n


NOALLOC_SCRATCH_BYTES = 128 << 20   # KDA_NOALLOC_SCRATCH_BYTES of include/kda.h


def recurrent_bwd_noalloc(q, k, v, g, beta, dout, d_final_state=None, scale=None,
                          initial_state=None, *, need_d_initial_state=True, out=None):
    """``kda_recurrent_bwd_noalloc``: :func:`recurrent_bwd` without a
    workspace, for callers that cannot allocate: the library's own scratch
    array (``NOALLOC_SCRATCH_BYTES`` per GPU) serves instead, so sizes whose
    :func:`recurrent_bwd_workspace_size` exceeds it are rejected.  Calls that
    overlap in time on one GPU race on that array.  Pass ``out`` (the six
    result tensors) to allocate nothing on this side either."""
    return recurrent_bwd(q, k, v, g, beta, dout, d_final_state, scale, initial_state,
                         need_d_initial_state=need_d_initial_state, out=out, _noalloc=True)


def chunk_bwd_workspace_size(B, T, H, HV, K, V, dtype=torch.bfloat16) -> int:
    """Bytes of workspace ``kda_chunk_bwd`` needs for these sizes."""
    n = _load().kda_chunk_bwd_workspace_size(B, T, H, HV, K, V, _dtype_code(dtype))
    if n < 0:
        raise KDAError(KDA_EINVAL, _load().kda_last_error().decode(errors="replace"))
    return n


def chunk_bwd(q, k, v, g, beta, dout, d_final_state=None, scale=None, initial_state=None,
              *, workspace=None, need_d_initial_state=True, out=None, saved_states=None,
              final_state=None):
    """``kda_chunk_bwd``: :func:`recurrent_bwd` in the chunk form on the
    matrix cores, for bf16 inputs with -5 <= g <= 0 (the inputs of
    :func:`chunk_fwd`).  Same arguments and results; ``workspace`` of at
    least :func:`chunk_bwd_workspace_size` bytes.  With ``saved_states``
    (the snapshots of :func:`chunk_fwd_snapshots` at snapshot_every = 1024,
    [B, T // 1024, HV, K, V]; None allowed when T <= 1024) and
    ``final_state`` (the forward's final state, needed with d_final_state)
    it calls ``kda_chunk_bwd_saved``, which does not run the forward again."""
    saved = saved_states is not None or final_state is not None
    return recurrent_bwd(q, k, v, g, beta, dout, d_final_state, scale, initial_state,
                         workspace=workspace, need_d_initial_state=need_d_initial_state,
                         out=out, _chunked=True, _saved=(saved_states, final_state) if saved else None)


def recurrent_bwd(q, k, v, g, beta, dout, d_final_state=None, scale=None, initial_state=None,
                  *, workspace=None, need_d_initial_state=True, out=None, _noalloc=False,
                  _chunked=False, _saved=None):
    """``kda_recurrent_bwd``: gradients of the forward pass with the same
    inputs (any finite g).  dout [B,T,HV,V] is dL/do (v's dtype),
    d_final_state [B,HV,K,V] fp32 (or None) is dL/dS_T.  Returns (dq, dk
    [B,T,H,K] and dv [B,T,HV,V] in q's dtype, dg [B,T,HV,K], dbeta [B,T,HV],
    dS0 [B,HV,K,V] fp32 or None).  ``workspace`` (a uint8 GPU tensor of at
    least :func:`recurrent_bwd_workspace_size` bytes) may be passed to avoid
    an allocation, and ``out`` (the six result tensors, dS0 may be None) to
    write into."""
    _need(q, "q")
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    dt, dev = q.dtype, q.device
    _need(k, "k", dt, (B, T, H, K), dev)
    _need(v, "v", dt, (B, T, HV, V), dev)
    _need(g, "g", torch.float32, (B, T, HV, K), dev)
    _need(beta, "beta", torch.float32, (B, T, HV), dev)
    _need(dout, "dout", dt, (B, T, HV, V), dev)
    for t_, n_ in ((initial_state, "initial_state"), (d_final_state, "d_final_state")):
        if t_ is not None:
            _need(t_, n_, torch.float32, (B, HV, K, V), dev)
    if _saved is not None:
        if _saved[0] is not None:
            _need(_saved[0], "saved_states", torch.float32, (B, T // 1024, HV, K, V), dev)
        if _saved[1] is not None:
            _need(_saved[1], "final_state", torch.float32, (B, HV, K, V), dev)
    if not _noalloc:
        nbytes = (chunk_bwd_workspace_size(B, T, H, HV, K, V, dt) if _chunked
                  else recurrent_bwd_workspace_size(B, T, H, HV, K, V))
        if workspace is None:
            workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
        else:
            _need(workspace, "workspace", torch.uint8, None, dev)
    if out is None:
        dq = torch.empty(B, T, H, K, dtype=dt, device=dev)
        dk = torch.empty(B, T, H, K, dtype=dt, device=dev)
        dv = torch.empty(B, T, HV, V, dtype=dt, device=dev)
        dg = torch.empty(B, T, HV, K, dtype=torch.float32, device=dev)
        db = torch.empty(B, T, HV, dtype=torch.float32, device=dev)
        dS0 = torch.empty(B, HV, K, V, dtype=torch.float32, device=dev) if need_d_initial_state else None
    else:
        dq, dk, dv, dg, db, dS0 = out
        for t_, n_, d_, s_ in ((dq, "dq", dt, (B, T, H, K)), (dk, "dk", dt, (B, T, H, K)),
                               (dv, "dv", dt, (B, T, HV, V)), (dg, "dg", torch.float32, (B, T, HV, K)),
                               (db, "dbeta", torch.float32, (B, T, HV))):
            _need(t_, n_, d_, s_, dev)
        if dS0 is not None:
            _need(dS0, "dS0", torch.float32, (B, HV, K, V), dev)
    with torch.cuda.device(dev):
        if _noalloc:
            _check(_load().kda_recurrent_bwd_noalloc(
                _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(dout),
                _ptr(d_final_state), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(db), _ptr(dS0),
                B, T, H, HV, K, V, float(scale) if scale else 0.0, _dtype_code(dt), _stream_handle(dev)))
        elif _saved is not None:
            _check(_load().kda_chunk_bwd_saved(
                _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(_saved[0]),
                _ptr(_saved[1]), _ptr(dout), _ptr(d_final_state), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg),
                _ptr(db), _ptr(dS0), B, T, H, HV, K, V, float(scale) if scale else 0.0, _dtype_code(dt),
                _ptr(workspace), workspace.numel(), _stream_handle(dev)))
        else:
            entry = _load().kda_chunk_bwd if _chunked else _load().kda_recurrent_bwd
            _check(entry(
                _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(dout),
                _ptr(d_final_state), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(db), _ptr(dS0),
                B, T, H, HV, K, V, float(scale) if scale else 0.0, _dtype_code(dt), _ptr(workspace),
                workspace.numel(), _stream_handle(dev)))
    return dq, dk, dv, dg, db, dS0


def chunk_fwd(q, k, v, g, beta, scale=None, initial_state=None, output_final_state=False,
              *, chunk_size=32, out=None, final_state=None, workspace=None):
    """Chunk-parallel KDA prefill (``kda_chunk_fwd``).

    q, k [B,T,H,K]; v [B,T,HV,V] (all bf16 or all fp32); g [B,T,HV,K] fp32 with
    -5 <= g <= 0; beta [B,T,HV] fp32; initial_state [B,HV,K,V] fp32 or None.
    Returns (o [B,T,HV,V] in v's dtype, final state [B,HV,K,V] fp32 or None).
    ``final_state`` may be passed (even the initial_state tensor itself, to
    resume in place); ``out`` may be passed to avoid an allocation, and
    ``workspace`` (a uint8 GPU tensor of at least
    :func:`chunk_fwd_workspace_size` bytes) to avoid one for scratch.
    """
    (B, T, H, HV, K, V), out, final_state = _prefill_args(
        q, k, v, g, beta, initial_state, output_final_state, out, final_state)
    dev = q.device
    ws = _prefill_workspace(workspace, (B, T, H, HV, K, V), chunk_size, q.dtype, dev)
    with torch.cuda.device(dev):
        _check(_load().kda_chunk_fwd(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(out),
            _ptr(final_state), B, T, H, HV, K, V, float(scale) if scale else 0.0,
            int(chunk_size), _dtype_code(q.dtype), _ptr(ws), ws.numel() if ws is not None else 0,
            _stream_handle(dev)))
    return out, final_state


def chunk_fwd_gated(q, k, v, z, beta_logit, A_log, dt_bias, gate_lower_bound=-5.0, scale=None,
                    initial_state=None, output_final_state=False, *, out_gate=None,
                    out_gate_eps=1e-6, chunk_size=32, out=None, final_state=None, workspace=None):
    """``kda_chunk_fwd_gated``: :func:`chunk_fwd` with the gate
    g = lb * sigmoid(exp(A_log) (z + dt_bias)) and beta = sigmoid(beta_logit)
    formed in the kernel, and, with ``out_gate``, the output gate
    y = sigmoid(out_gate) * o / sqrt(mean(o^2) + eps) applied to o.  bf16 only.
    z [B,T,HV,K] fp32; beta_logit [B,T,HV] fp32; A_log [HV]; dt_bias [HV*K];
    out_gate [B,T,HV,V] bf16 or None.  Returns (y or o, final state or None)."""
    (B, T, H, HV, K, V), out, final_state = _prefill_args(
        q, k, v, z, beta_logit, initial_state, output_final_state, out, final_state)
    dev = q.device
    _need(A_log, "A_log", torch.float32, (HV,), dev)
    _need(dt_bias, "dt_bias", torch.float32, (HV * K,), dev)
    if out_gate is not None:
        _need(out_gate, "out_gate", q.dtype, (B, T, HV, V), dev)
    ws = _prefill_workspace(workspace, (B, T, H, HV, K, V), chunk_size, q.dtype, dev)
    with torch.cuda.device(dev):
        _check(_load().kda_chunk_fwd_gated(
            _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(beta_logit), _ptr(A_log), _ptr(dt_bias),
            float(gate_lower_bound), _ptr(initial_state), _ptr(out_gate), float(out_gate_eps),
            _ptr(out), _ptr(final_state), B, T, H, HV, K, V, float(scale) if scale else 0.0,
            int(chunk_size), _dtype_code(q.dtype), _ptr(ws), ws.numel() if ws is not None else 0,
            _stream_handle(dev)))
    return out, final_state


class _KDA(torch.autograd.Function):
    """Forward by kda_chunk_fwd (chunked, bounded gate), kda_chunk_fwd_unbounded
    (chunked, bf16, any g <= 0) or kda_recurrent_fwd; backward by kda_chunk_bwd
    (after a chunked bf16 forward with the bounded gate) or kda_recurrent_bwd:
    all compute the same function and its gradients."""

    @staticmethod
    def forward(ctx, q, k, v, g, beta, initial_state, scale, chunked, bounded_gate):
        unbounded = chunked and not bounded_gate and q.dtype == torch.bfloat16
        ctx.chunked = chunked and bounded_gate and q.dtype == torch.bfloat16
        snaps = None
        if ctx.chunked:
            # the states every 1024 tokens, so that the backward does not run
            # the forward again (kda_chunk_bwd_saved)
            o, S, snaps = chunk_fwd_snapshots(q, k, v, g, beta, 1024, scale=scale, initial_state=initial_state,
                                              output_final_state=True)
        else:
            fwd = chunk_fwd_unbounded if unbounded else chunk_fwd if chunked and bounded_gate else recurrent_fwd
            o, S = fwd(q, k, v, g, beta, scale=scale, initial_state=initial_state, output_final_state=True)
        ctx.save_for_backward(q, k, v, g, beta, initial_state, snaps, S)
        ctx.scale = scale
        return o, S

    @staticmethod
    def backward(ctx, do, dS):
        q, k, v, g, beta, S0, snaps, ST = ctx.saved_tensors
        do = torch.zeros_like(v) if do is None else do.contiguous()
        dS = None if dS is None else dS.contiguous()
        if ctx.chunked:
            dq, dk, dv, dg, db, dS0 = chunk_bwd(q, k, v, g, beta, do, dS, scale=ctx.scale, initial_state=S0,
                                                need_d_initial_state=S0 is not None, saved_states=snaps,
                                                final_state=ST)
        else:
            dq, dk, dv, dg, db, dS0 = recurrent_bwd(q, k, v, g, beta, do, dS, scale=ctx.scale, initial_state=S0,
                                                    need_d_initial_state=S0 is not None)
        return dq, dk, dv, dg, db, dS0, None, None, None


def kda(q, k, v, g, beta, scale=None, initial_state=None, output_final_state=False, *, chunked=True,
        bounded_gate=True):
    """KDA forward with autograd: the interface of naive_kda on the
    "K3/kda/ops/reference/recurrent.py" page.  Returns (o, final state or
    None); gradients reach q, k, v, g, beta and initial_state.  The forward:
    chunked with ``bounded_gate`` (-5 <= g <= 0), kda_chunk_fwd (for bf16 its
    snapshot form, keeping the state every 1024 tokens for the backward);
    chunked without it, kda_chunk_fwd_unbounded for bf16 inputs (any g <= 0,
    each token's g floored at -17) and kda_recurrent_fwd for fp32; not
    chunked, kda_recurrent_fwd (any g).  The backward is kda_chunk_bwd_saved
    (given those states) after a chunked bf16 forward with the bounded gate,
    else kda_recurrent_bwd (which takes g as given: where the forward floored
    it, the two differ by the gradient of less than e^-17 of the state)."""
    o, S = _KDA.apply(q, k, v, g, beta, initial_state, scale, chunked, bounded_gate)
    return o, (S if output_final_state else None)


def _conv_fields(pro, C, B, dev, conv_weight, conv_state, conv_ring, conv_pos, need_state):
    """The conv fields of the prologue struct: conv_state is [B, C, KW]
    (oldest register first), or with ``conv_ring`` the [KW, B, C] ring whose
    oldest register sits in slot ``conv_pos``."""
    KW = conv_weight.shape[-1]
    _need(conv_weight, "conv_weight", torch.float32, (C, KW), dev)
    pro.conv_weight = conv_weight.data_ptr()
    if conv_state is not None or need_state:
        _need(conv_state, "conv_state", torch.float32, (KW, B, C) if conv_ring else (B, C, KW), dev)
        pro.conv_state = conv_state.data_ptr()
    pro.conv_kernel = KW
    if conv_ring:
        pro.conv_ring = 1
        pro.conv_pos = int(conv_pos)


def _prologue_struct(C, dev, conv_weight, conv_state, l2norm_qk, l2_eps, gate_mode, A_log,
                     dt_bias, gate_lower_bound, beta_is_logit, HV, K, B, conv_ring=False, conv_pos=0):
    pro = DecodePrologue()
    use = False
    if conv_weight is not None:
        _conv_fields(pro, C, B, dev, conv_weight, conv_state, conv_ring, conv_pos, False)
        use = True
    if l2norm_qk:
        pro.l2norm_qk = 1
        pro.l2_eps = float(l2_eps)
        use = True
    if gate_mode != GATE_DIRECT:
        _need(A_log, "A_log", torch.float32, (HV,), dev)
        _need(dt_bias, "dt_bias", torch.float32, (HV * K,), dev)
        pro.gate_mode = int(gate_mode)
        pro.A_log = A_log.data_ptr()
        pro.dt_bias = dt_bias.data_ptr()
        pro.gate_lower_bound = float(gate_lower_bound)
        use = True
    if beta_is_logit:
        pro.beta_is_logit = 1
        use = True
    return pro, use


def prefill_prologue(x, gate, beta, *, H, HV, K, V, conv_weight=None, conv_state=None,
                     l2norm_qk=False, l2_eps=1e-6, gate_mode=GATE_DIRECT, A_log=None,
                     dt_bias=None, gate_lower_bound=-5.0, beta_is_logit=False, out=None,
                     conv_ring=False, conv_pos=0):
    """``kda_prefill_prologue``: the decode prologue's stages over all T tokens.

    x [B,T,2HK+HV*V] (bf16 or fp32), gate [B,T,HV,K] fp32 (g or z), beta
    [B,T,HV] fp32 (or logits); ``conv_state`` [B,C,KW] fp32 (with
    ``conv_ring``: the [KW,B,C] ring, oldest register in slot ``conv_pos``;
    the caller then advances conv_pos by T mod KW) is read and then
    overwritten with the registers after the last token.  Returns
    (q [B,T,H,K], k, v [B,T,HV,V] in x's dtype, g [B,T,HV,K] fp32, beta [B,T,HV] fp32)
    -- the inputs of :func:`chunk_fwd`.  ``out`` may supply those five tensors.
    With ``gate`` and ``beta`` both None the gate and beta stages are skipped
    (g and beta come back as None): the inputs of :func:`chunk_fwd_gated`,
    which forms them itself.
    """
    _need(x, "x")
    B, T = x.shape[0], x.shape[1]
    C = 2 * H * K + HV * V
    dt = x.dtype
    dev = x.device
    if tuple(x.shape) != (B, T, C):
        raise ValueError("x has shape %s, expected %s" % (tuple(x.shape), (B, T, C)))
    gate_stage = gate is not None or beta is not None
    if gate_stage:
        _need(gate, "gate", torch.float32, (B, T, HV, K), dev)
        _need(beta, "beta", torch.float32, (B, T, HV), dev)
    if out is None:
        out = (torch.empty(B, T, H, K, dtype=dt, device=dev), torch.empty(B, T, H, K, dtype=dt, device=dev),
               torch.empty(B, T, HV, V, dtype=dt, device=dev),
               torch.empty(B, T, HV, K, dtype=torch.float32, device=dev) if gate_stage else None,
               torch.empty(B, T, HV, dtype=torch.float32, device=dev) if gate_stage else None)
    q, k, v, g, bo = out
    _need(q, "q", dt, (B, T, H, K), dev)
    _need(k, "k", dt, (B, T, H, K), dev)
    _need(v, "v", dt, (B, T, HV, V), dev)
    if gate_stage:
        _need(g, "g", torch.float32, (B, T, HV, K), dev)
        _need(bo, "beta_out", torch.float32, (B, T, HV), dev)
    else:
        g = bo = None
    pro, use = _prologue_struct(C, dev, conv_weight, conv_state, l2norm_qk, l2_eps, gate_mode,
                                A_log, dt_bias, gate_lower_bound, beta_is_logit, HV, K, B,
                                conv_ring, conv_pos)
    with torch.cuda.device(dev):
        _check(_load().kda_prefill_prologue(
            _ptr(x), _ptr(gate), _ptr(beta), ctypes.byref(pro) if use else None,
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(bo), B, T, H, HV, K, V,
            _dtype_code(dt), _stream_handle(dev)))
    return q, k, v, g, bo


def output_gate(o, gate, eps=1e-6, *, out=None):
    """``kda_output_gate``: y = sigmoid(gate) * o / sqrt(mean(o^2) + eps) over
    the last dimension (the head dimension).  ``out`` may be ``o`` (in place)."""
    _need(o, "o")
    dev = o.device
    D = o.shape[-1]
    _need(gate, "gate", o.dtype, tuple(o.shape), dev)
    if out is None:
        out = torch.empty_like(o)
    else:
        _need(out, "out", o.dtype, tuple(o.shape), dev)
    with torch.cuda.device(dev):
        _check(_load().kda_output_gate(_ptr(o), _ptr(gate), _ptr(out), o.numel() // D, D,
                                       float(eps), _dtype_code(o.dtype), _stream_handle(dev)))
    return out


def decode_step(qkv, gate, beta, state, *, H, HV, K, V, scale=None, out=None,
                conv_weight=None, conv_state=None, l2norm_qk=False, l2_eps=1e-6,
                gate_mode=GATE_DIRECT, A_log=None, dt_bias=None, gate_lower_bound=-5.0,
                beta_is_logit=False, conv_ring=False, conv_pos=0):
    """One decode token (``kda_decode_step``); ``state`` (and ``conv_state``)
    are updated in place.  qkv [B, 2HK+HV*V] (bf16 or fp32), gate [B,HV,K] fp32
    (g, or z for the BOUNDED/SOFTPLUS gate modes), beta [B,HV] fp32.
    ``conv_state`` is [B,C,KW], or with ``conv_ring`` the [KW,B,C] ring whose
    oldest register sits in slot ``conv_pos`` (the caller then advances
    conv_pos by 1 mod KW).  Returns out [B,HV,V] in qkv's dtype."""
    _need(qkv, "qkv")
    B = qkv.shape[0]
    C = 2 * H * K + HV * V
    dt = qkv.dtype
    dev = qkv.device
    if tuple(qkv.shape) != (B, C):
        raise ValueError("qkv has shape %s, expected %s" % (tuple(qkv.shape), (B, C)))
    _need(gate, "gate", torch.float32, (B, HV, K), dev)
    _need(beta, "beta", torch.float32, (B, HV), dev)
    _need(state, "state", torch.float32, (B, HV, K, V), dev)
    if out is None:
        out = torch.empty(B, HV, V, dtype=dt, device=dev)
    else:
        _need(out, "out", dt, (B, HV, V), dev)
    pro = DecodePrologue()
    use_pro = False
    if conv_weight is not None:
        _conv_fields(pro, C, B, dev, conv_weight, conv_state, conv_ring, conv_pos, True)
        use_pro = True
    if l2norm_qk:
        pro.l2norm_qk = 1
        pro.l2_eps = float(l2_eps)
        use_pro = True
    if gate_mode != GATE_DIRECT:
        _need(A_log, "A_log", torch.float32, (HV,), dev)
        _need(dt_bias, "dt_bias", torch.float32, (HV * K,), dev)
        pro.gate_mode = int(gate_mode)
        pro.A_log = A_log.data_ptr()
        pro.dt_bias = dt_bias.data_ptr()
        pro.gate_lower_bound = float(gate_lower_bound)
        use_pro = True
    if beta_is_logit:
        pro.beta_is_logit = 1
        use_pro = True
    with torch.cuda.device(dev):
        _check(_load().kda_decode_step(
            _ptr(qkv), _ptr(gate), _ptr(beta), _ptr(state), _ptr(out),
            ctypes.byref(pro) if use_pro else None, B, H, HV, K, V,
            float(scale) if scale else 0.0, _dtype_code(dt), _stream_handle(dev)))
    return out
