"""KDA CPU oracle -- TEST INFRASTRUCTURE ONLY.

Plain, slow fp64 reference for the Kimi Delta Attention forward pass, used to
check the HIP library.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the product package never
does, and the two share no code.

The arithmetic lives in ``kda_oracle.c`` (token loop and decode step, compiled
with gcc) and ``chunk_mirror.py`` (the chunk algebra in numpy).  This module
only marshals arrays: every input is upcast exactly to float64 (bf16 and fp32
values are exactly representable) before the C code runs.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math) next to its source."""
    if force or not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True, cwd=_HERE)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB_PATH)
            P = ctypes.c_void_p
            L = ctypes.c_long
            D = ctypes.c_double
            I = ctypes.c_int
            lib.kda_oracle_threads.argtypes = []
            lib.kda_oracle_threads.restype = I
            lib.kda_oracle_fwd.argtypes = [P] * 8 + [L] * 6 + [D]
            lib.kda_oracle_fwd.restype = I
            lib.kda_oracle_fwd_snapshots.argtypes = [P] * 9 + [L] * 7 + [D]
            lib.kda_oracle_fwd_snapshots.restype = I
            lib.kda_oracle_bwd.argtypes = [P] * 14 + [L] * 6 + [D]
            lib.kda_oracle_bwd.restype = I
            lib.kda_oracle_decode_step.argtypes = (
                [P, P, P, L, I, D, P, P, P, I, D, P, I, P, P] + [L] * 5 + [D])
            lib.kda_oracle_decode_step.restype = I
            lib.kda_oracle_prefill_prologue.argtypes = (
                [P, P, P, L, I, D, P, P, P, I, D, P, I, P, P, P, P, P] + [L] * 6)
            lib.kda_oracle_prefill_prologue.restype = I
            lib.kda_oracle_output_gate.argtypes = [P, P, P, L, L, D]
            lib.kda_oracle_output_gate.restype = I
            lib.kda_oracle_gate.argtypes = [P, P, P, I, D, P, L, L, L]
            lib.kda_oracle_gate.restype = I
            lib.kda_oracle_conv_update.argtypes = [P, P, P, P, L, L, L]
            lib.kda_oracle_conv_update.restype = I
            lib.kda_oracle_l2norm_rows.argtypes = [P, L, L, D]
            lib.kda_oracle_l2norm_rows.restype = I
            lib.kda_oracle_sigmoid.argtypes = [D]
            lib.kda_oracle_sigmoid.restype = D
            lib.kda_oracle_softplus.argtypes = [D]
            lib.kda_oracle_softplus.restype = D
            _lib = lib
    return _lib


def f64(x) -> np.ndarray:
    """Exact upcast of a numpy array or (CPU or device) torch tensor to float64."""
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def kda_fwd(q, k, v, g, beta, scale=None, initial_state=None, output_final_state=True,
            snapshot_every=None):
    """Token-by-token KDA forward in fp64.

    Follows naive_kda_fwd on the "K3/kda/ops/reference/recurrent.py" page:
    q, k [B,T,H,K]; v [B,T,HV,V]; g [B,T,HV,K]; beta [B,T,HV];
    initial_state [B,HV,K,V] or None.  Returns (o [B,T,HV,V], S_T or None),
    and with ``snapshot_every`` a third array [B, T // every, HV, K, V]: the
    state after each whole multiple of ``every`` tokens (the prefix snapshots
    that the prefix-cache test on the "metrale_model_weights/kimi_k3_host/kda.rs"
    page resumes decoding from).
    """
    q, k, v, g, beta = (f64(a) for a in (q, k, v, g, beta))
    S0 = f64(initial_state)
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    assert k.shape == q.shape and v.shape[:2] == (B, T)
    assert g.shape == (B, T, HV, K) and beta.shape == (B, T, HV)
    if S0 is not None:
        assert S0.shape == (B, HV, K, V)
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    o = np.zeros((B, T, HV, V), dtype=np.float64)
    S = np.zeros((B, HV, K, V), dtype=np.float64)
    snaps, every = None, 0
    if snapshot_every is not None:
        every = int(snapshot_every)
        assert every >= 1
        snaps = np.zeros((B, T // every, HV, K, V), dtype=np.float64)
    rc = _load().kda_oracle_fwd_snapshots(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(o), _ptr(S),
        _ptr(snaps), every, B, T, H, HV, K, V, float(scale))
    if rc != 0:
        raise RuntimeError("kda_oracle_fwd failed with status %d" % rc)
    if snapshot_every is not None:
        return o, (S if output_final_state else None), snaps
    return o, (S if output_final_state else None)


def kda_bwd(q, k, v, g, beta, dout, d_final_state=None, scale=None, initial_state=None):
    """Gradients of kda_fwd in fp64 by back-propagation through time, as the
    backward of KDAFunction on the "K3/kda/ops/reference/recurrent.py" page
    derives them, with the gradient of the initial state kept.

    dout [B,T,HV,V] is dL/do, d_final_state [B,HV,K,V] (or None = 0) is
    dL/dS_T.  Returns (dq, dk [B,T,H,K], dv [B,T,HV,V], dg [B,T,HV,K],
    dbeta [B,T,HV], dS0 [B,HV,K,V]).
    """
    q, k, v, g, beta, do = (f64(a) for a in (q, k, v, g, beta, dout))
    S0, dST = f64(initial_state), f64(d_final_state)
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    assert k.shape == q.shape and v.shape[:2] == (B, T) and do.shape == v.shape
    assert g.shape == (B, T, HV, K) and beta.shape == (B, T, HV)
    for st in (S0, dST):
        if st is not None:
            assert st.shape == (B, HV, K, V)
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    dq = np.zeros((B, T, H, K))
    dk = np.zeros((B, T, H, K))
    dv = np.zeros((B, T, HV, V))
    dg = np.zeros((B, T, HV, K))
    db = np.zeros((B, T, HV))
    dS0 = np.zeros((B, HV, K, V))
    rc = _load().kda_oracle_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(do), _ptr(dST),
        _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(db), _ptr(dS0), B, T, H, HV, K, V, float(scale))
    if rc != 0:
        raise RuntimeError("kda_oracle_bwd failed with status %d" % rc)
    return dq, dk, dv, dg, db, dS0


def kda_decode_step(x, state, H, HV, K, V, *, conv_w=None, conv_state=None,
                    l2norm_qk=False, eps=1e-6, gate_in=None, A_log=None, dt_bias=None,
                    gate_bounded=True, lower_bound=-5.0, beta=None, beta_is_logit=False,
                    scale=None):
    """One decode token (the kda_decode_token / kda_recurrent_step flow on the
    "metrale_model_weights/kimi_k3_host/kda.rs" page) in fp64.

    ``state`` (float64 [B,HV,K,V]) and ``conv_state`` (float64 [B,C,KW]) are
    updated in place; they must already be float64 contiguous numpy arrays.
    Returns out [B,HV,V].
    """
    x = f64(x)
    B = x.shape[0]
    Cch = 2 * H * K + HV * V
    assert x.shape == (B, Cch)
    assert isinstance(state, np.ndarray) and state.dtype == np.float64
    assert state.flags.c_contiguous and state.shape == (B, HV, K, V)
    gate_in = f64(gate_in).reshape(B, HV * K)
    beta = f64(beta).reshape(B, HV)
    KW = 0
    cw = None
    if conv_w is not None:
        cw = f64(conv_w)
        KW = cw.shape[-1]
        assert cw.shape == (Cch, KW)
        assert isinstance(conv_state, np.ndarray) and conv_state.dtype == np.float64
        assert conv_state.flags.c_contiguous and conv_state.shape == (B, Cch, KW)
    al = f64(A_log)
    dtb = f64(dt_bias)
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    out = np.zeros((B, HV, V), dtype=np.float64)
    rc = _load().kda_oracle_decode_step(
        _ptr(x), _ptr(cw), _ptr(conv_state if cw is not None else None), KW,
        int(bool(l2norm_qk)), float(eps), _ptr(gate_in), _ptr(al), _ptr(dtb),
        int(bool(gate_bounded)), float(lower_bound), _ptr(beta), int(bool(beta_is_logit)),
        _ptr(state), _ptr(out), B, H, HV, K, V, float(scale))
    if rc != 0:
        raise RuntimeError("kda_oracle_decode_step failed with status %d" % rc)
    return out


def prefill_prologue(x, H, HV, K, V, *, conv_w=None, conv_state=None, l2norm_qk=False,
                     eps=1e-6, gate_in=None, A_log=None, dt_bias=None, gate_bounded=True,
                     lower_bound=-5.0, beta=None, beta_is_logit=False):
    """The decode prologue's stages over T tokens of each sequence, in fp64
    (conv_update, l2norm_rows, bounded_gate and the beta sigmoid of the
    "metrale_model_weights/kimi_k3_host/kda.rs" page, token after token).

    x [B,T,2HK+HV*V]; gate_in [B,T,HV,K]; beta [B,T,HV]; ``conv_state``
    (float64 [B,C,KW]) is updated in place.  Returns (q [B,T,H,K], k, v
    [B,T,HV,V], g [B,T,HV,K], beta [B,T,HV]).
    """
    x = f64(x)
    B, T, Cch = x.shape
    assert Cch == 2 * H * K + HV * V
    gate_in = f64(gate_in).reshape(B, T, HV, K)
    beta = f64(beta).reshape(B, T, HV)
    KW = 0
    cw = None
    if conv_w is not None:
        cw = f64(conv_w)
        KW = cw.shape[-1]
        assert cw.shape == (Cch, KW)
        assert isinstance(conv_state, np.ndarray) and conv_state.dtype == np.float64
        assert conv_state.flags.c_contiguous and conv_state.shape == (B, Cch, KW)
    q = np.zeros((B, T, H, K))
    k = np.zeros((B, T, H, K))
    v = np.zeros((B, T, HV, V))
    g = np.zeros((B, T, HV, K))
    bo = np.zeros((B, T, HV))
    rc = _load().kda_oracle_prefill_prologue(
        _ptr(x), _ptr(cw), _ptr(conv_state if cw is not None else None), KW,
        int(bool(l2norm_qk)), float(eps), _ptr(gate_in), _ptr(f64(A_log)), _ptr(f64(dt_bias)),
        int(bool(gate_bounded)), float(lower_bound), _ptr(beta), int(bool(beta_is_logit)),
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(bo), B, T, H, HV, K, V)
    if rc != 0:
        raise RuntimeError("kda_oracle_prefill_prologue failed with status %d" % rc)
    return q, k, v, g, bo


def output_gate(o, gate_in, eps):
    """full_rank_output_gate ("kda.rs"): rows of the last dimension,
    y = sigmoid(gate) * o / sqrt(mean(o^2) + eps)."""
    o = f64(o)
    gi = f64(gate_in)
    assert gi.shape == o.shape
    d = o.shape[-1]
    y = np.zeros_like(o)
    rc = _load().kda_oracle_output_gate(_ptr(o), _ptr(gi), _ptr(y), o.size // d, d, float(eps))
    if rc != 0:
        raise RuntimeError("kda_oracle_output_gate failed")
    return y


def gate(z, A_log, dt_bias, HV, K, bounded=True, lower_bound=-5.0):
    """Gate stage alone ("kda.rs" bounded_gate): z [rows, HV*K] -> g [rows, HV*K]."""
    z = f64(z)
    rows = z.size // (HV * K)
    g = np.zeros_like(z)
    _load().kda_oracle_gate(_ptr(z), _ptr(f64(A_log)), _ptr(f64(dt_bias)), int(bool(bounded)),
                            float(lower_bound), _ptr(g), rows, HV, K)
    return g


def conv_update(state, x, w):
    """Short-conv stage alone ("kda.rs" conv_update); state [rows,C,KW] in place."""
    x = f64(x)
    w = f64(w)
    rows, C = x.shape
    KW = w.shape[-1]
    assert state.dtype == np.float64 and state.shape == (rows, C, KW)
    y = np.zeros_like(x)
    rc = _load().kda_oracle_conv_update(_ptr(state), _ptr(x), _ptr(w), _ptr(y), rows, C, KW)
    if rc != 0:
        raise RuntimeError("kda_oracle_conv_update failed")
    return y


def l2norm_rows(x, d, eps=1e-6):
    """L2 norm stage alone ("kda.rs" l2norm_rows) on rows of length d."""
    x = f64(x).copy()
    _load().kda_oracle_l2norm_rows(_ptr(x), x.size // d, d, float(eps))
    return x


def sigmoid(x: float) -> float:
    return _load().kda_oracle_sigmoid(float(x))


def softplus(x: float) -> float:
    return _load().kda_oracle_softplus(float(x))


def omp_threads() -> int:
    """Threads the oracle's OpenMP loops use."""
    return int(_load().kda_oracle_threads())
