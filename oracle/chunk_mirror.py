"""Chunk-form mirror of the KDA forward -- TEST INFRASTRUCTURE ONLY.

A float64 numpy restatement of the chunk algebra on the
"src/tinycenn_lm/research_layers.py" page (function ``delta_recurrence``),
mapped onto KDA.  That page's recurrence is
    Sbar_t = diag(exp(log_decay_t)) S_{t-1},  S_t = Sbar_t + k_t (z_t - erase_t^T Sbar_t)^T
and KDA is the case write-key = k, erase = beta*k, z = beta*v, with the query
scaled by the readout scale.  The page states the chunk solve is algebraically
identical to the token recurrence; the oracle tests check exactly that against
the token loop in ``kda_oracle.c``.

Two modes:
  * ``literal``  -- the page's own scaling: decay = exp(chunk-local cumsum),
    write = k / decay, read = erase * decay, a unit-lower-triangular solve per
    chunk against z - read @ M, the within-chunk output tril(qr @ write^T) @ R
    (diagonal included) and the carry M <- decay_last * (M + write^T @ R).
    Safe in float64 for the test sizes (exp(+-160) is far from overflow).
  * ``refpoint`` -- the same algebra with every exponential taken of a
    difference of chunk-local cumulative sums around a reference row r:
    (x_i e^{G_i - G_r}) . (y_j e^{G_r - G_j}), the solve applied to the
    M-independent right-hand side [beta*v | beta*k*Gamma] (U = U0 - W M by
    linearity), and the state-write operand k e^{G_last - G_j}, which is <= 1.
Nothing is shared with the HIP library.  Library primitives used as steps:
numpy matmul and scipy's triangular solve.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.linalg import solve_triangular


def _expand(x, G):
    # repeat_interleave over the head axis (axis 2), as the recurrent.py page does
    return np.repeat(x, G, axis=2)


def kda_chunk_fwd(q, k, v, g, beta, scale=None, initial_state=None, chunk=32,
                  mode="literal", ref_row=None):
    """Chunked KDA forward in float64.  Shapes as in the token oracle:
    q,k [B,T,H,K]; v [B,T,HV,V]; g [B,T,HV,K]; beta [B,T,HV]; S0 [B,HV,K,V].
    Returns (o [B,T,HV,V], S_T [B,HV,K,V])."""
    q, k, v, g, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta))
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    G = HV // H
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    qe = _expand(q, G) * scale          # [B,T,HV,K]
    ke = _expand(k, G)
    M = np.zeros((B, HV, K, V)) if initial_state is None else np.array(
        initial_state, dtype=np.float64)
    o = np.zeros((B, T, HV, V))
    for start in range(0, T, chunk):
        stop = min(start + chunk, T)
        n = stop - start
        # [B,HV,n,*] views of this chunk
        qc = qe[:, start:stop].transpose(0, 2, 1, 3)
        kc = ke[:, start:stop].transpose(0, 2, 1, 3)
        vc = v[:, start:stop].transpose(0, 2, 1, 3)
        gc = g[:, start:stop].transpose(0, 2, 1, 3)
        bc = beta[:, start:stop].transpose(0, 2, 1)[..., None]   # [B,HV,n,1]
        Gc = np.cumsum(gc, axis=2)                                # chunk-local cumsum
        if mode == "literal":
            decay = np.exp(Gc)
            write = kc / decay
            read = bc * kc * decay                                # erase * decay
            inter = read @ np.swapaxes(write, -1, -2)
            system = np.tril(inter, -1) + np.eye(n)
            rhs = bc * vc - read @ M
            R = np.empty_like(rhs)
            for b in range(B):
                for h in range(HV):
                    R[b, h] = solve_triangular(system[b, h], rhs[b, h], lower=True,
                                               unit_diagonal=True)
            qr = qc * decay
            within = np.tril(qr @ np.swapaxes(write, -1, -2))
            o[:, start:stop] = (qr @ M + within @ R).transpose(0, 2, 1, 3)
            M = decay[:, :, -1, :, None] * (M + np.swapaxes(write, -1, -2) @ R)
        elif mode == "refpoint":
            r = (n - 1) // 2 if ref_row is None else min(ref_row, n - 1)
            Gr = Gc[:, :, r:r + 1, :]
            up = np.exp(Gc - Gr)           # e^{G_i - G_r}
            dn = np.exp(Gr - Gc)           # e^{G_r - G_j}
            Akk = np.tril((bc * kc * up) @ np.swapaxes(kc * dn, -1, -2), -1)
            Aqk = np.tril((qc * up) @ np.swapaxes(kc * dn, -1, -2))
            Gam = np.exp(Gc)
            kbar = kc * np.exp(Gc[:, :, -1:, :] - Gc)
            Tinv = np.empty_like(Akk)
            eye = np.eye(n)
            for b in range(B):
                for h in range(HV):
                    Tinv[b, h] = solve_triangular(eye + Akk[b, h], eye, lower=True,
                                                  unit_diagonal=True)
            W = Tinv @ (bc * kc * Gam)
            U0 = Tinv @ (bc * vc)
            U = U0 - W @ M
            o[:, start:stop] = ((qc * Gam) @ M + Aqk @ U).transpose(0, 2, 1, 3)
            M = Gam[:, :, -1, :, None] * M + np.swapaxes(kbar, -1, -2) @ U
        else:
            raise ValueError("mode must be 'literal' or 'refpoint'")
    return o, M
