"""Pins for the CPU oracle: checks against what the pages and the mathematics
fix, never against the oracle's own formula retyped.

Each test names the mistake class it would catch (dropped term, wrong sign,
wrong index, transposed operand, wrong order of the steps).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import chunk_mirror

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


def rand_inputs(B, T, H, HV, K, V, g_scale=5.0, s0=True, rng=RNG, unit_qk=True):
    q = rng.standard_normal((B, T, H, K))
    k = rng.standard_normal((B, T, H, K))
    if unit_qk:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, HV, V))
    g = -g_scale / (1.0 + np.exp(-rng.standard_normal((B, T, HV, K))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, HV))))
    S0 = rng.standard_normal((B, HV, K, V)) * 0.3 if s0 else None
    return q, k, v, g, beta, S0


def rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# ---------------------------------------------------------------- worked examples

def test_hand_expansion_two_tokens():
    """Hand expansion of the four steps (decay, residual, write, readout) for
    T=2 (tests/golden/hand_expansion_T2.json).  Catches a wrong step order, a
    dropped decay, a wrong residual sign, readout-before-write."""
    d = json.load(open(os.path.join(GOLDEN, "hand_expansion_T2.json")))
    S0 = np.array(d["S0"])[None, None]
    g = np.log(np.array(d["decay_exp_g"]))[None, :, None, :]
    k = np.array(d["k"])[None, :, None, :]
    v = np.array(d["v"])[None, :, None, :]
    q = np.array(d["q"])[None, :, None, :]
    beta = np.array(d["beta"])[None, :, None]
    o, S = oracle.kda_fwd(q, k, v, g, beta, scale=1.0, initial_state=S0)
    np.testing.assert_allclose(o[0, :, 0], np.array(d["o"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(S[0, 0], np.array(d["S_T"]), rtol=0, atol=1e-14)


def _fraction_reference(q, k, v, d, beta, S0, scale):
    """Exact rational evaluation of the recurrence in its projection form
    S_t = (I - beta_t k_t k_t^T) D_t S_{t-1} + beta_t k_t v_t^T, o_t = scale q_t^T S_t
    (D_t = diag(exp g_t)); algebraically the same map as the page's four steps."""
    T = len(q)
    K, V = len(S0), len(S0[0])
    S = [row[:] for row in S0]
    outs = []
    for t in range(T):
        DS = [[d[t][i] * S[i][j] for j in range(V)] for i in range(K)]
        P = [[(1 if i == m else 0) - beta[t] * k[t][i] * k[t][m] for m in range(K)]
             for i in range(K)]
        S = [[sum(P[i][m] * DS[m][j] for m in range(K)) + beta[t] * k[t][i] * v[t][j]
              for j in range(V)] for i in range(K)]
        outs.append([scale * sum(q[t][i] * S[i][j] for i in range(K)) for j in range(V)])
    return outs, S


@pytest.mark.parametrize("T,K,V", [(1, 1, 1), (3, 2, 3), (5, 3, 2), (8, 4, 4)])
def test_brute_force_rational(T, K, V):
    """Brute force with exact rationals on tiny inputs; decays are exact
    fractions passed as g = log(d).  Catches any arithmetic slip, transposed
    state (K != V), scale on the wrong operand."""
    rng = np.random.default_rng(T * 100 + K * 10 + V)
    fr = lambda lo, hi: Fraction(int(rng.integers(lo, hi)), 8)
    q = [[fr(-8, 9) for _ in range(K)] for _ in range(T)]
    k = [[fr(-8, 9) for _ in range(K)] for _ in range(T)]
    v = [[fr(-16, 17) for _ in range(V)] for _ in range(T)]
    d = [[Fraction(int(rng.integers(1, 9)), 8) for _ in range(K)] for _ in range(T)]
    beta = [Fraction(int(rng.integers(0, 9)), 8) for _ in range(T)]
    S0 = [[fr(-8, 9) for _ in range(V)] for _ in range(K)]
    scale = Fraction(1, 2)
    exp_o, exp_S = _fraction_reference(q, k, v, d, beta, S0, scale)
    A = lambda x: np.array([[float(e) for e in row] for row in x])
    o, S = oracle.kda_fwd(A(q)[None, :, None], A(k)[None, :, None], A(v)[None, :, None],
                          np.log(A(d))[None, :, None], np.array([float(b) for b in beta])[None, :, None],
                          scale=0.5, initial_state=A(S0)[None, None])
    np.testing.assert_allclose(o[0, :, 0], A(exp_o), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S[0, 0], A(exp_S), rtol=1e-12, atol=1e-12)


def test_scalar_closed_form():
    """K=V=1: S_t = e^{g_t}(1 - beta_t k_t^2) S_{t-1} + beta_t k_t v_t, o_t = s q_t S_t."""
    rng = np.random.default_rng(7)
    T = 50
    q, k, v = (rng.standard_normal(T) for _ in range(3))
    g = -rng.random(T)
    beta = rng.random(T)
    s = 0.7
    S = 0.25
    exp_o = []
    for t in range(T):
        S = math.exp(g[t]) * (1 - beta[t] * k[t] ** 2) * S + beta[t] * k[t] * v[t]
        exp_o.append(s * q[t] * S)
    o, ST = oracle.kda_fwd(q[None, :, None, None], k[None, :, None, None], v[None, :, None, None],
                           g[None, :, None, None], beta[None, :, None], scale=s,
                           initial_state=np.full((1, 1, 1, 1), 0.25))
    np.testing.assert_allclose(o[0, :, 0, 0], exp_o, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(ST[0, 0, 0, 0], S, rtol=1e-13)


# ---------------------------------------------------------------- closed forms

def test_beta_zero_is_pure_decay():
    """beta = 0: nothing is written, so S_T = exp(sum_t g_t) (.) S0 and
    o_t = s q_t^T (exp(G_t) (.) S0), G_t the running sum of g (decay per K row)."""
    B, T, H, HV, K, V = 2, 20, 2, 4, 8, 5
    q, k, v, g, beta, S0 = rand_inputs(B, T, H, HV, K, V, g_scale=0.5)
    beta[:] = 0.0
    o, S = oracle.kda_fwd(q, k, v, g, beta, initial_state=S0)
    G = np.cumsum(g, axis=1)                          # [B,T,HV,K]
    np.testing.assert_allclose(S, np.exp(G[:, -1])[..., None] * S0, rtol=1e-13, atol=1e-15)
    s = 1 / math.sqrt(K)
    qe = np.repeat(q, HV // H, axis=2)
    exp_o = s * np.einsum("bthk,bthk,bhkv->bthv", qe, np.exp(G), S0)
    np.testing.assert_allclose(o, exp_o, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("K", [4, 32, 128])
def test_unit_key_recall(K):
    """g = 0, beta = 1, |k| = 1, q = sqrt(K) k: the write erases the old
    prediction along k and stores v, so o_t = v_t exactly for any S0 and any
    history (the delta-rule intuition on the sec-01.tex page)."""
    B, T, H, HV, V = 1, 40, 1, 2, 6
    q, k, v, g, beta, S0 = rand_inputs(B, T, H, HV, K, V)
    g[:] = 0.0
    beta[:] = 1.0
    q = math.sqrt(K) * k
    o, _ = oracle.kda_fwd(q, k, v, g, beta, initial_state=S0)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- invariants

def test_linearity_in_state_and_values():
    """The map (S0, v) -> (o, S_T) is linear for fixed q,k,g,beta
    (S_t = (I - beta k k^T) D S + beta k v^T).  Catches any stray nonlinearity."""
    B, T, H, HV, K, V = 1, 17, 1, 1, 6, 7
    q, k, v, g, beta, S0 = rand_inputs(B, T, H, HV, K, V)
    _, _, v2, _, _, S02 = rand_inputs(B, T, H, HV, K, V)
    o1, S1 = oracle.kda_fwd(q, k, v, g, beta, initial_state=S0)
    o2, S2 = oracle.kda_fwd(q, k, v2, g, beta, initial_state=S02)
    o3, S3 = oracle.kda_fwd(q, k, 2 * v - 3 * v2, g, beta, initial_state=2 * S0 - 3 * S02)
    np.testing.assert_allclose(o3, 2 * o1 - 3 * o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S3, 2 * S1 - 3 * S2, rtol=1e-12, atol=1e-12)


def test_gqa_equals_explicit_repeat():
    """H < HV equals H = HV with q, k repeat_interleave'd (value head hv reads
    q/k head hv // (HV/H), never hv % H)."""
    B, T, H, HV, K, V = 2, 12, 2, 6, 8, 8
    q, k, v, g, beta, S0 = rand_inputs(B, T, H, HV, K, V)
    o1, S1 = oracle.kda_fwd(q, k, v, g, beta, initial_state=S0)
    qe, ke = np.repeat(q, 3, axis=2), np.repeat(k, 3, axis=2)
    o2, S2 = oracle.kda_fwd(qe, ke, v, g, beta, initial_state=S0)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(S1, S2)
    # and a tiled (hv % H) mapping is really different
    o3, _ = oracle.kda_fwd(np.tile(q, (1, 1, 3, 1)), np.tile(k, (1, 1, 3, 1)), v, g, beta,
                           initial_state=S0)
    assert np.max(np.abs(o3 - o1)) > 1e-3


def test_value_columns_independent():
    """Columns [a,b) of a full run equal a run on v[..., a:b], S0[..., a:b]:
    state columns only couple through K.  This is what lets the GPU split V."""
    B, T, H, HV, K, V = 1, 30, 1, 2, 8, 12
    q, k, v, g, beta, S0 = rand_inputs(B, T, H, HV, K, V)
    o, S = oracle.kda_fwd(q, k, v, g, beta, initial_state=S0)
    o2, S2 = oracle.kda_fwd(q, k, v[..., 4:9], g, beta, initial_state=S0[..., 4:9])
    np.testing.assert_allclose(o2, o[..., 4:9], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(S2, S[..., 4:9], rtol=1e-13, atol=1e-15)


def test_split_resume():
    """fwd(T1) then fwd(T2, S0 = S_T1) equals fwd(T1+T2)."""
    B, T, H, HV, K, V = 2, 33, 1, 2, 8, 4
    q, k, v, g, beta, S0 = rand_inputs(B, T, H, HV, K, V)
    o, S = oracle.kda_fwd(q, k, v, g, beta, initial_state=S0)
    a = 13
    oa, Sa = oracle.kda_fwd(q[:, :a], k[:, :a], v[:, :a], g[:, :a], beta[:, :a], initial_state=S0)
    ob, Sb = oracle.kda_fwd(q[:, a:], k[:, a:], v[:, a:], g[:, a:], beta[:, a:], initial_state=Sa)
    np.testing.assert_allclose(np.concatenate([oa, ob], axis=1), o, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(Sb, S, rtol=1e-13, atol=1e-15)


def _fraction_states(q, k, v, d, beta, S0):
    """All states S_1..S_T of the projection form of the recurrence, exactly."""
    T = len(q)
    K, V = len(S0), len(S0[0])
    S = [row[:] for row in S0]
    states = []
    for t in range(T):
        DS = [[d[t][i] * S[i][j] for j in range(V)] for i in range(K)]
        S = [[DS[i][j] - beta[t] * k[t][i] * sum(k[t][m] * DS[m][j] for m in range(K))
              + beta[t] * k[t][i] * v[t][j] for j in range(V)] for i in range(K)]
        states.append(S)
    return states


@pytest.mark.parametrize("T,every", [(8, 2), (7, 3), (6, 6), (5, 8)])
def test_snapshots_brute_force_rational(T, every):
    """Prefix snapshots (the state clones that kda.rs prefix_hit_wrong_slot_diverges
    resumes from) against exact rationals: snapshot j is S after token
    (j+1)*every, T // every of them.  Catches an off-by-one token, a snapshot
    taken before the write, a wrong count."""
    K, V = 3, 2
    rng = np.random.default_rng(T * 10 + every)
    fr = lambda lo, hi: Fraction(int(rng.integers(lo, hi)), 8)
    q = [[fr(-8, 9) for _ in range(K)] for _ in range(T)]
    k = [[fr(-8, 9) for _ in range(K)] for _ in range(T)]
    v = [[fr(-16, 17) for _ in range(V)] for _ in range(T)]
    d = [[Fraction(int(rng.integers(1, 9)), 8) for _ in range(K)] for _ in range(T)]
    beta = [Fraction(int(rng.integers(0, 9)), 8) for _ in range(T)]
    S0 = [[fr(-8, 9) for _ in range(V)] for _ in range(K)]
    states = _fraction_states(q, k, v, d, beta, S0)
    A = lambda x: np.array([[float(e) for e in row] for row in x])
    _, _, snaps = oracle.kda_fwd(
        A(q)[None, :, None], A(k)[None, :, None], A(v)[None, :, None],
        np.log(A(d))[None, :, None], np.array([float(b) for b in beta])[None, :, None],
        scale=0.5, initial_state=A(S0)[None, None], snapshot_every=every)
    assert snaps.shape == (1, T // every, 1, K, V)
    for j in range(T // every):
        np.testing.assert_allclose(snaps[0, j, 0], A(states[(j + 1) * every - 1]),
                                   rtol=1e-12, atol=1e-12)


def test_snapshots_beta_zero_closed_form():
    """beta = 0: snapshot j = exp(G_{(j+1)e}) (.) S0 for every (b, hv), laid out
    [B, T // e, HV, K, V].  Catches a transposed (b, j, hv) layout."""
    B, T, H, HV, K, V, e = 2, 20, 1, 3, 4, 5, 6
    q, k, v, g, beta, S0 = rand_inputs(B, T, H, HV, K, V, g_scale=0.5)
    beta[:] = 0.0
    _, S, snaps = oracle.kda_fwd(q, k, v, g, beta, initial_state=S0, snapshot_every=e)
    G = np.cumsum(g, axis=1)
    assert snaps.shape == (B, 3, HV, K, V)
    for j in range(3):
        np.testing.assert_allclose(snaps[:, j], np.exp(G[:, (j + 1) * e - 1])[..., None] * S0,
                                   rtol=1e-13, atol=1e-15)


def test_snapshot_resume_equals_full_run():
    """Resuming from snapshot j over the rest of the tokens gives the full run's
    later outputs and final state; resuming from snapshot j-1 does not."""
    B, T, H, HV, K, V, e = 2, 40, 1, 2, 8, 4, 8
    q, k, v, g, beta, S0 = rand_inputs(B, T, H, HV, K, V)
    o, S, snaps = oracle.kda_fwd(q, k, v, g, beta, initial_state=S0, snapshot_every=e)
    j = 2
    a = (j + 1) * e
    ob, Sb = oracle.kda_fwd(q[:, a:], k[:, a:], v[:, a:], g[:, a:], beta[:, a:],
                            initial_state=snaps[:, j])
    np.testing.assert_allclose(ob, o[:, a:], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(Sb, S, rtol=1e-12, atol=1e-14)
    ow, _ = oracle.kda_fwd(q[:, a:], k[:, a:], v[:, a:], g[:, a:], beta[:, a:],
                           initial_state=snaps[:, j - 1])
    assert np.max(np.abs(ow - o[:, a:])) > 1e-4


def test_default_scale_and_zero_state():
    """scale=None means 1/sqrt(K); initial_state=None means zeros."""
    B, T, H, HV, K, V = 1, 5, 1, 1, 16, 4
    q, k, v, g, beta, _ = rand_inputs(B, T, H, HV, K, V)
    o1, S1 = oracle.kda_fwd(q, k, v, g, beta)
    o2, S2 = oracle.kda_fwd(q, k, v, g, beta, scale=0.25, initial_state=np.zeros((B, HV, K, V)))
    np.testing.assert_allclose(o1, o2, rtol=1e-14, atol=0)
    np.testing.assert_array_equal(S1, S2)


# ---------------------------------------------------------------- chunk algebra

def test_chunk_one_is_token_loop():
    """Chunk size 1 of the research_layers.py chunk form equals the token loop."""
    q, k, v, g, beta, S0 = rand_inputs(2, 9, 1, 2, 4, 3)
    o, S = oracle.kda_fwd(q, k, v, g, beta, initial_state=S0)
    oc, Sc = chunk_mirror.kda_chunk_fwd(q, k, v, g, beta, initial_state=S0, chunk=1)
    assert rel(oc, o) < 1e-13 and rel(Sc, S) < 1e-13


@pytest.mark.parametrize("mode", ["literal", "refpoint"])
@pytest.mark.parametrize("chunk", [2, 4, 16, 32, 64])
def test_chunk_form_equals_token_loop(mode, chunk):
    """The chunk form (cumulative decay, unit-lower-triangular solve, carry)
    reaches the token loop's result, including a ragged last chunk and GQA."""
    q, k, v, g, beta, S0 = rand_inputs(2, 2 * chunk + 3, 2, 4, 8, 6)
    o, S = oracle.kda_fwd(q, k, v, g, beta, initial_state=S0)
    oc, Sc = chunk_mirror.kda_chunk_fwd(q, k, v, g, beta, initial_state=S0, chunk=chunk, mode=mode)
    assert rel(oc, o) < 1e-11, rel(oc, o)
    assert rel(Sc, S) < 1e-11, rel(Sc, S)


# ---------------------------------------------------------------- decode prologue

def test_decode_equals_prefill():
    """T decode steps (no prologue, g and beta given) equal the forward over T."""
    B, T, H, HV, K, V = 2, 10, 2, 4, 8, 6
    q, k, v, g, beta, S0 = rand_inputs(B, T, H, HV, K, V)
    o, S = oracle.kda_fwd(q, k, v, g, beta, initial_state=S0)
    state = S0.copy()
    outs = []
    for t in range(T):
        x = np.concatenate([q[:, t].reshape(B, -1), k[:, t].reshape(B, -1),
                            v[:, t].reshape(B, -1)], axis=1)
        outs.append(oracle.kda_decode_step(x, state, H, HV, K, V, gate_in=g[:, t],
                                           beta=beta[:, t]))
    np.testing.assert_allclose(np.stack(outs, 1), o, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(state, S, rtol=1e-13, atol=1e-15)


def _silu(a):
    return a / (1.0 + math.exp(-a))


def _softplus(x):
    return math.log(1.0 + math.exp(x))


def test_conv_state_advances():
    """kda.rs conv_kernel_4_state_advances: with w=1 and x_t = t+1 the newest
    value sits in the last slot and the state reads [1,2,3,4] after 4 steps;
    the outputs are SiLU of the running register sums 1, 3, 6, 10."""
    d = json.load(open(os.path.join(GOLDEN, "kda_rs_unit_examples.json")))["conv"]
    ch = 3 * d["heads"] * d["head_dim"]
    KW = d["kernel"]
    state = np.zeros((1, ch, KW))
    w = np.full((ch, KW), d["weight"])
    sums = np.cumsum(d["x_per_step"])
    for t, xv in enumerate(d["x_per_step"]):
        y = oracle.conv_update(state, np.full((1, ch), xv), w)
        assert np.all(state[0, :, KW - 1] == xv)
        np.testing.assert_allclose(y[0], _silu(sums[t]), rtol=1e-15)
    assert np.all(state[0] == np.array(d["page_final_state_row"]))


def test_conv_weight_orientation():
    """Weight slot j multiplies register slot j (oldest first): a one-hot
    weight on slot 0 returns the input from KW-1 steps ago."""
    KW, ch = 4, 3
    state = np.zeros((1, ch, KW))
    w = np.zeros((ch, KW))
    w[:, 0] = 1.0
    ys = [oracle.conv_update(state, np.full((1, ch), float(t + 1)), w)[0, 0] for t in range(6)]
    np.testing.assert_allclose(ys, [0, 0, 0, _silu(1), _silu(2), _silu(3)], rtol=1e-15)


def test_gate_closed_forms():
    """kda.rs omitted_lower_bound_is_neg_exp_a_softplus: with A_log=0 the
    unbounded gate is -softplus(z+dt_bias); the -5 lower-bounded gate is
    -5*sigmoid(z+dt_bias) and differs from it by more than 0.1."""
    d = json.load(open(os.path.join(GOLDEN, "kda_rs_unit_examples.json")))["gate"]
    z = np.array(d["z"])[None]
    g_unb = oracle.gate(z, d["A_log"], d["dt_bias"], HV=1, K=2, bounded=False)
    g_bnd = oracle.gate(z, d["A_log"], d["dt_bias"], HV=1, K=2, bounded=True,
                        lower_bound=d["bounded_lb"])
    xs = [zz + dd for zz, dd in zip(d["z"], d["dt_bias"])]
    for i, x in enumerate(xs):
        assert abs(g_unb[0, i] - (-_softplus(x))) < d["page_tolerance_vs_neg_softplus"]
        np.testing.assert_allclose(g_unb[0, i], -_softplus(x), rtol=1e-14)
        np.testing.assert_allclose(g_bnd[0, i], d["bounded_lb"] / (1 + math.exp(-x)), rtol=1e-14)
    assert abs(g_bnd[0, 0] - g_unb[0, 0]) > d["page_min_gap_bounded_vs_unbounded"]
    # A_log scales the pre-activation by exp(A_log) per head
    g2 = oracle.gate(z, [math.log(3.0)], d["dt_bias"], HV=1, K=2, bounded=True)
    np.testing.assert_allclose(g2[0, 0], -5.0 / (1 + math.exp(-3.0 * xs[0])), rtol=1e-14)


def _gate_cases():
    """Closed forms of "kda.rs" bounded_gate at A_log = ln 3 (decay factor 3),
    chosen so that the value is exact: softplus(ln 3) = ln 4, so the unbounded
    gate is -3 ln 4 = -6 ln 2; at x = ln(3)/3 the lower-bounded gate is
    -5 sigmoid(ln 3) = -5 * 3/4.  Misplacing the factor (-softplus(3x) gives
    -ln 28; -5 sigmoid(x) gives -3.0) fails them."""
    ln3 = math.log(3.0)
    return [
        # (bounded, z + dt_bias, expected g)
        (False, ln3, -6.0 * math.log(2.0)),
        (False, 0.0, -3.0 * math.log(2.0)),
        (True, ln3 / 3.0, -3.75),
        (True, 0.0, -2.5),
    ]


def test_gate_exp_alog_factor():
    """The gate entry point: exp(A_log) multiplies softplus(x) on the
    unbounded branch and x inside the sigmoid on the bounded one."""
    for bounded, x, want in _gate_cases():
        z = np.array([[x - 0.25, x + 0.5]])           # z + dt_bias = x on both channels
        g = oracle.gate(z, [math.log(3.0)], [0.25, -0.5], HV=1, K=2, bounded=bounded)
        np.testing.assert_allclose(g[0], [want, want], rtol=1e-14)


def test_gate_exp_alog_factor_in_decode_step():
    """The same gate inside the decode step: one head, K = V = 1, no conv or
    L2 norm, beta = 0 and state 1.  The step only decays, so the new state and
    the readout (q = 1, scale 1) are both exp(g): 1/64 on the unbounded case
    with x = ln 3."""
    for bounded, x, want in _gate_cases():
        state = np.ones((1, 1, 1, 1))
        xq = np.array([[1.0, 0.5, 2.0]])               # q | k | v
        o = oracle.kda_decode_step(xq, state, 1, 1, 1, 1, gate_in=np.array([[x - 0.1]]),
                                   A_log=[math.log(3.0)], dt_bias=[0.1], gate_bounded=bounded,
                                   beta=np.array([[0.0]]), beta_is_logit=False, scale=1.0)
        np.testing.assert_allclose(o[0, 0, 0], math.exp(want), rtol=1e-13)
        np.testing.assert_allclose(state[0, 0, 0, 0], math.exp(want), rtol=1e-13)
    # the unbounded case at x = ln 3 is exactly 2^-6
    state = np.ones((1, 1, 1, 1))
    o = oracle.kda_decode_step(np.array([[1.0, 0.5, 2.0]]), state, 1, 1, 1, 1,
                               gate_in=np.array([[math.log(3.0)]]), A_log=[math.log(3.0)],
                               dt_bias=[0.0], gate_bounded=False, beta=np.array([[0.0]]),
                               beta_is_logit=False, scale=1.0)
    assert abs(o[0, 0, 0] - 1.0 / 64.0) < 1e-15


def test_gate_exp_alog_factor_in_prefill_prologue():
    """The same gate inside the prefill prologue, on every token and head:
    two value heads with A_log = ln 3 and 0 (decay factors 3 and 1)."""
    for bounded, x, want in _gate_cases():
        H = HV = 2
        K = V = 1
        T = 3
        xin = np.zeros((1, T, 2 * H * K + HV * V))
        dt = np.array([0.2, -0.3])
        z = np.empty((1, T, HV, K))
        z[..., 0, 0] = x - dt[0]
        z[..., 1, 0] = 0.0 - dt[1]                       # head 1: x = 0, factor 1
        _, _, _, g, _ = oracle.prefill_prologue(xin, H, HV, K, V, gate_in=z,
                                                A_log=[math.log(3.0), 0.0], dt_bias=dt,
                                                gate_bounded=bounded, beta=np.zeros((1, T, HV)))
        np.testing.assert_allclose(g[0, :, 0, 0], [want] * T, rtol=1e-14)
        # factor 1 at x = 0: -ln 2 unbounded, -5/2 bounded
        np.testing.assert_allclose(g[0, :, 1, 0], [-2.5 if bounded else -math.log(2.0)] * T,
                                   rtol=1e-14)


def test_l2norm_eps_inside_root():
    """kda.rs l2norm_rows: x / sqrt(sum x^2 + eps)."""
    x = np.array([[3.0, 4.0], [0.0, 0.0]])
    y = oracle.l2norm_rows(x, 2, eps=1e-6)
    np.testing.assert_allclose(y[0], [3 / math.sqrt(25 + 1e-6), 4 / math.sqrt(25 + 1e-6)], rtol=1e-15)
    assert np.all(y[1] == 0.0)


def test_beta_logit_zero_still_writes():
    """kda.rs beta_zero_is_sigmoid_half_not_zero: a beta logit of 0 means
    beta = 0.5.  From a zero state the step stores beta*k(x)v, so
    o = scale*(q.k)*beta*v; here q = k = [1,0]/sqrt(1+eps), v = [1, 0.5]."""
    d = json.load(open(os.path.join(GOLDEN, "kda_rs_unit_examples.json")))["beta_logit_step"]
    H = HV = d["heads"]
    K = V = d["head_dim"]
    x = np.array(d["qkv"])[None]
    outs = []
    for logit in d["logits"]:
        state = np.zeros((1, HV, K, V))
        o = oracle.kda_decode_step(x, state, H, HV, K, V, l2norm_qk=True, eps=d["eps"],
                                   gate_in=np.array(d["gate"])[None], beta=np.array([[logit]]),
                                   beta_is_logit=True)
        qk = 1.0 / (1.0 + d["eps"])
        beta = 1.0 / (1.0 + math.exp(-logit))
        np.testing.assert_allclose(o[0, 0], qk * beta * np.array([1.0, 0.5]) / math.sqrt(2), rtol=1e-14)
        outs.append(o)
    assert np.max(np.abs(outs[0])) > 1e-6
    assert not np.array_equal(outs[0], outs[1])


def test_snapshot_restore_bitwise():
    """kda.rs prefix_hit_wrong_slot_diverges: decoding from a copy of the state
    taken after step 2 equals sequential decoding bit for bit (conv state too);
    restoring the step-1 snapshot instead diverges by more than 1e-4."""
    d = json.load(open(os.path.join(GOLDEN, "kda_rs_unit_examples.json")))["prefix"]
    H = HV = d["heads"]
    K = V = d["head_dim"]
    KW = d["kernel"]
    ch = 2 * H * K + HV * V
    w = np.full((ch, KW), d["conv_weight"])
    z = np.array(d["gate_z"])[None]
    kw = dict(conv_w=w, l2norm_qk=True, gate_in=z, A_log=np.array(d["gate_A_log"]),
              dt_bias=np.array(d["gate_dt_bias"]), gate_bounded=True, lower_bound=d["gate_lb"],
              beta=np.array([[d["beta_logit"]]]), beta_is_logit=True)
    st, cs = np.zeros((1, HV, K, V)), np.zeros((1, ch, KW))
    snaps = []
    for xv in d["x_steps"]:
        oracle.kda_decode_step(np.full((1, ch), xv), st, H, HV, K, V, conv_state=cs, **kw)
        snaps.append((st.copy(), cs.copy()))
    x3 = np.full((1, ch), d["x_final"])
    y_seq = oracle.kda_decode_step(x3, st, H, HV, K, V, conv_state=cs, **kw)
    s1, c1 = snaps[1][0].copy(), snaps[1][1].copy()
    y_hit = oracle.kda_decode_step(x3, s1, H, HV, K, V, conv_state=c1, **kw)
    np.testing.assert_array_equal(y_hit, y_seq)
    np.testing.assert_array_equal(c1, cs)
    s0, c0 = snaps[0][0].copy(), snaps[0][1].copy()
    y_wrong = oracle.kda_decode_step(x3, s0, H, HV, K, V, conv_state=c0, **kw)
    assert np.max(np.abs(y_hit - y_wrong)) > d["page_min_wrong_slot_gap"]


def test_decode_prologue_composition():
    """The fused decode equals its stages run one after another (conv+SiLU,
    per-head L2 norm of q and k, bounded gate, sigmoid(beta)), then the plain
    step; with GQA (H < HV)."""
    rng = np.random.default_rng(3)
    B, H, HV, K, V, KW = 3, 2, 4, 8, 4, 4
    ch = 2 * H * K + HV * V
    w = rng.standard_normal((ch, KW))
    A_log, dtb = rng.standard_normal(HV), rng.standard_normal(HV * K)
    st_a = rng.standard_normal((B, HV, K, V))
    cs_a = rng.standard_normal((B, ch, KW))
    st_b, cs_b = st_a.copy(), cs_a.copy()
    for _ in range(3):
        x, z, bl = rng.standard_normal((B, ch)), rng.standard_normal((B, HV * K)), rng.standard_normal((B, HV))
        o_a = oracle.kda_decode_step(x, st_a, H, HV, K, V, conv_w=w, conv_state=cs_a, l2norm_qk=True,
                                     gate_in=z, A_log=A_log, dt_bias=dtb, beta=bl, beta_is_logit=True)
        y = oracle.conv_update(cs_b, x, w)
        y[:, :2 * H * K] = oracle.l2norm_rows(y[:, :2 * H * K], K)
        g = oracle.gate(z, A_log, dtb, HV, K)
        beta = 1.0 / (1.0 + np.exp(-bl))
        o_b = oracle.kda_decode_step(y, st_b, H, HV, K, V, gate_in=g, beta=beta)
        np.testing.assert_allclose(o_a, o_b, rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(st_a, st_b, rtol=1e-13, atol=1e-15)
        np.testing.assert_array_equal(cs_a, cs_b)


# ---------------------------------------------------------------- prefill prologue, output gate

def test_prefill_prologue_conv_page_example():
    """kda.rs conv_kernel_4_state_advances over T = 4 tokens of one prefill:
    w = 1, x_t = t + 1 on every channel; the outputs are SiLU of the running
    sums 1, 3, 6, 10 and the register ends as [1, 2, 3, 4].  Catches a window
    that does not carry from token to token, or runs the wrong way in time."""
    d = json.load(open(os.path.join(GOLDEN, "kda_rs_unit_examples.json")))["conv"]
    H = HV = d["heads"]
    K = V = d["head_dim"]
    KW = d["kernel"]
    ch = 2 * H * K + HV * V
    T = len(d["x_per_step"])
    x = np.repeat(np.array(d["x_per_step"])[None, :, None], ch, axis=2)
    cs = np.zeros((1, ch, KW))
    q, k, v, _, _ = oracle.prefill_prologue(
        x, H, HV, K, V, conv_w=np.full((ch, KW), d["weight"]), conv_state=cs,
        gate_in=np.zeros((1, T, HV, K)), beta=np.zeros((1, T, HV)))
    sums = np.cumsum(d["x_per_step"])
    for t in range(T):
        for arr in (q, k, v):
            np.testing.assert_allclose(arr[0, t].ravel(), _silu(sums[t]), rtol=1e-15)
    assert np.all(cs[0] == np.array(d["page_final_state_row"]))


@pytest.mark.parametrize("bounded", [True, False])
def test_prefill_prologue_then_fwd_equals_decode_loop(bounded):
    """T decode steps with the full prologue (conv + SiLU, L2 norm, gate, beta
    logits) from zero state equal the prologue over the T tokens followed by
    the token loop: same outputs, same recurrent state, same conv register.
    The decode step is pinned separately against the kda.rs examples."""
    rng = np.random.default_rng(7)
    B, T, H, HV, K, V, KW = 2, 9, 1, 2, 4, 3, 4
    ch = 2 * H * K + HV * V
    x = rng.standard_normal((B, T, ch))
    w = rng.standard_normal((ch, KW))
    z = rng.standard_normal((B, T, HV, K))
    A_log = rng.standard_normal(HV) * 0.5
    dt = rng.standard_normal(HV * K) * 0.5
    bl = rng.standard_normal((B, T, HV))
    cs0 = rng.standard_normal((B, ch, KW)) * 0.5
    kw = dict(l2norm_qk=True, eps=1e-6, A_log=A_log, dt_bias=dt, gate_bounded=bounded,
              lower_bound=-5.0, beta_is_logit=True)
    st = np.zeros((B, HV, K, V))
    cs = cs0.copy()
    outs = []
    for t in range(T):
        outs.append(oracle.kda_decode_step(x[:, t], st, H, HV, K, V, conv_w=w, conv_state=cs,
                                           gate_in=z[:, t], beta=bl[:, t], **kw))
    cs2 = cs0.copy()
    q, k, v, g, beta = oracle.prefill_prologue(x, H, HV, K, V, conv_w=w, conv_state=cs2,
                                               gate_in=z, beta=bl, **kw)
    o, S = oracle.kda_fwd(q, k, v, g, beta)
    np.testing.assert_allclose(o, np.stack(outs, 1), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S, st, rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(cs2, cs)


def test_output_gate_closed_forms():
    """kda.rs full_rank_output_gate: y = sigmoid(g) o / sqrt(mean(o^2) + eps).
    o = [3, -4], g = 0, eps = 0: mean square 12.5, so y = [3, -4] / (2 sqrt 12.5);
    g = log 3 gives sigmoid = 3/4 exactly; an all-zero row stays zero (eps > 0);
    with eps = 0, y is invariant to scaling o by c > 0 and flips sign for c < 0.
    Catches sum in place of mean, a missing root, tanh in place of sigmoid."""
    o = np.array([[3.0, -4.0]])
    y = oracle.output_gate(o, np.zeros_like(o), 0.0)
    np.testing.assert_allclose(y, o / (2 * math.sqrt(12.5)), rtol=1e-15)
    y = oracle.output_gate(o, np.full_like(o, math.log(3.0)), 0.0)
    np.testing.assert_allclose(y, 0.75 * o / math.sqrt(12.5), rtol=1e-14)
    z = oracle.output_gate(np.zeros((2, 8)), np.ones((2, 8)), 1e-6)
    assert np.all(z == 0.0)
    rng = np.random.default_rng(3)
    o = rng.standard_normal((5, 16))
    gt = rng.standard_normal((5, 16))
    y = oracle.output_gate(o, gt, 0.0)
    np.testing.assert_allclose(oracle.output_gate(7.5 * o, gt, 0.0), y, rtol=1e-13)
    np.testing.assert_allclose(oracle.output_gate(-0.25 * o, gt, 0.0), -y, rtol=1e-13)
    # with the gate saturated, every row has mean square ms / (ms + eps)
    eps = 0.3
    y = oracle.output_gate(o, np.full_like(o, 60.0), eps)
    ms = np.mean(o * o, axis=1)
    np.testing.assert_allclose(np.mean(y * y, axis=1), ms / (ms + eps), rtol=1e-13)


# ---------------------------------------------------------------- backward

def _loss(inp, Wo, WS, scale=None):
    """L = sum(o * Wo) + sum(S_T * WS), by the forward oracle."""
    o, S = oracle.kda_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                          scale=scale, initial_state=inp["S0"])
    return float((o * Wo).sum() + (S * WS).sum())


@pytest.mark.parametrize("with_dST", [True, False])
def test_backward_matches_finite_differences(with_dST):
    """Every gradient of kda_bwd against central differences of the forward
    oracle, entry by entry (GQA, nonzero S0, unnormalised q and k)."""
    B, T, H, HV, K, V = 2, 5, 1, 2, 3, 2
    rng = np.random.default_rng(7)
    inp = dict(q=rng.standard_normal((B, T, H, K)), k=rng.standard_normal((B, T, H, K)),
               v=rng.standard_normal((B, T, HV, V)), g=-2.0 * rng.random((B, T, HV, K)),
               beta=rng.random((B, T, HV)), S0=rng.standard_normal((B, HV, K, V)))
    Wo = rng.standard_normal((B, T, HV, V))
    WS = rng.standard_normal((B, HV, K, V)) if with_dST else np.zeros((B, HV, K, V))
    grads = oracle.kda_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], Wo,
                           WS if with_dST else None, initial_state=inp["S0"])
    h = 1e-6
    for name, grad in zip(("q", "k", "v", "g", "beta", "S0"), grads):
        x = inp[name]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + h
            lp = _loss(inp, Wo, WS)
            x[idx] = keep - h
            lm = _loss(inp, Wo, WS)
            x[idx] = keep
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-7, err_msg="d" + name)


def test_backward_explicit_scale():
    """A given scale enters dq linearly and the other gradients through o."""
    B, T, H, HV, K, V = 1, 4, 2, 2, 3, 3
    rng = np.random.default_rng(8)
    inp = dict(q=rng.standard_normal((B, T, H, K)), k=rng.standard_normal((B, T, H, K)),
               v=rng.standard_normal((B, T, HV, V)), g=-rng.random((B, T, HV, K)),
               beta=rng.random((B, T, HV)), S0=None)
    Wo = rng.standard_normal((B, T, HV, V))
    WS = np.zeros((B, HV, K, V))
    dq = oracle.kda_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], Wo, scale=0.7)[0]
    h = 1e-6
    idx = (0, 2, 1, 2)
    inp["q"][idx] += h
    lp = _loss(inp, Wo, WS, scale=0.7)
    inp["q"][idx] -= 2 * h
    lm = _loss(inp, Wo, WS, scale=0.7)
    assert abs(dq[idx] - (lp - lm) / (2 * h)) < 1e-7


def test_backward_empty_sequence_and_beta_zero():
    """T = 0: dS0 = dS_T and nothing else.  beta = 0: nothing is written, so
    dL/dv = 0 exactly, and dS0 = exp(sum of g) (.) dS_T + sum over t of
    exp(G_t) (.) (s q_t (x) dout_t)  (the state only decays)."""
    rng = np.random.default_rng(9)
    B, H, HV, K, V = 1, 1, 1, 3, 2
    dST = rng.standard_normal((B, HV, K, V))
    z = lambda *s: np.zeros(s)
    dq, dk, dv, dg, db, dS0 = oracle.kda_bwd(z(B, 0, H, K), z(B, 0, H, K), z(B, 0, HV, V), z(B, 0, HV, K),
                                             z(B, 0, HV), z(B, 0, HV, V), dST, initial_state=z(B, HV, K, V))
    assert dq.size == 0 and dv.size == 0 and dg.size == 0 and db.size == 0
    np.testing.assert_array_equal(dS0, dST)
    T = 4
    q, k = rng.standard_normal((B, T, H, K)), rng.standard_normal((B, T, H, K))
    v, g = rng.standard_normal((B, T, HV, V)), -rng.random((B, T, HV, K))
    do = rng.standard_normal((B, T, HV, V))
    dq, dk, dv, dg, db, dS0 = oracle.kda_bwd(q, k, v, g, np.zeros((B, T, HV)), do, dST,
                                             initial_state=rng.standard_normal((B, HV, K, V)))
    assert np.all(dv == 0.0)
    s = 1 / math.sqrt(K)
    G = np.cumsum(g[0, :, 0], axis=0)                    # [T, K]
    want = np.exp(G[-1])[:, None] * dST[0, 0]
    for t in range(T):
        want += np.exp(G[t])[:, None] * np.outer(s * q[0, t, 0], do[0, t, 0])
    np.testing.assert_allclose(dS0[0, 0], want, rtol=1e-12, atol=1e-14)


def test_backward_gqa_equals_explicit_repeat():
    """dq and dk of a q/k head are the sums over the value heads it serves
    (the repeat_interleave reversed)."""
    B, T, H, HV, K, V = 1, 6, 2, 4, 3, 2
    rng = np.random.default_rng(10)
    q, k = rng.standard_normal((B, T, H, K)), rng.standard_normal((B, T, H, K))
    v, g = rng.standard_normal((B, T, HV, V)), -rng.random((B, T, HV, K))
    beta, do = rng.random((B, T, HV)), rng.standard_normal((B, T, HV, V))
    a = oracle.kda_bwd(q, k, v, g, beta, do)
    qr, kr = np.repeat(q, HV // H, axis=2), np.repeat(k, HV // H, axis=2)
    r = oracle.kda_bwd(qr, kr, v, g, beta, do)
    np.testing.assert_allclose(a[0], r[0].reshape(B, T, H, HV // H, K).sum(3), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(a[1], r[1].reshape(B, T, H, HV // H, K).sum(3), rtol=1e-13, atol=1e-14)
    for i in range(2, 6):
        np.testing.assert_allclose(a[i], r[i], rtol=1e-13, atol=1e-14)


def test_dg_from_read_write_rescaling():
    """The identity the GPU backward forms dg from: adding eps to g_u scales
    every read at t >= u against every write at s < u by e^eps, so
    dg_u = sum_{t>=u} (qs_t*dqs_t - k_t*(S_dec,t dr_t) - beta_t k_t*da_t)
           + sum_V S_T * dL/dS_T.
    Its terms come from a plain numpy pass here; the sum must equal the
    oracle's dg (pinned by finite differences above)."""
    B, T, H, HV, K, V = 1, 9, 1, 1, 4, 3
    rng = np.random.default_rng(21)
    q, k = rng.standard_normal((T, K)), rng.standard_normal((T, K))
    v, g = rng.standard_normal((T, V)), -3.0 * rng.random((T, K))
    beta, S0 = rng.random(T), rng.standard_normal((K, V))
    do, dST = rng.standard_normal((T, V)), rng.standard_normal((K, V))
    s = 1 / math.sqrt(K)
    S, Sdec, St, r = S0.copy(), [], [], []
    for t in range(T):
        Sd = np.exp(g[t])[:, None] * S
        rt = v[t] - k[t] @ Sd
        S = Sd + np.outer(beta[t] * k[t], rt)
        Sdec.append(Sd); St.append(S.copy()); r.append(rt)
    D = dST.copy()
    e = np.zeros((T, K))
    for t in range(T - 1, -1, -1):
        D = D + np.outer(s * q[t], do[t])
        dqs = St[t] @ do[t]
        da = D @ r[t]
        dr = (beta[t] * k[t]) @ D
        e[t] = s * q[t] * dqs - k[t] * (Sdec[t] @ dr) - beta[t] * k[t] * da
        D = np.exp(g[t])[:, None] * (D - np.outer(k[t], dr))
    dg_identity = np.cumsum(e[::-1], axis=0)[::-1] + (S * dST).sum(axis=1)
    ref = oracle.kda_bwd(q[None, :, None], k[None, :, None], v[None, :, None], g[None, :, None],
                         beta[None, :, None], do[None, :, None], dST[None, None],
                         initial_state=S0[None, None])[3][0, :, 0]
    np.testing.assert_allclose(dg_identity, ref, rtol=1e-11, atol=1e-12)
