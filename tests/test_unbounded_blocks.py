"""The block split behind kda_chunk_fwd_unbounded's in-chunk matrices, on the
CPU: every entry (i, j <= i) of A_qk and A_kk of a chunk is formed in exactly
one block, as a row factor times a column factor around that block's
reference row, and in fp32 the products reproduce the fp64 definition

    A_qk[i][j] = sum_c q_ic k_jc 2^(G_ic - G_jc)      (j <= i)
    A_kk[i][j] = sum_c k_ic k_jc 2^(G_ic - G_jc)      (j < i, beta not applied)

with G the chunk-local cumulative sum of max(g, -17) in base 2, for gates far
below any bounded range, without an overflow."""
import numpy as np
import pytest

FLOOR = -17.0
C = 32


def family(w, x):
    """(row, its reference row) for operand slot x of block family w; the
    column side uses the same map (F1: rows 16..31 against columns 0..15)."""
    if w == 0:
        return (16 + x, 15), (x, 15)
    if w == 1:
        r = 8 + x if x < 8 else 16 + x
        c = x if x < 8 else 8 + x
        ref = 7 if x < 8 else 23
        return (r, ref), (c, ref)
    o = 16 * (w - 2)
    ref = o + (3 if x < 8 else 11)
    return (o + x, ref), (o + x, ref)


def keeps(w, r, x):
    """Which slot pairs (tile row r, tile column x) of family w are entries of
    the lower triangle that this family owns."""
    if w == 0:
        return True
    return (r < 8) == (x < 8)


def blocked(q, k, G):
    Aq = np.full((C, C), np.nan, np.float32)
    Ak = np.full((C, C), np.nan, np.float32)
    owner = np.zeros((C, C), int)
    with np.errstate(over="ignore", invalid="ignore", under="ignore"):
        for w in range(4):
            for r in range(16):
                (ri, rr), _ = family(w, r)
                fr = np.exp2(G[ri] - G[rr])
                assert np.all(np.isfinite(fr)), "row factor overflow"
                for x in range(16):
                    if not keeps(w, r, x):
                        continue
                    _, (cj, rc) = family(w, x)
                    if cj > ri:
                        continue
                    fc = np.exp2(G[rc] - G[cj])
                    assert np.all(np.isfinite(fc)), "column factor overflow"
                    b = (k[cj] * fc).astype(np.float32)
                    Aq[ri, cj] = np.float32(np.dot((q[ri] * fr).astype(np.float32), b))
                    if cj < ri:
                        Ak[ri, cj] = np.float32(np.dot((k[ri] * fr).astype(np.float32), b))
                    owner[ri, cj] += 1
    return Aq, Ak, owner


@pytest.mark.parametrize("seed,kind", [(0, "heavy"), (1, "extreme"), (2, "floor"), (3, "mild")])
def test_block_split_reproduces_definition(seed, kind):
    rng = np.random.default_rng(seed)
    K = 32
    q = (rng.standard_normal((C, K)) / np.sqrt(K)).astype(np.float32)
    k = (rng.standard_normal((C, K)) / np.sqrt(K)).astype(np.float32)
    if kind == "heavy":
        g = -np.exp(1.5 * rng.standard_normal((C, K)))
    elif kind == "extreme":
        g = -np.exp(3.0 * rng.standard_normal((C, K)))
        g[::7] = -1.0e4
    elif kind == "floor":
        g = -17.0 + 4.0 * (rng.random((C, K)) - 0.5)
    else:
        g = -5.0 / (1.0 + np.exp(-rng.standard_normal((C, K))))
    gf = (np.maximum(g, FLOOR) / np.log(2.0)).astype(np.float32)
    G = np.cumsum(gf, axis=0, dtype=np.float32)
    Aq, Ak, owner = blocked(q, k, G)
    # every lower entry (diagonal included) owned by exactly one block
    assert np.array_equal(owner, np.tril(np.ones((C, C), int)))
    G64 = np.cumsum(np.maximum(g, FLOOR) / np.log(2.0), axis=0)
    for i in range(C):
        for j in range(i + 1):
            f = np.exp2(G64[i] - G64[j])
            want = float(np.sum(q[i].astype(np.float64) * k[j] * f))
            scale = float(np.sum(np.abs(q[i].astype(np.float64) * k[j]))) + 1e-30
            assert abs(Aq[i, j] - want) <= 2e-5 * scale, (i, j, Aq[i, j], want)
            if j < i:
                want = float(np.sum(k[i].astype(np.float64) * k[j] * f))
                scale = float(np.sum(np.abs(k[i].astype(np.float64) * k[j]))) + 1e-30
                assert abs(Ak[i, j] - want) <= 2e-5 * scale, (i, j, Ak[i, j], want)


def test_single_reference_row_overflows():
    """The one reference row of the bounded kernels (row 15) does not survive
    these gates: a row factor 2^(G_0 - G_15) overflows fp32."""
    g = np.full((C, 4), -17.0)
    G = np.cumsum((g / np.log(2.0)).astype(np.float32), axis=0, dtype=np.float32)
    with np.errstate(over="ignore"):
        assert not np.all(np.isfinite(np.exp2(G[0] - G[15]).astype(np.float32)))
