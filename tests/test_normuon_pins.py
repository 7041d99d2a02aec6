"""Pins for the NorMuon / MeqMuon normalisations in the fp64 oracle.

The MeqMuon page describes row-wise (NorMuon) and column-wise normalisation
of the orthogonalised update and an automatic choice between them, without
formulas.  The normalisations are pinned here by brute force on small
matrices and by the cases where they reduce to the identity (an update whose
rows, or columns, are orthonormal); the choice of direction is a reading of
the page ("parity unpinned"), checked only for being the documented rule.
"""
import math

import numpy as np
import pytest

from oracle import (frobenius_inner, meqmuon_direction, muon_step, normuon_cols, normuon_rows)


def brute_rows(O):
    """Row equalisation written out element by element."""
    O = np.asarray(O, np.float64)
    rows, cols = O.shape
    total = 0.0
    for i in range(rows):
        for j in range(cols):
            total += O[i, j] * O[i, j]
    target = math.sqrt(total / rows)
    out = np.zeros_like(O)
    for i in range(rows):
        n = math.sqrt(sum(O[i, j] * O[i, j] for j in range(cols)))
        if n > 0:
            for j in range(cols):
                out[i, j] = O[i, j] * target / n
    return out


@pytest.mark.parametrize("shape", [(3, 5), (5, 3), (7, 7), (1, 6), (6, 1)])
def test_rows_brute_force(shape):
    O = np.random.default_rng(51).standard_normal(shape)
    assert np.max(np.abs(normuon_rows(O) - brute_rows(O))) < 1e-14


@pytest.mark.parametrize("shape", [(3, 5), (5, 3), (7, 7)])
def test_cols_is_rows_of_transpose(shape):
    O = np.random.default_rng(52).standard_normal(shape)
    assert np.max(np.abs(normuon_cols(O) - brute_rows(O.T).T)) < 1e-14


def test_equal_norms_and_kept_frobenius_norm():
    O = np.random.default_rng(53).standard_normal((9, 13)) * np.arange(1, 10)[:, None]
    R = normuon_rows(O)
    rn = np.linalg.norm(R, axis=1)
    assert np.max(np.abs(rn - rn[0])) < 1e-13
    assert abs(np.linalg.norm(R) - np.linalg.norm(O)) < 1e-12
    # each row keeps its direction
    for i in range(9):
        cos = frobenius_inner(R[i], O[i]) / (np.linalg.norm(R[i]) * np.linalg.norm(O[i]))
        assert abs(cos - 1) < 1e-14


def test_identity_on_orthonormal_rows_and_columns():
    rng = np.random.default_rng(54)
    Q, _ = np.linalg.qr(rng.standard_normal((12, 5)))   # 12 x 5, orthonormal columns
    assert np.max(np.abs(normuon_cols(Q) - Q)) < 1e-14   # tall: columns already equal
    assert np.max(np.abs(normuon_rows(Q.T) - Q.T)) < 1e-14  # wide: rows already equal


def test_zero_rows_and_zero_matrix():
    O = np.random.default_rng(55).standard_normal((4, 6))
    O[2] = 0.0
    R = normuon_rows(O)
    assert not R[2].any()
    target = np.linalg.norm(O) / 2.0                      # sqrt(4 rows)
    assert np.allclose(np.linalg.norm(R[[0, 1, 3]], axis=1), target, rtol=0, atol=1e-14)
    assert not normuon_rows(np.zeros((3, 3))).any()


def test_scale_covariance():
    O = np.random.default_rng(56).standard_normal((6, 4))
    assert np.max(np.abs(normuon_rows(3.5 * O) - 3.5 * normuon_rows(O))) < 1e-13


def test_meqmuon_direction_rule():
    """Reading of the page: the direction whose norms vary more (std / mean)
    is equalised; ties go to rows."""
    rng = np.random.default_rng(57)
    O = rng.standard_normal((16, 16))
    O[3] *= 40.0                                          # one dominant row
    assert meqmuon_direction(O) == "rows"
    assert meqmuon_direction(O.T) == "cols"
    Q, _ = np.linalg.qr(rng.standard_normal((10, 4)))
    assert meqmuon_direction(Q.T) == "cols"               # rows equal, columns spread
    assert meqmuon_direction(np.ones((5, 5))) == "rows"   # tie


def semi_orthogonal(rows, cols, rng):
    p, q = min(rows, cols), max(rows, cols)
    Q, _ = np.linalg.qr(rng.standard_normal((q, p)))
    return Q.T if rows < cols else Q


@pytest.mark.parametrize("shape", [(8, 24), (24, 8)])
def test_normuon_step_on_semi_orthogonal_gradient(shape):
    """G = Q semi-orthogonal, M = 0: O = f^5(1/sqrt(p)) Q, whose short-side
    vectors all have the same norm.  For a wide W those are the rows, so
    NorMuon's step equals Muon's; for a tall W the rows differ (columns are
    the equal ones), and the step equals Muon's with O's rows equalised."""
    rng = np.random.default_rng(58)
    W = rng.standard_normal(shape) * 0.02
    Q = semi_orthogonal(*shape, rng)
    Wn, _, st = muon_step(W, Q, np.zeros(shape), variant="normuon")
    Wm, _, _ = muon_step(W, Q, np.zeros(shape), variant="muon")
    if shape[0] < shape[1]:
        assert np.max(np.abs(Wn - Wm)) < 1e-15
    else:
        d = 1 - 0.02 * 0.1
        O = -(Wm - d * W) / (0.02 * 0.2 * math.sqrt(max(shape)))
        assert np.max(np.abs(Wn - (d * W - 0.02 * 0.2 * math.sqrt(max(shape)) * brute_rows(O)))) < 1e-15
        assert abs(st["norm2_Ot"] - st["norm2_O"]) < 1e-12 * st["norm2_O"]


def spread_loops(O, rows_first):
    """std / mean of the row (or column) norms, written out with loops."""
    O = np.asarray(O, np.float64)
    n0, n1 = O.shape if rows_first else O.T.shape
    A = O if rows_first else O.T
    norms = [math.sqrt(sum(A[i, j] ** 2 for j in range(n1))) for i in range(n0)]
    mean = sum(norms) / n0
    var = sum((x - mean) ** 2 for x in norms) / n0
    return math.sqrt(var) / mean


MEQ_CASES = [("row", (20, 12)), ("col", (20, 12)), ("row", (12, 20)), ("col", (12, 20))]


def meq_case(heavy, shape):
    rng = np.random.default_rng(59)
    W = rng.standard_normal(shape) * 0.02
    G = rng.standard_normal(shape) * 1e-3
    if heavy == "row":
        G[5] *= 30.0
    else:
        G[:, 5] *= 30.0
    return W, G


@pytest.mark.parametrize("heavy,shape", MEQ_CASES)
def test_meqmuon_step_follows_its_choice(heavy, shape):
    """MeqMuon equalises the direction whose norms in O vary more (computed
    here with loops), and the step is Muon's with that direction equalised."""
    W, G = meq_case(heavy, shape)
    Wq, _, _ = muon_step(W, G, np.zeros(shape), variant="meqmuon")
    Wr, _, _ = muon_step(W, G, np.zeros(shape), variant="normuon")
    Wm, _, _ = muon_step(W, G, np.zeros(shape), variant="muon")
    d, step = 1 - 0.02 * 0.1, 0.02 * 0.2 * math.sqrt(max(shape))
    O = -(Wm - d * W) / step
    rows = spread_loops(O, True) >= spread_loops(O, False)
    expect = d * W - step * (brute_rows(O) if rows else brute_rows(O.T).T)
    assert np.max(np.abs(Wq - expect)) < 1e-14
    if rows:
        assert np.max(np.abs(Wq - Wr)) < 1e-15


def test_meqmuon_cases_cover_both_directions():
    """Orthogonalisation evens out the short side: a dominant gradient row of
    a tall matrix or column of a wide one leaves O spread along the long side."""
    seen = set()
    for heavy, shape in MEQ_CASES:
        W, G = meq_case(heavy, shape)
        Wm, _, _ = muon_step(W, G, np.zeros(shape), variant="muon")
        O = -(Wm - (1 - 0.002) * W) / (0.02 * 0.2 * math.sqrt(max(shape)))
        seen.add(meqmuon_direction(O))
    assert seen == {"rows", "cols"}


# Shapes on both sides of square, from nearly square to very elongated.
FORCED_SHAPES = [(4, 9), (9, 4), (16, 40), (40, 16), (3, 100), (100, 3), (64, 256), (256, 64),
                 (31, 33), (33, 31)]


@pytest.mark.parametrize("shape", FORCED_SHAPES)
def test_meqmuon_forced_direction(shape):
    """The cases the page's sentence decides on its own (MeqMuon picks the
    direction that is imbalanced): in a semi-orthogonal O the short side's
    vectors all have norm 1 (spread 0) while the long side's differ, so the
    long side's vectors are equalised — columns of a wide O, rows of a tall
    one — whatever rule settles two imbalanced directions."""
    rng = np.random.default_rng(61 + shape[0] + 7 * shape[1])
    Q = semi_orthogonal(*shape, rng)
    wide = shape[0] < shape[1]
    assert meqmuon_direction(Q) == ("cols" if wide else "rows")
    assert meqmuon_direction(2.5 * Q) == ("cols" if wide else "rows")


@pytest.mark.parametrize("shape", FORCED_SHAPES)
def test_meqmuon_forced_step(shape):
    """The whole step on a semi-orthogonal gradient Q (M = 0): O = f^5(x0) Q
    keeps Q's equal short-side norms, so MeqMuon's step is Muon's with the
    long side's vectors of O equalised (brute force), and NorMuon's equals
    it for a tall W (rows are the long side's vectors there)."""
    rng = np.random.default_rng(62 + shape[0] + 7 * shape[1])
    W = rng.standard_normal(shape) * 0.02
    Q = semi_orthogonal(*shape, rng)
    M0 = np.zeros(shape)
    Wq, _, _ = muon_step(W, Q, M0, variant="meqmuon")
    Wm, _, _ = muon_step(W, Q, M0, variant="muon")
    d, step = 1 - 0.02 * 0.1, 0.02 * 0.2 * math.sqrt(max(shape))
    O = -(Wm - d * W) / step
    wide = shape[0] < shape[1]
    expect = d * W - step * (brute_rows(O.T).T if wide else brute_rows(O))
    assert np.max(np.abs(Wq - expect)) < 1e-14
    if not wide:
        Wr, _, _ = muon_step(W, Q, M0, variant="normuon")
        assert np.max(np.abs(Wq - Wr)) < 1e-15
