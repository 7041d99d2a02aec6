"""Pins for the fp64 oracle, against what the pages and the mathematics fix.

None of these re-types the oracle's own formulas: each checks the oracle
against a different route to the same number (a singular-value closed form, a
textbook algorithm, a scalar recursion, an invariant the MuonGS page states,
or an independent library routine), chosen so that a dropped term, a wrong
sign or a transposed operand anywhere in the oracle fails at least one test.
"""
import json
import os

import numpy as np
import pytest

from oracle import (NS_COEFFICIENTS, NS_EPS, RMS_MATCH, frobenius_inner, muon_step,
                    muongs_project, nesterov_momentum, newton_schulz, update_scale)

HERE = os.path.dirname(os.path.abspath(__file__))
CLASSICAL = (15 / 8, -10 / 8, 3 / 8)


def relerr(x, y):
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    return float(np.linalg.norm(x - y) / max(np.linalg.norm(y), 1e-300))


def f_scalar(x, a, b, c):
    """The odd quintic the iteration applies to every singular value."""
    return a * x + b * x ** 3 + c * x ** 5


def f_iter(x, coeffs, n):
    for _ in range(n):
        x = f_scalar(x, *coeffs)
    return x


def semi_orthogonal(rows, cols, rng):
    """An exactly (to rounding) semi-orthogonal rows x cols matrix via QR."""
    p, q = min(rows, cols), max(rows, cols)
    Q, _ = np.linalg.qr(rng.standard_normal((q, p)))   # q x p, orthonormal columns
    return Q.T if rows < cols else Q


# ---------------------------------------------------------------- page numbers
def test_constants_match_pages():
    """The oracle's constants are the numbers the pages print (cited fixture)."""
    with open(os.path.join(HERE, "golden", "page_constants.json")) as fh:
        fx = json.load(fh)
    assert tuple(fx["ns_coefficients"]["value"]) == NS_COEFFICIENTS
    assert fx["ns_eps"]["value"] == NS_EPS
    assert fx["rms_match_constant"]["value"] == RMS_MATCH
    from oracle import DEFAULT_LR, DEFAULT_MOMENTUM, DEFAULT_NS_STEPS, DEFAULT_WEIGHT_DECAY
    assert fx["lr"]["value"] == DEFAULT_LR
    assert fx["momentum"]["value"] == DEFAULT_MOMENTUM
    assert fx["ns_steps"]["value"] == DEFAULT_NS_STEPS
    assert fx["weight_decay_example"]["value"] == DEFAULT_WEIGHT_DECAY


# -------------------------------------------- P-1: singular-value closed form
@pytest.mark.parametrize("shape", [(3, 5), (8, 8), (16, 40), (40, 16), (1, 7), (7, 1), (24, 24)])
@pytest.mark.parametrize("coeffs", [NS_COEFFICIENTS, CLASSICAL, (2.0, -1.5, 0.5), (1.1, 0.3, -0.2)])
@pytest.mark.parametrize("steps", [0, 1, 2, 5])
def test_ns_equals_singular_value_polynomial(shape, coeffs, steps):
    """NS(U) = U_s diag(f^N(sigma_i / (||U||_F + eps))) V_s^T.

    Every term of X <- aX + b(XX^T)X + c(XX^T)^2 X acts on the singular values
    alone, so the iteration is f^N applied to the normalised spectrum.  A sign
    error, a dropped term, X@B instead of B@X, X^T X instead of X X^T or a
    spectral instead of a Frobenius normalisation all break this identity.
    """
    rng = np.random.default_rng(hash((shape, steps)) % (2 ** 32))
    U = rng.standard_normal(shape) * 0.37
    Us, s, Vt = np.linalg.svd(U, full_matrices=False)
    fro = float(np.sqrt(np.sum(s ** 2)))
    expected = Us @ np.diag(f_iter(s / (fro + NS_EPS), coeffs, steps)) @ Vt
    got = newton_schulz(U, *coeffs, steps)
    assert got.shape == U.shape
    assert relerr(got, expected) < 1e-12


def test_ns_row_vector_brute_force():
    """p = 1: X X^T is the scalar x^2, so O = f^N(|u|/(|u|+eps)) u/|u| directly."""
    u = np.array([[0.3, -1.2, 0.05, 2.0, -0.7]])
    nrm = float(np.sqrt(np.sum(u ** 2)))
    x0 = nrm / (nrm + NS_EPS)
    expected = f_iter(x0, NS_COEFFICIENTS, 5) * u / nrm
    assert relerr(newton_schulz(u, *NS_COEFFICIENTS, 5), expected) < 1e-14
    assert relerr(newton_schulz(u.T, *NS_COEFFICIENTS, 5), expected.T) < 1e-14


# ------------------------------------ P-2: classical coefficients, polar factor
def test_classical_coefficients_from_conditions():
    """f(1) = 1, f'(1) = 0, f''(1) = 0 fix the classical quintic."""
    Msys = np.array([[1.0, 1.0, 1.0], [1.0, 3.0, 5.0], [0.0, 6.0, 20.0]])
    abc = np.linalg.solve(Msys, np.array([1.0, 0.0, 0.0]))
    assert np.allclose(abc, CLASSICAL, atol=1e-15, rtol=0)
    # The pages' coefficients trade exactness at 1 for speed near 0: f(1) = 0.701.
    assert abs(f_scalar(1.0, *NS_COEFFICIENTS) - 0.7010) < 1e-12


@pytest.mark.parametrize("shape", [(3, 5), (8, 8), (16, 40), (40, 16)])
def test_classical_ns_converges_to_polar_factor(shape):
    """With the classical coefficients the iteration reaches U V^T (the polar
    factor (MM^T)^{-1/2} M the pages say NS approximates)."""
    rng = np.random.default_rng(7)
    U = rng.standard_normal(shape)
    Us, s, Vt = np.linalg.svd(U, full_matrices=False)
    assert s.min() / np.sqrt(np.sum(s ** 2)) > 1e-3  # full rank, well within reach
    polar = Us @ Vt
    assert relerr(newton_schulz(U, *CLASSICAL, 40), polar) < 1e-12


def test_pages_coefficients_do_not_converge():
    """The printed (3.4445, -4.7750, 2.0315) leave singular values spread in
    roughly [0.68, 1.2] after 5 steps instead of reaching 1."""
    rng = np.random.default_rng(3)
    O = newton_schulz(rng.standard_normal((64, 160)), *NS_COEFFICIENTS, 5)
    s = np.linalg.svd(O, compute_uv=False)
    assert 0.6 < s.min() < 0.95 and 1.0 < s.max() < 1.21


# ----------------------------------------- P-3: scalar special case, full step
@pytest.mark.parametrize("shape", [(4, 9), (8, 8), (16, 6), (32, 64)])
@pytest.mark.parametrize("variant", ["muon", "muongs"])
def test_semi_orthogonal_gradient_step(shape, variant):
    """G = Q semi-orthogonal, M = 0: U = (1+mu) Q, every singular value of X_0
    is x0 = (1+mu)/((1+mu) sqrt(p) + eps), so O = f^5(x0) Q and
    W' = (1 - lr wd) W - lr s f^5(x0) Q.  (MuonGS: W chosen orthogonal to Q.)"""
    rng = np.random.default_rng(11)
    rows, cols = shape
    p = min(shape)
    Q = semi_orthogonal(rows, cols, rng)
    W = rng.standard_normal(shape) * 0.02
    if variant == "muongs":
        W = W - frobenius_inner(W, Q) / frobenius_inner(Q, Q) * Q
    lr, mu, wd = 0.02, 0.95, 0.1
    Wn, Mn, st = muon_step(W, Q, np.zeros(shape), lr=lr, momentum=mu, weight_decay=wd,
                           ns_steps=5, variant=variant)
    x0 = (1 + mu) / ((1 + mu) * np.sqrt(p) + NS_EPS)
    fo = f_iter(x0, NS_COEFFICIENTS, 5)
    s = 0.2 * np.sqrt(max(rows, cols))
    expected = (1 - lr * wd) * W - lr * s * fo * Q
    assert relerr(Wn, expected) < 1e-12
    assert relerr(Mn, Q) < 1e-15


def test_scalar_values_for_config_widths():
    """f^5(1/sqrt(p)) for the p of the configs: the NS gain a semi-orthogonal
    gradient sees.  Checked through the matrix iteration on exactly
    semi-orthogonal inputs of each width."""
    rng = np.random.default_rng(5)
    for p in (4, 8, 64, 256):
        Q = semi_orthogonal(p, 2 * p, rng)
        O = newton_schulz(Q, *NS_COEFFICIENTS, 5)
        expected = f_iter(1.0 / (np.sqrt(p) + NS_EPS), NS_COEFFICIENTS, 5)
        assert relerr(O, expected * Q) < 1e-12


# ------------------------------------------------------------- P-4: RMS 0.2
@pytest.mark.parametrize("shape", [(8, 8), (16, 48), (48, 16), (256, 512)])
def test_rms_of_scaled_semi_orthogonal_update(shape):
    """||O||_F^2 = p for a semi-orthogonal O, so RMS(0.2 sqrt(max) O) = 0.2."""
    rng = np.random.default_rng(2)
    Q = semi_orthogonal(*shape, rng)
    upd = update_scale(*shape) * Q
    assert abs(np.sqrt(np.mean(upd ** 2)) - 0.2) < 1e-14


@pytest.mark.parametrize("shape", [(16, 48), (48, 16), (32, 32)])
def test_rms_end_to_end_converged(shape):
    """Classical coefficients, 40 steps, wd = 0: RMS(W' - W) / lr = 0.2."""
    rng = np.random.default_rng(4)
    W = rng.standard_normal(shape) * 0.02
    G = rng.standard_normal(shape) * 1e-3
    Wn, _, _ = muon_step(W, G, np.zeros(shape), lr=0.02, weight_decay=0.0, ns_steps=40,
                         a=CLASSICAL[0], b=CLASSICAL[1], c=CLASSICAL[2])
    assert abs(np.sqrt(np.mean((Wn - W) ** 2)) / 0.02 - 0.2) < 1e-10


# --------------------------------------------------- P-5: MuonGS invariants
@pytest.mark.parametrize("shape", [(16, 40), (40, 16), (32, 32), (64, 128)])
@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_muongs_invariants(shape, wd):
    """[MuonGS page, "전제와 한계"]: <W, O~> = 0, ||O~|| <= ||O||, and
    r'^2 = (1 - lr wd)^2 r^2 + (lr s)^2 ||O~||^2 (the page's identity at wd = 0,
    with its step size eta equal to lr * s here)."""
    rng = np.random.default_rng(21)
    W = rng.standard_normal(shape) * 0.02
    G = rng.standard_normal(shape) * 1e-3
    M = rng.standard_normal(shape) * 1e-3
    lr = 0.02
    s = 0.2 * np.sqrt(max(shape))
    Wn, _, st = muon_step(W, G, M, lr=lr, weight_decay=wd, variant="muongs")
    Ot = -(Wn - (1 - lr * wd) * W) / (lr * s)
    cos = frobenius_inner(W, Ot) / np.sqrt(frobenius_inner(W, W) * frobenius_inner(Ot, Ot))
    assert abs(cos) < 1e-12
    assert frobenius_inner(Ot, Ot) <= st["norm2_O"] * (1 + 1e-12)
    assert abs(frobenius_inner(Ot, Ot) / st["norm2_Ot"] - 1) < 1e-10
    r2n = (1 - lr * wd) ** 2 * st["r2"] + (lr * s) ** 2 * st["norm2_Ot"]
    assert abs(frobenius_inner(Wn, Wn) / r2n - 1) < 1e-12
    # Gaussian inputs keep the spectrum of O below 1 on average: ||O~|| <= sqrt(p).
    assert np.sqrt(st["norm2_Ot"]) <= np.sqrt(min(shape))


def test_muongs_radial_update_vanishes():
    """If O is parallel to W the projection removes all of it: W' = (1-lr wd) W."""
    rng = np.random.default_rng(8)
    Q = semi_orthogonal(12, 20, rng)
    W = 0.02 * Q
    Wn, _, _ = muon_step(W, Q, np.zeros_like(Q), lr=0.02, weight_decay=0.1, variant="muongs")
    assert relerr(Wn, (1 - 0.002) * W) < 1e-13


def test_muongs_zero_weight_keeps_update():
    """r = 0: no radial direction, O~ = O (Muon and MuonGS agree)."""
    rng = np.random.default_rng(9)
    G = rng.standard_normal((8, 12))
    W = np.zeros((8, 12))
    a, _, _ = muon_step(W, G, np.zeros_like(G), variant="muon")
    b, _, _ = muon_step(W, G, np.zeros_like(G), variant="muongs")
    assert np.array_equal(a, b)
    assert np.array_equal(muongs_project(W, G), G)


def test_muongs_norm_growth_bound_over_steps():
    """[MuonGS page, Thm 4.1]: with wd = 0, r_T^2 <= r_0^2 + p sum (lr s)^2."""
    rng = np.random.default_rng(12)
    shape = (32, 96)
    p = min(shape)
    W = rng.standard_normal(shape) * 0.02
    M = np.zeros(shape)
    r0 = frobenius_inner(W, W)
    lr = 0.02
    s = 0.2 * np.sqrt(max(shape))
    for t in range(10):
        G = rng.standard_normal(shape) * 1e-3
        W, M, _ = muon_step(W, G, M, lr=lr, weight_decay=0.0, variant="muongs")
        assert frobenius_inner(W, W) <= r0 + p * (t + 1) * (lr * s) ** 2


# --------------------------------------------------- P-6: momentum, Nesterov
def test_momentum_closed_form():
    """M_t = sum_k mu^(t-k) G_k from M_0 = 0 (SGD-momentum buffer)."""
    rng = np.random.default_rng(13)
    mu = 0.95
    Gs = [rng.standard_normal((5, 7)) for _ in range(6)]
    M = np.zeros((5, 7))
    for t, G in enumerate(Gs):
        M, _ = nesterov_momentum(G, M, mu)
        expected = sum(mu ** (t - k) * Gs[k] for k in range(t + 1))
        assert relerr(M, expected) < 1e-14


def test_nesterov_reproduces_textbook_nag():
    """Plain SGD on the look-ahead direction U reproduces classical Nesterov
    accelerated gradient (v <- mu v - lr grad(theta + mu v); theta <- theta + v):
    the iterate phi = theta + mu v of NAG equals phi <- phi - lr U with U from
    ``nesterov_momentum``.  Pins both M' = mu M + G and U = G + mu M'."""
    rng = np.random.default_rng(14)
    n = 6
    H = rng.standard_normal((n, n))
    H = H @ H.T / n + np.eye(n)
    grad = lambda x: H @ x  # noqa: E731
    lr, mu = 0.05, 0.9
    theta = rng.standard_normal(n)
    v = np.zeros(n)
    phi = theta.copy()
    M = np.zeros(n)
    for _ in range(25):
        v = mu * v - lr * grad(theta + mu * v)
        theta = theta + v
        M, U = nesterov_momentum(grad(phi), M, mu)
        phi = phi - lr * U
        assert np.allclose(phi, theta + mu * v, rtol=0, atol=1e-12)


# ------------------------------------------ P-7..P-9: symmetries, zero case
@pytest.mark.parametrize("variant", ["muon", "muongs"])
def test_transpose_equivariance(variant):
    rng = np.random.default_rng(15)
    W = rng.standard_normal((24, 40)) * 0.02
    G = rng.standard_normal((24, 40)) * 1e-3
    M = rng.standard_normal((24, 40)) * 1e-3
    a, am, _ = muon_step(W, G, M, variant=variant)
    b, bm, _ = muon_step(W.T, G.T, M.T, variant=variant)
    assert relerr(b, a.T) < 1e-14 and relerr(bm, am.T) == 0.0


def test_scale_invariance():
    """Scaling G and M by k > 0 leaves W' unchanged up to the eps term."""
    rng = np.random.default_rng(16)
    W = rng.standard_normal((20, 30)) * 0.02
    G = rng.standard_normal((20, 30))
    M = rng.standard_normal((20, 30))
    a, _, _ = muon_step(W, G, M)
    b, _, _ = muon_step(W, 8.0 * G, 8.0 * M)
    assert relerr(b - W, a - W) < 1e-8


@pytest.mark.parametrize("variant", ["muon", "muongs"])
def test_zero_gradient_and_momentum(variant):
    """G = M = 0: X_0 = 0/(0 + eps) = 0, so O = 0 and W' = (1 - lr wd) W."""
    rng = np.random.default_rng(17)
    W = rng.standard_normal((10, 14)) * 0.02
    Wn, Mn, st = muon_step(W, np.zeros_like(W), np.zeros_like(W), lr=0.02,
                           weight_decay=0.1, variant=variant)
    assert np.array_equal(Wn, (1 - 0.02 * 0.1) * W)
    assert not Mn.any() and st["norm2_O"] == 0.0


def test_non_2d_rejected():
    with pytest.raises(ValueError):
        muon_step(np.zeros(5), np.zeros(5), np.zeros(5))


# --------------------------- P-11: torch.optim.Muon as an independent routine
@pytest.mark.parametrize("shape", [(48, 80), (80, 48)])
def test_against_torch_optim_muon(shape):
    """torch.optim.Muon with Moonlight's RMS matching agrees with the oracle's
    two-step trajectory to bf16 accuracy (it runs its iteration in bf16).
    Two steps, so the momentum buffer is non-zero in the second: this checks
    the Nesterov direction, the 0.2 sqrt(max) scale, the decay with the
    unscaled lr, the update sign and the short-side transposition."""
    torch = pytest.importorskip("torch")
    if not hasattr(torch.optim, "Muon"):
        pytest.skip("torch.optim.Muon not available")
    rng = np.random.default_rng(18)
    W0 = rng.standard_normal(shape) * 0.02
    Gs = [rng.standard_normal(shape) * 1e-3 for _ in range(2)]
    p = torch.nn.Parameter(torch.tensor(W0, dtype=torch.float32))
    opt = torch.optim.Muon([p], lr=0.02, momentum=0.95, weight_decay=0.1, nesterov=True,
                           adjust_lr_fn="match_rms_adamw")
    W, M = W0, np.zeros(shape)
    for G in Gs:
        p.grad = torch.tensor(G, dtype=torch.float32)
        opt.step()
        W, M, _ = muon_step(W, G, M, lr=0.02, momentum=0.95, weight_decay=0.1)
    got = p.detach().double().numpy()
    assert relerr(got - W0, W - W0) < 2e-2


# ------------------------------------------- MuonH and Keller's shape scale
@pytest.mark.parametrize("shape", [(16, 40), (40, 16), (24, 24)])
@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_muonh_keeps_the_norm(shape, wd):
    """MuonH holds ||W||_F fixed (the [GS] page's fixed-radius control), and
    W' points along (1 - lr wd) W - lr s O."""
    rng = np.random.default_rng(31)
    W = rng.standard_normal(shape) * 0.02
    G = rng.standard_normal(shape) * 1e-3
    Wn, _, st = muon_step(W, G, np.zeros(shape), weight_decay=wd, variant="muonh")
    assert abs(np.linalg.norm(Wn) / np.linalg.norm(W) - 1) < 1e-13
    Wm, _, _ = muon_step(W, G, np.zeros(shape), weight_decay=wd, variant="muon")
    cos = frobenius_inner(Wn, Wm) / (np.linalg.norm(Wn) * np.linalg.norm(Wm))
    assert abs(cos - 1) < 1e-13


def test_muonh_orthogonal_update_closed_form():
    """O orthogonal to W (W chosen so), wd = 0: ||W - lr s O||^2 = r^2 +
    (lr s)^2 ||O||^2, so W' = r (W - lr s O) / sqrt(r^2 + (lr s)^2 ||O||^2), and
    the effective step size per unit radius is lr / r every step (C_T = lr T / R)."""
    rng = np.random.default_rng(32)
    shape = (12, 30)
    Q = semi_orthogonal(*shape, rng)
    W = rng.standard_normal(shape) * 0.02
    W = W - frobenius_inner(W, Q) / frobenius_inner(Q, Q) * Q
    r = np.linalg.norm(W)
    Wn, _, _ = muon_step(W, Q, np.zeros(shape), weight_decay=0.0, variant="muonh")
    O = newton_schulz(1.95 * Q, *NS_COEFFICIENTS, 5)
    s = 0.2 * np.sqrt(30)
    expect = r * (W - 0.02 * s * O) / np.sqrt(r ** 2 + (0.02 * s) ** 2 * np.sum(O ** 2))
    assert relerr(Wn, expect) < 1e-12
    # fixed radius: T steps accumulate C_T = sum lr/||W_t|| = lr T / r exactly
    Wt, C = W, 0.0
    for t in range(5):
        C += 0.02 / np.linalg.norm(Wt)
        Wt, _, _ = muon_step(Wt, rng.standard_normal(shape) * 1e-3, np.zeros(shape),
                             weight_decay=0.0, variant="muonh")
    assert abs(C / (0.02 * 5 / r) - 1) < 1e-12


@pytest.mark.parametrize("shape,factor", [((64, 64), 1.0), ((256, 64), 2.0), ((64, 256), 1.0),
                                          ((90, 10), 3.0)])
def test_keller_shape_factor(shape, factor):
    """[LS] code block, last line: update = X * max(1, rows/cols)^0.5."""
    assert update_scale(*shape, scale="keller") == pytest.approx(factor, rel=0, abs=1e-15)
    rng = np.random.default_rng(33)
    W = rng.standard_normal(shape) * 0.02
    G = rng.standard_normal(shape) * 1e-3
    Wk, _, _ = muon_step(W, G, np.zeros(shape), scale="keller")
    Wm, _, _ = muon_step(W, G, np.zeros(shape))
    dk = Wk - (1 - 0.002) * W
    dm = Wm - (1 - 0.002) * W
    # same direction, magnitudes in the ratio of the two factors
    assert relerr(dk, dm * factor / (0.2 * np.sqrt(max(shape)))) < 1e-12
