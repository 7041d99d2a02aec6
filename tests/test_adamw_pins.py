"""Pins for the fp64 AdamW oracle (the hybrid optimizer's non-Muon half).

Each test reaches the oracle's numbers by another route: an independent
library routine (``torch.optim.AdamW`` in float64), the closed forms of the
first step and of a constant gradient (where the bias corrections cancel the
moments' start from zero exactly), the moments written as weighted sums, and
the zero case.  A dropped bias correction, swapped betas, eps inside the
square root, decay scaled without lr or applied after the Adam term, or a
sign error fails at least one of them.
"""
import json
import os

import numpy as np
import pytest

from oracle import AUX_BETAS, AUX_EPS, AUX_LR, AUX_WEIGHT_DECAY, adamw_step

HERE = os.path.dirname(os.path.abspath(__file__))


def relerr(x, y):
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    return float(np.linalg.norm(x - y) / max(np.linalg.norm(y), 1e-300))


def test_aux_constants_match_pages():
    """betas, eps, weight decay and peak lrs are the [GS] page's (cited fixture)."""
    with open(os.path.join(HERE, "golden", "page_constants.json")) as fh:
        fx = json.load(fh)
    assert tuple(fx["aux_adamw_betas"]["value"]) == AUX_BETAS
    assert fx["aux_adamw_eps"]["value"] == AUX_EPS
    assert fx["aux_adamw_weight_decay"]["value"] == AUX_WEIGHT_DECAY
    assert fx["aux_adamw_peak_lr"]["value"] == AUX_LR


HYPER = [
    dict(lr=AUX_LR["vector"], beta1=AUX_BETAS[0], beta2=AUX_BETAS[1], eps=AUX_EPS,
         weight_decay=AUX_WEIGHT_DECAY),
    dict(lr=AUX_LR["embedding"], beta1=AUX_BETAS[0], beta2=AUX_BETAS[1], eps=AUX_EPS,
         weight_decay=AUX_WEIGHT_DECAY),
    dict(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.01),
    dict(lr=1e-2, beta1=0.5, beta2=0.999, eps=1e-3, weight_decay=0.3),
]


@pytest.mark.parametrize("hp", HYPER)
@pytest.mark.parametrize("shape", [(37,), (12, 20), (3, 4, 5)])
def test_against_torch_optim_adamw(hp, shape):
    """torch.optim.AdamW (the routine [MX] section 5 hands the non-Muon
    parameters to), run in float64 on the CPU, follows the same trajectory
    over six steps: weights and both moments."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(41)
    p0 = rng.standard_normal(shape) * 0.02
    grads = [rng.standard_normal(shape) * 1e-3 * (k + 1) for k in range(6)]
    tp = torch.nn.Parameter(torch.tensor(p0, dtype=torch.float64))
    opt = torch.optim.AdamW([tp], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                            weight_decay=hp["weight_decay"], foreach=False)
    p, m, v = p0, np.zeros(shape), np.zeros(shape)
    for t, g in enumerate(grads, start=1):
        tp.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        p, m, v = adamw_step(p, g, m, v, step=t, **hp)
    st = opt.state[tp]
    assert relerr(tp.detach().numpy() - p0, p - p0) < 1e-12
    assert relerr(st["exp_avg"].numpy(), m) < 1e-12
    assert relerr(st["exp_avg_sq"].numpy(), v) < 1e-12


@pytest.mark.parametrize("hp", HYPER)
def test_first_step_closed_form(hp):
    """From zero moments, step 1: m^ = g and v^ = g^2 exactly, so the update
    is lr g / (|g| + eps) on top of the decay (1 - lr wd) p."""
    rng = np.random.default_rng(42)
    p = rng.standard_normal(200) * 0.02
    g = rng.standard_normal(200) * 1e-3
    g[:5] = [0.0, -0.0, 1e-30, -1e-30, 5.0]
    pn, mn, vn = adamw_step(p, g, np.zeros(200), np.zeros(200), step=1, **hp)
    expect = (1 - hp["lr"] * hp["weight_decay"]) * p - hp["lr"] * g / (np.abs(g) + hp["eps"])
    assert np.max(np.abs(pn - expect)) <= 1e-15 * np.max(np.abs(p) + hp["lr"])
    assert np.array_equal(mn, (1 - hp["beta1"]) * g)


@pytest.mark.parametrize("hp", HYPER)
def test_constant_gradient_closed_form(hp):
    """A gradient held constant for T steps: the bias corrections make
    m^ = g and v^ = g^2 at every step, so each step applies the same update u
    and p_T = d^T p_0 - u (1 - d^T) / (1 - d) with d = 1 - lr wd."""
    rng = np.random.default_rng(43)
    p0 = rng.standard_normal(64) * 0.02
    g = rng.standard_normal(64) * 1e-3
    p, m, v = p0, np.zeros(64), np.zeros(64)
    T = 9
    for t in range(1, T + 1):
        p, m, v = adamw_step(p, g, m, v, step=t, **hp)
    d = 1 - hp["lr"] * hp["weight_decay"]
    u = hp["lr"] * g / (np.abs(g) + hp["eps"])
    expect = d ** T * p0 - u * (1 - d ** T) / (1 - d)
    assert relerr(p, expect) < 1e-12


def test_moments_are_weighted_sums():
    """m_T = (1-b1) sum_k b1^(T-k) g_k and v_T = (1-b2) sum_k b2^(T-k) g_k^2."""
    rng = np.random.default_rng(44)
    b1, b2 = AUX_BETAS
    grads = [rng.standard_normal(50) for _ in range(7)]
    p, m, v = np.zeros(50), np.zeros(50), np.zeros(50)
    for t, g in enumerate(grads, start=1):
        p, m, v = adamw_step(p, g, m, v, lr=1e-3, step=t)
    T = len(grads)
    m_ref = (1 - b1) * sum(b1 ** (T - k) * g for k, g in enumerate(grads, start=1))
    v_ref = (1 - b2) * sum(b2 ** (T - k) * g * g for k, g in enumerate(grads, start=1))
    assert relerr(m, m_ref) < 1e-14
    assert relerr(v, v_ref) < 1e-14


def test_zero_gradient_and_state():
    """g = m = v = 0: the Adam term is 0/(0+eps) = 0; only the decay acts."""
    p = np.linspace(-1, 1, 33)
    pn, mn, vn = adamw_step(p, np.zeros(33), np.zeros(33), np.zeros(33), lr=0.7, step=3)
    assert np.array_equal(pn, p - 0.7 * AUX_WEIGHT_DECAY * p)
    assert not mn.any() and not vn.any()


def test_gradient_scale_invariance_without_eps():
    """With eps = 0 AdamW is invariant to a positive rescale of every gradient."""
    rng = np.random.default_rng(45)
    p0 = rng.standard_normal(40)
    grads = [rng.standard_normal(40) for _ in range(4)]
    out = []
    for k in (1.0, 1e-4):
        p, m, v = p0, np.zeros(40), np.zeros(40)
        for t, g in enumerate(grads, start=1):
            p, m, v = adamw_step(p, k * g, m, v, lr=0.01, eps=0.0, step=t)
        out.append(p)
    assert relerr(out[1] - p0, out[0] - p0) < 1e-13


def test_rejects_bad_step_and_shapes():
    z = np.zeros(4)
    with pytest.raises(ValueError):
        adamw_step(z, z, z, z, lr=0.1, step=0)
    with pytest.raises(ValueError):
        adamw_step(z, np.zeros(5), z, z, lr=0.1, step=1)
