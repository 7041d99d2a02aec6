"""Shared helpers for the GPU parity tests (not collected by pytest).

The HIP path and the oracle consume the very same inputs: tensors are drawn
once (seeded), copied to the host and promoted to float64 for the oracle.
"""
import math

import numpy as np
import torch

import oracle

# Tolerances on the relative Frobenius error of the update dW = W' - W, per
# matrix: 1e-5 for the float32 path, 3e-2 for the bf16 matrix-core path.  The
# momentum buffer is float32 elementwise arithmetic on both paths: 1e-6.
TOL_F32 = 1e-5
TOL_BF16 = 3e-2
TOL_M = 1e-6
# Per 64x64 tile of a bf16 update: a bound that a corrupted sub-tile (a
# zeroed or stale 32x32 block moves its 64x64 tile's relative error to 0.5
# or more) cannot meet, while the bf16 arithmetic's own error (about 1.2e-2
# per matrix, nearly uniform over the tiles) meets it with a wide margin.
TOL_BF16_TILE = 0.1
TILE = 64

HP = dict(lr=0.02, momentum=0.95, weight_decay=0.1, ns_steps=5)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def relF(x, y) -> float:
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    d = np.linalg.norm(y)
    return float(np.linalg.norm(x - y) / d) if d > 0 else float(np.linalg.norm(x))


def oracle_step(W, G, M, variant="muon", **hp):
    kw = dict(HP)
    kw.update(hp)
    a, b, c = kw.pop("ns_coefficients", oracle.NS_COEFFICIENTS)
    return oracle.muon_step(f64(W), f64(G), f64(M), a=a, b=b, c=c, variant=variant, **kw)


def step_factor(shape, scale="moonlight"):
    return oracle.update_scale(*shape, scale)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even)."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).double().numpy()


def tile_relF(d_gpu, d_ref, tile=TILE):
    """Largest relative Frobenius error over the tile x tile blocks (ragged
    at the edges) of two update matrices; blocks whose reference is exactly
    zero are compared on the absolute error."""
    rows, cols = d_ref.shape
    worst = 0.0
    for i in range(0, rows, tile):
        for j in range(0, cols, tile):
            r = d_ref[i:i + tile, j:j + tile]
            e = np.linalg.norm(d_gpu[i:i + tile, j:j + tile] - r)
            n = np.linalg.norm(r)
            worst = max(worst, e / n if n > 0 else e)
    return float(worst)


def check_against_oracle(W0, G, M0, W1, M1, variant="muon", tol=None, stats=None,
                         rounding_floor=False, tile_check=True, **hp):
    """W0/M0 inputs, W1/M1 GPU outputs.  Returns the relative errors.

    The error is the relative Frobenius error of the update dW = W' - W.  One
    degenerate case is measured differently: when the MuonGS projection
    removes (almost) all of O (O parallel to W, e.g. any 1 x 1 matrix), the
    reference update is the weight decay alone and the GPU's result is the
    cancellation of two terms of size lr*s*||O||; its error is then taken
    relative to that size, the scale at which float32 can resolve it.
    """
    tol = tol if tol is not None else (TOL_F32 if W0.dtype == torch.float32 else TOL_BF16)
    kw = dict(HP)
    kw.update(hp)
    Wr, Mr, st = oracle_step(W0, G, M0, variant=variant, **hp)
    w0 = f64(W0)
    dref = Wr - w0
    denom = np.linalg.norm(dref)
    if variant == "muongs" and st["norm2_Ot"] < 1e-6 * st["norm2_O"]:
        s_ = step_factor(W0.shape, kw.get("scale", "moonlight"))
        denom = max(denom, kw["lr"] * s_ * math.sqrt(st["norm2_O"]))
    e_dw = float(np.linalg.norm(f64(W1) - w0 - dref) / denom) if denom > 0 else \
        float(np.linalg.norm(f64(W1) - w0))
    if rounding_floor and W0.dtype == torch.bfloat16 and denom > 0:
        # Updates much smaller than a bf16 weight's resolution: allow, on top
        # of the tolerance, what rounding the exact W' to bf16 costs itself.
        tol += float(np.linalg.norm(bf16_round(Wr) - Wr) / denom)
    e_m = relF(f64(M1), Mr)
    assert e_dw <= tol, f"relF(dW) = {e_dw:.3e} > {tol:.1e}"
    assert e_m <= TOL_M, f"relF(M') = {e_m:.3e} > {TOL_M:.1e}"
    if (tile_check and W0.dtype == torch.bfloat16 and not rounding_floor and denom > 0
            and denom == np.linalg.norm(dref)):
        # every 64x64 tile on its own (not only the matrix as a whole)
        e_t = tile_relF(f64(W1) - w0, dref)
        assert e_t <= TOL_BF16_TILE, f"worst 64x64 tile relF(dW) = {e_t:.3e} > {TOL_BF16_TILE}"
    if stats is not None:
        s = stats.detach().cpu().double().numpy()
        o_tol = 1e-4 if W0.dtype == torch.float32 else 5e-2
        assert abs(s[0] - st["norm_U"]) <= 1e-5 * st["norm_U"]
        assert abs(s[1] - st["r2"]) <= 1e-5 * st["r2"]
        # <W,O>, ||O||^2 and ||O~||^2 are compared on the scale of ||O||^2.
        assert abs(s[3] - st["norm2_O"]) <= o_tol * st["norm2_O"]
        assert abs(s[4] - st["norm2_Ot"]) <= o_tol * st["norm2_O"]
        assert abs(s[2] - st["dot_WO"]) <= o_tol * math.sqrt(st["r2"] * st["norm2_O"])
    return e_dw, e_m, st


def check_bf16_elementwise(W1, Wr, slack):
    """Every bf16 output lies within one bf16 ulp of the exact result rounded
    to bf16, plus `slack` (per element: what the bf16 storage of the iterate
    may move the exact result)."""
    w1 = f64(W1)
    ref = bf16_round(Wr)
    ulp = np.abs(bf16_round(np.nextafter(np.abs(ref), np.inf) * 1.0040) - np.abs(ref))
    ulp = np.maximum(ulp, 2.0 ** -133)
    excess = np.abs(w1 - ref) - (ulp * 1.0001 + slack)
    assert np.all(excess <= 0), float(np.max(excess))


def recovered_update(W0, W1, lr, wd):
    """O~ implied by the GPU result: -(W' - (1 - lr wd) W) / (lr s)."""
    rows, cols = W0.shape
    s = 0.2 * math.sqrt(max(rows, cols))
    w0, w1 = f64(W0), f64(W1)
    return -(w1 - (1 - lr * wd) * w0) / (lr * s), s


def check_muongs_invariants(W0, W1, lr, wd, cos_tol, r2_tol, ratio_max=1.0):
    """MuonGS page, section "전제와 한계": the update is orthogonal to W,
    r'^2 = (1 - lr wd)^2 r^2 + (lr s)^2 ||O~||^2 and ||O~||_F <= sqrt(p) (on
    these inputs: the pages' coefficients can exceed it on flat spectra) —
    asserted on GPU output.  Returns ||O~|| / sqrt(p)."""
    Ot, s = recovered_update(W0, W1, lr, wd)
    w0, w1 = f64(W0), f64(W1)
    cos = float(np.sum(w0 * Ot) / math.sqrt(np.sum(w0 * w0) * np.sum(Ot * Ot)))
    assert abs(cos) <= cos_tol, f"cos(W, O~) = {cos:.2e}"
    r2n = (1 - lr * wd) ** 2 * np.sum(w0 * w0) + (lr * s) ** 2 * np.sum(Ot * Ot)
    assert abs(np.sum(w1 * w1) / r2n - 1) <= r2_tol
    p = min(W0.shape)
    ratio = float(np.sqrt(np.sum(Ot * Ot)) / math.sqrt(p))
    assert ratio <= ratio_max, f"||O~|| / sqrt(p) = {ratio:.4f} > {ratio_max}"
    return ratio
