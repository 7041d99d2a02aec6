"""Muon / MuonGS optimizer step: plain fp64 NumPy oracle.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
helper with the HIP library and imports nothing from it.

It is deliberately slow and literal: every step is written in the order and
notation of the pages it follows, in float64, with NumPy's ``@`` as the only
library primitive (no symmetric tricks, no blocking, no fusion).

Citation keys (the pages this follows; a section, code block or equation is
named after the key):

  [LS] "LLM Pretraining Loss Spike 진단과 처방: 배치 사이즈, Gradient
       Accumulation, 그리고 Muon 전환 판단" (juhoplayground.github.io), section
       "AdamW에서 Muon으로 갈아탈 것인가".
  [GS] "MuonGS: Pretraining LLMs with Relaxed Weight-Norm Control"
       (onedev.kr paper summary).
  [MS] "[논문 AI 리뷰] MUON IS SCALABLE FOR LLM TRAINING TECHNICAL REPORT"
       (blog.pieroot.xyz), section "2. Key Methods and Approach".
  [MX] "[Deep Learning] Muon — 행렬 업데이트를 직교화하는 옵티마이저"
       (codersblog.github.io).
  [ME] "행과 열을 함께 정규화하는 사전학습 옵티마이저 MeqMuon 공개"
       (ailog.hnlab.kr), section "핵심 내용".

Readings taken where the pages are silent (each is listed with its reason in
the design notes of the repository):

  * Momentum is the SGD form M' = mu*M + G ("before Newton-Schulz, Muon is
    just SGD-momentum", [LS]); Nesterov look-ahead U = G + mu*M' (the pages
    name Nesterov as the default but print no formula).
  * The Newton-Schulz iteration runs on the shorter side: a tall matrix
    (rows > cols) is transposed first and the result transposed back ([MX]
    section 2: a rectangular update becomes semi-orthogonal).
  * Update scale is Moonlight's 0.2*sqrt(max(A, B)) ([MS] eq. 4); weight decay
    is decoupled and uses the unscaled learning rate ([LS] Moonlight section,
    "AdamW식 weight decay"; [MX] section 3 step 5).
  * MuonGS projects O against the pre-decay W; if ||W||_F == 0 the projection
    is the identity.  Weight decay, when non-zero, is applied in every variant.

Parity status: every function here is pinned by the ``-m "not gpu"`` tests
(closed forms, invariants, library special cases), except the direction
MeqMuon chooses (``meqmuon_direction``): the page gives no rule, so that
choice is "parity unpinned" (the two normalisations it chooses between are
pinned).
"""
from __future__ import annotations

import numpy as np

# [LS] section "Muon head의 실체는 하이브리드 옵티마이저다", the Newton-Schulz
# snippet: the quintic coefficients as printed (a, b, c).
NS_COEFFICIENTS = (3.4445, -4.7750, 2.0315)
# Same snippet: the small constant added to the Frobenius norm before the
# first iterate is scaled by its reciprocal.
NS_EPS = 1e-7
# [LS] same section, the listed defaults: lr 0.02, momentum 0.95 (Nesterov),
# ns_steps 5.  Weight decay 0.1 is [MX] section 5's example.
DEFAULT_LR = 0.02
DEFAULT_MOMENTUM = 0.95
DEFAULT_NS_STEPS = 5
DEFAULT_WEIGHT_DECAY = 0.1
# [MS] eq. 4 (and [LS] Moonlight section): the constant that matches AdamW's
# update RMS.
RMS_MATCH = 0.2

VARIANT_MUON = "muon"
VARIANT_MUONGS = "muongs"
VARIANT_MUONH = "muonh"
VARIANT_NORMUON = "normuon"
VARIANT_MEQMUON = "meqmuon"
SCALE_MOONLIGHT = "moonlight"
SCALE_KELLER = "keller"


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def frobenius_inner(X, Y) -> float:
    """<X, Y>_F = sum_ij X_ij Y_ij  ([GS] "전제와 한계": the <W_t, O_t>_F term)."""
    return float(np.sum(_f64(X) * _f64(Y)))


def nesterov_momentum(G, M, momentum):
    """Momentum accumulation, then the Nesterov look-ahead.

    [MX] section 3, step 2 (accumulate the previous state with the current
    gradient; Nesterov by default) and [LS] "Muon head" section (SGD-momentum,
    momentum 0.95, nesterov True):

        M' = mu * M + G          (SGD-momentum buffer)
        U  = G + mu * M'         (Nesterov look-ahead; the matrix handed to NS)

    Returns (M', U).
    """
    G = _f64(G)
    M = _f64(M)
    M_new = momentum * M + G
    U = G + momentum * M_new
    return M_new, U


def newton_schulz(U, a, b, c, steps, eps=NS_EPS):
    """Approximate the orthogonal polar factor (U U^T)^{-1/2} U.

    [MS] section 2: the iteration X_k = a X + b (X X^T) X + c (X X^T)^2 X,
    evaluated term by term as written there, with P = X X^T:

        Y = P X          the cubic term  (X X^T) X
        Z = P Y          the quintic term (X X^T)^2 X
        X <- a X + b Y + c Z

    The start X_0 is U divided by its Frobenius norm plus the small constant
    NS_EPS (the [LS] Newton-Schulz snippet normalises this way, with that
    stabiliser added to the norm).  The iteration runs on the shorter
    side ([MX] section 2): a tall U (rows > cols) is transposed before and
    after.  ``steps == 0`` returns the scaled X_0.
    """
    U = _f64(U)
    if U.ndim != 2:
        raise ValueError("Newton-Schulz needs a 2-D matrix")
    transposed = U.shape[0] > U.shape[1]
    X = U.T if transposed else U
    X = X / (np.linalg.norm(X, "fro") + eps)
    for _ in range(steps):
        P = X @ X.T
        Y = P @ X
        Z = P @ Y
        X = a * X + b * Y + c * Z
    return X.T if transposed else X


def muongs_project(W, O):
    """Gram-Schmidt radial projection of the update ([GS] "전제와 한계"):

        O~ = O - (<W, O>_F / r^2) W,   r = ||W||_F.

    With r == 0 there is no radial direction and O is returned unchanged.
    """
    W = _f64(W)
    O = _f64(O)
    r2 = frobenius_inner(W, W)
    if r2 == 0.0:
        return O.copy()
    return O - (frobenius_inner(W, O) / r2) * W


def update_scale(rows, cols, scale=SCALE_MOONLIGHT):
    """Shape factor of the update.

    Moonlight RMS matching, [MS] eq. 4: 0.2 * sqrt(max(A, B)).
    Keller's shape correction, the last line of the [LS] Newton-Schulz code
    block: max(1, A/B)^0.5 with A x B the weight's own shape.
    """
    if scale == SCALE_MOONLIGHT:
        return RMS_MATCH * float(np.sqrt(max(rows, cols)))
    if scale == SCALE_KELLER:
        return float(np.sqrt(max(1.0, rows / cols)))
    raise ValueError(f"unknown scale {scale!r}")


def muonh_renormalise(W, W_hat):
    """MuonH, the fixed-radius control the [GS] page compares against
    ("고정 반경 제약을 쓰는 MuonH"; fixed-norm control gives C_T = eta T / R):
    the stepped weight is put back on the sphere of the weight's norm before
    the step, R = ||W||_F:  W' = R * W_hat / ||W_hat||_F  (W_hat if zero)."""
    R = np.sqrt(frobenius_inner(W, W))
    n = np.sqrt(frobenius_inner(W_hat, W_hat))
    return W_hat * (R / n) if n > 0 else W_hat


def _equalise(O, axis):
    """Every row (axis=1: norms taken along each row) or column (axis=0) of
    O rescaled to the mean norm ||O||_F / sqrt(count); zero ones stay zero."""
    O = _f64(O)
    norms = np.sqrt(np.sum(O * O, axis=axis, keepdims=True))
    count = O.shape[1 - axis]
    target = np.sqrt(frobenius_inner(O, O) / count)
    scale = np.divide(target, norms, out=np.zeros_like(norms), where=norms > 0)
    return O * scale


def normuon_rows(O):
    """[ME] "핵심 내용": NorMuon normalises the size of the orthogonalised
    update row by row.  Reading (the page prints no formula): each row of O
    gets the mean row norm ||O||_F / sqrt(rows), so ||O||_F is kept."""
    return _equalise(O, axis=1)


def normuon_cols(O):
    """The same along columns (MeqMuon's other direction, [ME])."""
    return _equalise(O, axis=0)


def _spread(norms):
    """Coefficient of variation (std / mean) of a set of norms (0 if all 0)."""
    mean = float(np.mean(norms))
    return float(np.std(norms)) / mean if mean > 0 else 0.0


def meqmuon_direction(O):
    """[ME]: MeqMuon picks row or column normalisation per matrix by itself.
    Reading (no rule on the page; parity unpinned for this choice): the
    direction whose norms are more spread out (larger std / mean) is
    equalised; ties go to rows."""
    O = _f64(O)
    rn = np.sqrt(np.sum(O * O, axis=1))
    cn = np.sqrt(np.sum(O * O, axis=0))
    return "rows" if _spread(rn) >= _spread(cn) else "cols"


def muon_step(W, G, M, *, lr=DEFAULT_LR, momentum=DEFAULT_MOMENTUM,
              weight_decay=DEFAULT_WEIGHT_DECAY, ns_steps=DEFAULT_NS_STEPS,
              a=NS_COEFFICIENTS[0], b=NS_COEFFICIENTS[1], c=NS_COEFFICIENTS[2],
              variant=VARIANT_MUON, eps=NS_EPS, scale=SCALE_MOONLIGHT):
    """One Muon (or MuonGS) step on one 2-D hidden weight, in fp64.

    The order is [MX] section 3: momentum (Nesterov), magnitude normalisation,
    Newton-Schulz, then the shape scale and decoupled weight decay, then the
    parameter update.  MuonGS ([GS]) replaces O by its projection O~ before
    the update.

        M'  = mu M + G;  U = G + mu M'
        O   = NS_{a,b,c}^{ns_steps}(U)
        O~  = O - (<W,O>/||W||^2) W        (MuonGS only)
        O~  = rows (or columns) of O at equal norm   (NorMuon, MeqMuon)
        s   = 0.2 sqrt(max(A, B))           (or Keller's max(1, A/B)^0.5)
        W'  = (1 - lr*wd) W - lr * s * O~
        W'  = ||W|| W' / ||W'||             (MuonH only)

    Returns (W', M', stats) where stats holds the scalars the library can
    report: norm_U = ||U||_F, r2 = ||W||_F^2, dot_WO = <W,O>_F,
    norm2_O = ||O||_F^2 and norm2_Ot = ||O~||_F^2 (O~ = O for plain Muon).
    """
    W = _f64(W)
    G = _f64(G)
    M = _f64(M)
    if W.ndim != 2:
        # [MX] section 5: a non-2-D parameter is an error for Muon.
        raise ValueError("Muon updates 2-D weight matrices only")
    if G.shape != W.shape or M.shape != W.shape:
        raise ValueError("W, G and M must have the same shape")
    if variant not in (VARIANT_MUON, VARIANT_MUONGS, VARIANT_MUONH, VARIANT_NORMUON,
                       VARIANT_MEQMUON):
        raise ValueError(f"unknown variant {variant!r}")
    rows, cols = W.shape

    M_new, U = nesterov_momentum(G, M, momentum)
    O = newton_schulz(U, a, b, c, ns_steps, eps)
    if variant == VARIANT_MUONGS:
        O_t = muongs_project(W, O)
    elif variant == VARIANT_NORMUON:
        O_t = normuon_rows(O)
    elif variant == VARIANT_MEQMUON:
        O_t = normuon_rows(O) if meqmuon_direction(O) == "rows" else normuon_cols(O)
    else:
        O_t = O
    s = update_scale(rows, cols, scale)
    W_new = (1.0 - lr * weight_decay) * W - lr * s * O_t
    if variant == VARIANT_MUONH:
        W_new = muonh_renormalise(W, W_new)

    stats = {
        "norm_U": float(np.linalg.norm(U, "fro")),
        "r2": frobenius_inner(W, W),
        "dot_WO": frobenius_inner(W, O),
        "norm2_O": frobenius_inner(O, O),
        "norm2_Ot": frobenius_inner(O_t, O_t),
    }
    return W_new, M_new, stats
