"""AdamW for the parameters the hybrid optimizer keeps off Muon: plain fp64
NumPy oracle.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library and imports nothing from it.

What the pages fix (citation keys as in ``muon_oracle``):

  * [LS] section "Muon head의 실체는 하이브리드 옵티마이저다": Muon is for
    hidden 2-D weights only; the input embedding, the output layer and the
    internal gains and biases go to a standard method such as AdamW.
  * [MX] section 5: the non-Muon parameters are handed to
    ``torch.optim.AdamW`` (so AdamW in its decoupled-decay form).
  * [GS], the experiments paragraph of "전제와 한계": embeddings, output head
    and 1-D parameters use AdamW with betas (0.8, 0.95), eps 1e-10, weight
    decay 1e-3 and peak learning rates 0.7 / 0.004 / 0.015 respectively.

The pages name AdamW but print no update rule.  The reading taken is the
textbook decoupled AdamW with bias correction (the rule ``torch.optim.AdamW``
implements), at step t = 1, 2, ...:

    m' = beta1 m + (1 - beta1) g
    v' = beta2 v + (1 - beta2) g^2
    m^ = m' / (1 - beta1^t),   v^ = v' / (1 - beta2^t)
    p' = p - lr wd p - lr m^ / (sqrt(v^) + eps)

Parity status: pinned by the ``-m "not gpu"`` tests (``torch.optim.AdamW`` in
float64 as an independent routine, the first-step and constant-gradient
closed forms, the moment sums, the zero case); not "parity unpinned".
"""
from __future__ import annotations

import numpy as np

# [GS] experiments paragraph: betas, eps and weight decay of the auxiliary
# AdamW, and its peak learning rates for embedding / output head / 1-D params.
AUX_BETAS = (0.8, 0.95)
AUX_EPS = 1e-10
AUX_WEIGHT_DECAY = 1e-3
AUX_LR = {"embedding": 0.7, "head": 0.004, "vector": 0.015}


def adamw_step(p, g, m, v, *, lr, beta1=AUX_BETAS[0], beta2=AUX_BETAS[1],
               eps=AUX_EPS, weight_decay=AUX_WEIGHT_DECAY, step):
    """One decoupled AdamW step on one parameter tensor of any shape, in fp64.

    ``step`` is the 1-based count of this update (it sets the bias
    corrections).  Returns (p', m', v').
    """
    if int(step) != step or step < 1:
        raise ValueError("step counts updates from 1")
    p = np.asarray(p, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if not (p.shape == g.shape == m.shape == v.shape):
        raise ValueError("p, g, m and v must have the same shape")
    m_new = beta1 * m + (1.0 - beta1) * g
    v_new = beta2 * v + (1.0 - beta2) * (g * g)
    m_hat = m_new / (1.0 - beta1 ** step)
    v_hat = v_new / (1.0 - beta2 ** step)
    p_new = p - lr * weight_decay * p - lr * m_hat / (np.sqrt(v_hat) + eps)
    return p_new, m_new, v_new
