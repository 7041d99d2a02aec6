"""fp64 CPU oracle for the Muon step.  Test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package; the HIP library never does.
"""
from .muon_oracle import (  # noqa: F401
    DEFAULT_LR, DEFAULT_MOMENTUM, DEFAULT_NS_STEPS, DEFAULT_WEIGHT_DECAY,
    NS_COEFFICIENTS, NS_EPS, RMS_MATCH, SCALE_KELLER, SCALE_MOONLIGHT, VARIANT_MEQMUON,
    VARIANT_MUON, VARIANT_MUONGS, VARIANT_MUONH, VARIANT_NORMUON, frobenius_inner,
    meqmuon_direction, muon_step, muongs_project, muonh_renormalise, nesterov_momentum,
    newton_schulz, normuon_cols, normuon_rows, update_scale,
)
from .adamw_oracle import (  # noqa: F401
    AUX_BETAS, AUX_EPS, AUX_LR, AUX_WEIGHT_DECAY, adamw_step,
)
