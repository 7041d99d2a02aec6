"""Muon optimizer step for MI355X (gfx950): HIP kernels behind a C ABI.

The HIP library (libmuon.so, built in-tree by ``muon_step_03_amd.build``) is
loaded on first use; without it every entry point raises.
"""
from .api import (  # noqa: F401
    MuonError, MuonStep, NS_COEFFICIENTS, muon_step, muon_step_batched, muon_step_grouped,
    pointer_table, stacked_group, table_group, workspace_bytes, workspace_bytes_grouped,
)
