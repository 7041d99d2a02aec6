"""Muon optimizer step (and the AdamW step of the hybrid optimizer) for
MI355X (gfx950): HIP kernels behind a C ABI.

The HIP library (libmuon.so, built in-tree by ``muon_step_03_amd.build``) is
loaded on first use; without it every entry point raises.
"""
from .api import (  # noqa: F401
    AUX_BETAS, AUX_EPS, AUX_LR, AUX_WEIGHT_DECAY, AdamWStep, HybridMuonAdamW, MuonError,
    MuonStep, NS_COEFFICIENTS, adamw_step, adamw_step_grouped, adamw_tensor, muon_step,
    muon_step_batched, muon_step_grouped, muon_step_grouped_noalloc, pointer_table,
    stacked_chunks, stacked_group, chunk_size, table_group, workspace_bytes,
    workspace_bytes_grouped,
)
