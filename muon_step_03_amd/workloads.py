"""Seeded synthetic inputs for the Muon step: shapes, value distributions, seeds.

This module holds no arithmetic of the method itself.  It only draws the
inputs (W, G, M) that both the HIP library and the fp64 oracle consume, so the
two sides see exactly the same numbers.

Shapes follow the model set-ups of the MuonGS summary page ("MuonGS:
Pretraining LLMs with Relaxed Weight-Norm Control", experiment paragraph):
GPT-160M (12 layers, hidden 768), GPT-400M (24 layers, hidden 1024) and a
32-layer MoE with hidden 512, 64 routed experts and 1 shared expert per layer.
Hidden-layer weights only: 4 attention projections and the MLP up/down
projections per layer (embeddings and head are not Muon parameters).

Distributions: W ~ N(0, 0.02^2), G ~ N(0, (1e-3)^2), M = 0.  The large-matrix
stress set draws each gradient row with its own standard deviation
1e-3 * exp(z), z ~ N(0, 1) (heavy-tailed rows).

Seeds: the generator for (workload w, step t, tensor kind k, shape group g) is
seeded with 1000*w + 100*g + 10*t + k, k = 0 for W and 1 for G, so every
group is reproducible on its own.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

F32 = "f32"
BF16 = "bf16"

W_STD = 0.02
G_STD = 1e-3


@dataclass(frozen=True)
class Group:
    """``count`` matrices of one shape, stored as one [count, rows, cols] stack."""
    count: int
    rows: int
    cols: int


@dataclass(frozen=True)
class Workload:
    name: str
    index: int                 # used in the seed
    dtype: str                 # dtype of W and G; the momentum M is always fp32
    groups: tuple              # tuple[Group, ...]
    heavy_tailed_rows: bool = False
    description: str = ""
    # Matrices per layer, for documentation only.
    layout: dict = field(default_factory=dict)

    @property
    def n_matrices(self) -> int:
        return sum(g.count for g in self.groups)

    @property
    def n_elements(self) -> int:
        return sum(g.count * g.rows * g.cols for g in self.groups)


def _layered(n_layers, per_layer):
    """Collapse a per-layer list of (rows, cols) into shape groups."""
    counts = {}
    for rc in per_layer:
        counts[rc] = counts.get(rc, 0) + n_layers
    return tuple(Group(c, r, k) for (r, k), c in counts.items())


WORKLOADS = {
    "fp32_256x512": Workload(
        "fp32_256x512", 1, F32, (Group(1, 256, 512),),
        description="single fp32 256x512 matrix"),
    "gpt160m": Workload(
        "gpt160m", 2, BF16,
        _layered(12, [(768, 768)] * 4 + [(768, 3072), (3072, 768)]),
        description="GPT-160M hidden set: 12 x {4x 768x768, 768x3072, 3072x768}"),
    "gpt400m": Workload(
        "gpt400m", 3, BF16,
        _layered(24, [(1024, 1024)] * 4 + [(1024, 4096), (4096, 1024)]),
        description="GPT-400M hidden set: 24 x {4x 1024x1024, 1024x4096, 4096x1024}"),
    "moe1b": Workload(
        "moe1b", 4, BF16,
        _layered(32, [(512, 512)] * 4 + [(512, 1408), (1408, 512)] * 65),
        description="MoE: 32 x {4x 512x512 attn, 65 experts x (512x1408 up, 1408x512 down)}"),
    "stress2k": Workload(
        "stress2k", 5, BF16,
        (Group(1024, 2048, 5632), Group(1024, 5632, 2048)),
        heavy_tailed_rows=True,
        description="2048 MLP matrices of a 2k-hidden model (1024 of each orientation), "
                    "heavy-tailed gradient rows"),
}


def torch_dtype(dtype: str):
    return {F32: torch.float32, BF16: torch.bfloat16}[dtype]


def seed_for(workload_index: int, group_index: int, step: int, kind: int) -> int:
    return 1000 * workload_index + 100 * group_index + 10 * step + kind


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def make_weights(wl: Workload, device="cpu", groups=None):
    """W stacks, one [count, rows, cols] tensor per group, N(0, 0.02^2)."""
    out = []
    for gi, grp in enumerate(wl.groups):
        if groups is not None and gi not in groups:
            out.append(None)
            continue
        gen = _gen(device, seed_for(wl.index, gi, 0, 0))
        w = torch.empty((grp.count, grp.rows, grp.cols), dtype=torch.float32, device=device)
        w.normal_(0.0, W_STD, generator=gen)
        out.append(w.to(torch_dtype(wl.dtype)))
        del w
    return out


def make_grads(wl: Workload, step: int = 0, device="cpu", groups=None):
    """G stacks for one step; heavy-tailed rows where the workload asks for them."""
    out = []
    for gi, grp in enumerate(wl.groups):
        if groups is not None and gi not in groups:
            out.append(None)
            continue
        gen = _gen(device, seed_for(wl.index, gi, step, 1))
        g = torch.empty((grp.count, grp.rows, grp.cols), dtype=torch.float32, device=device)
        g.normal_(0.0, 1.0, generator=gen)
        if wl.heavy_tailed_rows:
            z = torch.empty((grp.count, grp.rows, 1), dtype=torch.float32, device=device)
            z.normal_(0.0, 1.0, generator=gen)
            g.mul_(torch.exp(z).mul_(G_STD))
        else:
            g.mul_(G_STD)
        out.append(g.to(torch_dtype(wl.dtype)))
        del g
    return out


def make_momentum(wl: Workload, device="cpu", groups=None):
    """Momentum buffers start at zero (fp32)."""
    return [None if (groups is not None and gi not in groups) else
            torch.zeros((grp.count, grp.rows, grp.cols), dtype=torch.float32, device=device)
            for gi, grp in enumerate(wl.groups)]


def random_matrix(rows, cols, std, seed, dtype=torch.float32, device="cpu"):
    """One seeded Gaussian matrix (small test cases and ragged shapes)."""
    gen = _gen(device, seed)
    x = torch.empty((rows, cols), dtype=torch.float32, device=device)
    x.normal_(0.0, std, generator=gen)
    return x.to(dtype)


# ------------------------------------------------------- AdamW-side tensors
# The parameters the hybrid optimizer gives to AdamW: input embedding, output
# head (untied) and the 1-D gains, two per layer plus a final one.  The pages
# give no vocabulary size; 50304 (GPT-2's 50257 tokens padded to a multiple
# of 128, as NanoGPT-family models do) stands in.  Roles select the
# per-tensor learning rate (embedding / head / vector).
AUX_VOCAB = 50304


@dataclass(frozen=True)
class AuxTensor:
    role: str      # "embedding", "head" or "vector"
    shape: tuple


def _aux(hidden, n_layers):
    return ((AuxTensor("embedding", (AUX_VOCAB, hidden)), AuxTensor("head", (AUX_VOCAB, hidden)))
            + tuple(AuxTensor("vector", (hidden,)) for _ in range(2 * n_layers + 1)))


AUX_SETS = {
    "gpt160m": _aux(768, 12),
    "gpt400m": _aux(1024, 24),
    "moe1b": _aux(512, 32),
}


def aux_seed(workload_index: int, step: int, kind: int) -> int:
    """Seed of the generator that draws every AdamW-side tensor of one kind
    (0 parameters, 1 gradients), in table order."""
    return 1_000_000 + 1000 * workload_index + 10 * step + kind


def make_aux_params(name: str, device="cpu", dtype=BF16):
    """Embedding and head ~ N(0, 0.02^2); gains ~ 1 + N(0, 0.02^2)."""
    wl = WORKLOADS[name]
    gen = _gen(device, aux_seed(wl.index, 0, 0))
    out = []
    for t in AUX_SETS[name]:
        x = torch.empty(t.shape, dtype=torch.float32, device=device)
        x.normal_(0.0, W_STD, generator=gen)
        if t.role == "vector":
            x.add_(1.0)
        out.append(x.to(torch_dtype(dtype)))
    return out


def make_aux_grads(name: str, step: int = 0, device="cpu", dtype=BF16):
    """Gradients ~ N(0, (1e-3)^2)."""
    wl = WORKLOADS[name]
    gen = _gen(device, aux_seed(wl.index, step, 1))
    out = []
    for t in AUX_SETS[name]:
        x = torch.empty(t.shape, dtype=torch.float32, device=device)
        x.normal_(0.0, G_STD, generator=gen)
        out.append(x.to(torch_dtype(dtype)))
    return out


def make_aux_moments(name: str, device="cpu"):
    """First and second moments start at zero (float32, flattened)."""
    return [(torch.zeros(math.prod(t.shape), dtype=torch.float32, device=device),
             torch.zeros(math.prod(t.shape), dtype=torch.float32, device=device))
            for t in AUX_SETS[name]]
