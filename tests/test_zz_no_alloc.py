"""muon_step_grouped_noalloc (the entry point for callers that cannot
allocate: its workspace is the library's static per-GPU array) against
muon_step_grouped with a caller-allocated workspace, through the C ABI.

Both run the same kernels on the same inputs, so the results must be
bitwise equal; two calls in a row, the second on a smaller input, show that
whatever the first call left in the shared array does not matter."""
import pytest
import torch

from muon_step_03_amd import (MuonError, _lib, muon_step_grouped, muon_step_grouped_noalloc,
                              stacked_group, workspace_bytes_grouped)
from muon_step_03_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"
HP = dict(lr=0.02, momentum=0.95, weight_decay=0.1, ns_steps=5)


def stacks(shapes, dtype, seed):
    Ws = [wl.random_matrix(c * r, k, 0.02, seed + i, dtype, DEV).view(c, r, k)
          for i, (c, r, k) in enumerate(shapes)]
    Gs = [wl.random_matrix(c * r, k, 1e-3, seed + 50 + i, dtype, DEV).view(c, r, k)
          for i, (c, r, k) in enumerate(shapes)]
    Ms = [wl.random_matrix(c * r, k, 1e-3, seed + 100 + i, torch.float32, DEV).view(c, r, k)
          for i, (c, r, k) in enumerate(shapes)]
    return Ws, Gs, Ms


def both_ways(shapes, dtype, seed, variant, with_stats):
    Ws, Gs, Ms = stacks(shapes, dtype, seed)
    n = sum(c for c, _, _ in shapes)
    groups_a = [stacked_group(W.clone(), G, M.clone()) for W, G, M in zip(Ws, Gs, Ms)]
    need = workspace_bytes_grouped(groups_a, dtype)
    assert 0 < need <= _lib.MUON_NOALLOC_WORKSPACE_BYTES
    outs = []
    for noalloc in (False, True):
        W1 = [W.clone() for W in Ws]
        M1 = [M.clone() for M in Ms]
        st = torch.full((5 * n,), float("nan"), device=DEV) if with_stats else None
        groups = [stacked_group(W, G, M) for W, G, M in zip(W1, Gs, M1)]
        if noalloc:
            muon_step_grouped_noalloc(groups, dtype, variant=variant, stats=st, **HP)
        else:
            muon_step_grouped(groups, dtype, variant=variant, stats=st, **HP)
        torch.cuda.synchronize()
        outs.append((W1, M1, st))
    (Wa, Ma, sa), (Wb, Mb, sb) = outs
    for x, y in zip(Wa + Ma, Wb + Mb):
        assert torch.equal(x, y)
    if with_stats:
        assert torch.equal(sa, sb) and bool(torch.isfinite(sb).all())
    assert not any(torch.equal(x, W) for x, W in zip(Wb, Ws))   # the step ran


@pytest.mark.parametrize("variant,with_stats", [("muon", False), ("muongs", True)])
def test_noalloc_matches_grouped_two_calls(variant, with_stats):
    # first call: 20 matrices in three groups (56.3 MiB of the 64 MiB array);
    # then two small calls on top of what the first left in it
    both_ways([(12, 512, 1408), (6, 768, 256), (2, 200, 130)], torch.bfloat16, 2100, variant,
              with_stats)
    both_ways([(2, 128, 384)], torch.bfloat16, 2200, variant, with_stats)
    both_ways([(1, 256, 512)], torch.float32, 2300, variant, with_stats)


def test_noalloc_rejects_more_than_its_workspace():
    shapes = [(8, 1024, 4096)]
    Ws, Gs, Ms = stacks(shapes, torch.bfloat16, 2400)
    W0 = Ws[0].clone()
    groups = [stacked_group(Ws[0], Gs[0], Ms[0])]
    assert workspace_bytes_grouped(groups, torch.bfloat16) > _lib.MUON_NOALLOC_WORKSPACE_BYTES
    with pytest.raises(MuonError) as ei:
        muon_step_grouped_noalloc(groups, torch.bfloat16, **HP)
    assert ei.value.status == _lib.MUON_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert torch.equal(Ws[0], W0)
