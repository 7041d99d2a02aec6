"""Parity of the HIP Muon step with the fp64 oracle, through the C ABI.

Small cases are compared element by element over whole matrices (ragged
shapes spanning several tiles); the full-size workloads run in the launch
configuration the benchmark times (one grouped launch sequence over the whole
model) and are compared on sampled matrices the oracle computes one by one.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from muon_step_03_amd import (MuonError, MuonStep, muon_step, muon_step_batched,
                              muon_step_grouped, stacked_group)
from muon_step_03_amd import workloads as wl
from _parity import (HP, TOL_BF16, TOL_F32, TOL_M, bf16_round, check_against_oracle,
                     check_bf16_elementwise, check_muongs_invariants, f64, oracle_step, relF)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def inputs(rows, cols, dtype, seed, m_std=0.0, g_std=1e-3):
    W = wl.random_matrix(rows, cols, 0.02, seed, dtype, DEV)
    G = wl.random_matrix(rows, cols, g_std, seed + 1, dtype, DEV)
    if m_std:
        M = wl.random_matrix(rows, cols, m_std, seed + 2, torch.float32, DEV)
    else:
        M = torch.zeros(rows, cols, dtype=torch.float32, device=DEV)
    return W, G, M


def gpu_step(W, G, M, stats=True, **kw):
    W1, M1 = W.clone(), M.clone()
    st = torch.zeros(5, dtype=torch.float32, device=DEV) if stats else None
    hp = dict(HP)
    hp.update(kw)
    muon_step(W1, G, M1, stats=st, **hp)
    torch.cuda.synchronize()
    return W1, M1, st


# ------------------------------------------------ the fp32 256x512 workload
@pytest.mark.parametrize("variant,wd", [("muon", 0.1), ("muongs", 0.1), ("muongs", 0.0)])
def test_fp32_256x512(variant, wd):
    w = wl.WORKLOADS["fp32_256x512"]
    W = wl.make_weights(w, DEV)[0][0]
    G = wl.make_grads(w, 0, DEV)[0][0]
    M = wl.make_momentum(w, DEV)[0][0]
    W1, M1, st = gpu_step(W, G, M, variant=variant, weight_decay=wd)
    e, _, ost = check_against_oracle(W, G, M, W1, M1, variant=variant, stats=st, weight_decay=wd)
    print(f"fp32 256x512 {variant} wd={wd}: relF(dW) = {e:.2e}")
    if variant == "muongs":
        # ||O~|| <= sqrt(p) on these inputs (asserted inside)
        check_muongs_invariants(W, W1, 0.02, wd, cos_tol=1e-6, r2_tol=1e-6)


# -------------------------------------------- ragged shapes, whole matrices
F32_SHAPES = [(100, 300), (300, 100), (37, 5), (5, 37), (1, 1), (1, 70), (70, 1), (65, 129),
              (129, 65), (200, 200)]
BF16_SHAPES = [(200, 300), (300, 200), (257, 129), (129, 257), (1, 300), (300, 1), (64, 1000),
               (1000, 64), (384, 384), (130, 130)]


@pytest.mark.parametrize("shape", F32_SHAPES)
@pytest.mark.parametrize("variant", ["muon", "muongs"])
def test_fp32_ragged(shape, variant):
    W, G, M = inputs(*shape, torch.float32, seed=hash(shape) % 10000, m_std=1e-3)
    W1, M1, st = gpu_step(W, G, M, variant=variant)
    check_against_oracle(W, G, M, W1, M1, variant=variant, stats=st)


@pytest.mark.parametrize("shape", BF16_SHAPES)
@pytest.mark.parametrize("variant", ["muon", "muongs"])
def test_bf16_ragged(shape, variant):
    W, G, M = inputs(*shape, torch.bfloat16, seed=hash(shape) % 10000, m_std=1e-3)
    W1, M1, st = gpu_step(W, G, M, variant=variant)
    e, _, _ = check_against_oracle(W, G, M, W1, M1, variant=variant, stats=st)
    print(f"bf16 {shape} {variant}: relF(dW) = {e:.2e}")


# 256x256 tiles: matrices whose short side is at least 512 and whose padded
# sides are multiples of 256, in a launch holding at least 4 (symmetric
# products) and 8 (update) such tiles per CU.  Here 110 matrices of
# 1024x1100 (10 symmetric and 20 update tiles each, ragged long side) next
# to a group of 1152x1200, whose padded short side keeps the 128-wide tiles:
# the Gram and the update then run as two launches per iteration, read off
# the library's launch count; the polynomial of a short side below 2048
# takes the 128-wide tiles in both groups (one launch).
@pytest.mark.parametrize("variant,stats", [("muon", True), ("muongs", True), ("muon", False)])
def test_bf16_large_tiles(variant, stats):
    import ctypes
    from muon_step_03_amd import _lib
    shapes = [(110, 1024, 1100), (3, 1152, 1200)]
    Ws = [wl.random_matrix(c * r, k, 0.02, 900 + i, torch.bfloat16, DEV).view(c, r, k)
          for i, (c, r, k) in enumerate(shapes)]
    Gs = [wl.random_matrix(c * r, k, 1e-3, 910 + i, torch.bfloat16, DEV).view(c, r, k)
          for i, (c, r, k) in enumerate(shapes)]
    Ms = [wl.random_matrix(c * r, k, 1e-3, 920 + i, torch.float32, DEV).view(c, r, k)
          for i, (c, r, k) in enumerate(shapes)]
    picks = [(0, 0), (0, 57), (0, 109), (1, 2)]
    before = {pk: (Ws[pk[0]][pk[1]].clone(), Ms[pk[0]][pk[1]].clone()) for pk in picks}
    st = torch.zeros(113 * 5, device=DEV) if stats else None
    L = _lib.lib()
    n = _lib.MUON_NUM_PHASES
    ms, cnt = (ctypes.c_double * n)(), (ctypes.c_int64 * n)()
    assert L.muon_profile_read(ms, cnt, n) == 0      # drop earlier records
    ms, cnt = (ctypes.c_double * n)(), (ctypes.c_int64 * n)()
    L.muon_profile_enable(1)
    muon_step_grouped([stacked_group(W, G, M) for W, G, M in zip(Ws, Gs, Ms)], torch.bfloat16,
                      variant=variant, stats=st, **HP)
    torch.cuda.synchronize()
    L.muon_profile_enable(0)
    assert L.muon_profile_read(ms, cnt, n) == 0
    names = [L.muon_phase_name(i).decode() for i in range(n)]
    launches = {names[i]: cnt[i] for i in range(n)}
    assert launches["gram"] == 10 and launches["poly"] == 5, launches
    assert launches["update"] + launches["update_tail"] == 10, launches
    for gi, i in picks:
        W0, M0 = before[(gi, i)]
        s5 = st[(110 * gi + i) * 5:(110 * gi + i + 1) * 5] if stats else None
        e, _, _ = check_against_oracle(W0, Gs[gi][i], M0, Ws[gi][i], Ms[gi][i], variant=variant,
                                       stats=s5)
        print(f"bf16 {shapes[gi][1:]} #{i} {variant} stats={stats}: relF(dW) = {e:.2e}")


# Short sides padded to 512 take the 512x128 update tiles (one tile spans the
# short side; the long side is padded to a multiple of 128): ragged short and
# long sides, wide and tall, with the step applied by the last update (no
# statistics) and by the separate tail (MuonGS with statistics), in a grouped
# call like the MoE experts'.
SHORT512 = [(3, 400, 1000), (2, 1000, 400), (2, 450, 777), (2, 777, 450), (2, 512, 512),
            (3, 500, 1408), (2, 1408, 512)]


@pytest.mark.parametrize("variant,with_stats", [("muon", False), ("muongs", True)])
def test_bf16_short_side_512(variant, with_stats):
    Ws = [wl.random_matrix(c * r, k, 0.02, 1100 + i, torch.bfloat16, DEV).view(c, r, k)
          for i, (c, r, k) in enumerate(SHORT512)]
    Gs = [wl.random_matrix(c * r, k, 1e-3, 1150 + i, torch.bfloat16, DEV).view(c, r, k)
          for i, (c, r, k) in enumerate(SHORT512)]
    Ms = [wl.random_matrix(c * r, k, 1e-3, 1200 + i, torch.float32, DEV).view(c, r, k)
          for i, (c, r, k) in enumerate(SHORT512)]
    W0 = [w.clone() for w in Ws]
    M0 = [m.clone() for m in Ms]
    n = sum(c for c, _, _ in SHORT512)
    st = torch.full((5 * n,), float("nan"), device=DEV) if with_stats else None
    muon_step_grouped([stacked_group(W, G, M) for W, G, M in zip(Ws, Gs, Ms)], torch.bfloat16,
                      variant=variant, stats=st, **HP)
    torch.cuda.synchronize()
    k = 0
    for gi, (c, r, cols) in enumerate(SHORT512):
        for i in range(c):
            s5 = st[5 * k:5 * k + 5] if with_stats else None
            e, _, _ = check_against_oracle(W0[gi][i], Gs[gi][i], M0[gi][i], Ws[gi][i], Ms[gi][i],
                                           variant=variant, stats=s5)
            if variant == "muongs":
                check_muongs_invariants(W0[gi][i], Ws[gi][i], 0.02, 0.1, cos_tol=1e-3,
                                        r2_tol=1e-3, ratio_max=1.01)
            k += 1
        print(f"{r}x{cols} {variant}: relF(dW) = {e:.2e}")


# Plain Muon without statistics: on the bf16 path the last Newton-Schulz
# update applies the step to W itself whenever the weight's row length is a
# multiple of 8 (the other shapes here take the separate tail).
# (An 8x8 square matrix is not among them: with p = 8 the smallest singular
# directions carry much of the update, the iteration multiplies
# perturbations there by up to a^5 = 487, and X0's bf16 storage alone then
# exceeds the 3e-2 bar on some inputs — 2 of 40 seeds in an fp64 emulation
# of the bf16 path.  16x16, 8x64 and 64x8 keep the smallest shapes covered.)
FUSED_SHAPES = [(256, 512), (512, 256), (200, 304), (304, 200), (1000, 64), (64, 1000),
                (257, 129), (129, 257), (16, 16), (8, 64), (64, 8), (384, 384)]


@pytest.mark.parametrize("shape", FUSED_SHAPES)
@pytest.mark.parametrize("ns", [1, 5])
def test_bf16_without_stats(shape, ns):
    """The step applied by the last update (no statistics) and the separate
    tail (statistics requested) on the same inputs, each against the oracle.
    The bar is the bf16 tolerance plus what rounding the exact W' to bf16
    costs on its own (relative to the update): one iteration leaves ||O||
    near 3.4 instead of near sqrt(p), and the update of a 16x16 matrix is a
    few bf16 spacings of W, so there the final rounding is a visible share of
    the error on both paths."""
    W, G, M = inputs(*shape, torch.bfloat16, seed=hash(shape) % 10000 + ns, m_std=1e-3)
    W1, M1, _ = gpu_step(W, G, M, stats=False, ns_steps=ns)
    W2, M2, st = gpu_step(W, G, M, stats=True, ns_steps=ns)
    assert torch.equal(M1, M2)
    e_f, _, _ = check_against_oracle(W, G, M, W1, M1, ns_steps=ns, rounding_floor=True)
    e_s, _, _ = check_against_oracle(W, G, M, W2, M2, ns_steps=ns, rounding_floor=True, stats=st)
    print(f"bf16 {shape} ns={ns}: relF(dW) fused {e_f:.2e}, separate tail {e_s:.2e}")


def test_fused_and_separate_tail_agree():
    """The same step with statistics (separate tail, O rounded to bf16 first)
    and without (step applied in the last update from fp32 O): both meet the
    bar, and they differ by no more than the bf16 rounding of O can move W'."""
    shape = (768, 3072)
    W, G, M = inputs(*shape, torch.bfloat16, seed=91, m_std=1e-3)
    Wf, Mf, _ = gpu_step(W, G, M, stats=False)
    Ws, Ms, st = gpu_step(W, G, M, stats=True)
    check_against_oracle(W, G, M, Wf, Mf)
    check_against_oracle(W, G, M, Ws, Ms, stats=st)
    assert torch.equal(Mf, Ms)
    step = 0.02 * 0.2 * math.sqrt(max(shape))
    O_bound = 2.0 ** -8 * 1.25 * step        # |O| <= ~1.2: half a bf16 ulp of O, scaled
    w_ulp = 2.0 ** -7 * np.maximum(np.abs(f64(Wf)), np.abs(f64(Ws)))
    assert np.all(np.abs(f64(Wf) - f64(Ws)) <= O_bound + w_ulp)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shape", [(96, 200), (200, 96), (128, 128)])
@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_muonh(dtype, shape, wd):
    """MuonH keeps ||W||_F: checked on the GPU output itself (bf16 rounding of
    W' moves the norm by far less than 1e-3), and the update against the oracle."""
    W, G, M = inputs(*shape, dtype, seed=77, m_std=1e-3)
    W1, M1, st = gpu_step(W, G, M, variant="muonh", weight_decay=wd)
    check_against_oracle(W, G, M, W1, M1, variant="muonh", stats=st, weight_decay=wd)
    n0, n1 = np.linalg.norm(f64(W)), np.linalg.norm(f64(W1))
    assert abs(n1 / n0 - 1) < (1e-6 if dtype == torch.float32 else 1e-3)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shape", [(256, 64), (64, 256), (130, 130)])
@pytest.mark.parametrize("variant", ["muon", "muongs", "muonh"])
def test_keller_scale(dtype, shape, variant):
    """Keller's factor max(1, rows/cols)^0.5 is 1 for wide matrices (Moonlight's
    would be 0.2*sqrt(256) = 3.2), so the bf16 update is 3x closer to a bf16
    weight's resolution: the bf16 check adds the exact W' rounding cost."""
    W, G, M = inputs(*shape, dtype, seed=78, m_std=1e-3)
    W1, M1, st = gpu_step(W, G, M, variant=variant, scale="keller")
    check_against_oracle(W, G, M, W1, M1, variant=variant, stats=st, scale="keller",
                         rounding_floor=True)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("ns", [0, 1, 2])
def test_few_ns_steps(dtype, ns):
    """ns_steps = 0 returns the normalised look-ahead itself.  Its norm is 1
    (not about sqrt(p)), so the bf16 update is below the resolution of a bf16
    weight: there W' is checked element by element against the exact W'
    rounded to bf16."""
    W, G, M = inputs(160, 96, dtype, seed=31 + ns, m_std=1e-3)
    W1, M1, st = gpu_step(W, G, M, ns_steps=ns)
    if dtype == torch.bfloat16 and ns == 0:
        Wr, Mr, _ = oracle_step(W, G, M, ns_steps=0)
        _, U = oracle.nesterov_momentum(f64(G), f64(M), 0.95)
        O = oracle.newton_schulz(U, *oracle.NS_COEFFICIENTS, 0)
        step = 0.02 * 0.2 * math.sqrt(max(W.shape))
        # X0 holds U rounded to bf16: up to 2^-9 relative per element, so
        # lr*s*2^-8*|O| bounds what it can move W' before the final rounding.
        check_bf16_elementwise(W1, Wr, slack=step * 2.0 ** -8 * np.abs(O))
        assert relF(f64(M1), Mr) <= 1e-6
    else:
        check_against_oracle(W, G, M, W1, M1, stats=st, ns_steps=ns)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_classical_coefficients_converge(dtype):
    """(15/8, -10/8, 3/8) with 30 steps: the step's update has RMS 0.2*lr."""
    W, G, M = inputs(128, 384, dtype, seed=41)
    coeffs = (15 / 8, -10 / 8, 3 / 8)
    W1, M1, st = gpu_step(W, G, M, ns_steps=30, ns_coefficients=coeffs, weight_decay=0.0)
    check_against_oracle(W, G, M, W1, M1, stats=st, ns_steps=30, ns_coefficients=coeffs,
                         weight_decay=0.0)
    rms = float(np.sqrt(np.mean((f64(W1) - f64(W)) ** 2))) / 0.02
    assert abs(rms - 0.2) < (1e-5 if dtype == torch.float32 else 1e-2)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shape", [(256, 512), (512, 256), (768, 768)])
def test_semi_orthogonal_gradient(dtype, shape):
    """G = Q semi-orthogonal, M = 0: W' = (1 - lr wd) W - lr s f^5(x0) Q with
    the scalar f^5 of the pages' quintic."""
    rows, cols = shape
    p = min(shape)
    gen = torch.Generator().manual_seed(5)
    A = torch.randn(max(shape), p, generator=gen, dtype=torch.float64)
    Q, _ = torch.linalg.qr(A)
    Q = (Q.T if rows < cols else Q).contiguous()
    G = Q.to(dtype).to(DEV)
    W = wl.random_matrix(rows, cols, 0.02, 6, dtype, DEV)
    M = torch.zeros(rows, cols, dtype=torch.float32, device=DEV)
    W1, M1, st = gpu_step(W, G, M)
    check_against_oracle(W, G, M, W1, M1, stats=st)
    q = f64(G)
    x = (1 + 0.95) * math.sqrt(1.0) / ((1 + 0.95) * float(np.linalg.norm(q)) + 1e-7)
    a, b, c = oracle.NS_COEFFICIENTS
    for _ in range(5):
        x = a * x + b * x ** 3 + c * x ** 5
    s = 0.2 * math.sqrt(max(shape))
    expect = (1 - 0.002) * f64(W) - 0.02 * s * x * q
    tol = TOL_F32 if dtype == torch.float32 else TOL_BF16
    assert relF(f64(W1) - f64(W), expect - f64(W)) <= tol


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("variant", ["muon", "muongs"])
def test_zero_gradient_and_momentum(dtype, variant):
    """G = M = 0: O = 0, W' = (1 - lr wd) W, M' = 0."""
    W = wl.random_matrix(96, 160, 0.02, 8, dtype, DEV)
    G = torch.zeros_like(W)
    M = torch.zeros(96, 160, dtype=torch.float32, device=DEV)
    W1, M1, st = gpu_step(W, G, M, variant=variant)
    decay = torch.tensor(1 - 0.02 * 0.1, dtype=torch.float32)
    expect = (W.float() * decay.to(DEV)).to(dtype)
    assert torch.equal(W1, expect)
    assert not M1.any()
    assert st[3].item() == 0.0


def test_nan_gradient_propagates():
    W, G, M = inputs(64, 128, torch.float32, seed=9)
    G[3, 7] = float("nan")
    W1, M1, st = gpu_step(W, G, M)
    assert math.isnan(st[0].item())
    assert torch.isnan(W1).all()
    assert torch.isnan(M1[3, 7]) and torch.isfinite(M1[0, 0])


# ----------------------------------------------------- bitwise properties
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_batched_equals_single_and_deterministic(dtype):
    shape = (192, 320)
    mats = [inputs(*shape, dtype, seed=100 + 3 * i, m_std=1e-3) for i in range(5)]
    singles = []
    for W, G, M in mats:
        W1, M1, _ = gpu_step(W, G, M, stats=False)
        singles.append((W1, M1))
    for rep in range(2):
        Ws = [W.clone() for W, _, _ in mats]
        Ms = [M.clone() for _, _, M in mats]
        muon_step_batched(Ws, [G for _, G, _ in mats], Ms, **HP)
        torch.cuda.synchronize()
        for (W1, M1), W2, M2 in zip(singles, Ws, Ms):
            assert torch.equal(W1, W2) and torch.equal(M1, M2)


def test_stacked_equals_tables():
    shape = (256, 640)
    W = torch.stack([wl.random_matrix(*shape, 0.02, 200 + i, torch.bfloat16, DEV) for i in range(4)])
    G = torch.stack([wl.random_matrix(*shape, 1e-3, 300 + i, torch.bfloat16, DEV) for i in range(4)])
    M = torch.stack([wl.random_matrix(*shape, 1e-3, 400 + i, torch.float32, DEV) for i in range(4)])
    Wa, Ma = W.clone(), M.clone()
    muon_step_grouped([stacked_group(Wa, G, Ma)], torch.bfloat16, **HP)
    Wb, Mb = W.clone(), M.clone()
    muon_step_batched(list(Wb), list(G), list(Mb), **HP)
    torch.cuda.synchronize()
    assert torch.equal(Wa, Wb) and torch.equal(Ma, Mb)


@pytest.mark.parametrize("dtype,shape", [(torch.float32, (160, 416)), (torch.bfloat16, (160, 416)),
                                         (torch.bfloat16, (512, 1408))])
def test_transpose_equivariance(dtype, shape):
    """The step of W^T is the transpose of W's, bit for bit (plain Muon): a
    tall matrix is iterated as its transpose, the per-element arithmetic of
    the head and the tail does not depend on the orientation, and ||U||_F is
    summed in fp64, so the different tiling of the two orientations does not
    move the norm's fp32 rounding."""
    W, G, M = inputs(*shape, dtype, seed=55, m_std=1e-3)
    W1, M1, _ = gpu_step(W, G, M)
    W2, M2, _ = gpu_step(W.T.contiguous(), G.T.contiguous(), M.T.contiguous())
    assert torch.equal(M2.T, M1)
    assert torch.equal(W2.T, W1), relF(f64(W2).T - f64(W), f64(W1) - f64(W))


@pytest.mark.parametrize("variant", ["muon", "muongs", "muonh", "normuon", "meqmuon"])
def test_workspace_contents_do_not_matter(variant):
    """The step must not read workspace it has not written: a zeroed and a
    NaN-filled workspace (0xFF bytes) give bitwise identical results on the
    full grouped GPT-160M launch.  Catches pipeline races that read an LDS
    stage before its load landed, or a tile left unwritten."""
    from muon_step_03_amd import workspace_bytes_grouped
    w = wl.WORKLOADS["gpt160m"]
    Gs = wl.make_grads(w, 0, DEV)
    outs = []
    for fill in (0x00, 0xFF):
        Ws, Ms = wl.make_weights(w, DEV), wl.make_momentum(w, DEV)
        groups = [stacked_group(Ws[i], Gs[i], Ms[i]) for i in range(len(w.groups))]
        ws = torch.full((workspace_bytes_grouped(groups, torch.bfloat16),), fill,
                        dtype=torch.uint8, device=DEV)
        muon_step_grouped(groups, torch.bfloat16, variant=variant, workspace=ws, **HP)
        torch.cuda.synchronize()
        outs.append((Ws, Ms))
    for (Wa, Ma), (Wb, Mb) in zip(zip(*outs[0]), zip(*outs[1])):
        assert torch.isfinite(Wa.float()).all()
        assert torch.equal(Wa, Wb) and torch.equal(Ma, Mb)


# ------------------------------------------- full-size workloads, sampled
def run_workload(w, step, Ws, Ms, variant, stats=None):
    Gs = wl.make_grads(w, step, DEV)
    groups = [stacked_group(Ws[i], Gs[i], Ms[i]) for i in range(len(w.groups))]
    W0 = [x.clone() for x in Ws]
    M0 = [x.clone() for x in Ms]
    muon_step_grouped(groups, wl.torch_dtype(w.dtype), variant=variant, stats=stats, **HP)
    torch.cuda.synchronize()
    return W0, Gs, M0


def sampled(w, per_group=2):
    """The first, a middle and the last matrix of every group (per_group >= 2),
    or the first and a middle one."""
    out = []
    for gi, g in enumerate(w.groups):
        idx = {0, g.count // 2} | ({g.count - 1} if per_group >= 2 else set())
        out += [(gi, i) for i in sorted(idx)]
    return out


def slice_boundary_matrices(w):
    """The matrices next to a boundary between the eight XCD slices of any
    Newton-Schulz launch of a grouped call over the workload.  Each launch
    gives XCD x the contiguous tiles [n x / 8, n (x + 1) / 8) of a group's
    n = count x tiles-per-matrix tiles; the tiles per matrix are those of the
    128-wide symmetric tiles ((p_pad/128)(p_pad/128 + 1)/2) and update tiles
    ((p_pad/128)(q_pad/256)), and, for matrices that may take them, of the
    256x256 ones, or of the 512x128 update tiles (q_pad/128 of them) when the
    padded short side is 512.  For every boundary b the matrices holding
    tiles b - 1 and b are returned (one matrix when b falls inside it)."""
    out = set()
    for gi, g in enumerate(w.groups):
        p, q = min(g.rows, g.cols), max(g.rows, g.cols)
        pp = -(-p // 128) * 128
        nt = pp // 128
        if pp == 512:
            qp = -(-q // 128) * 128
            per = {nt * (nt + 1) // 2, 3, qp // 128}
        else:
            qp = -(-q // 256) * 256
            per = {nt * (nt + 1) // 2, nt * (qp // 256)}
            if p >= 512 and pp % 256 == 0:
                nb = pp // 256
                per |= {nb * (nb + 1) // 2, nb * (qp // 256)}
        for tiles in per:
            n = g.count * tiles
            for x in range(1, 8):
                b = n * x // 8
                out |= {(gi, (b - 1) // tiles), (gi, b // tiles)}
    return sorted(k for k in out if 0 <= k[1] < w.groups[k[0]].count)


def graded_matrices(w):
    return sorted(set(sampled(w)) | set(slice_boundary_matrices(w)))


@pytest.mark.parametrize("variant,with_stats", [("muon", True), ("muongs", True), ("muon", False)])
def test_gpt160m_full_set(variant, with_stats):
    """The grouped launch the benchmark times (without statistics: the step
    is applied by the last update), and with per-matrix statistics; graded
    on the first, middle and last matrix of every group and on every matrix
    next to an XCD slice boundary of the launches."""
    w = wl.WORKLOADS["gpt160m"]
    Ws, Ms = wl.make_weights(w, DEV), wl.make_momentum(w, DEV)
    stats = torch.zeros(w.n_matrices * 5, device=DEV) if with_stats else None
    W0, Gs, M0 = run_workload(w, 0, Ws, Ms, variant, stats)
    base = np.cumsum([0] + [g.count for g in w.groups])
    picks = graded_matrices(w)
    worst = 0.0
    for gi, i in picks:
        st = stats[(base[gi] + i) * 5:(base[gi] + i + 1) * 5] if with_stats else None
        e, _, _ = check_against_oracle(W0[gi][i], Gs[gi][i], M0[gi][i], Ws[gi][i], Ms[gi][i],
                                       variant=variant, stats=st)
        worst = max(worst, e)
        if variant == "muongs":
            check_muongs_invariants(W0[gi][i], Ws[gi][i], 0.02, 0.1, cos_tol=1e-3, r2_tol=1e-3,
                                    ratio_max=1.01)
    print(f"gpt160m {variant}: {len(picks)} of {w.n_matrices} matrices graded, "
          f"worst relF(dW) = {worst:.2e}")


def test_gpt400m_consecutive_steps():
    """Ten consecutive Muon and MuonGS steps with a fresh gradient every step
    (the GPT-400M configuration).  Graded against the oracle from the GPU's
    own W_t, M_t (teacher forcing): step 0 on the first, middle and last
    matrix of every group and every matrix next to an XCD slice boundary,
    steps 4 and 9 on the first and a middle matrix of every group, with the
    MuonGS invariants on those matrices; every step leaves W and M finite.
    The free-running drift (the oracle's own ten steps in fp64 from the same
    start, against the GPU's ten) is reported, not graded."""
    w = wl.WORKLOADS["gpt400m"]
    drift_picks = sampled(w, per_group=1)
    for variant in ("muon", "muongs"):
        Ws, Ms = wl.make_weights(w, DEV), wl.make_momentum(w, DEV)
        free = {k: (f64(Ws[k[0]][k[1]]), f64(Ms[k[0]][k[1]])) for k in drift_picks}
        start = {k: v[0].copy() for k, v in free.items()}
        worst = 0.0
        for step in range(10):
            W0, Gs, M0 = run_workload(w, step, Ws, Ms, variant)
            assert all(bool(torch.isfinite(x).all()) for x in Ws + Ms), step
            for k in drift_picks:
                Wf, Mf, _ = oracle.muon_step(free[k][0], f64(Gs[k[0]][k[1]]), free[k][1],
                                             variant=variant, **HP)
                free[k] = (Wf, Mf)
            if step == 0:
                picks = graded_matrices(w)
            elif step in (4, 9):
                picks = sampled(w, per_group=1)
            else:
                continue
            for gi, i in picks:
                e, _, _ = check_against_oracle(W0[gi][i], Gs[gi][i], M0[gi][i], Ws[gi][i],
                                               Ms[gi][i], variant=variant)
                worst = max(worst, e)
                if variant == "muongs":
                    check_muongs_invariants(W0[gi][i], Ws[gi][i], 0.02, 0.1, cos_tol=1e-3,
                                            r2_tol=1e-3, ratio_max=1.01)
            print(f"gpt400m step {step} {variant}: {len(picks)} matrices graded, "
                  f"worst relF(dW) = {worst:.2e}", flush=True)
        for gi, i in drift_picks:
            w10, w0 = f64(Ws[gi][i]), start[(gi, i)]
            d = relF(w10 - w0, free[(gi, i)][0] - w0)
            print(f"gpt400m {variant} {w.groups[gi]} #{i}: free-running 10-step drift "
                  f"relF(W_10 - W_0) = {d:.2e} (reported, not graded)")


def test_moe_full_set():
    """The whole MoE-1B set (4288 matrices) in one grouped call, graded on the
    first, middle and last matrix of every group and every matrix next to an
    XCD slice boundary of its launches."""
    w = wl.WORKLOADS["moe1b"]
    Ws, Ms = wl.make_weights(w, DEV), wl.make_momentum(w, DEV)
    W0, Gs, M0 = run_workload(w, 0, Ws, Ms, "muon")
    picks = graded_matrices(w)
    worst = 0.0
    for gi, i in picks:
        e, _, _ = check_against_oracle(W0[gi][i], Gs[gi][i], M0[gi][i], Ws[gi][i], Ms[gi][i])
        worst = max(worst, e)
    print(f"moe1b: {len(picks)} of {w.n_matrices} matrices graded, worst relF(dW) = {worst:.2e}")


def test_stress_matrices_sampled():
    """The 2k-hidden MLP shapes (2048x5632 and its transpose) with heavy-tailed
    gradient rows, on 4 matrices of each orientation."""
    w = wl.WORKLOADS["stress2k"]
    small = wl.Workload("stress2k-4", w.index, w.dtype,
                        tuple(wl.Group(4, g.rows, g.cols) for g in w.groups),
                        heavy_tailed_rows=True)
    Ws, Ms = wl.make_weights(small, DEV), wl.make_momentum(small, DEV)
    W0, Gs, M0 = run_workload(small, 0, Ws, Ms, "muon")
    for gi, i in [(0, 0), (1, 3)]:
        e, _, _ = check_against_oracle(W0[gi][i], Gs[gi][i], M0[gi][i], Ws[gi][i], Ms[gi][i])
        print(f"stress {small.groups[gi]} #{i}: relF(dW) = {e:.2e}")


@pytest.mark.timeout(900)
def test_stress_full_size_chunked():
    """The whole 2k-hidden stress set (1024 matrices of 2048x5632 and 1024 of
    5632x2048, heavy-tailed gradient rows: 23.6 G elements, 189 GB of W, G
    and M) in the calls the benchmark times: its workspace would not fit
    beside the tensors, so the step runs as a few grouped calls over even
    chunks of both groups.  The first and last matrix of each shape, copied
    before the step, are checked against the oracle."""
    from muon_step_03_amd import stacked_chunks
    w = wl.WORKLOADS["stress2k"]
    torch.cuda.empty_cache()
    Ws, Gs, Ms = wl.make_weights(w, DEV), wl.make_grads(w, 0, DEV), wl.make_momentum(w, DEV)
    torch.cuda.empty_cache()
    picks = sampled(w)
    before = {(gi, i): (Ws[gi][i].clone(), Gs[gi][i].clone(), Ms[gi][i].clone()) for gi, i in picks}
    calls, ws_bytes = stacked_chunks(zip(Ws, Gs, Ms), torch.bfloat16, 32 << 30)
    assert len(calls) > 1
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    for groups in calls:
        muon_step_grouped(groups, torch.bfloat16, workspace=ws, **HP)
    torch.cuda.synchronize()
    print(f"stress2k: {len(calls)} calls of {calls[0][0].count} matrices per shape, "
          f"workspace {ws_bytes / 2**30:.1f} GiB", flush=True)
    after = {k: (Ws[k[0]][k[1]].cpu(), Ms[k[0]][k[1]].cpu()) for k in picks}
    del Ws, Gs, Ms, ws, calls
    torch.cuda.empty_cache()
    for gi, i in picks:
        W0, G, M0 = (x.cpu() for x in before[(gi, i)])
        e, _, _ = check_against_oracle(W0, G, M0, *after[(gi, i)])
        print(f"stress2k {w.groups[gi]} #{i}: relF(dW) = {e:.2e}", flush=True)


def test_optimizer_front_end_two_steps():
    shapes = [(256, 256), (256, 1024), (1024, 256), (256, 256)]
    params = [torch.nn.Parameter(wl.random_matrix(*s, 0.02, 500 + i, torch.bfloat16, DEV))
              for i, s in enumerate(shapes)]
    opt = MuonStep(params, lr=0.02, momentum=0.95, weight_decay=0.1, variant="muongs")
    for step in range(2):
        W0 = [p.detach().clone() for p in params]
        M0 = [m.clone() for m in opt.momentum_buffers]
        for i, p in enumerate(params):
            p.grad = wl.random_matrix(*shapes[i], 1e-3, 600 + 10 * step + i, torch.bfloat16, DEV)
        opt.step()
        torch.cuda.synchronize()
        for i, p in enumerate(params):
            check_against_oracle(W0[i], p.grad, M0[i], p.detach(), opt.momentum_buffers[i],
                                 variant="muongs")


def test_errors_surface_as_exceptions():
    W, G, M = inputs(64, 64, torch.float32, seed=1)
    with pytest.raises(ValueError):
        muon_step(W, G, M, workspace=torch.empty(16, dtype=torch.uint8, device=DEV))
    with pytest.raises(MuonError):
        muon_step(W, G, M, ns_steps=-1)
    with pytest.raises(ValueError):
        muon_step(W[0], G[0], M[0])


# ------------------------------------------------------ NorMuon and MeqMuon
def spreads(O):
    """std/mean of the row norms and of the column norms of O (fp64)."""
    rn, cn = np.linalg.norm(O, axis=1), np.linalg.norm(O, axis=0)
    return float(np.std(rn) / np.mean(rn)), float(np.std(cn) / np.mean(cn))


def recovered_o(W0, W1, shape, wd=0.1, lr=0.02):
    step = lr * 0.2 * math.sqrt(max(shape))
    return -(f64(W1) - (1 - lr * wd) * f64(W0)) / step


# the last two span several 256-row / 256-column chunks of the norm sums,
# ragged on both sides
NORM_SHAPES = [(96, 256), (256, 96), (200, 200), (130, 70), (70, 130), (300, 520), (600, 260)]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shape", NORM_SHAPES)
@pytest.mark.parametrize("heavy", ["row", "col"])
@pytest.mark.parametrize("variant", ["normuon", "meqmuon"])
def test_row_column_equalisation(dtype, shape, heavy, variant):
    """Against the oracle, with a dominant gradient row or column so that
    both MeqMuon directions occur.  The direction is a floating-point choice
    on spreads of a few percent, which the bf16 Newton-Schulz iteration moves
    by a few percent of themselves: the inputs (drawn on the host, fixed
    seeds) keep the two spreads at least 16 % apart, and the test asserts a
    10 % margin.  On the GPU's own output, the equalised direction's norms
    are equal and the other direction's are not."""
    seed = 7100 + 10 * NORM_SHAPES.index(shape) + (heavy == "col")
    W = wl.random_matrix(*shape, 0.02, seed, dtype)
    G = wl.random_matrix(*shape, 1e-3, seed + 1, torch.float32)
    if heavy == "row":
        G[shape[0] // 3] *= 20
    else:
        G[:, shape[1] // 3] *= 20
    G = G.to(dtype)
    M = wl.random_matrix(*shape, 1e-3, seed + 2, torch.float32)
    Wm, _, _ = oracle_step(W, G, M, variant="muon")
    O = recovered_o(W, torch.from_numpy(Wm), shape)
    sr, sc = spreads(O)
    assert abs(sr - sc) > 0.1 * max(sr, sc), (sr, sc)
    rows = variant == "normuon" or sr >= sc
    W, G, M = W.to(DEV), G.to(DEV), M.to(DEV)
    W1, M1, st = gpu_step(W, G, M, variant=variant)
    check_against_oracle(W, G, M, W1, M1, variant=variant, stats=st)
    On = recovered_o(W, W1, shape)
    n = np.linalg.norm(On, axis=1 if rows else 0)
    other = np.linalg.norm(On, axis=0 if rows else 1)
    # bf16: rounding W' to bf16 alone leaves the equalised norms 1.5e-3 to
    # 3.5e-3 apart on these inputs; the other direction's norms stay at
    # least 5 % apart
    tol = 1e-4 if dtype == torch.float32 else 1e-2
    dev = np.max(np.abs(n / np.mean(n) - 1))
    dev_other = np.max(np.abs(other / np.mean(other) - 1))
    print(f"{variant} {shape} heavy {heavy} {dtype}: spreads rows {sr:.4f} cols {sc:.4f}, "
          f"equalised {'rows' if rows else 'cols'} to {dev:.1e} (other {dev_other:.1e})")
    assert dev < tol
    assert dev_other > 3e-2


@pytest.mark.parametrize("variant", ["normuon", "meqmuon"])
def test_equalisation_gpt160m_grouped(variant):
    """The grouped launch over the 72 GPT-160M matrices (three shape groups).
    A nearly orthogonal square O has row and column spreads of about 1 % and
    close to each other, and the bf16 path's O (1.3e-2 from the oracle's)
    moves them by a few percent of themselves, so MeqMuon's choice can go
    either way between the bf16 path and fp64 (measured: spreads 0.0090 and
    0.0094, 4.6 % apart, decided differently).  The direction the GPU took is
    read off its output (the equalised side), must be the oracle's wherever
    the two spreads differ by more than 10 % (the margin the equalisation
    test keeps its inputs at), and the result is compared with the oracle's
    step for that direction."""
    w = wl.WORKLOADS["gpt160m"]
    Ws, Ms = wl.make_weights(w, DEV), wl.make_momentum(w, DEV)
    W0, Gs, M0 = run_workload(w, 0, Ws, Ms, variant)
    for gi, i in sampled(w):
        shape = (w.groups[gi].rows, w.groups[gi].cols)
        Wm, Mr, _ = oracle_step(W0[gi][i], Gs[gi][i], M0[gi][i], variant="muon")
        O = recovered_o(W0[gi][i], torch.from_numpy(Wm), shape)
        On = recovered_o(W0[gi][i], Ws[gi][i], shape)
        rn, cn = np.linalg.norm(On, axis=1), np.linalg.norm(On, axis=0)
        gpu_rows = np.std(rn) / np.mean(rn) <= np.std(cn) / np.mean(cn)
        sr, sc = spreads(O)
        if variant == "normuon" or abs(sr - sc) > 0.1 * max(sr, sc):
            assert gpu_rows == (variant == "normuon" or sr >= sc), (sr, sc)
        ref = oracle.normuon_rows(O) if gpu_rows else oracle.normuon_cols(O)
        step = 0.02 * 0.2 * math.sqrt(max(shape))
        Wr = (1 - 0.002) * f64(W0[gi][i]) - step * ref
        e = relF(f64(Ws[gi][i]) - f64(W0[gi][i]), Wr - f64(W0[gi][i]))
        assert e <= TOL_BF16, e
        assert relF(f64(Ms[gi][i]), Mr) <= TOL_M
        print(f"gpt160m {w.groups[gi]} #{i} {variant}: spreads {sr:.4f}/{sc:.4f}, "
              f"{'rows' if gpu_rows else 'cols'}, relF(dW) = {e:.2e}")


# ------------------------------------------- launch sequences and front end
# Eleven shape groups: more than the eight one launch sequence takes, so the
# call runs two sequences (the second with its own workspace regions and
# statistics offset); three row lengths are not multiples of 8, so without
# statistics those groups take the separate tail while the others have the
# step applied by their last update, in the same launches.
MANY_GROUPS = [(3, 64, 96), (2, 96, 64), (4, 128, 128), (2, 100, 130), (3, 130, 100),
               (2, 256, 72), (1, 72, 256), (2, 33, 257), (2, 200, 304), (1, 384, 128),
               (2, 48, 48)]


@pytest.mark.parametrize("variant,with_stats", [("muon", False), ("muon", True), ("muongs", True)])
def test_more_groups_than_one_launch_sequence(variant, with_stats):
    Ws = [wl.random_matrix(c * r, k, 0.02, 1300 + i, torch.bfloat16, DEV).view(c, r, k)
          for i, (c, r, k) in enumerate(MANY_GROUPS)]
    Gs = [wl.random_matrix(c * r, k, 1e-3, 1400 + i, torch.bfloat16, DEV).view(c, r, k)
          for i, (c, r, k) in enumerate(MANY_GROUPS)]
    Ms = [wl.random_matrix(c * r, k, 1e-3, 1500 + i, torch.float32, DEV).view(c, r, k)
          for i, (c, r, k) in enumerate(MANY_GROUPS)]
    W0 = [w.clone() for w in Ws]
    M0 = [m.clone() for m in Ms]
    total = sum(c for c, _, _ in MANY_GROUPS)
    st = torch.full((total * 5,), float("nan"), device=DEV) if with_stats else None
    muon_step_grouped([stacked_group(W, G, M) for W, G, M in zip(Ws, Gs, Ms)], torch.bfloat16,
                      variant=variant, stats=st, **HP)
    torch.cuda.synchronize()
    if with_stats:
        assert bool(torch.isfinite(st).all())   # every matrix's row written
    k = 0
    for gi, (c, r, cols) in enumerate(MANY_GROUPS):
        for i in range(c):
            s5 = st[5 * k:5 * k + 5] if with_stats else None
            e, _, _ = check_against_oracle(W0[gi][i], Gs[gi][i], M0[gi][i], Ws[gi][i], Ms[gi][i],
                                           variant=variant, stats=s5, rounding_floor=min(r, cols) < 64)
            k += 1
        print(f"group {gi} {r}x{cols} {variant} stats={with_stats}: relF(dW) = {e:.2e}")


def test_side_stream_matches_default_stream():
    """A call on a stream other than the current one, with allocations on the
    current stream made before anything is synchronised: the binding's own
    workspace must not be handed out again while the kernels still use it,
    so the result is bitwise that of the same call on the current stream."""
    w = wl.WORKLOADS["gpt160m"]
    Gs = wl.make_grads(w, 0, DEV)
    Wa, Ma = wl.make_weights(w, DEV), wl.make_momentum(w, DEV)
    Wb, Mb = [x.clone() for x in Wa], [x.clone() for x in Ma]
    torch.cuda.synchronize()
    muon_step_grouped([stacked_group(W, G, M) for W, G, M in zip(Wa, Gs, Ma)], torch.bfloat16,
                      **HP)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    muon_step_grouped([stacked_group(W, G, M) for W, G, M in zip(Wb, Gs, Mb)], torch.bfloat16,
                      stream=side, **HP)
    # the current stream allocates and writes while the side stream still runs
    junk = [torch.full((1 << 26,), 7, dtype=torch.uint8, device=DEV) for _ in range(8)]
    torch.cuda.synchronize()
    del junk
    for x, y in zip(Wa + Ma, Wb + Mb):
        assert torch.equal(x, y)


def test_checkpoint_split_run_is_bitwise():
    """The optimizer state is the momentum buffer alone (one per matrix): k
    steps, W and M copied to the host and restored into fresh tensors (and a
    fresh workspace), then the remaining steps, give bitwise the weights and
    momenta of an uninterrupted run."""
    shapes = [(4, 256, 640), (2, 640, 256), (3, 200, 130)]
    def fresh():
        return ([wl.random_matrix(c * r, k, 0.02, 1600 + i, torch.bfloat16, DEV).view(c, r, k)
                 for i, (c, r, k) in enumerate(shapes)],
                [torch.zeros(c, r, k, device=DEV) for c, r, k in shapes])
    def grads(step):
        return [wl.random_matrix(c * r, k, 1e-3, 1700 + 10 * step + i, torch.bfloat16, DEV)
                .view(c, r, k) for i, (c, r, k) in enumerate(shapes)]
    def run(Ws, Ms, steps):
        for t in steps:
            Gs = grads(t)
            muon_step_grouped([stacked_group(W, G, M) for W, G, M in zip(Ws, Gs, Ms)],
                              torch.bfloat16, **HP)
        torch.cuda.synchronize()
    Wa, Ma = fresh()
    run(Wa, Ma, range(6))
    Wb, Mb = fresh()
    run(Wb, Mb, range(3))
    saved = [(W.cpu(), M.cpu()) for W, M in zip(Wb, Mb)]
    del Wb, Mb
    torch.cuda.empty_cache()
    Wc = [W.to(DEV) for W, _ in saved]
    Mc = [M.to(DEV) for _, M in saved]
    run(Wc, Mc, range(3, 6))
    for x, y in zip(Wa + Ma, Wc + Mc):
        assert torch.equal(x, y)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("k", [0.125, 8.0])
def test_gradient_scale_invariance(dtype, k):
    """Scaling G and M by k > 0 scales U by k and leaves O, hence W', unchanged
    up to the 1e-7 in the normaliser; M' scales by k exactly.  With k a power
    of two every stored value scales exactly, and what remains is the
    rounding of 1/(k ||U|| + eps) against 1/(||U|| + eps) / k (about 1e-6
    relative here, where ||U|| = 0.53).  The iteration multiplies such a
    perturbation along the smallest singular directions by up to a^5 = 487,
    so in fp32 the two updates agree to the fp32 parity bar (measured
    2.6e-6).  In bf16 the same perturbation flips a few dozen roundings of
    the first A, and from there the two rounding sequences part: the two
    updates then differ about as much as either differs from the oracle
    (measured 1.07e-2), so in bf16 each is held to the oracle's bar on its
    own inputs and their difference to that bar."""
    W, G, M = inputs(192, 320, dtype, seed=61, m_std=1e-3)
    W1, M1, _ = gpu_step(W, G, M, stats=False)
    Gk = (G.float() * k).to(dtype)
    Wk, Mk, _ = gpu_step(W, Gk, M * k, stats=False)
    d1, dk = f64(W1) - f64(W), f64(Wk) - f64(W)
    e = relF(dk, d1)
    print(f"{dtype} k={k}: relF(dW_k, dW_1) = {e:.2e}")
    assert e <= (TOL_F32 if dtype == torch.float32 else TOL_BF16)
    assert torch.equal(Mk, M1 * k)
    check_against_oracle(W, Gk, M * k, Wk, Mk)


def test_optimizer_front_end_stats_and_rebinding():
    """MuonStep over two dtypes: each dtype's call writes its own rows of the
    statistics buffer (in stats_order), and a parameter whose .data is
    rebound between steps is updated in its new storage."""
    shapes = [((256, 512), torch.bfloat16), ((128, 96), torch.float32),
              ((512, 256), torch.bfloat16), ((128, 96), torch.float32)]
    params = [torch.nn.Parameter(wl.random_matrix(*s, 0.02, 1800 + i, dt, DEV))
              for i, (s, dt) in enumerate(shapes)]
    opt = MuonStep(params, variant="muongs")
    assert sorted(opt.stats_order) == list(range(len(params)))
    for step in range(2):
        if step == 1:
            params[2].data = params[2].data.clone()     # new storage
        W0 = [p.detach().clone() for p in params]
        M0 = [m.clone() for m in opt.momentum_buffers]
        for i, p in enumerate(params):
            p.grad = wl.random_matrix(*shapes[i][0], 1e-3, 1900 + 10 * step + i, shapes[i][1], DEV)
        stats = torch.full((len(params) * 5,), float("nan"), device=DEV)
        opt.step(stats=stats)
        torch.cuda.synchronize()
        for row, i in enumerate(opt.stats_order):
            check_against_oracle(W0[i], params[i].grad, M0[i], params[i].detach(),
                                 opt.momentum_buffers[i], variant="muongs",
                                 stats=stats[5 * row:5 * row + 5])


_TRACE_CHILD = r'''
import sys
import torch
sys.path.insert(0, sys.argv[1])
sys.path.insert(0, sys.argv[1] + "/tests")
from _parity import HP
from muon_step_03_amd import muon_step_grouped, stacked_group
from muon_step_03_amd import workloads as wl
shapes = [(3, 256, 640), (2, 640, 256)]
Ws = [wl.random_matrix(c * r, k, 0.02, 1900 + i, torch.bfloat16, "cuda").view(c, r, k)
      for i, (c, r, k) in enumerate(shapes)]
Gs = [wl.random_matrix(c * r, k, 1e-3, 1950 + i, torch.bfloat16, "cuda").view(c, r, k)
      for i, (c, r, k) in enumerate(shapes)]
Ms = [torch.zeros(c, r, k, device="cuda") for c, r, k in shapes]
for variant in ("muon", "muongs"):
    muon_step_grouped([stacked_group(W, G, M) for W, G, M in zip(Ws, Gs, Ms)], torch.bfloat16,
                      variant=variant, **HP)
torch.cuda.synchronize()
torch.save({"W": [W.cpu() for W in Ws], "M": [M.cpu() for M in Ms]}, sys.argv[2])
'''


def test_trace_ranges_leave_results_unchanged(tmp_path):
    """With MUON_TRACE=1 (roctx ranges around calls and launches; read once
    per process, so the traced run is a child process) a Muon and a MuonGS
    step give bitwise the weights and momenta of the same steps untraced."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    script = tmp_path / "child.py"
    script.write_text(_TRACE_CHILD)
    out = tmp_path / "traced.pt"
    env = dict(os.environ, MUON_TRACE="1")
    r = subprocess.run([sys.executable, str(script), root, str(out)], env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "no roctx library" not in r.stderr
    traced = torch.load(str(out), weights_only=True)
    shapes = [(3, 256, 640), (2, 640, 256)]
    Ws = [wl.random_matrix(c * r, k, 0.02, 1900 + i, torch.bfloat16, DEV).view(c, r, k)
          for i, (c, r, k) in enumerate(shapes)]
    Gs = [wl.random_matrix(c * r, k, 1e-3, 1950 + i, torch.bfloat16, DEV).view(c, r, k)
          for i, (c, r, k) in enumerate(shapes)]
    Ms = [torch.zeros(c, r, k, device=DEV) for c, r, k in shapes]
    for variant in ("muon", "muongs"):
        muon_step_grouped([stacked_group(W, G, M) for W, G, M in zip(Ws, Gs, Ms)],
                          torch.bfloat16, variant=variant, **HP)
    torch.cuda.synchronize()
    for x, y in zip(Ws + Ms, traced["W"] + traced["M"]):
        assert torch.equal(x.cpu(), y)
