"""GPU parity of the AdamW entry points against the fp64 oracle, through the C ABI.

Per element: the float32 moments within a few float32 roundings of the exact
values; the parameter within the float32 arithmetic's error of the exact
value, plus half a bf16 spacing when the parameter is stored in bf16 (the
final round-to-nearest-even).  The relative Frobenius error of the update
P' - P is also held to the fp32 / bf16 bars of the Muon step.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from muon_step_03_amd import (AUX_BETAS, AUX_EPS, AUX_LR, AUX_WEIGHT_DECAY, AdamWStep,
                              HybridMuonAdamW, adamw_step, adamw_step_grouped, adamw_tensor)
from muon_step_03_amd import workloads as wl

from _parity import f64, relF

pytestmark = pytest.mark.gpu
DEV = "cuda"
U32 = 2.0 ** -24


def bf16_spacing(x):
    """Spacing of bf16 numbers at |x| (the larger binade at a boundary)."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def check_adamw(P0, G, m0, v0, P1, m1, v1, *, lr, step, betas=AUX_BETAS, eps=AUX_EPS,
                weight_decay=AUX_WEIGHT_DECAY):
    b1, b2 = betas
    p0, g, mm, vv = f64(P0).ravel(), f64(G).ravel(), f64(m0).ravel(), f64(v0).ravel()
    Pr, mr, vr = oracle.adamw_step(p0, g, mm, vv, lr=lr, beta1=b1, beta2=b2, eps=eps,
                                   weight_decay=weight_decay, step=step)
    gm1, gv1, gp1 = f64(m1).ravel(), f64(v1).ravel(), f64(P1).ravel()
    # moments: two products and a sum in float32
    assert np.all(np.abs(gm1 - mr) <= 4 * U32 * (b1 * np.abs(mm) + (1 - b1) * np.abs(g)) + 1e-45)
    assert np.all(np.abs(gv1 - vr) <= 6 * U32 * (b2 * vv + (1 - b2) * g * g) + 1e-45)
    # parameter: decay term and Adam term, each a few roundings (the Adam
    # term's sqrt, scale, add and divide), then the final rounding.  m' can
    # nearly cancel (b1 m against (1 - b1) g); its absolute rounding error
    # then reaches the Adam term scaled by lr / ((1 - b1^t) denom).
    decay = 1 - lr * weight_decay
    adam = Pr - decay * p0
    dm = 4 * U32 * (b1 * np.abs(mm) + (1 - b1) * np.abs(g))
    denom = np.sqrt(vr / (1 - b2 ** step)) + eps
    slack = (4 * U32 * np.abs(decay * p0) + 16 * U32 * np.abs(adam)
             + lr / (1 - b1 ** step) * dm / denom)
    if P1.dtype == torch.bfloat16:
        slack = slack + 0.5 * bf16_spacing(np.maximum(np.abs(Pr), np.abs(gp1)))
    excess = np.abs(gp1 - Pr) - slack
    assert np.all(excess <= 0), float(np.max(excess))
    if np.any(Pr != p0):
        if P1.dtype == torch.float32:
            assert relF(gp1 - p0, Pr - p0) <= 1e-5
        else:
            # a small update (lr 3e-4 on weights of 0.02) is partly below a
            # bf16 weight's spacing: the bar adds what storing the exact
            # result in bf16 costs.
            floor = relF(f64(torch.from_numpy(Pr).to(torch.bfloat16)) - p0, Pr - p0)
            assert relF(gp1 - p0, Pr - p0) <= 3e-2 + floor
    return Pr, mr, vr


def state(n, seed, step):
    """Moments as after step-1 updates: m ~ N(0, (1e-3)^2); v ~ (1e-3 z)^2."""
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    if step == 1:
        return (torch.zeros(n, dtype=torch.float32, device=DEV),
                torch.zeros(n, dtype=torch.float32, device=DEV))
    m = torch.randn(n, generator=gen, device=DEV) * 1e-3
    v = (torch.randn(n, generator=gen, device=DEV) * 1e-3) ** 2
    return m, v


def tensors(n, dtype, seed):
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    P = (torch.randn(n, generator=gen, device=DEV) * 0.02).to(dtype)
    G = (torch.randn(n, generator=gen, device=DEV) * 1e-3).to(dtype)
    return P, G


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("n", [1, 3, 4095, 4096, 4097, 3 * 4096 + 5, 100_003])
@pytest.mark.parametrize("step", [1, 7])
def test_single_tensor(dtype, n, step):
    """Sizes below, at and past one block's chunk (4096 elements) and ragged
    tails; step 1 from zero moments and a later step from non-zero ones."""
    P, G = tensors(n, dtype, seed=n)
    m, v = state(n, seed=n + 1, step=step)
    P0, m0, v0 = P.clone(), m.clone(), v.clone()
    adamw_step(P, G, m, v, lr=AUX_LR["vector"], step=step)
    torch.cuda.synchronize()
    check_adamw(P0, G, m0, v0, P, m, v, lr=AUX_LR["vector"], step=step)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_unaligned_pointers(dtype):
    """Views starting one element into their storage take the per-element
    path; results are the same as from aligned copies."""
    n = 9000
    Pb, Gb = tensors(n + 1, dtype, seed=5)
    mb, vb = state(n + 1, seed=6, step=3)
    P, G, m, v = Pb[1:], Gb[1:], mb[1:], vb[1:]
    heads = (Pb[:1].clone(), mb[:1].clone(), vb[:1].clone())
    Pa, Ga, ma, va = P.clone(), G.clone(), m.clone(), v.clone()
    P0, m0, v0 = P.clone(), m.clone(), v.clone()
    adamw_step(P, G, m, v, lr=0.004, step=3)
    adamw_step(Pa, Ga, ma, va, lr=0.004, step=3)
    torch.cuda.synchronize()
    check_adamw(P0, G, m0, v0, P, m, v, lr=0.004, step=3)
    assert torch.equal(P, Pa) and torch.equal(m, ma) and torch.equal(v, va)
    # the element before each view is untouched
    assert all(torch.equal(a, b) for a, b in zip(heads, (Pb[:1], mb[:1], vb[:1])))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_grouped_equals_single_bitwise(dtype):
    """40 tensors (two launches of up to 32) with their own lr and weight decay:
    the grouped call equals one call per tensor bit for bit, and the oracle."""
    sizes = [1, 7, 64, 768, 4096, 5000, 12345, 65536] * 5
    lrs = [0.7, 0.004, 0.015, 3e-4]
    wds = [1e-3, 0.0, 0.1]
    A, B, base = [], [], []
    for i, n in enumerate(sizes):
        P, G = tensors(n, dtype, seed=100 + i)
        m, v = state(n, seed=200 + i, step=4)
        base.append((P.clone(), G, m.clone(), v.clone()))
        A.append((P, G, m, v))
        B.append((P.clone(), G, m.clone(), v.clone()))
    adamw_step_grouped([adamw_tensor(*t, lr=lrs[i % 4], weight_decay=wds[i % 3])
                        for i, t in enumerate(A)], dtype, step=4)
    for i, t in enumerate(B):
        adamw_step(*t, lr=lrs[i % 4], weight_decay=wds[i % 3], step=4)
    torch.cuda.synchronize()
    for i, (a, b, z) in enumerate(zip(A, B, base)):
        assert torch.equal(a[0], b[0]) and torch.equal(a[2], b[2]) and torch.equal(a[3], b[3]), i
        check_adamw(z[0], z[1], z[2], z[3], a[0], a[2], a[3], lr=lrs[i % 4], step=4,
                    weight_decay=wds[i % 3])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_three_steps_teacher_forced(dtype):
    """Steps 1..3 with fresh gradients; each GPU step is checked against the
    oracle run from the GPU's own previous state."""
    n = 50_000
    P, _ = tensors(n, dtype, seed=9)
    m = torch.zeros(n, dtype=torch.float32, device=DEV)
    v = torch.zeros(n, dtype=torch.float32, device=DEV)
    for t in (1, 2, 3):
        _, G = tensors(n, dtype, seed=10 + t)
        P0, m0, v0 = P.clone(), m.clone(), v.clone()
        adamw_step(P, G, m, v, lr=AUX_LR["embedding"], step=t)
        torch.cuda.synchronize()
        check_adamw(P0, G, m0, v0, P, m, v, lr=AUX_LR["embedding"], step=t)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_zero_gradient_and_state(dtype):
    """g = m = v = 0: the Adam term is 0 / eps = 0; P' = (1 - lr wd) P rounded."""
    n = 10_000
    P, _ = tensors(n, dtype, seed=12)
    G = torch.zeros(n, dtype=dtype, device=DEV)
    m = torch.zeros(n, dtype=torch.float32, device=DEV)
    v = torch.zeros(n, dtype=torch.float32, device=DEV)
    P0 = P.clone()
    adamw_step(P, G, m, v, lr=0.7, step=5, weight_decay=1e-3)
    torch.cuda.synchronize()
    assert not m.any() and not v.any()
    want = (P0.float() * np.float32(1 - 0.7 * 1e-3)).to(dtype)
    assert torch.equal(P, want)


def test_nan_gradient_propagates():
    n = 5000
    P, G = tensors(n, torch.bfloat16, seed=13)
    G[17] = float("nan")
    m, v = state(n, seed=14, step=2)
    adamw_step(P, G, m, v, lr=0.015, step=2)
    torch.cuda.synchronize()
    assert torch.isnan(P[17]) and torch.isnan(m[17]) and torch.isnan(v[17])
    assert torch.isfinite(P[:17]).all() and torch.isfinite(P[18:]).all()


def test_deterministic():
    n = 70_000
    out = []
    for _ in range(2):
        P, G = tensors(n, torch.bfloat16, seed=15)
        m, v = state(n, seed=16, step=6)
        adamw_step(P, G, m, v, lr=0.004, step=6)
        out.append((P, m, v))
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(out[0], out[1]))


@pytest.mark.parametrize("name", ["gpt160m"])
def test_aux_set_of_model(name):
    """The whole AdamW side of GPT-160M (embedding and head 50304x768, 25
    gains) in the grouped call the benchmark times: two steps, each checked
    against the oracle on every element."""
    Ps = wl.make_aux_params(name, device=DEV)
    moments = wl.make_aux_moments(name, device=DEV)
    roles = [t.role for t in wl.AUX_SETS[name]]
    for step in (1, 2):
        Gs = wl.make_aux_grads(name, step, device=DEV)
        before = [(P.clone(), m.clone(), v.clone()) for P, (m, v) in zip(Ps, moments)]
        adamw_step_grouped([adamw_tensor(P, G, m, v, lr=AUX_LR[r])
                            for P, G, (m, v), r in zip(Ps, Gs, moments, roles)],
                           torch.bfloat16, step=step)
        torch.cuda.synchronize()
        for P, G, (m, v), (P0, m0, v0), r in zip(Ps, Gs, moments, before, roles):
            check_adamw(P0, G, m0, v0, P, m, v, lr=AUX_LR[r], step=step)
        del before


def test_hybrid_optimizer_front_end():
    """HybridMuonAdamW: Muon on the 2-D hidden weights, AdamW on embedding,
    head and gains, each half matching its oracle over two steps."""
    torch.manual_seed(3)
    hidden = [torch.nn.Parameter((torch.randn(96, 160) * 0.02).to(DEV)),
              torch.nn.Parameter((torch.randn(160, 96) * 0.02).to(DEV))]
    emb = torch.nn.Parameter((torch.randn(300, 96) * 0.02).to(DEV))
    gain = torch.nn.Parameter(torch.ones(96, device=DEV))
    opt = HybridMuonAdamW(hidden, [dict(params=[emb], lr=AUX_LR["embedding"]),
                                   dict(params=[gain], lr=AUX_LR["vector"])])
    Ms = [np.zeros(p.shape) for p in hidden]
    ms = [np.zeros(p.numel()) for p in (emb, gain)]
    vs = [np.zeros(p.numel()) for p in (emb, gain)]
    for t in (1, 2):
        for p in hidden + [emb, gain]:
            p.grad = torch.randn_like(p) * 1e-3
        W0 = [f64(p.detach()) for p in hidden]
        A0 = [f64(p.detach()).ravel() for p in (emb, gain)]
        grads = [f64(p.grad) for p in hidden + [emb, gain]]
        opt.step()
        torch.cuda.synchronize()
        for i, p in enumerate(hidden):
            Wr, Ms[i], _ = oracle.muon_step(W0[i], grads[i], Ms[i])
            assert relF(f64(p.detach()) - W0[i], Wr - W0[i]) <= 1e-5
        for j, (p, lr) in enumerate(((emb, AUX_LR["embedding"]), (gain, AUX_LR["vector"]))):
            Pr, ms[j], vs[j] = oracle.adamw_step(A0[j], grads[2 + j].ravel(), ms[j], vs[j],
                                                 lr=lr, step=t)
            assert relF(f64(p.detach()).ravel() - A0[j], Pr - A0[j]) <= 1e-5


def test_front_end_errors():
    P = torch.zeros(10, device=DEV, dtype=torch.bfloat16)
    f = torch.zeros(10, device=DEV)
    with pytest.raises(TypeError):     # gradient dtype differs from the parameter's
        adamw_tensor(P, f, f.clone(), f.clone(), lr=0.1)
    with pytest.raises(ValueError):    # moment size differs
        adamw_tensor(P, P.clone(), torch.zeros(9, device=DEV), f, lr=0.1)
    with pytest.raises(TypeError):
        adamw_tensor(P.half(), P.half(), f, f.clone(), lr=0.1)
    p = torch.nn.Parameter(torch.zeros(4, device=DEV))
    opt = AdamWStep([dict(params=[p], lr=0.1)])
    with pytest.raises(RuntimeError):
        opt.step()
    assert math.isfinite(AUX_EPS)
