"""AdamW step of the hybrid optimizer (Moonlight guide, "The Coordinate-Wise Limitation of
AdamW" and "The Hybrid Optimization Strategy") against the fp64 oracle.

The kernel works in fp32 and rounds the parameter once to its dtype. Bounds per element:
moments within 4 fp32 roundings of their inputs' magnitudes; the parameter within half a unit
in the last place of its dtype plus the propagated fp32 error of the update.
"""
import numpy as np
import pytest

import oracle
from helpers import say, to_np

pytestmark = pytest.mark.gpu
U32 = 2.0 ** -24
MANT = {"f32": 23, "bf16": 7, "f16": 10}


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


@pytest.fixture(scope="module")
def ops():
    from newton_schulz_matrix_muon_amd import ops as o
    o.lib()
    return o


def _dt(torch, name):
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[name]


MIN_EXP = {"f32": -126, "bf16": -126, "f16": -14}     # smallest normal exponent


def _half_ulp(x, name):
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** MIN_EXP[name])))
    return 2.0 ** (e - MANT[name] - 1)


def check_step(p0, g, m0, v0, p1, m1, v1, hp, name):
    """p0, g, m0, v0: exact fp64 inputs; p1, m1, v1: the kernel's outputs (fp64 copies)."""
    lr, b1, b2, eps, wd, step, bc = hp
    # the kernel receives the hyper-parameters as fp32: give the oracle those same values
    lr, b1, b2, eps, wd = (float(np.float32(x)) for x in (lr, b1, b2, eps, wd))
    pr, mr, vr = oracle.adamw_step(p0, g, m0, v0, lr, b1, b2, eps, wd, step, bc)
    dm = 4 * U32 * (b1 * np.abs(m0) + (1 - b1) * np.abs(g)) + 1e-38
    dv = 4 * U32 * (b2 * np.abs(v0) + (1 - b2) * g * g) + 1e-38
    assert np.all(np.abs(m1 - mr) <= dm)
    assert np.all(np.abs(v1 - vr) <= dv)
    c1 = 1 / (1 - b1 ** step) if bc else 1.0
    c2 = 1 / (1 - b2 ** step) if bc else 1.0
    den = np.sqrt(vr * c2) + eps
    upd = mr * c1 / den
    dupd = dm * c1 / den + 8 * U32 * np.abs(upd) + np.abs(upd) * dv * c2 / (2 * np.maximum(vr * c2, 1e-300) ** 0.5 * den)
    slack = 4 * U32 * (abs(1 - lr * wd) * np.abs(p0) + lr * np.abs(upd)) + lr * dupd
    ok = np.abs(p1 - pr) <= _half_ulp(pr, name) * (1 + 1e-6) + slack
    assert ok.all(), (np.flatnonzero(~ok)[:5], p1[~ok][:5], pr[~ok][:5])


@pytest.mark.parametrize("name", ["bf16", "f32", "f16"])
@pytest.mark.parametrize("bc", [False, True])
def test_adamw_multi_tensor_two_steps(torch, ops, name, bc):
    say(f"case adamw {name} bias_correction={bc}")
    gen = torch.Generator(device="cuda").manual_seed(77)
    sizes = [0, 1, 4099, 8192, 100_003, 7168]
    dt = _dt(torch, name)
    ps = [(0.02 * torch.randn(n, generator=gen, device="cuda")).to(dt) for n in sizes]
    ms = [torch.zeros(n, device="cuda") for n in sizes]
    vs = [torch.zeros(n, device="cuda") for n in sizes]
    hp = dict(lr=3e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, bias_correction=bc)
    for step in (1, 2):
        gs = [(torch.randn(n, generator=gen, device="cuda") * (1e-3 if i % 2 else 1.0)).to(dt)
              for i, n in enumerate(sizes)]
        before = [(to_np(p), to_np(g), to_np(m), to_np(v)) for p, g, m, v in zip(ps, gs, ms, vs)]
        ops.adamw_step(ps, gs, ms, vs, step=step, **hp)
        torch.cuda.synchronize()
        for (p0, g0, m0, v0), p, m, v in zip(before, ps, ms, vs):
            check_step(p0, g0, m0, v0, to_np(p), to_np(m), to_np(v),
                       (3e-3, 0.9, 0.95, 1e-8, 0.1, step, bc), name)


def test_adamw_many_tensors_and_unaligned_views(torch, ops):
    """More tensors than one launch's table (48) and views that are not vector-aligned."""
    say("case adamw 70 tensors + unaligned views")
    gen = torch.Generator(device="cuda").manual_seed(5)
    base = torch.randn(70 * 301 + 3, generator=gen, device="cuda").to(torch.bfloat16)
    ps = [base[1 + 301 * i: 1 + 301 * i + 300] for i in range(70)]        # offset by one element
    gs = [torch.randn(300, generator=gen, device="cuda").to(torch.bfloat16) for _ in range(70)]
    ms = [torch.randn(300, generator=gen, device="cuda") * 1e-2 for _ in range(70)]
    vs = [torch.rand(300, generator=gen, device="cuda") * 1e-4 for _ in range(70)]
    before = [(to_np(p), to_np(g), to_np(m), to_np(v)) for p, g, m, v in zip(ps, gs, ms, vs)]
    gaps = torch.tensor([0] + [301 * (i + 1) for i in range(70)] + [70 * 301 + 1, 70 * 301 + 2], device="cuda")
    gap_vals = base[gaps].clone()
    ops.timing_reset()
    ops.timing_enable(True)
    ops.adamw_step(ps, gs, ms, vs, lr=1e-2, beta1=0.8, beta2=0.99, eps=1e-6, weight_decay=0.05)
    ops.timing_enable(False)
    assert ops.timing_query()["adamw"][1] == 2                            # 48 + 22 tensors
    torch.cuda.synchronize()
    for (p0, g0, m0, v0), p, m, v in zip(before, ps, ms, vs):
        check_step(p0, g0, m0, v0, to_np(p), to_np(m), to_np(v), (1e-2, 0.8, 0.99, 1e-6, 0.05, 1, False), "bf16")
    # the elements between the views are untouched
    assert torch.equal(base[gaps], gap_vals)


def test_adamw_embedding_size_sampled(torch, ops):
    """A Kimi-K2-sized token embedding, 163840 x 7168 bf16 (1.17 G parameters), one step,
    checked on 20 000 sampled elements."""
    say("case adamw embedding 163840 x 7168 bf16")
    n = 163840 * 7168
    gen = torch.Generator(device="cuda").manual_seed(11)
    p = (0.02 * torch.randn(n, generator=gen, device="cuda")).to(torch.bfloat16)
    g = (1e-3 * torch.randn(n, generator=gen, device="cuda")).to(torch.bfloat16)
    m = torch.zeros(n, device="cuda")
    v = torch.zeros(n, device="cuda")
    idx = torch.randint(0, n, (20000,), generator=gen, device="cuda")
    p0, g0 = to_np(p[idx]), to_np(g[idx])
    ops.adamw_step([p], [g], [m], [v], lr=2e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    torch.cuda.synchronize()
    z = np.zeros_like(p0)
    check_step(p0, g0, z, z, to_np(p[idx]), to_np(m[idx]), to_np(v[idx]), (2e-4, 0.9, 0.95, 1e-8, 0.1, 1, False), "bf16")
