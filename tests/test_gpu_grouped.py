"""Grouped calls: several batches of different shapes (and orientations) in one call.

A grouped call must give, bit for bit, what separate single-group calls give (same kernels,
same tiles; only the launches are shared), and each group must still match the oracle. The
groups mirror the structure of the Kimi-K2 optimizer step timed in the Gram Newton-Schulz
article (expert up/gate matrices, expert down matrices in the transposed orientation, a dense
FFN matrix) at reduced sizes.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from helpers import rel_fro, say, to_np

pytestmark = pytest.mark.gpu
TOL = 2e-2
SHAPES = [(3, 200, 456), (2, 456, 200), (1, 300, 700)]


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


def _inputs(torch, shapes, seed):
    Gs = [synth.torch_lowrank_plus_noise(b, r, c, power=0.7, noise=0.05, workload_index=1,
                                         seed_offset=seed + 10 * i, device="cuda")
          for i, (b, r, c) in enumerate(shapes)]
    Ws = [synth.torch_weights(b, r, c, workload_index=1, device="cuda", seed_offset=seed + 20 * i)
          for i, (b, r, c) in enumerate(shapes)]
    return Gs, Ws


@pytest.mark.parametrize("variant", ["gram", "standard"])
def test_grouped_ns_equals_single_calls(torch, ops, variant):
    say(f"case grouped NS {variant}")
    Gs, _ = _inputs(torch, SHAPES, 7000)
    if variant == "gram":
        outs = ops.gram_ns_grouped(Gs)
        singles = [ops.gram_ns(G) for G in Gs]
    else:
        outs = ops.muon_ns_grouped(Gs)
        singles = [ops.muon_ns(G) for G in Gs]
    torch.cuda.synchronize()
    for O, S in zip(outs, singles):
        assert torch.equal(O, S)
    ns = (lambda x: oracle.ns_gram(x, restarts=(2,))) if variant == "gram" else oracle.ns_standard
    for G, O in zip(Gs, outs):
        assert rel_fro(to_np(O[-1]), ns(to_np(G[-1]))) < TOL


@pytest.mark.parametrize("variant", ["gram", "standard"])
def test_grouped_muon_step_equals_single_calls(torch, ops, variant):
    say(f"case grouped muon_step {variant}")
    code = ops.GRAM if variant == "gram" else ops.STANDARD
    kw = dict(lr=0.02, momentum=0.95, weight_decay=0.01, nesterov=True, scale_coeff=0.2, variant=code)
    Gs, Ws = _inputs(torch, SHAPES, 8000)
    W1 = [W.clone() for W in Ws]
    M0 = [torch.zeros(G.shape, dtype=torch.float32, device="cuda") for G in Gs]
    M1 = [M.clone() for M in M0]
    U0 = [torch.empty(G.shape, dtype=torch.float32, device="cuda") for G in Gs]
    U1 = [U.clone() for U in U0]
    flags = torch.zeros(sum(G.shape[0] for G in Gs), dtype=torch.int32, device="cuda")
    ops.muon_step_grouped(Ws, Gs, M0, U_outs=U0, flags=flags, **kw)
    for W, G, M, U in zip(W1, Gs, M1, U1):
        ops.muon_step(W, G, M, U_out=U, **kw)
    torch.cuda.synchronize()
    for a, b in zip(Ws + M0 + U0, W1 + M1 + U1):
        assert torch.equal(a, b)
    assert int(flags.abs().sum()) == 0
    ns = (lambda x: oracle.ns_gram(x, restarts=(2,))) if code == ops.GRAM else oracle.ns_standard
    for G, U in zip(Gs, U0):
        _, _, Un = oracle.muon_step(np.zeros(G.shape[1:]), to_np(G[0]), np.zeros(G.shape[1:]), 0.02,
                                    0.95, 0.01, nesterov=True, scale_coeff=0.2, ns=ns)
        assert rel_fro(to_np(U[0]), Un) < TOL


def test_grouped_fallback_when_the_workspace_holds_one_group(torch, ops):
    """A workspace too small for all groups side by side runs them one after another."""
    say("case grouped fallback")
    Gs, _ = _inputs(torch, SHAPES, 9000)
    p = ops.ns_params(io_dtype=ops.BF16)
    singles = [ops.workspace_bytes(ops.GRAM, G, p) for G in Gs]
    assert ops.workspace_bytes_grouped(ops.GRAM, Gs, p) > max(singles)
    ws = torch.empty(max(singles), dtype=torch.uint8, device="cuda")
    outs = ops.gram_ns_grouped(Gs, workspace=ws)
    ref = [ops.gram_ns(G) for G in Gs]
    torch.cuda.synchronize()
    for O, S in zip(outs, ref):
        assert torch.equal(O, S)


def test_grouped_flags_follow_the_group_order(torch, ops):
    say("case grouped flags")
    Gs, _ = _inputs(torch, SHAPES, 9500)
    Gs[1][1].zero_()                      # group 1, matrix 1: zero input
    Gs[2][0, 5, 7] = float("nan")         # group 2, matrix 0: non-finite input
    flags = torch.zeros(6, dtype=torch.int32, device="cuda")
    outs = ops.gram_ns_grouped(Gs, flags=flags)
    torch.cuda.synchronize()
    f = flags.cpu().tolist()
    assert f[0] == f[1] == f[2] == f[3] == 0
    assert f[4] & 2 and not f[4] & 1      # 3 + 1: the zero matrix
    assert f[5] & 1                       # 3 + 2 + 0: the NaN matrix
    assert torch.count_nonzero(outs[1][1]) == 0


def test_grouped_k2_structure_reduced(torch, ops):
    """Expert up/gate (n x m), expert down (m x n) and one dense matrix, scaled down 4x."""
    say("case grouped K2 structure, reduced")
    shapes = [(8, 512, 1792), (4, 1792, 512), (1, 1792, 4608)]
    Gs = [synth.torch_gaussian_plus_spike(b, r, c, workload_index=2, device="cuda") for b, r, c in shapes]
    outs = ops.gram_ns_grouped(Gs)
    singles = [ops.gram_ns(G) for G in Gs]
    torch.cuda.synchronize()
    for O, S in zip(outs, singles):
        assert torch.equal(O, S)
    O = to_np(outs[2][0])
    assert rel_fro(O, oracle.ns_gram(to_np(Gs[2][0]), restarts=(2,))) < TOL
    assert math.isfinite(float(outs[0].float().abs().max()))


@pytest.mark.timeout(900)
def test_grouped_k2_full_size_equals_single_calls(torch, ops):
    """The whole Kimi-K2 Muon step's matrices at full size in one grouped call (432 x 2048 x
    7168 up/gate, 216 x 7168 x 2048 down, 3 x 7168 x 18432 dense): the 256 x 256 kernels with
    every group's tiles split over the XCDs, bit for bit equal to one call per group; the first
    matrix of every group (the dense one included) against the oracle."""
    say("case grouped K2 full size")
    shapes = [(432, 2048, 7168), (216, 7168, 2048), (3, 7168, 18432)]
    Gs = [synth.torch_gaussian_plus_spike(b, r, c, workload_index=2, device="cuda") for b, r, c in shapes]
    outs = ops.gram_ns_grouped(Gs)
    torch.cuda.synchronize()
    for G, O in zip(Gs, outs):
        S = ops.gram_ns(G)
        torch.cuda.synchronize()
        assert torch.equal(O, S)
        del S
    for i in (0, 1, 2):
        e = rel_fro(to_np(outs[i][0]), oracle.ns_gram(to_np(Gs[i][0]), restarts=(2,)))
        say(f"  group {i} matrix 0: rel_F {e:.3e}")
        assert e < TOL
