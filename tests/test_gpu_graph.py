"""HIP graph capture of the fused Muon step.

The library's call path makes no allocation, memset or host synchronisation (the workspace is
passed in, timing is off), so a whole step can be captured once into a HIP graph and replayed.
Each replay is checked bit for bit against the same step run eagerly (the kernels are
deterministic), with unrelated eager work and a device synchronisation between replays.
"""

import numpy as np
import pytest

import synth
from helpers import say

pytestmark = pytest.mark.gpu

REPLAYS = 3
HYPER = dict(lr=0.02, momentum=0.95, weight_decay=0.1, nesterov=True)


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


def batch(torch, seed, B, r, c, scale=1.0, dtype=None):
    a = np.stack([scale * synth.lowrank_plus_noise(synth.host_rng(seed, b), r, c, 0.7, 0.05)
                  for b in range(B)])
    return torch.tensor(a, dtype=dtype or torch.bfloat16, device="cuda")


@pytest.mark.parametrize("variant", ["standard", "gram_stabilized"])
@pytest.mark.parametrize("shape", [(4, 512, 1408), (3, 1408, 512)])
def test_captured_muon_step_replays_match_eager(torch, ops, variant, shape):
    B, r, c = shape
    say(f"case graph capture muon_step {variant} {shape}")
    code = ops.STANDARD if variant == "standard" else ops.GRAM
    G = batch(torch, 301, B, r, c)
    W0 = batch(torch, 302, B, r, c, 0.02)
    M0 = batch(torch, 303, B, r, c, 0.5, torch.float32)  # momentum is fp32

    W_e, M_e = W0.clone(), M0.clone()
    ops.muon_step(W_e, G, M_e, variant=code, **HYPER)
    torch.cuda.synchronize()

    p = ops.ns_params(io_dtype=ops.BF16, restart_mask=ops.STABILIZED_RESTART_MASK
                      if code == ops.GRAM else 0)
    ws = torch.empty(ops.workspace_bytes(code, G, p), dtype=torch.uint8, device="cuda")
    W_s, M_s = W0.clone(), M0.clone()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ops.muon_step(W_s, G, M_s, variant=code, workspace=ws, **HYPER)
    torch.cuda.synchronize()

    other_G = batch(torch, 304, 2, 256, 640)
    for rep in range(REPLAYS):
        W_s.copy_(W0)
        M_s.copy_(M0)
        # Unrelated eager work between replays, on the same stream and device.
        W_o = torch.zeros_like(other_G)
        M_o = torch.zeros_like(other_G, dtype=torch.float32)
        ops.muon_step(W_o, other_G, M_o, variant=code, **HYPER)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(W_s, W_e), (variant, shape, rep, "W")
        assert torch.equal(M_s, M_e), (variant, shape, rep, "M")
        assert torch.isfinite(W_o.float()).all()


def test_captured_grouped_step_replays_match_eager(torch, ops):
    say("case graph capture muon_step_grouped")
    shapes = [(3, 512, 1408), (2, 1408, 512), (1, 768, 768)]
    Gs = [batch(torch, 310 + i, *s) for i, s in enumerate(shapes)]
    W0 = [batch(torch, 320 + i, *s, scale=0.02) for i, s in enumerate(shapes)]
    M0 = [batch(torch, 330 + i, *s, scale=0.5, dtype=torch.float32) for i, s in enumerate(shapes)]

    W_e, M_e = [w.clone() for w in W0], [m.clone() for m in M0]
    ops.muon_step_grouped(W_e, Gs, M_e, **HYPER)
    torch.cuda.synchronize()

    p = ops.ns_params(io_dtype=ops.BF16, restart_mask=ops.STABILIZED_RESTART_MASK)
    ws = torch.empty(ops.workspace_bytes_grouped(ops.GRAM, Gs, p), dtype=torch.uint8,
                     device="cuda")
    W_s, M_s = [w.clone() for w in W0], [m.clone() for m in M0]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ops.muon_step_grouped(W_s, Gs, M_s, workspace=ws, **HYPER)
    torch.cuda.synchronize()

    for rep in range(REPLAYS):
        for w, w0 in zip(W_s, W0):
            w.copy_(w0)
        for m, m0 in zip(M_s, M0):
            m.copy_(m0)
        extra = torch.zeros_like(Gs[0])
        ops.muon_step(extra, Gs[0], torch.zeros_like(Gs[0], dtype=torch.float32), **HYPER)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for g, (ws_, we, ms_, me) in enumerate(zip(W_s, W_e, M_s, M_e)):
            assert torch.equal(ws_, we), (rep, g, "W")
            assert torch.equal(ms_, me), (rep, g, "M")
