"""Checkpoint / resume and run-to-run determinism of the fused Muon step (Moonlight guide, "The
Scalable Muon Optimizer: Theory and Mechanics": the momentum buffer is the optimizer's only
state). The library keeps nothing between calls (the caller owns W and M), so saving (W, M)
after step t and restoring it reproduces step t + 1 bit for bit; and one step from one state
gives bit-identical W, M (and U) on every run: the Frobenius norm is reduced in a fixed order and
every output element is computed by one thread, so a difference would expose a race."""
import pytest

import synth
from helpers import say

pytestmark = pytest.mark.gpu


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


# small-tile path, and the large-tile persistent path with ragged edges in both orientations
SHAPES = [(6, 256, 512), (24, 1000, 1512), (24, 1512, 1000)]


@pytest.mark.parametrize("variant", ["gram", "standard"])
@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("with_u", [False, True])
def test_resume_from_saved_state_is_bit_identical(torch, ops, shape, variant, with_u):
    B, r, c = shape
    say(f"case resume {shape} {variant} U_out={with_u}")
    code = ops.GRAM if variant == "gram" else ops.STANDARD
    G1, G2 = (synth.torch_lowrank_plus_noise(B, r, c, power=0.7, noise=0.05, workload_index=1,
                                             seed_offset=s, device="cuda").to(torch.bfloat16) for s in (41, 42))
    W = synth.torch_weights(B, r, c, workload_index=1, device="cuda", dtype=torch.bfloat16)
    M = torch.zeros(B, r, c, dtype=torch.float32, device="cuda")
    kw = dict(lr=0.02, momentum=0.95, weight_decay=0.1, nesterov=True, variant=code)

    def step(W, M, G):
        U = torch.empty(B, r, c, dtype=torch.bfloat16, device="cuda") if with_u else None
        ops.muon_step(W, G, M, U_out=U, **kw)
        return U

    step(W, M, G1)                                   # step t
    W_saved, M_saved = W.clone(), M.clone()          # checkpoint
    U_a = step(W, M, G2)                             # step t + 1
    runs = []
    for _ in range(2):                               # restore, then step t + 1 again (twice)
        W_r, M_r = W_saved.clone(), M_saved.clone()
        U_r = step(W_r, M_r, G2)
        runs.append((W_r, M_r, U_r))
    torch.cuda.synchronize()
    for W_r, M_r, U_r in runs:
        assert torch.equal(W_r, W) and torch.equal(M_r, M)
        if with_u:
            assert torch.equal(U_r, U_a)
    assert not torch.equal(W, W_saved)               # the step did change W
