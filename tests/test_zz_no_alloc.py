"""muon_step_noalloc (the Muon step on the library's static device scratch) against muon_step
with a caller workspace of the same size: both process the batch in the same chunks with the
same kernels, so W, M and U agree bit for bit. Two calls in a row, the second on a smaller
input, so the second call runs on scratch that still holds the first call's contents."""
import os
import re

import pytest

import synth
from helpers import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


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


def test_scratch_size_matches_the_header(ops):
    text = open(os.path.join(ROOT, "include", "muon_ns.h")).read()
    m = re.search(r"#define MNS_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == ops.NOALLOC_SCRATCH_BYTES


# (batch, rows, cols, variant): the first call needs several scratch-sized chunks (a
# 2048 x 7168 matrix takes ~100 MB with stabilized Gram NS), the second is smaller and
# transposed (rows > cols), ragged, and standard NS
CALLS = [(5, 2048, 7168, "gram"), (7, 700, 300, "standard")]


def test_noalloc_step_equals_the_workspace_step_twice(torch, ops):
    kw = dict(lr=0.02, momentum=0.95, weight_decay=0.01, scale_coeff=0.2, nesterov=True)
    ws = torch.empty(ops.NOALLOC_SCRATCH_BYTES, dtype=torch.uint8, device="cuda")
    for i, (B, r, c, variant) in enumerate(CALLS):
        say(f"case noalloc call {i}: {B}x{r}x{c} {variant}")
        code = ops.GRAM if variant == "gram" else ops.STANDARD
        G = synth.torch_gaussian_plus_spike(B, r, c, workload_index=7, device="cuda")
        W0 = synth.torch_weights(B, r, c, workload_index=7, device="cuda")
        M0 = 0.01 * torch.randn(B, r, c, device="cuda", dtype=torch.float32)
        W1, M1 = W0.clone(), M0.clone()
        W2, M2 = W0.clone(), M0.clone()
        U1 = torch.empty(B, r, c, dtype=torch.float32, device="cuda")
        U2 = torch.empty_like(U1)
        f1 = torch.full((B,), -1, dtype=torch.int32, device="cuda")
        f2 = torch.full((B,), -1, dtype=torch.int32, device="cuda")
        ops.muon_step(W1, G, M1, variant=code, workspace=ws, U_out=U1, flags=f1, **kw)
        ops.muon_step_noalloc(W2, G, M2, variant=code, U_out=U2, flags=f2, **kw)
        torch.cuda.synchronize()
        assert int(f1.abs().sum()) == 0 and torch.equal(f1, f2)
        assert torch.equal(W1, W2) and torch.equal(M1, M2) and torch.equal(U1, U2)
        assert not torch.equal(W1, W0)
        # and the fused weight-update epilogue (no U_out) of both entry points
        W3, M3 = W0.clone(), M0.clone()
        W4, M4 = W0.clone(), M0.clone()
        ops.muon_step(W3, G, M3, variant=code, workspace=ws, **kw)
        ops.muon_step_noalloc(W4, G, M4, variant=code, **kw)
        torch.cuda.synchronize()
        assert torch.equal(W3, W4) and torch.equal(M3, M4)
        say(f"  call {i}: bit-equal W, M, U and flags")
        del G, W0, M0, W1, M1, W2, M2, U1, U2, W3, M3, W4, M4
        torch.cuda.empty_cache()
