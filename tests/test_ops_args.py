"""The Python binding rejects misuse before any library call: wrong dtypes, short or
mis-typed flag buffers, mismatched shapes, group-list lengths and host tensors raise in
ops.py, so nothing reaches a kernel as a bad pointer. CPU only: every case raises before the
library (or a GPU) is touched."""
import pytest
import torch

from newton_schulz_matrix_muon_amd import ops


def _step_tensors(b=3, r=8, c=16):
    W = torch.zeros(b, r, c, dtype=torch.bfloat16)
    G = torch.zeros(b, r, c, dtype=torch.bfloat16)
    M = torch.zeros(b, r, c, dtype=torch.float32)
    return W, G, M


STEP_KW = dict(lr=0.02, momentum=0.95, weight_decay=0.01)


def test_muon_step_rejects_a_momentum_buffer_that_is_not_fp32():
    W, G, M = _step_tensors()
    with pytest.raises(TypeError, match="float32"):
        ops.muon_step(W, G, M.to(torch.bfloat16), **STEP_KW)


def test_muon_step_rejects_mismatched_shapes():
    W, G, M = _step_tensors()
    with pytest.raises(ValueError, match="shape"):
        ops.muon_step(W[:2], G, M, **STEP_KW)
    with pytest.raises(ValueError, match="U_out"):
        ops.muon_step(W, G, M, U_out=torch.zeros(3, 8, 15), **STEP_KW)


@pytest.mark.parametrize("bad, exc", [(torch.zeros(3, dtype=torch.int64), TypeError),
                                      (torch.zeros(2, dtype=torch.int32), ValueError),
                                      (torch.zeros(6, dtype=torch.int32)[::2], ValueError)])
def test_flags_must_be_int32_contiguous_and_cover_the_batch(bad, exc):
    W, G, M = _step_tensors()
    with pytest.raises(exc, match="flags"):
        ops.muon_step(W, G, M, flags=bad, **STEP_KW)
    with pytest.raises(exc, match="flags"):
        ops.gram_ns(G, flags=bad)
    with pytest.raises(exc, match="flags"):
        ops.muon_ns(G, flags=bad)


def test_host_tensors_are_rejected():
    W, G, M = _step_tensors()
    with pytest.raises(ValueError, match="device"):
        ops.muon_step(W, G, M, **STEP_KW)
    with pytest.raises(ValueError, match="device"):
        ops.gram_ns(G)
    with pytest.raises(ValueError, match="device"):
        ops.gram_trace(G)


def test_ns_out_must_match_the_input():
    _, G, _ = _step_tensors()
    with pytest.raises(TypeError, match="dtype"):
        ops.gram_ns(G, out=torch.empty(3, 8, 16, dtype=torch.float16))
    with pytest.raises(ValueError, match="shape"):
        ops.muon_ns(G, out=torch.empty(3, 16, 8, dtype=torch.bfloat16))


def test_grouped_calls_check_lists_flags_and_buffers():
    W, G, M = _step_tensors()
    W2, G2, M2 = _step_tensors(2, 16, 8)
    with pytest.raises(ValueError, match="groups"):
        ops.gram_ns_grouped([G] * 5)
    with pytest.raises(ValueError, match="entries"):
        ops.muon_step_grouped([W], [G, G2], [M, M2], **STEP_KW)
    with pytest.raises(TypeError, match="float32"):
        ops.muon_step_grouped([W, W2], [G, G2], [M, M2.double()], **STEP_KW)
    # flags must cover the matrices of every group (3 + 2 here)
    with pytest.raises(ValueError, match="flags"):
        ops.muon_step_grouped([W, W2], [G, G2], [M, M2], flags=torch.zeros(4, dtype=torch.int32),
                              **STEP_KW)
    with pytest.raises(ValueError, match="flags"):
        ops.muon_ns_grouped([G, G2], flags=torch.zeros(3, dtype=torch.int32))
    with pytest.raises(ValueError, match="device"):
        ops.muon_step_grouped([W, W2], [G, G2], [M, M2], flags=torch.zeros(5, dtype=torch.int32),
                              **STEP_KW)


def test_adamw_checks_dtypes_and_sizes():
    p = torch.zeros(10, dtype=torch.bfloat16)
    g = torch.zeros(10, dtype=torch.bfloat16)
    m = torch.zeros(10)
    v = torch.zeros(10)
    with pytest.raises(TypeError, match="grads"):
        ops.adamw_step([p], [g.float()], [m], [v], lr=1e-3)
    with pytest.raises(TypeError, match="float32"):
        ops.adamw_step([p], [g], [m.to(torch.bfloat16)], [v], lr=1e-3)
    with pytest.raises(TypeError, match="params"):
        ops.adamw_step([p, p.half()], [g, g.half()], [m, m.clone()], [v, v.clone()], lr=1e-3)
    with pytest.raises(ValueError, match="sizes"):
        ops.adamw_step([p], [g[:9]], [m], [v], lr=1e-3)
    with pytest.raises(ValueError, match="device"):
        ops.adamw_step([p], [g], [m], [v], lr=1e-3)
