"""Restart schedule x iterate precision x coefficient ablation of Gram Newton-Schulz on the
stability inputs (Gram NS article, sections on the fp16 instability and the restarted variant;
Moonlight guide, Newton-Schulz section, for the cubic 0.5 X (3I - X^T X)).

Inputs: the first matrix of nine stability classes (n in {512, 1024} with n:m in {1:1, 1:2,
1:4, 1:8}, and 2048 x 2048), G = U diag(s) V^T with s_j = exp(Uniform(ln 1e-6, 0)).
Runs: restart sets {}, {2}, {1, 3}, {1, 2, 3, 4}; iterates fp16 and bf16 (input stored in
fp16) and fp32 (input stored in fp32); quintic (3.4445, -4.7750, 2.0315) and cubic
(1.5, -0.5, 0) coefficients, K = 5. Each run is compared with the fp64 oracle's Gram
iteration with the same coefficients (in fp64 the restart set does not change the result).

Asserted: every output is finite; the fp32-iterate runs are within 1e-3 of the oracle for
every restart set and both coefficient sets; with fp16 iterates, restarting (any non-empty
set) is at least as accurate as the naive form for the quintic. Everything else is reported
(printed; JSON when MNS_REPORT_DIR is set).
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from helpers import rel_fro, say

pytestmark = pytest.mark.gpu
WORKLOAD = 4
MASKS = {"none": 0, "{2}": 1 << 2, "{1,3}": (1 << 1) | (1 << 3), "{1,2,3,4}": 0b11110}
COEFFS = {"quintic": [[3.4445, -4.7750, 2.0315]] * 5, "cubic": [[1.5, -0.5, 0.0]] * 5}
CLASSES = [0, 1, 2, 3, 4, 5, 6, 7, 8]       # class c: n = (512, 1024, 2048)[c // 4], m = n (1, 2, 4, 8)[c % 4]


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


@pytest.fixture(scope="module")
def ablation(torch, ops):
    shapes = synth.stability_classes(12)
    res = {}
    for c in CLASSES:
        n, m = shapes[c]
        G32 = synth.torch_loguniform_spectrum(1, n, m, workload_index=WORKLOAD, seed_offset=1000 * c,
                                              device="cuda", chunk=1)
        G16 = G32.to(torch.float16)
        inputs = {"f16": G16, "f32": G32}
        refs = {(io, cn): oracle.ns_gram(inputs[io][0].double().cpu().numpy(), coeffs=cf, restarts=())
                for io in inputs for cn, cf in COEFFS.items()}
        for cn, cf in COEFFS.items():
            for it in ("f16", "bf16", "f32"):
                io = "f32" if it == "f32" else "f16"
                itc = {"f16": ops.F16, "bf16": ops.BF16, "f32": ops.F32}[it]
                for mn, mask in MASKS.items():
                    O = ops.gram_ns(inputs[io], coeffs=cf, iter_dtype=itc, restart_mask=mask)
                    Oh = O[0].double().cpu().numpy()
                    fin = bool(np.isfinite(Oh).all())
                    res[(c, cn, it, mn)] = rel_fro(Oh, refs[(io, cn)]) if fin else float("inf")
        say(f"ablation class {c} ({n} x {m}) done")
    return res


def test_ablation_report_and_bounds(ablation):
    res = ablation
    rows = {}
    for (c, cn, it, mn), e in res.items():
        rows.setdefault((cn, it, mn), []).append(e)
    say(f"{'coeffs':8s} {'iterates':8s} {'restarts':10s}  rel_F median / max over {len(CLASSES)} matrices")
    for (cn, it, mn), es in sorted(rows.items()):
        say(f"{cn:8s} {it:8s} {mn:10s}  {np.median(es):.2e} / {max(es):.2e}")
    out = os.environ.get("MNS_REPORT_DIR")
    if out:
        os.makedirs(out, exist_ok=True)
        with open(os.path.join(out, "ablation_restart_precision_coeffs.json"), "w") as f:
            json.dump({"/".join(map(str, k)): v for k, v in res.items()}, f, indent=1)
    assert all(np.isfinite(e) for e in res.values())
    assert all(e <= 1e-3 for (c, cn, it, mn), e in res.items() if it == "f32"), \
        {k: v for k, v in res.items() if k[2] == "f32" and v > 1e-3}
    for c in CLASSES:
        naive = res[(c, "quintic", "f16", "none")]
        for mn in ("{2}", "{1,3}", "{1,2,3,4}"):
            assert res[(c, "quintic", "f16", mn)] <= naive, (c, mn, res[(c, "quintic", "f16", mn)], naive)
