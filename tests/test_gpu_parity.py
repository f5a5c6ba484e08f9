"""GPU parity: the HIP path through the C ABI against the fp64 oracle, element by element.

Bars: relative Frobenius error <= 1e-4 on the fp32 path and <= 2e-2 on the bf16/fp16 path,
against the oracle's same variant, steps, coefficients and restart set, and every output
singular value inside the oracle output's band widened by the same tolerance.
"""

import numpy as np
import pytest

import oracle
import synth
from helpers import band_ok, rel_fro, say, to_np, w_update_ok

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2, "f16": 2e-2}


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


def tdtype(torch, name):
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[name]


def oracle_fn(variant):
    if variant == "standard":
        return lambda g: oracle.ns_standard(g)
    if variant == "gram_naive":
        return lambda g: oracle.ns_gram(g, restarts=())
    return lambda g: oracle.ns_gram(g, restarts=(2,))


def gpu_fn(ops, variant, **kw):
    if variant == "standard":
        return lambda G: ops.muon_ns(G, **kw)
    if variant == "gram_naive":
        return lambda G: ops.gram_ns(G, restart_mask=0, **kw)
    return lambda G: ops.gram_ns(G, restart_mask=1 << 2, **kw)


def check_batch(Gd, Od, variant, tol, label, band=True):
    G = to_np(Gd)
    O = to_np(Od)
    if G.ndim == 2:
        G, O = G[None], O[None]
    ref_fn = oracle_fn(variant)
    worst = 0.0
    for b in range(G.shape[0]):
        ref = ref_fn(G[b])
        e = rel_fro(O[b], ref)
        worst = max(worst, e)
        assert np.all(np.isfinite(O[b])), f"{label}[{b}] non-finite"
        assert e <= tol, f"{label}[{b}] rel_F {e:.3e} > {tol}"
        if band:
            ok, info = band_ok(O[b], ref, tol)
            assert ok, f"{label}[{b}] band {info}"
    say(f"  {label}: worst rel_F {worst:.3e} (tol {tol})")
    return worst


VARIANTS = ["standard", "gram_naive", "gram_stabilized"]


# ------------------------------------------------------------------ fp32 path

@pytest.mark.parametrize("variant", VARIANTS)
def test_small_fp32_128x512(torch, ops, variant):
    say(f"case small_fp32 128x512 {variant}")
    rng = synth.host_rng(0, 0)
    G = synth.lowrank_plus_noise(rng, 128, 512, power=1.0, noise=0.01)
    Gd = torch.tensor(G, dtype=torch.float32, device="cuda")
    Od = gpu_fn(ops, variant)(Gd)
    torch.cuda.synchronize()
    check_batch(Gd, Od, variant, TOL["f32"], f"f32/{variant}")


@pytest.mark.parametrize("shape", [(97, 211), (211, 97), (130, 130), (1, 40), (40, 1), (3, 5)])
def test_ragged_fp32(torch, ops, shape):
    say(f"case ragged_fp32 {shape}")
    r, c = shape
    G = synth.lowrank_plus_noise(synth.host_rng(90, r * 1000 + c), r, c, power=0.5, noise=0.05)
    Gd = torch.tensor(np.stack([G, -0.5 * G]), dtype=torch.float32, device="cuda")
    for variant in VARIANTS:
        Od = gpu_fn(ops, variant)(Gd)
        torch.cuda.synchronize()
        check_batch(Gd, Od, variant, TOL["f32"], f"f32{shape}/{variant}")


# ------------------------------------------------------------------ half-precision paths

@pytest.mark.parametrize("shape", [(97, 211), (211, 97), (300, 700), (700, 300), (257, 257),
                                   (1, 64), (64, 1), (5, 3), (128, 1024)])
@pytest.mark.parametrize("io", ["bf16", "f16"])
def test_ragged_half(torch, ops, shape, io):
    say(f"case ragged_half {io} {shape}")
    r, c = shape
    Gs = [synth.lowrank_plus_noise(synth.host_rng(91, 10 * b + r * 7 + c), r, c, power=0.7,
                                   noise=0.05) for b in range(3)]
    Gd = torch.tensor(np.stack(Gs), dtype=tdtype(torch, io), device="cuda")
    for variant in VARIANTS:
        Od = gpu_fn(ops, variant)(Gd)
        torch.cuda.synchronize()
        check_batch(Gd, Od, variant, TOL[io], f"{io}{shape}/{variant}")


def test_strided_batch_and_bf16_iterates(torch, ops):
    say("case strided batch 4 x 200 x 456 in a 4 x 220 x 500 buffer, iterates bf16 and f16")
    base = torch.zeros(4, 220, 500, dtype=torch.bfloat16, device="cuda")
    Gs = [synth.lowrank_plus_noise(synth.host_rng(92, b), 200, 456, 0.7, 0.05) for b in range(4)]
    base[:, :200, :456] = torch.tensor(np.stack(Gs), dtype=torch.bfloat16, device="cuda")
    Gv = base[:, :200, :456]
    outb = torch.full((4, 210, 480), float("nan"), dtype=torch.bfloat16, device="cuda")
    Ov = outb[:, :200, :456]
    for it in (ops.F16, ops.BF16):
        for variant, fn in (("standard", lambda: ops.muon_ns(Gv, out=Ov, iter_dtype=it)),
                            ("gram_stabilized", lambda: ops.gram_ns(Gv, out=Ov, iter_dtype=it))):
            fn()
            torch.cuda.synchronize()
            check_batch(Gv, Ov, variant, TOL["bf16"], f"strided/it{it}/{variant}")
    # nothing outside the view was written
    assert torch.isnan(outb[:, 200:, :].float()).all() and torch.isnan(outb[:, :, 456:].float()).all()


def test_custom_coefficients_and_restart_masks(torch, ops):
    say("case cubic coefficients K=9, restart masks")
    G = synth.lowrank_plus_noise(synth.host_rng(93, 0), 150, 390, 0.5, 0.02)
    Gd = torch.tensor(G, dtype=torch.float32, device="cuda")
    cub = [[1.5, -0.5, 0.0]] * 9
    O = to_np(ops.muon_ns(Gd, steps=9, coeffs=cub))
    ref = oracle.ns_standard(to_np(Gd), coeffs=cub)
    assert rel_fro(O, ref) < 1e-4
    for mask in (0, 1 << 1, (1 << 1) | (1 << 3), 0b11111110):
        restarts = [k for k in range(1, 9) if (mask >> k) & 1]
        O = to_np(ops.gram_ns(Gd, steps=9, coeffs=cub, restart_mask=mask))
        ref = oracle.ns_gram(to_np(Gd), coeffs=cub, restarts=restarts)
        e = rel_fro(O, ref)
        say(f"  mask {mask:#x}: rel_F {e:.2e}")
        assert e < 1e-4
    # single step (K = 1): the first step is also the last
    for io in ("f32", "bf16"):
        Gx = Gd.to(tdtype(torch, io))
        for variant in VARIANTS:
            O = to_np(gpu_fn(ops, variant, steps=1)(Gx))
            ref = oracle.ns_gram(to_np(Gx), steps=1, restarts=()) if variant != "standard" \
                else oracle.ns_standard(to_np(Gx), steps=1)
            assert rel_fro(O, ref) < TOL[io], (io, variant)


# ------------------------------------------------------------------ degenerate inputs

def test_zero_and_nonfinite_inputs_set_flags(torch, ops):
    say("case zero / NaN inputs")
    G = torch.zeros(3, 64, 160, dtype=torch.bfloat16, device="cuda")
    G[1] = torch.tensor(synth.host_rng(98, 0).standard_normal((64, 160)), dtype=torch.bfloat16,
                        device="cuda")
    G[2, 5, 7] = float("nan")
    for variant in VARIANTS:
        flags = torch.full((3,), -1, dtype=torch.int32, device="cuda")
        O = gpu_fn(ops, variant, flags=flags)(G)
        torch.cuda.synchronize()
        f = flags.cpu().tolist()
        assert f[0] == 2 and torch.all(O[0] == 0), (variant, f)
        assert f[1] == 0
        assert f[2] & 1 and f[2] & 4, (variant, f)


def test_deterministic_reruns(torch, ops):
    say("case determinism")
    G = torch.tensor(np.stack([synth.lowrank_plus_noise(synth.host_rng(94, b), 256, 640, 0.7, 0.05)
                               for b in range(2)]), dtype=torch.bfloat16, device="cuda")
    for variant in VARIANTS:
        a = gpu_fn(ops, variant)(G)
        b = gpu_fn(ops, variant)(G)
        torch.cuda.synchronize()
        assert torch.equal(a, b), variant


def test_small_workspace_processes_in_chunks(torch, ops):
    say("case chunked workspace")
    G = torch.tensor(np.stack([synth.lowrank_plus_noise(synth.host_rng(95, b), 100, 260, 0.7, 0.05)
                               for b in range(5)]), dtype=torch.bfloat16, device="cuda")
    for variant, code in (("standard", ops.STANDARD), ("gram_stabilized", ops.GRAM)):
        p = ops.ns_params(io_dtype=ops.BF16, restart_mask=4 if code == ops.GRAM else 0)
        need2 = ops.workspace_bytes(code, G, p, max_batch_chunk=2)
        ws = torch.empty(need2, dtype=torch.uint8, device="cuda")
        fn = ops.muon_ns if code == ops.STANDARD else ops.gram_ns
        O = fn(G, workspace=ws)
        full = fn(G)
        torch.cuda.synchronize()
        assert torch.equal(O, full)
        check_batch(G, O, variant, TOL["bf16"], f"chunked/{variant}")


# ------------------------------------------------------------------ Muon step

@pytest.mark.parametrize("variant", ["standard", "gram_stabilized"])
@pytest.mark.parametrize("wdt", ["bf16", "f32"])
def test_muon_step_two_steps(torch, ops, variant, wdt):
    say(f"case muon_step {variant} W {wdt}")
    B, r, c = 3, 176, 256
    rng = synth.host_rng(96, 0)
    Gs1 = np.stack([synth.lowrank_plus_noise(rng, r, c, 0.7, 0.05) for _ in range(B)])
    Gs2 = np.stack([synth.lowrank_plus_noise(rng, r, c, 0.7, 0.05) for _ in range(B)])
    W0 = 0.02 * rng.standard_normal((B, r, c))
    Wd = torch.tensor(W0, dtype=tdtype(torch, wdt), device="cuda")
    Md = torch.zeros(B, r, c, dtype=torch.float32, device="cuda")
    Ud = torch.empty(B, r, c, dtype=torch.float32, device="cuda")
    W = to_np(Wd)
    M = np.zeros((B, r, c))
    lr, mu, wd = 0.02, 0.95, 0.1
    code = ops.GRAM if variant == "gram_stabilized" else ops.STANDARD
    ns = oracle_fn(variant)
    for step, Gs in enumerate((Gs1, Gs2)):
        Gd = torch.tensor(Gs, dtype=torch.bfloat16, device="cuda")
        ops.muon_step(Wd, Gd, Md, lr=lr, momentum=mu, weight_decay=wd, nesterov=True,
                      variant=code, U_out=Ud)
        torch.cuda.synchronize()
        Gh = to_np(Gd)
        Wg, Mg, Ug = to_np(Wd), to_np(Md), to_np(Ud)
        for b in range(B):
            # the oracle starts from the GPU's stored state each step (N rounded as stored)
            Wn, Mn, Un = oracle.muon_step(W[b], Gh[b], M[b], lr, mu, wd, nesterov=True,
                                          scale_coeff=0.2, ns=ns)
            assert rel_fro(Mg[b], Mn) < 1e-6
            eu = rel_fro(Ug[b], Un)
            assert eu < TOL["bf16"], (step, b, eu)
            # the weight change matches the oracle's to the update tolerance
            dW = np.linalg.norm(Wg[b] - Wn) / np.linalg.norm(lr * Un)
            assert dW < TOL["bf16"], (step, b, dW)
            # and W is the update formula applied to the returned U, rounded once
            ok, frac = w_update_ok(Wg[b], W[b], Ug[b], lr, wd, wdt)
            assert ok, (step, b, frac)
        say(f"  step {step}: worst U rel_F {max(rel_fro(Ug[b], oracle.muon_step(W[b], Gh[b], M[b], lr, mu, wd, True, 0.2, ns)[2]) for b in range(B)):.3e}")
        W, M = Wg, Mg


@pytest.mark.parametrize("variant,dt,nesterov", [("gram_stabilized", "f16", False),
                                                 ("standard", "f32", True),
                                                 ("gram_naive", "bf16", False)])
def test_muon_step_dtypes_and_momentum_forms(torch, ops, variant, dt, nesterov):
    """fp16 and fp32 gradients and weights, plain (non-Nesterov) momentum from a nonzero state,
    and the naive Gram form, on a ragged shape: M, U and W against the oracle's Muon step."""
    say(f"case muon_step {variant} {dt} nesterov={nesterov}")
    B, r, c = 2, 200, 328
    rng = synth.host_rng(99, 0)
    G = np.stack([synth.lowrank_plus_noise(rng, r, c, 0.7, 0.05) for _ in range(B)])
    Wd = torch.tensor(0.02 * rng.standard_normal((B, r, c)), dtype=tdtype(torch, dt), device="cuda")
    Md = torch.tensor(0.1 * rng.standard_normal((B, r, c)), dtype=torch.float32, device="cuda")
    Gd = torch.tensor(G, dtype=tdtype(torch, dt), device="cuda")
    Ud = torch.empty(B, r, c, dtype=torch.float32, device="cuda")
    W, M = to_np(Wd), to_np(Md)
    lr, mu, wd = 0.02, 0.9, 0.05
    code = ops.STANDARD if variant == "standard" else ops.GRAM
    extra = {"restart_mask": 0} if variant == "gram_naive" else {}
    ops.muon_step(Wd, Gd, Md, lr=lr, momentum=mu, weight_decay=wd, nesterov=nesterov,
                  variant=code, U_out=Ud, **extra)
    torch.cuda.synchronize()
    Gh, Wg, Mg, Ug = to_np(Gd), to_np(Wd), to_np(Md), to_np(Ud)
    for b in range(B):
        Wn, Mn, Un = oracle.muon_step(W[b], Gh[b], M[b], lr, mu, wd, nesterov=nesterov,
                                      scale_coeff=0.2, ns=oracle_fn(variant))
        assert rel_fro(Mg[b], Mn) < 1e-6, b
        assert rel_fro(Ug[b], Un) < TOL[dt], (b, rel_fro(Ug[b], Un))
        ok, frac = w_update_ok(Wg[b], W[b], Ug[b], lr, wd, dt)
        assert ok, (b, frac)


def test_muon_step_with_zero_gradient_only_decays(torch, ops):
    """G = 0 and M = 0: N has zero norm, the orthogonalized update is exactly zero (flag bit 1),
    and W only decays: W <- (1 - lr wd) W, rounded once."""
    say("case muon_step zero gradient")
    B, r, c = 2, 96, 160
    rng = synth.host_rng(100, 0)
    W0 = 0.02 * rng.standard_normal((B, r, c))
    for variant, code in (("standard", ops.STANDARD), ("gram_stabilized", ops.GRAM)):
        Wd = torch.tensor(W0, dtype=torch.bfloat16, device="cuda")
        W = to_np(Wd)
        Gd = torch.zeros(B, r, c, dtype=torch.bfloat16, device="cuda")
        Md = torch.zeros(B, r, c, dtype=torch.float32, device="cuda")
        Ud = torch.full((B, r, c), float("nan"), dtype=torch.float32, device="cuda")
        flags = torch.full((B,), -1, dtype=torch.int32, device="cuda")
        ops.muon_step(Wd, Gd, Md, lr=0.02, momentum=0.95, weight_decay=0.1, nesterov=True,
                      variant=code, U_out=Ud, flags=flags)
        torch.cuda.synchronize()
        assert flags.cpu().tolist() == [2, 2], (variant, flags.cpu().tolist())
        assert torch.all(Ud == 0) and torch.all(Md == 0), variant
        ok, frac = w_update_ok(to_np(Wd), W, np.zeros_like(W), 0.02, 0.1, "bf16")
        assert ok, (variant, frac)


def test_muon_step_transposed_orientation(torch, ops):
    say("case muon_step 300 x 120 (rows > cols)")
    rng = synth.host_rng(97, 0)
    G = synth.lowrank_plus_noise(rng, 300, 120, 0.7, 0.05)
    W0 = 0.02 * rng.standard_normal((300, 120))
    Wd = torch.tensor(W0, dtype=torch.float32, device="cuda")
    Gd = torch.tensor(G, dtype=torch.bfloat16, device="cuda")
    Md = torch.zeros(300, 120, dtype=torch.float32, device="cuda")
    Ud = torch.empty(300, 120, dtype=torch.bfloat16, device="cuda")
    ops.muon_step(Wd, Gd, Md, lr=0.05, momentum=0.9, weight_decay=0.01, nesterov=False,
                  variant=ops.GRAM, U_out=Ud)
    torch.cuda.synchronize()
    Wn, Mn, Un = oracle.muon_step(W0, to_np(Gd), np.zeros((300, 120)), 0.05, 0.9, 0.01,
                                  nesterov=False, ns=oracle_fn("gram_stabilized"))
    assert rel_fro(to_np(Ud), Un) < 2e-2
    assert np.linalg.norm(to_np(Wd) - Wn) / np.linalg.norm(0.05 * Un) < 2e-2


@pytest.mark.parametrize("shape,wdt", [((6, 256, 512), "bf16"), ((4, 512, 256), "bf16"), ((3, 264, 520), "f16"),
                                       ((2, 256, 768), "f32"),
                                       # large enough for the 256 x 256 tiles: W row pass and,
                                       # for the tall batch, the transposed column pass
                                       ((24, 1000, 1512), "bf16"), ((24, 1512, 1000), "bf16")])
def test_muon_step_weight_update_without_u_out(torch, ops, shape, wdt):
    """Without U_out the last product updates W in its own epilogue; it must agree with the
    path that also writes U (to one unit in the last place of W) and flag non-finite outputs.
    U of the first matrix is checked against the oracle's Muon step."""
    say(f"case muon_step W update without U_out {shape} {wdt}")
    B, r, c = shape
    dt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[wdt]
    G = synth.torch_lowrank_plus_noise(B, r, c, power=0.7, noise=0.05, workload_index=1,
                                       seed_offset=31, device="cuda").to(dt if wdt != "f32" else torch.bfloat16)
    W0 = synth.torch_weights(B, r, c, workload_index=1, device="cuda", dtype=dt)
    kw = dict(lr=0.02, momentum=0.95, weight_decay=0.1, nesterov=True, scale_coeff=0.2, variant=ops.GRAM)
    W1, W2 = W0.clone(), W0.clone()
    M1 = torch.zeros(shape, dtype=torch.float32, device="cuda")
    M2 = M1.clone()
    U = torch.empty(shape, dtype=torch.float32, device="cuda")
    ops.muon_step(W1, G, M1, U_out=U, **kw)
    ops.muon_step(W2, G, M2, **kw)
    torch.cuda.synchronize()
    assert torch.equal(M1, M2)
    a, b, w0, u = (t.double().cpu().numpy() for t in (W1, W2, W0, U))
    # both paths evaluate the same expressions; the compiler may contract them into fused
    # multiply-adds differently, which moves the fp32 result by a few roundings of its operands
    # and the stored W by at most one unit in its last place
    mant = {"bf16": 7, "f16": 10, "f32": 23}[wdt]
    e = np.floor(np.log2(np.maximum(np.maximum(np.abs(a), np.abs(b)), 2.0 ** -14)))
    tol = 2.0 ** (e - mant) + 4 * 2.0 ** -24 * ((1 - 0.02 * 0.1) * np.abs(w0) + 0.02 * np.abs(u))
    assert np.all(np.abs(a - b) <= tol), float(np.max(np.abs(a - b) / tol))
    _, _, Un = oracle.muon_step(np.zeros((r, c)), to_np(G[0]), np.zeros((r, c)), 0.02, 0.95, 0.1,
                                nesterov=True, scale_coeff=0.2, ns=lambda x: oracle.ns_gram(x, restarts=(2,)))
    assert rel_fro(u[0], Un) < 2e-2
    # a NaN in one gradient: that matrix's flags report the non-finite output
    G[1, 3, 5] = float("nan")
    flags = torch.zeros(B, dtype=torch.int32, device="cuda")
    ops.muon_step(W2, G, M2, flags=flags, **kw)
    torch.cuda.synchronize()
    f = flags.cpu().tolist()
    assert f[1] & 4 and f[1] & 1 and f[0] == 0
