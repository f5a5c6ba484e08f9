"""Parity at the workloads' full sizes, in the launch configuration the bench uses.

* expert batch 64 x 1408 x 2048 bf16: two fused Muon steps (Nesterov, mu 0.95, lr 2e-4,
  wd 0.1, scale 0.2 sqrt(2048)); sampled matrices checked against the oracle.
* Kimi-K2 expert batch 648 x 2048 x 7168 bf16 (the bench's workload, whole batch in one
  workspace chunk): sampled matrices against the oracle for both variants.
* Kimi-K2 dense 3 x 7168 x 18432 bf16: its own seeded input (power law i^-0.5 plus 0.05
  noise) against the oracle element by element, and a power-law input with a known SVD built
  from Kronecker products of small orthogonal factors, sampled output entries against the
  closed form U p(S) V^T (a property that holds at any size).
"""
import math

import numpy as np
import pytest

import oracle
import synth
from helpers import band_ok, band_ok_gram, bf16_steps, gram_singular_range, rel_fro, say, to_np, w_update_ok

pytestmark = pytest.mark.gpu
TOL = 2e-2


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


@pytest.mark.parametrize("variant", ["standard", "gram_stabilized"])
def test_expert_batch_1408x2048_muon_step(torch, ops, variant):
    say(f"case expert 64x1408x2048 muon_step {variant}")
    B, r, c = 64, 1408, 2048
    code = ops.GRAM if variant == "gram_stabilized" else ops.STANDARD
    ns = (lambda x: oracle.ns_gram(x, restarts=(2,))) if code == ops.GRAM else oracle.ns_standard
    W = synth.torch_weights(B, r, c, workload_index=1, device="cuda")
    M = torch.zeros(B, r, c, dtype=torch.float32, device="cuda")
    U = torch.empty(B, r, c, dtype=torch.float32, device="cuda")
    lr, mu, wd = 2e-4, 0.95, 0.1
    picks = [0, 37, 63]
    Wh = {b: to_np(W[b]) for b in picks}
    Mh = {b: np.zeros((r, c)) for b in picks}
    for step in range(2):
        G = synth.torch_lowrank_plus_noise(B, r, c, power=0.7, noise=0.05, workload_index=1,
                                           seed_offset=1000 * step, device="cuda")
        ops.muon_step(W, G, M, lr=lr, momentum=mu, weight_decay=wd, nesterov=True,
                      scale_coeff=0.2, variant=code, U_out=U)
        torch.cuda.synchronize()
        for b in picks:
            Wn, Mn, Un = oracle.muon_step(Wh[b], to_np(G[b]), Mh[b], lr, mu, wd, nesterov=True,
                                          scale_coeff=0.2, ns=ns)
            Ug, Wg, Mg = to_np(U[b]), to_np(W[b]), to_np(M[b])
            e = rel_fro(Ug, Un)
            ok, info = band_ok(Ug, Un, TOL)
            say(f"  step {step} matrix {b}: U rel_F {e:.3e}, band {info}")
            assert e <= TOL and ok
            assert rel_fro(Mg, Mn) < 1e-6
            # bf16 weights: the update applied to the returned U, rounded once ...
            ok, frac = w_update_ok(Wg, Wh[b], Ug, lr, wd, "bf16")
            assert ok, f"W update off at step {step}: {frac:.2e} of entries"
            # ... and the oracle's weights up to one bf16 step plus lr |U - U_oracle| (the
            # update's own deviation, bounded by the U check above)
            big = np.maximum(np.abs(Wn), np.abs(Wg)).astype(np.float32)
            ulp = np.spacing(big).astype(np.float64) * 2 ** 16
            dev = np.abs(Wg - Wn) - lr * np.abs(Ug - Un)
            say(f"    W: {np.mean(bf16_steps(Wg, Wn) == 0):.4f} of entries equal to the oracle's rounded W")
            assert np.all(dev <= ulp + 1e-12)
            Wh[b], Mh[b] = Wg, Mg


# Matrices on both sides of the boundaries where the persistent tile walk of the 648-matrix
# batch hands over from one XCD's share of the tile list to the next (648 / 8 = 81 matrices per
# share), plus the first and the last matrix.
K2_PICKS = [0, 80, 81, 161, 162, 323, 324, 647]


def w_frobenius_bound_ok(Wg, Wn, Un, lr, tol):
    """W after a step, against the oracle's fp64 W: the GPU's W is the exact update rounded once
    to bf16 with its own U, so ||W_gpu - W_oracle||_F <= ||half a bf16 step of W||_F +
    lr ||U_gpu - U_oracle||_F, and the second term is at most lr tol ||U_oracle||_F when U meets
    the tolerance. Returns (ok, lhs, rhs)."""
    big = np.maximum(np.abs(Wn), np.abs(Wg)).astype(np.float32)
    half_ulp = 0.5 * np.spacing(big).astype(np.float64) * 2 ** 16
    lhs = float(np.linalg.norm(Wg - Wn))
    rhs = float(np.linalg.norm(half_ulp) + lr * tol * np.linalg.norm(Un)) * (1 + 1e-6)
    return lhs <= rhs, lhs, rhs


def test_k2_expert_batch_timed_muon_step(torch, ops):
    """The exact call the bench times: muon_step over 648 x 2048 x 7168 bf16 with stabilized
    Gram NS, Nesterov momentum, bf16 W, fp32 M, the bench's workspace, no U_out and no flags
    (so the last product updates W in its typed weight-update epilogue on the persistent
    grid). Two steps, the second from the nonzero momentum the first left; W and M of the
    matrices at the XCD-share boundaries against the oracle's Muon step."""
    B, r, c = 648, 2048, 7168
    say(f"case k2 experts {B}x{r}x{c}: timed muon_step call, generating")
    G1 = synth.torch_gaussian_plus_spike(B, r, c, workload_index=2, device="cuda")
    G2 = synth.torch_gaussian_plus_spike(B, r, c, workload_index=12, device="cuda")
    W = synth.torch_weights(B, r, c, workload_index=2, device="cuda", seed_offset=500_000)
    M = torch.zeros(B, r, c, dtype=torch.float32, device="cuda")
    p_g = ops.ns_params(io_dtype=ops.BF16, restart_mask=1 << 2)
    p_s = ops.ns_params(io_dtype=ops.BF16, restart_mask=0)
    ws = torch.empty(max(ops.workspace_bytes(ops.GRAM, G1, p_g),
                         ops.workspace_bytes(ops.STANDARD, G1, p_s)), dtype=torch.uint8, device="cuda")
    kw = dict(lr=0.02, momentum=0.95, weight_decay=0.01, scale_coeff=0.2, nesterov=True)
    ns = lambda x: oracle.ns_gram(x, restarts=(2,))
    Wh = {b: to_np(W[b]) for b in K2_PICKS}
    Mh = {b: np.zeros((r, c)) for b in K2_PICKS}
    for step, G in enumerate((G1, G2)):
        say(f"  step {step}: muon_step on the whole batch")
        ops.muon_step(W, G, M, variant=ops.GRAM, workspace=ws, **kw)
        torch.cuda.synchronize()
        for b in K2_PICKS:
            Wn, Mn, Un = oracle.muon_step(Wh[b], to_np(G[b]), Mh[b], kw["lr"], kw["momentum"],
                                          kw["weight_decay"], nesterov=True, scale_coeff=0.2, ns=ns)
            Wg, Mg = to_np(W[b]), to_np(M[b])
            ok, lhs, rhs = w_frobenius_bound_ok(Wg, Wn, Un, kw["lr"], TOL)
            em = rel_fro(Mg, Mn)
            say(f"    matrix {b}: ||W - W_oracle||_F {lhs:.4e} (bound {rhs:.4e}), M rel_F {em:.2e}")
            assert ok
            assert em < 1e-6
            assert bool(torch.isfinite(W[b].float()).all())
            Wh[b], Mh[b] = Wg, Mg


def test_k2_expert_batch_648x2048x7168_sampled(torch, ops):
    B, r, c = 648, 2048, 7168
    say(f"case k2 experts {B}x{r}x{c}: generating")
    G = synth.torch_gaussian_plus_spike(B, r, c, workload_index=2, device="cuda")
    p_g = ops.ns_params(io_dtype=ops.BF16, restart_mask=1 << 2)
    p_s = ops.ns_params(io_dtype=ops.BF16, restart_mask=0)
    ws = torch.empty(max(ops.workspace_bytes(ops.GRAM, G, p_g),
                         ops.workspace_bytes(ops.STANDARD, G, p_s)), dtype=torch.uint8, device="cuda")
    O = torch.empty_like(G)
    flags = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    picks = K2_PICKS
    Gh = {b: to_np(G[b]) for b in picks}
    for variant in ("gram_stabilized", "standard"):
        say(f"  running {variant} on the whole batch")
        if variant == "standard":
            ops.muon_ns(G, out=O, workspace=ws, flags=flags)
            ref_fn = oracle.ns_standard
        else:
            ops.gram_ns(G, out=O, workspace=ws, flags=flags)
            ref_fn = lambda x: oracle.ns_gram(x, restarts=(2,))
        torch.cuda.synchronize()
        assert int(flags.abs().sum()) == 0, "flags raised"
        assert bool(torch.isfinite(O.float()).all())
        for b in picks:
            ref = ref_fn(Gh[b])
            got = to_np(O[b])
            e = rel_fro(got, ref)
            ok, info = band_ok(got, ref, TOL)
            say(f"  {variant} matrix {b}: rel_F {e:.3e}, band {info}")
            assert e <= TOL and ok


@pytest.fixture(scope="module")
def dense_ffn(torch):
    """The dense FFN batch as the bench generates it: 3 x 7168 x 18432 bf16, U diag(i^-0.5) V^T
    plus 0.05 N(0, 1) noise, normalised. The fp64 reference of matrix 0 (the oracle's stabilized
    Gram iteration on the stored bf16 values; in fp64 the standard and Gram forms agree to
    ~1e-12, which the oracle's own tests pin) and its singular-value range are computed once."""
    n, m = 7168, 18432
    say(f"case k2 dense 3x{n}x{m} power law + noise: generating")
    G = synth.torch_lowrank_plus_noise(3, n, m, power=0.5, noise=0.05, workload_index=3,
                                       device="cuda", chunk=1)
    G0 = to_np(G[0])
    say("  oracle on matrix 0 (fp64, host)")
    ref = oracle.ns_gram(G0, restarts=(2,))
    rng_ = gram_singular_range(ref)
    return G, ref, rng_


@pytest.mark.timeout(900)
@pytest.mark.parametrize("variant", ["gram_stabilized", "standard"])
def test_k2_dense_3x7168x18432_own_input(torch, ops, dense_ffn, variant):
    """The dense FFN batch on its own input, in the bench's launch configuration (all three
    matrices in one call): matrix 0 against the fp64 oracle element by element (relative
    Frobenius error) and the band of its singular values."""
    G, ref, ref_range = dense_ffn
    say(f"  dense FFN {variant}")
    flags = torch.zeros(3, dtype=torch.int32, device="cuda")
    O = ops.gram_ns(G, flags=flags) if variant != "standard" else ops.muon_ns(G, flags=flags)
    torch.cuda.synchronize()
    assert int(flags.abs().sum()) == 0
    assert bool(torch.isfinite(O.float()).all())
    got = to_np(O[0])
    e = rel_fro(got, ref)
    ok, info = band_ok_gram(got, ref, TOL, ref_range)
    say(f"  {variant} matrix 0: rel_F {e:.3e}, band {info}")
    assert e <= TOL and ok


@pytest.mark.parametrize("variant", ["standard", "gram_stabilized"])
def test_expert_batch_1408x2048_bf16_iterates(torch, ops, variant):
    """The expert batch with every iterate stored in bf16 (64 x 1408 x 2048, the input as the
    workload defines it), NS alone on the whole batch; sampled matrices against the oracle.
    The library's default for bf16 input keeps the normalised iterates in fp16."""
    say(f"case expert 64x1408x2048 bf16 iterates {variant}")
    B, r, c = 64, 1408, 2048
    G = synth.torch_lowrank_plus_noise(B, r, c, power=0.7, noise=0.05, workload_index=1,
                                       device="cuda")
    if variant == "standard":
        O = ops.muon_ns(G, iter_dtype=ops.BF16)
        ns = oracle.ns_standard
    else:
        O = ops.gram_ns(G, iter_dtype=ops.BF16)
        ns = lambda x: oracle.ns_gram(x, restarts=(2,))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(O.float()).all())
    for b in (0, 37, 63):
        ref = ns(to_np(G[b]))
        e = rel_fro(to_np(O[b]), ref)
        ok, info = band_ok(to_np(O[b]), ref, TOL)
        say(f"  matrix {b}: rel_F {e:.3e}, band {info}")
        assert e <= TOL and ok


def test_k2_dense_3x7168x18432_structured(torch, ops):
    n, m = 7168, 18432
    say(f"case k2 dense 3x{n}x{m} with known SVD")
    spec = np.arange(1, n + 1, dtype=np.float64) ** -0.5
    rng = np.random.default_rng([3, 7])
    facs, Gs = [], torch.empty(3, n, m, dtype=torch.bfloat16, device="cuda")
    for b in range(3):
        Ua = synth.orthonormal(rng, 56, 56); Ub = synth.orthonormal(rng, 128, 128)
        Va = synth.orthonormal(rng, 144, 144); Vb = synth.orthonormal(rng, 128, 128)
        Ut = torch.kron(torch.tensor(Ua, device="cuda"), torch.tensor(Ub, device="cuda")).float()
        Vt = torch.kron(torch.tensor(Va, device="cuda"), torch.tensor(Vb, device="cuda"))[:, :n].float()
        st = torch.tensor(spec, device="cuda").float()
        Gs[b] = torch.matmul(Ut * st, Vt.t().contiguous()).to(torch.bfloat16)
        del Ut, Vt
        facs.append((Ua, Ub, Va, Vb))
    torch.cuda.synchronize()
    sel = np.random.default_rng(11)
    rows = np.sort(sel.choice(n, 48, replace=False))
    cols = np.sort(sel.choice(m, 48, replace=False))
    for variant in ("gram_stabilized", "standard"):
        O = ops.gram_ns(Gs) if variant != "standard" else ops.muon_ns(Gs)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(O.float()).all())
        for b in range(3):
            Ua, Ub, Va, Vb = facs[b]
            Ur = np.stack([np.kron(Ua[i // 128], Ub[i % 128]) for i in rows])
            Vr = np.stack([np.kron(Va[j // 128], Vb[j % 128])[:n] for j in cols])
            nrm = float(torch.linalg.vector_norm(Gs[b].double()).item())
            ref = oracle.ns_closed_form_entries(Ur, spec, Vr, fro_norm=nrm)
            got = to_np(O[b][torch.tensor(rows, device="cuda")][:, torch.tensor(cols, device="cuda")])
            e = rel_fro(got, ref)
            say(f"  {variant} matrix {b}: sampled-entry rel_F {e:.3e}")
            assert e <= TOL


def test_largest_accepted_matrix_32768x32768_structured(torch, ops):
    """The largest matrix the library accepts: one n x m iterate of exactly 2^31 bytes
    (32768 x 32768 bf16), where byte offsets reach the top of the 32-bit range and the
    out-of-range sentinel equals the operand size. Known SVD (Kronecker factors), sampled
    entries against the closed form, both variants."""
    n = 32768
    say(f"case largest matrix 1x{n}x{n} with known SVD")
    spec = np.arange(1, n + 1, dtype=np.float64) ** -0.5
    rng = np.random.default_rng([3, 9])
    Ua = synth.orthonormal(rng, 128, 128); Ub = synth.orthonormal(rng, 256, 256)
    Va = synth.orthonormal(rng, 128, 128); Vb = synth.orthonormal(rng, 256, 256)
    f32 = dict(dtype=torch.float32, device="cuda")
    Ut = torch.kron(torch.tensor(Ua, **f32), torch.tensor(Ub, **f32))
    Vt = torch.kron(torch.tensor(Va, **f32), torch.tensor(Vb, **f32))
    st = torch.tensor(spec, **f32)
    G = torch.matmul(Ut * st, Vt.t().contiguous()).to(torch.bfloat16).unsqueeze(0)
    del Ut, Vt
    nrm = float(sum(float((G[0, i:i + 2048].double() ** 2).sum()) for i in range(0, n, 2048)) ** 0.5)
    torch.cuda.synchronize()
    sel = np.random.default_rng(12)
    rows = np.sort(sel.choice(n, 48, replace=False))
    cols = np.sort(sel.choice(n, 48, replace=False))
    Ur = np.stack([np.kron(Ua[i // 256], Ub[i % 256]) for i in rows])
    Vr = np.stack([np.kron(Va[j // 256], Vb[j % 256]) for j in cols])
    ref = oracle.ns_closed_form_entries(Ur, spec, Vr, fro_norm=nrm)
    for variant in ("gram_stabilized", "standard"):
        flags = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        O = ops.gram_ns(G, flags=flags) if variant != "standard" else ops.muon_ns(G, flags=flags)
        torch.cuda.synchronize()
        assert int(flags.item()) == 0, (variant, int(flags.item()))
        got = to_np(O[0][torch.tensor(rows, device="cuda")][:, torch.tensor(cols, device="cuda")])
        e = rel_fro(got, ref)
        say(f"  {variant}: sampled-entry rel_F {e:.3e}")
        assert e <= TOL
        del O
    torch.cuda.empty_cache()


@pytest.mark.parametrize("variant", ["standard", "gram_stabilized"])
@pytest.mark.parametrize("shape", [(24, 1000, 1500), (24, 1500, 1000)])
def test_ragged_batch_on_the_large_tile_path(torch, ops, variant, shape):
    """n = 1000 (a k tail inside a 64-wide k-stage) and m = 1500 (not a multiple of 8 or of the
    256-wide tile), large enough that the rectangular products take the 256 x 256 DMA kernel
    with X read k-major; both orientations. Sampled matrices against the oracle."""
    say(f"case ragged large-tile {shape} {variant}")
    B, r, c = shape
    n, m = min(r, c), max(r, c)
    assert B * math.ceil(n / 256) * math.ceil(m / 256) >= 512      # the 256-tile policy applies
    code = ops.GRAM if variant == "gram_stabilized" else ops.STANDARD
    ns = (lambda x: oracle.ns_gram(x, restarts=(2,))) if code == ops.GRAM else oracle.ns_standard
    G = synth.torch_lowrank_plus_noise(B, r, c, power=0.7, noise=0.05, workload_index=1,
                                       seed_offset=4242, device="cuda")
    O = ops.gram_ns(G) if code == ops.GRAM else ops.muon_ns(G)
    torch.cuda.synchronize()
    assert O.shape == G.shape
    for b in (0, B - 1):
        ref = ns(to_np(G[b]))
        e = rel_fro(to_np(O[b]), ref)
        ok, info = band_ok(to_np(O[b]), ref, TOL)
        say(f"  matrix {b}: rel_F {e:.3e}, band {info}")
        assert e <= TOL and ok


@pytest.mark.parametrize("variant", ["standard", "gram_stabilized"])
def test_expert_batch_relative_noise(torch, ops, variant):
    """The second reading of the expert batch's noise: 0.05 of the signal's Frobenius norm
    instead of 0.05 N(0, 1) per entry, which keeps the i^-0.7 spectrum above the noise (the
    harder case: singular values spread over three decades). 64 x 1408 x 2048 bf16, NS alone;
    sampled matrices against the oracle."""
    say(f"case expert 64x1408x2048 relative noise {variant}")
    B, r, c = 64, 1408, 2048
    code = ops.GRAM if variant == "gram_stabilized" else ops.STANDARD
    ns = (lambda x: oracle.ns_gram(x, restarts=(2,))) if code == ops.GRAM else oracle.ns_standard
    G = synth.torch_lowrank_plus_noise(B, r, c, power=0.7, noise=0.05, workload_index=1,
                                       seed_offset=5000, device="cuda", relative=True)
    O = ops.gram_ns(G) if code == ops.GRAM else ops.muon_ns(G)
    torch.cuda.synchronize()
    for b in (0, 41):
        ref = ns(to_np(G[b]))
        e = rel_fro(to_np(O[b]), ref)
        ok, info = band_ok(to_np(O[b]), ref, TOL)
        say(f"  matrix {b}: rel_F {e:.3e}, band {info}")
        assert e <= TOL and ok
