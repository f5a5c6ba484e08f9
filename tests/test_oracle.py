"""Pins for the fp64 oracle against facts fixed by the pages and by the mathematics.

Nothing here compares the oracle with a copy of itself: each pin is a closed form
(the SVD of the input, exact rational arithmetic), a textbook limit (the polar
factor), a special case checkable by hand, or an identity between two different
formulations (odd polynomial in X versus polynomial in X X^T times X).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import ns as ons

HERE = os.path.dirname(os.path.abspath(__file__))
QUINTIC = (Fraction(34445, 10000), Fraction(-47750, 10000), Fraction(20315, 10000))


def exact_scalar_map(x: Fraction, steps=5, coeffs=QUINTIC) -> Fraction:
    """p_K(...p_1(x)) in exact rational arithmetic, p(s) = a s + b s^3 + c s^5."""
    a, b, c = coeffs
    for _ in range(steps):
        x = a * x + b * x ** 3 + c * x ** 5
    return x


def spectral_closed_form(G, steps=5, coeffs=(3.4445, -4.7750, 2.0315), eps=0.0):
    """U diag(p^K(s / (||G||_F + eps))) V^T from numpy's SVD, scalar map by plain loop."""
    U, s, Vt = np.linalg.svd(np.asarray(G, dtype=np.float64), full_matrices=False)
    x = s / (np.sqrt((s ** 2).sum()) + eps)
    a, b, c = coeffs
    for _ in range(steps):
        x = a * x + b * x ** 3 + c * x ** 5
    return (U * x) @ Vt


def rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


@pytest.fixture(params=[(24, 56), (56, 24), (32, 32), (7, 91)])
def G(request):
    rng = np.random.default_rng(1234 + sum(request.param))
    r, c = request.param
    return rng.standard_normal((r, c))


# ------------------------------------------------------------------ closed forms

def test_standard_matches_svd_closed_form(G):
    out = oracle.ns_standard(G, eps=0.0)
    assert out.shape == G.shape
    assert rel(out, spectral_closed_form(G)) < 1e-10


def test_gram_naive_and_stabilized_match_svd_closed_form(G):
    ref = spectral_closed_form(G)
    assert rel(oracle.ns_gram(G, eps=0.0, restarts=()), ref) < 1e-10
    assert rel(oracle.ns_gram(G, eps=0.0, restarts=(2,)), ref) < 1e-10
    assert rel(oracle.ns_gram(G, eps=0.0, restarts=(1, 3)), ref) < 1e-10


def test_closed_form_helper_matches_independent_spectral_map(G):
    assert rel(oracle.ns_svd_closed_form(G, eps=0.0), spectral_closed_form(G)) < 1e-12
    assert rel(oracle.ns_svd_closed_form(G, eps=1e-7), spectral_closed_form(G, eps=1e-7)) < 1e-12


def test_eps_is_added_to_the_frobenius_norm():
    rng = np.random.default_rng(5)
    G = 1e-6 * rng.standard_normal((8, 20))     # ||G|| ~ 1.3e-5, so eps = 1e-7 is visible
    for eps in (1e-7, 1e-6):
        assert rel(oracle.ns_standard(G, eps=eps), spectral_closed_form(G, eps=eps)) < 1e-10
    assert rel(oracle.ns_standard(G, eps=1e-7), spectral_closed_form(G, eps=0.0)) > 1e-4


def test_polar_limit_with_the_pages_cubic():
    """The guide's cubic 0.5 X (3I - X^T X) drives every singular value to 1: after many
    steps the output is the polar factor U V^T (guide, 'The Promise and Pitfalls of Matrix
    Orthogonalization': every singular value of the update equals 1)."""
    consts = json.load(open(os.path.join(HERE, "golden", "pages_constants.json")))
    cub = consts["cubic_iteration"]
    triple = (cub["a"], cub["b"], cub["c"])
    rng = np.random.default_rng(77)
    for (r, c) in [(16, 40), (40, 16), (20, 20)]:
        U0 = np.linalg.qr(rng.standard_normal((r, min(r, c))))[0]
        V0 = np.linalg.qr(rng.standard_normal((c, min(r, c))))[0]
        s = np.linspace(1.0, 0.05, min(r, c))
        G = (U0 * s) @ V0.T
        polar = U0 @ V0.T
        for fn in (oracle.ns_standard, lambda g, **k: oracle.ns_gram(g, restarts=(), **k),
                   lambda g, **k: oracle.ns_gram(g, restarts=(2,), **k)):
            out = fn(G, coeffs=oracle.default_coeffs(40, triple), eps=0.0)
            assert np.abs(out - polar).max() < 1e-12


def test_cubic_step_is_the_guides_half_three_identity_minus_gram():
    """One step with (1.5, -0.5, 0) equals the guide's listing: A = X X^T, B = 0.5 (3I - A), X <- B X."""
    rng = np.random.default_rng(3)
    G = rng.standard_normal((12, 30))
    X0 = G / np.linalg.norm(G)
    B = 0.5 * (3.0 * np.eye(12) - X0 @ X0.T)
    out = oracle.ns_standard(G, coeffs=[[1.5, -0.5, 0.0]], eps=0.0)
    assert np.abs(out - B @ X0).max() < 1e-15


# ------------------------------------------------------------------ special cases

def test_single_row_input_is_scaled_direction():
    g = np.random.default_rng(9).standard_normal((1, 300))
    p5 = float(exact_scalar_map(Fraction(1)))
    assert abs(p5 - 0.6964364094697522) < 1e-15
    out = oracle.ns_standard(g, eps=0.0)
    assert np.abs(out - p5 * g / np.linalg.norm(g)).max() < 1e-15
    out_t = oracle.ns_standard(g.T, eps=0.0)       # 300 x 1: transposed internally
    assert np.abs(out_t - p5 * g.T / np.linalg.norm(g)).max() < 1e-15
    assert np.abs(oracle.ns_gram(g, eps=0.0) - out).max() < 1e-15


def test_orthonormal_rows_map_to_a_multiple_of_themselves():
    n, m = 128, 512
    rng = np.random.default_rng(11)
    G = np.linalg.qr(rng.standard_normal((m, n)))[0].T     # n x m, orthonormal rows
    # p^5(1/sqrt(128)) in exact rational arithmetic from a 1e-15-close rational of 1/sqrt(128)
    fac = float(exact_scalar_map(Fraction(1.0 / math.sqrt(n)).limit_denominator(10 ** 15)))
    assert abs(fac - 0.7227621604452805) < 1e-12
    for out in (oracle.ns_standard(G, eps=0.0), oracle.ns_gram(G, eps=0.0, restarts=()),
                oracle.ns_gram(G, eps=0.0, restarts=(2,))):
        assert np.abs(out - fac * G).max() < 1e-13


def test_diagonal_and_permuted_inputs_act_elementwise():
    d = np.array([3.0, -1.0, 0.5, 2.0, -0.25, 1e-3])
    n = d.size
    G = np.zeros((n, 10))
    G[np.arange(n), np.arange(n)] = d
    nrm = np.linalg.norm(d)
    expect = np.zeros_like(G)
    for i, di in enumerate(d):
        expect[i, i] = math.copysign(float(exact_scalar_map(Fraction(abs(di) / nrm))), di)
    for fn in (oracle.ns_standard, oracle.ns_gram):
        assert np.abs(fn(G, eps=0.0) - expect).max() < 1e-14
    # row and column permutations are carried through
    pr = np.random.default_rng(2).permutation(n)
    pc = np.random.default_rng(3).permutation(10)
    Gp = G[pr][:, pc]
    assert np.abs(oracle.ns_standard(Gp, eps=0.0) - expect[pr][:, pc]).max() < 1e-14


def test_zero_matrix_gives_zero():
    Z = np.zeros((5, 9))
    assert np.all(oracle.ns_standard(Z) == 0.0)
    assert np.all(oracle.ns_gram(Z) == 0.0)
    assert np.all(oracle.ns_gram(Z, restarts=()) == 0.0)


# ------------------------------------------------------------------ Gram identity

def test_one_gram_step_equals_one_standard_step():
    """a X + b (X X^T) X + c (X X^T)^2 X == (a I + b R + c R^2) X with R = X X^T."""
    rng = np.random.default_rng(21)
    G = rng.standard_normal((10, 33))
    for k in (1, 2, 3):
        c = oracle.default_coeffs(k)
        assert rel(oracle.ns_gram(G, coeffs=c, eps=0.0, restarts=()),
                   oracle.ns_standard(G, coeffs=c, eps=0.0)) < 1e-13


def test_traced_gram_matrices_are_the_iterates_gram():
    rng = np.random.default_rng(22)
    G = rng.standard_normal((9, 27))
    trace = []
    oracle.ns_gram(G, eps=0.0, restarts=(), trace=trace)
    for k in range(1, 5):
        Xk = oracle.ns_standard(G, coeffs=oracle.default_coeffs(k), eps=0.0)
        assert rel(trace[k - 1], Xk @ Xk.T) < 1e-12


def test_restart_set_does_not_change_the_exact_result():
    rng = np.random.default_rng(23)
    G = rng.standard_normal((16, 48))
    base = oracle.ns_standard(G, eps=1e-7)
    for rs in [(), (1,), (2,), (3,), (1, 2, 3, 4), (4,)]:
        assert rel(oracle.ns_gram(G, eps=1e-7, restarts=rs), base) < 1e-12


def test_all_forms_reach_the_closed_form_on_a_wide_log_uniform_spectrum():
    """Singular values spread over six decades (the stability sweep's inputs): in fp64 the
    standard, naive Gram and stabilized Gram iterations all equal U p^K(S) V^T."""
    import synth
    G = synth.loguniform_spectrum(synth.host_rng(4, 999), 96, 384)
    ref = spectral_closed_form(G, eps=1e-7)
    assert rel(oracle.ns_standard(G), ref) < 1e-11
    assert rel(oracle.ns_gram(G, restarts=()), ref) < 1e-11
    assert rel(oracle.ns_gram(G, restarts=(2,)), ref) < 1e-11


# ------------------------------------------------------------------ invariants

def test_odd_scale_transpose_and_orthogonal_equivariance():
    rng = np.random.default_rng(31)
    G = rng.standard_normal((14, 35))
    O = oracle.ns_standard(G, eps=0.0)
    assert np.abs(oracle.ns_standard(-G, eps=0.0) + O).max() < 1e-14
    assert rel(oracle.ns_standard(7.5 * G, eps=0.0), O) < 1e-13
    assert np.abs(oracle.ns_standard(G.T, eps=0.0) - O.T).max() < 1e-14
    P = np.linalg.qr(rng.standard_normal((14, 14)))[0]
    Wm = np.linalg.qr(rng.standard_normal((35, 35)))[0]
    assert rel(oracle.ns_standard(P @ G @ Wm, eps=0.0), P @ O @ Wm) < 1e-12


def test_output_singular_values_are_the_scalar_map():
    rng = np.random.default_rng(32)
    G = rng.standard_normal((20, 50))
    s = np.linalg.svd(G, compute_uv=False)
    so = np.linalg.svd(oracle.ns_gram(G, eps=0.0), compute_uv=False)
    expect = np.sort([float(exact_scalar_map(Fraction(float(v)))) for v in s / np.linalg.norm(s)])
    assert np.abs(np.sort(so) - expect).max() < 1e-12


# ------------------------------------------------------------------ Muon step

def test_muon_step_from_zero_state():
    rng = np.random.default_rng(41)
    W = 0.02 * rng.standard_normal((12, 40))
    G = rng.standard_normal((12, 40))
    mu, lr, wd = 0.95, 0.02, 0.01
    for nesterov in (False, True):
        Wn, Mn, U = oracle.muon_step(W, G, np.zeros_like(G), lr=lr, momentum=mu,
                                     weight_decay=wd, nesterov=nesterov,
                                     ns=lambda x: oracle.ns_standard(x, eps=0.0))
        assert np.abs(Mn - (1 - mu) * G).max() < 1e-15
        O = spectral_closed_form(G)
        assert rel(U, 0.2 * math.sqrt(40) * O) < 1e-10
        assert rel(Wn, (1 - lr * wd) * W - lr * 0.2 * math.sqrt(40) * O) < 1e-10


def test_muon_step_lr_zero_and_weight_decay_only():
    rng = np.random.default_rng(42)
    W = rng.standard_normal((6, 8))
    G = rng.standard_normal((6, 8))
    Wn, _, _ = oracle.muon_step(W, G, np.zeros_like(G), lr=0.0, momentum=0.9, weight_decay=0.3)
    assert np.array_equal(Wn, W)
    Wn, Mn, U = oracle.muon_step(W, np.zeros_like(G), np.zeros_like(G), lr=0.1,
                                 momentum=0.9, weight_decay=0.3)
    assert np.all(U == 0) and np.all(Mn == 0)
    assert np.array_equal(Wn, (1 - 0.1 * 0.3) * W)


def test_ema_and_sum_momentum_give_the_same_update_direction():
    rng = np.random.default_rng(43)
    G1, G2 = rng.standard_normal((2, 10, 30))
    mu = 0.9
    ns = lambda x: oracle.ns_standard(x, eps=0.0)
    W = np.zeros((10, 30))
    _, M1, _ = oracle.muon_step(W, G1, np.zeros_like(G1), 0.0, mu, 0.0, ns=ns)
    _, _, U_ema = oracle.muon_step(W, G2, M1, 0.0, mu, 0.0, ns=ns)
    M_sum = mu * G1 + G2                         # sum form M <- mu M + G
    assert rel(U_ema, 0.2 * math.sqrt(30) * ns(M_sum)) < 1e-12


def test_update_rms_is_scale_coeff_when_orthogonal():
    rng = np.random.default_rng(44)
    for (r, c) in [(16, 64), (64, 16)]:
        G = rng.standard_normal((r, c))
        ns = lambda x: oracle.ns_standard(x, coeffs=oracle.default_coeffs(40, oracle.CUBIC), eps=0.0)
        _, _, U = oracle.muon_step(np.zeros((r, c)), G, np.zeros((r, c)), 1.0, 0.0, 0.0, ns=ns)
        assert abs(math.sqrt(np.mean(U ** 2)) - 0.2) < 1e-12


# ------------------------------------------------------------------ planted mistakes

def _closed_form_pin_fails(monkeypatch, attr, replacement):
    rng = np.random.default_rng(51)
    G = rng.standard_normal((12, 30))
    with monkeypatch.context() as mp:
        mp.setattr(ons, attr, replacement)
        bad = [rel(oracle.ns_standard(G, eps=0.0), spectral_closed_form(G)),
               rel(oracle.ns_gram(G, eps=0.0), spectral_closed_form(G))]
    return min(bad) > 1e-6


def test_pins_catch_planted_mistakes(monkeypatch):
    real_coeffs = ons._coeff_array
    # a flipped sign on b
    assert _closed_form_pin_fails(
        monkeypatch, "_coeff_array",
        lambda c, s: real_coeffs(c, s) * np.array([1.0, -1.0, 1.0]))
    # the guide's extra 1/sqrt(min dim) in the normalisation
    assert _closed_form_pin_fails(
        monkeypatch, "frobenius_normalize",
        lambda X, eps=1e-7: X / ((np.linalg.norm(X) + eps) * math.sqrt(X.shape[0])))
    # spectral-norm instead of Frobenius normalisation
    assert _closed_form_pin_fails(
        monkeypatch, "frobenius_normalize",
        lambda X, eps=1e-7: X / (np.linalg.norm(X, 2) + eps))


def test_closed_form_entries_of_a_structured_input():
    """Known-SVD inputs built from Kronecker products of small orthogonal factors (used for the
    full-size checks): selected entries match the iteration run on the dense matrix."""
    import synth
    rng = np.random.default_rng(61)
    n, m = 24, 60
    spec = np.arange(1, n + 1) ** -0.5
    G, (Ua, Ub, Va, Vb) = synth.structured_known_svd(rng, n, m, spec, na=4, ma=5)
    U = np.kron(Ua, Ub)
    V = np.kron(Va, Vb)[:, :n]
    assert np.abs(U.T @ U - np.eye(n)).max() < 1e-12 and np.abs(V.T @ V - np.eye(n)).max() < 1e-12
    full = oracle.ns_standard(G)
    rows, cols = [0, 5, 23], [1, 17, 59]
    blk = oracle.ns_closed_form_entries(U[rows], spec, V[cols])
    assert np.abs(blk - full[np.ix_(rows, cols)]).max() < 1e-12
    # with an explicit norm (the stored matrix's) as well
    blk2 = oracle.ns_closed_form_entries(U[rows], spec, V[cols], fro_norm=np.linalg.norm(G))
    assert np.abs(blk2 - blk).max() < 1e-12


# ------------------------------------------------------------------ Nesterov momentum

def _disjoint_diagonal_pair(n=6, m=10):
    """Two gradients whose nonzeros sit on disjoint parts of the diagonal: every linear
    combination of them is diagonal, so Newton-Schulz acts entry by entry on it."""
    d1 = np.array([3.0, -1.25, 0.5])
    d2 = np.array([-2.0, 0.75, 1.5])
    G1, G2 = np.zeros((n, m)), np.zeros((n, m))
    G1[[0, 1, 2], [0, 1, 2]] = d1
    G2[[3, 4, 5], [3, 4, 5]] = d2
    return G1, G2


def _diagonal_ns_exact(N):
    """sign(d) p^5(|d| / ||d||) on the diagonal of a diagonal N, the scalar map in exact
    rational arithmetic (only the norm is a float)."""
    d = np.diag(N)
    nrm = np.linalg.norm(d)
    out = np.zeros_like(N)
    for i, di in enumerate(d):
        if di != 0.0:
            out[i, i] = math.copysign(float(exact_scalar_map(Fraction(abs(di) / nrm))), di)
    return out


def _two_step_updates(nesterov):
    """Two Muon steps from zero momentum on the disjoint diagonal pair: returns (M2, U2)."""
    G1, G2 = _disjoint_diagonal_pair()
    mu = 0.9
    ns = lambda x: oracle.ns_standard(x, eps=0.0)
    W = np.zeros_like(G1)
    _, M1, _ = oracle.muon_step(W, G1, np.zeros_like(G1), 0.0, mu, 0.0, nesterov=nesterov, ns=ns)
    _, M2, U2 = oracle.muon_step(W, G2, M1, 0.0, mu, 0.0, nesterov=nesterov, ns=ns)
    return M2, U2


def _nesterov_pin_holds():
    """Second step from a nonzero state: with M1 = (1 - mu) G1 the buffer is
    M2 = mu (1 - mu) G1 + (1 - mu) G2 and the Nesterov input is
    N2 = mu^2 (1 - mu) G1 + (1 - mu^2) G2; the update is 0.2 sqrt(10) NS(N2), entry by entry."""
    G1, G2 = _disjoint_diagonal_pair()
    mu = 0.9
    M2, U2 = _two_step_updates(nesterov=True)
    N2 = mu ** 2 * (1 - mu) * G1 + (1 - mu ** 2) * G2
    ok_m = np.abs(M2 - (mu * (1 - mu) * G1 + (1 - mu) * G2)).max() < 1e-15
    ok_u = np.abs(U2 - 0.2 * math.sqrt(10) * _diagonal_ns_exact(N2)).max() < 1e-13
    return ok_m and ok_u


def test_nesterov_momentum_two_steps_on_disjoint_diagonals():
    assert _nesterov_pin_holds()


def test_plain_momentum_two_steps_on_disjoint_diagonals():
    """Without Nesterov the buffer itself is orthogonalized: N2 = M2."""
    G1, G2 = _disjoint_diagonal_pair()
    mu = 0.9
    M2, U2 = _two_step_updates(nesterov=False)
    M2_exact = mu * (1 - mu) * G1 + (1 - mu) * G2
    assert np.abs(M2 - M2_exact).max() < 1e-15
    assert np.abs(U2 - 0.2 * math.sqrt(10) * _diagonal_ns_exact(M2_exact)).max() < 1e-13
    # and the two rules give different updates from this nonzero state
    _, U2n = _two_step_updates(nesterov=True)
    assert np.abs(U2 - U2n).max() > 1e-3


def test_nesterov_pin_catches_a_pre_update_momentum(monkeypatch):
    """Planted mistake: the Nesterov input formed from the buffer before its update,
    N = mu M_old + (1 - mu) G. From zero state this still gives N proportional to G, so only
    the nonzero-state pin above can catch it."""
    def wrong(M, G, momentum, nesterov):
        M_new = momentum * M + (1.0 - momentum) * G
        N = momentum * M + (1.0 - momentum) * G if nesterov else M_new
        return M_new, N
    with monkeypatch.context() as mp:
        mp.setattr(ons, "momentum_update", wrong)
        assert not _nesterov_pin_holds()
    assert _nesterov_pin_holds()


def test_nesterov_input_from_a_random_nonzero_state():
    """With the identity in place of Newton-Schulz the update exposes the orthogonalized
    input: 0.2 sqrt(max dim) (mu (mu M + (1 - mu) G) + (1 - mu) G) with Nesterov, and
    0.2 sqrt(max dim) (mu M + (1 - mu) G) without."""
    rng = np.random.default_rng(45)
    W = rng.standard_normal((7, 19))
    G = rng.standard_normal((7, 19))
    M = rng.standard_normal((7, 19))
    mu = 0.95
    s = 0.2 * math.sqrt(19)
    _, Mn, U = oracle.muon_step(W, G, M, 0.0, mu, 0.0, nesterov=True, ns=lambda x: x)
    assert np.abs(Mn - (mu * M + (1 - mu) * G)).max() < 1e-15
    assert np.abs(U / s - (mu * (mu * M + (1 - mu) * G) + (1 - mu) * G)).max() < 1e-14
    _, Mn, U = oracle.muon_step(W, G, M, 0.0, mu, 0.0, nesterov=False, ns=lambda x: x)
    assert np.abs(U / s - (mu * M + (1 - mu) * G)).max() < 1e-14
