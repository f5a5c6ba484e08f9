"""Plain, slow, obviously-correct fp64 oracle for the Muon hot path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg, never by the product path. It shares no code
with the HIP library (no kernels, helpers, tables or constants).

Everything is numpy float64 on the CPU; ``@`` (BLAS matmul) and ``numpy.linalg``
routines are the only library primitives used. Inputs are upcast exactly from
whatever dtype they were stored in.

Sources (web pages):
* "Moonlight 16B Guide: Scalable MoE & Muon Optimizer" (aifetchly blog):
  - "The Scalable Muon Optimizer: Theory and Mechanics" (the four-step box:
    momentum, Newton-Schulz loop, update scale, decoupled weight decay);
  - "The Newton-Schulz Iteration for Matrix Orthogonalization" (normalisation and
    the odd polynomial iteration);
  - "Innovation 1" (decoupled weight decay) and "Innovation 2" (update scale);
  - "End-to-End PyTorch Implementation" (orientation: transpose so rows <= cols;
    eps added to the Frobenius norm; left Gram X X^T; momentum buffer update).
* Jiqizhixin article on Gram Newton-Schulz ("Muon ... 2x speed-up in trillion-
  parameter MoE"): sections on standard Newton-Schulz and its three products,
  the Gram reformulation (an odd polynomial p(X) equals q(X X^T) X), the fp16
  instability of the naive Gram form, and the stabilized variant that restarts
  after step 2 and re-forms the Gram matrix.

Readings of points the pages leave open:
* coefficients: one triple (a_k, b_k, c_k) per step; the step maps
  X -> a X + b (X X^T) X + c (X X^T)^2 X, i.e. each singular value s -> a s + b s^3 + c s^5.
  Default: the quintic (3.4445, -4.7750, 2.0315) for every step; the pages' own
  cubic 0.5 * X (3I - X^T X) is (1.5, -0.5, 0).
* normalisation: X0 = G / (||G||_F + eps), eps = 1e-7 (Frobenius only; the extra
  1/sqrt(min dim) factor of the guide is not applied).
* Gram accumulation: X_k = Z_k X_{k-1} with Z_k = a I + b R + c R^2, hence
  Q_k = Z_k Q_{k-1} and R_k = Z_k R_{k-1} Z_k; the output is Q_K X_0.
* restart (stabilized variant): after each step k in ``restarts`` (k < K), form
  X_k = Q_k X explicitly, set R = X_k X_k^T, Q = I and continue from X_k.
"""
from __future__ import annotations

import math
from typing import Callable, Iterable, Optional, Sequence

import numpy as np

# Per-step coefficient triples (a, b, c).
QUINTIC = (3.4445, -4.7750, 2.0315)
CUBIC = (1.5, -0.5, 0.0)


def default_coeffs(steps: int = 5, triple: Sequence[float] = QUINTIC) -> np.ndarray:
    """The same (a, b, c) for every one of ``steps`` steps, as a [steps, 3] fp64 array."""
    return np.tile(np.asarray(triple, dtype=np.float64), (steps, 1))


def _coeff_array(coeffs, steps: Optional[int]) -> np.ndarray:
    if coeffs is None:
        coeffs = default_coeffs(5 if steps is None else steps)
    c = np.asarray(coeffs, dtype=np.float64)
    if c.ndim == 1:
        c = np.tile(c, (5 if steps is None else steps, 1))
    if steps is not None and c.shape[0] != steps:
        raise ValueError("coefficient rows != steps")
    return c


def orient(G: np.ndarray):
    """Return (X, transposed): X = G if rows <= cols else G^T (guide's PyTorch listing)."""
    G = np.asarray(G, dtype=np.float64)
    if G.ndim != 2:
        raise ValueError("Newton-Schulz needs a 2-D matrix")
    if G.shape[0] > G.shape[1]:
        return G.T.copy(), True
    return G.copy(), False


def frobenius_normalize(X: np.ndarray, eps: float = 1e-7) -> np.ndarray:
    """X / (||X||_F + eps): the guide's Frobenius normalisation with eps added to the norm."""
    return X / (math.sqrt(float(np.sum(X * X))) + eps)


def ns_standard(G, coeffs=None, eps: float = 1e-7, steps: Optional[int] = None) -> np.ndarray:
    """Standard Newton-Schulz on X (Jiqizhixin article, "standard Newton-Schulz": three
    products per step, X X^T, A^2 and B X).

    For k = 1..K:  A = X X^T;  B = b_k A + c_k A^2;  X <- a_k X + B X.
    Rows > cols are handled by working on G^T and transposing the result back.
    """
    c = _coeff_array(coeffs, steps)
    X, transposed = orient(G)
    X = frobenius_normalize(X, eps)
    for a_k, b_k, c_k in c:
        A = X @ X.T
        B = b_k * A + c_k * (A @ A)
        X = a_k * X + B @ X
    return X.T if transposed else X


def ns_gram(G, coeffs=None, eps: float = 1e-7, restarts: Iterable[int] = (2,),
            steps: Optional[int] = None, trace: Optional[list] = None) -> np.ndarray:
    """Gram Newton-Schulz (Jiqizhixin article, Gram reformulation + stabilized variant).

    Iterates on the n x n Gram matrix R = X X^T instead of the n x m X:
      start  R = X0 X0^T, Q = I, Y = X0
      step k: Z = a_k I + b_k R + c_k R^2;  Q <- Z Q
              if k in restarts and k < K:  Y <- Q Y;  R <- Y Y^T;  Q <- I
              elif k < K:                  R <- Z R Z
      output Q Y
    ``restarts=()`` is the naive variant; ``restarts=(2,)`` the stabilized one.
    If ``trace`` is a list, the R in use after each step is appended to it
    (for the negative-eigenvalue report).
    """
    c = _coeff_array(coeffs, steps)
    K = c.shape[0]
    rs = set(int(k) for k in restarts)
    X, transposed = orient(G)
    Y = frobenius_normalize(X, eps)
    n = Y.shape[0]
    R = Y @ Y.T
    Q = np.eye(n)
    for k, (a_k, b_k, c_k) in enumerate(c, start=1):
        Z = a_k * np.eye(n) + b_k * R + c_k * (R @ R)
        Q = Z @ Q
        if k < K and k in rs:
            Y = Q @ Y
            R = Y @ Y.T
            Q = np.eye(n)
        elif k < K:
            R = Z @ R @ Z
        if trace is not None:
            trace.append(R.copy())
    O = Q @ Y
    return O.T if transposed else O


def scalar_ns_map(s, coeffs=None, steps: Optional[int] = None):
    """The scalar map each singular value undergoes: s -> a s + b s^3 + c s^5, composed over steps."""
    c = _coeff_array(coeffs, steps)
    s = np.asarray(s, dtype=np.float64)
    for a_k, b_k, c_k in c:
        s = a_k * s + b_k * s ** 3 + c_k * s ** 5
    return s


def ns_svd_closed_form(G, coeffs=None, eps: float = 1e-7, steps: Optional[int] = None) -> np.ndarray:
    """What the iteration reaches, written through the SVD: G = U S V^T ->
    U diag(p_K(...p_1(s/(||G||_F+eps)))) V^T (each step is an odd polynomial in X,
    which acts on the singular values only)."""
    G = np.asarray(G, dtype=np.float64)
    U, s, Vt = np.linalg.svd(G, full_matrices=False)
    nrm = math.sqrt(float(np.sum(G * G))) + eps
    return (U * scalar_ns_map(s / nrm, coeffs, steps)) @ Vt


def ns_closed_form_entries(U_rows, spectrum, V_rows, coeffs=None, eps: float = 1e-7,
                           steps: Optional[int] = None, fro_norm: Optional[float] = None) -> np.ndarray:
    """Selected entries of the output for an input with a known SVD G = U diag(spectrum) V^T:
    rows i of U (``U_rows``, k x r) and rows j of V (``V_rows``, l x r) give the k x l block
    U_rows diag(p_K(...p_1(spectrum / (||G||_F + eps)))) V_rows^T. ``fro_norm`` defaults to
    ||spectrum||_2 (= ||G||_F)."""
    s = np.asarray(spectrum, dtype=np.float64)
    nrm = float(np.linalg.norm(s)) if fro_norm is None else float(fro_norm)
    f = scalar_ns_map(s / (nrm + eps), coeffs, steps)
    return (np.asarray(U_rows, dtype=np.float64) * f) @ np.asarray(V_rows, dtype=np.float64).T


def momentum_update(M, G, momentum: float, nesterov: bool):
    """Momentum accumulation of the guide's "Scalable Muon Optimizer" box, in its EMA form:
    M_new = mu M + (1 - mu) G. The matrix handed to Newton-Schulz is M_new, or with Nesterov
    the same rule applied once more to the updated buffer: N = mu M_new + (1 - mu) G.
    Returns (M_new, N)."""
    M_new = momentum * M + (1.0 - momentum) * G
    N = momentum * M_new + (1.0 - momentum) * G if nesterov else M_new
    return M_new, N


def muon_step(W, G, M, lr: float, momentum: float, weight_decay: float,
              nesterov: bool = False, scale_coeff: float = 0.2,
              ns: Optional[Callable] = None):
    """One Muon step for one matrix parameter (guide, "Scalable Muon Optimizer" box):

      1. M <- mu M + (1 - mu) G                       (momentum accumulation)
         N = mu M + (1 - mu) G if nesterov else M     (Nesterov: the same rule once more)
      2. O = NS(N)                                    (Newton-Schulz orthogonalisation)
      3. U = scale_coeff * sqrt(max(d_out, d_in)) * O (update-scale alignment)
      4. W <- (1 - lr * wd) W - lr * U                (decoupled weight decay)

    Returns (W_new, M_new, U) in fp64.
    """
    ns = ns_standard if ns is None else ns
    W = np.asarray(W, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    M = np.asarray(M, dtype=np.float64)
    M_new, N = momentum_update(M, G, momentum, nesterov)
    O = ns(N)
    d_out, d_in = W.shape
    U = scale_coeff * math.sqrt(max(d_out, d_in)) * O
    W_new = (1.0 - lr * weight_decay) * W - lr * U
    return W_new, M_new, U
