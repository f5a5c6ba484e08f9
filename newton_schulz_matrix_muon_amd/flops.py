"""Algorithmic flop accounting for the Newton-Schulz variants (host logic only).

Conventions:
* a product whose result is symmetric (X X^T, and products of commuting symmetric
  n x n iterates) is computed as its upper triangle only and counts n (n + 1) k
  flops for an inner dimension k;
* a rectangular product (n x n) . (n x m) counts 2 n^2 m;
* ``standard_dense_flops`` is the count the Gram Newton-Schulz article gives for one
  standard iteration on an n x m X (X X^T 2 m n^2, A^2 2 n^3, B X 2 m n^2), times K.

``gram_flops`` is the method's count (every n x n product symmetric-aware). The kernels
execute the accumulated product Q <- Z Q as a full n x n product (2 n^3), which keeps the
order in which the steps act on X under rounding; ``gram_executed_flops`` counts that.
"""
from __future__ import annotations

from typing import Iterable


def sym_flops(n: int, k: int) -> int:
    """Upper-triangle product with an n x n symmetric result and inner dimension k."""
    return n * (n + 1) * k


def rect_flops(n: int, m: int) -> int:
    """(n x n) . (n x m)."""
    return 2 * n * n * m


def orient(rows: int, cols: int):
    """(n, m) with n <= m."""
    return (rows, cols) if rows <= cols else (cols, rows)


def standard_flops(rows: int, cols: int, steps: int = 5) -> int:
    """Standard iteration with symmetric-aware A = X X^T and A^2 products."""
    n, m = orient(rows, cols)
    return steps * (sym_flops(n, m) + sym_flops(n, n) + rect_flops(n, m))


def standard_dense_flops(rows: int, cols: int, steps: int = 5) -> int:
    """The article's count: 2 m n^2 + 2 n^3 + 2 m n^2 per iteration."""
    n, m = orient(rows, cols)
    return steps * (2 * m * n * n + 2 * n ** 3 + 2 * m * n * n)


def gram_products(steps: int, restarts: Iterable[int]):
    """Counts of (symmetric n x n products, Gram formations X X^T, rectangular Q X products)."""
    rs = set(int(k) for k in restarts)
    sym = 0
    gram = 1          # R0 = X0 X0^T
    rect = 1          # final Q X
    q_is_identity = True
    for k in range(1, steps + 1):
        sym += 1      # R^2 for Z_k
        if not q_is_identity:
            sym += 1  # Q <- Z Q
        q_is_identity = False
        if k < steps and k in rs:
            rect += 1
            gram += 1
            q_is_identity = True
        elif k < steps:
            sym += 2  # R <- Z (R Z)
    return sym, gram, rect


def gram_flops(rows: int, cols: int, steps: int = 5, restarts: Iterable[int] = (2,)) -> int:
    n, m = orient(rows, cols)
    sym, gram, rect = gram_products(steps, restarts)
    return sym * sym_flops(n, n) + gram * sym_flops(n, m) + rect * rect_flops(n, m)


def gram_products_executed(steps: int, restarts: Iterable[int]):
    """Counts of (symmetric n x n products, full n x n products, Gram formations, rectangular
    products) as the kernels execute them: the Q <- Z Q updates are full products."""
    rs = set(int(k) for k in restarts)
    sym = full = 0
    gram = rect = 1
    q_is_identity = True
    for k in range(1, steps + 1):
        sym += 1
        if not q_is_identity:
            full += 1
        q_is_identity = False
        if k < steps and k in rs:
            rect += 1
            gram += 1
            q_is_identity = True
        elif k < steps:
            sym += 2
    return sym, full, gram, rect


def gram_executed_flops(rows: int, cols: int, steps: int = 5, restarts: Iterable[int] = (2,)) -> int:
    n, m = orient(rows, cols)
    sym, full, gram, rect = gram_products_executed(steps, restarts)
    return (sym * sym_flops(n, n) + full * 2 * n ** 3 + gram * sym_flops(n, m)
            + rect * rect_flops(n, m))
