"""fp64 reference of the gate / beta projections -- TEST INFRASTRUCTURE.

The PR #55426 report ("Fix KDA projection overlap on Hopper", "Implementation
breakdown" items 1-3 and "Key source snippets") runs the projections upstream
of the KDA forward as two skinny GEMMs with bf16 operands and fp32
accumulation: the first against the stacked gate-first-factor / beta weight
(F_A and beta, 144 rows at the test shape), the second, 128 deep, against the
gate's second factor (F_B, 1536 x 128).  Read here as

    P = round_bf16(hidden @ w_ab^T)            exact sum, one rounding
    G = round_bf16(P[:, :128] @ w_b^T)

with rounding to nearest even.  The products are formed in fp64, which is
exact for bf16 operands (8-bit significands: each product has at most 16
significant bits) and leaves only the summation's rounding, far below a bf16
unit; the one rounding to bf16 is then done exactly (round_bf16).

Only the test suite may import this module.
"""
from __future__ import annotations

import numpy as np

RANK = 128  # inner dimension of the gate's second factor


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float64 (exact)."""
    b = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even, in one
    step (no intermediate fp32 rounding).  Normal range only: |x| in
    [2^-126, 2^128) or zero, which is all the projections produce here."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)                  # x = m 2^e, 0.5 <= |m| < 1
    r = np.round(m * 256.0)             # 8 significant bits; numpy rounds half to even
    return np.ldexp(r / 256.0, e)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16-representable float64 values -> their uint16 bit patterns."""
    f = np.asarray(x, np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def gate_proj(hidden_bits, w_ab_bits, w_b_bits):
    """The two projections.  Arguments are uint16 bf16 bit patterns:
    hidden [M, K], w_ab [n_ab, K] (n_ab >= 128), w_b [n_b, 128].
    Returns (P, G, P_exact, G_exact): the bf16-rounded results as float64
    [M, n_ab] and [M, n_b], and the unrounded sums (G_exact is the exact sum
    of the rounded P)."""
    h = bf16_to_f64(hidden_bits)
    wab = bf16_to_f64(w_ab_bits)
    wb = bf16_to_f64(w_b_bits)
    assert h.ndim == 2 and wab.ndim == 2 and wb.ndim == 2
    assert wab.shape[1] == h.shape[1] and wab.shape[0] >= RANK and wb.shape[1] == RANK
    p_exact = h @ wab.T
    p = round_bf16(p_exact)
    g_exact = p[:, :RANK] @ wb.T
    g = round_bf16(g_exact)
    return p, g, p_exact, g_exact
