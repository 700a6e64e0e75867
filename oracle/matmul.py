"""Matrix product C = A B in float64 (test infrastructure only).

The tiled kernel of "Guia Prático de Programação de GPU com Tiles" (Passo a
Passo, step 5 "Multiplicação de Matrizes Tiled — Acumulação no Loop K")
splits A and B into blocks and adds, for each output tile, the products of
an A block and a B block over the K loop into an fp32 accumulator.  Summed
over all K blocks that is the plain product

    C[i, j] = sum_k A[i, k] * B[k, j],

which this module writes out as one float64 matrix product of the exact input
values (bf16 values are exact in float64; every product of two bf16 numbers
and every partial sum of a few thousand of them is far inside float64's
precision, so only the final rounding of a long sum differs from the real
number, by at most about K * 2^-53 relative).

Reading: A is [M, K] and B is [K, N], both row-major (the page's strides are
left undefined; row-major is the plain layout of its index expressions).
"""

from __future__ import annotations

import numpy as np

from .full_softmax import _as_f64


def matmul(a, b) -> np.ndarray:
    """C = A B in float64; a [M, K], b [K, N] (numpy arrays or CPU tensors)."""
    a, b = _as_f64(a), _as_f64(b)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[0]:
        raise ValueError(f"shapes {a.shape} and {b.shape} do not chain")
    return a @ b


def matmul_rows(a, b, rows) -> np.ndarray:
    """Rows ``rows`` of C = A B in float64 (for sampled checks of large C)."""
    a, b = _as_f64(a), _as_f64(b)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[0]:
        raise ValueError(f"shapes {a.shape} and {b.shape} do not chain")
    return a[np.asarray(rows)] @ b
