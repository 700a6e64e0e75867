"""Row softmax and fused GELU in float64 (test infrastructure only).

Both follow "Guia Prático de Programação de GPU com Tiles" (Passo a Passo):

* step 4 "Softmax por Linha": per row, subtract the row maximum, take the
  exponentials, divide by their sum.  Entries past the row's length are not
  part of it (the page loads them as -inf, which contributes exp(-inf) = 0).
* step 3 "GELU Fundido": h = x * w + b elementwise, then the tanh
  approximation of GELU, 0.5 h (1 + tanh(sqrt(2/pi) (h + 0.044715 h^3))).
  The page builds tanh from exponentials; tanh itself is the function meant,
  and numpy's tanh evaluates it without overflow for every argument.  For
  very negative h, 1 + tanh(...) cancels: the result then carries an
  absolute error of a few float64 ulps of h (about 1e-16 |h|).

Inputs are used exactly as given (bf16 values upcast to float64).
"""

from __future__ import annotations

import math

import numpy as np

from .full_softmax import _as_f64

GELU_C = math.sqrt(2.0 / math.pi)
GELU_A = 0.044715


def softmax_rows(x, n_cols: int | None = None) -> np.ndarray:
    """Softmax of the first n_cols columns of every row of x [n_rows, >= n_cols]."""
    x = _as_f64(x)
    if x.ndim != 2:
        raise ValueError("x must be 2-D")
    n = x.shape[1] if n_cols is None else int(n_cols)
    if not 1 <= n <= x.shape[1]:
        raise ValueError("need 1 <= n_cols <= row length")
    r = x[:, :n]
    m = r.max(axis=1, keepdims=True)
    e = np.exp(r - m)
    return e / e.sum(axis=1, keepdims=True)


def gelu_fused(x, w, b) -> np.ndarray:
    """0.5 h (1 + tanh(sqrt(2/pi) (h + 0.044715 h^3))) with h = x*w + b, elementwise."""
    x, w, b = _as_f64(x), _as_f64(w), _as_f64(b)
    if not (x.shape == w.shape == b.shape):
        raise ValueError("x, w, b must share one shape")
    h = x * w + b
    return 0.5 * h * (1.0 + np.tanh(GELU_C * (h + GELU_A * h ** 3)))
