"""Pins for ``oracle.softmax_rows`` and ``oracle.gelu_fused`` (CPU only).

Facts that do not come from the oracle:
  * library routines: torch.softmax and torch.nn.functional.gelu(approximate=
    "tanh") in float64;
  * closed forms: a constant row gives 1/n; two entries give the logistic
    function of their difference; gelu(0) = 0; gelu(h) - gelu(-h) = h (tanh
    is odd); gelu(h) -> h for large h and -> 0 for very negative h;
  * invariants: rows sum to 1; softmax is unchanged by adding a constant to
    a row; large entries (1e4) do not overflow;
  * planted mistakes (no max subtraction, the wrong axis, a wrong GELU
    constant, the cube dropped) fail these pins.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import rowwise as rowwise_mod
from tiled_attention_tileattn_amd.inputs import random_gelu_inputs, random_rows


@pytest.mark.parametrize("shape", [(1, 1), (3, 7), (16, 300), (5, 2049)])
def test_softmax_matches_torch(shape):
    x = random_rows(*shape, seed=sum(shape), scale=3.0)
    ref = torch.softmax(x.double(), dim=1).numpy()
    np.testing.assert_allclose(oracle.softmax_rows(x), ref, rtol=1e-13, atol=1e-300)


def test_softmax_closed_forms():
    np.testing.assert_allclose(oracle.softmax_rows(np.full((2, 10), 3.5)), np.full((2, 10), 0.1), rtol=1e-15)
    a, b = 0.7, -1.9
    p = oracle.softmax_rows(np.array([[a, b]]))[0]
    assert abs(p[0] - 1.0 / (1.0 + math.exp(b - a))) < 1e-15
    assert abs(p[1] - 1.0 / (1.0 + math.exp(a - b))) < 1e-15


def test_softmax_invariants():
    x = random_rows(8, 500, seed=3, scale=5.0).double().numpy()
    p = oracle.softmax_rows(x)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=1e-13)
    np.testing.assert_allclose(oracle.softmax_rows(x + 123.25), p, rtol=1e-12)
    big = np.array([[1e4, 1e4 - 1.0, -1e4]])
    q = oracle.softmax_rows(big)[0]
    assert np.isfinite(q).all() and abs(q[0] - 1 / (1 + math.exp(-1))) < 1e-15


def test_softmax_prefix_columns_and_minus_inf():
    x = random_rows(4, 20, seed=4).double().numpy()
    np.testing.assert_allclose(oracle.softmax_rows(x, 13), oracle.softmax_rows(x[:, :13]), rtol=0)
    y = x.copy()
    y[:, 5] = -np.inf
    p = oracle.softmax_rows(y)
    assert np.all(p[:, 5] == 0)
    np.testing.assert_allclose(np.delete(p, 5, axis=1), oracle.softmax_rows(np.delete(x, 5, axis=1)),
                               rtol=1e-14)


@pytest.mark.parametrize("scale", [1.0, 10.0])
def test_gelu_matches_torch(scale):
    # Both sides evaluate 0.5 h (1 + tanh z): for very negative h, 1 + tanh z
    # cancels and each carries an absolute error of a few float64 ulps of h.
    x, w, b = random_gelu_inputs(4096, seed=5, scale=scale)
    h = (x.double() * w.double() + b.double()).numpy()
    ref = F.gelu(torch.from_numpy(h), approximate="tanh").numpy()
    g = oracle.gelu_fused(x, w, b)
    assert np.all(np.abs(g - ref) <= 1e-13 * np.abs(ref) + 1e-15 * np.abs(h))


def test_gelu_closed_forms():
    one = np.ones(5)
    h = np.array([0.0, 0.3, -1.7, 4.0, -12.5])
    g = oracle.gelu_fused(h, one, np.zeros(5))
    gm = oracle.gelu_fused(-h, one, np.zeros(5))
    assert g[0] == 0.0
    np.testing.assert_allclose(g - gm, h, rtol=0, atol=1e-14)
    big = oracle.gelu_fused(np.array([40.0, -40.0, -200.0]), np.ones(3), np.zeros(3))
    assert big[0] == 40.0 and abs(big[1]) < 1e-300 and np.isfinite(big).all()
    # the fused input: h = x*w + b
    np.testing.assert_allclose(oracle.gelu_fused(np.array([2.0]), np.array([0.5]), np.array([-0.25])),
                               oracle.gelu_fused(np.array([0.75]), np.ones(1), np.zeros(1)), rtol=0)


# ---- planted mistakes -----------------------------------------------------
def _softmax_no_max(x, n_cols=None):
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(x)
    return e / e.sum(axis=1, keepdims=True)


def _softmax_wrong_axis(x, n_cols=None):
    x = np.asarray(x.double().numpy() if hasattr(x, "double") else x, dtype=np.float64)
    e = np.exp(x - x.max(axis=0, keepdims=True))
    return e / e.sum(axis=0, keepdims=True)


def _gelu_factory(c, a):
    def g(x, w, b):
        x, w, b = (np.asarray(t.double().numpy() if hasattr(t, "double") else t, dtype=np.float64)
                   for t in (x, w, b))
        h = x * w + b
        return 0.5 * h * (1.0 + np.tanh(c * (h + a * h ** 3)))
    return g


def _softmax_pins_pass():
    try:
        with np.errstate(over="ignore", invalid="ignore"):
            test_softmax_matches_torch((16, 300))
            test_softmax_invariants()
        return True
    except (AssertionError, ValueError):
        return False


def _gelu_pins_pass():
    try:
        test_gelu_matches_torch(1.0)
        test_gelu_closed_forms()
        return True
    except (AssertionError, ValueError):
        return False


@pytest.mark.parametrize("mutant", [_softmax_no_max, _softmax_wrong_axis])
def test_planted_softmax_mistakes_are_caught(mutant, monkeypatch):
    assert _softmax_pins_pass()
    monkeypatch.setattr(oracle, "softmax_rows", mutant)
    assert not _softmax_pins_pass()


@pytest.mark.parametrize("consts", [(math.sqrt(2 / math.pi), 0.0), (math.sqrt(1 / math.pi), 0.044715),
                                    (math.sqrt(2 / math.pi), 0.04715)])
def test_planted_gelu_mistakes_are_caught(consts, monkeypatch):
    assert _gelu_pins_pass()
    monkeypatch.setattr(oracle, "gelu_fused", _gelu_factory(*consts))
    assert not _gelu_pins_pass()


def test_module_constants_are_the_pages():
    assert rowwise_mod.GELU_A == 0.044715
    assert abs(rowwise_mod.GELU_C - 0.7978845608028654) < 1e-16
