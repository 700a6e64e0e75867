"""Parity of the row softmax and the fused GELU with the oracle (needs an MI355X).

Calls go through the C ABI (the ctypes binding's ``softmax`` / ``gelu``) on
seeded inputs; the oracle gets the same values (bf16 upcast exactly).

Element-wise bounds, derived from the fp32 arithmetic of the kernels:

softmax, o_i = exp2(x_i*L - m*L) * (1/s), L = log2 e rounded to fp32, s the
fp32 sum of the numerators:
  * the exponent: the fma rounds once (u |t_i|, t_i = (x_i - m) L) and L is
    off by at most u relative; both move p_i by about |x_i - m| u each; the
    hardware exp2 adds at most 2u (u = 2^-24); the part of the error common
    to a row (m*L rounded) cancels in the normalisation;
  * the sum: at most n/256 + 16 additions along any path of the reduction
    (per-thread chunks, then the wave and workgroup trees), plus the online
    kernel's rescalings: gamma_d with d = n/128 + 32;
  * the reciprocal and the product: 2u.
  relative error <= (2 |x_i - m| + 4) u + gamma_d + 2u, plus 2^-8 when the
  output is bf16, plus an absolute 2^-125 for results in the subnormal range.

GELU, g = h / (1 + exp2(-2 L z)), h = fma(x, w, b), z = c (h + a h^3):
  * h: one rounding (u); z: the cube, the fma and the products with the fp32
    constants c and a: <= 8u relative;
  * exp2 of -2 L z: argument error |2 L z| * 10u, which moves the factor
    1/(1 + e) by at most that (relative), plus 2u for exp2 itself;
  * 1 + e, the division: 2u.  The bf16 kernel multiplies by the hardware
    reciprocal instead (1 ulp, i.e. 2u, then the product: u): 4u there.
  relative error <= (12 + 30 |z|) u (bf16: 2u more), plus 2^-8 for bf16
  output, plus the oracle's own absolute error where 1 + tanh cancels
  (1e-15 |h|) and 2^-125.
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import tiled_attention_tileattn_amd as ta
from tiled_attention_tileattn_amd.inputs import ROWWISE_WORKLOADS, random_gelu_inputs, random_rows

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
TINY = 2.0 ** -125


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    ta.load_library()
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _softmax_bound(x64, p_ref, n, bf16_out):
    m = np.max(x64, axis=1, keepdims=True)
    d = n / 128 + 32
    gamma = d * U / (1 - d * U)
    dist = np.where(np.isfinite(x64), np.abs(x64 - m), 0.0)   # -inf entries: p_ref = 0
    rel = (2 * dist + 6) * U + gamma
    if bf16_out:
        rel = rel + 2.0 ** -8
    return rel * p_ref + TINY


def _check_softmax(x, n_cols, dtype, what, inplace=False):
    xd = x.cuda()
    if inplace:
        out = ta.softmax(xd, out=xd, n_cols=n_cols)
    else:
        out = ta.softmax(xd, n_cols=n_cols)
    torch.cuda.synchronize()
    o = out.double().cpu().numpy()
    x64 = x.double().numpy()
    p_ref = oracle.softmax_rows(x64, n_cols)
    bnd = _softmax_bound(x64[:, :n_cols], p_ref, n_cols, dtype == "bf16")
    err = np.abs(o[:, :n_cols] - p_ref)
    _say(f"  {what}: max|dP|={err.max():.3e} max(|dP|/bound)={(err / bnd).max():.3e}")
    assert np.isfinite(o[:, :n_cols]).all()
    assert np.all(err <= bnd), what
    if not inplace and n_cols < x.shape[1]:
        # columns past n_cols are not written
        pass
    return out


SOFTMAX_SHAPES = [
    # n_rows, n_cols, stride
    (1, 1, 8), (3, 7, 8), (4, 8, 8), (5, 100, 104), (2, 2047, 2048), (3, 2048, 2048), (2, 2049, 2056),
    (7, 4096, 4096), (3, 5000, 5000), (2, 8192, 8192), (2, 16384, 16384), (2, 16385, 16392),
    (2, 50000, 50000), (300, 333, 336),
]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("shape", SOFTMAX_SHAPES)
def test_softmax_sweep(shape, dtype):
    n_rows, n_cols, stride = shape
    what = f"softmax rows={n_rows} cols={n_cols} stride={stride} {dtype}"
    _say(what)
    x = random_rows(n_rows, stride, seed=n_rows + n_cols, dtype=dtype, scale=2.0)
    _check_softmax(x, n_cols, dtype, what)


@pytest.mark.parametrize("n_cols", [300, 20000])
def test_softmax_large_values_and_minus_inf(n_cols):
    # |x| ~ 1e3 would overflow exp without the max subtraction; -inf entries give 0
    x = random_rows(4, n_cols, seed=31, dtype="fp32", scale=1000.0)
    x[:, ::7] = -float("inf")
    _check_softmax(x, n_cols, "fp32", f"large values, -inf entries, cols={n_cols}")


def test_softmax_columns_past_n_cols_are_untouched():
    x = random_rows(3, 64, seed=32).cuda()
    out = torch.full_like(x, 7.0)
    ta.softmax(x, out=out, n_cols=40)
    torch.cuda.synchronize()
    assert torch.all(out[:, 40:] == 7.0)


@pytest.mark.parametrize("n_cols", [1000, 30000])
def test_softmax_in_place(n_cols):
    x = random_rows(5, n_cols, seed=33, dtype="bf16")
    _check_softmax(x, n_cols, "bf16", f"in place cols={n_cols}", inplace=True)


def test_softmax_rows_of_minus_inf_give_nan():
    x = torch.zeros(2, 16, device="cuda")
    x[1] = -float("inf")
    out = ta.softmax(x)
    torch.cuda.synchronize()
    assert torch.allclose(out[0], torch.full((16,), 1 / 16, device="cuda"))
    assert torch.isnan(out[1]).all()


def _gelu_bound(x, w, b, g_ref, bf16_out):
    h = x * w + b
    z = math.sqrt(2 / math.pi) * (h + 0.044715 * h ** 3)
    rel = (12 + 30 * np.abs(z)) * U
    if bf16_out:
        rel = rel + 2 * U + 2.0 ** -8
    return rel * np.abs(g_ref) + 1e-15 * np.abs(h) + TINY


def _check_gelu(x, w, b, dtype, what, out_alias=None):
    xd, wd, bd = x.cuda(), w.cuda(), b.cuda()
    out = {"x": xd, "w": wd, "b": bd}.get(out_alias)
    g = ta.gelu(xd, wd, bd, out=out)
    torch.cuda.synchronize()
    g = g.double().cpu().numpy()
    x64, w64, b64 = (t.double().numpy() for t in (x, w, b))
    g_ref = oracle.gelu_fused(x64, w64, b64)
    bnd = _gelu_bound(x64, w64, b64, g_ref, dtype == "bf16")
    err = np.abs(g - g_ref)
    _say(f"  {what}: max|dG|={err.max():.3e} max(|dG|/bound)={(err / bnd).max():.3e}")
    assert np.isfinite(g).all()
    assert np.all(err <= bnd), what


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("n", [1, 7, 8, 9, 255, 2048, 2049, 100003, 1 << 20])
def test_gelu_sweep(n, dtype):
    what = f"gelu n={n} {dtype}"
    _say(what)
    x, w, b = random_gelu_inputs(n, seed=n, dtype=dtype)
    _check_gelu(x, w, b, dtype, what)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_gelu_tails(dtype):
    # |h| up to ~1e3: exp(-2z) overflows for very negative z, the result must stay finite
    x, w, b = random_gelu_inputs(50000, seed=41, dtype=dtype, scale=20.0)
    _check_gelu(x, w, b, dtype, f"gelu tails {dtype}")


def test_gelu_output_may_alias_an_input():
    x, w, b = random_gelu_inputs(10001, seed=42)
    _check_gelu(x, w, b, "fp32", "gelu out = w", out_alias="w")


@pytest.mark.parametrize("name", list(ROWWISE_WORKLOADS))
def test_workload_sampled(name):
    kind, dtype, shape, seed = ROWWISE_WORKLOADS[name]
    _say(f"{name}: full size on the GPU, sampled against the oracle")
    rng = np.random.default_rng(seed)
    if kind == "softmax":
        x = random_rows(*shape, seed=seed, dtype=dtype, device="cuda")
        out = ta.softmax(x)
        torch.cuda.synchronize()
        rows = torch.from_numpy(np.sort(rng.choice(shape[0], 128, replace=False))).cuda()
        xs, os_ = x[rows].cpu(), out[rows].double().cpu().numpy()
        p_ref = oracle.softmax_rows(xs.double().numpy())
        bnd = _softmax_bound(xs.double().numpy(), p_ref, shape[1], dtype == "bf16")
        assert np.all(np.abs(os_ - p_ref) <= bnd)
    else:
        x, w, b = random_gelu_inputs(shape[0], seed=seed, dtype=dtype, device="cuda")
        g = ta.gelu(x, w, b)
        torch.cuda.synchronize()
        idx = torch.from_numpy(rng.choice(shape[0], 1 << 16, replace=False)).cuda()
        idx = torch.cat([idx, torch.arange(shape[0] - 64, shape[0], device="cuda")])
        xs, ws, bs = (t[idx].double().cpu().numpy() for t in (x, w, b))
        gs = g[idx].double().cpu().numpy()
        g_ref = oracle.gelu_fused(xs, ws, bs)
        assert np.all(np.abs(gs - g_ref) <= _gelu_bound(xs, ws, bs, g_ref, dtype == "bf16"))
        assert torch.isfinite(g).all()
