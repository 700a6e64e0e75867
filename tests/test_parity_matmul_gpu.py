"""Parity of the matrix product (tileattn_matmul) with the oracle (needs an MI355X).

Calls go through the C ABI (the ctypes binding's ``matmul``) on seeded inputs
from ``tiled_attention_tileattn_amd.inputs``; ``oracle.matmul`` gets the same
bf16 values.

Two kinds of check:
  * integer-valued inputs (|a|, |b| <= 4): every product and partial sum is
    exact in fp32, so an fp32 C must equal the oracle bit for bit and a bf16 C
    must equal the oracle rounded to nearest even;
  * N(0, 1) inputs: each element within the error bound of fp32 summation of
    exact products in any order, |C - C_ref| <= gamma_K * (|A| |B|) with
    gamma_K = K u / (1 - K u), u = 2^-23 (covers truncating as well as
    rounding adders); a bf16 C adds its own rounding, 2^-8 |C_ref|.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import tiled_attention_tileattn_amd as ta
from tiled_attention_tileattn_amd.inputs import MATMUL_WORKLOADS, random_matrices

pytestmark = pytest.mark.gpu


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


def _bound(a64, b64, c_ref, K, out_bf16):
    u = 2.0 ** -23
    g = K * u / (1 - K * u)
    bnd = g * (np.abs(a64) @ np.abs(b64))
    if out_bf16:
        bnd = bnd * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(c_ref)
    return bnd


def _gpu(a, b, out_dtype):
    c = ta.matmul(a.cuda(), b.cuda(), out_dtype=out_dtype)
    torch.cuda.synchronize()
    return c.cpu()


SHAPES = [
    # M, N, K
    (1, 8, 8), (7, 16, 24), (64, 64, 64), (256, 256, 64), (255, 248, 56), (257, 264, 72),
    (300, 520, 136), (513, 1000, 200), (1024, 1024, 1024), (40, 2056, 8), (1000, 8, 1000),
]


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shape", SHAPES)
def test_integer_inputs_exact(shape, out_dtype):
    M, N, K = shape
    _say(f"integer M={M} N={N} K={K} {out_dtype}")
    a, b = random_matrices(M, N, K, seed=M + N + K, integer=True)
    c = _gpu(a, b, out_dtype)
    c_ref = oracle.matmul(a, b)
    want = torch.from_numpy(c_ref).to(torch.float32)
    if out_dtype == torch.bfloat16:
        want = want.to(torch.bfloat16)
    assert torch.equal(c, want), f"{shape}: differs"


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shape", SHAPES)
def test_gaussian_inputs_within_fp32_bound(shape, out_dtype):
    M, N, K = shape
    _say(f"gaussian M={M} N={N} K={K} {out_dtype}")
    a, b = random_matrices(M, N, K, seed=3 * (M + N + K))
    c = _gpu(a, b, out_dtype).double().numpy()
    a64, b64 = a.double().numpy(), b.double().numpy()
    c_ref = oracle.matmul(a, b)
    err = np.abs(c - c_ref)
    bnd = _bound(a64, b64, c_ref, K, out_dtype == torch.bfloat16)
    _say(f"  max|dC|={err.max():.3e} max(|dC|/bound)={(err / np.maximum(bnd, 1e-300)).max():.3e}")
    assert np.all(err <= bnd)


def test_k_zero_writes_zeros():
    a = torch.zeros((5, 0), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((0, 16), dtype=torch.bfloat16, device="cuda")
    out = torch.full((5, 16), float("nan"), device="cuda")
    ta.matmul(a, b, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), torch.zeros(5, 16))


def test_empty_m_or_n_is_a_noop():
    for M, N in [(0, 16), (4, 0)]:
        a = torch.zeros((M, 8), dtype=torch.bfloat16, device="cuda")
        b = torch.zeros((8, N), dtype=torch.bfloat16, device="cuda")
        c = ta.matmul(a, b)
        torch.cuda.synchronize()
        assert c.shape == (M, N)


def test_deterministic_and_stream_ordered():
    a, b = random_matrices(700, 600, 504, seed=8, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        c1 = ta.matmul(a, b, stream=s)
        c2 = ta.matmul(a, b, stream=s)
    s.synchronize()
    assert torch.equal(c1, c2)


@pytest.mark.parametrize("name", list(MATMUL_WORKLOADS))
def test_workload_sampled_rows(name):
    M, N, K, seed = MATMUL_WORKLOADS[name]
    _say(f"{name}: M={M} N={N} K={K}, 256 sampled rows, fp32 C")
    a, b = random_matrices(M, N, K, seed=seed)
    c = ta.matmul(a.cuda(), b.cuda())
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(seed).choice(M, 256, replace=False))
    rows = np.unique(np.concatenate([rows, [0, 255, 256, M - 1]]))
    c_s = c[torch.from_numpy(rows).cuda()].double().cpu().numpy()
    a64, b64 = a.double().numpy(), b.double().numpy()
    c_ref = oracle.matmul_rows(a, b, rows)
    err = np.abs(c_s - c_ref)
    bnd = _bound(a64[rows], b64, c_ref, K, False)
    _say(f"  max|dC|={err.max():.3e} max(|dC|/bound)={(err / bnd).max():.3e}")
    assert np.all(err <= bnd)
    assert torch.isfinite(c).all()


@pytest.mark.parametrize("name", list(MATMUL_WORKLOADS))
def test_workload_integer_sampled_rows_exact(name):
    M, N, K, seed = MATMUL_WORKLOADS[name]
    _say(f"{name}: integer inputs, 256 sampled rows exact")
    a, b = random_matrices(M, N, K, seed=seed + 1, integer=True)
    c = ta.matmul(a.cuda(), b.cuda())
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(seed + 1).choice(M, 256, replace=False))
    c_s = c[torch.from_numpy(rows).cuda()].cpu()
    want = torch.from_numpy(oracle.matmul_rows(a, b, rows)).to(torch.float32)
    assert torch.equal(c_s, want)
