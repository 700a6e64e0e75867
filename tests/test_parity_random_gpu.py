"""Randomized parity sweep over the 16-bit kernel's instance families (needs
an MI355X).

Each case draws, from its own seed, a shape (batch, GQA ratio, Sq and Sk from
1 to ~700 keys, head dimension), causal or not, bf16 or fp16, and one of:
plain, linear (ALiBi) bias, random block map, or both.  Small grids run the
key split, grids of heads x query tiles beyond half the chip the 256-row
kernel; both are drawn.  Each output is checked against the fp64 oracle with
the plain path's tolerances (rows a block map leaves empty: o = 0,
lse = -inf exactly).
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import tiled_attention_tileattn_amd as ta
from tiled_attention_tileattn_amd.inputs import alibi_slopes, random_block_mask, random_qkv

pytestmark = pytest.mark.gpu

TOL = {"bf16": dict(max=2e-2, mean=2e-3, lse=1e-3), "fp16": dict(max=4e-3, mean=4e-4, lse=1e-3)}
N_CASES = 40


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


def _draw(case):
    rng = np.random.default_rng(1000 + case)
    big = case % 4 == 3  # every fourth case: a grid for the 256-row kernel
    D = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 4, 8]))
    if big:  # 2 x 64 heads x >= 2 query tiles of 256: over half of 256 CUs
        B, Hkv = 2, 64 // G
        Sq = int(rng.integers(260, 520))
    else:
        B, Hkv = int(rng.integers(1, 3)), int(rng.choice([1, 2]))
        Sq = int(rng.integers(1, 700))
    Sk = Sq if rng.random() < 0.5 else int(rng.integers(1, 520 if big else 700))
    causal = bool(rng.random() < 0.5)
    dtype = str(rng.choice(["bf16", "fp16"]))
    variant = str(rng.choice(["plain", "alibi", "mask", "alibi+mask"]))
    return B, Hkv * G, Hkv, Sq, Sk, D, causal, dtype, variant


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_case(case):
    B, Hq, Hkv, Sq, Sk, D, causal, dtype, variant = _draw(case)
    what = f"case {case}: B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Sk={Sk} D={D} causal={causal} {dtype} {variant}"
    _say(what)
    q, k, v = random_qkv(B, Hq, Hkv, Sq, Sk, D, dtype=dtype, seed=2000 + case)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    slopes = alibi_slopes(Hq) if "alibi" in variant else None
    mask = random_block_mask(Hq if case % 2 else 1, Sq, Sk, seed=3000 + case, p_visible=0.6) \
        if "mask" in variant else None
    o, lse = ta.forward(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale,
                        alibi_slopes=None if slopes is None else slopes.cuda(),
                        block_mask=None if mask is None else mask.cuda())
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_ext(q, k, v, scale, causal, slopes, mask)
    o = o.to("cpu", torch.float64).numpy()
    lse = lse.to("cpu", torch.float64).numpy()
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: empty rows differ"
    assert np.all(o[empty] == 0), f"{what}: empty rows not zero"
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    live = ~empty
    tol = TOL[dtype]
    err = np.abs(o[live] - o_ref[live]) if live.any() else np.zeros(1)
    lerr = np.abs(lse[live] - lse_ref[live]) if live.any() else np.zeros(1)
    _say(f"  max|dO|={err.max():.3e} mean|dO|={err.mean():.3e} max|dlse|={lerr.max():.3e}")
    assert err.max() <= tol["max"], what
    assert err.mean() <= tol["mean"], what
    assert lerr.max() <= tol["lse"], what
