"""Parity of the ALiBi / block-sparse path (tileattn_fwd_ext) with the oracle.

Calls go through the C ABI (the ctypes binding's ``forward`` with
``alibi_slopes`` / ``block_mask``) on seeded inputs; ``oracle.attention_ext``
gets the same input values (the slopes as the float32 numbers the GPU gets).
Tolerances on O and lse are those of the plain path for the same dtype.
Rows with no visible key must come out exactly o = 0, lse = -inf.
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


def _run(B, Hq, Hkv, Sq, Sk, D, causal, dtype, seed, use_slopes, mask_heads, p_visible=0.6,
         empty_qblocks=(), scale=None):
    """use_slopes: False, True (the geometric slopes) or a list of Hq slopes."""
    what = (f"B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Sk={Sk} D={D} causal={causal} {dtype} seed={seed} "
            f"slopes={use_slopes} mask_heads={mask_heads} scale={scale}")
    _say(what)
    q, k, v = random_qkv(B, Hq, Hkv, Sq, Sk, D, dtype=dtype, seed=seed)
    scale = float(np.float32(1.0 / math.sqrt(D))) if scale is None else scale
    if isinstance(use_slopes, (list, tuple)):
        slopes = torch.tensor(use_slopes, dtype=torch.float32)
    else:
        slopes = alibi_slopes(Hq) if use_slopes else None
    mask = None
    if mask_heads:
        mask = random_block_mask(mask_heads, Sq, Sk, seed=seed + 1, p_visible=p_visible)
        for qb in empty_qblocks:
            mask[:, qb, :] = 0
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
    live = ~empty
    tol = TOL[dtype]
    assert np.isfinite(o).all()
    err = np.abs(o[live] - o_ref[live]) if live.any() else np.zeros(1)
    lerr = np.abs(lse[live] - lse_ref[live]) if live.any() else np.zeros(1)
    _say(f"  max|dO|={err.max():.3e} mean|dO|={err.mean():.3e} max|dlse|={lerr.max():.3e} "
         f"empty rows={int(empty.sum())}")
    assert err.max() <= tol["max"], what
    assert err.mean() <= tol["mean"], what
    assert lerr.max() <= tol["lse"], what
    return o, lse


SHAPES = [
    # B, Hq, Hkv, Sq, Sk, D
    (1, 4, 2, 300, 300, 128),
    (2, 2, 1, 129, 257, 64),
    (1, 8, 4, 513, 200, 128),
    (1, 2, 2, 64, 64, 64),
    (1, 1, 1, 1, 70, 128),
    (1, 4, 1, 700, 640, 128),
]
KINDS = [(True, 0), (False, 1), (False, "Hq"), (True, "Hq")]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("shape", SHAPES)
def test_ext_sweep(shape, kind, causal, dtype):
    use_slopes, mh = kind
    mh = shape[1] if mh == "Hq" else mh
    _run(*shape, causal=causal, dtype=dtype, seed=sum(shape) + 3 * causal, use_slopes=use_slopes,
         mask_heads=mh)


@pytest.mark.parametrize("causal", [False, True])
def test_ext_rows_with_no_visible_key(causal):
    # query blocks 1 and 3 see nothing; block 0 keeps key block 0 by the mask recipe
    _run(1, 4, 2, 300, 300, 128, causal, "bf16", seed=90, use_slopes=True, mask_heads=4,
         empty_qblocks=(1, 3))


def test_ext_mask_with_nothing_visible():
    _run(1, 2, 1, 130, 200, 64, True, "fp16", seed=91, use_slopes=False, mask_heads=1,
         p_visible=0.0, empty_qblocks=(0, 1, 2))


def test_ext_identity_extras_match_plain_kernel():
    q, k, v = (t.cuda() for t in random_qkv(1, 8, 2, 520, 520, 128, dtype="bf16", seed=92))
    o0, l0 = ta.forward(q, k, v, causal=True)
    ones = torch.ones(1, 9, 9, dtype=torch.uint8, device="cuda")
    zero = torch.zeros(8, dtype=torch.float32, device="cuda")
    o1, l1 = ta.forward(q, k, v, causal=True, alibi_slopes=zero, block_mask=ones)
    torch.cuda.synchronize()
    assert (o1.float() - o0.float()).abs().max().item() <= 2e-2
    assert (l1 - l0).abs().max().item() <= 1e-4


def test_ext_headline_shape_slice():
    # the headline shape restricted to one KV head (4 query heads), ALiBi +
    # a 50% block mask, against the full oracle on those heads
    _run(1, 4, 1, 8192, 8192, 128, True, "bf16", seed=93, use_slopes=True, mask_heads=4,
         p_visible=0.5)


@pytest.mark.parametrize("scale", [0.0, 1e-30, 1.0])
@pytest.mark.parametrize("mask_heads", [0, 2])
def test_ext_scale_edges(scale, mask_heads):
    # scale 0 (and below 2^-64): the scores are the bias alone
    _run(1, 2, 1, 200, 330, 64, True, "bf16", seed=94, use_slopes=True, mask_heads=mask_heads,
         scale=scale)


@pytest.mark.parametrize("causal", [False, True])
def test_ext_steep_slopes(causal):
    # slopes up to 4 per key: the weight sits on the few keys next to the row
    _run(1, 4, 2, 333, 333, 128, causal, "bf16", seed=95, use_slopes=[4.0, 1.0, 0.25, 0.0],
         mask_heads=0)


@pytest.mark.parametrize("kind", KINDS)
def test_ext_packed_heads_256_rows(kind):
    # 8 query heads per KV head on 256-row workgroups: with a block mask the
    # workgroup packs 4 heads x 64 positions (each 64-position query block
    # whole), without one (bias only) 8 heads x 32 positions; every wave
    # takes its own head's slope and mask plane.
    use_slopes, mh = kind
    mh = 64 if mh == "Hq" else mh
    _run(2, 64, 8, 600, 600, 64, True, "bf16", seed=96, use_slopes=use_slopes, mask_heads=mh)
