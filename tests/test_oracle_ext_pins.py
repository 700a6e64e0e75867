"""Pins for ``oracle.attention_ext`` (ALiBi bias, block-sparse mask), CPU only.

The function is checked against facts that do not come from it:
  * it reduces to ``oracle.attention`` (pinned separately) when the slopes
    are zero and the mask shows everything;
  * PyTorch's scaled_dot_product_attention in float64 with the bias and the
    mask given as an additive float mask (a library routine), and
    torch.logsumexp over the same masked scores for lse;
  * closed forms: with Q = 0 every score is the bias alone, so the weights
    are a geometric sequence in the query-key distance and lse is the log of
    a geometric sum;
  * a mask that shows one block is plain attention of that block's rows
    against that block's keys; a mask that shows nothing gives o = 0,
    lse = -inf;
  * planted mistakes in the oracle (bias sign, distance direction, mask
    transposed) fail these pins.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import biased as biased_mod
from tiled_attention_tileattn_amd.inputs import random_qkv

BLOCK = 64


def _slopes(Hq, base=8.0):
    # the geometric slopes of the ALiBi paper: 2^(-base*h/Hq), h = 1..Hq
    return np.array([2.0 ** (-base * (h + 1) / Hq) for h in range(Hq)])


def _random_mask(Hm, Sq, Sk, seed, p=0.6):
    rng = np.random.default_rng(seed)
    nq, nk = -(-Sq // BLOCK), -(-Sk // BLOCK)
    m = (rng.random((Hm, nq, nk)) < p).astype(np.uint8)
    m[:, :, 0] = 1          # every row keeps key block 0 (so no row is empty)
    return m


def _sdpa_reference(q, k, v, scale, causal, slopes, mask):
    """o and lse from torch (float64), bias and mask as one additive mask."""
    q, k, v = (t.double() for t in (q, k, v))
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    k = k.repeat_interleave(G, dim=1)
    v = v.repeat_interleave(G, dim=1)
    i = torch.arange(Sq, dtype=torch.float64)[:, None]
    j = torch.arange(Sk, dtype=torch.float64)[None, :]
    add = torch.zeros(Hq, Sq, Sk, dtype=torch.float64)
    if slopes is not None:
        dist = (i - j) if causal else (i - j).abs()
        add = add - torch.as_tensor(slopes, dtype=torch.float64)[:, None, None] * dist
    vis = torch.ones(Hq, Sq, Sk, dtype=torch.bool)
    if causal:
        vis &= (j <= i)
    if mask is not None:
        mt = torch.as_tensor(mask).bool()
        mt = mt.expand(Hq, -1, -1) if mt.shape[0] == 1 else mt
        full = mt.repeat_interleave(BLOCK, dim=1).repeat_interleave(BLOCK, dim=2)[:, :Sq, :Sk]
        vis &= full
    add = add.masked_fill(~vis, float("-inf"))
    o = F.scaled_dot_product_attention(q, k, v, attn_mask=add[None], scale=scale)
    s = torch.einsum("bhid,bhjd->bhij", q, k) * scale + add[None]
    lse = torch.logsumexp(s, dim=-1)
    return o.numpy(), lse.numpy()


CASES = [
    # B, Hq, Hkv, Sq, Sk, D, causal
    (1, 4, 2, 70, 90, 16, False),
    (2, 2, 1, 130, 130, 8, True),
    (1, 8, 4, 65, 200, 16, True),
    (1, 2, 2, 1, 1, 8, False),
]


@pytest.mark.parametrize("case", CASES)
def test_reduces_to_plain_attention(case):
    B, Hq, Hkv, Sq, Sk, D, causal = case
    q, k, v = random_qkv(B, Hq, Hkv, Sq, Sk, D, dtype="fp32", seed=61)
    o0, l0 = oracle.attention(q, k, v, 0.3, causal)
    ones = np.ones((1, -(-Sq // BLOCK), -(-Sk // BLOCK)), dtype=np.uint8)
    for slopes, mask in [(None, None), (np.zeros(Hq), None), (None, ones), (np.zeros(Hq), ones)]:
        o, l = oracle.attention_ext(q, k, v, 0.3, causal, slopes, mask)
        np.testing.assert_allclose(o, o0, atol=1e-12)
        np.testing.assert_allclose(l, l0, atol=1e-12)


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("per_head", [False, True])
def test_matches_sdpa_with_additive_mask(case, per_head):
    B, Hq, Hkv, Sq, Sk, D, causal = case
    q, k, v = random_qkv(B, Hq, Hkv, Sq, Sk, D, dtype="fp32", seed=62 + Sq)
    slopes = _slopes(Hq)
    mask = _random_mask(Hq if per_head else 1, Sq, Sk, seed=Sk)
    scale = 1.0 / math.sqrt(D)
    o, l = oracle.attention_ext(q, k, v, scale, causal, slopes, mask)
    o_ref, l_ref = _sdpa_reference(q, k, v, scale, causal, slopes, mask)
    np.testing.assert_allclose(o, o_ref, atol=1e-10)
    np.testing.assert_allclose(l, l_ref, atol=1e-10)


@pytest.mark.parametrize("causal", [True, False])
def test_alibi_with_zero_queries_is_geometric(causal):
    Hq, S, D = 3, 40, 8
    _, k, v = random_qkv(1, Hq, 1, S, S, D, dtype="fp32", seed=63)
    q = torch.zeros(1, Hq, S, D)
    slopes = np.array([0.5, 0.1, 1.3])
    o, l = oracle.attention_ext(q, k, v, 0.7, causal, slopes, None)
    vv = v[0, 0].double().numpy()
    for h, m in enumerate(slopes):
        r = math.exp(-m)
        for i in (0, 1, 17, S - 1):
            if causal:
                # weights r^(i-j), j = 0..i; sum = (1 - r^(i+1)) / (1 - r)
                w = np.array([r ** (i - j) for j in range(i + 1)])
                lse = math.log((1 - r ** (i + 1)) / (1 - r))
                ref = w @ vv[: i + 1] / w.sum()
            else:
                # weights r^|i-j|; sum = (1 - r^(i+1))/(1 - r) + r (1 - r^(S-1-i))/(1 - r)
                w = np.array([r ** abs(i - j) for j in range(S)])
                lse = math.log((1 - r ** (i + 1)) / (1 - r) + r * (1 - r ** (S - 1 - i)) / (1 - r))
                ref = w @ vv / w.sum()
            assert abs(l[0, h, i] - lse) < 1e-12
            np.testing.assert_allclose(o[0, h, i], ref, atol=1e-12)


def test_single_visible_block_is_plain_attention_of_that_block():
    Sq, Sk, D = 150, 200, 16
    q, k, v = random_qkv(1, 2, 1, Sq, Sk, D, dtype="fp32", seed=64)
    mask = np.zeros((1, 3, 4), dtype=np.uint8)
    mask[0, 1, 2] = 1                               # rows 64..127 see keys 128..191
    o, l = oracle.attention_ext(q, k, v, 0.25, False, None, mask)
    o_blk, l_blk = oracle.attention(q[:, :, 64:128], k[:, :, 128:192], v[:, :, 128:192], 0.25, False)
    np.testing.assert_allclose(o[:, :, 64:128], o_blk, atol=1e-12)
    np.testing.assert_allclose(l[:, :, 64:128], l_blk, atol=1e-12)
    rest = np.r_[0:64, 128:150]
    assert np.all(o[:, :, rest] == 0) and np.all(np.isneginf(l[:, :, rest]))


def test_mask_that_shows_nothing_gives_empty_rows():
    q, k, v = random_qkv(1, 2, 2, 10, 70, 8, dtype="fp32", seed=65)
    o, l = oracle.attention_ext(q, k, v, 1.0, True, _slopes(2), np.zeros((1, 1, 2), np.uint8))
    assert np.all(o == 0) and np.all(np.isneginf(l))


def test_shared_mask_equals_identical_per_head_planes():
    q, k, v = random_qkv(1, 4, 2, 100, 100, 8, dtype="fp32", seed=66)
    m1 = _random_mask(1, 100, 100, seed=3)
    o1, l1 = oracle.attention_ext(q, k, v, 0.5, True, _slopes(4), m1)
    o2, l2 = oracle.attention_ext(q, k, v, 0.5, True, _slopes(4), np.repeat(m1, 4, axis=0))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_rejects_bad_mask_and_slopes():
    q, k, v = random_qkv(1, 2, 1, 10, 10, 8, dtype="fp32", seed=67)
    with pytest.raises(ValueError):
        oracle.attention_ext(q, k, v, 1.0, False, np.ones(3), None)
    with pytest.raises(ValueError):
        oracle.attention_ext(q, k, v, 1.0, False, None, np.ones((2 + 1, 1, 1), np.uint8))


# ---- planted mistakes -----------------------------------------------------
def _mutant(kind):
    orig = biased_mod._rows

    def rows(qh, kh, vh, r, scale, causal, slope, plane, block):
        if kind == "bias_sign" and slope is not None:
            slope = -slope
        if kind == "mask_transposed" and plane is not None:
            plane = plane.T
        if kind == "distance_direction" and slope is not None and causal:
            # b = -m (j - i) instead of -m (i - j)
            Sk = kh.shape[0]
            s = (qh @ kh.T) * scale - slope * (np.arange(Sk)[None, :] - r[:, None])
            vis = biased_mod._visible(r, Sk, causal, plane, block)
            s = np.where(vis, s, -np.inf)
            mx = s.max(axis=1, keepdims=True)
            e = np.exp(s - mx)
            return (e / e.sum(axis=1, keepdims=True)) @ vh, mx[:, 0] + np.log(e.sum(axis=1))
        return orig(qh, kh, vh, r, scale, causal, slope, plane, block)

    return rows


def _ext_pins_pass():
    try:
        test_matches_sdpa_with_additive_mask(CASES[1], True)
        test_matches_sdpa_with_additive_mask(CASES[0], False)
        test_alibi_with_zero_queries_is_geometric(True)
        test_single_visible_block_is_plain_attention_of_that_block()
        return True
    except (AssertionError, ValueError, IndexError):
        return False


@pytest.mark.parametrize("kind", ["bias_sign", "mask_transposed", "distance_direction"])
def test_planted_mistakes_are_caught(kind, monkeypatch):
    assert _ext_pins_pass()
    monkeypatch.setattr(biased_mod, "_rows", _mutant(kind))
    assert not _ext_pins_pass()
