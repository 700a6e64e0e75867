"""Pins of the CPU oracle to facts outside the oracle (CPU only).

Each test ties the oracle to something it does not compute itself: a closed
form, an invariant of softmax attention, an independent library routine, or
a brute-force loop.  ``test_planted_mistakes_are_caught`` plants plausible
mistakes in a copy of the oracle and checks that at least one pin fails for
each, so the pins are known to have teeth.
"""

import math

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle
from oracle import full_softmax as oracle_mod
from tiled_attention_tileattn_amd.inputs import WORKLOADS, make_inputs, random_qkv

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def _f64(x):
    return torch.as_tensor(x, dtype=torch.float64) if not torch.is_tensor(x) else x.to(torch.float64)


# ---------------------------------------------------------------------------
# Library routine: PyTorch SDPA in float64 on the CPU (top-left causal, GQA).
# ---------------------------------------------------------------------------
def _torch_reference(q, k, v, scale, causal):
    q, k, v = _f64(q), _f64(k), _f64(v)
    Hq, Hkv = q.shape[1], k.shape[1]
    o = F.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=scale,
                                       enable_gqa=(Hq != Hkv))
    kr = k.repeat_interleave(Hq // Hkv, dim=1)
    s = torch.matmul(q, kr.transpose(-1, -2).contiguous()) * scale
    if causal:
        Sq, Sk = q.shape[2], k.shape[2]
        vis = torch.ones(Sq, Sk, dtype=torch.bool).tril()
        s = s.masked_fill(~vis, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return o.numpy(), lse.numpy()


SHAPES = [
    # B, Hq, Hkv, Sq, Sk, D, causal
    (1, 1, 1, 5, 5, 8, False),
    (2, 4, 2, 7, 11, 16, True),
    (1, 8, 1, 13, 3, 8, True),
    (2, 6, 3, 16, 16, 32, False),
    (1, 4, 4, 1, 9, 64, True),
    (1, 2, 1, 9, 1, 64, False),
]


@pytest.mark.parametrize("shape", SHAPES)
def test_matches_torch_sdpa(shape):
    B, Hq, Hkv, Sq, Sk, D, causal = shape
    q, k, v = random_qkv(B, Hq, Hkv, Sq, Sk, D, dtype="fp32", seed=11)
    scale = 1.0 / math.sqrt(D)
    o, lse = oracle.attention(q, k, v, scale, causal)
    o_ref, lse_ref = _torch_reference(q, k, v, scale, causal)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Brute force by the definition (pure Python, math.fsum).
# ---------------------------------------------------------------------------
BRUTE = [
    (1, 1, 1, 1, 1, 4, False), (1, 1, 1, 1, 1, 4, True),
    (1, 2, 1, 3, 7, 4, True), (1, 4, 2, 7, 3, 8, True), (2, 4, 4, 13, 16, 4, False),
    (1, 8, 1, 16, 13, 4, True), (1, 2, 2, 16, 16, 8, True), (1, 8, 8, 2, 2, 4, False),
]


@pytest.mark.parametrize("shape", BRUTE)
def test_bruteforce_agrees(shape):
    B, Hq, Hkv, Sq, Sk, D, causal = shape
    q, k, v = random_qkv(B, Hq, Hkv, Sq, Sk, D, dtype="bf16", seed=sum(shape[:6]))
    scale = float(np.float32(1.0 / math.sqrt(D)))
    o, lse = oracle.attention(q, k, v, scale, causal)
    ob, lb = oracle.attention_bruteforce(q, k, v, scale, causal)
    np.testing.assert_allclose(o, np.array(ob), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(lb), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Closed forms.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_single_key_returns_value_row(causal):
    q, k, v = random_qkv(2, 4, 2, 9, 1, 16, dtype="bf16", seed=3)
    scale = 0.25
    o, lse = oracle.attention(q, k, v, scale, causal)
    qd, kd, vd = _f64(q).numpy(), _f64(k).numpy(), _f64(v).numpy()
    for b in range(2):
        for h in range(4):
            hk = h // 2
            np.testing.assert_array_equal(o[b, h], np.broadcast_to(vd[b, hk, 0], o[b, h].shape))
            dots = np.array([math.fsum(qd[b, h, i] * kd[b, hk, 0]) for i in range(9)])
            np.testing.assert_allclose(lse[b, h], scale * dots, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_gives_mean_of_visible_values(causal):
    B, Hq, Hkv, Sq, Sk, D = 1, 4, 2, 12, 10, 8
    _, k, v = random_qkv(B, Hq, Hkv, Sq, Sk, D, dtype="fp32", seed=5)
    q = torch.zeros(B, Hq, Sq, D)
    o, lse = oracle.attention(q, k, v, 0.125, causal)
    vd = _f64(v).numpy()
    for h in range(Hq):
        for i in range(Sq):
            n = min(i + 1, Sk) if causal else Sk
            mean = np.array([math.fsum(vd[0, h // 2, :n, d]) / n for d in range(D)])
            np.testing.assert_allclose(o[0, h, i], mean, rtol=0, atol=1e-13)
            assert abs(lse[0, h, i] - math.log(n)) < 1e-13


def test_zero_scale_gives_mean_for_any_query():
    q, k, v = random_qkv(1, 2, 1, 6, 6, 8, dtype="fp32", seed=8)
    o, lse = oracle.attention(q, k, v, 0.0, causal=True)
    vd = _f64(v).numpy()
    for i in range(6):
        np.testing.assert_allclose(o[0, 1, i], vd[0, 0, : i + 1].mean(axis=0), atol=1e-13)
        assert abs(lse[0, 1, i] - math.log(i + 1)) < 1e-13


@pytest.mark.parametrize("c", [0.75, -1.5])
@pytest.mark.parametrize("causal", [False, True])
def test_constant_values_return_the_constant(c, causal):
    q, k, _ = random_qkv(1, 4, 1, 11, 11, 16, dtype="bf16", seed=9)
    v = torch.full((1, 1, 11, 16), c, dtype=torch.bfloat16)
    o, _ = oracle.attention(q, k, v, 0.25, causal)
    np.testing.assert_allclose(o, c, rtol=0, atol=1e-14)


def test_two_keys_logistic_weights():
    """Two keys: weights are logistic in the score difference; lse = logaddexp."""
    q, k, v = random_qkv(1, 3, 1, 4, 2, 8, dtype="fp32", seed=13)
    scale = 0.5
    o, lse = oracle.attention(q, k, v, scale, causal=False)
    qd, kd, vd = _f64(q).numpy()[0], _f64(k).numpy()[0, 0], _f64(v).numpy()[0, 0]
    for h in range(3):
        s0 = scale * (qd[h] @ kd[0])
        s1 = scale * (qd[h] @ kd[1])
        w0 = scipy.special.expit(s0 - s1)
        np.testing.assert_allclose(o[0, h], w0[:, None] * vd[0] + (1 - w0)[:, None] * vd[1],
                                   rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[0, h], np.logaddexp(s0, s1), rtol=0, atol=1e-13)


def test_hand_worked_example():
    """Scores 0 and ln 3 give weights 1/4 and 3/4 (worked by hand)."""
    ln3 = math.log(3.0)
    q = torch.tensor([[[[ln3, 0.0], [ln3, 0.0]]]], dtype=torch.float64)    # Sq=2
    k = torch.tensor([[[[0.0, 1.0], [1.0, 0.0]]]], dtype=torch.float64)    # s = [0, ln3]
    v = torch.tensor([[[[4.0, 0.0], [0.0, 8.0]]]], dtype=torch.float64)
    o, lse = oracle.attention(q, k, v, 1.0, causal=False)
    np.testing.assert_allclose(o[0, 0], [[1.0, 6.0], [1.0, 6.0]], atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], [math.log(4.0)] * 2, atol=1e-14)
    o, lse = oracle.attention(q, k, v, 1.0, causal=True)
    np.testing.assert_allclose(o[0, 0], [[4.0, 0.0], [1.0, 6.0]], atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], [0.0, math.log(4.0)], atol=1e-14)


# ---------------------------------------------------------------------------
# Invariants.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_softmax_rows_sum_to_one(causal):
    q, k, v = random_qkv(1, 4, 2, 20, 17, 16, dtype="bf16", seed=21)
    scale = 0.25
    _, lse = oracle.attention(q, k, v, scale, causal)
    s = torch.matmul(_f64(q), _f64(k).repeat_interleave(2, 1).transpose(-1, -2).contiguous()) * scale
    for i in range(20):
        n = min(i + 1, 17) if causal else 17
        tot = torch.exp(s[0, :, i, :n] - torch.as_tensor(lse[0, :, i])[:, None]).sum(-1)
        np.testing.assert_allclose(tot.numpy(), 1.0, rtol=0, atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv():
    q, k, v = random_qkv(2, 8, 2, 10, 14, 16, dtype="bf16", seed=31)
    o1, l1 = oracle.attention(q, k, v, 0.25, True)
    o2, l2 = oracle.attention(q, k.repeat_interleave(4, 1), v.repeat_interleave(4, 1), 0.25, True)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_key_permutation_invariance_noncausal():
    q, k, v = random_qkv(1, 2, 1, 7, 15, 16, dtype="bf16", seed=41)
    perm = torch.randperm(15, generator=torch.Generator().manual_seed(0))
    o1, l1 = oracle.attention(q, k, v, 0.25, False)
    o2, l2 = oracle.attention(q, k[:, :, perm], v[:, :, perm], 0.25, False)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)


def test_causal_row_zero_is_first_value_row():
    q, k, v = random_qkv(2, 4, 2, 5, 8, 16, dtype="bf16", seed=51)
    o, _ = oracle.attention(q, k, v, 0.25, True)
    vd = _f64(v).numpy()
    for h in range(4):
        np.testing.assert_array_equal(o[:, h, 0], vd[:, h // 2, 0])


def test_rows_sampler_matches_full():
    q, k, v = random_qkv(2, 4, 2, 33, 29, 16, dtype="bf16", seed=61)
    o, lse = oracle.attention(q, k, v, 0.25, True)
    rows = np.array([0, 5, 32, 33, 100, 2 * 4 * 33 - 1, 77])
    o_s, l_s = oracle.attention_rows(q, k, v, 0.25, True, rows)
    # Same definition; only BLAS blocking (hence rounding order) may differ.
    np.testing.assert_allclose(o_s, o.reshape(-1, 16)[rows], rtol=0, atol=1e-13)
    np.testing.assert_allclose(l_s, lse.reshape(-1)[rows], rtol=0, atol=1e-13)


def test_threads_do_not_change_results():
    q, k, v = random_qkv(1, 6, 3, 40, 40, 16, dtype="bf16", seed=71)
    o1, l1 = oracle.attention(q, k, v, 0.25, True, threads=1)
    o2, l2 = oracle.attention(q, k, v, 0.25, True, threads=4)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


# ---------------------------------------------------------------------------
# The pins have teeth: plausible mistakes planted in a copy of the oracle.
# ---------------------------------------------------------------------------
def _mutant_head_rows(kind):
    orig = oracle_mod._head_rows

    def wrong(qh, kh, vh, rows, scale, causal):
        if kind == "no_scale":
            return orig(qh, kh, vh, rows, 1.0, causal)
        if kind == "strict_causal":       # j < i instead of j <= i
            Sk = kh.shape[0]
            s = (qh @ kh.T) * scale
            s = np.where(np.arange(Sk)[None, :] < np.maximum(rows[:, None], 1), s, -np.inf)
            m = s.max(1, keepdims=True)
            e = np.exp(s - m)
            return (e / e.sum(1, keepdims=True)) @ vh, m[:, 0] + np.log(e.sum(1))
        if kind == "lse_log2":
            o, lse = orig(qh, kh, vh, rows, scale, causal)
            return o, lse / math.log(2.0)
        if kind == "k_transposed_rows":   # keys read in reverse order
            return orig(qh, kh[::-1].copy(), vh, rows, scale, causal)
        if kind == "no_max_shift_sign":   # wrong sign inside the exponent
            s = (qh @ kh.T) * scale
            if causal:
                s = np.where(np.arange(kh.shape[0])[None, :] <= rows[:, None], s, np.inf)
            e = np.exp(-s)
            e = np.where(np.isfinite(s), e, 0.0)
            return (e / e.sum(1, keepdims=True)) @ vh, np.log(e.sum(1))
        raise AssertionError(kind)

    return wrong


def _mutant_gqa(q, k, v, scale, causal):
    """GQA mapping h % Hkv instead of h // G."""
    Hq, Hkv = q.shape[1], k.shape[1]
    idx = torch.arange(Hq) % Hkv
    return oracle.attention(q, k[:, idx].contiguous(), v[:, idx].contiguous(), scale, causal)


def _pins_pass(attn):
    """Run a compact subset of the pins against an attention function."""
    try:
        for shape in [SHAPES[1], SHAPES[2], SHAPES[3]]:
            B, Hq, Hkv, Sq, Sk, D, causal = shape
            q, k, v = random_qkv(B, Hq, Hkv, Sq, Sk, D, dtype="fp32", seed=11)
            o, lse = attn(q, k, v, 1.0 / math.sqrt(D), causal)
            o_ref, lse_ref = _torch_reference(q, k, v, 1.0 / math.sqrt(D), causal)
            np.testing.assert_allclose(o, o_ref, atol=1e-9)
            np.testing.assert_allclose(lse, lse_ref, atol=1e-9)
        return True
    except AssertionError:
        return False


@pytest.mark.parametrize("kind", ["no_scale", "strict_causal", "lse_log2", "k_transposed_rows",
                                  "no_max_shift_sign", "gqa_modulo"])
def test_planted_mistakes_are_caught(kind, monkeypatch):
    assert _pins_pass(oracle.attention)
    if kind == "gqa_modulo":
        assert not _pins_pass(_mutant_gqa)
        return
    monkeypatch.setattr(oracle_mod, "_head_rows", _mutant_head_rows(kind))
    assert not _pins_pass(oracle.attention)


# ---------------------------------------------------------------------------
# Seeded input generator.
# ---------------------------------------------------------------------------
def test_inputs_are_deterministic_and_follow_the_recipe():
    w = WORKLOADS["tiny_fp32"]
    q1, k1, v1 = make_inputs(w)
    q2, k2, v2 = make_inputs(w)
    assert torch.equal(q1, q2) and torch.equal(k1, k2) and torch.equal(v1, v2)
    g = torch.Generator("cpu").manual_seed(0)
    assert torch.equal(q1, torch.randn(1, 1, 128, 64, generator=g))
    assert q1.dtype == torch.float32 and q1.is_contiguous()
    wb = WORKLOADS["mha_bf16"].with_(Sq=16, Sk=16)
    qb, _, _ = make_inputs(wb)
    assert qb.dtype == torch.bfloat16
    g = torch.Generator("cpu").manual_seed(1)
    assert torch.equal(qb, torch.randn(4, 8, 16, 64, generator=g).to(torch.bfloat16))
    wh = WORKLOADS["causal_gqa_fp16"].with_(Sq=16, Sk=16)
    qh, kh, vh = make_inputs(wh)
    assert qh.dtype == kh.dtype == vh.dtype == torch.float16
    g = torch.Generator("cpu").manual_seed(5)
    assert torch.equal(qh, torch.randn(1, 32, 16, 128, generator=g).to(torch.float16))


def test_oracle_takes_fp16_values_exactly():
    # fp16 inputs reach the oracle as their exact binary16 values, and the
    # result is the same as for those values given in float64.
    q, k, v = random_qkv(1, 2, 1, 9, 11, 16, dtype="fp16", seed=51)
    o16, l16 = oracle.attention(q, k, v, 0.25, True)
    o64, l64 = oracle.attention(q.double(), k.double(), v.double(), 0.25, True)
    assert np.array_equal(o16, o64) and np.array_equal(l16, l64)


def test_long_context_sample_is_reproducible():
    w = WORKLOADS["longctx_gqa_bf16"].with_(Sq=64, Sk=64)
    *_, s1 = make_inputs(w, with_sample=True)
    *_, s2 = make_inputs(w, with_sample=True)
    assert np.array_equal(s1, s2) and len(s1) == 256 and len(set(s1.tolist())) == 256
    q, k, _ = make_inputs(w)
    assert abs(float(q.float().std()) - 0.5) < 0.02 and abs(float(k.float().std()) - 0.5) < 0.02


def test_workload_flop_counts():
    assert WORKLOADS["causal_gqa_bf16"].flop() == 549755813888
    assert WORKLOADS["mha_bf16"].flop() == 8589934592
    assert WORKLOADS["tiny_fp32"].scale == 0.125
