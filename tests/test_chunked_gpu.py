"""Parity of the chunked key split (``tileattn_fwd_ws``) with the fp64 oracle
(needs an MI355X).

Where few query tiles cover long key ranges, ``tileattn_fwd_ws`` cuts each
query tile's key tiles into chunks that run as separate workgroups and merges
their partial softmax states in a second kernel.  Every case below asserts
that the library does take chunks for it (a workspace size above zero), so
the tests exercise that path and not the plain one.

Cases: several chunks per query tile with an odd, one-tile or ragged last
chunk; causal query tiles with one chunk beside tiles with several (the
light ones write their rows directly, the heavy ones go through the merge);
Sq > Sk causal; single query rows (decode); fp16; and, at full size, one KV
head's share of the causal GQA 8K workload (B=1, Hq=4, Hkv=1, S=8192) on
sampled rows, plus every row against the unsplit kernel.
Tolerances are the plain path's (bf16: max 2e-2, mean 2e-3; fp16: max 4e-3,
mean 4e-4; lse 1e-3): the split changes only the order in which the same
fp32 partial sums are added.
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import tiled_attention_tileattn_amd as ta
from tiled_attention_tileattn_amd.inputs import WORKLOADS, alibi_slopes, make_inputs, random_qkv

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


def _check(o, lse, o_ref, lse_ref, dtype, what):
    tol = TOL[dtype]
    o = o.detach().to("cpu", torch.float64).numpy()
    lse = lse.detach().to("cpu", torch.float64).numpy()
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    err = np.abs(o - o_ref)
    lerr = float(np.abs(lse - lse_ref).max())
    _say(f"  {what}: max|dO|={err.max():.3e} mean|dO|={err.mean():.3e} max|dlse|={lerr:.3e}")
    assert err.max() <= tol["max"], what
    assert err.mean() <= tol["mean"], what
    assert lerr <= tol["lse"], what


CASES = [
    # B, Hq, Hkv, Sq, Sk, D, causal, dtype
    (1, 1, 1, 128, 4096, 64, False, "bf16"),     # 64 key tiles in 4 chunks of 16
    (1, 2, 1, 200, 3390, 128, False, "bf16"),    # 53 tiles: 3 x 16 + 5, ragged Sq and Sk
    (1, 1, 1, 4096, 4096, 128, True, "bf16"),    # causal: 1 to 4 chunks per query tile
    (1, 2, 2, 5000, 3500, 64, True, "fp16"),     # causal, Sq > Sk
    (2, 4, 1, 1, 8192, 128, False, "bf16"),      # one query row per head, 8 chunks
    (1, 4, 2, 64, 20000, 128, False, "fp16"),    # 313 tiles: 19 chunks of 16 and one of 9
    (1, 2, 1, 3, 16 * 1024 + 70, 64, False, "bf16"),  # 258 tiles = 16 x 16 + 2
]


@pytest.mark.parametrize("case", CASES)
def test_chunked_matches_oracle_and_plain_kernel(case):
    B, Hq, Hkv, Sq, Sk, D, causal, dtype = case
    what = f"B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Sk={Sk} D={D} causal={causal} {dtype}"
    _say(what)
    assert ta.tileattn_fwd_workspace_size(B, Hq, Hkv, Sq, Sk, D, causal) > 0, "no chunks for this case"
    q, k, v = random_qkv(B, Hq, Hkv, Sq, Sk, D, dtype=dtype, seed=Sq + Sk + D)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o, lse = ta.forward(qd, kd, vd, causal=causal, scale=scale)
    o1, lse1 = ta.forward(qd, kd, vd, causal=causal, scale=scale, key_chunks=False)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(q, k, v, scale, causal)
    _check(o, lse, o_ref, lse_ref, dtype, "chunked")
    _check(o1, lse1, o_ref, lse_ref, dtype, "plain")
    d = (o.double() - o1.double()).abs()
    assert d.max().item() <= TOL[dtype]["max"] and d.mean().item() <= TOL[dtype]["mean"]


def test_chunked_is_deterministic_and_reusable():
    # The same workspace for two different problems in a row, then the first
    # again: every result is bitwise the one of a fresh call.
    B, Hq, Hkv, D = 1, 4, 1, 128
    scale = float(np.float32(1.0 / math.sqrt(D)))
    a = [t.cuda() for t in random_qkv(B, Hq, Hkv, 300, 5000, D, dtype="bf16", seed=91)]
    b = [t.cuda() for t in random_qkv(B, Hq, Hkv, 4000, 4000, D, dtype="bf16", seed=92)]
    n_a = ta.tileattn_fwd_workspace_size(B, Hq, Hkv, 300, 5000, D, False)
    n_b = ta.tileattn_fwd_workspace_size(B, Hq, Hkv, 4000, 4000, D, True)
    assert n_a > 0 and n_b > 0
    ws = torch.empty(max(n_a, n_b), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def run(x, Sq, Sk, causal):
        o = torch.empty_like(x[0])
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device="cuda")
        rc = ta.tileattn_fwd_ws(x[0].data_ptr(), x[1].data_ptr(), x[2].data_ptr(), o.data_ptr(),
                                lse.data_ptr(), B, Hq, Hkv, Sq, Sk, D, scale, causal, None, 0,
                                ws.data_ptr(), ws.numel(), stream)
        assert rc == 0, ta.tileattn_strerror(rc)
        return o, lse

    ra1 = run(a, 300, 5000, False)
    rb = run(b, 4000, 4000, True)
    ra2 = run(a, 300, 5000, False)
    fa = ta.forward(*a, causal=False, scale=scale)
    fb = ta.forward(*b, causal=True, scale=scale)
    torch.cuda.synchronize()
    for x, y in ((ra1, fa), (ra2, fa), (rb, fb)):
        assert torch.equal(x[0], y[0]) and torch.equal(x[1], y[1])


def test_head_shard_of_causal_gqa_8k_sampled_rows():
    # One KV head's share of the headline workload: 4 query heads of 64 query
    # tiles, the heaviest with 128 key tiles in two chunks.  Rows: a seeded
    # sample plus the edges of the first, a middle and the last query tile
    # of every head, against the oracle; every row against the unsplit kernel.
    w = WORKLOADS["causal_gqa_bf16"]
    q, k, v = make_inputs(w)
    q, k, v = q[:, :4].contiguous(), k[:, :1].contiguous(), v[:, :1].contiguous()
    B, Hq, Hkv, Sq, Sk, D = 1, 4, 1, w.Sq, w.Sk, w.D
    assert ta.tileattn_fwd_workspace_size(B, Hq, Hkv, Sq, Sk, D, True) > 0
    _say("head shard of causal_gqa_bf16 (chunked)")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o, lse = ta.forward(qd, kd, vd, causal=True, scale=w.scale)
    o1, lse1 = ta.forward(qd, kd, vd, causal=True, scale=w.scale, key_chunks=False)
    torch.cuda.synchronize()
    rng = np.random.default_rng(8192)
    rows = set(rng.choice(Hq * Sq, 192, replace=False).tolist())
    for h in range(Hq):
        for r in (0, 1, 127, 128, 4095, 4096, 4223, Sq - 129, Sq - 128, Sq - 2, Sq - 1):
            rows.add(h * Sq + r)
    rows = np.array(sorted(rows), dtype=np.int64)
    idx = torch.as_tensor(rows, device="cuda")
    o_ref, lse_ref = oracle.attention_rows(q, k, v, w.scale, True, rows)
    _check(o.reshape(-1, D)[idx], lse.reshape(-1)[idx], o_ref, lse_ref, "bf16", f"{len(rows)} rows")
    d = (o.double() - o1.double()).abs()
    dl = (lse - lse1).abs().max().item()
    _say(f"  vs unsplit, all rows: max|dO|={d.max().item():.3e} mean|dO|={d.mean().item():.3e} max|dlse|={dl:.3e}")
    assert d.max().item() <= 2e-2 and d.mean().item() <= 2e-3 and dl <= 1e-3


def test_decode_rows_against_32k_keys():
    # Decode shape at full context: 1 query row per head, 32 query heads over
    # 8 KV heads of 32768 keys (the long-context workload's heads), all rows.
    B, Hq, Hkv, Sq, Sk, D = 1, 32, 8, 1, 32768, 128
    assert ta.tileattn_fwd_workspace_size(B, Hq, Hkv, Sq, Sk, D, False) > 0
    _say("decode rows against 32K keys (chunked)")
    q, k, v = random_qkv(B, Hq, Hkv, Sq, Sk, D, dtype="bf16", seed=32768, q_std=0.5, k_std=0.5)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    o, lse = ta.forward(q.cuda(), k.cuda(), v.cuda(), causal=False, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(q, k, v, scale, False)
    _check(o, lse, o_ref, lse_ref, "bf16", "all rows")


def _draw(case):
    # Seeded shapes that the chunked key split takes: short queries against
    # 3K-40K keys (non-causal), or causal heads of 3K-4.5K positions (one or
    # two heads, to keep the oracle within a few seconds).
    rng = np.random.default_rng(5000 + case)
    D = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 4, 8]))
    dtype = str(rng.choice(["bf16", "fp16"]))
    if case % 2:
        B, Hkv = 1, 1
        Hq = int(rng.choice([1, 2]))
        G = Hq
        Sq = Sk = int(rng.integers(3100, 4500))
        causal = True
    else:
        B, Hkv = int(rng.integers(1, 3)), int(rng.choice([1, 2]))
        Hq = Hkv * G
        Sq = int(rng.integers(1, 300))
        Sk = int(rng.integers(3100, 40000))
        causal = False  # top-left causal rows this short would see < 300 keys
    return B, Hq, Hkv, Sq, Sk, D, causal, dtype


@pytest.mark.parametrize("case", range(12))
def test_chunked_random_case(case):
    B, Hq, Hkv, Sq, Sk, D, causal, dtype = _draw(case)
    what = f"case {case}: B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Sk={Sk} D={D} causal={causal} {dtype}"
    _say(what)
    assert ta.tileattn_fwd_workspace_size(B, Hq, Hkv, Sq, Sk, D, causal) > 0, "no chunks for this case"
    q, k, v = random_qkv(B, Hq, Hkv, Sq, Sk, D, dtype=dtype, seed=6000 + case)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    o, lse = ta.forward(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(q, k, v, scale, causal)
    _check(o, lse, o_ref, lse_ref, dtype, what)


ALIBI_CASES = [
    # B, Hq, Hkv, Sq, Sk, D, causal, dtype, slopes ("geo": the ALiBi recipe)
    (1, 4, 1, 4000, 4000, 128, True, "bf16", "geo"),     # causal: walks its chunk from the diagonal down
    (1, 8, 2, 1, 20000, 128, False, "bf16", "geo"),      # decode rows, |i - j| bias
    (2, 2, 2, 150, 7000, 64, False, "fp16", "geo"),
    (1, 2, 1, 3300, 3300, 64, True, "fp16", [0.5, 0.0]),  # a steep slope and none
]


@pytest.mark.parametrize("case", ALIBI_CASES)
def test_chunked_alibi(case):
    # The linear bias through tileattn_fwd_ws: every chunk starts its scores
    # from the bias of its own key tiles.  Against the biased oracle, and
    # against tileattn_fwd_ext (no chunks).
    B, Hq, Hkv, Sq, Sk, D, causal, dtype, sl = case
    what = f"ALiBi B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Sk={Sk} D={D} causal={causal} {dtype}"
    _say(what)
    assert ta.tileattn_fwd_workspace_size(B, Hq, Hkv, Sq, Sk, D, causal) > 0
    q, k, v = random_qkv(B, Hq, Hkv, Sq, Sk, D, dtype=dtype, seed=Sq + Sk)
    slopes = alibi_slopes(Hq) if sl == "geo" else torch.tensor(sl, dtype=torch.float32)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    qd, kd, vd, sd = q.cuda(), k.cuda(), v.cuda(), slopes.cuda()
    o, lse = ta.forward(qd, kd, vd, causal=causal, scale=scale, alibi_slopes=sd)
    o1, lse1 = ta.forward(qd, kd, vd, causal=causal, scale=scale, alibi_slopes=sd, key_chunks=False)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_ext(q, k, v, scale, causal, slopes, None)
    _check(o, lse, o_ref, lse_ref, dtype, "chunked")
    _check(o1, lse1, o_ref, lse_ref, dtype, "unsplit")


def test_chunked_on_a_side_stream():
    # forward() on a stream other than the current one: the workspace it
    # allocates is recorded on that stream, so back-to-back calls there (each
    # freeing its workspace to the allocator on return) still give the same
    # result as one call on the current stream.
    B, Hq, Hkv, Sq, Sk, D = 1, 8, 2, 64, 12000, 128
    assert ta.tileattn_fwd_workspace_size(B, Hq, Hkv, Sq, Sk, D, False) > 0
    q, k, v = (t.cuda() for t in random_qkv(B, Hq, Hkv, Sq, Sk, D, dtype="bf16", seed=77))
    o_ref, l_ref = ta.forward(q, k, v)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    outs = [ta.forward(q, k, v, stream=side) for _ in range(4)]
    side.synchronize()
    for o, lse in outs:
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
