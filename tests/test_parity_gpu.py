"""Parity of the HIP kernels with the CPU fp64 oracle (needs an MI355X).

Every comparison calls the library through the C ABI (the ctypes binding)
on seeded inputs from ``tiled_attention_tileattn_amd.inputs`` and compares
element by element with ``oracle`` on the same input values.

Tolerances (on O, over all compared elements):
    bf16 inputs: max |err| <= 2e-2 and mean |err| <= 2e-3
    fp16 inputs: max |err| <= 4e-3 and mean |err| <= 4e-4
    fp32 inputs: max |err| <= 1e-4
The fp16 bound scales the bf16 one by the ratio of the two formats' unit
roundoffs (2^-11 / 2^-8 = 1/8) and rounds up: the error is dominated by the
rounding of P and of O to the 16-bit dtype.
On lse (not specified elsewhere; derived from the arithmetic: fp32 sums of
exact products and the hardware exp2/log): <= 1e-3 (bf16, fp16), <= 1e-4 (fp32).
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import tiled_attention_tileattn_amd as ta
from tiled_attention_tileattn_amd.inputs import WORKLOADS, make_inputs, random_qkv

pytestmark = pytest.mark.gpu

TOL = {"bf16": dict(max=2e-2, mean=2e-3, lse=1e-3), "fp16": dict(max=4e-3, mean=4e-4, lse=1e-3),
       "fp32": dict(max=1e-4, mean=1e-4, lse=1e-4)}


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


def _gpu_forward(q, k, v, causal, scale):
    qd, kd, vd = (t.to("cuda") for t in (q, k, v))
    o, lse = ta.forward(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


def _errs(o_gpu, o_ref):
    err = np.abs(o_gpu.astype(np.float64) - o_ref)
    return float(err.max()), float(err.mean())


def _check(o, lse, o_ref, lse_ref, dtype, what=""):
    tol = TOL[dtype]
    o = o.detach().to("cpu", torch.float64).numpy()
    lse = lse.detach().to("cpu", torch.float64).numpy()
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    mx, mean = _errs(o, o_ref)
    lmx = float(np.abs(lse - lse_ref).max()) if lse.size else 0.0
    _say(f"  {what}: max|dO|={mx:.3e} mean|dO|={mean:.3e} max|dlse|={lmx:.3e}")
    assert mx <= tol["max"], f"{what}: max abs err {mx}"
    assert mean <= tol["mean"], f"{what}: mean abs err {mean}"
    assert lmx <= tol["lse"], f"{what}: lse err {lmx}"


def _parity(B, Hq, Hkv, Sq, Sk, D, causal, dtype, seed, scale=None, q_std=1.0, k_std=1.0):
    scale = float(np.float32(1.0 / math.sqrt(D))) if scale is None else scale
    what = f"B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Sk={Sk} D={D} causal={causal} {dtype} seed={seed}"
    _say(what)
    q, k, v = random_qkv(B, Hq, Hkv, Sq, Sk, D, dtype=dtype, seed=seed, q_std=q_std, k_std=k_std)
    o, lse = _gpu_forward(q, k, v, causal, scale)
    o_ref, lse_ref = oracle.attention(q, k, v, scale, causal)
    _check(o, lse, o_ref, lse_ref, dtype, what)
    return q, k, v, o, lse


# ---------------------------------------------------------------------------
# Small sweep: tails around the 128-row / 64-key tiles, Sq != Sk, GQA ratios.
# ---------------------------------------------------------------------------
SWEEP = [
    # B, Hq, Hkv, Sq, Sk, D
    (1, 1, 1, 1, 1, 64), (1, 2, 1, 2, 2, 128), (1, 4, 2, 7, 13, 64), (2, 2, 2, 13, 7, 128),
    (1, 8, 1, 16, 16, 128), (1, 2, 2, 17, 17, 64), (1, 4, 1, 64, 64, 128), (1, 2, 1, 127, 129, 128),
    (2, 4, 4, 128, 128, 64), (1, 8, 2, 129, 127, 128), (1, 4, 2, 300, 300, 128),
    (1, 2, 2, 300, 65, 64), (1, 2, 1, 63, 300, 128), (1, 16, 2, 257, 257, 128),
    (1, 1, 1, 1, 300, 128), (1, 1, 1, 300, 1, 64),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SWEEP)
def test_sweep_bf16(shape, causal):
    _parity(*shape, causal=causal, dtype="bf16", seed=sum(shape))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SWEEP[1::2])
def test_sweep_fp16(shape, causal):
    _parity(*shape, causal=causal, dtype="fp16", seed=3 + sum(shape))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SWEEP[::2])
def test_sweep_fp32(shape, causal):
    _parity(*shape, causal=causal, dtype="fp32", seed=7 + sum(shape))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("heavy_half", [0, 1])
def test_key_split_merge_with_the_row_max_in_one_half(heavy_half, D):
    # This grid is small enough for the key split: one wave group takes key
    # tiles 0-9 (keys 0-639), the other tiles 10-19, the last one past Sk.
    # Keys of one half scaled by 3 put every row's max in that half, so the
    # merge scales the other half's partial state down by a large factor.
    B, Hq, Hkv, Sq, Sk = 1, 4, 2, 200, 1153
    scale = float(np.float32(1.0 / math.sqrt(D)))
    what = f"key split, max in half {heavy_half}, D={D}"
    _say(what)
    q, k, v = random_qkv(B, Hq, Hkv, Sq, Sk, D, dtype="bf16", seed=90 + heavy_half + D)
    sl = slice(0, 640) if heavy_half == 0 else slice(640, Sk)
    k[:, :, sl] = (k[:, :, sl].float() * 3).to(k.dtype)
    o, lse = _gpu_forward(q, k, v, False, scale)
    o_ref, lse_ref = oracle.attention(q, k, v, scale, False)
    _check(o, lse, o_ref, lse_ref, "bf16", what)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_scale_edge_values(dtype):
    # scale = 0: every visible key weighs the same; large scale: peaky softmax.
    _parity(1, 4, 2, 150, 150, 128, True, dtype, seed=3, scale=0.0)
    _parity(1, 4, 2, 150, 150, 64, False, dtype, seed=4, scale=1.0)
    _parity(1, 2, 1, 200, 200, 128, True, dtype, seed=5, q_std=4.0, k_std=4.0)


# ---------------------------------------------------------------------------
# Closed forms and invariants on the kernel's outputs.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_single_key_returns_value_row(causal):
    q, k, v = random_qkv(2, 8, 2, 200, 1, 128, dtype="bf16", seed=11)
    o, lse = _gpu_forward(q, k, v, causal, 0.0883883461356163)
    expect = v.repeat_interleave(4, dim=1).expand(2, 8, 200, 128)
    assert torch.equal(o.cpu(), expect), "Sk=1 must return v[0] exactly"


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_returns_mean_of_visible_values(causal):
    B, Hq, Hkv, S, D = 1, 4, 2, 333, 128
    _, k, v = random_qkv(B, Hq, Hkv, S, S, D, dtype="bf16", seed=12)
    q = torch.zeros(B, Hq, S, D, dtype=torch.bfloat16)
    o, lse = _gpu_forward(q, k, v, causal, 0.0883883461356163)
    vd = v.double().repeat_interleave(2, dim=1)
    if causal:
        mean = vd.cumsum(2) / torch.arange(1, S + 1, dtype=torch.float64)[None, None, :, None]
        lse_ref = torch.log(torch.arange(1, S + 1, dtype=torch.float64)).expand(B, Hq, S)
    else:
        mean = vd.mean(2, keepdim=True).expand(B, Hq, S, D)
        lse_ref = torch.full((B, Hq, S), math.log(S), dtype=torch.float64)
    _check(o, lse, mean.numpy(), lse_ref.numpy(), "bf16", f"zero query causal={causal}")


@pytest.mark.parametrize("c", [0.75, -1.5])
def test_constant_values_return_the_constant(c):
    q, k, _ = random_qkv(1, 4, 1, 257, 257, 128, dtype="bf16", seed=13)
    v = torch.full((1, 1, 257, 128), c, dtype=torch.bfloat16)
    o, _ = _gpu_forward(q, k, v, True, 0.0883883461356163)
    err = (o.cpu().double() - c).abs().max().item()
    assert err <= abs(c) * 2 ** -7, err   # within one bf16 ulp of c


def test_causal_row_zero_is_first_value_row():
    q, k, v = random_qkv(2, 8, 4, 130, 130, 128, dtype="bf16", seed=14)
    o, _ = _gpu_forward(q, k, v, True, 0.0883883461356163)
    assert torch.equal(o.cpu()[:, :, 0], v.repeat_interleave(2, dim=1)[:, :, 0])


# Shapes that exercise each branch of the workgroup -> (batch, head group,
# query tile) map (head groups: the query heads of a KV head one workgroup
# packs):
# whole (batch, kv head) slots per XCD (slots a multiple of 8), slots spread
# over XCDs by query-tile residue (1, 2 or 4 slots), and the uneven fallback.
MAP_CASES = [
    # B, Hq, Hkv, S, D, causal
    (1, 8, 1, 2048, 128, True),     # 1 slot, 8 query tiles: residue split over 8 XCDs
    (2, 4, 2, 1024, 128, True),     # 4 slots, 4 query tiles: residue split over 2 XCDs
    (1, 4, 2, 2048, 64, False),     # 2 slots, 8 query tiles: residue split over 4 XCDs
    (8, 2, 2, 512, 64, True),       # 16 slots: 2 whole slots per XCD
    (1, 8, 2, 1030, 64, True),      # 2 slots, 33 query tiles (4 heads x 32): fallback order
    (3, 4, 1, 600, 64, False),      # 3 slots: fallback order
]


@pytest.mark.parametrize("case", MAP_CASES)
def test_workgroup_map_cases(case):
    # These grids are small enough for the key split's 128-row workgroups;
    # the map is the same function for both workgroup sizes.
    B, Hq, Hkv, S, D, causal = case
    _parity(B, Hq, Hkv, S, S, D, causal, "bf16", seed=B * 100 + Hq + S)


# Grids of more than half a chip of 256-row workgroups keep the 8-wave
# ping-pong kernel: many heads over short, ragged sequences.
EIGHT_WAVE_CASES = [
    # B, Hq, Hkv, Sq, Sk, D, dtype
    (2, 64, 8, 300, 300, 128, "bf16"),
    (4, 40, 8, 129, 257, 64, "bf16"),
    (3, 64, 16, 200, 333, 128, "fp16"),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", EIGHT_WAVE_CASES)
def test_eight_wave_grids(case, causal):
    B, Hq, Hkv, Sq, Sk, D, dtype = case
    st, bm, _, _ = ta.tileattn_launch_shape(2, B, Hq, Hkv, Sq, Sk, D, int(causal))
    assert st == 0 and bm == 256
    _parity(B, Hq, Hkv, Sq, Sk, D, causal, dtype, seed=B + Hq + Sq + Sk)


def test_small_grids_take_128_row_workgroups():
    # The workload and sweep shapes on either side of the switch.
    assert ta.tileattn_launch_shape(2, 4, 8, 8, 1024, 1024, 64, 0)[1] == 128   # mha_bf16
    assert ta.tileattn_launch_shape(2, 1, 32, 8, 8192, 8192, 128, 1)[1] == 256  # causal GQA 8K
    assert ta.tileattn_launch_shape(2, 1, 4, 2, 300, 300, 128, 1)[1] == 128


def test_eight_wave_residue_map_on_sampled_rows():
    # One (batch, kv head) slot and 192 query tiles of 8 heads x 32
    # positions: the 8-wave kernel's residue split over the XCDs (192
    # workgroups).
    B, Hq, Hkv, S, D = 1, 8, 1, 6144, 128
    assert ta.tileattn_launch_shape(2, B, Hq, Hkv, S, S, D, 1)[1] == 256
    q, k, v = random_qkv(B, Hq, Hkv, S, S, D, dtype="bf16", seed=20)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    o, lse = _gpu_forward(q, k, v, True, scale)
    rng = np.random.default_rng(20)
    rows = np.unique(np.concatenate([rng.integers(0, B * Hq * S, 384),
                                     [h * S + i for h in range(Hq) for i in (0, 255, 256, S - 1)]]))
    o_rows = o.reshape(-1, D)[torch.as_tensor(rows, device="cuda")]
    l_rows = lse.reshape(-1)[torch.as_tensor(rows, device="cuda")]
    o_ref, lse_ref = oracle.attention_rows(q, k, v, scale, True, rows)
    _check(o_rows, l_rows, o_ref, lse_ref, "bf16", f"residue map, 8 waves ({len(rows)} rows)")


def test_gqa_equals_mha_with_repeated_kv_bitwise():
    # Both grids take 256-row workgroups (GQA: 4 heads x 64 positions each;
    # MHA: 256 positions of one head).  There every row visits key tiles
    # 0, 1, ... in order, and the tiles past its diagonal that a larger
    # workgroup adds contribute exact zeros, so the rows agree bit for bit.
    # (The key split divides each workgroup's tiles between its two wave
    # groups, at a point that depends on the workgroup's extent, so there the
    # two layouts agree only up to rounding.)
    q, k, v = random_qkv(1, 64, 16, 600, 600, 128, dtype="bf16", seed=15)
    assert ta.tileattn_launch_shape(2, 1, 64, 16, 600, 600, 128, 1)[1] == 256
    assert ta.tileattn_launch_shape(2, 1, 64, 64, 600, 600, 128, 1)[1] == 256
    o1, l1 = _gpu_forward(q, k, v, True, 0.0883883461356163)
    o2, l2 = _gpu_forward(q, k.repeat_interleave(4, 1).contiguous(),
                          v.repeat_interleave(4, 1).contiguous(), True, 0.0883883461356163)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_rows_sum_to_one_from_lse():
    q, k, v = random_qkv(1, 4, 2, 200, 180, 128, dtype="bf16", seed=16)
    scale = 0.0883883461356163
    _, lse = _gpu_forward(q, k, v, True, scale)
    s = torch.matmul(q.double(), k.double().repeat_interleave(2, 1).transpose(-1, -2).contiguous()) * scale
    vis = torch.ones(200, 180, dtype=torch.bool).tril()
    tot = (torch.exp(s - lse.cpu().double()[..., None]) * vis).sum(-1)
    assert (tot - 1).abs().max().item() < 2e-3


def test_deterministic_and_stream_ordered():
    q, k, v = (t.cuda() for t in random_qkv(1, 8, 2, 520, 520, 128, dtype="bf16", seed=17))
    o1, l1 = ta.forward(q, k, v, causal=True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o2, l2 = ta.forward(q, k, v, causal=True, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_empty_query_set_is_a_noop():
    q = torch.zeros(1, 4, 0, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 2, 5, 128, dtype=torch.bfloat16, device="cuda")
    o, lse = ta.forward(q, k, k, causal=True)
    assert o.shape == (1, 4, 0, 128) and lse.shape == (1, 4, 0)


# ---------------------------------------------------------------------------
# The workloads at full size.
# ---------------------------------------------------------------------------
def _edge_rows(w, n_extra, seed):
    """Flat row indices: first/last rows of heads, tile boundaries, plus random."""
    rows = set()
    for b in (0, w.B - 1):
        for h in (0, w.Hq // 2, w.Hq - 1):
            for i in (0, 1, 63, 64, 127, 128, w.Sq // 2, w.Sq - 2, w.Sq - 1):
                if 0 <= i < w.Sq:
                    rows.add((b * w.Hq + h) * w.Sq + i)
    rng = np.random.default_rng(seed)
    rows.update(rng.integers(0, w.B * w.Hq * w.Sq, size=n_extra).tolist())
    return np.array(sorted(rows), dtype=np.int64)


# Every row of O and lse against the full oracle, errors taken over all
# elements: the two small workloads, causal MHA at 4K, causal GQA at 8K
# (the headline) and the same shape in fp16.  The full oracle costs about
# 0.5 s (4K) and 2 s (8K) on the host's cores.
FULL_WORKLOADS = ["tiny_fp32", "mha_bf16", "causal_mha_bf16", "causal_gqa_bf16", "causal_gqa_fp16"]


@pytest.mark.parametrize("name", FULL_WORKLOADS)
def test_workload_full_oracle(name):
    w = WORKLOADS[name]
    _say(f"workload {name} (full oracle)")
    q, k, v = make_inputs(w)
    o, lse = _gpu_forward(q, k, v, w.causal, w.scale)
    o_ref, lse_ref = oracle.attention(q, k, v, w.scale, w.causal)
    _check(o, lse, o_ref, lse_ref, w.dtype, f"{name} (all {w.B * w.Hq * w.Sq} rows)")


def test_longctx_workload_sampled_rows():
    # 32K keys: the full oracle would cost minutes, so the 256 seeded rows of
    # the workload's own sample plus head and tile edges are compared, and
    # properties that hold for every row are checked on all of them.
    w = WORKLOADS["longctx_gqa_bf16"]
    _say("workload longctx_gqa_bf16 (sampled rows)")
    q, k, v, rows = make_inputs(w, with_sample=True)
    rows = np.union1d(rows, _edge_rows(w, 0, 0))
    o, lse = _gpu_forward(q, k, v, w.causal, w.scale)
    o_rows = o.reshape(-1, w.D)[torch.as_tensor(rows, device="cuda")]
    l_rows = lse.reshape(-1)[torch.as_tensor(rows, device="cuda")]
    o_ref, lse_ref = oracle.attention_rows(q, k, v, w.scale, w.causal, rows)
    _check(o_rows, l_rows, o_ref, lse_ref, w.dtype, f"longctx_gqa_bf16 ({len(rows)} rows)")
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    G = w.Hq // w.Hkv
    v0 = v[:, :, 0].to("cuda").repeat_interleave(G, dim=1)
    assert torch.equal(o[:, :, 0], v0)


def test_key_permutation_invariance():
    # Non-causal attention does not depend on the order of the keys: permuting
    # the rows of K and V together leaves O unchanged (up to the rounding of
    # the different summation order), and both launches match the oracle.
    B, Hq, Hkv, Sq, Sk, D = 1, 8, 2, 300, 517, 128
    scale = float(np.float32(1.0 / math.sqrt(D)))
    q, k, v = random_qkv(B, Hq, Hkv, Sq, Sk, D, dtype="bf16", seed=21)
    perm = torch.randperm(Sk, generator=torch.Generator().manual_seed(21))
    kp, vp = k[:, :, perm].contiguous(), v[:, :, perm].contiguous()
    o1, l1 = _gpu_forward(q, k, v, False, scale)
    o2, l2 = _gpu_forward(q, kp, vp, False, scale)
    o_ref, lse_ref = oracle.attention(q, k, v, scale, False)
    _check(o1, l1, o_ref, lse_ref, "bf16", "keys in order")
    _check(o2, l2, o_ref, lse_ref, "bf16", "keys permuted")
    d = (o1.double() - o2.double()).abs()
    assert d.max().item() <= 2e-2 and d.mean().item() <= 2e-3
    assert (l1.double() - l2.double()).abs().max().item() <= 1e-3


def test_forward_refuses_outputs_that_overlap_inputs():
    q, k, v = (t.cuda() for t in random_qkv(1, 2, 1, 64, 64, 64, dtype="bf16", seed=18))
    with pytest.raises(ValueError, match="must not overlap"):
        ta.forward(q, k, v, out=q)
    lse_in_k = k.view(torch.float32).reshape(-1)[: 2 * 64].view(1, 2, 64)
    with pytest.raises(ValueError, match="must not overlap"):
        ta.forward(q, k, v, lse=lse_in_k)


def test_million_keys_few_queries():
    # 2^20 + 37 keys: 16385 key tiles per workgroup, the 32-bit buffer
    # offsets of K and V up to 256 MiB, and a ragged last tile; 3 query rows
    # keep the oracle cheap.
    _parity(1, 2, 1, 3, (1 << 20) + 37, 128, False, "bf16", seed=19)


# Head packing: a workgroup holds the largest power of two (up to 8 on 256
# rows, 4 on 128) of the query heads sharing a KV head, each on a slice of
# positions: G = 16, 8 and 6 (2 heads), 3 (none); decode-like rows.
PACK_CASES = [
    # B, Hq, Hkv, Sq, Sk, D, causal, dtype
    (1, 16, 1, 300, 300, 128, True, "bf16"),    # key split, 4 heads x 32 positions
    (2, 64, 8, 600, 600, 128, True, "bf16"),    # 256 rows: 8 heads x 32 positions
    (2, 48, 8, 520, 700, 64, True, "fp16"),     # 256 rows: 2 heads x 128 positions
    (1, 24, 8, 100, 100, 128, False, "bf16"),   # G = 3: one head per workgroup
    (1, 32, 8, 1, 2000, 128, False, "bf16"),    # one row per head, 4 heads a workgroup
    (4, 32, 8, 3, 700, 64, True, "fp16"),       # three rows per head, causal
]


@pytest.mark.parametrize("case", PACK_CASES)
def test_head_packing(case):
    B, Hq, Hkv, Sq, Sk, D, causal, dtype = case
    _parity(B, Hq, Hkv, Sq, Sk, D, causal, dtype, seed=Hq + Sq + Sk)


# Grids on either side of the workgroup-size switch (at most 128 workgroups
# of 256 rows on a 256-CU device take 128-row workgroups instead).
SWITCH_CASES = [
    # B, Hq, Hkv, Sq, Sk, D, causal, dtype
    (1, 64, 8, 512, 300, 128, True, "bf16"),    # 128 -> 128-row workgroups
    (1, 43, 43, 700, 700, 64, False, "bf16"),   # 129 -> 256-row
    (2, 32, 16, 260, 512, 128, False, "fp16"),  # 128 -> 128-row
    (5, 13, 13, 500, 257, 64, True, "fp16"),    # 130 -> 256-row
]


@pytest.mark.parametrize("case", SWITCH_CASES)
def test_workgroup_size_switch(case):
    B, Hq, Hkv, Sq, Sk, D, causal, dtype = case
    G, p = Hq // Hkv, 1
    while 2 * p <= 8 and G % (2 * p) == 0:
        p *= 2
    wg256 = B * (Hq // p) * -(-Sq // (256 // p))   # 256-row workgroups, p heads packed
    expect = 128 if 2 * wg256 <= torch.cuda.get_device_properties(0).multi_processor_count else 256
    assert ta.tileattn_launch_shape(2, B, Hq, Hkv, Sq, Sk, D, int(causal))[1] == expect
    _parity(B, Hq, Hkv, Sq, Sk, D, causal, dtype, seed=wg256 + Sq)
