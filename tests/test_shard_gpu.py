"""What one GPU can show of a multi-GPU split (needs an MI355X).

* Head sharding: each of 8 GPUs would run the kernel on one KV head and its
  query heads, with no communication.  At the 32K shape (B=1, Hq=64, Hkv=8)
  a shard still fills the chip with 256-row workgroups, runs the same kernel
  instance as the full launch, and must give its rows bit for bit.  At the
  8K headline shape (B=1, Hq=32, Hkv=8) a shard's grid is small enough for
  the key split (128-row workgroups, each key range in two halves merged at
  the end), so it rounds differently; there its rows must agree with the full
  launch's within the plain path's bf16 tolerances.
* Key sharding (non-causal): each shard computes (O_g, lse_g) over its keys;
  the exact result is lse = ln sum_g exp(lse_g), O = sum_g exp(lse_g - lse) O_g.
  The merge is done on the host here and compared with the oracle over all
  keys, with the plain path's bf16 tolerances.
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


def _head_shards(name):
    w = WORKLOADS[name]
    q, k, v = make_inputs(w, device="cuda")
    o, lse = ta.forward(q, k, v, causal=w.causal, scale=w.scale)
    G = w.Hq // w.Hkv
    for g in range(w.Hkv):
        hs = slice(g * G, (g + 1) * G)
        o_s, lse_s = ta.forward(q[:, hs].contiguous(), k[:, g:g + 1].contiguous(),
                                v[:, g:g + 1].contiguous(), causal=w.causal, scale=w.scale)
        torch.cuda.synchronize()
        yield g, o_s, lse_s, o[:, hs], lse[:, hs]


def test_head_shards_of_causal_gqa_32k_match_the_full_launch_bitwise():
    _say("head shards of longctx_gqa_bf16")
    for g, o_s, lse_s, o_f, lse_f in _head_shards("longctx_gqa_bf16"):
        assert torch.equal(o_s, o_f), f"shard {g}: O differs"
        assert torch.equal(lse_s, lse_f), f"shard {g}: lse differs"


def test_head_shards_of_causal_gqa_8k_match_the_full_launch():
    _say("head shards of causal_gqa_bf16")
    for g, o_s, lse_s, o_f, lse_f in _head_shards("causal_gqa_bf16"):
        d = (o_s.float() - o_f.float()).abs()
        dl = (lse_s - lse_f).abs().max().item()
        _say(f"  shard {g}: max|dO|={d.max().item():.3e} mean|dO|={d.mean().item():.3e} max|dlse|={dl:.3e}")
        assert d.max().item() <= 2e-2 and d.mean().item() <= 2e-3 and dl <= 1e-4, f"shard {g}"


@pytest.mark.parametrize("split", [[700], [64, 1000], [333, 334]])
def test_key_shards_merge_to_the_full_result(split):
    B, Hq, Hkv, Sq, Sk, D = 1, 8, 2, 600, 1500, 128
    _say(f"key shards at {split} of Sk={Sk}")
    q, k, v = random_qkv(B, Hq, Hkv, Sq, Sk, D, dtype="bf16", seed=70 + len(split))
    scale = float(np.float32(1.0 / math.sqrt(D)))
    qd = q.cuda()
    bounds = [0] + list(split) + [Sk]
    parts = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        ks = k[:, :, a:b].contiguous().cuda()
        vs = v[:, :, a:b].contiguous().cuda()
        parts.append(ta.forward(qd, ks, vs, causal=False, scale=scale))
    torch.cuda.synchronize()
    lses = torch.stack([p[1].double() for p in parts])                 # [n, B, Hq, Sq]
    lse = torch.logsumexp(lses, dim=0)
    o = sum(torch.exp(l - lse)[..., None] * p[0].double() for l, p in zip(lses, parts))
    o_ref, lse_ref = oracle.attention(q, k, v, scale, False)
    err = np.abs(o.cpu().numpy() - o_ref)
    lerr = np.abs(lse.cpu().numpy() - lse_ref)
    _say(f"  max|dO|={err.max():.3e} mean|dO|={err.mean():.3e} max|dlse|={lerr.max():.3e}")
    assert err.max() <= 2e-2 and err.mean() <= 2e-3 and lerr.max() <= 1e-3
