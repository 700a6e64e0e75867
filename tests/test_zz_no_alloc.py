"""The allocation-free entry point (``tileattn_fwd_noalloc``) against the
workspace entry point (``tileattn_fwd_ws``) it is a variant of (needs an
MI355X).

Both run the same kernels on the same inputs, the first with the library's
static device workspace, the second with a torch allocation, so their
results must be bitwise equal.  Two calls in a row on the shared static
array, the second on a smaller problem, check that nothing the first call
left in it reaches the second's results; a problem the library runs without
chunks goes through the same entry point unchanged.
"""

import math
import sys

import numpy as np
import pytest
import torch

import tiled_attention_tileattn_amd as ta
from tiled_attention_tileattn_amd.inputs import alibi_slopes, random_qkv

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


def _both(B, Hq, Hkv, Sq, Sk, D, causal, dtype, seed, slopes=None):
    _say(f"no-alloc vs workspace entry: B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Sk={Sk} D={D} "
         f"causal={causal} {dtype}")
    q, k, v = (t.cuda() for t in random_qkv(B, Hq, Hkv, Sq, Sk, D, dtype=dtype, seed=seed))
    scale = float(np.float32(1.0 / math.sqrt(D)))
    is_f16 = int(dtype == "fp16")
    stream = torch.cuda.current_stream().cuda_stream
    outs = []
    for static in (True, False):
        o = torch.full_like(q, float("nan"))
        lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device="cuda")
        args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                B, Hq, Hkv, Sq, Sk, D, scale, causal, None if slopes is None else slopes.data_ptr(), is_f16)
        if static:
            rc = ta.tileattn_fwd_noalloc(*args, stream)
        else:
            n = ta.tileattn_fwd_workspace_size(B, Hq, Hkv, Sq, Sk, D, causal)
            ws = torch.empty(max(n, 16), dtype=torch.uint8, device="cuda")
            rc = ta.tileattn_fwd_ws(*args, ws.data_ptr(), n, stream)
        assert rc == 0, ta.tileattn_strerror(rc)
        torch.cuda.synchronize()
        outs.append((o, lse))
    (o1, l1), (o2, l2) = outs
    assert torch.isfinite(o1.float()).all() and torch.isfinite(l1).all()
    assert torch.equal(o1, o2), "O differs"
    assert torch.equal(l1, l2), "lse differs"


def test_noalloc_matches_workspace_entry_two_calls_in_a_row():
    # One KV head's share of the causal GQA 8K workload: the largest split
    # here (34 MB of partial states), then a smaller one on the same array.
    assert ta.tileattn_fwd_workspace_size(1, 4, 1, 8192, 8192, 128, True) > \
        ta.tileattn_fwd_workspace_size(1, 2, 1, 200, 3390, 128, False) > 0
    _both(1, 4, 1, 8192, 8192, 128, True, "bf16", seed=3)
    _both(1, 2, 1, 200, 3390, 128, False, "bf16", seed=4)


def test_noalloc_with_linear_bias():
    _both(1, 8, 2, 2, 12000, 64, False, "bf16", seed=7, slopes=alibi_slopes(8).cuda())


def test_noalloc_fp16_decode_and_unsplit_problem():
    _both(1, 32, 8, 1, 32768, 128, False, "fp16", seed=5)
    assert ta.tileattn_fwd_workspace_size(2, 16, 16, 512, 512, 64, True) == 0
    _both(2, 16, 16, 512, 512, 64, True, "bf16", seed=6)
