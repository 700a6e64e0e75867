"""Race check of the attention kernels' LDS double buffering (needs an MI355X).

``libtileattn_synccheck.so`` is the same attention source built with
TILEATTN_SYNC_CHECK: extra workgroup barriers close the staging step and both
phases of every tile iteration.  That changes only the order in which the
waves reach LDS, never the arithmetic, so its outputs must equal the product
library's bit for bit.  Any difference would mean that some LDS read races the
write it depends on, which a tolerance check against the oracle could miss.
Both libraries are called through their C ABI (``tileattn_fwd_ext``, and
``tileattn_fwd_ws`` for the chunked key split and its merge kernel) on the
same device buffers.
"""

import ctypes
import os
import sys

import pytest
import torch

import tiled_attention_tileattn_amd as ta
from tiled_attention_tileattn_amd.build import SYNC_CHECK_OUT
from tiled_attention_tileattn_amd.inputs import alibi_slopes, random_block_mask, random_qkv

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _ext(lib):
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    fn = lib.tileattn_fwd_ext
    fn.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, vp, i, i, vp]
    fn.restype = i
    return fn


@pytest.fixture(scope="module")
def libs():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    if not os.path.exists(SYNC_CHECK_OUT):
        raise RuntimeError(f"{SYNC_CHECK_OUT} is missing: run __graft_entry__.build() first")
    torch.cuda.set_device(0)
    return _ext(ta.load_library()), _ext(ctypes.CDLL(SYNC_CHECK_OUT))


CASES = [
    # B, Hq, Hkv, Sq, Sk, D, causal, ALiBi, block mask, fp16
    (1, 4, 2, 300, 300, 128, True, False, False, False),
    (1, 8, 2, 1000, 1000, 128, True, False, False, False),
    (2, 4, 4, 513, 700, 64, False, False, False, False),
    (1, 4, 1, 777, 777, 128, True, True, False, False),
    (1, 4, 2, 640, 640, 128, True, False, True, False),
    (1, 2, 2, 520, 520, 128, False, True, True, True),
    (1, 4, 2, 2048, 2048, 128, True, False, False, True),
    # Grids over half a chip of 256-row workgroups: the 8-wave ping-pong
    # kernel (the small plain shapes above run 128-row workgroups).
    (2, 64, 8, 300, 300, 128, True, False, False, False),
    (3, 64, 16, 520, 400, 64, False, False, False, True),
]


@pytest.mark.parametrize("case", CASES)
def test_barrier_build_is_bit_identical(libs, case):
    B, Hq, Hkv, Sq, Sk, D, causal, alibi, masked, f16 = case
    bm = 256 if (alibi or masked) else ta.tileattn_launch_shape(2, B, Hq, Hkv, Sq, Sk, D, int(causal))[1]
    _say(f"sync check B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Sk={Sk} D={D} causal={causal} "
         f"alibi={alibi} mask={masked} fp16={f16} rows/workgroup={bm}")
    q, k, v = (t.cuda() for t in random_qkv(B, Hq, Hkv, Sq, Sk, D, dtype="fp16" if f16 else "bf16",
                                           seed=Sq + Sk + D))
    slopes = alibi_slopes(Hq).cuda() if alibi else None
    mask = random_block_mask(Hq, Sq, Sk, seed=Sq, p_visible=0.6).cuda() if masked else None
    scale = 1.0 / D ** 0.5
    outs = []
    for fn in libs:
        o = torch.empty_like(q)
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device="cuda")
        rc = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                B, Hq, Hkv, Sq, Sk, D, scale, int(causal),
                None if slopes is None else slopes.data_ptr(),
                None if mask is None else mask.data_ptr(), Hq if masked else 1, int(f16),
                torch.cuda.current_stream().cuda_stream)
        assert rc == 0, ta.tileattn_strerror(rc)
        outs.append((o, lse))
    torch.cuda.synchronize()
    (o1, l1), (o2, l2) = outs
    assert torch.equal(o1, o2), "O differs between the product and the barrier build"
    assert torch.equal(l1, l2), "lse differs between the product and the barrier build"


CHUNK_CASES = [
    # B, Hq, Hkv, Sq, Sk, D, causal, fp16: shapes the chunked key split takes
    (1, 4, 1, 4000, 4000, 128, True, False),
    (1, 32, 8, 3, 9000, 64, False, True),
]


@pytest.mark.parametrize("case", CHUNK_CASES)
def test_chunked_barrier_build_is_bit_identical(libs, case):
    # The chunked key split (tileattn_fwd_ws: partial states through global
    # memory, then the merge kernel) in both builds.
    B, Hq, Hkv, Sq, Sk, D, causal, f16 = case
    need = ta.tileattn_fwd_workspace_size(B, Hq, Hkv, Sq, Sk, D, causal)
    assert need > 0
    _say(f"sync check, chunked: B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Sk={Sk} D={D} causal={causal} fp16={f16}")
    q, k, v = (t.cuda() for t in random_qkv(B, Hq, Hkv, Sq, Sk, D, dtype="fp16" if f16 else "bf16",
                                           seed=Sq + Sk))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    outs = []
    for lib in (ta.load_library(), ctypes.CDLL(SYNC_CHECK_OUT)):
        fn = lib.tileattn_fwd_ws
        fn.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, i, vp, ctypes.c_size_t, vp]
        fn.restype = i
        o = torch.empty_like(q)
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device="cuda")
        rc = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                B, Hq, Hkv, Sq, Sk, D, 1.0 / D ** 0.5, int(causal), None, int(f16), ws.data_ptr(), need,
                torch.cuda.current_stream().cuda_stream)
        assert rc == 0, ta.tileattn_strerror(rc)
        torch.cuda.synchronize()
        outs.append((o, lse))
    (o1, l1), (o2, l2) = outs
    assert torch.equal(o1, o2), "O differs between the product and the barrier build"
    assert torch.equal(l1, l2), "lse differs between the product and the barrier build"
