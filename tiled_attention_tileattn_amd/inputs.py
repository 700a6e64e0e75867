"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module draws random numbers and nothing else: it holds none of the
attention arithmetic, so both the GPU path and the CPU oracle can be fed from
it without sharing any of the method's code.

Recipe (the same for every workload):
    g = torch.Generator("cpu").manual_seed(seed)
    q = randn([B, Hq,  Sq, D]) * q_std      (float32, drawn first)
    k = randn([B, Hkv, Sk, D]) * k_std      (drawn second)
    v = randn([B, Hkv, Sk, D]) * v_std      (drawn third)
    then cast to the workload dtype (bfloat16 and float16 casts round to nearest even).
A row sample for the long-context workload continues the same generator
after v: randperm(B * Hq * Sq)[:n], flat indices into [B, Hq, Sq].
"""

from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Sk: int
    D: int
    causal: bool
    dtype: str          # "bf16", "fp16" or "fp32"
    seed: int
    q_std: float = 1.0
    k_std: float = 1.0
    v_std: float = 1.0
    sample_rows: int = 0   # >0: the oracle is checked on this many sampled rows

    @property
    def scale(self) -> float:
        """1/sqrt(D), as the float32 value the GPU receives."""
        return float(np.float32(1.0 / math.sqrt(self.D)))

    @property
    def torch_dtype(self):
        return {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[self.dtype]

    def flop(self) -> float:
        """Counted attention FLOP: 4*B*Hq*Sq*Sk*D, halved when causal."""
        f = 4.0 * self.B * self.Hq * self.Sq * self.Sk * self.D
        return f / 2 if self.causal else f

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads: a tiny fp32 case, plain multi-head bf16, causal multi-head,
# causal grouped-query at 8K (the headline), and long-context grouped-query at 32K;
# plus the headline shape in fp16, the dtype of the first page's own kernel.
WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 1, 1, 1, 128, 128, 64, False, "fp32", 0),
    "mha_bf16": Workload("mha_bf16", 4, 8, 8, 1024, 1024, 64, False, "bf16", 1),
    "causal_mha_bf16": Workload("causal_mha_bf16", 2, 16, 16, 4096, 4096, 128, True, "bf16", 2),
    "causal_gqa_bf16": Workload("causal_gqa_bf16", 1, 32, 8, 8192, 8192, 128, True, "bf16", 3),
    "longctx_gqa_bf16": Workload("longctx_gqa_bf16", 1, 64, 8, 32768, 32768, 128, True, "bf16", 4,
                                 q_std=0.5, k_std=0.5, sample_rows=256),
    "causal_gqa_fp16": Workload("causal_gqa_fp16", 1, 32, 8, 8192, 8192, 128, True, "fp16", 5),
}

HEADLINE = "causal_gqa_bf16"


def make_inputs(w: Workload, device: str | torch.device = "cpu", with_sample: bool = False):
    """Draw (q, k, v[, sample]) for workload ``w`` following the module recipe.

    The draw always happens on the CPU generator, so the values do not depend
    on ``device``; the tensors are then moved there.
    """
    g = torch.Generator("cpu").manual_seed(w.seed)
    q = torch.randn((w.B, w.Hq, w.Sq, w.D), generator=g, dtype=torch.float32)
    k = torch.randn((w.B, w.Hkv, w.Sk, w.D), generator=g, dtype=torch.float32)
    v = torch.randn((w.B, w.Hkv, w.Sk, w.D), generator=g, dtype=torch.float32)
    if w.q_std != 1.0:
        q.mul_(w.q_std)
    if w.k_std != 1.0:
        k.mul_(w.k_std)
    if w.v_std != 1.0:
        v.mul_(w.v_std)
    dt = w.torch_dtype
    q, k, v = (t.to(dt).contiguous().to(device) for t in (q, k, v))
    if not with_sample:
        return q, k, v
    n = w.sample_rows if w.sample_rows > 0 else 256
    total = w.B * w.Hq * w.Sq
    sample = torch.randperm(total, generator=g)[: min(n, total)].numpy()
    return q, k, v, sample


def random_qkv(B, Hq, Hkv, Sq, Sk, D, dtype="bf16", seed=0, q_std=1.0, k_std=1.0, v_std=1.0,
               device="cpu"):
    """Ad-hoc shapes for tests, same recipe as ``make_inputs``."""
    w = Workload("adhoc", B, Hq, Hkv, Sq, Sk, D, False, dtype, seed, q_std, k_std, v_std)
    return make_inputs(w, device=device)


def alibi_slopes(Hq: int, base: float = 8.0) -> torch.Tensor:
    """ALiBi slopes, the geometric sequence 2^(-base*h/Hq), h = 1..Hq, as float32.

    This is the slope recipe of "Train Short, Test Long: Attention with
    Linear Biases"; the kernel takes any slopes, these are the inputs used.
    """
    return torch.tensor([2.0 ** (-base * (h + 1) / Hq) for h in range(Hq)], dtype=torch.float32)


def random_block_mask(mask_heads: int, Sq: int, Sk: int, seed: int, p_visible: float = 0.5,
                      block: int = 64) -> torch.Tensor:
    """Seeded uint8 block map [mask_heads, ceil(Sq/block), ceil(Sk/block)].

    Each block is visible with probability p_visible (numpy default_rng);
    key block 0 is always visible, so no query row is left without a key.
    """
    rng = np.random.default_rng(seed)
    nq, nk = -(-Sq // block), -(-Sk // block)
    m = (rng.random((mask_heads, nq, nk)) < p_visible).astype(np.uint8)
    m[:, :, 0] = 1
    return torch.from_numpy(m).contiguous()


def window_block_mask(Sq: int, Sk: int, window_blocks: int, block: int = 64) -> torch.Tensor:
    """Local-window block map [1, nq, nk]: query block qb sees key blocks
    qb - window_blocks + 1 .. qb, plus key block 0 (a "sink" every row keeps)."""
    nq, nk = -(-Sq // block), -(-Sk // block)
    m = np.zeros((1, nq, nk), dtype=np.uint8)
    for qb in range(nq):
        m[0, qb, max(0, qb - window_blocks + 1): min(nk, qb + 1)] = 1
        m[0, qb, 0] = 1
    return torch.from_numpy(m).contiguous()


# ---- matrix product inputs ---------------------------------------------------
# name -> (M, N, K, seed): the square bf16 product timed next to the attention.
MATMUL_WORKLOADS = {
    "matmul_bf16_8k": (8192, 8192, 8192, 11),
}


def random_matrices(M: int, N: int, K: int, seed: int, integer: bool = False,
                    device: str | torch.device = "cpu"):
    """Seeded bf16 A [M, K] and B [K, N] for the matrix product.

    Draws from torch.Generator('cpu').manual_seed(seed), A first and then B:
    N(0, 1) float32 values cast to bf16 (round to nearest even), or with
    ``integer`` integers uniform in [-4, 4] (exact in bf16; every product and
    every partial sum of up to 2^19 of them is then exact in fp32).
    """
    g = torch.Generator("cpu").manual_seed(seed)
    if integer:
        a = torch.randint(-4, 5, (M, K), generator=g, dtype=torch.int32).to(torch.float32)
        b = torch.randint(-4, 5, (K, N), generator=g, dtype=torch.int32).to(torch.float32)
    else:
        a = torch.randn((M, K), generator=g, dtype=torch.float32)
        b = torch.randn((K, N), generator=g, dtype=torch.float32)
    return a.to(torch.bfloat16).to(device).contiguous(), b.to(torch.bfloat16).to(device).contiguous()


# ---- row softmax and fused GELU inputs -----------------------------------------
# name -> (kind, dtype, shape, seed): the memory-bound kernels timed next to
# the attention (an 8K-column softmax over 64K rows; 2^28-element GELU).
ROWWISE_WORKLOADS = {
    "softmax_bf16_64k_x_8k": ("softmax", "bf16", (65536, 8192), 21),
    "softmax_fp32_64k_x_8k": ("softmax", "fp32", (65536, 8192), 22),
    "gelu_fp32_256m": ("gelu", "fp32", (1 << 28,), 23),
    "gelu_bf16_256m": ("gelu", "bf16", (1 << 28,), 24),
}


DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


def _randn(shape, gen, device, scale, dtype):
    t = torch.randn(shape, generator=gen, dtype=torch.float32, device=device)
    if scale != 1.0:
        t = t * scale
    return t.to(DTYPES[dtype]).contiguous()


def random_rows(n_rows: int, n_cols: int, seed: int, dtype: str = "fp32", scale: float = 1.0,
                device: str | torch.device = "cpu") -> torch.Tensor:
    """Seeded [n_rows, n_cols] softmax input: N(0, scale^2) float32 draws from a
    torch generator on ``device`` seeded with ``seed``, cast to ``dtype``
    (bf16: round to nearest even).  CPU and GPU draws differ; each is
    reproducible."""
    g = torch.Generator(device).manual_seed(seed)
    return _randn((n_rows, n_cols), g, device, scale, dtype)


def random_gelu_inputs(n: int, seed: int, dtype: str = "fp32", scale: float = 1.0,
                       device: str | torch.device = "cpu"):
    """Seeded x, w, b of n elements for the fused GELU: N(0, scale^2) draws in
    that order from one generator on ``device``, cast to ``dtype``."""
    g = torch.Generator(device).manual_seed(seed)
    return tuple(_randn((n,), g, device, scale, dtype) for _ in range(3))
