"""Exact attention forward in float64 with an explicit full softmax.

Test infrastructure only (see the package docstring).  Slow on purpose: the
whole ``Sq x Sk`` score block of a head is formed (in row blocks to bound
memory), the row maximum is subtracted, the exponentials are summed and
divided -- the textbook stable softmax of "Guia Prático de Programação de GPU
com Tiles" (Passo a Passo, step 4 "Softmax por Linha — Reduções em Tile") --
and the probabilities weight the value rows (step 6 "Flash Attention —
Softmax Online", whose running recurrence equals this full softmax).

Shapes (contiguous row-major, as handed to the GPU library):
    q   [B, Hq,  Sq, D]
    k,v [B, Hkv, Sk, D]
    o   [B, Hq,  Sq, D]   (float64 here)
    lse [B, Hq,  Sq]      (float64 here)

Readings of points the pages leave open:
    * GQA: query head h reads key/value head h // (Hq // Hkv).
    * causal: key j is visible to query i iff j <= i (top-left aligned).
    * lse = m_i + ln(sum_j exp(s_ij - m_i)) over the visible keys, with s the
      scaled scores (natural logarithm).
    * inputs are used exactly as given (bf16 values upcast to float64, the
      scale as the float32 number the GPU receives, upcast).
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_ROW_BLOCK = 1024


def _as_f64(x) -> np.ndarray:
    """Upcast a numpy array or a (CPU) torch tensor to a float64 numpy array."""
    if hasattr(x, "detach"):  # torch tensor; bf16 has no numpy dtype
        import torch

        x = x.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be 4-D [B, H, S, D]")
    B, Hq, Sq, D = q.shape
    Bk, Hkv, Sk, Dk = k.shape
    if v.shape != k.shape or Bk != B or Dk != D:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    if Hkv < 1 or Hq % Hkv != 0:
        raise ValueError(f"Hq={Hq} must be a multiple of Hkv={Hkv}")
    if Sk < 1:
        raise ValueError("softmax over an empty key set is undefined (Sk >= 1)")
    return B, Hq, Hkv, Sq, Sk, D


def _head_rows(qh: np.ndarray, kh: np.ndarray, vh: np.ndarray, rows: np.ndarray,
               scale: float, causal: bool):
    """Attention of the query rows ``rows`` of one head against one K/V head.

    qh: [n, D] the selected query rows, rows: [n] their positions i.
    Returns (o [n, D], lse [n]) in float64.
    """
    Sk = kh.shape[0]
    s = (qh @ kh.T) * scale                                   # [n, Sk] scaled scores
    if causal:
        key_idx = np.arange(Sk)[None, :]
        s = np.where(key_idx <= rows[:, None], s, -np.inf)    # j <= i visible
    m = s.max(axis=1, keepdims=True)                          # row max (finite: key 0 visible)
    e = np.exp(s - m)                                         # masked -> exp(-inf) = 0
    denom = e.sum(axis=1, keepdims=True)
    p = e / denom                                             # explicit full softmax
    o = p @ vh
    lse = m[:, 0] + np.log(denom[:, 0])
    return o, lse


def _workers(n_tasks: int) -> int:
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    return max(1, min(cores, n_tasks))


def _run_pool(fn, tasks, threads: int | None):
    """Run fn over tasks on a thread pool, one BLAS thread per worker."""
    n = threads if threads is not None else _workers(len(tasks))
    if n <= 1 or len(tasks) <= 1:
        return [fn(t) for t in tasks]
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            with ThreadPoolExecutor(max_workers=n) as ex:
                return list(ex.map(fn, tasks))
    with ThreadPoolExecutor(max_workers=n) as ex:  # pragma: no cover
        return list(ex.map(fn, tasks))


def attention(q, k, v, scale: float, causal: bool, threads: int | None = None):
    """Full attention forward, every row of every head, in float64.

    Returns (o [B, Hq, Sq, D], lse [B, Hq, Sq]) as float64 numpy arrays.
    ``threads`` = worker threads over heads (default: all usable cores).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, Hq, Hkv, Sq, Sk, D = _check_shapes(q, k, v)
    G = Hq // Hkv
    scale = float(scale)
    o = np.empty((B, Hq, Sq, D), dtype=np.float64)
    lse = np.empty((B, Hq, Sq), dtype=np.float64)

    def one_head(bh):
        b, h = bh
        hk = h // G
        for r0 in range(0, Sq, _ROW_BLOCK):
            rows = np.arange(r0, min(Sq, r0 + _ROW_BLOCK))
            ob, lb = _head_rows(q[b, h, rows], k[b, hk], v[b, hk], rows, scale, causal)
            o[b, h, rows] = ob
            lse[b, h, rows] = lb

    tasks = [(b, h) for b in range(B) for h in range(Hq)]
    _run_pool(one_head, tasks, threads)
    return o, lse


def attention_rows(q, k, v, scale: float, causal: bool, flat_rows,
                   threads: int | None = None):
    """Attention for a sample of query rows given as flat indices into [B, Hq, Sq].

    Used where the full oracle is too slow (long sequences): each sampled row is
    computed exactly as in ``attention``.  Returns (o [n, D], lse [n]) float64,
    in the order of ``flat_rows``.
    """
    B, Hq, Sq, D = q.shape
    Hkv = k.shape[1]
    flat_rows = np.asarray(flat_rows, dtype=np.int64)
    b_idx = flat_rows // (Hq * Sq)
    h_idx = (flat_rows // Sq) % Hq
    i_idx = flat_rows % Sq
    G = Hq // Hkv
    o = np.empty((len(flat_rows), D), dtype=np.float64)
    lse = np.empty((len(flat_rows),), dtype=np.float64)

    # Group the sampled rows by (b, h) so each K/V head is upcast once per group.
    groups = {}
    for n, (b, h) in enumerate(zip(b_idx.tolist(), h_idx.tolist())):
        groups.setdefault((b, h), []).append(n)

    def one_group(item):
        (b, h), ns = item
        hk = h // G
        qh = _as_f64(q[b, h][i_idx[ns]])
        kh = _as_f64(k[b, hk])
        vh = _as_f64(v[b, hk])
        _check_shapes(qh[None, None], kh[None, None], vh[None, None])
        ob, lb = _head_rows(qh, kh, vh, i_idx[ns], float(scale), causal)
        o[ns] = ob
        lse[ns] = lb

    _run_pool(one_group, list(groups.items()), threads)
    return o, lse
