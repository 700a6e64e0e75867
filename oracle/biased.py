"""Exact attention forward with an ALiBi bias and a block-sparse mask, float64.

Test infrastructure only (see the package docstring).  The first page, "Guia
Prático de Programação de GPU com Tiles: de Kernels cuTile e Triton ao Flash
Attention", names ALiBi and block-sparse masking (FAQ, on how the tutorial
kernel compares with the official flash-attention library) as features the
library adds over its tutorial kernel, without defining them.  The readings
here are the plainest ones:

    * ALiBi (Press, Smith and Lewis, "Train Short, Test Long: Attention with
      Linear Biases"): a per-query-head slope m_h adds a bias linear in the
      query-key distance to the scaled score,
          s_ij = scale * <q_i, k_j> + b_ij,
          b_ij = -m_h * (i - j)      (causal; only j <= i is visible)
          b_ij = -m_h * |i - j|      (non-causal).
    * block-sparse: a byte map over blocks of ``block`` x ``block`` (query
      rows x keys), ``mask[hm, i // block, j // block] != 0`` makes the block
      visible; hm = h when the map has one plane per query head, else 0.  It
      is combined with the causal rule (both must allow a key).
    * a row with no visible key (possible only with a block mask) has no
      softmax; its output is o = 0 and lse = -inf.

Everything else is the plain definition of the full softmax as in
``full_softmax``: scores of all visible keys, minus the row max,
exponentiated, normalised, weighting the value rows; lse = m + ln(sum).
"""

from __future__ import annotations

import numpy as np

from .full_softmax import _as_f64, _check_shapes, _run_pool

_ROW_BLOCK = 1024


def _visible(rows: np.ndarray, Sk: int, causal: bool, mask_plane, block: int) -> np.ndarray:
    """Boolean [n, Sk]: key j visible to query row rows[n]."""
    keys = np.arange(Sk)[None, :]
    vis = np.ones((len(rows), Sk), dtype=bool)
    if causal:
        vis &= keys <= rows[:, None]
    if mask_plane is not None:
        vis &= mask_plane[rows[:, None] // block, keys // block] != 0
    return vis


def _rows(qh, kh, vh, rows, scale, causal, slope, mask_plane, block):
    Sk = kh.shape[0]
    s = (qh @ kh.T) * scale
    if slope is not None:
        dist = rows[:, None] - np.arange(Sk)[None, :]            # i - j
        s = s - slope * (dist if causal else np.abs(dist))
    vis = _visible(rows, Sk, causal, mask_plane, block)
    s = np.where(vis, s, -np.inf)
    o = np.zeros((len(rows), vh.shape[1]), dtype=np.float64)
    lse = np.full(len(rows), -np.inf, dtype=np.float64)
    live = vis.any(axis=1)                                        # rows with a visible key
    if live.any():
        sl = s[live]
        m = sl.max(axis=1, keepdims=True)
        e = np.exp(sl - m)
        denom = e.sum(axis=1, keepdims=True)
        o[live] = (e / denom) @ vh
        lse[live] = m[:, 0] + np.log(denom[:, 0])
    return o, lse


def attention_ext(q, k, v, scale: float, causal: bool, alibi_slopes=None, block_mask=None,
                  block: int = 64, threads: int | None = None):
    """Attention forward with optional ALiBi slopes [Hq] and block mask.

    block_mask: array-like [Hm, ceil(Sq/block), ceil(Sk/block)] with Hm = 1
    (shared by all heads) or Hq; nonzero = visible.
    Returns (o [B, Hq, Sq, D], lse [B, Hq, Sq]) float64.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, Hq, Hkv, Sq, Sk, D = _check_shapes(q, k, v)
    G = Hq // Hkv
    scale = float(scale)
    slopes = None if alibi_slopes is None else _as_f64(alibi_slopes).reshape(-1)
    if slopes is not None and slopes.shape[0] != Hq:
        raise ValueError("alibi_slopes must have Hq entries")
    bm = None
    if block_mask is not None:
        bm = np.asarray(block_mask.cpu() if hasattr(block_mask, "cpu") else block_mask)
        nq, nk = -(-Sq // block), -(-Sk // block)
        if bm.ndim != 3 or bm.shape[0] not in (1, Hq) or bm.shape[1:] != (nq, nk):
            raise ValueError(f"block_mask must be [1 or Hq, {nq}, {nk}], got {bm.shape}")
    o = np.empty((B, Hq, Sq, D), dtype=np.float64)
    lse = np.empty((B, Hq, Sq), dtype=np.float64)

    def one_head(bh):
        b, h = bh
        hk = h // G
        slope = None if slopes is None else slopes[h]
        plane = None if bm is None else bm[h if bm.shape[0] == Hq else 0]
        for r0 in range(0, Sq, _ROW_BLOCK):
            rows = np.arange(r0, min(Sq, r0 + _ROW_BLOCK))
            ob, lb = _rows(q[b, h, rows], k[b, hk], v[b, hk], rows, scale, causal, slope, plane, block)
            o[b, h, rows] = ob
            lse[b, h, rows] = lb

    _run_pool(one_head, [(b, h) for b in range(B) for h in range(Hq)], threads)
    return o, lse
