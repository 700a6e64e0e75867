"""Brute-force attention by the definition, in pure Python (tiny inputs only).

Test infrastructure only (see the package docstring).  Independent of the
numpy oracle: explicit loops, ``math.exp`` and ``math.fsum`` (exactly rounded
sums), no arrays.  It serves as a second, differently written statement of
the same definition -- per query row, the stable softmax of the scaled
dot products over the visible keys ("Guia Prático de Programação de GPU com
Tiles", Passo a Passo, steps 4 and 6) -- so a slip in the vectorised
oracle's indexing, masking or head mapping shows up as a disagreement on
shapes with S <= 16.
"""

from __future__ import annotations

import math


def _nested(x):
    """Return x as nested Python lists of floats (accepts numpy / torch / lists)."""
    if hasattr(x, "detach"):
        import torch

        x = x.detach().to("cpu", torch.float64).tolist()
    elif hasattr(x, "tolist"):
        x = x.astype("float64").tolist()
    return x


def attention_bruteforce(q, k, v, scale: float, causal: bool):
    """Return (o, lse) as nested lists: o[b][h][i][d], lse[b][h][i]."""
    q, k, v = _nested(q), _nested(k), _nested(v)
    B, Hq = len(q), len(q[0])
    Hkv = len(k[0])
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    group = Hq // Hkv
    scale = float(scale)
    o, lse = [], []
    for b in range(B):
        ob, lb = [], []
        for h in range(Hq):
            kv_head = h // group
            keys, vals = k[b][kv_head], v[b][kv_head]
            Sk, D = len(keys), len(vals[0])
            oh, lh = [], []
            for i, qrow in enumerate(q[b][h]):
                visible = [j for j in range(Sk) if (not causal) or j <= i]
                scores = [scale * math.fsum(qrow[d] * keys[j][d] for d in range(D))
                          for j in visible]
                top = max(scores)
                weights = [math.exp(s - top) for s in scores]
                total = math.fsum(weights)
                orow = [math.fsum(weights[n] * vals[j][d] for n, j in enumerate(visible)) / total
                        for d in range(D)]
                oh.append(orow)
                lh.append(top + math.log(total))
            ob.append(oh)
            lb.append(lh)
        o.append(ob)
        lse.append(lb)
    return o, lse
