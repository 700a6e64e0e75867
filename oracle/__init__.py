"""CPU fp64 oracle for exact attention (test infrastructure only).

This package is the checker, not the product.  Only the test suite, the
``smoke()`` entry of ``__graft_entry__`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The GPU library never calls into it, and it
shares no code with the GPU library: no kernels, no helpers, no constants.

What it computes, and where that is defined:

* Attention is the softmax of the scaled query-key products over the keys a
  query may see, weighted over the value rows.  The tiled online-softmax
  kernel of "Guia Prático de Programação de GPU com Tiles: de Kernels cuTile
  e Triton ao Flash Attention" (Passo a Passo, step 6 "Flash Attention —
  Softmax Online") reaches this same result block by block; the running
  max / running sum recurrence there telescopes exactly to the full softmax,
  so the oracle writes out the full softmax directly (fp64, explicit
  max-subtraction as in step 4 "Softmax por Linha").
* Grouped-query attention (query heads sharing a key/value head) is named
  as a feature of the final kernel of "Como Domar o Blackwell Sem Enlouquecer
  com CUDA" (section "O Que Tem Dentro Deste Tutorial").  Reading: query head
  ``h`` uses key/value head ``h // (Hq // Hkv)``.
* Causal masking is named as a feature of the production library in the FAQ
  of the first page.  Reading: key ``j`` is visible to query ``i`` iff
  ``j <= i`` (top-left aligned, also when ``Sq != Sk``).
* The per-row log-sum-exp is not on the pages.  Reading: natural log of the
  softmax denominator of the *scaled* scores, ``lse = m + ln(sum exp(s - m))``.

Modules:

* ``full_softmax`` — vectorised numpy fp64 definition (full and row-sampled).
* ``biased``    — the same definition with an ALiBi bias and a block-sparse
  mask (features the first page's FAQ names for the official library);
  the readings are in its docstring.
* ``brute``     — pure-Python triple loop with ``math.fsum``; tiny inputs only.
* ``matmul``    — the plain matrix product C = A B in float64, which the tiled
  fp32-accumulating K loop of the first page's step 5 ("Multiplicação de
  Matrizes Tiled") computes block by block.
* ``rowwise``   — the row softmax (step 4 "Softmax por Linha") and the fused
  GELU (step 3 "GELU Fundido") of the same page, in float64.

Every function here is pinned by ``-m "not gpu"`` tests against facts that
do not come from the oracle itself (closed forms, invariants, a library
routine, brute force); see ``tests/test_oracle_pins.py``,
``tests/test_oracle_ext_pins.py``, ``tests/test_oracle_matmul_pins.py`` and
``tests/test_oracle_rowwise_pins.py``.
"""

from .full_softmax import attention, attention_rows
from .biased import attention_ext
from .brute import attention_bruteforce
from .matmul import matmul, matmul_rows
from .rowwise import gelu_fused, softmax_rows

__all__ = ["attention", "attention_rows", "attention_ext", "attention_bruteforce",
           "matmul", "matmul_rows", "softmax_rows", "gelu_fused"]
