"""tileattn: exact attention forward for MI355X (gfx950), HIP kernels behind a C ABI.

``forward(q, k, v, causal, scale) -> (o, lse)``, ``matmul(a, b) -> c``,
``softmax(x) -> out`` and ``gelu(x, w, b) -> out`` are the torch-facing
entries; ``tileattn_fwd`` / ``tileattn_fwd_f16`` / ``tileattn_fwd_ext`` /
``tileattn_fwd_ws`` / ``tileattn_fwd_workspace_size`` / ``tileattn_fwd_noalloc`` /
``tileattn_fwd_f32`` / ``tileattn_matmul`` / ``tileattn_softmax`` /
``tileattn_gelu`` / ``tileattn_strerror`` /
``tileattn_launch_shape`` mirror the C functions of ``include/tileattn.h``.
The shared library is loaded on first use and must have been built
(``python -m tiled_attention_tileattn_amd.build``); there is no fallback.
"""

from .binding import (  # noqa: F401
    EXPORTED,
    LIB_PATH,
    TileAttnError,
    forward,
    gelu,
    load_library,
    matmul,
    softmax,
    tileattn_fwd,
    tileattn_fwd_ext,
    tileattn_fwd_f16,
    tileattn_fwd_f32,
    tileattn_fwd_noalloc,
    tileattn_fwd_workspace_size,
    tileattn_fwd_ws,
    tileattn_gelu,
    tileattn_launch_shape,
    tileattn_matmul,
    tileattn_softmax,
    tileattn_strerror,
)
