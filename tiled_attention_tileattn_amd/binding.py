"""Thin ctypes binding of ``libtileattn.so`` (argument marshalling only).

The raw functions mirror the C ABI of ``include/tileattn.h`` name for name and
take plain integers for device pointers and the stream.  ``forward`` is the
torch convenience wrapper: it checks tensors, allocates ``o``/``lse`` with
torch (the library itself allocates nothing) and passes torch's current HIP
stream.  Every step of the attention runs in the library's kernels; there is
no fallback of any kind -- if the library is missing, every call raises.
"""

from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtileattn.so")

EXPORTED = ("tileattn_fwd", "tileattn_fwd_f16", "tileattn_fwd_ext", "tileattn_fwd_ws",
            "tileattn_fwd_workspace_size", "tileattn_fwd_noalloc", "tileattn_fwd_f32", "tileattn_matmul", "tileattn_softmax", "tileattn_gelu", "tileattn_strerror",
            "tileattn_launch_shape")

DTYPE_F32, DTYPE_BF16 = 0, 1  # tileattn_dtype codes

STATUS = {
    0: "TILEATTN_OK",
    -1: "TILEATTN_ERR_NULL_POINTER",
    -2: "TILEATTN_ERR_BAD_SHAPE",
    -3: "TILEATTN_ERR_GQA_RATIO",
    -4: "TILEATTN_ERR_HEAD_DIM",
    -5: "TILEATTN_ERR_SCALE",
    -6: "TILEATTN_ERR_ALIGNMENT",
    -7: "TILEATTN_ERR_TOO_LARGE",
    -8: "TILEATTN_ERR_LAUNCH",
    -9: "TILEATTN_ERR_DTYPE",
    -10: "TILEATTN_ERR_WORKSPACE",
    -11: "TILEATTN_ERR_SCRATCH",
}

_lib = None


class TileAttnError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {STATUS.get(code, code)} ({tileattn_strerror(code)})")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build the HIP library first "
            "(python -m tiled_attention_tileattn_amd.build)")
    lib = ctypes.CDLL(path)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    sig = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
    lib.tileattn_fwd.argtypes = sig
    lib.tileattn_fwd.restype = i
    lib.tileattn_fwd_f16.argtypes = sig
    lib.tileattn_fwd_f16.restype = i
    lib.tileattn_fwd_ext.argtypes = sig[:13] + [vp, vp, i, i, vp]
    lib.tileattn_fwd_ext.restype = i
    lib.tileattn_fwd_ws.argtypes = sig[:13] + [vp, i, vp, ctypes.c_size_t, vp]
    lib.tileattn_fwd_ws.restype = i
    lib.tileattn_fwd_workspace_size.argtypes = [i] * 7
    lib.tileattn_fwd_workspace_size.restype = ctypes.c_longlong
    lib.tileattn_fwd_noalloc.argtypes = sig[:13] + [vp, i, vp]
    lib.tileattn_fwd_noalloc.restype = i
    lib.tileattn_fwd_f32.argtypes = sig
    lib.tileattn_fwd_f32.restype = i
    lib.tileattn_matmul.argtypes = [vp, vp, vp, i, i, i, i, vp]
    lib.tileattn_matmul.restype = i
    ll = ctypes.c_longlong
    lib.tileattn_softmax.argtypes = [vp, vp, i, i, ll, i, vp]
    lib.tileattn_softmax.restype = i
    lib.tileattn_gelu.argtypes = [vp, vp, vp, vp, ll, i, vp]
    lib.tileattn_gelu.restype = i
    lib.tileattn_strerror.argtypes = [i]
    lib.tileattn_strerror.restype = ctypes.c_char_p
    lib.tileattn_launch_shape.argtypes = [i, i, i, i, i, i, i, i, ctypes.POINTER(i),
                                          ctypes.POINTER(i), ctypes.POINTER(ctypes.c_longlong)]
    lib.tileattn_launch_shape.restype = i
    _lib = lib
    return lib


# ---- raw C-ABI mirrors (integers for pointers and stream) -------------------
def tileattn_fwd(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, causal, stream) -> int:
    return load_library().tileattn_fwd(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D,
                                       float(scale), int(bool(causal)), stream)


def tileattn_fwd_f16(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, causal, stream) -> int:
    return load_library().tileattn_fwd_f16(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D,
                                           float(scale), int(bool(causal)), stream)


def tileattn_fwd_ext(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, causal, alibi_slopes,
                     block_mask, mask_heads, is_f16, stream) -> int:
    return load_library().tileattn_fwd_ext(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, float(scale),
                                           int(bool(causal)), alibi_slopes, block_mask, mask_heads,
                                           int(bool(is_f16)), stream)


def tileattn_fwd_ws(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, causal, alibi_slopes, is_f16,
                    workspace, workspace_bytes, stream) -> int:
    return load_library().tileattn_fwd_ws(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, float(scale),
                                          int(bool(causal)), alibi_slopes, int(bool(is_f16)), workspace,
                                          workspace_bytes, stream)


def tileattn_fwd_workspace_size(B, Hq, Hkv, Sq, Sk, D, causal) -> int:
    return load_library().tileattn_fwd_workspace_size(B, Hq, Hkv, Sq, Sk, D, int(bool(causal)))


def tileattn_fwd_noalloc(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, causal, alibi_slopes, is_f16,
                         stream) -> int:
    return load_library().tileattn_fwd_noalloc(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, float(scale),
                                               int(bool(causal)), alibi_slopes, int(bool(is_f16)), stream)


def tileattn_fwd_f32(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, causal, stream) -> int:
    return load_library().tileattn_fwd_f32(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D,
                                           float(scale), int(bool(causal)), stream)


def tileattn_matmul(a, b, c, M, N, K, out_bf16, stream) -> int:
    return load_library().tileattn_matmul(a, b, c, M, N, K, int(bool(out_bf16)), stream)


def tileattn_softmax(x, out, n_rows, n_cols, stride, dtype, stream) -> int:
    return load_library().tileattn_softmax(x, out, n_rows, n_cols, stride, dtype, stream)


def tileattn_gelu(x, w, b, out, n, dtype, stream) -> int:
    return load_library().tileattn_gelu(x, w, b, out, n, dtype, stream)


def tileattn_strerror(status: int) -> str:
    return load_library().tileattn_strerror(int(status)).decode()


def tileattn_launch_shape(dtype_bytes, B, Hq, Hkv, Sq, Sk, D, causal):
    """Return (status, block_m, block_n, workgroups)."""
    bm, bn, wg = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_longlong(0)
    st = load_library().tileattn_launch_shape(dtype_bytes, B, Hq, Hkv, Sq, Sk, D, int(bool(causal)),
                                              ctypes.byref(bm), ctypes.byref(bn), ctypes.byref(wg))
    return st, bm.value, bn.value, wg.value


# ---- torch convenience wrapper ----------------------------------------------
def _overlap(a, b) -> bool:
    """The byte ranges of two contiguous tensors intersect."""
    a0, b0 = a.data_ptr(), b.data_ptr()
    a1, b1 = a0 + a.numel() * a.element_size(), b0 + b.numel() * b.element_size()
    return a0 < b1 and b0 < a1 and a1 > a0 and b1 > b0


def forward(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None,
            stream=None, alibi_slopes=None, block_mask=None, key_chunks: bool = True):
    """Attention forward on the GPU: returns (o, lse).

    q [B, Hq, Sq, D], k/v [B, Hkv, Sk, D]: contiguous bf16, fp16 or fp32 tensors on
    one HIP device.  ``scale`` defaults to 1/sqrt(D).  ``out``/``lse`` may be
    preallocated ([B, Hq, Sq, D] in q's dtype, [B, Hq, Sq] fp32).  ``stream``
    is a torch stream (default: the current stream of q's device).

    ``alibi_slopes`` (float32 [Hq]) and/or ``block_mask`` (uint8
    [1 or Hq, ceil(Sq/64), ceil(Sk/64)]), both on q's device, select
    ``tileattn_fwd_ext`` (bf16 or fp16 inputs only).

    bf16 / fp16 calls without a block mask go through ``tileattn_fwd_ws``
    when ``key_chunks`` is true (the default): where the library splits
    query tiles' key ranges over several workgroups, its workspace is a
    torch allocation on the launch stream.  ``key_chunks=False`` calls
    ``tileattn_fwd`` / ``tileattn_fwd_f16`` / ``tileattn_fwd_ext``, which
    never split.
    """
    import torch

    entry = {torch.bfloat16: tileattn_fwd, torch.float16: tileattn_fwd_f16,
             torch.float32: tileattn_fwd_f32}
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dim() != 4:
            raise ValueError(f"{name} must be a 4-D torch tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a HIP device, got {t.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in entry:
        raise ValueError("q, k, v must share one dtype: bfloat16, float16 or float32")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on the same device")
    B, Hq, Sq, D = q.shape
    Bk, Hkv, Sk, Dk = k.shape
    if v.shape != k.shape or Bk != B or Dk != D:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous tensor like q")
    if tuple(lse.shape) != (B, Hq, Sq) or lse.dtype != torch.float32 or not lse.is_contiguous() \
            or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 tensor [B, Hq, Sq] on q's device")
    for name, t in (("out", out), ("lse", lse)):
        if any(_overlap(t, u) for u in (q, k, v)):
            raise ValueError(f"{name} must not overlap q, k or v")
    ext = alibi_slopes is not None or block_mask is not None
    if ext:
        if q.dtype not in (torch.bfloat16, torch.float16):
            raise ValueError("alibi_slopes / block_mask need bfloat16 or float16 inputs")
        if alibi_slopes is not None and (alibi_slopes.dtype != torch.float32
                                         or tuple(alibi_slopes.shape) != (Hq,)
                                         or not alibi_slopes.is_contiguous()
                                         or alibi_slopes.device != q.device):
            raise ValueError("alibi_slopes must be a contiguous float32 tensor [Hq] on q's device")
        mask_heads = 1
        if block_mask is not None:
            nq, nk = -(-Sq // 64), -(-Sk // 64)
            if (block_mask.dtype != torch.uint8 or block_mask.dim() != 3
                    or block_mask.shape[0] not in (1, Hq) or tuple(block_mask.shape[1:]) != (nq, nk)
                    or not block_mask.is_contiguous() or block_mask.device != q.device):
                raise ValueError(f"block_mask must be a contiguous uint8 tensor [1 or Hq, {nq}, {nk}] "
                                 "on q's device")
            mask_heads = block_mask.shape[0]
    fn = tileattn_fwd_ext if ext else entry[q.dtype]
    with torch.cuda.device(q.device):
        s = stream if stream is not None else torch.cuda.current_stream(q.device)
        ws_bytes = 0
        if key_chunks and block_mask is None and q.dtype != torch.float32:
            ws_bytes = tileattn_fwd_workspace_size(B, Hq, Hkv, Sq, Sk, D, causal)
            if ws_bytes < 0:
                raise TileAttnError(ws_bytes, "tileattn_fwd_workspace_size")
        if ws_bytes > 0:
            fn = tileattn_fwd_ws
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
            if s != torch.cuda.current_stream(q.device):
                ws.record_stream(s)
            rc = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                    B, Hq, Hkv, Sq, Sk, D, scale, causal,
                    None if alibi_slopes is None else alibi_slopes.data_ptr(),
                    int(q.dtype == torch.float16), ws.data_ptr(), ws_bytes, s.cuda_stream)
        elif ext:
            rc = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                    B, Hq, Hkv, Sq, Sk, D, scale, causal,
                    None if alibi_slopes is None else alibi_slopes.data_ptr(),
                    None if block_mask is None else block_mask.data_ptr(), mask_heads,
                    int(q.dtype == torch.float16), s.cuda_stream)
        else:
            rc = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                    B, Hq, Hkv, Sq, Sk, D, scale, causal, s.cuda_stream)
    if rc != 0:
        raise TileAttnError(rc, fn.__name__)
    return out, lse


def matmul(a, b, out=None, out_dtype=None, stream=None):
    """C = A @ B on the GPU with an fp32 accumulator: returns C.

    a [M, K] and b [K, N]: contiguous bfloat16 tensors on one HIP device, N
    and K multiples of 8.  ``out_dtype`` is torch.float32 (default: the
    accumulator as it is) or torch.bfloat16; ``out`` may be preallocated
    ([M, N], contiguous, that dtype).  ``stream`` is a torch stream (default:
    the current stream of a's device).
    """
    import torch

    for name, t in (("a", a), ("b", b)):
        if not isinstance(t, torch.Tensor) or t.dim() != 2 or t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be a 2-D bfloat16 torch tensor")
        if t.device.type != "cuda" or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous tensor on a HIP device")
    if a.device != b.device:
        raise ValueError("a and b must be on the same device")
    M, K = a.shape
    Kb, N = b.shape
    if Kb != K:
        raise ValueError(f"shape mismatch a{tuple(a.shape)} b{tuple(b.shape)}")
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.float32
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out_dtype must be torch.float32 or torch.bfloat16")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    if tuple(out.shape) != (M, N) or out.dtype != out_dtype or not out.is_contiguous() \
            or out.device != a.device:
        raise ValueError(f"out must be a contiguous {out_dtype} tensor [{M}, {N}] on a's device")
    with torch.cuda.device(a.device):
        s = stream if stream is not None else torch.cuda.current_stream(a.device)
        rc = tileattn_matmul(a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K,
                             out_dtype == torch.bfloat16, s.cuda_stream)
    if rc != 0:
        raise TileAttnError(rc, "tileattn_matmul")
    return out


def _dtype_code(t):
    import torch

    codes = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}
    if t.dtype not in codes:
        raise ValueError("dtype must be torch.float32 or torch.bfloat16")
    return codes[t.dtype]


def softmax(x, out=None, n_cols=None, stream=None):
    """Row softmax on the GPU: returns out.

    x [n_rows, stride]: a contiguous float32 or bfloat16 tensor on a HIP
    device; the softmax runs over the first ``n_cols`` columns (default: all)
    of every row and writes them into ``out`` (same shape and dtype as x; may
    be x itself).  Columns past n_cols of out are left as they are.
    """
    import torch

    if not isinstance(x, torch.Tensor) or x.dim() != 2 or x.device.type != "cuda" or not x.is_contiguous():
        raise ValueError("x must be a contiguous 2-D tensor on a HIP device")
    code = _dtype_code(x)
    n_rows, stride = x.shape
    n_cols = stride if n_cols is None else int(n_cols)
    if out is None:
        out = torch.empty_like(x)
    if out.shape != x.shape or out.dtype != x.dtype or not out.is_contiguous() or out.device != x.device:
        raise ValueError("out must be a contiguous tensor like x")
    with torch.cuda.device(x.device):
        s = stream if stream is not None else torch.cuda.current_stream(x.device)
        rc = tileattn_softmax(x.data_ptr(), out.data_ptr(), n_rows, n_cols, stride, code, s.cuda_stream)
    if rc != 0:
        raise TileAttnError(rc, "tileattn_softmax")
    return out


def gelu(x, w, b, out=None, stream=None):
    """Fused GELU on the GPU: out = gelu_tanh(x * w + b) elementwise; returns out.

    x, w, b: contiguous float32 or bfloat16 tensors of one shape and dtype on
    one HIP device; ``out`` (same shape and dtype) may be one of them.
    """
    import torch

    for name, t in (("x", x), ("w", w), ("b", b)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous tensor on a HIP device")
    if not (x.shape == w.shape == b.shape) or not (x.dtype == w.dtype == b.dtype) \
            or not (x.device == w.device == b.device):
        raise ValueError("x, w, b must share shape, dtype and device")
    code = _dtype_code(x)
    if out is None:
        out = torch.empty_like(x)
    if out.shape != x.shape or out.dtype != x.dtype or not out.is_contiguous() or out.device != x.device:
        raise ValueError("out must be a contiguous tensor like x")
    with torch.cuda.device(x.device):
        s = stream if stream is not None else torch.cuda.current_stream(x.device)
        rc = tileattn_gelu(x.data_ptr(), w.data_ptr(), b.data_ptr(), out.data_ptr(), x.numel(), code,
                           s.cuda_stream)
    if rc != 0:
        raise TileAttnError(rc, "tileattn_gelu")
    return out
