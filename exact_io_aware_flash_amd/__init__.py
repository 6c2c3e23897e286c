"""Exact tiled attention with online softmax for AMD MI355X (gfx950).

Thin Python binding over the C ABI declared in include/flash_attn.h: it checks tensor
properties, allocates outputs with PyTorch, and passes raw device pointers and the current HIP
stream to libflash_attn.so.  Every step of the computation runs in the library's HIP kernels;
there is no fallback path.  If the library has not been built this module raises on use.

Build the library with `python -m exact_io_aware_flash_amd.build`.
"""
from __future__ import annotations

import ctypes
import math
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libflash_attn.so")

FA_OK = 0
FA_ERR_NULL = 1
FA_ERR_SHAPE = 2
FA_ERR_HEADDIM = 3
FA_ERR_ALIGN = 4
FA_ERR_SCALE = 5
FA_ERR_WORKSPACE = 6
FA_ERR_HIP = 7
FA_ERR_ALIAS = 8
FA_ERR_FLAG = 9
FA_ERR_SPLITS = 10
FA_ERR_SCRATCH = 11
FA_ERR_UNSUPPORTED = 12
NOALLOC_MAX_ROWS = 1 << 22
MASK_BLOCK = 128
MAX_SPLITS = 64

_lib = None


class FlashAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status}: {status_string(status)}")


def lib() -> ctypes.CDLL:
    """Load libflash_attn.so (raises if it is missing: there is no other implementation).  The
    environment variable FLASH_ATTN_LIB names another build of the same library instead (the
    checking builds: host sanitizers, LDS sentinels)."""
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("FLASH_ATTN_LIB") or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing; build it with `python -m exact_io_aware_flash_amd.build`")
    _lib = load(path)
    return _lib


def load(path: str) -> ctypes.CDLL:
    """Load a build of the library at `path` and declare its entry points."""
    L = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.flash_attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vp]
    L.flash_attn_fwd.restype = i
    L.flash_attn_fwd_f32.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vp]
    L.flash_attn_fwd_f32.restype = i
    L.flash_attn_bwd_workspace_bytes.argtypes = [i, i, i, i]
    L.flash_attn_bwd_workspace_bytes.restype = sz
    L.flash_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, f, i, vp, vp]
    L.flash_attn_bwd.restype = i
    L.flash_attn_bwd_f32.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, f, i, vp, vp]
    L.flash_attn_bwd_f32.restype = i
    L.flash_attn_bwd_preprocess.argtypes = [vp, vp, vp, vp, sz, i, i, i, i, vp]
    L.flash_attn_bwd_preprocess.restype = i
    L.flash_attn_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, sz, vp, vp, i, i, i, i, f, i, vp, vp]
    L.flash_attn_bwd_dkdv.restype = i
    L.flash_attn_bwd_dq.argtypes = [vp, vp, vp, vp, vp, vp, sz, vp, i, i, i, i, f, i, vp, vp]
    L.flash_attn_bwd_dq.restype = i
    L.flash_attn_fwd_splitkv_workspace_bytes.argtypes = [i, i, i, i, i]
    L.flash_attn_fwd_splitkv_workspace_bytes.restype = sz
    L.flash_attn_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i, vp, sz, vp]
    L.flash_attn_fwd_splitkv.restype = i
    L.flash_attn_merge.argtypes = [vp, vp, i, ctypes.c_int64, i, vp, vp, vp]
    L.flash_attn_merge.restype = i
    L.flash_attn_fwd_mxfp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vp]
    L.flash_attn_fwd_mxfp8.restype = i
    L.flash_attn_mxfp8_quantize_rows.argtypes = [vp, vp, vp, i, i, i, i, vp]
    L.flash_attn_mxfp8_quantize_rows.restype = i
    L.flash_attn_mxfp8_quantize_vt.argtypes = [vp, vp, vp, i, i, i, i, vp]
    L.flash_attn_mxfp8_quantize_vt.restype = i
    L.flash_attn_mxfp8_vt_cols.argtypes = [i]
    L.flash_attn_mxfp8_vt_cols.restype = ctypes.c_int64
    L.flash_attn_bwd_onepass_workspace_bytes.argtypes = [i, i, i, i]
    L.flash_attn_bwd_onepass_workspace_bytes.restype = sz
    L.flash_attn_bwd_onepass.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, f, i, vp, vp]
    L.flash_attn_bwd_onepass.restype = i
    L.flash_attn_fwd_pingpong.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vp]
    L.flash_attn_fwd_pingpong.restype = i
    L.flash_attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vp]
    L.flash_attn_bwd_noalloc.restype = i
    L.flash_attn_status_string.argtypes = [i]
    L.flash_attn_status_string.restype = ctypes.c_char_p
    return L


def status_string(status: int) -> str:
    return lib().flash_attn_status_string(status).decode()


def workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(lib().flash_attn_bwd_workspace_bytes(B, H, N, d))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream):
    """Context for the binding's own allocations.  With an explicit stream, tensors the binding
    allocates (outputs, the backward workspace, the split-key partials) are allocated on that
    stream, so the caching allocator does not hand their memory to later work on another stream
    while the kernels enqueued on `stream` may still use it."""
    import contextlib

    import torch

    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _check(t, name, dtype, shape, device):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name}: expected a tensor on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _mask_arg(block_mask, N, device):
    if block_mask is None:
        return None
    import torch

    nb = (N + MASK_BLOCK - 1) // MASK_BLOCK
    _check(block_mask, "block_mask", torch.uint8, (nb, nb), device)
    return block_mask


def fwd(q, k, v, scale: float | None = None, causal: bool = False, block_mask=None, out=None, lse=None,
        stream=None):
    """Forward pass.  q, k, v: [B, H, N, d] bf16 or float32 CUDA tensors (same dtype).
    block_mask: optional uint8 [nb, nb] CUDA tensor, nb = ceil(N / 128).
    Returns (o [B, H, N, d] in the input dtype, lse [B, H, N] float32, natural log)."""
    import torch

    B, H, N, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, name, q.dtype, (B, H, N, d), dev)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    with _on(stream):
        if out is None:
            out = torch.empty_like(q)
        if lse is None:
            lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    _check(out, "out", q.dtype, (B, H, N, d), dev)
    _check(lse, "lse", torch.float32, (B, H, N), dev)
    bm = _mask_arg(block_mask, N, dev)
    L = lib()
    if q.dtype == torch.bfloat16:
        fn, where = L.flash_attn_fwd, "flash_attn_fwd"
    elif q.dtype == torch.float32:
        fn, where = L.flash_attn_fwd_f32, "flash_attn_fwd_f32"
    else:
        raise TypeError(f"unsupported dtype {q.dtype}")
    st = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d, scale, int(bool(causal)), _ptr(bm),
            _stream(stream))
    if st != FA_OK:
        raise FlashAttnError(st, where)
    return out, lse


def fwd_pingpong(q, k, v, scale: float | None = None, causal: bool = False, out=None, lse=None, stream=None):
    """Forward (bf16, d = 128, no block mask) with the wave-specialised schedule; bitwise the
    same outputs as fwd().  Returns (o, lse)."""
    import torch

    B, H, N, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, name, torch.bfloat16, (B, H, N, d), dev)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    with _on(stream):
        out = torch.empty_like(q) if out is None else out
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev) if lse is None else lse
    _check(out, "out", torch.bfloat16, (B, H, N, d), dev)
    _check(lse, "lse", torch.float32, (B, H, N), dev)
    st = lib().flash_attn_fwd_pingpong(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d, scale,
                                       int(bool(causal)), None, _stream(stream))
    if st != FA_OK:
        raise FlashAttnError(st, "flash_attn_fwd_pingpong")
    return out, lse


def bwd(q, k, v, o, lse, do, scale: float | None = None, causal: bool = False, block_mask=None, dq=None, dk=None,
        dv=None, workspace=None, stream=None):
    """Backward pass for the forward call with the same q, k, v, scale, causal and block_mask.
    Returns (dq, dk, dv) in the input dtype."""
    import torch

    B, H, N, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check(t, name, q.dtype, (B, H, N, d), dev)
    _check(lse, "lse", torch.float32, (B, H, N), dev)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    with _on(stream):
        dq = torch.empty_like(q) if dq is None else dq
        dk = torch.empty_like(q) if dk is None else dk
        dv = torch.empty_like(q) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check(t, name, q.dtype, (B, H, N, d), dev)
    with _on(stream):
        need = workspace_bytes(B, H, N, d)
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    bm = _mask_arg(block_mask, N, dev)
    L = lib()
    if q.dtype == torch.bfloat16:
        fn, where = L.flash_attn_bwd, "flash_attn_bwd"
    elif q.dtype == torch.float32:
        fn, where = L.flash_attn_bwd_f32, "flash_attn_bwd_f32"
    else:
        raise TypeError(f"unsupported dtype {q.dtype}")
    st = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
            workspace.numel() * workspace.element_size(), B, H, N, d, scale, int(bool(causal)), _ptr(bm),
            _stream(stream))
    if st != FA_OK:
        raise FlashAttnError(st, where)
    return dq, dk, dv


def bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv, scale: float | None = None, causal: bool = False, block_mask=None,
                stream=None):
    """bf16 backward into caller-given dq, dk, dv through flash_attn_bwd_noalloc: the library's
    fixed per-device scratch holds D, so neither the library nor this function allocates device
    memory (B * H * N <= NOALLOC_MAX_ROWS).  Calls overlapping on one device race on the scratch."""
    import torch

    B, H, N, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do), ("dq", dq), ("dk", dk), ("dv", dv)):
        _check(t, name, torch.bfloat16, (B, H, N, d), dev)
    _check(lse, "lse", torch.float32, (B, H, N), dev)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    bm = _mask_arg(block_mask, N, dev)
    st = lib().flash_attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk),
                                      _ptr(dv), B, H, N, d, scale, int(bool(causal)), _ptr(bm), _stream(stream))
    if st != FA_OK:
        raise FlashAttnError(st, "flash_attn_bwd_noalloc")
    return dq, dk, dv


def onepass_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(lib().flash_attn_bwd_onepass_workspace_bytes(B, H, N, d))


def bwd_onepass(q, k, v, o, lse, do, scale: float | None = None, causal: bool = False, block_mask=None, dq=None,
                dk=None, dv=None, workspace=None, stream=None):
    """Backward (bf16, d = 128) in one pass over each key block: dK, dV and dQ from one
    recomputation of S and P, dQ summed with float32 atomics in the workspace (so dQ's rounding
    order varies run to run).  Returns (dq, dk, dv)."""
    import torch

    B, H, N, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check(t, name, torch.bfloat16, (B, H, N, d), dev)
    _check(lse, "lse", torch.float32, (B, H, N), dev)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    with _on(stream):
        dq = torch.empty_like(q) if dq is None else dq
        dk = torch.empty_like(q) if dk is None else dk
        dv = torch.empty_like(q) if dv is None else dv
        if workspace is None:
            need = onepass_workspace_bytes(B, H, N, d)
            if need == 0:
                raise FlashAttnError(FA_ERR_UNSUPPORTED, "bwd_onepass")
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    bm = _mask_arg(block_mask, N, dev)
    st = lib().flash_attn_bwd_onepass(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk),
                                      _ptr(dv), _ptr(workspace), _ws_bytes(workspace), B, H, N, d, scale,
                                      int(bool(causal)), _ptr(bm), _stream(stream))
    if st != FA_OK:
        raise FlashAttnError(st, "flash_attn_bwd_onepass")
    return dq, dk, dv


def splitkv_workspace_bytes(B: int, H: int, N: int, d: int, splits: int) -> int:
    return int(lib().flash_attn_fwd_splitkv_workspace_bytes(B, H, N, d, splits))


def default_splits(B: int, H: int, N: int) -> int:
    """Key ranges for fwd_splitkv when the caller gives none: enough that the grid has about
    1024 workgroups (four per compute unit), at most 8; 1 when the plain grid already has that."""
    wgs = B * H * ((N + 127) // 128)
    s = 1
    while s < 8 and wgs * s < 1024:
        s *= 2
    return s


def fwd_splitkv(q, k, v, scale: float | None = None, causal: bool = False, block_mask=None, splits: int | None = None,
                out=None, lse=None, workspace=None, stream=None):
    """Split-key forward (bf16): the key blocks are cut into `splits` ranges whose partial
    results are merged by log-sum-exp.  Same result as fwd() up to rounding order.
    Returns (o, lse)."""
    import torch

    B, H, N, d = q.shape
    if splits is None:
        splits = default_splits(B, H, N)
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, name, torch.bfloat16, (B, H, N, d), dev)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    with _on(stream):
        out = torch.empty_like(q) if out is None else out
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev) if lse is None else lse
    _check(out, "out", torch.bfloat16, (B, H, N, d), dev)
    _check(lse, "lse", torch.float32, (B, H, N), dev)
    with _on(stream):
        if workspace is None:
            need = splitkv_workspace_bytes(B, H, N, d, splits)
            if need == 0:
                raise FlashAttnError(FA_ERR_SPLITS, "fwd_splitkv")
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    bm = _mask_arg(block_mask, N, dev)
    st = lib().flash_attn_fwd_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d, scale,
                                      int(bool(causal)), _ptr(bm), int(splits), _ptr(workspace), _ws_bytes(workspace),
                                      _stream(stream))
    if st != FA_OK:
        raise FlashAttnError(st, "flash_attn_fwd_splitkv")
    return out, lse


def merge(o_parts, lse_parts, out=None, lse=None, stream=None):
    """Log-sum-exp merge of partial results over disjoint key sets of the same rows:
    o_parts float32 [P, ..., d], lse_parts float32 [P, ...] -> (o bf16 [..., d], lse float32 [...])."""
    import torch

    P = o_parts.shape[0]
    rows_shape = tuple(o_parts.shape[1:-1])
    d = o_parts.shape[-1]
    dev = o_parts.device
    _check(o_parts, "o_parts", torch.float32, (P, *rows_shape, d), dev)
    _check(lse_parts, "lse_parts", torch.float32, (P, *rows_shape), dev)
    with _on(stream):
        out = torch.empty((*rows_shape, d), dtype=torch.bfloat16, device=dev) if out is None else out
        lse = torch.empty(rows_shape, dtype=torch.float32, device=dev) if lse is None else lse
    _check(out, "out", torch.bfloat16, (*rows_shape, d), dev)
    _check(lse, "lse", torch.float32, rows_shape, dev)
    rows = int(math.prod(rows_shape))
    st = lib().flash_attn_merge(_ptr(o_parts), _ptr(lse_parts), P, rows, d, _ptr(out), _ptr(lse), _stream(stream))
    if st != FA_OK:
        raise FlashAttnError(st, "flash_attn_merge")
    return out, lse


# ---------------------------------------------------------------------------------------------
# The three backward stages one by one (bf16).  Enqueued in this order with one workspace they
# equal bwd().
def new_workspace(B: int, H: int, N: int, d: int, device):
    """A workspace tensor of flash_attn_bwd_workspace_bytes() bytes (torch allocations are
    256-byte aligned)."""
    import torch

    return torch.empty(workspace_bytes(B, H, N, d), dtype=torch.uint8, device=device)


def _ws_bytes(ws):
    return ws.numel() * ws.element_size()


def bwd_preprocess(q, o, do, workspace=None, stream=None):
    """Pre-pass: D = rowsum(dO * O) into `workspace`."""
    import torch

    B, H, N, d = o.shape
    for name, t in (("q", q), ("o", o), ("do", do)):
        _check(t, name, torch.bfloat16, (B, H, N, d), o.device)
    with _on(stream):
        workspace = new_workspace(B, H, N, d, o.device) if workspace is None else workspace
    st = lib().flash_attn_bwd_preprocess(_ptr(q), _ptr(o), _ptr(do), _ptr(workspace), _ws_bytes(workspace), B, H,
                                         N, d, _stream(stream))
    if st != FA_OK:
        raise FlashAttnError(st, "flash_attn_bwd_preprocess")
    return workspace


def bwd_dkdv(q, k, v, do, lse, workspace, scale=None, causal=False, block_mask=None, dk=None, dv=None, stream=None):
    import torch

    B, H, N, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("do", do)):
        _check(t, name, torch.bfloat16, (B, H, N, d), dev)
    _check(lse, "lse", torch.float32, (B, H, N), dev)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    with _on(stream):
        dk = torch.empty_like(q) if dk is None else dk
        dv = torch.empty_like(q) if dv is None else dv
    bm = _mask_arg(block_mask, N, dev)
    st = lib().flash_attn_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse), _ptr(workspace),
                                   _ws_bytes(workspace), _ptr(dk), _ptr(dv), B, H, N, d, scale, int(bool(causal)),
                                   _ptr(bm), _stream(stream))
    if st != FA_OK:
        raise FlashAttnError(st, "flash_attn_bwd_dkdv")
    return dk, dv


def bwd_dq(q, k, v, do, lse, workspace, scale=None, causal=False, block_mask=None, dq=None, stream=None):
    import torch

    B, H, N, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("do", do)):
        _check(t, name, torch.bfloat16, (B, H, N, d), dev)
    _check(lse, "lse", torch.float32, (B, H, N), dev)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    with _on(stream):
        dq = torch.empty_like(q) if dq is None else dq
    bm = _mask_arg(block_mask, N, dev)
    st = lib().flash_attn_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse), _ptr(workspace),
                                 _ws_bytes(workspace), _ptr(dq), B, H, N, d, scale, int(bool(causal)), _ptr(bm),
                                 _stream(stream))
    if st != FA_OK:
        raise FlashAttnError(st, "flash_attn_bwd_dq")
    return dq


# ---------------------------------------------------------------------------------------------
# Autograd entry: O = attention(Q, K, V) as a differentiable PyTorch operation.  The forward
# keeps O and LSE for the backward, which recomputes S and P tile by tile from them (the
# recomputation of the backward pass: "How FlashAttention Eliminates Transformer Memory
# Bottlenecks", Innovation #3).  Both directions run in the library's kernels.
class MXFP8:
    """An MX-FP8 tensor as the FP8 forward reads it: E4M3 codes (uint8) and E8M0 block scales
    (uint8, value 2^(s - 127)).  `transposed` marks V's feature-major layout."""

    def __init__(self, codes, scales, transposed: bool, shape):
        self.codes, self.scales, self.transposed, self.shape = codes, scales, transposed, tuple(shape)


def mxfp8_vt_cols(N: int) -> int:
    return int(lib().flash_attn_mxfp8_vt_cols(N))


def mxfp8_quantize(x, transposed: bool = False, stream=None) -> MXFP8:
    """MX-FP8 quantisation of a bf16 [B, H, N, d] CUDA tensor: blocks of 32 along d (Q, K), or
    with transposed=True blocks of 32 keys into V's transposed layout [B, H, d, Np]."""
    import torch

    B, H, N, d = x.shape
    _check(x, "x", torch.bfloat16, (B, H, N, d), x.device)
    L = lib()
    if transposed:
        npad = mxfp8_vt_cols(N)
        with _on(stream):
            codes = torch.empty((B, H, d, npad), dtype=torch.uint8, device=x.device)
            scales = torch.empty((B, H, npad // 32, 32, d // 32), dtype=torch.uint8, device=x.device)
        st = L.flash_attn_mxfp8_quantize_vt(_ptr(x), _ptr(codes), _ptr(scales), B, H, N, d, _stream(stream))
        where = "flash_attn_mxfp8_quantize_vt"
    else:
        with _on(stream):
            codes = torch.empty((B, H, N, d), dtype=torch.uint8, device=x.device)
            scales = torch.empty((B, H, N, d // 32), dtype=torch.uint8, device=x.device)
        st = L.flash_attn_mxfp8_quantize_rows(_ptr(x), _ptr(codes), _ptr(scales), B, H, N, d, _stream(stream))
        where = "flash_attn_mxfp8_quantize_rows"
    if st != FA_OK:
        raise FlashAttnError(st, where)
    return MXFP8(codes, scales, transposed, (B, H, N, d))


def fwd_mxfp8(q: MXFP8, k: MXFP8, vt: MXFP8, scale: float | None = None, causal: bool = False, block_mask=None,
              out=None, lse=None, stream=None):
    """MX-FP8 forward from quantised Q, K (row blocks) and V (transposed).  Returns
    (o [B, H, N, d] bf16, lse [B, H, N] float32)."""
    import torch

    B, H, N, d = q.shape
    if k.shape != q.shape or vt.shape != q.shape or q.transposed or k.transposed or not vt.transposed:
        raise ValueError("fwd_mxfp8: q, k row-quantised and vt transposed, all of one [B, H, N, d] shape")
    dev = q.codes.device
    npad = mxfp8_vt_cols(N)
    _check(q.codes, "q.codes", torch.uint8, (B, H, N, d), dev)
    _check(k.codes, "k.codes", torch.uint8, (B, H, N, d), dev)
    _check(q.scales, "q.scales", torch.uint8, (B, H, N, d // 32), dev)
    _check(k.scales, "k.scales", torch.uint8, (B, H, N, d // 32), dev)
    _check(vt.codes, "vt.codes", torch.uint8, (B, H, d, npad), dev)
    _check(vt.scales, "vt.scales", torch.uint8, (B, H, npad // 32, 32, d // 32), dev)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    with _on(stream):
        if out is None:
            out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=dev)
        if lse is None:
            lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    _check(out, "out", torch.bfloat16, (B, H, N, d), dev)
    _check(lse, "lse", torch.float32, (B, H, N), dev)
    bm = _mask_arg(block_mask, N, dev)
    st = lib().flash_attn_fwd_mxfp8(_ptr(q.codes), _ptr(q.scales), _ptr(k.codes), _ptr(k.scales), _ptr(vt.codes),
                                    _ptr(vt.scales), _ptr(out), _ptr(lse), B, H, N, d, scale, int(bool(causal)),
                                    _ptr(bm), _stream(stream))
    if st != FA_OK:
        raise FlashAttnError(st, "flash_attn_fwd_mxfp8")
    return out, lse


def _attention_fn():
    import torch

    class _Attention(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, scale, causal, block_mask):
            o, lse = fwd(q, k, v, scale, causal, block_mask)
            ctx.save_for_backward(q, k, v, o, lse)
            ctx.scale, ctx.causal, ctx.block_mask = scale, causal, block_mask
            return o

        @staticmethod
        def backward(ctx, do):
            q, k, v, o, lse = ctx.saved_tensors
            dq, dk, dv = bwd(q, k, v, o, lse, do.contiguous(), ctx.scale, ctx.causal, ctx.block_mask)
            return dq, dk, dv, None, None, None

    return _Attention


_ATTENTION = None


def attention(q, k, v, scale: float | None = None, causal: bool = False, block_mask=None):
    """Differentiable exact attention: returns O [B, H, N, d] (input dtype) for q, k, v of shape
    [B, H, N, d] (bf16 or float32, contiguous, on the GPU); gradients flow to q, k and v."""
    global _ATTENTION
    if _ATTENTION is None:
        _ATTENTION = _attention_fn()
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    return _ATTENTION.apply(q, k, v, float(scale), bool(causal), block_mask)
