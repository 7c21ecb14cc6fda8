"""ctypes binding of libfa_attn.so (argument marshalling only).

Every computation runs in the library's HIP kernels.  If the library has not
been built, loading raises; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import math
import os
import re

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libfa_attn.so")
HEADER = os.path.join(os.path.dirname(PKG_DIR), "include", "fa_attn.h")

F32, F16, BF16 = 0, 1, 2
MASK_NONE, MASK_CAUSAL = 0, 1

_lib = None


class FaError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_str(status)})")


def lib():
    """Load the shared library once (raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m io_aware_exact_12_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        L.attn_fwd.restype = ctypes.c_int
        L.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64,
                               ctypes.c_int, ctypes.c_float, ctypes.c_int, vp]
        L.attn_bwd.restype = ctypes.c_int
        L.attn_bwd.argtypes = [vp] * 9 + [i64, i64, i64, i64, ctypes.c_int, ctypes.c_float,
                                          ctypes.c_int, vp, ctypes.c_size_t, vp]
        L.attn_fwd_window.restype = ctypes.c_int
        L.attn_fwd_window.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                      i64, ctypes.c_float, ctypes.c_int, vp]
        L.attn_bwd_window.restype = ctypes.c_int
        L.attn_bwd_window.argtypes = [vp] * 9 + [i64, i64, i64, i64, i64, ctypes.c_float,
                                                 ctypes.c_int, vp, ctypes.c_size_t, vp]
        i64p = ctypes.POINTER(ctypes.c_int64)
        L.attn_fwd_strided.restype = ctypes.c_int
        L.attn_fwd_strided.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64p, i64p, i64p,
                                       ctypes.c_int, ctypes.c_float, ctypes.c_int, vp]
        L.attn_bwd_strided.restype = ctypes.c_int
        L.attn_bwd_strided.argtypes = [vp] * 9 + [i64, i64, i64, i64, i64p, i64p, ctypes.c_int,
                                                  ctypes.c_float, ctypes.c_int, vp, ctypes.c_size_t, vp]
        L.attn_fwd_dv.restype = ctypes.c_int
        L.attn_fwd_dv.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_int,
                                  ctypes.c_float, ctypes.c_int, vp]
        L.attn_bwd_dv.restype = ctypes.c_int
        L.attn_bwd_dv.argtypes = [vp] * 9 + [i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_float,
                                             ctypes.c_int, vp, ctypes.c_size_t, vp]
        L.attn_fwd_block_sparse.restype = ctypes.c_int
        L.attn_fwd_block_sparse.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, i64, i64,
                                            ctypes.c_int, ctypes.c_float, ctypes.c_int, vp]
        L.attn_bwd_block_sparse.restype = ctypes.c_int
        L.attn_bwd_block_sparse.argtypes = [vp] * 9 + [i64, i64, i64, i64, vp, i64, i64, ctypes.c_int,
                                                       ctypes.c_float, ctypes.c_int, vp, ctypes.c_size_t,
                                                       vp]
        L.attn_fwd_kv_outer.restype = ctypes.c_int
        L.attn_fwd_kv_outer.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int,
                                         ctypes.c_float, ctypes.c_int, vp, ctypes.c_size_t, vp]
        L.attn_fwd_kv_outer_workspace_bytes.restype = ctypes.c_size_t
        L.attn_fwd_kv_outer_workspace_bytes.argtypes = [i64, i64, i64, i64, ctypes.c_int]
        L.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.attn_bwd_workspace_bytes.argtypes = [i64, i64, i64, i64, ctypes.c_int]
        L.attn_bwd_block_sparse_workspace_bytes.restype = ctypes.c_size_t
        L.attn_bwd_block_sparse_workspace_bytes.argtypes = [i64, i64, i64, i64, ctypes.c_int]
        L.attn_bwd_noalloc.restype = ctypes.c_int
        L.attn_bwd_noalloc.argtypes = [vp] * 9 + [i64, i64, i64, i64, ctypes.c_int, ctypes.c_float,
                                                  ctypes.c_int, vp]
        L.attn_bwd_noalloc_max_rows.restype = ctypes.c_size_t
        L.attn_bwd_noalloc_max_rows.argtypes = []
        L.fa_status_str.restype = ctypes.c_char_p
        L.fa_status_str.argtypes = [ctypes.c_int]
        L.fa_abi_version.restype = ctypes.c_int
        L.fa_abi_version.argtypes = []
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().fa_status_str(int(status)).decode()


def declared_symbols(header: str = HEADER):
    """Names of the functions include/fa_attn.h declares."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


def attn_fwd_raw(q, k, v, o, lse, B, H, N, d, mask, scale, dtype, stream):
    """Direct call of the C entry point with integer pointers; returns the status."""
    return lib().attn_fwd(q, k, v, o, lse, B, H, N, d, mask, scale, dtype, stream)


def attn_bwd_raw(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, mask, scale, dtype, ws, ws_bytes,
                 stream):
    """Direct call of the C entry point with integer pointers; returns the status."""
    return lib().attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, mask, scale, dtype, ws,
                          ws_bytes, stream)


def attn_bwd_noalloc_raw(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, mask, scale, dtype, stream):
    """Direct call of the allocation-free backward entry point; returns the status."""
    return lib().attn_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, mask, scale, dtype,
                                  stream)


def noalloc_max_rows():
    """Largest B * H * N the allocation-free backward accepts."""
    return lib().attn_bwd_noalloc_max_rows()


def attn_fwd_window_raw(q, k, v, o, lse, B, H, N, d, window, scale, dtype, stream):
    """Direct call of the C entry point with integer pointers; returns the status."""
    return lib().attn_fwd_window(q, k, v, o, lse, B, H, N, d, window, scale, dtype, stream)


def attn_bwd_window_raw(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, window, scale, dtype, ws,
                        ws_bytes, stream):
    """Direct call of the C entry point with integer pointers; returns the status."""
    return lib().attn_bwd_window(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, window, scale,
                                 dtype, ws, ws_bytes, stream)


def bwd_workspace_bytes(B, H, N, d, dtype_code):
    return lib().attn_bwd_workspace_bytes(B, H, N, d, dtype_code)


def bwd_block_sparse_workspace_bytes(B, H, N, d, dtype_code):
    return lib().attn_bwd_block_sparse_workspace_bytes(B, H, N, d, dtype_code)


def _strides(st):
    """A host int64[3] array for the ABI (None stays None)."""
    return None if st is None else (ctypes.c_int64 * 3)(*[int(x) for x in st])


def attn_fwd_strided_raw(q, k, v, o, lse, B, H, N, d, q_st, kv_st, o_st, mask, scale, dtype, stream):
    return lib().attn_fwd_strided(q, k, v, o, lse, B, H, N, d, _strides(q_st), _strides(kv_st),
                                  _strides(o_st), mask, scale, dtype, stream)


def attn_bwd_strided_raw(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, in_st, grad_st, mask, scale,
                         dtype, ws, ws_bytes, stream):
    return lib().attn_bwd_strided(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, _strides(in_st),
                                  _strides(grad_st), mask, scale, dtype, ws, ws_bytes, stream)


def attn_fwd_dv_raw(q, k, v, o, lse, B, H, N, d, dv, mask, scale, dtype, stream):
    return lib().attn_fwd_dv(q, k, v, o, lse, B, H, N, d, dv, mask, scale, dtype, stream)


def attn_bwd_dv_raw(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, d_v, mask, scale, dtype, ws,
                    ws_bytes, stream):
    return lib().attn_bwd_dv(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, d_v, mask, scale, dtype,
                             ws, ws_bytes, stream)


def attn_fwd_block_sparse_raw(q, k, v, o, lse, B, H, N, d, block_mask, mask_batches, mask_heads,
                              mask, scale, dtype, stream):
    return lib().attn_fwd_block_sparse(q, k, v, o, lse, B, H, N, d, block_mask, mask_batches,
                                       mask_heads, mask, scale, dtype, stream)


def attn_bwd_block_sparse_raw(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, block_mask,
                              mask_batches, mask_heads, mask, scale, dtype, ws, ws_bytes, stream):
    return lib().attn_bwd_block_sparse(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, block_mask,
                                       mask_batches, mask_heads, mask, scale, dtype, ws, ws_bytes,
                                       stream)


def _check_block_mask(bm, B, H, N):
    import torch
    nb = -(-N // 64)
    if bm.dim() != 4 or tuple(bm.shape[-2:]) != (nb, nb) or bm.shape[0] not in (1, B) or \
            bm.shape[1] not in (1, H):
        raise ValueError(f"block_mask must be [1 or B, 1 or H, {nb}, {nb}], got {tuple(bm.shape)}")
    if bm.dtype != torch.uint8 or not bm.is_cuda or not bm.is_contiguous():
        raise ValueError("block_mask must be a contiguous uint8 device tensor")


def _layout(t):
    """{batch, head, row} element strides of a [B, H, N, d] tensor whose last
    axis is contiguous; axes of extent 1 get stride 0 (their stride is never
    used)."""
    return tuple(0 if t.shape[i] == 1 else t.stride(i) for i in range(3))


def attn_fwd_kv_outer_raw(q, k, v, o, lse, B, H, N, d, mask, scale, dtype, ws, ws_bytes, stream):
    return lib().attn_fwd_kv_outer(q, k, v, o, lse, B, H, N, d, mask, scale, dtype, ws, ws_bytes,
                                   stream)


def kv_outer_workspace_bytes(B, H, N, d, dtype_code):
    return lib().attn_fwd_kv_outer_workspace_bytes(B, H, N, d, dtype_code)


def check_buffer(t, name, shape, dtype, device, contiguous=True):
    """Reject a caller-supplied output or scratch tensor that does not match what
    the kernels will write through its raw pointer: its shape, dtype and device
    must be the given ones, and it must be contiguous (or, with
    ``contiguous=False``, have a contiguous last axis)."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not contiguous and t.dim() > 0 and t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError(f"{name} must have a contiguous last axis")


def check_workspace(ws, need, device):
    """A workspace must be a contiguous uint8 tensor of at least ``need`` bytes on ``device``."""
    import torch
    if ws.dtype != torch.uint8:
        raise TypeError(f"workspace must be uint8, got {ws.dtype}")
    if ws.device != device:
        raise ValueError(f"workspace must be on {device}, got {ws.device}")
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    if ws.numel() < need:
        raise ValueError(f"workspace holds {ws.numel()} bytes, {need} needed")


def _torch_dtype_code(t):
    import torch
    codes = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def attn_fwd(q, k, v, causal: bool = False, scale: float | None = None, *, out=None, lse=None,
             return_lse: bool = True, stream=None, window: int | None = None, block_mask=None):
    """Exact attention forward on the GPU: returns ``(o, lse)`` (lse None if not requested).

    q, k, v: contiguous device tensors [B, H, N, d] of one dtype (float32,
    float16 or bfloat16), d in {64, 96, 128, 256} (256: float16 or bfloat16).  ``scale`` defaults to 1/sqrt(d).
    ``window`` (causal only) calls ``attn_fwd_window``: query i sees keys
    i - window < j <= i.  ``block_mask`` (uint8 device tensor
    [1 or B, 1 or H, ceil(N/64), ceil(N/64)]) calls ``attn_fwd_block_sparse``.
    Non-contiguous q, k, v (last axis contiguous) call ``attn_fwd_strided``.
    Work is enqueued on ``stream`` (default: torch's current stream).
    """
    import torch
    if q.shape != k.shape or q.shape[:3] != v.shape[:3] or q.dim() != 4 or v.dim() != 4:
        raise ValueError(f"q, k must share one [B, H, N, d] shape and v be [B, H, N, dv], "
                         f"got {q.shape}, {k.shape}, {v.shape}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    for t in (q, k, v):
        if not t.is_cuda or t.stride(-1) != 1:
            raise ValueError("q, k, v must be device tensors with a contiguous last axis")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k and v must be on one device")
    B, H, N, d = q.shape
    dv = v.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q) if dv == d else torch.empty((B, H, N, dv), dtype=q.dtype, device=q.device)
    else:
        check_buffer(out, "out", (B, H, N, dv), q.dtype, q.device, contiguous=False)
    if return_lse and lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    elif return_lse:
        check_buffer(lse, "lse", (B, H, N), torch.float32, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    if dv != d:
        # values of another width (v, o: [B, H, N, dv], all contiguous)
        if window is not None or block_mask is not None:
            raise ValueError("dv != d takes no window or block mask")
        if not all(t.is_contiguous() for t in (q, k, v, out)) or tuple(out.shape) != (B, H, N, dv):
            raise ValueError("dv != d takes contiguous q, k, v and a contiguous [B, H, N, dv] out")
        st = attn_fwd_dv_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                             lse.data_ptr() if return_lse else None, B, H, N, d, dv,
                             MASK_CAUSAL if causal else MASK_NONE, float(scale), _torch_dtype_code(q),
                             stream.cuda_stream)
        if st != 0:
            raise FaError(st, "attn_fwd_dv")
        return out, (lse if return_lse else None)
    if block_mask is not None:
        bm = block_mask
        _check_block_mask(bm, B, H, N)
        if window is not None or not all(t.is_contiguous() for t in (q, k, v, out)):
            raise ValueError("a block-sparse mask takes contiguous q, k, v, out and no window")
        st = attn_fwd_block_sparse_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                       lse.data_ptr() if return_lse else None, B, H, N, d,
                                       bm.data_ptr(), bm.shape[0], bm.shape[1],
                                       MASK_CAUSAL if causal else MASK_NONE, float(scale),
                                       _torch_dtype_code(q), stream.cuda_stream)
        if st != 0:
            raise FaError(st, "attn_fwd_block_sparse")
        return out, (lse if return_lse else None)
    if not all(t.is_contiguous() for t in (q, k, v, out)):
        # strided views (transposed, packed, or k and v broadcast over heads)
        if window is not None:
            raise ValueError("a sliding window takes contiguous q, k, v")
        if _layout(k) != _layout(v):
            raise ValueError("k and v must share one layout")
        if out.shape != q.shape or out.stride(-1) != 1:
            raise ValueError("out must be [B, H, N, d] with a contiguous last axis")
        st = attn_fwd_strided_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                  lse.data_ptr() if return_lse else None, B, H, N, d, _layout(q),
                                  _layout(k), _layout(out), MASK_CAUSAL if causal else MASK_NONE,
                                  float(scale), _torch_dtype_code(q), stream.cuda_stream)
        if st != 0:
            raise FaError(st, "attn_fwd_strided")
        return out, (lse if return_lse else None)
    if window is not None:
        if not causal:
            raise ValueError("a sliding window needs causal=True")
        st = lib().attn_fwd_window(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                   lse.data_ptr() if return_lse else None, B, H, N, d, int(window),
                                   float(scale), _torch_dtype_code(q), stream.cuda_stream)
        if st != 0:
            raise FaError(st, "attn_fwd_window")
        return out, (lse if return_lse else None)
    st = lib().attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                        lse.data_ptr() if return_lse else None, B, H, N, d,
                        MASK_CAUSAL if causal else MASK_NONE, float(scale), _torch_dtype_code(q),
                        stream.cuda_stream)
    if st != 0:
        raise FaError(st, "attn_fwd")
    return out, (lse if return_lse else None)


def attn_fwd_kv_outer(q, k, v, causal: bool = False, scale: float | None = None, *, out=None,
                      lse=None, workspace=None, stream=None):
    """The forward in the original key/value-outer loop order (``attn_fwd_kv_outer``):
    returns ``(o, lse)``.  Same arguments as ``attn_fwd`` (fp16/bf16 only);
    ``workspace`` is a uint8 device tensor of at least
    ``kv_outer_workspace_bytes`` bytes, allocated here when not given.
    """
    import torch
    if q.shape != k.shape or q.shape != v.shape or q.dim() != 4:
        raise ValueError(f"q, k, v must share one [B, H, N, d] shape, got {q.shape}, {k.shape}, {v.shape}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous device tensors")
    B, H, N, d = q.shape
    code = _torch_dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        check_buffer(out, "out", (B, H, N, d), q.dtype, q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        check_buffer(lse, "lse", (B, H, N), torch.float32, q.device)
    need = kv_outer_workspace_bytes(B, H, N, d, code)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    else:
        check_workspace(workspace, need, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = lib().attn_fwd_kv_outer(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                 lse.data_ptr(), B, H, N, d, MASK_CAUSAL if causal else MASK_NONE,
                                 float(scale), code, workspace.data_ptr(),
                                 workspace.numel() * workspace.element_size(), stream.cuda_stream)
    if st != 0:
        raise FaError(st, "attn_fwd_kv_outer")
    return out, lse


def attn_bwd(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None, *,
             dq=None, dk=None, dv=None, workspace=None, stream=None, window: int | None = None,
             block_mask=None):
    """Gradients (dq, dk, dv) of sum(o * dout) for o, lse = attn_fwd(q, k, v, causal, scale,
    window=window) (``window`` calls ``attn_bwd_window``).

    All tensors are contiguous device tensors; q, k, v, o, dout share one
    [B, H, N, d] shape and dtype (float16 or bfloat16), lse is float32 [B, H, N].
    v, o and dout may instead be [B, H, N, dv] (contiguous, no window or block
    mask), which calls ``attn_bwd_dv``.
    ``workspace`` (a uint8 device tensor) is allocated when not given.
    """
    import torch
    shape = q.shape
    d_v = v.shape[-1] if v.dim() == 4 else None
    vshape = shape[:3] + (d_v,)
    for t, want in ((k, shape), (v, vshape), (o, vshape), (dout, vshape)):
        if t.shape != want or t.dtype != q.dtype:
            raise ValueError("q, k must share one [B, H, N, d] shape, v, o, dout one [B, H, N, dv], "
                             "all one dtype")
    for t in (q, k, v, o, dout):
        if not t.is_cuda or t.stride(-1) != 1:
            raise ValueError("inputs must be device tensors with a contiguous last axis")
    if any(t.device != q.device for t in (k, v, o, dout)):
        raise ValueError("q, k, v, o and dout must be on one device")
    check_buffer(lse, "lse", tuple(shape[:3]), torch.float32, q.device)
    B, H, N, d = shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    code = _torch_dtype_code(q)
    for g, name, like in ((dq, "dq", q), (dk, "dk", k), (dv, "dv", v)):
        if g is not None:
            check_buffer(g, name, tuple(like.shape), like.dtype, q.device, contiguous=False)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = (bwd_block_sparse_workspace_bytes if block_mask is not None else bwd_workspace_bytes)(
        B, H, N, d, code)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    else:
        check_workspace(workspace, need, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    if d_v != d:
        if window is not None or block_mask is not None:
            raise ValueError("dv != d takes no window or block mask")
        if not all(t.is_contiguous() for t in (q, k, v, o, dout, dq, dk, dv)):
            raise ValueError("dv != d takes contiguous tensors")
        st = attn_bwd_dv_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                             lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d,
                             d_v, MASK_CAUSAL if causal else MASK_NONE, float(scale), code,
                             workspace.data_ptr(), ws_bytes, stream.cuda_stream)
        if st != 0:
            raise FaError(st, "attn_bwd_dv")
        return dq, dk, dv
    if block_mask is not None:
        _check_block_mask(block_mask, B, H, N)
        if window is not None or not all(t.is_contiguous() for t in (q, k, v, o, dout, dq, dk, dv)):
            raise ValueError("a block-sparse mask takes contiguous tensors and no window")
        st = attn_bwd_block_sparse_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                       dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                       dv.data_ptr(), B, H, N, d, block_mask.data_ptr(),
                                       block_mask.shape[0], block_mask.shape[1],
                                       MASK_CAUSAL if causal else MASK_NONE, float(scale), code,
                                       workspace.data_ptr(), ws_bytes, stream.cuda_stream)
        if st != 0:
            raise FaError(st, "attn_bwd_block_sparse")
        return dq, dk, dv
    if not all(t.is_contiguous() for t in (q, k, v, o, dout, dq, dk, dv)):
        # strided views: q, k, v, o, dout share one layout, dq, dk, dv another
        if window is not None:
            raise ValueError("a sliding window takes contiguous tensors")
        lay = _layout(q)
        if any(_layout(t) != lay for t in (k, v, o, dout)):
            raise ValueError("q, k, v, o and dout must share one layout")
        glay = _layout(dq)
        if any(_layout(t) != glay or t.stride(-1) != 1 for t in (dq, dk, dv)):
            raise ValueError("dq, dk and dv must share one layout with a contiguous last axis")
        st = attn_bwd_strided_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                  dv.data_ptr(), B, H, N, d, lay, glay,
                                  MASK_CAUSAL if causal else MASK_NONE, float(scale), code,
                                  workspace.data_ptr(), ws_bytes, stream.cuda_stream)
        if st != 0:
            raise FaError(st, "attn_bwd_strided")
        return dq, dk, dv
    if window is not None:
        if not causal:
            raise ValueError("a sliding window needs causal=True")
        st = lib().attn_bwd_window(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                   dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                   dv.data_ptr(), B, H, N, d, int(window), float(scale), code,
                                   workspace.data_ptr(), ws_bytes, stream.cuda_stream)
        if st != 0:
            raise FaError(st, "attn_bwd_window")
        return dq, dk, dv
    st = lib().attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                        lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d,
                        MASK_CAUSAL if causal else MASK_NONE, float(scale), code,
                        workspace.data_ptr(), ws_bytes, stream.cuda_stream)
    if st != 0:
        raise FaError(st, "attn_bwd")
    return dq, dk, dv


def attn_bwd_noalloc(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None, *,
                     dq, dk, dv, stream=None):
    """attn_bwd through the allocation-free entry point (``attn_bwd_noalloc``):
    the caller passes dq, dk and dv, and the backward's scratch is the
    library's fixed per-GPU array, so nothing is allocated here or in the
    library.  Contiguous [B, H, N, d] fp16 / bf16 tensors only; B * H * N at
    most ``noalloc_max_rows()``.  Calls that overlap on one GPU race on the
    shared scratch."""
    import torch
    shape = q.shape
    for t in (k, v, o, dout):
        if t.shape != shape or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k, v, o and dout must share one [B, H, N, d] shape, dtype and device")
    for t in (q, k, v, o, dout):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("inputs must be contiguous device tensors")
    check_buffer(lse, "lse", tuple(shape[:3]), torch.float32, q.device)
    for g, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        check_buffer(g, name, tuple(shape), q.dtype, q.device)
    B, H, N, d = shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = attn_bwd_noalloc_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                              dv.data_ptr(), B, H, N, d, MASK_CAUSAL if causal else MASK_NONE,
                              float(scale), _torch_dtype_code(q), stream.cuda_stream)
    if st != 0:
        raise FaError(st, "attn_bwd_noalloc")
    return dq, dk, dv
