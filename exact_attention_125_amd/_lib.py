"""ctypes binding of ``libfa.so`` (include/fa.h) — argument marshalling only.

Tensors are torch tensors on the GPU; torch provides device memory and the current HIP
stream, nothing else.  Every step of the computation runs in the library's HIP kernels.
If the library is missing this module raises on import: there is no fallback path.

Argument names follow the ``flash_attn_fn(q, k, v, dropout_p, softmax_scale, causal,
window_size, alibi_slopes)`` call listed in "告别OOM和训练慢：用Flash Attention加速你的PyTorch大模型
（含A100环境配置）" §4.2 (``fwd_kv`` / ``bwd_kv`` take dropout and ALiBi; ``fwd`` / ``bwd`` do
not) and the (batch, num_heads, seq_len, head_dim) layout of the SDPA call in "Flash Attention
3.7 核心原理与实战：加速Transformer模型训练与推理" §3.2.

Caller-supplied outputs (``out``, ``lse``, ``dq``, ``dk``, ``dv``) are checked against the
inputs before the call: the library sees only their addresses, so an output of the wrong
size, type or layout would make the kernels write outside it.
"""
from __future__ import annotations

import ctypes
import math
import os
import types

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_F16, FA_BF16 = 0, 1
STATUS_NAMES = {
    0: "FA_OK", 1: "FA_ERR_NULL_PTR", 2: "FA_ERR_BAD_SHAPE", 3: "FA_ERR_UNSUPPORTED_HEAD_DIM",
    4: "FA_ERR_BAD_DTYPE", 5: "FA_ERR_BAD_WINDOW", 6: "FA_ERR_MISALIGNED", 7: "FA_ERR_BAD_SCALE",
    8: "FA_ERR_WORKSPACE", 9: "FA_ERR_HIP", 10: "FA_ERR_ALIAS", 11: "FA_ERR_BAD_STAGES",
    12: "FA_ERR_BAD_DROPOUT", 13: "FA_ERR_TOO_LARGE",
}
NOALLOC_SCRATCH_BYTES = 16 << 20   # FA_NOALLOC_SCRATCH_BYTES
BWD_DELTA, BWD_DKDV, BWD_DQ, BWD_ALL = 1, 2, 4, 7

# Every function include/fa.h declares, with its ctypes signature.
_P, _I, _F, _S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_U64, _U32 = ctypes.c_ulonglong, ctypes.c_uint
SIGNATURES = {
    "fa_version": (_I, []),
    "fa_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _I, _P]),
    "fa_bwd_workspace_size": (_S, [_I, _I, _I, _I]),
    "fa_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _S,
                    _I, _I, _I, _I, _I, _F, _I, _I, _I, _P]),
    "fa_bwd_stages": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _S,
                           _I, _I, _I, _I, _I, _F, _I, _I, _I, ctypes.c_uint, _P]),
    "fa_fwd_varlen": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _I, _P]),
    "fa_bwd_varlen": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _S, _P,
                           _I, _I, _I, _I, _I, _F, _I, _I, _I, ctypes.c_uint, _P]),
    "fa_fwd_packed": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I, _P]),
    "fa_bwd_packed": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _S, _P,
                           _I, _I, _I, _I, _I, _I, _F, _I, _I, _I, ctypes.c_uint, _P]),
    "fa_fwd_kv_workspace_size": (_S, [_I, _I, _I, _I, _I]),
    "fa_fwd_kv": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I, _P, _P,
                       _P, _F, _U64, _U32, _P, _S, _P]),
    "fa_bwd_kv": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _S, _I, _I, _I, _I, _I, _I, _F,
                       _I, _I, _I, _P, _P, _P, _F, _U64, _U32, _P]),
    "fa_fwd_kv_fp8": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _F, _F, _I, _I,
                           _I, _P, _P, _S, _P]),
    "fa_fwd_fp8": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _F, _F, _F, _I, _I, _I, _P]),
    "fa_bwd_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P,
                            _I, _I, _I, _I, _I, _F, _I, _I, _I, _P]),
    "fa_status_string": (ctypes.c_char_p, [_I]),
    "fa_last_error_detail": (ctypes.c_char_p, []),
}


class FaStrides(ctypes.Structure):
    """``fa_strides``: element strides of one [B, H, rows, d] operand."""
    _fields_ = [("batch", ctypes.c_longlong), ("head", ctypes.c_longlong), ("row", ctypes.c_longlong)]


class FaError(RuntimeError):
    def __init__(self, status: int, lib):
        self.status = status
        msg = lib.fa_status_string(status).decode()
        detail = lib.fa_last_error_detail().decode()
        super().__init__(msg + (f" ({detail})" if detail else ""))


def load(path: str = LIB_PATH):
    """Load the library and attach signatures.  Raises if it is not built."""
    if not os.path.exists(path):
        raise ImportError(f"{path} not found: build it with `python exact_attention_125_amd/build.py`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = load()


def lib():
    return _lib


def _check(status: int):
    if status != 0:
        raise FaError(status, _lib)


def _dtype_code(t):
    import torch
    if t.dtype == torch.float16:
        return FA_F16
    if t.dtype == torch.bfloat16:
        return FA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: use float16 or bfloat16")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_tensors(*ts):
    ref = ts[0]
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must be on a GPU device")
        if t.device != ref.device:
            raise ValueError("tensors must be on the same device")
        if t.dtype != ref.dtype:
            raise ValueError("q, k, v (and o, dout) must share one dtype")
        if t.dim() != 4 or tuple(t.shape) != tuple(ref.shape):
            raise ValueError(f"expected [B, H, N, d] tensors of one shape, got {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous [B, H, N, d]")


def _check_out(t, like, name, dense=True):
    """An output buffer for a result shaped like ``like``: same device, dtype and shape, last
    dimension contiguous, no row shared between elements (no zero stride), and dense
    [B, H, N, d] when the entry point takes no strides (``dense``)."""
    if t.device != like.device:
        raise ValueError(f"{name} must be on {like.device}, got {t.device}")
    if t.dtype != like.dtype:
        raise ValueError(f"{name} must be {like.dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(like.shape):
        raise ValueError(f"{name} must have shape {tuple(like.shape)}, got {tuple(t.shape)}")
    if t.numel() == 0:
        return
    if t.stride(-1) != 1 or any(s == 0 for s, n in zip(t.stride(), t.shape) if n > 1):
        raise ValueError(f"{name} must have a contiguous last dimension and no shared rows")
    if dense and not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous [B, H, N, d] tensor")


def _check_lse(lse, q, name="lse"):
    """A float32 [B, H, N_q] contiguous tensor on q's device."""
    import torch
    B, H, n = q.shape[0], q.shape[1], q.shape[2]
    if lse.device != q.device or lse.dtype != torch.float32:
        raise ValueError(f"{name} must be a float32 tensor on {q.device}")
    if tuple(lse.shape) != (B, H, n) or not lse.is_contiguous():
        raise ValueError(f"{name} must be a contiguous [B, H, N_q] = {(B, H, n)} tensor")


def _resolve(q, softmax_scale, window_size):
    scale = 1.0 / math.sqrt(q.shape[-1]) if softmax_scale is None else float(softmax_scale)
    wl, wr = (int(window_size[0]), int(window_size[1]))
    return scale, wl, wr


def _check_workspace(ws, q):
    """A contiguous device buffer on q's device (its size is checked by the library)."""
    if ws.device != q.device or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {q.device}")


def _check_seqlens(seqlens, q):
    import torch
    if not seqlens.is_cuda or seqlens.device != q.device:
        raise ValueError("seqlens must be on the device of q")
    if seqlens.dtype != torch.int32 or seqlens.dim() != 1 or seqlens.shape[0] != q.shape[0]:
        raise ValueError("seqlens must be an int32 [B] tensor")
    if not seqlens.is_contiguous():
        raise ValueError("seqlens must be contiguous")


def fwd(q, k, v, softmax_scale=None, causal=False, window_size=(-1, -1), out=None, lse=None,
        return_lse=True, seqlens=None):
    """Forward pass.  Returns ``(o, lse)`` (``lse`` None when ``return_lse`` is False).
    ``seqlens`` (int32 [B] on the device) makes it a padded batch (``fa_fwd_varlen``)."""
    import torch
    _check_tensors(q, k, v)
    B, H, N, d = q.shape
    scale, wl, wr = _resolve(q, softmax_scale, window_size)
    if out is not None:
        _check_out(out, q, "out")
    o = torch.empty_like(q) if out is None else out
    if return_lse and lse is None:
        lse = torch.empty((B, H, N), device=q.device, dtype=torch.float32)
    if not return_lse:
        lse = None
    if lse is not None:
        _check_lse(lse, q)
    if seqlens is not None:
        _check_seqlens(seqlens, q)
        _check(_lib.fa_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(seqlens),
                                  B, H, N, d, _dtype_code(q), scale, int(bool(causal)), wl, wr,
                                  _stream(q.device)))
        return o, lse
    _check(_lib.fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                       _dtype_code(q), scale, int(bool(causal)), wl, wr, _stream(q.device)))
    return o, lse


def bwd(dout, q, k, v, o, lse, softmax_scale=None, causal=False, window_size=(-1, -1),
        dq=None, dk=None, dv=None, workspace=None, stages=BWD_ALL, seqlens=None):
    """Backward pass.  Returns ``(dq, dk, dv)``.  ``stages`` (a mask of BWD_DELTA, BWD_DKDV,
    BWD_DQ) runs a subset of the three stages; later stages need the earlier ones' results
    in the same ``workspace`` and outputs (BWD_DELTA with BWD_DQ in one call run as one
    kernel, before BWD_DKDV).  ``seqlens`` (int32 [B] on the device) makes it a
    padded batch (``fa_bwd_varlen``)."""
    import torch
    _check_tensors(q, k, v, o, dout)
    B, H, N, d = q.shape
    scale, wl, wr = _resolve(q, softmax_scale, window_size)
    _check_lse(lse, q)
    for g, like, name in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
        if g is not None:
            _check_out(g, like, name)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = _lib.fa_bwd_workspace_size(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), device=q.device, dtype=torch.uint8)
    _check_workspace(workspace, q)
    if seqlens is not None:
        _check_seqlens(seqlens, q)
        _check(_lib.fa_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                  _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _ptr(seqlens),
                                  B, H, N, d, _dtype_code(q), scale, int(bool(causal)), wl, wr,
                                  int(stages), _stream(q.device)))
        return dq, dk, dv
    _check(_lib.fa_bwd_stages(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                              _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                              workspace.numel() * workspace.element_size(),
                              B, H, N, d, _dtype_code(q), scale, int(bool(causal)), wl, wr,
                              int(stages), _stream(q.device)))
    return dq, dk, dv


def fwd_fp8(q, k, v, q_descale, k_descale, v_descale, softmax_scale=None, causal=False,
            window_size=(-1, -1), out_dtype=None, out=None, return_lse=True):
    """``fa_fwd_fp8``: attention over FP8 E4M3 q, k, v [B, H, N, d] (``torch.float8_e4m3fn`` or
    their ``uint8`` codes, contiguous, on one device), element value ``descale * value(code)``
    per tensor.  Returns ``(o, lse)``, ``o`` of ``out_dtype`` (bfloat16 by default, or the dtype
    of ``out``)."""
    import torch
    for t in (q, k, v):
        if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise ValueError("q, k, v must be float8_e4m3fn or uint8 (E4M3 codes)")
        if not t.is_cuda or t.device != q.device:
            raise ValueError("q, k, v must be on one GPU device")
        if t.dim() != 4 or tuple(t.shape) != tuple(q.shape) or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous [B, H, N, d] tensors of one shape")
    B, H, N, d = q.shape
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.bfloat16
    if out_dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("out_dtype must be float16 or bfloat16")
    like = types.SimpleNamespace(device=q.device, dtype=out_dtype, shape=(B, H, N, d))
    if out is not None:
        _check_out(out, like, "out")
    o = torch.empty((B, H, N, d), dtype=out_dtype, device=q.device) if out is None else out
    lse = torch.empty((B, H, N), device=q.device, dtype=torch.float32) if return_lse else None
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    wl, wr = (int(window_size[0]), int(window_size[1]))
    _check(_lib.fa_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                           FA_BF16 if out_dtype == torch.bfloat16 else FA_F16, scale,
                           float(q_descale), float(k_descale), float(v_descale),
                           int(bool(causal)), wl, wr, _stream(q.device)))
    return o, lse


def bwd_noalloc(dout, q, k, v, o, lse, dq, dk, dv, softmax_scale=None, causal=False,
                window_size=(-1, -1)):
    """``fa_bwd_noalloc``: ``bwd`` into caller-supplied ``dq``, ``dk``, ``dv`` with the per-query
    statistics in the library's static device scratch (no allocation by the library or by
    this wrapper).  Calls that overlap on one device race on that scratch."""
    _check_tensors(q, k, v, o, dout)
    B, H, N, d = q.shape
    scale, wl, wr = _resolve(q, softmax_scale, window_size)
    _check_lse(lse, q)
    for g, like, name in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
        _check_out(g, like, name)
    _check(_lib.fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                               _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, _dtype_code(q), scale,
                               int(bool(causal)), wl, wr, _stream(q.device)))
    return dq, dk, dv


def _check_packed(q, cu_seqlens, max_seqlen):
    """[H, total, d] operands and the offsets of a packed batch; returns (B, H, total, d)."""
    import torch
    if q.dim() != 3:
        raise ValueError("packed operands are [H, total, d] tensors")
    if (not cu_seqlens.is_cuda or cu_seqlens.device != q.device or cu_seqlens.dtype != torch.int32
            or cu_seqlens.dim() != 1 or cu_seqlens.shape[0] < 1 or not cu_seqlens.is_contiguous()):
        raise ValueError("cu_seqlens must be a contiguous int32 [B + 1] tensor on q's device")
    if int(max_seqlen) < 0:
        raise ValueError("max_seqlen must be >= 0")
    H, total, d = q.shape
    return cu_seqlens.shape[0] - 1, H, total, d


def fwd_packed(q, k, v, cu_seqlens, max_seqlen, softmax_scale=None, causal=False,
               window_size=(-1, -1), out=None, lse=None, return_lse=True):
    """``fa_fwd_packed``: q, k, v [H, total, d] holding every sequence's rows per head, sequence
    b at rows cu_seqlens[b] .. cu_seqlens[b+1]-1 (int32 [B + 1] on the device); ``max_seqlen``
    the longest sequence.  Returns ``(o, lse)``, ``lse`` [H, total] float32 (rows no sequence
    covers are left as allocated)."""
    import torch
    for t in (q, k, v):
        if not t.is_cuda or t.device != q.device or t.dtype != q.dtype:
            raise ValueError("q, k, v must share one GPU device and dtype")
        if tuple(t.shape) != tuple(q.shape) or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous [H, total, d] tensors of one shape")
    B, H, total, d = _check_packed(q, cu_seqlens, max_seqlen)
    scale, wl, wr = _resolve(q, softmax_scale, window_size)
    if out is not None:
        _check_out(out, q, "out")
    o = torch.empty_like(q) if out is None else out
    if return_lse and lse is None:
        lse = torch.empty((H, total), device=q.device, dtype=torch.float32)
    if not return_lse:
        lse = None
    if lse is not None and (lse.device != q.device or lse.dtype != torch.float32
                            or tuple(lse.shape) != (H, total) or not lse.is_contiguous()):
        raise ValueError(f"lse must be a contiguous float32 [H, total] = {(H, total)} tensor")
    _check(_lib.fa_fwd_packed(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens),
                              B, H, total, int(max_seqlen), d, _dtype_code(q), scale,
                              int(bool(causal)), wl, wr, _stream(q.device)))
    return o, lse


def bwd_packed(dout, q, k, v, o, lse, cu_seqlens, max_seqlen, softmax_scale=None, causal=False,
               window_size=(-1, -1), dq=None, dk=None, dv=None, workspace=None, stages=BWD_ALL):
    """``fa_bwd_packed``: gradients ``(dq, dk, dv)`` of ``fwd_packed`` ([H, total, d])."""
    import torch
    for t in (k, v, o, dout):
        if not t.is_cuda or t.device != q.device or t.dtype != q.dtype:
            raise ValueError("q, k, v, o, dout must share one GPU device and dtype")
        if tuple(t.shape) != tuple(q.shape) or not t.is_contiguous():
            raise ValueError("q, k, v, o, dout must be contiguous [H, total, d] tensors")
    B, H, total, d = _check_packed(q, cu_seqlens, max_seqlen)
    scale, wl, wr = _resolve(q, softmax_scale, window_size)
    if (lse.device != q.device or lse.dtype != torch.float32 or tuple(lse.shape) != (H, total)
            or not lse.is_contiguous()):
        raise ValueError(f"lse must be a contiguous float32 [H, total] = {(H, total)} tensor")
    for g, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        if g is not None:
            _check_out(g, q, name)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = _lib.fa_bwd_workspace_size(B, H, int(max_seqlen), d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), device=q.device, dtype=torch.uint8)
    _check_workspace(workspace, q)
    _check(_lib.fa_bwd_packed(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                              _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _ptr(cu_seqlens),
                              B, H, total, int(max_seqlen), d, _dtype_code(q), scale,
                              int(bool(causal)), wl, wr, int(stages), _stream(q.device)))
    return dq, dk, dv


def bwd_workspace_size(B, H, N, d) -> int:
    return int(_lib.fa_bwd_workspace_size(B, H, N, d))


def fwd_kv_workspace_size(B, H, n_q, n_k, d) -> int:
    return int(_lib.fa_fwd_kv_workspace_size(B, H, n_q, n_k, d))


def _check_kv_tensors(q, k, v):
    for t in (q, k, v):
        if not t.is_cuda or t.device != q.device:
            raise ValueError("q, k, v must be on one GPU device")
        if t.dtype != q.dtype:
            raise ValueError("q, k, v must share one dtype")
        if t.dim() != 4 or t.stride(-1) != 1:
            raise ValueError("expected [B, H, N, d] tensors with a contiguous last dimension")
    B, H, n_q, d = q.shape
    if tuple(k.shape) != (B, H, k.shape[2], d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"k, v must be [B, H, N_k, d] to match q {tuple(q.shape)}")


def _check_slopes(slopes, q):
    import torch
    if slopes is None:
        return
    if not slopes.is_cuda or slopes.device != q.device or slopes.dtype != torch.float32:
        raise ValueError("alibi_slopes must be a float32 tensor on the device of q")
    if slopes.dim() != 1 or slopes.shape[0] != q.shape[1] or not slopes.is_contiguous():
        raise ValueError("alibi_slopes must be a contiguous [heads] tensor")


def _check_blocks(block_mask, q, n_k):
    import torch
    if block_mask is None:
        return
    shape = (q.shape[1], -(-q.shape[2] // 64), -(-n_k // 64))
    if (not block_mask.is_cuda or block_mask.device != q.device
            or block_mask.dtype not in (torch.uint8, torch.bool)):
        raise ValueError("block_mask must be a uint8 or bool tensor on the device of q")
    if tuple(block_mask.shape) != shape or not block_mask.is_contiguous():
        raise ValueError(f"block_mask must be a contiguous [heads, ceil(N_q/64), ceil(N_k/64)] "
                         f"= {shape} tensor")


def _check_key_padding(key_padding_mask, q, n_k):
    import torch
    if key_padding_mask is None:
        return
    shape = (q.shape[0], n_k)
    if (not key_padding_mask.is_cuda or key_padding_mask.device != q.device
            or key_padding_mask.dtype not in (torch.uint8, torch.bool)):
        raise ValueError("key_padding_mask must be a uint8 or bool tensor on the device of q")
    if tuple(key_padding_mask.shape) != shape or not key_padding_mask.is_contiguous():
        raise ValueError(f"key_padding_mask must be a contiguous [batch, N_k] = {shape} tensor")


def fwd_kv(q, k, v, softmax_scale=None, causal=False, window_size=(-1, -1), out=None,
           return_lse=True, workspace=None, alibi_slopes=None, dropout_p=0.0, dropout_seed=0,
           dropout_offset=0, block_mask=None, key_padding_mask=None):
    """``fa_fwd_kv``: q [B, H, N_q, d] over k, v [B, H, N_k, d], the queries being the last N_q
    key positions.  Any strides with a contiguous last dimension (for example transposed
    views of [B, N, H, d] memory).  ``alibi_slopes``: float32 [H] on the device, or None.
    ``dropout_p`` / ``dropout_seed`` / ``dropout_offset``: attention dropout with masks from
    the library's Philox stream (the same three values go to ``bwd_kv``).  ``block_mask``:
    uint8 / bool [H, ceil(N_q/64), ceil(N_k/64)] on the device selecting 64 x 64 blocks.
    ``key_padding_mask``: uint8 / bool [B, N_k] on the device, True (nonzero) where a key is
    padding.  Returns ``(o, lse)``; ``o`` has the strides of ``q``."""
    import torch
    _check_kv_tensors(q, k, v)
    _check_slopes(alibi_slopes, q)
    _check_blocks(block_mask, q, k.shape[2])
    _check_key_padding(key_padding_mask, q, k.shape[2])
    B, H, n_q, d = q.shape
    n_k = k.shape[2]
    scale, wl, wr = _resolve(q, softmax_scale, window_size)
    if out is not None:
        _check_out(out, q, "out", dense=False)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, n_q), device=q.device, dtype=torch.float32) if return_lse else None
    st = (FaStrides * 4)(*(FaStrides(*t.stride()[:3]) for t in (q, k, v, o)))
    need = fwd_kv_workspace_size(B, H, n_q, n_k, d)
    if workspace is None and need > 0:
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    if workspace is not None:
        _check_workspace(workspace, q)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.fa_fwd_kv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), st, B, H, n_q, n_k, d,
                          _dtype_code(q), scale, int(bool(causal)), wl, wr, _ptr(alibi_slopes),
                          _ptr(block_mask), _ptr(key_padding_mask), float(dropout_p),
                          int(dropout_seed), int(dropout_offset), _ptr(workspace), ws_bytes,
                          _stream(q.device)))
    return o, lse


def fwd_kv_fp8(q, k, v, k_descale, v_descale, softmax_scale=None, causal=False,
               window_size=(-1, -1), out=None, return_lse=True, workspace=None,
               key_padding_mask=None):
    """``fa_fwd_kv_fp8``: a decode step (N_q <= 4) of q [B, H, N_q, d] (fp16 / bf16) over an
    FP8 E4M3 cache k, v [B, H, N_k, d] (``torch.float8_e4m3fn`` or its ``uint8`` codes), key
    element ``k_descale * value``, value element ``v_descale * value``.  Any strides with a
    contiguous last dimension.  ``key_padding_mask`` as in ``fwd_kv``.  Returns ``(o, lse)``;
    ``o`` has the strides of ``q``."""
    import torch
    for t in (k, v):
        if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise ValueError("k, v must be float8_e4m3fn or uint8 (E4M3 codes)")
        if not t.is_cuda or t.device != q.device or t.dim() != 4 or t.stride(-1) != 1:
            raise ValueError("k, v must be [B, H, N_k, d] on q's device, last dimension contiguous")
    if q.dtype not in (torch.float16, torch.bfloat16) or q.dim() != 4 or q.stride(-1) != 1:
        raise ValueError("q must be an fp16 / bf16 [B, H, N_q, d] tensor, last dimension contiguous")
    B, H, n_q, d = q.shape
    n_k = k.shape[2]
    if tuple(k.shape) != (B, H, n_k, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"k, v must be [B, H, N_k, d] to match q {tuple(q.shape)}")
    scale, wl, wr = _resolve(q, softmax_scale, window_size)
    if not q.is_cuda:
        raise ValueError("q must be on a GPU device")
    _check_key_padding(key_padding_mask, q, n_k)
    if out is not None:
        _check_out(out, q, "out", dense=False)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, n_q), device=q.device, dtype=torch.float32) if return_lse else None
    st = (FaStrides * 4)(*(FaStrides(*t.stride()[:3]) for t in (q, k, v, o)))
    need = fwd_kv_workspace_size(B, H, n_q, n_k, d)
    if workspace is None and need > 0:
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    if workspace is not None:
        _check_workspace(workspace, q)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.fa_fwd_kv_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), st, B, H, n_q, n_k,
                              d, _dtype_code(q), scale, float(k_descale), float(v_descale),
                              int(bool(causal)), wl, wr, _ptr(key_padding_mask),
                              _ptr(workspace), ws_bytes, _stream(q.device)))
    return o, lse


def bwd_kv(dout, q, k, v, o, lse, softmax_scale=None, causal=False, window_size=(-1, -1),
           dq=None, dk=None, dv=None, workspace=None, alibi_slopes=None, dropout_p=0.0,
           dropout_seed=0, dropout_offset=0, block_mask=None, key_padding_mask=None):
    """``fa_bwd_kv``: gradients ``(dq, dk, dv)`` of ``fwd_kv``.  Any strides with a contiguous
    last dimension; new gradients take the strides of q, k, v."""
    import torch
    _check_kv_tensors(q, k, v)
    _check_slopes(alibi_slopes, q)
    _check_blocks(block_mask, q, k.shape[2])
    _check_key_padding(key_padding_mask, q, k.shape[2])
    for t in (o, dout):
        if t.dtype != q.dtype or tuple(t.shape) != tuple(q.shape) or t.stride(-1) != 1:
            raise ValueError("o and dout must match q")
    B, H, n_q, d = q.shape
    n_k = k.shape[2]
    scale, wl, wr = _resolve(q, softmax_scale, window_size)
    _check_lse(lse, q)
    for g, like, name in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
        if g is not None:
            _check_out(g, like, name, dense=False)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for g, t in ((dk, k), (dv, v)):
        if any(st == 0 for st in g.stride()[:3]) and g.numel() > 0:
            raise ValueError("gradient outputs must not share rows (stride 0): pass dense ones")
    need = _lib.fa_bwd_workspace_size(B, H, n_q, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), device=q.device, dtype=torch.uint8)
    _check_workspace(workspace, q)
    st = (FaStrides * 8)(*(FaStrides(*t.stride()[:3]) for t in (q, k, v, o, dout, dq, dk, dv)))
    _check(_lib.fa_bwd_kv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                          _ptr(dk), _ptr(dv), st, _ptr(workspace),
                          workspace.numel() * workspace.element_size(), B, H, n_q, n_k, d,
                          _dtype_code(q), scale, int(bool(causal)), wl, wr, _ptr(alibi_slopes),
                          _ptr(block_mask), _ptr(key_padding_mask), float(dropout_p),
                          int(dropout_seed), int(dropout_offset), _stream(q.device)))
    return dq, dk, dv
