"""Fused exact attention for AMD Instinct MI355X (gfx950).

Thin Python binding over libfa.so (include/fa.h): it checks tensors,
allocates outputs with torch and passes raw device pointers and the current
HIP stream to the C ABI. Every step of the computation runs in the HIP
kernels; there is no fallback path.

    o, lse = forward(q, k, v, causal=False, scale=None)
    dq, dk, dv = backward(q, k, v, o, lse, do, causal=False, scale=None)
    o = attention(q, k, v, causal=False, scale=None)   # autograd-aware
    o, lse = forward_varlen(q, k, v, cu_seqlens, max_seqlen, causal=False, scale=None)

Tensors are contiguous [B, H, N, D] of float32, float16 or bfloat16 on the
GPU (k and v may have H_kv heads, H_kv dividing H: query head h reads K/V
head h // (H // H_kv)); the default scale is 1/sqrt(D).
"""

import math

import torch

from . import _lib
from ._lib import FaError  # noqa: F401

_DTYPES = {torch.float32: _lib.FA_FP32, torch.float16: _lib.FA_FP16,
           torch.bfloat16: _lib.FA_BF16}


def _stream_handle(t):
    """hipStream_t of torch's current stream on t's device (None = default)."""
    return torch.cuda.current_stream(t.device).cuda_stream or None


def _check_qkv(q, k, v):
    """Checks q [B, H, N, D] and k, v [B, H_kv, N, D] with H_kv dividing H;
    returns H_kv."""
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or k.shape[0] != q.shape[0] or \
            k.shape[2:] != q.shape[2:] or k.shape[1] < 1 or q.shape[1] % k.shape[1] != 0:
        raise ValueError(f"need q [B, H, N, D] and k, v [B, H_kv, N, D] with H_kv dividing H, "
                         f"got {tuple(q.shape)}, {tuple(k.shape)}, {tuple(v.shape)}")
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError(f"dtype must be float32, float16 or bfloat16 (all equal), got "
                        f"{q.dtype}, {k.dtype}, {v.dtype}")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")
    return k.shape[1]


def _check_buffer(name, t, shape, dtype, device):
    """A tensor handed to a kernel as a raw pointer: it must be contiguous,
    of the given shape and dtype, on `device` (the inputs' GPU). Anything
    else would let a kernel read or write outside the tensor."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_workspace(name, t, need, device):
    """A caller's workspace: uint8, contiguous, on `device`, at least `need`
    bytes (the library also checks the byte count it is given)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device != device or t.dtype != torch.uint8 or t.dim() != 1 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous 1-D uint8 tensor on {device}")
    if t.numel() < need:
        raise ValueError(f"{name} holds {t.numel()} bytes, {need} needed")


def default_scale(D):
    return 1.0 / math.sqrt(D)


def forward(q, k, v, causal=False, scale=None, out=None, lse=None, dropout_p=0.0, seed=0,
            offset=0):
    """Fused forward. Returns (o, lse): o like q, lse fp32 [B, H, N] (natural log).

    dropout_p > 0 drops attention probabilities with counter-based bits keyed by
    (seed, offset); the same arguments to `backward` regenerate them. k and v
    may have fewer heads than q (grouped K/V heads).
    """
    H_kv = _check_qkv(q, k, v)
    B, H, N, D = q.shape
    if scale is None:
        scale = default_scale(D)
    if out is None:
        out = torch.empty_like(q)
    _check_buffer("out", out, q.shape, q.dtype, q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_buffer("lse", lse, (B, H, N), torch.float32, q.device)
    lib = _lib.load()
    with torch.cuda.device(q.device):
        if H_kv != H:
            st = lib.fa_forward_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                    lse.data_ptr(), B, H, H_kv, N, D, float(scale),
                                    int(bool(causal)), _DTYPES[q.dtype], float(dropout_p),
                                    int(seed), int(offset), _stream_handle(q))
            _lib.check("fa_forward_gqa", st)
        elif dropout_p:
            st = lib.fa_forward_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                        lse.data_ptr(), B, H, N, D, float(scale),
                                        int(bool(causal)), _DTYPES[q.dtype], float(dropout_p),
                                        int(seed), int(offset), _stream_handle(q))
            _lib.check("fa_forward_dropout", st)
        else:
            st = lib.fa_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                lse.data_ptr(), B, H, N, D, float(scale), int(bool(causal)),
                                _DTYPES[q.dtype], _stream_handle(q))
            _lib.check("fa_forward", st)
    return out, lse


def forward_varlen(q, k, v, cu_seqlens, max_seqlen, causal=False, scale=None, out=None,
                   lse=None, dropout_p=0.0, seed=0, offset=0):
    """Forward over a packed batch of variable-length sequences with grouped K/V heads.

    q: [total, H, D]; k, v: [total, H_kv, D] (H_kv divides H); cu_seqlens: int32
    [batch + 1] on q's device, sequence b being tokens cu_seqlens[b] .. cu_seqlens[b+1]-1.
    max_seqlen sizes the grid and must be at least the longest sequence: the
    offsets stay on the device (no synchronisation), so a longer sequence is
    not detected; it is cut to its first max_seqlen tokens and its later rows
    are not written.
    dropout_p > 0 drops probabilities as `forward` does, with the bits of a
    dense batch of the same sequences.
    Returns (o [total, H, D], lse fp32 [H, total]).
    """
    if q.dim() != 3 or k.dim() != 3 or k.shape != v.shape or q.shape[0] != k.shape[0] \
            or q.shape[2] != k.shape[2]:
        raise ValueError(f"need q [total, H, D] and k, v [total, H_kv, D], got "
                         f"{tuple(q.shape)}, {tuple(k.shape)}, {tuple(v.shape)}")
    if q.dtype not in (torch.float16, torch.bfloat16) or k.dtype != q.dtype or \
            v.dtype != q.dtype:
        raise TypeError("dtype must be float16 or bfloat16 (all equal)")
    for name, t in (("q", q), ("k", k), ("v", v), ("cu_seqlens", cu_seqlens)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be int32 [batch + 1]")
    if not (q.device == k.device == v.device == cu_seqlens.device):
        raise ValueError("q, k, v and cu_seqlens must be on one device")
    total, H, D = q.shape
    if scale is None:
        scale = default_scale(D)
    if out is None:
        out = torch.empty_like(q)
    _check_buffer("out", out, q.shape, q.dtype, q.device)
    if lse is None:
        lse = torch.empty((H, total), dtype=torch.float32, device=q.device)
    _check_buffer("lse", lse, (H, total), torch.float32, q.device)
    lib = _lib.load()
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
            cu_seqlens.data_ptr(), cu_seqlens.numel() - 1, int(max_seqlen), total, H, k.shape[1],
            D, float(scale), int(bool(causal)), _DTYPES[q.dtype])
    with torch.cuda.device(q.device):
        if dropout_p:
            st = lib.fa_forward_varlen_dropout(*args, float(dropout_p), int(seed), int(offset),
                                               _stream_handle(q))
            _lib.check("fa_forward_varlen_dropout", st)
        else:
            st = lib.fa_forward_varlen(*args, _stream_handle(q))
            _lib.check("fa_forward_varlen", st)
    return out, lse


def decode_workspace_bytes(batch, s_q, H, H_kv, max_seqlen_k, D):
    return int(_lib.load().fa_decode_workspace_bytes(batch, s_q, H, H_kv, max_seqlen_k, D))


def decode(q, k_cache, v_cache, cache_seqlens, max_seqlen_k=None, scale=None, out=None, lse=None,
           workspace=None):
    """Attention of s_q new tokens per sequence against a key/value cache.

    q: [B, s_q, H, D]; k_cache, v_cache: [B, cap, H_kv, D]; cache_seqlens: int32 [B]
    on q's device (cached tokens per sequence, the new ones included as the
    last s_q). New token t sees keys 0 .. L_b - s_q + t. max_seqlen_k bounds the
    lengths (default: cap). Returns (o [B, s_q, H, D], lse fp32 [B, H, s_q]).
    """
    if q.dim() != 4 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape or \
            q.shape[0] != k_cache.shape[0] or q.shape[3] != k_cache.shape[3]:
        raise ValueError(f"need q [B, s_q, H, D] and caches [B, cap, H_kv, D], got "
                         f"{tuple(q.shape)}, {tuple(k_cache.shape)}, {tuple(v_cache.shape)}")
    if q.dtype not in (torch.float16, torch.bfloat16) or k_cache.dtype != q.dtype or \
            v_cache.dtype != q.dtype:
        raise TypeError("dtype must be float16 or bfloat16 (all equal)")
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                    ("cache_seqlens", cache_seqlens)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    B, s_q, H, D = q.shape
    cap, H_kv = k_cache.shape[1], k_cache.shape[2]
    if cache_seqlens.dtype != torch.int32 or cache_seqlens.shape != (B,):
        raise ValueError("cache_seqlens must be int32 [B]")
    if not (q.device == k_cache.device == v_cache.device == cache_seqlens.device):
        raise ValueError("q, the caches and cache_seqlens must be on one device")
    if max_seqlen_k is None:
        max_seqlen_k = cap
    if scale is None:
        scale = default_scale(D)
    if out is None:
        out = torch.empty_like(q)
    _check_buffer("out", out, q.shape, q.dtype, q.device)
    if lse is None:
        lse = torch.empty((B, H, s_q), dtype=torch.float32, device=q.device)
    _check_buffer("lse", lse, (B, H, s_q), torch.float32, q.device)
    need = decode_workspace_bytes(B, s_q, H, H_kv, max_seqlen_k, D)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _check_workspace("workspace", workspace, need, q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() if workspace is not None else 0
    lib = _lib.load()
    with torch.cuda.device(q.device):
        st = lib.fa_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                           cache_seqlens.data_ptr(), out.data_ptr(), lse.data_ptr(), ws_ptr,
                           ws_len, B, s_q, cap, int(max_seqlen_k), H, H_kv, D, float(scale),
                           _DTYPES[q.dtype], _stream_handle(q))
    _lib.check("fa_decode", st)
    return out, lse


def backward_workspace_bytes(B, H, N, D):
    return int(_lib.load().fa_backward_workspace_bytes(B, H, N, D))


def backward(q, k, v, o, lse, do, causal=False, scale=None, workspace=None, dropout_p=0.0,
             seed=0, offset=0, out=None):
    """Backward from the forward's o and lse (and its dropout arguments).
    Returns (dq, dk, dv), dk and dv shaped like k (with grouped K/V heads, the
    sums over each K/V head's query heads); `out` may give the three output
    tensors."""
    H_kv = _check_qkv(q, k, v)
    for name, t in (("o", o), ("do", do)):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must match q (shape, dtype, device, contiguous)")
    B, H, N, D = q.shape
    _check_buffer("lse", lse, (B, H, N), torch.float32, q.device)
    for name, t in (("o", o), ("do", do)):
        _check_buffer(name, t, q.shape, q.dtype, q.device)
    if scale is None:
        scale = default_scale(D)
    need = backward_workspace_bytes(B, H, N, D)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check_workspace("workspace", workspace, need, q.device)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = out
        for name, t, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
            _check_buffer(name, t, like.shape, q.dtype, q.device)
    lib = _lib.load()
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
            lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
            workspace.numel())
    args = ptrs + (B, H, N, D, float(scale), int(bool(causal)), _DTYPES[q.dtype])
    with torch.cuda.device(q.device):
        if H_kv != H:
            st = lib.fa_backward_gqa(*ptrs, B, H, H_kv, N, D, float(scale), int(bool(causal)),
                                     _DTYPES[q.dtype], float(dropout_p), int(seed), int(offset),
                                     _stream_handle(q))
            _lib.check("fa_backward_gqa", st)
        elif dropout_p:
            st = lib.fa_backward_dropout(*args, float(dropout_p), int(seed), int(offset),
                                         _stream_handle(q))
            _lib.check("fa_backward_dropout", st)
        else:
            st = lib.fa_backward(*args, _stream_handle(q))
            _lib.check("fa_backward", st)
    return dq, dk, dv


def backward_varlen(q, k, v, o, lse, do, cu_seqlens, max_seqlen, causal=False, scale=None,
                    workspace=None, out=None, dropout_p=0.0, seed=0, offset=0):
    """Backward of forward_varlen from its o and lse [H, total] (and its
    dropout arguments). Returns
    (dq [total, H, D], dk, dv [total, H_kv, D]); dk and dv sum over the query
    heads that share each K/V head. `out` may give the three output tensors
    (rows of tokens outside every sequence are left as they are)."""
    if q.dim() != 3 or k.dim() != 3 or k.shape != v.shape or q.shape[0] != k.shape[0] \
            or q.shape[2] != k.shape[2]:
        raise ValueError(f"need q [total, H, D] and k, v [total, H_kv, D], got "
                         f"{tuple(q.shape)}, {tuple(k.shape)}, {tuple(v.shape)}")
    if q.dtype not in (torch.float16, torch.bfloat16) or k.dtype != q.dtype or \
            v.dtype != q.dtype:
        raise TypeError("dtype must be float16 or bfloat16 (all equal)")
    for name, t in (("o", o), ("do", do)):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError(f"{name} must match q (shape, dtype)")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do), ("lse", lse),
                    ("cu_seqlens", cu_seqlens)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    total, H, D = q.shape
    _check_buffer("lse", lse, (H, total), torch.float32, q.device)
    for name, t in (("k", k), ("v", v), ("o", o), ("do", do), ("cu_seqlens", cu_seqlens)):
        if t.device != q.device:
            raise ValueError(f"{name} must be on {q.device}")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be int32 [batch + 1]")
    if scale is None:
        scale = default_scale(D)
    need = backward_workspace_bytes(1, H, total, D)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check_workspace("workspace", workspace, need, q.device)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = out
        for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
            _check_buffer(name, t, ref.shape, ref.dtype, q.device)
    lib = _lib.load()
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
            lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), cu_seqlens.data_ptr(),
            workspace.data_ptr(), workspace.numel(), cu_seqlens.numel() - 1, int(max_seqlen),
            total, H, k.shape[1], D, float(scale), int(bool(causal)), _DTYPES[q.dtype])
    with torch.cuda.device(q.device):
        if dropout_p:
            st = lib.fa_backward_varlen_dropout(*args, float(dropout_p), int(seed), int(offset),
                                                _stream_handle(q))
            _lib.check("fa_backward_varlen_dropout", st)
        else:
            st = lib.fa_backward_varlen(*args, _stream_handle(q))
            _lib.check("fa_backward_varlen", st)
    return dq, dk, dv


class _FlashAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, causal, scale, dropout_p, seed, offset):
        o, lse = forward(q, k, v, causal, scale, dropout_p=dropout_p, seed=seed, offset=offset)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.causal, ctx.scale = causal, scale
        ctx.dropout = (dropout_p, seed, offset)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        p, seed, offset = ctx.dropout
        dq, dk, dv = backward(q, k, v, o, lse, do.contiguous(), ctx.causal, ctx.scale,
                              dropout_p=p, seed=seed, offset=offset)
        return dq, dk, dv, None, None, None, None, None


def attention(q, k, v, causal=False, scale=None, dropout_p=0.0, seed=0, offset=0):
    """Autograd-aware fused attention (O only), with optional dropout."""
    if scale is None:
        scale = default_scale(q.shape[-1])
    return _FlashAttention.apply(q, k, v, causal, scale, dropout_p, seed, offset)


class _FlashAttentionVarlen(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, cu_seqlens, max_seqlen, causal, scale, dropout_p, seed, offset):
        o, lse = forward_varlen(q, k, v, cu_seqlens, max_seqlen, causal, scale,
                                dropout_p=dropout_p, seed=seed, offset=offset)
        ctx.save_for_backward(q, k, v, o, lse, cu_seqlens)
        ctx.max_seqlen, ctx.causal, ctx.scale = max_seqlen, causal, scale
        ctx.dropout = (dropout_p, seed, offset)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse, cu = ctx.saved_tensors
        p, seed, offset = ctx.dropout
        dq, dk, dv = backward_varlen(q, k, v, o, lse, do.contiguous(), cu, ctx.max_seqlen,
                                     ctx.causal, ctx.scale, dropout_p=p, seed=seed,
                                     offset=offset)
        return dq, dk, dv, None, None, None, None, None, None, None


def attention_varlen(q, k, v, cu_seqlens, max_seqlen, causal=False, scale=None, dropout_p=0.0,
                     seed=0, offset=0):
    """Autograd-aware fused attention over a packed variable-length batch with
    grouped K/V heads (O only), with optional dropout."""
    if scale is None:
        scale = default_scale(q.shape[-1])
    return _FlashAttentionVarlen.apply(q, k, v, cu_seqlens, max_seqlen, causal, scale, dropout_p,
                                       seed, offset)
