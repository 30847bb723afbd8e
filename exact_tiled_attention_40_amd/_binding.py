"""ctypes marshalling for libfa.so (see include/fa.h for the contract).

Tensors are torch tensors on the GPU; torch only provides device memory and
the current stream.  Shapes: fixed length q, k, v are [B, N, H, d] (any
token stride, unit stride inside a token, e.g. views into a packed
[B, N, 3, H, d] tensor); varlen q, k, v are [total, H, d] with int32
cu_seqlens on the device.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libfa.so")

FA_DTYPE_F16 = 0
FA_DTYPE_BF16 = 1
FA_MASK_BLOCK = 128       # rows and columns of one block-mask entry
FA_MASK_MAX_N = 65536     # longest sequence the block-sparse calls accept
FA_DECODE_MAX_Q = 8       # new query tokens per sequence in one decode step
FA_NOALLOC_MAX_ROWS = 1 << 22  # B*N*H limit of fa_backward_noalloc
_DTYPES = {torch.float16: FA_DTYPE_F16, torch.bfloat16: FA_DTYPE_BF16}


class FAError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"fa error {code}: {msg}")
        self.code = code


def library_path() -> str:
    return _LIB_PATH


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with `python exact_tiled_attention_40_amd/build.py`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i, f, i64, u64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_int64, ctypes.c_uint64
    lib.fa_forward.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, f, u64, vp, i, i64]
    lib.fa_forward.restype = i
    lib.fa_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, f, u64, vp, i, i64,
                                vp, ctypes.c_size_t]
    lib.fa_backward.restype = i
    lib.fa_backward_noalloc.argtypes = lib.fa_backward.argtypes[:-2]
    lib.fa_backward_noalloc.restype = i
    lib.fa_backward_stage.argtypes = [i] + lib.fa_backward.argtypes
    lib.fa_backward_stage.restype = i
    lib.fa_backward_workspace_size.argtypes = [i, i, i, i]
    lib.fa_backward_workspace_size.restype = ctypes.c_size_t
    lib.fa_forward_block_sparse.argtypes = lib.fa_forward.argtypes + [vp]
    lib.fa_forward_block_sparse.restype = i
    lib.fa_backward_block_sparse.argtypes = lib.fa_backward.argtypes + [vp]
    lib.fa_backward_block_sparse.restype = i
    lib.fa_backward_block_sparse_stage.argtypes = [i] + lib.fa_backward_block_sparse.argtypes
    lib.fa_backward_block_sparse_stage.restype = i
    lib.fa_dropout_bits_size.argtypes = [i, i, i]
    lib.fa_dropout_bits_size.restype = ctypes.c_size_t
    lib.fa_forward_keep.argtypes = lib.fa_forward.argtypes + [vp, ctypes.c_size_t]
    lib.fa_forward_keep.restype = i
    lib.fa_backward_keep.argtypes = lib.fa_backward.argtypes + [vp, ctypes.c_size_t]
    lib.fa_backward_keep.restype = i
    lib.fa_backward_keep_stage.argtypes = [i] + lib.fa_backward_keep.argtypes
    lib.fa_backward_keep_stage.restype = i
    lib.fa_decode_workspace_size.argtypes = [i, i, i, i, i]
    lib.fa_decode_workspace_size.restype = ctypes.c_size_t
    lib.fa_decode.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, i, vp, ctypes.c_size_t]
    lib.fa_decode.restype = i
    lib.fa_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp, i, vp, ctypes.c_size_t]
    lib.fa_decode_paged.restype = i
    lib.fa_dropout_mask.argtypes = [vp, i, i, i, f, u64, vp]
    lib.fa_dropout_mask.restype = i
    lib.fa_strerror.argtypes = [i]
    lib.fa_strerror.restype = ctypes.c_char_p
    return lib


_lib = _load()


def fa_strerror(code: int) -> str:
    return _lib.fa_strerror(int(code)).decode()


def _check(code: int):
    if code != 0:
        raise FAError(code, fa_strerror(code))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _geometry(q, cu_seqlens, max_seqlen):
    """(B, N, H, d, ld) of a q/k/v tensor."""
    if cu_seqlens is None:
        if q.dim() != 4:
            raise ValueError("fixed-length q/k/v must be [B, N, H, d]")
        B, N, H, d = q.shape
        if q.stride(3) != 1 or q.stride(2) != d:
            raise ValueError("head dim and heads must be contiguous inside a token")
        if q.stride(0) != N * q.stride(1):
            raise ValueError("tokens of consecutive batches must be evenly spaced")
        return B, N, H, d, q.stride(1)
    if q.dim() != 3:
        raise ValueError("varlen q/k/v must be [total, H, d]")
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda or cu_seqlens.dim() != 1 \
            or not cu_seqlens.is_contiguous() or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be a contiguous 1-d int32 device tensor of nseq + 1 prefix sums")
    if max_seqlen is None:
        raise ValueError("varlen needs max_seqlen")
    _, H, d = q.shape
    if q.stride(2) != 1 or q.stride(1) != d:
        raise ValueError("head dim and heads must be contiguous inside a token")
    return cu_seqlens.numel() - 1, int(max_seqlen), H, d, q.stride(0)


def _same_geometry(ref, *ts):
    for t in ts:
        if t.shape != ref.shape or t.stride() != ref.stride() or t.dtype != ref.dtype or t.device != ref.device:
            raise ValueError("q, k, v (and dq, dk, dv) must share shape, strides, dtype and device")


def _check_like(name, t, shape, dtype, device):
    """t must be a contiguous tensor of the given shape, dtype and device."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != device:
        raise ValueError(f"{name} must be {dtype} {tuple(shape)} on {device}, got {t.dtype} {tuple(t.shape)} "
                         f"on {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _block_mask(block_mask, B, H, N, device):
    nb = -(-N // FA_MASK_BLOCK)
    if block_mask.dtype != torch.uint8 or block_mask.device != device or not block_mask.is_contiguous():
        raise ValueError("block_mask must be a contiguous uint8 tensor on q's device")
    if tuple(block_mask.shape) != (B, H, nb, nb):
        raise ValueError(f"block_mask must be [B, H, nb, nb] = {(B, H, nb, nb)}")
    return _ptr(block_mask)


def fa_forward(q, k, v, *, scale=None, causal=False, cu_seqlens=None, max_seqlen=None, dropout_p=0.0, seed=0,
               out=None, lse=None, stream=None, block_mask=None):
    """Returns (o, lse).  o is contiguous with q's logical shape; lse is float32
    [B, N, H] (fixed length) or [total, H] (varlen).  With ``block_mask``
    (uint8 [B, H, nb, nb], nb = ceil(N / FA_MASK_BLOCK)) this calls
    fa_forward_block_sparse."""
    _same_geometry(q, k, v)
    if q.dtype not in _DTYPES:
        raise FAError(3, fa_strerror(3))
    B, N, H, d, ld = _geometry(q, cu_seqlens, max_seqlen)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    _check_like("out", out, q.shape, q.dtype, q.device)
    _check_like("lse", lse, q.shape[:-1], torch.float32, q.device)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d, float(scale), int(bool(causal)),
            _ptr(cu_seqlens), float(dropout_p), int(seed) & (2**64 - 1), _stream(stream), _DTYPES[q.dtype], ld)
    if block_mask is None:
        _check(_lib.fa_forward(*args))
    else:
        _check(_lib.fa_forward_block_sparse(*args, _block_mask(block_mask, B, H, N, q.device)))
    return out, lse


def fa_dropout_bits_size(B: int, N: int, H: int) -> int:
    """Bytes of the keep-bit buffer of fa_forward_keep / fa_backward_keep (0
    when N exceeds FA_MASK_MAX_N)."""
    return int(_lib.fa_dropout_bits_size(B, N, H))


def _keep_bits(keep_bits, B, N, H, device):
    if keep_bits is None:
        return None, 0
    if keep_bits.device != device or not keep_bits.is_contiguous():
        raise ValueError("keep_bits must be a contiguous tensor on q's device")
    return _ptr(keep_bits), keep_bits.numel() * keep_bits.element_size()


def fa_forward_keep(q, k, v, *, keep_bits, scale=None, causal=False, cu_seqlens=None, max_seqlen=None,
                    dropout_p=0.0, seed=0, out=None, lse=None, stream=None):
    """fa_forward that also stores its dropout decisions into ``keep_bits``
    (a device buffer of fa_dropout_bits_size(B, N, H) bytes, e.g. uint8 or
    int32; unused, and may be None, when dropout_p == 0).  Returns (o, lse)."""
    _same_geometry(q, k, v)
    if q.dtype not in _DTYPES:
        raise FAError(3, fa_strerror(3))
    B, N, H, d, ld = _geometry(q, cu_seqlens, max_seqlen)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    _check_like("out", out, q.shape, q.dtype, q.device)
    _check_like("lse", lse, q.shape[:-1], torch.float32, q.device)
    kb, kb_bytes = _keep_bits(keep_bits, B, N, H, q.device)
    _check(_lib.fa_forward_keep(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d, float(scale),
                                int(bool(causal)), _ptr(cu_seqlens), float(dropout_p), int(seed) & (2**64 - 1),
                                _stream(stream), _DTYPES[q.dtype], ld, kb, kb_bytes))
    return out, lse


def fa_backward_workspace_size(B: int, N: int, H: int, d: int) -> int:
    return int(_lib.fa_backward_workspace_size(B, N, H, d))


def fa_backward(q, k, v, o, lse, dout, *, scale=None, causal=False, cu_seqlens=None, max_seqlen=None,
                dropout_p=0.0, seed=0, dq=None, dk=None, dv=None, workspace=None, stream=None, block_mask=None):
    """Returns (dq, dk, dv).  Freshly allocated gradients are contiguous; pass
    dq/dk/dv views (e.g. into a packed [B, N, 3, H, d] buffer) with q's
    strides to write in place.  With ``block_mask`` this calls
    fa_backward_block_sparse (same mask as the forward)."""
    return _backward(None, q, k, v, o, lse, dout, scale=scale, causal=causal, cu_seqlens=cu_seqlens,
                     max_seqlen=max_seqlen, dropout_p=dropout_p, seed=seed, dq=dq, dk=dk, dv=dv,
                     workspace=workspace, stream=stream, block_mask=block_mask)


def fa_backward_stage(stage, q, k, v, o, lse, dout, *, scale=None, causal=False, cu_seqlens=None,
                      max_seqlen=None, dropout_p=0.0, seed=0, dq=None, dk=None, dv=None, workspace=None,
                      stream=None, block_mask=None):
    """One backward stage (0: D and dQ, 1: dK and dV); the caller passes the
    same dq/dk/dv and workspace to both, stage 0 first.  With ``block_mask``
    this calls fa_backward_block_sparse_stage."""
    if dq is None or dk is None or dv is None or workspace is None:
        raise ValueError("fa_backward_stage needs explicit dq, dk, dv and workspace")
    return _backward(int(stage), q, k, v, o, lse, dout, scale=scale, causal=causal, cu_seqlens=cu_seqlens,
                     max_seqlen=max_seqlen, dropout_p=dropout_p, seed=seed, dq=dq, dk=dk, dv=dv,
                     workspace=workspace, stream=stream, block_mask=block_mask)


def fa_backward_keep(q, k, v, o, lse, dout, *, keep_bits, scale=None, causal=False, cu_seqlens=None,
                     max_seqlen=None, dropout_p=0.0, seed=0, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """fa_backward reading the dropout decisions fa_forward_keep stored in
    ``keep_bits`` (same shapes, lengths, dropout_p and seed)."""
    return _backward(None, q, k, v, o, lse, dout, scale=scale, causal=causal, cu_seqlens=cu_seqlens,
                     max_seqlen=max_seqlen, dropout_p=dropout_p, seed=seed, dq=dq, dk=dk, dv=dv,
                     workspace=workspace, stream=stream, keep_bits=keep_bits, keep=True)


def fa_backward_keep_stage(stage, q, k, v, o, lse, dout, *, keep_bits, scale=None, causal=False, cu_seqlens=None,
                           max_seqlen=None, dropout_p=0.0, seed=0, dq=None, dk=None, dv=None, workspace=None,
                           stream=None):
    """One stage of fa_backward_keep (0: D and dQ, 1: dK and dV)."""
    if dq is None or dk is None or dv is None or workspace is None:
        raise ValueError("fa_backward_keep_stage needs explicit dq, dk, dv and workspace")
    return _backward(int(stage), q, k, v, o, lse, dout, scale=scale, causal=causal, cu_seqlens=cu_seqlens,
                     max_seqlen=max_seqlen, dropout_p=dropout_p, seed=seed, dq=dq, dk=dk, dv=dv,
                     workspace=workspace, stream=stream, keep_bits=keep_bits, keep=True)


def _backward(stage, q, k, v, o, lse, dout, *, scale, causal, cu_seqlens, max_seqlen, dropout_p, seed, dq, dk,
              dv, workspace, stream, block_mask=None, keep_bits=None, keep=False):
    _same_geometry(q, k, v)
    if q.dtype not in _DTYPES:
        raise FAError(3, fa_strerror(3))
    B, N, H, d, ld = _geometry(q, cu_seqlens, max_seqlen)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check_like("o", o, q.shape, q.dtype, q.device)
    _check_like("dout", dout, q.shape, q.dtype, q.device)
    _check_like("lse", lse, q.shape[:-1], torch.float32, q.device)
    if dq is None and dk is None and dv is None:
        if ld != H * d:
            raise ValueError("pass dq/dk/dv explicitly for strided q/k/v")
        dq, dk, dv = (torch.empty(q.shape, dtype=q.dtype, device=q.device) for _ in range(3))
    _same_geometry(q, dq, dk, dv)
    need = fa_backward_workspace_size(B, N, H, d)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    elif workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d,
            float(scale), int(bool(causal)), _ptr(cu_seqlens), float(dropout_p), int(seed) & (2**64 - 1),
            _stream(stream), _DTYPES[q.dtype], ld, _ptr(workspace), workspace.numel() * workspace.element_size())
    if keep:
        kb, kb_bytes = _keep_bits(keep_bits, B, N, H, q.device)
        if stage is None:
            _check(_lib.fa_backward_keep(*args, kb, kb_bytes))
        else:
            _check(_lib.fa_backward_keep_stage(stage, *args, kb, kb_bytes))
    elif block_mask is not None:
        m = _block_mask(block_mask, B, H, N, q.device)
        if stage is None:
            _check(_lib.fa_backward_block_sparse(*args, m))
        else:
            _check(_lib.fa_backward_block_sparse_stage(stage, *args, m))
    elif stage is None:
        _check(_lib.fa_backward(*args))
    else:
        _check(_lib.fa_backward_stage(stage, *args))
    return dq, dk, dv


def fa_backward_noalloc(q, k, v, o, lse, dout, *, dq, dk, dv, scale=None, causal=False, cu_seqlens=None,
                        max_seqlen=None, dropout_p=0.0, seed=0, stream=None):
    """fa_backward without a workspace: the library's fixed per-GPU scratch
    holds the backward's row arrays (B*N*H <= FA_NOALLOC_MAX_ROWS), so
    neither this call nor the library allocates; the caller passes dq, dk,
    dv.  Calls that overlap on one GPU race."""
    _same_geometry(q, k, v)
    if q.dtype not in _DTYPES:
        raise FAError(3, fa_strerror(3))
    B, N, H, d, ld = _geometry(q, cu_seqlens, max_seqlen)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check_like("o", o, q.shape, q.dtype, q.device)
    _check_like("dout", dout, q.shape, q.dtype, q.device)
    _check_like("lse", lse, q.shape[:-1], torch.float32, q.device)
    _same_geometry(q, dq, dk, dv)
    _check(_lib.fa_backward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                                    _ptr(dv), B, H, N, d, float(scale), int(bool(causal)), _ptr(cu_seqlens),
                                    float(dropout_p), int(seed) & (2**64 - 1), _stream(stream), _DTYPES[q.dtype], ld))
    return dq, dk, dv


def fa_dropout_mask(b: int, h: int, N: int, dropout_p: float, seed: int, *, out=None, device="cuda",
                    stream=None):
    """uint8 [N, N] keep mask (1 = kept) of head (b, h) as the kernels draw it."""
    if out is None:
        out = torch.empty((N, N), dtype=torch.uint8, device=device)
    _check(_lib.fa_dropout_mask(_ptr(out), b, h, N, float(dropout_p), int(seed) & (2**64 - 1), _stream(stream)))
    return out


def fa_decode_workspace_size(B: int, H: int, nq: int, nk_max: int, d: int) -> int:
    return int(_lib.fa_decode_workspace_size(B, H, nq, nk_max, d))


def fa_decode(q, k_cache, v_cache, *, seqlens_k=None, scale=None, causal=False, out=None, lse=None,
              workspace=None, stream=None):
    """One KV-cache decode step.  q [B, nq, H, d]; k_cache, v_cache
    [B, nk_max, H, d] (contiguous); seqlens_k optional int32 [B] on the
    device.  Returns (o [B, nq, H, d], lse float32 [B, nq, H])."""
    if q.dtype not in _DTYPES or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise FAError(3, fa_strerror(3))
    for t in (q, k_cache, v_cache):
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError("q, k_cache and v_cache must be contiguous 4-d tensors")
    B, nq, H, d = q.shape
    nk = k_cache.shape[1]
    if tuple(k_cache.shape) != (B, nk, H, d) or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache, v_cache must be [B, nk_max, H, d] with q's B, H, d")
    if seqlens_k is not None and (seqlens_k.dtype != torch.int32 or not seqlens_k.is_cuda or seqlens_k.numel() != B):
        raise ValueError("seqlens_k must be an int32 device tensor of B entries")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, nq, H), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(max(1, fa_decode_workspace_size(B, H, nq, nk, d)), dtype=torch.uint8,
                                device=q.device)
    _check(_lib.fa_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens_k), _ptr(out), _ptr(lse), B, H, nq,
                          nk, d, float(scale), int(bool(causal)), _stream(stream), _DTYPES[q.dtype], _ptr(workspace),
                          workspace.numel() * workspace.element_size()))
    return out, lse


def fa_decode_paged(q, k_pages, v_pages, block_table, *, seqlens_k=None, scale=None, causal=False, out=None,
                    lse=None, workspace=None, stream=None):
    """One KV-cache decode step over a paged cache.  q [B, nq, H, d];
    k_pages, v_pages [num_pages, page_size, H, d] (contiguous, page_size a
    power of two); block_table int32 [B, max_pages] on the device (cache
    position j of sequence b is token j % page_size of page
    block_table[b, j // page_size]); seqlens_k optional int32 [B] on the
    device.  Returns (o [B, nq, H, d], lse float32 [B, nq, H])."""
    if q.dtype not in _DTYPES or k_pages.dtype != q.dtype or v_pages.dtype != q.dtype:
        raise FAError(3, fa_strerror(3))
    for t in (q, k_pages, v_pages):
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError("q, k_pages and v_pages must be contiguous 4-d tensors")
    B, nq, H, d = q.shape
    num_pages, page_size = k_pages.shape[:2]
    if tuple(k_pages.shape) != (num_pages, page_size, H, d) or v_pages.shape != k_pages.shape:
        raise ValueError("k_pages, v_pages must be [num_pages, page_size, H, d] with q's H, d")
    if (block_table.dtype != torch.int32 or not block_table.is_cuda or block_table.dim() != 2
            or block_table.shape[0] != B or not block_table.is_contiguous()):
        raise ValueError("block_table must be a contiguous int32 device tensor [B, max_pages]")
    max_pages = block_table.shape[1]
    if seqlens_k is not None and (seqlens_k.dtype != torch.int32 or not seqlens_k.is_cuda or seqlens_k.numel() != B):
        raise ValueError("seqlens_k must be an int32 device tensor of B entries")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, nq, H), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(max(1, fa_decode_workspace_size(B, H, nq, max_pages * page_size, d)),
                                dtype=torch.uint8, device=q.device)
    _check(_lib.fa_decode_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(seqlens_k), _ptr(out),
                                _ptr(lse), B, H, nq, num_pages, page_size, max_pages, d, float(scale),
                                int(bool(causal)), _stream(stream), _DTYPES[q.dtype], _ptr(workspace),
                                workspace.numel() * workspace.element_size()))
    return out, lse
