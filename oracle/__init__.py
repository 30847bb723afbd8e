"""Plain fp64 CPU oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
the GPU library and never imports it.

The arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP over heads or
rows); this module builds and loads it with ctypes and marshals numpy arrays.
What each function computes, with its source passages, is stated in the
header of ``oracle.c``: the three-step definition S = QK^T, P = softmax(S),
O = PV of the lab write-up (section 2.1), its analytic backward, the
online-softmax recurrence of section 3.2, and Philox-4x32-10 dropout bits.

Layout: tensors are float64 numpy arrays [tokens, H, d]; a fixed-length batch
[B, N, H, d] is passed reshaped to [B*N, H, d].  Sequence s covers tokens
``starts[s] .. starts[s] + lens[s] - 1``.  LSE is [tokens, H].
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int)
        u32p = ctypes.POINTER(ctypes.c_uint32)
        lib.oracle_rows_head.argtypes = [dp, dp, dp, dp, ctypes.c_long, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_double, ctypes.c_int, ctypes.c_int, ip, dp, dp, dp]
        lib.oracle_rows_head.restype = None
        lib.oracle_philox4x32_10.argtypes = [u32p, u32p, u32p]
        lib.oracle_philox4x32_10.restype = None
        lib.oracle_keep.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int]
        lib.oracle_keep.restype = ctypes.c_int
        lib.oracle_keep_mask.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.POINTER(ctypes.c_uint8)]
        lib.oracle_keep_mask.restype = None
        u8p = ctypes.POINTER(ctypes.c_uint8)
        common = [ctypes.c_int, ip, ip, ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_int,
                  ctypes.c_double, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int, ip,
                  u8p, ctypes.c_int, ctypes.c_int]
        lib.oracle_fwd.argtypes = [dp, dp, dp, dp, dp] + common
        lib.oracle_fwd.restype = None
        lib.oracle_bwd.argtypes = [dp, dp, dp, dp, dp, dp, dp] + common
        lib.oracle_bwd.restype = None
        lib.oracle_fwd_head_tiled.argtypes = [dp, dp, dp, ctypes.c_long, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_double, ctypes.c_int, ctypes.c_double,
                                              ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_int, ctypes.c_int, dp, dp,
                                              ctypes.c_long]
        lib.oracle_fwd_head_tiled.restype = None
        lib.oracle_decode.argtypes = [dp, dp, dp, dp, dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ip, ctypes.c_double, ctypes.c_int]
        lib.oracle_decode.restype = None
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _dptr(a: np.ndarray):
    assert a.dtype == np.float64 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _iptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int))


def dropout_threshold(p: float) -> int:
    """floor(p * 2^16) for the float32 value of p (an element is kept iff its
    16-bit Philox value is >= this threshold)."""
    return int(math.floor(float(np.float32(p)) * 65536.0))


def _seq_layout(tokens: int, N: int | None, lengths):
    if lengths is None:
        assert tokens % N == 0
        nseq = tokens // N
        starts = np.arange(nseq, dtype=np.int32) * N
        lens = np.full(nseq, N, dtype=np.int32)
    else:
        lens = np.ascontiguousarray(np.asarray(lengths, dtype=np.int32))
        starts = np.zeros(len(lens), dtype=np.int32)
        if len(lens) > 1:
            starts[1:] = np.cumsum(lens[:-1])
        assert int(lens.sum()) == tokens
    return starts, lens


def _sel(heads):
    if heads is None:
        return 0, None
    a = np.ascontiguousarray(np.asarray(heads, dtype=np.int32).reshape(-1, 2))
    return a.shape[0], a


def _prep(*xs):
    return [np.ascontiguousarray(x, dtype=np.float64) for x in xs]


def _mask(block_mask, block: int, nseq: int, H: int, lens):
    """(pointer, block, blocks per side) of an optional [nseq, H, nb, nb] block mask."""
    if block_mask is None:
        return None, 1, 0, None
    m = np.ascontiguousarray(np.asarray(block_mask, dtype=np.uint8))
    nb = -(-int(max(lens)) // block) if len(lens) else 0
    assert m.ndim == 4 and m.shape[0] == nseq and m.shape[1] == H and m.shape[2] == m.shape[3], m.shape
    assert m.shape[2] >= nb
    return m.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), int(block), int(m.shape[2]), m


def forward(q, k, v, *, scale: float, causal: bool, N: int | None = None, lengths=None,
            dropout_p: float = 0.0, seed: int = 0, heads=None, block_mask=None, block: int = 128):
    """O and LSE of attention.  q, k, v: float64 [tokens, H, d].

    Fixed length: pass N (sequence length; tokens = B*N).  Varlen: pass the
    list of sequence lengths.  ``heads`` = optional list of (sequence, head)
    pairs to compute; other entries of O and LSE are returned as NaN.
    Dropout keep bits depend on (seed, sequence index, head, row, col).
    ``block_mask`` = optional uint8 [sequences, H, nb, nb]: element (i, j) of
    a head is visible only if entry (i // block, j // block) is nonzero; rows
    with no visible key get O = 0 and LSE = -inf."""
    lib = _load()
    q, k, v = _prep(q, k, v)
    T, H, d = q.shape
    starts, lens = _seq_layout(T, N, lengths)
    nsel, sel = _sel(heads)
    mptr, blk, nb, _keep = _mask(block_mask, block, len(lens), H, lens)
    o = np.full_like(q, np.nan)
    lse = np.full((T, H), np.nan, dtype=np.float64)
    lib.oracle_fwd(_dptr(q), _dptr(k), _dptr(v), _dptr(o), _dptr(lse), len(lens), _iptr(starts),
                   _iptr(lens), H, d, float(scale), int(bool(causal)), float(np.float32(dropout_p)),
                   dropout_threshold(dropout_p) if dropout_p > 0 else 0, int(seed) & (2**64 - 1),
                   nsel, _iptr(sel), mptr, blk, nb)
    return o, lse


def backward(q, k, v, dout, *, scale: float, causal: bool, N: int | None = None, lengths=None,
             dropout_p: float = 0.0, seed: int = 0, heads=None, block_mask=None, block: int = 128):
    """dQ, dK, dV of L = sum(O * dout), with O = forward(q, k, v) (same
    optional block mask)."""
    lib = _load()
    q, k, v, dout = _prep(q, k, v, dout)
    T, H, d = q.shape
    starts, lens = _seq_layout(T, N, lengths)
    nsel, sel = _sel(heads)
    mptr, blk, nb, _keep = _mask(block_mask, block, len(lens), H, lens)
    dq = np.full_like(q, np.nan)
    dk = np.full_like(q, np.nan)
    dv = np.full_like(q, np.nan)
    lib.oracle_bwd(_dptr(q), _dptr(k), _dptr(v), _dptr(dout), _dptr(dq), _dptr(dk), _dptr(dv),
                   len(lens), _iptr(starts), _iptr(lens), H, d, float(scale), int(bool(causal)),
                   float(np.float32(dropout_p)), dropout_threshold(dropout_p) if dropout_p > 0 else 0,
                   int(seed) & (2**64 - 1), nsel, _iptr(sel), mptr, blk, nb)
    return dq, dk, dv


def forward_tiled_head(q, k, v, *, scale: float, causal: bool, Br: int, Bc: int,
                       dropout_p: float = 0.0, seed: int = 0, b: int = 0, h: int = 0):
    """Online-softmax recurrence (fp64) on one head; q, k, v: [L, d]."""
    lib = _load()
    q, k, v = _prep(q, k, v)
    L, d = q.shape
    o = np.zeros_like(q)
    lse = np.zeros(L, dtype=np.float64)
    lib.oracle_fwd_head_tiled(_dptr(q), _dptr(k), _dptr(v), d, L, d, float(scale), int(bool(causal)),
                              float(np.float32(dropout_p)),
                              dropout_threshold(dropout_p) if dropout_p > 0 else 0,
                              int(seed) & (2**64 - 1), b, h, Br, Bc, _dptr(o), _dptr(lse), 1)
    return o, lse


def decode(q, k_cache, v_cache, *, scale: float, causal: bool, seqlens_k=None):
    """KV-cache decode step: q [B, nq, H, d] against the first seqlens_k[b]
    tokens of k_cache, v_cache [B, nk_max, H, d] (all nk_max if None); the nq
    queries are the last nq positions of their sequence (causal: query t sees
    keys j <= L - nq + t).  Returns O [B, nq, H, d] and LSE [B, nq, H]."""
    lib = _load()
    q, k, v = _prep(q, k_cache, v_cache)
    B, nq, H, d = q.shape
    nk = k.shape[1]
    assert k.shape == (B, nk, H, d) and v.shape == k.shape
    lk = None if seqlens_k is None else np.ascontiguousarray(np.asarray(seqlens_k, dtype=np.int32))
    o = np.zeros_like(q)
    lse = np.zeros((B, nq, H), dtype=np.float64)
    lib.oracle_decode(_dptr(q), _dptr(k), _dptr(v), _dptr(o), _dptr(lse), B, H, nq, nk, d, _iptr(lk),
                      float(scale), int(bool(causal)))
    return o, lse


def decode_paged(q, k_pages, v_pages, block_table, *, scale: float, causal: bool, seqlens_k=None):
    """The decode step over a paged cache: k_pages, v_pages [num_pages, P,
    H, d] hold pages of P tokens, and cache position j of sequence b is token
    j % P of page block_table[b][j // P].  Gathers each sequence's valid
    positions (all max_pages * P if seqlens_k is None) into the contiguous
    [B, nk_max, H, d] layout and runs decode() on it; table entries past a
    sequence's length are not used."""
    kp = np.asarray(k_pages, dtype=np.float64)
    vp = np.asarray(v_pages, dtype=np.float64)
    table = np.asarray(block_table, dtype=np.int64)
    B, max_pages = table.shape
    P = kp.shape[1]
    nk = max_pages * P
    lens = np.full(B, nk, dtype=np.int64) if seqlens_k is None else np.clip(np.asarray(seqlens_k), 0, nk)
    k = np.zeros((B, nk) + kp.shape[2:])
    v = np.zeros_like(k)
    for b in range(B):
        pos = np.arange(lens[b])
        page = table[b, pos // P]
        if len(page) and (page.min() < 0 or page.max() >= kp.shape[0]):
            raise ValueError("block table entry outside the page pool")
        k[b, :lens[b]] = kp[page, pos % P]
        v[b, :lens[b]] = vp[page, pos % P]
    return decode(q, k, v, scale=scale, causal=causal, seqlens_k=lens.astype(np.int32))


def rows_head(q, k, v, dout=None, *, scale: float, causal: bool, rows):
    """O, LSE (and dQ if dout is given) of the listed query rows of one head,
    without forming P: q, k, v, dout float64 [L, d] (any row stride).
    Returns o [n, d], lse [n], dq [n, d] or None.  No dropout, no mask."""
    lib = _load()
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    L, d = q.shape
    ld = q.strides[0] // 8
    for t in (k, v) + ((dout,) if dout is not None else ()):
        t = np.asarray(t)
        if t.shape != (L, d) or t.strides != q.strides or t.dtype != np.float64:
            raise ValueError("q, k, v, dout must share shape and strides")
    if q.strides[1] != 8:
        raise ValueError("rows must be contiguous in the head dimension")
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
    if rows.size and (rows.min() < 0 or rows.max() >= L):
        raise ValueError("row out of range")
    n = rows.size
    o = np.zeros((n, d))
    lse = np.zeros(n)
    dq = np.zeros((n, d)) if dout is not None else None
    dptr = ctypes.POINTER(ctypes.c_double)
    lib.oracle_rows_head(q.ctypes.data_as(dptr), k.ctypes.data_as(dptr), v.ctypes.data_as(dptr),
                         dout.ctypes.data_as(dptr) if dout is not None else None, ld, L, d, float(scale),
                         int(bool(causal)), n, rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int)), _dptr(o),
                         _dptr(lse), _dptr(dq) if dq is not None else None)
    return o, lse, dq


def philox4x32_10(counter, key):
    """Raw Philox-4x32-10 block: four uint32 words for a 4-word counter and 2-word key."""
    lib = _load()
    c = (ctypes.c_uint32 * 4)(*[int(x) & 0xFFFFFFFF for x in counter])
    kk = (ctypes.c_uint32 * 2)(*[int(x) & 0xFFFFFFFF for x in key])
    out = (ctypes.c_uint32 * 4)()
    lib.oracle_philox4x32_10(c, kk, out)
    return [int(x) for x in out]


def keep(seed: int, thresh: int, b: int, h: int, i: int, j: int) -> bool:
    """Keep bit of one element for an explicit threshold (kept iff word >= thresh)."""
    return bool(_load().oracle_keep(int(seed) & (2**64 - 1), int(thresh), b, h, i, j))


def keep_mask(seed: int, dropout_p: float, b: int, h: int, L: int) -> np.ndarray:
    """Dropout keep mask (uint8, 1 = kept) of one head, [L, L] (rows = queries)."""
    lib = _load()
    m = np.zeros((L, L), dtype=np.uint8)
    lib.oracle_keep_mask(int(seed) & (2**64 - 1), dropout_threshold(dropout_p), b, h, L,
                         m.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)))
    return m


def max_threads() -> int:
    return int(_load().oracle_max_threads())
