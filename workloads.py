"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers; it holds none of the attention
arithmetic, so both the oracle-side tests and the GPU path can use it.

Recipe (every workload): a CPU ``torch.Generator`` seeded with the
workload's seed draws, in this order, [the varlen sequence lengths], q, k, v,
dO as float32 standard normals, each rounded once (round to nearest even) to
the workload's dtype.  The long-sequence workload then multiplies the
rounded K by 4 (exact in fp16 and bf16).  The packed-QKV workload draws q, k
and v together as one [B, N, 3, H, d] tensor and
uses views into it.  Varlen lengths are discrete uniform on [128, 4096],
both ends included.

Shapes follow the pages: the [batch, seq, heads, head_dim] layout of the lab
write-up (section 4.2), its experiment shapes (section 5: batch 4, 8 heads,
head_dim 128, seqlen 4096 and 8192), the packed-QKV example of the
tiemojia.cn article (B=2, N=2048, H=12, d=64, fp16) and the varlen and
dropout arguments of the FlashAttention library overview.  The pages train
language models on real text; no dataset or weights are used here, the
normal draws stand in for activations.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import torch

DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int                  # batch (fixed length) or number of sequences (varlen)
    H: int
    N: int                  # sequence length (varlen: maximum length)
    d: int
    dtype: str              # "f16" | "bf16"
    causal: bool
    packed: bool = False    # q, k, v are views into one [B, N, 3, H, d] tensor
    dropout_p: float = 0.0
    k_mult: float = 1.0
    varlen: bool = False
    len_range: tuple = (128, 4096)
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


# The five workloads, by name; the seed of each is fixed (1001 .. 1005).
WORKLOADS = {w.name: w for w in (
    Workload("tiny_B1_H2_N128_d64_f16", 1, 2, 128, 64, "f16", False, seed=1001),
    Workload("packed_qkv_B2_H12_N2048_d64_f16", 2, 12, 2048, 64, "f16", False, packed=True, seed=1002),
    Workload("causal_B4_H8_N4096_d128_bf16", 4, 8, 4096, 128, "bf16", True, seed=1003),
    Workload("long_causal_B1_H16_N8192_d128_bf16_kx4", 1, 16, 8192, 128, "bf16", True, k_mult=4.0,
             seed=1004),
    Workload("varlen16_H32_d128_bf16_causal_p0.1", 16, 32, 4096, 128, "bf16", True, dropout_p=0.1,
             varlen=True, seed=1005),
)}

# the workload the benchmark times: causal B=4, H=8, N=4096, d=128, bf16
HEADLINE = "causal_B4_H8_N4096_d128_bf16"


@dataclasses.dataclass
class Inputs:
    wl: Workload
    q: torch.Tensor         # [B, N, H, d] or [T, H, d] (may be a strided view)
    k: torch.Tensor
    v: torch.Tensor
    do: torch.Tensor        # contiguous, same logical shape as q
    lengths: Optional[list]
    cu_seqlens: Optional[torch.Tensor]   # int32 [nseq + 1] (varlen only)
    qkv: Optional[torch.Tensor] = None   # the packed tensor (packed only)

    @property
    def tokens(self) -> int:
        return int(self.q.shape[0] * self.q.shape[1]) if not self.wl.varlen else int(self.q.shape[0])


def make_inputs(wl: Workload, seed: Optional[int] = None, with_do: bool = True) -> Inputs:
    g = torch.Generator().manual_seed(wl.seed if seed is None else seed)
    dt = DTYPES[wl.dtype]
    lengths = None
    cu = None
    if wl.varlen:
        lo, hi = wl.len_range
        lengths = [int(x) for x in torch.randint(lo, hi + 1, (wl.B,), generator=g)]
        cu = torch.zeros(wl.B + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
        shape = (sum(lengths), wl.H, wl.d)
    else:
        shape = (wl.B, wl.N, wl.H, wl.d)
    qkv = None
    if wl.packed:
        assert not wl.varlen
        qkv = torch.randn(wl.B, wl.N, 3, wl.H, wl.d, generator=g).to(dt)
        q, k, v = qkv.unbind(2)
        if wl.k_mult != 1.0:
            qkv[:, :, 1] *= wl.k_mult
    else:
        q = torch.randn(*shape, generator=g).to(dt)
        k = torch.randn(*shape, generator=g).to(dt)
        v = torch.randn(*shape, generator=g).to(dt)
        if wl.k_mult != 1.0:
            k = k * wl.k_mult
    do = torch.randn(*shape, generator=g).to(dt) if with_do else None
    return Inputs(wl, q, k, v, do, lengths, cu, qkv)


def custom(B: int, H: int, N: int, d: int, dtype: str = "bf16", causal: bool = False, *,
           lengths: Optional[Sequence[int]] = None, dropout_p: float = 0.0, packed: bool = False,
           k_mult: float = 1.0, seed: int = 7) -> Inputs:
    """Same recipe at an arbitrary shape (edge and ragged cases)."""
    varlen = lengths is not None
    wl = Workload(f"custom_B{B}_H{H}_N{N}_d{d}_{dtype}", len(lengths) if varlen else B, H,
                  max(lengths) if varlen and len(lengths) else N, d, dtype, causal, packed=packed,
                  dropout_p=dropout_p, k_mult=k_mult, varlen=varlen, seed=seed)
    if varlen:
        g = torch.Generator().manual_seed(seed)
        dt = DTYPES[dtype]
        T = int(sum(lengths))
        q = torch.randn(T, H, d, generator=g).to(dt)
        k = torch.randn(T, H, d, generator=g).to(dt)
        v = torch.randn(T, H, d, generator=g).to(dt)
        if k_mult != 1.0:
            k = k * k_mult
        do = torch.randn(T, H, d, generator=g).to(dt)
        cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
        if len(lengths):
            cu[1:] = torch.cumsum(torch.tensor(list(lengths), dtype=torch.int64), 0).to(torch.int32)
        return Inputs(wl, q, k, v, do, list(lengths), cu)
    return make_inputs(wl)


def ragged_lengths(n: int, lo: int, hi: int, seed: int) -> list:
    """n sequence lengths, discrete uniform on [lo, hi] (numpy generator)."""
    import numpy as np
    return [int(x) for x in np.random.default_rng(seed).integers(lo, hi + 1, n)]


def as_f64_tokens(x: torch.Tensor):
    """[B, N, H, d] or [T, H, d] (any strides) -> contiguous float64 numpy [tokens, H, d]."""
    x = x.detach().to("cpu")
    if x.dim() == 4:
        x = x.reshape(x.shape[0] * x.shape[1], x.shape[2], x.shape[3])
    return x.to(torch.float64).contiguous().numpy()


def block_mask(B: int, H: int, N: int, density: float, seed: int, *, block: int = 128,
               keep_diagonal: bool = True) -> torch.Tensor:
    """Random uint8 block mask [B, H, nb, nb] (nb = ceil(N / block)) for
    block-sparse attention: each entry is 1 with probability ``density``
    (a seeded CPU torch.Generator draws one uniform per entry, row-major);
    with ``keep_diagonal`` the diagonal blocks are forced to 1, so that no
    query row is left without keys."""
    nb = -(-N // block)
    g = torch.Generator().manual_seed(seed)
    m = (torch.rand(B, H, nb, nb, generator=g) < density).to(torch.uint8)
    if keep_diagonal:
        idx = torch.arange(nb)
        m[:, :, idx, idx] = 1
    return m


# ------------------------------------------------------------ KV-cache decode

@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int
    H: int
    nq: int                  # new query tokens per sequence
    nk: int                  # cache capacity per sequence
    d: int
    dtype: str
    causal: bool
    ragged: bool = False     # valid cache lengths ~ U{1..nk} per sequence (else all nk)
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


# The lab write-up's inference case (section 6.1): one new token per sequence
# against a long cache, at its section-5 head shape (32 heads of 128 would be
# the LLaMA-7B layout of the how-to; 8192 cached tokens).
DECODE_WORKLOADS = {w.name: w for w in (
    DecodeWorkload("decode_B8_H32_nq1_Nk8192_d128_bf16", 8, 32, 1, 8192, 128, "bf16", True, seed=1101),
    DecodeWorkload("decode_B16_H8_nq4_Nk4096_d64_f16_ragged", 16, 8, 4, 4096, 64, "f16", True, ragged=True,
                   seed=1102),
)}
DECODE_HEADLINE = "decode_B8_H32_nq1_Nk8192_d128_bf16"


@dataclasses.dataclass
class DecodeInputs:
    wl: DecodeWorkload
    q: torch.Tensor          # [B, nq, H, d]
    k: torch.Tensor          # [B, nk, H, d]
    v: torch.Tensor
    seqlens: Optional[torch.Tensor]  # int32 [B] or None


def make_decode_inputs(wl: DecodeWorkload, lengths: Optional[Sequence[int]] = None) -> DecodeInputs:
    """Same recipe as make_inputs: [lengths], q, k_cache, v_cache as fp32
    normals rounded once to the dtype.  Ragged lengths ~ U{1..nk} unless given."""
    g = torch.Generator().manual_seed(wl.seed)
    dt = DTYPES[wl.dtype]
    seq = None
    if lengths is not None:
        seq = torch.tensor(list(lengths), dtype=torch.int32)
    elif wl.ragged:
        seq = torch.randint(1, wl.nk + 1, (wl.B,), generator=g).to(torch.int32)
    q = torch.randn(wl.B, wl.nq, wl.H, wl.d, generator=g).to(dt)
    k = torch.randn(wl.B, wl.nk, wl.H, wl.d, generator=g).to(dt)
    v = torch.randn(wl.B, wl.nk, wl.H, wl.d, generator=g).to(dt)
    return DecodeInputs(wl, q, k, v, seq)


def paged_cache(k: torch.Tensor, v: torch.Tensor, page_size: int, seed: int,
                lengths: Optional[Sequence[int]] = None, spare: int = 2):
    """The caches k, v [B, nk, H, d] laid out as a paged cache: pools
    [num_pages, page_size, H, d] whose pages sit in a seeded random order,
    with `spare` unused pages, and a table [B, ceil(nk / page_size)] (int32)
    naming the pool page of each page of each sequence.  Unused pages and the
    padding rows of a last partial page hold NaN; table entries of pages at or
    past a sequence's length are -1 (lengths = all nk if None).  Layout only:
    the cache contents are those of k and v."""
    B, nk, H, d = k.shape
    max_pages = -(-nk // page_size)
    n = B * max_pages + spare
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(seed))
    kp = torch.full((n, page_size, H, d), float("nan"), dtype=k.dtype)
    vp = torch.full_like(kp, float("nan"))
    table = torch.full((B, max_pages), -1, dtype=torch.int32)
    for b in range(B):
        L = nk if lengths is None else int(lengths[b])
        for p in range(max_pages):
            lo, hi = p * page_size, min((p + 1) * page_size, nk)
            slot = int(perm[b * max_pages + p])
            kp[slot, :hi - lo] = k[b, lo:hi]
            vp[slot, :hi - lo] = v[b, lo:hi]
            if lo < L:
                table[b, p] = slot
    return kp, vp, table
