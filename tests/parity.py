"""Helpers shared by the GPU parity tests: run the HIP path, run the oracle
on the same (rounded) inputs, and compare against the stated tolerances.

Tolerances (attention parity bars): O max abs <= 1e-2 (fp16) / 2e-2 (bf16);
LSE max abs <= 1e-3; dQ, dK, dV relative Frobenius error <= 1e-2; dropout
masks bit-exact.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from workloads import Inputs, as_f64_tokens

O_TOL = {"f16": 1e-2, "bf16": 2e-2}
LSE_TOL = 1e-3
GRAD_TOL = 1e-2
# Per-head gradient bar: 1e-2 like the whole tensor, except on heads of
# fewer than SHORT_HEAD tokens, where reading O back in 16 bits for
# D = dO . O alone can move a head's dQ or dK by more than 1e-2 of its norm
# (pinned in test_tolerance_floor.py); those heads are held to TINY_HEAD_BAR.
SHORT_HEAD = 16
TINY_HEAD_BAR = 4e-2


def head_bar(rows: int) -> float:
    return GRAD_TOL if rows >= SHORT_HEAD else TINY_HEAD_BAR


def to_gpu(x: Inputs):
    """Device copies; packed q/k/v stay views into one device qkv tensor."""
    dev = torch.device("cuda")
    if x.qkv is not None:
        qkv = x.qkv.to(dev)
        q, k, v = qkv.unbind(2)
    else:
        q, k, v = (t.to(dev) for t in (x.q, x.k, x.v))
    do = x.do.to(dev) if x.do is not None else None
    cu = x.cu_seqlens.to(dev) if x.cu_seqlens is not None else None
    return q, k, v, do, cu


def seq_kwargs(x: Inputs):
    if x.wl.varlen:
        return dict(lengths=x.lengths)
    return dict(N=x.wl.N)


def select_heads(x: Inputs, n: int | None, seed: int = 0):
    """All (sequence, head) pairs, or n of them chosen by a fixed seed (always
    including the first and last sequence and head)."""
    nseq = len(x.lengths) if x.wl.varlen else x.wl.B
    pairs = [(s, h) for s in range(nseq) for h in range(x.wl.H)]
    if n is None or n >= len(pairs):
        return None, pairs
    rng = np.random.default_rng(seed)
    pick = {pairs[0], pairs[-1]}
    while len(pick) < n:
        pick.add(pairs[int(rng.integers(len(pairs)))])
    pick = sorted(pick)
    return pick, pick


def token_rows(x: Inputs, s: int):
    if x.wl.varlen:
        st = int(sum(x.lengths[:s]))
        return slice(st, st + x.lengths[s])
    return slice(s * x.wl.N, (s + 1) * x.wl.N)


def oracle_forward(x: Inputs, heads):
    return oracle.forward(as_f64_tokens(x.q), as_f64_tokens(x.k), as_f64_tokens(x.v), scale=x.wl.scale,
                          causal=x.wl.causal, dropout_p=x.wl.dropout_p, seed=x.wl.seed, heads=heads,
                          **seq_kwargs(x))


def oracle_backward(x: Inputs, heads):
    return oracle.backward(as_f64_tokens(x.q), as_f64_tokens(x.k), as_f64_tokens(x.v), as_f64_tokens(x.do),
                           scale=x.wl.scale, causal=x.wl.causal, dropout_p=x.wl.dropout_p, seed=x.wl.seed,
                           heads=heads, **seq_kwargs(x))


def tokens_f64(t: torch.Tensor) -> np.ndarray:
    return as_f64_tokens(t.detach().float().cpu())


def compare_forward(x: Inputs, o_gpu, lse_gpu, pairs, o_ref, lse_ref):
    """Max abs errors of O and LSE over the given (sequence, head) pairs."""
    o = tokens_f64(o_gpu)
    lse = lse_gpu.detach().cpu().double().numpy().reshape(o.shape[0], -1)
    eo = el = 0.0
    for s, h in pairs:
        r = token_rows(x, s)
        eo = max(eo, float(np.abs(o[r, h] - o_ref[r, h]).max(initial=0.0)))
        el = max(el, float(np.abs(lse[r, h] - lse_ref[r, h]).max(initial=0.0)))
    return eo, el


def rel_fro(x: Inputs, g_gpu, g_ref, pairs, floor_ref=None):
    """(||G - G*||_F / ||G*||_F over the given heads, worst single head, heads
    over their per-head bar).

    Both errors use the reference's own norm as the denominator.  Only where
    a reference gradient vanishes exactly (dQ and dK of a head whose rows
    each see a single key, e.g. one token) would the ratio be undefined;
    there, and only there, the denominator is ||floor_ref||_F of the same
    head (the dV reference, the scale of the gradients), so that rounding
    noise is measured against that scale.  The third result lists
    (sequence, head, rows, error) of every head above head_bar(rows)."""
    g = tokens_f64(g_gpu) if isinstance(g_gpu, torch.Tensor) else g_gpu
    num = den = fnum = fden = 0.0
    worst = 0.0
    over = []
    for s, h in pairs:
        r = token_rows(x, s)
        a, b = g[r, h], g_ref[r, h]
        n, d = float(((a - b) ** 2).sum()), float((b ** 2).sum())
        num += n
        den += d
        if d == 0.0 and floor_ref is not None:
            d = float((floor_ref[r, h] ** 2).sum())
            fnum += n
            fden += d
        e = (n / d) ** 0.5 if d > 0 else (0.0 if n == 0 else float("inf"))
        worst = max(worst, e)
        if e > head_bar(r.stop - r.start):
            over.append((s, h, r.stop - r.start, e))
    if den > 0:
        total = (num / den) ** 0.5
    elif fden > 0:
        total = (fnum / fden) ** 0.5
    else:
        total = 0.0 if num == 0 else float("inf")
    return total, worst, over
