"""Dropout keep bits recovered bit for bit through the fused kernels (needs
an MI355X).

With Q = 0 every visible score is 0, so P is uniform, 1/n_i over the n_i
keys query i sees (n_i = i + 1 causal, L otherwise).

Forward: with K = 0 and one-hot V rows (v_j = e_{j-o} for o <= j < o + d,
else 0), O[i][c] = keep(i, o + c) / (n_i (1 - p)) for a visible key o + c,
so O[i][c] != 0 exactly when the forward kernel kept element (i, o + c).

Key-side backward: with one-hot dO rows (dO_i = e_{i-o} for o <= i < o + d),
dV_j = sum_i Z_ij dO_i gives dV_j[c] = keep(o + c, j) / (n_{o+c} (1 - p)), so
the key-side kernel's bits are read off dV the same way.

Query-side backward: with one-hot K rows (k_j = e_{j-o}), every V row and
every dO row e_0, dP_ij = dO_i . v_j = 1 and dQ_i[c] = scale dS_{i,o+c}
with dS_ij = (keep_ij / (1 - p) - D_i) / n_i, D_i = dO_i . O_i = O_i[0].
A kept element gives dS above, a dropped one below
(0.5 / (1 - p) - D_i) / n_i, half a step of 1 / (n_i (1 - p)) on either
side, so the query-side kernel's bits are read off dQ against that
threshold (D_i taken from the forward's own O).

Sliding o over the sequence covers every (query, key) pair; the bits must
equal the oracle's keep mask (Philox-4x32-10 as the oracle header defines
it) wherever a pair is visible, and invisible pairs must contribute exactly
nothing.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from conftest import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DT = {"bf16": torch.bfloat16, "f16": torch.float16}


def _onehot_rows(T, H, d, starts, lengths, o, dtype, dev):
    """[T, H, d] with row starts[s] + o + c of every sequence = e_c (c < d)."""
    x = torch.zeros(T, H, d, dtype=dtype, device=dev)
    rows, cols = [], []
    for st, L in zip(starts, lengths):
        w = max(0, min(d, L - o))
        rows.append(torch.arange(w) + int(st) + o)
        cols.append(torch.arange(w))
    if rows:
        r = torch.cat(rows).to(dev)
        c = torch.cat(cols).to(dev)
        x[r, :, c] = 1
    return x


def probe(lengths, H, d, dtype, causal, p, seed, varlen, heads=None):
    """Keep bits [seq][head] (L x L, -1 where not read) seen by the forward,
    the key-side backward and the query-side backward, for the given heads
    (all if None)."""
    import exact_tiled_attention_40_amd as fa
    dev = torch.device("cuda")
    heads = list(range(H)) if heads is None else list(heads)
    nseq, N = len(lengths), max(lengths)
    T = sum(lengths) if varlen else nseq * N
    starts = np.cumsum([0] + list(lengths))[:-1] if varlen else [s * N for s in range(nseq)]
    kw = dict(causal=causal, dropout_p=p, seed=seed)
    if varlen:
        cu = torch.tensor(np.cumsum([0] + list(lengths)), dtype=torch.int32, device=dev)
        kw.update(cu_seqlens=cu, max_seqlen=N)
    shape = (T, H, d) if varlen else (nseq, N, H, d)
    dt = DT[dtype]
    scale = 1.0 / np.sqrt(d)
    zero = torch.zeros(shape, dtype=dt, device=dev)
    e0 = torch.zeros(T, H, d, dtype=dt, device=dev)
    e0[:, :, 0] = 1
    e0 = e0.reshape(shape)
    hsel = torch.tensor(heads, device=dev)
    bits = {kind: [[np.full((L, L), -1, np.int8) for _ in heads] for L in lengths] for kind in ("fwd", "kv", "q")}
    for o in range(0, N, d):
        x = _onehot_rows(T, H, d, starts, lengths, o, dt, dev).reshape(shape)
        # forward (one-hot V) and key side (one-hot dO)
        out, lse = fa.fa_forward(zero, zero, x, **kw)
        _, _, dv = fa.fa_backward(zero, zero, x, out, lse, x, **kw)
        # query side: one-hot K, V = dO = e_0
        out0, lse0 = fa.fa_forward(zero, x, e0, scale=scale, **kw)
        dq, _, _ = fa.fa_backward(zero, x, e0, out0, lse0, e0, scale=scale, **kw)
        torch.cuda.synchronize()
        out = out.reshape(T, H, d)[:, hsel].float().cpu().numpy()
        dv = dv.reshape(T, H, d)[:, hsel].float().cpu().numpy()
        dq = dq.reshape(T, H, d)[:, hsel].float().cpu().numpy()
        dd = out0.reshape(T, H, d)[:, hsel, 0].float().cpu().numpy()
        for s, L in enumerate(lengths):
            if L <= o:
                continue
            w = min(d, L - o)
            sl = slice(starts[s], starts[s] + L)
            n = (np.arange(L) + 1 if causal else np.full(L, L)).astype(np.float64)
            for t in range(len(heads)):
                bits["fwd"][s][t][:, o:o + w] = out[sl, t, :w] != 0
                bits["kv"][s][t][o:o + w, :] = (dv[sl, t, :w] != 0).T
                thr = scale * (0.5 / (1.0 - np.float32(p)) - dd[sl, t]) / n
                got = dq[sl, t, :w]
                vis = (np.arange(w)[None, :] + o <= np.arange(L)[:, None]) if causal else np.ones((L, w), bool)
                b = np.where(vis, got > thr[:, None], got != 0).astype(np.int8)
                bits["q"][s][t][:, o:o + w] = b
    return heads, bits


def check_probe(lengths, H, d, dtype, causal, p, seed, varlen, heads=None):
    heads, bits = probe(lengths, H, d, dtype, causal, p, seed, varlen, heads)
    for s, L in enumerate(lengths):
        vis = np.tril(np.ones((L, L), bool)) if causal else np.ones((L, L), bool)
        for t, h in enumerate(heads):
            ref = oracle.keep_mask(seed, p, s, h, L).astype(bool)
            counts = {}
            for kind in ("fwd", "kv", "q"):
                b = bits[kind][s][t]
                assert (b >= 0).all(), (kind, s, h)
                counts[kind] = int((b[vis].astype(bool) != ref[vis]).sum())
                # invisible pairs contribute nothing
                assert not b[~vis].any(), (kind, s, h)
            print(f"[seq {s} head {h} L={L}] mismatches: forward {counts['fwd']}, key side {counts['kv']}, "
                  f"query side {counts['q']}; kept {ref[vis].mean():.4f}", flush=True)
            assert counts == {"fwd": 0, "kv": 0, "q": 0}, counts


@pytest.mark.parametrize("lengths,H,d,dtype,causal,p,seed,varlen", [
    ([300, 300], 2, 128, "bf16", True, 0.3, 2**40 + 17, False),
    ([200], 3, 64, "f16", False, 0.5, 1005, False),
    ([5, 130, 77, 260], 2, 128, "bf16", True, 0.1, 99, True),
    ([70, 33], 1, 32, "f16", False, 0.25, 7, True),
    ([150, 90], 2, 96, "bf16", True, 0.2, 12345, True),
    ([300, 77], 2, 160, "bf16", True, 0.1, 31, True),
    ([200], 2, 192, "f16", False, 0.3, 32, False),
    ([260, 130], 2, 256, "bf16", True, 0.2, 33, True),
])
def test_keep_bits_through_fused_kernels(lengths, H, d, dtype, causal, p, seed, varlen):
    check_probe(lengths, H, d, dtype, causal, p, seed, varlen)


def test_keep_bits_varlen_workload_shape():
    """The varlen dropout workload's own shape: its 16 drawn sequence lengths
    (up to 4096 tokens, packed), H = 32, d = 128, bf16, causal, p = 0.1, its
    seed; heads 0 and 31 of every sequence, sequence 15 included."""
    wl = workloads.WORKLOADS["varlen16_H32_d128_bf16_causal_p0.1"]
    lengths = workloads.make_inputs(wl, with_do=False).lengths
    print(f"[varlen workload shape] lengths {lengths}", flush=True)
    check_probe(lengths, wl.H, wl.d, wl.dtype, wl.causal, wl.dropout_p, wl.seed, True, heads=[0, 31])
