"""Dropout keep bits recovered bit for bit through the fused kernels (needs
an MI355X).

With Q = K = 0 every visible score is 0, so P is uniform, 1/n_i over the n_i
keys query i sees.  Forward: with one-hot V rows (v_j = e_{j-o} for
o <= j < o + d, else 0), O[i][c] = keep(i, o + c) / (n_i (1 - p)) for a
visible key o + c and 0 otherwise, so O[i][c] != 0 exactly when the forward
kernel kept element (i, o + c).  Key-side backward: with one-hot dO rows
(dO_i = e_{i-o} for o <= i < o + d), dV_j = sum_i Z_ij dO_i gives
dV_j[c] = keep(o + c, j) / (n_{o+c} (1 - p)) for a visible pair, so the key
side's keep bits are read off dV the same way.  Sliding o over the sequence
covers every (query, key) pair; the bits must equal the oracle's keep mask
(Philox-4x32-10 as the header defines it) everywhere a pair is visible.
"""
import numpy as np
import pytest
import torch

import oracle
from conftest import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DT = {"bf16": torch.bfloat16, "f16": torch.float16}


def probe(lengths, H, d, dtype, causal, p, seed, varlen):
    """Keep bits [seq][h] (L x L, -1 where not visible) seen by the forward
    and by the key-side backward."""
    import exact_tiled_attention_40_amd as fa
    dev = torch.device("cuda")
    nseq, N = len(lengths), max(lengths)
    T = sum(lengths) if varlen else nseq * N
    starts = np.cumsum([0] + list(lengths))[:-1] if varlen else [s * N for s in range(nseq)]
    kw = dict(causal=causal, dropout_p=p, seed=seed)
    if varlen:
        cu = torch.tensor(np.cumsum([0] + list(lengths)), dtype=torch.int32, device=dev)
        kw.update(cu_seqlens=cu, max_seqlen=N)
    shape = (T, H, d) if varlen else (nseq, N, H, d)
    q = torch.zeros(shape, dtype=DT[dtype], device=dev)
    k = torch.zeros_like(q)
    fwd_bits = [[np.full((L, L), -1, np.int8) for _ in range(H)] for L in lengths]
    bwd_bits = [[np.full((L, L), -1, np.int8) for _ in range(H)] for L in lengths]
    for o in range(0, N, d):
        onehot = torch.zeros(T, H, d, dtype=torch.float32)
        for s, L in enumerate(lengths):
            for c in range(min(d, L - o) if L > o else 0):
                onehot[starts[s] + o + c, :, c] = 1.0
        x = onehot.to(DT[dtype]).to(dev).reshape(shape)
        out, lse = fa.fa_forward(q, k, x, **kw)
        dq, dk, dv = fa.fa_backward(q, k, x, out, lse, x, **kw)
        torch.cuda.synchronize()
        out = out.reshape(T, H, d).float().cpu().numpy()
        dv = dv.reshape(T, H, d).float().cpu().numpy()
        for s, L in enumerate(lengths):
            if L <= o:
                continue
            w = min(d, L - o)
            rows = out[starts[s]:starts[s] + L]        # [L, H, d]: O[i][c] <-> (i, o + c)
            keys = dv[starts[s]:starts[s] + L]         # [L, H, d]: dV[j][c] <-> (o + c, j)
            for h in range(H):
                fwd_bits[s][h][:, o:o + w] = rows[:, h, :w] != 0
                bwd_bits[s][h][o:o + w, :] = (keys[:, h, :w] != 0).T
    return fwd_bits, bwd_bits


@pytest.mark.parametrize("lengths,H,d,dtype,causal,p,seed,varlen", [
    ([300, 300], 2, 128, "bf16", True, 0.3, 2**40 + 17, False),
    ([200], 3, 64, "f16", False, 0.5, 1005, False),
    ([5, 130, 77, 260], 2, 128, "bf16", True, 0.1, 99, True),
    ([70, 33], 1, 32, "f16", False, 0.25, 7, True),
])
def test_keep_bits_through_fused_kernels(lengths, H, d, dtype, causal, p, seed, varlen):
    fwd_bits, bwd_bits = probe(lengths, H, d, dtype, causal, p, seed, varlen)
    for s, L in enumerate(lengths):
        vis = np.tril(np.ones((L, L), bool)) if causal else np.ones((L, L), bool)
        for h in range(len(fwd_bits[s])):
            ref = oracle.keep_mask(seed, p, s, h, L).astype(bool)
            f, b = fwd_bits[s][h], bwd_bits[s][h]
            assert (f[vis] >= 0).all() and (b[vis] >= 0).all()
            nf = int((f[vis].astype(bool) != ref[vis]).sum())
            nb = int((b[vis].astype(bool) != ref[vis]).sum())
            print(f"[seq {s} head {h} L={L}] forward mismatches {nf}, key-side mismatches {nb}, "
                  f"kept {ref[vis].mean():.3f}", flush=True)
            assert nf == 0 and nb == 0
            # masked-out pairs contribute nothing
            assert not f[~vis].any() and not b[~vis].any()
