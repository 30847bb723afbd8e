"""GPU parity of the block-sparse calls (fa_forward_block_sparse,
fa_backward_block_sparse) against the fp64 oracle with the same block mask
(needs an MI355X)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from conftest import gpu_available
from parity import GRAD_TOL, LSE_TOL, O_TOL, rel_fro, seq_kwargs, to_gpu, tokens_f64, token_rows
from workloads import as_f64_tokens

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def run(x, bm, backward=True):
    import exact_tiled_attention_40_amd as fa
    q, k, v, do, cu = to_gpu(x)
    kw = dict(scale=x.wl.scale, causal=x.wl.causal, cu_seqlens=cu, max_seqlen=x.wl.N if cu is not None else None,
              dropout_p=x.wl.dropout_p, seed=x.wl.seed)
    m = bm.cuda() if bm is not None else None
    o, lse = fa.fa_forward(q, k, v, block_mask=m, **kw)
    grads = fa.fa_backward(q, k, v, o, lse, do, block_mask=m, **kw) if backward else None
    torch.cuda.synchronize()
    return o, lse, grads


def reference(x, bm):
    kw = dict(scale=x.wl.scale, causal=x.wl.causal, dropout_p=x.wl.dropout_p, seed=x.wl.seed,
              block_mask=bm.numpy(), block=128, **seq_kwargs(x))
    q, k, v, do = (as_f64_tokens(t) for t in (x.q, x.k, x.v, x.do))
    o, lse = oracle.forward(q, k, v, **kw)
    return o, lse, oracle.backward(q, k, v, do, **kw)


def check(x, bm):
    o, lse, grads = run(x, bm)
    o_ref, lse_ref, g_ref = reference(x, bm)
    og = tokens_f64(o)
    lg = lse.detach().cpu().double().numpy().reshape(og.shape[0], -1)
    empty = np.isneginf(lse_ref)
    # rows that see no key: O = 0 and LSE = -inf exactly
    assert np.all(og[empty.nonzero()[0], empty.nonzero()[1]] == 0.0)
    assert np.all(np.isneginf(lg[empty]))
    ok = ~empty
    eo = float(np.abs(og - o_ref).max())
    el = float(np.abs(lg[ok] - lse_ref[ok]).max(initial=0.0))
    print(f"[{x.wl.name}] O max abs {eo:.3e}, LSE max abs {el:.3e}, empty rows {int(empty.sum())}", flush=True)
    assert eo <= O_TOL[x.wl.dtype] and el <= LSE_TOL
    nseq = len(x.lengths) if x.wl.varlen else x.wl.B
    pairs = [(s, h) for s in range(nseq) for h in range(x.wl.H)]
    for name, g, r in zip(("dQ", "dK", "dV"), grads, g_ref):
        assert torch.isfinite(g.float()).all(), name
        e, worst, over = rel_fro(x, g, r, pairs, floor_ref=g_ref[2])
        print(f"[{x.wl.name}] {name} rel Frobenius {e:.3e} (worst head {worst:.3e})", flush=True)
        assert e <= GRAD_TOL and not over, (name, e, over)
    # structural zeros: dQ of rows that see no key, dK and dV of keys that no
    # query sees
    dq, dk, dv = (tokens_f64(g) for g in grads)
    bmn = bm.numpy()
    for s in range(nseq):
        r = token_rows(x, s)
        L = r.stop - r.start
        idx = np.arange(L) // 128
        for h in range(x.wl.H):
            em = bmn[s, h][idx][:, idx].astype(bool)
            if x.wl.causal:
                em &= np.tril(np.ones((L, L), dtype=bool))
            no_key = ~em.any(axis=1)
            unseen = ~em.any(axis=0)
            assert np.array_equal(no_key, empty[r, h])
            assert np.all(dq[r, h][no_key] == 0.0)
            assert np.all(dk[r, h][unseen] == 0.0) and np.all(dv[r, h][unseen] == 0.0)


CASES = [
    # B, H, N, d, dtype, causal, density
    (1, 2, 512, 128, "bf16", False, 0.5),
    (2, 2, 700, 64, "f16", True, 0.5),
    (1, 1, 1000, 128, "bf16", True, 0.3),
    (1, 3, 384, 64, "bf16", False, 0.0),
    (2, 1, 1111, 128, "f16", False, 0.7),
    (1, 2, 600, 32, "bf16", True, 0.5),
    (1, 2, 500, 96, "f16", False, 0.4),
    (1, 2, 640, 160, "bf16", True, 0.5),
    (2, 1, 500, 192, "f16", False, 0.5),
    (1, 2, 777, 256, "bf16", True, 0.4),
]


@pytest.mark.parametrize("B,H,N,d,dtype,causal,density", CASES)
def test_block_sparse_small(B, H, N, d, dtype, causal, density):
    x = workloads.custom(B, H, N, d, dtype, causal, seed=300 + N)
    check(x, workloads.block_mask(B, H, N, density, seed=400 + N))


@pytest.mark.parametrize("causal", [False, True])
def test_block_sparse_empty_rows_and_unseen_keys(causal):
    B, H, N, d = 1, 2, 640, 128
    x = workloads.custom(B, H, N, d, "bf16", causal, seed=501)
    bm = workloads.block_mask(B, H, N, 0.6, seed=502, keep_diagonal=False)
    bm[0, 0, 2, :] = 0      # queries 256..383 of head 0 see nothing
    bm[0, 1, :, 1] = 0      # keys 128..255 of head 1 are seen by no query
    bm[0, 1, 4, :] = 1
    check(x, bm)


def test_block_sparse_varlen_dropout():
    lengths = [300, 700, 129, 1]
    x = workloads.custom(len(lengths), 2, max(lengths), 128, "bf16", True, lengths=lengths, dropout_p=0.2,
                         seed=511)
    check(x, workloads.block_mask(len(lengths), 2, max(lengths), 0.5, seed=512))


@pytest.mark.parametrize("d,causal", [(64, False), (128, True)])
def test_block_sparse_all_ones_equals_dense(d, causal):
    B, H, N = 2, 2, 777
    x = workloads.custom(B, H, N, d, "bf16", causal, seed=520 + d)
    ones = torch.ones(workloads.block_mask(B, H, N, 1.0, seed=0).shape, dtype=torch.uint8)
    o1, l1, g1 = run(x, ones)
    o0, l0, g0 = run(x, None)
    assert torch.equal(o1, o0) and torch.equal(l1, l0)
    for a, b in zip(g1, g0):
        assert torch.equal(a, b)


def test_block_sparse_headline_shape_sampled():
    # the causal B4 H8 N4096 d128 bf16 shape at 50 % block density: the
    # forward on every head against the oracle for two heads
    wl = workloads.WORKLOADS[workloads.HEADLINE]
    x = workloads.make_inputs(wl)
    bm = workloads.block_mask(wl.B, wl.H, wl.N, 0.5, seed=530)
    o, lse, _ = run(x, bm, backward=False)
    for s, h in [(0, 0), (wl.B - 1, wl.H - 1)]:
        r = token_rows(x, s)
        q, k, v = (as_f64_tokens(t)[r, h:h + 1] for t in (x.q, x.k, x.v))
        o_ref, lse_ref = oracle.forward(q, k, v, scale=wl.scale, causal=True, N=wl.N,
                                        block_mask=bm[s:s + 1, h:h + 1].numpy(), block=128)
        og = tokens_f64(o)[r, h:h + 1]
        lg = lse.detach().cpu().double().numpy().reshape(-1, wl.H)[r, h:h + 1]
        print(f"[headline sparse] head ({s},{h}) O max abs {np.abs(og - o_ref).max():.3e}", flush=True)
        assert np.abs(og - o_ref).max() <= O_TOL["bf16"]
        assert np.abs(lg - lse_ref).max() <= LSE_TOL
