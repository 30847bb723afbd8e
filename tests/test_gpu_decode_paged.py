"""GPU parity of fa_decode_paged (the decode step over a paged KV cache)
against the fp64 oracle, and against fa_decode on the same cache (needs an
MI355X).  The pools are scattered in a random page order with unused pages
and padding rows set to NaN, and table entries past each length set to -1,
so a read of anything outside the sequence's pages shows up in the output."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from conftest import gpu_available
from parity import LSE_TOL, O_TOL

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def make(B, H, nq, nk, d, dtype, causal, lengths, seed):
    wl = workloads.DecodeWorkload(f"paged_B{B}_H{H}_nq{nq}_Nk{nk}_d{d}_{dtype}", B, H, nq, nk, d, dtype, causal,
                                  seed=seed)
    return workloads.make_decode_inputs(wl, lengths=lengths)


@pytest.mark.parametrize("B,H,nq,nk,d,dtype,causal,page,lengths", [
    (3, 2, 4, 2048, 128, "bf16", True, 16, [2048, 1000, 0]),
    (2, 4, 1, 3000, 64, "f16", False, 64, [3000, 1]),
    (1, 3, 8, 1500, 128, "f16", True, 1, [1500]),
    (2, 2, 2, 5000, 128, "bf16", True, 4096, [5000, 4097]),
    (4, 1, 5, 777, 64, "bf16", False, 256, [777, 200, 256, 0]),
    (2, 3, 3, 2100, 128, "f16", True, 32, [1025, 2100]),
])
def test_decode_paged_matches_oracle(B, H, nq, nk, d, dtype, causal, page, lengths):
    import exact_tiled_attention_40_amd as fa
    x = make(B, H, nq, nk, d, dtype, causal, lengths, seed=800 + nk + page)
    kp, vp, table = workloads.paged_cache(x.k, x.v, page, seed=900 + page, lengths=lengths)
    dev = torch.device("cuda")
    print(f"[paged B{B} H{H} nq{nq} nk{nk} d{d} {dtype} causal={causal} page={page} pool={kp.shape[0]}]", flush=True)
    o, lse = fa.fa_decode_paged(x.q.to(dev), kp.to(dev), vp.to(dev), table.to(dev), seqlens_k=x.seqlens.to(dev),
                                scale=x.wl.scale, causal=causal)
    torch.cuda.synchronize()
    o = o.float().cpu().double().numpy()
    lse = lse.cpu().double().numpy()
    o_ref, lse_ref = oracle.decode_paged(x.q.double().numpy(), kp.double().numpy(), vp.double().numpy(),
                                         table.numpy(), scale=x.wl.scale, causal=causal,
                                         seqlens_k=x.seqlens.numpy())
    empty = np.isneginf(lse_ref)
    assert np.all(o[empty] == 0.0) and np.all(np.isneginf(lse[empty]))
    eo = float(np.abs(o - o_ref).max())
    el = float(np.abs(lse[~empty] - lse_ref[~empty]).max(initial=0.0))
    print(f"  O max abs {eo:.3e}, LSE max abs {el:.3e}, empty {int(empty.sum())}", flush=True)
    assert np.isfinite(o).all()
    assert eo <= O_TOL[dtype] and el <= LSE_TOL


@pytest.mark.parametrize("page,causal", [(16, True), (128, False), (2048, True)])
def test_decode_paged_identity_table_equals_contiguous(page, causal):
    # the contiguous cache read as pages in order: the same kernel arithmetic
    # over the same keys, so the outputs agree bit for bit
    import exact_tiled_attention_40_amd as fa
    B, H, nq, nk, d = 3, 4, 4, 4096, 128
    x = make(B, H, nq, nk, d, "bf16", causal, [4096, 2500, 17], seed=850 + page)
    dev = torch.device("cuda")
    q, k, v, lens = (t.to(dev) for t in (x.q, x.k, x.v, x.seqlens))
    max_pages = nk // page
    table = torch.arange(B * max_pages, dtype=torch.int32, device=dev).reshape(B, max_pages)
    o1, l1 = fa.fa_decode(q, k, v, seqlens_k=lens, causal=causal)
    o2, l2 = fa.fa_decode_paged(q, k.view(B * max_pages, page, H, d), v.view(B * max_pages, page, H, d), table,
                                seqlens_k=lens, causal=causal)
    torch.cuda.synchronize()
    print(f"[identity page={page} causal={causal}] max |dO| {(o1.float() - o2.float()).abs().max().item():.3e}",
          flush=True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
