"""GPU parity of fa_decode (KV-cache decode step) against the fp64 oracle
(needs an MI355X)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from conftest import gpu_available
from parity import LSE_TOL, O_TOL

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def run(x):
    import exact_tiled_attention_40_amd as fa
    dev = torch.device("cuda")
    q, k, v = (t.to(dev) for t in (x.q, x.k, x.v))
    lens = x.seqlens.to(dev) if x.seqlens is not None else None
    o, lse = fa.fa_decode(q, k, v, seqlens_k=lens, scale=x.wl.scale, causal=x.wl.causal)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), lse.cpu().double().numpy()


def check(x):
    o, lse = run(x)
    o_ref, lse_ref = oracle.decode(x.q.double().numpy(), x.k.double().numpy(), x.v.double().numpy(),
                                   scale=x.wl.scale, causal=x.wl.causal,
                                   seqlens_k=None if x.seqlens is None else x.seqlens.numpy())
    empty = np.isneginf(lse_ref)
    assert np.all(o[empty] == 0.0) and np.all(np.isneginf(lse[empty]))
    eo = float(np.abs(o - o_ref).max())
    el = float(np.abs(lse[~empty] - lse_ref[~empty]).max(initial=0.0))
    print(f"[{x.wl.name}] O max abs {eo:.3e}, LSE max abs {el:.3e}, empty {int(empty.sum())}", flush=True)
    assert eo <= O_TOL[x.wl.dtype] and el <= LSE_TOL


def wl(B, H, nq, nk, d, dtype, causal, seed):
    return workloads.DecodeWorkload(f"decode_B{B}_H{H}_nq{nq}_Nk{nk}_d{d}_{dtype}", B, H, nq, nk, d, dtype, causal,
                                    seed=seed)


@pytest.mark.parametrize("B,H,nq,nk,d,dtype,causal", [
    (2, 4, 1, 1000, 128, "bf16", False),
    (1, 2, 1, 1, 64, "f16", True),
    (3, 2, 4, 2048, 64, "f16", True),
    (2, 3, 2, 513, 128, "bf16", True),
    (1, 8, 3, 4097, 128, "f16", False),
    (4, 1, 4, 511, 64, "bf16", False),
    # five to eight new tokens (speculative or chunked steps)
    (2, 3, 5, 1100, 128, "bf16", True),
    (3, 2, 8, 2500, 64, "f16", True),
    (1, 4, 8, 300, 128, "f16", False),
    (2, 2, 7, 6, 64, "bf16", True),
])
def test_decode_small(B, H, nq, nk, d, dtype, causal):
    check(workloads.make_decode_inputs(wl(B, H, nq, nk, d, dtype, causal, seed=700 + nk)))


def test_decode_ragged_lengths_and_empty_queries():
    # lengths 0 and 1 with 4 causal queries: queries that see no key
    x = workloads.make_decode_inputs(wl(5, 2, 4, 1500, 128, "bf16", True, seed=710), lengths=[1500, 0, 1, 3, 513])
    check(x)
    x = workloads.make_decode_inputs(wl(3, 2, 2, 700, 64, "f16", False, seed=711), lengths=[0, 700, 512])
    check(x)


@pytest.mark.parametrize("name", list(workloads.DECODE_WORKLOADS))
def test_decode_workload(name):
    check(workloads.make_decode_inputs(workloads.DECODE_WORKLOADS[name]))
