"""fa_backward_noalloc (the backward on the library's fixed per-GPU scratch)
against fa_backward (caller workspace) through the C ABI (needs an MI355X).

Two calls in a row, the second on a smaller problem than the first, so the
scratch still holds the first call's rows when the second runs: both must
equal fa_backward bit for bit (same kernels, deterministic), and so must a
repeat of the first call after the second.
"""
import pytest
import torch

import workloads
from conftest import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _case(x):
    import exact_tiled_attention_40_amd as fa
    dev = torch.device("cuda")
    q, k, v, do = (t.to(dev) for t in (x.q, x.k, x.v, x.do))
    cu = x.cu_seqlens.to(dev) if x.cu_seqlens is not None else None
    kw = dict(scale=x.wl.scale, causal=x.wl.causal, cu_seqlens=cu, max_seqlen=x.wl.N if cu is not None else None,
              dropout_p=x.wl.dropout_p, seed=x.wl.seed)
    o, lse = fa.fa_forward(q, k, v, **kw)
    ref = fa.fa_backward(q, k, v, o, lse, do, **kw)
    torch.cuda.synchronize()
    return q, k, v, o, lse, do, kw, ref


def _noalloc(case):
    import exact_tiled_attention_40_amd as fa
    q, k, v, o, lse, do, kw, _ = case
    # outputs filled with NaN: every element must be written
    grads = [torch.full_like(q, float("nan")) for _ in range(3)]
    fa.fa_backward_noalloc(q, k, v, o, lse, do, dq=grads[0], dk=grads[1], dv=grads[2], **kw)
    torch.cuda.synchronize()
    return grads


def test_noalloc_backward_equals_fa_backward_twice_second_smaller():
    big = _case(workloads.custom(2, 4, 1000, 128, "bf16", True, dropout_p=0.1, seed=61))
    small = _case(workloads.custom(0, 2, 0, 64, "f16", False, lengths=[5, 130, 77], seed=62))
    for name, case in (("B2 H4 N1000 d128 bf16 causal p=0.1", big), ("varlen 3 seqs H2 d64 f16", small),
                       ("B2 H4 N1000 d128 bf16 causal p=0.1, again", big)):
        print(f"[noalloc] {name}", flush=True)
        got = _noalloc(case)
        for gn, a, b in zip(("dQ", "dK", "dV"), got, case[-1]):
            assert torch.equal(a, b), (name, gn)


def test_noalloc_backward_at_the_scratch_limit():
    # B*N*H = FA_NOALLOC_MAX_ROWS exactly (1024 sequences of 64 tokens, 64
    # heads): the scratch's last rows are written and read
    import exact_tiled_attention_40_amd as fa
    B, N, H = 1024, 64, 64
    assert B * N * H == fa.FA_NOALLOC_MAX_ROWS
    case = _case(workloads.custom(B, H, N, 32, "bf16", False, dropout_p=0.2, seed=63))
    print("[noalloc] B1024 H64 N64 d32 bf16 p=0.2 (B*N*H at the limit)", flush=True)
    got = _noalloc(case)
    for gn, a, b in zip(("dQ", "dK", "dV"), got, case[-1]):
        assert torch.equal(a, b), gn
