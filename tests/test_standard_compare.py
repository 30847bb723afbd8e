"""The standard-attention side of the comparison measurement computes the
same attention as the oracle (fp64 on the CPU, no dropout), so a timing
against it compares equal work.  With dropout, its inverted scaling keeps
the expectation of O: averaged over many masks it approaches the undropped
O."""
import numpy as np
import pytest
import torch

import bench
import oracle


@pytest.mark.parametrize("B,N,H,d,causal", [(2, 37, 3, 16, True), (1, 50, 2, 32, False)])
def test_standard_step_matches_oracle(B, N, H, d, causal):
    g = torch.Generator().manual_seed(11)
    q, k, v, do = (torch.randn(B, N, H, d, generator=g, dtype=torch.float64) for _ in range(4))
    scale = d ** -0.5
    o, dq, dk, dv = bench.standard_attention_step(q, k, v, do, scale=scale, causal=causal)
    tok = lambda t: t.reshape(B * N, H, d).contiguous().numpy()
    o_ref, _ = oracle.forward(tok(q), tok(k), tok(v), scale=scale, causal=causal, N=N)
    dq_ref, dk_ref, dv_ref = oracle.backward(tok(q), tok(k), tok(v), tok(do), scale=scale, causal=causal, N=N)
    for got, ref in ((o, o_ref), (dq, dq_ref), (dk, dk_ref), (dv, dv_ref)):
        np.testing.assert_allclose(tok(got), ref, rtol=1e-10, atol=1e-12)


def test_standard_step_dropout_is_unbiased():
    g = torch.Generator().manual_seed(5)
    B, N, H, d = 1, 24, 1, 8
    q, k, v, do = (torch.randn(B, N, H, d, generator=g, dtype=torch.float64) for _ in range(4))
    o0 = bench.standard_attention_step(q, k, v, do, scale=0.3, causal=True)[0]
    draws = torch.Generator().manual_seed(7)
    acc = torch.zeros_like(o0)
    n = 2000
    for _ in range(n):
        acc += bench.standard_attention_step(q, k, v, do, scale=0.3, causal=True, dropout_p=0.25,
                                             generator=draws)[0]
    # each element is a mean of n draws with per-draw spread below max|v| / (1 - p)
    bound = 5 * v.abs().max() / 0.75 / n ** 0.5
    assert (acc / n - o0).abs().max() < bound
