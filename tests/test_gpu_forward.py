"""GPU parity of fa_forward against the fp64 oracle (needs an MI355X)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import LSE_TOL, O_TOL, compare_forward, oracle_forward, select_heads, to_gpu
from conftest import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def run_forward(x, **kw):
    import exact_tiled_attention_40_amd as fa
    q, k, v, _, cu = to_gpu(x)
    o, lse = fa.fa_forward(q, k, v, scale=x.wl.scale, causal=x.wl.causal, cu_seqlens=cu,
                           max_seqlen=x.wl.N if cu is not None else None, dropout_p=x.wl.dropout_p,
                           seed=x.wl.seed, **kw)
    torch.cuda.synchronize()
    return o, lse


def check(x, n_heads=None):
    o, lse = run_forward(x)
    heads, pairs = select_heads(x, n_heads)
    o_ref, lse_ref = oracle_forward(x, heads)
    eo, el = compare_forward(x, o, lse, pairs, o_ref, lse_ref)
    print(f"[{x.wl.name}] O max abs {eo:.3e}  LSE max abs {el:.3e}", flush=True)
    assert np.isfinite(o.float().cpu().numpy()).all()
    assert eo <= O_TOL[x.wl.dtype], eo
    assert el <= LSE_TOL, el
    return o, lse


SMALL = [
    # B, H, N, d, dtype, causal
    (1, 1, 1, 64, "f16", False),
    (1, 1, 1, 128, "bf16", True),
    (2, 3, 77, 64, "bf16", True),
    (1, 2, 128, 64, "f16", False),
    (1, 2, 200, 128, "bf16", False),
    (2, 2, 257, 128, "f16", True),
    (1, 1, 129, 128, "bf16", True),
    (1, 4, 384, 64, "bf16", True),
    (3, 1, 191, 128, "f16", False),
    (1, 2, 1000, 128, "bf16", True),
    # the smaller and in-between head sizes
    (1, 2, 1, 32, "bf16", True),
    (2, 2, 333, 32, "f16", False),
    (1, 3, 517, 32, "bf16", True),
    (1, 1, 1, 96, "f16", False),
    (2, 2, 300, 96, "bf16", True),
    (1, 2, 700, 96, "f16", False),
    # heads above 128 (four waves, one per SIMD; 256: split dK/dV columns)
    (1, 2, 1, 160, "bf16", True),
    (2, 2, 200, 160, "f16", False),
    (1, 3, 333, 160, "bf16", True),
    (1, 1, 1, 192, "f16", False),
    (2, 2, 257, 192, "bf16", True),
    (1, 2, 600, 192, "f16", False),
    (1, 1, 1, 256, "bf16", True),
    (1, 2, 129, 256, "f16", False),
    (2, 2, 300, 256, "bf16", True),
    (1, 2, 777, 256, "bf16", False),
]


@pytest.mark.parametrize("B,H,N,d,dtype,causal", SMALL)
def test_forward_small(B, H, N, d, dtype, causal):
    check(workloads.custom(B, H, N, d, dtype, causal, seed=11 + N))


@pytest.mark.parametrize("d", [64, 128, 192])
def test_forward_packed_qkv(d):
    check(workloads.custom(2, 3, 150, d, "f16", False, packed=True, seed=5))


@pytest.mark.parametrize("causal", [False, True])
def test_forward_varlen_ragged(causal):
    x = workloads.custom(0, 2, 0, 128, "bf16", causal, lengths=[1, 63, 64, 65, 200, 129, 7], seed=9)
    check(x)


@pytest.mark.parametrize("d,dtype", [(160, "f16"), (192, "bf16"), (256, "bf16")])
def test_forward_varlen_ragged_large_heads(d, dtype):
    check(workloads.custom(0, 2, 0, d, dtype, True, lengths=[1, 63, 64, 65, 200, 129, 7, 700], dropout_p=0.1,
                           seed=d))


def test_forward_varlen_dropout():
    x = workloads.custom(0, 2, 0, 128, "bf16", True, lengths=[5, 130, 77], dropout_p=0.3, seed=19)
    check(x)


@pytest.mark.parametrize("d,causal", [(64, False), (128, True), (160, True), (192, False), (256, True)])
def test_forward_fixed_dropout(d, causal):
    check(workloads.custom(2, 2, 150, d, "f16", causal, dropout_p=0.2, seed=21))


def test_forward_large_scores():
    # K x 16: score std 16 / sqrt(d) stresses the running-max rescale
    check(workloads.custom(1, 2, 300, 128, "bf16", True, k_mult=16.0, seed=23))


def test_forward_deterministic():
    x = workloads.custom(1, 4, 333, 128, "bf16", True, seed=31)
    o1, l1 = run_forward(x)
    o2, l2 = run_forward(x)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_forward_writes_only_its_outputs():
    import exact_tiled_attention_40_amd as fa
    x = workloads.custom(1, 2, 100, 64, "bf16", True, seed=33)
    q, k, v, _, _ = to_gpu(x)
    n = q.numel()
    buf = torch.full((n + 4096,), 7.0, dtype=q.dtype, device="cuda")
    lbuf = torch.full((q.shape[0] * q.shape[1] * q.shape[2] + 512,), 9.0, dtype=torch.float32, device="cuda")
    o = buf[2048:2048 + n].view(q.shape)
    lse = lbuf[256:256 + lbuf.numel() - 512].view(q.shape[:-1])
    fa.fa_forward(q, k, v, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert (buf[:2048] == 7.0).all() and (buf[2048 + n:] == 7.0).all()
    assert (lbuf[:256] == 9.0).all() and (lbuf[-256:] == 9.0).all()


def test_dropout_mask_bit_exact():
    import exact_tiled_attention_40_amd as fa
    wl = workloads.WORKLOADS["varlen16_H32_d128_bf16_causal_p0.1"]
    for (b, h, N, p, seed) in [(0, 0, 128, 0.1, 1001), (3, 7, 77, 0.5, 2**40 + 3), (15, 31, 300, 0.1, 1005),
                               (15, 31, 4096, wl.dropout_p, wl.seed)]:
        m = fa.fa_dropout_mask(b, h, N, p, seed).cpu().numpy()
        ref = oracle.keep_mask(seed, p, b, h, N)
        assert np.array_equal(m, ref), (b, h, N)


def test_dropout_mask_independent_of_length():
    """The keep decision of (i, j) depends on (seed, b, h, i, j) only: the
    mask of a shorter sequence is the top-left block of a longer one's (the
    export of a packed variable-length sequence relies on it)."""
    import exact_tiled_attention_40_amd as fa
    for (b, h, n_small, n_big, p, seed) in [(5, 2, 100, 300, 0.2, 77), (15, 31, 1, 4096, 0.1, 1005)]:
        small = fa.fa_dropout_mask(b, h, n_small, p, seed).cpu().numpy()
        big = fa.fa_dropout_mask(b, h, n_big, p, seed).cpu().numpy()
        assert np.array_equal(big[:n_small, :n_small], small), (b, h, n_small, n_big)
