"""Stored dropout decisions: fa_forward_keep / fa_backward_keep (needs an
MI355X).

The keep-bit calls trade the backward's rehashing of the dropout mask for one
bit per (query, key) pair stored by the forward.  They must give bitwise the
outputs of fa_forward / fa_backward with the same arguments; the bits the
forward stores must equal the oracle's keep mask (Philox-4x32-10 as the
oracle header defines it) on every pair a query sees; and the forward must
write nothing outside the documented words (the buffer starts as random
garbage, with a guard region after it).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from conftest import gpu_available
from parity import to_gpu

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DT = {"bf16": torch.bfloat16, "f16": torch.float16}
GUARD = 4096  # bytes after the buffer that must stay untouched


def _inputs(lengths, H, d, dtype, varlen, seed):
    g = torch.Generator().manual_seed(seed)
    nseq, N = len(lengths), max(lengths)
    shape = (sum(lengths), H, d) if varlen else (nseq, N, H, d)
    q, k, v, do = (torch.randn(shape, generator=g, dtype=torch.float32).to(DT[dtype]).cuda() for _ in range(4))
    kw = {}
    if varlen:
        cu = torch.tensor(np.cumsum([0] + list(lengths)), dtype=torch.int32).cuda()
        kw = dict(cu_seqlens=cu, max_seqlen=N)
    return q, k, v, do, kw


def _garbage(nbytes, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randint(0, 256, (nbytes + GUARD,), generator=g, dtype=torch.uint8).cuda()


def decode_bits(buf, B, H, N, b, h, L):
    """[L, L] keep bits of sequence b, head h from the stored words."""
    nkt, npad = (N + 63) // 64, (N + 3) // 4 * 4
    per_head = nkt * 2 * npad * 4
    words = buf[(b * H + h) * per_head:(b * H + h + 1) * per_head].cpu().numpy().view(np.uint32)
    words = words.reshape(nkt, 2, npad)
    per_query = np.ascontiguousarray(words[:, :, :L].transpose(2, 0, 1))  # [L, nkt, 2]
    bits = np.unpackbits(per_query.view(np.uint8), bitorder="little").reshape(L, nkt * 64)
    return bits[:, :L]


def run_pair(lengths, H, d, dtype, causal, p, seed, varlen, heads=None, check_bits=True):
    import exact_tiled_attention_40_amd as fa
    q, k, v, do, kw = _inputs(lengths, H, d, dtype, varlen, seed + 1)
    B, N = len(lengths), max(lengths)
    kw.update(causal=causal, dropout_p=p, seed=seed)
    need = fa.fa_dropout_bits_size(B, N, H)
    assert need == B * H * ((N + 63) // 64) * 2 * ((N + 3) // 4 * 4) * 4
    buf = _garbage(need, seed + 2)
    guard = buf[need:].clone()
    o_ref, lse_ref = fa.fa_forward(q, k, v, **kw)
    o, lse = fa.fa_forward_keep(q, k, v, keep_bits=buf[:need], **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), "forward_keep differs from forward"
    assert torch.equal(buf[need:], guard), "forward_keep wrote past the buffer"
    g_ref = fa.fa_backward(q, k, v, o_ref, lse_ref, do, **kw)
    g = fa.fa_backward_keep(q, k, v, o, lse, do, keep_bits=buf[:need], **kw)
    torch.cuda.synchronize()
    for name, a, r in zip(("dQ", "dK", "dV"), g, g_ref):
        assert torch.isfinite(a.float()).all(), name
        assert torch.equal(a, r), f"backward_keep {name} differs from backward"
    if not check_bits:
        return buf
    heads = range(H) if heads is None else heads
    for s, L in enumerate(lengths):
        vis = np.tril(np.ones((L, L), bool)) if causal else np.ones((L, L), bool)
        for h in heads:
            got = decode_bits(buf, B, H, N, s, h, L).astype(bool)
            ref = oracle.keep_mask(seed, p, s, h, L).astype(bool)
            bad = int((got[vis] != ref[vis]).sum())
            assert bad == 0, (s, h, L, bad)
    print(f"[{lengths} H{H} d{d} {dtype} causal={causal} p={p} varlen={varlen}] outputs bitwise equal, "
          f"bits equal to the oracle's", flush=True)
    return buf


@pytest.mark.parametrize("lengths,H,d,dtype,causal,p,seed,varlen", [
    ([300, 300], 2, 128, "bf16", True, 0.3, 2**40 + 17, False),
    ([200], 3, 64, "f16", False, 0.5, 1005, False),
    ([129, 129], 4, 64, "bf16", True, 0.1, 5, False),
    ([5, 130, 77, 260], 2, 128, "bf16", True, 0.1, 99, True),
    ([70, 33], 1, 32, "f16", False, 0.25, 7, True),
    ([150, 90], 2, 96, "bf16", True, 0.2, 12345, True),
    ([301, 77], 2, 160, "bf16", True, 0.1, 31, True),
    ([201], 2, 192, "f16", False, 0.3, 32, False),
    ([260, 130], 2, 256, "bf16", True, 0.2, 33, True),
    ([1, 3], 2, 128, "bf16", True, 0.4, 8, True),
])
def test_keep_bits_match_hash_path_and_oracle(lengths, H, d, dtype, causal, p, seed, varlen):
    run_pair(lengths, H, d, dtype, causal, p, seed, varlen)


def test_keep_bits_without_dropout_is_the_plain_call():
    import exact_tiled_attention_40_amd as fa
    q, k, v, do, kw = _inputs([200, 200], 2, 64, "bf16", False, 3)
    o_ref, lse_ref = fa.fa_forward(q, k, v, causal=True)
    o, lse = fa.fa_forward_keep(q, k, v, keep_bits=None, causal=True)
    g_ref = fa.fa_backward(q, k, v, o_ref, lse_ref, do, causal=True)
    g = fa.fa_backward_keep(q, k, v, o, lse, do, keep_bits=None, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
    for a, r in zip(g, g_ref):
        assert torch.equal(a, r)


def test_keep_bits_varlen_workload_shape():
    """The varlen dropout workload at its full size (16 packed sequences up to
    4096 tokens, H 32, d 128, bf16, causal, p 0.1, its seed): every output
    bitwise equal to the hashing path; bits checked on heads 0 and 31 of
    sequences 0, 7 and 15."""
    import exact_tiled_attention_40_amd as fa
    wl = workloads.WORKLOADS["varlen16_H32_d128_bf16_causal_p0.1"]
    x = workloads.make_inputs(wl)
    q, k, v, do, cu = to_gpu(x)
    kw = dict(scale=wl.scale, causal=wl.causal, dropout_p=wl.dropout_p, seed=wl.seed, cu_seqlens=cu,
              max_seqlen=wl.N)
    need = fa.fa_dropout_bits_size(wl.B, wl.N, wl.H)
    print(f"[varlen workload] lengths {x.lengths}, keep bits {need / 2**20:.0f} MiB", flush=True)
    buf = _garbage(need, 11)
    guard = buf[need:].clone()
    o_ref, lse_ref = fa.fa_forward(q, k, v, **kw)
    o, lse = fa.fa_forward_keep(q, k, v, keep_bits=buf[:need], **kw)
    g_ref = fa.fa_backward(q, k, v, o_ref, lse_ref, do, **kw)
    g = fa.fa_backward_keep(q, k, v, o, lse, do, keep_bits=buf[:need], **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
    assert torch.equal(buf[need:], guard)
    for name, a, r in zip(("dQ", "dK", "dV"), g, g_ref):
        assert torch.equal(a, r), name
    for s in (0, 7, 15):
        L = x.lengths[s]
        vis = np.tril(np.ones((L, L), bool))
        for h in (0, 31):
            got = decode_bits(buf, wl.B, wl.H, wl.N, s, h, L).astype(bool)
            ref = oracle.keep_mask(wl.seed, wl.dropout_p, s, h, L).astype(bool)
            assert int((got[vis] != ref[vis]).sum()) == 0, (s, h)
            print(f"[varlen workload seq {s} head {h} L={L}] bits equal, kept {ref[vis].mean():.4f}", flush=True)


def test_keep_bits_at_the_longest_sequence():
    """One sequence of FA_MASK_MAX_N = 65536 tokens (the largest the keep-bit
    buffer addresses: 512 MiB per head), causal, p = 0.1: every output
    bitwise equal to the hashing path, and the stored bits of the first 4096
    queries against the first 4096 keys equal to the oracle's keep mask (a
    decision depends on (seed, b, h, i, j) only, so the oracle's mask of a
    4096-token sequence covers them)."""
    import exact_tiled_attention_40_amd as fa
    N, H, d, p, seed = fa.FA_MASK_MAX_N, 1, 64, 0.1, 4242
    q, k, v, do, kw = _inputs([N], H, d, "bf16", False, seed)
    kw.update(causal=True, dropout_p=p, seed=seed)
    need = fa.fa_dropout_bits_size(1, N, H)
    assert need == N * (N // 64) * 8
    buf = _garbage(need, 5)
    guard = buf[need:].clone()
    o_ref, lse_ref = fa.fa_forward(q, k, v, **kw)
    o, lse = fa.fa_forward_keep(q, k, v, keep_bits=buf[:need], **kw)
    g_ref = fa.fa_backward(q, k, v, o_ref, lse_ref, do, **kw)
    g = fa.fa_backward_keep(q, k, v, o, lse, do, keep_bits=buf[:need], **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
    assert torch.equal(buf[need:], guard)
    for name, a, r in zip(("dQ", "dK", "dV"), g, g_ref):
        assert torch.equal(a, r), name
    L = 4096
    words = buf[:need].view(torch.int32).view(N // 64, 2, N)[: L // 64, :, :L].cpu().numpy().view(np.uint32)
    per_query = np.ascontiguousarray(words.transpose(2, 0, 1))  # [L, L/64, 2]
    got = np.unpackbits(per_query.view(np.uint8), bitorder="little").reshape(L, L).astype(bool)
    ref = oracle.keep_mask(seed, p, 0, 0, L).astype(bool)
    vis = np.tril(np.ones((L, L), bool))
    assert int((got[vis] != ref[vis]).sum()) == 0
    print(f"[keep bits N={N}] outputs bitwise equal; first {L} rows' bits equal the oracle, kept "
          f"{ref[vis].mean():.4f}", flush=True)
