"""GPU parity on degenerate and extreme grids (needs an MI355X): many heads
of very short sequences (grids of thousands of workgroups, most of them one
partial tile), packed batches with empty sequences, and hundreds of ragged
sequences; forward and backward against the fp64 oracle, every head."""
import numpy as np
import pytest

import workloads
from conftest import gpu_available
from test_gpu_backward import check as check_backward
from test_gpu_forward import check as check_forward

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


CASES = [
    ("many_heads_tiny_causal", lambda: workloads.custom(64, 40, 5, 128, "bf16", True, seed=41)),
    ("many_heads_short", lambda: workloads.custom(33, 17, 70, 64, "f16", False, seed=42)),
    ("empty_sequences_causal", lambda: workloads.custom(0, 2, 0, 128, "bf16", True, lengths=[0, 5, 0, 130, 0, 1],
                                                        seed=43)),
    ("empty_sequences_dropout", lambda: workloads.custom(0, 3, 0, 64, "f16", False, lengths=[0, 0, 77, 0, 200],
                                                         dropout_p=0.2, seed=44)),
    ("three_hundred_sequences", lambda: workloads.custom(0, 3, 0, 64, "f16", False, lengths=workloads.ragged_lengths(300, 0, 40, 45),
                                                         seed=45)),
    ("three_hundred_sequences_causal_d96", lambda: workloads.custom(0, 2, 0, 96, "bf16", True,
                                                                    lengths=workloads.ragged_lengths(300, 1, 90, 46), seed=46)),
]


@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
def test_edge_forward(name, make):
    check_forward(make())


@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
def test_edge_backward(name, make):
    check_backward(make())


@pytest.mark.parametrize("dropout_p", [0.0, 0.15])
def test_varlen_guard_regions(dropout_p):
    """Packed varlen tensors followed by a guard region of 300 tokens: NaN in
    every input past the last token (q, k, v, dO, and O, LSE as the backward
    reads them) must not reach any output, no output past the last token may
    be written (O, LSE, dQ, dK, dV hold a sentinel there), and the outputs
    must still match the oracle."""
    import torch

    import exact_tiled_attention_40_amd as fa
    from parity import GRAD_TOL, LSE_TOL, O_TOL, oracle_backward, oracle_forward, rel_fro, tokens_f64
    lengths = [1, 63, 64, 65, 200, 129, 7, 256]
    x = workloads.custom(0, 2, 0, 128, "bf16", True, lengths=lengths, dropout_p=dropout_p, seed=47)
    T, G = sum(lengths), 300
    H, d = x.wl.H, x.wl.d
    dev = torch.device("cuda")

    def guarded(t, fill):
        buf = torch.full((T + G,) + tuple(t.shape[1:]), fill, dtype=t.dtype, device=dev)
        buf[:T] = t.to(dev)
        return buf

    q, k, v, do = (guarded(t, float("nan")) for t in (x.q, x.k, x.v, x.do))
    ob = torch.full((T + G, H, d), -7.0, dtype=torch.bfloat16, device=dev)
    lb = torch.full((T + G, H), -7.0, dtype=torch.float32, device=dev)
    grads = [torch.full((T + G, H, d), -7.0, dtype=torch.bfloat16, device=dev) for _ in range(3)]
    cu = x.cu_seqlens.to(dev)
    kw = dict(scale=x.wl.scale, causal=True, cu_seqlens=cu, max_seqlen=max(lengths), dropout_p=dropout_p,
              seed=x.wl.seed)
    print(f"[varlen guard p={dropout_p}] forward + backward", flush=True)
    fa.fa_forward(q[:T], k[:T], v[:T], out=ob[:T], lse=lb[:T], **kw)
    torch.cuda.synchronize()
    # the backward's O and LSE inputs get their own NaN guard
    o_in, l_in = guarded(ob[:T], float("nan")), guarded(lb[:T], float("nan"))
    fa.fa_backward(q[:T], k[:T], v[:T], o_in[:T], l_in[:T], do[:T], dq=grads[0][:T], dk=grads[1][:T],
                   dv=grads[2][:T], **kw)
    torch.cuda.synchronize()
    for name, t in (("O", ob), ("LSE", lb), ("dQ", grads[0]), ("dK", grads[1]), ("dV", grads[2])):
        assert (t[T:] == -7.0).all(), f"{name} written past the last token"
        assert torch.isfinite(t[:T].float()).all(), f"{name} not finite"
    pairs = [(s, h) for s in range(len(lengths)) for h in range(H)]
    o_ref, lse_ref = oracle_forward(x, pairs)
    eo = float(np.abs(tokens_f64(ob[:T]) - o_ref).max())
    el = float(np.abs(lb[:T].double().cpu().numpy() - lse_ref).max())
    assert eo <= O_TOL["bf16"] and el <= LSE_TOL, (eo, el)
    refs = oracle_backward(x, pairs)
    for name, g, r in zip(("dQ", "dK", "dV"), grads, refs):
        e, worst, over = rel_fro(x, g[:T], r, pairs, floor_ref=refs[2])
        print(f"[varlen guard p={dropout_p}] {name} {e:.3e} (worst head {worst:.3e})", flush=True)
        assert e <= GRAD_TOL and not over, (name, e, over)
