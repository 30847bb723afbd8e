"""The library on a side stream and inside a captured HIP graph (needs an
MI355X): forward + backward enqueued on a non-default stream, and the same
calls captured once into a graph and replayed several times with other GPU
work and synchronisations between replays; every result must equal the
eager one on the default stream bit for bit (the kernels are deterministic
and allocate nothing, so a replay recomputes exactly the same values)."""
import pytest
import torch

import workloads
from conftest import gpu_available
from parity import to_gpu

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def run(fa, q, k, v, do, out, **kw):
    o, lse, dq, dk, dv, ws, kb = out
    if kb is None:
        fa.fa_forward(q, k, v, out=o, lse=lse, **kw)
        fa.fa_backward(q, k, v, o, lse, do, dq=dq, dk=dk, dv=dv, workspace=ws, **kw)
    else:
        fa.fa_forward_keep(q, k, v, keep_bits=kb, out=o, lse=lse, **kw)
        fa.fa_backward_keep(q, k, v, o, lse, do, keep_bits=kb, dq=dq, dk=dk, dv=dv, workspace=ws, **kw)


# dropout with the hashing calls, and with the stored-keep-bit calls (whose
# bit buffer is cleared before every replay as well)
@pytest.mark.parametrize("dropout_p,keep", [(0.0, False), (0.2, False), (0.2, True)])
def test_side_stream_and_graph_replay_match_eager(dropout_p, keep):
    import exact_tiled_attention_40_amd as fa
    x = workloads.custom(2, 3, 300, 128, "bf16", True, dropout_p=dropout_p, seed=81)
    q, k, v, do, _ = to_gpu(x)
    kw = dict(causal=True, dropout_p=dropout_p, seed=x.wl.seed)

    def buffers():
        ws = torch.empty(fa.fa_backward_workspace_size(2, 300, 3, 128), dtype=torch.uint8, device="cuda")
        kb = torch.zeros(fa.fa_dropout_bits_size(2, 300, 3), dtype=torch.uint8, device="cuda") if keep else None
        return (torch.empty_like(q), torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda"),
                torch.empty_like(q), torch.empty_like(q), torch.empty_like(q), ws, kb)

    ref = buffers()
    run(fa, q, k, v, do, ref, **kw)
    torch.cuda.synchronize()

    # a side stream
    side = torch.cuda.Stream()
    got = buffers()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(fa, q, k, v, do, got, **kw)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for a, b in zip(ref[:5], got[:5]):
        assert torch.equal(a, b)

    # a captured graph, replayed with eager work in between
    cap = buffers()
    g = torch.cuda.CUDAGraph()
    capture_stream = torch.cuda.Stream()
    capture_stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(capture_stream):
        run(fa, q, k, v, do, cap, **kw)  # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(capture_stream)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=capture_stream):
        run(fa, q, k, v, do, cap, **kw)
    for rep in range(4):
        for t in cap[:5] + ((cap[6],) if keep else ()):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref[:5], cap[:5]):
            assert torch.equal(a, b), rep
        if keep:
            assert torch.equal(ref[6], cap[6]), rep
        # unrelated eager work between replays
        (q.float() * 2).sum().item()
