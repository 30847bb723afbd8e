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


def ragged(n, lo, hi, seed):
    return [int(x) for x in np.random.default_rng(seed).integers(lo, hi + 1, n)]


CASES = [
    ("many_heads_tiny_causal", lambda: workloads.custom(64, 40, 5, 128, "bf16", True, seed=41)),
    ("many_heads_short", lambda: workloads.custom(33, 17, 70, 64, "f16", False, seed=42)),
    ("empty_sequences_causal", lambda: workloads.custom(0, 2, 0, 128, "bf16", True, lengths=[0, 5, 0, 130, 0, 1],
                                                        seed=43)),
    ("empty_sequences_dropout", lambda: workloads.custom(0, 3, 0, 64, "f16", False, lengths=[0, 0, 77, 0, 200],
                                                         dropout_p=0.2, seed=44)),
    ("three_hundred_sequences", lambda: workloads.custom(0, 3, 0, 64, "f16", False, lengths=ragged(300, 0, 40, 45),
                                                         seed=45)),
    ("three_hundred_sequences_causal_d96", lambda: workloads.custom(0, 2, 0, 96, "bf16", True,
                                                                    lengths=ragged(300, 1, 90, 46), seed=46)),
]


@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
def test_edge_forward(name, make):
    check_forward(make())


@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
def test_edge_backward(name, make):
    check_backward(make())
