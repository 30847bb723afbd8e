"""Pins for the fp64 CPU oracle (no GPU).

Each test ties the oracle to something other than itself: a hand-worked
example, a closed form, an invariant the mathematics fixes, torch's own fp64
scaled_dot_product_attention and autograd, central finite differences, and
rocRAND's independent Philox-4x32-10 engine.
"""
import json
import math
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden")


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def fwd(q, k, v, scale, causal, **kw):
    """[L, d] single-head helper."""
    o, lse = oracle.forward(q[:, None, :], k[:, None, :], v[:, None, :], scale=scale, causal=causal,
                            N=q.shape[0], **kw)
    return o[:, 0, :], lse[:, 0]


def bwd(q, k, v, do, scale, causal, **kw):
    g = oracle.backward(q[:, None, :], k[:, None, :], v[:, None, :], do[:, None, :], scale=scale,
                        causal=causal, N=q.shape[0], **kw)
    return [x[:, 0, :] for x in g]


# ----------------------------------------------------------------- golden

def test_hand_worked_two_token_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_two_token.json")))
    x = g["inputs"]
    q, k, v, do = (np.array(x[n], dtype=np.float64)[:, None] for n in ("q", "k", "v", "dout"))
    for causal, key in ((False, "noncausal"), (True, "causal")):
        o, lse = fwd(q, k, v, x["scale"], causal)
        np.testing.assert_allclose(o[:, 0], g[key]["o"], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse, g[key]["lse"], rtol=0, atol=1e-14)
    dq, dk, dv = bwd(q, k, v, do, x["scale"], False)
    e = g["noncausal"]
    np.testing.assert_allclose(dq[:, 0], e["dq"], atol=1e-14)
    np.testing.assert_allclose(dk[:, 0], e["dk"], atol=1e-14)
    np.testing.assert_allclose(dv[:, 0], e["dv"], atol=1e-14)


# ----------------------------------------------------------- closed forms

@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_gives_mean_of_visible_values(causal):
    L, d = 37, 8
    q = np.zeros((L, d)); k = rnd((L, d), 1); v = rnd((L, d), 2)
    o, lse = fwd(q, k, v, 0.7, causal)
    for i in range(L):
        n = i + 1 if causal else L
        np.testing.assert_allclose(o[i], v[:n].mean(0), atol=1e-13)
        assert abs(lse[i] - math.log(n)) < 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_identical_key_rows(causal):
    L, d = 29, 16
    u = rnd((d,), 3)
    q = rnd((L, d), 4); k = np.tile(u, (L, 1)); v = rnd((L, d), 5)
    o, lse = fwd(q, k, v, 0.25, causal)
    for i in range(L):
        n = i + 1 if causal else L
        np.testing.assert_allclose(o[i], v[:n].mean(0), atol=1e-13)
        assert abs(lse[i] - (0.25 * q[i] @ u + math.log(n))) < 1e-12


def test_single_dominant_score():
    L, d = 20, 8
    q = rnd((L, d), 6); k = rnd((L, d), 7) * 0.01; v = rnd((L, d), 8)
    i, jstar = 5, 13
    k[jstar] = 400.0 * q[i] / (q[i] @ q[i])        # s_i,j* = scale * 400 dominates the row
    o, _ = fwd(q, k, v, 0.5, False)
    np.testing.assert_allclose(o[i], v[jstar], atol=1e-12)


def test_causal_row_zero_is_first_value():
    L, d = 16, 8
    q, k, v = rnd((L, d), 9), rnd((L, d), 10), rnd((L, d), 11)
    o, lse = fwd(q, k, v, 0.3, True)
    np.testing.assert_allclose(o[0], v[0], atol=0)
    assert abs(lse[0] - 0.3 * q[0] @ k[0]) < 1e-14


# ------------------------------------------------------------- invariants

def test_key_shift_invariance():
    L, d, s = 24, 8, 0.4
    q, k, v = rnd((L, d), 12), rnd((L, d), 13), rnd((L, d), 14)
    u = rnd((d,), 15)
    o1, l1 = fwd(q, k, v, s, True)
    o2, l2 = fwd(q, k + u, v, s, True)
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    np.testing.assert_allclose(l2, l1 + s * q @ u, atol=1e-12)


def test_permutations_and_linearity():
    L, d, s = 19, 8, 0.35
    q, k, v = rnd((L, d), 16), rnd((L, d), 17), rnd((L, d), 18)
    o, lse = fwd(q, k, v, s, False)
    perm = np.random.default_rng(19).permutation(L)
    o_kv, _ = fwd(q, k[perm], v[perm], s, False)
    np.testing.assert_allclose(o_kv, o, atol=1e-12)
    o_q, l_q = fwd(q[perm], k, v, s, False)
    np.testing.assert_allclose(o_q, o[perm], atol=1e-12)
    np.testing.assert_allclose(l_q, lse[perm], atol=1e-12)
    v2 = rnd((L, d), 20)
    o2, _ = fwd(q, k, v2, s, False)
    o3, _ = fwd(q, k, 2.0 * v - 3.0 * v2, s, False)
    np.testing.assert_allclose(o3, 2.0 * o - 3.0 * o2, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_lse_bounds(causal):
    L, d, s = 33, 16, 0.25
    q, k, v = rnd((L, d), 21), rnd((L, d), 22) * 3, rnd((L, d), 23)
    _, lse = fwd(q, k, v, s, causal)
    S = s * q @ k.T
    for i in range(L):
        n = i + 1 if causal else L
        m = S[i, :n].max()
        assert m - 1e-12 <= lse[i] <= m + math.log(n) + 1e-12


# --------------------------------------------------- library cross-check

def _torch_ref(q, k, v, scale, causal):
    """torch fp64 SDPA over [B,H,N,d] from [B,N,H,d]."""
    tq, tk, tv = (torch.tensor(x).permute(0, 2, 1, 3) for x in (q, k, v))
    return torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_fp64(causal):
    B, N, H, d, s = 2, 45, 3, 16, 0.3
    q, k, v = rnd((B, N, H, d), 24), rnd((B, N, H, d), 25), rnd((B, N, H, d), 26)
    o, lse = oracle.forward(q.reshape(-1, H, d), k.reshape(-1, H, d), v.reshape(-1, H, d), scale=s,
                            causal=causal, N=N)
    ref = _torch_ref(q, k, v, s, causal).permute(0, 2, 1, 3).numpy()
    np.testing.assert_allclose(o.reshape(B, N, H, d), ref, atol=1e-12)
    # LSE through torch.logsumexp on a masked score matrix
    S = torch.einsum("bnhd,bmhd->bhnm", torch.tensor(q), torch.tensor(k)) * s
    if causal:
        S = S.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
    ref_lse = torch.logsumexp(S, -1).permute(0, 2, 1).numpy()
    np.testing.assert_allclose(lse.reshape(B, N, H), ref_lse, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_grads_match_torch_autograd_fp64(causal):
    B, N, H, d, s = 1, 33, 2, 8, 0.4
    q, k, v, do = (rnd((B, N, H, d), 30 + t) for t in range(4))
    dq, dk, dv = oracle.backward(*(x.reshape(-1, H, d) for x in (q, k, v, do)), scale=s, causal=causal, N=N)
    tq, tk, tv = (torch.tensor(x).permute(0, 2, 1, 3).requires_grad_() for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=s)
    out.backward(torch.tensor(do).permute(0, 2, 1, 3))
    for mine, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(mine.reshape(B, N, H, d), t.grad.permute(0, 2, 1, 3).numpy(), atol=1e-12)


# ------------------------------------------------- tiled == definition

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Br,Bc", [(1, 1), (3, 3), (16, 16), (64, 64), (37, 37), (3, 16), (16, 3),
                                   (64, 5)])
def test_online_softmax_tiled_equals_definition(causal, Br, Bc):
    L, d, s = 37, 8, 0.5
    q, k, v = rnd((L, d), 40), rnd((L, d), 41) * 4.0, rnd((L, d), 42)
    o, lse = fwd(q, k, v, s, causal)
    ot, lt = oracle.forward_tiled_head(q, k, v, scale=s, causal=causal, Br=Br, Bc=Bc)
    np.testing.assert_allclose(ot, o, atol=1e-12)
    np.testing.assert_allclose(lt, lse, atol=1e-12)


def test_online_softmax_tiled_equals_definition_with_dropout():
    L, d, s = 40, 8, 0.5
    q, k, v = rnd((L, d), 43), rnd((L, d), 44), rnd((L, d), 45)
    o, lse = fwd(q, k, v, s, True, dropout_p=0.3, seed=99)
    ot, lt = oracle.forward_tiled_head(q, k, v, scale=s, causal=True, Br=7, Bc=9, dropout_p=0.3, seed=99)
    np.testing.assert_allclose(ot, o, atol=1e-12)
    np.testing.assert_allclose(lt, lse, atol=1e-12)


# -------------------------------------------------- finite differences

def _loss(q, k, v, do, s, causal, **kw):
    o, _ = fwd(q, k, v, s, causal, **kw)
    return float((o * do).sum())


@pytest.mark.parametrize("L,d", [(6, 4), (16, 8)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p", [0.0, 0.4])
def test_backward_finite_differences(L, d, causal, p):
    s = 0.6
    q, k, v, do = (rnd((L, d), 50 + t) for t in range(4))
    kw = dict(dropout_p=p, seed=1234) if p else {}
    dq, dk, dv = bwd(q, k, v, do, s, causal, **kw)
    h = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for trial in range(3):
            delta = rnd((L, d), 100 + 10 * which + trial)
            args = [q, k, v]
            plus = [a + h * delta if t == which else a for t, a in enumerate(args)]
            minus = [a - h * delta if t == which else a for t, a in enumerate(args)]
            fd = (_loss(*plus, do, s, causal, **kw) - _loss(*minus, do, s, causal, **kw)) / (2 * h)
            an = float((grad * delta).sum())
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (which, fd, an)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_sum_invariants(causal):
    L, d = 31, 8
    q, k, v, do = (rnd((L, d), 60 + t) for t in range(4))
    dq, dk, dv = bwd(q, k, v, do, 0.3, causal)
    np.testing.assert_allclose(dk.sum(0), 0.0, atol=1e-12)           # rows of dS sum to zero
    np.testing.assert_allclose(dv.sum(0), do.sum(0), atol=1e-12)     # columns of P sum ... rows sum to 1


# ------------------------------------------------------------- varlen

def test_varlen_equals_separate_sequences():
    lens = [5, 1, 17, 9]
    H, d, s = 2, 8, 0.4
    T = sum(lens)
    q, k, v, do = (rnd((T, H, d), 70 + t) for t in range(4))
    o, lse = oracle.forward(q, k, v, scale=s, causal=True, lengths=lens)
    dq, dk, dv = oracle.backward(q, k, v, do, scale=s, causal=True, lengths=lens)
    st = 0
    for L in lens:
        sl = slice(st, st + L)
        o1, l1 = oracle.forward(q[sl], k[sl], v[sl], scale=s, causal=True, N=L)
        g1 = oracle.backward(q[sl], k[sl], v[sl], do[sl], scale=s, causal=True, N=L)
        np.testing.assert_array_equal(o[sl], o1)
        np.testing.assert_array_equal(lse[sl], l1)
        for a, b in zip((dq, dk, dv), g1):
            np.testing.assert_array_equal(a[sl], b)
        # and each sequence against torch's SDPA
        ref = _torch_ref(q[None, sl], k[None, sl], v[None, sl], s, True).permute(0, 2, 1, 3).numpy()[0]
        np.testing.assert_allclose(o[sl], ref, atol=1e-12)
        st += L


def test_head_selection_computes_only_requested_heads():
    B, N, H, d = 2, 12, 3, 8
    q, k, v, do = (rnd((B * N, H, d), 80 + t) for t in range(4))
    o, lse = oracle.forward(q, k, v, scale=0.3, causal=True, N=N)
    os_, ls = oracle.forward(q, k, v, scale=0.3, causal=True, N=N, heads=[(1, 2), (0, 1)])
    for b, h in ((1, 2), (0, 1)):
        np.testing.assert_array_equal(os_[b * N:(b + 1) * N, h], o[b * N:(b + 1) * N, h])
        np.testing.assert_array_equal(ls[b * N:(b + 1) * N, h], lse[b * N:(b + 1) * N, h])
    assert np.isnan(os_[0:N, 0]).all()


# -------------------------------------------------------------- dropout

@pytest.fixture(scope="module")
def rocrand_philox(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("philox") / "philox_rocrand")
    subprocess.check_call([hipcc, "--offload-arch=gfx950", "-O1", os.path.join(HERE, "helpers", "philox_rocrand.cpp"),
                           "-o", exe], stderr=subprocess.DEVNULL)
    return exe


def test_philox_matches_rocrand(rocrand_philox):
    rng = np.random.default_rng(90)
    # the helper reaches counter word 1 through a 64-bit offset of 4 * block,
    # so word 1 stays below 2^30 (the attention counter uses col / 4 there)
    cases = [[0, 0, 0, 0, 0, 0], [1, 2, 3, 4, 5, 6], [0xFFFFFFFF, 2**30 - 1] + [0xFFFFFFFF] * 4]
    for _ in range(200):
        c = list(map(int, rng.integers(0, 2**32, 6)))
        c[1] %= 2**30
        cases.append(c)
    inp = "\n".join(" ".join(str(x) for x in c) for c in cases) + "\n"
    out = subprocess.run([rocrand_philox], input=inp, capture_output=True, text=True, check=True).stdout
    ref = [list(map(int, line.split())) for line in out.strip().splitlines()]
    assert len(ref) == len(cases)
    for c, r in zip(cases, ref):
        assert oracle.philox4x32_10(c[:4], c[4:]) == r, c


def test_keep_mask_uses_documented_counter_layout():
    seed, p = 0x123456789ABCDEF0, 0.25
    t = oracle.dropout_threshold(p)
    m = oracle.keep_mask(seed, p, b=3, h=5, L=13)
    assert t == int(0.25 * 65536)
    for i in range(13):
        for j in range(13):
            words = oracle.philox4x32_10([i, j // 8, 5, 3], [seed & 0xFFFFFFFF, seed >> 32])
            value = (words[(j % 8) // 2] >> (16 * (j % 2))) & 0xFFFF
            assert m[i, j] == (value >= t)


def test_keep_threshold_boundary():
    # an element whose 16-bit Philox value equals the threshold is kept; one
    # above is dropped (both halves of a word: columns 6 and 7 share word 3)
    seed, b, h, i = 42, 1, 2, 3
    words = oracle.philox4x32_10([i, 0, h, b], [seed, 0])
    for j, v in ((6, words[3] & 0xFFFF), (7, words[3] >> 16)):
        assert oracle.keep(seed, v, b, h, i, j)
        assert not oracle.keep(seed, v + 1, b, h, i, j)


def test_dropout_threshold_values():
    assert oracle.dropout_threshold(0.1) == 6553           # floor(0.1f * 65536)
    assert oracle.dropout_threshold(0.5) == 32768
    assert oracle.dropout_threshold(0.999) == 65470


def test_keep_rate_statistics():
    p = 0.1
    m = oracle.keep_mask(1005, p, b=0, h=0, L=700)
    n = m.size
    expect = 1.0 - oracle.dropout_threshold(p) / 2**16
    sigma = math.sqrt(n * expect * (1 - expect))
    assert abs(int(m.sum()) - n * expect) < 5 * sigma
    # different heads / batches give different masks
    assert (m != oracle.keep_mask(1005, p, b=0, h=1, L=700)).mean() > 0.1
    assert (m != oracle.keep_mask(1005, p, b=1, h=0, L=700)).mean() > 0.1


def test_dropout_forward_matches_masked_torch_reference():
    L, d, s, p, seed = 23, 8, 0.45, 0.3, 77
    q, k, v = rnd((L, d), 91), rnd((L, d), 92), rnd((L, d), 93)
    for causal in (False, True):
        o, lse = fwd(q, k, v, s, causal, dropout_p=p, seed=seed)
        o_nd, lse_nd = fwd(q, k, v, s, causal)
        np.testing.assert_allclose(lse, lse_nd, atol=0)          # LSE excludes dropout
        S = torch.tensor(q) @ torch.tensor(k).T * s
        if causal:
            S = S.masked_fill(torch.triu(torch.ones(L, L, dtype=torch.bool), 1), float("-inf"))
        P = torch.softmax(S, -1)
        keep = torch.tensor(oracle.keep_mask(seed, p, 0, 0, L), dtype=torch.float64)
        ref = (P * keep / (1.0 - float(np.float32(p)))) @ torch.tensor(v)
        np.testing.assert_allclose(o, ref.numpy(), atol=1e-12)


def test_dropout_one_hot_probe_recovers_mask():
    # Q = K = 0 and one-hot V rows: O[i][c] = keep(i, o + c) / (n_i (1 - p))
    L, d, p, seed = 24, 8, 0.5, 5
    q = np.zeros((L, d)); k = np.zeros((L, d))
    for off in range(0, L, d):
        v = np.zeros((L, d))
        for c in range(d):
            if off + c < L:
                v[off + c, c] = 1.0
        o, _ = fwd(q, k, v, 1.0, True, dropout_p=p, seed=seed)
        mask = oracle.keep_mask(seed, p, 0, 0, L)
        for i in range(L):
            for c in range(d):
                j = off + c
                want = mask[i, j] / ((i + 1) * (1 - p)) if j <= i else 0.0
                assert abs(o[i, c] - want) < 1e-14


def test_tiny_dropout_probability_equals_no_dropout():
    L, d = 20, 8
    q, k, v = rnd((L, d), 94), rnd((L, d), 95), rnd((L, d), 96)
    assert oracle.dropout_threshold(1e-12) == 0          # every element kept
    o1, _ = fwd(q, k, v, 0.5, True, dropout_p=1e-12, seed=3)
    o2, _ = fwd(q, k, v, 0.5, True)
    np.testing.assert_allclose(o1, o2, atol=1e-12)


# ------------------------------------------------------------ block mask
# Block-sparse attention (the block-sparse mode of the coreui.cn
# FlashAttention-2 how-to, section 5.2): element (i, j) is visible only where the block mask entry of
# (i // block, j // block) is nonzero.

def _element_mask(bm, N, block, causal):
    """[B, H, N, N] boolean element mask (True = visible) from a block mask."""
    idx = np.arange(N) // block
    m = bm[:, :, idx][:, :, :, idx].astype(bool)
    if causal:
        m = m & np.tril(np.ones((N, N), dtype=bool))
    return m


def _random_block_mask(B, H, nb, seed, density=0.5):
    bm = (np.random.default_rng(seed).random((B, H, nb, nb)) < density).astype(np.uint8)
    for r in range(nb):
        bm[:, :, r, r] = 1  # every row keeps its diagonal block: no empty row
    return bm


@pytest.mark.parametrize("causal", [False, True])
def test_block_mask_matches_torch_sdpa_fp64(causal):
    B, N, H, d, s, blk = 2, 45, 3, 16, 0.3, 8
    nb = -(-N // blk)
    q, k, v = rnd((B, N, H, d), 200), rnd((B, N, H, d), 201), rnd((B, N, H, d), 202)
    bm = _random_block_mask(B, H, nb, 203)
    o, lse = oracle.forward(q.reshape(-1, H, d), k.reshape(-1, H, d), v.reshape(-1, H, d), scale=s,
                            causal=causal, N=N, block_mask=bm, block=blk)
    em = torch.tensor(_element_mask(bm, N, blk, causal))
    tq, tk, tv = (torch.tensor(x).permute(0, 2, 1, 3) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=em, scale=s)
    np.testing.assert_allclose(o.reshape(B, N, H, d), ref.permute(0, 2, 1, 3).numpy(), atol=1e-12)
    S = torch.einsum("bhnd,bhmd->bhnm", tq, tk) * s
    ref_lse = torch.logsumexp(S.masked_fill(~em, float("-inf")), -1).permute(0, 2, 1).numpy()
    np.testing.assert_allclose(lse.reshape(B, N, H), ref_lse, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_block_mask_grads_match_torch_autograd_fp64(causal):
    B, N, H, d, s, blk = 1, 37, 2, 8, 0.4, 6
    nb = -(-N // blk)
    q, k, v, do = (rnd((B, N, H, d), 210 + t) for t in range(4))
    bm = _random_block_mask(B, H, nb, 215)
    dq, dk, dv = oracle.backward(*(x.reshape(-1, H, d) for x in (q, k, v, do)), scale=s, causal=causal, N=N,
                                 block_mask=bm, block=blk)
    em = torch.tensor(_element_mask(bm, N, blk, causal))
    tq, tk, tv = (torch.tensor(x).permute(0, 2, 1, 3).requires_grad_() for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=em, scale=s)
    out.backward(torch.tensor(do).permute(0, 2, 1, 3))
    for mine, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(mine.reshape(B, N, H, d), t.grad.permute(0, 2, 1, 3).numpy(), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_block_mask_all_ones_equals_dense(causal):
    N, H, d, blk = 29, 2, 8, 8
    q, k, v, do = (rnd((N, H, d), 220 + t) for t in range(4))
    bm = np.ones((1, H, 4, 4), dtype=np.uint8)
    o0, l0 = oracle.forward(q, k, v, scale=0.5, causal=causal, N=N)
    o1, l1 = oracle.forward(q, k, v, scale=0.5, causal=causal, N=N, block_mask=bm, block=blk)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    g0 = oracle.backward(q, k, v, do, scale=0.5, causal=causal, N=N)
    g1 = oracle.backward(q, k, v, do, scale=0.5, causal=causal, N=N, block_mask=bm, block=blk)
    for a, b in zip(g0, g1):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("causal", [False, True])
def test_block_diagonal_mask_equals_separate_sequences(causal):
    # a block-diagonal mask cuts one sequence into independent pieces of one
    # block each, which is what the varlen layout computes
    N, H, d, blk = 40, 2, 8, 8
    nb = N // blk
    q, k, v, do = (rnd((N, H, d), 230 + t) for t in range(4))
    bm = np.zeros((1, H, nb, nb), dtype=np.uint8)
    for r in range(nb):
        bm[0, :, r, r] = 1
    o1, l1 = oracle.forward(q, k, v, scale=0.7, causal=causal, N=N, block_mask=bm, block=blk)
    o2, l2 = oracle.forward(q, k, v, scale=0.7, causal=causal, lengths=[blk] * nb)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)
    g1 = oracle.backward(q, k, v, do, scale=0.7, causal=causal, N=N, block_mask=bm, block=blk)
    g2 = oracle.backward(q, k, v, do, scale=0.7, causal=causal, lengths=[blk] * nb)
    for a, b in zip(g1, g2):
        np.testing.assert_allclose(a, b, atol=1e-13)


def test_block_mask_empty_rows_and_unseen_keys():
    N, d, blk = 24, 8, 8
    q, k, v, do = (rnd((N, d), 240 + t) for t in range(4))
    bm = np.ones((1, 1, 3, 3), dtype=np.uint8)
    bm[0, 0, 1, :] = 0      # queries 8..15 see nothing
    bm[0, 0, :, 2] = 0      # keys 16..23 are seen by no query
    o, lse = fwd(q, k, v, 0.5, False, block_mask=bm, block=blk)
    assert np.all(o[8:16] == 0.0) and np.all(np.isneginf(lse[8:16]))
    assert np.all(np.isfinite(lse[:8])) and np.all(np.isfinite(lse[16:]))
    dq, dk, dv = bwd(q, k, v, do, 0.5, False, block_mask=bm, block=blk)
    assert np.all(dq[8:16] == 0.0)
    assert np.all(dk[16:] == 0.0) and np.all(dv[16:] == 0.0)
    # the remaining rows see exactly keys 0..15: plain attention over them
    S = q @ k[:16].T * 0.5
    P = np.exp(S - S.max(1, keepdims=True))
    P /= P.sum(1, keepdims=True)
    np.testing.assert_allclose(o[:8], (P @ v[:16])[:8], atol=1e-12)
    np.testing.assert_allclose(o[16:], (P @ v[:16])[16:], atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_block_mask_backward_finite_differences(causal):
    L, d, s, blk = 12, 4, 0.6, 4
    q, k, v, do = (rnd((L, d), 250 + t) for t in range(4))
    bm = np.array([[[[1, 0, 1], [0, 0, 0], [1, 1, 0]]]], dtype=np.uint8)  # row block 1 empty
    kw = dict(block_mask=bm, block=blk)
    dq, dk, dv = bwd(q, k, v, do, s, causal, **kw)

    def loss(qq, kk, vv):
        o, _ = fwd(qq, kk, vv, s, causal, **kw)
        return float((o * do).sum())

    h = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for trial in range(3):
            delta = rnd((L, d), 260 + 10 * which + trial)
            args = [q, k, v]
            plus = [a + h * delta if t == which else a for t, a in enumerate(args)]
            minus = [a - h * delta if t == which else a for t, a in enumerate(args)]
            fd = (loss(*plus) - loss(*minus)) / (2 * h)
            an = float((grad * delta).sum())
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (which, fd, an)


# ------------------------------------------------------------ KV-cache decode
# The decode step (lab write-up, section 6.1): nq new queries at the end of
# their sequence attend to the cached keys and values.

@pytest.mark.parametrize("nq", [1, 3, 40])
def test_decode_is_the_last_rows_of_causal_attention(nq):
    L, H, d = 40, 2, 8
    q, k, v = rnd((L, H, d), 600), rnd((L, H, d), 601), rnd((L, H, d), 602)
    o_full, l_full = oracle.forward(q, k, v, scale=0.4, causal=True, N=L)
    o, lse = oracle.decode(q[None, L - nq:], k[None], v[None], scale=0.4, causal=True)
    np.testing.assert_allclose(o[0], o_full[L - nq:], atol=1e-13)
    np.testing.assert_allclose(lse[0], l_full[L - nq:], atol=1e-13)


def test_decode_matches_torch_sdpa_fp64():
    B, H, d, nk, nq = 3, 2, 16, 50, 4
    q, kc, vc = rnd((B, nq, H, d), 610), rnd((B, nk, H, d), 611), rnd((B, nk, H, d), 612)
    lens = [50, 17, 4]
    for causal in (False, True):
        o, lse = oracle.decode(q, kc, vc, scale=0.3, causal=causal, seqlens_k=lens)
        for b, L in enumerate(lens):
            tq, tk, tv = (torch.tensor(x[b]).permute(1, 0, 2) for x in (q, kc[:, :L], vc[:, :L]))
            mask = None
            if causal:  # bottom-right: query t sees keys j <= L - nq + t
                mask = torch.arange(L)[None, :] <= (L - nq + torch.arange(nq))[:, None]
            ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=0.3)
            np.testing.assert_allclose(o[b], ref.permute(1, 0, 2).numpy(), atol=1e-12)
            S = torch.einsum("htd,hjd->htj", tq, tk) * 0.3
            if mask is not None:
                S = S.masked_fill(~mask, float("-inf"))
            np.testing.assert_allclose(lse[b], torch.logsumexp(S, -1).T.numpy(), atol=1e-12)


def test_decode_queries_that_see_no_key():
    # causal with fewer cached keys than new queries: the first queries see nothing
    B, H, d, nk, nq = 1, 1, 8, 6, 4
    q, kc, vc = rnd((B, nq, H, d), 620), rnd((B, nk, H, d), 621), rnd((B, nk, H, d), 622)
    o, lse = oracle.decode(q, kc, vc, scale=0.5, causal=True, seqlens_k=[2])
    # L - nq + t + 1 = t - 1 keys: t = 0, 1 see none, t = 2 sees key 0, t = 3 keys 0, 1
    assert np.all(o[0, :2] == 0.0) and np.all(np.isneginf(lse[0, :2]))
    np.testing.assert_allclose(o[0, 2, 0], vc[0, 0, 0], atol=1e-15)
    assert np.isclose(lse[0, 2, 0], 0.5 * float(q[0, 2, 0] @ kc[0, 0, 0]), atol=1e-14)


def paged_from_contiguous(kc, P, rng, spare=3):
    """Scatter a contiguous [B, nk, H, d] cache into a shuffled page pool:
    page p of sequence b goes to pool slot perm[b * max_pages + p]; `spare`
    unused slots hold NaN.  Returns (pool, table)."""
    B, nk, H, d = kc.shape
    max_pages = nk // P
    n = B * max_pages + spare
    perm = rng.permutation(n)
    pool = np.full((n, P, H, d), np.nan)
    table = np.zeros((B, max_pages), dtype=np.int32)
    for b in range(B):
        for p in range(max_pages):
            slot = perm[b * max_pages + p]
            pool[slot] = kc[b, p * P:(p + 1) * P]
            table[b, p] = slot
    return pool, table


@pytest.mark.parametrize("P,causal", [(4, False), (8, True), (1, True), (32, False)])
def test_decode_paged_equals_contiguous_decode(P, causal):
    # the cache scattered page by page into a shuffled pool (with unused NaN
    # pages, and table entries past each length set to -1) decodes exactly as
    # the contiguous cache does
    B, H, d, nq, nk = 3, 2, 8, 3, 32
    q, kc, vc = rnd((B, nq, H, d), 630), rnd((B, nk, H, d), 631), rnd((B, nk, H, d), 632)
    lens = np.array([32, 13, 0], dtype=np.int32)
    rng = np.random.default_rng(P)
    kp, table = paged_from_contiguous(kc, P, rng)
    vp, table_v = paged_from_contiguous(vc, P, np.random.default_rng(P))
    assert (table == table_v).all()
    for b in range(B):
        table[b, (lens[b] + P - 1) // P:] = -1
    o_ref, lse_ref = oracle.decode(q, kc, vc, scale=0.4, causal=causal, seqlens_k=lens)
    o, lse = oracle.decode_paged(q, kp, vp, table, scale=0.4, causal=causal, seqlens_k=lens)
    assert np.array_equal(o, o_ref) and np.array_equal(lse, lse_ref)


def test_decode_paged_rejects_entries_outside_the_pool():
    q, kp, vp = rnd((1, 1, 1, 4), 640), rnd((2, 4, 1, 4), 641), rnd((2, 4, 1, 4), 642)
    with pytest.raises(ValueError):
        oracle.decode_paged(q, kp, vp, np.array([[0, 2]], dtype=np.int32), scale=1.0, causal=False)


@pytest.mark.parametrize("causal", [False, True])
def test_rows_head_equals_full_head(causal):
    # the row-subset oracle (for sequences too long to form P) gives the same
    # O, LSE and dQ rows as the full-head definition, on a strided head view
    L, H, d, s = 41, 3, 8, 0.37
    q, k, v, do = (rnd((L, H, d), 700 + i) for i in range(4))
    o, lse = oracle.forward(q, k, v, scale=s, causal=causal, N=L)
    dq, _, _ = oracle.backward(q, k, v, do, scale=s, causal=causal, N=L)
    rows = [0, 1, 5, 17, 39, 40]
    for h in range(H):
        ro, rl, rdq = oracle.rows_head(q[:, h], k[:, h], v[:, h], do[:, h], scale=s, causal=causal, rows=rows)
        np.testing.assert_allclose(ro, o[rows, h], atol=1e-13)
        np.testing.assert_allclose(rl, lse[rows, h], atol=1e-13)
        np.testing.assert_allclose(rdq, dq[rows, h], atol=1e-13)
    ro, rl, none = oracle.rows_head(q[:, 0], k[:, 0], v[:, 0], scale=s, causal=causal, rows=rows)
    assert none is None
    np.testing.assert_allclose(ro, o[rows, 0], atol=1e-13)


@pytest.mark.parametrize("openmp", [False, True])
def test_oracle_runs_clean_under_sanitizers(tmp_path, openmp):
    # every oracle entry point on exactly sized heap buffers (empty sequences,
    # block masks, dropout, head selection, decode with an empty cache, row
    # subsets) under AddressSanitizer + UndefinedBehaviorSanitizer, serial and
    # with OpenMP threads
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_sanitize")
    cmd = [gcc, "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", os.path.join(os.path.dirname(HERE), "oracle", "oracle.c"),
           os.path.join(HERE, "helpers", "oracle_sanitize.c"), "-lm", "-o", exe]
    if openmp:
        cmd.insert(1, "-fopenmp")
    subprocess.check_call(cmd)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", OMP_NUM_THREADS="4")
    r = subprocess.run([exe], capture_output=True, text=True, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "clean" in r.stdout
