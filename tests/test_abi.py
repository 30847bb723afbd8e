"""Host-side tests of the C-ABI library (no GPU needed).

The library validates every argument on the host before its first HIP call,
so each error code can be forced here without a device.  Valid calls are
never made on the CPU.
"""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))
HEADER = os.path.join(ROOT, "include", "fa.h")
LIB = os.path.join(ROOT, "exact_tiled_attention_40_amd", "libfa.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libfa.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(fa_[a-z_0-9]+)\s*\(", src, flags=re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted([
        "fa_backward", "fa_backward_block_sparse", "fa_backward_block_sparse_stage", "fa_backward_keep",
        "fa_backward_keep_stage", "fa_backward_noalloc", "fa_backward_stage",
        "fa_backward_workspace_size", "fa_decode", "fa_decode_paged", "fa_decode_workspace_size",
        "fa_dropout_bits_size", "fa_dropout_mask", "fa_forward", "fa_forward_block_sparse", "fa_forward_keep",
        "fa_strerror"])


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for name in declared_functions():
        assert name in exported, name
    lib = ctypes.CDLL(LIB)
    for name in declared_functions():
        getattr(lib, name)


@pytest.fixture(scope="module")
def lib():
    L = ctypes.CDLL(LIB)
    vp, i, f, i64, u64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_int64, ctypes.c_uint64
    L.fa_forward.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, f, u64, vp, i, i64]
    L.fa_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, f, u64, vp, i, i64, vp,
                              ctypes.c_size_t]
    L.fa_backward_stage.argtypes = [i] + L.fa_backward.argtypes
    L.fa_backward_workspace_size.argtypes = [i, i, i, i]
    L.fa_backward_workspace_size.restype = ctypes.c_size_t
    L.fa_dropout_mask.argtypes = [vp, i, i, i, f, u64, vp]
    L.fa_forward_block_sparse.argtypes = L.fa_forward.argtypes + [vp]
    L.fa_backward_block_sparse.argtypes = L.fa_backward.argtypes + [vp]
    L.fa_backward_block_sparse_stage.argtypes = [i] + L.fa_backward_block_sparse.argtypes
    L.fa_decode_workspace_size.argtypes = [i, i, i, i, i]
    L.fa_decode_workspace_size.restype = ctypes.c_size_t
    L.fa_decode.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, i, vp, ctypes.c_size_t]
    L.fa_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp, i, vp, ctypes.c_size_t]
    L.fa_dropout_bits_size.argtypes = [i, i, i]
    L.fa_dropout_bits_size.restype = ctypes.c_size_t
    L.fa_forward_keep.argtypes = L.fa_forward.argtypes + [vp, ctypes.c_size_t]
    L.fa_backward_keep.argtypes = L.fa_backward.argtypes + [vp, ctypes.c_size_t]
    L.fa_backward_keep_stage.argtypes = [i] + L.fa_backward_keep.argtypes
    L.fa_strerror.argtypes = [i]
    L.fa_strerror.restype = ctypes.c_char_p
    return L


P = 0x10000  # a fake, 16-byte aligned "device" address: never dereferenced on error paths

FWD_OK = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=2, N=128, d=64, scale=0.125, causal=0, cu=None, p=0.0,
              seed=0, stream=None, dtype=1, ld=0)


def fwd(lib, **over):
    a = dict(FWD_OK, **over)
    return lib.fa_forward(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"], a["scale"],
                          a["causal"], a["cu"], a["p"], a["seed"], a["stream"], a["dtype"], a["ld"])


@pytest.mark.parametrize("over,code", [
    (dict(q=None), 1), (dict(lse=None), 1), (dict(o=None), 1),
    (dict(B=0), 2), (dict(H=0), 2), (dict(N=0), 2), (dict(N=-5), 2), (dict(B=70000, N=70000), 2),
    (dict(d=16), 3), (dict(d=48), 3), (dict(d=224), 3), (dict(d=288), 3), (dict(dtype=2), 3), (dict(dtype=-1), 3),
    (dict(scale=float("nan")), 4), (dict(scale=float("inf")), 4), (dict(scale=0.0), 4), (dict(scale=-1.0), 4),
    (dict(p=1.0), 4), (dict(p=-0.1), 4), (dict(p=float("nan")), 4),
    (dict(ld=100), 5), (dict(ld=127), 5), (dict(q=P + 8), 5), (dict(o=P + 2), 5), (dict(lse=P + 4), 5),
    (dict(ld=(1 << 24) + 8), 3), (dict(H=(1 << 18) + 1, d=64), 3),
])
def test_forward_rejects_bad_arguments(lib, over, code):
    assert fwd(lib, **over) == code


def test_backward_checks(lib):
    need = lib.fa_backward_workspace_size(1, 128, 2, 64)
    assert need >= 128 * 2 * 4

    def bwd(ws=P, nbytes=None, **over):
        a = dict(FWD_OK, **over)
        return lib.fa_backward(a["q"], a["k"], a["v"], a["o"], a["lse"], P, P, P, P, a["B"], a["H"], a["N"], a["d"],
                               a["scale"], a["causal"], a["cu"], a["p"], a["seed"], None, a["dtype"], a["ld"], ws,
                               need if nbytes is None else nbytes)
    assert bwd(ws=None) == 6
    assert bwd(nbytes=need - 1) == 6
    assert bwd(ws=P + 4) == 5
    assert bwd(d=80) == 3
    assert bwd(q=None) == 1
    assert bwd(scale=0.0) == 4
    a = dict(FWD_OK)
    for stage in (-1, 2):
        assert lib.fa_backward_stage(stage, P, P, P, P, P, P, P, P, P, 1, 2, 128, 64, 0.125, 0, None, 0.0, 0, None, 1,
                                     0, P, need) == 4
    assert lib.fa_backward_stage(1, P, P, P, P, P, P, P, P, P, 1, 2, 128, 80, 0.125, 0, None, 0.0, 0, None, 1, 0,
                                 P, need) == 3


def test_workspace_size_edge_cases(lib):
    assert lib.fa_backward_workspace_size(0, 1, 1, 64) == 0
    assert lib.fa_backward_workspace_size(1, 1, 1, 64) > 0
    assert lib.fa_backward_workspace_size(2**31 - 1, 2**31 - 1, 2**31 - 1, 128) == 0   # overflow


def test_dropout_bits_checks(lib):
    # one bit per (query, key) pair, keys padded to 64 per query
    assert lib.fa_dropout_bits_size(2, 100, 3) == 2 * 3 * 100 * 128 // 8
    assert lib.fa_dropout_bits_size(1, 4096, 1) == 4096 * 4096 // 8
    assert lib.fa_dropout_bits_size(1, 101, 1) == 2 * 2 * 104 * 4   # rows padded to a multiple of 4
    assert lib.fa_dropout_bits_size(1, 65537, 1) == 0
    assert lib.fa_dropout_bits_size(0, 64, 1) == 0
    need = lib.fa_backward_workspace_size(1, 128, 2, 64)
    kneed = lib.fa_dropout_bits_size(1, 128, 2)
    fargs = [P, P, P, P, P, 1, 2, 128, 64, 0.125, 1, None, 0.1, 3, None, 1, 0]
    assert lib.fa_forward_keep(*fargs, None, kneed) == 1
    assert lib.fa_forward_keep(*fargs, P, kneed - 1) == 6
    assert lib.fa_forward_keep(*fargs, P + 4, kneed) == 5
    bargs = [P] * 9 + [1, 2, 128, 64, 0.125, 1, None, 0.1, 3, None, 1, 0, P, need]
    assert lib.fa_backward_keep(*bargs, None, kneed) == 1
    assert lib.fa_backward_keep(*bargs, P, 0) == 6
    assert lib.fa_backward_keep_stage(5, *bargs, P, kneed) == 4
    assert lib.fa_backward_keep(*bargs[:12], 80, *bargs[13:], P, kneed) == 3


def test_dropout_mask_checks(lib):
    assert lib.fa_dropout_mask(None, 0, 0, 8, 0.1, 1, None) == 1
    assert lib.fa_dropout_mask(P, 0, 0, 0, 0.1, 1, None) == 2
    assert lib.fa_dropout_mask(P, -1, 0, 8, 0.1, 1, None) == 2
    assert lib.fa_dropout_mask(P, 0, 0, 8, 1.5, 1, None) == 4


def test_strerror_covers_every_code(lib):
    msgs = [lib.fa_strerror(c).decode() for c in range(9)]
    assert len(set(msgs)) == 9
    assert lib.fa_strerror(99).decode().startswith("unknown")


def test_binding_fails_loudly_without_library(tmp_path):
    # the Python binding has no fallback: with libfa.so missing, import raises
    import shutil
    import sys
    pkg = tmp_path / "exact_tiled_attention_40_amd"
    shutil.copytree(os.path.join(ROOT, "exact_tiled_attention_40_amd"), pkg,
                    ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    code = "import exact_tiled_attention_40_amd"
    r = subprocess.run([sys.executable, "-c", code], cwd=tmp_path, capture_output=True, text=True)
    assert r.returncode != 0 and "libfa.so is missing" in r.stderr


# ------------------------------------------------------------ block-sparse

def fwd_bs(lib, mask=P, **over):
    a = dict(FWD_OK, **over)
    return lib.fa_forward_block_sparse(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"],
                                       a["scale"], a["causal"], a["cu"], a["p"], a["seed"], a["stream"],
                                       a["dtype"], a["ld"], mask)


def test_block_sparse_forward_rejects_bad_arguments(lib):
    assert fwd_bs(lib, mask=None) == 1                    # no mask
    assert fwd_bs(lib, N=65537) == 3                      # longer than FA_MASK_MAX_N
    assert fwd_bs(lib, q=None) == 1                       # the dense checks still apply
    assert fwd_bs(lib, d=224) == 3
    assert fwd_bs(lib, scale=float("nan")) == 4
    assert fwd_bs(lib, o=P + 2) == 5


def test_block_sparse_backward_rejects_bad_arguments(lib):
    need = lib.fa_backward_workspace_size(1, 128, 2, 64)

    def call(mask=P, N=128, ws=P, wsb=need):
        return lib.fa_backward_block_sparse(P, P, P, P, P, P, P, P, P, 1, 2, N, 64, 0.125, 0, None, 0.0, 0,
                                            None, 1, 0, ws, wsb, mask)
    assert call(mask=None) == 1
    assert call(N=70000, wsb=lib.fa_backward_workspace_size(1, 70000, 2, 64)) == 3
    assert call(ws=None) == 6
    assert call(wsb=need - 1) == 6
    stage_args = (P, P, P, P, P, P, P, P, P, 1, 2, 128, 64, 0.125, 0, None, 0.0, 0, None, 1, 0, P, need)
    assert lib.fa_backward_block_sparse_stage(2, *stage_args, P) == 4
    assert lib.fa_backward_block_sparse_stage(-1, *stage_args, P) == 4
    assert lib.fa_backward_block_sparse_stage(0, *stage_args, None) == 1


# ------------------------------------------------------------ decode

def test_decode_workspace_size(lib):
    # B * H * ceil(nk / 1024) * nq * (d + 2) floats
    assert lib.fa_decode_workspace_size(2, 3, 4, 1000, 128) == 2 * 3 * 1 * 4 * 130 * 4
    assert lib.fa_decode_workspace_size(2, 3, 4, 1025, 128) == 2 * 3 * 2 * 4 * 130 * 4
    assert lib.fa_decode_workspace_size(1, 1, 1, 512, 64) == 66 * 4
    assert lib.fa_decode_workspace_size(0, 1, 1, 512, 64) == 0
    assert lib.fa_decode_workspace_size(1, 1, 1, 0, 64) == 0


def test_decode_rejects_bad_arguments(lib):
    need = lib.fa_decode_workspace_size(1, 2, 1, 1024, 128)

    def call(q=P, k=P, v=P, lens=None, o=P, lse=P, B=1, H=2, nq=1, nk=1024, d=128, scale=0.1, causal=0, dtype=1,
             ws=P, wsb=need):
        return lib.fa_decode(q, k, v, lens, o, lse, B, H, nq, nk, d, scale, causal, None, dtype, ws, wsb)
    assert call(q=None) == 1 and call(k=None) == 1 and call(lse=None) == 1
    assert call(B=0) == 2 and call(H=0) == 2 and call(nq=0) == 2 and call(nk=0) == 2
    assert call(nq=9) == 3 and call(d=32) == 3 and call(d=96) == 3 and call(dtype=7) == 3
    assert call(scale=float("nan")) == 4 and call(scale=0.0) == 4
    assert call(q=P + 8) == 5 and call(lse=P + 4) == 5 and call(lens=P + 2) == 5
    assert call(ws=None) == 6 and call(wsb=need - 1) == 6
    assert call(ws=P + 4) == 5


def test_decode_paged_rejects_bad_arguments(lib):
    need = lib.fa_decode_workspace_size(1, 2, 1, 16 * 64, 128)

    def call(q=P, k=P, v=P, table=P, lens=None, o=P, lse=P, B=1, H=2, nq=1, num_pages=20, page_size=64,
             max_pages=16, d=128, scale=0.1, causal=0, dtype=1, ws=P, wsb=need):
        return lib.fa_decode_paged(q, k, v, table, lens, o, lse, B, H, nq, num_pages, page_size, max_pages, d, scale,
                                   causal, None, dtype, ws, wsb)
    assert call(table=None) == 1 and call(k=None) == 1 and call(o=None) == 1
    assert call(num_pages=0) == 2 and call(page_size=0) == 2 and call(max_pages=0) == 2 and call(B=0) == 2
    assert call(page_size=48) == 3 and call(page_size=3) == 3 and call(nq=9) == 3 and call(d=96) == 3
    assert call(page_size=1 << 30, max_pages=4) == 2          # capacity above 2^31 - 1 tokens
    assert call(table=P + 2) == 5 and call(lens=P + 2) == 5 and call(v=P + 8) == 5
    assert call(wsb=need - 1) == 6 and call(ws=None) == 6
    assert call(scale=float("inf")) == 4


def test_abi_front_end_under_sanitizers(tmp_path):
    # fa_api.cpp built for the host with AddressSanitizer + UBSan against
    # recording stubs of the kernel launchers: every entry point's error and
    # accepted paths, and the launch description the launchers receive
    # (dropout threshold and scale, token stride, mask blocks, workspace
    # carving, backward stages).  No GPU, no HIP runtime call.
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "abi_host_check")
    host_sanitizers = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined".split()
    subprocess.check_call([hipcc, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", *host_sanitizers,
                           "-fno-omit-frame-pointer", "-I" + os.path.join(ROOT, "include"),
                           os.path.join(ROOT, "exact_tiled_attention_40_amd", "csrc", "fa_api.cpp"),
                           os.path.join(HERE, "helpers", "abi_host_check.cpp"), "-o", exe],
                          stderr=subprocess.DEVNULL)
    r = subprocess.run([exe], capture_output=True, text=True, env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0"))
    assert r.returncode == 0, r.stdout + r.stderr
    assert "clean" in r.stdout


# ------------------------------------------------------------ binding checks

def test_binding_rejects_mismatched_outputs_before_the_library():
    # the binding checks every caller-given output and auxiliary tensor before
    # a pointer reaches the library (CPU tensors here: a call that passed
    # the checks would need a GPU, so only rejections are exercised)
    import torch
    import exact_tiled_attention_40_amd as fa
    q = torch.zeros(1, 8, 2, 64, dtype=torch.bfloat16)
    bad_out = [torch.zeros(1, 8, 2, 32, dtype=torch.bfloat16), torch.zeros(1, 8, 2, 64, dtype=torch.float16),
               torch.zeros(1, 8, 64, 2, dtype=torch.bfloat16).transpose(2, 3)]
    for out in bad_out:
        with pytest.raises(ValueError):
            fa.fa_forward(q, q, q, out=out)
    for lse in (torch.zeros(1, 8, 2, dtype=torch.float16), torch.zeros(1, 8, 3), torch.zeros(1, 2, 8).transpose(1, 2)):
        with pytest.raises(ValueError):
            fa.fa_forward(q, q, q, out=torch.zeros_like(q), lse=lse)
    lse = torch.zeros(1, 8, 2)
    for o, dout, l in ((q[..., :32], q, lse), (q, q.float(), lse), (q, q, lse.double()), (q, q, lse[:, :4])):
        with pytest.raises(ValueError):
            fa.fa_backward(q, q, q, o, l, dout)
    with pytest.raises(ValueError):
        fa.fa_backward(q, q, q, q, lse, q, workspace=torch.zeros(64, dtype=torch.uint8)[::2])
    qv = torch.zeros(20, 2, 64, dtype=torch.bfloat16)
    for cu in (torch.tensor([0, 20], dtype=torch.int64), torch.tensor([0, 20], dtype=torch.int32)):
        with pytest.raises(ValueError):  # int64, or not on the device
            fa.fa_forward(qv, qv, qv, cu_seqlens=cu, max_seqlen=20)


def test_noalloc_backward_rejects_before_any_hip_call(lib):
    vp, i, f, i64, u64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_int64, ctypes.c_uint64
    lib.fa_backward_noalloc.argtypes = [vp] * 9 + [i, i, i, i, f, i, vp, f, u64, vp, i, i64]

    def call(B=1, H=1, N=128, d=64, p=0.0, first=P):
        return lib.fa_backward_noalloc(first, P, P, P, P, P, P, P, P, B, H, N, d, 0.125, 1, None, p, 0, None, 1, 0)

    max_rows = 1 << 22
    assert call(N=max_rows + 1) == 8                  # FA_ERR_SCRATCH_LIMIT
    assert call(B=4, H=32, N=32769, d=128) == 8
    assert call(first=None) == 1 and call(d=80) == 3 and call(p=1.0) == 4
    assert "FA_NOALLOC_MAX_ROWS" in lib.fa_strerror(8).decode()
    assert lib.fa_backward_workspace_size(1, max_rows, 1, 64) == 2 * 4 * max_rows   # the scratch holds the limit
