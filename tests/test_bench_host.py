"""Host-side pieces of bench.py that need no GPU: the visible-pair counts
behind the flop convention, and the shader-clock reader."""
import numpy as np

import bench
import workloads


def test_visible_pairs_counts():
    wl = workloads.WORKLOADS[workloads.HEADLINE]          # causal B4 H8 N4096
    assert bench.visible_pairs(wl) == 4 * 8 * 4096 * 4097 // 2 == 268_500_992
    wl2 = workloads.WORKLOADS["packed_qkv_B2_H12_N2048_d64_f16"]   # non-causal
    assert bench.visible_pairs(wl2) == 2 * 12 * 2048 * 2048


def test_visible_pairs_under_full_block_mask_equals_dense():
    wl = workloads.WORKLOADS[workloads.HEADLINE]
    nb = (wl.N + 127) // 128
    full = np.ones((wl.B, wl.H, nb, nb), np.uint8)
    # the causal pair count only sees the lower triangle; upper blocks add nothing
    assert bench.visible_pairs_masked(wl, full) == bench.visible_pairs(wl)
    diag = np.zeros_like(full)
    diag[..., np.arange(nb), np.arange(nb)] = 1
    assert bench.visible_pairs_masked(wl, diag) == wl.B * wl.H * nb * (128 * 129 // 2)


def test_clock_reader_parses_current_level(tmp_path):
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("0: 500Mhz\n1: 1987Mhz *\n2: 2400Mhz\n")
    c = bench.ClockSampler()
    c.path = str(f)
    assert c._read() == 1987
    f.write_text("0: 500Mhz\n1: 2100Mhz\n")   # no current marker
    assert c._read() is None
    c.samples = [300, 900, 2000, 1900, 2100, 2050]   # ramping up from idle, then settled
    s = c.summary()
    assert (s["median"], s["min"], s["max"], s["samples"]) == (2050, 1900, 2100, 3)


def test_cpu_baseline_reports_forward_and_backward():
    wl = workloads.WORKLOADS["tiny_B1_H2_N128_d64_f16"]
    x = workloads.make_inputs(wl)
    r = bench.cpu_baseline(wl, x, 0, repeats=3, warmup=1)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["cores"] == min(2, r["host_threads"])
    pairs = 2 * 128 * 128
    assert abs(r["fwd"]["gflop"] - 4 * 64 * pairs / 1e9) < 1e-12
    assert abs(r["bwd"]["gflop"] - 10 * 64 * pairs / 1e9) < 1e-12
    assert r["fwd"]["seconds"] > 0 and r["bwd"]["seconds"] > 0
    assert abs(r["value"] - 14 * 64 * pairs / (r["fwd"]["seconds"] + r["bwd"]["seconds"]) / 1e12) < 1e-9
    assert r["cpu_model"] and "median of 3" in r["timing"]
    # a varlen workload's pairs follow its drawn lengths (one short sequence here)
    wlv = workloads.custom(0, 2, 0, 64, "f16", True, lengths=[5, 17], dropout_p=0.1, seed=3)
    rv = bench.cpu_baseline(wlv.wl, wlv, 0, repeats=1, warmup=0)
    assert abs(rv["fwd"]["gflop"] - 4 * 64 * 2 * (15 + 153) / 1e9) < 1e-12
