#!/usr/bin/env python3
"""Attention forward + backward throughput on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--block-density P] [--keep-bits] [--decode [--page-size P]]
    python bench.py --compare-standard [--seqlens 512,1024,...] [--dropout P]

A step is one pass of the whole hot path over one batch of synthetic input:
fa_forward (fused tiled forward) followed by the two backward kernels
(query side: D and dQ; key side: dK and dV), with every input resident in
HBM.  The
default workload is the causal B=4, H=8, N=4096, d=128 bf16 one.
W untimed steps run first (repeated until the GPU clocks have settled, about
1.5 s), then exactly K timed steps bracketed by device synchronisation; HIP
events on the library's stream time each kernel of every step.  Rank 0
prints one JSON line.

Work convention: a visible (query, key) pair costs 4*d flops forward and
10*d flops backward (B*H*N(N+1)/2 pairs causal, B*H*N^2 otherwise); masked
work inside diagonal tiles is not counted.  With --block-density P the
block-sparse calls run under a random 128x128 block mask (each block on with
probability P, diagonal blocks on) and only the pairs it leaves visible
count.  Peak = MI355X dense bf16/fp16
MFMA, 2.5 PFLOP/s.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd+bwd TFLOP/s (% of MFMA bf16 peak), B4 H8 N4096 d128 causal"
PEAK_TFLOPS = 2500.0      # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0     # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")
KERNEL_SOURCES = {
    "fa_fwd_kernel": ["fa_fwd.hip", "fa_device.hpp"],
    "fa_bwd_dq_kernel": ["fa_bwd.hip", "fa_device.hpp"],
    "fa_bwd_dkdv_kernel": ["fa_bwd.hip", "fa_device.hpp"],
}


def visible_pairs(wl, lengths=None) -> int:
    lens = lengths if lengths is not None else [wl.N] * wl.B
    if wl.causal:
        return wl.H * sum(L * (L + 1) // 2 for L in lens)
    return wl.H * sum(L * L for L in lens)


def visible_pairs_masked(wl, bm) -> int:
    """Visible pairs under a [B, H, nb, nb] block mask (blocks of 128), with
    the causal rule j <= i where the workload is causal."""
    import numpy as np
    blk, N = 128, wl.N
    nb = bm.shape[-1]
    sizes = np.minimum(blk, N - blk * np.arange(nb))            # rows (= columns) of each block
    full = np.outer(sizes, sizes)                                 # pairs of a block with no causal cut
    if wl.causal:
        full = np.tril(full, -1) + np.diag(sizes * (sizes + 1) // 2)
    return int((bm.astype(np.int64) * full[None, None]).sum())


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "exact_tiled_attention_40_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    when they are missing or were taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256") != kernel_source_hash(kernel):
        return None
    return rec.get("traffic_bytes")


def cpu_model() -> str:
    """The host CPU's model name (first processor entry of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, x, n_heads: int, repeats: int = 3, warmup: int = 1):
    """The fp64 oracle (as it stands) on a bounded sample of the workload:
    n_heads (sequence, head) pairs at full length (0 = every pair), forward
    and backward timed separately, `warmup` untimed runs then the median of
    `repeats`; OpenMP runs one pair per host thread."""
    import statistics

    import oracle
    from workloads import as_f64_tokens
    oracle.build()
    nseq = len(x.lengths) if wl.varlen else wl.B
    all_pairs = [(s, h) for s in range(nseq) for h in range(wl.H)]
    if n_heads <= 0 or n_heads >= len(all_pairs):
        sel = all_pairs
    else:
        sel = all_pairs[::max(1, len(all_pairs) // n_heads)][:n_heads]
    q, k, v, do = (as_f64_tokens(t) for t in (x.q, x.k, x.v, x.do))
    kw = dict(scale=wl.scale, causal=wl.causal, dropout_p=wl.dropout_p, seed=wl.seed, heads=sel)
    kw.update(lengths=x.lengths) if wl.varlen else kw.update(N=wl.N)
    times = {"fwd": [], "bwd": []}
    for r in range(warmup + repeats):
        t0 = time.perf_counter()
        oracle.forward(q, k, v, **kw)
        t1 = time.perf_counter()
        oracle.backward(q, k, v, do, **kw)
        t2 = time.perf_counter()
        if r >= warmup:
            times["fwd"].append(t1 - t0)
            times["bwd"].append(t2 - t1)
    lens = x.lengths if wl.varlen else [wl.N] * wl.B
    pairs = sum((lens[s] * (lens[s] + 1) // 2) if wl.causal else lens[s] ** 2 for s, _ in sel)
    tf, tb = statistics.median(times["fwd"]), statistics.median(times["bwd"])
    ff, fb = 4.0 * wl.d * pairs, 10.0 * wl.d * pairs
    what = "every" if len(sel) == len(all_pairs) else f"{len(sel)} of the"
    threads = min(oracle.max_threads(), len(sel))
    return {"value": (ff + fb) / (tf + tb) / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "host_threads": oracle.max_threads(),
            "fwd": {"seconds": tf, "tflops": ff / tf / 1e12, "gflop": ff / 1e9},
            "bwd": {"seconds": tb, "tflops": fb / tb / 1e12, "gflop": fb / 1e9},
            "seconds": tf + tb, "timing": f"{warmup} warm-up run(s), median of {repeats}",
            "sample": f"{what} {len(all_pairs)} (sequence, head) pairs of the {wl.name} workload at full length, "
                      f"fp64 forward and backward timed separately, {(ff + fb) / 1e9:.1f} GFLOP per run "
                      f"(4*d and 10*d flops per visible pair)"}


def cpu_baseline_configs(args) -> int:
    """The oracle baseline on every workload, one JSON line each: the small
    and headline workloads (and any listed) with 1 warm-up and the median of
    3 over every (sequence, head) pair, the long and varlen ones in a single
    run.  Host work only; minutes in all."""
    import workloads
    names = args.workload.split(",") if args.workload else list(workloads.WORKLOADS)
    for name in names:
        wl = workloads.WORKLOADS[name]
        x = workloads.make_inputs(wl)
        big = wl.N * wl.N * wl.H * wl.B > 4096 * 4096 * 32 or wl.varlen
        rec = cpu_baseline(wl, x, 0, repeats=1 if big else 3, warmup=0 if big else 1)
        print(json.dumps({"workload": name, "cpu_baseline": rec}), flush=True)
    return 0


def copy_calibration(nbytes: int, steps: int) -> int:
    """A plain elementwise pass over nbytes of fp32 (y = -x: reads nbytes,
    writes nbytes), run `steps` times: the reference kernel that scales the
    FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(steps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_bytes_read": n * 4, "calibration_bytes_written": n * 4, "launches": steps}),
          flush=True)
    return 0


def _counter_means(csv_path: str, counter: str):
    """Mean value of a counter per kernel name over the dispatches of a
    rocprofv3 counter_collection.csv."""
    import csv
    import re
    acc = {}
    with open(csv_path) as fh:
        for row in csv.DictReader(fh):
            if row["Counter_Name"] != counter:
                continue
            m = re.search(r"(fa_\w+_kernel)", row["Kernel_Name"])
            name = m.group(1) if m else row["Kernel_Name"]
            acc.setdefault(name, {})
            acc[name][row["Dispatch_Id"]] = acc[name].get(row["Dispatch_Id"], 0.0) + float(row["Counter_Value"])
    return {k: sum(v.values()) / len(v) for k, v in acc.items()}


def pmc_summary(pmc_dir: str, calib_bytes: int) -> int:
    """Turn four rocprofv3 --pmc runs (fetch/, write/: this benchmark;
    calib_fetch/, calib_write/: the calibration pass of calib_bytes) into
    per-launch HBM traffic of each kernel, written to TRAFFIC_FILE together
    with the hash of the kernel sources it was measured on."""
    f = _counter_means(os.path.join(pmc_dir, "fetch", "run_counter_collection.csv"), "FETCH_SIZE")
    w = _counter_means(os.path.join(pmc_dir, "write", "run_counter_collection.csv"), "WRITE_SIZE")
    cf = _counter_means(os.path.join(pmc_dir, "calib_fetch", "run_counter_collection.csv"), "FETCH_SIZE")
    cw = _counter_means(os.path.join(pmc_dir, "calib_write", "run_counter_collection.csv"), "WRITE_SIZE")
    # the calibration kernel is the launch with the largest fetch
    calib = max(cf, key=cf.get)
    fetch_scale = calib_bytes / cf[calib]
    write_scale = calib_bytes / cw[calib]
    out = {"calibration": {"kernel": calib, "bytes": calib_bytes, "FETCH_SIZE": cf[calib], "WRITE_SIZE": cw[calib],
                           "fetch_bytes_per_unit": fetch_scale, "write_bytes_per_unit": write_scale}}
    for k in KERNEL_SOURCES:
        if k in f and k in w:
            out[k] = {"FETCH_SIZE": f[k], "WRITE_SIZE": w[k], "fetch_bytes": f[k] * fetch_scale,
                      "write_bytes": w[k] * write_scale, "traffic_bytes": f[k] * fetch_scale + w[k] * write_scale,
                      "source_sha256": kernel_source_hash(k)}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))
    return 0


def decode_bench(args) -> int:
    """One decode step = fa_decode (split kernel + merge kernel) over the
    workload's caches; HBM-bound, so the roofline is bytes against 8 TB/s.
    Algorithmic bytes = the valid K and V cache rows read once, plus q, o and
    lse."""
    import torch
    import exact_tiled_attention_40_amd as fa
    import workloads

    wl = workloads.DECODE_WORKLOADS[args.workload or workloads.DECODE_HEADLINE]
    x = workloads.make_decode_inputs(wl)
    dev = torch.device("cuda")
    q, k, v = (t.to(dev) for t in (x.q, x.k, x.v))
    lens = x.seqlens.to(dev) if x.seqlens is not None else None
    o = torch.empty_like(q)
    lse = torch.empty((wl.B, wl.nq, wl.H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    if args.page_size:
        # the same caches as a paged cache: shuffled pool pages and a block table
        kp, vp, table = workloads.paged_cache(x.k, x.v, args.page_size, seed=wl.seed + 1,
                                              lengths=None if x.seqlens is None else x.seqlens.tolist())
        kp, vp, table = kp.to(dev), vp.to(dev), table.to(dev)
        del k, v
        cap = table.shape[1] * args.page_size
        ws = torch.empty(fa.fa_decode_workspace_size(wl.B, wl.H, wl.nq, cap, wl.d), dtype=torch.uint8, device=dev)

        def step():
            fa.fa_decode_paged(q, kp, vp, table, seqlens_k=lens, scale=wl.scale, causal=wl.causal, out=o, lse=lse,
                               workspace=ws, stream=stream)
    else:
        ws = torch.empty(fa.fa_decode_workspace_size(wl.B, wl.H, wl.nq, wl.nk, wl.d), dtype=torch.uint8, device=dev)

        def step():
            fa.fa_decode(q, k, v, seqlens_k=lens, scale=wl.scale, causal=wl.causal, out=o, lse=lse, workspace=ws,
                         stream=stream)

    t_settle = time.perf_counter()
    with ClockSampler() as clock:
        while True:
            for _ in range(max(args.warmup, 1)):
                step()
            torch.cuda.synchronize()
            if time.perf_counter() - t_settle >= args.settle_s:
                break
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    valid = int(x.seqlens.clamp(0, wl.nk).sum()) if x.seqlens is not None else wl.B * wl.nk
    esz = 2
    kv_bytes = 2 * valid * wl.H * wl.d * esz
    io_bytes = wl.B * wl.nq * wl.H * (2 * wl.d * esz + 4)
    algo = kv_bytes + io_bytes
    gbs = algo / (ms * 1e-3) / 1e9
    line = {
        "metric": "KV-cache decode step GB/s (cache bytes read, % of HBM peak)",
        "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name + (f"_paged{args.page_size}" if args.page_size else ""), "B": wl.B, "H": wl.H,
                   "nq": wl.nq, "nk": wl.nk, "d": wl.d, "causal": wl.causal, "valid_cache_tokens": valid,
                   **({"page_size": args.page_size} if args.page_size else {})},
        "roofline": {"bound": "hbm", "kernel": "fa_decode_paged (split + merge)" if args.page_size
                     else "fa_decode (split + merge)", "achieved": gbs, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS, "traffic": None, "avg_launch_ms": ms,
                     "algorithmic_bytes_per_launch": algo},
        "wall_s_timed": wall,
        "observed_sclk_mhz": clock.summary(),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle
        qd, kd, vd = (t.double().numpy() for t in (x.q, x.k, x.v))
        t1 = time.perf_counter()
        oracle.decode(qd, kd, vd, scale=wl.scale, causal=wl.causal,
                      seqlens_k=None if x.seqlens is None else x.seqlens.numpy())
        sec = time.perf_counter() - t1
        line["cpu_baseline"] = {"value": algo / sec / 1e9, "unit": "GB/s", "cores": oracle.max_threads(),
                                "kind": "oracle", "seconds": sec,
                                "sample": "the whole decode step of the workload, fp64 (bytes counted as the "
                                          "kernel's 16-bit cache bytes)"}
    print(json.dumps(line), flush=True)
    return 0


class ClockSampler:
    """Samples the GPU shader clock (the current level of sysfs pp_dpm_sclk,
    the line marked '*') from a thread while the warm-up steps run, which are
    the same steps the timed region runs.  Reports the median, minimum and
    maximum in MHz once the clock has ramped up, or None where there is not
    exactly one such file."""

    def __init__(self, period_s: float = 0.05):
        import glob
        import threading
        files = glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")
        self.path = files[0] if len(files) == 1 else None
        self.period = period_s
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True) if self.path else None

    def _read(self):
        try:
            with open(self.path) as fh:
                for line in fh:
                    if line.rstrip().endswith("*"):
                        return int(line.split(":")[1].strip().lower().split("mhz")[0])
        except (OSError, ValueError, IndexError):
            return None
        return None

    def _run(self):
        while not self._stop.is_set():
            v = self._read()
            if v is not None:
                self.samples.append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        if self._thread:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        if self._thread:
            self._stop.set()
            self._thread.join()

    def summary(self):
        """Over the second half of the samples: the first ones catch the
        clock still ramping up from idle."""
        if not self.samples:
            return None
        v = sorted(self.samples[len(self.samples) // 2:])
        return {"median": v[len(v) // 2], "min": v[0], "max": v[-1], "samples": len(v),
                "source": "sysfs pp_dpm_sclk current level, second half of the warm-up steps"}


def standard_attention_step(q, k, v, do, *, scale, causal, dropout_p=0.0, generator=None):
    """Standard attention, forward then backward, with every intermediate
    written out (the three-step method of the FlashAttention write-ups,
    section 2.2 of the lab write-up): S = scale Q K^T and P = softmax(S) are
    full N x N matrices per head, and the backward materialises dP and dS as
    well.  torch eager ops in the inputs' dtype; this is the comparison side
    of the measurement, not part of the library.

    q, k, v, do: [B, N, H, d].  Returns (o, dq, dk, dv) in the same layout.
    Dropout draws its own mask from torch's generator: it costs what a
    materialised mask costs, but its bits are not the library's.  Operands of
    the batched products are made contiguous first, transposes included."""
    import torch
    qh, kh, vh, doh = (t.permute(0, 2, 1, 3).contiguous() for t in (q, k, v, do))
    n = qh.shape[2]
    s = torch.matmul(qh, kh.transpose(-1, -2).contiguous()) * scale
    if causal:
        hidden = torch.ones(n, n, dtype=torch.bool, device=s.device).triu_(1)
        s.masked_fill_(hidden, float("-inf"))
    p = torch.softmax(s, dim=-1)
    if dropout_p > 0:
        keep = torch.rand(p.shape, generator=generator, device=p.device) >= dropout_p
        z = p * keep / (1.0 - dropout_p)
    else:
        z = p
    o = torch.matmul(z, vh)
    dv = torch.matmul(z.transpose(-1, -2).contiguous(), doh)
    dz = torch.matmul(doh, vh.transpose(-1, -2).contiguous())
    dp = dz * keep / (1.0 - dropout_p) if dropout_p > 0 else dz
    ds = p * (dp - (p * dp).sum(dim=-1, keepdim=True))
    dq = torch.matmul(ds, kh) * scale
    dk = torch.matmul(ds.transpose(-1, -2).contiguous(), qh) * scale
    return tuple(t.permute(0, 2, 1, 3) for t in (o, dq, dk, dv))


def compare_standard(args) -> int:
    """Tiled kernels against standard (materialised) attention, forward +
    backward, at one or more sequence lengths of a fixed-length workload:
    step time and peak device memory each side allocates beyond its inputs
    (outputs, workspace and intermediates).  One JSON line per length."""
    import torch
    import exact_tiled_attention_40_amd as fa
    import workloads

    base = workloads.WORKLOADS[args.workload or workloads.HEADLINE]
    if base.varlen:
        print("the standard-attention comparison runs on the fixed-length workloads", file=sys.stderr)
        return 2
    if args.dropout >= 0:
        base = dataclasses.replace(base, dropout_p=args.dropout)
    lens = [int(s) for s in args.seqlens.split(",")] if args.seqlens else [base.N]
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()
    gen = torch.Generator(device=dev)
    gen.manual_seed(base.seed)
    for n in lens:
        wl = dataclasses.replace(base, N=n, name=base.name.replace(f"_N{base.N}_", f"_N{n}_"))
        x = workloads.make_inputs(wl)
        if x.qkv is not None:
            qkv = x.qkv.to(dev)
            q, k, v = qkv.unbind(2)   # views into the packed [B, N, 3, H, d] tensor
            do = x.do.to(dev)
        else:
            qkv = None
            q, k, v, do = (t.to(dev) for t in (x.q, x.k, x.v, x.do))
        kw = dict(scale=wl.scale, causal=wl.causal, dropout_p=wl.dropout_p, seed=wl.seed)

        def tiled():
            o, lse = fa.fa_forward(q, k, v, stream=stream, **kw)
            # packed inputs: the gradients go into one packed dqkv buffer
            gout = dict(zip(("dq", "dk", "dv"), torch.empty_like(qkv).unbind(2))) if qkv is not None else {}
            grads = fa.fa_backward(q, k, v, o, lse, do, stream=stream, **kw, **gout)
            return (o,) + tuple(grads)

        def standard():
            return standard_attention_step(q, k, v, do, scale=wl.scale, causal=wl.causal,
                                           dropout_p=wl.dropout_p, generator=gen)

        res = {}
        outs = {}
        for name, fn in (("tiled", tiled), ("standard", standard)):
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
            torch.cuda.reset_peak_memory_stats()
            held = torch.cuda.memory_allocated()
            outs[name] = fn()
            torch.cuda.synchronize()
            peak = torch.cuda.max_memory_allocated() - held
            outs[name] = tuple(t.float() for t in outs[name]) if wl.dropout_p == 0 else None
            t_settle = time.perf_counter()
            while True:
                for _ in range(max(args.warmup, 1)):
                    fn()
                torch.cuda.synchronize()
                if time.perf_counter() - t_settle >= args.settle_s:
                    break
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(args.steps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            res[name] = {"ms_per_step": e0.elapsed_time(e1) / args.steps, "peak_bytes": int(peak)}
        pairs = visible_pairs(wl)
        flops = 14.0 * wl.d * pairs
        for r in res.values():
            r["tflops"] = flops / (r["ms_per_step"] * 1e-3) / 1e12
        line = {
            "metric": "standard attention vs tiled attention, fwd+bwd step (speedup, memory ratio)",
            "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "N": n, "d": wl.d, "causal": wl.causal,
                       "dropout_p": wl.dropout_p, "dtype": wl.dtype, "packed_qkv": wl.packed},
            "steps": args.steps, "warmup": args.warmup, "data": "synthetic",
            "tiled": res["tiled"], "standard": res["standard"],
            "speedup": res["standard"]["ms_per_step"] / res["tiled"]["ms_per_step"],
            "memory_ratio": res["standard"]["peak_bytes"] / max(res["tiled"]["peak_bytes"], 1),
        }
        if outs["tiled"] is not None:
            # both sides compute the same attention (no dropout): largest
            # relative difference of each output, a check on the comparison
            line["max_rel_diff"] = {nm: float((a - b).abs().max() / b.abs().max().clamp_min(1e-30))
                                    for nm, a, b in zip(("o", "dq", "dk", "dv"), outs["tiled"], outs["standard"])}
        print(json.dumps(line), flush=True)
        del q, k, v, do, qkv, x, outs
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None, help="workload name (default: the causal B4 H8 N4096 d128 one)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=16,
                    help="oracle sample size in (sequence, head) pairs (about 10-30 s of host work); 0 = all")
    ap.add_argument("--cpu-baseline-configs", action="store_true",
                    help="time only the fp64 oracle on every workload (or the --workload list), one JSON line each")
    ap.add_argument("--copy-bytes", type=int, default=0, help="run only the counter calibration pass over this many bytes")
    ap.add_argument("--pmc-summary", default="", help="directory of rocprofv3 --pmc runs to turn into the traffic file")
    ap.add_argument("--calib-bytes", type=int, default=1 << 30, help="bytes of the calibration pass of --pmc-summary")
    ap.add_argument("--block-density", type=float, default=0.0,
                    help="time the block-sparse calls with a random 128x128 block mask of this density "
                         "(diagonal blocks kept); 0 = dense")
    ap.add_argument("--decode", action="store_true",
                    help="time fa_decode (KV-cache decode step) on a decode workload instead")
    ap.add_argument("--page-size", type=int, default=0,
                    help="with --decode: time fa_decode_paged on the same caches split into pages of this many "
                         "tokens (a power of two) in shuffled order")
    ap.add_argument("--keep-bits", action="store_true",
                    help="dropout workloads: time fa_forward_keep / fa_backward_keep_stage (the forward stores "
                         "its keep decisions, the backward reads them instead of hashing)")
    ap.add_argument("--head-dim", type=int, default=0,
                    help="run the chosen workload with this head size instead (32, 64, 96, 128, 160, 192 or 256)")
    ap.add_argument("--settle-s", type=float, default=1.5,
                    help="repeat the warm-up steps until this many seconds have passed (clock settling)")
    ap.add_argument("--compare-standard", action="store_true",
                    help="time standard (materialised) attention against the tiled kernels instead: step time "
                         "and peak memory, one JSON line per sequence length")
    ap.add_argument("--seqlens", default="", help="comma-separated sequence lengths for --compare-standard")
    ap.add_argument("--dropout", type=float, default=-1.0,
                    help="dropout probability for --compare-standard (default: the workload's)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the kernels shard by (batch, head) "
              f"and need no collective, so there is no multi-GPU run to time.", file=sys.stderr)
        return 2

    if args.copy_bytes:
        return copy_calibration(args.copy_bytes, args.steps)
    if args.cpu_baseline_configs:
        return cpu_baseline_configs(args)
    if args.pmc_summary:
        return pmc_summary(args.pmc_summary, args.calib_bytes)

    if args.decode:
        return decode_bench(args)
    if args.compare_standard:
        return compare_standard(args)

    import torch
    import exact_tiled_attention_40_amd as fa
    import workloads

    wl = workloads.WORKLOADS[args.workload or workloads.HEADLINE]
    if args.head_dim and args.head_dim != wl.d:
        # same recipe and seed at another head size (the head-size sweep)
        wl = dataclasses.replace(wl, name=wl.name.replace(f"_d{wl.d}_", f"_d{args.head_dim}_"), d=args.head_dim)
    x = workloads.make_inputs(wl)
    dev = torch.device("cuda")
    if x.qkv is not None:
        qkv = x.qkv.to(dev)
        q, k, v = qkv.unbind(2)
        dqkv = torch.empty_like(qkv)
        dq, dk, dv = dqkv.unbind(2)
    else:
        q, k, v = (t.to(dev) for t in (x.q, x.k, x.v))
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    do = x.do.to(dev)
    o = torch.empty(q.shape, dtype=q.dtype, device=dev)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
    ws = torch.empty(fa.fa_backward_workspace_size(wl.B, wl.N, wl.H, wl.d), dtype=torch.uint8, device=dev)
    kw = dict(scale=wl.scale, causal=wl.causal, dropout_p=wl.dropout_p, seed=wl.seed)
    if wl.varlen:
        # packed [total, H, d] tokens of B sequences of the drawn lengths
        kw.update(cu_seqlens=x.cu_seqlens.to(dev), max_seqlen=wl.N)
        if args.block_density > 0:
            print("block masks are timed on the fixed-length workloads", file=sys.stderr)
            return 2
    stream = torch.cuda.current_stream()
    bm = None
    if args.block_density > 0:
        bm = workloads.block_mask(wl.B, wl.H, wl.N, args.block_density, seed=wl.seed + 1000)
        kw["block_mask"] = bm.to(dev)

    keep = None
    if args.keep_bits:
        if bm is not None or wl.dropout_p == 0:
            print("--keep-bits times dense or varlen workloads with dropout", file=sys.stderr)
            return 2
        keep = torch.empty(fa.fa_dropout_bits_size(wl.B, wl.N, wl.H), dtype=torch.uint8, device=dev)

    def step(ev=None):
        if ev: ev[0].record(stream)
        if keep is None:
            fa.fa_forward(q, k, v, out=o, lse=lse, stream=stream, **kw)
        else:
            fa.fa_forward_keep(q, k, v, keep_bits=keep, out=o, lse=lse, stream=stream, **kw)
        if ev: ev[1].record(stream)
        for s in range(2):
            if keep is None:
                fa.fa_backward_stage(s, q, k, v, o, lse, do, dq=dq, dk=dk, dv=dv, workspace=ws, stream=stream,
                                     **kw)
            else:
                fa.fa_backward_keep_stage(s, q, k, v, o, lse, do, keep_bits=keep, dq=dq, dk=dk, dv=dv,
                                          workspace=ws, stream=stream, **kw)
            if ev: ev[2 + s].record(stream)

    # W warm-up steps, repeated until at least --settle-s seconds have passed:
    # the GPU clocks take about a second of load to settle, and a step is
    # under a millisecond.
    t_settle = time.perf_counter()
    with ClockSampler() as clock:
        while True:
            for _ in range(args.warmup):
                step()
            torch.cuda.synchronize()
            if time.perf_counter() - t_settle >= args.settle_s or args.warmup == 0:
                break
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    names = ["fa_fwd_kernel", "fa_bwd_dq_kernel", "fa_bwd_dkdv_kernel"]
    ms = {n: sum(ev[j].elapsed_time(ev[j + 1]) for ev in events) / args.steps for j, n in enumerate(names)}
    step_ms = events[0][0].elapsed_time(events[-1][3]) / args.steps

    pairs = visible_pairs(wl, x.lengths) if bm is None else visible_pairs_masked(wl, bm.numpy())
    fwd_flops = 4.0 * wl.d * pairs
    bwd_flops = 10.0 * wl.d * pairs
    total_tflops = (fwd_flops + bwd_flops) / (step_ms * 1e-3) / 1e12
    fwd_tflops = fwd_flops / (ms["fa_fwd_kernel"] * 1e-3) / 1e12
    bwd_ms = ms["fa_bwd_dq_kernel"] + ms["fa_bwd_dkdv_kernel"]
    bwd_tflops = bwd_flops / (bwd_ms * 1e-3) / 1e12

    # Algorithmic flops per launch: the forward's 4*d per visible pair; the
    # backward's 10*d per pair splits into S, dP, dV, dK (8*d, key-side
    # kernel) and dQ (2*d, query-side kernel, whose S and dP recomputation is
    # not counted).  Matrix-core work actually issued is 4*d, 6*d and 8*d.
    algo_flops = {"fa_fwd_kernel": fwd_flops, "fa_bwd_dq_kernel": 2.0 * wl.d * pairs,
                  "fa_bwd_dkdv_kernel": 8.0 * wl.d * pairs}
    issued_flops = {"fa_fwd_kernel": fwd_flops, "fa_bwd_dq_kernel": 6.0 * wl.d * pairs,
                    "fa_bwd_dkdv_kernel": 8.0 * wl.d * pairs}
    dom = max(names, key=lambda n: ms[n])
    achieved = algo_flops[dom] / (ms[dom] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_TFLOPS,
                # the traffic file holds the counters of the default workload's dense kernels
                "traffic": measured_traffic(dom) if wl.name == workloads.HEADLINE and bm is None else None,
                "avg_launch_ms": ms[dom], "algorithmic_flops_per_launch": algo_flops[dom]}
    per_kernel = {n: {"ms": ms[n], "algorithmic_tflops": algo_flops[n] / (ms[n] * 1e-3) / 1e12,
                      "issued_mfma_tflops": issued_flops[n] / (ms[n] * 1e-3) / 1e12} for n in names}

    line = {
        "metric": METRIC,
        "value": total_tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name + (f"_blocksparse{args.block_density:g}" if bm is not None else ""),
                   "B": wl.B, "H": wl.H, "N": wl.N, "d": wl.d, "causal": wl.causal,
                   "dropout_p": wl.dropout_p, "packed_qkv": wl.packed,
                   **({"dropout_keep_bits": True} if keep is not None else {}),
                   **({"block_density": args.block_density, "mask_blocks_on": int(bm.sum()),
                       "mask_blocks": int(bm.numel()), "visible_pairs": pairs} if bm is not None else {}),
                   **({"varlen": True, "total_tokens": int(sum(x.lengths)), "visible_pairs": pairs}
                      if wl.varlen else {})},
        "frac_of_peak": total_tflops / PEAK_TFLOPS,
        "fwd": {"tflops": fwd_tflops, "ms": ms["fa_fwd_kernel"], "frac": fwd_tflops / PEAK_TFLOPS},
        "bwd": {"tflops": bwd_tflops, "ms": bwd_ms, "frac": bwd_tflops / PEAK_TFLOPS},
        "kernels": per_kernel,
        "wall_s_timed": wall,
        "observed_sclk_mhz": clock.summary(),
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline and bm is None:
        line["cpu_baseline"] = cpu_baseline(wl, x, args.cpu_heads)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
