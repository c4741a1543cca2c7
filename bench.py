"""Benchmark of pair-biased triangle attention on one MI355X.

A step is one pass of the hot path over one batch: the starting-node AND the
ending-node triangle attention of a 1024 x 1024 x 128 bf16 pair tensor
(N(0,1) plus 2*exp(-|i-j|/32) on every channel), each = K1 (LayerNorm +
projections) then K2 (fused attention + gate + output projection).  Inputs
are resident in HBM before timing starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Prints ONE JSON line.  `value` = algorithmic TFLOP/s of the whole step;
`roofline` = the fused attention kernel (tri_attend) against the dense bf16
MFMA peak, its launch duration measured with HIP events on the stream it runs
on; `cpu_baseline` = the float64 oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 (vector and MFMA)
PEAK_HBM_GBS = 8000.0
DEFAULT_WORKLOAD = "startend-bf16-I1024-distogram"
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SRC = os.path.join(ROOT, "protein_pair_representation_amd", "csrc", "triattn_kernels.hip")


def flops(I, rows, with_bias):
    """Algorithmic flops (2 per multiply-add) of one variant; elementwise work not counted."""
    c, hd, H = 128, 128, 4
    proj = 2.0 * rows * I * c * (4 * hd + (H if with_bias else 0))
    attn = 4.0 * H * 32 * rows * I * I
    out = 2.0 * rows * I * hd * c
    return proj, attn, out


def k1_bytes(I, rows, es, with_bias):
    """Algorithmic HBM bytes of K1: read Z, write q, k, v^T, g (and the fp32 bias)."""
    return rows * I * 128 * es * 5 + (4 * I * I * 4 if with_bias else 0)


def k2_bytes(I, rows, es):
    """Algorithmic HBM bytes of K2: read q, k, v^T, g and the fp32 bias once, write out."""
    return rows * I * 128 * es * 5 + 4 * I * I * 4


def kernel_sha():
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def read_traffic(workload):
    """HBM bytes per tri_attend launch from the committed rocprofv3 --pmc summary, if current."""
    path = os.path.join(PROFILE_DIR, f"tri_attend_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m = re.search(r"traffic_bytes_per_launch=([0-9.eE+]+)\s+kernel_sha=([0-9a-f]+)", txt)
    if not m or m.group(2) != kernel_sha():
        return None
    return float(m.group(1))


def cpu_baseline(wl, z_host, w_host, target_s=12.0):
    """The float64 oracle on a bounded sample of rows of the workload, over a process pool."""
    import multiprocessing as mp

    import numpy as np
    from oracle import ref
    from protein_pair_representation_amd import inputs

    workers = max(1, min(16, os.cpu_count() or 1))
    I = wl.I
    p = ref.params(inputs.weights_f64(w_host), 4, 32)
    z64 = inputs.to_f64(z_host)
    t0 = time.perf_counter()
    bias = ref.pair_bias(z64, p)                    # whole bias, single process
    t_bias = time.perf_counter() - t0
    f_bias = 2.0 * I * I * 128 * 4
    # calibrate one row, then size the sample to about target_s of wall time
    t0 = time.perf_counter()
    ref.triangle_attn_rows(z64[:1], bias, p)
    t_row = time.perf_counter() - t0
    n_rows = int(max(workers, min(I, workers * max(1, round((target_s - t_bias) / max(t_row, 1e-3) / 1.0)))))
    n_rows = min(n_rows, I)
    rows = np.linspace(0, I - 1, n_rows).astype(int)
    chunks = [rows[i::workers] for i in range(workers)]
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(workers, initializer=_limit_blas) as pool:
        pool.starmap(_oracle_rows, [(z64[c], bias, p) for c in chunks if len(c)])
    t_rows = time.perf_counter() - t0
    proj, attn, out = flops(I, n_rows, False)
    total_f = f_bias + proj + attn + out
    total_t = t_bias + t_rows
    return {"value": total_f / total_t / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
            "sample": f"{wl.name}: whole pair bias (1 process) + starting-node rows {n_rows} of {I} "
                      f"({workers} processes, 1 BLAS thread each), float64 NumPy; {total_t:.1f} s"}


def _limit_blas():
    os.environ["OMP_NUM_THREADS"] = "1"
    os.environ["OPENBLAS_NUM_THREADS"] = "1"


def _oracle_rows(z_rows, bias, p):
    from oracle import ref
    return ref.triangle_attn_rows(z_rows, bias, p).shape


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the sharded path is described, not built.", file=sys.stderr)
        sys.exit(2)

    import torch
    from protein_pair_representation_amd import inputs
    from protein_pair_representation_amd import triattn as ta

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 3}))
        return

    wl = inputs.WORKLOADS[args.workload]
    dt = inputs.DTYPES[wl.dtype]
    es = 2 if wl.dtype == "bf16" else 4
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    w_host = inputs.workload_weights(wl)
    wd = {k: v.to(dev) for k, v in w_host.items()}
    I, R = wl.I, wl.n_rows
    variants = list(wl.variants)
    if "rows" in variants:
        bias = torch.empty((4, I, I), dtype=torch.float32, device=dev)
        parts = []
        for r0 in range(0, I, 512):
            zb = inputs.workload_z(wl, r0, min(512, I - r0)).to(dev)
            ta.triangle_attn_pair_bias(zb, wd, row0=r0, bias=bias)
            if r0 < R:
                parts.append(zb[:R - r0])
        z = torch.cat(parts)[:R].contiguous()
        z_host = None
    else:
        z_host = inputs.workload_z(wl)
        z = z_host.to(dev)
        bias = None
    torch.cuda.synchronize()

    ws = {v: ta.workspace(I, R, dt, v, dev) for v in variants}
    out = {v: torch.empty((R, I, 128), dtype=dt, device=dev) for v in variants}
    n_ev = 3 * len(variants)

    def step(evs):
        for n_, v in enumerate(variants):
            evs[3 * n_].record(stream)
            ta.triangle_attn_project(z, wd, variant=v, ws=ws[v], stream=stream)
            evs[3 * n_ + 1].record(stream)
            ta.triangle_attn_attend(ws[v], wd, I, R, dt, variant=v, bias=bias if v == "rows" else None,
                                    out=out[v], stream=stream)
            evs[3 * n_ + 2].record(stream)

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    warm = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    for _ in range(args.warmup):
        step(warm)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for v in variants:
        assert torch.isfinite(out[v]).all(), f"non-finite output ({v})"

    ms_step = (t1 - t0) * 1e3 / args.steps
    k1_ms = sum(e[3 * n_].elapsed_time(e[3 * n_ + 1]) for e in events for n_ in range(len(variants)))
    k2_ms = sum(e[3 * n_ + 1].elapsed_time(e[3 * n_ + 2]) for e in events for n_ in range(len(variants)))
    n_launch = args.steps * len(variants)
    k1_ms /= n_launch
    k2_ms /= n_launch

    step_flops = 0.0
    for v in variants:
        proj, attn, o = flops(I, R, v != "rows")
        step_flops += proj + attn + o
    _, attn1, out1 = flops(I, R, False)
    k2_flops = attn1 + out1
    k2_tflops = k2_flops / (k2_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS
    traffic = read_traffic(wl.name)
    k1b = k1_bytes(I, R, es, "rows" not in variants)
    value = step_flops / (ms_step * 1e-3) / 1e12

    res = {
        "metric": "pair-attention TFLOP/s (bf16) and % of MFMA peak at I=1024, c_z=128",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic (seeded N(0,1) pair tensor and weights, resident in HBM)",
        "config": {"workload": wl.name, "I": I, "rows": R, "c_z": 128, "heads": 4, "head_dim": 32,
                   "variants": variants},
        "pct_of_peak_step": round(100 * value / peak, 2),
        "roofline": {"kernel": "tri_attend", "bound": "mfma", "achieved": round(k2_tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(k2_tflops / peak, 4),
                     "traffic": traffic, "algorithmic_bytes": k2_bytes(I, R, es),
                     "flops_per_launch": k2_flops, "avg_launch_ms": round(k2_ms, 4)},
        "kernels": {"tri_project": {"avg_launch_ms": round(k1_ms, 4), "algorithmic_bytes": k1b,
                                    "GB/s": round(k1b / (k1_ms * 1e-3) / 1e9, 1),
                                    "frac_hbm": round(k1b / (k1_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
                    "tri_attend": {"avg_launch_ms": round(k2_ms, 4), "TFLOP/s": round(k2_tflops, 2)}},
        "kernel_sha": kernel_sha(),
    }
    if not args.no_cpu_baseline and z_host is not None:
        res["cpu_baseline"] = cpu_baseline(wl, z_host, w_host)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
