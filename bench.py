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
    """Algorithmic HBM bytes of K1: read Z, write q, k, v^T, g (and the fp32 pair bias)."""
    return rows * I * 128 * es * 5 + (4 * I * I * 4 if with_bias else 0)


def k2_bytes(I, rows, es):
    """Algorithmic HBM bytes of K2: read q, k, v^T, g and the packed bias (fp16 / fp32) once, write out."""
    return rows * I * 128 * es * 5 + 4 * I * I * es


def kernel_sha(path=KERNEL_SRC):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


AAQ_SRC = os.path.join(ROOT, "protein_pair_representation_amd", "csrc", "aaq_kernels.hip")
AAQ_CASES = [("encode", "A"), ("decode", "A"), ("encode", "B"), ("decode", "B")]


def aaq_traffic(workload):
    """{kernel label: HBM bytes per launch} from the committed codec --pmc summary, if current."""
    path = os.path.join(PROFILE_DIR, f"aaq_{workload}_pmc.txt")
    if not os.path.exists(path):
        return {}
    out = {}
    for m in re.finditer(r"^(aaq_\S+)_traffic_bytes_per_launch=([0-9.eE+]+)\s+kernel_sha=([0-9a-f]+)",
                         open(path).read(), re.M):
        if m.group(3) == kernel_sha(AAQ_SRC):
            out[m.group(1)] = float(m.group(2))
    return out


def aaq_codec(z, workload, stream, reps=20):
    """The AAQ codec on the workload's pair tensor: encode (bf16 tokens -> records) and
    decode (records -> bf16 tokens) for groups A and B, each timed over `reps` launches
    with HIP events on `stream`.  Algorithmic bytes = tokens x (token bytes + record bytes)."""
    import torch
    from protein_pair_representation_amd import aaq
    n = z.numel() // 128
    tb = 128 * z.element_size()
    rec = {g: aaq.aaq_encode(z, g, stream=stream) for g in ("A", "B")}
    y = torch.empty((n, 128), dtype=z.dtype, device=z.device)
    traffic = aaq_traffic(workload)
    res = {"tokens": n, "kernel_sha": kernel_sha(AAQ_SRC)}
    for op, g in AAQ_CASES:
        def launch():
            if op == "encode":
                aaq.aaq_encode(z, g, out=rec[g], stream=stream)
            else:
                aaq.aaq_decode(rec[g], g, z.dtype, out=y, stream=stream)
        launch()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            launch()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        nbytes = n * (tb + aaq.aaq_record_bytes(g))
        gbs = nbytes / (ms * 1e-3) / 1e9
        label = f"aaq_{op}_{g}_{'bf16' if z.dtype == torch.bfloat16 else 'f32'}"
        res[label] = {"avg_launch_ms": round(ms, 4), "algorithmic_bytes": nbytes, "GB/s": round(gbs, 1),
                      "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic.get(label)}
    return res


def aaq_project(z, wd, variant, stream, reps=20):
    """The projection stage (K1 + bias pack) fed by the pair tensor as bf16 tokens and
    as group-A records, each timed over `reps` calls with HIP events on `stream`."""
    import torch
    from protein_pair_representation_amd import aaq
    from protein_pair_representation_amd import triattn as ta
    R, I = z.shape[0], z.shape[1]
    rec = aaq.aaq_encode(z, "A", stream=stream)
    ws = ta.workspace(I, R, z.dtype, variant, z.device)
    runs = {"from_bf16_tokens": lambda: ta.triangle_attn_project(z, wd, variant=variant, ws=ws, stream=stream),
            "from_group_a_records": lambda: ta.triangle_attn_project_aaq(rec, wd, I, R, "A", variant=variant, ws=ws,
                                                                         stream=stream)}
    out = {"variant": variant}
    for name, fn in runs.items():
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        out[name + "_ms"] = round(e0.elapsed_time(e1) / reps, 4)
    return out


KNN_SRC = os.path.join(ROOT, "protein_pair_representation_amd", "csrc", "knn_kernels.hip")


def knn_bytes(L, k):
    """Algorithmic HBM bytes of one kNN encode: read coordinates (12 B) and single features
    (256 B) once per atom, write k neighbour indices (4 B) and k pair rows (32 B)."""
    return L * (12 + 256 + k * (4 + 32))


def knn_encoder(stream, reps=20, name="knn-L16384-k32"):
    """The kNN sparse pair encoder on its workload (atoms along a chain), timed over `reps`
    calls (three launches each) with HIP events on `stream`."""
    import torch
    from protein_pair_representation_amd import inputs
    from protein_pair_representation_amd import knn
    wl = inputs.KNN_WORKLOADS[name]
    L, k = wl["L"], wl["k"]
    a = {n_: t.cuda() for n_, t in inputs.make_atoms(wl["seed"], L).items()}
    nbr = torch.empty((L, k), dtype=torch.int32, device="cuda")
    pair = torch.empty((L, k, 16), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(knn.knn_workspace_bytes(L), dtype=torch.uint8, device="cuda")

    def launch():
        knn.knn_pair_encode(a["x"], a["s"], k, a["w_l"], a["w_m"], a["w_d"], nbr=nbr, pair=pair, ws=ws,
                            stream=stream)
    launch()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        launch()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nb = knn_bytes(L, k)
    return {"workload": name, "atoms": L, "k": k, "avg_call_ms": round(ms, 4),
            "pairs_per_s": round(L * k / (ms * 1e-3), 1), "algorithmic_bytes": nb,
            "GB/s": round(nb / (ms * 1e-3) / 1e9, 1), "frac_hbm": round(nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "kernel_sha": kernel_sha(KNN_SRC)}


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


def cpu_baseline(wl, z_host, w_host, target_s=20.0):
    """The float64 oracle on a bounded sample of rows of the workload, over a process pool.

    The whole pair bias is computed first (it is shared by every row), then rows
    spread evenly over the line are run one per worker and process; a first round
    of one row per worker sizes the remaining rounds to about `target_s` in total.
    """
    import multiprocessing as mp

    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import ref
    from protein_pair_representation_amd import inputs

    # one process per core of this process's CPU share, at most 16: the share of one GPU
    # on the GPU hosts (a box may show more cores than it allots to one GPU)
    allowed = len(os.sched_getaffinity(0))
    workers = max(1, min(16, allowed))
    I = wl.I
    p = ref.params(inputs.weights_f64(w_host), 4, 32)
    z64 = inputs.to_f64(z_host)
    t0 = time.perf_counter()
    with threadpool_limits(limits=workers):
        bias = ref.pair_bias(z64, p)
    t_bias = time.perf_counter() - t0
    f_bias = 2.0 * I * I * 128 * 4
    order = np.argsort((np.arange(I) * 0.6180339887498949) % 1.0, kind="stable")  # spread-out rows
    ctx = mp.get_context("fork")
    done = 0
    t0 = time.perf_counter()
    with ctx.Pool(workers, initializer=_limit_blas) as pool:
        def run_round(k):
            rows = order[k * workers:(k + 1) * workers]
            pool.starmap(_oracle_rows, [(z64[r:r + 1], bias, p) for r in rows])
            return len(rows)
        done += run_round(0)
        t_round = time.perf_counter() - t0
        rounds = int(max(0, min((I - done) // workers, (target_s - t_bias - t_round) // max(t_round, 1e-3))))
        for k in range(1, rounds + 1):
            done += run_round(k)
    t_rows = time.perf_counter() - t0
    proj, attn, out = flops(I, done, False)
    total_f = f_bias + proj + attn + out
    total_t = t_bias + t_rows
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    return {"value": round(total_f / total_t / 1e12, 5), "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
            "cpu_model": cpu_model, "host_cpu_count": os.cpu_count(), "cores_in_affinity": allowed,
            "cores_note": "workers = cores of this process's affinity, capped at 16 (one GPU's CPU share)",
            "sample": f"{wl.name}: the whole pair bias ({workers} BLAS threads) + starting-node rows {done} of {I} "
                      f"({workers} processes, 1 BLAS thread each), float64 NumPy; {total_t:.1f} s wall"}


def key_blocks(ws, wd, I, R, dt, variant, nb, stream, k2_flops, k2_ms, reps=10):
    """The attention stage as NB key blocks folded into a carried state, then finalize."""
    import torch
    from protein_pair_representation_amd import triattn as ta
    size = ((I + nb - 1) // nb + 63) // 64 * 64     # keys per block: a multiple of 64
    blocks = [(k0, min(size, I - k0)) for k0 in range(0, I, size)]
    st = ta.state(I, R, dt, variant)
    out = torch.empty((R, I, 128), dtype=dt, device="cuda")

    def once():
        for n, (k0, nk) in enumerate(blocks):
            ta.triangle_attn_attend_block(ws, wd, I, R, dt, k0, nk, n == 0, st, variant=variant, stream=stream)
        ta.triangle_attn_attend_finalize(ws, wd, I, R, dt, st, variant=variant, out=out, stream=stream)

    once()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        once()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return {"variant": variant, "blocks": len(blocks), "block_keys": size, "ms": round(ms, 4),
            "TFLOP/s": round(k2_flops / (ms * 1e-3) / 1e12, 2), "one_pass_ms": round(k2_ms, 4),
            "time_vs_one_pass": round(ms / k2_ms, 3)}


def kv_blocks(ws, wd, I, R, dt, variant, nb, stream, k2_flops, k2_ms, reps=10):
    """The ring step: NB caller-held key blocks (copies of the workspace's keys, values and
    bias columns, padded to 64 positions) folded into a carried state, the last one
    folded and finished in one launch (and, for comparison, every block folded, then
    a separate finalize)."""
    import torch
    from protein_pair_representation_amd import triattn as ta
    v = ta.workspace_views(ws, I, R, dt, variant)
    size = (I + nb - 1) // nb
    blocks = []
    for k0 in range(0, I, size):
        nk = min(size, I - k0)
        npos = (nk + 63) // 64 * 64
        kb = torch.zeros(v["k"].shape[:2] + (npos, 32), dtype=dt, device="cuda")
        vb = torch.zeros(v["vt"].shape[:3] + (npos,), dtype=dt, device="cuda")
        kb[:, :, :nk] = v["k"][:, :, k0:k0 + nk]
        vb[:, :, :, :nk] = v["vt"][:, :, :, k0:k0 + nk]
        blocks.append((kb, vb, v["bias_f32"][:, :, k0:k0 + nk].clone(), nk))   # a copy even for one block
    st = ta.state(I, R, dt, variant)
    out = torch.empty((R, I, 128), dtype=dt, device="cuda")

    def ring(fused_last):
        for n, (kb, vb, bb, nk) in enumerate(blocks):
            if fused_last and n == len(blocks) - 1:
                ta.triangle_attn_attend_kv_block_final(ws, wd, I, R, dt, kb, vb, bb, nk, n == 0, st,
                                                       variant=variant, out=out, stream=stream)
            else:
                ta.triangle_attn_attend_kv_block(ws, wd, I, R, dt, kb, vb, bb, nk, n == 0, st, variant=variant,
                                                 stream=stream)
        if not fused_last:
            ta.triangle_attn_attend_finalize(ws, wd, I, R, dt, st, variant=variant, out=out, stream=stream)

    def timed(fused_last):
        ring(fused_last)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            ring(fused_last)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ms_sep = timed(False)
    ms = timed(True)
    return {"variant": variant, "blocks": len(blocks), "block_keys": size, "ms": round(ms, 4),
            "TFLOP/s": round(k2_flops / (ms * 1e-3) / 1e12, 2), "one_pass_ms": round(k2_ms, 4),
            "time_vs_one_pass": round(ms / k2_ms, 3), "last_block": "folded and finished in one launch",
            "ms_with_separate_finalize": round(ms_sep, 4)}


def _limit_blas():
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)


def _oracle_rows(z_rows, bias, p):
    from oracle import ref
    return ref.triangle_attn_rows(z_rows, bias, p).shape


def _counter_csv(d):
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if len(files) != 1:
        raise SystemExit(f"expected one counter_collection.csv under {d}, found {files}")
    return files[0]


def _per_dispatch(path, counter):
    """{kernel name: [per-dispatch value]} for one counter (values summed over a dispatch's rows)."""
    import csv
    import collections
    acc = collections.defaultdict(float)
    names = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        acc[r["Dispatch_Id"]] += float(r["Counter_Value"])
        names[r["Dispatch_Id"]] = r["Kernel_Name"]
    out = collections.defaultdict(list)
    for k, v in acc.items():
        out[names[k]].append(v)
    return out


def _short(name):
    if "tri_attend" in name:
        # the one-pass kernels (bf16: tri_attend_fast; fp32: the unshifted form, template
        # flag true) do the work of one-pass calls; the shifted form only runs the
        # workgroups they flag (or key-block calls)
        if "tri_attend_fast" in name or "Lb1E" in name or "true>" in name:
            return "tri_attend"
        return "tri_attend_shifted"
    for key in ("tri_project", "tri_pack_bias", "copyBuffer"):
        if key in name:
            return key
    m = re.search(r"aaq_(encode|decode)_([ABC])_(bf16|f32)|knn_(prepare|select_encode)", name)
    if m:
        return m.group(0)
    return name[:60]


def summarize_pmc(run_dir, workload, copy_mib, family="tri"):
    """Write the HBM-traffic summary of tri_attend / tri_project from four rocprofv3 --pmc runs.

    run_dir holds pmc_fetch/ and pmc_write/ (bench.py under FETCH_SIZE and WRITE_SIZE)
    and pmc_copy_fetch/, pmc_copy_write/ (bench.py --copy-calibration under the same
    counters).  Each counter is scaled by (bytes the copy kernel moves) / (what the
    counter reads for it).
    """
    copy_bytes = copy_mib << 20
    cf = _per_dispatch(_counter_csv(os.path.join(run_dir, "pmc_copy_fetch")), "FETCH_SIZE")
    cw = _per_dispatch(_counter_csv(os.path.join(run_dir, "pmc_copy_write")), "WRITE_SIZE")
    copy_f = [v for k, v in cf.items() if "copyBuffer" in k][0]
    copy_w = [v for k, v in cw.items() if "copyBuffer" in k][0]
    f_scale = copy_bytes / (sum(copy_f) / len(copy_f) * 1024)
    w_scale = copy_bytes / (sum(copy_w) / len(copy_w) * 1024)
    kf = _per_dispatch(_counter_csv(os.path.join(run_dir, "pmc_fetch")), "FETCH_SIZE")
    kw = _per_dispatch(_counter_csv(os.path.join(run_dir, "pmc_write")), "WRITE_SIZE")
    lines = []
    per = {}
    for name in sorted(set(kf) | set(kw)):
        sh = _short(name)
        if not sh.startswith(family + "_"):
            continue
        f = kf.get(name, [0.0])
        w = kw.get(name, [0.0])
        fb = sum(f) / len(f) * 1024 * f_scale
        wb = sum(w) / len(w) * 1024 * w_scale
        per[sh] = fb + wb
        lines.append(f"{sh:14s} dispatches {len(f):3d}  FETCH_SIZE {sum(f) / len(f):12.1f} KiB  WRITE_SIZE "
                     f"{sum(w) / len(w):12.1f} KiB  -> HBM read {fb / 1e6:9.2f} MB  write {wb / 1e6:9.2f} MB")
    if family == "aaq":
        wl_path = os.path.join(PROFILE_DIR, f"aaq_{workload}_pmc.txt")
        sha = kernel_sha(AAQ_SRC)
        cmd_b = f"python3 $R/bench.py --workload {workload} --aaq-only --steps 3"
        tail = [f"{k}_traffic_bytes_per_launch={v:.6e} kernel_sha={sha}" for k, v in sorted(per.items())]
    else:
        wl_path = os.path.join(PROFILE_DIR, f"tri_attend_{workload}_pmc.txt")
        sha = kernel_sha()
        cmd_b = f"python3 $R/bench.py --workload {workload} --steps 3 --warmup 1 --no-cpu-baseline --key-blocks 0 --aaq 0 --knn 0 --other-workloads 0"
        tail = [f"traffic_bytes_per_launch={per.get('tri_attend', 0.0):.6e} kernel_sha={sha}",
                f"tri_project_traffic_bytes_per_launch={per.get('tri_project', 0.0):.6e} kernel_sha={sha}"]
    cmd_c = f"python3 $R/bench.py --copy-calibration {copy_mib}"
    txt = [f"# HBM traffic per dispatch, workload {workload}, gfx950 (MI355X)",
           "# commands (R = repository root, O = output directory, run from /tmp):",
           f"#   timeout -s KILL 100 rocprofv3 --pmc FETCH_SIZE --output-format csv -d $O/pmc_fetch -o f -- {cmd_b}",
           f"#   timeout -s KILL 100 rocprofv3 --pmc WRITE_SIZE --output-format csv -d $O/pmc_write -o w -- {cmd_b}",
           f"#   timeout -s KILL 100 rocprofv3 --pmc FETCH_SIZE --output-format csv -d $O/pmc_copy_fetch -o cf -- {cmd_c}",
           f"#   timeout -s KILL 100 rocprofv3 --pmc WRITE_SIZE --output-format csv -d $O/pmc_copy_write -o cw -- {cmd_c}",
           f"#   python3 bench.py --summarize-pmc $O --workload {workload}" + (" --family aaq" if family == "aaq" else ""),
           f"# calibration: a {copy_mib} MiB device copy reads FETCH_SIZE {sum(copy_f) / len(copy_f):.1f} KiB and "
           f"WRITE_SIZE {sum(copy_w) / len(copy_w):.1f} KiB;",
           f"#   scale factors FETCH x{f_scale:.4f}, WRITE x{w_scale:.4f}",
           *lines,
           *tail]
    open(wl_path, "w").write("\n".join(txt) + "\n")
    print("\n".join(txt))


SQ_PASSES = [
    "GRBM_GUI_ACTIVE SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES "
    "SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_VALU2 SQ_WAIT_INST_ANY SQ_WAIT_ANY",
    "GRBM_GUI_ACTIVE SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_SALU SQ_ACTIVE_INST_LDS SQ_WAIT_INST_LDS "
    "SQ_LDS_BANK_CONFLICT SQ_ACTIVE_INST_ANY",
    "GRBM_GUI_ACTIVE SQ_INSTS_VMEM SQ_INSTS_VALU_TRANS_F32 SQ_ACTIVE_INST_SCA SQ_WAVES SQ_BUSY_CU_CYCLES",
]


def _sq_target(workload, family):
    """(kernel short name, bench command, summary path, source hash) of an SQ summary."""
    if family == "knn":
        return ("knn_select_encode", "python3 $R/bench.py --knn-only --steps 3",
                os.path.join(PROFILE_DIR, "knn_select_encode_knn-L16384-k32_sq.txt"), kernel_sha(KNN_SRC))
    if family == "aaq":
        return ("aaq_encode_A_bf16", f"python3 $R/bench.py --workload {workload} --aaq-only --steps 3",
                os.path.join(PROFILE_DIR, f"aaq_encode_A_bf16_{workload}_sq.txt"), kernel_sha(AAQ_SRC))
    return ("tri_attend", f"python3 $R/bench.py --workload {workload} --steps 3 --warmup 1 --no-cpu-baseline "
            "--key-blocks 0 --aaq 0 --knn 0 --other-workloads 0",
            os.path.join(PROFILE_DIR, f"tri_attend_{workload}_sq.txt"), kernel_sha())


def summarize_sq(run_dir, workload, family="tri"):
    """Write a kernel's SQ counter summary (matrix-core and VALU activity): the
    one-pass attention kernel, or with family "knn" / "aaq" the kNN selection or
    the group-A encode kernel.

    run_dir holds sq1/ sq2/ sq3/: bench.py under the three counter sets of SQ_PASSES.
    rocprofv3 reports each counter summed over the device; GRBM_GUI_ACTIVE is summed
    over the 8 XCDs, so one XCD's busy cycles are GRBM_GUI_ACTIVE / 8, and the
    fractions below are per SIMD: counter / (GRBM_GUI_ACTIVE / 8 x 1024 SIMDs),
    with the quad-cycle counters (SQ_ACTIVE_INST_*) multiplied by 4.
    """
    import collections
    import csv
    import glob
    kname, cmd, path, sha = _sq_target(workload, family)
    acc = collections.defaultdict(list)
    durations = []
    for n in range(1, len(SQ_PASSES) + 1):
        files = glob.glob(os.path.join(run_dir, f"sq{n}", "**", "*counter_collection.csv"), recursive=True)
        if len(files) != 1:
            raise SystemExit(f"expected one counter_collection.csv under {run_dir}/sq{n}")
        per = collections.defaultdict(dict)
        for r in csv.DictReader(open(files[0])):
            if _short(r["Kernel_Name"]) != kname:
                continue
            per[r["Dispatch_Id"]][r["Counter_Name"]] = float(r["Counter_Value"])
            if n == 1 and r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                durations.append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
        for d in per.values():
            for k, v in d.items():
                acc[k].append(v)
    c = {k: sum(v) / len(v) for k, v in acc.items()}
    xcd_cycles = c["GRBM_GUI_ACTIVE"] / 8
    simd_cycles = xcd_cycles * 1024
    dur = sum(durations) / len(durations)
    waves = c.get("SQ_WAVES", 0.0)

    def frac(name, quad=False):
        return c[name] * (4 if quad else 1) / simd_cycles

    mfma, valu, coex = frac("SQ_VALU_MFMA_BUSY_CYCLES"), frac("SQ_ACTIVE_INST_VALU", True), \
        frac("SQ_VALU_MFMA_COEXEC_CYCLES")
    what = "the one-pass attention kernel (tri_attend)" if family == "tri" else kname
    if family == "knn":
        workload = "knn-L16384-k32"
    lines = [f"# SQ counters of {what}, workload {workload}, gfx950 (MI355X)",
             "# commands (R = repository root, O = output directory, run from /tmp), n = 1, 2, 3 over the counter sets:"]
    for n, pset in enumerate(SQ_PASSES, 1):
        lines.append(f"#   timeout -s KILL 100 rocprofv3 --pmc {pset} --output-format csv -d $O/sq{n} -o s -- {cmd}")
    lines.append(f"#   python3 bench.py --summarize-sq $O --workload {workload}"
                 + (f" --family {family}" if family != "tri" else ""))
    lines.append(f"# kernel_sha={sha}")
    lines.append("# normalisation: per SIMD, counter / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs);"
                 " SQ_ACTIVE_INST_* are in quad-cycles (x 4), SQ_WAVE_CYCLES and SQ_WAIT_* in quad-cycles too")
    lines += [f"{k:28s} {v:18.1f}" for k, v in sorted(c.items())]
    lines += [
        f"dispatches_per_pass        {len(durations)}",
        f"avg_dispatch_ms            {dur * 1e3:.4f}",
        f"effective_clock_ghz        {xcd_cycles / dur / 1e9:.3f}   (GRBM_GUI_ACTIVE / 8 / dispatch time)",
        f"mfma_busy                  {mfma:.4f}   (SQ_VALU_MFMA_BUSY_CYCLES per SIMD-cycle)",
        f"valu_active                {valu:.4f}   (4 x SQ_ACTIVE_INST_VALU, VALU cycles summed over the waves, per "
        "SIMD-cycle; MFMA issue included)",
        f"mfma_valu_coexec           {coex:.4f}   (SQ_VALU_MFMA_COEXEC_CYCLES per SIMD-cycle)",
        f"mfma_or_valu               {mfma + valu - coex:.4f}",
        f"wave_wait_inst_any         {c['SQ_WAIT_INST_ANY'] / c['SQ_WAVE_CYCLES']:.4f}   "
        "(SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES, both in quad-cycles: share of the waves' life waiting to issue)"
        if "SQ_WAIT_INST_ANY" in c else "",
        f"wave_wait_any              {c['SQ_WAIT_ANY'] / c['SQ_WAVE_CYCLES']:.4f}   "
        "(SQ_WAIT_ANY / SQ_WAVE_CYCLES: share of the waves' life in s_waitcnt)" if "SQ_WAIT_ANY" in c else "",
    ]
    if waves:
        lines += [f"valu_insts_per_wave        {c['SQ_INSTS_VALU'] / waves:.1f}",
                  f"mfma_insts_per_wave        {c['SQ_INSTS_MFMA'] / waves:.1f}",
                  f"trans_f32_insts_per_wave   {c['SQ_INSTS_VALU_TRANS_F32'] / waves:.1f}",
                  f"lds_insts_per_wave         {c['SQ_INSTS_LDS'] / waves:.1f}",
                  f"salu_insts_per_wave        {c['SQ_INSTS_SALU'] / waves:.1f}",
                  f"vmem_insts_per_wave        {c['SQ_INSTS_VMEM'] / waves:.1f}"]
    open(path, "w").write("\n".join(x for x in lines if x) + "\n")
    print("\n".join(lines))


def summarize_trace(run_dir, workload, steps, warmup, family="tri"):
    """Write the per-kernel duration summary from a rocprofv3 --kernel-trace --stats csv run."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*kernel_stats.csv"), recursive=True)
    if len(files) != 1:
        raise SystemExit(f"expected one kernel_stats.csv under {run_dir}, found {files}")
    rows = list(csv.DictReader(open(files[0])))
    if family == "aaq":
        run = f"python3 $R/bench.py --workload {workload} --aaq-only --steps {steps}"
        summ = f"python3 bench.py --summarize-trace $O/kt --workload {workload} --steps {steps} --family aaq"
        sha, path = kernel_sha(AAQ_SRC), os.path.join(PROFILE_DIR, f"aaq_{workload}_trace.txt")
    elif family == "knn":
        workload = "knn-L16384-k32"
        run = f"python3 $R/bench.py --knn-only --steps {steps}"
        summ = f"python3 bench.py --summarize-trace $O/kt --steps {steps} --family knn"
        sha, path = kernel_sha(KNN_SRC), os.path.join(PROFILE_DIR, "knn_knn-L16384-k32_trace.txt")
    else:
        run = (f"python3 $R/bench.py --workload {workload} --steps {steps} --warmup {warmup} --no-cpu-baseline "
               f"--key-blocks 0 --aaq 0 --knn 0 --other-workloads 0")
        summ = f"python3 bench.py --summarize-trace $O/kt --workload {workload} --steps {steps} --warmup {warmup}"
        sha, path = kernel_sha(), os.path.join(PROFILE_DIR, f"kernels_{workload}_trace.txt")
    out = [f"# rocprofv3 kernel statistics, workload {workload}, gfx950 (MI355X)",
           "# command (R = repository root, O = output directory, run from /tmp):",
           f"#   timeout -k 10 300 rocprofv3 --kernel-trace --stats --output-format csv -d $O/kt -o kt -- {run}",
           f"#   {summ}",
           f"# kernel_sha={sha}",
           f"{'kernel':16s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>6s}"]
    for r in rows:
        sh = _short(r["Name"])
        if not sh.startswith(family + "_"):
            continue
        out.append(f"{sh:16s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.1f} {float(r['MinNs']) / 1e3:10.1f} "
                   f"{float(r['MaxNs']) / 1e3:10.1f} {float(r['Percentage']):6.2f}")
    open(path, "w").write("\n".join(out) + "\n")
    print("\n".join(out))


ISSUE_PROBE_MODES = [  # (mode of csrc/issue_probe.hip, what one loop iteration issues, instructions per iteration)
    (0, "v_exp_f32, 8 independent", 8),
    (1, "v_exp_f16, 8 independent", 8),
    (2, "v_cvt_pk_bf16_f32, 8 chained", 8),
    (3, "v_mfma_f32_32x32x16_bf16, 4 independent", 4),
    (4, "v_mfma_f32_16x16x32_bf16, 4 independent", 4),
    (5, "phase: 4 + 2 products (in dependent pairs) alone", 6),
    (6, "phase: 16 exp + 8 P conversions + 9 widenings alone", 33),
    (7, "phase: both, one product per 5-6 VALU instructions", 39),
]


def issue_probe():
    """Issue costs of the attention loop's instructions on this GPU (no memory traffic in the
    measured loops), at two and three waves per SIMD; summary to profiles/issue_probe_gfx950.txt."""
    import ctypes
    from protein_pair_representation_amd.build import PROBE_PATH
    if not os.path.exists(PROBE_PATH):
        raise SystemExit(f"{PROBE_PATH} is missing: build it (python -m protein_pair_representation_amd.build)")
    lib = ctypes.CDLL(PROBE_PATH)
    lib.issue_probe_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_double)]
    lib.issue_probe_run.restype = ctypes.c_int
    src = os.path.join(ROOT, "protein_pair_representation_amd", "csrc", "issue_probe.hip")
    lines = ["# issue costs of the attention loop's instruction mix, gfx950 (MI355X); no memory traffic in the loops",
             "# command: python3 bench.py --issue-probe",
             f"# probe source sha={kernel_sha(src)}",
             "# SIMD-cycles per loop iteration = kernel time x core clock / (waves per SIMD x iterations)",
             f"{'loop body':54s} {'waves/SIMD':>10s} {'cyc/iter':>9s} {'cyc/instr':>9s} {'GHz':>5s}"]
    for mode, what, ninstr in ISSUE_PROBE_MODES:
        for w in (2, 3):
            cyc, ghz = ctypes.c_double(), ctypes.c_double()
            rc = lib.issue_probe_run(mode, w, ctypes.byref(cyc), ctypes.byref(ghz))
            if rc != 0:
                raise SystemExit(f"issue_probe_run({mode}, {w}) returned {rc}")
            lines.append(f"{what:54s} {w:10d} {cyc.value:9.1f} {cyc.value / ninstr:9.2f} {ghz.value:5.2f}")
    open(os.path.join(PROFILE_DIR, "issue_probe_gfx950.txt"), "w").write("\n".join(lines) + "\n")
    print("\n".join(lines), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--key-blocks", type=int, default=4, metavar="NB",
                    help="also time the key-block stage with NB blocks + finalize (0: skip)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration) and exit")
    ap.add_argument("--summarize-pmc", metavar="DIR",
                    help="write the HBM-traffic summary under profiles/ from rocprofv3 --pmc runs in DIR, and exit")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="write the kernel-duration summary under profiles/ from a rocprofv3 --stats run, and exit")
    ap.add_argument("--copy-mib", type=int, default=1024, help="size of the calibration copy (--summarize-pmc)")
    ap.add_argument("--aaq", type=int, default=1, help="also time the AAQ codec on the pair tensor (0: skip)")
    ap.add_argument("--aaq-only", action="store_true",
                    help="time only the AAQ codec (encode/decode, groups A and B) over --steps launches each")
    ap.add_argument("--knn", type=int, default=1, help="also time the kNN sparse pair encoder (0: skip)")
    ap.add_argument("--knn-only", action="store_true",
                    help="time only the kNN sparse pair encoder (knn-L16384-k32) over --steps calls")
    ap.add_argument("--other-workloads", type=int, default=1,
                    help="also measure the other workloads (fewer steps each; 0: skip)")
    ap.add_argument("--summarize-sq", metavar="DIR",
                    help="write the attention kernel's SQ counter summary under profiles/ from rocprofv3 --pmc runs "
                         "in DIR, and exit")
    ap.add_argument("--issue-probe", action="store_true",
                    help="measure the issue costs of the attention loop's instruction mix (libissueprobe.so), "
                         "write the summary under profiles/, and exit")
    ap.add_argument("--family", default="tri", choices=["tri", "aaq", "knn"],
                    help="kernel family of --summarize-pmc / --summarize-trace / --summarize-sq")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc, args.workload, args.copy_mib, args.family)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.workload, args.steps, args.warmup, args.family)
        return
    if args.summarize_sq:
        summarize_sq(args.summarize_sq, args.workload, args.family)
        return
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); "
              "row sharding over several GPUs is not implemented.", file=sys.stderr)
        sys.exit(2)

    import torch
    from protein_pair_representation_amd import inputs
    from protein_pair_representation_amd import triattn as ta

    if args.issue_probe:
        issue_probe()
        return

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 3}))
        return

    if args.knn_only:
        print(json.dumps({"knn": knn_encoder(torch.cuda.current_stream(), reps=args.steps)}), flush=True)
        return

    wl = inputs.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    if args.aaq_only:
        z = inputs.workload_z(wl).to(dev)
        print(json.dumps({"workload": wl.name, "aaq": aaq_codec(z, wl.name, stream, reps=args.steps)}), flush=True)
        return

    m = measure_workload(wl, args.steps, args.warmup, stream)
    res = {
        "metric": "pair-attention TFLOP/s (bf16) and % of MFMA peak at I=1024, c_z=128",
        "value": m["value"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic (seeded N(0,1) pair tensor and weights, resident in HBM)",
        "config": {"workload": wl.name, "I": wl.I, "rows": wl.n_rows, "c_z": 128, "heads": 4, "head_dim": 32,
                   "variants": list(wl.variants)},
        "pct_of_peak_step": m["pct_of_peak_step"],
        "roofline": m["roofline"],
        "kernels": m["kernels"],
        "kernel_sha": kernel_sha(),
    }
    z, wd, ws = m.pop("_z"), m.pop("_wd"), m.pop("_ws")
    variants = list(wl.variants)
    if args.key_blocks > 0 and variants[0] != "rows":
        dt = inputs.DTYPES[wl.dtype]
        v0, k2ms = variants[0], m["roofline"]["avg_launch_ms"]
        res["key_blocks"] = key_blocks(ws[v0], wd, wl.I, wl.n_rows, dt, v0, args.key_blocks, stream,
                                       m["k2_flops"], k2ms)
        # caller-held blocks (the ring step): as many blocks, then half as many larger ones
        res["kv_blocks"] = [kv_blocks(ws[v0], wd, wl.I, wl.n_rows, dt, v0, nb, stream, m["k2_flops"], k2ms)
                            for nb in sorted({args.key_blocks, max(1, args.key_blocks // 2)}, reverse=True)]
    if args.aaq > 0:
        res["aaq"] = aaq_codec(z, wl.name, stream)
        if wl.dtype == "bf16":
            res["aaq"]["project_stage"] = aaq_project(z, wd, variants[0], stream)
    if args.knn > 0:
        res["knn"] = knn_encoder(stream)
    del z, wd, ws
    torch.cuda.empty_cache()
    if args.other_workloads:
        # the other workloads (I = 64 fp32, I = 384, I = 2048 with outliers, the I = 4096 row block), each measured the same way (fewer steps)
        others = {}
        for name in inputs.WORKLOADS:
            if name == wl.name:
                continue
            o = inputs.WORKLOADS[name]
            steps = 10 if o.I < 4096 else 5
            mo = measure_workload(o, steps, 3, stream)
            for k in ("_z", "_wd", "_ws"):
                mo.pop(k)
            others[name] = {"steps": steps, "warmup": 3, "ms_per_step": mo["ms_per_step"], "TFLOP/s": mo["value"],
                            "dtype": o.dtype, "roofline": mo["roofline"], "kernels": mo["kernels"]}
            torch.cuda.empty_cache()
        res["other_workloads"] = others
    res["gpu_clock"] = gpu_clock()
    mhz = res["gpu_clock"]["sclk_mhz"]
    if mhz and res["dtype"] == "bf16":
        # the dense bf16 peak at the reported clock: 256 CUs x 4096 flops per cycle (2.5 PF at 2.4 GHz)
        at_clock = 256 * 4096 * mhz * 1e6 / 1e12
        res["roofline"]["peak_at_reported_clock"] = round(at_clock, 1)
        res["roofline"]["frac_at_reported_clock"] = round(res["roofline"]["achieved"] / at_clock, 4)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, inputs.workload_z(wl), inputs.workload_weights(wl))
    print(json.dumps(res), flush=True)


def gpu_clock():
    """Shader clock of GPU 0 as rocm-smi reports it right after the timed runs (a snapshot)."""
    import subprocess
    try:
        out = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=20)
        data = json.loads(out.stdout)
        card = data.get("card0") or next(iter(data.values()))
        sclk = next((v for k, v in card.items() if k.lower().startswith("sclk")), None)
        mhz = float(re.search(r"([0-9.]+)\s*Mhz", str(sclk), re.I).group(1)) if sclk else None
        return {"sclk_mhz": mhz, "source": "rocm-smi --showclocks (after the timed region)"}
    except Exception as e:  # the clock is context; its absence does not fail the bench
        return {"sclk_mhz": None, "source": f"rocm-smi unavailable: {type(e).__name__}"}


def measure_workload(wl, steps, warmup, stream):
    """Time `steps` steps of a workload (every variant: K1 + bias pack, then K2) with inputs
    resident in HBM; K1 and K2 are also timed per launch with HIP events on `stream`."""
    import torch
    from protein_pair_representation_amd import inputs
    from protein_pair_representation_amd import triattn as ta

    dt = inputs.DTYPES[wl.dtype]
    es = 2 if wl.dtype == "bf16" else 4
    dev = torch.device("cuda:0")
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
        del parts
    else:
        z = inputs.workload_z(wl).to(dev)
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

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(steps)]
    warm = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    for _ in range(warmup):
        step(warm)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_ in range(steps):
        step(events[s_])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for v in variants:
        assert torch.isfinite(out[v]).all(), f"non-finite output ({wl.name} {v})"

    ms_step = (t1 - t0) * 1e3 / steps
    k1_all = sorted(e[3 * n_].elapsed_time(e[3 * n_ + 1]) for e in events for n_ in range(len(variants)))
    k2_all = sorted(e[3 * n_ + 1].elapsed_time(e[3 * n_ + 2]) for e in events for n_ in range(len(variants)))
    k1_ms = sum(k1_all) / len(k1_all)
    k2_ms = sum(k2_all) / len(k2_all)
    step_flops = 0.0
    for v in variants:
        proj, attn, o = flops(I, R, v != "rows")
        step_flops += proj + attn + o
    _, attn1, out1 = flops(I, R, False)
    k2_flops = attn1 + out1
    k2_tflops = k2_flops / (k2_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS
    k1b = k1_bytes(I, R, es, "rows" not in variants)
    value = step_flops / (ms_step * 1e-3) / 1e12
    return {
        "value": round(value, 2), "ms_per_step": round(ms_step, 4), "pct_of_peak_step": round(100 * value / peak, 2),
        "k2_flops": k2_flops,
        "roofline": {"kernel": "tri_attend", "bound": "mfma", "achieved": round(k2_tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(k2_tflops / peak, 4),
                     "traffic": read_traffic(wl.name), "algorithmic_bytes": k2_bytes(I, R, es),
                     "flops_per_launch": k2_flops, "avg_launch_ms": round(k2_ms, 4)},
        "kernels": {"project_stage (tri_project + tri_pack_bias)": {
                        "avg_ms": round(k1_ms, 4), "algorithmic_bytes": k1b,
                        "min_ms": round(k1_all[0], 4), "median_ms": round(k1_all[len(k1_all) // 2], 4),
                        "GB/s": round(k1b / (k1_ms * 1e-3) / 1e9, 1),
                        "frac_hbm": round(k1b / (k1_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
                    "tri_attend": {"avg_launch_ms": round(k2_ms, 4), "TFLOP/s": round(k2_tflops, 2),
                                   "min_launch_ms": round(k2_all[0], 4),
                                   "median_launch_ms": round(k2_all[len(k2_all) // 2], 4)}},
        "_z": z, "_wd": wd, "_ws": ws,
    }


if __name__ == "__main__":
    main()
