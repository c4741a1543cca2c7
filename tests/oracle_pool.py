"""Whole-output comparison of a GPU result with the float64 oracle, over a process pool.

The oracle is evaluated row by row (starting node, row block) or column by
column (ending node) in forked worker processes, one BLAS thread each; every
worker compares its part with the GPU output and returns only the error sums,
so the full oracle output is never gathered in one place.
"""
from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np

from oracle import ref

_G: dict = {}


def _limit_blas():
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)


def workers() -> int:
    """Cores in this process's affinity, at most 16 (one GPU's share of a host's cores)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _part(task):
    kind, idx = task
    if kind == "end":
        want = ref.triangle_attn_end(_G["z64"], _G["p"], cols=idx, bias=_G["bias"])   # [I][n][c]
        got = _G["got"][:, idx]
    else:                                                                          # start / rows
        want = ref.triangle_attn_rows(_G["z64"][idx], _G["bias"], _G["p"])             # [n][I][c]
        got = _G["got"][idx]
    got = got.astype(np.float64)
    finite = np.isfinite(got)
    err = np.abs(np.where(finite, got, 0.0) - want)
    return float(err.sum()), float(np.abs(want).sum()), float(err.max()), int((~finite).sum()), int(err.size)


def compare(kind, z64, bias, p, got, index, chunk=8, progress=None):
    """Errors of got (float32/float64 numpy, the GPU output) against the oracle.

    kind "start" / "rows": got[i] for every row i in ``index`` of z64 (rows of Z
    with the given bias [H][I][I]); kind "end": got[:, j] for every column j in
    ``index``.  Returns (max abs, relative L1, non-finite count, elements).
    progress(done, total) is called as parts finish (long comparisons report
    through it).
    """
    index = list(index)
    tasks = [(kind, index[k:k + chunk]) for k in range(0, len(index), chunk)]
    _G.update(z64=z64, bias=bias, p=p, got=got)
    parts = []
    try:
        with mp.get_context("fork").Pool(min(workers(), len(tasks)), initializer=_limit_blas) as pool:
            for part in pool.imap_unordered(_part, tasks, chunksize=1):
                parts.append(part)
                if progress is not None:
                    progress(len(parts), len(tasks))
    finally:
        _G.clear()
    esum = sum(x[0] for x in parts)
    rsum = sum(x[1] for x in parts)
    return max(x[2] for x in parts), esum / max(rsum, 1e-300), sum(x[3] for x in parts), sum(x[4] for x in parts)
