"""Seeded synthetic inputs for pair-biased triangle attention.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the attention arithmetic, so both the fp64 oracle and the
HIP library can consume what it produces without sharing any of the method.

Recipe (every workload):

* ``numpy.random.SeedSequence(seed)`` is split into three children:
  child 0 draws the weights, child 1 the pair tensor Z, child 2 the outlier
  mask.  Z is drawn in blocks of ``Z_BLOCK_ROWS`` rows, each block from its own
  grandchild of child 1, so any block of rows can be regenerated on its own.
* Z entries are N(0, 1) (float32 draws).  Optional structure:
  - "distogram": 2*exp(-|i-j|/32) added to every channel of token (i, j), with
    0-based global indices (a smooth distance-like pair pattern, as the
    LightNobel article describes for pair activations, section 2.2.1);
  - "outliers": every entry independently with probability 0.01 is
    multiplied by 20 (per-token outlier channels at varying positions, LightNobel
    article section 2.2.2).
* Weights use the torch.nn.Linear convention, W[out][in]:
  w_q, w_k, w_v, w_g: [H*d][c_z]; w_b: [H][c_z]; w_o: [c_z][H*d], every entry
  N(0, 1/c_z), drawn in that order (q, k, v, b, g, o).  LayerNorm gamma = 1,
  beta = 0, gate bias b_g = 0, output bias b_o = 0.
* Everything is rounded (round-to-nearest-even) to the storage dtype once;
  the rounded values are the inputs of both sides.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

C_Z = 128
HEADS = 4
HEAD_DIM = 32
LN_EPS = 1e-5
Z_BLOCK_ROWS = 64

DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: pair tensor side I, rows handled, dtype, structure."""

    name: str
    I: int
    dtype: str  # "bf16" | "f32"
    seed: int
    variants: tuple = ("start",)
    rows: int | None = None  # row-block size (row-block variant); None = all I rows
    distogram: bool = False
    outliers: bool = False
    c_z: int = C_Z
    heads: int = HEADS
    head_dim: int = HEAD_DIM
    notes: str = field(default="", compare=False)

    @property
    def n_rows(self) -> int:
        return self.I if self.rows is None else self.rows


# The five workloads the library is built and measured against.
WORKLOADS = {
    "start-f32-I64": Workload("start-f32-I64", 64, "f32", 1, ("start",),
                              notes="fp32 correctness case, Z 64x64x128"),
    "start-bf16-I384": Workload("start-bf16-I384", 384, "bf16", 2, ("start",),
                                notes="bf16, Z 384x384x128, gating on"),
    "startend-bf16-I1024-distogram": Workload(
        "startend-bf16-I1024-distogram", 1024, "bf16", 3, ("start", "end"), distogram=True,
        notes="bf16, Z 1024x1024x128 + 2exp(-|i-j|/32); starting and ending node"),
    "start-bf16-I2048-outliers": Workload(
        "start-bf16-I2048-outliers", 2048, "bf16", 4, ("start",), outliers=True,
        notes="bf16, Z 2048x2048x128 with 1% of entries x20"),
    "rows-bf16-R1024-I4096": Workload(
        "rows-bf16-R1024-I4096", 4096, "bf16", 5, ("rows",), rows=1024,
        notes="bf16, rows 0..1023 of Z 4096x4096x128, full 4096x4096xH bias local"),
}


def _children(seed: int):
    return np.random.SeedSequence(seed).spawn(3)


def make_weights(seed: int, dtype: str = "bf16", c_z: int = C_Z, heads: int = HEADS,
                 head_dim: int = HEAD_DIM) -> dict:
    """Weights of one triangle-attention block (nn.Linear layout, storage dtype)."""
    rng = np.random.default_rng(_children(seed)[0])
    hd = heads * head_dim
    std = 1.0 / np.sqrt(c_z)
    shapes = [("w_q", (hd, c_z)), ("w_k", (hd, c_z)), ("w_v", (hd, c_z)),
              ("w_b", (heads, c_z)), ("w_g", (hd, c_z)), ("w_o", (c_z, hd))]
    tdt = DTYPES[dtype]
    w = {}
    for name, shape in shapes:
        w[name] = torch.from_numpy(rng.standard_normal(shape) * std).to(tdt).contiguous()
    w["ln_gamma"] = torch.ones(c_z, dtype=torch.float32)
    w["ln_beta"] = torch.zeros(c_z, dtype=torch.float32)
    w["b_g"] = torch.zeros(hd, dtype=torch.float32)
    w["b_o"] = torch.zeros(c_z, dtype=torch.float32)
    return w


def make_z_rows(seed: int, I: int, row0: int, n_rows: int, dtype: str = "bf16",
                c_z: int = C_Z, distogram: bool = False, outliers: bool = False) -> torch.Tensor:
    """Rows [row0, row0 + n_rows) of the seeded pair tensor Z (I x I x c_z), storage dtype."""
    if n_rows <= 0:
        return torch.empty((0, I, c_z), dtype=DTYPES[dtype])
    ch = _children(seed)
    b0, b1 = row0 // Z_BLOCK_ROWS, (row0 + n_rows - 1) // Z_BLOCK_ROWS
    n_blocks_total = (I + Z_BLOCK_ROWS - 1) // Z_BLOCK_ROWS
    z_blocks = ch[1].spawn(n_blocks_total)
    m_blocks = ch[2].spawn(n_blocks_total)
    out = torch.empty((n_rows, I, c_z), dtype=DTYPES[dtype])

    def block(b):
        r_lo = b * Z_BLOCK_ROWS
        r_hi = min(I, r_lo + Z_BLOCK_ROWS)
        zb = np.random.default_rng(z_blocks[b]).standard_normal(
            (r_hi - r_lo, I, c_z), dtype=np.float32)
        if outliers:
            mask = np.random.default_rng(m_blocks[b]).random((r_hi - r_lo, I, c_z),
                                                              dtype=np.float32) < 0.01
            zb[mask] *= 20.0
        if distogram:
            i = np.arange(r_lo, r_hi, dtype=np.float32)[:, None]
            j = np.arange(I, dtype=np.float32)[None, :]
            zb += (2.0 * np.exp(-np.abs(i - j) / 32.0)).astype(np.float32)[:, :, None]
        s_lo, s_hi = max(r_lo, row0), min(r_hi, row0 + n_rows)
        out[s_lo - row0:s_hi - row0] = torch.from_numpy(zb[s_lo - r_lo:s_hi - r_lo]).to(DTYPES[dtype])

    # blocks are independent (own generators, disjoint rows of out): drawn on threads
    blocks = range(b0, b1 + 1)
    if len(blocks) == 1:
        block(b0)
    else:
        with ThreadPoolExecutor(max(1, min(8, len(os.sched_getaffinity(0)), len(blocks)))) as ex:
            list(ex.map(block, blocks))
    return out


def make_z(seed: int, I: int, dtype: str = "bf16", c_z: int = C_Z, distogram: bool = False,
           outliers: bool = False) -> torch.Tensor:
    return make_z_rows(seed, I, 0, I, dtype, c_z, distogram, outliers)


def workload_z(w: Workload, row0: int = 0, n_rows: int | None = None) -> torch.Tensor:
    n = w.I if n_rows is None else n_rows
    return make_z_rows(w.seed, w.I, row0, n, w.dtype, w.c_z, w.distogram, w.outliers)


def workload_weights(w: Workload) -> dict:
    return make_weights(w.seed, w.dtype, w.c_z, w.heads, w.head_dim)


def random_bias(seed: int, heads: int, I: int, scale: float = 1.0, offset_per_query=None) -> torch.Tensor:
    """A caller-supplied fp32 pair bias [H][I][I] ~ N(0, scale^2) (row-block tests)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 7]))
    b = (rng.standard_normal((heads, I, I)) * scale).astype(np.float32)
    if offset_per_query is not None:
        b += np.asarray(offset_per_query, dtype=np.float32)[None, :, None]
    return torch.from_numpy(b)


TOKEN_KINDS = ("gaussian", "offset", "spikes", "tied_spikes", "zeros", "constant", "integers", "tiny")


def make_tokens(seed: int, n: int, dtype: str = "bf16", c_z: int = C_Z) -> torch.Tensor:
    """n synthetic tokens [n][c_z] of mixed shapes, for the quantization codec.

    Token t is of kind TOKEN_KINDS[t % 8]: N(0, 1) scaled by 10^U(-3, 2) per token
    ("gaussian"); the same plus an offset of 4 sigma, so every value has one sign
    ("offset"); N(0, 1) with 1 to 8 channels set to +-U(5, 40) ("spikes"); the same
    with every spike of one magnitude, signs random ("tied_spikes"); all zeros;
    one value repeated; integers in [-8, 7]; N(0, 1) x 1e-30.  Rounded once
    (nearest even) to the storage dtype.
    """
    rng = np.random.default_rng(np.random.SeedSequence([seed, 11]))
    x = rng.standard_normal((n, c_z))
    scale = 10.0 ** rng.uniform(-3, 2, (n, 1))
    kind = np.arange(n) % len(TOKEN_KINDS)
    n_sp = rng.integers(1, 9, n)
    mag = rng.uniform(5, 40, (n, c_z))
    sign = np.where(rng.random((n, c_z)) < 0.5, -1.0, 1.0)
    perm = np.argsort(rng.random((n, c_z)), axis=-1)
    spike = np.zeros((n, c_z), dtype=bool)
    np.put_along_axis(spike, perm[:, :8], (np.arange(8)[None, :] < n_sp[:, None]), axis=-1)
    ints = rng.integers(-8, 8, (n, c_z)).astype(np.float64)
    const = rng.standard_normal((n, 1)) * scale
    out = x * scale
    out = np.where((kind == 1)[:, None], (x + 4.0) * scale, out)
    out = np.where((kind == 2)[:, None], np.where(spike, sign * mag, x), out)
    out = np.where((kind == 3)[:, None], np.where(spike, sign * mag[:, :1], x), out)
    out = np.where((kind == 4)[:, None], 0.0, out)
    out = np.where((kind == 5)[:, None], np.broadcast_to(const, (n, c_z)), out)
    out = np.where((kind == 6)[:, None], ints, out)
    out = np.where((kind == 7)[:, None], x * 1e-30, out)
    return torch.from_numpy(out.astype(np.float32)).to(DTYPES[dtype]).contiguous()


ATOMS_PER_RESIDUE = 8
KNN_WORKLOADS = {
    "knn-L16384-k32": dict(L=16384, k=32, seed=6,
                           notes="16384 atoms (2048 residues x 8) along a random-walk chain, k = 32"),
}


def make_atoms(seed: int, L: int, c_s: int = 128, c_p: int = 16) -> dict:
    """Synthetic atoms for the kNN pair encoder: coordinates x [L][3] fp32, single
    features s [L][c_s] bf16, weights w_l, w_m [c_p][c_s] bf16 (N(0, 1/c_s)),
    w_d [c_p][4] fp32 (N(0, 1/4)).

    Coordinates: residues along a random walk of 3.8 A steps in uniformly random
    directions (a chain of alpha carbons), each carrying ATOMS_PER_RESIDUE atoms at
    N(0, 1.2 A) offsets from it per axis; L is cut from that chain.
    """
    rng = np.random.default_rng(np.random.SeedSequence([seed, 13]))
    n_res = (L + ATOMS_PER_RESIDUE - 1) // ATOMS_PER_RESIDUE
    steps = rng.standard_normal((n_res, 3))
    steps *= 3.8 / np.linalg.norm(steps, axis=1, keepdims=True)
    ca = np.cumsum(steps, axis=0)
    x = (np.repeat(ca, ATOMS_PER_RESIDUE, axis=0)[:L]
         + rng.standard_normal((n_res * ATOMS_PER_RESIDUE, 3))[:L] * 1.2).astype(np.float32)
    s = torch.from_numpy(rng.standard_normal((L, c_s)).astype(np.float32)).to(torch.bfloat16)
    w_l = torch.from_numpy(rng.standard_normal((c_p, c_s)) / np.sqrt(c_s)).to(torch.bfloat16)
    w_m = torch.from_numpy(rng.standard_normal((c_p, c_s)) / np.sqrt(c_s)).to(torch.bfloat16)
    w_d = torch.from_numpy((rng.standard_normal((c_p, 4)) * 0.5).astype(np.float32))
    return {"x": torch.from_numpy(x), "s": s.contiguous(), "w_l": w_l.contiguous(), "w_m": w_m.contiguous(),
            "w_d": w_d.contiguous()}


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of stored values (bf16/fp32) to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def weights_f64(w: dict) -> dict:
    return {k: to_f64(v) for k, v in w.items()}
