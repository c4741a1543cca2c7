"""k-nearest-neighbour sparse atom-pair encoder -- TEST INFRASTRUCTURE ONLY.

A plain CPU implementation of the low-memory pair encoder of the Design-CP
summary (section "Detalles de implementación", memory optimisation): the
atom-pair tensor P is built only at the k nearest neighbours of each atom
instead of for all L x L atom pairs.  The HIP library is checked against it;
the library never imports it.

What the page fixes: pair features of atoms, built at sparse k-nearest-
neighbour indices, never materialised densely.

Readings where the page is silent (each one a line of the design notes):

* neighbours: for atom l, the k atoms m != l with the smallest squared
  distance |x_l - x_m|^2, in ascending order, equal distances going to the
  lower index.  The squared distance is evaluated in float32 in a fixed
  order, ((dx*dx + dy*dy) + dz*dz) with d = x_l - x_m, each operation rounded
  to nearest even; the device selects with the same float32 values, so the
  neighbour lists agree exactly;
* pair features: p_lm = W_l s_l + W_m s_m + W_d phi(x_l - x_m) with
  phi(d) = (d_x, d_y, d_z, 1 / (1 + |d|^2)) -- each atom's single features
  projected, the relative position and an inverse-square distance, the
  feature set of AlphaFold 3's atom-pair embedding (Abramson et al. 2024,
  Algorithm 5), taken here as the plainest pair encoder;
* shapes: c_s = 128 single channels (bf16), c_p = 16 pair channels, weights
  in torch.nn.Linear layout (W[out][in]); |d|^2 in phi is the float32
  selection value; everything else in float64.

Parity status: pinned by ``tests/test_oracle_knn.py`` (pure-Python brute force,
closed forms on a lattice, translation and permutation invariance, planted
mistakes).  No function here is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

C_S = 128
C_P = 16


def sq_dist_f32(xl: np.ndarray, xm: np.ndarray) -> np.ndarray:
    """float32 squared distances ((dx*dx + dy*dy) + dz*dz), d = xl - xm (broadcast)."""
    xl = np.asarray(xl, dtype=np.float32)
    xm = np.asarray(xm, dtype=np.float32)
    d = xl - xm
    return (d[..., 0] * d[..., 0] + d[..., 1] * d[..., 1]) + d[..., 2] * d[..., 2]


def neighbours(x: np.ndarray, k: int, rows=None) -> tuple[np.ndarray, np.ndarray]:
    """Indices [R][k] (int64) and float32 squared distances [R][k] of the k nearest
    atoms of each atom in `rows` (default: all), excluding the atom itself."""
    x = np.asarray(x, dtype=np.float32)
    L = x.shape[0]
    rows = np.arange(L) if rows is None else np.asarray(rows)
    idx = np.empty((len(rows), k), dtype=np.int64)
    d2 = np.empty((len(rows), k), dtype=np.float32)
    cand = np.arange(L)
    for n, l in enumerate(rows):
        dl = sq_dist_f32(x[l], x)
        order = np.lexsort((cand, dl))          # primary: distance, then index
        order = order[order != l][:k]
        idx[n], d2[n] = order, dl[order]
    return idx, d2


def phi(x: np.ndarray, rows: np.ndarray, idx: np.ndarray, d2: np.ndarray) -> np.ndarray:
    """Geometric features [R][k][4]: x_l - x_m (exact in float64) and 1 / (1 + |d|^2)."""
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    d = x64[rows][:, None, :] - x64[idx]
    return np.concatenate([d, (1.0 / (1.0 + d2.astype(np.float64)))[..., None]], axis=-1)


def pair_features(x, s, w_l, w_m, w_d, k, rows=None):
    """(neighbour indices [R][k], pair tensor [R][k][c_p] float64) of the atoms in `rows`."""
    L = np.asarray(x).shape[0]
    rows = np.arange(L) if rows is None else np.asarray(rows)
    idx, d2 = neighbours(x, k, rows)
    s64 = np.asarray(s, dtype=np.float64)
    a = s64[rows] @ np.asarray(w_l, dtype=np.float64).T          # [R][c_p]
    b = s64 @ np.asarray(w_m, dtype=np.float64).T                # [L][c_p]
    p = a[:, None, :] + b[idx] + phi(x, rows, idx, d2) @ np.asarray(w_d, dtype=np.float64).T
    return idx, p
