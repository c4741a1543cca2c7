"""Pins for the kNN sparse atom-pair encoder oracle (CPU only).

* pure-Python brute force (explicit loops, Python's own sort) on integer
  lattices, where every squared distance is an exact integer, and on random
  float32 coordinates with float32 arithmetic written out term by term;
* closed forms: atoms on a line (neighbours alternate left/right, ties to the
  lower index), features equal to phi when only W_d is the identity, and to
  torch CPU linear layers when W_d = 0;
* invariances: integer translations, permutations of the atom order;
* planted mistakes: each mutant of the oracle must fail at least one pin.
"""
import numpy as np
import pytest
import torch

from oracle import knn

C_S, C_P = knn.C_S, knn.C_P


def brute_neighbours(coords, k):
    """Explicit loops over float32 scalars; ranking with sorted() on (d2, index)."""
    L = len(coords)
    out = []
    for l in range(L):
        cand = []
        for m in range(L):
            if m == l:
                continue
            dx = np.float32(coords[l][0]) - np.float32(coords[m][0])
            dy = np.float32(coords[l][1]) - np.float32(coords[m][1])
            dz = np.float32(coords[l][2]) - np.float32(coords[m][2])
            d2 = np.float32(np.float32(dx * dx) + np.float32(dy * dy))
            d2 = np.float32(d2 + np.float32(dz * dz))
            cand.append((float(d2), m))
        out.append([m for _, m in sorted(cand)[:k]])
    return out


def rand_weights(rng):
    w_l = rng.standard_normal((C_P, C_S)) / np.sqrt(C_S)
    w_m = rng.standard_normal((C_P, C_S)) / np.sqrt(C_S)
    w_d = rng.standard_normal((C_P, 4))
    return w_l, w_m, w_d


# ----------------------------------------------------------------------------------------
# Pins as functions of the oracle module.

def pin_brute_lattice(seed=0):
    rng = np.random.default_rng(seed)
    x = rng.integers(-4, 5, (40, 3)).astype(np.float32)   # many exact ties
    idx, _ = knn.neighbours(x, 7)
    assert [list(r) for r in idx] == brute_neighbours(x.tolist(), 7)


def pin_brute_float(seed=1):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((30, 3)) * 5).astype(np.float32)
    idx, d2 = knn.neighbours(x, 6)
    assert [list(r) for r in idx] == brute_neighbours(x.tolist(), 6)
    assert np.all(np.diff(d2, axis=1) >= 0)


def pin_line():
    L, k = 12, 4
    x = np.zeros((L, 3), dtype=np.float32)
    x[:, 0] = np.arange(L)
    idx, d2 = knn.neighbours(x, k)
    for l in range(L):
        order = sorted((abs(l - m), m) for m in range(L) if m != l)
        assert list(idx[l]) == [m for _, m in order[:k]], l
    assert list(idx[5]) == [4, 6, 3, 7] and list(d2[5]) == [1, 1, 4, 4]


def pin_phi_identity(seed=2):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((25, 3)) * 3).astype(np.float32)
    s = rng.standard_normal((25, C_S))
    w_d = np.zeros((C_P, 4))
    w_d[:4, :4] = np.eye(4)
    idx, p = knn.pair_features(x, s, np.zeros((C_P, C_S)), np.zeros((C_P, C_S)), w_d, 5)
    for l in range(25):
        for n in range(5):
            m = idx[l, n]
            d = x[l].astype(np.float64) - x[m].astype(np.float64)
            assert np.allclose(p[l, n, :3], d, rtol=0, atol=0)
            d2 = float(knn.sq_dist_f32(x[l], x[m]))
            assert p[l, n, 3] == 1.0 / (1.0 + d2)
            assert np.all(p[l, n, 4:] == 0)


def pin_linear_parts(seed=3):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((33, 3)) * 4).astype(np.float32)
    s = rng.standard_normal((33, C_S))
    w_l, w_m, _ = rand_weights(rng)
    idx, p = knn.pair_features(x, s, w_l, w_m, np.zeros((C_P, 4)), 6)
    st = torch.from_numpy(s)
    a = torch.nn.functional.linear(st, torch.from_numpy(w_l)).numpy()
    b = torch.nn.functional.linear(st, torch.from_numpy(w_m)).numpy()
    assert np.allclose(p, a[:, None, :] + b[idx], rtol=1e-12, atol=1e-12)


def pin_translation(seed=4):
    rng = np.random.default_rng(seed)
    x = rng.integers(-20, 21, (50, 3)).astype(np.float32)
    s = rng.standard_normal((50, C_S))
    w = rand_weights(rng)
    i0, p0 = knn.pair_features(x, s, *w, 8)
    i1, p1 = knn.pair_features(x + np.float32(1000), s, *w, 8)
    assert np.array_equal(i0, i1) and np.allclose(p0, p1, rtol=0, atol=1e-12)


def pin_permutation(seed=5):
    rng = np.random.default_rng(seed)
    L = 40
    x = (rng.standard_normal((L, 3)) * 6).astype(np.float32)
    s = rng.standard_normal((L, C_S))
    w = rand_weights(rng)
    perm = rng.permutation(L)           # new atom a is old atom perm[a]
    inv = np.argsort(perm)
    i0, p0 = knn.pair_features(x, s, *w, 6)
    i1, p1 = knn.pair_features(x[perm], s[perm], *w, 6)
    assert np.array_equal(perm[i1], i0[perm])
    assert np.allclose(p1, p0[perm], rtol=1e-12, atol=1e-12)
    assert np.array_equal(inv[perm], np.arange(L))


ALL_PINS = [pin_brute_lattice, pin_brute_float, pin_line, pin_phi_identity, pin_linear_parts,
            pin_translation, pin_permutation]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# ----------------------------------------------------------------------------------------
# Planted mistakes.

def _mut_self_included(_orig):
    def f(x, k, rows=None):
        x = np.asarray(x, dtype=np.float32)
        L = x.shape[0]
        rows = np.arange(L) if rows is None else np.asarray(rows)
        idx = np.empty((len(rows), k), dtype=np.int64)
        d2 = np.empty((len(rows), k), dtype=np.float32)
        for n, l in enumerate(rows):
            dl = knn.sq_dist_f32(x[l], x)
            order = np.lexsort((np.arange(L), dl))[:k]
            idx[n], d2[n] = order, dl[order]
        return idx, d2
    return f


def _mut_ties_high(_orig):
    def f(x, k, rows=None):
        x = np.asarray(x, dtype=np.float32)
        L = x.shape[0]
        rows = np.arange(L) if rows is None else np.asarray(rows)
        idx = np.empty((len(rows), k), dtype=np.int64)
        d2 = np.empty((len(rows), k), dtype=np.float32)
        for n, l in enumerate(rows):
            dl = knn.sq_dist_f32(x[l], x)
            order = np.lexsort((-np.arange(L), dl))
            order = order[order != l][:k]
            idx[n], d2[n] = order, dl[order]
        return idx, d2
    return f


def _mut_phi_sign(orig):
    def f(x, rows, idx, d2):
        ph = orig(x, rows, idx, d2)
        ph[..., :3] = -ph[..., :3]
        return ph
    return f


def _mut_phi_distance_not_squared(orig):
    def f(x, rows, idx, d2):
        ph = orig(x, rows, idx, d2)
        ph[..., 3] = 1.0 / (1.0 + np.sqrt(d2.astype(np.float64)))
        return ph
    return f


def _mut_sq_dist_dropped_z(_orig):
    def f(xl, xm):
        d = np.asarray(xl, dtype=np.float32) - np.asarray(xm, dtype=np.float32)
        return d[..., 0] * d[..., 0] + d[..., 1] * d[..., 1]
    return f


def _mut_features_swapped(orig):
    def f(x, s, w_l, w_m, w_d, k, rows=None):
        return orig(x, s, w_m, w_l, w_d, k, rows)
    return f


MUTANTS = [("neighbours", _mut_self_included), ("neighbours", _mut_ties_high), ("phi", _mut_phi_sign),
           ("phi", _mut_phi_distance_not_squared), ("sq_dist_f32", _mut_sq_dist_dropped_z),
           ("pair_features", _mut_features_swapped)]


@pytest.mark.parametrize("name,mut", MUTANTS, ids=[m.__name__ for _, m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, name, mut):
    monkeypatch.setattr(knn, name, mut(getattr(knn, name)))
    caught = []
    for pin in ALL_PINS:
        try:
            pin()
            caught.append(False)
        except (AssertionError, ValueError, IndexError):
            caught.append(True)
    assert any(caught), f"mutant {mut.__name__} of {name} passed every pin"
