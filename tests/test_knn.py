"""GPU parity of the kNN sparse atom-pair encoder (knn_pair_encode) against the
float64 oracle (oracle.knn).

* Neighbour lists are integer results: they must equal the oracle's bit for
  bit (both sides rank by the same float32 squared distance, ties to the lower
  index).
* Pair features are accumulated in float32 and stored bf16.  Per element the
  bar is |got - want| <= 2^-8 (|want| + delta) + delta, where 2^-8 |v| bounds the
  nearest-even rounding to bf16 (half an ulp of an 8-bit significand) and
  delta = 140 * 2^-24 * S bounds the float32 accumulation (at most 138 rounded
  operations on terms whose magnitudes sum to S = |s_l| . |w_l| + |s_m| . |w_m|
  + |phi| . |w_d|); the relative L1 error must also stay within 5e-3.
* At the full size (16384 atoms, k = 32) sampled rows are checked against the
  oracle, and every row against properties that fix the k nearest at any size.
"""
import numpy as np
import pytest
import torch

from oracle import knn as oknn
from protein_pair_representation_amd import inputs
from protein_pair_representation_amd import knn as kn

from test_parity import say

pytestmark = pytest.mark.gpu


def run(a: dict, k: int):
    d = {n: t.cuda() for n, t in a.items()}
    nbr, pair = kn.knn_pair_encode(d["x"], d["s"], k, d["w_l"], d["w_m"], d["w_d"])
    torch.cuda.synchronize()
    return nbr.cpu().numpy(), pair.cpu().float().numpy()


def oracle(a: dict, k: int, rows=None):
    return oknn.pair_features(a["x"].numpy(), inputs.to_f64(a["s"]), inputs.to_f64(a["w_l"]),
                              inputs.to_f64(a["w_m"]), inputs.to_f64(a["w_d"]), k, rows)


def magnitude(a: dict, idx: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """S[r][n][o]: the sum of the magnitudes of the terms of pair (rows[r], idx[r][n])."""
    s = np.abs(inputs.to_f64(a["s"]))
    sa = s[rows] @ np.abs(inputs.to_f64(a["w_l"])).T
    sb = s @ np.abs(inputs.to_f64(a["w_m"])).T
    x = a["x"].numpy()
    d2 = oknn.sq_dist_f32(x[rows][:, None, :], x[idx])
    ph = np.abs(oknn.phi(x, rows, idx, d2)) @ np.abs(inputs.to_f64(a["w_d"])).T
    return sa[:, None, :] + sb[idx] + ph


def check_pairs(a, got, want, idx, rows, what):
    delta = 140 * 2.0 ** -24 * magnitude(a, idx, rows)
    bound = 2.0 ** -8 * (np.abs(want) + delta) + delta
    err = np.abs(got - want)
    rel_l1 = err.sum() / max(np.abs(want).sum(), 1e-300)
    worst = float((err / bound).max()) if err.size else 0.0
    say(f"  {what}: pair max abs {err.max() if err.size else 0:.3e}, rel L1 {rel_l1:.3e}, "
        f"worst err/bound {worst:.3f}")
    assert np.all(err <= bound), f"{what}: {int((err > bound).sum())} elements beyond the bound"
    assert rel_l1 <= 5e-3


def synthetic(seed, L, scatter=None):
    a = inputs.make_atoms(seed, L)
    if scatter is not None:
        a["x"] = torch.from_numpy(scatter(np.random.default_rng(seed + 1), a["x"].numpy()).astype(np.float32))
    return a


@pytest.mark.parametrize("L,k", [(2, 1), (33, 32), (65, 64), (64, 63), (130, 7), (200, 32), (1000, 32),
                                 (1000, 16), (777, 64), (2049, 32)])
def test_chain(L, k):
    say(f"[knn] chain L={L} k={k}")
    a = synthetic(100 + L + k, L)
    nbr, pair = run(a, k)
    idx, want = oracle(a, k)
    assert np.array_equal(nbr, idx), f"neighbours differ in {int((nbr != idx).any(1).sum())} rows"
    check_pairs(a, pair, want, idx, np.arange(L), f"L={L} k={k}")


def test_lattice_ties():
    """Integer coordinates on a small grid: most distances tie exactly, so the
    order is decided by the index rule alone."""
    L, k = 700, 32
    say(f"[knn] lattice ties L={L} k={k}")
    a = synthetic(7, L, lambda r, x: r.integers(-4, 5, (L, 3)))
    nbr, pair = run(a, k)
    idx, want = oracle(a, k)
    assert np.array_equal(nbr, idx)
    check_pairs(a, pair, want, idx, np.arange(L), "lattice")


def test_duplicate_atoms():
    """Groups of atoms at the same position: zero distances, phi_4 = 1."""
    L, k = 300, 24
    say(f"[knn] duplicates L={L} k={k}")
    a = synthetic(8, L, lambda r, x: np.repeat(x[::5], 5, axis=0)[:L])
    nbr, pair = run(a, k)
    idx, want = oracle(a, k)
    assert np.array_equal(nbr, idx)
    check_pairs(a, pair, want, idx, np.arange(L), "duplicates")


def test_shuffled_order():
    """Atoms in random order: the chunk boxes are loose and nearly every chunk
    is scanned; the result is the same as for any order."""
    L, k = 3000, 32
    say(f"[knn] shuffled L={L} k={k}")
    a = synthetic(9, L, lambda r, x: x[r.permutation(L)])
    nbr, pair = run(a, k)
    idx, want = oracle(a, k)
    assert np.array_equal(nbr, idx)
    check_pairs(a, pair, want, idx, np.arange(L), "shuffled")


def test_far_clusters():
    """Two chains 10^4 A apart plus a lone far atom: boxes far beyond the k-th
    distance are skipped, the lone atom's neighbours all lie in another chunk."""
    L, k = 1500, 32

    def place(r, x):
        x = x.copy()
        x[700:] += 1.0e4
        x[L - 1] = (-5.0e4, 0.0, 0.0)
        return x

    say(f"[knn] far clusters L={L} k={k}")
    a = synthetic(10, L, place)
    nbr, pair = run(a, k)
    idx, want = oracle(a, k)
    assert np.array_equal(nbr, idx)
    check_pairs(a, pair, want, idx, np.arange(L), "far clusters")


def test_empty():
    a = synthetic(11, 8)
    d = {n: t.cuda() for n, t in a.items()}
    nbr, pair = kn.knn_pair_encode(d["x"][:0], d["s"][:0], 4, d["w_l"], d["w_m"], d["w_d"])
    torch.cuda.synchronize()
    assert nbr.shape == (0, 4) and pair.shape == (0, 4, 16)


def ranks_are_exact(x: np.ndarray, nbr: np.ndarray, k: int, block: int = 512):
    """Every row: no self, sorted by (d2, index), and exactly k - 1 atoms rank
    ahead of the last entry -- which fixes the k nearest uniquely."""
    L = x.shape[0]
    ids = np.arange(L)
    for r0 in range(0, L, block):
        rows = ids[r0:r0 + block]
        d2 = oknn.sq_dist_f32(x[rows][:, None, :], x[None, :, :])        # float32, same order
        d2[np.arange(len(rows)), rows] = np.inf                          # self never ranks
        nb = nbr[rows]
        assert np.all(nb >= 0) and np.all(nb < L) and np.all(nb != rows[:, None])
        dn = np.take_along_axis(d2, nb, axis=1)
        step_ok = (dn[:, 1:] > dn[:, :-1]) | ((dn[:, 1:] == dn[:, :-1]) & (nb[:, 1:] > nb[:, :-1]))
        assert np.all(step_ok), f"rows from {r0}: list not in (d2, index) order"
        last_d, last_i = dn[:, -1:], nb[:, -1:]
        ahead = (d2 < last_d) | ((d2 == last_d) & (ids[None, :] < last_i))
        assert np.all(ahead.sum(1) == k - 1), f"rows from {r0}: not the k nearest"


def test_workload_16384():
    """The full-size workload: sampled rows against the oracle, every row
    against the ranking properties."""
    wl = inputs.KNN_WORKLOADS["knn-L16384-k32"]
    L, k = wl["L"], wl["k"]
    say(f"[knn] knn-L16384-k32 (L={L} k={k})")
    a = inputs.make_atoms(wl["seed"], L)
    nbr, pair = run(a, k)
    rng = np.random.default_rng(0)
    rows = np.unique(np.r_[0:64, L - 64:L, rng.integers(0, L, 128)])
    idx, want = oracle(a, k, rows)
    assert np.array_equal(nbr[rows], idx)
    check_pairs(a, pair[rows], want, idx, rows, "sampled rows")
    ranks_are_exact(a["x"].numpy(), nbr.astype(np.int64), k)


@pytest.mark.parametrize("L,k", [(100003, 64), (1 << 20, 32)])
def test_large_sampled(L, k):
    """Large and ragged atom counts (past the 16384-atom workload): sampled rows
    against the oracle, every sampled list bit-exact."""
    say(f"[knn] large L={L} k={k}")
    a = inputs.make_atoms(40 + k, L)
    nbr, pair = run(a, k)
    rng = np.random.default_rng(1)
    rows = np.unique(np.r_[0:8, L - 8:L, rng.integers(0, L, 48)])
    idx, want = oracle(a, k, rows)
    assert np.array_equal(nbr[rows], idx)
    check_pairs(a, pair[rows], want, idx, rows, f"L={L} sampled rows")


def test_max_atoms():
    """The largest supported count, 2^24 atoms (k = 32): neighbour lists of
    sampled rows bit for bit against the oracle's ranking, and their pair
    features from the oracle's phi and the stored single features."""
    L, k = 1 << 24, 32
    say(f"[knn] max atoms L={L} k={k}")
    a = inputs.make_atoms(77, L)
    d = {n: t.cuda() for n, t in a.items()}
    nbr, pair = kn.knn_pair_encode(d["x"], d["s"], k, d["w_l"], d["w_m"], d["w_d"])
    torch.cuda.synchronize()
    rows = np.array([0, 1, L // 2, L - 2, L - 1, 12345678, 9876543, 4242424])
    rt = torch.as_tensor(rows, device="cuda")
    got_nbr = nbr[rt].cpu().numpy()
    got_pair = pair[rt].cpu().float().numpy()
    del d, nbr, pair
    torch.cuda.empty_cache()
    x = a["x"].numpy()
    idx, d2 = oknn.neighbours(x, k, rows)
    assert np.array_equal(got_nbr, idx)
    s = inputs.to_f64(a["s"][torch.as_tensor(np.concatenate([rows, idx.ravel()]))])
    sr, sm = s[:len(rows)], s[len(rows):].reshape(len(rows), k, -1)
    want = (sr @ inputs.to_f64(a["w_l"]).T)[:, None, :] + sm @ inputs.to_f64(a["w_m"]).T \
        + oknn.phi(x, rows, idx, d2) @ inputs.to_f64(a["w_d"]).T
    err = np.abs(got_pair - want)
    say(f"  L={L}: pair max abs {err.max():.3e}, rel L1 {err.sum() / np.abs(want).sum():.3e}")
    assert err.sum() / np.abs(want).sum() <= 5e-3 and np.all(err <= 2.0 ** -8 * np.abs(want) + 1e-3)
