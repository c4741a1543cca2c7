"""Pins for the AAQ codec oracle (CPU only).

The codec oracle (LightNobel article, section 2.2) is checked against things
other than itself:
* closed forms of the 3-sigma rule: m equal spikes on a flat token are
  outliers exactly when (n - m) / m > 9; a spike placed just above / below the
  threshold separates the population from the sample deviation;
* exact rational arithmetic (fractions.Fraction) for the candidates and the
  3-sigma decisions of random tokens, with Python's own sort for the ranking;
* hand-derived records: an INT8 token with scale 1 and one INT16 outlier whose
  float32 scale is worked out by hand, an INT4 token with scale 1, and ties;
* tokens that lie on a power-of-two grid encode to their grid codes and
  decode exactly; scaling by 2^k scales s and keeps the codes;
* error bounds: inliers within s/2, outliers within s_o/2;
* planted mistakes: each mutant of the oracle must fail at least one pin.
"""
import struct
from fractions import Fraction

import numpy as np
import pytest

from oracle import aaq

N = aaq.HZ


def spikes_token(m, a=40.0, b=1.0, chans=None):
    x = np.full(N, b, dtype=np.float32)
    chans = list(range(0, 10 * m, 10)) if chans is None else chans
    x[chans] = a
    return x, sorted(chans)


def outlier_set(rec, group):
    f = aaq.fields(rec, group)
    return [sorted(int(c) for c in f["chans"][t, :f["n"][t]]) for t in range(rec.shape[0])]


def threshold_spike(rest, ratio):
    """Value a such that, with the 127 values `rest` and a at channel 0, the
    token has (a - mu)^2 / var = ratio (population variance), rounded to fp32."""
    r = rest.astype(np.float64)
    n = N
    s1, s2 = r.sum(), (r * r).sum()
    # (a - mu)^2 * n^2 = ((n-1) a - s1)^2 ;  var * n^2 = n (s2 + a^2) - (s1 + a)^2
    # solve ((n-1)a - s1)^2 = ratio * (n (s2 + a^2) - (s1 + a)^2) for the larger root
    A = (n - 1) ** 2 - ratio * (n - 1)
    B = -2 * (n - 1) * s1 + 2 * ratio * s1
    C = s1 * s1 - ratio * (n * s2 - s1 * s1)
    a = (-B + np.sqrt(B * B - 4 * A * C)) / (2 * A)
    return np.float32(a)


def exact_ratio(x, c):
    fr = [Fraction(float(v)) for v in x]
    mu = sum(fr) / len(fr)
    var = sum((v - mu) ** 2 for v in fr) / len(fr)
    return (fr[c] - mu) ** 2 / var


# ----------------------------------------------------------------------------------------
# Pins as functions of the oracle module, so planted mistakes can be re-checked.

def pin_spikes():
    """m spikes of 40 on a flat token of 1: (a - mu)^2 / var = (n - m) / m."""
    for m in range(1, 14):
        x, chans = spikes_token(m)
        got = outlier_set(aaq.encode(x[None], "A"), "A")[0]
        want = chans[:5] if (N - m) / m > 9 else []
        assert got == want, (m, got, want)


def pin_ties():
    """Six spikes of equal magnitude (signs mixed): the five lowest channels win."""
    chans = [100, 7, 64, 3, 90, 50]
    x = np.full(N, 0.5, dtype=np.float32)
    x[chans] = [30.0, 30.0, -30.0, 30.0, -30.0, 30.0]
    got = outlier_set(aaq.encode(x[None], "B"), "B")[0]
    assert got == [3, 7, 50, 64, 90], got


def pin_population_sigma(seed=7):
    """A spike with exact ratio just above 9 is an outlier, just below it is not;
    a ratio of 9.03 is below 9 for the sample variance (x 127/128)."""
    rng = np.random.default_rng(seed)
    rest = rng.standard_normal(N - 1).astype(np.float32)
    for ratio, want in ((9.03, [0]), (8.97, [])):
        a = threshold_spike(rest, ratio)
        x = np.concatenate([[a], rest]).astype(np.float32)
        r = exact_ratio(x, 0)
        assert (r > 9) == bool(want) and abs(float(r) - ratio) < 1e-3
        got = outlier_set(aaq.encode(x[None], "A"), "A")[0]
        assert got == want, (ratio, got)


def pin_exact_rational(seed=11, tokens=48):
    """Random bf16-valued tokens with planted spikes: outlier sets equal the
    exact-arithmetic decisions over Python's own ranking."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((tokens, N)).astype(np.float32)
    spike = rng.random((tokens, N)) < 0.03
    x = np.where(spike, x * rng.uniform(3, 25, (tokens, N)), x).astype(np.float32)
    x[0, :6] = 9.0  # a tie at the fifth place
    x = (x.view(np.uint32) & 0xFFFF0000).view(np.float32)  # bf16 values
    got = outlier_set(aaq.encode(x, "A"), "A")
    for t in range(tokens):
        fr = [Fraction(float(v)) for v in x[t]]
        mu = sum(fr) / N
        var = sum((v - mu) ** 2 for v in fr) / N
        cand = sorted(range(N), key=lambda c: (abs(fr[c]), -c), reverse=True)[:5]
        want = sorted(c for c in cand if (fr[c] - mu) ** 2 > 9 * var)
        assert got[t] == want, (t, got[t], want)


def pin_int8_record():
    """x_c = 2c - 128, x_127 = 127, x_5 = 4096.  Inliers span [-128, 127]:
    s = 255 / 255 = 1, z = 128, q_c = x_c + 128.  The one outlier is 4096:
    s_o = fl32(4096 / 32767) = 2^-3 + 2^-18 (4096/32767 = 2^-3 + 256.0078 ulps of
    2^-26), bits 0x3E000100; 1 / s_o = fl32(8 (1 - 2^-15 + 2^-30)) = 8 - 2^-12;
    q_o = rint(4096 (8 - 2^-12)) = 32767; decoding gives fl32(32767 s_o) = 4096
    (the exact product is 4096 - 3.8e-6, under half an ulp of 2^-12)."""
    x = np.array([2 * c - 128 for c in range(N)], dtype=np.float32)
    x[127], x[5] = 127, 4096
    rec = aaq.encode(x[None], "A")[0]
    codes = bytes((2 * c) for c in range(N))
    codes = codes[:5] + bytes([128]) + codes[6:127] + bytes([255])
    meta = (struct.pack("<I", 0x3F800000) + struct.pack("<I", 0x3E000100)
            + struct.pack("<5h", 32767, 0, 0, 0, 0) + bytes([5, 0, 0, 0, 0]) + bytes([128, 1])
            + bytes(7))
    assert rec.tobytes() == codes + meta
    y = aaq.decode(rec[None], "A")[0]
    assert np.array_equal(y, x)


def pin_int4_record():
    """x_c = (c mod 16) - 8: s = 15 / 15 = 1, z = 8, q_c = c mod 16; byte j holds
    q_2j in its low nibble and q_2j+1 in its high nibble.  Group C gives the same
    codes with s and z right after them; group B finds no outlier (no value is
    3 sigma away: sigma^2 = 21.25)."""
    x = np.array([(c % 16) - 8 for c in range(N)], dtype=np.float32)
    codes = bytes((((2 * j) % 16) | (((2 * j + 1) % 16) << 4)) for j in range(64))
    rec_b = aaq.encode(x[None], "B")[0]
    meta_b = struct.pack("<I", 0x3F800000) + bytes(4) + bytes(10) + bytes(5) + bytes([8, 0]) + bytes(7)
    assert rec_b.tobytes() == codes + meta_b
    rec_c = aaq.encode(x[None], "C")[0]
    assert rec_c.tobytes() == codes + struct.pack("<I", 0x3F800000) + bytes([8]) + bytes(11)
    for g, r in (("B", rec_b), ("C", rec_c)):
        assert np.array_equal(aaq.decode(r[None], g)[0], x)


def pin_grid(seed=5):
    """Tokens on the grid s (q - z) with s = 2^-e and codes 0 and qmax present
    encode to exactly (s, z, q) and decode exactly.  Codes drawn uniformly stay
    within 3 sigma (a uniform spread reaches about 1.7 sigma), so A and B find no
    outlier."""
    rng = np.random.default_rng(seed)
    for group, bits in (("A", 8), ("B", 4), ("C", 4)):
        qmax = (1 << bits) - 1
        for t in range(20):
            e = int(rng.integers(-6, 7))
            s = np.float32(2.0 ** e)
            z = int(rng.integers(1, qmax))
            q = rng.integers(0, qmax + 1, N)
            q[rng.permutation(N)[:2]] = [0, qmax]
            x = (s * (q - z)).astype(np.float32)
            rec = aaq.encode(x[None], group)
            f = aaq.fields(rec, group)
            lo, hi = min(0, int(q.min()) - z), max(0, int(q.max()) - z)
            s_want = np.float32(s * (hi - lo) / qmax)
            assert f["s"][0] == s_want, (group, t, f["s"][0], s_want)
            assert s_want == s and f["z"][0] == z and np.array_equal(f["q"][0], q), (group, t)
            assert np.array_equal(aaq.decode(rec, group)[0], x), (group, t)
            if group != "C":
                assert f["n"][0] == 0


def pin_scaling(seed=9):
    """x -> 2^k x: codes, zero points and outlier channels unchanged, scales x 2^k."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((16, N)).astype(np.float32)
    x[rng.random((16, N)) < 0.02] *= 30
    for group in ("A", "B", "C"):
        f0 = aaq.fields(aaq.encode(x, group), group)
        for k in (-3, 5):
            fk = aaq.fields(aaq.encode(x * np.float32(2.0 ** k), group), group)
            assert np.array_equal(f0["q"], fk["q"]) and np.array_equal(f0["z"], fk["z"])
            assert np.array_equal(fk["s"], f0["s"] * np.float32(2.0 ** k))
            if group != "C":
                assert np.array_equal(f0["chans"], fk["chans"]) and np.array_equal(f0["q_o"], fk["q_o"])


def pin_error_bounds(seed=13):
    """Inliers decode within s/2, outliers within s_o/2 (plus float32 rounding);
    codes stay in range; at most five outliers."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((64, N)) * rng.uniform(0.01, 10, (64, 1))).astype(np.float32)
    x[rng.random((64, N)) < 0.02] *= rng.uniform(-40, 40)
    x[3] = 0.0
    x[4] = np.float32(2.5)
    for group, bits in (("A", 8), ("B", 4), ("C", 4)):
        rec = aaq.encode(x, group)
        f = aaq.fields(rec, group)
        y = aaq.decode(rec, group)
        assert f["q"].min() >= 0 and f["q"].max() <= (1 << bits) - 1
        out = np.zeros(x.shape, dtype=bool)
        if group != "C":
            assert f["n"].max() <= 5
            for t in range(x.shape[0]):
                out[t, f["chans"][t, :f["n"][t]]] = True
            err_o = np.abs(y - x)[out]
            bound_o = np.broadcast_to(f["s_o"][:, None], x.shape)[out] * 0.5000001 + np.abs(x[out]) * 2e-7
            assert (err_o <= bound_o).all()
        err = np.abs(y - x)[~out]
        bound = np.broadcast_to(f["s"][:, None], x.shape)[~out] * 0.5000001 + np.abs(x[~out]) * 2e-7
        assert (err <= bound).all(), (group, (err - bound).max())
        assert np.array_equal(y[3], x[3])


ALL_PINS = [pin_spikes, pin_ties, pin_population_sigma, pin_exact_rational, pin_int8_record,
            pin_int4_record, pin_grid, pin_scaling, pin_error_bounds]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_record_sizes():
    assert [aaq.record_bytes(g) for g in "ABC"] == [160, 96, 80]


def test_margin_reports_threshold_distance():
    rng = np.random.default_rng(3)
    rest = rng.standard_normal(N - 1).astype(np.float32)
    a = threshold_spike(rest, 9.0 * (1 + 1e-4))
    x = np.concatenate([[a], rest]).astype(np.float32)[None]
    m = aaq.threshold_margin(x)[0]
    assert 1e-5 < m < 1e-3


# ----------------------------------------------------------------------------------------
# Planted mistakes.

def _mut_k4(_orig):
    return lambda x, k=4: _orig(x, 4)


def _mut_ties_high(_orig):
    def f(x, k=aaq.TOP_K):
        n, hz = x.shape
        ch = np.broadcast_to(np.arange(hz)[::-1], (n, hz))
        return np.lexsort((ch, -np.abs(x)), axis=-1)[:, :k]
    return f


def _mut_sample_var(_orig):
    def f(x):
        mu, var = _orig(x)
        return mu, var * x.shape[-1] / (x.shape[-1] - 1)
    return f


def _mut_two_sigma(_orig):
    def f(x, cand):
        mu, var = aaq.token_stats(x)
        xc = np.take_along_axis(x, cand, axis=-1).astype(np.float64)
        ok = np.abs(xc - mu[:, None]) > 2.0 * np.sqrt(var)[:, None]
        mask = np.zeros(x.shape, dtype=bool)
        np.put_along_axis(mask, cand, ok, axis=-1)
        return mask
    return f


def _mut_zero_point_sign(_orig):
    def f(x, inlier, bits):
        s, z, q = _orig(x, inlier, bits)
        qmax = (1 << bits) - 1
        inv = np.where(s > 0, np.float32(1) / np.where(s > 0, s, 1), 0).astype(np.float32)
        z2 = np.clip(qmax - z, 0, qmax)
        q2 = np.clip(np.rint(x.astype(np.float32) * inv[:, None]).astype(np.int64) + z2[:, None], 0, qmax)
        return s, z2, np.where(inlier, q2, z2[:, None])
    return f


def _mut_floor(_orig):
    def f(x, inlier, bits):
        s, z, q = _orig(x, inlier, bits)
        qmax = (1 << bits) - 1
        inv = np.where(s > 0, np.float32(1) / np.where(s > 0, s, 1), 0).astype(np.float32)
        q2 = np.clip(np.floor(x.astype(np.float32) * inv[:, None]).astype(np.int64) + z[:, None], 0, qmax)
        return s, z, np.where(inlier, q2, z[:, None])
    return f


def _mut_no_zero_in_range(_orig):
    def f(x, inlier, bits):
        qmax = (1 << bits) - 1
        x = x.astype(np.float32)
        rmin = np.where(inlier, x, np.inf).min(axis=-1).astype(np.float32)
        rmax = np.where(inlier, x, -np.inf).max(axis=-1).astype(np.float32)
        s = ((rmax - rmin) / np.float32(qmax)).astype(np.float32)
        inv = np.where(s > 0, np.float32(1) / np.where(s > 0, s, 1), 0).astype(np.float32)
        z = np.clip(np.rint(-rmin * inv), 0, qmax).astype(np.int64)
        q = np.clip(np.rint(x * inv[:, None]).astype(np.int64) + z[:, None], 0, qmax)
        return s, z, np.where(inlier, q, z[:, None])
    return f


def _mut_outlier_scale_32768(_orig):
    def f(x, outlier):
        s_o, q = _orig(x, outlier)
        s2 = (s_o * np.float32(32767) / np.float32(32768)).astype(np.float32)
        inv = np.where(s2 > 0, np.float32(1) / np.where(s2 > 0, s2, 1), 0).astype(np.float32)
        q2 = np.clip(np.rint(x.astype(np.float32) * inv[:, None]).astype(np.int64), -32767, 32767)
        return s2, np.where(outlier, q2, 0)
    return f


def _mut_nibbles_swapped(_orig):
    def f(q, bits):
        if bits == 8:
            return _orig(q, bits)
        return (q[:, 1::2] | (q[:, 0::2] << 4)).astype(np.uint8)
    return f


def _mut_decode_drops_outliers(_orig):
    def f(rec, group):
        bits, _, rb, cb = aaq.GROUPS[group]
        rec = np.asarray(rec, dtype=np.uint8).reshape(-1, rb)
        fl = aaq.fields(rec, group)
        return ((fl["q"] - fl["z"][:, None]).astype(np.float32) * fl["s"][:, None]).astype(np.float32)
    return f


MUTANTS = [
    ("topk_candidates", _mut_k4), ("topk_candidates", _mut_ties_high), ("token_stats", _mut_sample_var),
    ("confirm_outliers", _mut_two_sigma), ("quantize_inliers", _mut_zero_point_sign),
    ("quantize_inliers", _mut_floor), ("quantize_inliers", _mut_no_zero_in_range),
    ("quantize_outliers", _mut_outlier_scale_32768), ("_pack_codes", _mut_nibbles_swapped),
    ("decode", _mut_decode_drops_outliers),
]


@pytest.mark.parametrize("name,mut", MUTANTS, ids=[m.__name__ for _, m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, name, mut):
    monkeypatch.setattr(aaq, name, mut(getattr(aaq, name)))
    caught = []
    for pin in ALL_PINS:
        try:
            pin()
            caught.append(False)
        except (AssertionError, ValueError, IndexError):
            caught.append(True)
    assert any(caught), f"mutant {mut.__name__} of {name} passed every pin"
