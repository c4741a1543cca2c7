"""Token-wise adaptive activation quantization (AAQ) codec -- TEST INFRASTRUCTURE ONLY.

A plain CPU codec for the pair representation, written from the LightNobel
article (section 2.2 "Adaptive activation quantization": 2.2.1 token-wise
granularity, 2.2.2 dynamic outlier handling, 2.2.3 multi-precision groups;
section 2.3.2 memory subsystem, token-interleaved storage).  The HIP library
is checked against it; the library never imports it.

What the article fixes:

* each token -- one Hz-vector of the (Ns, Ns, Hz) pair tensor, Hz = 128 -- is
  quantized on its own, with its own scale and zero point (2.2.1);
* outliers: the k = 5 entries of largest magnitude are candidates, a 3-sigma
  rule confirms them, confirmed ones are stored separately as INT16, the rest
  (the inliers) at INT4 or INT8 (2.2.2);
* group A (residual path): INT8 + outliers; group B (after LayerNorm, before
  a linear layer): INT4 + outliers; group C (everything else): INT4, no
  outlier handling (2.2.3);
* a token's codes, outliers and metadata sit next to each other (2.3.2).

Readings where the article is silent (each one a line of the design notes):

* candidates are ranked by |x|; equal magnitudes go to the lower channel;
* the 3-sigma rule uses the mean mu and the population standard deviation
  sigma of all Hz values of the token (float64, two passes); a candidate is
  confirmed when |x - mu| > 3 sigma, sigma = sqrt(variance), in float64;
* inliers: affine (asymmetric) uniform quantization with an integer zero point
  over the inlier range widened to contain 0, so that 0 is exact and the zero
  point fits the code range -- the scheme of Jacob et al., "Quantization and
  Training of Neural Networks for Efficient Integer-Arithmetic-Only
  Inference" (2018):  s = (rmax - rmin) / (2^b - 1),  z = rint(-rmin / s),
  q = clamp(rint(x / s) + z, 0, 2^b - 1),  x^ = s (q - z);
  a token whose inliers are all zero gets s = 0, z = 0, codes 0;
* outliers: symmetric INT16 with a scale of their own,
  s_o = max|x_o| / 32767, q_o = rint(x_o / s_o), x^ = s_o q_o;
* scales are stored as float32 and every step that turns a value into a code
  is done in float32 in this order: s = (rmax - rmin) / qmax; inv = 1 / s;
  z = rint(-rmin * inv); q = rint(x * inv) + z (each operation rounded to
  nearest even), likewise for the outliers; decoding multiplies in float32.
  The device codec makes the same float32 decisions, so codes agree bit for
  bit except where the float64 3-sigma test is within rounding of its
  threshold (summation order);
* record layouts (little endian), fixed size per token, tokens back to back:
    group A, 160 B: codes u8[128] (channel c at byte c; an outlier's channel
      holds z) | meta (32 B)
    group B,  96 B: codes u4[128] (byte j: channel 2j low nibble, 2j+1 high)
      | meta (32 B)
    group C,  80 B: codes u4[128] | f32 s | u8 z | 11 zero bytes
  meta: f32 s | f32 s_o | i16 q_o[5] | u8 channel[5] | u8 z | u8 n | 7 zero
    bytes; outlier slots in ascending channel order, unused slots zero,
    s_o = 0 when n = 0.

Parity status: pinned by ``tests/test_oracle_aaq.py`` (exact rational 3-sigma
decisions, closed forms of the 3-sigma rule, hand-derived records, tie cases,
error bounds, power-of-two grids and scaling, planted mistakes).  No function here is
"parity unpinned".
"""
from __future__ import annotations

import numpy as np

HZ = 128
TOP_K = 5
SIGMA_RULE = 3.0
OUTLIER_QMAX = 32767

GROUPS = {
    # name: (inlier bits, outlier handling, record bytes, code bytes)
    "A": (8, True, 160, 128),
    "B": (4, True, 96, 64),
    "C": (4, False, 80, 64),
}

f32 = np.float32


def record_bytes(group: str) -> int:
    return GROUPS[group][2]


# ----------------------------------------------------------------------------------------
# Section 2.2.2: dynamic top-k candidates, 3-sigma confirmation.

def topk_candidates(x: np.ndarray, k: int = TOP_K) -> np.ndarray:
    """Channels of the k largest |x| per token, [N, k]; ties go to the lower channel."""
    n, hz = x.shape
    ch = np.broadcast_to(np.arange(hz), (n, hz))
    order = np.lexsort((ch, -np.abs(x)), axis=-1)  # primary key: -|x|, then channel
    return order[:, :k]


def token_stats(x: np.ndarray):
    """Mean and population variance of each token's Hz values, float64, two passes."""
    x64 = x.astype(np.float64)
    mu = x64.sum(axis=-1) / x.shape[-1]
    var = ((x64 - mu[:, None]) ** 2).sum(axis=-1) / x.shape[-1]
    return mu, var


def confirm_outliers(x: np.ndarray, cand: np.ndarray) -> np.ndarray:
    """Boolean [N, Hz] mask: candidates with |x - mu| > 3 sigma."""
    mu, var = token_stats(x)
    xc = np.take_along_axis(x, cand, axis=-1).astype(np.float64)
    d = xc - mu[:, None]
    ok = np.abs(d) > SIGMA_RULE * np.sqrt(var)[:, None]
    mask = np.zeros(x.shape, dtype=bool)
    np.put_along_axis(mask, cand, ok, axis=-1)
    return mask


# ----------------------------------------------------------------------------------------
# Section 2.2.1 / 2.2.3: token-wise asymmetric INT-b inliers, INT16 outliers.

def quantize_inliers(x: np.ndarray, inlier: np.ndarray, bits: int):
    """Per-token scale s, zero point z and codes q of the inliers (float32 decisions)."""
    qmax = (1 << bits) - 1
    x = x.astype(f32)
    big = f32(np.inf)
    rmin = np.minimum(np.where(inlier, x, big).min(axis=-1), f32(0))
    rmax = np.maximum(np.where(inlier, x, -big).max(axis=-1), f32(0))
    s = ((rmax - rmin) / f32(qmax)).astype(f32)
    with np.errstate(divide="ignore"):
        inv = np.where(s > 0, f32(1) / s, f32(0)).astype(f32)
    z = np.clip(np.rint(-rmin * inv), 0, qmax).astype(np.int64)
    q = np.clip(np.rint(x * inv[:, None]).astype(np.int64) + z[:, None], 0, qmax)
    q = np.where(inlier, q, z[:, None])
    return s, z, q


def quantize_outliers(x: np.ndarray, outlier: np.ndarray):
    """Per-token INT16 scale and codes of the confirmed outliers (float32 decisions)."""
    x = x.astype(f32)
    amax = np.where(outlier, np.abs(x), f32(0)).max(axis=-1).astype(f32)
    s_o = (amax / f32(OUTLIER_QMAX)).astype(f32)
    with np.errstate(divide="ignore"):
        inv = np.where(s_o > 0, f32(1) / s_o, f32(0)).astype(f32)
    q = np.clip(np.rint(x * inv[:, None]).astype(np.int64), -OUTLIER_QMAX, OUTLIER_QMAX)
    return s_o, np.where(outlier, q, 0)


def outlier_mask(x: np.ndarray, group: str) -> np.ndarray:
    if not GROUPS[group][1]:
        return np.zeros(x.shape, dtype=bool)
    return confirm_outliers(x, topk_candidates(x))


# ----------------------------------------------------------------------------------------
# Section 2.3.2: token-interleaved records.

def _pack_codes(q: np.ndarray, bits: int) -> np.ndarray:
    if bits == 8:
        return q.astype(np.uint8)
    return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)


def _unpack_codes(b: np.ndarray, bits: int) -> np.ndarray:
    if bits == 8:
        return b.astype(np.int64)
    q = np.empty((b.shape[0], 2 * b.shape[1]), dtype=np.int64)
    q[:, 0::2] = b & 15
    q[:, 1::2] = b >> 4
    return q


def encode(x: np.ndarray, group: str) -> np.ndarray:
    """Encode tokens x [N, Hz] (the stored bf16 / fp32 values) into records [N, bytes] u8."""
    bits, handles_outliers, rb, cb = GROUPS[group]
    x = np.asarray(x, dtype=f32).reshape(-1, HZ)
    n = x.shape[0]
    out_mask = outlier_mask(x, group)
    s, z, q = quantize_inliers(x, ~out_mask, bits)
    rec = np.zeros((n, rb), dtype=np.uint8)
    rec[:, :cb] = _pack_codes(q, bits)
    meta = rec[:, cb:]
    meta[:, 0:4] = s.astype("<f4").view(np.uint8).reshape(n, 4)
    if not handles_outliers:
        meta[:, 4] = z
        return rec
    s_o, q_o = quantize_outliers(x, out_mask)
    meta[:, 4:8] = s_o.astype("<f4").view(np.uint8).reshape(n, 4)
    for t in range(n):
        chans = np.flatnonzero(out_mask[t])  # ascending channel order
        vals = q_o[t, chans].astype("<i2").view(np.uint8)
        meta[t, 8:8 + 2 * len(chans)] = vals
        meta[t, 18:18 + len(chans)] = chans
        meta[t, 24] = len(chans)
    meta[:, 23] = z
    return rec


def decode(rec: np.ndarray, group: str) -> np.ndarray:
    """Decode records [N, bytes] into float32 tokens [N, Hz]: s (q - z), outliers s_o q_o."""
    bits, handles_outliers, rb, cb = GROUPS[group]
    rec = np.asarray(rec, dtype=np.uint8).reshape(-1, rb)
    n = rec.shape[0]
    q = _unpack_codes(rec[:, :cb], bits)
    meta = rec[:, cb:]
    s = np.ascontiguousarray(meta[:, 0:4]).view("<f4").reshape(n).astype(f32)
    z = (meta[:, 23] if handles_outliers else meta[:, 4]).astype(np.int64)
    y = (q - z[:, None]).astype(f32) * s[:, None]
    if handles_outliers:
        s_o = np.ascontiguousarray(meta[:, 4:8]).view("<f4").reshape(n).astype(f32)
        q_o = np.ascontiguousarray(meta[:, 8:18]).view("<i2").reshape(n, TOP_K).astype(f32)
        for t in range(n):
            for slot in range(int(meta[t, 24])):
                y[t, meta[t, 18 + slot]] = q_o[t, slot] * s_o[t]
    return y.astype(f32)


def fields(rec: np.ndarray, group: str) -> dict:
    """The record's fields as arrays (codes [N, Hz], s, z, and for A/B s_o, n, chans, q_o)."""
    bits, handles_outliers, rb, cb = GROUPS[group]
    rec = np.asarray(rec, dtype=np.uint8).reshape(-1, rb)
    n = rec.shape[0]
    meta = rec[:, cb:]
    f = {"q": _unpack_codes(rec[:, :cb], bits),
         "s": np.ascontiguousarray(meta[:, 0:4]).view("<f4").reshape(n).copy()}
    if handles_outliers:
        f["z"] = meta[:, 23].astype(np.int64)
        f["s_o"] = np.ascontiguousarray(meta[:, 4:8]).view("<f4").reshape(n).copy()
        f["q_o"] = np.ascontiguousarray(meta[:, 8:18]).view("<i2").reshape(n, TOP_K).astype(np.int64)
        f["chans"] = meta[:, 18:23].astype(np.int64)
        f["n"] = meta[:, 24].astype(np.int64)
    else:
        f["z"] = meta[:, 4].astype(np.int64)
    return f


def threshold_margin(x: np.ndarray) -> np.ndarray:
    """Per token, the smallest relative distance ||x - mu| - 3 sigma| / (3 sigma) over its
    top-k candidates: how close the float64 3-sigma decisions came to their threshold."""
    x = np.asarray(x, dtype=f32).reshape(-1, HZ)
    cand = topk_candidates(x)
    mu, var = token_stats(x)
    d = np.take_along_axis(x, cand, axis=-1).astype(np.float64) - mu[:, None]
    thr = SIGMA_RULE * np.sqrt(var)[:, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        m = np.abs(np.abs(d) - thr) / thr
    return np.where(thr > 0, m, np.inf).min(axis=-1)
