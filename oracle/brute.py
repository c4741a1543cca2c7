"""Pure-Python scalar-loop triangle attention for tiny inputs -- TEST INFRASTRUCTURE ONLY.

Written independently of ``oracle.ref`` (no shared helpers) from the same
definition: per-token LayerNorm with the biased variance, nn.Linear-style
projections, a per-head additive pair bias, softmax over keys, a sigmoid gate
and an output projection (gated triangular attention, the operator the
LightNobel article names in section 3.1; equations as read in ``oracle.ref``).
Every value is a Python float and every sum an explicit loop.
"""
from __future__ import annotations

import math


def _tolist(a):
    return a.tolist() if hasattr(a, "tolist") else a


def _token_features(zt, p):
    """LayerNorm + projections of one token (list of c_z floats)."""
    c = len(zt)
    mean = 0.0
    for x in zt:
        mean += x
    mean /= c
    var = 0.0
    for x in zt:
        var += (x - mean) * (x - mean)
    var /= c
    inv = 1.0 / math.sqrt(var + p["eps"])
    xn = [(zt[t] - mean) * inv * p["ln_gamma"][t] + p["ln_beta"][t] for t in range(c)]

    def lin(w, b=None):
        res = []
        for o in range(len(w)):
            acc = 0.0
            for t in range(c):
                acc += xn[t] * w[o][t]
            if b is not None:
                acc += b[o]
            res.append(acc)
        return res

    q = lin(p["w_q"])
    k = lin(p["w_k"])
    v = lin(p["w_v"])
    g = [1.0 / (1.0 + math.exp(-x)) for x in lin(p["w_g"], p["b_g"])]
    b = lin(p["w_b"])
    return q, k, v, g, b


def _prep(z, p):
    z = _tolist(z)
    pl = {k: _tolist(v) for k, v in p.items()}
    R, I = len(z), len(z[0])
    feats = [[_token_features(z[r][c], pl) for c in range(I)] for r in range(R)]
    return z, pl, feats


def _out_token(o_heads, g, pl):
    """o_heads: flat list over (h, e); returns the c_z-vector (g*o) W_o^T + b_o."""
    og = [o_heads[t] * g[t] for t in range(len(g))]
    res = []
    for c in range(len(pl["w_o"])):
        acc = pl["b_o"][c]
        for t in range(len(og)):
            acc += og[t] * pl["w_o"][c][t]
        res.append(acc)
    return res


def _attend_one(qv, keys, vals, biases, H, d):
    """o for one query: qv flat (h,e); keys/vals: lists over key of flat (h,e); biases[h][key]."""
    o = [0.0] * (H * d)
    scale = 1.0 / math.sqrt(d)
    for h in range(H):
        s = []
        for kk in range(len(keys)):
            dot = 0.0
            for e in range(d):
                dot += qv[h * d + e] * keys[kk][h * d + e]
            s.append(dot * scale + biases[h][kk])
        m = max(s)
        ex = [math.exp(x - m) for x in s]
        tot = 0.0
        for x in ex:
            tot += x
        for kk in range(len(keys)):
            a = ex[kk] / tot
            for e in range(d):
                o[h * d + e] += a * vals[kk][h * d + e]
    return o


def start(z, p):
    """Starting node: out[i][j] over keys k of row i, bias b_jk."""
    z, pl, f = _prep(z, p)
    I, H, d = len(z), pl["heads"], pl["head_dim"]
    out = []
    for i in range(I):
        row = []
        for j in range(I):
            keys = [f[i][k][1] for k in range(I)]
            vals = [f[i][k][2] for k in range(I)]
            biases = [[f[j][k][4][h] for k in range(I)] for h in range(H)]
            o = _attend_one(f[i][j][0], keys, vals, biases, H, d)
            row.append(_out_token(o, f[i][j][3], pl))
        out.append(row)
    return out


def end(z, p):
    """Ending node: out[i][j] over keys k of column j, bias b_ki."""
    z, pl, f = _prep(z, p)
    I, H, d = len(z), pl["heads"], pl["head_dim"]
    out = []
    for i in range(I):
        row = []
        for j in range(I):
            keys = [f[k][j][1] for k in range(I)]
            vals = [f[k][j][2] for k in range(I)]
            biases = [[f[k][i][4][h] for k in range(I)] for h in range(H)]
            o = _attend_one(f[i][j][0], keys, vals, biases, H, d)
            row.append(_out_token(o, f[i][j][3], pl))
        out.append(row)
    return out


def rows(z_rows, bias, p):
    """Row block with a given bias[h][j][k]."""
    z, pl, f = _prep(z_rows, p)
    bias = _tolist(bias)
    R, I, H, d = len(z), len(z[0]), pl["heads"], pl["head_dim"]
    out = []
    for r in range(R):
        row = []
        for j in range(I):
            keys = [f[r][k][1] for k in range(I)]
            vals = [f[r][k][2] for k in range(I)]
            biases = [[bias[h][j][k] for k in range(I)] for h in range(H)]
            o = _attend_one(f[r][j][0], keys, vals, biases, H, d)
            row.append(_out_token(o, f[r][j][3], pl))
        out.append(row)
    return out


def pair_bias(z, p):
    """bias[h][r][k] of every token of z."""
    z, pl, f = _prep(z, p)
    H = pl["heads"]
    return [[[f[r][k][4][h] for k in range(len(z[0]))] for r in range(len(z))] for h in range(H)]
