"""float64 NumPy oracle for gated triangle self-attention -- TEST INFRASTRUCTURE ONLY.

What the pages fix, and what is read into them:

* The operand is the pair representation Z, an I x I array of c_z-vectors
  ("tokens"), with c_z usually 128 (LightNobel article, section 1.1, the
  (Ns, Ns, Hz) pair representation).  Linear layers and layer normalisation act
  on each token on its own (LightNobel article, section 2.2.1).
* The operator is triangular attention (LightNobel article, section 3.1, which
  names it among the protein-specific operators).  The pages never write its
  equations; this oracle takes the standard gated form used by AlphaFold-family
  trunks as the plainest reading:

    x_ij   = LayerNorm(z_ij)                      (biased variance, eps 1e-5)
    q,k,v  = x W_q^T, x W_k^T, x W_v^T            (H heads of width d)
    b_jk^h = x_jk . W_b[h]                        (pair bias, one scalar per head)
    g_ij   = sigmoid(x_ij W_g^T + b_g)
    start: o_ij^h = sum_k softmax_k(q_ij^h . k_ik^h / sqrt(d) + b_jk^h) v_ik^h
    end:   o_ij^h = sum_k softmax_k(q_ij^h . k_kj^h / sqrt(d) + b_ki^h) v_kj^h
    out_ij = (g_ij * o_ij) W_o^T + b_o

* Attention is pairwise over the O(I^2) pair tensor (Design-CP summary, problem
  statement); the row-block form -- a block of query rows attends with its
  own keys/values and a bias that is held whole -- follows the 1D row sharding
  of the Design-CP summary, Methodology section 1.

Weights use the torch.nn.Linear convention W[out][in].  The pair bias is a
head-major array bias[h][j][k] = b_jk^h.  Everything is float64; inputs are
upcast from their stored (bf16 / fp32) values before use.
"""
from __future__ import annotations

import numpy as np

SOFTMAX_SUM_TOL = 1e-12


def layer_norm(z, gamma, beta, eps):
    """Per-token LayerNorm over the last axis with the biased variance."""
    mu = z.mean(axis=-1, keepdims=True)
    var = ((z - mu) ** 2).mean(axis=-1, keepdims=True)
    return (z - mu) / np.sqrt(var + eps) * gamma + beta


def linear(x, w, b=None):
    """y = x W^T (+ b), W stored [out][in] as in torch.nn.Linear."""
    y = x @ w.T
    return y if b is None else y + b


def sigmoid(x):
    with np.errstate(over="ignore"):  # exp(-x) = inf for x << 0 gives exactly 0
        return 1.0 / (1.0 + np.exp(-x))


def softmax(s):
    """Softmax over the last axis, full matrix materialised; rows checked to sum to 1."""
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    a = e / e.sum(axis=-1, keepdims=True)
    assert np.all(a >= 0.0)
    assert np.all(np.abs(a.sum(axis=-1) - 1.0) <= SOFTMAX_SUM_TOL)
    return a


def project(z, p):
    """LayerNorm then the q/k/v/gate/bias projections of tokens z[..., c_z].

    Returns q, k, v, g shaped [..., H, d] and the pair bias shaped [..., H].
    """
    H, d = p["heads"], p["head_dim"]
    x = layer_norm(z, p["ln_gamma"], p["ln_beta"], p["eps"])
    lead = z.shape[:-1]
    q = linear(x, p["w_q"]).reshape(*lead, H, d)
    k = linear(x, p["w_k"]).reshape(*lead, H, d)
    v = linear(x, p["w_v"]).reshape(*lead, H, d)
    g = sigmoid(linear(x, p["w_g"], p["b_g"])).reshape(*lead, H, d)
    b = linear(x, p["w_b"])
    return q, k, v, g, b


def pair_bias(z, p, chunk_rows=64):
    """bias[h][r][k] = b^h of token z[r][k]; rows are processed in chunks to bound memory."""
    R, I = z.shape[0], z.shape[1]
    out = np.empty((p["heads"], R, I))
    for r0 in range(0, R, chunk_rows):
        x = layer_norm(z[r0:r0 + chunk_rows], p["ln_gamma"], p["ln_beta"], p["eps"])
        out[:, r0:r0 + chunk_rows, :] = np.moveaxis(linear(x, p["w_b"]), -1, 0)
    return out


def attend(q, k, v, bias, head_dim):
    """One attention problem per head with an additive bias, full softmax.

    q: [J, H, d] queries, k, v: [K, H, d] keys/values, bias: [H][J][K].
    Returns o: [J, H, d] with o[j,h] = sum_k softmax_k(q[j,h].k[k,h]/sqrt(d) + bias[h,j,k]) v[k,h].
    """
    s = np.einsum("jhd,khd->hjk", q, k) / np.sqrt(head_dim) + bias
    a = softmax(s)
    return np.einsum("hjk,khd->jhd", a, v)


def gate_and_project_out(o, g, p):
    """out = (g * o) W_o^T + b_o, with o, g: [..., H, d]."""
    lead = o.shape[:-2]
    og = (g * o).reshape(*lead, p["heads"] * p["head_dim"])
    return linear(og, p["w_o"], p["b_o"])


def triangle_attn_start(z, p, rows=None):
    """Starting-node triangle attention of Z [I][I][c_z]; returns out [I][I][c_z].

    ``rows`` (optional) restricts the output to those rows i (the bias still
    comes from all of Z); the result is then [len(rows)][I][c_z].
    """
    I = z.shape[0]
    bias = pair_bias(z, p)
    rows = range(I) if rows is None else rows
    out = []
    for i in rows:
        q, k, v, g, _ = project(z[i], p)
        o = attend(q, k, v, bias, p["head_dim"])
        out.append(gate_and_project_out(o, g, p))
    return np.stack(out)


def triangle_attn_end(z, p, cols=None, bias=None):
    """Ending-node triangle attention, written directly (no transposition of Z).

    For every column j: queries q_ij and gates g_ij over i, keys/values k_kj,
    v_kj over k, and bias b_ki: bias_T[h][i][k] = bias[h][k][i].
    ``cols`` (optional) restricts the output to those columns j; the result is
    then [I][len(cols)][c_z] (all rows i, the chosen columns).  ``bias``
    (optional) is pair_bias(z, p) computed beforehand, for callers that
    evaluate the columns in several parts.
    """
    I = z.shape[0]
    bias = pair_bias(z, p) if bias is None else bias
    bias_t = np.transpose(bias, (0, 2, 1))
    cols = list(range(I)) if cols is None else list(cols)
    out = np.empty((I, len(cols), z.shape[2]))
    for n, j in enumerate(cols):
        q, k, v, g, _ = project(z[:, j], p)          # token (i, j) for i = 0..I-1
        o = attend(q, k, v, bias_t, p["head_dim"])    # query i, key k
        out[:, n] = gate_and_project_out(o, g, p)
    return out


def triangle_attn_rows(z_rows, bias, p):
    """Row-block triangle attention: rows z_rows [R][I][c_z] with a given bias [H][I][I]."""
    out = []
    for zi in z_rows:
        q, k, v, g, _ = project(zi, p)
        o = attend(q, k, v, bias, p["head_dim"])
        out.append(gate_and_project_out(o, g, p))
    return np.stack(out) if out else np.zeros((0,) + z_rows.shape[1:])


def params(weights_f64: dict, heads: int, head_dim: int, eps: float = 1e-5) -> dict:
    """Bundle float64 weight arrays with the shape constants the oracle needs."""
    p = dict(weights_f64)
    p.update(heads=heads, head_dim=head_dim, eps=eps)
    return p



def triangle_attn_rows_queries(z_rows, bias_q, queries, p):
    """Row-block attention evaluated only at some query positions.

    For every line r of z_rows [R][I][c_z] and every n, the output token of
    query position queries[n]; bias_q[h][n][k] is the bias of that query
    against key k.  Same definition as triangle_attn_rows, restricted to the
    chosen queries (large problems are checked on such samples).
    """
    queries = np.asarray(queries)
    out = []
    for zi in z_rows:
        q, k, v, g, _ = project(zi, p)
        o = attend(q[queries], k, v, bias_q, p["head_dim"])
        out.append(gate_and_project_out(o, g[queries], p))
    return np.stack(out)
