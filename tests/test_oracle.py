"""Pins for the float64 oracle (CPU only).

The oracle is checked against things other than itself:
* a pure-Python brute force written separately (tiny I);
* torch CPU library routines in float64 (layer_norm, linear,
  scaled_dot_product_attention with an additive float mask);
* closed forms (I = 1, two keys with one channel pair, uniform attention,
  zero gate, a bias that does not depend on the row);
* invariants (rows sum to one, start/end transposition, LayerNorm shift,
  per-query bias shift, permutation equivariance, row blocks);
* planted mistakes: each mutant of the oracle must fail at least one pin.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import brute, ref

SHAPES = [(8, 2, 4), (128, 4, 32)]


def rand_params(rng, c, H, d, gamma_beta=False, b_g=False, b_o=False):
    hd = H * d
    s = 1.0 / math.sqrt(c)
    p = {
        "w_q": rng.standard_normal((hd, c)) * s, "w_k": rng.standard_normal((hd, c)) * s,
        "w_v": rng.standard_normal((hd, c)) * s, "w_b": rng.standard_normal((H, c)) * s,
        "w_g": rng.standard_normal((hd, c)) * s, "w_o": rng.standard_normal((c, hd)) * s,
        "ln_gamma": 1.0 + 0.3 * rng.standard_normal(c) if gamma_beta else np.ones(c),
        "ln_beta": 0.2 * rng.standard_normal(c) if gamma_beta else np.zeros(c),
        "b_g": 0.5 * rng.standard_normal(hd) if b_g else np.zeros(hd),
        "b_o": 0.5 * rng.standard_normal(c) if b_o else np.zeros(c),
    }
    return ref.params(p, H, d, 1e-5)


def rand_z(rng, I, c, R=None):
    return rng.standard_normal((I if R is None else R, I, c))


# ----------------------------------------------------------------------------------------
# Pins written as functions of the oracle module, so planted mistakes can be re-checked.

def torch_start(z, p):
    """Starting-node attention composed from torch CPU float64 library routines."""
    I, c = z.shape[0], z.shape[2]
    H, d = p["heads"], p["head_dim"]
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    x = F.layer_norm(t(z), (c,), weight=t(p["ln_gamma"]), bias=t(p["ln_beta"]), eps=p["eps"])
    q = F.linear(x, t(p["w_q"])).view(I, I, H, d).permute(0, 2, 1, 3)  # [i, h, j, d]
    k = F.linear(x, t(p["w_k"])).view(I, I, H, d).permute(0, 2, 1, 3)
    v = F.linear(x, t(p["w_v"])).view(I, I, H, d).permute(0, 2, 1, 3)
    g = torch.sigmoid(F.linear(x, t(p["w_g"]), t(p["b_g"])))          # [i, j, hd]
    bias = F.linear(x, t(p["w_b"])).permute(2, 0, 1)                  # [h, j, k]
    o = F.scaled_dot_product_attention(q, k, v, attn_mask=bias)       # [i, h, j, d]
    o = o.permute(0, 2, 1, 3).reshape(I, I, H * d)
    return F.linear(o * g, t(p["w_o"]), t(p["b_o"])).numpy()


def two_key_closed_form(z, w, b_g, b_o, eps):
    """c_z = 2, H = 1, d = 1, I = 2, gamma = 1, beta = 0, derived by hand.

    A 2-channel token (a, b) normalises to s * (1, -1) with delta = (a - b) / 2
    and s = delta / sqrt(delta^2 + eps).  Each projection of it is s times the
    difference of the two weight columns.  Over two keys the softmax is the
    logistic function of the score difference.
    """
    I = 2
    s = np.empty((I, I))
    for i in range(I):
        for j in range(I):
            delta = (z[i, j, 0] - z[i, j, 1]) / 2.0
            s[i, j] = delta / math.sqrt(delta * delta + eps)
    col = {n: w[n][:, 0] - w[n][:, 1] for n in ("w_q", "w_k", "w_v", "w_g", "w_b")}
    out = np.empty((I, I, 2))
    for i in range(I):
        for j in range(I):
            q = s[i, j] * col["w_q"][0]
            sc = [q * s[i, k] * col["w_k"][0] + s[j, k] * col["w_b"][0] for k in range(I)]
            a0 = 1.0 / (1.0 + math.exp(-(sc[0] - sc[1])))
            o = a0 * s[i, 0] * col["w_v"][0] + (1.0 - a0) * s[i, 1] * col["w_v"][0]
            gate = 1.0 / (1.0 + math.exp(-(s[i, j] * col["w_g"][0] + b_g[0])))
            for c in range(2):
                out[i, j, c] = gate * o * w["w_o"][c, 0] + b_o[c]
    return out


def pin_brute(seed=0):
    rng = np.random.default_rng(seed)
    errs = []
    for (c, H, d), I in [((8, 2, 4), 5), ((128, 4, 32), 3)]:
        p = rand_params(rng, c, H, d, gamma_beta=True, b_g=True, b_o=True)
        z = rand_z(rng, I, c)
        errs.append(np.abs(ref.triangle_attn_start(z, p) - np.array(brute.start(z, p))).max())
        errs.append(np.abs(ref.triangle_attn_end(z, p) - np.array(brute.end(z, p))).max())
        bias = rng.standard_normal((H, I, I))
        zr = rand_z(rng, I, c, R=2)
        errs.append(np.abs(ref.triangle_attn_rows(zr, bias, p) - np.array(brute.rows(zr, bias, p))).max())
        errs.append(np.abs(ref.pair_bias(z, p) - np.array(brute.pair_bias(z, p))).max())
    return max(errs)


def pin_torch(seed=1):
    rng = np.random.default_rng(seed)
    errs = []
    for (c, H, d), I in [((8, 2, 4), 6), ((128, 4, 32), 9)]:
        p = rand_params(rng, c, H, d, gamma_beta=True, b_g=True, b_o=True)
        z = rand_z(rng, I, c)
        errs.append(np.abs(ref.triangle_attn_start(z, p) - torch_start(z, p)).max())
    return max(errs)


def pin_closed_two_key(seed=2):
    rng = np.random.default_rng(seed)
    p = rand_params(rng, 2, 1, 1, b_g=True, b_o=True)
    z = rand_z(rng, 2, 2)
    return np.abs(ref.triangle_attn_start(z, p) - two_key_closed_form(z, p, p["b_g"], p["b_o"], p["eps"])).max()


def pin_transpose(seed=3):
    rng = np.random.default_rng(seed)
    p = rand_params(rng, 8, 2, 4, gamma_beta=True, b_g=True)
    z = rand_z(rng, 7, 8)
    a = ref.triangle_attn_end(z, p)
    b = np.transpose(ref.triangle_attn_start(np.transpose(z, (1, 0, 2)), p), (1, 0, 2))
    return np.abs(a - b).max()


def pin_uniform(seed=4):
    """W_q = 0 and W_b = 0: every key gets the same weight, o_ij = mean_k v_ik."""
    rng = np.random.default_rng(seed)
    c, H, d, I = 16, 2, 4, 6
    p = rand_params(rng, c, H, d, gamma_beta=True, b_g=True, b_o=True)
    p["w_q"] = np.zeros_like(p["w_q"])
    p["w_b"] = np.zeros_like(p["w_b"])
    z = rand_z(rng, I, c)
    x = (z - z.mean(-1, keepdims=True)) / np.sqrt(z.var(-1, keepdims=True) + p["eps"]) * p["ln_gamma"] + p["ln_beta"]
    v = x @ p["w_v"].T                                 # [i, k, hd]
    g = 1.0 / (1.0 + np.exp(-(x @ p["w_g"].T + p["b_g"])))
    o = np.repeat(v.mean(axis=1, keepdims=True), I, axis=1)
    want = (g * o) @ p["w_o"].T + p["b_o"]
    return np.abs(ref.triangle_attn_start(z, p) - want).max()


def pin_i1(seed=5):
    """I = 1: the softmax over one key is 1, so out = (sigmoid(g) * v) W_o^T + b_o."""
    rng = np.random.default_rng(seed)
    c, H, d = 128, 4, 32
    p = rand_params(rng, c, H, d, gamma_beta=True, b_g=True, b_o=True)
    z = rand_z(rng, 1, c)
    x = F.layer_norm(torch.from_numpy(z), (c,), torch.from_numpy(p["ln_gamma"]),
                     torch.from_numpy(p["ln_beta"]), p["eps"]).numpy()
    v = x @ p["w_v"].T
    g = 1.0 / (1.0 + np.exp(-(x @ p["w_g"].T + p["b_g"])))
    want = (g * v) @ p["w_o"].T + p["b_o"]
    return max(np.abs(ref.triangle_attn_start(z, p) - want).max(),
               np.abs(ref.triangle_attn_end(z, p) - want).max())


ALL_PINS = [pin_brute, pin_torch, pin_closed_two_key, pin_transpose, pin_uniform, pin_i1]
PIN_TOL = 1e-10


# ----------------------------------------------------------------------------------------
# The pins themselves.

@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    assert pin() <= PIN_TOL


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("I", [1, 2, 4])
def test_brute_small_shapes(seed, I):
    rng = np.random.default_rng(100 + seed)
    p = rand_params(rng, 8, 2, 4, gamma_beta=True, b_g=True, b_o=True)
    z = rand_z(rng, I, 8)
    assert np.abs(ref.triangle_attn_start(z, p) - np.array(brute.start(z, p))).max() <= 1e-12
    assert np.abs(ref.triangle_attn_end(z, p) - np.array(brute.end(z, p))).max() <= 1e-12


def test_brute_real_channels_i2():
    rng = np.random.default_rng(7)
    p = rand_params(rng, 128, 4, 32)
    z = rand_z(rng, 2, 128)
    assert np.abs(ref.triangle_attn_start(z, p) - np.array(brute.start(z, p))).max() <= 1e-12


def test_torch_sdpa_real_shape():
    rng = np.random.default_rng(8)
    p = rand_params(rng, 128, 4, 32)
    z = rand_z(rng, 24, 128)
    assert np.abs(ref.triangle_attn_start(z, p) - torch_start(z, p)).max() <= 1e-12


def test_softmax_rows_sum_to_one_and_nonneg():
    rng = np.random.default_rng(9)
    s = rng.standard_normal((3, 5, 7)) * 30
    a = ref.softmax(s)
    assert np.all(a >= 0) and np.abs(a.sum(-1) - 1).max() <= 1e-12
    # shift invariance of the softmax along keys
    assert np.abs(ref.softmax(s + rng.standard_normal((3, 5, 1)) * 50) - a).max() <= 1e-12


def test_zero_gate_gives_output_bias_exactly():
    rng = np.random.default_rng(10)
    p = rand_params(rng, 128, 4, 32, b_o=True)
    p["w_g"] = np.zeros_like(p["w_g"])
    p["b_g"] = np.full(128, -1e4)
    z = rand_z(rng, 5, 128)
    out = ref.triangle_attn_start(z, p)
    assert np.array_equal(out, np.broadcast_to(p["b_o"], out.shape))
    p["b_o"] = np.zeros(128)
    assert np.array_equal(ref.triangle_attn_end(z, p), np.zeros_like(out))


def test_row_independent_bias_is_plain_matmul():
    """W_q = 0: A[j,k] = softmax_k(b_jk) is the same for every row, so O_i = A V_i."""
    rng = np.random.default_rng(11)
    c, H, d, I = 16, 2, 8, 7
    p = rand_params(rng, c, H, d, b_g=True)
    p["w_q"] = np.zeros_like(p["w_q"])
    z = rand_z(rng, I, c)
    bias = ref.pair_bias(z, p)                                   # [h, j, k]
    a = np.exp(bias - bias.max(-1, keepdims=True))
    a /= a.sum(-1, keepdims=True)
    x = F.layer_norm(torch.from_numpy(z), (c,), eps=p["eps"]).numpy()
    v = (x @ p["w_v"].T).reshape(I, I, H, d)
    g = (1 / (1 + np.exp(-(x @ p["w_g"].T + p["b_g"])))).reshape(I, I, H, d)
    o = np.stack([np.stack([a[h] @ v[i, :, h, :] for h in range(H)], axis=1) for i in range(I)])
    want = (g * o).reshape(I, I, H * d) @ p["w_o"].T + p["b_o"]
    assert np.abs(ref.triangle_attn_start(z, p) - want).max() <= 1e-12


def test_layernorm_shift_invariance():
    rng = np.random.default_rng(12)
    p = rand_params(rng, 128, 4, 32)
    z = rand_z(rng, 6, 128)
    shift = rng.standard_normal((6, 6, 1)) * 5
    assert np.abs(ref.triangle_attn_start(z + shift, p) - ref.triangle_attn_start(z, p)).max() <= 1e-10


def test_distogram_offset_invariance():
    """The distogram-like term 2exp(-|i-j|/32) is the same on every channel of a token."""
    rng = np.random.default_rng(13)
    p = rand_params(rng, 128, 4, 32)
    I = 8
    z = rand_z(rng, I, 128)
    i = np.arange(I)[:, None]
    dist = (2 * np.exp(-np.abs(i - i.T) / 32.0))[:, :, None]
    for f in (ref.triangle_attn_start, ref.triangle_attn_end):
        assert np.abs(f(z + dist, p) - f(z, p)).max() <= 1e-10


def test_per_query_bias_shift_invariance():
    rng = np.random.default_rng(14)
    p = rand_params(rng, 128, 4, 32)
    I = 9
    zr = rand_z(rng, I, 128, R=3)
    bias = rng.standard_normal((4, I, I))
    shift = rng.standard_normal((1, I, 1)) * 30
    a = ref.triangle_attn_rows(zr, bias, p)
    assert np.abs(ref.triangle_attn_rows(zr, bias + shift, p) - a).max() <= 1e-10


def test_permutation_equivariance():
    rng = np.random.default_rng(15)
    p = rand_params(rng, 32, 2, 8, gamma_beta=True, b_g=True)
    I = 7
    z = rand_z(rng, I, 32)
    pi = rng.permutation(I)
    zp = z[pi][:, pi]
    for f in (ref.triangle_attn_start, ref.triangle_attn_end):
        assert np.abs(f(zp, p) - f(z, p)[pi][:, pi]).max() <= 1e-12


def test_rows_equal_full_rows_and_subsets():
    rng = np.random.default_rng(16)
    p = rand_params(rng, 128, 4, 32, b_g=True)
    I = 10
    z = rand_z(rng, I, 128)
    full = ref.triangle_attn_start(z, p)
    bias = ref.pair_bias(z, p)
    assert np.array_equal(ref.triangle_attn_rows(z[3:7], bias, p), full[3:7])
    assert np.array_equal(ref.triangle_attn_start(z, p, rows=[2, 9]), full[[2, 9]])
    full_end = ref.triangle_attn_end(z, p)
    assert np.array_equal(ref.triangle_attn_end(z, p, cols=[0, 5]), full_end[:, [0, 5]])


def test_pair_bias_chunking():
    rng = np.random.default_rng(17)
    p = rand_params(rng, 16, 2, 4)
    z = rand_z(rng, 9, 16)
    assert np.abs(ref.pair_bias(z, p, chunk_rows=2) - ref.pair_bias(z, p, chunk_rows=64)).max() == 0.0


# ----------------------------------------------------------------------------------------
# Planted mistakes: each must be caught by at least one pin.

def _mut_bias_transposed(orig):
    return lambda q, k, v, bias, d: orig(q, k, v, np.transpose(bias, (0, 2, 1)), d)


def _mut_no_scale(orig):
    return lambda q, k, v, bias, d: orig(q, k, v, bias, 1)


def _mut_softmax_axis(_orig):
    def f(s):
        e = np.exp(s - s.max(axis=-2, keepdims=True))
        return e / e.sum(axis=-2, keepdims=True)
    return f


def _mut_unbiased_var(_orig):
    def f(z, gamma, beta, eps):
        mu = z.mean(-1, keepdims=True)
        return (z - mu) / np.sqrt(z.var(-1, ddof=1, keepdims=True) + eps) * gamma + beta
    return f


def _mut_ln_no_beta(_orig):
    def f(z, gamma, beta, eps):
        mu = z.mean(-1, keepdims=True)
        return (z - mu) / np.sqrt(((z - mu) ** 2).mean(-1, keepdims=True) + eps) * gamma
    return f


def _mut_out_untransposed(_orig):
    def f(o, g, p):
        lead = o.shape[:-2]
        return (g * o).reshape(*lead, -1) @ p["w_o"] + p["b_o"]
    return f


def _mut_no_out_bias(_orig):
    def f(o, g, p):
        lead = o.shape[:-2]
        return (g * o).reshape(*lead, -1) @ p["w_o"].T
    return f


def _mut_gate_no_sigmoid(_orig):
    return lambda x: x


def _mut_sigmoid_sign(_orig):
    return lambda x: 1.0 / (1.0 + np.exp(x))


def _mut_exp_minus_max_dropped(_orig):
    def f(s):
        e = np.exp(s)
        return e / (e.sum(-1, keepdims=True) + 1e-3)
    return f


def _mut_head_split(orig):
    def f(z, p):
        q, k, v, g, b = orig(z, p)
        sw = lambda a: a.reshape(*a.shape[:-2], -1).reshape(*a.shape[:-2], a.shape[-1], a.shape[-2]).swapaxes(-1, -2)
        return sw(q), sw(k), sw(v), sw(g), b
    return f


def _mut_end_bias_untransposed(_orig):
    def f(z, p, cols=None):
        I = z.shape[0]
        bias = ref.pair_bias(z, p)
        out = np.empty((I, I, z.shape[2]))
        for j in range(I):
            q, k, v, g, _ = ref.project(z[:, j], p)
            out[:, j] = ref.gate_and_project_out(ref.attend(q, k, v, bias, p["head_dim"]), g, p)
        return out
    return f


def _mut_end_keys_of_row(_orig):
    def f(z, p, cols=None):
        I = z.shape[0]
        bias_t = np.transpose(ref.pair_bias(z, p), (0, 2, 1))
        out = np.empty((I, I, z.shape[2]))
        for j in range(I):
            q, _, _, g, _ = ref.project(z[:, j], p)
            _, k, v, _, _ = ref.project(z[j], p)
            out[:, j] = ref.gate_and_project_out(ref.attend(q, k, v, bias_t, p["head_dim"]), g, p)
        return out
    return f


MUTANTS = [
    ("attend", _mut_bias_transposed), ("attend", _mut_no_scale), ("softmax", _mut_softmax_axis),
    ("layer_norm", _mut_unbiased_var), ("layer_norm", _mut_ln_no_beta),
    ("gate_and_project_out", _mut_out_untransposed), ("gate_and_project_out", _mut_no_out_bias),
    ("sigmoid", _mut_gate_no_sigmoid), ("sigmoid", _mut_sigmoid_sign),
    ("softmax", _mut_exp_minus_max_dropped), ("project", _mut_head_split),
    ("triangle_attn_end", _mut_end_bias_untransposed), ("triangle_attn_end", _mut_end_keys_of_row),
]


@pytest.mark.parametrize("name,mut", MUTANTS, ids=[m.__name__ for _, m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, name, mut):
    monkeypatch.setattr(ref, name, mut(getattr(ref, name)))
    caught = []
    for pin in ALL_PINS:
        try:
            caught.append(pin() > PIN_TOL)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(True)
    assert any(caught), f"mutant {mut.__name__} of {name} passed every pin"


def test_rows_queries_is_restriction_of_rows_start_and_end():
    rng = np.random.default_rng(18)
    p = rand_params(rng, 128, 4, 32, gamma_beta=True, b_g=True)
    I = 11
    z = rand_z(rng, I, 128)
    js = [0, 4, 10]
    full = ref.triangle_attn_start(z, p)
    got = ref.triangle_attn_rows_queries(z[[2, 7]], ref.pair_bias(z[js], p), js, p)
    assert np.abs(got - full[[2, 7]][:, js]).max() <= 1e-12
    # ending node: line = column j, queries = rows i, bias of query i against key k is b_ki
    full_end = ref.triangle_attn_end(z, p)
    is_ = [1, 9]
    bias_q = ref.pair_bias(np.transpose(z[:, is_], (1, 0, 2)), p)  # [h][n][k] = b(z[k, i_n])
    got = ref.triangle_attn_rows_queries(np.transpose(z[:, [3, 6]], (1, 0, 2)), bias_q, is_, p)
    assert np.abs(got - np.transpose(full_end[is_][:, [3, 6]], (1, 0, 2))).max() <= 1e-12
