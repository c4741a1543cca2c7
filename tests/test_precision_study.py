"""Precision study: the attention stage with 8-bit (e4m3) operands, and the key-block
state's dtype (CPU only).

The fused attention kernel keeps q, k, v^T and the probabilities P in bf16 and
accumulates in fp32.  An 8-bit variant (fp8 MFMA on gfx950) would round q, k
or v to e4m3.  This model reproduces the kernel's roundings on the CPU -- the
projections rounded to bf16, the shifted base-2 bias to fp16, the scores to
fp32, P to bf16, the gated head outputs and the result to bf16 -- optionally
with q and k, or v, rounded to e4m3 with a per-tensor scale (amax / 448), and
compares each variant with the float64 oracle on the same inputs.

What it shows: the bf16 pipeline meets the bf16 bar (relative L1 <= 5e-3,
max abs <= 2e-2), and every e4m3 variant misses it several times over --
with a per-tensor scale, with MX-style power-of-two scales per token and head
(the block scales gfx950's scaled fp8 MFMA takes), with one scale per 64-key
tile, and with P in e4m3 scaled per row -- so an 8-bit attention variant cannot
be built to the same parity bar.

The same model, with the keys folded in blocks into a carried state as the key-block
stage does, shows why that state holds O / l in fp16: over seven folds it costs about
0.5% of relative L1 against an fp32 state, where a bf16 state would reach the bar.

Two 16-bit alternatives are modelled as well.  The projection stage feeds the
LayerNorm output x to the bf16 matrix core as hi + lo (two products per weight
fragment): x rounded to bf16 alone costs about 25% more relative L1, while x and
the weights in fp16 (one product) match the hi + lo split.  And the softmax
operands in fp16 (scores rounded to fp16 before the exponential, P and v in fp16)
would lower the error slightly; on gfx950 an fp16 exponential issues at the same
rate as the fp32 one, so that variant would not be faster.
"""
import numpy as np
import pytest
import torch

from oracle import ref
from protein_pair_representation_amd import inputs

LOG2E = 1.4426950408889634
E4M3_MAX = 448.0
BAR_REL_L1, BAR_MAX_ABS = 5e-3, 2e-2


def rnd(x, dtype):
    return torch.from_numpy(np.asarray(x, dtype=np.float64)).to(dtype).to(torch.float64).numpy()


def e4m3(x):
    s = np.abs(x).max() / E4M3_MAX
    return rnd(x / s, torch.float8_e4m3fn) * s


def e4m3_blocks(x, axis_len, axis=-1):
    """e4m3 with one power-of-two scale per block of `axis_len` consecutive elements
    along `axis` (the shared 8-bit exponent of the MX block formats gfx950's scaled
    fp8 MFMA takes): each block's amax is brought just under 448."""
    x = np.moveaxis(x, axis, -1)
    shp = x.shape
    xb = x.reshape(shp[:-1] + (shp[-1] // axis_len, axis_len))
    amax = np.abs(xb).max(-1, keepdims=True)
    s = np.where(amax > 0, 2.0 ** np.ceil(np.log2(np.maximum(amax, 1e-300) / E4M3_MAX)), 1.0)
    y = (rnd(xb / s, torch.float8_e4m3fn) * s).reshape(shp)
    return np.moveaxis(y, -1, axis)


# 8-bit variants of the operands: per-tensor scale (as above), MX-style blocks along
# the contraction (32 channels of a head for q and k: one scale per token and head),
# per 64-key tile for k and v (one scale per line, head and key tile), and P in
# e4m3 with one scale per query row (the row maximum of a tile brought to 448)
VARIANTS = {
    "qk-e4m3": dict(qk8="tensor"),
    "v-e4m3": dict(v8="tensor"),
    "qkv-e4m3": dict(qk8="tensor", v8="tensor"),
    "qk-e4m3-mx32": dict(qk8="mx"),
    "k-e4m3-tile64": dict(k8="tile"),
    "v-e4m3-tile64": dict(v8="tile"),
    "p-e4m3-row": dict(p8="row"),
}


def _q8(x, mode, d):
    if mode == "tensor":
        return e4m3(x)
    if mode == "mx":                                           # per token and head (32 channels)
        return e4m3_blocks(x, d, axis=-1)
    raise ValueError(mode)


def _tile8(x, d, tile=64):
    """x [I][keys][H*d]: one scale per (line, key tile of 64, head)."""
    I, K, C = x.shape
    y = np.empty_like(x)
    for k0 in range(0, K, tile):
        for h in range(C // d):
            blk = x[:, k0:k0 + tile, h * d:(h + 1) * d]
            amax = np.abs(blk).max(axis=(1, 2), keepdims=True)
            s = np.maximum(amax, 1e-300) / E4M3_MAX
            y[:, k0:k0 + tile, h * d:(h + 1) * d] = rnd(blk / s, torch.float8_e4m3fn) * s
    return y


def model(z, p, qk8=None, v8=None, k8=None, p8=None):
    """Starting-node attention of z [I][I][c_z] with the kernel's roundings, and the
    chosen operands in e4m3 (qk8 "tensor"/"mx", k8 / v8 "tensor"/"tile", p8 "row")."""
    H, d = p["heads"], p["head_dim"]
    x = rnd(ref.layer_norm(z, p["ln_gamma"], p["ln_beta"], p["eps"]), torch.float32)
    q = rnd(x @ p["w_q"].T * (LOG2E / np.sqrt(d)), torch.bfloat16)
    k = rnd(x @ p["w_k"].T, torch.bfloat16)
    v = rnd(x @ p["w_v"].T, torch.bfloat16)
    g = rnd(ref.sigmoid(x @ p["w_g"].T + p["b_g"]), torch.bfloat16)
    if qk8:
        q, k = _q8(q, qk8, d), _q8(k, qk8, d)
    if k8 == "tile":
        k = _tile8(k, d)
    if v8 == "tensor":
        v = e4m3(v)
    elif v8 == "tile":
        v = _tile8(v, d)
    b = np.moveaxis(x @ p["w_b"].T, -1, 0)                         # [H][j][k]
    b = rnd((b - b.max(-1, keepdims=True)) * LOG2E, torch.float16)
    out = []
    for i in range(z.shape[0]):
        heads = []
        for h in range(H):
            sl = slice(h * d, (h + 1) * d)
            s = rnd(q[i, :, sl] @ k[i, :, sl].T + b[h], torch.float32)
            pr = np.exp2(s - s.max(-1, keepdims=True))
            if p8 == "row":                                       # values in (0, 1]: scale 448
                pr = rnd(pr * E4M3_MAX, torch.float8_e4m3fn) / E4M3_MAX
            else:
                pr = rnd(pr, torch.bfloat16)
            o = (pr @ v[i, :, sl]) / pr.sum(-1, keepdims=True)
            heads.append(rnd(o * g[i, :, sl], torch.bfloat16))
        out.append(rnd(np.concatenate(heads, -1) @ p["w_o"].T + p["b_o"], torch.bfloat16))
    return np.stack(out)


@pytest.fixture(scope="module")
def case():
    I, seed = 128, 2
    w = inputs.make_weights(seed, "bf16")
    p = ref.params(inputs.weights_f64(w), 4, 32)
    z = inputs.to_f64(inputs.make_z(seed, I, "bf16"))
    return z, p, ref.triangle_attn_start(z, p)


def errors(got, want):
    err = np.abs(got - want)
    return err.max(), err.sum() / np.abs(want).sum()


def test_bf16_pipeline_meets_the_bar(case):
    z, p, want = case
    mx, rl1 = errors(model(z, p), want)
    assert mx <= BAR_MAX_ABS and rl1 <= BAR_REL_L1, (mx, rl1)


@pytest.mark.parametrize("name", list(VARIANTS))
def test_e4m3_operands_miss_the_bar(case, name):
    """Every 8-bit variant misses the bf16 bar by a wide margin: finer scales fix the
    range, not the 3-bit mantissa, whose rounding (up to 1/16 relative) dominates."""
    z, p, want = case
    mx, rl1 = errors(model(z, p, **VARIANTS[name]), want)
    print(f"{name}: max abs {mx:.2e}, rel L1 {rl1:.2e}")
    assert rl1 > 2 * BAR_REL_L1, (name, mx, rl1)


def fold_model(z, p, block, state_dtype):
    """Starting-node attention with the keys folded in blocks of `block` into a carried
    state, as the key-block stage does: per block the running shift m moves to the new
    maximum, P (bf16) is taken against it, and the carried O / l is rounded to
    `state_dtype` after every block but the last (the last block's O / l goes straight
    to the gate).  Projections, bias and output are rounded as in `model`."""
    H, d = p["heads"], p["head_dim"]
    x = rnd(ref.layer_norm(z, p["ln_gamma"], p["ln_beta"], p["eps"]), torch.float32)
    q = rnd(x @ p["w_q"].T * (LOG2E / np.sqrt(d)), torch.bfloat16)
    k = rnd(x @ p["w_k"].T, torch.bfloat16)
    v = rnd(x @ p["w_v"].T, torch.bfloat16)
    g = rnd(ref.sigmoid(x @ p["w_g"].T + p["b_g"]), torch.bfloat16)
    b = np.moveaxis(x @ p["w_b"].T, -1, 0)
    b = rnd((b - b.max(-1, keepdims=True)) * LOG2E, torch.float16)
    I = z.shape[0]
    starts = list(range(0, I, block))
    out = []
    for i in range(I):
        heads = []
        for h in range(H):
            sl = slice(h * d, (h + 1) * d)
            s = rnd(q[i, :, sl] @ k[i, :, sl].T + b[h], torch.float32)
            m = np.full((I, 1), -np.inf)
            l = np.zeros((I, 1))
            on = np.zeros((I, d))
            for n, k0 in enumerate(starts):
                sb = s[:, k0:k0 + block]
                m_new = np.maximum(m, sb.max(-1, keepdims=True))
                pb = rnd(np.exp2(sb - m_new), torch.bfloat16)
                alpha = np.exp2(m - m_new)
                l_new = l * alpha + pb.sum(-1, keepdims=True)
                o_full = on * l * alpha + pb @ v[i, k0:k0 + block, sl]
                on = o_full / l_new
                if n < len(starts) - 1:
                    on = rnd(on, state_dtype)
                m, l = m_new, l_new
            heads.append(rnd(on * g[i, :, sl], torch.bfloat16))
        out.append(rnd(np.concatenate(heads, -1) @ p["w_o"].T + p["b_o"], torch.bfloat16))
    return np.stack(out)


@pytest.mark.parametrize("block", [64, 16])
def test_fp16_state_holds_the_bar(case, block):
    """The key-block state carries O / l in fp16 for bf16 problems.  Folding the keys in
    blocks of 64 (2 roundings of the state at I = 128) or 16 (7 roundings) keeps the
    bf16 bar, within 10% of the relative L1 an fp32 state gives."""
    z, p, want = case
    mx16, rl16 = errors(fold_model(z, p, block, torch.float16), want)
    mx32, rl32 = errors(fold_model(z, p, block, torch.float32), want)
    print(f"block {block}: fp16 state max abs {mx16:.2e} rel L1 {rl16:.3e}; fp32 state {mx32:.2e} {rl32:.3e}")
    assert mx16 <= BAR_MAX_ABS and rl16 <= BAR_REL_L1, (mx16, rl16)
    assert rl16 <= 1.1 * rl32, (rl16, rl32)


def test_bf16_state_would_cost_more(case):
    """The same fold with O / l carried in bf16 (a state half the size of fp32's, like
    fp16's) loses more: the reason the state uses fp16, not bf16."""
    z, p, want = case
    _, rl16 = errors(fold_model(z, p, 16, torch.float16), want)
    _, rlb = errors(fold_model(z, p, 16, torch.bfloat16), want)
    print(f"block 16: fp16 state rel L1 {rl16:.3e}, bf16 state {rlb:.3e}")
    assert rlb > rl16, (rlb, rl16)


def model16(z, p, xmode="hilo", w16=False, pv=torch.bfloat16, s16=False):
    """Starting-node attention with the kernel's roundings and 16-bit alternatives:
    xmode = "hilo" (the LayerNorm output seen to about fp32, as the hi + lo products do),
    "bf16" or "fp16"; w16 rounds the projection weights to fp16 (the bf16 weights
    convert exactly, up to fp16's range); pv is the dtype of P and v; s16 rounds
    the scores to fp16 before the exponential (an fp16 exponential's input).  The
    gate is projected from bf16 x unless x is fp16, as the projection kernel does."""
    H, d = p["heads"], p["head_dim"]
    x0 = ref.layer_norm(z, p["ln_gamma"], p["ln_beta"], p["eps"])
    x = {"hilo": rnd(x0, torch.float32), "bf16": rnd(x0, torch.bfloat16), "fp16": rnd(x0, torch.float16)}[xmode]
    xg = x if xmode == "fp16" else rnd(x0, torch.bfloat16)
    W = {n: (rnd(p[n], torch.float16) if w16 else p[n]) for n in ("w_q", "w_k", "w_v", "w_g", "w_b")}
    q = rnd(x @ W["w_q"].T * (LOG2E / np.sqrt(d)), torch.bfloat16)
    k = rnd(x @ W["w_k"].T, torch.bfloat16)
    v = rnd(x @ W["w_v"].T, pv)
    g = rnd(ref.sigmoid(xg @ W["w_g"].T + p["b_g"]), torch.bfloat16)
    b = np.moveaxis(x @ W["w_b"].T, -1, 0)
    b = rnd((b - b.max(-1, keepdims=True)) * LOG2E, torch.float16)
    out = []
    for i in range(z.shape[0]):
        heads = []
        for h in range(H):
            sl = slice(h * d, (h + 1) * d)
            s = rnd(q[i, :, sl] @ k[i, :, sl].T + b[h], torch.float32)
            if s16:
                s = rnd(s, torch.float16)
            pr = rnd(np.exp2(s), pv)
            o = (pr @ v[i, :, sl]) / pr.sum(-1, keepdims=True)
            heads.append(rnd(o * g[i, :, sl], torch.bfloat16))
        out.append(rnd(np.concatenate(heads, -1) @ p["w_o"].T + p["b_o"], torch.bfloat16))
    return np.stack(out)


def test_projection_needs_more_than_bf16_x(case):
    """x rounded to bf16 before the projections costs about 25% more relative L1 than
    the hi + lo split the projection kernel uses (at I = 128 it sits at the bar); x
    and the weights in fp16 with one product match the split."""
    z, p, want = case
    _, r_hilo = errors(model16(z, p, xmode="hilo"), want)
    _, r_bf16 = errors(model16(z, p, xmode="bf16"), want)
    mx16, r_fp16 = errors(model16(z, p, xmode="fp16", w16=True), want)
    print(f"x hi+lo {r_hilo:.3e}, x bf16 {r_bf16:.3e}, x and W fp16 {r_fp16:.3e}")
    assert r_bf16 > 1.15 * r_hilo, (r_bf16, r_hilo)
    assert r_fp16 <= 1.02 * r_hilo and mx16 <= BAR_MAX_ABS, (r_fp16, r_hilo, mx16)


def test_fp16_softmax_operands_hold_the_bar(case):
    """Scores rounded to fp16 before the exponential, P and v in fp16: within the bar
    and no worse than the bf16 P and v the kernel uses."""
    z, p, want = case
    _, r_bf16 = errors(model16(z, p), want)
    mx, r_f16 = errors(model16(z, p, pv=torch.float16, s16=True), want)
    print(f"P, v bf16 {r_bf16:.3e}; scores, P, v fp16 {r_f16:.3e} (max abs {mx:.2e})")
    assert mx <= BAR_MAX_ABS and r_f16 <= r_bf16, (mx, r_f16, r_bf16)
