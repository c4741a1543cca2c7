"""Precision study: the attention stage with 8-bit (e4m3) operands (CPU only).

The fused attention kernel keeps q, k, v^T and the probabilities P in bf16 and
accumulates in fp32.  An 8-bit variant (fp8 MFMA on gfx950) would round q, k
or v to e4m3.  This model reproduces the kernel's roundings on the CPU -- the
projections rounded to bf16, the shifted base-2 bias to fp16, the scores to
fp32, P to bf16, the gated head outputs and the result to bf16 -- optionally
with q and k, or v, rounded to e4m3 with a per-tensor scale (amax / 448), and
compares each variant with the float64 oracle on the same inputs.

What it shows: the bf16 pipeline meets the bf16 bar (relative L1 <= 5e-3,
max abs <= 2e-2), and every e4m3 variant misses it several times over, so an
8-bit attention variant cannot be built to the same parity bar.
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


def model(z, p, qk8=False, v8=False):
    """Starting-node attention of z [I][I][c_z] with the kernel's roundings."""
    H, d = p["heads"], p["head_dim"]
    x = rnd(ref.layer_norm(z, p["ln_gamma"], p["ln_beta"], p["eps"]), torch.float32)
    q = rnd(x @ p["w_q"].T * (LOG2E / np.sqrt(d)), torch.bfloat16)
    k = rnd(x @ p["w_k"].T, torch.bfloat16)
    v = rnd(x @ p["w_v"].T, torch.bfloat16)
    g = rnd(ref.sigmoid(x @ p["w_g"].T + p["b_g"]), torch.bfloat16)
    if qk8:
        q, k = e4m3(q), e4m3(k)
    if v8:
        v = e4m3(v)
    b = np.moveaxis(x @ p["w_b"].T, -1, 0)                         # [H][j][k]
    b = rnd((b - b.max(-1, keepdims=True)) * LOG2E, torch.float16)
    out = []
    for i in range(z.shape[0]):
        heads = []
        for h in range(H):
            sl = slice(h * d, (h + 1) * d)
            s = rnd(q[i, :, sl] @ k[i, :, sl].T + b[h], torch.float32)
            pr = rnd(np.exp2(s - s.max(-1, keepdims=True)), torch.bfloat16)
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


@pytest.mark.parametrize("qk8,v8", [(True, False), (False, True), (True, True)], ids=["qk-e4m3", "v-e4m3", "qkv-e4m3"])
def test_e4m3_operands_miss_the_bar(case, qk8, v8):
    z, p, want = case
    mx, rl1 = errors(model(z, p, qk8=qk8, v8=v8), want)
    assert rl1 > 4 * BAR_REL_L1, (mx, rl1)
