"""GPU parity of the projection stage fed by token-wise quantized records
(triangle_attn_project_aaq), followed by the unchanged attention stage.

Expected values: the float64 oracle run on the oracle's own decode of the same
records (the records themselves are written by the oracle's encoder), with the
bf16 bars of the other parity tests.  A second check needs no oracle: tokens
that lie on a power-of-two grid decode to exactly their bf16 values, so the
workspace filled from their records must equal, bit for bit, the one filled
from the bf16 tokens.
"""
import numpy as np
import pytest
import torch

from oracle import aaq as oaq
from oracle import ref
from protein_pair_representation_amd import inputs
from protein_pair_representation_amd import triattn as ta

from test_parity import check, dev, params64, say, weights_with_extras

pytestmark = pytest.mark.gpu


def encode(z: torch.Tensor, group: str) -> np.ndarray:
    return oaq.encode(z.float().numpy().reshape(-1, 128), group)


def decoded(rec: np.ndarray, group: str, shape) -> np.ndarray:
    return oaq.decode(rec, group).astype(np.float64).reshape(shape)


@pytest.mark.parametrize("I", [65, 200])
@pytest.mark.parametrize("group", ["A", "B", "C"])
@pytest.mark.parametrize("variant", ["start", "end"])
def test_full_variants(variant, group, I):
    say(f"[aaq->K1] {variant} group {group} I={I}")
    w = weights_with_extras(700 + I, "bf16")
    z = inputs.make_z(700 + I, I, "bf16", outliers=True)
    rec = encode(z, group)
    wd = dev(w)
    ws = ta.triangle_attn_project_aaq(torch.from_numpy(rec).cuda(), wd, I, I, group, variant=variant)
    out = ta.triangle_attn_attend(ws, wd, I, I, torch.bfloat16, variant=variant)
    torch.cuda.synchronize()
    f = ref.triangle_attn_start if variant == "start" else ref.triangle_attn_end
    check(out, f(decoded(rec, group, (I, I, 128)), params64(w)), "bf16", f"{variant} {group} I={I}")


@pytest.mark.parametrize("group", ["A", "B"])
def test_row_block(group):
    I, R = 160, 40
    say(f"[aaq->K1] row block R={R} of I={I}, group {group}")
    w = weights_with_extras(800, "bf16")
    zr = inputs.make_z_rows(800, I, 0, R, "bf16", outliers=True)
    rec = encode(zr, group)
    bias = inputs.random_bias(800, 4, I, scale=1.0)
    wd = dev(w)
    ws = ta.triangle_attn_project_aaq(torch.from_numpy(rec).cuda(), wd, I, R, group, variant="rows")
    out = ta.triangle_attn_attend(ws, wd, I, R, torch.bfloat16, variant="rows", bias=bias.cuda())
    torch.cuda.synchronize()
    want = ref.triangle_attn_rows(decoded(rec, group, (R, I, 128)), inputs.to_f64(bias), params64(w))
    check(out, want, "bf16", f"rows {group}")


@pytest.mark.parametrize("group", ["A", "B", "C"])
def test_exact_grid_equals_bf16_path(group):
    """Tokens s (q - z) with s = 2^-5 and codes spread over the whole range (no
    value beyond 3 sigma) decode exactly to their bf16 values: the workspace from
    the records equals the workspace from the bf16 tokens bit for bit."""
    I = 96
    say(f"[aaq->K1] exact grid, group {group}")
    qmax = 255 if group == "A" else 15
    rng = np.random.default_rng(5)
    q = rng.integers(0, qmax + 1, (I * I, 128))
    q[:, 0], q[:, 1] = 0, qmax
    zp = rng.integers(1, qmax, (I * I, 1))
    x = ((q - zp) * 2.0 ** -5).astype(np.float32)
    z = torch.from_numpy(x.reshape(I, I, 128)).to(torch.bfloat16)
    assert torch.equal(z.float(), torch.from_numpy(x.reshape(I, I, 128)))
    rec = encode(z, group)
    assert np.array_equal(oaq.decode(rec, group), x)
    w = weights_with_extras(900, "bf16")
    wd = dev(w)
    for variant in ("start", "end"):
        ws_q = ta.triangle_attn_project_aaq(torch.from_numpy(rec).cuda(), wd, I, I, group, variant=variant)
        ws_z = ta.triangle_attn_project(z.cuda(), wd, variant=variant)
        torch.cuda.synchronize()
        vq = ta.workspace_views(ws_q, I, I, torch.bfloat16, variant)
        vz = ta.workspace_views(ws_z, I, I, torch.bfloat16, variant)
        # what the projection writes (the packed bias tiles follow from bias_f32 by the
        # same packing kernel; their query rows past I are never written)
        for name in ("q", "k", "vt", "g", "bias_f32"):
            a, b = vq[name], vz[name]
            same = torch.equal(a.view(torch.int16) if a.element_size() == 2 else a.view(torch.int32),
                               b.view(torch.int16) if b.element_size() == 2 else b.view(torch.int32))
            assert same, f"{variant}: {name} differs"


def test_workload_1024_group_a():
    """The I = 1024 pair tensor (starting node) as group-A records; sampled rows
    and queries against the oracle on the decoded tensor."""
    wl = inputs.WORKLOADS["startend-bf16-I1024-distogram"]
    say("[aaq->K1] startend-bf16-I1024-distogram as group A records (oracle encode)")
    z = inputs.workload_z(wl)
    I = wl.I
    rec = encode(z, "A")
    w = inputs.workload_weights(wl)
    wd = dev(w)
    ws = ta.triangle_attn_project_aaq(torch.from_numpy(rec).cuda(), wd, I, I, "A", variant="start")
    out = ta.triangle_attn_attend(ws, wd, I, I, torch.bfloat16, variant="start")
    torch.cuda.synchronize()
    zd = oaq.decode(rec, "A").reshape(I, I, 128)
    p = params64(w)
    lines, qs = [0, 511, I - 1], np.r_[0:32, I - 32:I]
    bias_q = ref.pair_bias(zd[qs].astype(np.float64), p)
    want = ref.triangle_attn_rows_queries(zd[lines].astype(np.float64), bias_q, qs, p)
    js = torch.as_tensor(qs, dtype=torch.long)
    check(out[lines][:, js].cpu(), want, "bf16", "I=1024 group A sampled")
