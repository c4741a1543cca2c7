"""GPU parity: the HIP library (through the C ABI) against the float64 oracle.

Tolerances (compared element by element on the stored outputs, upcast exactly):
  bf16 inputs, fp32 accumulation: max |gpu - ref| <= 2e-2 and
                                  sum |gpu - ref| / sum |ref| <= 5e-3
  fp32:                           max |gpu - ref| <= 1e-5
Small and ragged sizes are compared on every output, and so is the I = 1024
workload (both variants, over a process pool).  The I = 2048 and the row-block
I = 4096 workloads are compared on ten and eight whole lines (every query block),
with every output checked to be written and finite; with TRIATTN_FULL_PARITY=1
they are also compared on every output.
"""
import os

import numpy as np
import pytest
import torch

import oracle_pool
from oracle import ref
from protein_pair_representation_amd import inputs
from protein_pair_representation_amd import triattn as ta

pytestmark = pytest.mark.gpu

BF16_MAX_ABS, BF16_REL_L1, F32_MAX_ABS = 2e-2, 5e-3, 1e-5
TDT = {"bf16": torch.bfloat16, "f32": torch.float32}


def say(msg):
    print(msg, flush=True)


def check(gpu, want, dtype, what=""):
    got = inputs.to_f64(gpu)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - want)
    rel = err.sum() / max(np.abs(want).sum(), 1e-300)
    say(f"    {what}: max abs {err.max():.3e}, rel L1 {rel:.3e}")
    if dtype == "f32":
        assert err.max() <= F32_MAX_ABS, f"{what}: max abs {err.max():.3e}"
    else:
        assert err.max() <= BF16_MAX_ABS and rel <= BF16_REL_L1, f"{what}: max abs {err.max():.3e}, rel L1 {rel:.3e}"
    return float(err.max())


def weights_with_extras(seed, dtype, extras=True):
    """Seeded weights; with extras the LayerNorm affine and both biases are non-trivial."""
    w = inputs.make_weights(seed, dtype)
    if extras:
        g = torch.Generator().manual_seed(seed)
        w["ln_gamma"] = 1.0 + 0.2 * torch.randn(128, generator=g)
        w["ln_beta"] = 0.1 * torch.randn(128, generator=g)
        w["b_g"] = 0.5 * torch.randn(128, generator=g)
        w["b_o"] = 0.1 * torch.randn(128, generator=g)
    return w


def dev(w):
    return {k: v.cuda() for k, v in w.items()}


def params64(w):
    return ref.params(inputs.weights_f64(w), 4, 32, 1e-5)


def guarded(shape, dtype, margin=4096):
    """A tensor with guard bands on both sides, filled with a sentinel; returns (buffer, view)."""
    n = int(np.prod(shape))
    buf = torch.full((n + 2 * margin,), 7.0, dtype=dtype, device="cuda")
    return buf, buf[margin:margin + n].view(shape)


def guards_intact(buf, margin=4096):
    return bool(torch.all(buf[:margin] == 7.0)) and bool(torch.all(buf[-margin:] == 7.0))


# ------------------------------------------------------------------ small and ragged sizes, full output

SMALL = [(1, "bf16"), (5, "bf16"), (63, "bf16"), (64, "f32"), (65, "bf16"), (65, "f32"), (130, "bf16"),
         (200, "f32"), (257, "bf16")]


@pytest.mark.parametrize("I,dtype", SMALL)
@pytest.mark.parametrize("variant", ["start", "end"])
def test_small_full(I, dtype, variant):
    say(f"[parity] {variant} I={I} {dtype}")
    w = weights_with_extras(100 + I, dtype)
    z = inputs.make_z(100 + I, I, dtype)
    buf, out = guarded((I, I, 128), TDT[dtype])
    fn = ta.triangle_attn_start if variant == "start" else ta.triangle_attn_end
    fn(z.cuda(), dev(w), out=out)
    torch.cuda.synchronize()
    assert guards_intact(buf), "write outside the output"
    f = ref.triangle_attn_start if variant == "start" else ref.triangle_attn_end
    check(out, f(inputs.to_f64(z), params64(w)), dtype, f"{variant} I={I}")


@pytest.mark.parametrize("I,R,dtype", [(5, 3, "bf16"), (130, 1, "f32"), (130, 64, "bf16"), (257, 33, "bf16")])
def test_rows_given_bias(I, R, dtype):
    """Row block with a caller-supplied fp32 bias carrying large per-query offsets."""
    say(f"[parity] rows I={I} R={R} {dtype}")
    w = weights_with_extras(200 + I, dtype)
    zr = inputs.make_z_rows(200 + I, I, 7 % I, R, dtype)
    offs = np.linspace(-30, 30, I)
    bias = inputs.random_bias(I, 4, I, scale=2.0, offset_per_query=offs)
    buf, out = guarded((R, I, 128), TDT[dtype])
    ta.triangle_attn_start_rows(zr.cuda(), bias.cuda(), dev(w), out=out)
    torch.cuda.synchronize()
    assert guards_intact(buf)
    check(out, ref.triangle_attn_rows(inputs.to_f64(zr), inputs.to_f64(bias), params64(w)), dtype, "rows")


@pytest.mark.parametrize("I,R,row0,dtype", [(5, 2, 3, "bf16"), (130, 40, 17, "bf16"), (200, 200, 0, "f32")])
def test_pair_bias(I, R, row0, dtype):
    say(f"[parity] pair_bias I={I} R={R} row0={row0} {dtype}")
    w = weights_with_extras(300 + I, dtype)
    zr = inputs.make_z_rows(300 + I, I, row0, R, dtype)
    bbuf = torch.full((4 * I * I + 2 * 4096,), 7.0, dtype=torch.float32, device="cuda")
    bias = bbuf[4096:4096 + 4 * I * I].view(4, I, I)
    ta.triangle_attn_pair_bias(zr.cuda(), dev(w), row0=row0, bias=bias)
    torch.cuda.synchronize()
    assert guards_intact(bbuf)
    got = inputs.to_f64(bias)
    want = ref.pair_bias(inputs.to_f64(zr), params64(w))
    # bf16: LayerNorm output is rounded to bf16 before the projection
    tol = 1e-5 if dtype == "f32" else 2e-2
    assert np.abs(got[:, row0:row0 + R] - want).max() <= tol
    untouched = np.ones(I, bool)
    untouched[row0:row0 + R] = False
    assert np.all(got[:, untouched] == 7.0)


# ------------------------------------------------------------------ invariants on the GPU

def test_end_is_transposed_start_bitwise():
    say("[invariant] end(Z) == start(Z^T)^T")
    w = dev(weights_with_extras(5, "bf16"))
    z = inputs.make_z(5, 190, "bf16").cuda()
    a = ta.triangle_attn_end(z, w)
    b = ta.triangle_attn_start(z.transpose(0, 1).contiguous(), w).transpose(0, 1)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_rows_equal_start_rows_bitwise():
    say("[invariant] rows == rows of start")
    w = dev(weights_with_extras(6, "bf16"))
    I = 300
    z = inputs.make_z(6, I, "bf16").cuda()
    full = ta.triangle_attn_start(z, w)
    bias = torch.empty((4, I, I), dtype=torch.float32, device="cuda")
    for r0 in range(0, I, 128):  # bias assembled from row blocks, as a 1D-sharded run would
        ta.triangle_attn_pair_bias(z[r0:r0 + 128], w, row0=r0, bias=bias)
    part = ta.triangle_attn_start_rows(z[100:217].contiguous(), bias, w)
    torch.cuda.synchronize()
    assert torch.equal(part, full[100:217])


def test_repeatable_bitwise():
    say("[invariant] repeatability")
    w = dev(weights_with_extras(7, "bf16"))
    z = inputs.make_z(7, 333, "bf16").cuda()
    a = ta.triangle_attn_start(z, w)
    b = ta.triangle_attn_start(z, w)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ------------------------------------------------------------------ heads that need a softmax shift
# One-pass attention first runs every head without a shift (scores used as
# base-2 exponents directly); a workgroup (2 lines x 128 queries) runs again with
# the lazily introduced shift when one of its heads has a first key tile whose
# maximum lies more than 64 (base 2) from 0, or a row sum past 2^64.  These cases
# force that second run, for a few workgroups or for the whole grid.

@pytest.mark.parametrize("I,R,dtype,qsel", [(130, 8, "bf16", None), (257, 5, "bf16", (32, 64)),
                                             (200, 4, "f32", None), (257, 3, "f32", (200, 232)),
                                             (1024, 6, "bf16", None), (1024, 6, "bf16", (512, 544))])
def test_first_key_tile_far_below(I, R, dtype, qsel):
    """Keys 0..63 (the first key tile) carry a bias 60 below N(0, 1) for all
    queries, or for one 32-query block only (then one wave of the workgroup asks
    for the shifted form and the whole workgroup takes it)."""
    say(f"[parity] shift: first key tile far below, I={I} R={R} {dtype} queries={qsel}")
    w = weights_with_extras(400 + I, dtype)
    zr = inputs.make_z_rows(400 + I, I, 0, R, dtype)
    bias = inputs.random_bias(400 + I, 4, I)
    q = slice(None) if qsel is None else slice(*qsel)
    bias[:, q, :64] -= 60.0
    out = ta.triangle_attn_start_rows(zr.cuda(), bias.cuda(), dev(w))
    torch.cuda.synchronize()
    check(out, ref.triangle_attn_rows(inputs.to_f64(zr), inputs.to_f64(bias), params64(w)), dtype,
          "first tile far below")


def test_shift_flags_do_not_carry_over():
    """One workspace for three row-block calls: a bias that needs the shifted form
    in some workgroups, then an ordinary one, then the first again.  Each call
    sets every workgroup's flag afresh, so each result matches its own oracle."""
    I, R = 257, 6
    say(f"[parity] shift flags over reused workspace I={I} R={R}")
    w = weights_with_extras(450, "bf16")
    zr = inputs.make_z_rows(450, I, 0, R, "bf16")
    plain = inputs.random_bias(451, 4, I)
    far = plain.clone()
    far[:, 100:180, :64] -= 60.0
    ws = ta.workspace(I, R, torch.bfloat16, "rows")
    want = {}
    for name, b in (("far", far), ("plain", plain), ("far again", far)):
        out = ta.triangle_attn_start_rows(zr.cuda(), b.cuda(), dev(w), ws=ws)
        torch.cuda.synchronize()
        key = "far" if name.startswith("far") else "plain"
        if key not in want:
            want[key] = ref.triangle_attn_rows(inputs.to_f64(zr), inputs.to_f64(b), params64(w))
        check(out, want[key], "bf16", name)


def test_large_logits_f32():
    """W_q and W_k scaled by 6: logits with a standard deviation of ~50 (base 2),
    so first key tiles reach past 64 and row sums past 2^64 (exp2 itself would
    overflow fp32 past 128).  The bar is looser than the fp32 one: the scores are
    accumulated in fp32 from terms up to ~40 in size, so they carry errors up to
    ~1e-4 (natural-log units); a perturbation ds of the scores moves a softmax
    average of v by at most 2 max|ds| max|v| (|v| < 8 here), and the output
    projection does not amplify it beyond 2e-3."""
    I = 200
    say(f"[parity] shift: large logits I={I} f32")
    w = weights_with_extras(500, "f32")
    w["w_q"] = w["w_q"] * 6.0
    w["w_k"] = w["w_k"] * 6.0
    z = inputs.make_z(500, I, "f32")
    out = ta.triangle_attn_start(z.cuda(), dev(w))
    torch.cuda.synchronize()
    got = inputs.to_f64(out)
    want = ref.triangle_attn_start(inputs.to_f64(z), params64(w))
    assert np.all(np.isfinite(got))
    err = np.abs(got - want).max()
    say(f"    large logits: max abs {err:.3e}")
    assert err <= 2e-3


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero_gate(dtype):
    say(f"[invariant] zero gate {dtype}")
    w = weights_with_extras(8, dtype)
    w["w_g"] = torch.zeros_like(w["w_g"])
    w["b_g"] = torch.full((128,), -1e4)
    w["b_o"] = torch.arange(128, dtype=torch.float32) / 8 - 8   # exact in bf16
    z = inputs.make_z(8, 77, dtype).cuda()
    out = ta.triangle_attn_start(z, dev(w))
    torch.cuda.synchronize()
    want = w["b_o"].to(TDT[dtype]).cuda().expand(77, 77, 128)
    assert torch.equal(out, want)


def test_output_may_alias_input():
    say("[invariant] out == z")
    w = dev(weights_with_extras(9, "bf16"))
    z = inputs.make_z(9, 100, "bf16").cuda()
    want = ta.triangle_attn_start(z, w)
    z2 = z.clone()
    ta.triangle_attn_start(z2, w, out=z2)
    torch.cuda.synchronize()
    assert torch.equal(z2, want)


def test_stream_argument():
    say("[invariant] side stream")
    w = dev(weights_with_extras(10, "bf16"))
    z = inputs.make_z(10, 129, "bf16").cuda()
    want = ta.triangle_attn_start(z, w)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        got = ta.triangle_attn_start(z, w, stream=s)
    s.synchronize()
    assert torch.equal(got, want)


# ------------------------------------------------------------------ stage 1 against oracle intermediates

def untile_bias(raw, P):
    """[H][P][P] from the workspace's tiled bias layout (documented in include/triattn.h)."""
    t = raw.reshape(4, P // 32, P // 64, 2, 2, 32, 16)       # h, jb, kb, st, hh, jj, i
    t = t.transpose(0, 1, 5, 2, 3, 4, 6)                      # h, jb, jj, kb, st, hh, i
    return t.reshape(4, P, P)


@pytest.mark.parametrize("variant,dtype", [("start", "bf16"), ("end", "bf16"), ("start", "f32")])
def test_projection_stage(variant, dtype):
    say(f"[stage] project {variant} {dtype}")
    I = 70
    w = weights_with_extras(11, dtype)
    z = inputs.make_z(11, I, dtype)
    ws = ta.triangle_attn_project(z.cuda(), dev(w), variant=variant)
    torch.cuda.synchronize()
    v = {k: inputs.to_f64(t) for k, t in ta.workspace_views(ws, I, I, TDT[dtype], variant).items()}
    z64 = inputs.to_f64(z)
    if variant == "end":
        z64 = np.transpose(z64, (1, 0, 2))  # line = column of Z
    q, k, vv, g, b = ref.project(z64, params64(w))   # [L][P][H][d], bias [L][P][H]
    tol = 1e-5 if dtype == "f32" else 3e-2
    log2e = 1.0 / np.log(2.0)
    assert np.abs(v["q"][:, :, :I].transpose(0, 2, 1, 3) - q * log2e / np.sqrt(32)).max() <= tol
    assert np.abs(v["k"][:, :, :I].transpose(0, 2, 1, 3) - k).max() <= tol
    assert np.abs(v["vt"][:, :, :, :I].transpose(0, 3, 1, 2) - vv).max() <= tol
    assert np.abs(v["g"][:, :, :I].transpose(0, 2, 1, 3) - g).max() <= tol
    # bias[h][line][pos] = log2(e) b(token at (line, pos)); for end this is the transposed bias
    # K1's fp32 bias: bias_f32[h][line][pos] = b(token at (line, pos)) (end: transposed bias)
    bt = np.transpose(b, (2, 0, 1))
    assert np.abs(v["bias_f32"] - bt).max() <= (1e-5 if dtype == "f32" else 2e-2)
    # packed bias: per query row shifted by its maximum, base 2, compute dtype, tiled
    lay = ta.triangle_attn_workspace_layout(I, I, TDT[dtype], variant)
    packed = untile_bias(v["bias_tiles"], lay.positions)
    f32b = v["bias_f32"]
    want = (f32b - f32b.max(axis=2, keepdims=True)) * log2e
    rel = 1e-6 if dtype == "f32" else 2.0 ** -10  # fp16: round to nearest of 11 significant bits
    assert np.all(np.abs(packed[:, :I, :I] - want) <= rel * np.abs(want) + 1e-5)
    assert np.all(packed[:, :(I + 31) // 32 * 32, I:] <= -29000.0)
    assert np.all(np.isfinite(packed[:, I:(I + 31) // 32 * 32, :I]))
    assert np.all(np.isfinite(v["q"])) and np.all(np.isfinite(v["vt"]))


# ------------------------------------------------------------------ the five workloads

def _workload(name):
    w = inputs.WORKLOADS[name]
    return w, inputs.workload_weights(w)


@pytest.mark.parametrize("name", ["start-f32-I64", "start-bf16-I384"])
def test_workload_full(name):
    say(f"[workload] {name} full")
    wl, w = _workload(name)
    z = inputs.workload_z(wl)
    out = ta.triangle_attn_start(z.cuda(), dev(w))
    torch.cuda.synchronize()
    check(out, ref.triangle_attn_start(inputs.to_f64(z), params64(w)), wl.dtype, name)


def _nan_out(shape):
    """Output buffer filled with NaN: any token the kernels leave unwritten fails the comparison."""
    return torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")


def _check_pool(kind, z64, bias, p, got, index, expect_elems, what):
    maxabs, rel, nonfin, n = oracle_pool.compare(kind, z64, bias, p, got, index)
    say(f"    {what}: {n} outputs, max abs {maxabs:.3e}, rel L1 {rel:.3e}, non-finite {nonfin}")
    assert n == expect_elems, (n, expect_elems)
    assert nonfin == 0, f"{what}: {nonfin} non-finite outputs"
    assert maxabs <= BF16_MAX_ABS and rel <= BF16_REL_L1, f"{what}: max abs {maxabs:.3e}, rel L1 {rel:.3e}"


@pytest.mark.timeout(1500)
@pytest.mark.parametrize("variant", ["start", "end"])
def test_workload_i1024_every_token(variant):
    """The metric workload (I = 1024 with the distogram term), both variants,
    compared with the oracle on all I x I x 128 outputs."""
    name = "startend-bf16-I1024-distogram"
    say(f"[workload] {name} {variant}: every token")
    wl, w = _workload(name)
    I = wl.I
    z = inputs.workload_z(wl)
    out = _nan_out((I, I, 128))
    fn = ta.triangle_attn_start if variant == "start" else ta.triangle_attn_end
    fn(z.cuda(), dev(w), out=out)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    p = params64(w)
    z64 = inputs.to_f64(z)
    bias = ref.pair_bias(z64, p)
    _check_pool(variant, z64, bias, p, got, range(I), I * I * 128, f"{name} {variant}")


# lines of the larger workloads compared in full (every query): both lines of
# some line pairs, first and last lines, lines from both halves, and at I = 2048
# line pairs of every residue mod 4 (the XCD pair that serves a line pair)
LINES_I2048 = [0, 1, 2, 5, 510, 777, 1024, 1025, 2046, 2047]
LINES_R1024 = [0, 1, 255, 510, 511, 512, 1022, 1023]


@pytest.mark.timeout(1500)
def test_workload_i2048_outliers_lines():
    """I = 2048 with outlier channels: ten whole lines (every query block) against the oracle."""
    name = "start-bf16-I2048-outliers"
    say(f"[workload] {name}: lines {LINES_I2048}, every query")
    wl, w = _workload(name)
    I = wl.I
    z = inputs.workload_z(wl)
    out = _nan_out((I, I, 128))
    ta.triangle_attn_start(z.cuda(), dev(w), out=out)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any(), "unwritten outputs"
    got = out[LINES_I2048].float().cpu().numpy()
    p = params64(w)
    bias = ref.pair_bias(inputs.to_f64(z), p)
    z64 = inputs.to_f64(z[LINES_I2048])
    _check_pool("rows", z64, bias, p, got, range(len(LINES_I2048)), len(LINES_I2048) * I * 128, name)


@pytest.mark.timeout(1500)
def test_workload_rows_4096():
    """Row block of 1024 rows of I = 4096, bias of the whole pair tensor: eight
    whole lines (every query block) against the oracle, every output finite."""
    name = "rows-bf16-R1024-I4096"
    say(f"[workload] {name}: lines {LINES_R1024}, every query")
    wl, w = _workload(name)
    I, R = wl.I, wl.n_rows
    wd = dev(w)
    p = params64(w)
    bias = torch.empty((4, I, I), dtype=torch.float32, device="cuda")
    bias64 = np.empty((4, I, I))
    host_rows, dev_rows = [], []
    for r0 in range(0, I, 512):                                    # whole bias, built block by block
        zb = inputs.workload_z(wl, r0, 512)
        zbd = zb.cuda()
        ta.triangle_attn_pair_bias(zbd, wd, row0=r0, bias=bias)
        bias64[:, r0:r0 + 512] = ref.pair_bias(inputs.to_f64(zb), p)
        if r0 < R:
            host_rows.append(zb)
            dev_rows.append(zbd)
        say(f"  bias rows {r0}..{r0 + 511} done")
    z_rows_dev = torch.cat(dev_rows)
    out = _nan_out((R, I, 128))
    ta.triangle_attn_start_rows(z_rows_dev, bias, wd, out=out)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any(), "unwritten or non-finite outputs"
    got = out[LINES_R1024].float().cpu().numpy()
    z64 = inputs.to_f64(torch.cat(host_rows)[LINES_R1024])
    _check_pool("rows", z64, bias64, p, got, range(len(LINES_R1024)), len(LINES_R1024) * I * 128, name)


# Every output of the I = 2048 and I = 4096 row-block workloads: the oracle takes about
# 7 and 13 minutes of host time on 16 cores, so these run only when asked for
# (TRIATTN_FULL_PARITY=1); the line tests above cover every query block of both.
FULL_PARITY = os.environ.get("TRIATTN_FULL_PARITY") == "1"
full_only = pytest.mark.skipif(not FULL_PARITY, reason="every output of a large workload takes 7-13 min of "
                               "host time for the oracle: set TRIATTN_FULL_PARITY=1")


def _progress(what):
    step = {"n": 0}

    def report(done, total):
        if done * 20 >= (step["n"] + 1) * total or done == total:
            step["n"] = done * 20 // total
            say(f"    {what}: oracle {done}/{total} parts")
    return report


@full_only
@pytest.mark.timeout(1500)
def test_workload_i2048_outliers_every_token():
    """I = 2048 with outlier channels: all 2048 x 2048 x 128 outputs against the oracle."""
    name = "start-bf16-I2048-outliers"
    say(f"[workload] {name}: every token")
    wl, w = _workload(name)
    I = wl.I
    z = inputs.workload_z(wl)
    out = _nan_out((I, I, 128))
    ta.triangle_attn_start(z.cuda(), dev(w), out=out)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    del out
    p = params64(w)
    z64 = inputs.to_f64(z)
    bias = ref.pair_bias(z64, p)
    maxabs, rel, nonfin, n = oracle_pool.compare("start", z64, bias, p, got, range(I), chunk=4,
                                                 progress=_progress(name))
    say(f"    {name}: {n} outputs, max abs {maxabs:.3e}, rel L1 {rel:.3e}, non-finite {nonfin}")
    assert n == I * I * 128 and nonfin == 0
    assert maxabs <= BF16_MAX_ABS and rel <= BF16_REL_L1, f"{name}: max abs {maxabs:.3e}, rel L1 {rel:.3e}"


@full_only
@pytest.mark.timeout(1500)
def test_workload_rows_4096_every_token():
    """Row block of 1024 rows of I = 4096: all 1024 x 4096 x 128 outputs against the oracle."""
    name = "rows-bf16-R1024-I4096"
    say(f"[workload] {name}: every token")
    wl, w = _workload(name)
    I, R = wl.I, wl.n_rows
    wd = dev(w)
    p = params64(w)
    bias = torch.empty((4, I, I), dtype=torch.float32, device="cuda")
    bias64 = np.empty((4, I, I))
    host_rows, dev_rows = [], []
    for r0 in range(0, I, 512):
        zb = inputs.workload_z(wl, r0, 512)
        zbd = zb.cuda()
        ta.triangle_attn_pair_bias(zbd, wd, row0=r0, bias=bias)
        bias64[:, r0:r0 + 512] = ref.pair_bias(inputs.to_f64(zb), p)
        if r0 < R:
            host_rows.append(zb)
            dev_rows.append(zbd)
        say(f"  bias rows {r0}..{r0 + 511} done")
    out = _nan_out((R, I, 128))
    ta.triangle_attn_start_rows(torch.cat(dev_rows), bias, wd, out=out)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    del out, bias, dev_rows
    z64 = inputs.to_f64(torch.cat(host_rows))
    maxabs, rel, nonfin, n = oracle_pool.compare("rows", z64, bias64, p, got, range(R), chunk=2,
                                                 progress=_progress(name))
    say(f"    {name}: {n} outputs, max abs {maxabs:.3e}, rel L1 {rel:.3e}, non-finite {nonfin}")
    assert n == R * I * 128 and nonfin == 0
    assert maxabs <= BF16_MAX_ABS and rel <= BF16_REL_L1, f"{name}: max abs {maxabs:.3e}, rel L1 {rel:.3e}"


def test_small_bf16_i48_seed11():
    """Regression: I = 48, bf16, seed 11 (weights and pair tensor), starting node, in
    full.  Before the LayerNorm output entered the projections as two bf16 parts
    this case sat at relative L1 5.001e-3, just over the bar."""
    say("[parity] start I=48 bf16 seed 11")
    w = inputs.make_weights(11, "bf16")
    z = inputs.make_z(11, 48, "bf16")
    out = ta.triangle_attn_start(z.cuda(), dev(w))
    torch.cuda.synchronize()
    check(out, ref.triangle_attn_start(inputs.to_f64(z), params64(w)), "bf16", "start I=48 seed 11")
