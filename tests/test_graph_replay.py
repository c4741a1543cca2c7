"""The entry points under stream capture: captured once into a graph with
torch.cuda.graph and replayed, they give bit for bit the eager result.

The library only enqueues kernels on the stream it is given (no allocation, no
memset, no synchronisation), so a caller may capture it.  Each replay runs after
other eager work and a synchronisation, into an output first filled with NaN,
and is compared with the eager call on the same inputs and workspace.
"""
import pytest
import torch

from protein_pair_representation_amd import inputs
from protein_pair_representation_amd import triattn as ta

from test_parity import TDT, dev, say, weights_with_extras

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _replay_check(call, out, want, other):
    """Capture call() (which writes `out`) into a graph and replay it REPLAYS times."""
    side = torch.cuda.Stream()                     # warm-up outside the capture, as torch asks
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(REPLAYS):
        out.fill_(float("nan"))
        other()                                    # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {rep} differs from the eager result"


@pytest.mark.parametrize("I,dtype,variant", [(64, "f32", "start"), (130, "bf16", "end"), (384, "bf16", "start")])
def test_full_variant_replays(I, dtype, variant):
    say(f"[graph] {variant} I={I} {dtype}")
    w = dev(weights_with_extras(950 + I, dtype))
    z = inputs.make_z(950 + I, I, dtype).cuda()
    fn = ta.triangle_attn_start if variant == "start" else ta.triangle_attn_end
    ws = ta.workspace(I, I, TDT[dtype], variant)
    want = fn(z, w, ws=ws)
    torch.cuda.synchronize()
    out = torch.empty_like(want)
    z2 = inputs.make_z(951 + I, I, dtype).cuda()
    out2 = torch.empty_like(want)
    _replay_check(lambda: fn(z, w, out=out, ws=ws), out, want,
                  lambda: ta.triangle_attn_end(z2, w, out=out2))


def test_row_block_replays():
    I, R = 257, 40
    say(f"[graph] rows I={I} R={R} bf16")
    w = dev(weights_with_extras(960, "bf16"))
    zr = inputs.make_z_rows(960, I, 0, R, "bf16").cuda()
    bias = inputs.random_bias(961, 4, I).cuda()
    ws = ta.workspace(I, R, torch.bfloat16, "rows")
    want = ta.triangle_attn_start_rows(zr, bias, w, ws=ws)
    torch.cuda.synchronize()
    out = torch.empty_like(want)
    _replay_check(lambda: ta.triangle_attn_start_rows(zr, bias, w, out=out, ws=ws), out, want,
                  lambda: ta.triangle_attn_start_rows(zr, bias, w))
