"""triangle_attn_start_noalloc: the allocation-free entry point, through the C ABI.

Its output must equal triangle_attn_start's on the same inputs (same kernels on a
static workspace instead of a caller's), on two calls in a row, the second on a
smaller problem (the static array keeps the first call's contents), and both must
meet the bar against the oracle.  A problem larger than the static workspace is
rejected before anything is enqueued.
"""
import numpy as np
import pytest
import torch

from oracle import ref
from protein_pair_representation_amd import inputs
from protein_pair_representation_amd import triattn as ta

from test_parity import TDT, check, dev, guarded, guards_intact, params64, say, weights_with_extras

pytestmark = pytest.mark.gpu


def test_noalloc_matches_start_twice():
    for I, dtype in ((200, "bf16"), (77, "bf16"), (130, "f32"), (64, "f32")):
        say(f"[no-alloc] start I={I} {dtype}")
        w = dev(weights_with_extras(900 + I, dtype))
        z = inputs.make_z(900 + I, I, dtype)
        zd = z.cuda()
        want = ta.triangle_attn_start(zd, w)
        buf, out = guarded((I, I, 128), TDT[dtype])
        ta.triangle_attn_start_noalloc(zd, w, out=out)
        torch.cuda.synchronize()
        assert guards_intact(buf), "write outside the output"
        assert torch.equal(out, want), "static-workspace result differs from triangle_attn_start"
        check(out, ref.triangle_attn_start(inputs.to_f64(z), params64({k: v.cpu() for k, v in w.items()})), dtype,
              f"no-alloc I={I}")


def test_noalloc_side_stream():
    I = 150
    say(f"[no-alloc] start I={I} bf16 on a side stream")
    w = dev(weights_with_extras(950, "bf16"))
    z = inputs.make_z(950, I, "bf16").cuda()
    want = ta.triangle_attn_start(z, w)
    out = torch.empty_like(z)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ta.triangle_attn_start_noalloc(z, w, out=out, stream=s)
    s.synchronize()
    assert torch.equal(out, want)


def test_noalloc_rejects_too_large():
    I = 512                                        # workspace ~ 340 MB > 256 MiB
    say(f"[no-alloc] I={I} rejected")
    w = dev(weights_with_extras(960, "bf16"))
    z = torch.zeros((I, I, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(z, 7.0)
    with pytest.raises(ta.TriAttnError) as e:
        ta.triangle_attn_start_noalloc(z, w, out=out)
    assert e.value.code == -12
    torch.cuda.synchronize()
    assert bool(torch.all(out == 7.0)), "out touched by a rejected call"
