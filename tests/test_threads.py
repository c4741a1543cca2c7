"""Concurrent callers: host threads, each with its own stream and workspace, call
the library at the same time (ctypes releases the GIL during a foreign call, so
the library's host code runs concurrently) and get bit for bit what one caller
gets alone."""
import threading

import pytest
import torch

from protein_pair_representation_amd import inputs
from protein_pair_representation_amd import triattn as ta

from test_parity import TDT, dev, say, weights_with_extras

pytestmark = pytest.mark.gpu

THREADS, ROUNDS = 4, 5


def test_threads_on_their_own_streams():
    say(f"[threads] {THREADS} threads x {ROUNDS} rounds, start and end, bf16 and fp32")
    cases = [(130, "bf16", "start"), (96, "f32", "end"), (257, "bf16", "end"), (64, "f32", "start")]
    work = []
    for n, (I, dtype, variant) in enumerate(cases):
        w = dev(weights_with_extras(970 + n, dtype))
        z = inputs.make_z(970 + n, I, dtype).cuda()
        fn = ta.triangle_attn_start if variant == "start" else ta.triangle_attn_end
        want = fn(z, w)
        work.append((fn, z, w, want, I, dtype, variant))
    torch.cuda.synchronize()
    errors = []
    barrier = threading.Barrier(THREADS)

    def run(t):
        try:
            fn, z, w, want, I, dtype, variant = work[t % len(work)]
            stream = torch.cuda.Stream()
            ws = ta.workspace(I, I, TDT[dtype], variant)
            out = torch.empty_like(want)
            barrier.wait()
            for r in range(ROUNDS):
                with torch.cuda.stream(stream):
                    out.fill_(float("nan"))
                    fn(z, w, out=out, ws=ws, stream=stream)
                stream.synchronize()
                if not torch.equal(out, want):
                    errors.append(f"thread {t} round {r}: differs from the single caller's result")
        except Exception as e:  # reported below
            errors.append(f"thread {t}: {e!r}")

    threads = [threading.Thread(target=run, args=(t,)) for t in range(THREADS)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
