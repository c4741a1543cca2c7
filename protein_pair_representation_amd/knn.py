"""Python binding of the kNN sparse atom-pair encoder in libtriattn.so (ctypes):
argument marshalling only.

Low-memory pair encoding (Design-CP summary, implementation details): atom-pair
features are built only at each atom's k nearest neighbours.  The functions
carry the names of the C entry points they call; the kernels do all of the work.
"""
from __future__ import annotations

import ctypes

import torch

from . import triattn as _ta

SINGLE_CHANNELS = 128
PAIR_CHANNELS = 16
MAX_K = 64


def knn_workspace_bytes(L: int) -> int:
    n = ctypes.c_size_t(0)
    _ta._check(_ta.load_library().knn_workspace_bytes(L, ctypes.byref(n)))
    return n.value


def knn_pair_encode(x: torch.Tensor, s: torch.Tensor, k: int, w_l: torch.Tensor, w_m: torch.Tensor,
                    w_d: torch.Tensor, nbr: torch.Tensor | None = None, pair: torch.Tensor | None = None,
                    ws: torch.Tensor | None = None, stream=None) -> tuple[torch.Tensor, torch.Tensor]:
    """(nbr int32 [L, k], pair bf16 [L, k, 16]) of the atoms x fp32 [L, 3] with single
    features s bf16 [L, 128]; weights w_l, w_m bf16 [16, 128], w_d fp32 [16, 4] (GPU)."""
    _ta._dev(x, "x", torch.float32)
    _ta._dev(s, "s", torch.bfloat16)
    for t, n, dt, shape in ((w_l, "w_l", torch.bfloat16, (PAIR_CHANNELS, SINGLE_CHANNELS)),
                            (w_m, "w_m", torch.bfloat16, (PAIR_CHANNELS, SINGLE_CHANNELS)),
                            (w_d, "w_d", torch.float32, (PAIR_CHANNELS, 4))):
        _ta._dev(t, n, dt)
        if tuple(t.shape) != shape:
            raise ValueError(f"{n} must have shape {shape}")
    L = x.shape[0]
    if tuple(x.shape) != (L, 3) or tuple(s.shape) != (L, SINGLE_CHANNELS):
        raise ValueError("x must be [L, 3] and s [L, 128]")
    if nbr is None:
        nbr = torch.empty((L, k), dtype=torch.int32, device=x.device)
    if pair is None:
        pair = torch.empty((L, k, PAIR_CHANNELS), dtype=torch.bfloat16, device=x.device)
    if ws is None:
        ws = torch.empty(max(knn_workspace_bytes(L), 1), dtype=torch.uint8, device=x.device)
    _ta._dev(nbr, "nbr", torch.int32)
    _ta._dev(pair, "pair", torch.bfloat16)
    _ta._dev(ws, "ws", torch.uint8)
    if nbr.numel() != L * k or pair.numel() != L * k * PAIR_CHANNELS:
        raise ValueError(f"nbr must hold {L} x {k} and pair {L} x {k} x {PAIR_CHANNELS} values")
    _ta._check(_ta.load_library().knn_pair_encode(
        _ta._ptr(x), _ta._ptr(s), L, k, _ta._ptr(w_l), _ta._ptr(w_m), _ta._ptr(w_d), _ta._ptr(nbr),
        _ta._ptr(pair), _ta._ptr(ws), ws.numel(), _ta._stream(stream)))
    return nbr, pair
