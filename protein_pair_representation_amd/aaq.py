"""Python binding of the AAQ codec in libtriattn.so (ctypes): argument marshalling only.

Token-wise adaptive activation quantization of the pair representation
(LightNobel article, section 2.2): every 128-channel token becomes one
fixed-size record holding its INT8 / INT4 codes, its scale and zero point, and
up to five INT16 outliers.  The functions carry the names of the C entry
points they call; the kernels do all of the work.
"""
from __future__ import annotations

import ctypes

import torch

from . import triattn as _ta

GROUPS = {"A": 0, "B": 1, "C": 2}
CHANNELS = 128


def _group(g) -> int:
    code = GROUPS.get(g, g) if isinstance(g, str) else int(g)
    if code not in GROUPS.values():
        raise ValueError(f"unknown AAQ group {g!r}")
    return code


def aaq_record_bytes(group) -> int:
    rc = _ta.load_library().aaq_record_bytes(_group(group))
    _ta._check(min(rc, 0))
    return rc


def aaq_encode(x: torch.Tensor, group, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Records [n, record_bytes] (uint8) of the tokens of x [..., 128] (bf16 / fp32, GPU)."""
    _ta._dev(x, "x")
    if x.dtype not in _ta._DTYPE_CODE:
        raise TypeError(f"x must be bfloat16 or float32, got {x.dtype}")
    if x.shape[-1] != CHANNELS:
        raise ValueError(f"x must have {CHANNELS} channels in its last axis")
    n = x.numel() // CHANNELS
    rb = aaq_record_bytes(group)
    if out is None:
        out = torch.empty((n, rb), dtype=torch.uint8, device=x.device)
    _ta._dev(out, "out", torch.uint8)
    if out.numel() != n * rb:
        raise ValueError(f"out must hold {n} x {rb} bytes")
    _ta._check(_ta.load_library().aaq_encode(_ta._ptr(x), _ta._DTYPE_CODE[x.dtype], n, _group(group),
                                               _ta._ptr(out), _ta._stream(stream)))
    return out


def aaq_decode(records: torch.Tensor, group, dtype: torch.dtype = torch.bfloat16,
               out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Tokens [n, 128] (dtype) decoded from records [n, record_bytes] (uint8, GPU)."""
    _ta._dev(records, "records", torch.uint8)
    rb = aaq_record_bytes(group)
    if records.numel() % rb:
        raise ValueError(f"records must be a whole number of {rb}-byte records")
    n = records.numel() // rb
    if dtype not in _ta._DTYPE_CODE:
        raise TypeError(f"dtype must be bfloat16 or float32, got {dtype}")
    if out is None:
        out = torch.empty((n, CHANNELS), dtype=dtype, device=records.device)
    _ta._dev(out, "out", dtype)
    if out.numel() != n * CHANNELS:
        raise ValueError(f"out must hold {n} x {CHANNELS} values")
    _ta._check(_ta.load_library().aaq_decode(_ta._ptr(records), _group(group), n, _ta._ptr(out),
                                               _ta._DTYPE_CODE[dtype], _ta._stream(stream)))
    return out
