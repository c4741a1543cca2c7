"""Python binding of libtriattn.so (ctypes): argument marshalling only.

Each function has the name of the C entry point it calls and takes torch
tensors on the GPU; torch provides device memory (outputs and workspaces it
allocates when the caller passes none) and the current HIP stream.  Every step
of the computation runs in the library's HIP kernels.  If the library has not
been built, loading fails loudly; there is no other code path.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

from .build import LIB_PATH, ROOT

C_Z, HEADS, HEAD_DIM = 128, 4, 32
TA_BF16, TA_F32 = 1, 2
TA_START, TA_END, TA_ROWS = 0, 1, 2
VARIANTS = {"start": TA_START, "end": TA_END, "rows": TA_ROWS}
_DTYPE_CODE = {torch.bfloat16: TA_BF16, torch.float32: TA_F32}

_WEIGHT_FIELDS = ["ln_gamma", "ln_beta", "w_q", "w_k", "w_v", "w_g", "w_b", "b_g", "w_o", "b_o"]


class TaProblem(ctypes.Structure):
    _fields_ = [("I", ctypes.c_int32), ("rows", ctypes.c_int32), ("c_z", ctypes.c_int32),
                ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("ln_eps", ctypes.c_float)]


class TaWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _WEIGHT_FIELDS]


class TaWsLayout(ctypes.Structure):
    _fields_ = [("q", ctypes.c_size_t), ("k", ctypes.c_size_t), ("vt", ctypes.c_size_t),
                ("g", ctypes.c_size_t), ("o", ctypes.c_size_t), ("bias", ctypes.c_size_t),
                ("bias_f32", ctypes.c_size_t), ("redo", ctypes.c_size_t),
                ("total", ctypes.c_size_t),
                ("lines", ctypes.c_int32), ("positions", ctypes.c_int32)]


class TriAttnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"triattn error {code}: {msg}")
        self.code = code


_lib = None


def header_functions() -> list:
    """Names of the functions include/triattn.h, aaq.h and knn.h declare."""
    names = set()
    for h in ("triattn.h", "aaq.h", "knn.h"):
        text = open(os.path.join(ROOT, "include", h)).read()
        names |= set(re.findall(r"\b((?:triangle_attn|aaq|knn)_\w+)\s*\(", text))
    return sorted(names)


def load_library(path: str | None = None) -> ctypes.CDLL:
    """The library at `path`, or the in-tree build (TRIATTN_LIB overrides it, e.g. with
    the sanitizer build of the host code); loaded once."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    default = os.environ.get("TRIATTN_LIB") or LIB_PATH
    path = path or default
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first (python -m protein_pair_representation_amd.build)")
    lib = ctypes.CDLL(path)
    P, W, L = ctypes.POINTER(TaProblem), ctypes.POINTER(TaWeights), ctypes.POINTER(TaWsLayout)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    sig = {
        "triangle_attn_abi_version": ([], i32),
        "triangle_attn_strerror": ([i32], ctypes.c_char_p),
        "triangle_attn_workspace_layout": ([P, i32, L], i32),
        "triangle_attn_start": ([P, W, vp, vp, vp, sz, vp], i32),
        "triangle_attn_start_noalloc": ([P, W, vp, vp, vp], i32),
        "triangle_attn_end": ([P, W, vp, vp, vp, sz, vp], i32),
        "triangle_attn_start_rows": ([P, W, vp, vp, vp, vp, sz, vp], i32),
        "triangle_attn_pair_bias": ([P, W, vp, ctypes.c_int32, vp, vp], i32),
        "triangle_attn_project": ([P, i32, W, vp, vp, sz, vp], i32),
        "triangle_attn_attend": ([P, i32, W, vp, vp, vp, sz, vp], i32),
        "triangle_attn_state_bytes": ([P, i32, ctypes.POINTER(sz)], i32),
        "triangle_attn_attend_block": ([P, i32, W, vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, vp, sz,
                                        vp], i32),
        "triangle_attn_attend_finalize": ([P, i32, W, vp, vp, vp, sz, vp], i32),
        "triangle_attn_attend_kv_block": ([P, i32, W, vp, vp, ctypes.c_int32, vp, ctypes.c_int32, ctypes.c_int32,
                                           vp, vp, sz, vp], i32),
        "triangle_attn_attend_kv_block_final": ([P, i32, W, vp, vp, ctypes.c_int32, vp, ctypes.c_int32,
                                                 ctypes.c_int32, vp, vp, vp, sz, vp], i32),
        "triangle_attn_project_aaq": ([P, i32, W, vp, i32, vp, sz, vp], i32),
        "aaq_record_bytes": ([i32], i32),
        "aaq_encode": ([vp, i32, ctypes.c_int64, i32, vp, vp], i32),
        "aaq_decode": ([vp, i32, ctypes.c_int64, vp, i32, vp], i32),
        "knn_workspace_bytes": ([ctypes.c_int64, ctypes.POINTER(sz)], i32),
        "knn_pair_encode": ([vp, vp, ctypes.c_int64, i32, vp, vp, vp, vp, vp, vp, sz, vp], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes, fn.restype = args, res
    if path == default:
        _lib = lib
    return lib


def _check(rc: int):
    if rc != 0:
        raise TriAttnError(rc, load_library().triangle_attn_strerror(rc).decode())


def problem(I: int, rows: int, dtype: torch.dtype, eps: float = 1e-5) -> TaProblem:
    if dtype not in _DTYPE_CODE:
        raise TypeError(f"unsupported dtype {dtype}")
    return TaProblem(I, rows, C_Z, HEADS, HEAD_DIM, _DTYPE_CODE[dtype], eps)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def weights_struct(w: dict, dtype: torch.dtype) -> TaWeights:
    """ctypes struct of device pointers from a dict of GPU tensors (b_g, b_o optional)."""
    s = TaWeights()
    for n in _WEIGHT_FIELDS:
        t = w.get(n)
        if t is None:
            if n in ("b_g", "b_o"):
                continue
            raise KeyError(f"weight {n} missing")
        _dev(t, n, torch.float32 if n in ("ln_gamma", "ln_beta", "b_g", "b_o") else dtype)
        setattr(s, n, t.data_ptr())
    return s


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def triangle_attn_workspace_layout(I: int, rows: int, dtype: torch.dtype, variant: str) -> TaWsLayout:
    lay = TaWsLayout()
    _check(load_library().triangle_attn_workspace_layout(ctypes.byref(problem(I, rows, dtype)),
                                                         VARIANTS[variant], ctypes.byref(lay)))
    return lay


def workspace(I: int, rows: int, dtype: torch.dtype, variant: str, device=None) -> torch.Tensor:
    lay = triangle_attn_workspace_layout(I, rows, dtype, variant)
    return torch.empty(lay.total, dtype=torch.uint8, device=device or "cuda")


def _full(fn_name, variant, z, weights, out, ws, stream, eps):
    _dev(z, "z")
    I = z.shape[0]
    if z.shape != (I, I, C_Z):
        raise ValueError(f"z must be [I][I][{C_Z}], got {tuple(z.shape)}")
    out = torch.empty_like(z) if out is None else _dev(out, "out", z.dtype)
    ws = workspace(I, I, z.dtype, variant, z.device) if ws is None else _dev(ws, "ws")
    fn = getattr(load_library(), fn_name)
    _check(fn(ctypes.byref(problem(I, I, z.dtype, eps)), ctypes.byref(weights_struct(weights, z.dtype)),
              _ptr(z), _ptr(out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return out


def triangle_attn_start(z, weights, out=None, ws=None, stream=None, eps=1e-5):
    """Starting-node triangle attention of z [I][I][128] (bf16 or fp32)."""
    return _full("triangle_attn_start", "start", z, weights, out, ws, stream, eps)


def triangle_attn_end(z, weights, out=None, ws=None, stream=None, eps=1e-5):
    """Ending-node triangle attention of z [I][I][128]."""
    return _full("triangle_attn_end", "end", z, weights, out, ws, stream, eps)


def triangle_attn_start_rows(z_rows, bias, weights, out=None, ws=None, stream=None, eps=1e-5):
    """Row block: z_rows [R][I][128] with the whole fp32 pair bias [4][I][I]."""
    _dev(z_rows, "z_rows")
    _dev(bias, "bias", torch.float32)
    R, I = z_rows.shape[0], z_rows.shape[1]
    if z_rows.shape != (R, I, C_Z) or bias.shape != (HEADS, I, I):
        raise ValueError("z_rows must be [R][I][128] and bias [4][I][I]")
    out = torch.empty_like(z_rows) if out is None else _dev(out, "out", z_rows.dtype)
    ws = workspace(I, R, z_rows.dtype, "rows", z_rows.device) if ws is None else _dev(ws, "ws")
    _check(load_library().triangle_attn_start_rows(
        ctypes.byref(problem(I, R, z_rows.dtype, eps)), ctypes.byref(weights_struct(weights, z_rows.dtype)),
        _ptr(z_rows), _ptr(bias), _ptr(out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return out


def triangle_attn_pair_bias(z_rows, weights, row0=0, bias=None, I=None, stream=None, eps=1e-5):
    """Writes bias[h][row0 + r][k] for the rows of z_rows into a whole fp32 [4][I][I] array."""
    _dev(z_rows, "z_rows")
    R, I_ = z_rows.shape[0], z_rows.shape[1]
    I = I_ if I is None else I
    if I != I_:
        raise ValueError("z_rows must have I columns")
    bias = torch.zeros((HEADS, I, I), dtype=torch.float32, device=z_rows.device) if bias is None \
        else _dev(bias, "bias", torch.float32)
    _check(load_library().triangle_attn_pair_bias(
        ctypes.byref(problem(I, R, z_rows.dtype, eps)), ctypes.byref(weights_struct(weights, z_rows.dtype)),
        _ptr(z_rows), int(row0), _ptr(bias), _stream(stream)))
    return bias


def triangle_attn_start_noalloc(z, weights, out, stream=None, eps=1e-5):
    """triangle_attn_start on the library's static workspace (no workspace argument;
    the caller passes the output, so nothing is allocated here either)."""
    _dev(z, "z")
    I = z.shape[0]
    if z.shape != (I, I, C_Z):
        raise ValueError(f"z must be [I][I][{C_Z}], got {tuple(z.shape)}")
    _dev(out, "out", z.dtype)
    _check(load_library().triangle_attn_start_noalloc(
        ctypes.byref(problem(I, I, z.dtype, eps)), ctypes.byref(weights_struct(weights, z.dtype)), _ptr(z),
        _ptr(out), _stream(stream)))
    return out


def triangle_attn_project(z, weights, variant="start", ws=None, stream=None, eps=1e-5):
    """Stage 1 only: LayerNorm + projections into a workspace (returned)."""
    _dev(z, "z")
    R, I = z.shape[0], z.shape[1]
    ws = workspace(I, R, z.dtype, variant, z.device) if ws is None else _dev(ws, "ws")
    _check(load_library().triangle_attn_project(
        ctypes.byref(problem(I, R, z.dtype, eps)), VARIANTS[variant],
        ctypes.byref(weights_struct(weights, z.dtype)), _ptr(z), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)))
    return ws


def triangle_attn_project_aaq(records, weights, I, rows, group, variant="start", ws=None, stream=None, eps=1e-5):
    """Stage 1 from token-wise quantized records [rows * I, record bytes] (uint8, GPU)
    of group "A", "B" or "C"; bf16 workspace (returned)."""
    _dev(records, "records", torch.uint8)
    code = {"A": 0, "B": 1, "C": 2}.get(group, group)
    ws = workspace(I, rows, torch.bfloat16, variant, records.device) if ws is None else _dev(ws, "ws")
    _check(load_library().triangle_attn_project_aaq(
        ctypes.byref(problem(I, rows, torch.bfloat16, eps)), VARIANTS[variant],
        ctypes.byref(weights_struct(weights, torch.bfloat16)), _ptr(records), int(code), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))
    return ws


def triangle_attn_attend(ws, weights, I, rows, dtype, variant="start", bias=None, out=None, stream=None,
                         eps=1e-5):
    """Stage 2 only: fused attention + gate + output projection from a filled workspace."""
    _dev(ws, "ws")
    out = torch.empty((rows, I, C_Z), dtype=dtype, device=ws.device) if out is None else _dev(out, "out", dtype)
    _check(load_library().triangle_attn_attend(
        ctypes.byref(problem(I, rows, dtype, eps)), VARIANTS[variant], ctypes.byref(weights_struct(weights, dtype)),
        _ptr(bias), _ptr(out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return out


def triangle_attn_state_bytes(I: int, rows: int, dtype: torch.dtype, variant: str) -> int:
    n = ctypes.c_size_t()
    _check(load_library().triangle_attn_state_bytes(ctypes.byref(problem(I, rows, dtype)), VARIANTS[variant],
                                                    ctypes.byref(n)))
    return n.value


def state(I: int, rows: int, dtype: torch.dtype, variant: str, device=None) -> torch.Tensor:
    """A carried softmax state buffer for triangle_attn_attend_block (uninitialised; held as
    a float32 tensor of triangle_attn_state_bytes bytes: its regions have their own dtypes,
    see state_views)."""
    n = triangle_attn_state_bytes(I, rows, dtype, variant)
    return torch.empty(n // 4, dtype=torch.float32, device=device or "cuda")


def triangle_attn_attend_block(ws, weights, I, rows, dtype, key0, nkeys, first, st, variant="start", bias=None,
                               stream=None, eps=1e-5):
    """Fold keys [key0, key0 + nkeys) into the carried state `st` (see include/triattn.h)."""
    _dev(ws, "ws")
    _dev(st, "state", torch.float32)
    _check(load_library().triangle_attn_attend_block(
        ctypes.byref(problem(I, rows, dtype, eps)), VARIANTS[variant], ctypes.byref(weights_struct(weights, dtype)),
        _ptr(bias), int(key0), int(nkeys), int(bool(first)), _ptr(st), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)))
    return st


def triangle_attn_attend_kv_block(ws, weights, I, rows, dtype, k_blk, vt_blk, bias_blk, nkeys, first, st,
                                  variant="start", stream=None, eps=1e-5):
    """Fold one caller-held key block into the carried state `st` (see include/triattn.h).

    k_blk [L][H][NB][d] and vt_blk [L][H][d][NB] in the compute dtype (NB = the block's
    padded key count), bias_blk fp32 [H][I][nkeys]."""
    _dev(ws, "ws")
    _dev(st, "state", torch.float32)
    _dev(k_blk, "k_blk", dtype)
    _dev(vt_blk, "vt_blk", dtype)
    _dev(bias_blk, "bias_blk", torch.float32)
    nb = k_blk.shape[2]
    _check(load_library().triangle_attn_attend_kv_block(
        ctypes.byref(problem(I, rows, dtype, eps)), VARIANTS[variant], ctypes.byref(weights_struct(weights, dtype)),
        _ptr(k_blk), _ptr(vt_blk), int(nb), _ptr(bias_blk), int(nkeys), int(bool(first)), _ptr(st), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))
    return st


def triangle_attn_attend_kv_block_final(ws, weights, I, rows, dtype, k_blk, vt_blk, bias_blk, nkeys, first, st,
                                        variant="start", out=None, stream=None, eps=1e-5):
    """Fold the last caller-held key block and finish the rows into `out` (see include/triattn.h)."""
    _dev(ws, "ws")
    _dev(st, "state", torch.float32)
    _dev(k_blk, "k_blk", dtype)
    _dev(vt_blk, "vt_blk", dtype)
    _dev(bias_blk, "bias_blk", torch.float32)
    out = torch.empty((rows, I, C_Z), dtype=dtype, device=ws.device) if out is None else _dev(out, "out", dtype)
    nb = k_blk.shape[2]
    _check(load_library().triangle_attn_attend_kv_block_final(
        ctypes.byref(problem(I, rows, dtype, eps)), VARIANTS[variant], ctypes.byref(weights_struct(weights, dtype)),
        _ptr(k_blk), _ptr(vt_blk), int(nb), _ptr(bias_blk), int(nkeys), int(bool(first)), _ptr(st), _ptr(out),
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return out


def triangle_attn_attend_finalize(ws, weights, I, rows, dtype, st, variant="start", out=None, stream=None,
                                  eps=1e-5):
    """o = O / l, gate and output projection of a carried state."""
    _dev(ws, "ws")
    _dev(st, "state", torch.float32)
    out = torch.empty((rows, I, C_Z), dtype=dtype, device=ws.device) if out is None else _dev(out, "out", dtype)
    _check(load_library().triangle_attn_attend_finalize(
        ctypes.byref(problem(I, rows, dtype, eps)), VARIANTS[variant], ctypes.byref(weights_struct(weights, dtype)),
        _ptr(st), _ptr(out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return out


def state_views(st: torch.Tensor, I: int, rows: int, dtype: torch.dtype, variant: str) -> dict:
    """O / l [L][H][P][d] (float16 for bf16 problems, float32 for fp32) and (m, l) [L][H][P][2]
    (float32) views of a state buffer."""
    lay = triangle_attn_workspace_layout(I, rows, dtype, variant)
    L, P = lay.lines, lay.positions
    n_o = L * HEADS * P * HEAD_DIM
    odt = torch.float16 if dtype == torch.bfloat16 else torch.float32
    o_bytes = n_o * torch.tensor([], dtype=odt).element_size()
    off_ml = ((o_bytes + 255) // 256 * 256) // 4
    return {"O": st.view(odt)[:n_o].view(L, HEADS, P, HEAD_DIM),
            "ml": st[off_ml:off_ml + L * HEADS * P * 2].view(L, HEADS, P, 2)}


def workspace_views(ws: torch.Tensor, I: int, rows: int, dtype: torch.dtype, variant: str) -> dict:
    """Typed views of the intermediates in a workspace (layouts documented in include/triattn.h)."""
    lay = triangle_attn_workspace_layout(I, rows, dtype, variant)
    L, P = lay.lines, lay.positions
    es = torch.tensor([], dtype=dtype).element_size()
    n = L * HEADS * P * HEAD_DIM

    def view(off, shape, dt, count, esz):
        return ws[off:off + count * esz].view(dt).view(shape)

    v = {
        "q": view(lay.q, (L, HEADS, P, HEAD_DIM), dtype, n, es),
        "k": view(lay.k, (L, HEADS, P, HEAD_DIM), dtype, n, es),
        "vt": view(lay.vt, (L, HEADS, HEAD_DIM, P), dtype, n, es),
        "g": view(lay.g, (L, HEADS, P, HEAD_DIM), dtype, n, es),
        "o": view(lay.o, (L, HEADS, P, HEAD_DIM), dtype, n, es),
    }
    bdt = torch.float16 if dtype == torch.bfloat16 else torch.float32   # packed bias element type
    v["bias_tiles"] = view(lay.bias, (HEADS * P * P,), bdt, HEADS * P * P, es)
    if variant != "rows":
        v["bias_f32"] = view(lay.bias_f32, (HEADS, I, I), torch.float32, HEADS * I * I, 4)
    return v
