"""The C ABI on the host: the library loads, exports what the header declares,
and rejects every bad argument before anything touches the device.

Pointers here are fake device addresses: every case fails validation, which
never dereferences a pointer and makes no HIP call, so this runs without a GPU.
"""
import ctypes
import os

import pytest
import torch

from protein_pair_representation_amd import triattn as ta

A = 0x7F0000000000  # a 256-byte aligned fake device address
MB = 1 << 20


@pytest.fixture(scope="module")
def lib():
    return ta.load_library()


def prob(I=64, rows=None, dtype=ta.TA_BF16, c_z=128, heads=4, hd=32, eps=1e-5):
    return ta.TaProblem(I, I if rows is None else rows, c_z, heads, hd, dtype, eps)


def weights(base=A + 900 * MB, **over):
    w = ta.TaWeights()
    for n_, name in enumerate(ta._WEIGHT_FIELDS):
        setattr(w, name, base + n_ * MB)
    for k, v in over.items():
        setattr(w, k, v)
    return w


def layout(lib, p, variant):
    lay = ta.TaWsLayout()
    rc = lib.triangle_attn_workspace_layout(ctypes.byref(p), variant, ctypes.byref(lay))
    return rc, lay


def test_exports_match_header(lib):
    names = ta.header_functions()
    assert len(names) == 21
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_strerror(lib):
    assert lib.triangle_attn_abi_version() == 7
    for code in range(0, -13, -1):
        msg = lib.triangle_attn_strerror(code).decode()
        assert msg and msg != "unknown error code"
    assert lib.triangle_attn_strerror(-99).decode() == "unknown error code"


@pytest.mark.parametrize("p,variant,code", [
    (None, ta.TA_START, -1),
    (prob(dtype=3), ta.TA_START, -4),
    (prob(c_z=64), ta.TA_START, -3),
    (prob(heads=8), ta.TA_START, -3),
    (prob(hd=16), ta.TA_START, -3),
    (prob(I=0), ta.TA_START, -2),
    (prob(I=70000), ta.TA_START, -2),
    (prob(I=64, rows=32), ta.TA_START, -2),
    (prob(I=64, rows=32), ta.TA_END, -2),
    (prob(I=64, rows=65), ta.TA_ROWS, -2),
    (prob(I=64, rows=0), ta.TA_ROWS, -2),
    (prob(eps=0.0), ta.TA_START, -10),
    (prob(eps=float("nan")), ta.TA_START, -10),
    (prob(), 7, -9),
])
def test_layout_rejects(lib, p, variant, code):
    lay = ta.TaWsLayout()
    rc = lib.triangle_attn_workspace_layout(None if p is None else ctypes.byref(p), variant, ctypes.byref(lay))
    assert rc == code


@pytest.mark.parametrize("I,rows,variant,dtype", [
    (64, 64, ta.TA_START, ta.TA_F32), (384, 384, ta.TA_START, ta.TA_BF16), (1000, 1000, ta.TA_END, ta.TA_BF16),
    (4096, 1024, ta.TA_ROWS, ta.TA_BF16), (5, 3, ta.TA_ROWS, ta.TA_F32), (1, 1, ta.TA_START, ta.TA_BF16)])
def test_layout_sizes(lib, I, rows, variant, dtype):
    rc, lay = layout(lib, prob(I, rows, dtype), variant)
    assert rc == 0
    es = 2 if dtype == ta.TA_BF16 else 4
    P = (I + 255) // 256 * 256
    region = lines = rows if variant == ta.TA_ROWS else I
    region = (lines * 4 * P * 32 * es + 255) // 256 * 256
    assert lay.lines == lines and lay.positions == P
    assert (lay.q, lay.k, lay.vt, lay.g, lay.o) == (0, region, 2 * region, 3 * region, 4 * region)
    assert lay.bias == 5 * region
    packed = (4 * P * P * es + 255) // 256 * 256
    if variant == ta.TA_ROWS:
        assert lay.bias_f32 == ctypes.c_size_t(-1).value and lay.redo == 5 * region + packed
    else:
        assert lay.bias_f32 == 5 * region + packed
        assert lay.redo == lay.bias_f32 + (4 * I * I * 4 + 255) // 256 * 256
    # one int32 flag per attention workgroup of 2 lines x 128 queries
    assert lay.total == lay.redo + (((lines + 1) // 2) * ((I + 127) // 128) * 4 + 255) // 256 * 256


def _start(lib, p=None, w="default", z=A, out=A + 100 * MB, ws=A + 200 * MB, ws_bytes=1 << 40, fn="start"):
    p = prob() if p is None else p
    w = weights() if w == "default" else w
    f = getattr(lib, "triangle_attn_" + fn)
    return f(ctypes.byref(p), None if w is None else ctypes.byref(w), z, out, ws, ws_bytes, None)


@pytest.mark.parametrize("fn", ["start", "end"])
def test_start_end_reject(lib, fn):
    assert _start(lib, w=None, fn=fn) == -1
    assert _start(lib, w=weights(w_q=None), fn=fn) == -1
    assert _start(lib, w=weights(ln_gamma=None), fn=fn) == -1
    assert _start(lib, z=None, fn=fn) == -1
    assert _start(lib, out=None, fn=fn) == -1
    assert _start(lib, ws=None, fn=fn) == -1
    assert _start(lib, z=A + 8, fn=fn) == -6
    assert _start(lib, out=A + 4, fn=fn) == -6
    assert _start(lib, w=weights(w_o=A + 900 * MB + 8), fn=fn) == -6
    assert _start(lib, w=weights(b_g=A + 900 * MB + 2), fn=fn) == -6
    rc, lay = layout(lib, prob(), ta.TA_START)
    assert _start(lib, ws_bytes=lay.total - 1, fn=fn) == -5
    # out overlapping the workspace, or partially overlapping z
    assert _start(lib, out=A + 200 * MB + 4096, fn=fn) == -7
    assert _start(lib, out=A + 256, fn=fn) == -7
    # out overlapping a weight
    assert _start(lib, out=A + 900 * MB, fn=fn) == -7
    # workspace overlapping z
    assert _start(lib, ws=A + 1024, fn=fn) == -7
    assert _start(lib, p=prob(dtype=0), fn=fn) == -4


def test_rows_reject(lib):
    p = prob(I=64, rows=16)
    w = weights()
    f = lib.triangle_attn_start_rows
    call = lambda bias=A + 300 * MB, z=A, out=A + 100 * MB, ws=A + 200 * MB: f(
        ctypes.byref(p), ctypes.byref(w), z, bias, out, ws, 1 << 40, None)
    assert call(bias=None) == -1
    assert call(bias=A + 300 * MB + 4) == -6
    assert call(out=A + 300 * MB) == -7          # out on the bias
    assert call(ws=A + 300 * MB) == -7           # workspace on the bias
    q = prob(I=64, rows=65)
    assert f(ctypes.byref(q), ctypes.byref(w), A, A + 300 * MB, A + 100 * MB, A + 200 * MB, 1 << 40, None) == -2


def test_pair_bias_reject(lib):
    w = weights()
    f = lib.triangle_attn_pair_bias
    p = prob(I=64, rows=16)
    assert f(ctypes.byref(p), ctypes.byref(w), A, -1, A + 100 * MB, None) == -2
    assert f(ctypes.byref(p), ctypes.byref(w), A, 49, A + 100 * MB, None) == -2
    assert f(ctypes.byref(p), ctypes.byref(w), None, 0, A + 100 * MB, None) == -1
    assert f(ctypes.byref(p), ctypes.byref(w), A, 0, None, None) == -1
    assert f(ctypes.byref(p), ctypes.byref(w), A, 0, A + 100 * MB + 8, None) == -6
    assert f(ctypes.byref(p), ctypes.byref(w), A, 0, A + 1024, None) == -7  # bias over z


def test_stage_entries_reject(lib):
    w = weights()
    p = prob()
    rc, lay = layout(lib, p, ta.TA_START)
    assert lib.triangle_attn_project(ctypes.byref(p), ta.TA_START, ctypes.byref(w), A, A + 200 * MB,
                                     lay.total - 1, None) == -5
    assert lib.triangle_attn_project(ctypes.byref(p), 5, ctypes.byref(w), A, A + 200 * MB, lay.total, None) == -9
    # start/end keep their bias in the workspace: passing one is a variant error
    assert lib.triangle_attn_attend(ctypes.byref(p), ta.TA_START, ctypes.byref(w), A + 300 * MB, A + 100 * MB,
                                    A + 200 * MB, lay.total, None) == -9
    pr = prob(I=64, rows=8)
    rc, lr = layout(lib, pr, ta.TA_ROWS)
    assert lib.triangle_attn_attend(ctypes.byref(pr), ta.TA_ROWS, ctypes.byref(w), None, A + 100 * MB,
                                    A + 200 * MB, lr.total, None) == -1


def test_python_binding_rejects_cpu_tensors():
    import torch
    z = torch.zeros(4, 4, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ta.triangle_attn_start(z, {})


def test_state_bytes(lib):
    """O / l in the bias dtype (fp16 for bf16, fp32 for fp32), then (m, l) and the shift
    scratch in fp32, each region starting at a 256-byte boundary."""
    n = ctypes.c_size_t()
    P = 1024
    ml = (1000 * 4 * P * 2 * 4 + 255) // 256 * 256
    for dt, es in [(ta.TA_BF16, 2), (ta.TA_F32, 4)]:
        p = prob(I=1000, dtype=dt)
        assert lib.triangle_attn_state_bytes(ctypes.byref(p), ta.TA_START, ctypes.byref(n)) == 0
        o = (1000 * 4 * P * 32 * es + 255) // 256 * 256
        assert n.value == o + ml + 4 * P * 4             # + the [H][P] shift scratch of caller-held blocks
    p = prob(I=1000, dtype=ta.TA_BF16)
    assert lib.triangle_attn_state_bytes(ctypes.byref(p), ta.TA_START, None) == -1
    assert lib.triangle_attn_state_bytes(ctypes.byref(prob(I=64, rows=32)), ta.TA_START, ctypes.byref(n)) == -2


@pytest.mark.parametrize("dtype,odt", [(torch.bfloat16, torch.float16), (torch.float32, torch.float32)])
def test_state_views_layout(dtype, odt):
    """The binding's typed views of a state buffer (a CPU tensor of the library's size)
    sit where the header places them: O / l first in the bias dtype, (m, l) at the next
    256-byte boundary, and the shift scratch after that within the buffer."""
    I, rows = 200, 200
    n = ta.triangle_attn_state_bytes(I, rows, dtype, "start")
    st = torch.zeros(n // 4, dtype=torch.float32)
    v = ta.state_views(st, I, rows, dtype, "start")
    lay = ta.triangle_attn_workspace_layout(I, rows, dtype, "start")
    L, P = lay.lines, lay.positions
    assert v["O"].dtype == odt and v["O"].shape == (L, 4, P, 32)
    assert v["ml"].dtype == torch.float32 and v["ml"].shape == (L, 4, P, 2)
    base = st.data_ptr()
    o_bytes = L * 4 * P * 32 * v["O"].element_size()
    assert v["O"].data_ptr() == base
    assert v["ml"].data_ptr() - base == (o_bytes + 255) // 256 * 256
    ml_end = v["ml"].data_ptr() - base + L * 4 * P * 2 * 4
    assert (ml_end + 255) // 256 * 256 + 4 * P * 4 == n       # the [H][P] shift scratch closes the buffer


def test_block_rejects(lib):
    p = prob(I=200)
    w = weights()
    rc, lay = layout(lib, p, ta.TA_START)
    f = lib.triangle_attn_attend_block
    call = lambda key0=0, nkeys=64, first=1, st=A + 300 * MB, ws=A + 200 * MB, variant=ta.TA_START, bias=None, \
        wsb=lay.total: f(ctypes.byref(p), variant, ctypes.byref(w), bias, key0, nkeys, first, st, ws, wsb, None)
    assert call(key0=32) == -2              # not a multiple of 64
    assert call(key0=-64) == -2
    assert call(key0=200) == -2
    assert call(nkeys=0) == -2
    assert call(key0=192, nkeys=64) == -2   # past I
    assert call(key0=64, nkeys=100) == -2   # ragged block that does not end at I
    assert call(st=None) == -1
    assert call(st=A + 300 * MB + 4) == -6
    assert call(st=A + 200 * MB + 4096) == -7   # state inside the workspace
    assert call(wsb=lay.total - 1) == -5
    assert call(variant=9) == -9
    pr = prob(I=200, rows=8)
    rc, lr = layout(lib, pr, ta.TA_ROWS)
    assert f(ctypes.byref(pr), ta.TA_ROWS, ctypes.byref(w), None, 0, 64, 1, A + 300 * MB, A + 200 * MB, lr.total,
             None) == -1                # the first block of a row block needs the bias
    fin = lib.triangle_attn_attend_finalize
    assert fin(ctypes.byref(p), ta.TA_START, ctypes.byref(w), None, A + 100 * MB, A + 200 * MB, lay.total, None) == -1
    assert fin(ctypes.byref(p), ta.TA_START, ctypes.byref(w), A + 300 * MB, A + 200 * MB + 512, A + 200 * MB,
               lay.total, None) == -7   # out inside the workspace


def test_noalloc_rejects(lib):
    """The static-workspace entry point validates before it looks up its array (no GPU here)."""
    w = weights()
    f = lib.triangle_attn_start_noalloc
    call = lambda p, z=A, out=A + 100 * MB, ww=w: f(ctypes.byref(p), None if ww is None else ctypes.byref(ww), z,
                                                   out, None)
    assert call(prob(I=512)) == -12                     # workspace past 256 MiB
    assert call(prob(I=300, dtype=ta.TA_F32)) == -12
    assert call(prob(I=64, rows=32)) == -2
    assert call(prob(I=64), ww=None) == -1
    assert call(prob(I=64), z=None) == -1
    assert call(prob(I=64), out=None) == -1
    assert f(None, ctypes.byref(w), A, A, None) == -1


def test_kv_block_rejects(lib):
    """The ring step on caller-held blocks: shapes, pointers, alignment and overlaps."""
    p = prob(I=200)                          # P = 256
    w = weights()
    rc, lay = layout(lib, p, ta.TA_START)
    f = lib.triangle_attn_attend_kv_block
    K, V, B, ST, WS = A + 400 * MB, A + 450 * MB, A + 500 * MB, A + 300 * MB, A + 200 * MB

    def call(k=K, vt=V, npos=128, bias=B, nkeys=100, first=1, st=ST, ws=WS, wsb=lay.total, variant=ta.TA_START):
        return f(ctypes.byref(p), variant, ctypes.byref(w), k, vt, npos, bias, nkeys, first, st, ws, wsb, None)

    assert call() != -2 and call() != -1     # (the valid shape reaches the launch; no GPU here)
    assert call(nkeys=0) == -2
    assert call(nkeys=201) == -2             # more keys than I
    assert call(nkeys=129) == -2             # more keys than positions
    assert call(npos=96) == -2               # positions not a multiple of 64
    assert call(npos=320) == -2              # positions past the workspace's P
    assert call(k=None) == -1 and call(vt=None) == -1 and call(bias=None) == -1
    assert call(st=None) == -1 and call(ws=None) == -1
    assert call(k=K + 8) == -6 and call(bias=B + 4) == -6 and call(st=ST + 4) == -6
    assert call(wsb=lay.total - 1) == -5
    assert call(st=K + 4096) == -7           # state over the key block
    assert call(k=WS + 4096) == -7           # key block inside the workspace
    assert call(bias=ST + 256) == -7         # bias block inside the state
    assert call(variant=9) == -9


def test_kv_block_final_rejects(lib):
    """The last ring step: the key-block checks, plus the output buffer."""
    p = prob(I=200)
    w = weights()
    rc, lay = layout(lib, p, ta.TA_START)
    f = lib.triangle_attn_attend_kv_block_final
    K, V, B, ST, WS, OUT = A + 400 * MB, A + 450 * MB, A + 500 * MB, A + 300 * MB, A + 200 * MB, A + 600 * MB

    def call(k=K, npos=128, nkeys=100, st=ST, out=OUT, ws=WS):
        return f(ctypes.byref(p), ta.TA_START, ctypes.byref(w), k, V, npos, B, nkeys, 0, st, out, ws, lay.total,
                 None)

    assert call() != -2 and call() != -1
    assert call(out=None) == -1
    assert call(out=OUT + 8) == -6
    assert call(nkeys=0) == -2 and call(npos=96) == -2
    assert call(out=K + 4096) == -7          # out over the key block
    assert call(out=WS + 4096) == -7         # out inside the workspace
    assert call(out=ST + 256) == -7          # out inside the state
    assert call(out=A + 900 * MB) == -7      # out over a weight
    assert call(k=OUT) == -7                 # key block over out


# ----------------------------------------------------------------------------------------- AAQ codec

def test_aaq_record_bytes(lib):
    assert [lib.aaq_record_bytes(g) for g in (0, 1, 2)] == [160, 96, 80]
    assert lib.aaq_record_bytes(3) == -11 and lib.aaq_record_bytes(-1) == -11


@pytest.mark.parametrize("x,dtype,n,group,rec,code", [
    (A, ta.TA_BF16, 8, 3, A + 64 * MB, -11),
    (A, 3, 8, 0, A + 64 * MB, -4),
    (A, ta.TA_BF16, -1, 0, A + 64 * MB, -2),
    (A, ta.TA_BF16, (1 << 40) + 1, 0, A + 64 * MB, -2),
    (None, ta.TA_BF16, 8, 0, A + 64 * MB, -1),
    (A, ta.TA_F32, 8, 1, None, -1),
    (A + 8, ta.TA_BF16, 8, 0, A + 64 * MB, -6),
    (A, ta.TA_BF16, 8, 2, A + 64 * MB + 4, -6),
    (A, ta.TA_BF16, 8, 0, A + 1024, -7),       # records start inside x (8 x 256 B)
    (A + 1024, ta.TA_F32, 8, 0, A, -7),        # x starts inside the records (8 x 160 B)
    (None, ta.TA_BF16, 0, 0, None, 0),         # n = 0: valid, nothing enqueued
])
def test_aaq_rejects(lib, x, dtype, n, group, rec, code):
    assert lib.aaq_encode(x, dtype, n, group, rec, None) == code
    assert lib.aaq_decode(rec, group, n, x, dtype, None) == code


def test_project_aaq_rejects(lib):
    W = ctypes.byref(weights())
    ws = A + 1024 * MB
    p = prob(I=64)
    rec = A + 512 * MB
    lay = ta.TaWsLayout()
    assert lib.triangle_attn_workspace_layout(ctypes.byref(p), ta.TA_START, ctypes.byref(lay)) == 0
    f = lib.triangle_attn_project_aaq
    assert f(ctypes.byref(prob(I=64, dtype=ta.TA_F32)), ta.TA_START, W, rec, 0, ws, lay.total, None) == -4
    assert f(ctypes.byref(p), ta.TA_START, W, rec, 3, ws, lay.total, None) == -11
    assert f(ctypes.byref(p), ta.TA_START, W, None, 0, ws, lay.total, None) == -1
    assert f(ctypes.byref(p), ta.TA_START, W, rec + 8, 0, ws, lay.total, None) == -6
    assert f(ctypes.byref(p), ta.TA_START, W, rec, 0, ws, lay.total - 16, None) == -5
    assert f(ctypes.byref(p), ta.TA_START, W, ws + 4096, 0, ws, lay.total, None) == -7   # records inside ws
    assert f(ctypes.byref(p), 7, W, rec, 0, ws, lay.total, None) == -9


def test_knn_workspace_bytes(lib):
    n = ctypes.c_size_t()
    assert lib.knn_workspace_bytes(16384, ctypes.byref(n)) == 0
    # A and B halves fp32 [L][32], float4 coordinates per 64-atom chunk, two float4 per chunk
    assert n.value == 16384 * 128 + 256 * 64 * 16 + 256 * 32
    assert lib.knn_workspace_bytes(100, ctypes.byref(n)) == 0 and n.value == 100 * 128 + 2 * 64 * 16 + 2 * 32
    assert lib.knn_workspace_bytes(0, ctypes.byref(n)) == 0 and n.value == 0
    assert lib.knn_workspace_bytes(-1, ctypes.byref(n)) == -2
    assert lib.knn_workspace_bytes((1 << 24) + 1, ctypes.byref(n)) == -2
    assert lib.knn_workspace_bytes(10, None) == -1


def test_knn_rejects(lib):
    L, k = 1000, 32
    n = ctypes.c_size_t()
    lib.knn_workspace_bytes(L, ctypes.byref(n))
    args = dict(x=A, s=A + 1 * MB, L=L, k=k, w_l=A + 2 * MB, w_m=A + 3 * MB, w_d=A + 4 * MB,
                nbr=A + 5 * MB, pair=A + 10 * MB, ws=A + 20 * MB, ws_bytes=n.value)

    def call(**over):
        a = dict(args, **over)
        return lib.knn_pair_encode(a["x"], a["s"], a["L"], a["k"], a["w_l"], a["w_m"], a["w_d"], a["nbr"],
                                   a["pair"], a["ws"], a["ws_bytes"], None)

    assert call(k=0) == -2 and call(k=65) == -2 and call(L=-1) == -2 and call(L=(1 << 24) + 1) == -2
    assert call(L=1, k=1) == -2 and call(L=32, k=32) == -2
    assert call(L=0, x=None, s=None) == 0                   # nothing to do, nothing enqueued
    for name in ("x", "s", "w_l", "w_m", "w_d", "nbr", "pair", "ws"):
        assert call(**{name: None}) == -1, name
        assert call(**{name: args[name] + 4}) == -6, name
    assert call(ws_bytes=n.value - 1) == -5
    assert call(pair=A + 5 * MB + 256) == -7                 # pair overlaps nbr
    assert call(nbr=A) == -7                                 # nbr overlaps x
    assert call(ws=A + 10 * MB + 1024) == -7                 # ws overlaps pair
    assert call(pair=A + 1 * MB) == -7                       # pair overlaps s


def test_issue_probe_library_exports():
    """The measurement-only probe library (bench.py --issue-probe) loads, exports its
    two functions, and rejects bad arguments before any GPU call."""
    import ctypes
    from protein_pair_representation_amd.build import PROBE_PATH
    if not os.path.exists(PROBE_PATH):
        pytest.skip("libissueprobe.so not built")
    lib = ctypes.CDLL(PROBE_PATH)
    assert lib.issue_probe_modes() == 8
    lib.issue_probe_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_double)]
    c, g = ctypes.c_double(), ctypes.c_double()
    for mode, waves in ((-1, 2), (8, 2), (0, 0), (0, 5)):
        assert lib.issue_probe_run(mode, waves, ctypes.byref(c), ctypes.byref(g)) == -1
    assert lib.issue_probe_run(0, 2, None, ctypes.byref(g)) == -1
