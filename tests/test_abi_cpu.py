"""The C-ABI library loads, exports what include/lisa.h declares, and rejects
bad arguments on the host before touching the GPU (CPU only: every call here
fails validation, so nothing is enqueued)."""

import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lisa.h")

lisa = pytest.importorskip("vision_transformer_token_amd.lisa", reason="liblisa.so not built")
lib = lisa.raw

OK, NULL, SHAPE, PARAM, DTYPE, UNSUP, WS, ALIGN, HIP = range(9)


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(lisa_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == [
        "lisa_apply", "lisa_attention_forward", "lisa_attention_workspace_size", "lisa_backward",
        "lisa_backward_after_forward",
        "lisa_backward_workspace_size", "lisa_forward", "lisa_forward_mlp", "lisa_forward_mlp_workspace_size",
        "lisa_forward_noalloc", "lisa_forward_phases", "lisa_forward_schedule",
        "lisa_reduce", "lisa_status_str", "lisa_workspace_check", "lisa_workspace_size"]


def test_library_exports_every_declared_symbol():
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_problem_struct_matches_header():
    import re

    hdr = open(os.path.join(os.path.dirname(__file__), "..", "include", "lisa.h")).read()
    body = hdr[hdr.index("typedef struct lisa_problem {"):hdr.index("} lisa_problem;")]
    names = re.findall(r"^\s*(?:int32_t|float)\s+(\w+);", body, re.M)
    assert names == [f[0] for f in lisa.Problem._fields_]
    assert ctypes.sizeof(lisa.Problem) == 4 * len(names) == 44


def test_stage_list_matches_header():
    """lisa.STAGES and LISA_PHASES are the header's LISA_STAGE_* enum, in order."""
    hdr = open(HEADER).read()
    assert int(re.search(r"#define LISA_PHASES (\d+)", hdr).group(1)) == lisa.LISA_PHASES
    body = hdr[hdr.index("LISA_STAGE_START = 0"):]
    body = body[:body.index("};")]
    names = [n.lower() for n in re.findall(r"LISA_STAGE_(\w+)", body)]
    assert names == lisa.STAGES
    assert len(names) < lisa.LISA_PHASES  # the last entry holds the rank


def prob(**kw):
    base = dict(batch=2, heads=3, grid_h=5, grid_w=7, d_h=64, d_v=64, T=3, dtype=lisa.LISA_BF16,
                eps=1e-6)
    base.update(kw)
    return lisa.Problem(**base)


# Fake, aligned device addresses: never dereferenced, since validation fails first.
A = 0x10000000
Q, K, V, Y, W_, AL, WS_ = (A + i * 0x1000000 for i in range(7))


def forward(p, q=Q, k=K, v=V, w=W_, beta=0.5, alpha=AL, y=Y, ws=WS_, ws_bytes=None, fn=None):
    if ws_bytes is None:
        ws_bytes = lisa.lisa_workspace_size(p) if p is not None else 0
    f = fn or lib.lisa_forward
    return f(None if p is None else ctypes.byref(p), q, k, v, w, ctypes.c_float(beta), alpha, y, ws,
             ctypes.c_size_t(ws_bytes), None)


def test_workspace_size():
    assert lib.lisa_workspace_size(None) == 0
    assert lisa.lisa_workspace_size(prob(batch=0)) == 0
    assert lisa.lisa_workspace_size(prob(d_h=32)) == 0
    a = lisa.lisa_workspace_size(prob())
    b = lisa.lisa_workspace_size(prob(batch=4))
    assert 0 < a < b and a % 256 == 0
    # long sequences: partial count is capped, so the size stays linear in batch*heads
    big = lisa.lisa_workspace_size(prob(batch=1, heads=1, grid_h=400, grid_w=400))
    assert 0 < big < 64 << 20


@pytest.mark.parametrize("fn", ["lisa_forward", "lisa_apply"])
def test_forward_argument_errors(fn):
    f = getattr(lib, fn)
    assert forward(None, fn=f) == NULL
    assert forward(prob(dtype=7), fn=f) == DTYPE
    for bad in (dict(batch=0), dict(heads=-1), dict(grid_h=0), dict(grid_w=0), dict(d_h=0),
                dict(grid_h=5000, grid_w=5000)):
        assert forward(prob(**bad), fn=f) == SHAPE, bad
    for bad in (dict(d_h=32), dict(d_v=128), dict(batch=300, heads=300)):
        assert forward(prob(**bad), fn=f) == UNSUP, bad
    for bad in (dict(T=0), dict(T=17), dict(feature=2), dict(feature=-1), dict(eps=0.0), dict(eps=-1e-6), dict(eps=math.nan),
                dict(eps=math.inf), dict(schedule=3), dict(schedule=-1)):
        assert forward(prob(**bad), fn=f) == PARAM, bad
    for beta in (1.0, -0.1, math.nan):
        assert forward(prob(), w=None, beta=beta, fn=f) == PARAM
    for name in ("q", "k", "v", "alpha", "y"):
        assert forward(prob(), fn=f, **{name: None}) == NULL, name
    for name in ("q", "k", "v", "y"):
        assert forward(prob(), fn=f, **{name: A + 8}) == ALIGN, name
    assert forward(prob(), w=A + 2, fn=f) == ALIGN
    assert forward(prob(), alpha=A + 2, fn=f) == ALIGN
    p = prob()
    need = lisa.lisa_workspace_size(p)
    assert forward(p, ws=None, fn=f) == WS
    assert forward(p, ws_bytes=need - 1, fn=f) == WS
    assert forward(p, ws=WS_ + 128, fn=f) == WS
    # Y overlapping an input or the workspace
    assert forward(p, y=Q + 64, fn=f) == PARAM
    assert forward(p, y=WS_, fn=f) == PARAM


def test_reduce_argument_errors():
    def reduce(p, q=Q, k=K, v=V, s=A, kv=A + 0x100000, m=A + 0x200000, ws=WS_, ws_bytes=None):
        if ws_bytes is None:
            ws_bytes = lisa.lisa_workspace_size(p) if p is not None else 0
        return lib.lisa_reduce(None if p is None else ctypes.byref(p), q, k, v, s, kv, m, ws,
                               ctypes.c_size_t(ws_bytes), None)

    assert reduce(None) == NULL
    assert reduce(prob(dtype=3)) == DTYPE
    assert reduce(prob(grid_h=0)) == SHAPE
    assert reduce(prob(d_v=16)) == UNSUP
    assert reduce(prob(T=0)) == PARAM
    assert reduce(prob(), q=None) == NULL
    assert reduce(prob(), k=A + 4) == ALIGN
    assert reduce(prob(), s=A + 2) == ALIGN
    assert reduce(prob(), ws=None) == WS
    p = prob()
    assert reduce(p, ws_bytes=lisa.lisa_workspace_size(p) - 256) == WS


DY, DQ, DK, DV, DW, DA = (A + (8 + i) * 0x1000000 for i in range(6))


BACKWARD_FN = [lib.lisa_backward]


def backward(p, q=Q, k=K, v=V, w=W_, beta=0.5, alpha=AL, dy=DY, dq=DQ, dk=DK, dv=DV, dw=DW, da=DA, ws=WS_,
             ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lisa.lisa_backward_workspace_size(p) if p is not None else 0
    return BACKWARD_FN[0](None if p is None else ctypes.byref(p), q, k, v, w, ctypes.c_float(beta), alpha,
                          dy, dq, dk, dv, dw, da, ws, ctypes.c_size_t(ws_bytes), None)


def test_backward_workspace_covers_the_forward():
    for T in (1, 3, 8):
        p = prob(T=T, grid_h=40, grid_w=33)
        assert lisa.lisa_backward_workspace_size(p) >= lisa.lisa_workspace_size(p) > 0
    assert lisa.lisa_backward_workspace_size(prob(T=9)) == 0
    # The forward takes up to 16 walk terms, the backward up to 8.
    assert lisa.lisa_workspace_size(prob(T=16)) > 0
    assert lisa.lisa_workspace_size(prob(T=17)) == 0
    # The ELU feature map: forward only.
    assert lisa.lisa_workspace_size(prob(feature=1)) == lisa.lisa_workspace_size(prob())
    assert lisa.lisa_backward_workspace_size(prob(feature=1)) == 0


@pytest.fixture(params=["lisa_backward", "lisa_backward_after_forward"])
def backward_entry(request):
    """Both backward entry points check their arguments the same way."""
    BACKWARD_FN[0] = getattr(lib, request.param)
    yield request.param
    BACKWARD_FN[0] = lib.lisa_backward


def test_backward_argument_errors(backward_entry):
    assert backward(None) == NULL
    assert backward(prob(dtype=3)) == DTYPE
    assert backward(prob(grid_w=-1)) == SHAPE
    assert backward(prob(d_h=32)) == UNSUP
    assert backward(prob(T=9)) == PARAM
    assert backward(prob(feature=1), ws_bytes=1 << 30) == UNSUP
    assert backward(prob(), w=None, beta=1.0) == PARAM
    for name in ("q", "k", "v", "alpha", "dy", "dq", "dk", "dv", "da"):
        assert backward(prob(), **{name: None}) == NULL, name
    assert backward(prob(), dy=DY + 8) == ALIGN
    assert backward(prob(), dq=DQ + 4) == ALIGN
    assert backward(prob(), dw=DW + 2) == ALIGN
    p = prob()
    assert backward(p, ws=None) == WS
    assert backward(p, ws_bytes=lisa.lisa_workspace_size(p)) == WS  # the forward's size is not enough
    assert backward(p, ws=WS_ + 128) == WS
    # outputs overlapping an input, each other or the workspace
    assert backward(p, dq=Q + 256) == PARAM
    assert backward(p, dk=DQ) == PARAM
    assert backward(p, dv=WS_ + 1024) == PARAM
    assert backward(p, da=AL) == PARAM
    assert backward(p, dw=DY) == PARAM


def test_status_strings():
    seen = set()
    for code in range(11):
        s = lisa.lisa_status_str(code)
        assert s and s not in seen
        seen.add(s)
    assert lisa.lisa_status_str(42) == "unknown status"


def test_workspace_check_argument_errors():
    """Checked before any HIP call: no device is touched."""
    check = lib.lisa_workspace_check
    assert check(None, ctypes.c_size_t(4096), None) == NULL
    assert check(WS_, ctypes.c_size_t(255), None) == WS
    assert check(WS_ + 128, ctypes.c_size_t(4096), None) == WS


W1_, B1_, W2_, B2_ = (A + (16 + i) * 0x1000000 for i in range(4))


def forward_mlp(p, hidden=64, w1=W1_, b1=B1_, w2=W2_, b2=B2_, mlp=True, q=Q, alpha=AL, ws=WS_, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lisa.lisa_forward_mlp_workspace_size(p, hidden) if p is not None else 0
    m = lisa.WeightMlp(hidden, w1, b1, w2, b2)
    return lib.lisa_forward_mlp(None if p is None else ctypes.byref(p), q, K, V,
                                ctypes.byref(m) if mlp else None, alpha, Y, ws, ctypes.c_size_t(ws_bytes), None)


def test_mlp_struct_matches_header():
    assert ctypes.sizeof(lisa.WeightMlp) == 8 + 4 * 8


def test_mlp_workspace_size():
    p = prob(grid_h=40, grid_w=33)
    for hidden in (32, 64, 128):
        # bf16: W1 [heads, hidden, 128] kept once more at 2 bytes per element
        assert lisa.lisa_forward_mlp_workspace_size(p, hidden) >= lisa.lisa_workspace_size(p) + 3 * hidden * 128 * 2
    for hidden in (0, 16, 48, 160):
        assert lisa.lisa_forward_mlp_workspace_size(p, hidden) == 0
    assert lisa.lisa_forward_mlp_workspace_size(prob(T=9), 64) == 0


def test_mlp_argument_errors():
    assert forward_mlp(None) == NULL
    assert forward_mlp(prob(), mlp=False) == NULL
    assert forward_mlp(prob(dtype=3)) == DTYPE
    assert forward_mlp(prob(grid_h=0)) == SHAPE
    assert forward_mlp(prob(d_h=32)) == UNSUP
    assert forward_mlp(prob(T=0)) == PARAM
    assert forward_mlp(prob(T=9), ws_bytes=1 << 30) == PARAM
    assert forward_mlp(prob(feature=1), ws_bytes=1 << 30) == UNSUP
    assert lisa.lisa_forward_mlp_workspace_size(prob(feature=1), 64) == 0
    for hidden in (16, 48, 160):
        assert forward_mlp(prob(), hidden=hidden, ws_bytes=1 << 30) == PARAM, hidden
    for name in ("w1", "b1", "w2", "b2"):
        assert forward_mlp(prob(), **{name: None}) == NULL, name
    assert forward_mlp(prob(), b2=B2_ + 2) == ALIGN
    assert forward_mlp(prob(), q=None) == NULL
    assert forward_mlp(prob(), alpha=AL + 1) == ALIGN
    p = prob()
    assert forward_mlp(p, ws_bytes=lisa.lisa_workspace_size(p)) == WS
    assert forward_mlp(p, ws=None) == WS


X_, WQ_, BQ_, WO_, BO_ = (A + (24 + i) * 0x1000000 for i in range(5))


def attention(p, x=X_, wq=WQ_, bq=BQ_, wo=WO_, bo=BO_, w=W_, beta=0.5, alpha=AL, y=Y, ws=WS_, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lisa.lisa_attention_workspace_size(p) if p is not None else 0
    return lib.lisa_attention_forward(None if p is None else ctypes.byref(p), x, wq, bq, wo, bo, w,
                                      ctypes.c_float(beta), alpha, y, ws, ctypes.c_size_t(ws_bytes), None)


def test_attention_workspace_size():
    p = prob(grid_h=40, grid_w=33)
    tensor = 2 * 3 * 40 * 33 * 64 * 2
    assert lisa.lisa_attention_workspace_size(p) >= lisa.lisa_workspace_size(p) + 4 * tensor
    assert lisa.lisa_attention_workspace_size(prob(T=17)) == 0
    assert lisa.lisa_attention_workspace_size(prob(T=16)) > 0


def test_attention_argument_errors():
    assert attention(None) == NULL
    assert attention(prob(dtype=3)) == DTYPE
    assert attention(prob(grid_h=0)) == SHAPE
    assert attention(prob(d_h=32)) == UNSUP
    assert attention(prob(T=17)) == PARAM
    assert attention(prob(), w=None, beta=1.0) == PARAM
    for name in ("x", "wq", "bq", "wo", "bo", "alpha", "y"):
        assert attention(prob(), **{name: None}) == NULL, name
    assert attention(prob(), x=X_ + 8) == ALIGN
    assert attention(prob(), wo=WO_ + 4) == ALIGN
    assert attention(prob(), bq=BQ_ + 2) == ALIGN
    p = prob()
    assert attention(p, ws_bytes=lisa.lisa_workspace_size(p)) == WS
    assert attention(p, ws=None) == WS
    assert attention(p, y=X_) == PARAM
    assert attention(p, y=WS_) == PARAM



def test_forward_noalloc_argument_errors():
    """lisa_forward_noalloc: every check that needs no device comes first, so
    these fail before any HIP call (no GPU here)."""
    f = lib.lisa_forward_noalloc

    def call(p, q=Q, k=K, v=V, w=W_, beta=0.5, alpha=AL, y=Y):
        return f(None if p is None else ctypes.byref(p), q, k, v, w, ctypes.c_float(beta), alpha, y, None)

    assert call(None) == NULL
    assert call(prob(batch=0)) == SHAPE
    assert call(prob(d_h=32)) == UNSUP
    assert call(prob(T=0)) == PARAM
    assert call(prob(), w=None, beta=1.0) == PARAM
    assert call(prob(), q=None) == NULL
    assert call(prob(), y=None) == NULL
    assert call(prob(), v=V + 8) == ALIGN
    assert call(prob(), y=Q) == PARAM
    # More (batch, head) slices than the fixed scratch's counters cover.
    assert call(prob(batch=8193, heads=1, grid_h=1, grid_w=1)) == lisa.LISA_ERR_SCRATCH


def test_forward_schedule_argument_errors():
    """lisa_forward_schedule checks the problem before it looks for a device."""
    out = ctypes.c_int32(-1)
    assert lib.lisa_forward_schedule(None, ctypes.byref(out)) == NULL
    assert lib.lisa_forward_schedule(ctypes.byref(prob(schedule=3)), ctypes.byref(out)) == PARAM
    assert lib.lisa_forward_schedule(ctypes.byref(prob(T=0)), ctypes.byref(out)) == PARAM
    assert lib.lisa_forward_schedule(ctypes.byref(prob()), None) == NULL
    assert out.value == -1
