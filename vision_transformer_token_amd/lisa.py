"""Thin ctypes binding of liblisa.so (C ABI in include/lisa.h).

Argument marshalling only: every step of the LiSA forward pass runs in the
library's HIP kernels.  PyTorch supplies device memory and the current
stream.  There is no fallback: if the library is missing, importing this
module raises.
"""

import ctypes
import os

import torch

__all__ = [
    "LisaError",
    "Problem",
    "LISA_FP32",
    "LISA_BF16",
    "lisa_workspace_size",
    "lisa_forward",
    "lisa_forward_mlp",
    "lisa_attention_forward",
    "lisa_attention_workspace_size",
    "lisa_forward_mlp_workspace_size",
    "WeightMlp",
    "lisa_reduce",
    "lisa_apply",
    "lisa_status_str",
    "make_problem",
    "new_workspace",
    "library_path",
    "lisa_workspace_check",
    "lisa_backward",
    "lisa_backward_after_forward",
    "lisa_backward_workspace_size",
    "LISA_ERR_NULL",
    "LISA_ERR_SHAPE",
    "LISA_ERR_PARAM",
    "LISA_ERR_DTYPE",
    "LISA_ERR_UNSUPPORTED",
    "LISA_ERR_WORKSPACE",
    "LISA_ERR_ALIGN",
    "LISA_ERR_HIP",
    "LISA_ERR_STALLED",
    "LISA_ERR_SCRATCH",
    "lisa_forward_noalloc",
    "lisa_forward_phases",
    "lisa_forward_schedule",
    "LISA_PHASES",
    "STAGES",
    "FEATURES",
    "SCHEDULES",
]

LISA_PHASES = 16
# Stage indices of lisa_forward_phases (LISA_STAGE_* in include/lisa.h).
STAGES = ["start", "staged", "kv", "local", "s", "m", "mwait", "combine", "cwait", "frags", "out", "end", "kvsweep",
          "cstaged", "csummed"]

LISA_FP32 = 0
LISA_BF16 = 1
LISA_OK = 0
LISA_ERR_NULL = 1
LISA_ERR_SHAPE = 2
LISA_ERR_PARAM = 3
LISA_ERR_DTYPE = 4
LISA_ERR_UNSUPPORTED = 5
LISA_ERR_WORKSPACE = 6
LISA_ERR_ALIGN = 7
LISA_ERR_HIP = 8
LISA_ERR_STALLED = 9
LISA_ERR_SCRATCH = 10

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path():
    return os.path.join(_HERE, "liblisa.so")


if not os.path.exists(library_path()):
    raise ImportError(
        f"{library_path()} is not built; run `python -m vision_transformer_token_amd.build` "
        "(or __graft_entry__.build()) first"
    )

_lib = ctypes.CDLL(library_path())


class Problem(ctypes.Structure):
    """struct lisa_problem."""

    _fields_ = [
        ("batch", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("grid_h", ctypes.c_int32),
        ("grid_w", ctypes.c_int32),
        ("d_h", ctypes.c_int32),
        ("d_v", ctypes.c_int32),
        ("T", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("eps", ctypes.c_float),
        ("feature", ctypes.c_int32),
        ("schedule", ctypes.c_int32),
    ]


# lisa_feature: phi of the global branch.
FEATURES = {"relu": 0, "elu": 1}
# lisa_schedule: which forward kernel runs the pass.
SCHEDULES = {"auto": 0, "streaming": 1, "resident": 2}


class WeightMlp(ctypes.Structure):
    """struct lisa_weight_mlp (device pointers)."""

    _fields_ = [
        ("hidden", ctypes.c_int32),
        ("w1", ctypes.c_void_p),
        ("b1", ctypes.c_void_p),
        ("w2", ctypes.c_void_p),
        ("b2", ctypes.c_void_p),
    ]


_P = ctypes.POINTER(Problem)
_vp = ctypes.c_void_p
_lib.lisa_workspace_size.argtypes = [_P]
_lib.lisa_workspace_size.restype = ctypes.c_size_t
_lib.lisa_forward.argtypes = [_P, _vp, _vp, _vp, _vp, ctypes.c_float, _vp, _vp, _vp, ctypes.c_size_t, _vp]
_lib.lisa_forward.restype = ctypes.c_int
_lib.lisa_forward_noalloc.argtypes = [_P, _vp, _vp, _vp, _vp, ctypes.c_float, _vp, _vp, _vp]
_lib.lisa_forward_noalloc.restype = ctypes.c_int
_lib.lisa_forward_phases.argtypes = [_P, _vp, _vp, _vp, _vp, ctypes.c_float, _vp, _vp, _vp, ctypes.c_size_t, _vp,
                                     ctypes.c_size_t, _vp]
_lib.lisa_forward_phases.restype = ctypes.c_int
_lib.lisa_apply.argtypes = _lib.lisa_forward.argtypes
_lib.lisa_apply.restype = ctypes.c_int
_lib.lisa_reduce.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
_lib.lisa_reduce.restype = ctypes.c_int
_lib.lisa_forward_mlp_workspace_size.argtypes = [_P, ctypes.c_int32]
_lib.lisa_forward_mlp_workspace_size.restype = ctypes.c_size_t
_lib.lisa_forward_mlp.argtypes = [_P, _vp, _vp, _vp, ctypes.POINTER(WeightMlp), _vp, _vp, _vp, ctypes.c_size_t, _vp]
_lib.lisa_forward_mlp.restype = ctypes.c_int
_lib.lisa_attention_workspace_size.argtypes = [_P]
_lib.lisa_attention_workspace_size.restype = ctypes.c_size_t
_lib.lisa_attention_forward.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp, _vp, _vp,
                                        ctypes.c_size_t, _vp]
_lib.lisa_attention_forward.restype = ctypes.c_int
_lib.lisa_backward_workspace_size.argtypes = [_P]
_lib.lisa_backward_workspace_size.restype = ctypes.c_size_t
_lib.lisa_backward.argtypes = [_P, _vp, _vp, _vp, _vp, ctypes.c_float, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                               _vp, ctypes.c_size_t, _vp]
_lib.lisa_backward.restype = ctypes.c_int
_lib.lisa_backward_after_forward.argtypes = _lib.lisa_backward.argtypes
_lib.lisa_backward_after_forward.restype = ctypes.c_int
_lib.lisa_workspace_check.argtypes = [_vp, ctypes.c_size_t, _vp]
_lib.lisa_workspace_check.restype = ctypes.c_int
_lib.lisa_status_str.argtypes = [ctypes.c_int]
_lib.lisa_status_str.restype = ctypes.c_char_p


class LisaError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {lisa_status_str(status)} (status {status})")


def lisa_status_str(status):
    return _lib.lisa_status_str(int(status)).decode()


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return LISA_BF16
    if t.dtype == torch.float32:
        return LISA_FP32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def make_problem(q, v, *, grid, T, eps=1e-6, feature="relu", schedule="auto"):
    """Problem for q [B, heads, n, d_h] and v [B, heads, n, d_v] on an H x W
    grid; ``feature`` is phi of the global branch, "relu" or "elu" (ELU + 1);
    ``schedule`` the forward kernel, "auto", "streaming" or "resident"."""
    H, W = grid
    B, heads, n, d_h = q.shape
    return Problem(B, heads, H, W, d_h, v.shape[-1], T, _dtype_code(q), eps, FEATURES[feature],
                   SCHEDULES[schedule])


def lisa_forward_schedule(problem):
    """The kernel lisa_forward runs for ``problem`` on the current device:
    "streaming" or "resident"."""
    out = ctypes.c_int32(-1)
    st = _lib.lisa_forward_schedule(ctypes.byref(problem), ctypes.byref(out))
    if st != LISA_OK:
        raise LisaError(st, "lisa_forward_schedule")
    return {v: k for k, v in SCHEDULES.items()}[out.value]


def lisa_workspace_size(problem):
    return int(_lib.lisa_workspace_size(ctypes.byref(problem)))


def new_workspace(problem, device):
    """Zero-filled workspace for ``problem`` (the ABI requires zeros on first use)."""
    nbytes = lisa_workspace_size(problem)
    if nbytes == 0:
        raise LisaError(2, "lisa_workspace_size")
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _check_tensors(**ts):
    for name, t in ts.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def _call_forward(fn, where, q, k, v, *, grid, T, alpha, weights=None, beta=None, eps=1e-6,
                  out=None, workspace=None, stream=None, feature="relu", schedule="auto"):
    _check_tensors(q=q, k=k, v=v, alpha=alpha, weights=weights, out=out, workspace=workspace)
    if weights is not None and weights.dtype != torch.float32:
        raise TypeError("weights must be float32")
    if alpha.dtype != torch.float32:
        raise TypeError("alpha must be float32")
    if weights is None and beta is None:
        raise ValueError("give adaptive weights or beta")
    prob = make_problem(q, v, grid=grid, T=T, eps=eps, feature=feature, schedule=schedule)
    if out is None:
        out = torch.empty_like(v)
    if workspace is None:
        workspace = new_workspace(prob, q.device)
    st = fn(
        ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(weights),
        ctypes.c_float(0.0 if beta is None else beta), _ptr(alpha), _ptr(out),
        _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream(stream, q.device),
    )
    if st != LISA_OK:
        raise LisaError(st, where)
    return out


def lisa_forward(q, k, v, *, grid, T, alpha, weights=None, beta=None, eps=1e-6, out=None,
                 workspace=None, stream=None, feature="relu", schedule="auto"):
    """Y = LiSA(q, k, v) on the GPU; see include/lisa.h.

    q, k: [B, heads, n, 64], v: [B, heads, n, 64], bf16 or fp32, contiguous
    GPU tensors with n = grid[0] * grid[1]; weights [B, heads, n, T] fp32 or
    None with ``beta``; alpha [heads] fp32.  ``workspace`` (a zero-filled
    uint8 tensor of lisa_workspace_size bytes) is allocated when not given.
    """
    return _call_forward(_lib.lisa_forward, "lisa_forward", q, k, v, grid=grid, T=T, alpha=alpha,
                         weights=weights, beta=beta, eps=eps, out=out, workspace=workspace,
                         stream=stream, feature=feature, schedule=schedule)


def lisa_forward_noalloc(q, k, v, *, grid, T, alpha, weights=None, beta=None, eps=1e-6, out=None, stream=None,
                         feature="relu", schedule="auto"):
    """lisa_forward without a workspace (the library's fixed device scratch;
    nothing is allocated by the call itself; ``out`` is allocated here when
    not given); see include/lisa.h."""
    _check_tensors(q=q, k=k, v=v, alpha=alpha, weights=weights, out=out)
    if weights is not None and weights.dtype != torch.float32:
        raise TypeError("weights must be float32")
    if alpha.dtype != torch.float32:
        raise TypeError("alpha must be float32")
    if weights is None and beta is None:
        raise ValueError("give adaptive weights or beta")
    prob = make_problem(q, v, grid=grid, T=T, eps=eps, feature=feature, schedule=schedule)
    if out is None:
        out = torch.empty_like(v)
    st = _lib.lisa_forward_noalloc(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(weights),
                                   ctypes.c_float(0.0 if beta is None else beta), _ptr(alpha), _ptr(out),
                                   _stream(stream, q.device))
    if st != LISA_OK:
        raise LisaError(st, "lisa_forward_noalloc")
    return out


def lisa_forward_phases(q, k, v, *, grid, T, alpha, stamps, weights=None, beta=None, eps=1e-6, out=None,
                        workspace=None, stream=None):
    """lisa_forward that also writes each workgroup's stage timeline into
    ``stamps`` (an int64 GPU tensor of at least compute units * LISA_PHASES
    entries); see include/lisa.h."""
    _check_tensors(stamps=stamps)
    if stamps.dtype != torch.int64:
        raise TypeError("stamps must be int64")

    def fn(prob, q_, k_, v_, w_, beta_, a_, y_, ws_, nb_, st_):
        return _lib.lisa_forward_phases(prob, q_, k_, v_, w_, beta_, a_, y_, ws_, nb_, _ptr(stamps),
                                        ctypes.c_size_t(stamps.numel()), st_)

    return _call_forward(fn, "lisa_forward_phases", q, k, v, grid=grid, T=T, alpha=alpha, weights=weights,
                         beta=beta, eps=eps, out=out, workspace=workspace, stream=stream)


def lisa_forward_mlp_workspace_size(problem, hidden):
    return int(_lib.lisa_forward_mlp_workspace_size(ctypes.byref(problem), int(hidden)))


def lisa_forward_mlp(q, k, v, *, grid, T, alpha, w1, b1, w2, b2, eps=1e-6, out=None, workspace=None,
                     stream=None, schedule="auto"):
    """Y = LiSA(q, k, v) with the walk weights predicted from concat(q_i, k_i)
    by the two-layer MLP (w1 [heads, hidden, 2 d_h], b1 [heads, hidden],
    w2 [heads, T, hidden], b2 [heads, T], fp32 GPU tensors); see include/lisa.h."""
    _check_tensors(q=q, k=k, v=v, alpha=alpha, w1=w1, b1=b1, w2=w2, b2=b2, out=out, workspace=workspace)
    for name, t in (("alpha", alpha), ("w1", w1), ("b1", b1), ("w2", w2), ("b2", b2)):
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    hidden = w1.shape[1]
    prob = make_problem(q, v, grid=grid, T=T, eps=eps, schedule=schedule)
    if workspace is None:
        nbytes = lisa_forward_mlp_workspace_size(prob, hidden)
        if nbytes == 0:
            raise LisaError(2, "lisa_forward_mlp_workspace_size")
        workspace = torch.zeros(nbytes, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty_like(v)
    mlp = WeightMlp(hidden, w1.data_ptr(), b1.data_ptr(), w2.data_ptr(), b2.data_ptr())
    st = _lib.lisa_forward_mlp(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(mlp), _ptr(alpha),
                               _ptr(out), _ptr(workspace), ctypes.c_size_t(workspace.numel()),
                               _stream(stream, q.device))
    if st != LISA_OK:
        raise LisaError(st, "lisa_forward_mlp")
    return out


def lisa_attention_workspace_size(problem):
    return int(_lib.lisa_attention_workspace_size(ctypes.byref(problem)))


def lisa_attention_forward(x, w_qkv, b_qkv, w_o, b_o, *, heads, grid, T, alpha, weights=None, beta=None,
                           eps=1e-6, out=None, workspace=None, stream=None, feature="relu", schedule="auto"):
    """The LiSA attention layer: x [B, n, C] (bf16 or fp32, C = 64 heads),
    w_qkv [3C, C] and w_o [C, C] in x's dtype, b_qkv [3C] and b_o [C] fp32;
    see include/lisa.h."""
    _check_tensors(x=x, w_qkv=w_qkv, b_qkv=b_qkv, w_o=w_o, b_o=b_o, alpha=alpha, weights=weights, out=out,
                   workspace=workspace)
    if weights is None and beta is None:
        raise ValueError("give adaptive weights or beta")
    B, n, C = x.shape
    if C != 64 * heads:
        raise ValueError("x's channels must be 64 * heads")
    prob = Problem(B, heads, grid[0], grid[1], 64, 64, T, _dtype_code(x), eps, FEATURES[feature],
                   SCHEDULES[schedule])
    if workspace is None:
        nbytes = lisa_attention_workspace_size(prob)
        if nbytes == 0:
            raise LisaError(2, "lisa_attention_workspace_size")
        workspace = torch.zeros(nbytes, dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty_like(x)
    st = _lib.lisa_attention_forward(
        ctypes.byref(prob), _ptr(x), _ptr(w_qkv), _ptr(b_qkv), _ptr(w_o), _ptr(b_o), _ptr(weights),
        ctypes.c_float(0.0 if beta is None else beta), _ptr(alpha), _ptr(out), _ptr(workspace),
        ctypes.c_size_t(workspace.numel()), _stream(stream, x.device))
    if st != LISA_OK:
        raise LisaError(st, "lisa_attention_forward")
    return out


def lisa_apply(q, k, v, *, grid, T, alpha, workspace, weights=None, beta=None, eps=1e-6, out=None,
               stream=None, feature="relu", schedule="auto"):
    """Output stage alone, from the statistics a previous lisa_reduce left in ``workspace``."""
    return _call_forward(_lib.lisa_apply, "lisa_apply", q, k, v, grid=grid, T=T, alpha=alpha,
                         weights=weights, beta=beta, eps=eps, out=out, workspace=workspace,
                         stream=stream, feature=feature, schedule=schedule)


def lisa_reduce(q, k, v, *, grid, eps=1e-6, T=3, workspace=None, outputs=True, stream=None, feature="relu",
                schedule="auto"):
    """Statistics stage: returns (s, phi(K)^T V, M) as fp32 tensors, or None if not ``outputs``."""
    _check_tensors(q=q, k=k, v=v, workspace=workspace)
    prob = make_problem(q, v, grid=grid, T=T, eps=eps, feature=feature, schedule=schedule)
    if workspace is None:
        workspace = new_workspace(prob, q.device)
    B, heads = q.shape[:2]
    d_h, d_v = q.shape[-1], v.shape[-1]
    s = kv = m = None
    if outputs:
        s = torch.empty(B, heads, d_h, dtype=torch.float32, device=q.device)
        kv = torch.empty(B, heads, d_h, d_v, dtype=torch.float32, device=q.device)
        m = torch.empty(B, heads, d_h, d_h, dtype=torch.float32, device=q.device)
    st = _lib.lisa_reduce(
        ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(s), _ptr(kv), _ptr(m),
        _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream(stream, q.device),
    )
    if st != LISA_OK:
        raise LisaError(st, "lisa_reduce")
    return (s, kv, m) if outputs else None


def lisa_backward_workspace_size(problem):
    return int(_lib.lisa_backward_workspace_size(ctypes.byref(problem)))


def lisa_backward(q, k, v, dy, *, grid, T, alpha, weights=None, beta=None, eps=1e-6, workspace=None,
                  out=None, stream=None):
    """Gradients of lisa_forward for the output gradient ``dy``; see include/lisa.h.

    Returns a dict with "dq", "dk", "dv" (dtype of q), "dweights" (fp32
    [B, heads, n, T], None with geometric weights) and "dalpha" (fp32
    [heads]).  ``workspace`` (zero-filled, lisa_backward_workspace_size
    bytes) is allocated when not given; ``out`` (a dict like the result)
    supplies the output tensors.
    """
    return _backward(_lib.lisa_backward, "lisa_backward", q, k, v, dy, grid=grid, T=T, alpha=alpha,
                     weights=weights, beta=beta, eps=eps, workspace=workspace, out=out, stream=stream)


def lisa_backward_after_forward(q, k, v, dy, *, grid, T, alpha, workspace, weights=None, beta=None, eps=1e-6,
                                out=None, stream=None):
    """lisa_backward that reuses the slice statistics a lisa_forward (or
    lisa_forward_mlp, lisa_reduce) of the same problem and inputs left in
    ``workspace`` (lisa_backward_workspace_size bytes) just before; see
    include/lisa.h.  Same results as lisa_backward."""
    if workspace is None:
        raise ValueError("lisa_backward_after_forward needs the forward's workspace")
    return _backward(_lib.lisa_backward_after_forward, "lisa_backward_after_forward", q, k, v, dy, grid=grid,
                     T=T, alpha=alpha, weights=weights, beta=beta, eps=eps, workspace=workspace, out=out,
                     stream=stream)


def _backward(fn, name, q, k, v, dy, *, grid, T, alpha, weights, beta, eps, workspace, out, stream):
    _check_tensors(q=q, k=k, v=v, dy=dy, alpha=alpha, weights=weights, workspace=workspace)
    if weights is not None and weights.dtype != torch.float32:
        raise TypeError("weights must be float32")
    if alpha.dtype != torch.float32:
        raise TypeError("alpha must be float32")
    if weights is None and beta is None:
        raise ValueError("give adaptive weights or beta")
    prob = make_problem(q, v, grid=grid, T=T, eps=eps)
    if workspace is None:
        nbytes = lisa_backward_workspace_size(prob)
        if nbytes == 0:
            raise LisaError(2, "lisa_backward_workspace_size")
        workspace = torch.zeros(nbytes, dtype=torch.uint8, device=q.device)
    if out is None:
        out = {
            "dq": torch.empty_like(q),
            "dk": torch.empty_like(k),
            "dv": torch.empty_like(v),
            "dweights": None if weights is None else torch.empty_like(weights),
            "dalpha": torch.empty_like(alpha),
        }
    _check_tensors(**{k_: t for k_, t in out.items()})
    st = fn(
        ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(weights),
        ctypes.c_float(0.0 if beta is None else beta), _ptr(alpha), _ptr(dy), _ptr(out["dq"]),
        _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dweights"]), _ptr(out["dalpha"]), _ptr(workspace),
        ctypes.c_size_t(workspace.numel()), _stream(stream, q.device),
    )
    if st != LISA_OK:
        raise LisaError(st, name)
    return out


def lisa_workspace_check(workspace, stream=None):
    """Synchronise ``stream`` and read (and clear) the workspace's stall flag;
    see include/lisa.h.  Returns LISA_OK, or LISA_ERR_STALLED when a call on
    this workspace abandoned a wait (its outputs are then undefined)."""
    _check_tensors(workspace=workspace)
    st = _lib.lisa_workspace_check(_ptr(workspace), ctypes.c_size_t(workspace.numel() * workspace.element_size()),
                                   _stream(stream, workspace.device))
    if st not in (LISA_OK, LISA_ERR_STALLED):
        raise LisaError(st, "lisa_workspace_check")
    return st


# Raw entry points for callers that marshal their own pointers (tests, bench).
raw = _lib
