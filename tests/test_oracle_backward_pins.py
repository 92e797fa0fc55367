"""Pins of the backward oracle (oracle/backward.py) to facts other than itself (CPU only).

- Central finite differences of the forward oracle, along random directions
  for every input and element by element on a tiny grid.
- G is linear in V and in the walk weights: dV and the weight gradient of the
  global branch against explicit n x n powers of S.
- alpha: dalpha = sum dY (G - L); alpha = 0 / 1 isolates the two branches;
  T = 1 reduces the global branch to w_0 V.
- Planted mistakes (in a patched copy, on the CPU) are each caught.
"""

import inspect
import math

import numpy as np
import pytest

from oracle import lisa as olisa
from oracle import backward as oback


def _problem(rng, B, heads, H, W, dh, dv, T, adaptive, eps=1e-3):
    n = H * W
    p = dict(
        Q=rng.standard_normal((B, heads, n, dh)),
        K=rng.standard_normal((B, heads, n, dh)),
        V=rng.standard_normal((B, heads, n, dv)),
        alpha=rng.uniform(0.1, 0.9, heads),
        H=H, W=W, T=T, eps=eps,
    )
    if adaptive:
        lg = rng.standard_normal((B, heads, n, T))
        p["weights"] = np.exp(lg) / np.exp(lg).sum(-1, keepdims=True)
    else:
        p["beta"] = float(rng.uniform(0.1, 0.9))
    return p


def _loss(p, dY, **over):
    q = dict(p, **over)
    return float((dY * olisa.lisa_forward(**q)).sum())


def _grads(p, dY, module=oback):
    return module.lisa_backward(dY=dY, **p)


@pytest.mark.parametrize("case", [
    (1, 2, 4, 5, 6, 6, 3, True),
    (2, 1, 3, 7, 4, 5, 5, True),
    (1, 1, 6, 2, 8, 3, 2, False),
    (1, 1, 1, 1, 4, 4, 4, True),   # n = 1
    (1, 2, 1, 6, 3, 3, 8, True),   # one grid row, T = 8
    (1, 1, 5, 5, 4, 4, 1, True),   # T = 1
])
def test_directional_finite_differences(case):
    B, heads, H, W, dh, dv, T, adaptive = case
    rng = np.random.default_rng(hash(case) % 2**32)
    p = _problem(rng, B, heads, H, W, dh, dv, T, adaptive)
    dY = rng.standard_normal(p["V"].shape)
    g = _grads(p, dY)
    h = 1e-6
    inputs = [("Q", "dq"), ("K", "dk"), ("V", "dv"), ("alpha", "dalpha")]
    if adaptive:
        inputs.append(("weights", "dweights"))
    for name, key in inputs:
        D = rng.standard_normal(np.shape(p[name]))
        fd = (_loss(p, dY, **{name: p[name] + h * D}) - _loss(p, dY, **{name: p[name] - h * D})) / (2 * h)
        an = float((g[key] * D).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_elementwise_finite_differences_tiny():
    rng = np.random.default_rng(7)
    p = _problem(rng, 1, 1, 3, 3, 3, 2, 3, True)
    dY = rng.standard_normal(p["V"].shape)
    g = _grads(p, dY)
    h = 1e-6
    for name, key in (("Q", "dq"), ("K", "dk"), ("V", "dv"), ("weights", "dweights")):
        x = p[name]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            e = np.zeros_like(x)
            e[idx] = h
            fd[idx] = (_loss(p, dY, **{name: x + e}) - _loss(p, dY, **{name: x - e})) / (2 * h)
        assert np.max(np.abs(fd - g[key])) <= 1e-7 * max(1.0, np.max(np.abs(fd))), name


def _dense_powers(q, k, eps, T):
    """S = diag(r) phi(Q) phi(K)^T formed explicitly, and S^0 .. S^(T-1)."""
    qp, kp = np.maximum(q, 0), np.maximum(k, 0)
    S = (qp @ kp.T) / (qp @ kp.sum(0) + eps)[:, None]
    out = [np.eye(len(q))]
    for _ in range(1, T):
        out.append(out[-1] @ S)
    return out


@pytest.mark.parametrize("seed", range(4))
def test_linear_parts_against_dense_powers(seed):
    """alpha = 1: dV = sum_k (S^k)^T diag(w_k) dY and dw_k(i) = dY_i . (S^k V)_i."""
    rng = np.random.default_rng(100 + seed)
    T = int(rng.integers(1, 7))
    p = _problem(rng, 1, 1, 4, 6, 5, 3, T, True)
    p["alpha"] = np.ones(1)
    dY = rng.standard_normal(p["V"].shape)
    g = _grads(p, dY)
    q, k, v, w, dy = p["Q"][0, 0], p["K"][0, 0], p["V"][0, 0], p["weights"][0, 0], dY[0, 0]
    Sk = _dense_powers(q, k, p["eps"], T)
    dv = sum(Sk[j].T @ (w[:, j : j + 1] * dy) for j in range(T))
    dw = np.stack([(dy * (Sk[j] @ v)).sum(1) for j in range(T)], axis=1)
    assert np.allclose(g["dv"][0, 0], dv, rtol=1e-11, atol=1e-12)
    assert np.allclose(g["dweights"][0, 0], dw, rtol=1e-11, atol=1e-12)


def test_alpha_gradient_and_branch_isolation():
    rng = np.random.default_rng(3)
    p = _problem(rng, 2, 2, 5, 4, 4, 4, 3, True)
    dY = rng.standard_normal(p["V"].shape)
    g = _grads(p, dY)
    G = np.empty_like(p["V"])
    L = np.empty_like(p["V"])
    for b in range(2):
        for h in range(2):
            G[b, h] = olisa.global_branch(p["Q"][b, h], p["K"][b, h], p["V"][b, h], p["weights"][b, h], p["eps"])
            L[b, h] = olisa.local_branch(p["Q"][b, h], p["K"][b, h], p["V"][b, h], 5, 4)
    assert np.allclose(g["dalpha"], (dY * (G - L)).sum(axis=(0, 2, 3)), rtol=1e-12)
    # alpha = 0: only the local branch, whose gradient ignores the weights.
    g0 = _grads(dict(p, alpha=np.zeros(2)), dY)
    assert np.all(g0["dweights"] == 0)
    # alpha = 1: only the global branch; T = 1 there leaves w_0 V alone.
    g1 = _grads(dict(p, alpha=np.ones(2), T=1, weights=p["weights"][..., :1]), dY)
    assert np.all(g1["dq"] == 0) and np.all(g1["dk"] == 0)
    assert np.allclose(g1["dv"], p["weights"][..., :1] * dY, rtol=0, atol=0)


def test_local_branch_single_cell_window():
    """A 1 x 1 grid: L = V whatever Q and K are, so dQ = dK = 0 and dV = dL."""
    rng = np.random.default_rng(9)
    q, k, v, dl = (rng.standard_normal((1, 4)) for _ in range(4))
    dq, dk, dv = oback.local_branch_backward(q, k, v, 1, 1, dl)
    assert np.all(dq == 0) and np.all(dk == 0) and np.allclose(dv, dl)


# --------------------------------------------------------------------------
# Planted mistakes: each edit below is a plausible slip in the adjoint; a
# patched copy of the module must fail the finite-difference pin.
# --------------------------------------------------------------------------
MISTAKES = {
    "drop ds": ("    dKp += ds[None, :]\n", "    pass\n"),
    "sign of dz": ("    dz = -(r * r) * dr", "    dz = (r * r) * dr"),
    "no M^T propagation": ("        dP[k - 1] = dP[k - 1] + M.T @ dP[k]", "        dP[k - 1] = dP[k - 1]"),
    "M instead of M^T": ("        dP[k - 1] = dP[k - 1] + M.T @ dP[k]", "        dP[k - 1] = dP[k - 1] + M @ dP[k]"),
    "softmax centring": ("    dz = p * (dLv - (dLg * L).sum(-1, keepdims=True))", "    dz = p * dLv"),
    "local scale": ("            g = dz[r0:r1, c0:c1, t : t + 1] * sc", "            g = dz[r0:r1, c0:c1, t : t + 1]"),
    "relu mask of K": ("    dK = dKp * (K > 0.0)", "    dK = dKp"),
}


def _patched_module(old, new):
    import types

    src = inspect.getsource(oback)
    assert src.count(old) == 1, old
    mod = types.ModuleType("oracle.backward_mutant")
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), "<mutant>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("mistake", sorted(MISTAKES))
def test_planted_mistakes_are_caught(mistake):
    mod = _patched_module(*MISTAKES[mistake])
    rng = np.random.default_rng(11)
    p = _problem(rng, 1, 1, 4, 5, 5, 4, 4, True)
    dY = rng.standard_normal(p["V"].shape)
    g = _grads(p, dY, module=mod)
    h = 1e-6
    worst = 0.0
    for name, key in (("Q", "dq"), ("K", "dk"), ("V", "dv")):
        D = rng.standard_normal(p[name].shape)
        fd = (_loss(p, dY, **{name: p[name] + h * D}) - _loss(p, dY, **{name: p[name] - h * D})) / (2 * h)
        an = float((g[key] * D).sum())
        worst = max(worst, abs(fd - an) / max(1.0, abs(an)))
    assert worst > 1e-4, f"{mistake} not caught ({worst:.2e})"
