"""Pins of the LiSA attention layer oracle (oracle/layer.py), CPU only.

- PyTorch's linear, view and permute in float64 around the operator oracle
  (itself pinned by tests/test_oracle_pins.py).
- Closed forms: identity projections give the operator on X's heads; V = 0
  (its projection rows zero) gives Y = bo exactly; a permutation of the heads
  (rows of Wqkv and columns of Wo, with alpha and the weights) leaves Y alone.
- Planted mistakes (in a patched copy, on the CPU) each fail a pin.
"""

import inspect
import types

import numpy as np
import pytest
import torch

from oracle import layer as olayer
from oracle import lisa as olisa


def _problem(rng, B, heads, H, W, T, dh=8, adaptive=True):
    C, n = heads * dh, H * W
    p = dict(
        X=rng.standard_normal((B, n, C)),
        Wqkv=rng.standard_normal((3 * C, C)) / np.sqrt(C),
        bqkv=rng.standard_normal(3 * C) * 0.1,
        Wo=rng.standard_normal((C, C)) / np.sqrt(C),
        bo=rng.standard_normal(C) * 0.1,
    )
    kw = dict(heads=heads, H=H, W=W, T=T, alpha=rng.uniform(0, 1, heads))
    if adaptive:
        lg = rng.standard_normal((B, heads, n, T))
        kw["weights"] = np.exp(lg) / np.exp(lg).sum(-1, keepdims=True)
    else:
        kw["beta"] = 0.5
    return p, kw


@pytest.mark.parametrize("case", [(2, 3, 4, 5, 3, True), (1, 1, 6, 6, 1, False), (3, 2, 1, 7, 5, True)])
def test_against_torch(case, module=olayer):
    B, heads, H, W, T, adaptive = case
    rng = np.random.default_rng(sum(case))
    p, kw = _problem(rng, B, heads, H, W, T, adaptive=adaptive)
    y = module.lisa_layer(**p, **kw)
    F = torch.nn.functional
    t = {k: torch.from_numpy(v) for k, v in p.items()}
    C, n = t["X"].shape[-1], H * W
    q, k, v = F.linear(t["X"], t["Wqkv"], t["bqkv"]).split(C, dim=-1)
    hs = lambda z: z.view(B, n, heads, C // heads).permute(0, 2, 1, 3).numpy()  # noqa: E731
    o = olisa.lisa_forward(hs(q), hs(k), hs(v), H=H, W=W, T=T, alpha=kw["alpha"], weights=kw.get("weights"),
                           beta=kw.get("beta"))
    o = torch.from_numpy(o).permute(0, 2, 1, 3).reshape(B, n, C)
    ref = F.linear(o, t["Wo"], t["bo"]).numpy()
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-13)


def test_identity_projections():
    rng = np.random.default_rng(1)
    p, kw = _problem(rng, 2, 2, 4, 4, 3)
    C = p["X"].shape[-1]
    eye = np.eye(C)
    y = olayer.lisa_layer(p["X"], np.vstack([eye, eye, eye]), np.zeros(3 * C), eye, np.zeros(C), **kw)
    xs = p["X"].reshape(2, 16, 2, C // 2).transpose(0, 2, 1, 3)
    ref = olisa.lisa_forward(xs, xs, xs, H=4, W=4, T=3, alpha=kw["alpha"], weights=kw["weights"])
    assert np.allclose(y, ref.transpose(0, 2, 1, 3).reshape(2, 16, C), rtol=1e-13, atol=1e-14)


def test_zero_values_give_the_output_bias():
    rng = np.random.default_rng(2)
    p, kw = _problem(rng, 2, 3, 5, 4, 4)
    C = p["X"].shape[-1]
    p["Wqkv"][2 * C:] = 0
    p["bqkv"][2 * C:] = 0
    y = olayer.lisa_layer(**p, **kw)
    assert np.all(y == np.broadcast_to(p["bo"], y.shape))


def test_head_permutation():
    rng = np.random.default_rng(3)
    heads, dh = 3, 8
    p, kw = _problem(rng, 2, heads, 4, 6, 3, dh=dh)
    perm = np.array([2, 0, 1])
    ch = np.concatenate([np.arange(h * dh, (h + 1) * dh) for h in perm])
    C = heads * dh
    rows = np.concatenate([ch, C + ch, 2 * C + ch])
    kw2 = dict(kw, alpha=kw["alpha"][perm], weights=kw["weights"][:, perm])
    y2 = olayer.lisa_layer(p["X"], p["Wqkv"][rows], p["bqkv"][rows], p["Wo"][:, ch], p["bo"], **kw2)
    assert np.allclose(olayer.lisa_layer(**p, **kw), y2, rtol=1e-12, atol=1e-13)


MISTAKES = {
    "heads interleaved": ("return t.reshape(B, n, heads, C // heads).transpose(0, 2, 1, 3)",
                          "return t.reshape(B, n, C // heads, heads).transpose(0, 3, 1, 2)"),
    "k and v swapped": ("q, k, v = (split_heads(", "q, v, k = (split_heads("),
    "no output bias": ("@ np.asarray(Wo, np.float64).T + np.asarray(bo, np.float64)", "@ np.asarray(Wo, np.float64).T"),
    "Wo not transposed": ("@ np.asarray(Wo, np.float64).T +", "@ np.asarray(Wo, np.float64) +"),
}


@pytest.mark.parametrize("mistake", sorted(MISTAKES))
def test_planted_mistakes_are_caught(mistake):
    old, new = MISTAKES[mistake]
    src = inspect.getsource(olayer)
    assert src.count(old) == 1, old
    mod = types.ModuleType("oracle.layer_mutant")
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), "<mutant>", "exec"), mod.__dict__)
    with pytest.raises(AssertionError):
        test_against_torch((2, 3, 4, 5, 3, True), module=mod)
