"""Pins of the walk-weight predictor oracle (oracle/predictor.py), CPU only.

- A hand-worked example (tests/golden/predictor_hand.json).
- PyTorch's linear, relu and softmax in float64, head by head.
- Special cases: W2 = 0 gives softmax(b2) for every token; with b2 the logs
  of the geometric weights the fused forward equals the geometric forward.
- The weights lie on the simplex.
- Planted mistakes (in a patched copy, on the CPU) each fail a pin.
"""

import inspect
import json
import math
import os
import types

import numpy as np
import pytest
import torch

from oracle import lisa as olisa
from oracle import predictor as opred

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _hand():
    with open(os.path.join(GOLDEN, "predictor_hand.json")) as f:
        g = json.load(f)
    arr = lambda k: np.array(g[k], dtype=np.float64)  # noqa: E731
    Q = arr("Q")[None, None]
    K = arr("K")[None, None]
    return g, Q, K, arr("W1")[None], arr("b1")[None], arr("W2")[None], arr("b2")[None]


def _expected_hand(g):
    out = []
    for l0, l1 in g["logits"]:
        z = math.exp(l1 - l0)
        out.append([1.0 / (1.0 + z), z / (1.0 + z)])
    return np.array(out)


def test_hand_example(module=opred):
    g, Q, K, W1, b1, W2, b2 = _hand()
    w = module.predicted_weights(Q, K, W1, b1, W2, b2)[0, 0]
    assert np.allclose(w, _expected_hand(g), rtol=1e-15, atol=0)


def _random(rng, B, heads, n, dh, hidden, T, scale=0.3):
    Q = rng.standard_normal((B, heads, n, dh))
    K = rng.standard_normal((B, heads, n, dh))
    W1 = rng.standard_normal((heads, hidden, 2 * dh)) * scale
    b1 = rng.standard_normal((heads, hidden)) * scale
    W2 = rng.standard_normal((heads, T, hidden)) * scale
    b2 = rng.standard_normal((heads, T)) * scale
    return Q, K, W1, b1, W2, b2


@pytest.mark.parametrize("shape", [(2, 3, 7, 5, 4, 3), (1, 1, 1, 8, 32, 8), (3, 2, 10, 64, 32, 1)])
def test_against_torch(shape):
    B, heads, n, dh, hidden, T = shape
    rng = np.random.default_rng(sum(shape))
    Q, K, W1, b1, W2, b2 = _random(rng, B, heads, n, dh, hidden, T)
    w = opred.predicted_weights(Q, K, W1, b1, W2, b2)
    F = torch.nn.functional
    for h in range(heads):
        x = torch.cat([torch.from_numpy(Q[:, h]), torch.from_numpy(K[:, h])], dim=-1)
        hid = F.relu(F.linear(x, torch.from_numpy(W1[h]), torch.from_numpy(b1[h])))
        ref = F.softmax(F.linear(hid, torch.from_numpy(W2[h]), torch.from_numpy(b2[h])), dim=-1)
        assert np.allclose(w[:, h], ref.numpy(), rtol=1e-13, atol=1e-15)


def test_simplex():
    rng = np.random.default_rng(5)
    w = opred.predicted_weights(*_random(rng, 2, 2, 50, 16, 32, 5, scale=2.0))
    assert np.all(w > 0) and np.allclose(w.sum(-1), 1.0, rtol=0, atol=1e-14)


def test_constant_output():
    rng = np.random.default_rng(6)
    Q, K, W1, b1, W2, b2 = _random(rng, 2, 3, 9, 8, 32, 4)
    w = opred.predicted_weights(Q, K, W1, b1, 0 * W2, b2)
    for h in range(3):
        e = np.exp(b2[h] - b2[h].max())
        assert np.allclose(w[:, h], e / e.sum(), rtol=1e-14, atol=0)
    assert np.allclose(opred.predicted_weights(Q, K, W1, b1, 0 * W2, 0 * b2), 1 / 4, rtol=1e-15, atol=0)


def test_geometric_special_case():
    """W2 = 0, b2 = log of the geometric weights: the fused forward is the
    geometric forward (an independent path through beta)."""
    rng = np.random.default_rng(7)
    B, heads, H, W, dh, T, beta = 2, 2, 4, 5, 6, 4, 0.6
    n = H * W
    Q, K, W1, b1, W2, b2 = _random(rng, B, heads, n, dh, 32, T)
    V = rng.standard_normal((B, heads, n, dh))
    alpha = rng.uniform(0, 1, heads)
    b2 = np.tile(np.log(olisa.geometric_weights(beta, T)), (heads, 1))
    y = opred.lisa_forward_mlp(Q, K, V, H=H, W=W, T=T, alpha=alpha, W1=W1, b1=b1, W2=0 * W2, b2=b2)
    ref = olisa.lisa_forward(Q, K, V, H=H, W=W, T=T, alpha=alpha, beta=beta)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-13)


MISTAKES = {
    "key first": ("np.concatenate([Q, K], axis=-1)", "np.concatenate([K, Q], axis=-1)"),
    "no relu": ("hid = np.maximum(hid + np.asarray(b1, np.float64)[None, :, None, :], 0.0)",
                "hid = hid + np.asarray(b1, np.float64)[None, :, None, :]"),
    "no b1": ("hid = np.maximum(hid + np.asarray(b1, np.float64)[None, :, None, :], 0.0)",
              "hid = np.maximum(hid, 0.0)"),
    "W2 transposed": ('np.einsum("bhnj,htj->bhnt", hid, np.asarray(W2, np.float64))',
                      'np.einsum("bhnj,hjt->bhnt", hid, np.asarray(W2, np.float64))'),
    "no b2": ("logits = logits + np.asarray(b2, np.float64)[None, :, None, :]", "logits = logits"),
}


@pytest.mark.parametrize("mistake", sorted(MISTAKES))
def test_planted_mistakes_are_caught(mistake):
    old, new = MISTAKES[mistake]
    src = inspect.getsource(opred)
    assert src.count(old) == 1, old
    mod = types.ModuleType("oracle.predictor_mutant")
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), "<mutant>", "exec"), mod.__dict__)
    with pytest.raises(AssertionError):
        test_hand_example(module=mod)
