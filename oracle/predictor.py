"""LiSA's per-token walk-weight predictor: float64 CPU reference (test
infrastructure only; only tests/, smoke() and bench.py's cpu_baseline may
import it).

Source: the reading note "LiSA:面向长程视觉建模的线性随机注意力" of
"LiSA: Linear Stochastic Attention for Long-Range Visual Modeling"
(arXiv:2611.04216v2), §2.4 (Eq. 10; supplementary Sec. 8): the adaptive
weights beta_k are predicted for every token and every head, from the
token's query and key concatenated, by a small two-layer MLP followed by a
softmax over the T weights.  The note gives no widths, activation or bias;
the readings taken here:

  M1  the input is concat(Q_i, K_i) of the head, query first, the vectors as
      given to the operator (before phi);
  M2  layer 1: h = ReLU(W1 x + b1), the hidden width a free parameter; ReLU is
      the plainest choice (it is also the operator's own feature map);
  M3  layer 2: logits = W2 h + b2 with T outputs, then w = softmax(logits)
      over the T weights of the token;
  M4  each head has its own parameters: W1 [heads, hidden, 2 d_h],
      b1 [heads, hidden], W2 [heads, T, hidden], b2 [heads, T].

Pinned by tests/test_oracle_predictor_pins.py: a hand-worked example
(tests/golden/predictor_hand.json), PyTorch's linear / relu / softmax in
float64, the constant-output and geometric special cases, and planted
mistakes.  Parity unpinned: the note prints no numeric example of the
predictor, so that M1-M4 are the paper's exact network rests on its prose.
"""

import numpy as np

from .lisa import lisa_forward

__all__ = ["predicted_weights", "lisa_forward_mlp"]


def predicted_weights(Q, K, W1, b1, W2, b2):
    """Walk weights [B, heads, n, T] from Q, K [B, heads, n, d_h] (M1-M4)."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    x = np.concatenate([Q, K], axis=-1)                         # [B, h, n, 2 d_h]
    hid = np.einsum("bhnc,hjc->bhnj", x, np.asarray(W1, np.float64))
    hid = np.maximum(hid + np.asarray(b1, np.float64)[None, :, None, :], 0.0)
    logits = np.einsum("bhnj,htj->bhnt", hid, np.asarray(W2, np.float64))
    logits = logits + np.asarray(b2, np.float64)[None, :, None, :]
    logits = logits - logits.max(axis=-1, keepdims=True)
    e = np.exp(logits)
    return e / e.sum(axis=-1, keepdims=True)


def lisa_forward_mlp(Q, K, V, *, H, W, T, alpha, W1, b1, W2, b2, eps=1e-6):
    """The forward pass with the walk weights predicted from Q and K."""
    w = predicted_weights(Q, K, W1, b1, W2, b2)
    assert w.shape[-1] == T, "W2 and b2 must have T outputs"
    return lisa_forward(Q, K, V, H=H, W=W, T=T, alpha=alpha, weights=w, eps=eps)
