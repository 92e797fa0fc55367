"""A LiSA attention layer around the operator: float64 CPU reference (test
infrastructure only; only tests/, smoke() and bench.py's cpu_baseline may
import it).

Source: the reading note "LiSA:面向长程视觉建模的线性随机注意力" of
"LiSA: Linear Stochastic Attention for Long-Range Visual Modeling"
(arXiv:2611.04216v2): the operator takes n tokens X in R^{n x d} and
projects them to Q, K, V (§2.1); it is a plug-in module replacing the
attention of DeiT-T and PVT-T (§4, abstract).  The note does not write the
layer out; the readings taken here are those of a ViT attention block:

  A1  one projection with bias gives Q, K, V: [Q | K | V] = X Wqkv^T + bqkv,
      Wqkv [3C, C], C = heads * d_h, in that order;
  A2  head h takes channels h d_h .. (h + 1) d_h - 1 of Q, K and V;
  A3  the heads' outputs are concatenated in the same channel order and
      projected with bias: Y = concat_h(LiSA_h) Wo^T + bo, Wo [C, C];
  A4  K and V keep the token grid of Q (the local branch needs them on the
      same grid; the PVT-T workload is 56 x 56 for all three).

Pinned by tests/test_oracle_layer_pins.py: PyTorch's linear and reshapes in
float64 around the (separately pinned) operator, the identity-projection and
zero-V closed forms, and planted mistakes.  Parity unpinned: the note prints
no layer, so A1-A4 rest on the usual ViT block.
"""

import numpy as np

from .lisa import lisa_forward

__all__ = ["lisa_layer", "split_heads", "merge_heads"]


def split_heads(t, heads):
    """[B, n, C] -> [B, heads, n, C / heads] (A2)."""
    B, n, C = t.shape
    return t.reshape(B, n, heads, C // heads).transpose(0, 2, 1, 3)


def merge_heads(t):
    """[B, heads, n, d] -> [B, n, heads * d] (A3)."""
    B, heads, n, d = t.shape
    return t.transpose(0, 2, 1, 3).reshape(B, n, heads * d)


def lisa_layer(X, Wqkv, bqkv, Wo, bo, *, heads, H, W, T, alpha, weights=None, beta=None, eps=1e-6,
               feature="relu"):
    """Y [B, n, C] of the LiSA attention layer (A1-A4), float64; ``feature``
    is phi of the operator's global branch."""
    X = np.asarray(X, dtype=np.float64)
    C = X.shape[-1]
    qkv = X @ np.asarray(Wqkv, np.float64).T + np.asarray(bqkv, np.float64)
    q, k, v = (split_heads(qkv[..., i * C:(i + 1) * C], heads) for i in range(3))
    y = lisa_forward(q, k, v, H=H, W=W, T=T, alpha=alpha, weights=weights, beta=beta, eps=eps, feature=feature)
    return merge_heads(y) @ np.asarray(Wo, np.float64).T + np.asarray(bo, np.float64)
