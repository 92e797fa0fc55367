"""LiSA forward pass: float64 CPU reference (test infrastructure only).

Source.  "[note §x]" cites the web page "LiSA:面向长程视觉建模的线性随机注意力",
a reading note of "LiSA: Linear Stochastic Attention for Long-Range Visual
Modeling" (arXiv:2611.04216v2), by the note's own section number, with the
paper's equation / table numbers as the note quotes them.  The note lost every
display formula in extraction; each formula below is the plainest reading of
the surrounding prose, and the readings are listed here:

  R1  phi = ReLU, applied to Q and K of the global branch only [note §2.1].
      The local branch uses Q and K as given (the note does not say it uses
      phi there).  The alternative the note's supplementary comparison names
      (ELU, Table 8) is read as phi(x) = ELU(x) + 1 = x + 1 (x > 0), e^x
      (x <= 0): the shift keeps every feature positive, so S stays a
      row-stochastic walk matrix; ELU alone could make row sums vanish.
  R2  s = sum_j phi(K_j); r_i = 1 / (phi(Q_i) . s + eps); Qt = diag(r) phi(Q);
      S = Qt phi(K)^T.  The note only says a tiny stabilising term is ignored
      when calling S row-stochastic [note §2.2]; eps sits in the row
      denominator.
  R3  The walk is truncated to T terms k = 0..T-1, term 0 being S^0 = I
      (with T = 1 only the self loop S^0 = I remains) [note §2.2].
  R4  Geometric weights w_k = (1-beta) beta^k / (1-beta^T): the geometric
      series of a walk that continues with probability beta, renormalised by
      1/(1-beta^T) over the first T terms [note §2.2, Eq. 4; §2.5].
  R5  Adaptive weights beta_k(i) are per token and per head [note §2.4,
      Eq. 10]; weight k of token i multiplies row i of S^k V.  They are used
      as given, without renormalisation.
  R6  Local branch: masked exponential similarity exp(q_i . k_j / sqrt(d_h))
      over token i itself and its (up to 8) spatial neighbours in the 3x3
      window, row-normalised [note §2.4, Fig. 2].  The note gives no scale;
      the usual 1/sqrt(d_h) of dot-product attention is taken.
  R7  Windows are clipped at the grid border (no padding tokens, no
      wrap-around): corners have 4 cells, edges 6, interior 9.
  R8  The row maximum is subtracted before exp (mathematically identical).
  R9  Y = alpha * G + (1 - alpha) * L with one learnable alpha per head; the
      alpha ablation's "global only" end is alpha = 1 and "local only" is
      alpha = 0 [note §2.4; §4.4, Table 6].
  R10 Tokens are in row-major grid order, i = row * W + col, n = H * W; there
      is no class token.  Tensors are [B, heads, n, d].

What pins this module (tests/test_oracle_pins.py): the low-rank recurrence
against explicit n x n powers of S; the local branch three ways (vectorised,
explicit loop, dense masked softmax from scipy); row sums of S; the walk-mass
proposition [note §2.5]; the untruncated closed form (1-beta)(I - beta S)^-1 V
[note §2.3]; the T = 1 identity; the one-hop case against textbook normalised
linear attention [note §2.1, Eq. 3]; invariants (constant V, linearity in V,
permutation equivariance); and hand-derived examples in tests/golden/.
Parity unpinned: the note prints no numeric input/output example, so that the
readings R1-R10 are the paper's exact formulas rests on the prose alone.
"""

import math

import numpy as np

__all__ = [
    "feature_map",
    "geometric_weights",
    "walk_weights",
    "normaliser",
    "stats",
    "global_branch",
    "neighbour_offsets",
    "local_branch",
    "local_branch_loop",
    "mix",
    "lisa_forward",
    "lisa_bruteforce",
]


FEATURES = ("relu", "elu")


def feature_map(x, feature="relu"):
    """phi(x): ReLU(x), the default non-negative feature map [note §2.1], or
    ELU(x) + 1 with feature="elu" (the supplementary alternative, Table 8)."""
    x = np.asarray(x, dtype=np.float64)
    if feature == "relu":
        return np.maximum(x, 0.0)
    if feature == "elu":
        return np.where(x > 0.0, x + 1.0, np.exp(np.minimum(x, 0.0)))
    raise ValueError(f"feature must be one of {FEATURES}")


def geometric_weights(beta, T):
    """w_k = (1-beta) beta^k / (1-beta^T) for k = 0..T-1 [note §2.2, Eq. 4].

    A walk continues with probability beta and stops with 1-beta; keeping the
    first T path lengths and dividing by their total mass 1-beta^T makes the
    weights sum to one [note §2.5].
    """
    if not (0.0 <= beta < 1.0):
        raise ValueError("beta must lie in [0, 1)")
    if T < 1:
        raise ValueError("T must be >= 1")
    k = np.arange(T, dtype=np.float64)
    return (1.0 - beta) * np.power(float(beta), k) / (1.0 - float(beta) ** T)


def walk_weights(n, T, weights=None, beta=None):
    """Per-token step weights, shape [n, T].

    Adaptive weights beta_k(i) are given per token [note §2.4, Eq. 10] and
    used as they are; otherwise the geometric weights of ``beta`` are shared by
    every token.
    """
    if weights is not None:
        w = np.asarray(weights, dtype=np.float64)
        if w.shape != (n, T):
            raise ValueError(f"weights must be [{n}, {T}], got {w.shape}")
        return w
    if beta is None:
        raise ValueError("give either adaptive weights or beta")
    return np.broadcast_to(geometric_weights(beta, T), (n, T))


def normaliser(Q, K, eps, feature="relu"):
    """Column sum s of phi(K) and row normaliser r of one (batch, head) slice.

    s = sum_j phi(K_j) and r_i = 1 / (phi(Q_i) . s + eps), so that
    Qt = diag(r) phi(Q) turns S = Qt phi(K)^T into a row-stochastic matrix up
    to the eps term [note §2.2].  Returns (phi(Q), phi(K), s, r).
    """
    Qp = feature_map(Q, feature)
    Kp = feature_map(K, feature)
    s = Kp.sum(axis=0)
    r = 1.0 / (Qp @ s + eps)
    return Qp, Kp, s, r


def stats(Q, K, V, eps, feature="relu"):
    """The d_h-space statistics of one slice: (s, K^T V, M = K^T Qt).

    These are the only quantities that depend on all tokens [note §2.3,
    Eq. 8]: K^T V (d_h x d_v) and M = phi(K)^T Qt (d_h x d_h), never the
    n x n matrix S.
    """
    V = np.asarray(V, dtype=np.float64)
    Qp, Kp, s, r = normaliser(Q, K, eps, feature)
    Qt = r[:, None] * Qp
    return s, Kp.T @ V, Kp.T @ Qt


def global_branch(Q, K, V, w, eps, feature="relu"):
    """G = sum_{k<T} diag(w[:, k]) S^k V for one slice, without forming S.

    Uses S^k V = Qt M^(k-1) (K^T V) for k >= 1 [note §2.3, Eq. 8]: the
    d_h x d_h power chain P_1 = K^T V, P_k = M P_(k-1) is built in feature
    space, and each term is one token-dimension projection Qt P_k added with
    its weight, as the paper's Algorithm 1 does per truncation term.  Term 0
    is S^0 V = V [note §2.2].
    """
    V = np.asarray(V, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    T = w.shape[1]
    Qp, Kp, s, r = normaliser(Q, K, eps, feature)
    Qt = r[:, None] * Qp
    M = Kp.T @ Qt
    P = Kp.T @ V  # P_1
    G = w[:, 0:1] * V
    for k in range(1, T):
        G = G + w[:, k : k + 1] * (Qt @ P)
        P = M @ P
    return G


def neighbour_offsets():
    """The 3x3 window: (d_row, d_col) for d_row, d_col in {-1, 0, 1} [note §2.4]."""
    return [(dr, dc) for dr in (-1, 0, 1) for dc in (-1, 0, 1)]


def local_branch(Q, K, V, H, W):
    """3x3 local attention of one slice, vectorised with shifted grid slices.

    L_i = sum_{j in N(i)} e_ij V_j / sum_{j in N(i)} e_ij with
    e_ij = exp(q_i . k_j / sqrt(d_h)), N(i) the valid cells of the 3x3 window
    around token i, self included [note §2.4, Fig. 2].  Readings R6-R8.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    n, dh = Q.shape
    dv = V.shape[1]
    if n != H * W:
        raise ValueError("n must equal H * W")
    Qg = Q.reshape(H, W, dh)
    Kg = K.reshape(H, W, dh)
    Vg = V.reshape(H, W, dv)
    offs = neighbour_offsets()
    logits = np.full((H, W, len(offs)), -np.inf)
    values = np.zeros((H, W, len(offs), dv))
    for t, (dr, dc) in enumerate(offs):
        # Centre cells whose neighbour (row+dr, col+dc) lies on the grid.
        r0, r1 = max(0, -dr), min(H, H - dr)
        c0, c1 = max(0, -dc), min(W, W - dc)
        if r0 >= r1 or c0 >= c1:
            continue
        kc = Kg[r0 + dr : r1 + dr, c0 + dc : c1 + dc]
        logits[r0:r1, c0:c1, t] = (Qg[r0:r1, c0:c1] * kc).sum(-1) / math.sqrt(dh)
        values[r0:r1, c0:c1, t] = Vg[r0 + dr : r1 + dr, c0 + dc : c1 + dc]
    m = logits.max(axis=-1, keepdims=True)
    e = np.exp(logits - m)  # exp(-inf) = 0 drops the cells off the grid
    p = e / e.sum(axis=-1, keepdims=True)
    L = (p[..., None] * values).sum(axis=2)
    return L.reshape(n, dv)


def local_branch_loop(Q, K, V, H, W):
    """The same 3x3 local attention, one token and one neighbour at a time.

    Pure Python loops; for tiny grids only.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    n, dh = Q.shape
    L = np.zeros((n, V.shape[1]))
    for row in range(H):
        for col in range(W):
            i = row * W + col
            nbrs = []
            for rr in range(row - 1, row + 2):
                for cc in range(col - 1, col + 2):
                    if 0 <= rr < H and 0 <= cc < W:
                        nbrs.append(rr * W + cc)
            sims = [float(np.dot(Q[i], K[j])) / math.sqrt(dh) for j in nbrs]
            top = max(sims)
            ex = [math.exp(x - top) for x in sims]
            tot = sum(ex)
            for e_j, j in zip(ex, nbrs):
                L[i] += (e_j / tot) * V[j]
    return L


def mix(G, L, alpha):
    """Y = alpha G + (1 - alpha) L [note §2.4; alpha endpoints of Table 6]."""
    return alpha * G + (1.0 - alpha) * L


def _check(Q, K, V, H, W, T, alpha, weights, beta):
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if Q.ndim != 4 or K.shape != Q.shape or V.shape[:3] != Q.shape[:3]:
        raise ValueError("Q, K must be [B, heads, n, d_h] and V [B, heads, n, d_v]")
    B, heads, n, _ = Q.shape
    if n != H * W:
        raise ValueError("n must equal H * W")
    alpha = np.broadcast_to(np.asarray(alpha, dtype=np.float64), (heads,))
    if weights is not None:
        weights = np.asarray(weights, dtype=np.float64)
        if weights.shape != (B, heads, n, T):
            raise ValueError("weights must be [B, heads, n, T]")
    elif beta is None:
        raise ValueError("give either adaptive weights or beta")
    return Q, K, V, alpha, weights


def lisa_forward(Q, K, V, *, H, W, T, alpha, weights=None, beta=None, eps=1e-6, feature="relu"):
    """LiSA forward pass, [B, heads, n, d] float64 in and out.

    Per (batch, head): global branch (low-rank form), local branch, alpha-mix.
    ``weights`` are adaptive per-token weights [B, heads, n, T]; without them
    the geometric weights of ``beta`` are used.  ``alpha`` has one entry per
    head.  ``feature`` picks phi of the global branch ("relu" or "elu").
    """
    Q, K, V, alpha, weights = _check(Q, K, V, H, W, T, alpha, weights, beta)
    B, heads, n, _ = Q.shape
    Y = np.empty((B, heads, n, V.shape[-1]))
    for b in range(B):
        for h in range(heads):
            w = walk_weights(n, T, None if weights is None else weights[b, h], beta)
            G = global_branch(Q[b, h], K[b, h], V[b, h], w, eps, feature)
            L = local_branch(Q[b, h], K[b, h], V[b, h], H, W)
            Y[b, h] = mix(G, L, alpha[h])
    return Y


def lisa_bruteforce(Q, K, V, *, H, W, T, alpha, weights=None, beta=None, eps=1e-6, feature="relu"):
    """The same forward pass with every n x n matrix formed explicitly.

    Global: S = Qt phi(K)^T built densely [note §2.2] and its powers S^k by
    repeated dense products; G = sum_k diag(w_k) S^k V.  Local: a dense n x n
    logit matrix q_i . k_j / sqrt(d_h), masked to the 3x3 window by grid
    coordinates, normalised row-wise by scipy's softmax.  For tiny grids only.
    """
    from scipy.special import softmax

    Q, K, V, alpha, weights = _check(Q, K, V, H, W, T, alpha, weights, beta)
    B, heads, n, dh = Q.shape
    rows = np.arange(n) // W
    cols = np.arange(n) % W
    window = (np.abs(rows[:, None] - rows[None, :]) <= 1) & (
        np.abs(cols[:, None] - cols[None, :]) <= 1
    )
    Y = np.empty((B, heads, n, V.shape[-1]))
    for b in range(B):
        for h in range(heads):
            q, k, v = Q[b, h], K[b, h], V[b, h]
            w = walk_weights(n, T, None if weights is None else weights[b, h], beta)
            if feature == "relu":
                qp, kp = np.maximum(q, 0.0), np.maximum(k, 0.0)
            elif feature == "elu":
                # ELU(x) + 1, written from its definition: alpha (e^x - 1) below zero, x above.
                qp = np.where(q > 0, q, np.expm1(np.minimum(q, 0.0))) + 1.0
                kp = np.where(k > 0, k, np.expm1(np.minimum(k, 0.0))) + 1.0
            else:
                raise ValueError("unknown feature map")
            S = (qp @ kp.T) / (qp @ kp.sum(axis=0) + eps)[:, None]
            Sk = np.eye(n)
            G = np.zeros_like(v)
            for step in range(T):
                G += w[:, step : step + 1] * (Sk @ v)
                Sk = Sk @ S
            logits = np.where(window, (q @ k.T) / math.sqrt(dh), -np.inf)
            A = softmax(logits, axis=1)
            L = A @ v
            Y[b, h] = alpha[h] * G + (1.0 - alpha[h]) * L
    return Y
