"""LiSA backward pass: float64 CPU reference (test infrastructure only).

The gradients of ``oracle.lisa.lisa_forward``'s output, contracted with an
output gradient dY, with respect to Q, K, V, the adaptive walk weights and
alpha.  The reading note trains every model it reports [note §3] and chooses
the truncation T with the cost of backpropagation in mind [note §2.3]; it
prints no backward formulas.  The derivative of the forward pass is exact, so
this module is that derivative written out: the adjoint of each forward step,
taken in reverse order, in the forward's notation (see ``oracle.lisa``):

  forward (one slice)                     adjoint
  phi(Q), phi(K)     ReLU                 d/dx max(x, 0) = 1 for x > 0, else 0
  s = sum_j phi(K_j)                      dphi(K_j) += ds
  r_i = 1 / (phi(Q_i).s + eps)            d(phi(Q_i).s) = -r_i^2 dr_i
  Qt_i = r_i phi(Q_i)                     dphi(Q_i) += r_i dQt_i, dr_i = dQt_i.phi(Q_i)
  M = phi(K)^T Qt,  P_1 = phi(K)^T V      dphi(K) += Qt dM^T + V dP_1^T,
                                          dQt += phi(K) dM, dV += phi(K) dP_1
  P_k = M P_(k-1)                         dM += dP_k P_(k-1)^T, dP_(k-1) += M^T dP_k
  G = w_0 V + sum_k w_k Qt P_k            dV += w_0 dG, dQt += sum_k w_k dG P_k^T,
                                          dP_k = Qt^T diag(w_k) dG,
                                          dw_k(i) = dG_i . (Qt P_k)_i
  L_i = sum_j p_ij V_j, p = softmax_j(q_i.k_j / sqrt(d_h)) over the 3x3 window
                                          dz_ij = p_ij (dL_i.V_j - dL_i.L_i),
                                          dq_i += sum_j dz_ij k_j / sqrt(d_h),
                                          dk_j += sum_i dz_ij q_i / sqrt(d_h),
                                          dV_j += sum_i p_ij dL_i
  Y = alpha G + (1 - alpha) L             dG = alpha dY, dL = (1 - alpha) dY,
                                          dalpha = sum dY (G - L)

Reading (in addition to oracle.lisa's R1-R10):
  B1  The ReLU's derivative at exactly 0 is taken as 0.
  B2  With geometric weights the weights are not an input: no weight
      gradient is formed (beta's gradient is out of scope).

What pins this module (tests/test_oracle_pins.py): central finite differences
of ``oracle.lisa.lisa_forward`` along random directions for every input and
element-wise on a tiny grid; dV and the weight gradients against explicit
n x n powers of S (G is linear in V and in the weights); alpha's gradient
against G - L; and the branch isolation alpha = 0 / 1.
"""

import math

import numpy as np

from .lisa import _check, neighbour_offsets, walk_weights

__all__ = ["global_branch_backward", "local_branch_backward", "lisa_backward"]


def global_branch_backward(Q, K, V, w, eps, dG):
    """Gradients of the global branch G of one slice (``oracle.lisa.global_branch``).

    Returns (dQ, dK, dV, dw) for dG = dLoss/dG, each with the shape of its
    input (dw: [n, T]).  The forward quantities are recomputed in float64.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    dG = np.asarray(dG, dtype=np.float64)
    T = w.shape[1]
    # Forward [note §2.2, §2.3].
    Qp = np.maximum(Q, 0.0)
    Kp = np.maximum(K, 0.0)
    s = Kp.sum(axis=0)
    r = 1.0 / (Qp @ s + eps)
    Qt = r[:, None] * Qp
    M = Kp.T @ Qt
    P = [None, Kp.T @ V]  # P[k] = M^(k-1) phi(K)^T V, k >= 1
    for k in range(2, T):
        P.append(M @ P[k - 1])
    # G = w_0 V + sum_k w_k Qt P_k.
    dw = np.zeros_like(w)
    dw[:, 0] = (dG * V).sum(axis=1)
    dV = w[:, 0:1] * dG
    dQt = np.zeros_like(Qt)
    dP = [None] + [None] * (T - 1)
    for k in range(1, T):
        dw[:, k] = (dG * (Qt @ P[k])).sum(axis=1)
        dQt += (w[:, k : k + 1] * dG) @ P[k].T
        dP[k] = Qt.T @ (w[:, k : k + 1] * dG)
    # P_k = M P_(k-1), from the last term down.
    dM = np.zeros_like(M)
    for k in range(T - 1, 1, -1):
        dM += dP[k] @ P[k - 1].T
        dP[k - 1] = dP[k - 1] + M.T @ dP[k]
    # M = phi(K)^T Qt and P_1 = phi(K)^T V.
    dKp = np.zeros_like(Kp)
    if T >= 2:
        dKp += Qt @ dM.T + V @ dP[1].T
        dQt += Kp @ dM
        dV += Kp @ dP[1]
    # Qt = diag(r) phi(Q), r = 1 / (phi(Q) s + eps).
    dr = (dQt * Qp).sum(axis=1)
    dz = -(r * r) * dr  # d(phi(Q_i) . s)
    dQp = r[:, None] * dQt + dz[:, None] * s[None, :]
    ds = Qp.T @ dz
    # s = sum_j phi(K_j).
    dKp += ds[None, :]
    dQ = dQp * (Q > 0.0)
    dK = dKp * (K > 0.0)
    return dQ, dK, dV, dw


def local_branch_backward(Q, K, V, H, W, dL):
    """Gradients of the 3x3 local branch of one slice (``oracle.lisa.local_branch``).

    Returns (dQ, dK, dV) for dL = dLoss/dL, with the same shifted-slice
    arrangement as the forward: slot t of a token is its neighbour at
    offset t, absent (probability 0) off the grid [note §2.4].
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    dL = np.asarray(dL, dtype=np.float64)
    n, dh = Q.shape
    dv = V.shape[1]
    sc = 1.0 / math.sqrt(dh)
    Qg, Kg, Vg, dLg = Q.reshape(H, W, dh), K.reshape(H, W, dh), V.reshape(H, W, dv), dL.reshape(H, W, dv)
    offs = neighbour_offsets()
    logits = np.full((H, W, len(offs)), -np.inf)
    spans = []
    for t, (dr, dc) in enumerate(offs):
        r0, r1 = max(0, -dr), min(H, H - dr)
        c0, c1 = max(0, -dc), min(W, W - dc)
        spans.append((r0, r1, c0, c1))
        if r0 < r1 and c0 < c1:
            kc = Kg[r0 + dr : r1 + dr, c0 + dc : c1 + dc]
            logits[r0:r1, c0:c1, t] = (Qg[r0:r1, c0:c1] * kc).sum(-1) * sc
    m = logits.max(axis=-1, keepdims=True)
    e = np.exp(logits - m)
    p = e / e.sum(axis=-1, keepdims=True)  # [H, W, 9]
    # L_i, then dL_i . V_j for every slot.
    L = np.zeros((H, W, dv))
    dLv = np.zeros((H, W, len(offs)))
    for t, (dr, dc) in enumerate(offs):
        r0, r1, c0, c1 = spans[t]
        if r0 < r1 and c0 < c1:
            vc = Vg[r0 + dr : r1 + dr, c0 + dc : c1 + dc]
            L[r0:r1, c0:c1] += p[r0:r1, c0:c1, t : t + 1] * vc
            dLv[r0:r1, c0:c1, t] = (dLg[r0:r1, c0:c1] * vc).sum(-1)
    dz = p * (dLv - (dLg * L).sum(-1, keepdims=True))
    dQ = np.zeros_like(Qg)
    dK = np.zeros_like(Kg)
    dV = np.zeros_like(Vg)
    for t, (dr, dc) in enumerate(offs):
        r0, r1, c0, c1 = spans[t]
        if r0 < r1 and c0 < c1:
            g = dz[r0:r1, c0:c1, t : t + 1] * sc
            dQ[r0:r1, c0:c1] += g * Kg[r0 + dr : r1 + dr, c0 + dc : c1 + dc]
            dK[r0 + dr : r1 + dr, c0 + dc : c1 + dc] += g * Qg[r0:r1, c0:c1]
            dV[r0 + dr : r1 + dr, c0 + dc : c1 + dc] += p[r0:r1, c0:c1, t : t + 1] * dLg[r0:r1, c0:c1]
    return dQ.reshape(n, dh), dK.reshape(n, dh), dV.reshape(n, dv)


def lisa_backward(Q, K, V, *, H, W, T, alpha, dY, weights=None, beta=None, eps=1e-6):
    """Gradients of ``oracle.lisa.lisa_forward`` for the output gradient dY.

    Returns a dict with "dq", "dk", "dv" ([B, heads, n, d]), "dweights"
    ([B, heads, n, T], None with geometric weights) and "dalpha" ([heads]),
    all float64.
    """
    from .lisa import global_branch, local_branch

    Q, K, V, alpha, weights = _check(Q, K, V, H, W, T, alpha, weights, beta)
    dY = np.asarray(dY, dtype=np.float64)
    B, heads, n, _ = Q.shape
    if dY.shape != V.shape:
        raise ValueError("dY must have the shape of V")
    dq, dk, dv = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    dw = None if weights is None else np.zeros_like(weights)
    dalpha = np.zeros(heads)
    for b in range(B):
        for h in range(heads):
            q, k, v, dy = Q[b, h], K[b, h], V[b, h], dY[b, h]
            w = walk_weights(n, T, None if weights is None else weights[b, h], beta)
            G = global_branch(q, k, v, w, eps)
            L = local_branch(q, k, v, H, W)
            dalpha[h] += (dy * (G - L)).sum()
            gq, gk, gv, gw = global_branch_backward(q, k, v, w, eps, alpha[h] * dy)
            lq, lk, lv = local_branch_backward(q, k, v, H, W, (1.0 - alpha[h]) * dy)
            dq[b, h] = gq + lq
            dk[b, h] = gk + lk
            dv[b, h] = gv + lv
            if dw is not None:
                dw[b, h] = gw
    return {"dq": dq, "dk": dk, "dv": dv, "dweights": dw, "dalpha": dalpha}
