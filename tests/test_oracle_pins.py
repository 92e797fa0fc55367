"""Pins of the CPU oracle to facts other than itself (CPU only).

Each test checks oracle/lisa.py against something the reading note or the
mathematics fixes: brute force with explicit n x n matrices, closed forms,
invariants, special cases, and hand-worked examples in tests/golden/.  The
last group plants plausible mistakes in a copy of the oracle and checks that
some pin catches each of them.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import lisa as olisa

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_slice(rng, n, dh, dv, relu=False, scale=1.0):
    Q = rng.standard_normal((n, dh)) * scale
    K = rng.standard_normal((n, dh)) * scale
    V = rng.standard_normal((n, dv))
    if relu:
        Q, K = np.maximum(Q, 0), np.maximum(K, 0)
    return Q, K, V


def _rand_problem(rng, B, heads, H, W, dh, dv, T, adaptive):
    n = H * W
    Q = rng.standard_normal((B, heads, n, dh))
    K = rng.standard_normal((B, heads, n, dh))
    V = rng.standard_normal((B, heads, n, dv))
    alpha = rng.uniform(0, 1, heads)
    if adaptive:
        lg = rng.standard_normal((B, heads, n, T))
        w = np.exp(lg) / np.exp(lg).sum(-1, keepdims=True)
        return dict(Q=Q, K=K, V=V, alpha=alpha, weights=w, beta=None)
    return dict(Q=Q, K=K, V=V, alpha=alpha, weights=None, beta=float(rng.uniform(0, 0.95)))


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# --------------------------------------------------------------------------
# P1: low-rank recurrence == explicit n x n powers (note §2.3, Eq. 8), and
#     vectorised local branch == dense masked softmax (note §2.4).
# --------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(12))
def test_lowrank_equals_bruteforce(seed):
    rng = np.random.default_rng(seed)
    H, W = int(rng.integers(1, 8)), int(rng.integers(1, 8))
    dh = int(rng.choice([1, 2, 8]))
    dv = int(rng.choice([1, 3, 8]))
    T = int(rng.integers(1, 9))
    p = _rand_problem(rng, 2, 2, H, W, dh, dv, T, adaptive=bool(seed % 2))
    a = oracle.lisa_forward(p["Q"], p["K"], p["V"], H=H, W=W, T=T, alpha=p["alpha"],
                            weights=p["weights"], beta=p["beta"], eps=1e-6)
    b = oracle.lisa_bruteforce(p["Q"], p["K"], p["V"], H=H, W=W, T=T, alpha=p["alpha"],
                               weights=p["weights"], beta=p["beta"], eps=1e-6)
    assert _rel(a, b) < 1e-11


def test_lowrank_equals_bruteforce_6x6_deep():
    rng = np.random.default_rng(99)
    for T in (1, 3, 5, 8):
        p = _rand_problem(rng, 1, 1, 6, 6, 8, 8, T, adaptive=True)
        a = oracle.lisa_forward(p["Q"], p["K"], p["V"], H=6, W=6, T=T, alpha=[0.3],
                                weights=p["weights"])
        b = oracle.lisa_bruteforce(p["Q"], p["K"], p["V"], H=6, W=6, T=T, alpha=[0.3],
                                   weights=p["weights"])
        assert _rel(a, b) < 1e-12


# --------------------------------------------------------------------------
# P2: rows of S sum to 1 - eps * r_i (note §2.2: row-stochastic up to the
#     stabilising term).
# --------------------------------------------------------------------------
def test_rows_of_S_sum_to_one_up_to_eps():
    rng = np.random.default_rng(2)
    Q, K, _ = _rand_slice(rng, 50, 16, 4)
    eps = 1e-3
    Qp, Kp, s, r = olisa.normaliser(Q, K, eps)
    S = (r[:, None] * Qp) @ Kp.T
    assert np.all(S >= 0)
    np.testing.assert_allclose(S.sum(axis=1), 1.0 - eps * r, rtol=0, atol=1e-14)
    # rank of S is at most d_h (note §2.2: product of two narrow matrices)
    assert np.linalg.matrix_rank(S) <= 16


# --------------------------------------------------------------------------
# P3: geometric weights, hand values (note §2.2 Eq. 4, §2.5).
# --------------------------------------------------------------------------
def test_geometric_weights_golden():
    with open(os.path.join(GOLDEN, "geometric_weights.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        beta = float(Fraction(case["beta"]))
        w = oracle.geometric_weights(beta, case["T"])
        ref = np.array([float(Fraction(x)) for x in case["w"]])
        np.testing.assert_allclose(w, ref, rtol=1e-15, atol=1e-16)
        assert abs(w.sum() - 1.0) < 1e-15


def test_geometric_weights_rejects_bad_beta():
    with pytest.raises(ValueError):
        oracle.geometric_weights(1.0, 3)
    with pytest.raises(ValueError):
        oracle.geometric_weights(-0.1, 3)


# --------------------------------------------------------------------------
# P4: walk mass (note §2.5, supplement proposition): the entry-wise sum of
#     S^k is n when S is row-stochastic, so the untruncated tail beyond T
#     carries mass n beta^T.
# --------------------------------------------------------------------------
def test_walk_mass_and_tail():
    rng = np.random.default_rng(4)
    n = 30
    Q, K, _ = _rand_slice(rng, n, 6, 1, relu=True)
    Q += 0.05  # no zero rows
    eps = 1e-12
    Qp, Kp, s, r = olisa.normaliser(Q, K, eps)
    S = (r[:, None] * Qp) @ Kp.T
    Sk = np.eye(n)
    for k in range(8):
        assert abs(Sk.sum() - n) < 1e-8
        Sk = Sk @ S
    beta, T = 0.6, 4
    tail = sum((1 - beta) * beta**k * n for k in range(T, 400))
    assert abs(tail - n * beta**T) < 1e-9


# --------------------------------------------------------------------------
# P5: M s = s - eps sum_i r_i phi(K_i); the spectral radius of M is <= 1, so
#     the power chain of note §2.3 cannot grow.
# --------------------------------------------------------------------------
def test_power_chain_eigenvector():
    rng = np.random.default_rng(5)
    Q, K, V = _rand_slice(rng, 80, 12, 12)
    eps = 1e-4
    s, KtV, M = olisa.stats(Q, K, V, eps)
    Qp, Kp, s2, r = olisa.normaliser(Q, K, eps)
    np.testing.assert_allclose(M @ s, s - eps * (r[:, None] * Kp).sum(0), rtol=1e-12, atol=1e-12)
    assert np.max(np.abs(np.linalg.eigvals(M))) <= 1 + 1e-12
    # K^T V and s against their sums over tokens written out
    np.testing.assert_allclose(s, sum(np.maximum(K[j], 0) for j in range(80)), rtol=1e-13)
    np.testing.assert_allclose(
        KtV, sum(np.outer(np.maximum(K[j], 0), V[j]) for j in range(80)), rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# P6: T = 1 keeps only S^0 = I (note §2.2) => G = V exactly; beta = 0 too.
# --------------------------------------------------------------------------
def test_T1_and_beta0_give_identity():
    rng = np.random.default_rng(6)
    Q, K, V = _rand_slice(rng, 20, 8, 8)
    G1 = olisa.global_branch(Q, K, V, olisa.walk_weights(20, 1, beta=0.7), 1e-6)
    assert np.array_equal(G1, V)
    G0 = olisa.global_branch(Q, K, V, olisa.walk_weights(20, 5, beta=0.0), 1e-6)
    assert np.array_equal(G0, V)


# --------------------------------------------------------------------------
# P7: untruncated closed form (note §2.3): with geometric weights and large T
#     the walk tends to (1-beta)(I - beta S)^-1 V (dense solve).
# --------------------------------------------------------------------------
def test_closed_form_large_T():
    rng = np.random.default_rng(7)
    n = 36
    Q, K, V = _rand_slice(rng, n, 8, 5)
    beta, T, eps = 0.5, 80, 1e-6
    G = olisa.global_branch(Q, K, V, olisa.walk_weights(n, T, beta=beta), eps)
    Qp, Kp, s, r = olisa.normaliser(Q, K, eps)
    S = (r[:, None] * Qp) @ Kp.T
    ref = (1 - beta) * np.linalg.solve(np.eye(n) - beta * S, V)
    assert _rel(G, ref) < 1e-13


# --------------------------------------------------------------------------
# P9: special cases.
# --------------------------------------------------------------------------
def test_zero_query_row_keeps_only_self_term():
    rng = np.random.default_rng(9)
    Q, K, V = _rand_slice(rng, 12, 4, 3)
    Q[5] = -np.abs(Q[5])  # ReLU(Q_5) = 0 => row 5 of S is 0
    w = olisa.walk_weights(12, 4, beta=0.4)
    G = olisa.global_branch(Q, K, V, w, 1e-6)
    np.testing.assert_allclose(G[5], w[5, 0] * V[5], rtol=1e-15, atol=1e-15)


def test_zero_keys_give_box_mean_and_counts():
    with open(os.path.join(GOLDEN, "neighbour_counts_3x4.json")) as f:
        g = json.load(f)
    H, W = g["H"], g["W"]
    n = H * W
    rng = np.random.default_rng(10)
    Q = rng.standard_normal((n, 5))
    K = np.zeros((n, 5))
    L = olisa.local_branch(Q, K, np.eye(n), H, W)  # V = I => L is the averaging matrix
    counts = np.round(1.0 / np.diag(L)).astype(int).reshape(H, W)
    assert counts.tolist() == g["counts"]
    np.testing.assert_allclose(L.sum(1), 1.0, rtol=0, atol=1e-15)
    # and with K = 0 the global branch keeps only the self term
    G = olisa.global_branch(Q, K, np.eye(n), olisa.walk_weights(n, 3, beta=0.5), 1e-6)
    np.testing.assert_allclose(G, olisa.geometric_weights(0.5, 3)[0] * np.eye(n), atol=1e-15)


def test_single_token_returns_v():
    rng = np.random.default_rng(11)
    Q = np.abs(rng.standard_normal((1, 1, 1, 8)))
    K = np.abs(rng.standard_normal((1, 1, 1, 8)))
    V = rng.standard_normal((1, 1, 1, 8))
    Y = oracle.lisa_forward(Q, K, V, H=1, W=1, T=5, alpha=[0.3], beta=0.5, eps=1e-6)
    # S = r q k^T is 1x1 and equals 1 - eps r, so every term is ~V
    np.testing.assert_allclose(Y, V, rtol=1e-6)


# --------------------------------------------------------------------------
# P10: one hop is textbook normalised linear attention (note §2.1, Eq. 3),
#      and the global branch is invariant to the scale of Q and of K.
# --------------------------------------------------------------------------
def test_one_hop_is_linear_attention():
    rng = np.random.default_rng(12)
    n = 40
    Q, K, V = _rand_slice(rng, n, 8, 6)
    w = np.zeros((n, 2))
    w[:, 1] = 1.0
    eps = 1e-6
    G = olisa.global_branch(Q, K, V, w, eps)
    Qp, Kp = np.maximum(Q, 0), np.maximum(K, 0)
    # phi(Q_i) (sum_j phi(K_j)^T V_j) / (phi(Q_i) . sum_j phi(K_j))
    num = np.stack([Qp[i] @ sum(np.outer(Kp[j], V[j]) for j in range(n)) for i in range(n)])
    den = np.array([Qp[i] @ Kp.sum(0) + eps for i in range(n)])
    np.testing.assert_allclose(G, num / den[:, None], rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------
# The ELU feature map (note §2.1: the supplementary comparison of ELU and
# ReLU, Table 8), read as phi(x) = ELU(x) + 1.
# --------------------------------------------------------------------------
def test_elu_feature_is_torch_elu_plus_one():
    import torch

    x = np.concatenate([np.linspace(-30.0, 30.0, 2001), [0.0, -0.0, 1e-300, -1e-300]])
    ref = torch.nn.functional.elu(torch.from_numpy(x), alpha=1.0).numpy() + 1.0
    # torch forms expm1(x) + 1, which rounds tiny e^x to within one ulp of 1.
    np.testing.assert_allclose(olisa.feature_map(x, "elu"), ref, rtol=1e-15, atol=2.3e-16)
    assert np.all(olisa.feature_map(x, "elu") > 0)
    with pytest.raises(ValueError):
        olisa.feature_map(x, "gelu")


@pytest.mark.parametrize("seed", range(6))
def test_lowrank_equals_bruteforce_elu(seed):
    rng = np.random.default_rng(500 + seed)
    H, W = int(rng.integers(1, 7)), int(rng.integers(1, 7))
    T = int(rng.integers(1, 17))
    p = _rand_problem(rng, 1, 2, H, W, 8, 5, T, adaptive=bool(seed % 2))
    kw = dict(H=H, W=W, T=T, alpha=p["alpha"], weights=p["weights"], beta=p["beta"], eps=1e-6,
              feature="elu")
    a = oracle.lisa_forward(p["Q"], p["K"], p["V"], **kw)
    b = oracle.lisa_bruteforce(p["Q"], p["K"], p["V"], **kw)
    assert _rel(a, b) < 1e-11
    # ELU differs from ReLU on these inputs (half of them are negative).
    c = oracle.lisa_forward(p["Q"], p["K"], p["V"], **dict(kw, feature="relu"))
    assert T == 1 or _rel(a, c) > 1e-3


def test_one_hop_with_elu_is_linear_attention():
    """One hop with phi = ELU + 1 is the linear attention of the elu(x) + 1
    feature map, written here with torch's ELU."""
    import torch

    rng = np.random.default_rng(14)
    n = 30
    Q, K, V = _rand_slice(rng, n, 8, 6)
    w = np.zeros((n, 2))
    w[:, 1] = 1.0
    eps = 1e-6
    G = olisa.global_branch(Q, K, V, w, eps, "elu")
    elu1 = lambda x: torch.nn.functional.elu(torch.from_numpy(x)).numpy() + 1.0
    Qp, Kp = elu1(Q), elu1(K)
    num = np.stack([Qp[i] @ sum(np.outer(Kp[j], V[j]) for j in range(n)) for i in range(n)])
    den = np.array([Qp[i] @ Kp.sum(0) + eps for i in range(n)])
    np.testing.assert_allclose(G, num / den[:, None], rtol=1e-12, atol=1e-14)
    # Every feature is positive, so S is row-stochastic up to eps r_i.
    Qp_, Kp_, s, r = olisa.normaliser(Q, K, eps, "elu")
    S = (r[:, None] * Qp_) @ Kp_.T
    np.testing.assert_allclose(S.sum(1), 1.0 - eps * r, rtol=0, atol=1e-13)
    assert np.all(S > 0)


def test_scale_invariance_of_global_branch():
    rng = np.random.default_rng(13)
    Q, K, V = _rand_slice(rng, 30, 8, 8, relu=True)
    Q += 0.1
    w = olisa.walk_weights(30, 4, beta=0.5)
    G = olisa.global_branch(Q, K, V, w, 1e-12)
    np.testing.assert_allclose(olisa.global_branch(7.0 * Q, K, V, w, 1e-12), G, rtol=1e-10)
    np.testing.assert_allclose(olisa.global_branch(Q, 0.2 * K, V, w, 1e-12), G, rtol=1e-10)


# --------------------------------------------------------------------------
# P11: invariants usable at any size.
# --------------------------------------------------------------------------
def test_constant_v_gives_constant_output():
    rng = np.random.default_rng(14)
    B, h, H, W, T = 2, 2, 5, 7, 4
    p = _rand_problem(rng, B, h, H, W, 8, 8, T, adaptive=True)
    V = np.ones_like(p["V"])
    Y = oracle.lisa_forward(p["Q"], p["K"], V, H=H, W=W, T=T, alpha=p["alpha"],
                            weights=p["weights"], eps=1e-9)
    np.testing.assert_allclose(Y, 1.0, atol=1e-7)


def test_linear_in_v():
    rng = np.random.default_rng(15)
    p = _rand_problem(rng, 1, 2, 4, 6, 8, 8, 3, adaptive=True)
    V2 = rng.standard_normal(p["V"].shape)
    kw = dict(H=4, W=6, T=3, alpha=p["alpha"], weights=p["weights"])
    Ya = oracle.lisa_forward(p["Q"], p["K"], p["V"], **kw)
    Yb = oracle.lisa_forward(p["Q"], p["K"], V2, **kw)
    Yc = oracle.lisa_forward(p["Q"], p["K"], 2.0 * p["V"] - 3.0 * V2, **kw)
    np.testing.assert_allclose(Yc, 2.0 * Ya - 3.0 * Yb, rtol=1e-10, atol=1e-12)


def test_global_branch_permutation_equivariant():
    rng = np.random.default_rng(16)
    n = 24
    Q, K, V = _rand_slice(rng, n, 8, 4)
    lg = rng.standard_normal((n, 4))
    w = np.exp(lg) / np.exp(lg).sum(1, keepdims=True)
    perm = rng.permutation(n)
    G = olisa.global_branch(Q, K, V, w, 1e-6)
    Gp = olisa.global_branch(Q[perm], K[perm], V[perm], w[perm], 1e-6)
    np.testing.assert_allclose(Gp, G[perm], rtol=1e-12, atol=1e-14)


def test_rank_one_closed_form():
    # d_h = 1 and every phi(Q_j) > 0 except one zero row: M is the scalar
    # mu = sum_j r_j K_j Q_j, so S^k V = mu^(k-1) S V and
    # G = w_0 V + (sum_{k>=1} w_k mu^(k-1)) S V.
    rng = np.random.default_rng(17)
    n = 10
    Q = np.abs(rng.standard_normal((n, 1))) + 0.1
    Q[3] = 0.0
    K = np.abs(rng.standard_normal((n, 1)))
    V = rng.standard_normal((n, 2))
    eps, T, beta = 1e-3, 6, 0.7
    w = olisa.geometric_weights(beta, T)
    s = K.sum()
    r = 1.0 / (Q[:, 0] * s + eps)
    mu = float((r * K[:, 0] * Q[:, 0]).sum())
    SV = (r * Q[:, 0])[:, None] * (K[:, 0] @ V)[None, :]
    ref = w[0] * V + sum(w[k] * mu ** (k - 1) for k in range(1, T)) * SV
    G = olisa.global_branch(Q, K, V, olisa.walk_weights(n, T, beta=beta), eps)
    np.testing.assert_allclose(G, ref, rtol=1e-13, atol=1e-15)


# --------------------------------------------------------------------------
# P12: local branch three ways, and alpha isolating each branch.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("H,W", [(1, 1), (1, 5), (5, 1), (2, 2), (3, 4), (6, 5)])
def test_local_branch_three_ways(H, W):
    rng = np.random.default_rng(H * 10 + W)
    n = H * W
    Q, K, V = _rand_slice(rng, n, 8, 3, scale=2.0)
    a = olisa.local_branch(Q, K, V, H, W)
    b = olisa.local_branch_loop(Q, K, V, H, W)
    one = lambda x: x[None, None]  # noqa: E731
    c = oracle.lisa_bruteforce(one(Q), one(K), one(V), H=H, W=W, T=1, alpha=[0.0], beta=0.5)[0, 0]
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(a, c, rtol=1e-12, atol=1e-14)


def test_alpha_isolates_branches():
    rng = np.random.default_rng(18)
    p = _rand_problem(rng, 1, 1, 4, 4, 8, 8, 3, adaptive=True)
    kw = dict(H=4, W=4, T=3, weights=p["weights"])
    Yg = oracle.lisa_forward(p["Q"], p["K"], p["V"], alpha=[1.0], **kw)[0, 0]
    Yl = oracle.lisa_forward(p["Q"], p["K"], p["V"], alpha=[0.0], **kw)[0, 0]
    G = olisa.global_branch(p["Q"][0, 0], p["K"][0, 0], p["V"][0, 0], p["weights"][0, 0], 1e-6)
    L = olisa.local_branch_loop(p["Q"][0, 0], p["K"][0, 0], p["V"][0, 0], 4, 4)
    np.testing.assert_allclose(Yg, G, rtol=1e-14)
    np.testing.assert_allclose(Yl, L, rtol=1e-12)


# --------------------------------------------------------------------------
# Hand-worked example (tests/golden/hand_1x2.json).
# --------------------------------------------------------------------------
def test_hand_example_1x2():
    with open(os.path.join(GOLDEN, "hand_1x2.json")) as f:
        g = json.load(f)
    Q = np.array(g["Q"], dtype=np.float64)[None, None]
    K = np.array(g["K"], dtype=np.float64)[None, None]
    V = np.array(g["V"], dtype=np.float64)[None, None]
    beta = float(Fraction(g["beta"]))
    alpha = float(Fraction(g["alpha"]))
    G = np.array([float(Fraction(x)) for x in g["G"]])
    Lref = []
    for i, row in enumerate(g["local_logits"]):
        e = [math.exp(float(Fraction(x))) for x in row]
        Lref.append(sum(ej * float(V[0, 0, j, 0]) for j, ej in enumerate(e)) / sum(e))
    Yref = alpha * G + (1 - alpha) * np.array(Lref)
    for fn in (oracle.lisa_forward, oracle.lisa_bruteforce):
        Y = fn(Q, K, V, H=1, W=2, T=g["T"], alpha=[alpha], beta=beta, eps=0.0)
        np.testing.assert_allclose(Y[0, 0, :, 0], Yref, rtol=1e-14)
    Gor = olisa.global_branch(Q[0, 0], K[0, 0], V[0, 0], olisa.walk_weights(2, 3, beta=beta), 0.0)
    np.testing.assert_allclose(Gor[:, 0], G, rtol=1e-15)


# --------------------------------------------------------------------------
# Planted mistakes: each plausible slip in the oracle must fail a pin above.
# The mistakes are planted in a monkeypatched copy, on the CPU.
# --------------------------------------------------------------------------
def _global_transposed_M(Q, K, V, w, eps, feature="relu"):
    Qp, Kp, s, r = olisa.normaliser(Q, K, eps)
    Qt = r[:, None] * Qp
    M = Qt.T @ Kp  # slip: Qt^T K instead of K^T Qt
    P = Kp.T @ V
    G = w[:, 0:1] * V
    for k in range(1, w.shape[1]):
        G = G + w[:, k : k + 1] * (Qt @ P)
        P = M @ P
    return G


def _global_no_self_term(Q, K, V, w, eps, feature="relu"):
    Qp, Kp, s, r = olisa.normaliser(Q, K, eps)
    Qt = r[:, None] * Qp
    M = Kp.T @ Qt
    P = Kp.T @ V
    G = np.zeros_like(np.asarray(V, dtype=np.float64))  # slip: term k = 0 dropped
    for k in range(1, w.shape[1]):
        G = G + w[:, k : k + 1] * (Qt @ P)
        P = M @ P
    return G


def _global_power_order(Q, K, V, w, eps, feature="relu"):
    Qp, Kp, s, r = olisa.normaliser(Q, K, eps)
    Qt = r[:, None] * Qp
    M = Kp.T @ Qt
    P = Kp.T @ V
    G = w[:, 0:1] * V
    for k in range(1, w.shape[1]):
        P = M @ P  # slip: power advanced before the projection (off by one)
        G = G + w[:, k : k + 1] * (Qt @ P)
    return G


def _local_wraparound(Q, K, V, H, W):
    Q = np.asarray(Q, dtype=np.float64)
    n, dh = Q.shape
    Qg, Kg, Vg = Q.reshape(H, W, dh), np.asarray(K).reshape(H, W, dh), np.asarray(V).reshape(H, W, -1)
    offs = olisa.neighbour_offsets()
    lg = np.stack([(Qg * np.roll(Kg, (-dr, -dc), (0, 1))).sum(-1) / math.sqrt(dh) for dr, dc in offs], -1)
    vals = np.stack([np.roll(Vg, (-dr, -dc), (0, 1)) for dr, dc in offs], 2)
    p = np.exp(lg - lg.max(-1, keepdims=True))
    p /= p.sum(-1, keepdims=True)
    return (p[..., None] * vals).sum(2).reshape(n, -1)


def _local_no_scale(Q, K, V, H, W):
    dh = np.asarray(Q).shape[1]
    return olisa_local_orig(np.asarray(Q) * math.sqrt(dh), K, V, H, W)


olisa_local_orig = olisa.local_branch


def _pins_pass():
    """Run a compact selection of the pins; True if all pass."""
    checks = [
        test_lowrank_equals_bruteforce_6x6_deep,
        test_T1_and_beta0_give_identity,
        test_one_hop_is_linear_attention,
        test_rank_one_closed_form,
        test_hand_example_1x2,
        lambda: test_local_branch_three_ways(3, 4),
        test_zero_keys_give_box_mean_and_counts,
    ]
    try:
        for c in checks:
            c()
    except AssertionError:
        return False
    return True


@pytest.mark.parametrize(
    "target,mistake",
    [
        ("global_branch", _global_transposed_M),
        ("global_branch", _global_no_self_term),
        ("global_branch", _global_power_order),
        ("local_branch", _local_wraparound),
        ("local_branch", _local_no_scale),
    ],
)
def test_planted_mistakes_are_caught(monkeypatch, target, mistake):
    assert _pins_pass()
    monkeypatch.setattr(olisa, target, mistake)
    assert not _pins_pass()
