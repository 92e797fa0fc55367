"""Parity of the HIP backward pass (lisa_backward, through the C ABI) with the
fp64 backward oracle, on the GPU.

Every output (dQ, dK, dV, the adaptive-weight gradient and dalpha) is
compared whole: relative L2, and per element against |ref| + rms(ref).
Tolerances: 1e-5 for fp32 inputs (fp32 arithmetic throughout); 1e-2 for bf16
inputs, where dQ, dK and dV are rounded to bf16 once (2^-9 relative per
element) and the statistics' M is formed from r_i phi(Q_i) rounded to bf16;
measured: about 1.7e-3 relative L2 and 3.4e-3 worst element.
"""

import zlib

import numpy as np
import pytest
import torch

import oracle
from vision_transformer_token_amd import workloads

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-5, "bf16": 1e-2}


@pytest.fixture(scope="module")
def lisa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from vision_transformer_token_amd import lisa as mod

    return mod


def f64(t):
    return None if t is None else t.double().cpu().numpy()


def make_dy(x, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(x["v"].shape, generator=g, dtype=torch.float32).to(x["v"].dtype)


def run_gpu(lisa, x, dy):
    d = {k: (x[k].cuda() if isinstance(x[k], torch.Tensor) else x[k]) for k in ("q", "k", "v", "weights", "alpha")}
    out = lisa.lisa_backward(d["q"], d["k"], d["v"], dy.cuda(), grid=(x["H"], x["W"]), T=x["T"],
                             alpha=d["alpha"], weights=d["weights"], beta=x["beta"], eps=x["eps"])
    torch.cuda.synchronize()
    return out


def run_oracle(x, dy):
    return oracle.lisa_backward(f64(x["q"]), f64(x["k"]), f64(x["v"]), H=x["H"], W=x["W"], T=x["T"],
                                alpha=f64(x["alpha"]), dY=f64(dy), weights=f64(x["weights"]), beta=x["beta"],
                                eps=x["eps"])


def compare(g, ref, dtype, label, floors=None):
    """floors: per output, an absolute error scale below which differences are
    rounding noise (used where the exact gradient is of order eps)."""
    floors = floors or {}
    worst = {}
    for key in ("dq", "dk", "dv", "dweights", "dalpha"):
        r = ref[key]
        if r is None:
            assert g[key] is None, key
            continue
        y = f64(g[key])
        diff = y - r
        assert np.all(np.isfinite(y)), key
        fl = floors.get(key, 0.0)
        nr = max(np.linalg.norm(r), fl * np.sqrt(r.size))
        rel = np.linalg.norm(diff) / nr if nr > 0 else np.linalg.norm(diff)
        rms = np.sqrt(np.mean(r**2))
        den = np.abs(r) + rms + fl
        el = np.max(np.abs(diff) / den) if np.all(den > 0) else np.max(np.abs(diff))
        worst[key] = (rel, el)
    print(f"[parity] backward {label}: " + " ".join(f"{k}={v[0]:.2e}/{v[1]:.2e}" for k, v in worst.items()),
          flush=True)
    for key, (rel, el) in worst.items():
        assert rel <= TOL[dtype] and el <= TOL[dtype], (label, key, rel, el)


SMALL = [
    # name, B, heads, H, W, T, dtype, weights mode
    ("ragged-a", 2, 3, 10, 13, 3, "fp32", "adaptive"),
    ("ragged-b", 1, 2, 17, 9, 5, "fp32", "geometric"),
    ("t1", 1, 2, 6, 7, 1, "fp32", "adaptive"),
    ("t2", 2, 1, 9, 11, 2, "fp32", "adaptive"),
    ("t8", 1, 1, 12, 12, 8, "fp32", "adaptive"),
    ("one-token", 3, 2, 1, 1, 3, "fp32", "adaptive"),
    ("one-row", 1, 2, 1, 40, 4, "fp32", "geometric"),
    ("two-blocks", 1, 1, 16, 17, 3, "fp32", "adaptive"),  # 272 tokens: 3 workgroups, a ragged one
    ("bf16-ragged", 2, 2, 13, 21, 3, "bf16", "adaptive"),
    ("bf16-t5", 1, 3, 20, 15, 5, "bf16", "adaptive"),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_backward_small(lisa, case):
    name, B, heads, H, W, T, dtype, mode = case
    w = workloads.small(name, B, heads, H, W, T, dtype=dtype, mode=mode, seed=zlib.crc32(name.encode()) % 1000)
    x = workloads.make_inputs(w)
    dy = make_dy(x, 17)
    floors = None
    if H * W == 1:
        # One token: its window holds it alone (L = V) and S = 1 - eps r, so
        # the exact dQ, dK and dalpha are of order eps, formed in fp32 as
        # differences of O(|dY| |V|) terms: compare them against that scale.
        scale = float(x["v"].abs().max() * dy.abs().max())
        floors = {"dq": scale, "dk": scale, "dalpha": scale * B}
    compare(run_gpu(lisa, x, dy), run_oracle(x, dy), dtype, w.describe(), floors)


@pytest.mark.parametrize("name", ["tiny_oracle_14x14", "deit_t_224", "pvt_t_stage1"])
def test_backward_workload(lisa, name):
    w = workloads.get(name)
    x = workloads.make_inputs(w)
    dy = make_dy(x, 29)
    compare(run_gpu(lisa, x, dy), run_oracle(x, dy), w.dtype, w.describe())


def test_backward_deterministic(lisa):
    w = workloads.small("det", 2, 2, 19, 23, 4, dtype="bf16", seed=3)
    x = workloads.make_inputs(w)
    dy = make_dy(x, 5)
    a, b = run_gpu(lisa, x, dy), run_gpu(lisa, x, dy)
    for key in ("dq", "dk", "dv", "dweights", "dalpha"):
        assert torch.equal(a[key], b[key]), key


AFTER = [
    # name, B, heads, H, W, T, dtype, weights mode, the call that leaves the statistics
    ("after-forward-bf16", 2, 2, 13, 21, 3, "bf16", "adaptive", "forward"),
    ("after-forward-fp32-geo", 1, 2, 17, 9, 5, "fp32", "geometric", "forward"),
    ("after-forward-t2", 2, 1, 9, 11, 2, "fp32", "adaptive", "forward"),  # T < 3: recomputed
    ("after-reduce", 1, 3, 20, 15, 4, "bf16", "adaptive", "reduce"),
    ("after-forward-mlp", 2, 1, 12, 17, 3, "bf16", "adaptive", "mlp"),
    ("after-forward-pvt", 32, 1, 56, 56, 3, "bf16", "adaptive", "forward"),
]


@pytest.mark.parametrize("case", AFTER, ids=[c[0] for c in AFTER])
def test_backward_after_forward_equals_backward(lisa, case):
    """lisa_backward_after_forward on the workspace a forward (or reduce) of the
    same inputs just used gives lisa_backward's gradients bit for bit."""
    name, B, heads, H, W, T, dtype, mode, first = case
    w = workloads.small(name, B, heads, H, W, T, dtype=dtype, mode=mode, seed=zlib.crc32(name.encode()) % 1000)
    x = workloads.make_inputs(w)
    dy = make_dy(x, 23).cuda()
    d = {k: (x[k].cuda() if isinstance(x[k], torch.Tensor) else x[k]) for k in ("q", "k", "v", "weights", "alpha")}
    kw = dict(grid=(H, W), T=T, alpha=d["alpha"], weights=d["weights"], beta=x["beta"], eps=x["eps"])
    prob = lisa.make_problem(d["q"], d["v"], grid=(H, W), T=T, eps=x["eps"])
    nbytes = lisa.lisa_backward_workspace_size(prob)
    if first == "mlp":
        nbytes = max(nbytes, lisa.lisa_forward_mlp_workspace_size(prob, 64))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    # Leave other statistics in the workspace first, so that a skipped
    # recomputation that should not have been skipped shows.
    lisa.lisa_reduce(d["k"], d["q"], -d["v"], grid=(H, W), eps=x["eps"], T=T, workspace=ws, outputs=False)
    if first == "forward":
        lisa.lisa_forward(d["q"], d["k"], d["v"], workspace=ws, **kw)
    elif first == "reduce":
        lisa.lisa_reduce(d["q"], d["k"], d["v"], grid=(H, W), eps=x["eps"], T=T, workspace=ws, outputs=False)
    else:
        prm = {k: t.cuda() for k, t in workloads.mlp_params(heads, 64, T, seed=7).items()}
        lisa.lisa_forward_mlp(d["q"], d["k"], d["v"], grid=(H, W), T=T, alpha=d["alpha"], eps=x["eps"],
                              workspace=ws, **prm)
    got = lisa.lisa_backward_after_forward(d["q"], d["k"], d["v"], dy, workspace=ws, **kw)
    ref = lisa.lisa_backward(d["q"], d["k"], d["v"], dy, **kw)
    torch.cuda.synchronize()
    print(f"[parity] backward after {first}: {w.describe()}", flush=True)
    for key in ("dq", "dk", "dv", "dweights", "dalpha"):
        if ref[key] is None:
            assert got[key] is None, key
        else:
            assert torch.equal(got[key], ref[key]), key
