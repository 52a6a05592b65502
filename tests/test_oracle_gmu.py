"""Pins for the oracle's Gated Memory Unit.

The definition (Paper-Notes reading notes, "Decoder-Hybrid-Decoder
Architecture for Efficient Reasoning with Long Generation", section 关键设计):
Y = (M ⊙ SiLU(X W1^T)) W2 with SiLU(z) = z·sigmoid(z), and the gate lifts the
2-D token-mixing matrix A of the earlier layer to a 3-D tensor
Ã_ijk = G_ik · A_ij.  None of these checks re-types the oracle's loops: they
use the 3-D brute force, hand-derived closed forms, torch's own SiLU/matmul
as library routines, and algebraic properties.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workload

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")))


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


@pytest.mark.parametrize("seed", [0, 1])
def test_three_d_mixing_identity_bruteforce(seed):
    """Pin (a): GMU(M = A·V) equals mixing V with the explicit 3-D tensor
    Ã_ijk = G_ik A_ij (G = SiLU(X W1^T)), then projecting with W2^T.  A gate
    applied to the wrong channel, a dropped M, or a wrong W2 orientation
    breaks the equality."""
    c = workload.tiny_gmu(seed)
    X, V, A = c.X.double(), c.V.double(), c.A
    W1, W2 = c.W1.double(), c.W2.double()
    G = torch.nn.functional.silu(X @ W1.T)                 # [T, d_inner], library SiLU
    T, d_inner = G.shape
    At = G[:, None, :] * A[:, :, None]                       # Ã[i, j, k], built element by element
    assert At.shape == (T, T, d_inner)
    Mt = (At * V[None, :, :]).sum(dim=1)                     # M̃[i, k] = Σ_j Ã_ijk V_jk
    Y_ref = (Mt @ W2.T).numpy()
    M = (A @ V).numpy()                                      # exact-ish fp64 memory for the identity
    Y = oracle.gmu(M, X.numpy(), W1.numpy(), W2.numpy())
    assert _rel(Y, Y_ref) <= 1e-12


def test_causality_of_mixing():
    """Perturbing token j > i (its value V_j or input X_j) leaves row i unchanged."""
    c = workload.tiny_gmu(0)
    A, V, X = c.A, c.V.double(), c.X.double()
    W1, W2 = c.W1.double().numpy(), c.W2.double().numpy()
    Y0 = oracle.gmu((A @ V).numpy(), X.numpy(), W1, W2)
    i = 20
    V2, X2 = V.clone(), X.clone()
    V2[i + 1:] += 3.0
    X2[i + 1:] -= 2.0
    Y1 = oracle.gmu((A @ V2).numpy(), X2.numpy(), W1, W2)
    assert np.array_equal(Y0[: i + 1], Y1[: i + 1])
    assert not np.array_equal(Y0[i + 1:], Y1[i + 1:])


@pytest.mark.parametrize("case", GOLDEN["gmu"], ids=lambda c: c["name"])
def test_closed_forms(case):
    Y = oracle.gmu(np.array(case["M"]), np.array(case["X"]), np.array(case["W1"]), np.array(case["W2"]))
    ns = {"ln": math.log}
    for val, expr in zip(np.array(case["Y"]).reshape(-1), case["expr"]):
        assert abs(eval(expr, {"__builtins__": {}}, ns) - val) <= 1e-15 * max(1.0, abs(val))
    np.testing.assert_allclose(Y, np.array(case["Y"]), rtol=1e-15, atol=1e-15)


def _rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


def test_special_cases():
    rows, dm, di = 5, 7, 11
    M, X = _rand((rows, di), 1), _rand((rows, dm), 2)
    W1, W2 = _rand((di, dm), 3, 0.3), _rand((dm, di), 4, 0.3)
    # W1 = 0: SiLU(0) = 0, so Y = 0.
    assert np.all(oracle.gmu(M, X, np.zeros_like(W1), W2) == 0.0)
    # M = 0 gives Y = 0.
    assert np.all(oracle.gmu(np.zeros_like(M), X, W1, W2) == 0.0)
    # M = 1 reduces the GMU to a bias-free SiLU MLP: silu(X W1^T) W2^T (torch as the library routine).
    mlp = torch.nn.functional.silu(torch.from_numpy(X) @ torch.from_numpy(W1).T) @ torch.from_numpy(W2).T
    assert _rel(oracle.gmu(np.ones_like(M), X, W1, W2), mlp.numpy()) <= 1e-13
    # Library cross-check of the full formula in torch fp64.
    full = (torch.from_numpy(M) * torch.nn.functional.silu(torch.from_numpy(X) @ torch.from_numpy(W1).T)) @ \
        torch.from_numpy(W2).T
    assert _rel(oracle.gmu(M, X, W1, W2), full.numpy()) <= 1e-13


def test_linearity_and_row_independence():
    rows, dm, di = 6, 9, 13
    M, M2, X = _rand((rows, di), 5), _rand((rows, di), 6), _rand((rows, dm), 7)
    W1, W2, W2b = _rand((di, dm), 8, 0.3), _rand((dm, di), 9, 0.3), _rand((dm, di), 10, 0.3)
    Y = oracle.gmu(M, X, W1, W2)
    # Linear in M.
    lhs = oracle.gmu(2.0 * M - 3.0 * M2, X, W1, W2)
    rhs = 2.0 * Y - 3.0 * oracle.gmu(M2, X, W1, W2)
    assert _rel(lhs, rhs) <= 1e-12
    # Linear in W2.
    assert _rel(oracle.gmu(M, X, W1, W2 + W2b), Y + oracle.gmu(M, X, W1, W2b)) <= 1e-12
    # Not linear in X (the gate is nonlinear).
    assert _rel(oracle.gmu(M, 2.0 * X, W1, W2), 2.0 * Y) > 1e-3
    # Rows are independent: a block call equals per-row calls bitwise.
    per_row = np.concatenate([oracle.gmu(M[r:r + 1], X[r:r + 1], W1, W2) for r in range(rows)])
    assert np.array_equal(per_row, Y)


def test_input_dtypes_widen_exactly():
    """fp32 and bf16 inputs are the same numbers as their fp64 widening."""
    g = workload.gmu_inputs(4, 64, 128, seed=3, dtype=torch.bfloat16)
    Yb = oracle.gmu(g.M, g.X, g.W1, g.W2)
    Yd = oracle.gmu(g.M.double().numpy(), g.X.double().numpy(), g.W1.double().numpy(), g.W2.double().numpy())
    assert np.array_equal(Yb, Yd)
    c = workload.tiny_gmu(0)
    Yf = oracle.gmu(c.M, c.X, c.W1, c.W2)
    Yd = oracle.gmu(c.M.double().numpy(), c.X.double().numpy(), c.W1.double().numpy(), c.W2.double().numpy())
    assert np.array_equal(Yf, Yd)


def test_byte_counts_gmu():
    rows, dm, di = 3, 16, 32
    g = workload.gmu_inputs(rows, dm, di, seed=1)
    _, nb = oracle.gmu(g.M, g.X, g.W1, g.W2, count_bytes=True)
    assert nb["state_in"] == rows * (dm + di) * 2
    assert nb["state_out"] == rows * dm * 2
    assert nb["weights"] == 2 * dm * di * 2
    assert nb["kv_cache"] == 0
