"""Pins for the oracle's SSM decode step (the Mamba layer whose output M the
GMU layers reuse).

What is computed: the pages say the GMU gates the token-mixing output M of
the self-decoder's last SSM layer and that this layer keeps a constant-size
state at decode time (Paper-Notes reading notes, "Decoder-Hybrid-Decoder
Architecture for Efficient Reasoning with Long Generation", sections 关键设计
and 整体框架; the SSM is Mamba with per-channel decay, section 消融实验).  The
step itself follows the published Mamba layer: input projection, causal
depthwise convolution and SiLU, data-dependent Δ/B/C, the zero-order-hold
state update, M = C·s + D·u, gate SiLU(z), output projection.

Pins:
- a hand-derived one-channel closed form (tests/golden/closed_forms.json);
- T recurrent steps against the parallel form built from torch fp64 library
  routines: F.linear for the projections, F.conv1d over the whole input
  history for the causal convolution (its tap order), F.softplus and F.silu,
  and the SSM as its materialised token-mixing matrix with decays from
  cumulative sums of Δ·A (the pages' reading of an SSM layer as a mixing
  matrix over tokens) — a different computation from the iterated update;
- special cases: no decay memory (A -> -inf), no step (Δ -> 0), a zero
  output projection, batch independence, the exact shift of the
  convolution window.
"""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import torch_model as tm
import workload

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")))


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _t64(a):
    return torch.as_tensor(np.asarray(a, np.float64)) if not isinstance(a, torch.Tensor) else a.detach().double()


def _f64(a):
    return _t64(a).numpy()


def _parallel(xs, w, conv0, s0):
    """T steps of one sequence in parallel form (tests/torch_model.py)."""
    return tm.mamba_parallel(xs, w, conv0, s0)


def _inputs(B, seed, d_model=64, d_inner=128, N=16, R=64, K=4, T=1):
    m = workload.mamba_inputs(B, d_model, d_inner, N, R, K, seed=seed)
    xs = workload.normal((T, B, d_model), seed=seed + 777)
    return m, xs


@pytest.mark.parametrize("case", GOLDEN["mamba_step"], ids=lambda c: c["name"])
def test_closed_form(case):
    w = {k: np.array(case[k]) for k in oracle.MAMBA_KEYS}
    M, y, co, so = oracle.mamba_step(np.array(case["x"]), w, np.array(case["conv_state"]), np.array(case["ssm_state"]))
    np.testing.assert_allclose(M, case["M"], rtol=1e-14)
    np.testing.assert_allclose(y, case["y"], rtol=1e-14)
    np.testing.assert_allclose(so, case["ssm_state_out"], rtol=1e-14)
    np.testing.assert_allclose(co, case["conv_state_out"], rtol=1e-14)


@pytest.mark.parametrize("T,K", [(1, 4), (6, 4), (9, 2), (5, 1)])
def test_recurrence_against_parallel_form(T, K):
    B = 2
    m, xs = _inputs(B, seed=10 + T + K, K=K, T=T)
    conv, ssm = m.conv_state, m.ssm_state
    Ms, ys = [], []
    for t in range(T):
        M, y, conv, ssm = oracle.mamba_step(xs[t], m.w, conv, ssm)
        Ms.append(M)
        ys.append(y)
    for b in range(B):
        Mp, yp, cp, sp = _parallel(xs[:, b], m.w, m.conv_state[b], m.ssm_state[b])
        assert _rel(np.stack(Ms)[:, b], Mp) <= 1e-11
        assert _rel(np.stack(ys)[:, b], yp) <= 1e-11
        if K > 1:
            assert _rel(conv[b], cp) <= 1e-13
        assert _rel(ssm[b], sp) <= 1e-11


def test_without_decay_memory_the_initial_state_is_forgotten():
    m, xs = _inputs(2, seed=20)
    m.w["A_log"] = torch.full_like(m.w["A_log"], 12.0)         # A = -e^12: exp(Δ A) underflows to 0
    a = oracle.mamba_step(xs[0], m.w, m.conv_state, m.ssm_state)
    b = oracle.mamba_step(xs[0], m.w, m.conv_state, 7.0 * m.ssm_state + 3.0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and np.array_equal(a[3], b[3])


def test_zero_step_keeps_the_state():
    m, xs = _inputs(2, seed=21)
    m.w["dt_bias"] = torch.full_like(m.w["dt_bias"], -60.0)     # Δ = softplus(-60) ~ 1e-26
    _, _, _, so = oracle.mamba_step(xs[0], m.w, m.conv_state, m.ssm_state)
    assert _rel(so, _f64(m.ssm_state)) <= 1e-20


def test_zero_output_projection_and_batch_independence():
    m, xs = _inputs(3, seed=22)
    M, y, co, so = oracle.mamba_step(xs[0], m.w, m.conv_state, m.ssm_state)
    for b in range(3):
        r = oracle.mamba_step(xs[0][b:b + 1], m.w, m.conv_state[b:b + 1], m.ssm_state[b:b + 1])
        assert np.array_equal(r[0][0], M[b]) and np.array_equal(r[1][0], y[b])
        assert np.array_equal(r[2][0], co[b]) and np.array_equal(r[3][0], so[b])
    m.w["W_out"] = torch.zeros_like(m.w["W_out"])
    assert np.count_nonzero(oracle.mamba_step(xs[0], m.w, m.conv_state, m.ssm_state)[1]) == 0


def test_convolution_window_shifts_exactly():
    m, xs = _inputs(2, seed=23)
    _, _, co, _ = oracle.mamba_step(xs[0], m.w, m.conv_state, m.ssm_state)
    assert np.array_equal(co[:, :, :-1], _f64(m.conv_state)[:, :, 1:])
    xi = F.linear(_t64(xs[0]), _t64(m.w["W_in"]))[:, :128].numpy()
    assert _rel(co[:, :, -1], xi) <= 1e-13


def test_rejects_bad_arguments():
    m, xs = _inputs(1, seed=24)
    with pytest.raises(ValueError):
        oracle.mamba_step(xs[0], m.w, m.conv_state[:, :, :2], m.ssm_state)
    w = dict(m.w)
    w["W_x"] = w["W_x"][:-1]
    with pytest.raises(ValueError):
        oracle.mamba_step(xs[0], w, m.conv_state, m.ssm_state)


@pytest.mark.parametrize("T,K", [(1, 4), (7, 4), (12, 1)])
def test_prefill_against_parallel_form(T, K):
    """oracle.mamba_prefill over a [B, T, d_model] prompt against the
    materialised mixing-matrix form, per sequence."""
    B = 2
    m, xs = _inputs(B, seed=30 + T + K, K=K, T=T)
    x = np.ascontiguousarray(np.transpose(_f64(xs), (1, 0, 2)))
    M, y, conv, ssm = oracle.mamba_prefill(x, m.w, m.conv_state, m.ssm_state)
    for b in range(B):
        Mp, yp, cp, sp = _parallel(xs[:, b], m.w, m.conv_state[b], m.ssm_state[b])
        assert _rel(M[b], Mp) <= 1e-11
        assert _rel(y[b], yp) <= 1e-11
        if K > 1:
            assert _rel(conv[b], cp) <= 1e-13
        assert _rel(ssm[b], sp) <= 1e-11


def test_prefill_pure_decay_closed_form():
    """With a zero input projection, bias and window the convolution sees
    zeros: u = SiLU(0) = 0, so δ = B = C = 0, M = y = 0, Δ = softplus(dt_bias)
    at every step and the state after T tokens is exp(T·Δ·A)·s0."""
    m, xs = _inputs(2, seed=40, T=5)
    m.w["W_in"] = torch.zeros_like(m.w["W_in"])
    m.w["conv_b"] = torch.zeros_like(m.w["conv_b"])
    m.conv_state.zero_()
    x = np.ascontiguousarray(np.transpose(_f64(xs), (1, 0, 2)))
    M, y, conv, ssm = oracle.mamba_prefill(x, m.w, m.conv_state, m.ssm_state)
    assert np.count_nonzero(M) == 0 and np.count_nonzero(y) == 0 and np.count_nonzero(conv) == 0
    dt = np.log1p(np.exp(_f64(m.w["dt_bias"])))                         # [d_inner]
    A = -np.exp(_f64(m.w["A_log"]))                                       # [d_inner, N]
    expect = np.exp(5 * dt[:, None] * A)[None] * _f64(m.ssm_state)
    assert _rel(ssm, expect) <= 1e-13


def test_prefill_in_two_parts_equals_one():
    """The states a prompt leaves carry it on exactly: prefill(x[:, :7]) then
    prefill(x[:, 7:]) from the returned states equals prefill(x)."""
    m, xs = _inputs(2, seed=41, T=11)
    x = np.ascontiguousarray(np.transpose(_f64(xs), (1, 0, 2)))
    M, y, conv, ssm = oracle.mamba_prefill(x, m.w, m.conv_state, m.ssm_state)
    M1, y1, c1, s1 = oracle.mamba_prefill(np.ascontiguousarray(x[:, :7]), m.w, m.conv_state, m.ssm_state)
    M2, y2, c2, s2 = oracle.mamba_prefill(np.ascontiguousarray(x[:, 7:]), m.w, c1, s1)
    assert np.array_equal(np.concatenate([M1, M2], 1), M) and np.array_equal(np.concatenate([y1, y2], 1), y)
    assert np.array_equal(c2, conv) and np.array_equal(s2, ssm)
