"""Pins for the oracle's differential-attention decode.

The pages name Differential Attention as part of their largest model and
remark that its serving implementation makes four plain attention passes
(Paper-Notes reading notes, "Decoder-Hybrid-Decoder Architecture for
Efficient Reasoning with Long Generation", section 局限性 / 可改进方向); they
do not define it.  The oracle follows the published definition
(Differential Transformer, Ye et al. 2024, section 2.1) read for one decode
query per sequence over the shared cache: query and key rows are two halves,
(q1 | q2) and (k1 | k2); value rows keep all D;
  o = softmax(scale q1 k1^T) V - lambda softmax(scale q2 k2^T) V,
  out = (1 - lambda_init) * o / RMS(o) * gamma     (RMS over the head, + eps).

Pins: each map against torch's fp64 scaled_dot_product_attention on the
halves (library routine; its default scale 1/sqrt(D/2) is the oracle's
default), hand-derived closed forms, the exchange symmetry at lambda = -1,
the independence of the second map at lambda = 0, the normalisation's scale
invariance, and ragged lengths against truncated caches.
"""
import json
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


def _f64(t):
    return t.double().numpy()


def _sdpa_default_scale(q, K, V):
    """torch fp64 SDPA at its default scale 1/sqrt(q width); GQA as repeated KV heads."""
    q, K, V = (torch.as_tensor(np.ascontiguousarray(t)) for t in (q, K, V))
    G = q.shape[1] // K.shape[1]
    out = torch.nn.functional.scaled_dot_product_attention(q[:, :, None, :], K.repeat_interleave(G, dim=1),
                                                           V.repeat_interleave(G, dim=1))
    return out[:, :, 0, :].numpy()


def _swap_halves(a):
    d = a.shape[-1] // 2
    return np.concatenate([a[..., d:], a[..., :d]], axis=-1)


@pytest.mark.parametrize("B,Hq,Hkv,D,L", [(2, 6, 2, 16, 37), (1, 24, 8, 128, 300), (2, 3, 1, 8, 1)])
@pytest.mark.parametrize("lam,lam_init", [(0.8, 0.8), (-0.3, 0.2)])
def test_maps_against_torch_sdpa(B, Hq, Hkv, D, L, lam, lam_init):
    x = workload.diffattn_inputs(B, Hq, Hkv, D, L, seed=B + L + D)
    q, K, V, g = _f64(x.q), _f64(x.K), _f64(x.V), _f64(x.gamma)
    d = D // 2
    eps = 1e-5
    out = oracle.diffattn(x.q, x.K, x.V, lam, lam_init, gamma=x.gamma, eps=eps)
    a1 = _sdpa_default_scale(q[..., :d], K[..., :d], V)
    a2 = _sdpa_default_scale(q[..., d:], K[..., d:], V)
    o = a1 - lam * a2
    ref = (1 - lam_init) * o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps) * g
    assert _rel(out, ref) <= 1e-12


@pytest.mark.parametrize("case", GOLDEN["diffattn"], ids=lambda c: c["name"])
def test_closed_forms(case):
    gamma = None if case["gamma"] is None else np.array(case["gamma"])
    out = oracle.diffattn(np.array(case["q"]), np.array(case["K"]), np.array(case["V"]), case["lam"],
                          case["lam_init"], gamma=gamma, lens=case["lens"], eps=case["eps"], scale=case["scale"])
    np.testing.assert_allclose(out, np.array(case["out"]), rtol=1e-14, atol=1e-14)


def test_exchange_symmetry_at_lambda_minus_one():
    """lambda = -1 adds the two maps, so exchanging the halves of every query
    and key row (map 1 <-> map 2) leaves the output unchanged."""
    x = workload.diffattn_inputs(2, 6, 3, 16, 45, seed=3)
    q, K, V = _f64(x.q), _f64(x.K), _f64(x.V)
    a = oracle.diffattn(q, K, V, -1.0, 0.3, gamma=x.gamma)
    b = oracle.diffattn(_swap_halves(q), _swap_halves(K), V, -1.0, 0.3, gamma=x.gamma)
    assert _rel(b, a) <= 1e-14
    # ... and at any other lambda it does change the output.
    c = oracle.diffattn(_swap_halves(q), _swap_halves(K), V, 0.5, 0.3, gamma=x.gamma)
    assert _rel(c, oracle.diffattn(q, K, V, 0.5, 0.3, gamma=x.gamma)) > 1e-3


def test_lambda_zero_ignores_second_map():
    x = workload.diffattn_inputs(2, 4, 2, 32, 50, seed=4)
    q, K, V = _f64(x.q), _f64(x.K), _f64(x.V)
    a = oracle.diffattn(q, K, V, 0.0, 0.5)
    rng = np.random.default_rng(0)
    q2, K2 = q.copy(), K.copy()
    q2[..., 16:] = rng.standard_normal(q2[..., 16:].shape) * 5
    K2[..., 16:] = rng.standard_normal(K2[..., 16:].shape) * 5
    assert np.array_equal(oracle.diffattn(q2, K2, V, 0.0, 0.5), a)


def test_normalisation_is_scale_invariant():
    """With eps = 0 the per-head RMS normalisation cancels any positive scale of V."""
    x = workload.diffattn_inputs(1, 6, 2, 16, 30, seed=5)
    q, K, V = _f64(x.q), _f64(x.K), _f64(x.V)
    a = oracle.diffattn(q, K, V, 0.6, 0.4, gamma=x.gamma, eps=0.0)
    b = oracle.diffattn(q, K, 7.5 * V, 0.6, 0.4, gamma=x.gamma, eps=0.0)
    assert _rel(b, a) <= 1e-14
    # (1 - lambda_init) scales the output linearly.
    c = oracle.diffattn(q, K, V, 0.6, 0.8, gamma=x.gamma, eps=0.0)
    assert _rel(c, a * (0.2 / 0.6)) <= 1e-14


def test_ragged_equals_truncated_cache():
    x = workload.diffattn_inputs(3, 6, 2, 16, 40, seed=6)
    q, K, V = _f64(x.q), _f64(x.K), _f64(x.V)
    lens = [40, 7, 1]
    out = oracle.diffattn(q, K, V, 0.8, 0.8, gamma=x.gamma, lens=lens)
    for b, n in enumerate(lens):
        ref = oracle.diffattn(q[b:b + 1], K[b:b + 1, :, :n], V[b:b + 1, :, :n], 0.8, 0.8, gamma=x.gamma)
        assert _rel(out[b:b + 1], ref) <= 1e-15


def test_rejects_bad_arguments():
    x = workload.diffattn_inputs(1, 2, 1, 8, 5, seed=7)
    with pytest.raises(ValueError):
        oracle.diffattn(x.q, x.K, x.V, 0.5, 0.5, lens=[6])
    with pytest.raises(ValueError):
        oracle.diffattn(x.q[..., :7], x.K[..., :7], x.V[..., :7], 0.5, 0.5)   # odd D
    with pytest.raises(ValueError):
        oracle.diffattn(x.q, x.K, x.V, 0.5, 0.5, gamma=np.ones(4))
