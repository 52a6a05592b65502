"""Pins for the oracle's shared-KV cross-attention decode.

What is computed (Paper-Notes reading notes, "Decoder-Hybrid-Decoder
Architecture for Efficient Reasoning with Long Generation", sections 现有痛点
and 整体框架): the new token's softmax attention over every position of the
single KV cache that the self-decoder's last full-attention layer wrote, with
no positional encoding (same page, 关键发现; the authors' abstract).
Grouped-query heads read KV head h // (Hq / Hkv).

Pins: torch's fp64 scaled_dot_product_attention (library routine) with the KV
heads repeated per group, a brute-force softmax without max-subtraction,
hand-derived closed forms, invariances, and the split-K/log-sum-exp identity.
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


def _sdpa(q, K, V, scale):
    """torch fp64 SDPA, GQA expressed as MHA with each KV head repeated G times."""
    q, K, V = (torch.as_tensor(np.asarray(t, np.float64)) for t in (q, K, V))
    G = q.shape[1] // K.shape[1]
    Kr, Vr = K.repeat_interleave(G, dim=1), V.repeat_interleave(G, dim=1)
    out = torch.nn.functional.scaled_dot_product_attention(q[:, :, None, :], Kr, Vr, scale=scale)
    return out[:, :, 0, :].numpy()


def _f64(t):
    return t.double().numpy()


@pytest.mark.parametrize("B,Hq,Hkv,D,L", [(2, 6, 2, 16, 37), (1, 24, 8, 128, 300), (3, 4, 4, 8, 1), (2, 3, 1, 32, 129)])
def test_against_torch_sdpa(B, Hq, Hkv, D, L):
    x = workload.xattn_inputs(B, Hq, Hkv, D, L, seed=B + L)
    scale = 1.0 / math.sqrt(D)
    out = oracle.xattn(x.q, x.K, x.V, scale)
    ref = _sdpa(_f64(x.q), _f64(x.K), _f64(x.V), scale)
    assert _rel(out, ref) <= 1e-12


def test_against_bruteforce_without_max_shift():
    """Small logits: plain e^{s} / Σ e^{s} without subtracting the max."""
    rng = np.random.default_rng(7)
    B, Hq, Hkv, D, L = 2, 4, 2, 8, 23
    q, K, V = rng.standard_normal((B, Hq, D)) * 0.3, rng.standard_normal((B, Hkv, L, D)), rng.standard_normal(
        (B, Hkv, L, D))
    scale = 0.7
    ref = np.zeros((B, Hq, D))
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            w = [math.exp(scale * float(np.dot(q[b, h], K[b, g, j]))) for j in range(L)]
            tot = sum(w)
            for j in range(L):
                ref[b, h] += (w[j] / tot) * V[b, g, j]
    assert _rel(oracle.xattn(q, K, V, scale), ref) <= 1e-13


@pytest.mark.parametrize("case", GOLDEN["xattn"], ids=lambda c: c["name"])
def test_closed_forms(case):
    out = oracle.xattn(np.array(case["q"]), np.array(case["K"]), np.array(case["V"]), case["scale"])
    np.testing.assert_allclose(out, np.array(case["out"]), rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("S", [1, 2, 7, 32])
def test_split_lse_merge_identity(S):
    """Chunked partials merged by log-sum-exp equal the direct softmax."""
    x = workload.xattn_inputs(2, 6, 2, 32, 301, seed=S)
    direct = oracle.xattn(x.q, x.K, x.V)
    chunked = oracle.xattn_chunked(x.q, x.K, x.V, S)
    assert _rel(chunked, direct) <= 1e-12


def test_split_identity_peaked_logits():
    """Large logits (near one-hot softmax) merge exactly too."""
    x = workload.xattn_inputs(1, 3, 1, 16, 200, seed=9)
    q = x.q.double() * 40.0
    direct = oracle.xattn(q, x.K, x.V, 0.25)
    for S in (3, 64, 200):
        assert _rel(oracle.xattn_chunked(q, x.K, x.V, S, 0.25), direct) <= 1e-12


def test_special_cases():
    rng = np.random.default_rng(11)
    B, Hq, Hkv, D, L = 2, 6, 3, 8, 17
    q, K, V = rng.standard_normal((B, Hq, D)), rng.standard_normal((B, Hkv, L, D)), rng.standard_normal(
        (B, Hkv, L, D))
    G = Hq // Hkv
    out = oracle.xattn(q, K, V, 0.5)
    # L = 1: out is the single value row of the group.
    o1 = oracle.xattn(q, K[:, :, :1], V[:, :, :1], 0.5)
    assert np.array_equal(o1, np.repeat(V[:, :, 0], G, axis=1))
    # q = 0: uniform weights, out = mean of V over positions.
    o0 = oracle.xattn(np.zeros_like(q), K, V, 0.5)
    assert _rel(o0, np.repeat(V.mean(axis=2), G, axis=1)) <= 1e-13
    # Identical keys: uniform weights as well.
    Kc = np.broadcast_to(K[:, :, :1], K.shape).copy()
    assert _rel(oracle.xattn(q, Kc, V, 0.5), np.repeat(V.mean(axis=2), G, axis=1)) <= 1e-13
    # Adding one vector c to every key shifts each head's logits equally: out unchanged.
    c = rng.standard_normal(D)
    assert _rel(oracle.xattn(q, K + c, V, 0.5), out) <= 1e-12
    # Scaling V scales the output.
    assert _rel(oracle.xattn(q, K, -2.5 * V, 0.5), -2.5 * out) <= 1e-13
    # Permuting positions (keys and values together) leaves out unchanged: no positional encoding.
    perm = rng.permutation(L)
    assert _rel(oracle.xattn(q, K[:, :, perm], V[:, :, perm], 0.5), out) <= 1e-13


def test_bf16_inputs_widen_exactly():
    x = workload.xattn_inputs(2, 6, 2, 16, 40, seed=5)
    assert np.array_equal(oracle.xattn(x.q, x.K, x.V), oracle.xattn(_f64(x.q), _f64(x.K), _f64(x.V)))


@pytest.mark.parametrize("L", [1, 16, 256, 4096])
def test_byte_counts_xattn(L):
    """Pin (c), attention side: the call reads every cached K and V element once,
    B·Hkv·L·D·2 bf16 values, so its state I/O grows linearly with L."""
    B, Hq, Hkv, D = 2, 6, 2, 16
    x = workload.xattn_inputs(B, Hq, Hkv, D, L, seed=1)
    _, nb = oracle.xattn(x.q, x.K, x.V, count_bytes=True)
    assert nb["kv_cache"] == B * Hkv * L * D * 2 * 2
    assert nb["state_in"] == B * Hq * D * 2
    assert nb["state_out"] == B * Hq * D * 2
    assert nb["weights"] == 0
