"""Pins for the oracle's self-decoder attention decode step.

What is computed (reading of the Paper-Notes page "Decoder-Hybrid-Decoder
Architecture for Efficient Reasoning with Long Generation", sections 整体框架
and 消融实验): the self-decoder's final full-attention layer writes the one
KV cache that the cross-decoder reads, and its other attention layers attend
over a sliding window (256 positions in the model the page favours).  One
decode step stores the new token's key and value rows (at its position, or
in ring slot position mod window) and attends over what is visible.

Pins: hand-derived closed forms; a ring driven token by token equals plain
attention (torch fp64 SDPA) over the last `window` tokens of the linear
history; the full-cache step equals the ragged attention oracle and SDPA on
the prefix; exactly one row per (sequence, KV head) changes; inactive
sequences change nothing.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")))


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _sdpa(q, K, V, scale):
    q, K, V = (torch.as_tensor(np.ascontiguousarray(t, dtype=np.float64)) for t in (q, K, V))
    G = q.shape[1] // K.shape[1]
    out = torch.nn.functional.scaled_dot_product_attention(q[:, :, None, :], K.repeat_interleave(G, dim=1),
                                                           V.repeat_interleave(G, dim=1), scale=scale)
    return out[:, :, 0, :].numpy()


@pytest.mark.parametrize("case", GOLDEN["selfattn"], ids=lambda c: c["name"])
def test_closed_forms(case):
    out, _, _ = oracle.selfattn(np.array(case["q"]), np.array(case["k_new"]), np.array(case["v_new"]),
                                np.array(case["K"]), np.array(case["V"]), case["pos"], window=case["window"],
                                scale=case["scale"])
    np.testing.assert_allclose(out, np.array(case["out"]), rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("W,T", [(4, 11), (8, 8), (8, 3), (16, 40)])
def test_ring_equals_attention_over_the_last_window(W, T):
    """Drive a ring of W slots with T tokens; at every step the output equals
    plain attention over the last min(t + 1, W) tokens of the linear history."""
    rng = np.random.default_rng(W * 100 + T)
    B, Hq, Hkv, D = 2, 6, 2, 8
    keys = rng.standard_normal((B, Hkv, T, D))
    vals = rng.standard_normal((B, Hkv, T, D))
    qs = rng.standard_normal((T, B, Hq, D))
    K = rng.standard_normal((B, Hkv, W, D)) * 50       # garbage in the unused slots
    V = rng.standard_normal((B, Hkv, W, D)) * 50
    scale = 1.0 / math.sqrt(D)
    for t in range(T):
        out, K, V = oracle.selfattn(qs[t], keys[:, :, t], vals[:, :, t], K, V, [t, t], window=W, scale=scale)
        lo = max(0, t + 1 - W)
        ref = _sdpa(qs[t], keys[:, :, lo:t + 1], vals[:, :, lo:t + 1], scale)
        assert _rel(out, ref) <= 1e-12, "step %d" % t


def test_full_cache_equals_ragged_attention_on_the_updated_cache():
    rng = np.random.default_rng(5)
    B, Hq, Hkv, D, L = 3, 6, 3, 16, 40
    q = rng.standard_normal((B, Hq, D))
    kn, vn = rng.standard_normal((B, Hkv, D)), rng.standard_normal((B, Hkv, D))
    K, V = rng.standard_normal((B, Hkv, L, D)), rng.standard_normal((B, Hkv, L, D))
    pos = [0, 17, 39]
    out, Ko, Vo = oracle.selfattn(q, kn, vn, K, V, pos, window=0)
    ref = oracle.xattn_varlen(q, Ko, Vo, [p + 1 for p in pos])
    assert _rel(out, ref) <= 1e-15
    for b, p in enumerate(pos):
        sd = _sdpa(q[b:b + 1], Ko[b:b + 1, :, :p + 1], Vo[b:b + 1, :, :p + 1], 1.0 / math.sqrt(D))
        assert _rel(out[b:b + 1], sd) <= 1e-12


@pytest.mark.parametrize("window", [0, 8])
def test_exactly_one_row_changes(window):
    rng = np.random.default_rng(6)
    B, Hq, Hkv, D = 3, 4, 2, 8
    L = window or 20
    q = rng.standard_normal((B, Hq, D))
    kn, vn = rng.standard_normal((B, Hkv, D)), rng.standard_normal((B, Hkv, D))
    K, V = rng.standard_normal((B, Hkv, L, D)), rng.standard_normal((B, Hkv, L, D))
    pos = [5, 19, -1]
    _, Ko, Vo = oracle.selfattn(q, kn, vn, K, V, pos, window=window)
    for b, p in enumerate(pos):
        for g in range(Hkv):
            slot = None if p < 0 else (p % window if window else p)
            for j in range(L):
                if j == slot:
                    assert np.array_equal(Ko[b, g, j], kn[b, g]) and np.array_equal(Vo[b, g, j], vn[b, g])
                else:
                    assert np.array_equal(Ko[b, g, j], K[b, g, j]) and np.array_equal(Vo[b, g, j], V[b, g, j])


def test_inactive_sequence_gives_zero_output():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((2, 2, 4))
    K, V = rng.standard_normal((2, 1, 6, 4)), rng.standard_normal((2, 1, 6, 4))
    out, _, _ = oracle.selfattn(q, np.ones((2, 1, 4)), np.ones((2, 1, 4)), K, V, [-1, 2])
    assert np.count_nonzero(out[0]) == 0 and np.count_nonzero(out[1]) > 0


def test_rejects_bad_arguments():
    q = np.zeros((1, 2, 4))
    K = np.zeros((1, 1, 6, 4))
    with pytest.raises(ValueError):
        oracle.selfattn(q, np.zeros((1, 1, 4)), np.zeros((1, 1, 4)), K, K, [6])            # position past the cache
    with pytest.raises(ValueError):
        oracle.selfattn(q, np.zeros((1, 1, 4)), np.zeros((1, 1, 4)), K, K, [2], window=4)  # L != window
