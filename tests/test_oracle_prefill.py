"""Pins for the oracle's prefill attention (causal, optionally over a sliding
window), the attention of the self-decoder's layers over the prompt.

What is computed (reading of the Paper-Notes page "Decoder-Hybrid-Decoder
Architecture for Efficient Reasoning with Long Generation", sections 领域现状
and 现有痛点: the decoder-decoder structure pre-fills in linear time; section
消融实验: the self-decoder's attention uses a 256-token sliding window): query
i attends to keys j <= i, and with a window W to j > i - W, grouped heads,
no positional encoding.

Pins: torch fp64 scaled_dot_product_attention with the explicit boolean
mask (library routine), a hand-derived closed form, window 1 returns the
token's own value, a window at least T equals plain causal attention bit for
bit, and the last token's output equals the decode attention oracle over
the prompt's keys.
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


def _inputs(B, T, Hq, Hkv, D, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, T, Hq, D)), rng.standard_normal((B, T, Hkv, D)),
            rng.standard_normal((B, T, Hkv, D)))


def _sdpa_masked(q, k, v, window, scale):
    q, k, v = (torch.as_tensor(t).transpose(1, 2) for t in (q, k, v))        # [B, H, T, D]
    G = q.shape[1] // k.shape[1]
    T = q.shape[2]
    i = torch.arange(T)[:, None]
    j = torch.arange(T)[None, :]
    mask = j <= i
    if window > 0:
        mask &= j > i - window
    out = torch.nn.functional.scaled_dot_product_attention(q, k.repeat_interleave(G, dim=1),
                                                           v.repeat_interleave(G, dim=1), attn_mask=mask, scale=scale)
    return out.transpose(1, 2).numpy()


@pytest.mark.parametrize("B,T,Hq,Hkv,D,window", [(2, 37, 6, 2, 16, 0), (1, 70, 3, 1, 32, 8), (2, 19, 4, 4, 8, 19),
                                                 (1, 50, 6, 3, 16, 1), (1, 64, 24, 8, 128, 16)])
def test_against_torch_sdpa_with_mask(B, T, Hq, Hkv, D, window):
    q, k, v = _inputs(B, T, Hq, Hkv, D, seed=T + window)
    scale = 1.0 / math.sqrt(D)
    assert _rel(oracle.attn_prefill(q, k, v, window, scale), _sdpa_masked(q, k, v, window, scale)) <= 1e-12


@pytest.mark.parametrize("case", GOLDEN["attn_prefill"], ids=lambda c: c["name"])
def test_closed_form(case):
    out = oracle.attn_prefill(np.array(case["q"]), np.array(case["k"]), np.array(case["v"]), case["window"],
                              case["scale"])
    np.testing.assert_allclose(out, np.array(case["out"]), rtol=1e-14, atol=1e-14)


def test_window_one_returns_the_own_value():
    q, k, v = _inputs(2, 20, 6, 2, 8, seed=3)
    out = oracle.attn_prefill(q, k, v, 1)
    assert np.array_equal(out, np.repeat(v, 3, axis=2))


def test_window_at_least_T_is_plain_causal():
    q, k, v = _inputs(1, 33, 4, 2, 8, seed=4)
    assert np.array_equal(oracle.attn_prefill(q, k, v, 33), oracle.attn_prefill(q, k, v, 0))
    assert np.array_equal(oracle.attn_prefill(q, k, v, 500), oracle.attn_prefill(q, k, v, 0))


def test_last_token_equals_decode_attention_over_the_prompt():
    q, k, v = _inputs(2, 45, 6, 2, 16, seed=5)
    out = oracle.attn_prefill(q, k, v, 0)
    dec = oracle.xattn(q[:, -1], np.ascontiguousarray(k.transpose(0, 2, 1, 3)),
                       np.ascontiguousarray(v.transpose(0, 2, 1, 3)))
    assert _rel(out[:, -1], dec) <= 1e-14
