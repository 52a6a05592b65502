"""Pins for the oracle's YOCO-style prefill (oracle.sambay_prefill).

What is computed: only the self-decoder runs over the prompt, its final
full-attention layer caches keys and values once, and the cross-decoder
runs on the last prompt token (Paper-Notes reading notes on
"Decoder-Hybrid-Decoder Architecture for Efficient Reasoning with Long
Generation", section 整体框架; Samba's alternation of SSM and sliding-window
layers, section 消融实验).  The composition is pinned against a different
computation, the recurrent one:
- prefill of T - 1 tokens followed by one decode step of the last token
  (oracle.sambay_decode_step: the per-token oracles mamba_step, selfattn on
  the ring or the full cache, the norms and MLPs, crossdecoder_ex) equals
  prefill of T tokens, to fp64 rounding, with every intermediate compared;
- causality: the cache rows of earlier positions do not depend on the last
  token; a window of at least T is plain causal attention;
- the vectorised bfloat16 rounding used for the residual stream equals the
  scalar definition, ties included.
"""
import numpy as np
import pytest
import torch

import oracle
import workload

B, T, DM, DI, NS, R, K, DF, HQ, HKV, D, W = 2, 9, 256, 128, 8, 16, 4, 64, 2, 1, 128, 4
SELF = ["mamba", "swa", "mamba", "attn"]
CROSS = ["xattn", "gmu"]


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _inputs(seed=3, T_=T, self_kinds=SELF, fresh=False):
    return workload.sambay_prefill_inputs(B, T_, DM, DI, NS, R, K, DF, HQ, HKV, D, W, T_, self_kinds, CROSS,
                                          seed=seed, fresh=fresh)


def _f64(t):
    return np.asarray(t.double().numpy() if isinstance(t, torch.Tensor) else t, np.float64)


def test_round_bf16_array_matches_the_scalar_definition():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(5000) * 10.0 ** rng.integers(-6, 6, 5000),
                        # exact ties between two bfloat16 neighbours, both parities
                        (1.0 + (2 * np.arange(1, 128) + 1) * 2.0 ** -8) * np.array([1, -1])[np.arange(127) % 2],
                        [0.0, -0.0, 1.0, 3.0 * 2.0 ** -20]])
    assert np.array_equal(oracle.round_bf16_array(x), oracle.round_bf16(x))


def _caches_after_prefill(inp, pre, T_pre):
    """Ring and shared-cache contents that a prefill of T_pre tokens leaves
    (from the per-layer keys and values it computed), and the SSM states."""
    layers = []
    K = V = None
    for i, ly in enumerate(inp.self_layers):
        st = dict(ly)
        r = pre["layers"][i]
        if ly["kind"] == "mamba":
            st["conv_state"], st["ssm_state"] = r["conv_state"], r["ssm_state"]
        elif ly["kind"] == "swa":
            kr, vr = np.zeros((B, HKV, W, D)), np.zeros((B, HKV, W, D))
            for p in range(max(0, T_pre - W), T_pre):
                kr[:, :, p % W], vr[:, :, p % W] = r["k"][:, p], r["v"][:, p]
            st["kring"], st["vring"] = kr, vr
        else:
            K, V = np.zeros((B, HKV, T_pre + 1, D)), np.zeros((B, HKV, T_pre + 1, D))
            K[:, :, :T_pre] = r["k"].transpose(0, 2, 1, 3)
            V[:, :, :T_pre] = r["v"].transpose(0, 2, 1, 3)
        layers.append(st)
    return layers, K, V


def test_prefill_equals_prefill_then_one_decode_step():
    """oracle.sambay_decode_step (per-token oracles, the recurrent form)
    after a prefill of T - 1 tokens equals a prefill of T tokens."""
    inp = _inputs()
    full = oracle.sambay_prefill(inp.x, inp.self_layers, inp.cross_layers, HQ, HKV, window=W, round_h=False)
    pre = oracle.sambay_prefill(inp.x[:, :T - 1], inp.self_layers, [], HQ, HKV, window=W, round_h=False)
    layers, K, V = _caches_after_prefill(inp, pre, T - 1)
    step = oracle.sambay_decode_step(inp.x[:, T - 1], layers, inp.cross_layers, HQ, HKV, np.full(B, T - 1), K, V,
                                     window=W, round_h=False)
    assert _rel(full["h_last"], step["h_self"]) <= 1e-11
    assert _rel(full["M_last"], step["M_last"]) <= 1e-11
    assert _rel(full["K"], step["K"]) <= 1e-12 and _rel(full["V"], step["V"]) <= 1e-12
    assert _rel(full["h_out"], step["h_out"]) <= 1e-11
    # the SSM states after the prompt: those after T-1 tokens stepped once more
    n = 0
    for i, ly in enumerate(inp.self_layers):
        if ly["kind"] == "mamba":
            n += 1
            assert _rel(full["layers"][i]["conv_state"], step["layers"][i]["conv_state"]) <= 1e-12
            assert _rel(full["layers"][i]["ssm_state"], step["layers"][i]["ssm_state"]) <= 1e-11
    assert n == 2


def test_decode_step_ring_holds_the_last_window_tokens():
    """After the step, a sliding-window layer's ring holds the keys of the
    last `window` tokens (prefill of T tokens), slot = position mod window."""
    inp = _inputs(seed=12)
    full = oracle.sambay_prefill(inp.x, inp.self_layers, [], HQ, HKV, window=W, round_h=False)
    pre = oracle.sambay_prefill(inp.x[:, :T - 1], inp.self_layers, [], HQ, HKV, window=W, round_h=False)
    layers, K, V = _caches_after_prefill(inp, pre, T - 1)
    step = oracle.sambay_decode_step(inp.x[:, T - 1], layers, [], HQ, HKV, np.full(B, T - 1), K, V, window=W,
                                     round_h=False)
    i = [j for j, ly in enumerate(inp.self_layers) if ly["kind"] == "swa"][0]
    for p in range(T - W, T):
        assert _rel(step["layers"][i]["kring"][:, :, p % W], full["layers"][i]["k"][:, p]) <= 1e-12


def test_cache_rows_of_earlier_positions_ignore_the_last_token():
    inp = _inputs(seed=4)
    a = oracle.sambay_prefill(inp.x, inp.self_layers, inp.cross_layers, HQ, HKV, window=W)
    x2 = inp.x.clone()
    x2[:, T - 1] = -x2[:, T - 1]
    b = oracle.sambay_prefill(x2, inp.self_layers, inp.cross_layers, HQ, HKV, window=W)
    assert np.array_equal(a["K"][:, :, :T - 1], b["K"][:, :, :T - 1])
    assert np.array_equal(a["V"][:, :, :T - 1], b["V"][:, :, :T - 1])
    assert not np.allclose(a["h_out"], b["h_out"])


def test_a_window_of_at_least_the_prompt_is_full_attention():
    inp = _inputs(seed=6)
    a = oracle.sambay_prefill(inp.x, inp.self_layers, inp.cross_layers, HQ, HKV, window=T)
    layers = [dict(ly, kind="attn") if ly["kind"] == "swa" else ly for ly in inp.self_layers]
    b = oracle.sambay_prefill(inp.x, layers, inp.cross_layers, HQ, HKV, window=T)
    assert np.array_equal(a["h_out"], b["h_out"])


def test_rounded_and_exact_residual_streams_stay_close():
    """The bf16 residual stream changes the result only at rounding level
    (the reading the library follows); a gross mistake would not."""
    inp = _inputs(seed=7)
    a = oracle.sambay_prefill(inp.x, inp.self_layers, inp.cross_layers, HQ, HKV, window=W, round_h=True)
    b = oracle.sambay_prefill(inp.x, inp.self_layers, inp.cross_layers, HQ, HKV, window=W, round_h=False)
    assert 0 < _rel(a["h_out"], b["h_out"]) <= 2e-2
