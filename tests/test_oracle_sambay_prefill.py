"""Pins for the oracle's YOCO-style prefill (oracle.sambay_prefill).

What is computed: only the self-decoder runs over the prompt, its final
full-attention layer caches keys and values once, and the cross-decoder
runs on the last prompt token (Paper-Notes reading notes on
"Decoder-Hybrid-Decoder Architecture for Efficient Reasoning with Long
Generation", section 整体框架; Samba's alternation of SSM and sliding-window
layers, section 消融实验).  The composition is pinned against a different
computation, the recurrent one:
- prefill of T - 1 tokens followed by one decode step of the last token
  through the per-token oracles (mamba_step, selfattn on the ring or the
  full cache, the norms and MLPs, crossdecoder_ex) equals prefill of T
  tokens, to fp64 rounding, with every intermediate compared;
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


def _decode_last_token(inp, pre, xs_last):
    """The token at position T-1 through the per-token oracles, from the
    states and cache rows that a prefill of the first T-1 tokens left."""
    h = _f64(xs_last)
    M_mem, K_full, V_full, states = None, None, None, {}
    pos = np.full(B, T - 1, dtype=np.int32)
    for i, ly in enumerate(inp.self_layers):
        xin = oracle.rmsnorm(h, ly["norm1"]) if ly.get("norm1") is not None else h
        st = pre["layers"][i]
        if ly["kind"] == "mamba":
            M, y, cs, ss = oracle.mamba_step(xin, ly["w"], st["conv_state"], st["ssm_state"])
            states[i] = (cs, ss)
            h = h + y
            M_mem = M
        else:
            q = (xin @ _f64(ly["wq"]).T).reshape(B, HQ, D)
            kn = (xin @ _f64(ly["wk"]).T).reshape(B, HKV, D)
            vn = (xin @ _f64(ly["wv"]).T).reshape(B, HKV, D)
            kp, vp = st["k"], st["v"]                                  # [B, T-1, Hkv, D]
            if ly["kind"] == "swa":
                Kc = np.zeros((B, HKV, W, D))
                Vc = np.zeros((B, HKV, W, D))
                for p in range(max(0, T - 1 - W), T - 1):
                    Kc[:, :, p % W], Vc[:, :, p % W] = kp[:, p], vp[:, p]
                o, _, _ = oracle.selfattn(q, kn, vn, Kc, Vc, pos, window=W)
            else:
                Kc = np.zeros((B, HKV, T, D))
                Vc = np.zeros((B, HKV, T, D))
                Kc[:, :, :T - 1] = kp.transpose(0, 2, 1, 3)
                Vc[:, :, :T - 1] = vp.transpose(0, 2, 1, 3)
                o, K_full, V_full = oracle.selfattn(q, kn, vn, Kc, Vc, pos, window=0)
            h = h + o.reshape(B, DM) @ _f64(ly["wo"]).T
        if ly.get("w_gate") is not None:
            h = h + oracle.swiglu(oracle.rmsnorm(h, ly["norm2"]), ly["w_gate"], ly["w_up"], ly["w_down"])
    h_out = oracle.crossdecoder_ex(h, M_mem, K_full, V_full, inp.cross_layers, HQ, round_bf16=False)
    return h, M_mem, K_full, V_full, h_out, states


def test_prefill_equals_prefill_then_one_decode_step():
    inp = _inputs()
    full = oracle.sambay_prefill(inp.x, inp.self_layers, inp.cross_layers, HQ, HKV, window=W, round_h=False)
    pre = oracle.sambay_prefill(inp.x[:, :T - 1], inp.self_layers, [], HQ, HKV, window=W, round_h=False)
    h, M, Kf, Vf, h_out, states = _decode_last_token(inp, pre, inp.x[:, T - 1])
    assert _rel(full["h_last"], h) <= 1e-11
    assert _rel(full["M_last"], M) <= 1e-11
    assert _rel(full["K"], Kf) <= 1e-12 and _rel(full["V"], Vf) <= 1e-12
    assert _rel(full["h_out"], h_out) <= 1e-11
    # the SSM states after the prompt: those after T-1 tokens stepped once more
    assert len(states) == 2
    for i, (cs, ss) in states.items():
        assert _rel(full["layers"][i]["conv_state"], cs) <= 1e-12
        assert _rel(full["layers"][i]["ssm_state"], ss) <= 1e-11


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
