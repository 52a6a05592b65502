"""Pins for the oracle's cross-decoder decode step, its bf16 residual rounding
and its byte counts.

Structure (Paper-Notes reading notes, "Decoder-Hybrid-Decoder Architecture for
Efficient Reasoning with Long Generation", section 整体框架): the cross-decoder
alternates cross-attention layers that reuse the one KV cache and GMU layers
that reuse the memory readout M of the self-decoder's last SSM layer.  The I/O
claim checked by counting (same page, 现有痛点 and 关键设计; the authors'
abstract): a cross-attention decode step reads O(d_kv·N) cache state, a GMU
step reads state whose size does not depend on N.
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


def test_round_bf16_fixture():
    g = GOLDEN["round_bf16"]
    assert np.array_equal(oracle.round_bf16(np.array(g["x"])), np.array(g["expected"]))


def test_round_bf16_matches_torch_on_binary32_inputs():
    """For values that are already binary32, direct rounding equals torch's
    float32 -> bfloat16 conversion (round to nearest even), ties included."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(4000) * np.exp(rng.uniform(-20, 20, 4000))).astype(np.float32)
    # Add exact ties: bf16 values plus half an ulp.
    base = torch.from_numpy(x[:500]).to(torch.bfloat16).float()
    ulp = torch.from_numpy(np.spacing(base.numpy().astype(np.float32)) * 65536.0)
    ties = (base + 0.5 * ulp).numpy().astype(np.float32)
    x = np.concatenate([x, ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(oracle.round_bf16(x.astype(np.float64)), ref)


def _tiny(kinds, B=3, Hq=4, Hkv=2, D=8, L=19, d_inner=48, seed=0):
    d_model = Hq * D
    return workload.crossdecoder_inputs(B, d_model, d_inner, Hq, Hkv, D, L, len(kinds), seed=seed, kinds=kinds), dict(
        B=B, Hq=Hq, Hkv=Hkv, D=D, L=L, d_model=d_model, d_inner=d_inner)


def _t64(t):
    return t.double()


def _gmu_layer_ref(h, M, W1, W2):
    return h + (M * torch.nn.functional.silu(h @ W1.T)) @ W2.T


def _xattn_layer_ref(h, K, V, Wq, Wo, Hq, scale):
    B = h.shape[0]
    q = (h @ Wq.T).reshape(B, Hq, -1)
    G = Hq // K.shape[1]
    o = torch.nn.functional.scaled_dot_product_attention(q[:, :, None, :], K.repeat_interleave(G, 1),
                                                         V.repeat_interleave(G, 1), scale=scale)[:, :, 0, :]
    return h + o.reshape(B, -1) @ Wo.T


def test_layers_against_torch_composition():
    """Each layer equals its definition composed from torch fp64 library calls,
    followed by the bf16 rounding of the residual stream."""
    kinds = ["xattn", "gmu", "xattn", "gmu"]
    x, s = _tiny(kinds)
    scale = 1.0 / math.sqrt(s["D"])
    h = _t64(x.h)
    for kind, wa, wb in x.layers:
        if kind == "xattn":
            h = _xattn_layer_ref(h, _t64(x.K), _t64(x.V), _t64(wa), _t64(wb), s["Hq"], scale)
        else:
            h = _gmu_layer_ref(h, _t64(x.M), _t64(wa), _t64(wb))
        h = torch.from_numpy(oracle.round_bf16(h.numpy()))
    out = oracle.crossdecoder(x.h, x.M, x.K, x.V, x.layers, s["Hq"], scale)
    # Both sides round h to bf16 after every layer; a last-bit difference before a
    # rounding can move one element by one bf16 ulp, so compare at that scale.
    assert _rel(out, h.numpy()) <= 2 ** -7
    # The pure fp64 variant (no rounding) against unrounded composition is tight.
    h = _t64(x.h)
    for kind, wa, wb in x.layers:
        h = _xattn_layer_ref(h, _t64(x.K), _t64(x.V), _t64(wa), _t64(wb), s["Hq"], scale) if kind == "xattn" \
            else _gmu_layer_ref(h, _t64(x.M), _t64(wa), _t64(wb))
    out = oracle.crossdecoder(x.h, x.M, x.K, x.V, x.layers, s["Hq"], scale, round_bf16=False)
    assert _rel(out, h.numpy()) <= 1e-12


def test_outputs_are_bf16_values():
    x, s = _tiny(["gmu", "xattn"])
    out = oracle.crossdecoder(x.h, x.M, x.K, x.V, x.layers, s["Hq"])
    assert np.array_equal(out, torch.from_numpy(out).to(torch.bfloat16).double().numpy())


def test_zero_output_weights_are_identity():
    """Wo = 0 or W2 = 0 makes the layer's branch vanish: h passes unchanged."""
    x, s = _tiny(["xattn", "gmu"])
    layers = [(k, wa, torch.zeros_like(wb)) for k, wa, wb in x.layers]
    out = oracle.crossdecoder(x.h, x.M, x.K, x.V, layers, s["Hq"])
    assert np.array_equal(out, x.h.double().numpy())


def test_layer_order_matters():
    x, s = _tiny(["xattn", "gmu"])
    a = oracle.crossdecoder(x.h, x.M, x.K, x.V, x.layers, s["Hq"])
    b = oracle.crossdecoder(x.h, x.M, x.K, x.V, x.layers[::-1], s["Hq"])
    assert _rel(a, b) > 1e-3


def test_all_gmu_and_all_xattn_stacks():
    """Structural special cases: an all-GMU stack (the pages' all-GMU ablation)
    and an all-attention stack run layer by layer through the primitives."""
    for kinds in (["gmu"] * 3, ["xattn"] * 3):
        x, s = _tiny(kinds)
        h = x.h.double().numpy()
        for kind, wa, wb in x.layers:
            if kind == "gmu":
                y = oracle.gmu(x.M.double().numpy(), h, wa.double().numpy(), wb.double().numpy())
            else:
                q = h @ wa.double().numpy().T
                o = oracle.xattn(q.reshape(s["B"], s["Hq"], s["D"]), x.K, x.V).reshape(s["B"], -1)
                y = o @ wb.double().numpy().T
            h = oracle.round_bf16(h + y)
        out = oracle.crossdecoder(x.h, x.M, x.K, x.V, x.layers, s["Hq"])
        assert _rel(out, h) <= 2 ** -7


# ------------------------------------------------------------ byte counts

def _analytic_layer_bytes(kind, B, d_model, d_inner, Hkv, D, N, e=2):
    """Distinct bytes one layer of a decode step touches, per category."""
    if kind == "xattn":
        return dict(kv_cache=B * Hkv * N * D * 2 * e, state_in=B * d_model * e, state_out=B * d_model * e,
                    weights=2 * d_model * d_model * e)
    return dict(kv_cache=0, state_in=B * (d_model + d_inner) * e, state_out=B * d_model * e,
                weights=2 * d_model * d_inner * e)


@pytest.mark.parametrize("N", [1, 16, 256, 4096])
def test_byte_counts_per_layer(N):
    """Pin (c): counted bytes equal the analytic formulas at every N; the GMU
    layer's state bytes do not change with N, the attention layer's cache
    bytes grow by Hkv·D·2·2 per cached position per sequence."""
    kinds = ["xattn", "gmu"]
    B, Hq, Hkv, D, d_inner = 2, 4, 2, 8, 48
    x, s = _tiny(kinds, B=B, Hq=Hq, Hkv=Hkv, D=D, L=N, d_inner=d_inner, seed=N)
    _, per_layer = oracle.crossdecoder(x.h, x.M, x.K, x.V, x.layers, Hq, count_bytes=True)
    for kind, got in zip(kinds, per_layer):
        assert got == _analytic_layer_bytes(kind, B, Hq * D, d_inner, Hkv, D, N)


def test_gmu_state_independent_of_N_and_attention_linear():
    B, Hq, Hkv, D, d_inner = 1, 4, 2, 8, 32
    gmu_state, kv = [], []
    Ns = [1, 16, 256, 4096]
    for N in Ns:
        x, s = _tiny(["xattn", "gmu"], B=B, Hq=Hq, Hkv=Hkv, D=D, L=N, d_inner=d_inner, seed=1)
        _, pl = oracle.crossdecoder(x.h, x.M, x.K, x.V, x.layers, Hq, count_bytes=True)
        gmu_state.append(pl[1]["state_in"] + pl[1]["state_out"] + pl[1]["kv_cache"])
        kv.append(pl[0]["kv_cache"])
    assert len(set(gmu_state)) == 1
    slopes = {(kv[i + 1] - kv[i]) / (Ns[i + 1] - Ns[i]) for i in range(len(Ns) - 1)}
    assert slopes == {Hkv * D * 2 * 2}


def test_analytic_bytes_at_model_width():
    """The same formulas at the full decode-step width: 4096 cache bytes per
    position per sequence (142.6 MB per sequence per attention layer at
    N = 34816) against 24576 GMU state bytes per sequence at any N."""
    c = workload.CROSSDECODER
    xa = _analytic_layer_bytes("xattn", 1, c["d_model"], c["d_inner"], c["Hkv"], c["D"], c["L"])
    gm = _analytic_layer_bytes("gmu", 1, c["d_model"], c["d_inner"], c["Hkv"], c["D"], c["L"])
    assert xa["kv_cache"] == 34816 * 4096 == 142_606_336
    assert gm["state_in"] + gm["state_out"] == 24_576
    step = sum(_analytic_layer_bytes(k, c["B"], c["d_model"], c["d_inner"], c["Hkv"], c["D"], c["L"])[cat]
               for k in workload.layer_kinds(c["n_layers"]) for cat in ("kv_cache", "weights"))
    assert step == 8 * 4_563_402_752 + 8 * 75_497_472 + 8 * 37_748_736
