"""Pins for the oracle's ragged-batch attention and the complete cross-decoder
layer (pre-RMSNorm mixer and pre-RMSNorm SwiGLU MLP).

The pages define the GMU and the cross-attention over the one shared KV cache
(Paper-Notes reading notes, "Decoder-Hybrid-Decoder Architecture for Efficient
Reasoning with Long Generation", sections 关键设计 and 整体框架) but not the
norm, the MLP or how a serving batch with sequences at different lengths is
laid out; those follow the plain Transformer readings stated in the oracle
and are pinned here by closed forms, by independent torch fp64 compositions
and by reduction to the already-pinned functions.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import torch_model as tm
import workload

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")))


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ------------------------------------------------------------- closed forms

@pytest.mark.parametrize("case", GOLDEN["rmsnorm"], ids=lambda c: c["name"])
def test_rmsnorm_closed_forms(case):
    y = oracle.rmsnorm(np.array(case["x"]), np.array(case["g"]), eps=case["eps"])
    np.testing.assert_allclose(y, np.array(case["y"]), rtol=1e-15, atol=1e-15)


@pytest.mark.parametrize("case", GOLDEN["swiglu"], ids=lambda c: c["name"])
def test_swiglu_closed_forms(case):
    y = oracle.swiglu(np.array(case["x"]), np.array(case["Wg"]), np.array(case["Wu"]), np.array(case["Wd"]))
    np.testing.assert_allclose(y, np.array(case["y"]), rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("case", GOLDEN["xattn_varlen"], ids=lambda c: c["name"])
def test_xattn_varlen_closed_forms(case):
    out = oracle.xattn_varlen(np.array(case["q"]), np.array(case["K"]), np.array(case["V"]), case["lens"],
                              scale=case["scale"])
    np.testing.assert_allclose(out, np.array(case["out"]), rtol=1e-14, atol=1e-14)


# ------------------------------------------------------- ragged attention

def _ragged(B=5, Hq=6, Hkv=2, D=16, L=77, seed=3):
    x = workload.xattn_inputs(B, Hq, Hkv, D, L, seed=seed)
    return x, [1, L, L - 1, 33, 40][:B]


def test_varlen_equals_attention_over_a_truncated_copy():
    """Sequence b's result equals the plain attention over a contiguous copy of
    its first lens[b] positions: catches a wrong (sequence, head) stride when the
    cache has room for more positions than are used."""
    x, lens = _ragged()
    out = oracle.xattn_varlen(x.q, x.K, x.V, lens)
    for b, n in enumerate(lens):
        ref = oracle.xattn(x.q[b:b + 1], x.K[b:b + 1, :, :n].contiguous(), x.V[b:b + 1, :, :n].contiguous())
        assert np.array_equal(out[b:b + 1], ref)


def test_varlen_full_lengths_equal_plain_attention():
    x, _ = _ragged()
    L = x.K.shape[2]
    assert np.array_equal(oracle.xattn_varlen(x.q, x.K, x.V, [L] * x.q.shape[0]), oracle.xattn(x.q, x.K, x.V))


def test_varlen_matches_torch_sdpa():
    """Independent implementation: torch fp64 scaled_dot_product_attention per
    sequence on the visible positions, KV heads repeated per query group."""
    x, lens = _ragged()
    out = oracle.xattn_varlen(x.q, x.K, x.V, lens)
    G = x.q.shape[1] // x.K.shape[1]
    for b, n in enumerate(lens):
        q = x.q[b].double().unsqueeze(1)                       # [Hq, 1, D]
        k = x.K[b, :, :n].double().repeat_interleave(G, 0)     # [Hq, n, D]
        v = x.V[b, :, :n].double().repeat_interleave(G, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v).squeeze(1).numpy()
        assert _rel(out[b], ref) < 1e-13


def test_varlen_single_position_returns_its_value():
    x, _ = _ragged()
    B = x.q.shape[0]
    out = oracle.xattn_varlen(x.q, x.K, x.V, [1] * B)
    G = x.q.shape[1] // x.K.shape[1]
    ref = x.V[:, :, 0].double().repeat_interleave(G, 1).numpy()
    assert np.array_equal(out, ref)


def test_varlen_never_reads_past_the_length():
    """NaN in every position past lens[b] leaves the result unchanged."""
    x, lens = _ragged()
    K, V = x.K.clone(), x.V.clone()
    for b, n in enumerate(lens):
        K[b, :, n:] = float("nan")
        V[b, :, n:] = float("nan")
    assert np.array_equal(oracle.xattn_varlen(x.q, K, V, lens), oracle.xattn_varlen(x.q, x.K, x.V, lens))


def test_varlen_zero_length_gives_zeros_and_bad_lengths_are_rejected():
    x, lens = _ragged()
    out = oracle.xattn_varlen(x.q, x.K, x.V, [0] + lens[1:])
    assert np.all(out[0] == 0.0) and np.array_equal(out[1:], oracle.xattn_varlen(x.q, x.K, x.V, lens)[1:])
    L = x.K.shape[2]
    with pytest.raises(ValueError):
        oracle.xattn_varlen(x.q, x.K, x.V, [L + 1] + lens[1:])
    with pytest.raises(ValueError):
        oracle.xattn_varlen(x.q, x.K, x.V, [-1] + lens[1:])


# ------------------------------------------------------- norm and MLP

def test_rmsnorm_matches_torch_and_is_scale_invariant():
    x = workload.normal((5, 48), seed=7, dtype=torch.float32)
    g = (1.0 + workload.normal((48,), std=0.1, seed=8, dtype=torch.float32)).to(torch.bfloat16)
    eps = 1e-5
    y = oracle.rmsnorm(x, g, eps)
    xd = x.double()
    ref = (xd / torch.sqrt((xd * xd).mean(-1, keepdim=True) + eps) * g.double()).numpy()
    assert _rel(y, ref) < 1e-14
    # Without eps the norm is invariant to a positive rescaling of the row.
    assert _rel(oracle.rmsnorm(7.0 * xd.numpy(), g, 0.0), oracle.rmsnorm(xd.numpy(), g, 0.0)) < 1e-14
    # eps keeps a zero row finite.
    assert np.all(oracle.rmsnorm(np.zeros((1, 48)), g, eps) == 0.0)


def test_swiglu_matches_torch():
    x = workload.normal((4, 40), seed=9, dtype=torch.float32)
    Wg = workload.normal((56, 40), std=0.2, seed=10)
    Wu = workload.normal((56, 40), std=0.2, seed=11)
    Wd = workload.normal((40, 56), std=0.2, seed=12)
    y = oracle.swiglu(x, Wg, Wu, Wd)
    xd = x.double()
    ref = ((torch.nn.functional.silu(xd @ Wg.double().T) * (xd @ Wu.double().T)) @ Wd.double().T).numpy()
    assert _rel(y, ref) < 1e-13


# ------------------------------------------------ complete cross-decoder

def _ex(kinds=("xattn", "gmu", "xattn", "gmu"), lens="ragged", norms=True, mlp=True, seed=0, B=3):
    Hq, Hkv, D, L, d_inner, d_ff = 4, 2, 8, 19, 48, 40
    d_model = Hq * D
    x = workload.crossdecoder_ex_inputs(B, d_model, d_inner, d_ff, Hq, Hkv, D, L, len(kinds), seed=seed,
                                        kinds=list(kinds), lens=lens, norms=norms, mlp=mlp)
    return x, Hq


def test_ex_without_norms_mlp_or_lengths_is_the_plain_step():
    """No norms, no MLP, every position visible: the complete step reduces to
    the (separately pinned) plain cross-decoder step."""
    x, Hq = _ex(lens=None, norms=False, mlp=False)
    plain = oracle.crossdecoder(x.h, x.M, x.K, x.V, [(l["kind"], l["w_a"], l["w_b"]) for l in x.layers], Hq)
    assert np.array_equal(oracle.crossdecoder_ex(x.h, x.M, x.K, x.V, x.layers, Hq), plain)


def _torch_ex(x, Hq, eps=1e-5):
    """Layer-by-layer composition from torch fp64 operations (tests/torch_model.py),
    h rounded to bf16 by the (separately pinned) oracle rounding after every
    residual add."""
    L = x.K.shape[2]
    lens = [L] * x.h.shape[0] if x.lens is None else [int(v) for v in x.lens]
    return tm.cross_decoder(x.h, x.M, x.K, x.V, lens, x.layers, Hq, eps=eps).numpy()


@pytest.mark.parametrize("kinds", [("xattn", "gmu", "xattn", "gmu"), ("gmu", "xattn"), ("xattn", "xattn")])
def test_ex_matches_torch_composition(kinds):
    x, Hq = _ex(kinds=kinds, lens=[19, 1, 7])
    got = oracle.crossdecoder_ex(x.h, x.M, x.K, x.V, x.layers, Hq, lens=x.lens)
    ref = _torch_ex(x, Hq)
    # Both round h to bf16 after every add; a rounding-boundary case may differ by one bf16 step.
    assert _rel(got, ref) < 1e-2
    assert np.mean(got == ref) > 0.95


def test_ex_zero_length_sequence_gets_no_attention():
    """A sequence with no visible position: its attention output is zero, so an
    all-attention stack without MLP leaves its h unchanged."""
    x, Hq = _ex(kinds=("xattn", "xattn"), lens=[0, 5, 19], norms=True, mlp=False)
    got = oracle.crossdecoder_ex(x.h, x.M, x.K, x.V, x.layers, Hq, lens=x.lens)
    assert np.array_equal(got[0], x.h[0].double().numpy())
    assert not np.array_equal(got[1], x.h[1].double().numpy())


def test_ex_mlp_changes_the_result_and_zero_down_projection_removes_it():
    x, Hq = _ex()
    with_mlp = oracle.crossdecoder_ex(x.h, x.M, x.K, x.V, x.layers, Hq, lens=x.lens)
    no_mlp = [dict(l, w_gate=None, w_up=None, w_down=None) for l in x.layers]
    zero_down = [dict(l, w_down=torch.zeros_like(l["w_down"])) for l in x.layers]
    base = oracle.crossdecoder_ex(x.h, x.M, x.K, x.V, no_mlp, Hq, lens=x.lens)
    assert not np.array_equal(with_mlp, base)
    assert np.array_equal(oracle.crossdecoder_ex(x.h, x.M, x.K, x.V, zero_down, Hq, lens=x.lens), base)


def test_ex_norm_gain_scales_the_branch_input():
    """Doubling norm1's gain doubles every branch input; for a GMU layer with M
    scaled by 1/2 and W2 unchanged this is not the identity (SiLU is not
    linear), so the gain must reach the product: compare against the torch
    composition with the doubled gain."""
    x, Hq = _ex(kinds=("gmu",), lens=None, mlp=False)
    x.layers[0]["norm1"] = (x.layers[0]["norm1"].float() * 2).to(torch.bfloat16)
    got = oracle.crossdecoder_ex(x.h, x.M, x.K, x.V, x.layers, Hq)
    assert _rel(got, _torch_ex(x, Hq)) < 1e-2
