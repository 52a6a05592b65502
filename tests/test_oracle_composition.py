"""Pins for the oracle's whole-model compositions (oracle.sambay_prefill and
oracle.sambay_decode_step) against an independent torch fp64 composition of
the same model (tests/torch_model.py).

What is composed (Paper-Notes reading notes on "Decoder-Hybrid-Decoder
Architecture for Efficient Reasoning with Long Generation", section 整体框架):
the self-decoder (SSM layers and sliding-window attention layers, ending in
one full-attention layer) runs first; that final layer's keys and values are
the single shared cache; the cross-decoder then alternates cross-attention
over that cache with GMU layers, and every GMU reuses the memory M of the
self-decoder's last SSM layer (section 关键设计).  Each layer is the plain
pre-norm layer: mixer on RMSNorm(h; norm1), then the SwiGLU MLP on
RMSNorm(h; norm2).

The torch side is a different computation: the SSM layer in parallel form
(materialised mixing matrix), attention over the prompt with an explicit
mask, and a decode step at position p computed as the full forward of that
sequence's p + 1 tokens, with no ring buffer, cache slot or carried state.
A misreading in either composition (an MLP without its norm, M taken from
the wrong SSM layer, the shared cache written by a sliding-window layer, a
ring slot off by one, a dropped residual) makes the two disagree far above
fp64 rounding; tests/test_oracle_mutations.py plants such mistakes in the
oracle's compositions and requires these pins to catch them.
"""
import numpy as np
import pytest
import torch

import oracle
import torch_model as tm
import workload

B, T, DM, DI, NS, R, KC, DF, HQ, HKV, D, W = 2, 9, 64, 96, 4, 8, 4, 48, 4, 2, 16, 4
L = 12                                # shared-cache capacity for the decode step (> every position used)
SAMBA = ["mamba", "swa", "mamba", "swa", "attn"]
TAIL_SSM = ["swa", "mamba", "attn", "mamba"]        # an SSM layer after the cache-producing layer
CROSS = ["xattn", "gmu", "xattn", "gmu"]


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _inputs(self_kinds, seed, fresh):
    return workload.sambay_prefill_inputs(B, T, DM, DI, NS, R, KC, DF, HQ, HKV, D, W, T, self_kinds, CROSS,
                                          seed=seed, fresh=fresh)


def _close(got, ref, round_h):
    """fp64 compositions of the same definitions agree to rounding; with the
    bf16 residual stream both round at the same points, and a value whose
    fp64 pre-rounding sums straddle a bf16 rounding boundary may land one
    bf16 step apart (then propagate), so that case is held to a bar two
    orders under what any composition mistake produces here, and most
    elements must still agree to fp64 rounding."""
    if round_h:
        got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
        near = np.abs(got - ref) <= 1e-10 * max(float(np.max(np.abs(ref))), 1e-300)
        return _rel(got, ref) <= 1e-2 and np.mean(near) > 0.9
    return _rel(got, ref) <= 1e-10


@pytest.mark.parametrize("self_kinds,seed,fresh,round_h", [
    (SAMBA, 1, False, False), (SAMBA, 2, True, True), (TAIL_SSM, 3, False, False), (TAIL_SSM, 4, False, True)])
def test_prefill_matches_torch_composition(self_kinds, seed, fresh, round_h):
    inp = _inputs(self_kinds, seed, fresh)
    got = oracle.sambay_prefill(inp.x, inp.self_layers, inp.cross_layers, HQ, HKV, window=W, round_h=round_h)
    for b in range(B):
        ref = tm.self_decoder(inp.x[b], inp.self_layers, HQ, HKV, W, round_h=round_h, seq=b)
        assert _close(got["h_last"][b], ref["h"][-1].numpy(), round_h)
        assert _close(got["M_last"][b], ref["M"][-1].numpy(), round_h)
        ia = self_kinds.index("attn")
        assert _close(got["K"][b], ref["layers"][ia]["k"].transpose(0, 1).numpy(), round_h)
        assert _close(got["V"][b], ref["layers"][ia]["v"].transpose(0, 1).numpy(), round_h)
        for i, kind in enumerate(self_kinds):
            if kind == "mamba":
                assert _close(got["layers"][i]["conv_state"][b], ref["layers"][i]["conv_state"], round_h)
                assert _close(got["layers"][i]["ssm_state"][b], ref["layers"][i]["ssm_state"], round_h)
            else:
                assert _close(got["layers"][i]["k"][b], ref["layers"][i]["k"].numpy(), round_h)
                assert _close(got["layers"][i]["v"][b], ref["layers"][i]["v"].numpy(), round_h)
        Kb = ref["layers"][ia]["k"].transpose(0, 1)[None]
        Vb = ref["layers"][ia]["v"].transpose(0, 1)[None]
        h_out = tm.cross_decoder(ref["h"][-1:], ref["M"][-1:], Kb, Vb, [T], inp.cross_layers, HQ, round_h=round_h)
        assert _close(got["h_out"][b], h_out[0].numpy(), round_h)


def _decode_state(inp, self_kinds, pos, round_h, seed):
    """The states a decode step at positions pos[b] starts from, built from
    the torch forward of each sequence's first pos[b] tokens: SSM windows
    and states, sliding-window rings (slot t mod W holds token t; slots of
    tokens that are no longer, or not yet, visible hold noise) and the shared
    cache (rows 0 .. pos[b]-1; the rest noise)."""
    rng = np.random.default_rng(seed)
    layers = [dict(ly) for ly in inp.self_layers]
    K = rng.standard_normal((B, HKV, L, D))
    V = rng.standard_normal((B, HKV, L, D))
    for i, kind in enumerate(self_kinds):
        if kind == "mamba":
            layers[i]["conv_state"] = np.array(tm.t64(inp.self_layers[i]["conv_state"]).numpy())
            layers[i]["ssm_state"] = np.array(tm.t64(inp.self_layers[i]["ssm_state"]).numpy())
        elif kind == "swa":
            layers[i]["kring"] = rng.standard_normal((B, HKV, W, D))
            layers[i]["vring"] = rng.standard_normal((B, HKV, W, D))
    for b in range(B):
        p = int(pos[b])
        pre = tm.self_decoder(inp.x[b, :p], inp.self_layers, HQ, HKV, W, round_h=round_h, seq=b)
        for i, kind in enumerate(self_kinds):
            r = pre["layers"][i]
            if kind == "mamba":
                layers[i]["conv_state"][b] = r["conv_state"]
                layers[i]["ssm_state"][b] = r["ssm_state"]
            elif kind == "swa":
                for t in range(max(0, p - W + 1), p):
                    layers[i]["kring"][b, :, t % W] = r["k"][t].numpy()
                    layers[i]["vring"][b, :, t % W] = r["v"][t].numpy()
            else:
                K[b, :, :p] = r["k"].transpose(0, 1).numpy()
                V[b, :, :p] = r["v"].transpose(0, 1).numpy()
    return layers, K, V


@pytest.mark.parametrize("self_kinds,seed,fresh,round_h", [
    (SAMBA, 5, False, False), (SAMBA, 6, True, True), (TAIL_SSM, 7, False, False)])
def test_decode_step_matches_torch_forward(self_kinds, seed, fresh, round_h):
    """One decode step at per-sequence positions (one past the window, one
    before the ring is full) equals the last token of the full forward."""
    inp = _inputs(self_kinds, seed, fresh)
    pos = np.array([T - 1, 2], dtype=np.int32)
    layers, K, V = _decode_state(inp, self_kinds, pos, round_h, seed)
    xnew = torch.stack([inp.x[b, int(pos[b])] for b in range(B)])
    got = oracle.sambay_decode_step(xnew, layers, inp.cross_layers, HQ, HKV, pos, K, V, window=W, round_h=round_h)
    ia = self_kinds.index("attn")
    for b in range(B):
        p = int(pos[b])
        ref = tm.self_decoder(inp.x[b, :p + 1], inp.self_layers, HQ, HKV, W, round_h=round_h, seq=b)
        assert _close(got["h_self"][b], ref["h"][-1].numpy(), round_h)
        assert _close(got["M_last"][b], ref["M"][-1].numpy(), round_h)
        # the shared cache: row p written by the final attention layer, the rest untouched
        assert _close(got["K"][b, :, :p + 1], ref["layers"][ia]["k"].transpose(0, 1).numpy(), round_h)
        assert _close(got["V"][b, :, :p + 1], ref["layers"][ia]["v"].transpose(0, 1).numpy(), round_h)
        assert np.array_equal(got["K"][b, :, p + 1:], K[b, :, p + 1:])
        for i, kind in enumerate(self_kinds):
            r = ref["layers"][i]
            if kind == "mamba":
                assert _close(got["layers"][i]["conv_state"][b], r["conv_state"], round_h)
                assert _close(got["layers"][i]["ssm_state"][b], r["ssm_state"], round_h)
            elif kind == "swa":
                assert _close(got["layers"][i]["kring"][b, :, p % W], r["k"][p].numpy(), round_h)
                assert _close(got["layers"][i]["vring"][b, :, p % W], r["v"][p].numpy(), round_h)
        Kb = ref["layers"][ia]["k"].transpose(0, 1)[None]
        Vb = ref["layers"][ia]["v"].transpose(0, 1)[None]
        h_out = tm.cross_decoder(ref["h"][-1:], ref["M"][-1:], Kb, Vb, [p + 1], inp.cross_layers, HQ,
                                 round_h=round_h)
        assert _close(got["h_out"][b], h_out[0].numpy(), round_h)


def test_the_composition_pins_are_not_vacuous():
    """Each composition choice the pins rely on changes the result by orders
    of magnitude more than the fp64 bar (1e-10) of the unrounded cases:
    dropping norm2, taking M from the first SSM layer, or letting the window
    layers see the whole prompt.  (The MLP branch is small next to h at
    these weight scales, so the rounded cases alone would not resolve a
    missing norm2; the unrounded ones do.)"""
    inp = _inputs(SAMBA, 8, False)
    base = oracle.sambay_prefill(inp.x, inp.self_layers, inp.cross_layers, HQ, HKV, window=W, round_h=False)
    no_norm2 = [dict(ly, norm2=None) for ly in inp.self_layers]
    a = oracle.sambay_prefill(inp.x, no_norm2, inp.cross_layers, HQ, HKV, window=W, round_h=False)
    assert _rel(a["h_last"], base["h_last"]) > 1e-5
    first_ssm = [ly for ly in inp.self_layers if ly["kind"] == "mamba"][0]
    ref = tm.self_decoder(inp.x[0], [first_ssm], HQ, HKV, W, round_h=False, seq=0)
    assert _rel(ref["M"][-1].numpy(), base["M_last"][0]) > 1e-1
    c = oracle.sambay_prefill(inp.x, inp.self_layers, inp.cross_layers, HQ, HKV, window=T, round_h=False)
    assert _rel(c["h_last"], base["h_last"]) > 1e-5
